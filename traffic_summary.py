"""Turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs into the traffic summaries.

    python traffic_summary.py [--score] <fetch_dir> <write_dir> \
        <copy_fetch_dir> <copy_write_dir> <out.md>

Without a flag the summary covers the decoder (dec_small_k on the small workload); with
--score, the action-scoring kernel (score_lse_res_k on bench.py's scoring leg: head
V=32000, d=1024, bf16, 65536 rows); with --sample, the sampling kernel (sample_topk_k, top-k 50 then top-p
0.95, on bench.py's sampling leg: 512 rows x V=32000).

Each directory holds the counter_collection.csv of one `rocprofv3 --pmc <counter>` run:
the decoder runs come from `bench.py --only-small --steps 1 --warmup 0`, the scoring and
sampling runs from `bench.py --only-scoring --steps 1 --warmup 0 --no-cpu-baseline`, the copy
runs from `bench.py --copy-kernel` (1 GiB read + 1 GiB written).  The counters report
KiB per dispatch; each is scaled by the ratio true bytes / counter bytes measured on the
copy kernel, and the decoder's per-launch traffic is reported together with the kernel
source hash so that a stale summary is never used for a changed kernel.
"""
from __future__ import annotations

import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return list(csv.DictReader(open(files[0])))


def _value(d, counter, kernel_sub):
    vals = [float(r["Counter_Value"]) for r in _rows(d)
            if r["Counter_Name"] == counter and kernel_sub in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"{counter} for a kernel matching {kernel_sub!r} not found in {d}")
    return max(vals)


def score_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, out):
    import bench  # noqa: E402
    copy_bytes = float(1 << 30)
    c_fetch = _value(cfetch_dir, "FETCH_SIZE", "copy") * 1024.0
    c_write = _value(cwrite_dir, "WRITE_SIZE", "copy") * 1024.0
    k_fetch = _value(fetch_dir, "FETCH_SIZE", "score_lse_res_k") * 1024.0
    k_write = _value(write_dir, "WRITE_SIZE", "score_lse_res_k") * 1024.0
    f_fetch, f_write = copy_bytes / c_fetch, copy_bytes / c_write
    traffic = k_fetch * f_fetch + k_write * f_write
    alg = bench.scoring_rows(65536, 1024, 32000)
    with open(out, "w") as f:
        f.write("# score_lse_res_k on the scoring leg (head V=32000, d=1024, bf16, 65536 rows): HBM traffic per launch\n\n")
        f.write("Commands (from the repository root on the GPU box, `cd /tmp && export TMPDIR=/tmp` first):\n\n")
        f.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -- python3 <repo>/bench.py --only-scoring --steps 1 --warmup 0 --no-cpu-baseline\n")
        f.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -- python3 <repo>/bench.py --only-scoring --steps 1 --warmup 0 --no-cpu-baseline\n")
        f.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <copy_fetch_dir> -- python3 <repo>/bench.py --copy-kernel\n")
        f.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <copy_write_dir> -- python3 <repo>/bench.py --copy-kernel\n")
        f.write("    python traffic_summary.py --score <fetch_dir> <write_dir> <copy_fetch_dir> <copy_write_dir> profiles/score_lse_res_k_head32000x1024_traffic.md\n\n")
        f.write("The kernel is bound by the matrix cores and the L2-to-CU path (the head is re-read from L2 once per\n")
        f.write("64-row block), not by HBM; the counters show that the s rows and the head leave HBM about once.\n\n")
        f.write(f"- copy kernel: 1 GiB read / 1 GiB written; FETCH_SIZE reads {c_fetch:.4e} B, WRITE_SIZE {c_write:.4e} B\n")
        f.write(f"- fetch scale: {f_fetch:.4f}\n")
        f.write(f"- write scale: {f_write:.4f}\n")
        f.write(f"- scoring FETCH_SIZE bytes per launch (raw): {k_fetch:.4e}\n")
        f.write(f"- scoring WRITE_SIZE bytes per launch (raw): {k_write:.4e}\n")
        f.write(f"- traffic bytes per launch: {traffic:.6e}\n")
        f.write(f"- algorithmic bytes per launch: {alg:.6e}\n")
        f.write(f"- traffic / algorithmic: {traffic / alg:.4f}\n")
        f.write(f"- kernel source sha256/16: `{bench.kernel_source_hash(bench.SCORE_SOURCES)}`\n")
    print(open(out).read())


def sample_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, out):
    import bench  # noqa: E402
    copy_bytes = float(1 << 30)
    c_fetch = _value(cfetch_dir, "FETCH_SIZE", "copy") * 1024.0
    c_write = _value(cwrite_dir, "WRITE_SIZE", "copy") * 1024.0
    k_fetch = _value(fetch_dir, "FETCH_SIZE", "sample_topk_k") * 1024.0
    k_write = _value(write_dir, "WRITE_SIZE", "sample_topk_k") * 1024.0
    f_fetch, f_write = copy_bytes / c_fetch, copy_bytes / c_write
    traffic = k_fetch * f_fetch + k_write * f_write
    alg = 512 * 32000 * 4.0 + 512 * 12.0
    with open(out, "w") as f:
        f.write("# sample_topk_k on the sampling leg (512 rows x V=32000 fp32 logits, top-k 50 then top-p 0.95): HBM traffic per launch\n\n")
        f.write("Commands (from the repository root on the GPU box, `cd /tmp && export TMPDIR=/tmp` first):\n\n")
        f.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -- python3 <repo>/bench.py --only-scoring --steps 1 --warmup 0 --no-cpu-baseline\n")
        f.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -- python3 <repo>/bench.py --only-scoring --steps 1 --warmup 0 --no-cpu-baseline\n")
        f.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <copy_fetch_dir> -- python3 <repo>/bench.py --copy-kernel\n")
        f.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <copy_write_dir> -- python3 <repo>/bench.py --copy-kernel\n")
        f.write("    python traffic_summary.py --sample <fetch_dir> <write_dir> <copy_fetch_dir> <copy_write_dir> profiles/sample_topk_k_512x32000_traffic.md\n\n")
        f.write("The lean top-k kernel's dispatches are taken (the leg's headline setting); the other two settings run sample_k.\n\n")
        f.write(f"- copy kernel: 1 GiB read / 1 GiB written; FETCH_SIZE reads {c_fetch:.4e} B, WRITE_SIZE {c_write:.4e} B\n")
        f.write(f"- fetch scale: {f_fetch:.4f}\n")
        f.write(f"- write scale: {f_write:.4f}\n")
        f.write(f"- sampling FETCH_SIZE bytes per launch (raw): {k_fetch:.4e}\n")
        f.write(f"- sampling WRITE_SIZE bytes per launch (raw): {k_write:.4e}\n")
        f.write(f"- traffic bytes per launch: {traffic:.6e}\n")
        f.write(f"- algorithmic bytes per launch: {alg:.6e}\n")
        f.write(f"- traffic / algorithmic: {traffic / alg:.4f}\n")
        f.write(f"- kernel source sha256/16: `{bench.kernel_source_hash(bench.SAMPLE_SOURCES)}`\n")
    print(open(out).read())


def mfma_summary(counter_dir, out):
    """Executed bf16 matrix operations of the scoring kernel against 2 N d V (N = 65536 rows,
    d = 1024, V = 32000), from a `rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16` run of the scoring
    leg; the counter is in units of 512 operations."""
    rows = _rows(counter_dir)
    per = {}
    for r in rows:
        if r["Counter_Name"] != "SQ_INSTS_VALU_MFMA_MOPS_BF16":
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    alg = 2.0 * 65536 * 1024 * 32000
    with open(out, "w") as f:
        f.write("# MFMA operation count: action scoring, head V=32000 x d=1024 (bf16), N=65536 rows\n\n")
        f.write("Commands (from the repository root on the GPU box, `cd /tmp && export TMPDIR=/tmp` first):\n\n")
        f.write("    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv -d <dir> -- python3 <repo>/bench.py --only-scoring --steps 1 --warmup 0 --no-cpu-baseline\n")
        f.write("    python traffic_summary.py --mfma <dir> profiles/score_lse_res_k_head32000x1024_mfma.md\n\n")
        f.write("`SQ_INSTS_VALU_MFMA_MOPS_BF16` counts bf16 matrix operations in units of 512.  Per dispatch,\n")
        f.write("averaged over the run's dispatches of each kernel that issues any:\n\n")
        f.write("| kernel | dispatches | executed bf16 FLOP (x 512) | algorithmic 2 N d V | executed / algorithmic |\n")
        f.write("|---|---:|---:|---:|---:|\n")
        for name, vals in sorted(per.items(), key=lambda kv: -max(kv[1])):
            avg = sum(vals) / len(vals) * 512.0
            if avg == 0:
                continue
            short = name.replace("rlt::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            if len(short) > 70:
                short = short[:67] + "..."
            f.write(f"| `{short}` | {len(vals)} | {avg:.4e} | {alg:.4e} | {avg / alg:.4f} |\n")
        f.write("\nThe scoring kernel sweeps the vocabulary in 512-column steps, 63 x 512 = 32256 columns for\n")
        f.write("V = 32000 (32256 / 32000 = 1.0080), so it executes that much more than the algorithmic count.\n")
    print(open(out).read())


def main(argv):
    if argv and argv[0] == "--mfma":
        return mfma_summary(*argv[1:])
    if argv and argv[0] == "--score":
        return score_summary(*argv[1:])
    if argv and argv[0] == "--sample":
        return sample_summary(*argv[1:])
    fetch_dir, write_dir, cfetch_dir, cwrite_dir, out = argv
    import bench  # noqa: E402  (repository root on sys.path)
    copy_bytes = float(1 << 30)
    c_fetch = _value(cfetch_dir, "FETCH_SIZE", "copy") * 1024.0
    c_write = _value(cwrite_dir, "WRITE_SIZE", "copy") * 1024.0
    k_fetch = _value(fetch_dir, "FETCH_SIZE", "dec_small_k") * 1024.0
    k_write = _value(write_dir, "WRITE_SIZE", "dec_small_k") * 1024.0
    f_fetch, f_write = copy_bytes / c_fetch, copy_bytes / c_write
    traffic = k_fetch * f_fetch + k_write * f_write
    from workloads import CONFIGS
    wl = CONFIGS["small"]
    alg = bench.algorithmic_decoder_bytes(wl.model, wl.batch, wl.seq_len)
    with open(out, "w") as f:
        f.write("# dec_small_k on the small workload: HBM traffic per launch (rocprofv3 counters)\n\n")
        f.write("Commands (from the repository root on the GPU box, `cd /tmp && export TMPDIR=/tmp` first):\n\n")
        f.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -- python3 <repo>/bench.py --only-small --steps 1 --warmup 0\n")
        f.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -- python3 <repo>/bench.py --only-small --steps 1 --warmup 0\n")
        f.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <copy_fetch_dir> -- python3 <repo>/bench.py --copy-kernel\n")
        f.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <copy_write_dir> -- python3 <repo>/bench.py --copy-kernel\n")
        f.write("    python traffic_summary.py <fetch_dir> <write_dir> <copy_fetch_dir> <copy_write_dir> profiles/dec_small_k_small_traffic.md\n\n")
        f.write(f"- copy kernel: 1 GiB read / 1 GiB written; FETCH_SIZE reads {c_fetch:.4e} B, WRITE_SIZE {c_write:.4e} B\n")
        f.write(f"- fetch scale: {f_fetch:.4f}\n")
        f.write(f"- write scale: {f_write:.4f}\n")
        f.write(f"- decoder FETCH_SIZE bytes per launch (raw): {k_fetch:.4e}\n")
        f.write(f"- decoder WRITE_SIZE bytes per launch (raw): {k_write:.4e}\n")
        f.write(f"- traffic bytes per launch: {traffic:.6e}\n")
        f.write(f"- algorithmic bytes per launch: {alg:.6e}\n")
        f.write(f"- traffic / algorithmic: {traffic / alg:.4f}\n")
        f.write(f"- kernel source sha256/16: `{bench.kernel_source_hash()}`\n")
    print(open(out).read())


if __name__ == "__main__":
    main(sys.argv[1:])
