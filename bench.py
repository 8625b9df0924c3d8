"""RLT exact-replay benchmark on one MI355X.

The headline is the decoder replay of the 48+48-layer reference model (d=2048, SwiGLU 5632,
W=256, G=1, V=32000, bf16) over B=64 sequences of T=4096 Zipf tokens.  One step = one
contiguous segment of that replay: --steps K splits t = 1..T into K segments, so the K timed
steps are together one exact replay from H_0 (the encoder has run over all T tokens before the
timed region, with the inputs resident in HBM).  value = B*T / (decoder time of the K steps)
in tokens/s; the roofline is the decoder's algorithmic bytes (weights once per step, window
cache read + write, memory rows 1..t of every layer, e_t in and s_t out) over that time,
against 8 TB/s and against the read and copy bandwidth measured on the box in the same run.

    python bench.py [--steps K] [--warmup W] [--config ref48] [--no-cpu-baseline]

Prints ONE JSON line.  Further legs in the same line: the small workload on the persistent
decoder, a 300M-class prefix, RL action scoring, token sampling, prefix snapshots.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
PCIE_PEAK_GBS = 64.0             # host link, PCIe 5.0 x16, one direction
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dec_small_k_small_traffic.md")
KERNEL_SOURCES = ["cross_token_recurrent_amd/csrc/dec_small.hip", "cross_token_recurrent_amd/csrc/device_common.h"]
SCORE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_lse_res_k_head32000x1024_traffic.md")
SCORE_SOURCES = ["cross_token_recurrent_amd/csrc/score.hip", "cross_token_recurrent_amd/csrc/device_common.h"]
SAMPLE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sample_topk_k_512x32000_traffic.md")
SAMPLE_SOURCES = ["cross_token_recurrent_amd/csrc/sample.hip", "cross_token_recurrent_amd/csrc/device_common.h"]


def kernel_source_hash(sources=None) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path: str = TRAFFIC_FILE, sources=None):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None when the
    summary is missing or was taken on a different version of the kernel's sources."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source sha256/16") != kernel_source_hash(sources):
        return None
    try:
        return float(fields["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def copy_kernel(gib: float = 1.0):
    """A plain device copy of known size (calibrates the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}), flush=True)


def algorithmic_decoder_bytes(cfg, B: int, T: int) -> float:
    """Bytes the decoder replay must move, summed over t = 1..T for the whole batch.

    Per step: the in-loop weights once (shared by the B sequences: per layer W_Q, W_K, W_V,
    W_O, W_Qx, W_Ox and the FFN; the merge's W_ge, W_gs, W_fb), and per sequence the window
    cache read + write, every layer's read of memory entries 1..t, e_t in and s_t out (fp32,
    plus the fp32 state)."""
    d, L, F, W = cfg.d_model, cfg.n_layers, cfg.ffn_dim, cfg.window
    p = 2 if cfg.dtype == "bf16" else 4
    ffn = (2 if cfg.ffn_kind == "gelu" else 3) * d * F
    p_loop = L * (6 * d * d + ffn) + 3 * d * d
    total = 0.0
    for t in range(1, T + 1):
        ring = L * 2 * d * p * (min(t - 1, W - 1) + 1)
        mem = L * 2 * d * p * t
        io = d * (p + 4 + 4)
        total += p_loop * p + B * (ring + mem + io)
    return total


def _oracle_one(args):
    """Worker: oracle replay of one sequence (imports only numpy/scipy and the oracle)."""
    cfg, weights, tok, t_limit = args
    import oracle
    m = oracle.OracleModel.from_config(cfg, weights)
    return oracle.replay(m, tok, t_limit)


def host_cores():
    """Cores this process may run on, and the BLAS threads numpy uses on them."""
    cores = len(os.sched_getaffinity(0))
    threads = min(cores, int(os.environ.get("OMP_NUM_THREADS", "0")) or cores)
    return cores, threads


def cpu_baseline(wl, weights, tokens, budget_s: float = 20.0):
    """The fp64 oracle (test infrastructure) timed on this host's cores over a bounded
    sample of whole sequences of the same workload, one sequence per worker process."""
    import multiprocessing as mp

    cores, _ = host_cores()
    # one probe sequence prefix sizes the sample to about budget_s of CPU work
    t_probe = min(wl.seq_len, 128)
    t0 = time.perf_counter()
    _oracle_one((wl.model, weights, tokens[0], t_probe))
    probe = time.perf_counter() - t0
    # cost grows ~linearly in t for the memory part; scale by (T/t_probe)^1.5 as an estimate
    est_seq = probe * (wl.seq_len / t_probe) ** 1.5
    n_seq = int(max(1, min(wl.batch, round(budget_s / max(est_seq, 1e-3)))))
    workers = min(cores, 16, n_seq)
    jobs = [(wl.model, weights, tokens[b], None) for b in range(n_seq)]
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_one, jobs)
    wall = time.perf_counter() - t0
    return {"value": n_seq * wl.seq_len / wall, "unit": "tokens/s", "cores": cores, "workers": workers,
            "kind": "oracle",
            "sample": f"{n_seq} of {wl.batch} sequences x T={wl.seq_len} (full replay incl. encoder and logits), "
                      f"fp64 numpy, one sequence per worker process ({workers} workers on {cores} cores), "
                      f"{wall:.1f} s wall"}


def cpu_baseline_prefix(wl, weights, tokens, budget_s: float = 15.0):
    """The fp64 oracle on a prefix of one sequence of a workload whose full sequences take the
    oracle hours: encoder over t_limit tokens, t_limit decoder steps, logits, with t_limit sized
    by an 8-position probe to about budget_s.  Optimistic as a rate for the whole replay, since
    late steps read more memory rows."""
    import oracle

    cores, threads = host_cores()
    t0 = time.perf_counter()
    m = oracle.OracleModel.from_config(wl.model, weights)
    t1 = time.perf_counter()
    oracle.replay(m, tokens[0], 8)
    probe = time.perf_counter() - t1
    t_limit = int(max(8, min(wl.seq_len, 8 * budget_s / max(probe, 1e-3))))
    t1 = time.perf_counter()
    oracle.replay(m, tokens[0], t_limit)
    wall = time.perf_counter() - t1
    del m
    return {"value": t_limit / wall, "unit": "tokens/s", "cores": cores, "threads": threads, "kind": "oracle",
            "sample": f"sequence 0, positions 1..{t_limit} of T={wl.seq_len} (encoder over {t_limit} tokens, "
                      f"{t_limit} decoder steps, logits), fp64 numpy on {threads} BLAS threads, {wall:.1f} s "
                      f"(+{t1 - t0:.1f} s to convert the weights to fp64, not counted); a prefix rate, "
                      f"optimistic for the whole replay"}


def measured_bandwidth(gib: float = 2.0, reps: int = 5):
    """Read and copy bandwidth of this GPU, measured in the same run with torch kernels."""
    import torch

    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    b.copy_(a)
    a.sum()
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(reps):
        b.copy_(a)
    ev[1].record(stream)
    torch.cuda.synchronize()
    copy = 2.0 * n * 4 * reps / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    ev[0].record(stream)
    for _ in range(reps):
        a.sum()
    ev[1].record(stream)
    torch.cuda.synchronize()
    read = 1.0 * n * 4 * reps / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBps": copy, "sum_read_GBps": read,
            "how": f"torch copy_ (bytes read + written) and torch sum (bytes read) over {gib:g} GiB fp32, "
                   f"{reps} each; the copy is the second roofline denominator"}


def hbm_roofline(nbytes: float, ms: float, bw, kernel: str, traffic=None, **extra):
    achieved = nbytes / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
         "traffic": traffic, "kernel": kernel}
    if bw:
        r["measured_copy_GBps"] = bw["copy_GBps"]
        r["frac_of_measured_copy"] = achieved / bw["copy_GBps"]
    r.update(extra)
    return r


def segment_sizes(T: int, K: int):
    """K contiguous segments covering positions 1..T (the first T % K one longer)."""
    return [T // K + (1 if i < T % K else 0) for i in range(K)]


def headline_replay(wl, steps: int, warmup: int, bw, with_cpu: bool = True):
    """The exact replay of one workload, timed as `steps` contiguous segments of the decoder
    (see the module docstring).  Returns the headline fields."""
    import torch

    import cross_token_recurrent_amd as rlt
    from workloads import make_tokens, make_weights

    cfg, B, T = wl.model, wl.batch, wl.seq_len
    if steps < 1 or steps > T:
        raise SystemExit(f"--steps must be in 1..{T} (segments of the {T}-position replay)")
    t_setup = time.perf_counter()
    weights = make_weights(cfg, wl.weight_seed)
    tokens = make_tokens(cfg.vocab, B, T, wl.token_dist, wl.token_seed)
    dev = torch.device("cuda:0")
    model = rlt.Model(cfg, weights, device=dev)
    state = rlt.State(model, B, T, keep_encoder_cache=False)
    tok = torch.from_numpy(tokens).to(dev)
    stream = torch.cuda.current_stream()
    seg = segment_sizes(T, steps)
    print(f"{wl.name}: model and state ready in {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    if warmup > 0:
        state.reset()
        rlt.rlt_encoder_forward(model, state, tok)
        for n in seg[:warmup]:
            rlt.rlt_decoder_replay(model, state, n)
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 3)]
    state.reset()
    ev[0].record(stream)
    rlt.rlt_encoder_forward(model, state, tok)
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[2].record(stream)
    for k, n in enumerate(seg):
        rlt.rlt_decoder_replay(model, state, n)
        ev[3 + k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    assert state.device_error() == 0
    enc_ms = ev[0].elapsed_time(ev[1])
    seg_ms = [ev[2 + k].elapsed_time(ev[3 + k]) for k in range(steps)]
    dec_ms = sum(seg_ms)
    segments, done, prev = [], 0, 0.0
    for n, ms in zip(seg, seg_ms):
        cum = algorithmic_decoder_bytes(cfg, B, done + n)
        gbs = (cum - prev) / (ms * 1e-3) / 1e9
        segments.append({"t": [done + 1, done + n], "ms": ms, "GBps": gbs, "frac_of_hbm": gbs / HBM_PEAK_GBS})
        done, prev = done + n, cum
    path = {1: "persistent-per-sequence", 2: "batched-phases"}[model.decoder_path(T)]
    del state, model
    torch.cuda.empty_cache()
    ms_step = wall * 1e3 / steps
    out = {
        "value": B * T / wall,
        "ms_per_step": ms_step,
        "decoder_event_ms": dec_ms,
        "decoder_tokens_per_s_events": B * T / (dec_ms * 1e-3),
        "end_to_end_tokens_per_s": B * T / ((enc_ms + dec_ms) * 1e-3),
        "phase_ms": {"encoder": enc_ms, "decoder_replay": dec_ms},
        "decoder_path": path,
        "roofline": hbm_roofline(prev, dec_ms, bw, "decoder step loop (one launch per product, window and "
                                 "cross-attention per layer; cross_part_k streams the memory rows)",
                                 traffic=None, algorithmic_bytes=prev, unit_of_work="one exact replay, t = 1..T"),
        "segments": segments,
    }
    if with_cpu:
        out["cpu_baseline"] = (cpu_baseline(wl, weights, tokens) if wl.seq_len * wl.model.d_model <= (1 << 20)
                               else cpu_baseline_prefix(wl, weights, tokens))
    return out


def scoring_rows(n: int, d: int, V: int) -> float:
    """Algorithmic HBM bytes of one scoring pass: s read once (fp32), the fragment-major
    bf16 head read once, the row log-sum-exp written."""
    return n * d * 4.0 + (V + 15) // 16 * 16 * d * 2.0 + n * 4.0


def _oracle_rows_per_s(fn, rows_total: int, budget_s: float = 6.0):
    """Time an oracle call on growing row samples until about budget_s of host work."""
    import time
    n, used, done = 8, 0.0, 0
    while used < budget_s and done < rows_total:
        t0 = time.perf_counter()
        fn(done, min(n, rows_total - done))
        used += time.perf_counter() - t0
        done += min(n, rows_total - done)
        n *= 2
    return done / used, done, used


def scoring_leg(steps: int, warmup: int, with_cpu: bool = True):
    """RL action scoring (rlt_score_actions) on the 300M-class head: V=32000, d=1024, bf16,
    N = 64 sequences x 1024 response positions.  The head GEMM dominates: 2*N*d*V flops
    per call, priced against the bf16 MFMA peak."""
    import numpy as np
    import torch

    import cross_token_recurrent_amd as rlt
    from workloads import ModelConfig, make_weights

    cfg = ModelConfig(vocab=32000, d_model=1024, n_heads=16, n_layers=1, ffn_dim=64, ffn_kind="swiglu",
                      window=4, mem_groups=1, dtype="bf16")
    dev = torch.device("cuda:0")
    weights = make_weights(cfg, 7)
    model = rlt.Model(cfg, weights, device=dev)
    n = 64 * 1024
    g = torch.Generator(device="cpu").manual_seed(8)
    s = torch.randn(n, cfg.d_model, generator=g).to(dev)
    acts = torch.randint(0, cfg.vocab, (n,), generator=g, dtype=torch.int32).to(dev)
    behav = torch.full((n,), -10.0, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        rlt.rlt_score_actions(model, s, acts, 1.0, behav, stream=stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(steps):
        rlt.rlt_score_actions(model, s, acts, 1.0, behav, stream=stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    # for context: the same scores through torch's library GEMM (bf16 logits written to HBM),
    # then log_softmax and a gather
    w_t = torch.from_numpy(weights["w_out"]).to(dev).to(torch.bfloat16).t().contiguous()
    s_b = s.to(torch.bfloat16)

    def unfused():
        z = torch.matmul(s_b, w_t).float()
        return z.log_softmax(-1).gather(1, acts.long()[:, None])[:, 0]

    unfused()
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(3):
        unfused()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms_unfused = ev[0].elapsed_time(ev[1]) / 3
    del w_t, s_b
    cpu = None
    if with_cpu:
        import numpy as np
        import oracle
        w_out = np.asarray(weights["w_out"], dtype=np.float64)
        s_host = s.cpu().numpy()
        a_host = acts.cpu().numpy()
        rate, done, used = _oracle_rows_per_s(
            lambda i, k: oracle.score_actions(w_out, s_host[i:i + k], a_host[i:i + k]), n)
        blas = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "0")) or 10 ** 6)
        cpu = {"value": rate, "unit": "rows/s", "cores": len(os.sched_getaffinity(0)), "threads": blas, "kind": "oracle",
               "sample": f"{done} of {n} rows through oracle.score_actions (fp64 numpy; the head product "
                         f"on up to {blas} BLAS threads), {used:.1f} s"}
    flops = 2.0 * n * cfg.d_model * cfg.vocab
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": f"RL action scoring, head V={cfg.vocab} d={cfg.d_model} bf16, N={n} rows "
                        f"(64 sequences x 1024 response positions), logp + ratio, logits never written",
            "rows_per_s": n / (ms * 1e-3), "ms_per_call": ms,
            "unfused_torch_ms_per_call": ms_unfused, "cpu_baseline": cpu,
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                         "traffic": measured_traffic(SCORE_TRAFFIC_FILE, SCORE_SOURCES),
                         "kernel": "score_lse_res_k (timed with score_finish_k)", "algorithmic_flops_per_call": flops,
                         "algorithmic_bytes_per_call": scoring_rows(n, cfg.d_model, cfg.vocab)}}


def sampling_leg(steps: int, warmup: int, with_cpu: bool = True):
    """Token sampling (rlt_sample_tokens) for one decode step of the 300M-class workload:
    512 rows x V=32000 fp32 logits, temperature 0.8, top-k 50 then top-p 0.95.  The kernel
    reads each logit once: N*V*4 + N*12 bytes per call, priced against HBM."""
    import torch

    import cross_token_recurrent_amd as rlt

    dev = torch.device("cuda:0")
    n, V = 512, 32000
    g = torch.Generator(device="cpu").manual_seed(9)
    logits = (torch.randn(n, V, generator=g) * 2.0).to(dev)
    u = torch.rand(n, generator=g).to(dev)
    stream = torch.cuda.current_stream()
    # The C-ABI call with its arguments marshalled once: a call through the Python binding
    # (output allocation, checks) takes longer on the host than the kernel on the GPU, so
    # back-to-back binding calls would time the host's launch gaps, not the kernel.
    from cross_token_recurrent_amd import rlt as rlt_binding
    lib = rlt_binding.load_library()
    tok = torch.empty(n, dtype=torch.int32, device=dev)
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    calls = max(20, steps)
    out = {}
    for name, k, p in (("top_k50_top_p0.95", 50, 0.95), ("top_p0.95", 0, 0.95), ("plain", 0, 1.0)):
        params = rlt_binding.rlt_sampling(0.8, k, p)
        args = (ctypes.c_void_p(logits.data_ptr()), n, V, ctypes.byref(params), ctypes.c_void_p(u.data_ptr()),
                ctypes.c_void_p(tok.data_ptr()), ctypes.c_void_p(logp.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        for _ in range(max(1, warmup)):
            if lib.rlt_sample_tokens(*args) != 0:
                raise RuntimeError(lib.rlt_last_error().decode())
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(calls):
            lib.rlt_sample_tokens(*args)
        ev[1].record(stream)
        torch.cuda.synchronize()
        out[name] = ev[0].elapsed_time(ev[1]) / calls
    ms = out["top_k50_top_p0.95"]
    cpu = None
    if with_cpu:
        import oracle
        l_host = logits.cpu().numpy()
        u_host = u.cpu().numpy()
        rate, done, used = _oracle_rows_per_s(
            lambda i, k: oracle.sample_tokens(l_host[i:i + k], u_host[i:i + k], 0.8, 50, 0.95), n)
        cpu = {"value": rate, "unit": "rows/s", "cores": len(os.sched_getaffinity(0)), "threads": 1, "kind": "oracle",
               "sample": f"{done} of {n} rows through oracle.sample_tokens (fp64 numpy), {used:.1f} s"}
    nbytes = n * V * 4.0 + n * 12.0
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"token sampling, {n} rows x V={V} fp32 logits, T=0.8, top-k 50 then top-p 0.95",
            "rows_per_s": n / (ms * 1e-3), "ms_per_call": ms,
            "ms_per_call_by_truncation": out, "cpu_baseline": cpu,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(SAMPLE_TRAFFIC_FILE, SAMPLE_SOURCES), "kernel": "sample_topk_k<16>",
                         "algorithmic_bytes_per_call": nbytes}}


def decoder_300m_leg(t0: int = 1024, n: int = 64, name: str = "300m"):
    """The batched decoder on the 300M-class workload (d=1024, 12+12 layers, SwiGLU 4096,
    W=128, G=L, V=32000, B=512, bf16): encode t0+n positions, replay 1..t0 (timed as a whole),
    then n more steps timed with HIP events; both against the decoder's algorithmic bytes.
    The workload's full T=2048 does not fit a bench run of minutes, so the late steps are
    taken at t0 = 1024."""
    import time

    import torch

    import cross_token_recurrent_amd as rlt
    from workloads import CONFIGS, make_tokens, make_weights

    wl = CONFIGS[name]
    cfg, B = wl.model, wl.batch
    w = make_weights(cfg, wl.weight_seed)
    model = rlt.Model(cfg, w, device=torch.device("cuda:0"))
    del w
    state = rlt.State(model, B, t0 + n)
    tok = torch.from_numpy(make_tokens(cfg.vocab, B, t0 + n, wl.token_dist, wl.token_seed)).cuda()
    stream = torch.cuda.current_stream()
    rlt.rlt_encoder_forward(model, state, tok)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    rlt.rlt_decoder_replay(model, state, t0)
    ev[1].record(stream)
    rlt.rlt_decoder_replay(model, state, n)
    ev[2].record(stream)
    torch.cuda.synchronize()
    ms_a, ms_b = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    bytes_a = algorithmic_decoder_bytes(cfg, B, t0)
    bytes_b = algorithmic_decoder_bytes(cfg, B, t0 + n) - bytes_a
    gbs_a, gbs_b = bytes_a / (ms_a * 1e-3) / 1e9, bytes_b / (ms_b * 1e-3) / 1e9
    path = {1: "persistent-per-sequence", 2: "batched-phases"}[model.decoder_path(t0 + n)]
    del state, model
    torch.cuda.empty_cache()
    return {"workload": f"{name}: RLT d={cfg.d_model} H={cfg.n_heads} L_E=L_D={cfg.n_layers} F={cfg.ffn_dim} "
                        f"{cfg.ffn_kind} W={cfg.window} G={cfg.mem_groups} V={cfg.vocab}, B={B}, Zipf tokens",
            "decoder_path": path,
            "steps_1_to_t0": {"t0": t0, "ms": ms_a, "tokens_per_s": B * t0 / (ms_a * 1e-3),
                              "achieved_GBps": gbs_a, "frac_of_hbm": gbs_a / HBM_PEAK_GBS},
            "late_steps": {"t": [t0 + 1, t0 + n], "ms_per_step": ms_b / n, "tokens_per_s": B * n / (ms_b * 1e-3),
                           "roofline": {"bound": "hbm", "achieved": gbs_b, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": gbs_b / HBM_PEAK_GBS, "traffic": None,
                                        "kernel": "batched decoder step (cross_part_k dominant)",
                                        "algorithmic_bytes": bytes_b}}}


def full_replay_leg(name: str = "long", chunk: int = 2048):
    """A large workload replayed over its full T: the encoder over all T positions, then the
    decoder over t = 1..T in segments of `chunk` steps, each timed with HIP events and set
    against its algorithmic bytes (cross-attention to M_{<=t} grows with t and dominates the
    late segments).  Used for the long-context workload (d=1024, 48+48 layers, SwiGLU 2816,
    W=512, G=1, B=16, T=32768), the 48+48-layer reference model (d=2048, SwiGLU 5632,
    W=256, G=1, B=64, T=4096) and the 300M-class workload (d=1024, 12+12 layers, SwiGLU
    4096, W=128, G=12, B=512, T=2048).  A line per segment goes to stderr as the run proceeds."""
    import time

    import torch

    import cross_token_recurrent_amd as rlt
    from workloads import CONFIGS, make_tokens, make_weights

    wl = CONFIGS[name]
    cfg, B, T = wl.model, wl.batch, wl.seq_len
    t_start = time.time()
    w = make_weights(cfg, wl.weight_seed)
    model = rlt.Model(cfg, w, device=torch.device("cuda:0"))
    del w
    state = rlt.State(model, B, T)
    tok = torch.from_numpy(make_tokens(cfg.vocab, B, T, wl.token_dist, wl.token_seed)).cuda()
    print(f"{name}: model and state ready in {time.time() - t_start:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    rlt.rlt_encoder_forward(model, state, tok)
    ev[1].record(stream)
    torch.cuda.synchronize()
    enc_ms = ev[0].elapsed_time(ev[1])
    print(f"{name}: encoder over {B} x {T} tokens in {enc_ms:.0f} ms", file=sys.stderr, flush=True)
    segments, done, prev_bytes = [], 0, 0.0
    while done < T:
        n = min(chunk, T - done)
        ev[0].record(stream)
        rlt.rlt_decoder_replay(model, state, n)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1])
        cum = algorithmic_decoder_bytes(cfg, B, done + n)
        gbs = (cum - prev_bytes) / (ms * 1e-3) / 1e9
        segments.append({"t": [done + 1, done + n], "ms_per_step": ms / n, "tokens_per_s": B * n / (ms * 1e-3),
                         "achieved_GBps": gbs, "frac_of_hbm": gbs / HBM_PEAK_GBS})
        print(f"{name}: steps {done + 1}..{done + n}: {ms / n:.2f} ms/step, {gbs:.0f} GB/s "
              f"({100 * gbs / HBM_PEAK_GBS:.1f} % of HBM)", file=sys.stderr, flush=True)
        done += n
        prev_bytes = cum
    assert state.device_error() == 0
    dec_ms = sum(s["ms_per_step"] * (s["t"][1] - s["t"][0] + 1) for s in segments)
    path = {1: "persistent-per-sequence", 2: "batched-phases"}[model.decoder_path(T)]
    del state, model
    torch.cuda.empty_cache()
    gbs_all = prev_bytes / (dec_ms * 1e-3) / 1e9
    late = segments[-1]
    return {"workload": f"{name}: RLT d={cfg.d_model} H={cfg.n_heads} L_E=L_D={cfg.n_layers} F={cfg.ffn_dim} "
                        f"{cfg.ffn_kind} W={cfg.window} G={cfg.mem_groups} V={cfg.vocab}, B={B}, T={T}, Zipf tokens",
            "decoder_path": path, "encoder_ms": enc_ms,
            "replay": {"ms": dec_ms, "tokens_per_s": B * T / (dec_ms * 1e-3), "achieved_GBps": gbs_all,
                       "frac_of_hbm": gbs_all / HBM_PEAK_GBS, "algorithmic_bytes": prev_bytes},
            "late_steps": {"t": late["t"], "ms_per_step": late["ms_per_step"], "tokens_per_s": late["tokens_per_s"],
                           "roofline": {"bound": "hbm", "achieved": late["achieved_GBps"], "peak": HBM_PEAK_GBS,
                                        "unit": "GB/s", "frac": late["frac_of_hbm"], "traffic": None,
                                        "kernel": "batched decoder step (cross_part_k dominant)"}},
            "segments": segments}


def snapshot_leg(model, state, steps: int):
    """Prefix snapshot of the benchmarked state (the whole replayed prefix, all B sequences)
    to pinned host memory and back: bytes per call / time, against the host link."""
    import torch

    import cross_token_recurrent_amd as rlt

    stream = torch.cuda.current_stream()
    nbytes = rlt.rlt_state_snapshot_bytes(state)
    buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    rlt.rlt_state_save(model, state, buf, stream=stream)
    rlt.rlt_state_restore(model, state, buf, stream=stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(steps):
        rlt.rlt_state_save(model, state, buf, stream=stream)
    ev[1].record(stream)
    for _ in range(steps):
        rlt.rlt_state_restore(model, state, buf, stream=stream)
    ev[2].record(stream)
    torch.cuda.synchronize()
    save_ms = ev[0].elapsed_time(ev[1]) / steps
    restore_ms = ev[1].elapsed_time(ev[2]) / steps
    gbs = nbytes / (save_ms * 1e-3) / 1e9
    return {"workload": "prefix snapshot of the benchmarked state (all sequences at t = T) to pinned host memory",
            "bytes": nbytes, "save_ms": save_ms, "restore_ms": restore_ms,
            "roofline": {"bound": "pcie", "achieved": gbs, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / PCIE_PEAK_GBS, "traffic": None, "kernel": "hipMemcpy2DAsync (save)",
                         "algorithmic_bytes_per_call": nbytes}}


def small_leg(steps: int, warmup: int, bw, with_cpu: bool = True):
    """The small workload (d=64, 4+4 layers, W=32, G=L, B=64, T=1024, bf16) on the persistent
    decoder: one step = reset to H_0 + encoder over all T tokens + decoder replay + logits for
    every position; the decoder launch is timed with HIP events."""
    import numpy as np
    import torch

    import cross_token_recurrent_amd as rlt
    from workloads import CONFIGS, make_tokens, make_weights

    wl = CONFIGS["small"]
    cfg, B, T = wl.model, wl.batch, wl.seq_len
    dev = torch.device("cuda:0")
    weights = make_weights(cfg, wl.weight_seed)
    tokens = make_tokens(cfg.vocab, B, T, wl.token_dist, wl.token_seed)
    model = rlt.Model(cfg, weights, device=dev)
    state = rlt.State(model, B, T, keep_encoder_cache=False)
    tok = torch.from_numpy(tokens).to(dev)
    S = torch.empty(B, T, cfg.d_model, dtype=torch.float32, device=dev)
    Z = torch.empty(B, T, cfg.vocab, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        state.reset()
        rlt.rlt_encoder_forward(model, state, tok)
        if ev:
            ev[1].record(stream)
        rlt.rlt_decoder_replay(model, state, T, S)
        if ev:
            ev[2].record(stream)
        rlt.rlt_logits(model, S, Z)
        if ev:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    head_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))
    path = model.decoder_path(T)
    dec_bytes = algorithmic_decoder_bytes(cfg, B, T)
    out = {
        "workload": f"{wl.name}: RLT d={cfg.d_model} H={cfg.n_heads} L_E=L_D={cfg.n_layers} F={cfg.ffn_dim} "
                    f"{cfg.ffn_kind} W={cfg.window} G={cfg.mem_groups} V={cfg.vocab}, B={B} T={T}, exact replay",
        "decoder_tokens_per_s": B * T / (dec_ms * 1e-3),
        "end_to_end_tokens_per_s": B * T / (wall / steps),
        "ms_per_step": wall * 1e3 / steps,
        "phase_ms": {"encoder": enc_ms, "decoder_replay": dec_ms, "logits": head_ms},
        "decoder_path": {1: "persistent-per-sequence", 2: "batched-phases"}[path],
        "roofline": hbm_roofline(dec_bytes, dec_ms, bw, "dec_small_k" if path == 1 else "batched decoder phases",
                                 traffic=measured_traffic() if path == 1 else None,
                                 algorithmic_bytes_per_launch=dec_bytes),
    }
    out["snapshot"] = snapshot_leg(model, state, 3)
    del state, model, S, Z
    torch.cuda.empty_cache()
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, weights, tokens)
    return out


def algorithmic_bptt_bytes(cfg, B: int, T: int) -> float:
    """HBM bytes the two sequential decoder kernels of the backward must move (fp32), the
    schedule of the tape pass, the recomputing sweep and its saved rows:
      tape, per step t: weights once (P_loop elements), the window rows (min(t, W-1) + 1) and the
        memory rows 1..t of every layer (keys and values), the tape written (layer inputs,
        window entry, s_t, s_{t-1}) and e_t read;
      sweep, per step: weights twice (W for the recompute, W^T for the adjoints), the window and
        memory rows twice (recompute; value rows for the output adjoint and key rows for the query
        adjoint), the tape read back, the saved rows of every product written
        (14 d + FFN_in + F per layer: product inputs and output adjoints), the merge adjoints and
        the logit adjoint of s_t.
    The token-parallel parts (encoder, logits, weight gradients) are not counted, so the rate
    derived from a whole call is conservative."""
    p = 4
    d, L, F, W = cfg.d_model, cfg.n_layers, cfg.ffn_dim, cfg.window
    f_in = 2 * F if cfg.ffn_kind == "swiglu" else F
    p_loop = L * (6 * d * d + (3 if cfg.ffn_kind == "swiglu" else 2) * F * d) + 3 * d * d
    sum_mem = T * (T + 1) / 2.0
    sum_win = sum(min(t, W - 1) + 1 for t in range(T))
    rows = B * L * 2 * d * p * (sum_win + sum_mem)
    tape = T * p_loop * p + rows + B * T * ((L + 1) * d + L * 2 * d + 3 * d) * p
    sweep = (2 * T * p_loop * p + 2 * rows + B * T * ((L + 1) * d + L * 2 * d) * p
             + B * T * L * (14 * d + f_in + F) * p + B * T * 4 * d * p)
    return float(tape + sweep)


def bptt_leg(steps: int, warmup: int, with_cpu: bool = True):
    """Full-BPTT backward of the small workload (d=64, 4+4 layers, W=32, G=L, V=512, B=64,
    T=1024): one call = encoder and decoder forward with the tape, loss, reverse sweep and every
    parameter gradient; timed with HIP events around the call."""
    import numpy as np
    import torch

    import cross_token_recurrent_amd as rlt
    from workloads import CONFIGS, make_tokens, make_weights

    wl = CONFIGS["small"]
    cfg, B, T = wl.model, wl.batch, wl.seq_len
    dev = torch.device("cuda:0")
    weights = make_weights(cfg, wl.weight_seed)
    tokens = make_tokens(cfg.vocab, B, T, wl.token_dist, wl.token_seed)
    c = rlt.make_config(cfg)
    table = rlt.rlt_param_table(c)
    total = sum(n for _, n in table.values())
    flat = torch.empty(total, dtype=torch.float32)
    for name, (off, n) in table.items():
        flat[off:off + n] = torch.from_numpy(np.ascontiguousarray(weights[name], dtype=np.float32).reshape(-1))
    flat = flat.to(dev)
    tok = torch.from_numpy(tokens.astype(np.int32)).to(dev)
    grads = torch.empty(total, dtype=torch.float32, device=dev)
    loss = torch.empty(B, dtype=torch.float32, device=dev)
    ws = torch.empty(rlt.rlt_bptt_workspace_bytes(c, B, T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        rlt.rlt_bptt(c, flat, tok, None, (), grads, loss, ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k in range(steps):
        rlt.rlt_bptt(c, flat, tok, None, (), grads, loss, ws)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
    avg = float(np.mean(ms))
    out = {
        "workload": f"{wl.name}: RLT d={cfg.d_model} H={cfg.n_heads} L_E=L_D={cfg.n_layers} F={cfg.ffn_dim} "
                    f"{cfg.ffn_kind} W={cfg.window} G={cfg.mem_groups} V={cfg.vocab}, B={B} T={T}, full BPTT of "
                    f"the summed next-token loss (fp32 arithmetic on the bf16-valued weights)",
        "ms_per_call": avg,
        "ms_min": float(np.min(ms)),
        "tokens_per_s": B * T / (avg * 1e-3),
        "roofline": hbm_roofline(algorithmic_bptt_bytes(cfg, B, T), avg, None,
                                 "rlt_bptt whole call (dec_sweep_k and dec_tape_k dominant: one workgroup per "
                                 "sequence, a latency-bound chain per step)",
                                 algorithmic_bytes=algorithmic_bptt_bytes(cfg, B, T),
                                 unit_of_work="one backward over B x T tokens"),
        "loss_mean_per_token": float(loss.sum().item()) / (B * (T - 1)),
        "workspace_GB": ws.numel() / 1e9,
    }
    del ws, grads, flat
    torch.cuda.empty_cache()
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline_bptt(wl, weights, tokens)
    return out


def _oracle_bptt_one(args):
    cfg, weights, tok = args
    import oracle
    m = oracle.OracleModel.from_config(cfg, weights)
    return oracle.bptt(m, tok)[0]


def cpu_baseline_bptt(wl, weights, tokens, n_seq: int = 4):
    """The fp64 backward oracle on n_seq whole sequences of the workload, one per worker."""
    import multiprocessing as mp

    cores, _ = host_cores()
    workers = min(cores, 16, n_seq)
    jobs = [(wl.model, weights, tokens[b]) for b in range(n_seq)]
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(workers) as pool:
        pool.map(_oracle_bptt_one, jobs)
    wall = time.perf_counter() - t0
    return {"value": n_seq * wl.seq_len / wall, "unit": "tokens/s", "cores": cores, "workers": workers,
            "kind": "oracle",
            "sample": f"{n_seq} of {wl.batch} sequences x T={wl.seq_len}, full BPTT (loss and every gradient), "
                      f"fp64 numpy, one sequence per worker process ({workers} workers on {cores} cores), "
                      f"{wall:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8, help="segments the headline replay is timed in")
    ap.add_argument("--warmup", type=int, default=2, help="segments of an untimed replay run first")
    ap.add_argument("--config", default="ref48", help="headline workload (a name from workloads.CONFIGS)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="only the headline replay")
    ap.add_argument("--no-scoring", action="store_true", help="skip the RL action-scoring measurement")
    ap.add_argument("--no-300m", action="store_true", help="skip the 300M-class batched decoder measurement")
    ap.add_argument("--only-small", action="store_true",
                    help="run only the small-workload leg (persistent decoder; for profiling)")
    ap.add_argument("--only-scoring", action="store_true",
                    help="run only the RL scoring and sampling legs (for profiling)")
    ap.add_argument("--only-300m", action="store_true",
                    help="run only the 300M-class batched decoder measurement (for profiling)")
    ap.add_argument("--only-ref48", action="store_true",
                    help="run only the same measurement on the 48+48-layer reference model (B=64)")
    ap.add_argument("--only-long", action="store_true",
                    help="run only the full replay of the long-context workload (B=16, T=32768; several minutes)")
    ap.add_argument("--full-300m", action="store_true",
                    help="run only the full replay of the 300M-class workload (B=512, T=2048)")
    ap.add_argument("--full-ref48", action="store_true",
                    help="run only the full replay of the 48+48-layer reference model (B=64, T=4096; minutes)")
    ap.add_argument("--only-bptt", action="store_true",
                    help="run only the full-BPTT backward of the small workload (B=64, T=1024)")
    ap.add_argument("--copy-kernel", action="store_true", help="run only a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.copy_kernel:
        copy_kernel()
        return
    if args.only_small:
        print(json.dumps({"small": small_leg(max(1, args.steps), args.warmup, None, False)}), flush=True)
        return
    if args.only_bptt:
        print(json.dumps({"bptt": bptt_leg(max(1, args.steps), args.warmup, not args.no_cpu_baseline)}), flush=True)
        return
    if args.only_scoring:
        print(json.dumps({"rl_scoring": scoring_leg(max(1, args.steps), args.warmup, not args.no_cpu_baseline),
                          "sampling": sampling_leg(max(1, args.steps), args.warmup, not args.no_cpu_baseline)}),
              flush=True)
        return
    if args.only_300m:
        print(json.dumps({"decoder_300m": decoder_300m_leg()}), flush=True)
        return
    if args.only_ref48:
        print(json.dumps({"decoder_ref48": decoder_300m_leg(1024, 32, "ref48")}), flush=True)
        return
    if args.only_long:
        print(json.dumps({"decoder_long": full_replay_leg("long", 2048)}), flush=True)
        return
    if args.full_ref48:
        print(json.dumps({"decoder_ref48_full": full_replay_leg("ref48", 512)}), flush=True)
        return
    if args.full_300m:
        print(json.dumps({"decoder_300m_full": full_replay_leg("300m", 256)}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the replay shards over sequences with no communication, "
              "so a multi-GPU figure is not measured here.", file=sys.stderr)
        sys.exit(2)

    from workloads import CONFIGS

    wl = CONFIGS[args.config]
    cfg = wl.model
    bw = measured_bandwidth()
    head = headline_replay(wl, args.steps, args.warmup, bw, not args.no_cpu_baseline)
    line = {
        "metric": "RLT replay decoder tokens/sec (B*T/s) at 1 GPU; % of HBM/MFMA roofline",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, uniform/Zipf token ids)",
        "config": {"workload": f"{wl.name}: RLT d={cfg.d_model} H={cfg.n_heads} L_E=L_D={cfg.n_layers} "
                               f"F={cfg.ffn_dim} {cfg.ffn_kind} W={cfg.window} G={cfg.mem_groups} V={cfg.vocab}, "
                               f"B={wl.batch} T={wl.seq_len}, exact replay timed as {args.steps} contiguous "
                               f"segments of the decoder (encoder over all T tokens before the timed region)",
                   "batch": wl.batch, "seq_len": wl.seq_len},
        "roofline": head.pop("roofline"),
        "cpu_baseline": head.pop("cpu_baseline", None),
        "measured_bandwidth": bw,
    }
    for k in ("value", "ms_per_step"):
        head.pop(k)
    line["replay"] = head
    if not args.no_legs:
        line["small"] = small_leg(max(3, min(args.steps, 20)), 2, bw, not args.no_cpu_baseline)
        if not args.no_300m:
            line["decoder_300m"] = decoder_300m_leg()
        if not args.no_scoring:
            line["rl_scoring"] = scoring_leg(max(3, min(args.steps, 10)), 2, not args.no_cpu_baseline)
            line["sampling"] = sampling_leg(max(3, min(args.steps, 10)), 2, not args.no_cpu_baseline)
        line["bptt"] = bptt_leg(3, 1, not args.no_cpu_baseline)
    add_copy_denominator(line, bw)
    print(json.dumps(line), flush=True)


def add_copy_denominator(x, bw) -> None:
    """Give every HBM roofline block of the line the copy bandwidth measured in the same run as its
    second denominator (the legs that build theirs without it included)."""
    if isinstance(x, dict):
        if x.get("bound") == "hbm" and "achieved" in x and "measured_copy_GBps" not in x and bw:
            x["measured_copy_GBps"] = bw["copy_GBps"]
            x["frac_of_measured_copy"] = x["achieved"] / bw["copy_GBps"]
        for v in x.values():
            add_copy_denominator(v, bw)
    elif isinstance(x, list):
        for v in x:
            add_copy_denominator(v, bw)


if __name__ == "__main__":
    main()
