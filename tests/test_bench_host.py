"""Host-side pieces of bench.py (no GPU): the one-GPU contract and the algorithmic byte
count that every roofline fraction is taken against."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def closed_form_bytes(cfg, B, T):
    """The decoder's bytes over t = 1..T summed in closed form: weights once per step, the
    window read + write (min(t-1, W-1) cached entries plus the current one), memory rows
    1..t in every layer, and e_t in / s_t out per sequence."""
    d, L, F, W = cfg.d_model, cfg.n_layers, cfg.ffn_dim, cfg.window
    p = 2 if cfg.dtype == "bf16" else 4
    ffn = (2 if cfg.ffn_kind == "gelu" else 3) * d * F
    p_loop = L * (6 * d * d + ffn) + 3 * d * d
    # sum_{k=0}^{T-1} min(k, W-1)
    cached = T * (T - 1) // 2 if T <= W else (W - 1) * W // 2 + (T - W) * (W - 1)
    ring = L * 2 * d * p * (cached + T)
    mem = L * 2 * d * p * T * (T + 1) // 2
    io = T * d * (p + 8)
    return T * p_loop * p + B * (ring + mem + io)


@pytest.mark.parametrize("name", ["tiny", "small", "300m", "ref48"])
def test_algorithmic_bytes_match_the_closed_form(name):
    wl = CONFIGS[name]
    for T in (1, wl.model.window - 1, wl.model.window, wl.model.window + 1, 97, wl.seq_len):
        got = bench.algorithmic_decoder_bytes(wl.model, wl.batch, T)
        want = closed_form_bytes(wl.model, wl.batch, T)
        assert abs(got - want) <= 1e-9 * want, (name, T, got, want)


def test_small_workload_bytes_are_the_quoted_figure():
    wl = CONFIGS["small"]
    assert round(bench.algorithmic_decoder_bytes(wl.model, wl.batch, wl.seq_len) / 1e9, 2) == 37.05


def test_every_hbm_roofline_block_gets_the_copy_denominator():
    """bench.py gives each HBM roofline block of its line, nested legs included, the copy
    bandwidth measured in the same run as a second denominator, and leaves other bounds and
    blocks that already carry one as they are."""
    import bench
    line = {"roofline": {"bound": "hbm", "achieved": 4000.0, "measured_copy_GBps": 4900.0},
            "leg": {"late_steps": {"roofline": {"bound": "hbm", "achieved": 2500.0}}},
            "scoring": {"roofline": {"bound": "mfma", "achieved": 1000.0}}}
    bench.add_copy_denominator(line, {"copy_GBps": 5000.0})
    assert line["roofline"]["measured_copy_GBps"] == 4900.0 and "frac_of_measured_copy" not in line["roofline"]
    late = line["leg"]["late_steps"]["roofline"]
    assert late["measured_copy_GBps"] == 5000.0 and late["frac_of_measured_copy"] == 0.5
    assert "measured_copy_GBps" not in line["scoring"]["roofline"]
