"""Action scoring on the GPU (rlt_score_actions) against the oracle's score_actions.

Scoring follows the RL contract of the pages ([FI] model-RL co-design paragraph): every
action is scored under the current weights, logp = log softmax(W_out s / temperature)[a],
and the behaviour log-probability recorded at sampling time is the denominator of the
importance ratio.

Tolerances.  The kernel rounds s to the storage type of W_out (the operand precision of
the token-parallel products) and accumulates in fp32.  Against the oracle fed the same
rounded operands the only difference is fp32 accumulation order, so logp must agree to
SCORE_ABS = 1e-4 absolute in both modes and the ratio to the matching relative bound.
In bf16 mode the result against the unrounded fp64 oracle is checked with the mode's
relative bound, |gpu - ref| <= 3e-2 * max(|ref|, 1).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import ModelConfig, make_weights

torch = pytest.importorskip("torch")
import cross_token_recurrent_amd as rlt  # noqa: E402

pytestmark = pytest.mark.gpu

SCORE_ABS = 1e-4
BF16_REL = 3e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load_library()
    return torch.device("cuda:0")


def _cfg(vocab, d, dtype):
    return ModelConfig(vocab=vocab, d_model=d, n_heads=max(1, d // 64), n_layers=1, ffn_dim=64,
                       ffn_kind="gelu", window=4, mem_groups=1, dtype=dtype)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _case(dev, vocab, d, dtype, n, seed, temperature=1.0, scale=1.0, with_behaviour=True, actions=None):
    cfg = _cfg(vocab, d, dtype)
    w = make_weights(cfg, seed)
    model = rlt.Model(cfg, w, device=dev)
    g = np.random.default_rng(seed + 1)
    S = (g.standard_normal((n, d)) * scale).astype(np.float32)
    if actions is None:
        actions = g.integers(0, vocab, size=n)
    actions = np.asarray(actions, dtype=np.int32)
    w_out = w["w_out"].astype(np.float64)
    S_op = _round_bf16(S) if dtype == "bf16" else S.astype(np.float64)
    lp_ref, _ = oracle.score_actions(w_out, S_op, actions, None, temperature)
    behav = (lp_ref + 0.1 * g.standard_normal(n)).astype(np.float32) if with_behaviour else None
    _, ratio_ref = oracle.score_actions(w_out, S_op, actions, behav, temperature) if with_behaviour else (None, None)
    lp, ratio = rlt.rlt_score_actions(model, torch.from_numpy(S).to(dev), torch.from_numpy(actions).to(dev),
                                      temperature, torch.from_numpy(behav).to(dev) if with_behaviour else None)
    torch.cuda.synchronize()
    lp = lp.cpu().numpy()
    assert np.isfinite(lp).all()
    err = float(np.abs(lp - lp_ref).max())
    assert err <= SCORE_ABS, f"logp max abs error {err:.3e}"
    if with_behaviour:
        ratio = ratio.cpu().numpy()
        rerr = float((np.abs(ratio - ratio_ref) / ratio_ref).max())
        assert rerr <= 2 * SCORE_ABS, f"ratio max relative error {rerr:.3e}"
    else:
        assert ratio is None
    if dtype == "bf16":
        lp_full, _ = oracle.score_actions(w_out, S.astype(np.float64), actions, None, temperature)
        rel = float((np.abs(lp - lp_full) / np.maximum(np.abs(lp_full), 1.0)).max())
        assert rel <= BF16_REL, f"logp vs unrounded oracle: {rel:.3e}"
    print(f"  V={vocab} d={d} {dtype} N={n} T={temperature}: logp max-abs {err:.3e}", flush=True)
    return lp, lp_ref


def test_score_tiny_fp32(dev):
    """Tiny fp32 head (vocab 256, d=64): ragged rows over three row tiles."""
    _case(dev, 256, 64, "fp32", 300, 11)


def test_score_small_bf16(dev):
    """Small bf16 head (vocab 512, d=64), temperature 0.7."""
    _case(dev, 512, 64, "bf16", 1000, 12, temperature=0.7)


def test_score_ragged_vocab(dev):
    """A vocabulary smaller than one column tile and not a multiple of 16 (V=97), and one of
    2.5 tiles (V=300), in both modes; no behaviour log-probs."""
    for dtype in ("fp32", "bf16"):
        _case(dev, 97, 64, dtype, 130, 13, with_behaviour=False)
        _case(dev, 300, 128, dtype, 129, 14, temperature=1.3)


def test_score_peaked_logits(dev):
    """Large logits (s scaled by 60, temperature 0.5): the running log-sum-exp must stay
    finite and exact when one column dominates each row."""
    for dtype in ("fp32", "bf16"):
        _case(dev, 512, 128, dtype, 200, 15, temperature=0.5, scale=60.0)


def test_score_first_and_last_action(dev):
    """Actions 0 and V-1 on every row pair (the first and last column of the head)."""
    acts = np.array([0, 96] * 40, dtype=np.int32)
    _case(dev, 97, 64, "fp32", 80, 16, actions=acts)
    acts = np.array([0, 511] * 70, dtype=np.int32)
    _case(dev, 512, 64, "bf16", 140, 17, actions=acts)


def test_score_resident_rows_paths(dev):
    """bf16 heads with d a multiple of 256 take the resident-rows kernel (64 rows per
    workgroup up to d=1024, 32 rows up to d=2048): ragged row tails (129 = 2*64 + 1,
    45 rows over two 32-row blocks), vocabularies below one 256-column step (97) and with a
    partial last step (300, 1000), large peaked logits."""
    _case(dev, 300, 256, "bf16", 129, 31, temperature=0.8)
    _case(dev, 97, 512, "bf16", 70, 32)
    _case(dev, 1000, 2048, "bf16", 45, 33, temperature=1.1)
    _case(dev, 512, 256, "bf16", 200, 34, temperature=0.5, scale=60.0)
    acts = np.array([0, 299] * 33, dtype=np.int32)
    _case(dev, 300, 768, "bf16", 66, 35, actions=acts)


def test_score_large_head_bf16(dev):
    """The 300M-class head (vocab 32000, d=1024, bf16) on 300 ragged rows."""
    _case(dev, 32000, 1024, "bf16", 300, 18, temperature=1.0)


def test_score_invalid_action_is_nan(dev):
    """Actions outside [0, V) give NaN (and a NaN ratio) on both kernel paths; 100 lies in the
    padding columns of the last 256-column step of the resident-rows path."""
    for d, dtype in ((64, "fp32"), (256, "bf16")):
        cfg = _cfg(97, d, dtype)
        model = rlt.Model(cfg, make_weights(cfg, 19), device=dev)
        S = torch.randn(5, d, generator=torch.Generator().manual_seed(1)).to(dev)
        acts = torch.tensor([-1, 97, 5, 1000, 100], dtype=torch.int32, device=dev)
        lp, ratio = rlt.rlt_score_actions(model, S, acts, 1.0, torch.zeros(5, device=dev))
        lp, ratio = lp.cpu().numpy(), ratio.cpu().numpy()
        assert np.isnan(lp[[0, 1, 3, 4]]).all() and np.isfinite(lp[2]), (d, lp)
        assert np.isnan(ratio[[0, 1, 3, 4]]).all() and np.isfinite(ratio[2])


def test_score_argument_errors(dev):
    cfg = _cfg(97, 64, "fp32")
    model = rlt.Model(cfg, make_weights(cfg, 20), device=dev)
    S = torch.zeros(2, 64, device=dev)
    acts = torch.zeros(2, dtype=torch.int32, device=dev)
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_score_actions(model, S, acts, temperature=0.0)
    assert ei.value.name == "RLT_ERR_INVALID"
    for bad in ((S.cpu(), acts), (S, acts.cpu()), (S.double(), acts), (S, acts[:1])):
        with pytest.raises(ValueError):
            rlt.rlt_score_actions(model, *bad)
    lib = rlt.load_library()
    import ctypes
    out = torch.empty(2, device=dev)
    rc = lib.rlt_score_actions(model.handle, ctypes.c_void_p(S.data_ptr()), ctypes.c_void_p(acts.data_ptr()), 2,
                               1.0, None, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(out.data_ptr()), None)
    assert rc != 0
    # the library itself refuses plain host memory before launching anything
    host = torch.zeros(2, 64)
    rc = lib.rlt_score_actions(model.handle, ctypes.c_void_p(host.data_ptr()), ctypes.c_void_p(acts.data_ptr()), 2,
                               1.0, None, ctypes.c_void_p(out.data_ptr()), None, None)
    assert rlt.RltError(rc, "").name == "RLT_ERR_INVALID" and b"GPU can access" in lib.rlt_last_error()


def test_score_after_replay(dev):
    """Replay, then score the response half of every sequence: the GPU chain
    (rlt_decoder_replay -> rlt_score_actions) against the oracle chain (replay -> score)."""
    from gpu_helpers import oracle_replay
    from workloads import make_tokens
    cfg = ModelConfig(vocab=256, d_model=64, n_heads=4, n_layers=2, ffn_dim=256, ffn_kind="gelu", window=8,
                      mem_groups=1, dtype="fp32")
    w = make_weights(cfg, 21)
    B, T, P = 3, 48, 24
    tok = make_tokens(cfg.vocab, B, T, "uniform", 22)
    model = rlt.Model(cfg, w, device=dev)
    state = rlt.State(model, B, T)
    tt = torch.from_numpy(tok).to(dev)
    rlt.rlt_encoder_forward(model, state, tt)
    S = torch.empty(B, T, cfg.d_model, dtype=torch.float32, device=dev)
    rlt.rlt_decoder_replay(model, state, T, S)
    # the action at position t is the token at t + 1 (next-token policy); score positions P-1 .. T-2
    acts = tt[:, P:].contiguous()
    Sr = S[:, P - 1:T - 1].contiguous()
    lp, _ = rlt.rlt_score_actions(model, Sr, acts)
    torch.cuda.synchronize()
    S_ref, _ = oracle_replay(cfg, w, tok)
    ref = np.stack([oracle.score_actions(w["w_out"], S_ref[b, P - 1:T - 1], tok[b, P:])[0] for b in range(B)])
    err = float(np.abs(lp.cpu().numpy() - ref).max())
    assert err <= SCORE_ABS, f"replay+score logp max abs error {err:.3e}"


def test_score_bench_size_sampled_rows(dev):
    """The launch the bench times: head V=32000, d=1024, bf16, N=65536 rows, with ratios; 48
    rows spread over the whole range (first, last, and seeded picks in between) are checked
    against the oracle on the same rounded operands, and every row must be finite."""
    cfg = _cfg(32000, 1024, "bf16")
    w = make_weights(cfg, 7)
    model = rlt.Model(cfg, w, device=dev)
    n = 64 * 1024
    g = np.random.default_rng(8)
    S = g.standard_normal((n, cfg.d_model)).astype(np.float32)
    acts = g.integers(0, cfg.vocab, size=n).astype(np.int32)
    behav = np.full(n, -10.0, np.float32)
    lp, ratio = rlt.rlt_score_actions(model, torch.from_numpy(S).to(dev), torch.from_numpy(acts).to(dev), 1.0,
                                      torch.from_numpy(behav).to(dev))
    torch.cuda.synchronize()
    lp, ratio = lp.cpu().numpy(), ratio.cpu().numpy()
    assert np.isfinite(lp).all() and np.isfinite(ratio).all()
    rows = np.unique(np.concatenate([[0, 63, 64, n - 1], g.choice(n, 44, replace=False)]))
    ref, rref = oracle.score_actions(w["w_out"].astype(np.float64), _round_bf16(S[rows]), acts[rows], behav[rows])
    err = float(np.abs(lp[rows] - ref).max())
    assert err <= SCORE_ABS, f"logp max abs error {err:.3e}"
    assert float((np.abs(ratio[rows] - rref) / rref).max()) <= 2 * SCORE_ABS
