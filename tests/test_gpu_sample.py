"""Token sampling on the GPU (rlt_sample_tokens, rlt_decoder_step_sample) against the
oracle's sample_tokens.

The draw is a deterministic function of the logits, the parameters and the caller's
uniforms ([FI] model-RL co-design paragraph: the sampler records the log-probability of the
distribution it drew from).  The kernel decides in fp32 and the oracle in fp64, so the two
agree on every token except where a decision sits on a boundary: u within BORDER of the
edge of a token's share, or the top-p mass within BORDER of the nucleus edge.  A test
accepts a differing token only if the oracle itself draws the GPU's token once u (or top_p)
is moved by BORDER, and the number of such rows must stay small.  The behaviour logp of the
drawn token must agree to LOGP_ABS.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
import cross_token_recurrent_amd as rlt  # noqa: E402

pytestmark = pytest.mark.gpu

BORDER = 1e-5
LOGP_ABS = 2e-5


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load_library()
    return torch.device("cuda:0")


def check_rows(logits, u, tok, logp, T, k, p, max_border_frac=0.02, border_eps=BORDER, logp_abs=LOGP_ABS):
    ref_tok, ref_lp = oracle.sample_tokens(logits.astype(np.float64), u.astype(np.float64), T, k, p)
    border = 0
    for i in range(logits.shape[0]):
        if tok[i] == ref_tok[i]:
            assert abs(logp[i] - ref_lp[i]) <= logp_abs, (i, logp[i], ref_lp[i])
            continue
        ok = False
        for du, dp in ((border_eps, 0.0), (-border_eps, 0.0), (0.0, border_eps), (0.0, -border_eps)):
            uu = min(max(float(u[i]) + du, 0.0), 1.0 - 1e-12)
            pp = min(max(p + dp, 1e-9), 1.0)
            t2, lp2 = oracle.sample_tokens(logits[i:i + 1].astype(np.float64), [uu], T, k, pp)
            if t2[0] == tok[i]:
                assert abs(logp[i] - lp2[0]) <= 1e-3, (i, logp[i], lp2[0])
                ok = True
                break
        assert ok, f"row {i}: GPU drew {tok[i]}, oracle {ref_tok[i]}, not a boundary case"
        border += 1
    assert border <= max(1, int(max_border_frac * logits.shape[0])), f"{border} boundary rows"
    return border


def _run(dev, logits, u, T, k, p):
    lt = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(dev)
    ut = torch.from_numpy(np.ascontiguousarray(u, dtype=np.float32)).to(dev)
    tok, lp = rlt.rlt_sample_tokens(lt, ut, T, k, p)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lp.cpu().numpy()


def _case(dev, N, V, T, k, p, seed, scale=2.0):
    g = np.random.default_rng(seed)
    logits = (g.standard_normal((N, V)) * scale).astype(np.float32)
    u = g.random(N).astype(np.float32)
    tok, lp = _run(dev, logits, u, T, k, p)
    b = check_rows(logits, u, tok, lp, T, k, p)
    print(f"  N={N} V={V} T={T} k={k} p={p}: {b} boundary rows", flush=True)


def test_sample_small_vocab_top_k_top_p(dev):
    """The small head (V=512): temperature 0.8, top-k 50, then top-p 0.9."""
    _case(dev, 256, 512, 0.8, 50, 0.9, 1)


def test_sample_plain_and_ragged_vocab(dev):
    """No truncation over V=97 (one value per thread, most threads padding), and V=1000 with
    top-p only (a ragged run of two values per thread)."""
    _case(dev, 200, 97, 1.3, 0, 1.0, 2)
    _case(dev, 100, 1000, 1.0, 0, 0.7, 3)


def test_sample_large_vocab(dev):
    """V=32000 (1024 threads, 32 values each): full nucleus 0.95; top-k 50 + top-p 0.9 (the
    bound from the per-thread maxima, then one wave over the survivors); top-k 2000 + top-p 0.8
    (k above the thread count: the prefix search) and top-k 1024 + top-p 0.5 (k at the thread
    count, where threads past V hold no element, so the bound is empty)."""
    _case(dev, 24, 32000, 1.0, 0, 0.95, 4)
    _case(dev, 24, 32000, 0.7, 50, 0.9, 5)
    _case(dev, 16, 32000, 1.0, 2000, 0.8, 9)
    _case(dev, 16, 32000, 1.0, 1024, 0.5, 10)


def test_sample_mid_vocab(dev):
    """8192 < V <= 16384 (1024 threads, 16 values each): top-k + top-p, top-p alone, and a
    ragged V that leaves the last thread partly empty."""
    _case(dev, 24, 12000, 0.9, 50, 0.9, 11)
    _case(dev, 24, 16384, 1.0, 0, 0.8, 12)
    _case(dev, 16, 9001, 1.0, 300, 0.95, 13)


def test_sample_top_values_in_few_threads(dev):
    """Logits that grow with the id put the largest values in the last threads' runs: the
    k-th largest per-thread maximum then admits more than one wave's list, and the search
    falls back to deciding the top bits over the whole row.  Falling logits put them in the
    first threads; a row whose top values are all in one thread's run is the extreme case."""
    V = 32000
    g = np.random.default_rng(14)
    rising = np.tile(np.linspace(-4.0, 4.0, V, dtype=np.float32), (8, 1))
    rising += (g.standard_normal((8, V)) * 1e-3).astype(np.float32)
    u = g.random(8).astype(np.float32)
    for logits in (rising, rising[:, ::-1].copy()):
        for k, p in ((50, 0.9), (1000, 0.95), (50, 1.0)):
            tok, lp = _run(dev, logits, u, 1.0, k, p)
            check_rows(logits, u, tok, lp, 1.0, k, p)
    one = (g.standard_normal((8, V)) * 0.5).astype(np.float32)
    one[:, 640:672] += 10.0   # ids 640..671: the run of thread 20
    tok, lp = _run(dev, one, u, 1.0, 40, 0.9)
    check_rows(one, u, tok, lp, 1.0, 40, 0.9)
    assert ((tok >= 640) & (tok < 672)).all()


def test_sample_lean_top_k(dev):
    """Top-k <= 128 with 4096 < V and V a multiple of 4 (the lean kernel, keys loaded straight
    into registers and the candidates ranked by id): V = 6000, 12000 and 32000; ties at the
    k-th place resolved by id; one call mixing rows finished on the bound's list and rows whose
    bound admits too many elements (logits growing with the id: the exact threshold over the
    whole row); and that exact path with more ties at the threshold than places left."""
    _case(dev, 24, 6000, 1.0, 100, 0.9, 15)
    _case(dev, 24, 12000, 0.7, 128, 1.0, 16)
    g = np.random.default_rng(17)
    V = 32000
    logits = (g.standard_normal((6, V)) * 0.5).astype(np.float32)
    logits[:, 100:110] = 5.0   # ten equal maxima; top-k 5 keeps ids 100..104
    u = g.random(6).astype(np.float32)
    tok, lp = _run(dev, logits, u, 1.0, 5, 1.0)
    assert ((tok >= 100) & (tok < 105)).all()
    check_rows(logits, u, tok, lp, 1.0, 5, 1.0)
    mixed = (g.standard_normal((8, V)) * 2.0).astype(np.float32)
    mixed[1::2] = np.linspace(-4.0, 4.0, V, dtype=np.float32)
    u = g.random(8).astype(np.float32)
    tok, lp = _run(dev, mixed, u, 0.9, 50, 0.9)
    check_rows(mixed, u, tok, lp, 0.9, 50, 0.9)
    assert (tok[1::2] >= V - 200).all()
    # the bound admits too many elements and the k-th place falls inside 100 equal logits:
    # top-k 50 keeps ids 31900..31949, top-p 0.9 of those the first 45
    tied = np.tile(np.linspace(-4.0, 4.0, V, dtype=np.float32), (6, 1))
    tied[:, V - 100:] = 10.0
    u = g.random(6).astype(np.float32)
    tok, lp = _run(dev, tied, u, 1.0, 50, 1.0)
    check_rows(tied, u, tok, lp, 1.0, 50, 1.0)
    assert ((tok >= V - 100) & (tok < V - 50)).all()
    tok, lp = _run(dev, tied, u, 1.0, 50, 0.9)
    check_rows(tied, u, tok, lp, 1.0, 50, 0.9)
    assert ((tok >= V - 100) & (tok < V - 55)).all()


def test_sample_lean_no_truncation(dev):
    """No truncation with 4096 < V and V a multiple of 4 (the lean kernel's two-level draw:
    the piece row of 2048 ids where the cumulative mass passes u*S, then a scan inside it):
    V = 6000, 12000 and 32000, top-k = V (no truncation either), and u at both edges."""
    _case(dev, 24, 6000, 0.7, 0, 1.0, 18)
    _case(dev, 24, 12000, 1.3, 0, 1.0, 19)
    _case(dev, 32, 32000, 1.0, 0, 1.0, 20)
    _case(dev, 8, 8192, 1.0, 8192, 1.0, 21)
    g = np.random.default_rng(22)
    logits = g.standard_normal((8, 32000)).astype(np.float32)
    for uu in (0.0, np.float32(1.0 - 2 ** -24)):
        u = np.full(8, uu, np.float32)
        tok, lp = _run(dev, logits, u, 1.0, 0, 1.0)
        check_rows(logits, u, tok, lp, 1.0, 0, 1.0, max_border_frac=1.0)
        if uu == 0.0:
            assert (tok == 0).all()


def test_sample_lean_nucleus(dev):
    """Top-p without top-k for 4096 < V, V a multiple of 4 (the lean kernel's search on the
    probabilities' bit patterns): V = 6000 and 12000; logits that grow with the id; equal logits
    (every id ties at the threshold: the nucleus p = 0.5 over V = 8192 is ids 0..4095 and u
    draws floor(4096 u)); logits within 1e-4 of each other (more than 512 ids share the first
    12 bits, so the block search decides every bit)."""
    _case(dev, 24, 6000, 0.9, 0, 0.9, 23)
    _case(dev, 24, 12000, 1.1, 0, 0.7, 24)
    g = np.random.default_rng(25)
    V = 32000
    rising = np.tile(np.linspace(-4.0, 4.0, V, dtype=np.float32), (6, 1))
    u = g.random(6).astype(np.float32)
    tok, lp = _run(dev, rising, u, 1.0, 0, 0.9)
    check_rows(rising, u, tok, lp, 1.0, 0, 0.9)
    flat = np.full((4, 8192), 0.7, np.float32)
    u = np.array([0.0, 0.25, 0.99, 0.5 + 1e-4], np.float32)
    tok, lp = _run(dev, flat, u, 1.0, 0, 0.5)
    assert list(tok) == [0, 1024, 4055, 2048]
    np.testing.assert_allclose(lp, -np.log(4096.0), atol=1e-6)
    near = (0.7 + 1e-4 * g.standard_normal((8, V))).astype(np.float32)
    u = g.random(8).astype(np.float32)
    tok, lp = _run(dev, near, u, 1.0, 0, 0.6)
    check_rows(near, u, tok, lp, 1.0, 0, 0.6)
    # 20 equal maxima spread over threads and pieces, the rest far below: the nucleus 0.5 ends
    # inside the ties, which keep the first 11 by id (the gathered-ties rank in one wave)
    ties = np.array([5, 700, 2049, 2050, 4000, 4097, 5000, 6000, 6001, 7000, 7001, 7500, 7600, 7700, 7800,
                     7900, 8000, 8100, 8150, 8191])
    tied = np.full((8, 8192), -10.0, np.float32)
    tied[:, ties] = 3.0
    u = ((np.arange(8) + 0.5) / 8).astype(np.float32)
    tok, lp = _run(dev, tied, u, 1.0, 0, 0.5)
    check_rows(tied, u, tok, lp, 1.0, 0, 0.5)
    assert np.isin(tok, ties[:11]).all() and tok[-1] == ties[10]
    # torch-generated rows (the bench's sampling input): in one row the fp32 mass above the
    # nucleus threshold rounds up to the target, so the tie at the threshold is not kept
    tg = torch.Generator(device="cpu").manual_seed(9)
    logits = (torch.randn(512, V, generator=tg) * 2.0).numpy()
    u = torch.rand(512, generator=tg).numpy()
    tok, lp = _run(dev, logits, u, 0.8, 0, 0.95)
    rows = np.arange(430, 450)
    check_rows(logits[rows], u[rows], tok[rows], lp[rows], 0.8, 0, 0.95, max_border_frac=0.1)


def test_sample_peaked_and_greedy(dev):
    """Peaked logits (scale 30): the nucleus holds one or two ids; top_k = 1 is the argmax
    with logp 0."""
    _case(dev, 64, 4096, 1.0, 0, 0.9, 6, scale=30.0)
    g = np.random.default_rng(7)
    logits = g.standard_normal((50, 3000)).astype(np.float32)
    u = g.random(50).astype(np.float32)
    tok, lp = _run(dev, logits, u, 1.0, 1, 1.0)
    assert np.array_equal(tok, logits.argmax(1)) and np.all(lp == 0.0)


def test_sample_ties_resolved_by_id(dev):
    """Equal logits: the nucleus p=0.5 over V=512 is ids 0..255 and u draws floor(256 u);
    top-k 300 over ties keeps ids 0..299; a tie at the k-th place between two equal maxima
    keeps the lower id."""
    V = 512
    logits = np.full((4, V), 0.7, np.float32)
    u = np.array([0.0, 0.25, 0.99, 0.5 + 1e-4], np.float32)
    tok, lp = _run(dev, logits, u, 1.0, 0, 0.5)
    assert list(tok) == [0, 64, 253, 128]
    np.testing.assert_allclose(lp, -np.log(256.0), atol=1e-6)
    tok, _ = _run(dev, logits[:1], np.array([0.999], np.float32), 1.0, 300, 1.0)
    assert tok[0] == 299
    z = np.array([[0.5, 2.0, -1.0, 2.0, 1.9]], np.float32)
    for uu in (0.0, 0.5, 0.999):
        tok, lp = _run(dev, z, np.array([uu], np.float32), 1.0, 1, 1.0)
        assert tok[0] == 1 and lp[0] == 0.0


def test_sample_u_edges(dev):
    """u = 0 draws the lowest kept id; u just below 1 draws the highest kept id."""
    g = np.random.default_rng(8)
    logits = g.standard_normal((8, 700)).astype(np.float32)
    for uu in (0.0, np.float32(1.0 - 2 ** -24)):
        u = np.full(8, uu, np.float32)
        tok, lp = _run(dev, logits, u, 1.0, 20, 1.0)
        check_rows(logits, u, tok, lp, 1.0, 20, 1.0, max_border_frac=1.0)


def test_sample_argument_errors(dev):
    lt = torch.zeros(2, 10, device=dev)
    ut = torch.zeros(2, device=dev)
    for T, k, p in ((0.0, 0, 1.0), (1.0, -1, 1.0), (1.0, 0, 0.0), (1.0, 0, 1.5)):
        with pytest.raises(rlt.RltError) as ei:
            rlt.rlt_sample_tokens(lt, ut, T, k, p)
        assert ei.value.name == "RLT_ERR_INVALID"
    big = torch.zeros(1, 32769, device=dev)
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_sample_tokens(big, ut[:1], 1.0, 0, 1.0)
    assert ei.value.name == "RLT_ERR_UNSUPPORTED"
    # plain host memory is refused by the library before anything is launched
    import ctypes
    lib = rlt.load_library()
    host = torch.zeros(2, 10)
    tok = torch.empty(2, dtype=torch.int32, device=dev)
    lp = torch.empty(2, device=dev)
    from cross_token_recurrent_amd.rlt import rlt_sampling
    params = rlt_sampling(1.0, 0, 1.0)
    rc = lib.rlt_sample_tokens(ctypes.c_void_p(host.data_ptr()), 2, 10, ctypes.byref(params),
                               ctypes.c_void_p(ut.data_ptr()), ctypes.c_void_p(tok.data_ptr()),
                               ctypes.c_void_p(lp.data_ptr()), None)
    assert rlt.RltError(rc, "").name == "RLT_ERR_INVALID" and b"GPU can access" in lib.rlt_last_error()


def test_decoder_step_sample(dev):
    """Generation: after a replayed prompt, rlt_decoder_step_sample equals rlt_decoder_step
    followed by a draw; the draw is checked against the oracle's sample of the oracle's own
    logits for that position (boundary rows allowed as above)."""
    from gpu_helpers import oracle_replay
    from workloads import ModelConfig, make_tokens, make_weights
    cfg = ModelConfig(vocab=256, d_model=64, n_heads=4, n_layers=2, ffn_dim=256, ffn_kind="gelu", window=8,
                      mem_groups=1, dtype="fp32")
    w = make_weights(cfg, 41)
    B, P = 16, 12
    tok = make_tokens(cfg.vocab, B, P + 1, "uniform", 42)
    model = rlt.Model(cfg, w, device=dev)
    state = rlt.State(model, B, P + 4, keep_encoder_cache=True)
    tt = torch.from_numpy(tok).to(dev)
    rlt.rlt_encoder_forward(model, state, tt[:, :P].contiguous())
    rlt.rlt_decoder_replay(model, state, P)
    u = np.random.default_rng(43).random(B).astype(np.float32)
    logits = torch.empty(B, cfg.vocab, device=dev)
    nxt, lp = rlt.rlt_decoder_step_sample(model, state, tt[:, P].contiguous(), torch.from_numpy(u).to(dev),
                                          0.9, 40, 0.9, logits=logits)
    torch.cuda.synchronize()
    assert state.position()[:2] == (P + 1, P + 1)
    _, Z_ref = oracle_replay(cfg, w, tok)
    z_ref = Z_ref[:, P]
    np.testing.assert_allclose(logits.cpu().numpy(), z_ref, rtol=0, atol=1e-4)
    # the GPU draws from its own logits (within 1e-4 of the oracle's): boundaries and logp
    # move by about that much
    check_rows(z_ref, u, nxt.cpu().numpy(), lp.cpu().numpy(), 0.9, 40, 0.9, max_border_frac=0.2,
               border_eps=1e-3, logp_abs=1e-3)


def test_sample_bench_size_sampled_rows(dev):
    """The launch the bench times: 512 rows x V=32000, T=0.8, top-k 50 then top-p 0.95; 64
    seeded rows (with the first and last) are checked against the oracle."""
    g = np.random.default_rng(9)
    logits = (g.standard_normal((512, 32000)) * 2.0).astype(np.float32)
    u = g.random(512).astype(np.float32)
    tok, lp = _run(dev, logits, u, 0.8, 50, 0.95)
    assert ((tok >= 0) & (tok < 32000)).all() and np.isfinite(lp).all() and (lp <= 0).all()
    rows = np.unique(np.concatenate([[0, 511], g.choice(512, 62, replace=False)]))
    check_rows(logits[rows], u[rows], tok[rows], lp[rows], 0.8, 50, 0.95)
