"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by
element on the same seeded inputs, plus the invariants the pages fix, on the GPU.

Pages: [FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer";
[DS] deepsonar "技术拆解 009｜RLT…"; [AL] alphalab "Recurrent Looped Transformer：路徑變深…".
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import check, oracle_replay
from workloads import CONFIGS, ModelConfig, make_tokens, make_weights, perturb_untied
from workloads.synth import bf16_round

torch = pytest.importorskip("torch")
import cross_token_recurrent_amd as rlt  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load_library()
    return torch.device("cuda:0")


def gpu_replay(cfg, weights, tokens, dev, keep=False, t_max=None, path=0):
    model = rlt.Model(cfg, weights, device=dev)
    model.set_decoder_path(path)
    B, T = tokens.shape
    state = rlt.State(model, B, t_max or T, keep)
    S, Z = rlt.replay(model, state, torch.from_numpy(tokens).to(dev))
    torch.cuda.synchronize()
    assert state.device_error() == 0
    return S.cpu().numpy(), Z.cpu().numpy(), model, state


def mcfg(**kw):
    base = dict(vocab=97, d_model=64, n_heads=4, n_layers=2, ffn_dim=128, ffn_kind="gelu", window=4,
                mem_groups=1, dtype="fp32")
    base.update(kw)
    return ModelConfig(**base)


# ---------------------------------------------------------------------------
# The configured workloads
# ---------------------------------------------------------------------------

def test_tiny_replay_all_sequences(dev):
    """Tiny RLT, fp32: all B=4 sequences, every t = 1..64, s_t and logits_t."""
    wl = CONFIGS["tiny"]
    cfg = wl.model
    w = make_weights(cfg, wl.weight_seed)
    tok = make_tokens(cfg.vocab, wl.batch, wl.seq_len, wl.token_dist, wl.token_seed)
    S, Z, model, _ = gpu_replay(cfg, w, tok, dev)
    assert model.decoder_path(wl.seq_len) == 1
    S_ref, Z_ref = oracle_replay(cfg, w, tok)
    check("tiny s_t", S, S_ref, "fp32")
    check("tiny logits", Z, Z_ref, "fp32")


def test_small_replay_full_size(dev):
    """Small RLT, bf16: B=64, T=1024 exactly as the benchmark launches it; sampled
    sequences checked against the oracle at every t."""
    wl = CONFIGS["small"]
    cfg = wl.model
    w = make_weights(cfg, wl.weight_seed)
    tok = make_tokens(cfg.vocab, wl.batch, wl.seq_len, wl.token_dist, wl.token_seed)
    S, Z, model, _ = gpu_replay(cfg, w, tok, dev)
    assert model.decoder_path(wl.seq_len) == 1
    seqs = [0, 21, 42, 63]
    S_ref, Z_ref = oracle_replay(cfg, w, tok, seqs)
    check("small s_t", S[seqs], S_ref, "bf16")
    check("small logits", Z[seqs], Z_ref, "bf16")


# ---------------------------------------------------------------------------
# Decoder and encoder in isolation
# ---------------------------------------------------------------------------

def _oracle_encoder(cfg, w, tok):
    m = oracle.OracleModel.from_config(cfg, w)
    es, mks, mvs = [], [], []
    for b in range(tok.shape[0]):
        st = oracle.init_state(m)
        oracle.encode(m, st, tok[b])
        es.append(np.array(st.e))
        mks.append(np.array(st.mem_k))
        mvs.append(np.array(st.mem_v))
    e = np.stack(es)                       # [B, T, d]
    mk = np.stack(mks, axis=1)             # [G, B, T, d]
    mv = np.stack(mvs, axis=1)
    return m, e, mk, mv


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decoder_with_injected_encoder_outputs(dev, dtype):
    """e and M injected from the oracle: the persistent decoder alone vs the oracle."""
    cfg = mcfg(dtype=dtype, window=5, mem_groups=2, n_layers=2, ffn_kind="swiglu")
    w = perturb_untied(make_weights(cfg, 11), cfg, 12)
    B, T = 3, 45
    tok = make_tokens(cfg.vocab, B, T, "uniform", 13)
    m, e, mk, mv = _oracle_encoder(cfg, w, tok)
    model = rlt.Model(cfg, w, device=dev)
    state = rlt.State(model, B, T)
    f32 = lambda a: torch.from_numpy(a.astype(np.float32)).to(dev)
    rlt.rlt_state_load_encoder_outputs(model, state, f32(e), f32(mk), f32(mv))
    S = torch.empty(B, T, cfg.d_model, dtype=torch.float32, device=dev)
    rlt.rlt_decoder_replay(model, state, T, S)
    torch.cuda.synchronize()
    # oracle decoder on the same encoder outputs, rounded on the host to what the state stores:
    # float32 as uploaded, then bf16 (round to nearest even) in bf16 mode
    def stored(a):
        a32 = a.astype(np.float32)
        return (bf16_round(a32) if dtype == "bf16" else a32).astype(np.float64)
    e_st, mk_st, mv_st = stored(e), stored(mk), stored(mv)
    S_ref = []
    for b in range(B):
        st = oracle.init_state(m)
        st.e = list(e_st[b])
        st.mem_k = [list(mk_st[g, b]) for g in range(cfg.mem_groups)]
        st.mem_v = [list(mv_st[g, b]) for g in range(cfg.mem_groups)]
        S_ref.append(oracle.decode(m, st, T))
    check(f"decoder-only s_t ({dtype})", S.cpu().numpy(), np.stack(S_ref), dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_encoder_outputs(dev, dtype):
    cfg = mcfg(dtype=dtype, mem_groups=2, ffn_kind="swiglu" if dtype == "bf16" else "gelu")
    w = perturb_untied(make_weights(cfg, 21), cfg, 22)
    B, T = 3, 150                         # several 128-row tiles and 64-key tiles, ragged tail
    tok = make_tokens(cfg.vocab, B, T, "uniform", 23)
    _, e, mk, mv = _oracle_encoder(cfg, w, tok)
    model = rlt.Model(cfg, w, device=dev)
    state = rlt.State(model, B, T)
    rlt.rlt_encoder_forward(model, state, torch.from_numpy(tok).to(dev))
    ge, gmk, gmv = (x.cpu().numpy() for x in rlt.rlt_state_read_encoder_outputs(model, state, 0, T))
    if dtype == "fp32":
        for name, g, r in (("e", ge, e), ("mem_k", gmk, mk), ("mem_v", gmv, mv)):
            err = np.abs(g - r).max()
            print(f"  encoder {name}: max-abs {err:.2e}")
            assert err < 2e-5, name
    else:
        for name, g, r in (("e", ge, e), ("mem_k", gmk, mk), ("mem_v", gmv, mv)):
            rr = (np.linalg.norm(g - r, axis=-1) / np.linalg.norm(r, axis=-1)).max()
            print(f"  encoder {name}: max row-rel {rr:.2e}")
            assert rr < 1.5e-2, name


# ---------------------------------------------------------------------------
# Shapes, windows, groups, FFN kinds, ragged and degenerate sizes
# ---------------------------------------------------------------------------

EDGE_CASES = [
    # (config overrides, B, T)
    (dict(window=1), 3, 20),                                           # W = 1: window holds only self
    (dict(window=40, n_layers=3, mem_groups=3, ffn_kind="swiglu"), 2, 24),  # W >= T, G = L
    (dict(), 1, 1),                                                    # T = 1, B = 1
    (dict(d_model=128, n_heads=4, ffn_dim=192, ffn_kind="swiglu", window=5, mem_groups=2, dtype="bf16"), 5, 70),
    (dict(d_model=64, n_heads=1, window=3, dtype="bf16"), 2, 33),      # head_dim 64
    (dict(d_model=128, n_heads=1, window=2, n_layers=1), 2, 17),       # head_dim 128
    (dict(d_model=128, n_heads=8, window=9, dtype="bf16", mem_groups=2), 3, 40),  # head_dim 16, H = 8
    (dict(d_model=64, n_heads=2, window=7, ffn_dim=64, n_layers=3), 2, 130),      # head_dim 32, T > 128
]


@pytest.mark.parametrize("path", [1, 2], ids=["persistent", "batched"])
@pytest.mark.parametrize("over,B,T", EDGE_CASES, ids=[f"case{i}" for i in range(len(EDGE_CASES))])
def test_edge_configs(dev, over, B, T, path):
    cfg = mcfg(**over)
    w = perturb_untied(make_weights(cfg, 31), cfg, 32)
    tok = make_tokens(cfg.vocab, B, T, "uniform", 33)
    S, Z, model, _ = gpu_replay(cfg, w, tok, dev, path=path)
    assert model.decoder_path(T) == path
    S_ref, Z_ref = oracle_replay(cfg, w, tok)
    check(f"{over} s_t", S, S_ref, cfg.dtype)
    check(f"{over} logits", Z, Z_ref, cfg.dtype)



# Past 16 key chunks of 256 rows (t >= 3840) the batched decoder folds the chunk partials of
# the cross-attention with a 256-thread combine; both sides of that switch against the oracle.
LONG_MEMORY = [
    (dict(n_heads=1, ffn_dim=64, window=5, mem_groups=2), 2, 4300),                  # head_dim 64, G = L
    (dict(n_heads=1, ffn_dim=64, window=9, dtype="bf16"), 2, 4100),                  # head_dim 64, bf16
    (dict(n_heads=4, ffn_dim=64, window=9, dtype="bf16"), 2, 4100),                  # head_dim 16, bf16
    (dict(d_model=128, n_heads=1, ffn_dim=64, window=3, dtype="bf16"), 1, 3900),     # head_dim 128, bf16
]


@pytest.mark.parametrize("over,B,T", LONG_MEMORY, ids=["dh64_fp32", "dh64_bf16", "dh16_bf16", "dh128_bf16"])
def test_batched_long_memory_combine(dev, over, B, T):
    cfg = mcfg(**over)
    w = make_weights(cfg, 91)
    tok = make_tokens(cfg.vocab, B, T, "uniform", 92)
    S, Z, model, _ = gpu_replay(cfg, w, tok, dev, path=2)
    S_ref, Z_ref = oracle_replay(cfg, w, tok)
    check(f"{over} s_t", S, S_ref, cfg.dtype)
    check(f"{over} logits", Z, Z_ref, cfg.dtype)

# The persistent decoder instantiates its product loop per FFN kind and FFN output shape
# (lanes per row x chunks per lane, or the generic loop): one case per shape class.
FFN_SHAPES = [
    dict(ffn_dim=384, dtype="bf16"),                                   # d=64: 16 lanes x 3 chunks
    dict(ffn_dim=512, ffn_kind="swiglu"),                              # d=64: 16 lanes x 4 chunks, fp32
    dict(ffn_dim=192, ffn_kind="swiglu", dtype="bf16"),                # d=64: 8 lanes x 3 chunks
    dict(ffn_dim=64, ffn_kind="swiglu", dtype="bf16"),                 # d=64: 8 lanes x 1 chunk
    dict(ffn_dim=320, dtype="bf16"),                                   # d=64: generic loop
    dict(d_model=128, ffn_dim=256, dtype="bf16"),                      # d=128: 8 lanes x 4 chunks
    dict(d_model=128, ffn_dim=384, ffn_kind="swiglu", dtype="bf16"),   # d=128: 8 lanes x 6 chunks
    dict(d_model=128, ffn_dim=512, n_layers=1, mem_groups=1),         # d=128: 8 lanes x 8 chunks, fp32
    dict(d_model=128, ffn_dim=320, ffn_kind="swiglu", dtype="bf16"),   # d=128: generic loop
]


@pytest.mark.parametrize("over", FFN_SHAPES, ids=[f"ffn{i}" for i in range(len(FFN_SHAPES))])
def test_ffn_shape_classes(dev, over):
    kw = dict(window=5, mem_groups=2)
    kw.update(over)
    cfg = mcfg(**kw)
    w = perturb_untied(make_weights(cfg, 51), cfg, 52)
    tok = make_tokens(cfg.vocab, 2, 20, "uniform", 53)
    S, Z, model, _ = gpu_replay(cfg, w, tok, dev, path=1)
    assert model.decoder_path(20) == 1
    S_ref, Z_ref = oracle_replay(cfg, w, tok)
    check(f"{over} s_t", S, S_ref, cfg.dtype)
    check(f"{over} logits", Z, Z_ref, cfg.dtype)


# ---------------------------------------------------------------------------
# Invariants on the GPU
# ---------------------------------------------------------------------------

def test_causality_bitwise(dev):
    """Outputs at t do not depend on tokens after t ([AL] §一), bit for bit."""
    cfg = mcfg(window=6, mem_groups=2, dtype="bf16")
    w = make_weights(cfg, 41)
    tok = make_tokens(cfg.vocab, 3, 80, "uniform", 42)
    S1, Z1, _, _ = gpu_replay(cfg, w, tok, dev)
    tok2 = tok.copy()
    tok2[:, 50:] = (tok2[:, 50:] + 7) % cfg.vocab
    S2, Z2, _, _ = gpu_replay(cfg, w, tok2, dev)
    assert np.array_equal(S1[:, :50], S2[:, :50]) and np.array_equal(Z1[:, :50], Z2[:, :50])
    assert not np.array_equal(S1[:, 50:], S2[:, 50:])


def test_run_to_run_determinism(dev):
    wl = CONFIGS["tiny"]
    cfg = wl.model.with_(dtype="bf16")
    w = make_weights(cfg, 5)
    tok = make_tokens(cfg.vocab, 4, 64, "uniform", 6)
    S1, Z1, model, state = gpu_replay(cfg, w, tok, dev)
    S2, Z2 = rlt.replay(model, state, torch.from_numpy(tok).to(dev))
    assert np.array_equal(S1, S2.cpu().numpy()) and np.array_equal(Z1, Z2.cpu().numpy())


@pytest.mark.parametrize("split", [0, 1, 32, 63, 64])
def test_prompt_split_invariance_and_incremental(dev, split):
    """Prefill of P prompt tokens then incremental steps equals full replay
    (Proposition 3.1, [FI] model-RL co-design; [DS] §2.5)."""
    wl = CONFIGS["tiny"]
    cfg = wl.model
    w = perturb_untied(make_weights(cfg, wl.weight_seed), cfg, 7)
    B, T = wl.batch, wl.seq_len
    tok = make_tokens(cfg.vocab, B, T, wl.token_dist, wl.token_seed)
    S_full, Z_full, model, _ = gpu_replay(cfg, w, tok, dev, keep=True)
    state = rlt.State(model, B, T, keep_encoder_cache=True)
    tt = torch.from_numpy(tok).to(dev)
    S = torch.empty(B, T, cfg.d_model, dtype=torch.float32, device=dev)
    Z = torch.empty(B, T, cfg.vocab, dtype=torch.float32, device=dev)
    if split > 0:
        rlt.rlt_encoder_forward(model, state, tt[:, :split].contiguous())
        Sp = torch.empty(B, split, cfg.d_model, dtype=torch.float32, device=dev)
        rlt.rlt_decoder_replay(model, state, split, Sp)
        S[:, :split] = Sp
        Z[:, :split] = rlt.rlt_logits(model, Sp)
    for t in range(split, T):
        s_t = torch.empty(B, cfg.d_model, dtype=torch.float32, device=dev)
        z_t = torch.empty(B, cfg.vocab, dtype=torch.float32, device=dev)
        rlt.rlt_decoder_step(model, state, tt[:, t].contiguous(), s_t, z_t)
        S[:, t] = s_t
        Z[:, t] = z_t
    torch.cuda.synchronize()
    assert state.position()[:2] == (T, T)
    np.testing.assert_allclose(S.cpu().numpy(), S_full, rtol=0, atol=1e-5)
    np.testing.assert_allclose(Z.cpu().numpy(), Z_full, rtol=0, atol=1e-5)
    S_ref, _ = oracle_replay(cfg, w, tok)
    check(f"split {split} s_t", S.cpu().numpy(), S_ref, "fp32")


def test_group_equivalence_bitwise(dev):
    cfg1 = mcfg(n_layers=3, mem_groups=1, window=4, dtype="bf16")
    cfgL = cfg1.with_(mem_groups=3)
    w1 = make_weights(cfg1, 51)
    wL = dict(w1)
    wL["wkm"] = np.repeat(w1["wkm"][:1], 3, axis=0)
    wL["wvm"] = np.repeat(w1["wvm"][:1], 3, axis=0)
    tok = make_tokens(cfg1.vocab, 2, 40, "uniform", 52)
    S1, Z1, _, _ = gpu_replay(cfg1, w1, tok, dev)
    SL, ZL, _, _ = gpu_replay(cfgL, wL, tok, dev)
    assert np.array_equal(S1, SL) and np.array_equal(Z1, ZL)


def test_window_at_least_T_equivalence(dev):
    cfg = mcfg(window=30, dtype="bf16")
    w = make_weights(cfg, 61)
    tok = make_tokens(cfg.vocab, 2, 30, "uniform", 62)
    S30, _, _, _ = gpu_replay(cfg, w, tok, dev)
    S99, _, _, _ = gpu_replay(cfg.with_(window=99), w, tok, dev)
    assert np.array_equal(S30, S99)


def test_logits_head(dev):
    cfg = mcfg(dtype="bf16", vocab=300)
    w = make_weights(cfg, 71)
    model = rlt.Model(cfg, w, device=dev)
    s = torch.randn(37, cfg.d_model, generator=torch.Generator().manual_seed(0)).to(dev)
    Z = rlt.rlt_logits(model, s).cpu().numpy()
    s_b = s.cpu().to(torch.bfloat16).double().numpy()
    ref = s_b @ w["w_out"].astype(np.float64).T
    assert np.abs(Z - ref).max() < 1e-4


# ---------------------------------------------------------------------------
# State contract errors ([FI] serving paragraph: a weight update invalidates states)
# ---------------------------------------------------------------------------

def test_state_contract_errors(dev):
    cfg = mcfg()
    w = make_weights(cfg, 81)
    model = rlt.Model(cfg, w, device=dev)
    state = rlt.State(model, 2, 8)
    tok = torch.from_numpy(make_tokens(cfg.vocab, 2, 8, "uniform", 82)).to(dev)
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_decoder_replay(model, state, 1)
    assert ei.value.name == "RLT_ERR_ORDER"
    rlt.rlt_encoder_forward(model, state, tok[:, :4].contiguous())
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_encoder_forward(model, state, tok[:, 4:].contiguous())
    assert ei.value.name == "RLT_ERR_NO_ENC_CACHE"
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_decoder_replay(model, state, 5)
    assert ei.value.name == "RLT_ERR_ORDER"
    rlt.rlt_decoder_replay(model, state, 4)
    assert state.position()[:2] == (4, 4)
    # capacity
    big = rlt.State(model, 2, 8, keep_encoder_cache=True)
    rlt.rlt_encoder_forward(model, big, tok)
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_encoder_forward(model, big, tok[:, :1].contiguous())
    assert ei.value.name == "RLT_ERR_CAPACITY"
    # weight update invalidates the state until reset
    w2 = dict(w)
    w2["w_fb"] = w["w_fb"] * 2
    model.update_weights(w2, version=2)
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_decoder_replay(model, state, 1)
    assert ei.value.name == "RLT_ERR_STALE_STATE"
    state.reset()
    assert state.position() == (0, 0, 2)
    # an out-of-range token is flagged on the device and replaced by id 0
    bad = tok.clone()
    bad[1, 3] = cfg.vocab + 5
    rlt.rlt_encoder_forward(model, state, bad)
    assert state.device_error() == 1


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_batched_decoder_matches_persistent_and_oracle(dev, name):
    """The two decoder implementations compute the same function on the same state."""
    wl = CONFIGS[name]
    cfg = wl.model
    B, T = min(wl.batch, 8), min(wl.seq_len, 200)
    w = perturb_untied(make_weights(cfg, wl.weight_seed), cfg, 90)
    tok = make_tokens(cfg.vocab, B, T, wl.token_dist, wl.token_seed)
    S1, Z1, _, _ = gpu_replay(cfg, w, tok, dev, path=1)
    S2, Z2, _, _ = gpu_replay(cfg, w, tok, dev, path=2)
    S_ref, Z_ref = oracle_replay(cfg, w, tok, [0, B - 1])
    check(f"{name} batched s_t", S2[[0, B - 1]], S_ref, cfg.dtype)
    check(f"{name} batched logits", Z2[[0, B - 1]], Z_ref, cfg.dtype)
    rel = np.linalg.norm(S1 - S2, axis=-1) / np.linalg.norm(S1, axis=-1)
    print(f"  persistent vs batched: max row-rel {rel.max():.2e}")
    assert rel.max() < (1e-5 if cfg.dtype == "fp32" else 2e-2)


def test_paths_can_alternate_on_one_state(dev):
    """Prefill with the batched path, continue with the persistent one: same state layout."""
    wl = CONFIGS["tiny"]
    cfg = wl.model
    w = make_weights(cfg, 3)
    B, T = 3, 40
    tok = make_tokens(cfg.vocab, B, T, "uniform", 4)
    S_ref, _, model, _ = gpu_replay(cfg, w, tok, dev, path=1)
    state = rlt.State(model, B, T)
    rlt.rlt_encoder_forward(model, state, torch.from_numpy(tok).to(dev))
    S = torch.empty(B, T, cfg.d_model, dtype=torch.float32, device=dev)
    model.set_decoder_path(2)
    Sa = torch.empty(B, 17, cfg.d_model, dtype=torch.float32, device=dev)
    rlt.rlt_decoder_replay(model, state, 17, Sa)
    model.set_decoder_path(1)
    Sb = torch.empty(B, T - 17, cfg.d_model, dtype=torch.float32, device=dev)
    rlt.rlt_decoder_replay(model, state, T - 17, Sb)
    S = torch.cat([Sa, Sb], 1).cpu().numpy()
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=2e-5)


# (B, FFN kind, FFN width): the weight-streaming products over one, two and four 16-row blocks
# with padding rows (B = 5, 6, 24, 40), a GELU input product wide enough (F = 6144 >= 384
# sixteen-column blocks) for two independent blocks per workgroup, two 64-row groups (B = 80),
# and past 512 rows the tiled products with K split over workgroups (B = 520).
# F = 1856 = 29 * 64: a K run (and, past 512 rows, a split of K) that no power of two divides
PRODUCT_CASES = [(6, "swiglu", 512), (5, "gelu", 512), (24, "swiglu", 512), (40, "gelu", 512), (8, "gelu", 6144),
                 (80, "swiglu", 512), (520, "swiglu", 512), (8, "gelu", 1856), (520, "gelu", 1856)]


@pytest.mark.parametrize("B,ffn,F", PRODUCT_CASES, ids=["ws_rows6", "ws_gelu_rows5", "ws_rows24", "ws_gelu_rows40",
                                                      "ws_gelu_two_blocks", "ws_row_groups80", "tiled_rows520",
                                                      "ws_gelu_f1856", "tiled_gelu_f1856"])
def test_batched_products_are_deterministic(dev, B, ffn, F):
    """The batched decoder's products add partial sums in fixed orders: a weight-streaming
    product (bf16, B <= 512, d = 256) adds its waves' K runs in wave order; past 512 rows the
    tiled products split K over workgroups and add the slices in slice order.  Two replays of
    the same input are bitwise equal, and both match the oracle (every sequence up to 80, the
    first and last of 520)."""
    cfg = mcfg(vocab=128, d_model=256, n_heads=4, n_layers=2, ffn_dim=F, ffn_kind=ffn, window=6,
               mem_groups=2, dtype="bf16")
    w = make_weights(cfg, 91)
    tok = make_tokens(cfg.vocab, B, 40, "uniform", 92)
    runs = [gpu_replay(cfg, w, tok, dev, path=2) for _ in range(2)]
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])
    seqs = list(range(B)) if B <= 80 else [0, B - 1]
    S_ref, Z_ref = oracle_replay(cfg, w, tok, seqs)
    check("batched s_t", runs[0][0][seqs], S_ref, "bf16")
    check("batched logits", runs[0][1][seqs], Z_ref, "bf16")
