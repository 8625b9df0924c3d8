"""Pins for the fp64 oracle: checks against library routines, closed forms and
invariants that the pages fix, chosen so that a plausible slip in the oracle
(a dropped residual, a wrong gain, a transposed projection, an off-by-one
window or memory range, a reset at the prompt/response split) fails one of them.

Pages: [FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer";
[DS] deepsonar "技术拆解 009｜RLT：给 Transformer 接一条时间回路…";
[AL] alphalab "Recurrent Looped Transformer：路徑變深，就真的更會推理嗎？（2026）".
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle as O
from workloads import CONFIGS, ModelConfig, make_tokens, make_weights, perturb_untied


@pytest.fixture(autouse=True)
def _fp64_default_dtype():
    """Library references in this module build fp64 tensors; the default dtype is set per
    test and restored, so collecting this module changes nothing for other modules."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def tiny_cfg(**kw):
    base = dict(vocab=37, d_model=16, n_heads=2, n_layers=2, ffn_dim=24, ffn_kind="gelu",
                window=3, mem_groups=1, dtype="fp32")
    base.update(kw)
    return ModelConfig(**base)


def model_for(cfg, seed=7, perturb=True, gate_bias_std=1.0, scale=None):
    w = make_weights(cfg, seed)
    if perturb:
        w = perturb_untied(w, cfg, seed + 1000, gate_bias_std)
    if scale is not None:  # larger weights make every term matter numerically
        w = {k: (v * scale if k not in ("b_g",) and not k.startswith("g_") else v) for k, v in w.items()}
    return O.OracleModel.from_config(cfg, w)


def toks(cfg, T, seed=3, B=1):
    return make_tokens(cfg.vocab, B, T, "uniform", seed)


# ---------------------------------------------------------------------------
# Independent torch fp64 formulations (library sdpa / rms_norm / gelu / silu)
# ---------------------------------------------------------------------------

def t64(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def torch_ffn(m, l, h):
    w = m.w
    if m.ffn_kind == "gelu":
        return F.linear(F.gelu(F.linear(h, t64(w["ffn_w1"][l]))), t64(w["ffn_w2"][l]))
    return F.linear(F.silu(F.linear(h, t64(w["ffn_gate"][l]))) * F.linear(h, t64(w["ffn_up"][l])),
                    t64(w["ffn_down"][l]))


def heads(x, H):  # [T, d] -> [H, T, dh]
    T, d = x.shape
    return x.reshape(T, H, d // H).transpose(0, 1)


def unheads(x):  # [H, T, dh] -> [T, d]
    H, T, dh = x.shape
    return x.transpose(0, 1).reshape(T, H * dh)


def torch_encoder(m, tokens):
    """Causal pre-norm encoder with library sdpa(is_causal=True)."""
    w, H, d, eps = m.w, m.n_heads, m.d_model, m.norm_eps
    x = t64(w["embed"])[torch.as_tensor(np.asarray(tokens, dtype=np.int64))]
    for l in range(m.n_layers):
        h = F.rms_norm(x, (d,), weight=t64(w["g_enc_attn"][l]), eps=eps)
        q, k, v = (F.linear(h, t64(w[n][l])) for n in ("wq", "wk", "wv"))
        a = F.scaled_dot_product_attention(heads(q, H), heads(k, H), heads(v, H), is_causal=True)
        x = x + F.linear(unheads(a), t64(w["wo"][l]))
        x = x + torch_ffn(m, l, F.rms_norm(x, (d,), weight=t64(w["g_enc_ffn"][l]), eps=eps))
    e = F.rms_norm(x, (d,), weight=t64(w["g_enc_final"]), eps=eps)
    mk = [F.linear(e, t64(w["wkm"][g])) for g in range(m.mem_groups)]
    mv = [F.linear(e, t64(w["wvm"][g])) for g in range(m.mem_groups)]
    return e, mk, mv


def torch_merge(m, e, s_prev):
    w = m.w
    gate = torch.sigmoid(F.linear(e, t64(w["w_ge"])) + F.linear(s_prev, t64(w["w_gs"])) + t64(w["b_g"]))
    return gate * e + (1 - gate) * F.linear(s_prev, t64(w["w_fb"]))


def torch_decoder_parallel(m, u, mk, mv):
    """Decoder stack evaluated token-parallel from given merged inputs u [T, d].

    Window as a band mask (key j visible to query i iff i-W < j <= i), memory
    as a causal mask, both through library sdpa with an explicit boolean mask.
    Equals the recurrence only when u does not depend on earlier outputs.
    """
    w, H, d, eps, W = m.w, m.n_heads, m.d_model, m.norm_eps, m.window
    T = u.shape[0]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    band = (j <= i) & (j > i - W)
    causal = j <= i
    y = u
    for l in range(m.n_layers):
        h = F.rms_norm(y, (d,), weight=t64(w["g_dec_self"][l]), eps=eps)
        q, k, v = (F.linear(h, t64(w[n][l])) for n in ("wq", "wk", "wv"))
        a = F.scaled_dot_product_attention(heads(q, H), heads(k, H), heads(v, H), attn_mask=band)
        y = y + F.linear(unheads(a), t64(w["wo"][l]))
        h = F.rms_norm(y, (d,), weight=t64(w["g_dec_cross"][l]), eps=eps)
        g = 0 if m.mem_groups == 1 else l
        qx = F.linear(h, t64(w["wqx"][l]))
        a = F.scaled_dot_product_attention(heads(qx, H), heads(mk[g], H), heads(mv[g], H), attn_mask=causal)
        y = y + F.linear(unheads(a), t64(w["wox"][l]))
        y = y + torch_ffn(m, l, F.rms_norm(y, (d,), weight=t64(w["g_dec_ffn"][l]), eps=eps))
    return F.rms_norm(y, (d,), weight=t64(w["g_dec_final"]), eps=eps)


# ---------------------------------------------------------------------------
# Sub-layers vs library routines
# ---------------------------------------------------------------------------

def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 24))
    g = rng.uniform(0.5, 1.5, 24)
    ref = F.rms_norm(t64(x), (24,), weight=t64(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), ref, rtol=0, atol=1e-14)


def test_gelu_silu_sigmoid_match_torch():
    x = np.linspace(-8, 8, 1001)
    np.testing.assert_allclose(O.gelu(x), F.gelu(t64(x)).numpy(), rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.silu(x), F.silu(t64(x)).numpy(), rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.sigmoid(x), torch.sigmoid(t64(x)).numpy(), rtol=0, atol=1e-15)
    # sigmoid saturates to exactly 1 / 0 at the gate-test biases used below
    assert O.sigmoid(np.array([39.0]))[0] == 1.0


def test_attend_matches_sdpa():
    rng = np.random.default_rng(1)
    for n in (1, 2, 7):
        q = rng.standard_normal(12)
        K = rng.standard_normal((n, 12))
        V = rng.standard_normal((n, 12))
        ref = F.scaled_dot_product_attention(heads(t64(q[None]), 3), heads(t64(K), 3), heads(t64(V), 3))
        np.testing.assert_allclose(O.attend(q, K, V, 3), unheads(ref).numpy()[0], rtol=0, atol=1e-13)
    # a single entry: softmax is exactly 1, output is exactly that value row
    q, K, V = rng.standard_normal(8), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.array_equal(O.attend(q, K, V, 2), V[0])


def test_causal_attention_matches_sdpa_with_offset():
    rng = np.random.default_rng(2)
    T, d, H = 300, 16, 4                       # > one 256-row block
    Q, K, V = (rng.standard_normal((T, d)) for _ in range(3))
    ref = unheads(F.scaled_dot_product_attention(heads(t64(Q), H), heads(t64(K), H), heads(t64(V), H),
                                                 is_causal=True)).numpy()
    np.testing.assert_allclose(O.causal_attention(Q, K, V, H, 0), ref, rtol=0, atol=1e-13)
    # queries for positions 100..299 over keys 0..299 == rows 100.. of the full pass
    np.testing.assert_allclose(O.causal_attention(Q[100:], K, V, H, 100), ref[100:], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Encoder vs library causal pass
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,G", [("gelu", 1), ("swiglu", 2)])
def test_encoder_matches_torch_causal_pass(kind, G):
    cfg = tiny_cfg(ffn_kind=kind, mem_groups=G)
    m = model_for(cfg, scale=8.0)
    tok = toks(cfg, 40)[0]
    st = O.init_state(m)
    e = O.encode(m, st, tok)
    e_ref, mk, mv = torch_encoder(m, tok)
    np.testing.assert_allclose(e, e_ref.numpy(), rtol=0, atol=1e-12)
    for g in range(G):
        np.testing.assert_allclose(np.array(st.mem_k[g]), mk[g].numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.array(st.mem_v[g]), mv[g].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Decoder vs token-parallel passes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("W", [1, 2, 3, 8, 64])
@pytest.mark.parametrize("kind,G", [("gelu", 1), ("swiglu", 2)])
def test_decoder_teacher_forced_parallel_pass(W, kind, G):
    """Given the oracle's own s_{t-1}, every s_t follows from a token-parallel pass.

    The merged inputs u_t = merge(e_t, s_{t-1}) are the only recurrent link;
    given all u_t, windows, memory causality, tying, norms and FFN are a masked
    parallel computation ([DS] §2.2, §2.4; [FI] decoder-state paragraph).
    """
    cfg = tiny_cfg(window=W, ffn_kind=kind, mem_groups=G)
    m = model_for(cfg, scale=6.0)
    T = 20
    tok = toks(cfg, T)[0]
    S, Z = O.replay(m, tok)
    e, mk, mv = torch_encoder(m, tok)
    s_prev = torch.cat([t64(m.w["s_star"])[None], t64(S[:-1])], 0)
    u = torch_merge(m, e, s_prev)
    s_par = torch_decoder_parallel(m, u, mk, mv)
    np.testing.assert_allclose(S, s_par.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(Z, S @ m.w["w_out"].T, rtol=0, atol=0)


def test_gate_saturated_decoder_is_token_parallel_and_negative_control():
    """b_g = +40: gate == 1 exactly, u_t = e_t, so the decoder equals a parallel
    pass with no recurrence.  With b_g = 0 that parallel pass must differ: a
    standard parallel SWA decoder pass is not the recurrence ([FI] model-hardware
    co-design principle)."""
    cfg = tiny_cfg(window=4, mem_groups=2)
    m = model_for(cfg, scale=6.0, gate_bias_std=0.0)
    tok = toks(cfg, 16)[0]
    e, mk, mv = torch_encoder(m, tok)
    m.w["b_g"] = np.full(cfg.d_model, 40.0)
    S_sat, _ = O.replay(m, tok)
    np.testing.assert_allclose(S_sat, torch_decoder_parallel(m, e, mk, mv).numpy(), rtol=0, atol=1e-11)
    m.w["b_g"] = np.zeros(cfg.d_model)
    S_rec, _ = O.replay(m, tok)
    diff = np.abs(S_rec - torch_decoder_parallel(m, e, mk, mv).numpy()).max()
    assert diff > 1e-3


def test_first_step_closed_form():
    """T = 1 expanded by hand: one window entry and one memory entry, so every
    softmax is exactly 1 and each attention returns its single value row."""
    for kind, G in (("gelu", 1), ("swiglu", 2)):
        cfg = tiny_cfg(ffn_kind=kind, mem_groups=G, window=5)
        m = model_for(cfg, scale=5.0)
        w, eps = m.w, m.norm_eps
        tok = toks(cfg, 1)[0]
        S, Z = O.replay(m, tok)
        # encoder, one position: attention over itself returns v
        x = w["embed"][tok[0]].copy()
        for l in range(cfg.n_layers):
            h = O.rms_norm(x, w["g_enc_attn"][l], eps)
            x = x + w["wo"][l] @ (w["wv"][l] @ h)
            x = x + m.ffn(l, O.rms_norm(x, w["g_enc_ffn"][l], eps))
        e = O.rms_norm(x, w["g_enc_final"], eps)
        s0 = w["s_star"]
        gate = 1 / (1 + np.exp(-(w["w_ge"] @ e + w["w_gs"] @ s0 + w["b_g"])))
        y = gate * e + (1 - gate) * (w["w_fb"] @ s0)
        for l in range(cfg.n_layers):
            h = O.rms_norm(y, w["g_dec_self"][l], eps)
            y = y + w["wo"][l] @ (w["wv"][l] @ h)
            g = 0 if G == 1 else l
            y = y + w["wox"][l] @ (w["wvm"][g] @ e)
            y = y + m.ffn(l, O.rms_norm(y, w["g_dec_ffn"][l], eps))
        s1 = O.rms_norm(y, w["g_dec_final"], eps)
        np.testing.assert_allclose(S[0], s1, rtol=0, atol=1e-13)
        np.testing.assert_allclose(Z[0], w["w_out"] @ s1, rtol=0, atol=1e-13)


def test_gate_closed_uses_feedback_only():
    """b_g = -40: gate == 0 exactly, so the decoder input is W_fb s_{t-1} and the
    token reaches the decoder only through the memory."""
    cfg = tiny_cfg(window=3)
    m = model_for(cfg, scale=4.0)
    m.w["b_g"] = np.full(cfg.d_model, -40.0)
    tok = toks(cfg, 6)[0]
    S, _ = O.replay(m, tok)
    e, mk, mv = torch_encoder(m, tok)
    s_prev = torch.cat([t64(m.w["s_star"])[None], t64(S[:-1])], 0)
    u = F.linear(s_prev, t64(m.w["w_fb"]))
    np.testing.assert_allclose(S, torch_decoder_parallel(m, u, mk, mv).numpy(), rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# Invariants the pages fix
# ---------------------------------------------------------------------------

def test_causality_bitwise():
    """Outputs at t never depend on tokens after t ([AL] §一: the memory shows no future tokens)."""
    cfg = tiny_cfg(window=4, mem_groups=2)
    m = model_for(cfg)
    tok = toks(cfg, 24)[0]
    S1, Z1 = O.replay(m, tok)
    tok2 = tok.copy()
    tok2[13:] = (tok2[13:] + 5) % cfg.vocab
    S2, Z2 = O.replay(m, tok2)
    assert np.array_equal(S1[:13], S2[:13]) and np.array_equal(Z1[:13], Z2[:13])
    assert not np.allclose(S1[13:], S2[13:])


@pytest.mark.parametrize("split", [0, 1, 7, 19, 20])
def test_prompt_split_invariance(split):
    """Proposition 3.1 ([FI] model-RL co-design principle): where the prompt
    ends does not change anything for a fixed token history - prefill then
    incremental generation from the same state, never a reset."""
    cfg = tiny_cfg(window=4, mem_groups=2, ffn_kind="swiglu")
    m = model_for(cfg)
    T = 20
    tok = toks(cfg, T)[0]
    S_ref, Z_ref = O.replay(m, tok)
    st = O.init_state(m)
    O.encode(m, st, tok[:split])
    S = list(O.decode(m, st, split))
    Z = list(O.logits(m, np.array(S))) if S else []
    for t in range(split, T):
        s, z = O.step(m, st, tok[t])
        S.append(s)
        Z.append(z)
    np.testing.assert_allclose(np.array(S), S_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.array(Z), Z_ref, rtol=0, atol=1e-12)
    assert st.t_dec == T and st.t_enc == T


def test_reset_at_split_would_be_detected():
    """A schedule that resets H to (s*, empty) at the split gives different
    outputs after it, so the split-invariance test is sensitive to resets."""
    cfg = tiny_cfg(window=4)
    m = model_for(cfg)
    tok = toks(cfg, 12)[0]
    S_ref, _ = O.replay(m, tok)
    st = O.init_state(m)
    O.encode(m, st, tok[:6])
    O.decode(m, st, 6)
    st.s = m.w["s_star"].copy()
    st.dec_cache = [[] for _ in range(cfg.n_layers)]
    S_after = [O.step(m, st, tok[t])[0] for t in range(6, 12)]
    assert np.abs(np.array(S_after) - S_ref[6:]).max() > 1e-4


def test_group_equivalence_bitwise():
    """G = L_D with every group's projections equal to group 0 == G = 1."""
    cfg1 = tiny_cfg(mem_groups=1, n_layers=3, window=3)
    cfgL = cfg1.with_(mem_groups=3)
    m1 = model_for(cfg1)
    wL = dict(m1.w)
    wL["wkm"] = np.repeat(m1.w["wkm"][:1], 3, axis=0)
    wL["wvm"] = np.repeat(m1.w["wvm"][:1], 3, axis=0)
    mL = O.OracleModel.from_config(cfgL, wL)
    tok = toks(cfg1, 15)[0]
    S1, Z1 = O.replay(m1, tok)
    SL, ZL = O.replay(mL, tok)
    assert np.array_equal(S1, SL) and np.array_equal(Z1, ZL)


def test_window_at_least_T_is_full_causal():
    cfg = tiny_cfg(window=16)
    m = model_for(cfg)
    tok = toks(cfg, 16)[0]
    S16, _ = O.replay(m, tok)
    m.window = 40
    S40, _ = O.replay(m, tok)
    assert np.array_equal(S16, S40)
    m.window = 15
    S15, _ = O.replay(m, tok)
    assert np.array_equal(S15[:15], S16[:15]) and not np.allclose(S15[15], S16[15])


def test_state_path_length_and_influence_of_s_star():
    """After t tokens the state path from s_0 crosses t*L_D decoder blocks
    ([FI] temporal-depth principle; [DS] §一).  s* influences later states
    through that path; with the gate saturated to the token side the path is cut."""
    cfg = tiny_cfg(window=3, n_layers=3)
    m = model_for(cfg, scale=3.0)
    tok = toks(cfg, 10)[0]
    st = O.init_state(m)
    O.encode(m, st, tok)
    for t in range(1, 11):
        O.decoder_step(m, st)
        assert st.depth == t * cfg.n_layers
    S0, _ = O.replay(m, tok)
    m.w["s_star"] = m.w["s_star"] + 1e-7
    S1, _ = O.replay(m, tok)
    assert (np.abs(S1 - S0).max(axis=1)[:8] > 1e-13).all()
    m.w["b_g"] = np.full(cfg.d_model, 40.0)
    Sa, _ = O.replay(m, tok)
    m.w["s_star"] = m.w["s_star"] - 1e-7
    Sb, _ = O.replay(m, tok)
    assert np.array_equal(Sa, Sb)


def test_incremental_matches_replay_on_tiny_config():
    """Generation consumes each token once; the step chain equals full replay."""
    wl = CONFIGS["tiny"]
    cfg = wl.model
    m = O.OracleModel.from_config(cfg, make_weights(cfg, wl.weight_seed))
    tok = make_tokens(cfg.vocab, 1, 24, "uniform", wl.token_seed)[0]
    S_ref, Z_ref = O.replay(m, tok)
    st = O.init_state(m)
    out = [O.step(m, st, x) for x in tok]
    np.testing.assert_allclose(np.array([o[0] for o in out]), S_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.array([o[1] for o in out]), Z_ref, rtol=0, atol=1e-12)


def test_errors():
    cfg = tiny_cfg()
    m = model_for(cfg)
    st = O.init_state(m)
    with pytest.raises(ValueError):
        O.decoder_step(m, st)
    with pytest.raises(ValueError):
        O.encode(m, st, [cfg.vocab])
    with pytest.raises(ValueError):
        O.OracleModel.from_config(cfg.with_(mem_groups=3, n_layers=2), make_weights(cfg, 1))
    with pytest.raises(ValueError):
        O.OracleModel.from_config(cfg.with_(d_model=15), make_weights(cfg, 1))


# ---------------------------------------------------------------------------
# Property tests over tiny random configurations
# ---------------------------------------------------------------------------

@settings(max_examples=25, deadline=None)
@given(d_heads=st.sampled_from([(8, 1), (8, 2), (16, 2), (16, 4)]),
       L=st.integers(1, 2), W=st.sampled_from([1, 2, 3, 12]),
       grouped=st.booleans(), kind=st.sampled_from(["gelu", "swiglu"]),
       T=st.integers(1, 12), seed=st.integers(0, 10_000))
def test_property_teacher_forced_and_split(d_heads, L, W, grouped, kind, T, seed):
    d, H = d_heads
    cfg = tiny_cfg(d_model=d, n_heads=H, n_layers=L, window=W, ffn_dim=2 * d,
                   mem_groups=L if grouped else 1, ffn_kind=kind, vocab=11)
    m = model_for(cfg, seed=seed, scale=5.0)
    tok = make_tokens(cfg.vocab, 1, T, "uniform", seed + 1)[0]
    S, _ = O.replay(m, tok)
    e, mk, mv = torch_encoder(m, tok)
    s_prev = torch.cat([t64(m.w["s_star"])[None], t64(S[:-1])], 0)
    s_par = torch_decoder_parallel(m, torch_merge(m, e, s_prev), mk, mv)
    np.testing.assert_allclose(S, s_par.numpy(), rtol=0, atol=1e-10)
    split = seed % (T + 1)
    st_ = O.init_state(m)
    O.encode(m, st_, tok[:split])
    S2 = list(O.decode(m, st_, split)) + [O.step(m, st_, x)[0] for x in tok[split:]]
    np.testing.assert_allclose(np.array(S2), S, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Action scoring ([FI] model-RL co-design paragraph): closed forms
# ---------------------------------------------------------------------------

def test_score_actions_zero_head_is_uniform():
    """W_out = 0: every action has probability 1/V at any temperature."""
    V, d = 13, 5
    rng = np.random.default_rng(3)
    S = rng.standard_normal((4, d))
    acts = [0, 12, 5, 7]
    behav = [-1.0, -2.5, math.log(1 / V), 0.0]
    for tau in (1.0, 0.3):
        lp, r = O.score_actions(np.zeros((V, d)), S, acts, behav, temperature=tau)
        np.testing.assert_allclose(lp, -math.log(V), rtol=0, atol=1e-15)
        np.testing.assert_allclose(r, [math.exp(-math.log(V) - b) for b in behav], rtol=1e-14)


def test_score_actions_one_dominant_logit():
    """Only row k of W_out is non-zero and aligned with s: z_k = c, every other logit 0, so
    logp_k = c - log(e^c + V - 1) and logp_other = -log(e^c + V - 1)."""
    V, d, k = 9, 4, 6
    s = np.array([0.5, -1.0, 2.0, 0.25])
    for c in (0.0, 3.0, 60.0, 700.0):
        W = np.zeros((V, d))
        W[k] = s * (c / float(s @ s))
        lp, _ = O.score_actions(W, s[None, :], [k])
        lq, _ = O.score_actions(W, s[None, :], [2])
        # log(e^c + V - 1) = c + log1p((V - 1) e^{-c}), stable for large c
        lse = c + math.log1p((V - 1) * math.exp(-c))
        assert abs(lp[0] - (c - lse)) < 1e-12 * max(1.0, c)
        assert abs(lq[0] - (-lse)) < 1e-12 * max(1.0, c)


def test_score_actions_normalised_and_hand_expanded():
    """exp(logp) over all V actions sums to one, and each logp matches a softmax expanded by
    hand (pure-Python loops, math.fsum) at two temperatures."""
    V, d = 7, 3
    rng = np.random.default_rng(11)
    W = rng.standard_normal((V, d))
    s = rng.standard_normal(d)
    for tau in (1.0, 0.7):
        lp, _ = O.score_actions(W, np.repeat(s[None, :], V, 0), list(range(V)), temperature=tau)
        assert abs(math.fsum(math.exp(x) for x in lp) - 1.0) < 1e-13
        z = [math.fsum(W[v, j] * s[j] for j in range(d)) / tau for v in range(V)]
        lse = math.log(math.fsum(math.exp(x) for x in z))
        for v in range(V):
            assert abs(lp[v] - (z[v] - lse)) < 1e-13


# ---------------------------------------------------------------------------
# Token sampling ([FI] model-RL co-design paragraph: the sampler records the
# log-probability of the distribution it actually drew from)
# ---------------------------------------------------------------------------

def test_sample_top1_is_argmax_with_lowest_id_on_ties():
    """top_k = 1 keeps only the best candidate: the argmax, the lowest id among equal
    maxima, with probability one (logp = 0) for every u."""
    z = np.array([[0.5, 2.0, -1.0, 2.0, 1.9]])
    for u in (0.0, 0.37, 0.999999):
        tok, lp = O.sample_tokens(z, [u], 1.0, 1, 1.0)
        assert tok[0] == 1 and lp[0] == 0.0
    tok, lp = O.sample_tokens(z, [0.5], 1.0, 0, 1e-12)   # a vanishing nucleus is the argmax too
    assert tok[0] == 1 and lp[0] == 0.0


def test_sample_untruncated_partitions_unit_interval_by_softmax():
    """Without truncation the draw is the inverse CDF of softmax(z / T) over ids in
    increasing order: every u strictly inside the interval of token v (bounds from the
    library softmax) draws v, and logp is the library log_softmax."""
    rng = np.random.default_rng(5)
    V = 11
    z = rng.standard_normal((1, V)) * 2.0
    for T in (1.0, 0.6, 3.0):
        p = torch.softmax(torch.from_numpy(z[0] / T), 0).numpy()
        ls = torch.log_softmax(torch.from_numpy(z[0] / T), 0).numpy()
        c = np.concatenate([[0.0], np.cumsum(p)])
        for v in range(V):
            for frac in (0.02, 0.5, 0.98):
                u = c[v] + frac * (c[v + 1] - c[v])
                tok, lp = O.sample_tokens(z, [u], T, 0, 1.0)
                assert tok[0] == v, (T, v, frac)
                assert abs(lp[0] - ls[v]) < 1e-12


def test_sample_hand_built_top_k_and_top_p_sets():
    """z = [1, 3, 2, 3, 0, 2.5]: the ranking (larger z, then smaller id) is 1, 3, 5, 2, 0, 4.
    top_k = 3 keeps {1, 3, 5}; top_p just below the mass share of {1, 3} keeps {1, 3}, just
    above it keeps {1, 3, 5}.  Draws run over the kept ids in increasing order and logp is
    the log of the renormalised share."""
    z = np.array([[1.0, 3.0, 2.0, 3.0, 0.0, 2.5]])
    e = np.exp(z[0] - 3.0)
    kept = [1, 3, 5]
    tot = math.fsum(e[v] for v in kept)
    bounds = np.cumsum([e[v] / tot for v in kept])
    for j, v in enumerate(kept):
        u = (bounds[j - 1] if j else 0.0) + 0.5 * (e[v] / tot)
        tok, lp = O.sample_tokens(z, [u], 1.0, 3, 1.0)
        assert tok[0] == v and abs(lp[0] - math.log(e[v] / tot)) < 1e-13
    share13 = (e[1] + e[3]) / math.fsum(e)
    tok, lp = O.sample_tokens(z, [0.99], 1.0, 0, share13 - 1e-9)
    assert tok[0] == 3 and abs(lp[0] - math.log(0.5)) < 1e-13
    tok, lp = O.sample_tokens(z, [0.99], 1.0, 0, share13 + 1e-9)
    assert tok[0] == 5
    assert abs(lp[0] - math.log(e[5] / (e[1] + e[3] + e[5]))) < 1e-13


def test_sample_top_k_is_applied_before_top_p():
    """z = [3, 2, 1, 0], k = 2, p = 0.7: renormalised over the top-2 the leader has share
    e/(e+1) = 0.731 >= 0.7, so only token 0 survives (logp 0).  Applying top-p over all
    four first (leader share 0.644 < 0.7) would keep two tokens."""
    z = np.array([[3.0, 2.0, 1.0, 0.0]])
    for u in (0.0, 0.5, 0.95):
        tok, lp = O.sample_tokens(z, [u], 1.0, 2, 0.7)
        assert tok[0] == 0 and lp[0] == 0.0


def test_sample_uniform_logits_nucleus():
    """Equal logits over V = 512 with top_p = 0.5 keep ids 0..255 (ties ranked by id), each
    with probability 1/256: u draws id floor(256 u)."""
    z = np.full((4, 512), 0.7)
    us = [0.0, 0.25, 0.99, 0.5 + 1e-6]
    tok, lp = O.sample_tokens(z, us, 1.0, 0, 0.5)
    assert list(tok) == [0, 64, 253, 128]
    np.testing.assert_allclose(lp, -math.log(256.0), rtol=0, atol=1e-13)
    tok, _ = O.sample_tokens(z[:1], [0.999], 1.0, 300, 1.0)   # top-k over ties: ids 0..299
    assert tok[0] == 299
