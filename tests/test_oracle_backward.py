"""Pins for the fp64 full-BPTT backward oracle (``oracle.rlt_backward``).

The hand-written adjoint is checked against things it does not share code with:
central finite differences of the forward oracle's loss (the forward being pinned in
test_oracle_pins.py), and torch fp64 autograd of an independent forward assembled from
library ops (rms_norm, sdpa, gelu/silu, cross_entropy), also with each detach applied by
``.detach()`` at the matching place.  Structural zeros pin the three state paths and
causality.

Pages: [FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer";
[DS] deepsonar "技术拆解 009｜RLT：给 Transformer 接一条时间回路…" (§2.5 full BPTT,
§2.6 second point: every detach is an approximation, §6 recipe).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from workloads import ModelConfig, make_tokens, make_weights, perturb_untied


def tiny_cfg(**kw):
    base = dict(vocab=13, d_model=8, n_heads=2, n_layers=2, ffn_dim=12, ffn_kind="gelu",
                window=3, mem_groups=1, dtype="fp32")
    base.update(kw)
    return ModelConfig(**base)


def model_for(cfg, seed=5, scale=8.0):
    """Weights scaled up from the synthetic init so every path carries a visible gradient."""
    w = perturb_untied(make_weights(cfg, seed), cfg, seed + 1000, 1.0)
    w = {k: (v * scale if k != "b_g" and not k.startswith("g_") else v) for k, v in w.items()}
    rng = np.random.default_rng(seed + 7)
    for k in w:                                    # gains away from 1 so their gradients matter
        if k.startswith("g_"):
            w[k] = w[k] * (1.0 + 0.3 * rng.standard_normal(w[k].shape)).astype(np.float32)
    return O.OracleModel.from_config(cfg, w)


def toks(cfg, T, seed=3):
    return make_tokens(cfg.vocab, 1, T, "uniform", seed)[0]


# ---------------------------------------------------------------------------
# Independent torch fp64 forward (library ops) for autograd
# ---------------------------------------------------------------------------

def torch_loss_and_grads(m, tokens, mask=None, detach=()):
    P = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True) for k, v in m.w.items()}
    d, H, L, W, eps = m.d_model, m.n_heads, m.n_layers, m.window, m.norm_eps
    dh = d // H
    tok = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
    T = tok.shape[0]

    def rms(x, g):
        return F.rms_norm(x, (d,), weight=g, eps=eps)

    def ffn(l, h):
        if m.ffn_kind == "gelu":
            return F.linear(F.gelu(F.linear(h, P["ffn_w1"][l])), P["ffn_w2"][l])
        return F.linear(F.silu(F.linear(h, P["ffn_gate"][l])) * F.linear(h, P["ffn_up"][l]), P["ffn_down"][l])

    def hd(x):  # [n, d] -> [H, n, dh]
        return x.reshape(x.shape[0], H, dh).transpose(0, 1)

    x = P["embed"][tok]
    for l in range(L):
        h = rms(x, P["g_enc_attn"][l])
        q, k, v = (F.linear(h, P[n][l]) for n in ("wq", "wk", "wv"))
        a = F.scaled_dot_product_attention(hd(q), hd(k), hd(v), is_causal=True)
        x = x + F.linear(a.transpose(0, 1).reshape(T, d), P["wo"][l])
        x = x + ffn(l, rms(x, P["g_enc_ffn"][l]))
    e = rms(x, P["g_enc_final"])
    MK = [F.linear(e, P["wkm"][g]) for g in range(m.mem_groups)]
    MV = [F.linear(e, P["wvm"][g]) for g in range(m.mem_groups)]
    if "memory" in detach:
        MK = [t.detach() for t in MK]
        MV = [t.detach() for t in MV]
    s = P["s_star"]
    caches = [[] for _ in range(L)]
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(T):
        s_in = s.detach() if ("s" in detach and t > 0) else s
        gate = torch.sigmoid(F.linear(e[t], P["w_ge"]) + F.linear(s_in, P["w_gs"]) + P["b_g"])
        y = gate * e[t] + (1 - gate) * F.linear(s_in, P["w_fb"])
        for l in range(L):
            h = rms(y, P["g_dec_self"][l])
            q, k, v = (F.linear(h, P[n][l]) for n in ("wq", "wk", "wv"))
            past = caches[l][max(0, len(caches[l]) - (W - 1)):] if W > 1 else []
            if "kv" in detach:
                past = [(pk.detach(), pv.detach()) for pk, pv in past]
            K = torch.stack([pk for pk, _ in past] + [k])
            V = torch.stack([pv for _, pv in past] + [v])
            a = F.scaled_dot_product_attention(hd(q[None]), hd(K), hd(V))
            y = y + F.linear(a.transpose(0, 1).reshape(d), P["wo"][l])
            caches[l].append((k, v))
            h = rms(y, P["g_dec_cross"][l])
            g = 0 if m.mem_groups == 1 else l
            qx = F.linear(h, P["wqx"][l])
            a = F.scaled_dot_product_attention(hd(qx[None]), hd(MK[g][:t + 1]), hd(MV[g][:t + 1]))
            y = y + F.linear(a.transpose(0, 1).reshape(d), P["wox"][l])
            y = y + ffn(l, rms(y, P["g_dec_ffn"][l]))
        s = rms(y, P["g_dec_final"])
        if t < T - 1:
            wt = 1.0 if mask is None else float(mask[t])
            loss = loss + wt * F.cross_entropy(F.linear(s, P["w_out"])[None], tok[t + 1:t + 2])
    loss.backward()
    return float(loss.detach()), {k: (np.zeros(v.shape) if v.grad is None else v.grad.numpy()) for k, v in P.items()}


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

CASES = [
    dict(),
    dict(ffn_kind="swiglu"),
    dict(mem_groups=2),
    dict(window=1),
    dict(window=9, ffn_kind="swiglu", mem_groups=2),
]


@pytest.mark.parametrize("kw", CASES, ids=["gelu", "swiglu", "G=L", "W=1", "W>T"])
def test_taped_loss_equals_replay_loss(kw):
    cfg = tiny_cfg(**kw)
    m = model_for(cfg)
    tk = toks(cfg, 7)
    loss, _, S = O.bptt(m, tk)
    S_ref, _ = O.replay(m, tk)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-13)
    assert abs(loss - O.next_token_loss(m, tk)) <= 1e-12 * max(1.0, abs(loss))


@pytest.mark.parametrize("kw", CASES[:3] + CASES[4:], ids=["gelu", "swiglu", "G=L", "W>T"])
def test_gradient_matches_central_differences(kw):
    """Every parameter tensor, a few entries each: (L(p+h) - L(p-h)) / 2h against the adjoint.
    An SFT-style mask (some positions unsupervised, others weighted) is used."""
    cfg = tiny_cfg(**kw)
    m = model_for(cfg)
    T = 7
    tk = toks(cfg, T)
    mask = np.array([1.0, 0.0, 0.5, 1.0, 0.0, 2.0])
    _, grads, _ = O.bptt(m, tk, mask)
    rng = np.random.default_rng(11)
    hstep = 1e-5
    checked = 0
    for name, val in m.w.items():
        flat = val.reshape(-1)
        picks = rng.choice(flat.size, size=min(3, flat.size), replace=False)
        if name == "embed":                        # rows of tokens that occur
            picks = np.array([int(tk[0]) * cfg.d_model, int(tk[3]) * cfg.d_model + 2])
        for i in picks:
            old = flat[i]
            flat[i] = old + hstep
            lp = O.next_token_loss(m, tk, mask)
            flat[i] = old - hstep
            lm = O.next_token_loss(m, tk, mask)
            flat[i] = old
            fd = (lp - lm) / (2 * hstep)
            an = grads[name].reshape(-1)[i]
            assert abs(fd - an) <= 1e-7 + 1e-6 * abs(an), (name, int(i), fd, an)
            checked += 1
    assert checked >= 3 * 20


DETACHES = [(), ("s",), ("kv",), ("memory",), ("s", "kv", "memory")]


@pytest.mark.parametrize("kw", CASES, ids=["gelu", "swiglu", "G=L", "W=1", "W>T"])
@pytest.mark.parametrize("detach", DETACHES, ids=["exact", "s", "kv", "memory", "all"])
def test_gradient_matches_torch_autograd(kw, detach):
    cfg = tiny_cfg(**kw)
    m = model_for(cfg)
    tk = toks(cfg, 8, seed=4)
    loss, grads, _ = O.bptt(m, tk, detach=detach)
    tloss, tgrads = torch_loss_and_grads(m, tk, detach=detach)
    assert abs(loss - tloss) <= 1e-11 * max(1.0, abs(tloss))
    for k in grads:
        ref = tgrads[k]
        np.testing.assert_allclose(grads[k], ref, rtol=1e-8, atol=1e-11 * max(1.0, np.abs(ref).max()),
                                   err_msg=k)


def test_each_detach_changes_the_gradient():
    """Each path carries gradient: cutting any one of them moves some gradient."""
    cfg = tiny_cfg(window=3, mem_groups=2)
    m = model_for(cfg)
    tk = toks(cfg, 8, seed=4)
    _, exact, _ = O.bptt(m, tk)
    for path in O.DETACH_PATHS:
        _, approx, _ = O.bptt(m, tk, detach=(path,))
        diff = max(np.abs(exact[k] - approx[k]).max() for k in exact)
        assert diff > 1e-6, path


def test_no_supervised_position_gives_zero_gradient():
    cfg = tiny_cfg()
    m = model_for(cfg)
    tk = toks(cfg, 6)
    loss, grads, _ = O.bptt(m, tk, mask=np.zeros(5))
    assert loss == 0.0
    assert all(not np.any(g) for g in grads.values())
    loss1, grads1, _ = O.bptt(m, tk[:1])           # T = 1: nothing to predict
    assert loss1 == 0.0 and all(not np.any(g) for g in grads1.values())


def test_state_paths_reach_s_star_and_cutting_them_isolates_it():
    """A loss at one late prediction reaches s* through the recurrence (s) and the window
    caches (kv).  With s cut, the caches alone carry s*'s influence at most W-1 positions
    forward per layer: step 0's layer-l entry is read at layer l by steps up to W-1 later,
    which changes their entries of layer l+1 and nothing below, so the last step reached is
    L (W-1).  With both cut, s* gets exactly nothing (memory does not depend on s)."""
    cfg = tiny_cfg(window=3)                       # L = 2: reach = 2 * (3 - 1) = 4
    m = model_for(cfg)
    T = 8
    tk = toks(cfg, T)
    reach = cfg.n_layers * (cfg.window - 1)

    def grad_s_star(t, detach=()):
        mask = np.zeros(T - 1)
        mask[t] = 1.0
        return O.bptt(m, tk, mask, detach=detach)[1]["s_star"]

    assert np.abs(grad_s_star(T - 2)).max() > 1e-8
    assert np.abs(grad_s_star(reach, ("s",))).max() > 1e-12
    assert not np.any(grad_s_star(reach + 1, ("s",)))
    assert not np.any(grad_s_star(T - 2, ("s",)))
    assert not np.any(grad_s_star(1, ("s", "kv")))


def test_memory_detach_leaves_memory_projections_without_gradient():
    cfg = tiny_cfg(mem_groups=2)
    m = model_for(cfg)
    tk = toks(cfg, 6)
    _, g, _ = O.bptt(m, tk, detach=("memory",))
    assert not np.any(g["wkm"]) and not np.any(g["wvm"])
    _, g, _ = O.bptt(m, tk)
    assert np.abs(g["wkm"]).max() > 0 and np.abs(g["wvm"]).max() > 0


def test_backward_is_causal_in_the_tokens():
    """The prediction at position t depends on tokens 0..t only (the target enters through
    the head): embedding rows of tokens that occur only later get no gradient."""
    cfg = tiny_cfg(vocab=16)
    m = model_for(cfg)
    tk = np.arange(8, dtype=np.int64)              # distinct ids: id == position
    mask = np.zeros(7)
    mask[3] = 1.0                                  # predict token 4 from positions 0..3
    _, g, _ = O.bptt(m, tk, mask)
    assert np.all(np.abs(g["embed"][:4]).max(axis=1) > 0)
    assert not np.any(g["embed"][4:])


def test_batch_is_sum_of_sequences():
    cfg = tiny_cfg()
    m = model_for(cfg)
    tk = make_tokens(cfg.vocab, 2, 5, "uniform", 9)
    total, grads = O.bptt_batch(m, tk)
    l0, g0, _ = O.bptt(m, tk[0])
    l1, g1, _ = O.bptt(m, tk[1])
    assert total == pytest.approx(l0 + l1, rel=1e-14)
    for k in grads:
        np.testing.assert_allclose(grads[k], g0[k] + g1[k], rtol=1e-13, atol=1e-15)


def test_errors():
    cfg = tiny_cfg()
    m = model_for(cfg)
    with pytest.raises(ValueError):
        O.bptt(m, [0, 1, 2], detach=("everything",))
    with pytest.raises(ValueError):
        O.bptt(m, [0, 1, 2], mask=[1.0])
    with pytest.raises(ValueError):
        O.bptt(m, [0, 99])
