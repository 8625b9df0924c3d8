"""Plain fp64 CPU oracle for the full-BPTT backward of RLT replay.

TEST INFRASTRUCTURE ONLY (same rule as ``rlt_oracle``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may import it.

Pages cited (titles as printed on each page):
  [FI] feinterview: "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer"
  [DS] deepsonar:   "技术拆解 009｜RLT：给 Transformer 接一条时间回路，潜变量推理与「无限时间深度」的真面目"

What is computed.  The pages train by full back-propagation through time: teacher forcing,
every valid next-token prediction supervised, gradient through the whole recurrent
trajectory ([DS] §2.5 and the build-your-own recipe in §6, steps on full BPTT; [FI]
model-RL co-design paragraph).  The exact gradient reaches the parameters through three
state paths, and cutting any of them is an approximation ([DS] §2.6, second point):
the recurrent output s_{t-1} fed into the merge, the decoder window keys/values, and the
encoder memory read by cross-attention.

Readings taken where the pages leave a step open:
  loss = sum over t = 1..T-1 of mask_t * CE(W_out s_t, tok_{t+1}) for one sequence (the
    pages' pseudo-code accumulates the per-step cross-entropy; a sum, not a mean);
    ``mask`` defaults to all ones (pretraining) and is zero where a position is not
    supervised (SFT keeps only assistant targets while the state runs over the whole
    sequence, [DS] §2.5);
  gradients are taken for every parameter, s* included ([DS] §6 lets s* be learned);
    tied encoder/decoder tensors collect both stacks' contributions;
  ``detach`` names explicit approximations, each cutting one path and nothing else:
    "s"      — s_{t-1} entering the merge at step t >= 2 is a constant (s* still gets the
               first merge's gradient);
    "kv"     — window entries of earlier positions are constants for later steps (the
               current position's own key/value still gets its gradient);
    "memory" — memory rows are constants for cross-attention (no gradient into W_KM,
               W_VM or the encoder through the memory; e_t still gets the merge's).
  The forward is the one of ``rlt_oracle`` (same sub-layers, same readings).

Method: one forward pass that keeps every intermediate (the tape), then the adjoint
recurrence in reverse time: per step, the adjoint of s_t (its own logit term plus what the
next merge sends back), through the final norm, the layers in reverse (FFN, cross-
attention, window attention), into the merge; window key/value adjoints and memory-row
adjoints are accumulated across the later steps that read them and consumed when their own
position is reached (window) or after the decoder sweep (memory); then the encoder in
reverse, token-parallel.  Every sub-layer's adjoint is written from its definition.

Pins (tests/test_oracle_backward.py): the taped loss equals the loss computed from
``rlt_oracle.replay``; central finite differences of that loss on every parameter tensor;
torch fp64 autograd of an independent forward built from library ops (also with each
detach); structural zeros (no supervised position, paths cut).
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

from .rlt_oracle import OracleModel, gelu, rms_norm, replay, sigmoid, silu

F64 = np.float64
DETACH_PATHS = ("s", "kv", "memory")


# ---------------------------------------------------------------------------
# Loss from the forward oracle
# ---------------------------------------------------------------------------

def _mask_or_default(mask: Optional[Sequence[float]], T: int) -> np.ndarray:
    if mask is None:
        return np.ones(max(T - 1, 0), dtype=F64)
    m = np.asarray(mask, dtype=F64)
    if m.shape != (max(T - 1, 0),):
        raise ValueError("mask must have one weight per predicted position (T-1)")
    return m


def next_token_loss(m: OracleModel, tokens: Sequence[int], mask: Optional[Sequence[float]] = None) -> float:
    """sum_t mask_t * CE(W_out s_t, tok_{t+1}), with s_t from ``rlt_oracle.replay``."""
    tok = np.asarray(tokens, dtype=np.int64)
    mk = _mask_or_default(mask, tok.shape[0])
    _, Z = replay(m, tok)
    loss = 0.0
    for t in range(tok.shape[0] - 1):
        z = Z[t]
        zmax = z.max()
        lse = zmax + math.log(float(np.exp(z - zmax).sum()))
        loss += mk[t] * (lse - z[tok[t + 1]])
    return float(loss)


# ---------------------------------------------------------------------------
# Sub-layer adjoints (rows are the leading axis; a single vector is one row)
# ---------------------------------------------------------------------------

def rms_norm_bwd(x: np.ndarray, gain: np.ndarray, dout: np.ndarray, eps: float
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Adjoint of out = g * x / r, r = sqrt(mean(x^2) + eps), per row.

    With n = x / r and dn = dout * g:  dx = (dn - n * mean(dn * n)) / r;  dg = sum_rows dout * n.
    """
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = x / r
    dn = dout * gain
    dx = (dn - n * np.mean(dn * n, axis=-1, keepdims=True)) / r
    dg = (dout * n).reshape(-1, x.shape[-1]).sum(axis=0)
    return dx, dg


def gelu_grad(u: np.ndarray) -> np.ndarray:
    """d/du [u Phi(u)] = Phi(u) + u phi(u)."""
    return 0.5 * (1.0 + _erf(u / math.sqrt(2.0))) + u * np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def silu_grad(u: np.ndarray) -> np.ndarray:
    """d/du [u sigma(u)] = sigma(u) (1 + u (1 - sigma(u)))."""
    sg = sigmoid(u)
    return sg * (1.0 + u * (1.0 - sg))


def attend_taped(q: np.ndarray, keys: np.ndarray, values: np.ndarray, n_heads: int
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Multi-head attention of one query (as ``rlt_oracle.attend``), also returning the
    per-head probabilities P [H, n]."""
    d = q.shape[0]
    dh = d // n_heads
    out = np.empty(d, dtype=F64)
    P = np.empty((n_heads, keys.shape[0]), dtype=F64)
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        z = keys[:, sl] @ q[sl] / math.sqrt(dh)
        p = np.exp(z - z.max())
        P[h] = p / p.sum()
        out[sl] = P[h] @ values[:, sl]
    return out, P


def attend_bwd(q: np.ndarray, keys: np.ndarray, values: np.ndarray, P: np.ndarray, dout: np.ndarray
               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Adjoint of one query's attention.  Per head, z_j = q.k_j / sqrt(dh), p = softmax(z),
    o = sum_j p_j v_j:  dv_j = p_j do;  dp_j = do.v_j;  dz_j = p_j (dp_j - sum_i p_i dp_i);
    dq = sum_j dz_j k_j / sqrt(dh);  dk_j = dz_j q / sqrt(dh)."""
    H = P.shape[0]
    d = q.shape[0]
    dh = d // H
    dq = np.empty(d, dtype=F64)
    dk = np.empty_like(keys)
    dv = np.empty_like(values)
    for h in range(H):
        sl = slice(h * dh, (h + 1) * dh)
        p = P[h]
        dp = values[:, sl] @ dout[sl]
        dz = p * (dp - p @ dp)
        dq[sl] = dz @ keys[:, sl] / math.sqrt(dh)
        dk[:, sl] = np.outer(dz, q[sl]) / math.sqrt(dh)
        dv[:, sl] = np.outer(p, dout[sl])
    return dq, dk, dv


def causal_attention_taped(Q: np.ndarray, K: np.ndarray, V: np.ndarray, n_heads: int
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """Causal MHA over one whole sequence (query i sees keys 0..i); also returns P [H, T, T]."""
    T, d = Q.shape
    dh = d // n_heads
    out = np.empty((T, d), dtype=F64)
    P = np.zeros((n_heads, T, T), dtype=F64)
    masked = np.arange(T)[None, :] > np.arange(T)[:, None]
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        z = Q[:, sl] @ K[:, sl].T / math.sqrt(dh)
        z[masked] = -np.inf
        p = np.exp(z - z.max(axis=1, keepdims=True))
        P[h] = p / p.sum(axis=1, keepdims=True)
        out[:, sl] = P[h] @ V[:, sl]
    return out, P


def causal_attention_bwd(Q, K, V, P, dO):
    """Adjoint of ``causal_attention_taped``: the single-query rule applied to every row
    (masked probabilities are exactly zero, so they contribute nothing)."""
    T, d = Q.shape
    H = P.shape[0]
    dh = d // H
    dQ, dK, dV = np.empty_like(Q), np.empty_like(K), np.empty_like(V)
    for h in range(H):
        sl = slice(h * dh, (h + 1) * dh)
        p = P[h]
        dP = dO[:, sl] @ V[:, sl].T
        dZ = p * (dP - (p * dP).sum(axis=1, keepdims=True))
        dQ[:, sl] = dZ @ K[:, sl] / math.sqrt(dh)
        dK[:, sl] = dZ.T @ Q[:, sl] / math.sqrt(dh)
        dV[:, sl] = p.T @ dO[:, sl]
    return dQ, dK, dV


class _Grads:
    """Gradient accumulators, one zero array per parameter."""

    def __init__(self, m: OracleModel):
        self.g = {k: np.zeros_like(v) for k, v in m.w.items()}

    def __getitem__(self, k):
        return self.g[k]


def ffn_fwd(m: OracleModel, l: int, h: np.ndarray):
    """Layer-l FFN on rows h; returns (out, saved pre-activations)."""
    w = m.w
    if m.ffn_kind == "gelu":
        u = h @ w["ffn_w1"][l].T
        return gelu(u) @ w["ffn_w2"][l].T, (u,)
    ug = h @ w["ffn_gate"][l].T
    uu = h @ w["ffn_up"][l].T
    return (silu(ug) * uu) @ w["ffn_down"][l].T, (ug, uu)


def ffn_bwd(m: OracleModel, G: _Grads, l: int, h: np.ndarray, saved, dout: np.ndarray) -> np.ndarray:
    """Adjoint of ``ffn_fwd`` on rows: accumulates the weight gradients, returns dh."""
    w = m.w
    if m.ffn_kind == "gelu":
        (u,) = saved
        G["ffn_w2"][l] += dout.T @ gelu(u)
        du = (dout @ w["ffn_w2"][l]) * gelu_grad(u)
        G["ffn_w1"][l] += du.T @ h
        return du @ w["ffn_w1"][l]
    ug, uu = saved
    a = silu(ug)
    G["ffn_down"][l] += dout.T @ (a * uu)
    da = dout @ w["ffn_down"][l]
    dug = da * uu * silu_grad(ug)
    duu = da * a
    G["ffn_gate"][l] += dug.T @ h
    G["ffn_up"][l] += duu.T @ h
    return dug @ w["ffn_gate"][l] + duu @ w["ffn_up"][l]


# ---------------------------------------------------------------------------
# Taped forward
# ---------------------------------------------------------------------------

def _encoder_taped(m: OracleModel, tok: np.ndarray):
    w, eps, H = m.w, m.norm_eps, m.n_heads
    x = w["embed"][tok].copy()
    tape = []
    for l in range(m.n_layers):
        x_in = x
        ha = rms_norm(x_in, w["g_enc_attn"][l], eps)
        Q, K, V = ha @ w["wq"][l].T, ha @ w["wk"][l].T, ha @ w["wv"][l].T
        A, P = causal_attention_taped(Q, K, V, H)
        x_mid = x_in + A @ w["wo"][l].T
        hf = rms_norm(x_mid, w["g_enc_ffn"][l], eps)
        fo, fs = ffn_fwd(m, l, hf)
        x = x_mid + fo
        tape.append((x_in, ha, Q, K, V, A, P, x_mid, hf, fs))
    e = rms_norm(x, w["g_enc_final"], eps)
    MK = [e @ w["wkm"][g].T for g in range(m.mem_groups)]
    MV = [e @ w["wvm"][g].T for g in range(m.mem_groups)]
    return e, MK, MV, x, tape


def _decoder_taped(m: OracleModel, e: np.ndarray, MK, MV):
    """Sequential decoder over all T positions, keeping every intermediate.

    The window of layer l at step t is positions max(0, t-W+1) .. t; their keys/values are
    kept in full arrays KC[l], VC[l] (row j = position j) and sliced per step."""
    w, eps, H, L, W = m.w, m.norm_eps, m.n_heads, m.n_layers, m.window
    T, d = e.shape
    KC = np.zeros((L, T, d))
    VC = np.zeros((L, T, d))
    S = np.empty((T, d))
    steps = []
    s = w["s_star"].copy()
    for t in range(T):
        s_prev = s
        f = w["w_fb"] @ s_prev
        gate = sigmoid(w["w_ge"] @ e[t] + w["w_gs"] @ s_prev + w["b_g"])
        y = gate * e[t] + (1.0 - gate) * f
        layers = []
        j0 = max(0, t - W + 1)
        for l in range(L):
            y_in = y
            h = rms_norm(y_in, w["g_dec_self"][l], eps)
            q, k, v = w["wq"][l] @ h, w["wk"][l] @ h, w["wv"][l] @ h
            KC[l, t], VC[l, t] = k, v
            o, P = attend_taped(q, KC[l, j0:t + 1], VC[l, j0:t + 1], H)
            y1 = y_in + w["wo"][l] @ o
            h2 = rms_norm(y1, w["g_dec_cross"][l], eps)
            g = m.group_of(l)
            qx = w["wqx"][l] @ h2
            o2, P2 = attend_taped(qx, MK[g][:t + 1], MV[g][:t + 1], H)
            y2 = y1 + w["wox"][l] @ o2
            h3 = rms_norm(y2, w["g_dec_ffn"][l], eps)
            fo, fs = ffn_fwd(m, l, h3[None, :])
            y = y2 + fo[0]
            layers.append((y_in, h, q, o, P, y1, h2, qx, o2, P2, y2, h3, fs))
        s = rms_norm(y, w["g_dec_final"], eps)
        S[t] = s
        steps.append((s_prev, f, gate, y, layers))
    return S, KC, VC, steps


# ---------------------------------------------------------------------------
# Full BPTT
# ---------------------------------------------------------------------------

def bptt(m: OracleModel, tokens: Sequence[int], mask: Optional[Sequence[float]] = None,
         detach: Iterable[str] = ()) -> Tuple[float, Dict[str, np.ndarray], np.ndarray]:
    """Loss and exact gradients of one sequence's next-token loss.

    Returns (loss, grads keyed like ``m.w``, S [T, d]).  ``detach`` (subset of "s", "kv",
    "memory") applies the named approximations; the default is the exact gradient."""
    detach = set(detach)
    bad = detach - set(DETACH_PATHS)
    if bad:
        raise ValueError(f"unknown detach path(s): {sorted(bad)}")
    w, eps, L, W = m.w, m.norm_eps, m.n_layers, m.window
    tok = np.asarray(tokens, dtype=np.int64)
    T = tok.shape[0]
    if T == 0:
        return 0.0, _Grads(m).g, np.zeros((0, m.d_model))
    if tok.min() < 0 or tok.max() >= m.vocab:
        raise ValueError("token id out of range")
    mk = _mask_or_default(mask, T)
    d = m.d_model

    e, MK, MV, x_last, enc_tape = _encoder_taped(m, tok)
    S, KC, VC, steps = _decoder_taped(m, e, MK, MV)

    G = _Grads(m)
    # Loss and its gradient on every s_t (off the loop: token-parallel).
    Z = S @ w["w_out"].T
    dS = np.zeros((T, d))
    loss = 0.0
    for t in range(T - 1):
        if mk[t] == 0.0:
            continue
        z = Z[t]
        p = np.exp(z - z.max())
        lse = z.max() + math.log(float(p.sum()))
        loss += mk[t] * (lse - z[tok[t + 1]])
        dz = p / p.sum()
        dz[tok[t + 1]] -= 1.0
        dz *= mk[t]
        G["w_out"][...] += np.outer(dz, S[t])
        dS[t] = w["w_out"].T @ dz

    # Decoder in reverse time.
    dKC = np.zeros((L, T, d))          # adjoint of window key of layer l at position j
    dVC = np.zeros((L, T, d))
    dMK = [np.zeros((T, d)) for _ in range(m.mem_groups)]
    dMV = [np.zeros((T, d)) for _ in range(m.mem_groups)]
    de = np.zeros((T, d))
    ds_carry = np.zeros(d)             # adjoint of s_t sent back by the merge of step t+1
    for t in range(T - 1, -1, -1):
        s_prev, f, gate, y_fin, layers = steps[t]
        ds = dS[t] + ds_carry
        dy, dg = rms_norm_bwd(y_fin, w["g_dec_final"], ds, eps)
        G["g_dec_final"][...] += dg
        j0 = max(0, t - W + 1)
        for l in range(L - 1, -1, -1):
            y_in, h, q, o, P, y1, h2, qx, o2, P2, y2, h3, fs = layers[l]
            g = m.group_of(l)
            # FFN sub-block
            dh3 = ffn_bwd(m, G, l, h3[None, :], fs, dy[None, :])[0]
            dx, dg = rms_norm_bwd(y2, w["g_dec_ffn"][l], dh3, eps)
            G["g_dec_ffn"][l] += dg
            dy = dy + dx
            # cross-attention sub-block
            G["wox"][l] += np.outer(dy, o2)
            do2 = w["wox"][l].T @ dy
            dqx, dmk, dmv = attend_bwd(qx, MK[g][:t + 1], MV[g][:t + 1], P2, do2)
            if "memory" not in detach:
                dMK[g][:t + 1] += dmk
                dMV[g][:t + 1] += dmv
            G["wqx"][l] += np.outer(dqx, h2)
            dx, dg = rms_norm_bwd(y1, w["g_dec_cross"][l], w["wqx"][l].T @ dqx, eps)
            G["g_dec_cross"][l] += dg
            dy = dy + dx
            # window self-attention sub-block
            G["wo"][l] += np.outer(dy, o)
            do = w["wo"][l].T @ dy
            dq, dk, dv = attend_bwd(q, KC[l, j0:t + 1], VC[l, j0:t + 1], P, do)
            dk_t = dk[-1] + dKC[l, t]
            dv_t = dv[-1] + dVC[l, t]
            if "kv" not in detach:
                dKC[l, j0:t] += dk[:-1]
                dVC[l, j0:t] += dv[:-1]
            G["wq"][l] += np.outer(dq, h)
            G["wk"][l] += np.outer(dk_t, h)
            G["wv"][l] += np.outer(dv_t, h)
            dh = w["wq"][l].T @ dq + w["wk"][l].T @ dk_t + w["wv"][l].T @ dv_t
            dx, dg = rms_norm_bwd(y_in, w["g_dec_self"][l], dh, eps)
            G["g_dec_self"][l] += dg
            dy = dy + dx
        # gated merge: y = gate * e + (1 - gate) * f,  gate = sigmoid(W_ge e + W_gs s + b_g)
        da = dy * (e[t] - f) * gate * (1.0 - gate)
        df = dy * (1.0 - gate)
        de[t] += dy * gate + w["w_ge"].T @ da
        G["w_fb"][...] += np.outer(df, s_prev)
        G["w_ge"][...] += np.outer(da, e[t])
        G["w_gs"][...] += np.outer(da, s_prev)
        G["b_g"][...] += da
        ds_prev = w["w_fb"].T @ df + w["w_gs"].T @ da
        if t == 0:
            G["s_star"][...] += ds_prev
        ds_carry = np.zeros(d) if "s" in detach else ds_prev

    # Memory rows back onto e.
    for g in range(m.mem_groups):
        G["wkm"][g] += dMK[g].T @ e
        G["wvm"][g] += dMV[g].T @ e
        de += dMK[g] @ w["wkm"][g] + dMV[g] @ w["wvm"][g]

    # Encoder in reverse (token-parallel).
    dx, dg = rms_norm_bwd(x_last, w["g_enc_final"], de, eps)
    G["g_enc_final"][...] += dg
    for l in range(L - 1, -1, -1):
        x_in, ha, Q, K, V, A, P, x_mid, hf, fs = enc_tape[l]
        dhf = ffn_bwd(m, G, l, hf, fs, dx)
        dxm, dg = rms_norm_bwd(x_mid, w["g_enc_ffn"][l], dhf, eps)
        G["g_enc_ffn"][l] += dg
        dx = dx + dxm
        G["wo"][l] += dx.T @ A
        dQ, dK, dV = causal_attention_bwd(Q, K, V, P, dx @ w["wo"][l])
        G["wq"][l] += dQ.T @ ha
        G["wk"][l] += dK.T @ ha
        G["wv"][l] += dV.T @ ha
        dha = dQ @ w["wq"][l] + dK @ w["wk"][l] + dV @ w["wv"][l]
        dxi, dg = rms_norm_bwd(x_in, w["g_enc_attn"][l], dha, eps)
        G["g_enc_attn"][l] += dg
        dx = dx + dxi
    np.add.at(G["embed"], tok, dx)
    return float(loss), G.g, S


def bptt_batch(m: OracleModel, tokens: np.ndarray, masks: Optional[np.ndarray] = None,
               detach: Iterable[str] = ()) -> Tuple[float, Dict[str, np.ndarray]]:
    """Sum of ``bptt`` over independent sequences (rows of ``tokens``)."""
    total, grads = 0.0, None
    for b in range(tokens.shape[0]):
        lb, gb, _ = bptt(m, tokens[b], None if masks is None else masks[b], detach)
        total += lb
        if grads is None:
            grads = gb
        else:
            for k in grads:
                grads[k] += gb[k]
    return total, grads
