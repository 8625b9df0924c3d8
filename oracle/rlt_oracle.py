"""Plain fp64 CPU oracle for Recurrent Looped Transformer (RLT) exact replay.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP path and imports nothing from it; the two meet only in the seeded
input generators of ``workloads/`` (which contain none of the method's
arithmetic).

Pages cited (titles as printed on each page):
  [FI] feinterview: "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer"
  [DS] deepsonar:   "技术拆解 009｜RLT：给 Transformer 接一条时间回路，潜变量推理与「无限时间深度」的真面目"
  [AL] alphalab:    "Recurrent Looped Transformer：路徑變深，就真的更會推理嗎？（2026）"

What is computed (everything in float64, one sequence at a time):

  Encoder ([FI] architecture paragraph; [DS] §2.1), for known tokens, causal:
      x_t = E[tok_t]
      per layer l: x_t += W_O^l MHA_causal(RMS(x; g_enc_attn^l))
                   x_t += FFN^l(RMS(x_t; g_enc_ffn^l))
      e_t = RMS(x_t; g_enc_final);  memory K^{M,g}_t = W_KM^g e_t, V^{M,g}_t = W_VM^g e_t
      for g = 1..G (G = 1 shared, or G = L_D one per decoder layer).

  Decoder ([FI] decoder-state paragraph; [DS] §2.2–§2.4; [AL] §一), sequential:
      H_0 = (s*, empty caches);  for t = 1..T:
        f = W_fb s_{t-1};  g = sigmoid(W_ge e_t + W_gs s_{t-1} + b_g);  y = g*e_t + (1-g)*f
        per layer l (attention and FFN weights are the encoder's layer l):
          h = RMS(y; g_dec_self^l);  q,k,v = W_Q^l h, W_K^l h, W_V^l h
          y += W_O^l MHA(q over C_l ++ [(k,v)])          (window of W incl. the current token)
          h = RMS(y; g_dec_cross^l);  y += W_Ox^l MHA(W_Qx^l h over memory group g(l), entries j <= t)
          y += FFN^l(RMS(y; g_dec_ffn^l))
          append (k,v) to C_l, drop the oldest entry beyond W-1
        s_t = RMS(y; g_dec_final);  logits_t = W_out s_t

Readings taken where the pages leave a step open:
  gated merge form (sigmoid gate between e_t and the feedback projection W_fb s_{t-1});
  decoder input built from e_t; memory projected from e_t with G groups;
  SWA keys/values are projections of the same normalised layer input as the query;
  pre-RMSNorm residual sub-blocks, eps = 1e-6; no positional encoding;
  MHA scale 1/sqrt(d_head), softmax with max subtraction; cross-attention has its own
  untied W_Qx, W_Ox; window at step t = positions max(1, t-W+1)..t; memory entry t is
  visible at step t; exact-erf GELU; SwiGLU = W_down(silu(W_gate h) * W_up h);
  logits from a separate head W_out; no biases except b_g.

Pins (tests/test_oracle_pins.py): library sub-layers (torch fp64 rms_norm, gelu, silu,
sdpa), causal encoder vs a torch sdpa pass, gate-saturated decoder vs a token-parallel
masked sdpa pass, W=1 and T=1 closed forms, causality, split invariance, incremental ==
replay, G equivalence, window >= T equivalence, state path length t*L_D; action scoring
against closed forms (zero head, one dominant logit, normalisation over all actions,
temperature on a hand-expanded softmax); token sampling against special cases (top-1 is the
argmax, the untruncated draw partitions [0, 1) by the library softmax, hand-built top-k and
top-p sets, truncation order, uniform logits).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64


# ---------------------------------------------------------------------------
# Sub-layers
# ---------------------------------------------------------------------------

def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMS(x; g) = g * x / sqrt(mean(x^2) + eps) over the last axis."""
    return gain * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, n_heads: int) -> np.ndarray:
    """Multi-head attention of ONE query vector over a list of keys/values.

    q [d], keys/values [n, d]; heads are contiguous slices of width d/H;
    per head: softmax_j(q_h . k_{j,h} / sqrt(d_h)) weighted sum of v_{j,h}.
    """
    d = q.shape[0]
    dh = d // n_heads
    out = np.empty(d, dtype=F64)
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        z = keys[:, sl] @ q[sl] / math.sqrt(dh)
        p = np.exp(z - z.max())
        out[sl] = (p / p.sum()) @ values[:, sl]
    return out


def causal_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, n_heads: int,
                     q_offset: int) -> np.ndarray:
    """Causal MHA for a block of queries.

    Q [n, d] are positions q_offset .. q_offset+n-1; K, V [q_offset+n, d] are
    positions 0 .. q_offset+n-1.  Query row i sees keys 0 .. q_offset+i.
    Rows are evaluated in blocks; each row gets its own exact softmax.
    """
    n, d = Q.shape
    dh = d // n_heads
    out = np.empty((n, d), dtype=F64)
    blk = 256
    for i0 in range(0, n, blk):
        i1 = min(n, i0 + blk)
        kmax = q_offset + i1                       # keys visible to the last row of the block
        rows = np.arange(q_offset + i0, q_offset + i1)[:, None]
        cols = np.arange(kmax)[None, :]
        masked = cols > rows
        for h in range(n_heads):
            sl = slice(h * dh, (h + 1) * dh)
            z = Q[i0:i1, sl] @ K[:kmax, sl].T / math.sqrt(dh)
            z[masked] = -np.inf
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            out[i0:i1, sl] = (p / p.sum(axis=1, keepdims=True)) @ V[:kmax, sl]
    return out


# ---------------------------------------------------------------------------
# Model parameters
# ---------------------------------------------------------------------------

@dataclass
class OracleModel:
    """fp64 copy of the parameters plus the shape constants.

    ``weights`` maps the canonical names of ``workloads.synth.PARAM_ORDER`` to
    arrays; per-layer tensors have a leading layer axis, memory projections a
    leading group axis.  Encoder layer l and decoder layer l use the SAME
    W_Q, W_K, W_V, W_O and FFN tensors (tying, [FI] tied-configuration
    paragraph); gains, cross-attention, memory projections and the merge are
    not shared.
    """
    vocab: int
    d_model: int
    n_heads: int
    n_layers: int
    ffn_dim: int
    ffn_kind: str
    window: int
    mem_groups: int
    norm_eps: float
    w: Dict[str, np.ndarray]

    @classmethod
    def from_config(cls, cfg, weights: Dict[str, np.ndarray]) -> "OracleModel":
        if cfg.d_model % cfg.n_heads != 0:
            raise ValueError("d_model must be a multiple of n_heads")
        if cfg.mem_groups not in (1, cfg.n_layers):
            raise ValueError("memory groups must be 1 or n_layers")
        if cfg.window < 1:
            raise ValueError("window must be >= 1")
        w = {k: np.asarray(v, dtype=F64) for k, v in weights.items()}
        return cls(cfg.vocab, cfg.d_model, cfg.n_heads, cfg.n_layers, cfg.ffn_dim,
                   cfg.ffn_kind, cfg.window, cfg.mem_groups, cfg.norm_eps, w)

    def ffn(self, l: int, h: np.ndarray) -> np.ndarray:
        """Layer-l FFN (shared by encoder layer l and decoder layer l)."""
        w = self.w
        if self.ffn_kind == "gelu":
            return gelu(h @ w["ffn_w1"][l].T) @ w["ffn_w2"][l].T
        return (silu(h @ w["ffn_gate"][l].T) * (h @ w["ffn_up"][l].T)) @ w["ffn_down"][l].T

    def group_of(self, l: int) -> int:
        """Memory group read by decoder layer l: 0 when G = 1, else l."""
        return 0 if self.mem_groups == 1 else l


# ---------------------------------------------------------------------------
# State H_t and the encoder side
# ---------------------------------------------------------------------------

@dataclass
class OracleState:
    """Complete state of one sequence.

    Decoder state H_t = (s_t, C^D_t) ([FI] decoder-state paragraph; [DS] §2.3):
    ``s`` and the per-layer window caches ``dec_cache[l]`` (explicit lists of
    (k, v), at most W-1 entries).  Encoder side: per-layer encoder key/value
    lists (for incremental encoding), and the produced e_t and memory rows.
    ``depth`` counts decoder blocks on the recurrent path from s_0.
    """
    s: np.ndarray
    dec_cache: List[List[Tuple[np.ndarray, np.ndarray]]]
    enc_k: List[List[np.ndarray]]
    enc_v: List[List[np.ndarray]]
    e: List[np.ndarray] = field(default_factory=list)
    mem_k: List[List[np.ndarray]] = field(default_factory=list)
    mem_v: List[List[np.ndarray]] = field(default_factory=list)
    t_dec: int = 0
    depth: int = 0

    @property
    def t_enc(self) -> int:
        return len(self.e)


def init_state(m: OracleModel) -> OracleState:
    """H_0 = (s*, empty caches), set once before the first token (no later reset)."""
    L, G = m.n_layers, m.mem_groups
    return OracleState(
        s=m.w["s_star"].copy(),
        dec_cache=[[] for _ in range(L)],
        enc_k=[[] for _ in range(L)],
        enc_v=[[] for _ in range(L)],
        mem_k=[[] for _ in range(G)],
        mem_v=[[] for _ in range(G)],
    )


def encode(m: OracleModel, st: OracleState, tokens: Sequence[int]) -> np.ndarray:
    """Append ``tokens`` (positions t_enc .. t_enc+n-1) to the causal encoder.

    Each new position attends to every earlier position (cached keys) and to
    the new positions up to itself.  Produces e_t and the G memory rows.
    Returns e for the new positions [n, d].
    """
    w = m.w
    tok = np.asarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    if n == 0:
        return np.zeros((0, m.d_model))
    if tok.min() < 0 or tok.max() >= m.vocab:
        raise ValueError("token id out of range")
    t0 = st.t_enc
    x = w["embed"][tok].copy()
    for l in range(m.n_layers):
        h = rms_norm(x, w["g_enc_attn"][l], m.norm_eps)
        q = h @ w["wq"][l].T
        k = h @ w["wk"][l].T
        v = h @ w["wv"][l].T
        st.enc_k[l].extend(list(k))
        st.enc_v[l].extend(list(v))
        K = np.array(st.enc_k[l])
        V = np.array(st.enc_v[l])
        x = x + causal_attention(q, K, V, m.n_heads, t0) @ w["wo"][l].T
        x = x + m.ffn(l, rms_norm(x, w["g_enc_ffn"][l], m.norm_eps))
    e = rms_norm(x, w["g_enc_final"], m.norm_eps)
    st.e.extend(list(e))
    for g in range(m.mem_groups):
        st.mem_k[g].extend(list(e @ w["wkm"][g].T))
        st.mem_v[g].extend(list(e @ w["wvm"][g].T))
    return e


# ---------------------------------------------------------------------------
# Decoder transition
# ---------------------------------------------------------------------------

def decoder_step(m: OracleModel, st: OracleState) -> np.ndarray:
    """One recurrent transition H_{t-1} -> H_t at position t = t_dec + 1.

    Requires the encoder to have produced e_t and memory row t.  Returns s_t.
    """
    w = m.w
    t = st.t_dec                        # 0-based index of the current position
    if t >= st.t_enc:
        raise ValueError("decoder would run ahead of the encoder")
    e_t = st.e[t]
    s_prev = st.s
    # Gated merge of e_t with the previous recurrent output.
    f = w["w_fb"] @ s_prev
    gate = sigmoid(w["w_ge"] @ e_t + w["w_gs"] @ s_prev + w["b_g"])
    y = gate * e_t + (1.0 - gate) * f
    for l in range(m.n_layers):
        # Causal sliding-window self-attention over the layer's cache + current entry.
        h = rms_norm(y, w["g_dec_self"][l], m.norm_eps)
        q = w["wq"][l] @ h
        k = w["wk"][l] @ h
        v = w["wv"][l] @ h
        cache = st.dec_cache[l]
        keys = np.array([kv[0] for kv in cache] + [k])
        vals = np.array([kv[1] for kv in cache] + [v])
        y = y + w["wo"][l] @ attend(q, keys, vals, m.n_heads)
        # Cross-attention from the current position to memory entries 1..t.
        h = rms_norm(y, w["g_dec_cross"][l], m.norm_eps)
        g = m.group_of(l)
        MK = np.array(st.mem_k[g][: t + 1])
        MV = np.array(st.mem_v[g][: t + 1])
        y = y + w["wox"][l] @ attend(w["wqx"][l] @ h, MK, MV, m.n_heads)
        # FFN (tied with encoder layer l).
        y = y + m.ffn(l, rms_norm(y, w["g_dec_ffn"][l], m.norm_eps))
        # Window bookkeeping: keep at most W-1 past entries.
        cache.append((k, v))
        while len(cache) > m.window - 1:
            cache.pop(0)
    st.s = rms_norm(y, w["g_dec_final"], m.norm_eps)
    st.t_dec += 1
    st.depth += m.n_layers
    return st.s


def decode(m: OracleModel, st: OracleState, n: int) -> np.ndarray:
    """Run ``n`` decoder transitions; returns S [n, d]."""
    out = np.empty((n, m.d_model), dtype=F64)
    for i in range(n):
        out[i] = decoder_step(m, st)
    return out


def logits(m: OracleModel, S: np.ndarray) -> np.ndarray:
    """Next-token logits read from s_t: W_out s_t (token-parallel, off the loop)."""
    return S @ m.w["w_out"].T


def score_actions(w_out: np.ndarray, S: np.ndarray, actions: Sequence[int],
                  behaviour_logp: Optional[Sequence[float]] = None, temperature: float = 1.0
                  ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Score each action under the current policy ([FI] model-RL co-design paragraph: the
    trainer rebuilds the states under the current weights, scores every action, and the
    recorded behaviour log-probability is the denominator of the importance ratio).

    Row i: z = (W_out s_i) / temperature;  logp_i = z[a_i] - log sum_v exp(z_v)
    (the log-sum-exp taken with its maximum subtracted);  ratio_i = exp(logp_i - behaviour_i).
    Reading: the current policy is the full softmax at the given temperature; any
    truncation the sampler used lives in the behaviour log-probabilities only.
    """
    S = np.asarray(S, dtype=F64)
    Z = (S @ np.asarray(w_out, dtype=F64).T) / float(temperature)
    logp = np.empty(S.shape[0], dtype=F64)
    for i, a in enumerate(actions):
        z = Z[i]
        zmax = z.max()
        lse = zmax + math.log(float(np.exp(z - zmax).sum()))
        logp[i] = z[int(a)] - lse
    ratio = None
    if behaviour_logp is not None:
        ratio = np.exp(logp - np.asarray(behaviour_logp, dtype=F64))
    return logp, ratio


def sample_tokens(logits: np.ndarray, uniforms: Sequence[float], temperature: float = 1.0, top_k: int = 0,
                  top_p: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Draw the next token of each row and record its behaviour log-probability under the
    distribution actually sampled ([FI] model-RL co-design paragraph: the sampler's
    log-probability is what the trainer's ratio divides by).

    Row i with uniform u_i in [0, 1):
      z = logits_i / temperature;
      candidates ranked by (larger z first, then smaller token id);
      top-k (k > 0 and k < V): keep the first k of that ranking;
      top-p (p < 1): keep the shortest prefix of the ranking whose mass, renormalised over the
        top-k survivors, reaches p (a candidate stays while the mass before it is below p);
      the kept tokens, taken in increasing id, partition [0, 1) in proportion to exp(z):
        the drawn token is the first whose cumulative share exceeds u_i;
      logp_i = z[drawn] - log sum_{kept} exp(z).
    Readings: truncation is applied top-k first, then top-p; ties are broken by token id;
    the uniforms are inputs, so the draw is a deterministic function of them.
    """
    Z = np.asarray(logits, dtype=F64) / float(temperature)
    n, V = Z.shape
    tok = np.empty(n, dtype=np.int64)
    logp = np.empty(n, dtype=F64)
    for i in range(n):
        z = Z[i]
        rank = np.lexsort((np.arange(V), -z))          # primary key -z, then id
        k = V if top_k <= 0 or top_k >= V else int(top_k)
        cand = rank[:k]
        zmax = z[cand[0]]
        if top_p < 1.0:
            w = np.exp(z[cand] - zmax)
            need = float(top_p) * float(w.sum())
            cum, keep = 0.0, 0
            for wj in w:
                if keep > 0 and cum >= need:
                    break
                cum += float(wj)
                keep += 1
            cand = cand[:keep]
        ids = np.sort(cand)
        w_ids = np.exp(z[ids] - zmax)
        total = float(w_ids.sum())
        target = float(uniforms[i]) * total
        pick, cum = int(ids[-1]), 0.0
        for v, wv in zip(ids, w_ids):
            cum += float(wv)
            if cum > target:
                pick = int(v)
                break
        tok[i] = pick
        logp[i] = z[pick] - zmax - math.log(total)
    return tok, logp


# ---------------------------------------------------------------------------
# Schedules
# ---------------------------------------------------------------------------

def replay(m: OracleModel, tokens: Sequence[int], t_limit: Optional[int] = None
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Exact current-policy replay of one sequence from H_0.

    Rebuilds encoder memory, every window cache and the recurrent output from
    the start under the given parameters ([FI] model-RL co-design principle;
    [AL] §四).  ``t_limit`` replays only the first t_limit positions, which by
    causality equals the first t_limit rows of the full replay.
    Returns (S [T, d], logits [T, V]).
    """
    tok = np.asarray(tokens)
    if t_limit is not None:
        tok = tok[:t_limit]
    st = init_state(m)
    encode(m, st, tok)
    S = decode(m, st, len(tok))
    return S, logits(m, S)


def step(m: OracleModel, st: OracleState, token: int) -> Tuple[np.ndarray, np.ndarray]:
    """Incremental generation step: encode one token, one transition, logits."""
    encode(m, st, [int(token)])
    s = decoder_step(m, st)
    return s, logits(m, s[None, :])[0]


def replay_batch(m: OracleModel, tokens: np.ndarray, seqs: Optional[Sequence[int]] = None,
                 t_limit: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """``replay`` for several independent sequences (rows of ``tokens``)."""
    seqs = list(range(tokens.shape[0])) if seqs is None else list(seqs)
    S_all, Z_all = [], []
    for b in seqs:
        S, Z = replay(m, tokens[b], t_limit)
        S_all.append(S)
        Z_all.append(Z)
    return np.stack(S_all), np.stack(Z_all)
