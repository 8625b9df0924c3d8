"""Seeded synthetic inputs: weights, token ids, and bf16 rounding of inputs.

Nothing here evaluates the model.  The generators draw parameters and token
ids from numpy's PCG64 ``default_rng`` in a fixed canonical order so that the
oracle and the HIP path consume bit-identical inputs.

Weight recipe: every matrix, the embedding E, the head W_out and the learned
start state s* are N(0, 0.02^2) draws (float32 ``standard_normal`` * 0.02);
RMSNorm gains are 1 and the gate bias b_g is 0.  In bf16 mode each draw is
rounded to bf16 (round-to-nearest-even) once, here, and both sides use the
rounded values (held as float32, which represents every bf16 value exactly).

Token recipe: int32 ids, either uniform on [0, V) or Zipf(1.1) on the finite
support [0, V) with P(k) proportional to (k+1)^-1.1, drawn by inverse CDF.
"""
from __future__ import annotations

from typing import Dict, Iterator, List, Tuple

import numpy as np

from .configs import ModelConfig

# Canonical parameter order.  "normal" tensors are drawn in this order from one
# generator; "ones"/"zeros" tensors consume no random numbers.
PARAM_ORDER: Tuple[str, ...] = (
    "embed", "w_out", "s_star", "w_ge", "w_gs", "w_fb", "b_g",
    "wq", "wk", "wv", "wo",
    "ffn_w1", "ffn_w2",                     # GELU FFN: W_2 gelu(W_1 h)
    "ffn_gate", "ffn_up", "ffn_down",       # SwiGLU FFN: W_down(silu(W_gate h) * W_up h)
    "wqx", "wox", "wkm", "wvm",
    "g_enc_attn", "g_enc_ffn", "g_enc_final",
    "g_dec_self", "g_dec_cross", "g_dec_ffn", "g_dec_final",
)


def param_shapes(cfg: ModelConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, init) for every parameter of ``cfg`` in canonical order.

    Matrices are [out, in] row-major (y = W x).  Per-layer tensors carry a
    leading L axis, the memory projections a leading G axis.
    """
    V, d, L, F, G = cfg.vocab, cfg.d_model, cfg.n_layers, cfg.ffn_dim, cfg.mem_groups
    out: List[Tuple[str, Tuple[int, ...], str]] = []
    for name in PARAM_ORDER:
        if name in ("embed", "w_out"):
            out.append((name, (V, d), "normal"))
        elif name == "s_star":
            out.append((name, (d,), "normal"))
        elif name in ("w_ge", "w_gs", "w_fb"):
            out.append((name, (d, d), "normal"))
        elif name == "b_g":
            out.append((name, (d,), "zeros"))
        elif name in ("wq", "wk", "wv", "wo", "wqx", "wox"):
            out.append((name, (L, d, d), "normal"))
        elif name == "ffn_w1":
            if cfg.ffn_kind == "gelu":
                out.append((name, (L, F, d), "normal"))
        elif name == "ffn_w2":
            if cfg.ffn_kind == "gelu":
                out.append((name, (L, d, F), "normal"))
        elif name in ("ffn_gate", "ffn_up"):
            if cfg.ffn_kind == "swiglu":
                out.append((name, (L, F, d), "normal"))
        elif name == "ffn_down":
            if cfg.ffn_kind == "swiglu":
                out.append((name, (L, d, F), "normal"))
        elif name in ("wkm", "wvm"):
            out.append((name, (G, d, d), "normal"))
        elif name in ("g_enc_attn", "g_enc_ffn", "g_dec_self", "g_dec_cross", "g_dec_ffn"):
            out.append((name, (L, d), "ones"))
        elif name in ("g_enc_final", "g_dec_final"):
            out.append((name, (d,), "ones"))
        else:  # pragma: no cover - PARAM_ORDER and this table are kept together
            raise KeyError(name)
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Inputs are finite (no NaN/Inf handling needed for synthetic draws).
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def iter_weights(cfg: ModelConfig, seed: int) -> Iterator[Tuple[str, np.ndarray]]:
    """Yield (name, float32 array) in canonical order (streams large models)."""
    rng = np.random.default_rng(seed)
    for name, shape, init in param_shapes(cfg):
        if init == "normal":
            w = rng.standard_normal(shape, dtype=np.float32)
            w *= np.float32(0.02)
            if cfg.dtype == "bf16":
                w = bf16_round(w)
        elif init == "ones":
            w = np.ones(shape, dtype=np.float32)
        else:
            w = np.zeros(shape, dtype=np.float32)
        yield name, w


def make_weights(cfg: ModelConfig, seed: int) -> Dict[str, np.ndarray]:
    return dict(iter_weights(cfg, seed))


def perturb_untied(weights: Dict[str, np.ndarray], cfg: ModelConfig, seed: int,
                   gate_bias_std: float = 1.0) -> Dict[str, np.ndarray]:
    """Copy of ``weights`` with RMSNorm gains ~ U(0.5, 1.5) and b_g ~ N(0, std^2).

    Used by tests so that parameters which the default init leaves at 1 or 0
    are exercised (a gain applied to the wrong sub-block then shows up).
    """
    rng = np.random.default_rng(seed)
    out = dict(weights)
    for name, shape, init in param_shapes(cfg):
        if init == "ones":
            g = rng.uniform(0.5, 1.5, size=shape).astype(np.float32)
            out[name] = bf16_round(g) if cfg.dtype == "bf16" else g
        elif name == "b_g":
            b = (rng.standard_normal(shape) * gate_bias_std).astype(np.float32)
            out[name] = bf16_round(b) if cfg.dtype == "bf16" else b
    return out


def make_tokens(vocab: int, batch: int, seq_len: int, dist: str, seed: int) -> np.ndarray:
    """int32 token ids [batch, seq_len]."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        return rng.integers(0, vocab, size=(batch, seq_len), dtype=np.int64).astype(np.int32)
    if dist.startswith("zipf"):
        a = float(dist[4:]) if len(dist) > 4 else 1.1
        pmf = (np.arange(1, vocab + 1, dtype=np.float64)) ** (-a)
        cdf = np.cumsum(pmf)
        cdf /= cdf[-1]
        u = rng.random(size=(batch, seq_len))
        ids = np.searchsorted(cdf, u, side="right")
        return np.minimum(ids, vocab - 1).astype(np.int32)
    raise ValueError(f"unknown token distribution {dist!r}")
