"""Shared helpers of the GPU parity tests: oracle runs (in worker processes that never
touch the GPU) and the comparison metrics of the two precision modes.

Tolerances: fp32 mode, max |gpu - oracle| <= 1e-4 over every element of s_t and
logits_t at every t; bf16 mode (bf16 storage, fp32 accumulate), per row (b, t):
||gpu - oracle||_2 / ||oracle||_2 <= 3e-2 for s_t (length d) and logits_t (length V).
"""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
from typing import Dict, Optional, Sequence

import numpy as np

FP32_MAX_ABS = 1e-4
BF16_ROW_REL = 3e-2


def _oracle_one(args):
    cfg, weights, tok, t_limit = args
    import oracle
    m = oracle.OracleModel.from_config(cfg, weights)
    return oracle.replay(m, tok, t_limit)


def oracle_replay(cfg, weights: Dict[str, np.ndarray], tokens: np.ndarray, seqs: Optional[Sequence[int]] = None,
                  t_limit: Optional[int] = None, workers: Optional[int] = None):
    """(S [nb, T, d], logits [nb, T, V]) for the chosen sequences, computed by the oracle
    in spawned worker processes (they import only numpy/scipy and the oracle)."""
    seqs = list(range(tokens.shape[0])) if seqs is None else list(seqs)
    jobs = [(cfg, weights, tokens[b], t_limit) for b in seqs]
    if workers is None:
        workers = min(len(jobs), 8, len(os.sched_getaffinity(0)))
    if workers <= 1 or len(jobs) == 1:
        out = [_oracle_one(j) for j in jobs]
    else:
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers) as pool:
            out = pool.map(_oracle_one, jobs)
    return np.stack([o[0] for o in out]), np.stack([o[1] for o in out])


def row_rel(x: np.ndarray, ref: np.ndarray) -> np.ndarray:
    num = np.linalg.norm(x.astype(np.float64) - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.maximum(den, 1e-30)


def check(name: str, gpu: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """Assert the mode's tolerance; returns the measured figure."""
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{name}: non-finite GPU values"
    if dtype == "fp32":
        err = float(np.abs(gpu.astype(np.float64) - ref).max())
        assert err <= FP32_MAX_ABS, f"{name}: max abs error {err:.3e} > {FP32_MAX_ABS}"
    else:
        rr = row_rel(gpu, ref)
        err = float(rr.max())
        assert err <= BF16_ROW_REL, f"{name}: worst row relative error {err:.3e} > {BF16_ROW_REL} at {np.unravel_index(rr.argmax(), rr.shape)}"
    print(f"  {name}: {'max-abs' if dtype == 'fp32' else 'max row-rel'} = {err:.3e}", flush=True)
    sys.stdout.flush()
    return err


def _oracle_bptt_one(args):
    cfg, weights, tok, mask, detach = args
    import oracle
    m = oracle.OracleModel.from_config(cfg, weights)
    loss, grads, _ = oracle.bptt(m, tok, mask, detach)
    return loss, grads


def oracle_bptt(cfg, weights: Dict[str, np.ndarray], tokens: np.ndarray, masks: Optional[np.ndarray] = None,
                detach=(), seqs: Optional[Sequence[int]] = None, workers: Optional[int] = None):
    """(per-sequence losses [nb], summed gradients {name: array}) of the fp64 backward oracle over
    the chosen sequences, computed in spawned worker processes."""
    seqs = list(range(tokens.shape[0])) if seqs is None else list(seqs)
    # masks, when given, has one row per chosen sequence
    jobs = [(cfg, weights, tokens[b], None if masks is None else masks[i], tuple(detach)) for i, b in enumerate(seqs)]
    if workers is None:
        workers = min(len(jobs), 8, len(os.sched_getaffinity(0)))
    if workers <= 1 or len(jobs) == 1:
        out = [_oracle_bptt_one(j) for j in jobs]
    else:
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers) as pool:
            out = pool.map(_oracle_bptt_one, jobs)
    grads = {k: sum(o[1][k] for o in out) for k in out[0][1]}
    return np.array([o[0] for o in out]), grads
