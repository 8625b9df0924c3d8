"""Prefix snapshots (rlt_state_save / rlt_state_restore) on the GPU.

A state saved after a prefix and restored, into a fresh state, a longer one or one that was
used before, must continue exactly as the uninterrupted state does (bitwise), and the
continuation must match the oracle's replay of the whole sequence ([FI] serving paragraph:
a conversation's state is kept and continued, and is only valid under its weights version).
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_helpers import check, oracle_replay
from workloads import ModelConfig, make_tokens, make_weights

torch = pytest.importorskip("torch")
import cross_token_recurrent_amd as rlt  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load_library()
    return torch.device("cuda:0")


def _cfg(dtype="fp32", **kw):
    base = dict(vocab=128, d_model=64, n_heads=4, n_layers=2, ffn_dim=128, ffn_kind="gelu", window=4,
                mem_groups=2, dtype=dtype)
    base.update(kw)
    return ModelConfig(**base)


def _steps(model, state, tt, t0, n):
    """n incremental steps from position t0: (S [B, n, d], Z [B, n, V])."""
    B = tt.shape[0]
    S = torch.empty(B, n, model.d_model, device=tt.device)
    Z = torch.empty(B, n, model.vocab, device=tt.device)
    for i in range(n):
        s = torch.empty(B, model.d_model, device=tt.device)
        z = torch.empty(B, model.vocab, device=tt.device)
        rlt.rlt_decoder_step(model, state, tt[:, t0 + i].contiguous(), s, z)
        S[:, i], Z[:, i] = s, z
    torch.cuda.synchronize()
    return S.cpu().numpy(), Z.cpu().numpy()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_snapshot_continuation_is_exact(dev, dtype):
    cfg = _cfg(dtype)
    w = make_weights(cfg, 61)
    B, P, n = 3, 20, 8
    tok = make_tokens(cfg.vocab, B, P + n, "uniform", 62)
    tt = torch.from_numpy(tok).to(dev)
    model = rlt.Model(cfg, w, device=dev)
    a = rlt.State(model, B, P + n, keep_encoder_cache=True)
    rlt.rlt_encoder_forward(model, a, tt[:, :P].contiguous())
    rlt.rlt_decoder_replay(model, a, P)
    snap = rlt.rlt_state_save(model, a)
    torch.cuda.synchronize()
    assert snap.numel() == rlt.rlt_state_snapshot_bytes(a)
    S_a, Z_a = _steps(model, a, tt, P, n)

    # into a longer fresh state
    b = rlt.State(model, B, 3 * (P + n), keep_encoder_cache=True)
    rlt.rlt_state_restore(model, b, snap)
    assert b.position()[:2] == (P, P)
    S_b, Z_b = _steps(model, b, tt, P, n)
    assert np.array_equal(S_a, S_b) and np.array_equal(Z_a, Z_b)

    # into a state that ran a longer, different sequence before
    c = rlt.State(model, B, P + n, keep_encoder_cache=True)
    other = torch.from_numpy(make_tokens(cfg.vocab, B, P + n, "uniform", 63)).to(dev)
    rlt.rlt_encoder_forward(model, c, other)
    rlt.rlt_decoder_replay(model, c, P + n)
    rlt.rlt_state_restore(model, c, snap)
    S_c, Z_c = _steps(model, c, tt, P, n)
    assert np.array_equal(S_a, S_c) and np.array_equal(Z_a, Z_c)

    _, Z_ref = oracle_replay(cfg, w, tok)
    check(f"{dtype} continued logits", Z_b, Z_ref[:, P:], dtype)


def test_snapshot_with_encoder_ahead_and_without_cache(dev):
    """t_dec < t_enc at the snapshot (the decoder finishes after the restore); a snapshot
    without an encoder cache restores into a state without one and replays the rest."""
    cfg = _cfg(window=3, mem_groups=1)
    w = make_weights(cfg, 64)
    B, T = 2, 24
    tok = make_tokens(cfg.vocab, B, T, "uniform", 65)
    tt = torch.from_numpy(tok).to(dev)
    model = rlt.Model(cfg, w, device=dev)
    a = rlt.State(model, B, T)
    rlt.rlt_encoder_forward(model, a, tt)
    rlt.rlt_decoder_replay(model, a, T - 7)
    snap = rlt.rlt_state_save(model, a)
    torch.cuda.synchronize()
    S_a = torch.empty(B, 7, cfg.d_model, device=dev)
    rlt.rlt_decoder_replay(model, a, 7, S_a)
    b = rlt.State(model, B, T)
    rlt.rlt_state_restore(model, b, snap)
    assert b.position()[:2] == (T, T - 7)
    S_b = torch.empty(B, 7, cfg.d_model, device=dev)
    rlt.rlt_decoder_replay(model, b, 7, S_b)
    torch.cuda.synchronize()
    assert torch.equal(S_a, S_b)


def test_snapshot_of_fresh_state_is_h0(dev):
    cfg = _cfg()
    w = make_weights(cfg, 66)
    model = rlt.Model(cfg, w, device=dev)
    B, T = 2, 12
    tt = torch.from_numpy(make_tokens(cfg.vocab, B, T, "uniform", 67)).to(dev)
    a = rlt.State(model, B, T)
    snap = rlt.rlt_state_save(model, a)
    torch.cuda.synchronize()
    b = rlt.State(model, B, T)
    rlt.rlt_encoder_forward(model, b, tt)
    rlt.rlt_decoder_replay(model, b, T)
    rlt.rlt_state_restore(model, b, snap)
    assert b.position()[:2] == (0, 0)
    out = []
    for st in (a, b):
        S = torch.empty(B, T, cfg.d_model, device=dev)
        rlt.rlt_encoder_forward(model, st, tt)
        rlt.rlt_decoder_replay(model, st, T, S)
        out.append(S)
    torch.cuda.synchronize()
    assert torch.equal(out[0], out[1])


def test_snapshot_errors(dev):
    cfg = _cfg()
    w = make_weights(cfg, 68)
    model = rlt.Model(cfg, w, device=dev)
    B, P = 2, 10
    tt = torch.from_numpy(make_tokens(cfg.vocab, B, P, "uniform", 69)).to(dev)
    a = rlt.State(model, B, P, keep_encoder_cache=False)
    rlt.rlt_encoder_forward(model, a, tt)
    rlt.rlt_decoder_replay(model, a, P)
    snap = rlt.rlt_state_save(model, a)
    torch.cuda.synchronize()

    def expect(name, state, buf):
        with pytest.raises(rlt.RltError) as ei:
            rlt.rlt_state_restore(model, state, buf)
        assert ei.value.name == name

    expect("RLT_ERR_INVALID", rlt.State(model, B + 1, P), snap)              # batch
    expect("RLT_ERR_CAPACITY", rlt.State(model, B, P - 1), snap)             # t_max < t_enc
    expect("RLT_ERR_NO_ENC_CACHE", rlt.State(model, B, P, keep_encoder_cache=True), snap)
    bad = snap.clone()
    bad[0] = ord("X")
    expect("RLT_ERR_INVALID", rlt.State(model, B, P), bad)                   # magic
    expect("RLT_ERR_INVALID", rlt.State(model, B, P), snap[: snap.numel() - 1].contiguous())
    import ctypes
    on_gpu = snap.to(dev)
    lib = rlt.load_library()
    target = rlt.State(model, B, P)
    rc = lib.rlt_state_restore(model.handle, target.handle, ctypes.c_void_p(on_gpu.data_ptr()), on_gpu.numel(), None)
    assert rlt.RltError(rc, "").name == "RLT_ERR_INVALID"                    # device memory
    small = torch.empty(snap.numel() - 1, dtype=torch.uint8)
    with pytest.raises(rlt.RltError):
        rlt.rlt_state_save(model, a, small)
    other = rlt.Model(_cfg(window=5), make_weights(_cfg(window=5), 70), device=dev)
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_state_restore(other, rlt.State(other, B, P), snap)          # configuration
    assert ei.value.name == "RLT_ERR_INVALID"
    model.update_weights(make_weights(cfg, 71), version=2)
    expect("RLT_ERR_STALE_STATE", rlt.State(model, B, P), snap)             # weights version
