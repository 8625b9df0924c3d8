"""Full-BPTT backward on the GPU (``rlt_bptt``) against the fp64 backward oracle.

Tolerance (the GPU side computes in fp32): per parameter tensor, max |gpu - oracle| <=
2e-5 * max |oracle| + 1e-7, and the per-sequence losses to 1e-5 relative.  Every product
rounds to fp32 (unit roundoff 6e-8) and the chains run over T steps and 2 L sub-layers; the
measured worst case over these cases is 2.4e-6, and the bound keeps a factor of about 8 over
it while a dropped or wrong term moves a tensor by a large part of its own scale.
"""
import numpy as np
import pytest
import torch

import cross_token_recurrent_amd as rlt
from tests.gpu_helpers import oracle_bptt
from workloads import CONFIGS, ModelConfig, make_tokens, make_weights, perturb_untied

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL_REL = 2e-5


def weights_for(cfg, seed=5, scale=4.0):
    w = perturb_untied(make_weights(cfg, seed), cfg, seed + 1000, 0.5)
    return {k: (v * np.float32(scale) if k != "b_g" and not k.startswith("g_") else v) for k, v in w.items()}


def flat(cfg_c, w):
    table = rlt.rlt_param_table(cfg_c)
    total = sum(n for _, n in table.values())
    out = torch.empty(total, dtype=torch.float32)
    for name, (off, n) in table.items():
        out[off:off + n] = torch.from_numpy(np.ascontiguousarray(w[name], dtype=np.float32).reshape(-1))
    return out.to(DEV), table


def run_gpu(cfg, w, tokens, masks=None, detach=()):
    c = rlt.make_config(cfg)
    wf, table = flat(c, w)
    tok = torch.from_numpy(tokens.astype(np.int32)).to(DEV)
    mk = None if masks is None else torch.from_numpy(masks.astype(np.float32)).to(DEV)
    loss, grads = rlt.rlt_bptt(c, wf, tok, mk, detach)
    torch.cuda.synchronize()
    g = grads.cpu().numpy()
    return loss.cpu().numpy(), {k: g[off:off + n].reshape(np.shape(w[k])) for k, (off, n) in table.items()}


def compare(tag, loss, grads, ref_loss, ref_grads):
    np.testing.assert_allclose(loss, ref_loss, rtol=1e-5, atol=1e-6, err_msg=f"{tag}: loss")
    worst = 0.0
    for k, ref in ref_grads.items():
        got = grads[k].astype(np.float64)
        assert np.isfinite(got).all(), f"{tag}: {k} not finite"
        scale = float(np.abs(ref).max())
        err = float(np.abs(got - ref).max())
        rel = err / max(scale, 1e-30)
        worst = max(worst, rel if scale > 1e-6 else 0.0)
        assert err <= TOL_REL * scale + 1e-7, f"{tag}: {k} max err {err:.3e} vs scale {scale:.3e} (rel {rel:.2e})"
    print(f"{tag}: worst per-tensor max-rel error {worst:.2e}", flush=True)


def tiny_cfg(**kw):
    base = CONFIGS["tiny"].model
    return base.with_(**kw)


CASES = {
    "tiny": dict(),
    "tiny_swiglu_G=L": dict(ffn_kind="swiglu", mem_groups=2),
    "tiny_W=1": dict(window=1),
    "tiny_W>T": dict(window=80),
    "tiny_dh32": dict(n_heads=2),
    "tiny_bf16_weights": dict(dtype="bf16"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_bptt_matches_oracle(name):
    cfg = tiny_cfg(**CASES[name])
    print(f"case {name}: {cfg}", flush=True)
    B, T = 4, 64
    w = weights_for(cfg)
    if cfg.dtype == "bf16":
        from workloads.synth import bf16_round
        w = {k: bf16_round(v) for k, v in w.items()}
    tokens = make_tokens(cfg.vocab, B, T, "uniform", 11)
    loss, grads = run_gpu(cfg, w, tokens)
    ref_loss, ref_grads = oracle_bptt(cfg, w, tokens)
    compare(name, loss, grads, ref_loss, ref_grads)


@pytest.mark.parametrize("detach", [("s",), ("kv",), ("memory",), ("s", "kv", "memory")])
def test_bptt_detach_matches_oracle(detach):
    cfg = tiny_cfg(mem_groups=2)
    B, T = 2, 40
    w = weights_for(cfg, seed=7)
    tokens = make_tokens(cfg.vocab, B, T, "uniform", 12)
    print(f"detach {detach}", flush=True)
    loss, grads = run_gpu(cfg, w, tokens, detach=detach)
    ref_loss, ref_grads = oracle_bptt(cfg, w, tokens, detach=detach)
    compare(f"detach {detach}", loss, grads, ref_loss, ref_grads)


def test_bptt_sft_mask_and_ragged_lengths():
    """A mask with zeros and non-unit weights; T = 1 (nothing to predict) and T = 2."""
    cfg = tiny_cfg()
    w = weights_for(cfg, seed=9)
    rng = np.random.default_rng(3)
    B, T = 3, 37
    tokens = make_tokens(cfg.vocab, B, T, "uniform", 13)
    masks = (rng.random((B, T - 1)) < 0.6).astype(np.float64) * rng.choice([0.5, 1.0, 2.0], size=(B, T - 1))
    loss, grads = run_gpu(cfg, w, tokens, masks)
    ref_loss, ref_grads = oracle_bptt(cfg, w, tokens, masks)
    compare("sft mask", loss, grads, ref_loss, ref_grads)
    for T in (1, 2):
        tokens = make_tokens(cfg.vocab, 2, T, "uniform", 14)
        loss, grads = run_gpu(cfg, w, tokens)
        ref_loss, ref_grads = oracle_bptt(cfg, w, tokens)
        compare(f"T={T}", loss, grads, ref_loss, ref_grads)


def test_bptt_small_workload_shape_every_sequence_prefix():
    """The small workload's model shape (d=64, 4+4 layers, W=32, G=L, GELU 256, V=512) over
    T=300: past the window wrap, every position and sequence."""
    cfg = CONFIGS["small"].model
    w = weights_for(cfg, seed=2, scale=2.0)
    from workloads.synth import bf16_round
    w = {k: bf16_round(v) for k, v in w.items()}
    tokens = make_tokens(cfg.vocab, 3, 300, "uniform", 102)
    loss, grads = run_gpu(cfg, w, tokens)
    ref_loss, ref_grads = oracle_bptt(cfg, w, tokens)
    compare("small shape T=300", loss, grads, ref_loss, ref_grads)


def test_bptt_errors():
    cfg = tiny_cfg()
    c = rlt.make_config(cfg)
    w = weights_for(cfg)
    wf, _ = flat(c, w)
    tok = torch.zeros((2, 8), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        rlt.rlt_bptt(c, wf, tok, detach=("everything",))
    big = rlt.make_config(cfg.with_(d_model=512, n_heads=8, ffn_dim=512))
    with pytest.raises(rlt.RltError):
        rlt.rlt_bptt_workspace_bytes(big, 2, 8)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(rlt.RltError):
        rlt.rlt_bptt(c, wf, tok, workspace=ws)
    bad = tok.clone()
    bad[1, 3] = cfg.vocab
    loss, _ = rlt.rlt_bptt(c, wf, bad)
    torch.cuda.synchronize()
    assert torch.isnan(loss).all()


def test_bptt_small_workload_full_size_sampled_sequences():
    """The small workload at its full size (B=64, T=1024, its own seeded weights and tokens), the
    launch configuration the bench times; the mask supervises sequences 0 and 63 only, so the
    gradient is the oracle's for those two sequences (the other 62 contribute exact zeros)."""
    wl = CONFIGS["small"]
    cfg, B, T = wl.model, wl.batch, wl.seq_len
    w = make_weights(cfg, wl.weight_seed)
    tokens = make_tokens(cfg.vocab, B, T, wl.token_dist, wl.token_seed)
    masks = np.zeros((B, T - 1))
    masks[0] = 1.0
    masks[B - 1] = 1.0
    loss, grads = run_gpu(cfg, w, tokens, masks)
    ref_loss, ref_grads = oracle_bptt(cfg, w, tokens, masks[[0, B - 1]], seqs=[0, B - 1])
    assert np.all(loss[1:B - 1] == 0.0)
    compare("small full size, sequences 0 and 63", loss[[0, B - 1]], grads, ref_loss, ref_grads)
