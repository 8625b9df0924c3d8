"""rlt_decoder_replay_noalloc (decoder replay whose scratch is the library's static per-GPU
array, for callers that cannot allocate) against rlt_decoder_replay, through the C ABI.

Two calls in a row on one GPU, the second with a smaller batch and sequence, so the second
call runs on the contents the first left in the shared array; both must equal the ordinary
entry point bit for bit (same kernels, same summation order).
"""
import numpy as np
import pytest

from workloads import ModelConfig, make_tokens, make_weights, perturb_untied

torch = pytest.importorskip("torch")
import cross_token_recurrent_amd as rlt  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load_library()
    return torch.device("cuda:0")


def _replay(model, tokens, dev, fn):
    B, T = tokens.shape
    state = rlt.State(model, B, T)
    rlt.rlt_encoder_forward(model, state, torch.from_numpy(tokens).to(dev))
    S = torch.empty(B, T, model.d_model, dtype=torch.float32, device=dev)
    fn(model, state, T, S)
    torch.cuda.synchronize()
    assert state.position()[:2] == (T, T)
    assert state.device_error() == 0
    return S.cpu().numpy()


# (config, path): the weight-streaming batched step (bf16, d = 256: fragment-major operands, norm
# partial sums, cross-attention arrival counters) and the persistent decoder (no scratch at all)
CASES = [
    (dict(vocab=128, d_model=256, n_heads=4, n_layers=2, ffn_dim=512, ffn_kind="swiglu", window=6, mem_groups=2,
          dtype="bf16"), 2),
    (dict(vocab=97, d_model=64, n_heads=4, n_layers=2, ffn_dim=128, ffn_kind="gelu", window=4, mem_groups=1,
          dtype="fp32"), 1),
]


@pytest.mark.parametrize("over,path", CASES, ids=["batched", "persistent"])
def test_noalloc_matches_replay_twice(dev, over, path):
    cfg = ModelConfig(**over)
    w = perturb_untied(make_weights(cfg, 301), cfg, 302)
    model = rlt.Model(cfg, w, device=dev)
    model.set_decoder_path(path)
    for B, T, seed in ((6, 40, 303), (3, 20, 304)):
        tok = make_tokens(cfg.vocab, B, T, "uniform", seed)
        ref = _replay(model, tok, dev, rlt.rlt_decoder_replay)
        got = _replay(model, tok, dev, rlt.rlt_decoder_replay_noalloc)
        print(f"  {path=} B={B} T={T}: max |noalloc - replay| = {np.abs(got - ref).max():.3e}", flush=True)
        assert np.array_equal(got, ref)


def test_noalloc_rejects_scratch_beyond_its_size(dev):
    cfg = ModelConfig(vocab=64, d_model=1024, n_heads=16, n_layers=1, ffn_dim=64, ffn_kind="gelu", window=2,
                      mem_groups=1, dtype="bf16")
    model = rlt.Model(cfg, make_weights(cfg, 305), device=dev)
    B, T = 2048, 64                      # about 140 MB of batched-decoder scratch
    state = rlt.State(model, B, T)
    tok = make_tokens(cfg.vocab, B, 1, "uniform", 306)
    rlt.rlt_encoder_forward(model, state, torch.from_numpy(tok).to(dev))
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_decoder_replay_noalloc(model, state, 1)
    assert ei.value.name == "RLT_ERR_UNSUPPORTED"
    assert state.position()[:2] == (1, 0)
    torch.cuda.synchronize()
