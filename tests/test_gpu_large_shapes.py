"""GPU parity at the large workloads' own kernel shapes, checked at every position.

The full-depth large workloads cannot be replayed by the fp64 oracle over their whole
length (hours per sequence), so these tests keep every dimension that selects a kernel
instance or a launch shape (d_model, heads, head_dim, FFN kind and width, window, memory
groups, batch, vocabulary, token distribution) and cut only the layer count to two.  The
replay is then long enough that the window ring wraps, the cross-attention memory spans
several key chunks and the encoder's causal attention runs over many key tiles, and the
sampled sequences are compared with the oracle at every position.

Pages: [FI] feinterview "普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer"
(model-RL co-design principle: replay rebuilds every state from the sequence start, so every
position must be right); [DS] deepsonar "技术拆解 009｜RLT…" §2.2 (window), §2.1 (memory).
"""
import sys
import time

import numpy as np
import pytest

from gpu_helpers import check, oracle_replay
from workloads import CONFIGS, make_tokens, make_weights, perturb_untied

torch = pytest.importorskip("torch")
import cross_token_recurrent_amd as rlt  # noqa: E402

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load_library()
    return torch.device("cuda:0")


# (workload, layers kept, T replayed, sequences compared).
#   300m:  B=512 (B*H = 8192 pairs: the one-wave window kernel), W=128 so the ring of 127 entries
#          wraps twice by t=300, two 256-key memory chunks, G = L.
#   ref48: B=64, d=2048, head_dim 128 (the weight-streaming products with two column blocks per
#          workgroup for QKV, the 8-wave window kernel), W=256 so the ring of 255 entries wraps
#          by t=300, two memory chunks, five 64-key encoder tiles, G = 1.
#   long:  B=16 (one 16-row block in every product), W=512 so the ring of 511 wraps three times
#          by t=2100, nine memory chunks, G = 1.
SHAPES = [
    ("300m", 2, 300, [0, 511]),
    ("ref48", 2, 300, [0, 63]),
    ("long", 2, 2100, [0]),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,layers,T,seqs", SHAPES, ids=[s[0] for s in SHAPES])
def test_large_shape_two_layers_every_position(dev, name, layers, T, seqs):
    wl = CONFIGS[name]
    cfg = wl.model.with_(n_layers=layers, mem_groups=layers if wl.model.mem_groups > 1 else 1)
    B = wl.batch
    log(f"  [{name} x{layers} layers] B={B} d={cfg.d_model} H={cfg.n_heads} F={cfg.ffn_dim} W={cfg.window} "
        f"G={cfg.mem_groups} T={T}, sequences {seqs}")
    w = perturb_untied(make_weights(cfg, wl.weight_seed), cfg, 200 + wl.index, gate_bias_std=0.5)
    tok = make_tokens(cfg.vocab, B, wl.seq_len, wl.token_dist, wl.token_seed)[:, :T].copy()
    model = rlt.Model(cfg, w, device=dev)
    assert model.decoder_path(T) == 2
    state = rlt.State(model, B, T)
    t0 = time.time()
    S, _ = rlt.replay(model, state, torch.from_numpy(tok).to(dev), with_logits=False)
    Z = rlt.rlt_logits(model, S[seqs].contiguous())
    torch.cuda.synchronize()
    assert state.device_error() == 0
    log(f"  [{name}] GPU replay done in {time.time() - t0:.1f} s")
    S_gpu, Z_gpu = S[seqs].cpu().numpy(), Z.cpu().numpy()
    del model, state, S, Z
    torch.cuda.empty_cache()
    t0 = time.time()
    # the 2048-wide weights (about 1 GB) are not worth pickling to worker processes
    S_ref, Z_ref = oracle_replay(cfg, w, tok, seqs, workers=1 if cfg.d_model >= 2048 else None)
    log(f"  [{name}] oracle done in {time.time() - t0:.1f} s")
    check(f"{name} x{layers} s_t", S_gpu, S_ref, cfg.dtype)
    check(f"{name} x{layers} logits", Z_gpu, Z_ref, cfg.dtype)
