"""C ABI checks that need no GPU: the library loads, exports every entry point the
header declares, its canonical parameter table agrees with the input generators, and
configuration errors are reported before anything touches a device."""
import ctypes
import re

import numpy as np
import pytest

import cross_token_recurrent_amd as rlt
from cross_token_recurrent_amd.rlt import HEADER_PATH, header_symbols, load_library, make_config, rlt_config
from workloads import CONFIGS, ModelConfig, param_shapes


def test_library_exports_every_header_symbol():
    lib = load_library()
    syms = header_symbols()
    assert len(syms) >= 20
    for s in syms:
        assert hasattr(lib, s), f"librlt.so does not export {s}"
    assert lib.rlt_version_string().startswith(b"librlt")


def test_header_declares_extern_c_and_error_codes():
    text = open(HEADER_PATH).read()
    assert 'extern "C"' in text
    for code in ("RLT_ERR_INVALID", "RLT_ERR_UNSUPPORTED", "RLT_ERR_CAPACITY", "RLT_ERR_ORDER",
                 "RLT_ERR_STALE_STATE", "RLT_ERR_NO_ENC_CACHE", "RLT_ERR_HIP"):
        assert re.search(rf"#define {code} \(-\d\)", text)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_param_table_matches_generators(name):
    cfg = CONFIGS[name].model
    table = rlt.rlt_param_table(make_config(cfg))
    shapes = param_shapes(cfg)
    assert list(table) == [n for n, _, _ in shapes]
    off = 0
    for n, shape, _ in shapes:
        o, numel = table[n]
        assert o == off and numel == int(np.prod(shape)), n
        off += numel


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_bytes(name):
    cfg = CONFIGS[name].model
    nbytes = rlt.rlt_model_workspace_bytes(make_config(cfg))
    esz = 2 if cfg.dtype == "bf16" else 4
    nparams = sum(int(np.prod(s)) for _, s, _ in param_shapes(cfg))
    # bf16 models with d >= 256 also hold fragment-major copies of the decoder weights and the head
    assert nparams * esz <= nbytes <= nparams * 4 + cfg.vocab * cfg.d_model * 2 + (1 << 20)


def _cfg(**kw):
    base = dict(vocab=64, d_model=64, n_heads=4, n_layers=2, ffn_dim=128, ffn_kind="gelu", window=4,
                mem_groups=1, dtype="bf16")
    base.update(kw)
    return make_config(ModelConfig(**base))


@pytest.mark.parametrize("bad,code", [
    (dict(window=0), "RLT_ERR_INVALID"),
    (dict(n_heads=3), "RLT_ERR_UNSUPPORTED"),        # d % H != 0
    (dict(mem_groups=3, n_layers=4), "RLT_ERR_UNSUPPORTED"),  # G not in {1, L}
    (dict(d_model=96, n_heads=6), "RLT_ERR_UNSUPPORTED"),     # d % 64
    (dict(n_heads=64), "RLT_ERR_UNSUPPORTED"),       # head_dim 1
    (dict(ffn_dim=100), "RLT_ERR_UNSUPPORTED"),
    (dict(vocab=0), "RLT_ERR_INVALID"),
])
def test_config_validation_before_any_device_call(bad, code):
    cfg = _cfg(**bad)
    with pytest.raises(rlt.RltError) as ei:
        rlt.rlt_model_workspace_bytes(cfg)
    assert ei.value.name == code
    # model creation rejects the same configuration before touching the device
    lib = load_library()
    h = ctypes.c_void_p()
    rc = lib.rlt_model_create(ctypes.byref(cfg), ctypes.c_void_p(256), 1, ctypes.c_void_p(256), 1 << 30, None,
                              ctypes.byref(h))
    assert rlt.rlt.ERRORS[rc] == code
    assert lib.rlt_last_error()


def test_bad_ffn_kind_dtype_eps():
    for field, value in (("ffn_kind", 7), ("dtype", 5), ("norm_eps", 0.0)):
        cfg = _cfg()
        setattr(cfg, field, value)
        with pytest.raises(rlt.RltError) as ei:
            rlt.rlt_model_workspace_bytes(cfg)
        assert ei.value.name == "RLT_ERR_INVALID"


def test_null_and_alignment_arguments_rejected():
    lib = load_library()
    cfg = _cfg()
    h = ctypes.c_void_p()
    assert lib.rlt_model_create(ctypes.byref(cfg), None, 1, ctypes.c_void_p(256), 1 << 30, None, ctypes.byref(h)) == -1
    assert lib.rlt_model_create(ctypes.byref(cfg), ctypes.c_void_p(256), 1, ctypes.c_void_p(257), 1 << 30, None,
                                ctypes.byref(h)) == -1
    assert lib.rlt_model_create(ctypes.byref(cfg), ctypes.c_void_p(256), 1, ctypes.c_void_p(256), 16, None,
                                ctypes.byref(h)) == -1
    assert b"too small" in lib.rlt_last_error()
    assert lib.rlt_encoder_forward(None, None, None, 1, None) == -1
    assert lib.rlt_decoder_replay(None, None, 1, None, None) == -1
    assert lib.rlt_state_reset(None, None, None) == -1


def test_binding_rejects_host_tensors_before_the_library():
    """The binding checks its tensors itself (active under python -O): host memory, a wrong
    dtype or a wrong size never reaches a kernel."""
    import torch
    with pytest.raises(ValueError, match="device memory"):
        rlt.rlt_sample_tokens(torch.zeros(2, 10), torch.zeros(2))
    with pytest.raises(ValueError, match="device memory"):
        rlt.Model(CONFIGS["tiny"].model, {}, device="cpu")
