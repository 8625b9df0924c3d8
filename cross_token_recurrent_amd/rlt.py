"""Thin Python binding of librlt.so (argument marshalling only).

Every function named ``rlt_*`` here calls the C entry point of the same name with
device pointers taken from torch tensors and the current torch stream; all compute
runs in the HIP kernels of the library.  The classes ``Model`` and ``State`` only own
the device buffers (allocated through torch) and the C handles.

There is no fallback: if librlt.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Tuple

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librlt.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "rlt.h")

RLT_OK = 0
ERRORS = {
    -1: "RLT_ERR_INVALID", -2: "RLT_ERR_UNSUPPORTED", -3: "RLT_ERR_CAPACITY", -4: "RLT_ERR_ORDER",
    -5: "RLT_ERR_STALE_STATE", -6: "RLT_ERR_NO_ENC_CACHE", -7: "RLT_ERR_HIP",
}
FFN_KINDS = {"gelu": 0, "swiglu": 1}
DTYPES = {"fp32": 0, "bf16": 1}


class RltError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


class rlt_config(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("ffn_dim", ctypes.c_int32), ("ffn_kind", ctypes.c_int32),
                ("window", ctypes.c_int32), ("mem_groups", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("norm_eps", ctypes.c_float)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
class rlt_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float)]


_SIGS = {
    "rlt_param_count": [ctypes.POINTER(rlt_config), ctypes.POINTER(_I32), ctypes.POINTER(ctypes.c_int64)],
    "rlt_param_info": [ctypes.POINTER(rlt_config), _I32, ctypes.POINTER(ctypes.c_char_p),
                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)],
    "rlt_model_workspace_bytes": [ctypes.POINTER(rlt_config), ctypes.POINTER(ctypes.c_size_t)],
    "rlt_model_create": [ctypes.POINTER(rlt_config), _P, ctypes.c_uint64, _P, ctypes.c_size_t, _P,
                         ctypes.POINTER(_P)],
    "rlt_model_update_weights": [_P, _P, ctypes.c_uint64, _P],
    "rlt_model_get_config": [_P, ctypes.POINTER(rlt_config), ctypes.POINTER(ctypes.c_uint64)],
    "rlt_model_release": [_P],
    "rlt_state_bytes": [_P, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "rlt_state_init": [_P, _P, ctypes.c_size_t, _I32, _I32, _I32, _P, ctypes.POINTER(_P)],
    "rlt_state_reset": [_P, _P, _P],
    "rlt_state_release": [_P],
    "rlt_state_position": [_P, ctypes.POINTER(_I32), ctypes.POINTER(_I32), ctypes.POINTER(ctypes.c_uint64)],
    "rlt_state_device_error": [_P, _P, ctypes.POINTER(_I32)],
    "rlt_state_snapshot_bytes": [_P, ctypes.POINTER(ctypes.c_size_t)],
    "rlt_state_save": [_P, _P, _P, ctypes.c_size_t, _P],
    "rlt_state_restore": [_P, _P, _P, ctypes.c_size_t, _P],
    "rlt_encoder_forward": [_P, _P, _P, _I32, _P],
    "rlt_decoder_replay": [_P, _P, _I32, _P, _P],
    "rlt_decoder_replay_noalloc": [_P, _P, _I32, _P, _P],
    "rlt_decoder_step": [_P, _P, _P, _P, _P, _P],
    "rlt_logits": [_P, _P, ctypes.c_int64, _P, _P],
    "rlt_score_actions": [_P, _P, _P, ctypes.c_int64, ctypes.c_float, _P, _P, _P, _P],
    "rlt_sample_tokens": [_P, ctypes.c_int64, _I32, ctypes.POINTER(rlt_sampling), _P, _P, _P, _P],
    "rlt_decoder_step_sample": [_P, _P, _P, ctypes.POINTER(rlt_sampling), _P, _P, _P, _P, _P, _P],
    "rlt_state_load_encoder_outputs": [_P, _P, _P, _P, _P, _I32, _P],
    "rlt_state_read_encoder_outputs": [_P, _P, _I32, _I32, _P, _P, _P, _P],
    "rlt_bptt_workspace_bytes": [ctypes.POINTER(rlt_config), _I32, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "rlt_bptt": [ctypes.POINTER(rlt_config), _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, ctypes.c_size_t, _P],
    "rlt_decoder_path": [_P, _I32, ctypes.POINTER(_I32)],
    "rlt_model_set_decoder_path": [_P, _I32],
    "rlt_last_error": [],
    "rlt_version_string": [],
}
_VOID = {"rlt_model_release", "rlt_state_release"}
_STR = {"rlt_last_error", "rlt_version_string"}

_lib: Optional[ctypes.CDLL] = None


def header_symbols() -> list:
    """Entry points declared in include/rlt.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"\b(rlt_[a-z_0-9]+)\s*\(", text)))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"librlt.so not built ({path}); run `python -m cross_token_recurrent_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None if name in _VOID else (ctypes.c_char_p if name in _STR else ctypes.c_int)
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != RLT_OK:
        raise RltError(rc, load_library().rlt_last_error().decode())


def _stream(stream=None) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(cond: bool, msg: str) -> None:
    """Argument check that stays active under ``python -O`` (a pointer of the wrong kind or
    size must never reach the library)."""
    if not cond:
        raise ValueError(msg)


def _tensor(t, name: str, dtype, device, shape=None, numel=None) -> None:
    """t must be a contiguous tensor of dtype on device (and of the given shape or size)."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.device == device, f"{name} must be on {device}, got {t.device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None:
        _need(t.numel() == numel, f"{name} must hold {numel} elements, got {t.numel()}")


def _host_bytes(t, name: str) -> None:
    _need(isinstance(t, torch.Tensor) and t.dtype == torch.uint8 and t.device.type == "cpu" and t.is_contiguous(),
          f"{name} must be a contiguous uint8 tensor in host memory")


def make_config(model_cfg) -> rlt_config:
    """rlt_config from any object with the model-shape attributes (e.g. workloads.ModelConfig)."""
    c = model_cfg
    return rlt_config(c.vocab, c.d_model, c.n_heads, c.n_layers, c.ffn_dim, FFN_KINDS[c.ffn_kind], c.window,
                      c.mem_groups, DTYPES[c.dtype], c.norm_eps)


# ---- C entry points with the same names -------------------------------------------------

def rlt_param_table(cfg: rlt_config) -> Dict[str, Tuple[int, int]]:
    lib = load_library()
    n, tot = _I32(), ctypes.c_int64()
    _check(lib.rlt_param_count(ctypes.byref(cfg), ctypes.byref(n), ctypes.byref(tot)))
    out = {}
    for i in range(n.value):
        name, off, numel = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib.rlt_param_info(ctypes.byref(cfg), i, ctypes.byref(name), ctypes.byref(off), ctypes.byref(numel)))
        out[name.value.decode()] = (off.value, numel.value)
    return out


def rlt_model_workspace_bytes(cfg: rlt_config) -> int:
    out = ctypes.c_size_t()
    _check(load_library().rlt_model_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def rlt_encoder_forward(model: "Model", state: "State", tokens: torch.Tensor, stream=None) -> None:
    _tensor(tokens, "tokens", torch.int32, state.device)
    _need(tokens.dim() == 2 and tokens.shape[0] == state.batch, f"tokens must be [{state.batch}, n]")
    _check(load_library().rlt_encoder_forward(model.handle, state.handle, _ptr(tokens), tokens.shape[1],
                                              _stream(stream)))


def rlt_decoder_replay(model: "Model", state: "State", n: int, s_out: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    if s_out is not None:
        _tensor(s_out, "s_out", torch.float32, state.device, shape=(state.batch, n, model.d_model))
    _check(load_library().rlt_decoder_replay(model.handle, state.handle, n, _ptr(s_out), _stream(stream)))


def rlt_decoder_replay_noalloc(model: "Model", state: "State", n: int, s_out: Optional[torch.Tensor] = None,
                               stream=None) -> None:
    if s_out is not None:
        _tensor(s_out, "s_out", torch.float32, state.device, shape=(state.batch, n, model.d_model))
    _check(load_library().rlt_decoder_replay_noalloc(model.handle, state.handle, n, _ptr(s_out), _stream(stream)))


def rlt_decoder_step(model: "Model", state: "State", tokens: torch.Tensor, s_out: Optional[torch.Tensor] = None,
                     logits: Optional[torch.Tensor] = None, stream=None) -> None:
    _tensor(tokens, "tokens", torch.int32, state.device, shape=(state.batch,))
    if s_out is not None:
        _tensor(s_out, "s_out", torch.float32, state.device, shape=(state.batch, model.d_model))
    if logits is not None:
        _tensor(logits, "logits", torch.float32, state.device, shape=(state.batch, model.vocab))
    _check(load_library().rlt_decoder_step(model.handle, state.handle, _ptr(tokens), _ptr(s_out), _ptr(logits),
                                           _stream(stream)))


def rlt_logits(model: "Model", s: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _tensor(s, "s", torch.float32, model.device)
    _need(s.dim() >= 1 and s.shape[-1] == model.d_model, f"s must be [..., {model.d_model}]")
    rows = s.numel() // model.d_model
    if out is None:
        out = torch.empty(*s.shape[:-1], model.vocab, dtype=torch.float32, device=s.device)
    _tensor(out, "out", torch.float32, model.device, numel=rows * model.vocab)
    _check(load_library().rlt_logits(model.handle, _ptr(s), rows, _ptr(out), _stream(stream)))
    return out


def rlt_score_actions(model: "Model", s: torch.Tensor, actions: torch.Tensor, temperature: float = 1.0,
                      behaviour_logp: Optional[torch.Tensor] = None, stream=None):
    """logp = log softmax(W_out s / temperature)[action] per row, and the importance ratio
    exp(logp - behaviour_logp) when behaviour_logp is given (else None)."""
    _tensor(s, "s", torch.float32, model.device)
    _need(s.dim() >= 1 and s.shape[-1] == model.d_model, f"s must be [..., {model.d_model}]")
    rows = s.numel() // model.d_model
    _tensor(actions, "actions", torch.int32, model.device, numel=rows)
    logp = torch.empty(*s.shape[:-1], dtype=torch.float32, device=s.device)
    ratio = None
    if behaviour_logp is not None:
        _tensor(behaviour_logp, "behaviour_logp", torch.float32, model.device, numel=rows)
        ratio = torch.empty_like(logp)
    _check(load_library().rlt_score_actions(model.handle, _ptr(s), _ptr(actions), rows, float(temperature),
                                            _ptr(behaviour_logp) if behaviour_logp is not None else None,
                                            _ptr(logp), _ptr(ratio) if ratio is not None else None,
                                            _stream(stream)))
    return logp, ratio


def rlt_sample_tokens(logits: torch.Tensor, uniforms: torch.Tensor, temperature: float = 1.0, top_k: int = 0,
                      top_p: float = 1.0, stream=None):
    """One draw per row of logits [..., V] with the caller's uniforms [...] in [0, 1):
    (tokens int32, behaviour logp fp32) under the truncated distribution actually sampled."""
    _need(isinstance(logits, torch.Tensor) and logits.is_cuda and logits.dim() >= 1,
          "logits must be a [..., V] tensor in device memory")
    _tensor(logits, "logits", torch.float32, logits.device)
    V = logits.shape[-1]
    _need(V >= 1, "logits must have at least one column")
    rows = logits.numel() // V
    _tensor(uniforms, "uniforms", torch.float32, logits.device, numel=rows)
    tok = torch.empty(*logits.shape[:-1], dtype=torch.int32, device=logits.device)
    logp = torch.empty(*logits.shape[:-1], dtype=torch.float32, device=logits.device)
    p = rlt_sampling(float(temperature), int(top_k), float(top_p))
    _check(load_library().rlt_sample_tokens(_ptr(logits), rows, V, ctypes.byref(p), _ptr(uniforms), _ptr(tok),
                                            _ptr(logp), _stream(stream)))
    return tok, logp


def rlt_decoder_step_sample(model: "Model", state: "State", tokens: torch.Tensor, uniforms: torch.Tensor,
                            temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                            s_out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                            stream=None):
    """Incremental step at the current position, then a draw of the next token per sequence:
    (next_tokens int32 [B], behaviour logp fp32 [B]).  ``logits`` [B, V] receives the step's
    logits (allocated when not given)."""
    _tensor(tokens, "tokens", torch.int32, state.device, shape=(state.batch,))
    _tensor(uniforms, "uniforms", torch.float32, state.device, numel=state.batch)
    if logits is None:
        logits = torch.empty(state.batch, model.vocab, dtype=torch.float32, device=state.device)
    _tensor(logits, "logits", torch.float32, state.device, shape=(state.batch, model.vocab))
    if s_out is not None:
        _tensor(s_out, "s_out", torch.float32, state.device, shape=(state.batch, model.d_model))
    nxt = torch.empty(state.batch, dtype=torch.int32, device=state.device)
    logp = torch.empty(state.batch, dtype=torch.float32, device=state.device)
    p = rlt_sampling(float(temperature), int(top_k), float(top_p))
    _check(load_library().rlt_decoder_step_sample(model.handle, state.handle, _ptr(tokens), ctypes.byref(p),
                                                  _ptr(uniforms), _ptr(nxt), _ptr(logp), _ptr(s_out), _ptr(logits),
                                                  _stream(stream)))
    return nxt, logp


def rlt_state_snapshot_bytes(state: "State") -> int:
    n = ctypes.c_size_t()
    _check(load_library().rlt_state_snapshot_bytes(state.handle, ctypes.byref(n)))
    return int(n.value)


def rlt_state_save(model: "Model", state: "State", out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Snapshot of the state at its current position into a host uint8 tensor (pinned when
    allocated here).  The copies are enqueued on the stream: synchronise before reading it."""
    n = rlt_state_snapshot_bytes(state)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    _host_bytes(out, "out")
    _check(load_library().rlt_state_save(model.handle, state.handle, ctypes.c_void_p(out.data_ptr()), out.numel(),
                                         _stream(stream)))
    return out


def rlt_state_restore(model: "Model", state: "State", snapshot: torch.Tensor, stream=None) -> None:
    """Reset `state` and load a snapshot into it (host uint8 tensor that must stay valid until
    the stream has run the copies)."""
    _host_bytes(snapshot, "snapshot")
    _check(load_library().rlt_state_restore(model.handle, state.handle, ctypes.c_void_p(snapshot.data_ptr()),
                                            snapshot.numel(), _stream(stream)))


def rlt_state_load_encoder_outputs(model: "Model", state: "State", e: torch.Tensor, mem_k: torch.Tensor,
                                   mem_v: torch.Tensor, stream=None) -> None:
    _need(isinstance(e, torch.Tensor) and e.dim() == 3, "e must be [B, n, d]")
    n = e.shape[1]
    G = model.mem_groups
    # contiguous copies are held by name until the call has enqueued its reads and the stream
    # has run them (a temporary freed early could be handed to the next allocation)
    e_c, mk_c, mv_c = (x.contiguous() if isinstance(x, torch.Tensor) else x for x in (e, mem_k, mem_v))
    _tensor(e_c, "e", torch.float32, state.device, shape=(state.batch, n, model.d_model))
    _tensor(mk_c, "mem_k", torch.float32, state.device, shape=(G, state.batch, n, model.d_model))
    _tensor(mv_c, "mem_v", torch.float32, state.device, shape=(G, state.batch, n, model.d_model))
    _check(load_library().rlt_state_load_encoder_outputs(model.handle, state.handle, _ptr(e_c), _ptr(mk_c),
                                                         _ptr(mv_c), n, _stream(stream)))
    (stream or torch.cuda.current_stream()).synchronize()


def rlt_state_read_encoder_outputs(model: "Model", state: "State", t0: int, n: int, stream=None):
    B, d, G = state.batch, model.d_model, model.mem_groups
    e = torch.empty(B, n, d, dtype=torch.float32, device=state.device)
    mk = torch.empty(G, B, n, d, dtype=torch.float32, device=state.device)
    mv = torch.empty_like(mk)
    _check(load_library().rlt_state_read_encoder_outputs(model.handle, state.handle, t0, n, _ptr(e), _ptr(mk),
                                                         _ptr(mv), _stream(stream)))
    return e, mk, mv


# ---- owners of device memory and handles --------------------------------------------------

DETACH_FLAGS = {"s": 1, "kv": 2, "memory": 4}


def rlt_bptt_workspace_bytes(cfg: rlt_config, batch: int, seq_len: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().rlt_bptt_workspace_bytes(ctypes.byref(cfg), batch, seq_len, ctypes.byref(out)))
    return out.value


def rlt_bptt(cfg: rlt_config, weights: torch.Tensor, tokens: torch.Tensor, mask: Optional[torch.Tensor] = None,
             detach=(), grads: Optional[torch.Tensor] = None, loss: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, stream=None):
    """Loss per sequence and the full-BPTT gradient (canonical flat layout) of the next-token loss.

    weights: flat fp32 canonical buffer on the device; tokens int32 [B, T]; mask fp32 [B, T-1] or
    None; detach: names from DETACH_FLAGS.  Returns (loss [B], grads [total])."""
    dev = weights.device
    total = sum(n for _, n in rlt_param_table(cfg).values())
    _tensor(weights, "weights", torch.float32, dev, numel=total)
    _need(tokens.dim() == 2, "tokens must be [batch, seq_len]")
    B, T = tokens.shape
    _tensor(tokens, "tokens", torch.int32, dev, shape=(B, T))
    if mask is not None:
        _tensor(mask, "mask", torch.float32, dev, shape=(B, max(T - 1, 0)))
    bits = 0
    for name in detach:
        _need(name in DETACH_FLAGS, f"unknown detach path {name!r}")
        bits |= DETACH_FLAGS[name]
    if grads is None:
        grads = torch.empty(total, dtype=torch.float32, device=dev)
    _tensor(grads, "grads", torch.float32, dev, numel=total)
    if loss is None:
        loss = torch.empty(B, dtype=torch.float32, device=dev)
    _tensor(loss, "loss", torch.float32, dev, shape=(B,))
    nbytes = rlt_bptt_workspace_bytes(cfg, B, T)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _tensor(workspace, "workspace", torch.uint8, dev)
    _check(load_library().rlt_bptt(ctypes.byref(cfg), _ptr(weights), _ptr(tokens), _ptr(mask), B, T, bits,
                                   _ptr(grads), _ptr(loss), _ptr(workspace), workspace.numel(), _stream(stream)))
    return loss, grads


class Model:
    """Packed weights (device workspace owned here) and the C model handle."""

    def __init__(self, model_cfg, weights: Dict[str, np.ndarray], version: int = 1, device="cuda:0",
                 stream=None):
        lib = load_library()
        self.cfg = make_config(model_cfg)
        dev = torch.device(device)
        _need(dev.type == "cuda", f"the model lives in device memory, not on {dev}")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.d_model, self.vocab = self.cfg.d_model, self.cfg.vocab
        self.mem_groups = self.cfg.mem_groups
        ws_bytes = rlt_model_workspace_bytes(self.cfg)
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        flat = self._flatten(weights)
        h = ctypes.c_void_p()
        _check(lib.rlt_model_create(ctypes.byref(self.cfg), _ptr(flat), version, _ptr(self.workspace), ws_bytes,
                                    _stream(stream), ctypes.byref(h)))
        self.handle = h
        self._sync(stream)   # the fp32 source buffer must outlive the pack kernels
        del flat

    def _flatten(self, weights: Dict[str, np.ndarray]) -> torch.Tensor:
        table = rlt_param_table(self.cfg)
        total = sum(n for _, n in table.values())
        flat = torch.empty(total, dtype=torch.float32, device=self.device)
        for name, (off, numel) in table.items():
            w = np.ascontiguousarray(weights[name], dtype=np.float32).reshape(-1)
            if w.size != numel:
                raise ValueError(f"weight {name}: {w.size} elements, expected {numel}")
            flat[off:off + numel].copy_(torch.from_numpy(w))
        return flat

    def _sync(self, stream=None):
        (stream or torch.cuda.current_stream()).synchronize()

    def update_weights(self, weights: Dict[str, np.ndarray], version: int, stream=None) -> None:
        flat = self._flatten(weights)
        _check(load_library().rlt_model_update_weights(self.handle, _ptr(flat), version, _stream(stream)))
        self._sync(stream)

    @property
    def version(self) -> int:
        v = ctypes.c_uint64()
        _check(load_library().rlt_model_get_config(self.handle, None, ctypes.byref(v)))
        return v.value

    def decoder_path(self, t_max: int) -> int:
        """RLT_PATH_PERSISTENT (1) or RLT_PATH_BATCHED (2) for a state of t_max positions."""
        p = _I32()
        _check(load_library().rlt_decoder_path(self.handle, t_max, ctypes.byref(p)))
        return p.value

    def set_decoder_path(self, path: int) -> None:
        """0 = automatic, 1 = persistent per-sequence kernel, 2 = batched per-phase kernels."""
        _check(load_library().rlt_model_set_decoder_path(self.handle, path))

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.rlt_model_release(self.handle)
            self.handle = None


class State:
    """H_t = (s_t, window caches) plus the encoder side, in one device blob owned here."""

    def __init__(self, model: Model, batch: int, t_max: int, keep_encoder_cache: bool = False, stream=None):
        lib = load_library()
        self.model, self.batch, self.t_max = model, batch, t_max
        self.device = model.device
        nbytes = ctypes.c_size_t()
        _check(lib.rlt_state_bytes(model.handle, batch, t_max, int(keep_encoder_cache), ctypes.byref(nbytes)))
        self.buffer = torch.empty(nbytes.value, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(lib.rlt_state_init(model.handle, _ptr(self.buffer), nbytes.value, batch, t_max,
                                  int(keep_encoder_cache), _stream(stream), ctypes.byref(h)))
        self.handle = h

    def reset(self, stream=None) -> None:
        _check(load_library().rlt_state_reset(self.model.handle, self.handle, _stream(stream)))

    def position(self) -> Tuple[int, int, int]:
        te, td, v = _I32(), _I32(), ctypes.c_uint64()
        _check(load_library().rlt_state_position(self.handle, ctypes.byref(te), ctypes.byref(td), ctypes.byref(v)))
        return te.value, td.value, v.value

    def device_error(self, stream=None) -> int:
        f = _I32()
        _check(load_library().rlt_state_device_error(self.handle, _stream(stream), ctypes.byref(f)))
        return f.value

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.rlt_state_release(self.handle)
            self.handle = None


def replay(model: Model, state: State, tokens: torch.Tensor, with_logits: bool = True, stream=None):
    """Exact replay from H_0: reset, encode all tokens, decode all positions, logits."""
    B, T = tokens.shape
    state.reset(stream)
    rlt_encoder_forward(model, state, tokens, stream)
    S = torch.empty(B, T, model.d_model, dtype=torch.float32, device=state.device)
    rlt_decoder_replay(model, state, T, S, stream)
    Z = rlt_logits(model, S, stream=stream) if with_logits else None
    return S, Z
