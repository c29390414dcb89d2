"""ctypes binding of liblola (include/lola.h): argument marshalling only.

Every function takes torch tensors that live on the GPU, passes their device
pointers and the current HIP stream to the C ABI and raises LolaError on a
non-zero status.  There is no fallback: without the built library or a GPU the
calls fail loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblola.so")

F32, BF16 = 0, 1

_STATUS = {0: "LOLA_OK", -1: "LOLA_ERR_INVALID_ARG", -2: "LOLA_ERR_UNSUPPORTED", -3: "LOLA_ERR_BAD_STATE",
           -4: "LOLA_ERR_WORKSPACE", -5: "LOLA_ERR_HIP"}

# Every symbol include/lola.h declares.
EXPORTS = ("lola_state_bytes", "lola_prefill_workspace_bytes", "lola_init_state", "lola_prefill_chunk",
           "lola_prefill_chunk_timed", "lola_prefill_chunk_noalloc", "lola_prefill_ragged", "lola_decode_step",
           "lola_read_cache", "lola_check_state", "lola_status_string")
NOALLOC_SCRATCH_BYTES = 64 << 20


class LolaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({status_string(status)})")


class LolaConfig(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("feat_half", ctypes.c_int32), ("window", ctypes.c_int32), ("cache_cap", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("policy", ctypes.c_int32), ("decode_mode", ctypes.c_int32)]


_lib = None


def lib():
    """Load liblola.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cp = ctypes.POINTER(LolaConfig)
        L.lola_state_bytes.argtypes = [cp, i32]
        L.lola_state_bytes.restype = sz
        L.lola_prefill_workspace_bytes.argtypes = [cp, i32, i32]
        L.lola_prefill_workspace_bytes.restype = sz
        L.lola_init_state.argtypes = [cp, i32, vp, vp, vp]
        L.lola_init_state.restype = ctypes.c_int
        L.lola_prefill_chunk.argtypes = [cp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.lola_prefill_chunk.restype = ctypes.c_int
        L.lola_prefill_chunk_timed.argtypes = [cp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp, vp]
        L.lola_prefill_chunk_timed.restype = ctypes.c_int
        L.lola_prefill_chunk_noalloc.argtypes = [cp, vp, i32, i32, vp, vp, vp, vp, vp]
        L.lola_prefill_chunk_noalloc.restype = ctypes.c_int
        L.lola_prefill_ragged.argtypes = [cp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lola_prefill_ragged.restype = ctypes.c_int
        L.lola_decode_step.argtypes = [cp, vp, i32, vp, vp, vp, vp, vp]
        L.lola_decode_step.restype = ctypes.c_int
        L.lola_read_cache.argtypes = [cp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.lola_read_cache.restype = ctypes.c_int
        L.lola_check_state.argtypes = [cp, vp, i32, vp]
        L.lola_check_state.restype = ctypes.c_int
        L.lola_status_string.argtypes = [ctypes.c_int]
        L.lola_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lola_status_string(status).decode()


def config(layer) -> LolaConfig:
    """C config from a LayerConfig-like object (inputs.LayerConfig)."""
    io = BF16 if layer.io_dtype == "bf16" else F32
    return LolaConfig(layer.n_q_heads, layer.n_kv_heads, layer.head_dim, layer.feat_half, layer.window,
                      layer.cache_cap, layer.chunk, io, float(layer.softmax_scale), int(layer.policy),
                      int(getattr(layer, "decode_mode", 0)))


def torch_dtype(layer):
    return torch.bfloat16 if layer.io_dtype == "bf16" else torch.float32


def _ptr(t):
    """Device address of a tensor the C ABI reads as densely packed: a strided view
    (a slice along a non-leading dimension, a transpose) is rejected, not copied."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("liblola takes densely packed tensors; got a strided view "
                         f"of shape {tuple(t.shape)} (call .contiguous() first)")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise LolaError(rc, what)


def state_bytes(layer, batch: int) -> int:
    return int(lib().lola_state_bytes(ctypes.byref(config(layer)), batch))


def workspace_bytes(layer, batch: int, max_tokens: int) -> int:
    return int(lib().lola_prefill_workspace_bytes(ctypes.byref(config(layer)), batch, max_tokens))


def init_state(layer, batch: int, W: torch.Tensor, state: torch.Tensor | None = None) -> torch.Tensor:
    """Allocate (unless given) and initialise a state buffer; W is [Hkv, feat_half, D] fp32 on the GPU."""
    n = state_bytes(layer, batch)
    if n == 0:
        raise LolaError(-2, "lola_state_bytes")
    if state is None:
        state = torch.empty(n, dtype=torch.uint8, device=W.device)
    _check(lib().lola_init_state(ctypes.byref(config(layer)), batch, _ptr(W), _ptr(state), _stream()),
           "lola_init_state")
    return state


def prefill(layer, state, q, k, v, out=None, workspace=None):
    """lola_prefill_chunk over n = k.shape[1] tokens of every sequence; returns out [B, n, Hq, D]."""
    B, n = k.shape[0], k.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    need = workspace_bytes(layer, B, n)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().lola_prefill_chunk(ctypes.byref(config(layer)), _ptr(state), B, n, _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream()), "lola_prefill_chunk")
    return out


def prefill_noalloc(layer, state, q, k, v, out=None):
    """lola_prefill_chunk_noalloc: as prefill(), with the library's static device scratch."""
    B, n = k.shape[0], k.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check(lib().lola_prefill_chunk_noalloc(ctypes.byref(config(layer)), _ptr(state), B, n, _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(out), _stream()), "lola_prefill_chunk_noalloc")
    return out


def prefill_ragged(layer, state, n_tokens, q, k, v, out=None, workspace=None):
    """lola_prefill_ragged: sequence b advances by n_tokens[b] (an int32 tensor on the GPU) of the
    k.shape[1] rows it is given; returns out [B, max_tokens, Hq, D] (rows past n_tokens[b] not written)."""
    B, n = k.shape[0], k.shape[1]
    if n_tokens.dtype != torch.int32 or n_tokens.numel() != B or not n_tokens.is_contiguous():
        raise ValueError("n_tokens must be a contiguous int32 tensor of one entry per sequence")
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(layer, B, n), dtype=torch.uint8, device=q.device)
    _check(lib().lola_prefill_ragged(ctypes.byref(config(layer)), _ptr(state), B, n, _ptr(n_tokens), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream()),
           "lola_prefill_ragged")
    return out


def prefill_timed(layer, state, q, k, v, events, out=None, workspace=None):
    """prefill() that records torch.cuda.Event objects (4, any may be None) around its launches."""
    B, n = k.shape[0], k.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(layer, B, n), dtype=torch.uint8, device=q.device)
    handles = (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
    _check(lib().lola_prefill_chunk_timed(ctypes.byref(config(layer)), _ptr(state), B, n, _ptr(q), _ptr(k),
                                          _ptr(v), _ptr(out), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(), handles),
           "lola_prefill_chunk_timed")
    return out


def decode(layer, state, q, k, v, out=None):
    """lola_decode_step: q [B, Hq, D], k, v [B, Hkv, D]; returns out [B, Hq, D]."""
    B = k.shape[0]
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check(lib().lola_decode_step(ctypes.byref(config(layer)), _ptr(state), B, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(out), _stream()), "lola_decode_step")
    return out


def read_cache(layer, state, batch: int, want_kv: bool = True, want_state: bool = True) -> dict:
    """lola_read_cache into fresh device tensors (cache in ascending position order)."""
    dev = state.device
    Hkv, C, D, F = layer.n_kv_heads, layer.cache_cap, layer.head_dim, 2 * layer.feat_half
    Cp = max(C, 1)
    res = {
        "count": torch.zeros((batch, Hkv), dtype=torch.int32, device=dev),
        "pos": torch.full((batch, Hkv, Cp), -1, dtype=torch.int64, device=dev),
        "tokens_seen": torch.zeros(batch, dtype=torch.int64, device=dev),
    }
    if want_kv:
        res["k"] = torch.zeros((batch, Hkv, Cp, D), dtype=torch_dtype(layer), device=dev)
        res["v"] = torch.zeros((batch, Hkv, Cp, D), dtype=torch_dtype(layer), device=dev)
    if want_state:
        res["H"] = torch.zeros((batch, Hkv, F, D), dtype=torch.float32, device=dev)
        res["s"] = torch.zeros((batch, Hkv, F), dtype=torch.float32, device=dev)
    _check(lib().lola_read_cache(ctypes.byref(config(layer)), _ptr(state), batch, _ptr(res["count"]),
                                 _ptr(res["pos"]) if C > 0 else None, _ptr(res.get("k")) if C > 0 else None,
                                 _ptr(res.get("v")) if C > 0 else None, _ptr(res.get("H")), _ptr(res.get("s")),
                                 _ptr(res["tokens_seen"]), _stream()), "lola_read_cache")
    return res


def check_state(layer, state, batch: int) -> int:
    """Synchronous header check; returns the status code (0 = matches)."""
    return int(lib().lola_check_state(ctypes.byref(config(layer)), _ptr(state), batch, _stream()))
