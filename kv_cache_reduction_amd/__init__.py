"""Python binding of libslim.so (Slim-Attention K-cache-only decode on MI355X).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libslim.so, which this module loads with ctypes.  torch tensors
supply device memory and the current HIP stream.  There is no fallback: if
the library is missing, importing this package raises ImportError.

Build it with ``python kv_cache_reduction_amd/build.py`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libslim.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python kv_cache_reduction_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

F32, BF16 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "workspace too small",
          4: "HIP runtime error", 5: "W_K is singular", 6: "an attend workgroup gave up waiting for its partner"}
TIMEOUT = 6

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

lib.slim_status_string.restype = ctypes.c_char_p
lib.slim_status_string.argtypes = [_i]
lib.slim_wkv.restype = _i
lib.slim_wkv.argtypes = [_vp, _vp, _i, _vp, _i]
lib.slim_prefill.restype = _i
lib.slim_prefill.argtypes = [_vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _vp, _vp]
lib.slim_decode_workspace_bytes.restype = _sz
lib.slim_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
for _name in ("slim_decode", "slim_decode_attend", "slim_decode_finish"):
    _fn = getattr(lib, _name)
    _fn.restype = _i
    _fn.argtypes = [_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _i, _f, _vp, _sz, _vp]
lib.slim_decode_noalloc.restype = _i
lib.slim_decode_noalloc.argtypes = [_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _i, _f, _vp]
NOALLOC_SCRATCH_BYTES = 80 << 20
lib.slim_decode_status.restype = _i
lib.slim_decode_status.argtypes = [_vp, _sz, _vp]
lib.slim_step_workspace_bytes.restype = _sz
lib.slim_step_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
lib.slim_step.restype = _i
lib.slim_step.argtypes = [_vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _f, _vp, _sz,
                          _vp]
lib.slim_multi_query_option.restype = _i
lib.slim_multi_query_option.argtypes = [_i, _i, _i, _i]
lib.slim_multi_query_workspace_bytes.restype = _sz
lib.slim_multi_query_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
lib.slim_multi_query.restype = _i
lib.slim_multi_query.argtypes = [_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]
lib.mha_decode_kv_workspace_bytes.restype = _sz
lib.mha_decode_kv_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
lib.mha_decode_kv.restype = _i
lib.mha_decode_kv.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _f, _vp, _sz, _vp]
lib.slim_probe_sink_floats.restype = _i
lib.slim_probe_sink_floats.argtypes = []
lib.slim_probe_read.restype = _i
lib.slim_probe_read.argtypes = [_vp, _sz, _vp, _vp]
lib.slim_probe_copy.restype = _i
lib.slim_probe_copy.argtypes = [_vp, _vp, _sz, _vp]


class SlimError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.slim_status_string(status).decode()} (status {status})")


def _check(status: int, what: str) -> None:
    if status != 0:
        raise SlimError(status, what)


def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t):
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# host: W_KV

def wkv(W_K: np.ndarray, W_V: np.ndarray, out_dtype: str = "bf16") -> np.ndarray:
    """W_KV = W_K^-1 . W_V from float64 host matrices (LU solve in the
    library).  Returns float32, or uint16 bf16 bit patterns for "bf16"."""
    W_K = np.ascontiguousarray(W_K, dtype=np.float64)
    W_V = np.ascontiguousarray(W_V, dtype=np.float64)
    d = W_K.shape[0]
    if W_K.shape != (d, d) or W_V.shape != (d, d):
        raise ValueError("W_K and W_V must be square and of equal size")
    out = np.empty((d, d), dtype=np.uint16 if out_dtype == "bf16" else np.float32)
    _check(lib.slim_wkv(W_K.ctypes.data, W_V.ctypes.data, d, out.ctypes.data,
                        BF16 if out_dtype == "bf16" else F32), "slim_wkv")
    return out


# ---------------------------------------------------------------------------
# device: prefill, decode, comparator

def prefill(X, W, K_cache, t0=None, stream=None) -> None:
    """K_cache[b, t0[b] + i, :] = round(X[b, i, :] . W).  X [B, n, d],
    W [d, d], K_cache [B, T_max, d], t0 int32 [B] on the device or None."""
    B, n, d = X.shape
    T_max = K_cache.shape[1]
    if W.shape != (d, d) or K_cache.shape != (B, T_max, d):
        raise ValueError("shape mismatch")
    _check(lib.slim_prefill(_dev(X), _dt(X), _dev(W), _dt(W), _dev(K_cache), _dt(K_cache),
                            B, n, d, T_max, None if t0 is None else _dev(t0), _stream(stream)),
           "slim_prefill")


def decode_workspace_bytes(B: int, H: int, dh: int, T_max: int, k_dtype) -> int:
    code = k_dtype if isinstance(k_dtype, int) else _dt_of(k_dtype)
    return int(lib.slim_decode_workspace_bytes(B, H, dh, T_max, code))


def _dt_of(dtype) -> int:
    torch = _torch()
    return {torch.float32: F32, torch.bfloat16: BF16}[dtype]


def workspace(nbytes: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _decode_args(q, K_cache, lengths, W_KV, out, H, dh, scale, ws):
    return _decode_core(q, K_cache, lengths, W_KV, out, H, dh, scale) + (_dev(ws), ws.numel())


def _decode_core(q, K_cache, lengths, W_KV, out, H, dh, scale):
    B, T_max, d = K_cache.shape
    if d != H * dh or q.shape != (B, d) or out.shape != (B, H, dh) or lengths.shape != (B,):
        raise ValueError("shape mismatch")
    if W_KV.shape != (d, d):
        raise ValueError("W_KV must be [d, d]")
    torch = _torch()
    if q.dtype != torch.float32 or out.dtype != torch.float32 or lengths.dtype != torch.int32:
        raise TypeError("q and out are float32, lengths int32")
    scale = 1.0 / math.sqrt(dh) if scale is None else float(scale)
    return (_dev(q), _dev(K_cache), _dt(K_cache), _dev(lengths), _dev(W_KV), _dt(W_KV), _dev(out),
            B, H, dh, T_max, scale)


def decode(q, K_cache, lengths, W_KV, out, H, dh, scale=None, ws=None, stream=None) -> None:
    """One Slim-Attention decode step (see slim_decode in include/slim.h)."""
    if ws is None:
        ws = workspace(decode_workspace_bytes(K_cache.shape[0], H, dh, K_cache.shape[1], K_cache.dtype),
                       q.device)
    _check(lib.slim_decode(*_decode_args(q, K_cache, lengths, W_KV, out, H, dh, scale, ws),
                           _stream(stream)), "slim_decode")


def decode_noalloc(q, K_cache, lengths, W_KV, out, H, dh, scale=None, stream=None) -> None:
    """slim_decode without a workspace (see slim_decode_noalloc in
    include/slim.h): the library's own device array serves as scratch."""
    _check(lib.slim_decode_noalloc(*_decode_core(q, K_cache, lengths, W_KV, out, H, dh, scale),
                                   _stream(stream)), "slim_decode_noalloc")


def decode_attend(q, K_cache, lengths, W_KV, out, H, dh, scale=None, ws=None, stream=None) -> None:
    _check(lib.slim_decode_attend(*_decode_args(q, K_cache, lengths, W_KV, out, H, dh, scale, ws),
                                  _stream(stream)), "slim_decode_attend")


def decode_finish(q, K_cache, lengths, W_KV, out, H, dh, scale=None, ws=None, stream=None) -> None:
    _check(lib.slim_decode_finish(*_decode_args(q, K_cache, lengths, W_KV, out, H, dh, scale, ws),
                                  _stream(stream)), "slim_decode_finish")


def decode_status(ws, stream=None) -> int:
    """Device-side outcome of the last decode or step on workspace `ws`
    (waits for the stream): 0, or TIMEOUT when an exchange wait gave up."""
    st = int(lib.slim_decode_status(_dev(ws), ws.numel(), _stream(stream)))
    if st not in (0, TIMEOUT):
        _check(st, "slim_decode_status")
    return st


def step_workspace_bytes(B: int, H: int, dh: int, T_max: int, k_dtype) -> int:
    code = k_dtype if isinstance(k_dtype, int) else _dt_of(k_dtype)
    return int(lib.slim_step_workspace_bytes(B, H, dh, T_max, code))


def step(x, W_Q, W_K, K_cache, lengths, lengths_next, W_KV, out, H, dh, scale=None, ws=None,
         stream=None) -> None:
    """One whole generation step (see slim_step in include/slim.h): q and k
    from x, attention over the cached rows, then k appended at row len_b and
    lengths_next written."""
    B, T_max, d = K_cache.shape
    if x.shape != (B, d) or W_Q.shape != (d, d) or W_K.shape != (d, d) or W_Q.dtype != W_K.dtype:
        raise ValueError("shape mismatch")
    if lengths_next.shape != (B,):
        raise ValueError("shape mismatch")
    torch = _torch()
    if x.dtype != torch.float32 or lengths_next.dtype != torch.int32:
        raise TypeError("x is float32, lengths int32")
    if ws is None:
        ws = workspace(step_workspace_bytes(B, H, dh, T_max, K_cache.dtype), x.device)
    a = _decode_args(x, K_cache, lengths, W_KV, out, H, dh, scale, ws)
    _check(lib.slim_step(_dev(x), _dev(W_Q), _dev(W_K), _dt(W_Q), _dev(K_cache), _dt(K_cache),
                         _dev(lengths), _dev(lengths_next), _dev(W_KV), _dt(W_KV), _dev(out),
                         B, H, dh, T_max, a[11], _dev(ws), ws.numel(), _stream(stream)), "slim_step")


def multi_query_option(n: int, H: int, dh: int, T: int) -> int:
    return int(lib.slim_multi_query_option(n, H, dh, T))


def multi_query_workspace_bytes(n: int, H: int, dh: int, T: int, w_dtype, option: int = 0) -> int:
    code = w_dtype if isinstance(w_dtype, int) else _dt_of(w_dtype)
    return int(lib.slim_multi_query_workspace_bytes(n, H, dh, T, BF16, code, option))


def multi_query(Q, K, W_KV, out, H, dh, limits=None, scale=None, option=0, ws=None, stream=None) -> None:
    """n queries over one context (see slim_multi_query in include/slim.h):
    Q [n, d] float32, K [T, d] bf16, W_KV [d, d], out [n, H, dh] float32,
    limits int32 [n] on the device or None (all rows)."""
    n, d = Q.shape
    T = K.shape[0]
    if K.shape != (T, d) or W_KV.shape != (d, d) or out.shape != (n, H, dh) or d != H * dh:
        raise ValueError("shape mismatch")
    if limits is not None and limits.shape != (n,):
        raise ValueError("limits must be [n]")
    torch = _torch()
    if Q.dtype != torch.float32 or out.dtype != torch.float32:
        raise TypeError("Q and out are float32")
    if ws is None:
        ws = workspace(multi_query_workspace_bytes(n, H, dh, T, W_KV.dtype, option), Q.device)
    scale = 1.0 / math.sqrt(dh) if scale is None else float(scale)
    _check(lib.slim_multi_query(_dev(Q), _dev(K), _dt(K), None if limits is None else _dev(limits),
                                _dev(W_KV), _dt(W_KV), _dev(out), n, H, dh, T, scale, int(option), _dev(ws),
                                ws.numel(), _stream(stream)), "slim_multi_query")


def mha_kv_workspace_bytes(B: int, H: int, dh: int, T_max: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dt_of(dtype)
    return int(lib.mha_decode_kv_workspace_bytes(B, H, dh, T_max, code))


def mha_decode_kv(q, K_cache, V_cache, lengths, out, H, dh, scale=None, ws=None, stream=None) -> None:
    """Comparator: standard MHA decode over explicit K and V caches."""
    B, T_max, d = K_cache.shape
    if V_cache.shape != K_cache.shape or V_cache.dtype != K_cache.dtype:
        raise ValueError("K and V caches must match")
    if d != H * dh or q.shape != (B, d) or out.shape != (B, H, dh) or lengths.shape != (B,):
        raise ValueError("shape mismatch")
    if ws is None:
        ws = workspace(mha_kv_workspace_bytes(B, H, dh, T_max, K_cache.dtype), q.device)
    scale = 1.0 / math.sqrt(dh) if scale is None else float(scale)
    _check(lib.mha_decode_kv(_dev(q), _dev(K_cache), _dev(V_cache), _dt(K_cache), _dev(lengths),
                             _dev(out), B, H, dh, T_max, scale, _dev(ws), ws.numel(), _stream(stream)),
           "mha_decode_kv")


# ---------------------------------------------------------------------------
# measurement probes

def probe_read(src, sink, stream=None) -> None:
    _check(lib.slim_probe_read(_dev(src), src.numel() * src.element_size(), _dev(sink),
                               _stream(stream)), "slim_probe_read")


def probe_copy(dst, src, stream=None) -> None:
    _check(lib.slim_probe_copy(_dev(dst), _dev(src), src.numel() * src.element_size(),
                               _stream(stream)), "slim_probe_copy")


def probe_sink_floats() -> int:
    return int(lib.slim_probe_sink_floats())
