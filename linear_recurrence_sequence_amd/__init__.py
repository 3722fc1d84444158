"""Python binding of libmsr (multi-scale retention on MI355X / gfx950).

Argument marshalling only: every function below checks the dtype, shape and
device of the tensors it is given (so that no wrong buffer reaches a
kernel) and builds the C call; every step of the computation runs in the
HIP kernels of ``libmsr.so``.  PyTorch supplies device memory and the
current stream.  The C functions carry the same names; their contracts are
documented in ``include/msr.h``.

If ``libmsr.so`` has not been built, importing works but the first call
raises ``MsrLibraryMissing`` -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MSR_F32", "MSR_BF16", "MsrError", "MsrLibraryMissing", "library_path", "lib",
    "msr_parallel_fwd", "msr_parallel_workspace_bytes",
    "msr_chunkwise_fwd", "msr_chunkwise_workspace_bytes", "msr_chunkwise_fwd_save", "msr_chunkwise_states_shape",
    "msr_chunkwise_bwd", "msr_chunkwise_bwd_workspace_bytes", "msr_chunkwise_bwd_saved",
    "msr_rglru_fwd", "msr_rglru_workspace_bytes",
    "msr_recurrent_step", "msr_layer_fwd", "msr_layer_workspace_bytes",
    "msr_layer_decode_step", "msr_layer_decode_workspace_bytes",
    "msr_layer_decode_step_noalloc", "msr_layer_decode_noalloc_max_bytes",
    "msr_retnet_block_fwd", "msr_retnet_block_workspace_bytes",
    "msr_status_str", "msr_last_error", "msr_trace_enable", "msr_trace_count", "msr_trace_get",
    "trace_totals",
]

MSR_F32, MSR_BF16 = 0, 1
EXPORTS = (
    "msr_parallel_fwd", "msr_parallel_workspace_bytes", "msr_chunkwise_fwd",
    "msr_chunkwise_workspace_bytes", "msr_chunkwise_fwd_save", "msr_chunkwise_bwd",
    "msr_chunkwise_bwd_workspace_bytes", "msr_chunkwise_bwd_saved",
    "msr_rglru_fwd", "msr_rglru_workspace_bytes", "msr_recurrent_step", "msr_layer_fwd",
    "msr_layer_workspace_bytes", "msr_layer_decode_step", "msr_layer_decode_workspace_bytes",
    "msr_layer_decode_step_noalloc", "msr_layer_decode_noalloc_max_bytes",
    "msr_retnet_block_fwd", "msr_retnet_block_workspace_bytes", "msr_status_str", "msr_last_error", "msr_trace_enable", "msr_trace_count", "msr_trace_get",
)

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    """The in-tree libmsr.so, or the build named by MSR_LIBRARY (e.g. the
    host-sanitizer build of build_sanitized.py)."""
    return os.environ.get("MSR_LIBRARY") or os.path.join(_HERE, "libmsr.so")


class MsrError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn}: {msr_status_str(status)} ({status}): {detail}")
        self.status = status


class MsrLibraryMissing(ImportError):
    pass


class MsrDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _F, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_DP = ctypes.POINTER(ctypes.c_double)


def lib():
    """Load libmsr.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise MsrLibraryMissing(
            f"{path} is missing: build it with `python -m linear_recurrence_sequence_amd.build`")
    L = ctypes.CDLL(path)
    sig = {
        "msr_parallel_fwd": (_I32, [_I32, MsrDims, _DP, _F, _I64, _F, _P, _P, _P, _P, _P, _SZ, _P]),
        "msr_parallel_workspace_bytes": (_SZ, [_I32, MsrDims, _F]),
        "msr_chunkwise_fwd": (_I32, [_I32, MsrDims, _I32, _DP, _F, _I64, _F, _P, _P, _P, _P, _P, _P, _P,
                                     _SZ, _P]),
        "msr_chunkwise_workspace_bytes": (_SZ, [_I32, MsrDims, _I32, _F]),
        "msr_chunkwise_fwd_save": (_I32, [_I32, MsrDims, _I32, _DP, _F, _I64, _F, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _SZ, _P]),
        "msr_chunkwise_bwd_saved": (_I32, [_I32, MsrDims, _I32, _DP, _F, _I64, _F, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P, _P, _SZ, _P]),
        "msr_chunkwise_bwd": (_I32, [_I32, MsrDims, _I32, _DP, _F, _I64, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, _SZ, _P]),
        "msr_chunkwise_bwd_workspace_bytes": (_SZ, [_I32, MsrDims, _I32, _F]),
        "msr_rglru_fwd": (_I32, [_I32, _I32, _I32, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "msr_rglru_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
        "msr_recurrent_step": (_I32, [_I32, _I32, _I32, _I32, _I32, _DP, _F, _I64, _F, _P, _P, _P, _P, _P,
                                      _P]),
        "msr_layer_fwd": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _DP, _F, _F, _P, _P, _P,
                                 _P, _P, _P, _P, _P, _SZ, _P]),
        "msr_layer_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
        "msr_layer_decode_step": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _DP, _F, _F, _I64, _P, _P, _P, _P,
                                         _P, _P, _P, _P, _P, _SZ, _P]),
        "msr_layer_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
        "msr_layer_decode_step_noalloc": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _DP, _F, _F, _I64, _P, _P, _P,
                                                 _P, _P, _P, _P, _P, _P]),
        "msr_layer_decode_noalloc_max_bytes": (_SZ, []),
        "msr_retnet_block_fwd": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _DP, _F, _F, _F,
                                        _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "msr_retnet_block_workspace_bytes": (_SZ, [_I32] * 9),
        "msr_trace_enable": (None, [_I32]),
        "msr_trace_count": (_I32, []),
        "msr_trace_get": (_I32, [_I32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_int64)]),
        "msr_status_str": (ctypes.c_char_p, [_I32]),
        "msr_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def msr_status_str(status: int) -> str:
    return lib().msr_status_str(int(status)).decode()


def msr_last_error() -> str:
    return lib().msr_last_error().decode()


def _check(fn, status):
    if status != 0:
        raise MsrError(fn, status, msr_last_error())


def msr_trace_enable(on: bool) -> None:
    lib().msr_trace_enable(1 if on else 0)


def msr_trace_count() -> int:
    return lib().msr_trace_count()


def msr_trace_get(i: int):
    name, ms, n = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
    _check("msr_trace_get", lib().msr_trace_get(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)))
    return name.value.decode(), ms.value, n.value


def trace_totals() -> dict:
    """{kernel name: (total ms, launches)} recorded since msr_trace_enable(True)."""
    return {name: (ms, n) for name, ms, n in (msr_trace_get(i) for i in range(msr_trace_count()))}


# ---------------------------------------------------------------- helpers --
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MSR_F32
    if t.dtype == torch.bfloat16:
        return MSR_BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _need(name, t, shape, dtype, device=None):
    """Check a caller's tensor before any pointer reaches the library: its
    dtype, exact shape and device (a wrong buffer would let a kernel read
    or write past the allocation).  None is allowed by the caller only
    where the argument is optional, so it is not checked here."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_ws(workspace, device):
    if workspace is not None and (workspace.device != device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")


def _gamma(gamma, heads):
    import numpy as np
    g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float64).reshape(-1))
    if g.size != heads:
        raise ValueError(f"gamma has {g.size} values for {heads} heads")
    return g, g.ctypes.data_as(_DP)


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return _torch().cuda.current_stream().cuda_stream


def _workspace(nbytes, workspace, device):
    if nbytes == 0:
        return workspace, 0
    if workspace is None:
        workspace = _torch().empty(nbytes, dtype=_torch().uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


# ------------------------------------------------------------ entry points --
def msr_parallel_workspace_bytes(dtype: int, batch, seqlen, heads, d_k, d_v, rope_base) -> int:
    return lib().msr_parallel_workspace_bytes(dtype, MsrDims(batch, seqlen, heads, d_k, d_v), rope_base)


def msr_chunkwise_workspace_bytes(dtype: int, batch, seqlen, heads, d_k, d_v, chunk, rope_base) -> int:
    return lib().msr_chunkwise_workspace_bytes(dtype, MsrDims(batch, seqlen, heads, d_k, d_v), chunk,
                                               rope_base)


def msr_layer_workspace_bytes(dtype: int, batch, seqlen, d_model, heads, d_k, d_v, chunk) -> int:
    return lib().msr_layer_workspace_bytes(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk)


def msr_parallel_fwd(Q, K, V, gamma, *, rope_base=0.0, pos0=0, qk_scale=1.0, O=None, workspace=None,
                     stream=None):
    """Parallel form (Eq. 5).  Q, K: [B, N, H, d_k]; V: [B, N, H, d_v]."""
    B, N, H, dk = Q.shape
    dv = V.shape[-1]
    dt = _dtype_code(Q)
    _need("K", K, Q.shape, Q.dtype, Q.device)
    _need("V", V, (B, N, H, dv), Q.dtype, Q.device)
    _need("O", O, (B, N, H, dv), Q.dtype, Q.device)
    _need_ws(workspace, Q.device)
    if O is None:
        O = _torch().empty((B, N, H, dv), dtype=Q.dtype, device=Q.device)
    _, gp = g = _gamma(gamma, H)
    dims = MsrDims(B, N, H, dk, dv)
    ws, wsb = _workspace(lib().msr_parallel_workspace_bytes(dt, dims, rope_base), workspace, Q.device)
    _check("msr_parallel_fwd", lib().msr_parallel_fwd(dt, dims, gp, rope_base, pos0, qk_scale, _ptr(Q), _ptr(K),
                                                      _ptr(V), _ptr(O), _ptr(ws), wsb, _stream(stream)))
    return O


def msr_chunkwise_fwd(Q, K, V, gamma, chunk, *, rope_base=0.0, pos0=0, qk_scale=1.0, S_in=None,
                      S_out=None, O=None, workspace=None, stream=None):
    """Chunkwise form (Eq. 7).  Returns O; S_out (if given) receives the
    final state [B, H, d_k, d_v] float32."""
    B, N, H, dk = Q.shape
    dv = V.shape[-1]
    dt = _dtype_code(Q)
    _check_core(Q, K, V, O, S_in, S_out, workspace)
    if O is None:
        O = _torch().empty((B, N, H, dv), dtype=Q.dtype, device=Q.device)
    _, gp = g = _gamma(gamma, H)
    dims = MsrDims(B, N, H, dk, dv)
    ws, wsb = _workspace(lib().msr_chunkwise_workspace_bytes(dt, dims, chunk, rope_base), workspace, Q.device)
    _check("msr_chunkwise_fwd", lib().msr_chunkwise_fwd(dt, dims, chunk, gp, rope_base, pos0, qk_scale, _ptr(Q),
                                                        _ptr(K), _ptr(V), _ptr(S_in), _ptr(S_out), _ptr(O),
                                                        _ptr(ws), wsb, _stream(stream)))
    return O


def _check_core(Q, K, V, O, S_in, S_out, workspace, R_chunks=None, chunk=None):
    """Shapes, dtypes and devices of a chunkwise call's tensors."""
    torch = _torch()
    B, N, H, dk = Q.shape
    dv = V.shape[-1]
    _need("K", K, Q.shape, Q.dtype, Q.device)
    _need("V", V, (B, N, H, dv), Q.dtype, Q.device)
    _need("O", O, (B, N, H, dv), Q.dtype, Q.device)
    _need("S_in", S_in, (B, H, dk, dv), torch.float32, Q.device)
    _need("S_out", S_out, (B, H, dk, dv), torch.float32, Q.device)
    if chunk is not None and chunk > 0:
        _need("R_chunks", R_chunks, msr_chunkwise_states_shape(B, N, H, dk, dv, chunk), Q.dtype, Q.device)
    _need_ws(workspace, Q.device)


def msr_chunkwise_states_shape(B, N, H, d_k, d_v, chunk):
    """Shape of the per-chunk states of msr_chunkwise_fwd_save: [B, H, NC, d_v, d_k]."""
    return (B, H, -(-N // chunk), d_v, d_k)


def msr_chunkwise_fwd_save(Q, K, V, gamma, chunk, R_chunks, *, rope_base=0.0, pos0=0, qk_scale=1.0, S_in=None,
                           S_out=None, O=None, workspace=None, stream=None):
    """msr_chunkwise_fwd that also writes every chunk's starting state
    (transposed) into R_chunks (msr_chunkwise_states_shape, Q's dtype).
    Returns O."""
    B, N, H, dk = Q.shape
    dv = V.shape[-1]
    dt = _dtype_code(Q)
    if R_chunks is None:
        raise ValueError("R_chunks is required")
    _check_core(Q, K, V, O, S_in, S_out, workspace, R_chunks, chunk)
    if O is None:
        O = _torch().empty((B, N, H, dv), dtype=Q.dtype, device=Q.device)
    _, gp = g = _gamma(gamma, H)
    dims = MsrDims(B, N, H, dk, dv)
    ws, wsb = _workspace(lib().msr_chunkwise_workspace_bytes(dt, dims, chunk, rope_base), workspace, Q.device)
    _check("msr_chunkwise_fwd_save", lib().msr_chunkwise_fwd_save(dt, dims, chunk, gp, rope_base, pos0, qk_scale,
                                                                  _ptr(Q), _ptr(K), _ptr(V), _ptr(S_in),
                                                                  _ptr(S_out), _ptr(R_chunks), _ptr(O), _ptr(ws),
                                                                  wsb, _stream(stream)))
    return O


def msr_chunkwise_bwd_workspace_bytes(dtype: int, batch, seqlen, heads, d_k, d_v, chunk, rope_base) -> int:
    return lib().msr_chunkwise_bwd_workspace_bytes(dtype, MsrDims(batch, seqlen, heads, d_k, d_v), chunk,
                                                   rope_base)


def msr_chunkwise_bwd(Q, K, V, dO, gamma, chunk, *, rope_base=0.0, pos0=0, qk_scale=1.0, S_in=None,
                      dS_out=None, dS_in=None, dQ=None, dK=None, dV=None, workspace=None, stream=None):
    """Backward of the chunkwise form.  Returns (dQ, dK, dV); dS_in (if
    given, [B, H, d_k, d_v] float32) receives the gradient of the initial
    state."""
    B, N, H, dk = Q.shape
    dv = V.shape[-1]
    dt = _dtype_code(Q)
    _check_bwd(Q, K, V, dO, S_in, dS_out, dS_in, dQ, dK, dV, workspace)
    t = _torch()
    dQ = t.empty_like(Q) if dQ is None else dQ
    dK = t.empty_like(K) if dK is None else dK
    dV = t.empty_like(V) if dV is None else dV
    _, gp = g = _gamma(gamma, H)
    dims = MsrDims(B, N, H, dk, dv)
    ws, wsb = _workspace(lib().msr_chunkwise_bwd_workspace_bytes(dt, dims, chunk, rope_base), workspace, Q.device)
    _check("msr_chunkwise_bwd", lib().msr_chunkwise_bwd(dt, dims, chunk, gp, rope_base, pos0, qk_scale, _ptr(Q),
                                                        _ptr(K), _ptr(V), _ptr(dO), _ptr(S_in), _ptr(dS_out),
                                                        _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dS_in), _ptr(ws), wsb,
                                                        _stream(stream)))
    return dQ, dK, dV


def _check_bwd(Q, K, V, dO, S_in, dS_out, dS_in, dQ, dK, dV, workspace, R_chunks=None, chunk=None):
    torch = _torch()
    B, N, H, dk = Q.shape
    dv = V.shape[-1]
    _check_core(Q, K, V, None, S_in, None, workspace, R_chunks, chunk)
    _need("dO", dO, (B, N, H, dv), Q.dtype, Q.device)
    _need("dS_out", dS_out, (B, H, dk, dv), torch.float32, Q.device)
    _need("dS_in", dS_in, (B, H, dk, dv), torch.float32, Q.device)
    _need("dQ", dQ, Q.shape, Q.dtype, Q.device)
    _need("dK", dK, Q.shape, Q.dtype, Q.device)
    _need("dV", dV, (B, N, H, dv), Q.dtype, Q.device)


def msr_chunkwise_bwd_saved(Q, K, V, dO, gamma, chunk, R_chunks, *, rope_base=0.0, pos0=0, qk_scale=1.0,
                            S_in=None, dS_out=None, dS_in=None, dQ=None, dK=None, dV=None, workspace=None,
                            stream=None):
    """msr_chunkwise_bwd with the forward's per-chunk states (from
    msr_chunkwise_fwd_save with the same arguments).  Returns (dQ, dK, dV)."""
    B, N, H, dk = Q.shape
    dv = V.shape[-1]
    dt = _dtype_code(Q)
    if R_chunks is None:
        raise ValueError("R_chunks is required")
    _check_bwd(Q, K, V, dO, S_in, dS_out, dS_in, dQ, dK, dV, workspace, R_chunks, chunk)
    t = _torch()
    dQ = t.empty_like(Q) if dQ is None else dQ
    dK = t.empty_like(K) if dK is None else dK
    dV = t.empty_like(V) if dV is None else dV
    _, gp = g = _gamma(gamma, H)
    dims = MsrDims(B, N, H, dk, dv)
    ws, wsb = _workspace(lib().msr_chunkwise_bwd_workspace_bytes(dt, dims, chunk, rope_base), workspace, Q.device)
    _check("msr_chunkwise_bwd_saved", lib().msr_chunkwise_bwd_saved(
        dt, dims, chunk, gp, rope_base, pos0, qk_scale, _ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(S_in),
        _ptr(dS_out), _ptr(R_chunks), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dS_in), _ptr(ws), wsb, _stream(stream)))
    return dQ, dK, dV


def msr_rglru_workspace_bytes(dtype: int, batch, seqlen, width) -> int:
    return lib().msr_rglru_workspace_bytes(dtype, batch, seqlen, width)


def msr_rglru_fwd(X, W_a, b_a, W_x, b_x, Lambda, *, c=8.0, h0=None, h_last=None, Y=None, workspace=None,
                  stream=None):
    """RG-LRU over a sequence.  X: [B, T, width]; W_a, W_x: [width, width];
    b_a, b_x, Lambda: [width] float32; h0, h_last: [B, width] float32.
    Returns Y [B, T, width]."""
    B, T, D = X.shape
    dt = _dtype_code(X)
    f32 = _torch().float32
    _need("W_a", W_a, (D, D), X.dtype, X.device)
    _need("W_x", W_x, (D, D), X.dtype, X.device)
    for name, t in (("b_a", b_a), ("b_x", b_x), ("Lambda", Lambda)):
        _need(name, t, (D,), f32, X.device)
    _need("h0", h0, (B, D), f32, X.device)
    _need("h_last", h_last, (B, D), f32, X.device)
    _need("Y", Y, X.shape, X.dtype, X.device)
    _need_ws(workspace, X.device)
    Y = _torch().empty_like(X) if Y is None else Y
    ws, wsb = _workspace(lib().msr_rglru_workspace_bytes(dt, B, T, D), workspace, X.device)
    _check("msr_rglru_fwd", lib().msr_rglru_fwd(dt, B, T, D, c, _ptr(X), _ptr(W_a), _ptr(b_a), _ptr(W_x), _ptr(b_x),
                                                _ptr(Lambda), _ptr(h0), _ptr(h_last), _ptr(Y), _ptr(ws), wsb,
                                                _stream(stream)))
    return Y


def msr_recurrent_step(q, k, v, S, gamma, *, pos, rope_base=0.0, qk_scale=1.0, o=None, stream=None):
    """Recurrent form, one step (Eq. 6), S updated in place.
    q, k: [B, H, d_k]; v: [B, H, d_v]; S: [B, H, d_k, d_v] float32."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if S is None:
        raise ValueError("S is required")
    _need("k", k, q.shape, q.dtype, q.device)
    _need("v", v, (B, H, dv), q.dtype, q.device)
    _need("S", S, (B, H, dk, dv), _torch().float32, q.device)
    _need("o", o, (B, H, dv), q.dtype, q.device)
    if o is None:
        o = _torch().empty((B, H, dv), dtype=q.dtype, device=q.device)
    _, gp = g = _gamma(gamma, H)
    _check("msr_recurrent_step", lib().msr_recurrent_step(dt, B, H, dk, dv, gp, rope_base, pos, qk_scale,
                                                          _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(o),
                                                          _stream(stream)))
    return o


def msr_layer_fwd(X, W_Q, W_K, W_V, W_G, W_O, gamma, heads, d_k, d_v, chunk, *, rope_base=10000.0,
                  gn_eps=1e-5, out=None, workspace=None, stream=None):
    """Gated MSR layer (Eq. 8).  X: [B, N, d_model]; returns [B, N, d_model]."""
    B, N, dm = X.shape
    dt = _dtype_code(X)
    _check_layer_weights(X, dm, heads, d_k, d_v, W_Q, W_K, W_V, W_G, W_O)
    _need("out", out, X.shape, X.dtype, X.device)
    _need_ws(workspace, X.device)
    if out is None:
        out = _torch().empty((B, N, dm), dtype=X.dtype, device=X.device)
    _, gp = g = _gamma(gamma, heads)
    nbytes = lib().msr_layer_workspace_bytes(dt, B, N, dm, heads, d_k, d_v, chunk)
    ws, wsb = _workspace(nbytes, workspace, X.device)
    _check("msr_layer_fwd", lib().msr_layer_fwd(dt, B, N, dm, heads, d_k, d_v, chunk, gp, rope_base, gn_eps,
                                                _ptr(X), _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_G), _ptr(W_O),
                                                _ptr(out), _ptr(ws), wsb, _stream(stream)))
    return out


def _check_layer_weights(X, dm, heads, d_k, d_v, W_Q, W_K, W_V, W_G, W_O):
    for name, t, shape in (("W_Q", W_Q, (dm, heads * d_k)), ("W_K", W_K, (dm, heads * d_k)),
                           ("W_V", W_V, (dm, heads * d_v)), ("W_G", W_G, (dm, heads * d_v)),
                           ("W_O", W_O, (heads * d_v, dm))):
        if t is None:
            raise ValueError(f"{name} is required")
        _need(name, t, shape, X.dtype, X.device)


def msr_retnet_block_workspace_bytes(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk, d_ffn):
    return lib().msr_retnet_block_workspace_bytes(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk, d_ffn)


def msr_retnet_block_fwd(X, W_Q, W_K, W_V, W_G, W_O, W_1, W_2, gamma, heads, d_k, d_v, chunk, *,
                         rope_base=10000.0, gn_eps=1e-5, ln_eps=1e-5, out=None, workspace=None, stream=None):
    """One RetNet block: Y = MSR(LN(X)) + X, out = gelu(LN(Y) W_1) W_2 + Y.  X: [B, N, d_model]."""
    B, N, dm = X.shape
    d_ffn = W_1.shape[1]
    dt = _dtype_code(X)
    _check_layer_weights(X, dm, heads, d_k, d_v, W_Q, W_K, W_V, W_G, W_O)
    _need("W_1", W_1, (dm, d_ffn), X.dtype, X.device)
    _need("W_2", W_2, (d_ffn, dm), X.dtype, X.device)
    _need("out", out, X.shape, X.dtype, X.device)
    _need_ws(workspace, X.device)
    if out is None:
        out = _torch().empty((B, N, dm), dtype=X.dtype, device=X.device)
    _, gp = g = _gamma(gamma, heads)
    nbytes = lib().msr_retnet_block_workspace_bytes(dt, B, N, dm, heads, d_k, d_v, chunk, d_ffn)
    ws, wsb = _workspace(nbytes, workspace, X.device)
    _check("msr_retnet_block_fwd",
           lib().msr_retnet_block_fwd(dt, B, N, dm, heads, d_k, d_v, chunk, d_ffn, gp, rope_base, gn_eps, ln_eps,
                                      _ptr(X), _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_G), _ptr(W_O), _ptr(W_1),
                                      _ptr(W_2), _ptr(out), _ptr(ws), wsb, _stream(stream)))
    return out


def msr_layer_decode_workspace_bytes(dtype, batch, d_model, heads, d_k, d_v):
    return lib().msr_layer_decode_workspace_bytes(dtype, batch, d_model, heads, d_k, d_v)


def msr_layer_decode_step(X, W_Q, W_K, W_V, W_G, W_O, S, gamma, heads, d_k, d_v, pos, *, rope_base=10000.0,
                          gn_eps=1e-5, out=None, workspace=None, stream=None):
    """One decode step of the gated MSR layer (Eq. 8 with Eq. 6).  X: [B, d_model] (the new token of each
    sequence); S: [B, heads, d_k, d_v] float32, updated in place; returns out [B, d_model]."""
    B, dm = X.shape
    dt = _dtype_code(X)
    _check_layer_weights(X, dm, heads, d_k, d_v, W_Q, W_K, W_V, W_G, W_O)
    if S is None:
        raise ValueError("S is required")
    _need("S", S, (B, heads, d_k, d_v), _torch().float32, X.device)
    _need("out", out, X.shape, X.dtype, X.device)
    _need_ws(workspace, X.device)
    if out is None:
        out = _torch().empty((B, dm), dtype=X.dtype, device=X.device)
    _, gp = g = _gamma(gamma, heads)
    nbytes = lib().msr_layer_decode_workspace_bytes(dt, B, dm, heads, d_k, d_v)
    ws, wsb = _workspace(nbytes, workspace, X.device)
    _check("msr_layer_decode_step",
           lib().msr_layer_decode_step(dt, B, dm, heads, d_k, d_v, gp, rope_base, gn_eps, int(pos), _ptr(X),
                                       _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_G), _ptr(W_O), _ptr(S), _ptr(out),
                                       _ptr(ws), wsb, _stream(stream)))
    return out


def msr_layer_decode_noalloc_max_bytes() -> int:
    return lib().msr_layer_decode_noalloc_max_bytes()


def msr_layer_decode_step_noalloc(X, W_Q, W_K, W_V, W_G, W_O, S, gamma, heads, d_k, d_v, pos, *,
                                  rope_base=10000.0, gn_eps=1e-5, out=None, stream=None):
    """msr_layer_decode_step on the library's static scratch (no workspace;
    the C call allocates nothing -- pass `out` to allocate nothing here
    either).  Calls that overlap on one GPU race."""
    B, dm = X.shape
    dt = _dtype_code(X)
    _check_layer_weights(X, dm, heads, d_k, d_v, W_Q, W_K, W_V, W_G, W_O)
    if S is None:
        raise ValueError("S is required")
    _need("S", S, (B, heads, d_k, d_v), _torch().float32, X.device)
    _need("out", out, X.shape, X.dtype, X.device)
    if out is None:
        out = _torch().empty((B, dm), dtype=X.dtype, device=X.device)
    _, gp = g = _gamma(gamma, heads)
    _check("msr_layer_decode_step_noalloc",
           lib().msr_layer_decode_step_noalloc(dt, B, dm, heads, d_k, d_v, gp, rope_base, gn_eps, int(pos), _ptr(X),
                                               _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_G), _ptr(W_O), _ptr(S),
                                               _ptr(out), _stream(stream)))
    return out
