"""MI355X (gfx950) fused causal attention, forward and backward.

A thin ctypes binding over ``libattn.so`` (C ABI in ``include/attn.h``).  Every
step of the computation runs in the library's HIP kernels; this module only
marshals torch tensors (device memory) and torch's current stream into the C
calls.  There is no fallback: if the library has not been built, importing the
binding raises.

Names mirror the C ABI:
    attn_fwd(Q, K, V, O, LSE, scale, causal=True, stream=None)
    attn_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal=True, stream=None)
    attn_bwd_atomic(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal=True, stream=None)
    attn_bwd_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, scale, causal=True, stream=None)
    attn_bwd_atomic_workspace_bytes(dtype, B, H, T, head_dim, causal=True)
    attn_bwd_workspace_bytes(dtype, B, H, T, head_dim, causal=True)
    attn_fwd_strided, attn_bwd_strided, attn_bwd_atomic_strided (same arguments)
    gemm(op, A, B, C, split_k=1, workspace=None, stream=None), gemm_workspace_bytes(op, M, N, K, split_k)
    attn_status_str(status), attn_last_error(), attn_init()
    attn_prof_enable(capacity), attn_prof_read()
Tensors are contiguous [B, H, T, head_dim] (float32 or bfloat16) on one GPU;
the *_strided calls accept any [B, H, T, head_dim] view whose last dimension
has stride 1 (for instance q, k, v = qkv.view(B, T, 3, H, d).permute(2, 0, 3,
1, 4) over a projection output) and pass its element strides through.  LSE is
float32 [B, H, T]; the workspace is any device tensor of at least
attn_bwd_workspace_bytes(...) bytes.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "AttnError", "ATTN_F32", "ATTN_BF16", "attn_fwd", "attn_bwd", "attn_bwd_atomic", "attn_bwd_noalloc",
    "NOALLOC_MAX_ROWS",
    "attn_fwd_strided", "attn_bwd_strided", "attn_bwd_atomic_strided",
    "GEMM_NT", "GEMM_NN", "GEMM_TN", "gemm", "gemm_workspace_bytes",
    "attn_bwd_workspace_bytes", "attn_bwd_atomic_workspace_bytes",
    "attn_status_str", "attn_last_error", "attn_prof_enable", "attn_prof_read", "attn_init", "library_path", "lib",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F32, ATTN_BF16 = 0, 1
GEMM_NT, GEMM_NN, GEMM_TN = 0, 1, 2
ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_ELAUNCH = 0, 1, 2, 3
NOALLOC_MAX_ROWS = 1 << 21  # ATTN_NOALLOC_MAX_ROWS in attn.h


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__("%s: %s (%s)" % (where, attn_status_str(status), detail))
        self.status = status


class _KernelTime(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


def _load():
    # torch ships its own HIP runtime (same SONAME as ROCm's).  Importing torch
    # first makes libattn.so bind to that copy instead of mapping a second HIP
    # runtime into the process, so device pointers and streams from torch are
    # valid in the library.
    import torch  # noqa: F401

    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            "libattn.so is not built; run `python causal_attention_attn_amd/build.py` "
            "(or __graft_entry__.build()) first"
        )
    L = ctypes.CDLL(_LIB_PATH)
    try:
        with open("/proc/self/maps") as f:
            hips = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        hips = set()
    if len(hips) > 1:
        raise ImportError("two HIP runtimes are mapped (%s); libattn.so must share torch's" % sorted(hips))
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    L.attn_fwd.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    L.attn_bwd.restype = i
    L.attn_bwd_noalloc.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    L.attn_bwd_noalloc.restype = i
    L.attn_bwd_atomic.argtypes = L.attn_bwd.argtypes
    L.attn_bwd_atomic.restype = i
    ll3 = ctypes.POINTER(ctypes.c_longlong)
    L.attn_fwd_strided.argtypes = [i, vp, vp, vp, vp, vp, ll3, i, i, i, i, f, i, vp]
    L.attn_fwd_strided.restype = i
    L.attn_bwd_strided.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ll3, i, i, i, i, f, i, vp]
    L.attn_bwd_strided.restype = i
    L.attn_bwd_atomic_strided.argtypes = L.attn_bwd_strided.argtypes
    L.attn_bwd_atomic_strided.restype = i
    L.gemm_workspace_bytes.argtypes = [i, i, i, i, i]
    L.gemm_workspace_bytes.restype = sz
    L.gemm_bf16.argtypes = [i, vp, i, vp, i, vp, i, i, i, i, i, i, vp, sz, vp]
    L.gemm_bf16.restype = i
    L.attn_bwd_atomic_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_bwd_atomic_workspace_bytes.restype = sz
    L.attn_init.argtypes = []
    L.attn_init.restype = i
    L.attn_status_str.argtypes = [i]
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_prof_enable.argtypes = [i]
    L.attn_prof_enable.restype = i
    L.attn_prof_read.argtypes = [ctypes.POINTER(_KernelTime), i]
    L.attn_prof_read.restype = i
    return L


lib = _load()


def library_path() -> str:
    return _LIB_PATH


def attn_init() -> None:
    """The library's one-time set-up on torch's current device (attn_init in
    attn.h).  Run at import for the current device when a GPU is present;
    call it again after switching to another device before capturing calls
    there into a HIP graph."""
    _check(lib.attn_init(), "attn_init")




def attn_status_str(status: int) -> str:
    return lib.attn_status_str(int(status)).decode()


def attn_last_error() -> str:
    return lib.attn_last_error().decode()


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where, attn_last_error())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _stream_handle(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _shape(Q):
    if Q.dim() != 4:
        raise ValueError("expected [B, H, T, head_dim], got %s" % (tuple(Q.shape),))
    return tuple(int(x) for x in Q.shape)


def _validate(where, Q, views, LSE, workspace=None):
    """Checks what the C ABI cannot see (it receives bare pointers): every
    [B, H, T, head_dim] tensor has Q's shape and element type, LSE is float32
    [B, H, T], and every tensor, the workspace included, lives on Q's GPU.
    Raises before anything reaches the library."""
    import torch

    B, H, T, d = _shape(Q)
    _dtype_code(Q)
    for name, t in views:
        if t is None:
            raise ValueError("%s: %s is missing" % (where, name))
        if tuple(t.shape) != (B, H, T, d):
            raise ValueError("%s: %s has shape %s, Q has %s" % (where, name, tuple(t.shape), (B, H, T, d)))
        if t.dtype != Q.dtype:
            raise TypeError("%s: %s is %s, Q is %s" % (where, name, t.dtype, Q.dtype))
    if LSE is None or LSE.dtype != torch.float32 or tuple(LSE.shape) != (B, H, T):
        raise ValueError("%s: LSE must be float32 of shape %s, got %s" % (
            where, (B, H, T), None if LSE is None else (LSE.dtype, tuple(LSE.shape))))
    tensors = [("Q", Q)] + list(views) + [("LSE", LSE)]
    if workspace is not None:
        tensors.append(("workspace", workspace))
    for name, t in tensors:
        if t.device.type != "cuda":
            raise ValueError("%s: %s is on %s; every tensor must be a GPU tensor" % (where, name, t.device))
        if t.device != Q.device:
            raise ValueError("%s: %s is on %s, Q on %s" % (where, name, t.device, Q.device))
    return B, H, T, d


def _p(t) -> int:
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return int(t.data_ptr())


def attn_fwd(Q, K, V, O, LSE, scale: float, causal: bool = True, stream=None) -> None:
    """Enqueue the forward pass on ``stream`` (default: torch's current stream)."""
    B, H, T, d = _validate("attn_fwd", Q, [("K", K), ("V", V), ("O", O)], LSE)
    _check(lib.attn_fwd(_dtype_code(Q), _p(Q), _p(K), _p(V), _p(O), _p(LSE), B, H, T, d, float(scale),
                        int(bool(causal)), _stream_handle(stream)), "attn_fwd")


def attn_bwd_workspace_bytes(dtype: int, B: int, H: int, T: int, head_dim: int, causal: bool = True) -> int:
    return int(lib.attn_bwd_workspace_bytes(int(dtype), B, H, T, head_dim, int(bool(causal))))


def _bwd(fn, name, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal, stream):
    B, H, T, d = _validate(name, Q, [("K", K), ("V", V), ("O", O), ("dO", dO), ("dQ", dQ), ("dK", dK),
                                     ("dV", dV)], LSE, workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(fn(_dtype_code(Q), _p(Q), _p(K), _p(V), _p(O), _p(dO), _p(LSE), _p(dQ), _p(dK), _p(dV),
              _p(workspace), nbytes, B, H, T, d, float(scale), int(bool(causal)), _stream_handle(stream)), name)


def attn_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale: float, causal: bool = True, stream=None) -> None:
    """Enqueue the (atomic-free, bitwise reproducible) backward pass on ``stream``
    (default: torch's current stream)."""
    _bwd(lib.attn_bwd, "attn_bwd", Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal, stream)


def attn_bwd_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, scale: float, causal: bool = True, stream=None) -> None:
    """attn_bwd with D in the library's static device array instead of a
    workspace (attn_bwd_noalloc in attn.h): B*H*T at most NOALLOC_MAX_ROWS;
    calls overlapping in time on one GPU race on that array."""
    B, H, T, d = _validate("attn_bwd_noalloc", Q, [("K", K), ("V", V), ("O", O), ("dO", dO), ("dQ", dQ),
                                                 ("dK", dK), ("dV", dV)], LSE)
    _check(lib.attn_bwd_noalloc(_dtype_code(Q), _p(Q), _p(K), _p(V), _p(O), _p(dO), _p(LSE), _p(dQ), _p(dK),
                                _p(dV), B, H, T, d, float(scale), int(bool(causal)), _stream_handle(stream)),
           "attn_bwd_noalloc")


def attn_bwd_atomic_workspace_bytes(dtype: int, B: int, H: int, T: int, head_dim: int, causal: bool = True) -> int:
    return int(lib.attn_bwd_atomic_workspace_bytes(int(dtype), B, H, T, head_dim, int(bool(causal))))


def attn_bwd_atomic(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale: float, causal: bool = True,
                    stream=None) -> None:
    """Backward with dQ accumulated by fp32 atomics inside the dK/dV kernel (bf16 only)."""
    _bwd(lib.attn_bwd_atomic, "attn_bwd_atomic", Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal,
         stream)


def _vp(t) -> int:
    """Address of a [B, H, T, head_dim] view (storage offset included)."""
    if t is None:
        return 0
    if t.dim() != 4 or (t.shape[3] > 1 and t.stride(3) != 1):
        raise ValueError("expected a [B, H, T, head_dim] view with unit stride in head_dim")
    return int(t.data_ptr())


def _strides(*ts):
    vals = []
    for t in ts:
        if t is None or t.dim() != 4:
            raise ValueError("expected [B, H, T, head_dim] views")
        vals += [int(t.stride(0)), int(t.stride(1)), int(t.stride(2))]
    return (ctypes.c_longlong * len(vals))(*vals)


def attn_fwd_strided(Q, K, V, O, LSE, scale: float, causal: bool = True, stream=None) -> None:
    """attn_fwd on strided [B, H, T, head_dim] views of Q, K, V and O."""
    B, H, T, d = _validate("attn_fwd_strided", Q, [("K", K), ("V", V), ("O", O)], LSE)
    _check(lib.attn_fwd_strided(_dtype_code(Q), _vp(Q), _vp(K), _vp(V), _vp(O), _p(LSE), _strides(Q, K, V, O),
                                B, H, T, d, float(scale), int(bool(causal)), _stream_handle(stream)),
           "attn_fwd_strided")


def _bwd_strided(fn, name, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale, causal, stream):
    B, H, T, d = _validate(name, Q, [("K", K), ("V", V), ("O", O), ("dO", dO), ("dQ", dQ), ("dK", dK),
                                     ("dV", dV)], LSE, workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(fn(_dtype_code(Q), _vp(Q), _vp(K), _vp(V), _vp(O), _vp(dO), _p(LSE), _vp(dQ), _vp(dK), _vp(dV),
              _p(workspace), nbytes, _strides(Q, K, V, O, dO, dQ, dK, dV), B, H, T, d, float(scale),
              int(bool(causal)), _stream_handle(stream)), name)


def attn_bwd_strided(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale: float, causal: bool = True,
                     stream=None) -> None:
    """attn_bwd on strided [B, H, T, head_dim] views."""
    _bwd_strided(lib.attn_bwd_strided, "attn_bwd_strided", Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale,
                 causal, stream)


def attn_bwd_atomic_strided(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, scale: float, causal: bool = True,
                            stream=None) -> None:
    """attn_bwd_atomic on strided [B, H, T, head_dim] views (bf16 only)."""
    _bwd_strided(lib.attn_bwd_atomic_strided, "attn_bwd_atomic_strided", Q, K, V, O, dO, LSE, dQ, dK, dV,
                 workspace, scale, causal, stream)


def gemm_workspace_bytes(op: int, M: int, N: int, K: int, split_k: int = 1) -> int:
    return int(lib.gemm_workspace_bytes(int(op), M, N, K, int(split_k)))


def _ld(t) -> int:
    """Leading dimension of a 2-D row-major view (unit stride along rows)."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D matrix with unit stride along its rows")
    return int(t.stride(0)) if t.shape[0] > 1 else int(t.shape[1])


def gemm(op: int, A, B, C, split_k: int = 1, workspace=None, stream=None) -> None:
    """C = op(A) op(B) on bf16 operands (GEMM_NT: A B^T, GEMM_NN: A B,
    GEMM_TN: A^T B); C is bfloat16 or float32.  Shapes come from the tensors:
    NT A [M, K] B [N, K]; NN A [M, K] B [K, N]; TN A [K, M] B [K, N]."""
    import torch

    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if op == GEMM_NT:
        (M, K), (N, K2) = A.shape, B.shape
    elif op == GEMM_NN:
        (M, K), (K2, N) = A.shape, B.shape
    elif op == GEMM_TN:
        (K, M), (K2, N) = A.shape, B.shape
    else:
        raise ValueError("unknown gemm op %r" % (op,))
    if K != K2 or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape), tuple(C.shape)))
    if C.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("C must be bfloat16 or float32, got %s" % C.dtype)
    for name, t in (("A", A), ("B", B), ("C", C), ("workspace", workspace)):
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("gemm: %s is on %s; every tensor must be a GPU tensor" % (name, t.device))
        if t.device != A.device:
            raise ValueError("gemm: %s is on %s, A on %s" % (name, t.device, A.device))
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.gemm_bf16(int(op), int(A.data_ptr()), _ld(A), int(B.data_ptr()), _ld(B), int(C.data_ptr()), _ld(C),
                         _dtype_code(C), int(M), int(N), int(K), int(split_k),
                         int(workspace.data_ptr()) if workspace is not None else 0, nbytes, _stream_handle(stream)),
           "gemm_bf16")


def attn_prof_enable(capacity: int) -> None:
    _check(lib.attn_prof_enable(int(capacity)), "attn_prof_enable")


def attn_prof_read() -> dict:
    """{kernel name: (launches, total_ms)} accumulated since the last read."""
    buf = (_KernelTime * 16)()
    n = lib.attn_prof_read(buf, 16)
    if n < 0:
        raise AttnError(ATTN_ELAUNCH, "attn_prof_read", "HIP event query failed")
    return {buf[i].kernel.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n, 16))}


def _init_current_device():
    import torch

    if torch.cuda.is_available():
        attn_init()


_init_current_device()
