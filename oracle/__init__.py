"""fp64 CPU oracle for causal scaled-dot-product attention (forward + backward).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, explicit T x T
matrices, no tiling) and follows the definition of attention that the Forge
paper's kernels compute (Forge, section "Attention kernel design": online
softmax forward with a saved logsumexp; section "Ecosystem survey": backward
through D = rowsum(dO o O)).  This module only builds the C file and marshals
numpy arrays through ctypes.

Parity pins (tests/test_oracle.py): central finite differences of L = <dO, O>
(Forge, section "Methodology and reproducibility": gradients are checked against
central finite differences), closed forms for uniform queries, equal keys, row
0 and T = 1, the key-shift and scale invariants, causality, and torch's CPU
float64 scaled_dot_product_attention.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_attn.so")

_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile attn_oracle.c with gcc -O2 (no -ffast-math) into a shared library."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
             "-o", tmp, src, "-lm"]
        )
        os.replace(tmp, out)
    return out


def load_library(path: str):
    """ctypes handle on a built oracle library (the default one, or a test build)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_attn_fwd.argtypes = [ctypes.c_int] * 3 + [ctypes.c_double, ctypes.c_int] + [dp] * 5 + [ctypes.c_int]
    lib.oracle_attn_fwd.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [ctypes.c_int] * 3 + [ctypes.c_double, ctypes.c_int] + [dp] * 10 + [ctypes.c_int]
    lib.oracle_attn_bwd.restype = ctypes.c_int
    lib.oracle_threads_default.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = load_library(_LIB)
    return _lib


def _threads(threads: int) -> int:
    """0 = one thread per CPU, at most 16 (a GPU host's per-GPU CPU share)."""
    return int(threads) if threads > 0 else max(1, min(16, os.cpu_count() or 1))


def _as_f64(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return int(_load().oracle_threads_default())


def attn_fwd(Q, K, V, scale: float, causal: bool, threads: int = 0, lib=None):
    """O [..., T, d] and LSE [..., T] in float64 for inputs shaped [..., T, d]."""
    Q, K, V = _as_f64(Q), _as_f64(K), _as_f64(V)
    assert Q.shape == K.shape == V.shape and Q.ndim >= 2
    T, d = Q.shape[-2:]
    BH = int(np.prod(Q.shape[:-2], dtype=np.int64)) if Q.ndim > 2 else 1
    O = np.empty_like(Q)
    LSE = np.empty(Q.shape[:-1], dtype=np.float64)
    rc = (lib or _load()).oracle_attn_fwd(BH, T, d, float(scale), int(bool(causal)), _ptr(Q), _ptr(K),
                                 _ptr(V), _ptr(O), _ptr(LSE), _threads(threads))
    if rc:
        raise RuntimeError("oracle_attn_fwd failed with code %d" % rc)
    return O, LSE


def attn_bwd(Q, K, V, dO, scale: float, causal: bool, threads: int = 0, lib=None):
    """dQ, dK, dV, O, LSE, D (= rowsum(dO o O)) in float64; the gradients are
    those of L = <dO, O> with O = softmax(scale Q K^T, mask) V."""
    Q, K, V, dO = _as_f64(Q), _as_f64(K), _as_f64(V), _as_f64(dO)
    assert Q.shape == K.shape == V.shape == dO.shape and Q.ndim >= 2
    T, d = Q.shape[-2:]
    BH = int(np.prod(Q.shape[:-2], dtype=np.int64)) if Q.ndim > 2 else 1
    dQ, dK, dV, O = (np.empty_like(Q) for _ in range(4))
    LSE = np.empty(Q.shape[:-1], dtype=np.float64)
    D = np.empty(Q.shape[:-1], dtype=np.float64)
    rc = (lib or _load()).oracle_attn_bwd(BH, T, d, float(scale), int(bool(causal)), _ptr(Q), _ptr(K),
                                 _ptr(V), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(O),
                                 _ptr(LSE), _ptr(D), _threads(threads))
    if rc:
        raise RuntimeError("oracle_attn_bwd failed with code %d" % rc)
    return dQ, dK, dV, O, LSE, D
