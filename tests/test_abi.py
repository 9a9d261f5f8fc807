"""C-ABI checks that need no GPU: every symbol declared in include/attn.h is
exported by libattn.so, status strings, workspace arithmetic, and host-side
argument validation (which returns before any HIP call, so fake, never
dereferenced pointers are safe).  The one case with fully valid arguments is
run only where no GPU is present, where it must report ATTN_ELAUNCH."""
import ctypes
import os
import re

import pytest

import causal_attention_attn_amd as ca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = ca.lib

# fake, 16-byte aligned, far-apart addresses (never dereferenced: validation fails first)
MB = 1 << 20
A = [0x100000000 + i * 256 * MB for i in range(12)]


def _gpu_present():
    import torch

    return torch.cuda.is_available()


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b((?:attn|gemm)_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_status_str", "attn_last_error",
            "attn_fwd_strided", "gemm_bf16", "gemm_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(L, n), "libattn.so does not export " + n
    nm = os.popen("nm -D --defined-only %s" % ca.library_path()).read()
    for n in names:
        assert re.search(r"\bT %s\b" % n, nm), n


def test_status_strings():
    assert [ca.attn_status_str(i) for i in range(4)] == ["ATTN_OK", "ATTN_EINVAL", "ATTN_EUNSUPPORTED", "ATTN_ELAUNCH"]
    assert ca.attn_status_str(17) == "unknown"


def test_workspace_bytes():
    assert ca.attn_bwd_workspace_bytes(ca.ATTN_BF16, 8, 12, 1024, 64) == 8 * 12 * 1024 * 4
    # the atomic path: D, then the fp32 dQ accumulator (B*H*T*d); bf16 only
    assert ca.attn_bwd_atomic_workspace_bytes(ca.ATTN_BF16, 8, 12, 1024, 64) == 8 * 12 * 1024 * 4 * (1 + 64)
    assert ca.attn_bwd_atomic_workspace_bytes(ca.ATTN_F32, 8, 12, 1024, 64) == 0
    assert "bf16 only" in ca.attn_last_error()
    assert ca.attn_bwd_workspace_bytes(ca.ATTN_F32, 1, 1, 3, 32) == 256  # padded to 256 bytes
    assert ca.attn_bwd_workspace_bytes(ca.ATTN_BF16, 1, 1, 1, 48) == 0
    assert "head_dim" in ca.attn_last_error()
    assert ca.attn_bwd_workspace_bytes(ca.ATTN_BF16, 0, 1, 1, 64) == 0


def fwd(dt=ca.ATTN_BF16, Q=A[0], K=A[1], V=A[2], O=A[3], LSE=A[4], B=2, H=3, T=100, d=64, scale=0.125, causal=1):
    return L.attn_fwd(dt, Q, K, V, O, LSE, B, H, T, d, ctypes.c_float(scale), causal, None)


def bwd(dt=ca.ATTN_BF16, Q=A[0], K=A[1], V=A[2], O=A[3], dO=A[4], LSE=A[5], dQ=A[6], dK=A[7], dV=A[8],
        ws=A[9], wsb=None, B=2, H=3, T=100, d=64, scale=0.125, causal=1, atomic=False):
    if wsb is None:
        wsb = (ca.attn_bwd_atomic_workspace_bytes if atomic else ca.attn_bwd_workspace_bytes)(dt, B, H, T, d)
    fn = L.attn_bwd_atomic if atomic else L.attn_bwd
    return fn(dt, Q, K, V, O, dO, LSE, dQ, dK, dV, ws, wsb, B, H, T, d, ctypes.c_float(scale), causal, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Q=0), ca.ATTN_EINVAL, "Q is null"),
    (dict(LSE=0), ca.ATTN_EINVAL, "LSE is null"),
    (dict(B=0), ca.ATTN_EINVAL, ">= 1"),
    (dict(T=-5), ca.ATTN_EINVAL, ">= 1"),
    (dict(d=48), ca.ATTN_EUNSUPPORTED, "head_dim"),
    (dict(d=256), ca.ATTN_EUNSUPPORTED, "head_dim"),
    (dict(dt=7), ca.ATTN_EUNSUPPORTED, "dtype"),
    (dict(scale=float("nan")), ca.ATTN_EINVAL, "finite"),
    (dict(scale=float("inf")), ca.ATTN_EINVAL, "finite"),
    (dict(K=A[1] + 8), ca.ATTN_EINVAL, "aligned"),
    (dict(O=A[0] + 1024), ca.ATTN_EINVAL, "overlaps input Q"),
    (dict(LSE=A[3] + 16), ca.ATTN_EINVAL, "overlaps output LSE"),
    (dict(B=65536, H=65536, T=65536), ca.ATTN_EINVAL, "exceeds"),
])
def test_fwd_validation(kw, status, msg):
    assert fwd(**kw) == status
    assert msg in ca.attn_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dO=0), ca.ATTN_EINVAL, "dO is null"),
    (dict(ws=0), ca.ATTN_EINVAL, "workspace is null"),
    (dict(wsb=16), ca.ATTN_EINVAL, "workspace too small"),
    (dict(dV=A[2]), ca.ATTN_EINVAL, "overlaps input V"),
    (dict(dK=A[6]), ca.ATTN_EINVAL, "output dQ overlaps output dK"),
    (dict(ws=A[8] + 64), ca.ATTN_EINVAL, "output dV overlaps output workspace"),
    (dict(d=16), ca.ATTN_EUNSUPPORTED, "head_dim"),
    (dict(H=0), ca.ATTN_EINVAL, ">= 1"),
    (dict(scale=float("-inf")), ca.ATTN_EINVAL, "finite"),
    (dict(LSE=A[5] + 4), ca.ATTN_EINVAL, "aligned"),
])
def test_bwd_validation(kw, status, msg):
    for atomic in (False, True):
        assert bwd(atomic=atomic, **kw) == status
        assert msg in ca.attn_last_error()


def test_atomic_path_needs_the_larger_workspace_and_bf16():
    small = ca.attn_bwd_workspace_bytes(ca.ATTN_BF16, 2, 3, 100, 64)
    assert bwd(wsb=small, atomic=True) == ca.ATTN_EINVAL and "workspace too small" in ca.attn_last_error()
    assert bwd(dt=ca.ATTN_F32, wsb=1 << 20, atomic=True) == ca.ATTN_EUNSUPPORTED


def test_valid_arguments_without_a_device_report_launch_error():
    if _gpu_present():
        pytest.skip("a GPU is present: fake pointers must not reach a real launch")
    assert fwd() == ca.ATTN_ELAUNCH
    assert bwd() == ca.ATTN_ELAUNCH
    assert bwd(atomic=True) == ca.ATTN_ELAUNCH
    assert ca.attn_last_error() != ""


def test_init_without_device():
    """attn_init launches nothing; where no GPU is present it reports ATTN_ELAUNCH."""
    if _gpu_present():
        pytest.skip("a GPU is present (attn_init is exercised by the GPU tests)")
    assert L.attn_init() == ca.ATTN_ELAUNCH
    assert "device" in ca.attn_last_error()
