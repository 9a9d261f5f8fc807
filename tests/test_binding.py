"""Python binding checks that need no GPU: every tensor handed to the C ABI
must have Q's shape and element type (LSE float32 [B, H, T]) and live on Q's
GPU.  The library only sees bare pointers, so these mismatches would reach the
kernels as out-of-bounds or host addresses; the binding must raise before any
library call.  The library handle is replaced by a recorder for each test, so
a call that got through would be seen."""
import pytest
import torch

import causal_attention_attn_amd as ca


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*args):
            self.calls.append(name)
            return 0
        return f


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(ca, "lib", r)
    return r


SHAPE = (2, 3, 17, 32)


def t(shape=SHAPE, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def fwd_args(**kw):
    a = dict(Q=t(), K=t(), V=t(), O=t(), LSE=torch.zeros(SHAPE[:3], dtype=torch.float32))
    a.update(kw)
    return a


def bwd_args(**kw):
    a = dict(Q=t(), K=t(), V=t(), O=t(), dO=t(), LSE=torch.zeros(SHAPE[:3], dtype=torch.float32),
             dQ=t(), dK=t(), dV=t(), workspace=torch.zeros(4096, dtype=torch.uint8))
    a.update(kw)
    return a


FWD_CASES = [
    (dict(K=t((2, 3, 16, 32))), ValueError, "K has shape"),
    (dict(O=t((2, 3, 17, 64))), ValueError, "O has shape"),
    (dict(V=t(dtype=torch.float32)), TypeError, "V is torch.float32"),
    (dict(O=t(dtype=torch.float32)), TypeError, "O is torch.float32"),
    (dict(LSE=torch.zeros(SHAPE[:3], dtype=torch.bfloat16)), ValueError, "LSE must be float32"),
    (dict(LSE=torch.zeros(SHAPE[:2], dtype=torch.float32)), ValueError, "LSE must be float32"),
    (dict(Q=t(dtype=torch.float16), K=t(dtype=torch.float16), V=t(dtype=torch.float16),
          O=t(dtype=torch.float16)), TypeError, "unsupported dtype"),
    (dict(), ValueError, "must be a GPU tensor"),  # consistent, but host tensors
]


@pytest.mark.parametrize("kw,exc,msg", FWD_CASES)
@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_strided"])
def test_fwd_rejects(rec, fn, kw, exc, msg):
    a = fwd_args(**kw)
    with pytest.raises(exc, match=msg):
        getattr(ca, fn)(a["Q"], a["K"], a["V"], a["O"], a["LSE"], 0.125, True)
    assert rec.calls == []


BWD_CASES = [
    (dict(dO=t((2, 3, 17, 16))), ValueError, "dO has shape"),
    (dict(dV=t((1, 3, 17, 32))), ValueError, "dV has shape"),
    (dict(dQ=t(dtype=torch.float32)), TypeError, "dQ is torch.float32"),
    (dict(LSE=torch.zeros((2, 3, 18), dtype=torch.float32)), ValueError, "LSE must be float32"),
    (dict(dK=None), ValueError, "dK is missing"),
    (dict(), ValueError, "must be a GPU tensor"),
]


@pytest.mark.parametrize("kw,exc,msg", BWD_CASES)
@pytest.mark.parametrize("fn", ["attn_bwd", "attn_bwd_atomic", "attn_bwd_strided", "attn_bwd_atomic_strided"])
def test_bwd_rejects(rec, fn, kw, exc, msg):
    a = bwd_args(**kw)
    with pytest.raises(exc, match=msg):
        getattr(ca, fn)(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"],
                        a["workspace"], 0.125, True)
    assert rec.calls == []


def test_gemm_rejects(rec):
    A = torch.zeros((64, 64), dtype=torch.bfloat16)
    B = torch.zeros((64, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="C must be bfloat16 or float32"):
        ca.gemm(ca.GEMM_NT, A, B, torch.zeros((64, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="shape mismatch"):
        ca.gemm(ca.GEMM_NT, A, B, torch.zeros((64, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        ca.gemm(ca.GEMM_NT, A, B, torch.zeros((64, 64), dtype=torch.bfloat16))
    assert rec.calls == []
