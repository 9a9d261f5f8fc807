"""attn_bwd_noalloc: attn_bwd with D in the library's static device array
instead of a caller workspace, for callers that cannot allocate.  Through the
C ABI it must give bitwise the results of attn_bwd (same kernels), call after
call with shrinking inputs (the array keeps the last call's contents), and
refuse inputs beyond its fixed size before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import causal_attention_attn_amd as ca

L = ca.lib


def test_oversize_rejected_on_host():
    """B*H*T one row past the limit: ATTN_EINVAL from the host check (fake,
    never dereferenced pointers; no GPU needed)."""
    p = [0x100000000 + i * (1 << 28) for i in range(9)]
    T = ca.NOALLOC_MAX_ROWS // 2 + 1  # B=1, H=2
    st = L.attn_bwd_noalloc(ca.ATTN_BF16, *p, 1, 2, T, 64, ctypes.c_float(0.125), 1, None)
    assert st == ca.ATTN_EINVAL
    assert "static scratch" in ca.attn_last_error()


def _run_pair(B, H, T, d, dtype, causal, seed):
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, T, d)
    Q, K, V, dO = (torch.randn(shape, generator=g).to(dtype).cuda() for _ in range(4))
    O = torch.empty(shape, dtype=dtype, device="cuda")
    LSE = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    scale = d ** -0.5
    ca.attn_fwd(Q, K, V, O, LSE, scale, causal)
    code = ca.ATTN_BF16 if dtype == torch.bfloat16 else ca.ATTN_F32
    ws = torch.empty(ca.attn_bwd_workspace_bytes(code, B, H, T, d, causal), dtype=torch.uint8, device="cuda")
    ref = [torch.full(shape, float("nan"), dtype=dtype, device="cuda") for _ in range(3)]
    ca.attn_bwd(Q, K, V, O, dO, LSE, *ref, ws, scale, causal)
    got = [torch.full(shape, float("nan"), dtype=dtype, device="cuda") for _ in range(3)]
    ca.attn_bwd_noalloc(Q, K, V, O, dO, LSE, *got, scale, causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert not torch.isnan(a).any(), "%s not fully written by attn_bwd_noalloc" % name
        assert torch.equal(a, b), "%s of attn_bwd_noalloc differs from attn_bwd" % name


@pytest.mark.gpu
def test_noalloc_equals_attn_bwd_twice_shrinking():
    """Two calls in a row, the second on a smaller input: both bitwise equal
    to attn_bwd on the same inputs."""
    print("[gpu] attn_bwd_noalloc B2 H3 T1000 d64 bf16, then B1 H2 T200 d64", flush=True)
    _run_pair(2, 3, 1000, 64, torch.bfloat16, True, seed=1)
    _run_pair(1, 2, 200, 64, torch.bfloat16, True, seed=2)


@pytest.mark.gpu
def test_noalloc_other_shapes():
    print("[gpu] attn_bwd_noalloc d128 bf16, d32 f32, limit-sized bf16", flush=True)
    _run_pair(1, 2, 333, 128, torch.bfloat16, True, seed=3)
    _run_pair(1, 2, 130, 32, torch.float32, False, seed=4)
    _run_pair(1, 32, ca.NOALLOC_MAX_ROWS // 32, 32, torch.bfloat16, True, seed=5)  # exactly at the limit
