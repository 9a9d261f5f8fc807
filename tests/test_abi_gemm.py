"""Host-side checks of the GEMM entry points (no GPU): workspace sizing and
argument validation, which fails before any HIP call (fake, never
dereferenced addresses).  The accepted call reports ATTN_ELAUNCH here and
runs only where no GPU is present."""
import ctypes

import pytest

import causal_attention_attn_amd as ca

L = ca.lib
MB = 1 << 20
P = [0x100000000 + i * 512 * MB for i in range(6)]


def _no_gpu():
    import torch

    return not torch.cuda.is_available()


def call(op=ca.GEMM_NT, A=P[0], lda=768, B=P[1], ldb=768, C=P[2], ldc=2304, ct=ca.ATTN_BF16, M=8192, N=2304, K=768,
         split=1, ws=0, wsb=0):
    return L.gemm_bf16(op, A, lda, B, ldb, C, ldc, ct, M, N, K, split, ws, wsb, None)


def test_workspace_bytes():
    assert ca.gemm_workspace_bytes(ca.GEMM_NT, 8192, 2304, 768, 1) == 0
    # dW of a GPT-2 MLP layer: K = 8192 tokens, 8 chunks of 1024
    assert ca.gemm_workspace_bytes(ca.GEMM_TN, 3072, 768, 8192, 8) == 8 * 3072 * 768 * 4
    # chunks of ceil(16/3) = 6 contraction tiles: 6 + 6 + 4, three partial products
    assert ca.gemm_workspace_bytes(ca.GEMM_TN, 64, 64, 1024, 3) == 3 * 64 * 64 * 4
    # 5 requested splits of 8 tiles -> chunks of 2 tiles -> 4 partial products
    assert ca.gemm_workspace_bytes(ca.GEMM_NN, 8, 8, 512, 5) == 4 * 8 * 8 * 4
    assert ca.gemm_workspace_bytes(ca.GEMM_NT, 8, 8, 100, 1) == 0 and "multiple of 64" in ca.attn_last_error()


def test_automatic_split():
    """split_k = 0 takes the largest split whose workgroups (128 x 128 output
    tiles x splits) all fit the 512 resident slots, with >= 8 contraction
    tiles per chunk; the workspace query shows which."""
    ws = lambda op, M, N, K: ca.gemm_workspace_bytes(op, M, N, K, 0)
    # GPT-2-small MLP: X W1^T has 1536 tiles and dY W1 384: neither is split
    assert ws(ca.GEMM_NT, 8192, 3072, 768) == 0
    assert ws(ca.GEMM_NN, 8192, 768, 3072) == 0
    # dY^T X: 144 tiles, 3 x 144 = 432 <= 512 < 4 x 144
    assert ws(ca.GEMM_TN, 3072, 768, 8192) == 3 * 3072 * 768 * 4
    # one tile, K = 1024 (16 contraction tiles): at most 2 chunks of >= 8
    assert ws(ca.GEMM_NT, 128, 128, 1024) == 2 * 128 * 128 * 4
    # one tile, K = 448 (7 contraction tiles): no chunk of 8, so unsplit
    assert ws(ca.GEMM_NT, 128, 128, 448) == 0
    assert ca.gemm_workspace_bytes(ca.GEMM_NT, 8, 8, 128, 3) == 0 and "split_k" in ca.attn_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(A=0), ca.ATTN_EINVAL, "A is null"),
    (dict(C=0), ca.ATTN_EINVAL, "C is null"),
    (dict(B=P[1] + 8), ca.ATTN_EINVAL, "aligned"),
    (dict(K=700, lda=704, ldb=704), ca.ATTN_EUNSUPPORTED, "multiple of 64"),
    (dict(N=2300, ldc=2304), ca.ATTN_EUNSUPPORTED, "multiple of 8"),
    (dict(op=ca.GEMM_TN, M=100, lda=104, ldb=2304, K=768, N=2304), ca.ATTN_EUNSUPPORTED, "multiple of 8"),
    (dict(op=7), ca.ATTN_EUNSUPPORTED, "gemm_op"),
    (dict(ct=5), ca.ATTN_EUNSUPPORTED, "dtype"),
    (dict(M=0), ca.ATTN_EINVAL, ">= 1"),
    (dict(lda=512), ca.ATTN_EINVAL, "leading dimension"),
    (dict(ldb=1 << 23), ca.ATTN_EINVAL, "below 2^23"),
    (dict(ldc=2308), ca.ATTN_EINVAL, "multiple of 8"),
    (dict(split=13), ca.ATTN_EINVAL, "split_k"),
    (dict(split=-1), ca.ATTN_EINVAL, "split_k"),
    (dict(split=4), ca.ATTN_EINVAL, "workspace too small"),
    (dict(C=P[0] + 4096), ca.ATTN_EINVAL, "output C overlaps input A"),
    (dict(split=4, ws=P[2] + 1024, wsb=1 << 30), ca.ATTN_EINVAL, "output C overlaps output workspace"),
])
def test_validation(kw, status, msg):
    assert call(**kw) == status
    assert msg in ca.attn_last_error()


@pytest.mark.skipif(not _no_gpu(), reason="fake pointers must not reach a real launch")
def test_valid_arguments_report_launch_error_without_a_device():
    assert call() == ca.ATTN_ELAUNCH
    # TN: A = dY [K, M], B = X [K, N]; split over the 8192-token contraction
    assert call(op=ca.GEMM_TN, lda=3072, ldb=768, ldc=768, M=3072, N=768, K=8192, split=8, ws=P[3],
                wsb=8 * 3072 * 768 * 4) == ca.ATTN_ELAUNCH
