"""GPU parity of the layer GEMMs (gemm_bf16 through the C ABI) against the
fp64 oracle (oracle/gemm.py) on the same seeded bf16 operands.

Bar, element by element: any fp32 summation order of K exact products errs
by at most gamma_K * sum_k |a_ik b_kj| (gamma_K = K u / (1 - K u),
u = 2^-24); a bf16 output adds one rounding of at most 2^-8 of the value.
Cases: every operation with ragged M (and N, K not multiples of the
128 x 128 x 64 tiles), padded leading dimensions, bf16 and fp32 outputs,
split_k of 1, 2, 3 and automatic; the GPT-2-small MLP products at full size
on sampled output rows; bitwise repeatability.  C is NaN-prefilled with
guard bands and row padding that must stay untouched.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import causal_attention_attn_amd as ca
from gpu_util import GUARD, log
from oracle import gemm as og

pytestmark = pytest.mark.gpu

OPC = {"NT": ca.GEMM_NT, "NN": ca.GEMM_NN, "TN": ca.GEMM_TN}
U32 = 2.0 ** -24


def _dev(bits, ld=None):
    """bf16 device matrix from uint16 bits, optionally with row padding to ld."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    rows, cols = t.shape
    if ld is None or ld == cols:
        return t.to("cuda")
    full = torch.zeros((rows, ld), dtype=torch.bfloat16)
    full[:, :cols] = t
    return full.to("cuda")[:, :cols]


class GuardedC:
    def __init__(self, M, N, ldc, dtype):
        self.full = torch.full((M * ldc + 2 * GUARD,), float("nan"), dtype=dtype, device="cuda")
        self.mat = self.full[GUARD:GUARD + M * ldc].view(M, ldc)
        self.view = self.mat[:, :N]
        self.M, self.N = M, N

    def check_untouched(self):
        g = torch.cat([self.full[:GUARD], self.full[GUARD + self.mat.numel():]])
        assert bool(torch.isnan(g).all()), "guard band written"
        if self.mat.shape[1] > self.N:
            assert bool(torch.isnan(self.mat[:, self.N:]).all()), "row padding written"


def run(op, A_bits, B_bits, M, N, K, ct=torch.bfloat16, split=1, pad=0):
    lda = (A_bits.shape[1] + pad) if pad else None
    ldb = (B_bits.shape[1] + pad) if pad else None
    A, B = _dev(A_bits, lda), _dev(B_bits, ldb)
    C = GuardedC(M, N, N + pad, ct)
    nb = ca.gemm_workspace_bytes(OPC[op], M, N, K, split)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda") if nb else None
    log("[gpu] gemm %s M=%d N=%d K=%d out=%s split=%d pad=%d" % (op, M, N, K, ct, split, pad))
    ca.gemm(OPC[op], A, B, C.view, split, ws)
    torch.cuda.synchronize()
    C.check_untouched()
    return C


def check(op, C, A, B, rows=None):
    got = C.view.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
        ref = og.gemm_rows(op, A, B, rows)
        bound_src = (np.abs(A), np.abs(B))
        absp = og.gemm_rows(op, *bound_src, rows)
    else:
        ref = og.gemm(op, A, B)
        absp = og.abs_product(op, A, B)
    assert not np.isnan(got).any(), "%d outputs never written" % int(np.isnan(got).sum())
    K = A.shape[1] if op in ("NT", "NN") else A.shape[0]
    gam = K * U32 / (1 - K * U32)
    tol = gam * absp
    if C.view.dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(tol, 1e-300)))
    assert np.all(err <= tol), "max err/bound = %.3g (max abs err %.3g)" % (worst, float(err.max()))
    return worst


SMALL = [("NT", 200, 136, 192), ("NN", 200, 136, 192), ("TN", 136, 264, 256), ("NT", 8, 8, 64),
         ("TN", 8, 128, 64), ("NN", 300, 392, 448)]


@pytest.mark.parametrize("op,M,N,K", SMALL)
@pytest.mark.parametrize("ct", [torch.bfloat16, torch.float32])
def test_small_ragged(op, M, N, K, ct):
    sa, sb = ai.gemm_operand_shapes(op, M, N, K)
    Ab, A = ai.make_matrix(sa, seed=M + 7 * N + 13 * K)
    Bb, B = ai.make_matrix(sb, seed=M + 7 * N + 13 * K + 1)
    for split in (1, 2, 3, 0):
        if split > K // 64:
            continue
        for pad in (0, 8):
            C = run(op, Ab, Bb, M, N, K, ct, split, pad)
            check(op, C, A, B)


# Shapes whose tile walk takes groups of 2, 4 and 1 m-tiles, the last group
# of a chunk partial where the group does not divide the m-tiles (the host
# test of the work order checks these choices: 5 x 8 tiles -> 2, 7 x 8 -> 4,
# 6 x 4 in two chunks -> 1, 6 x 6 in two chunks -> 4).  Every output must be
# written once: a tile the walk skipped stays NaN.
WALK = [("NT", 600, 1000, 192, 1), ("TN", 848, 1016, 128, 1), ("NN", 700, 512, 256, 2), ("NT", 768, 712, 256, 2)]


@pytest.mark.parametrize("op,M,N,K,split", WALK)
def test_walk_groups(op, M, N, K, split):
    sa, sb = ai.gemm_operand_shapes(op, M, N, K)
    Ab, A = ai.make_matrix(sa, seed=3 * M + N + K)
    Bb, B = ai.make_matrix(sb, seed=3 * M + N + K + 1)
    C = run(op, Ab, Bb, M, N, K, torch.bfloat16, split)
    check(op, C, A, B)


@pytest.mark.parametrize("name", ["mlp_fwd", "mlp_dx", "mlp_dw"])
def test_gpt2_mlp_products_sampled_rows(name):
    op, M, N, K = ai.GEMM_WORKLOADS[name]
    sa, sb = ai.gemm_operand_shapes(op, M, N, K)
    Ab, A = ai.make_matrix(sa, seed=100 + len(name))
    Bb, B = ai.make_matrix(sb, seed=200 + len(name))
    rows = [0, 1, 127, 128, M // 2 + 5, M - 1]
    for split in (1, 0):
        C = run(op, Ab, Bb, M, N, K, torch.bfloat16, split)
        w = check(op, C, A, B, rows)
        log("%s split=%d worst err/bound %.3g" % (name, split, w))


def test_repeatable():
    op, M, N, K = "TN", 264, 136, 1024
    sa, sb = ai.gemm_operand_shapes(op, M, N, K)
    Ab, _ = ai.make_matrix(sa, seed=5)
    Bb, _ = ai.make_matrix(sb, seed=6)
    for split in (1, 4, 0):
        a = run(op, Ab, Bb, M, N, K, torch.float32, split).view.clone()
        b = run(op, Ab, Bb, M, N, K, torch.float32, split).view.clone()
        assert torch.equal(a, b), split


@pytest.mark.parametrize("op", ["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (8000, 6144, 128)])
def test_large_tiles_sampled_rows(op, M, N, K):
    """Shapes with enough 256 x 256 tiles to fill the chip take the 8-wave
    large-tile kernel (the second with a ragged last row of tiles)."""
    sa, sb = ai.gemm_operand_shapes(op, M, N, K)
    Ab, A = ai.make_matrix(sa, seed=M + K)
    Bb, B = ai.make_matrix(sb, seed=N + K)
    rows = [0, 31, 32, 255, 256, M // 2 + 3, M - 65, M - 1]
    for ct in (torch.bfloat16, torch.float32):
        C = run(op, Ab, Bb, M, N, K, ct, 1)
        check(op, C, A, B, rows)
