/*
 * gemm.h -- C ABI of the layer products next to attention in a GPT-2
 * decoder step (same library, libattn.so): bf16 operands, fp32
 * accumulation on the gfx950 matrix cores, bf16 or fp32 output.
 *
 * The three products are the ones Forge times for its MLP ("Forge: Building
 * an LLM Training Framework from Scratch in C++ and Metal on Apple Silicon",
 * section "Results", GEMM table): the forward X W^T with weights stored
 * [out, in], the input gradient dX = dY W and the weight gradient
 * dW = dY^T X, whose contraction runs over all B*T tokens.  Forge notes
 * that this last case lags for want of a split of the contraction; here
 * split_k cuts it over workgroups.
 *
 * Conventions
 *   Layout     row-major with leading dimensions (elements between rows):
 *                GEMM_NT  C[M,N] = A[M,K] * B[N,K]^T    lda >= K, ldb >= K
 *                GEMM_NN  C[M,N] = A[M,K] * B[K,N]      lda >= K, ldb >= N
 *                GEMM_TN  C[M,N] = A[K,M]^T * B[K,N]    lda >= M, ldb >= N
 *              ldc >= N.  lda, ldb, ldc are multiples of 8 and below 2^23,
 *              and every pointer is 16-byte aligned (else ATTN_EINVAL).
 *   Shapes     M, N, K >= 1; K a multiple of 64; N a multiple of 8 (and M
 *              for GEMM_TN).  Other shapes: ATTN_EUNSUPPORTED.
 *   Numerics   every product of two bf16 values is exact in fp32; sums run
 *              in fp32 in a fixed order, so results are bitwise reproducible
 *              for a given split_k.  bf16 output is rounded to nearest even.
 *   split_k    1: one pass over K.  s > 1: the contraction is cut into
 *              chunks of ceil(K/64/s)*64; each chunk's fp32 partial product
 *              goes to the workspace and a second kernel adds them in chunk
 *              order.  0: chosen from the shape (gemm_workspace_bytes with
 *              split_k = 0 sizes the workspace for that choice).
 *   Ownership  device memory owned by the caller; the library enqueues on
 *              `stream` and never allocates, frees or synchronises.
 *   Errors     checked on the host before any launch, as for attn.h:
 *              EINVAL for null or misaligned pointers, bad leading
 *              dimensions or split_k, a short workspace, or C overlapping A,
 *              B or the workspace; attn_last_error() gives the detail.
 */
#ifndef ATTN_GEMM_H
#define ATTN_GEMM_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GEMM_NT = 0, GEMM_NN = 1, GEMM_TN = 2 } gemm_op;

/*
 * Bytes of fp32 workspace gemm_bf16 needs for this shape and split_k: 0 when
 * the contraction is not split, else (number of non-empty chunks) * M * N * 4
 * rounded up to 256.  Returns 0 with attn_last_error() set on invalid input.
 */
size_t gemm_workspace_bytes(gemm_op op, int M, int N, int K, int split_k);

/*
 * C = op(A) op(B) as in the table above; c_type is ATTN_BF16 or ATTN_F32.
 * workspace may be null when gemm_workspace_bytes(...) is 0.
 */
attn_status gemm_bf16(gemm_op op, const void *A, int lda, const void *B, int ldb, void *C, int ldc,
                      attn_dtype c_type, int M, int N, int K, int split_k, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GEMM_H */
