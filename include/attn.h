/*
 * attn.h -- C ABI of the MI355X (gfx950) fused causal attention library
 * (libattn.so): scaled-dot-product attention forward and backward for one
 * decoder layer, on caller-owned device memory and a caller stream.
 *
 * What is computed, per batch b and head h (Q, K, V, O, dO in R^{T x d},
 * s = scale, A_i = {j <= i} when causal, else all j):
 *   S = s Q K^T,  P_ij = exp(S_ij - LSE_i) on A_i and 0 elsewhere,
 *   LSE_i = ln sum_{j in A_i} exp(S_ij),  O = P V;
 *   backward of L = <dO, O>:  D_i = sum_c dO_ic O_ic,  dV = P^T dO,
 *   dS = P o (dO V^T - D 1^T),  dQ = s dS K,  dK = s dS^T Q.
 * Sources: Forge (S.-P. Boucher, 2026), section "Attention kernel design"
 * (tiled forward with online softmax; the saved logsumexp fixes the
 * normalisation of the backward; transposed score tiles by operand-role
 * exchange) and section "Ecosystem survey" (three-stage backward: a
 * preprocessing kernel for D = rowsum(dO o O) in float, a dQ kernel parallel
 * over queries and a dK/dV kernel parallel over key/value rows).  Causal masking
 * is the decoder-only convention of that paper's models (section "Introduction").
 *
 * Conventions shared by every entry point
 *   Layout     Q, K, V, O, dO, dQ, dK, dV: row-major [B, H, T, d] of the
 *              element type `dt` (fp32 or bf16), contiguous for the plain
 *              entry points and any view with a unit-stride d index for the
 *              *_strided ones; LSE and D: contiguous [B, H, T] fp32.  Every
 *              pointer is 16-byte aligned.
 *   Ownership  all pointers are device memory owned by the caller.  The
 *              library never allocates device memory, frees or synchronises on
 *              these calls: it enqueues kernels on `stream` (0 = the null
 *              stream) and returns before they run.  Device faults surface at
 *              the caller's next synchronisation.  With the timing hooks
 *              off (the default), a call records nothing but kernel
 *              launches (no memset, copy or event), so it can be captured
 *              into a HIP graph by stream capture and replayed on new
 *              contents of the same buffers.
 *   Causal     square self-attention, top-left aligned: query i sees keys
 *              j <= i.  causal = 0 lets every query see every key.
 *   Units      LSE is the natural-log logsumexp of the scaled scores.
 *   Values     inputs must be finite.  The library is built with NaN
 *              semantics relaxed (the maxima of the online softmax skip NaN
 *              quieting), so a NaN anywhere in Q, K, V, O, dO or LSE gives
 *              unspecified outputs (not necessarily NaN).  Infinite scores
 *              are not produced from finite inputs.
 *   Errors     arguments are checked on the host before anything is launched;
 *              on any non-OK status nothing was enqueued, and attn_last_error()
 *              returns a thread-local description.  ATTN_ELAUNCH reports a HIP
 *              error at launch (no device, no gfx950 code object, bad stream).
 *   Threads    the library holds no per-call state: calls from several host
 *              threads or on several streams are independent.  attn_fwd and
 *              attn_bwd are bitwise deterministic; attn_bwd_atomic is too
 *              except for the order of dQ's fp32 atomic additions.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_EINVAL = 1,      /* bad pointer, size, alignment, aliasing, scale or workspace */
    ATTN_EUNSUPPORTED = 2, /* head_dim not in {32, 64, 128} or unknown dtype */
    ATTN_ELAUNCH = 3       /* HIP reported an error when launching */
} attn_status;

/*
 * Optional one-time set-up on the calling thread's current device: reads the
 * device's compute-unit count and the occupancy of every kernel variant (the
 * work order of the causal kernels depends on both).  Without it each entry
 * point makes these queries on its first call on a device.  Calling attn_init
 * first, on each device, keeps those queries out of a later stream capture,
 * so that even the first call ever made can be captured into a HIP graph.
 * It also resolves the device address of attn_bwd_noalloc's static array.
 * Launches nothing.  ATTN_ELAUNCH when no device can be queried.
 */
attn_status attn_init(void);

/*
 * Forward pass (Forge, section "Attention kernel design": the tiled forward
 * with an online softmax that saves the logsumexp).
 *   Q, K, V  in  [B,H,T,head_dim], type dt
 *   O        out [B,H,T,head_dim], type dt (bf16 outputs are rounded to nearest even)
 *   LSE      out [B,H,T] fp32, natural log of sum_j exp(scale * q_i . k_j) over visible j
 *   scale    finite; any sign (1/sqrt(head_dim) is the usual choice)
 * EINVAL: a null pointer, B/H/T < 1, element count overflow, a non-finite
 * scale, a pointer not 16-byte aligned, or an output overlapping an input or
 * the other output.  EUNSUPPORTED: head_dim or dt outside the supported set.
 */
attn_status attn_fwd(attn_dtype dt, const void *Q, const void *K, const void *V, void *O,
                     float *LSE, int B, int H, int T, int head_dim, float scale, int causal,
                     hipStream_t stream);

/*
 * Bytes of device workspace attn_bwd needs for these sizes: the fp32 row
 * vector D = rowsum(dO o O) (Forge, section "Ecosystem survey"), padded to
 * 256 bytes.  Returns 0 when the arguments are invalid (see attn_last_error).
 */
size_t attn_bwd_workspace_bytes(attn_dtype dt, int B, int H, int T, int head_dim, int causal);

/*
 * Backward pass of L = <dO, O> with the three-stage, atomic-free structure of
 * Forge (section "Ecosystem survey"): a preprocessing kernel for
 * D = rowsum(dO o O) in fp32, a dK/dV kernel parallel over key/value rows and
 * a dQ kernel parallel over queries; P is recomputed from the saved logsumexp
 * (section "Attention kernel design").  Every output is bitwise reproducible.
 * The preprocessing is folded into the dQ kernel, which computes D for its
 * queries from the dO rows it already holds and stores it in the workspace;
 * the dK/dV kernel, enqueued after it on `stream`, reads it there.
 *   Q, K, V, O, dO  in  [B,H,T,head_dim], type dt; O is attn_fwd's output
 *   LSE             in  [B,H,T] fp32 from attn_fwd with the same Q, K, scale, causal
 *   dQ, dK, dV      out [B,H,T,head_dim], type dt
 *   workspace       caller-owned device scratch of >= attn_bwd_workspace_bytes(...)
 *                   bytes; contents on entry are ignored and on exit undefined
 * EINVAL additionally covers a workspace that is null, misaligned or too small
 * and outputs that overlap an input, another output or the workspace.
 */
attn_status attn_bwd(attn_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                     const void *dO, const float *LSE, void *dQ, void *dK, void *dV,
                     void *workspace, size_t workspace_bytes, int B, int H, int T,
                     int head_dim, float scale, int causal, hipStream_t stream);

/*
 * Workspace for attn_bwd_atomic: D as above followed by an fp32 dQ
 * accumulator of B*H*T*head_dim elements.  Returns 0 for invalid arguments
 * and for fp32 (ATTN_EUNSUPPORTED in attn_last_error).
 */
size_t attn_bwd_atomic_workspace_bytes(attn_dtype dt, int B, int H, int T, int head_dim, int causal);

/*
 * attn_bwd without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  Same arguments as attn_bwd minus the workspace, same
 * kernels and bitwise the same results.  D lives in a static device array of
 * ATTN_NOALLOC_MAX_ROWS floats (8 MiB), which each GPU the library runs on
 * holds until the process ends; B*H*T above ATTN_NOALLOC_MAX_ROWS gives
 * ATTN_EINVAL before anything is enqueued.  The call allocates nothing.  Every
 * call on one GPU shares that GPU's array, so calls that overlap in time on
 * one GPU (on different streams, or from different threads) race on it;
 * calls ordered on one stream do not.  The array's address on a device is
 * resolved by attn_init on that device, or by the first call there.
 */
#define ATTN_NOALLOC_MAX_ROWS ((size_t)1 << 21)
attn_status attn_bwd_noalloc(attn_dtype dt, const void *Q, const void *K, const void *V,
                             const void *O, const void *dO, const float *LSE, void *dQ, void *dK,
                             void *dV, int B, int H, int T, int head_dim, float scale, int causal,
                             hipStream_t stream);

/*
 * The backward pass with dQ folded into the dK/dV kernel: each key block's
 * dQ contribution is formed from the dS tile that kernel already holds and
 * added into the workspace's fp32 dQ accumulator with float atomics (zeroed
 * by the preprocess, then scaled and rounded by a final kernel).  It skips the
 * dQ pass's recomputation of S and dP; dK and dV are bitwise equal to
 * attn_bwd's, dQ differs by the run-dependent order of its fp32 additions.
 * bf16 only (EUNSUPPORTED for fp32).  Arguments and errors as for attn_bwd,
 * with attn_bwd_atomic_workspace_bytes(...) bytes of workspace.
 */
attn_status attn_bwd_atomic(attn_dtype dt, const void *Q, const void *K, const void *V,
                            const void *O, const void *dO, const float *LSE, void *dQ, void *dK,
                            void *dV, void *workspace, size_t workspace_bytes, int B, int H,
                            int T, int head_dim, float scale, int causal, hipStream_t stream);

/*
 * Strided views.  In a GPT-2 decoder layer (the llm.c workload of "How to
 * train an LLM on Apple Silicon without Python" (toolsonfire.com, 2026),
 * part "Starting Point"),
 * attention sits between the fused QKV projection, whose output rows are
 * [B, T, 3, H, d], and the output projection, which reads [B, T, H*d]; Forge
 * (section "System overview") hands such slices between kernels as views of
 * shared storage rather than copies.  The *_strided entry points take each
 * [B, H, T, d] tensor as a view: element (b, h, t, c) of tensor X sits at
 * X + b*s[0] + h*s[1] + t*s[2] + c (elements, not bytes), so Q, K and V can
 * be read straight out of the projection output and O, dQ, dK, dV written in
 * the layouts the neighbouring GEMMs use, with no permute kernels.
 *   strides   host array of int64 element strides, three per tensor
 *             (batch, head, token), in argument order: Q, K, V, O for
 *             attn_fwd_strided (12 values); Q, K, V, O, dO, dQ, dK, dV for the
 *             backward entry points (24 values).  Read during the call only.
 * Requirements (EINVAL otherwise): strides >= 0 and multiples of 16 bytes
 * (strides of extent-1 dimensions are ignored); each output view maps
 * distinct indices to distinct elements; no output may share an element
 * with an input, another output, LSE or the workspace.  Inputs may overlap
 * one another and may broadcast (stride 0).  Overlap is decided on the host
 * by a sufficient test: views whose byte ranges meet are accepted only when
 * they have identical strides and bases that differ by an offset that stays
 * injective as an extra index (the q, k, v or dq, dk, dv slices of one packed
 * buffer); other intersecting views are refused even if in fact disjoint.
 * LSE and the workspace stay contiguous.  Results equal the plain entry
 * points' bit for bit on the same values.  EUNSUPPORTED: a view whose
 * (T + 255) * token stride + head_dim exceeds 2^31 - 1 elements (the kernels
 * address rows within one (b, h) slab with 32-bit offsets; the same bound
 * applies to the plain entry points, whose token stride is head_dim).
 */
attn_status attn_fwd_strided(attn_dtype dt, const void *Q, const void *K, const void *V, void *O,
                             float *LSE, const long long *strides, int B, int H, int T,
                             int head_dim, float scale, int causal, hipStream_t stream);

attn_status attn_bwd_strided(attn_dtype dt, const void *Q, const void *K, const void *V,
                             const void *O, const void *dO, const float *LSE, void *dQ, void *dK,
                             void *dV, void *workspace, size_t workspace_bytes,
                             const long long *strides, int B, int H, int T, int head_dim,
                             float scale, int causal, hipStream_t stream);

attn_status attn_bwd_atomic_strided(attn_dtype dt, const void *Q, const void *K, const void *V,
                                    const void *O, const void *dO, const float *LSE, void *dQ,
                                    void *dK, void *dV, void *workspace, size_t workspace_bytes,
                                    const long long *strides, int B, int H, int T, int head_dim,
                                    float scale, int causal, hipStream_t stream);

/* Static name of a status code ("ATTN_OK", ...); "unknown" otherwise. */
const char *attn_status_str(attn_status s);

/* Thread-local text for the last non-OK status returned on this thread
 * ("" when none).  The pointer stays valid until the next call on the thread. */
const char *attn_last_error(void);

/*
 * Optional kernel timing (measurement only; Forge, section "Methodology and
 * reproducibility" times GPU execution separately from host encoding).
 * attn_prof_enable(capacity) with capacity > 0 creates `capacity` pairs of
 * HIP events once; afterwards every kernel the library launches is bracketed
 * by an event pair, stamped by the dispatch itself (hipExtLaunchKernel), until
 * the pairs run out.
 * attn_prof_enable(0) stops recording and releases the events.
 * attn_prof_read waits for the recorded events, then fills up to `max` records
 * (one per kernel name, in first-launch order) with the launch count and the
 * summed event time, clears the counters and returns the number of names (or
 * -1 on a HIP error).  Not meant to be called while another host thread
 * launches through the library.
 */
typedef struct {
    const char *kernel; /* static string naming the kernel */
    int launches;
    double total_ms;
} attn_kernel_time;

attn_status attn_prof_enable(int capacity);
int attn_prof_read(attn_kernel_time *out, int max);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
