// attn_launch.h -- internal interface between the C ABI (attn_api.hip) and
// the kernel translation units.  Not installed; the public header is attn.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace attn {

// Element strides of a [B, H, T, d] tensor whose head dimension is
// contiguous: element (b, h, t, c) sits at b*sb + h*sh + t*st + c.  Offsets
// inside one (b, h) slab, up to (T + 255) * st + d, fit in int32 (checked by
// the host), so row addressing stays 32-bit.
struct View {
    long long sb, sh;
    int st;
    // offset of the (b, h) slab with flat index bh = b*H + h
    __host__ __device__ __forceinline__ long long at(int bh, int H) const
    {
        const int b = bh / H;
        return (long long)b * sb + (long long)(bh - b * H) * sh;
    }
};

// Views of every [B, H, T, d] tensor of one call, and H (LSE and D are
// always contiguous [B, H, T]).
struct Layout {
    View q, k, v, o, dO, dq, dk, dv;
    int H;
};

// Optional kernel timing: when `acquire` is set it hands out an event pair
// for the next launch, which is then dispatched with hipExtLaunchKernel so the
// events are stamped by the dispatch itself (no extra packets on the stream).
struct KernelHook {
    bool (*acquire)(hipEvent_t *, hipEvent_t *, const char *) = nullptr;
    int cus = 0;  // compute units of the current device (0 if unknown)
    // set-up pass: every launcher runs its host-side choices (the per-kernel
    // occupancy queries included) and returns before launching anything
    bool dry = false;
};

// Bins for the serpentine work order (see serpentine() in attn_device.h): the
// compute-unit count when the whole grid is resident at once, so that the
// dispatcher deals it out in rounds of one workgroup per compute unit;
// otherwise 0 (plain heaviest-first order, which later waves then balance).
// Workgroups of KERN (THREADS each) resident at once on one compute unit,
// queried once per kernel; 0 if the query fails.
template <auto KERN, int THREADS> inline int resident_per_cu()
{
    static const int per_cu = [] {
        int n = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(KERN), THREADS, 0) ==
                       hipSuccess
                   ? n
                   : 0;
    }();
    return per_cu;
}

template <auto KERN, int THREADS> inline int serpentine_bins(int grid, const KernelHook &hook)
{
    return hook.cus > 0 && grid <= resident_per_cu<KERN, THREADS>() * hook.cus ? hook.cus : 0;
}

template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                                const KernelHook &hook, const char *name, Args... args)
{
    if (hook.dry) return hipSuccess;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hook.acquire && hook.acquire(&e0, &e1, name))
        hipExtLaunchKernelGGL(kern, grid, block, 0, stream, e0, e1, 0, static_cast<KArgs>(args)...);
    else
        hipLaunchKernelGGL(kern, grid, block, 0, stream, static_cast<KArgs>(args)...);
    return hipGetLastError();
}

// dt: 0 = fp32, 1 = bf16.  D in {32, 64, 128}.  Shapes are validated by the caller.
hipError_t launch_fwd(int dt, int D, const void *Q, const void *K, const void *V, void *O, float *LSE,
                      const Layout &lay, int BH, int T, float scale, int causal, hipStream_t stream,
                      const KernelHook &hook);

// dQacc == nullptr selects the deterministic Q-major dQ pass; otherwise dQ is
// accumulated with float atomics into dQacc (contiguous [BH*T, D] fp32, zeroed
// by the preprocess) and converted at the end (bf16 only: bwd_atomic_supported).
bool bwd_atomic_supported(int dt, int D);
hipError_t launch_bwd(int dt, int D, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                      const float *LSE, void *dQ, void *dK, void *dV, float *Dbuf, float *dQacc, const Layout &lay,
                      int BH, int T, float scale, int causal, hipStream_t stream, const KernelHook &hook);

// Layer GEMMs (gemm.hip), bf16 operands, row-major:
//   GEMM_KIND_NT  C[M,N] = A[M,K] B[N,K]^T
//   GEMM_KIND_NN  C[M,N] = A[M,K] B[K,N]
//   GEMM_KIND_TN  C[M,N] = A[K,M]^T B[K,N]
// K is a multiple of 64 and N (and M for TN) of 8; the caller has checked
// shapes, leading dimensions and alignment.  The contraction is cut into
// chunks of kchunk (a multiple of 64, gemm_split_chunk(K, splits) for a
// requested number of splits); with more than one chunk `part` holds one
// fp32 [M, N] partial product per chunk, summed in chunk order.
enum { GEMM_KIND_NT = 0, GEMM_KIND_NN = 1, GEMM_KIND_TN = 2 };
int gemm_split_chunk(int K, int splits);
int gemm_auto_splits(int M, int N, int K);
// Workgroups of the 128 x 128 GEMM tile resident at once on the current
// device (compute units x occupancy), read once per device; 512 (256 units,
// two each) where no device can be queried.
int gemm_resident_slots();
hipError_t launch_gemm(int op, int c_f32, const void *A, const void *B, void *C, float *part, int M, int N, int K,
                       int lda, int ldb, int ldc, int kchunk, hipStream_t stream, const KernelHook &hook);

}  // namespace attn
