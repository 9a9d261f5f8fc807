// attn_launch.h -- internal interface between the C ABI (attn_api.hip) and
// the kernel translation units.  Not installed; the public header is attn.h.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// Optional instrumentation around each kernel launch (event pairs on the
// launch stream); both hooks are null unless timing was enabled.
struct KernelHook {
    void (*on_begin)(hipStream_t) = nullptr;
    void (*on_end)(hipStream_t, const char *) = nullptr;
    void begin(hipStream_t s) const
    {
        if (on_begin) on_begin(s);
    }
    void end(hipStream_t s, const char *name) const
    {
        if (on_end) on_end(s, name);
    }
};

// dt: 0 = fp32, 1 = bf16.  D in {32, 64, 128}.  Shapes are validated by the caller.
hipError_t launch_fwd(int dt, int D, const void *Q, const void *K, const void *V, void *O, float *LSE, int BH,
                      int T, float scale, int causal, hipStream_t stream, const KernelHook &hook);

// dQacc == nullptr selects the deterministic Q-major dQ pass; otherwise dQ is
// accumulated with float atomics into dQacc ([BH*T, D] fp32, zeroed by the
// preprocess) and converted at the end (bf16 only: bwd_atomic_supported).
bool bwd_atomic_supported(int dt, int D);
hipError_t launch_bwd(int dt, int D, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                      const float *LSE, void *dQ, void *dK, void *dV, float *Dbuf, float *dQacc, int BH, int T,
                      float scale, int causal, hipStream_t stream, const KernelHook &hook);

}  // namespace attn
