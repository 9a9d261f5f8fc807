// attn_fwd.hip -- fused causal attention forward for gfx950.
//
// Forge (S.-P. Boucher, 2026), section "Attention kernel design": a query
// block per workgroup, K and V staged through on-chip memory, an online
// softmax that rescales the output accumulator per K/V block, and a saved
// logsumexp for the backward pass.  What differs on CDNA4:
//   * each wave owns 32 queries and computes the transposed score tile
//     S^T = K Q^T (32 keys x 32 queries) on the matrix cores, so that in the
//     32x32 accumulator a lane owns one query and 16 of the 32 keys.  The row
//     max and row sum are then in-register reductions plus one exchange with
//     the other half of the wave, and the per-query rescale of the output is a
//     per-lane multiply (Forge needed a diagonal-matrix product for it because
//     Metal leaves the fragment-to-lane map unspecified);
//   * the output is accumulated transposed, O^T += V^T P^T, so the bf16
//     probabilities are consumed straight from the score registers as the B
//     operand; V^T is gathered from the LDS tile;
//   * key blocks entirely above the causal diagonal are skipped, and the
//     workgroups with the most key blocks are dispatched first;
//   * softmax runs in base 2 with log2(e) folded into the scale; the stored
//     logsumexp is converted back to natural-log units.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

// Rescale threshold of the online softmax, in base-2 units: the running max
// m is only raised (and O, l rescaled) when a block's max exceeds it by more
// than this, so probabilities stay below 2^8 between rescales.  Any m that is
// at least the true max minus this bound gives the same normalised result.
constexpr float kLazyRescale = 8.f;

template <typename E, int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(const E *__restrict__ Q, const E *__restrict__ K,
                                                      const E *__restrict__ V, E *__restrict__ O,
                                                      float *__restrict__ LSE, int T, float c_log2,
                                                      int causal, int BH, int nqt)
{
    typedef typename Frag<E>::type FragE;
    constexpr int BM = 32 * NW;
    constexpr int NT = NW * 64;
    constexpr int STR = Tile<E, D>::kStride;
    constexpr int NC = D / 16;    // 16-wide chunks of the head dimension
    constexpr int NMB = D / 32;   // 32-row blocks of O^T
    constexpr int NSB = BN / 32;  // 32-key blocks per K/V tile
    __shared__ __attribute__((aligned(16))) E sK[2][BN * STR];
    __shared__ __attribute__((aligned(16))) E sV[2][BN * STR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int r32 = lane & 31, h = lane >> 5;
    const int bid = blockIdx.x;
    // heaviest query blocks first (causal work grows with the block index)
    const int qt = causal ? (nqt - 1 - bid / BH) : (bid / BH);
    const int bh = bid % BH;
    const size_t base = (size_t)bh * T * D;
    const int q0 = qt * BM;
    const int qw = q0 + 32 * w;
    const int myq = qw + r32;

    // Q^T as the B operand: lane (query r32, half h) holds Q[myq][16c + 8h + t].
    // A negative scale is folded into Q so that the max below is taken of
    // positively scaled scores; a zero scale becomes a scale far below the
    // rounding of any score, so masked (-inf) scores still map to zero.
    const float cs = fmaxf(fabsf(c_log2), 1e-30f);
    FragE qf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        qf[c] = myq < T ? load_row8(Q + base + (size_t)myq * D + 16 * c + 8 * h) : zero_frag<E>();
        if (c_log2 < 0.f) qf[c] = neg_frag<E>(qf[c]);
    }

    f32x16 o[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) o[mb] = zero16();
    float m = -INFINITY;  // running max of scaled scores (base-2 units)
    float lsum = 0.f;     // this lane's share of the running row sum

    const int kv_end = causal ? min(T, q0 + BM) : T;
    const int nkt = (kv_end + BN - 1) / BN;
    const int wave_last_key = causal ? min(qw + 31, T - 1) : T - 1;

    TileRegs<E, D, BN, NT> kr, vr;
    kr.load(K + base, 0, T, tid);
    vr.load(V + base, 0, T, tid);
    kr.template store<STR>(sK[0], tid);
    vr.template store<STR>(sV[0], tid);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const int k0 = kt * BN;
        const int buf = kt & 1;
        const bool more = kt + 1 < nkt;
        if (more) {  // next tile's HBM loads overlap this tile's math
            kr.load(K + base, k0 + BN, T, tid);
            vr.load(V + base, k0 + BN, T, tid);
        }
        if (qw < T && k0 <= wave_last_key) {
            const E *tK = sK[buf];
            const E *tV = sV[buf];
            f32x16 s[NSB];
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                s[sb] = zero16();
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    mma32(s[sb], load_row8(tK + (32 * sb + r32) * STR + 16 * c + 8 * h), qf[c]);
            }
            // keys above the diagonal or past T only occur in edge tiles
            const bool edge = (causal && k0 + BN - 1 > qw) || (k0 + BN > T);
            if (edge) {
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = k0 + 32 * sb + 8 * (j >> 2) + 4 * h + (j & 3);
                        if (key >= T || (causal && key > myq)) s[sb][j] = -INFINITY;
                    }
            }
            // every row of the wave sees at least key k0 of this tile, so mloc is finite
            float mloc = -INFINITY;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mloc = fmaxf(mloc, s[sb][j]);
            mloc = half_max(mloc) * cs;
            if (__any(mloc > m + kLazyRescale)) {
                const float mnew = fmaxf(m, mloc);
                const float alpha = fast_exp2(m - mnew);
                m = mnew;
                lsum *= alpha;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[mb][j] *= alpha;
            }
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                float p[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    p[j] = fast_exp2(fmaf(s[sb][j], cs, -m));
                    lsum += p[j];
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const FragE pf = pack8<E>(p + 8 * kk);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
                        mma32(o[mb], ColGather<E, STR>::load(tV, 32 * sb + 16 * kk + 4 * h, 32 * mb, lane), pf);
                }
            }
        }
        if (more) {
            kr.template store<STR>(sK[buf ^ 1], tid);
            vr.template store<STR>(sV[buf ^ 1], tid);
        }
        __syncthreads();
    }

    const float ltot = half_sum(lsum);  // both halves hold the same query
    if (myq < T) {
        const float inv = 1.f / ltot;
        E *orow = O + base + (size_t)myq * D;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * mb + 8 * g + 4 * h;
#pragma unroll
                for (int e = 0; e < 4; ++e) orow[d0 + e] = (E)(o[mb][4 * g + e] * inv);
            }
        if (h == 0) LSE[(size_t)bh * T + myq] = (m + __builtin_amdgcn_logf(ltot)) * kLn2;
    }
}

template <typename E, int D>
static hipError_t launch_fwd_t(const void *Q, const void *K, const void *V, void *O, float *LSE, int BH, int T,
                               float scale, int causal, hipStream_t stream, const KernelHook &hook)
{
    constexpr int NW = 4, BN = 64, BM = 32 * NW;
    const int nqt = (T + BM - 1) / BM;
    const float c_log2 = scale * kLog2e;
    hook.begin(stream);
    hipLaunchKernelGGL((fwd_kernel<E, D, NW, BN>), dim3(nqt * BH), dim3(NW * 64), 0, stream, (const E *)Q,
                       (const E *)K, (const E *)V, (E *)O, LSE, T, c_log2, causal, BH, nqt);
    hook.end(stream, "attn_fwd");
    return hipGetLastError();
}

hipError_t launch_fwd(int dt, int D, const void *Q, const void *K, const void *V, void *O, float *LSE, int BH,
                      int T, float scale, int causal, hipStream_t stream, const KernelHook &hook)
{
#define ATTN_FWD_CASE(E, DD) \
    if (D == DD) return launch_fwd_t<E, DD>(Q, K, V, O, LSE, BH, T, scale, causal, stream, hook);
    if (dt == 0) {
        ATTN_FWD_CASE(float, 32) ATTN_FWD_CASE(float, 64) ATTN_FWD_CASE(float, 128)
    } else {
        ATTN_FWD_CASE(bf16, 32) ATTN_FWD_CASE(bf16, 64) ATTN_FWD_CASE(bf16, 128)
    }
#undef ATTN_FWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace attn
