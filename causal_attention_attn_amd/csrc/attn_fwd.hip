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
#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

// Rescale threshold of the online softmax, in base-2 units: the running max
// m is only raised (and O, l rescaled) when a block's max exceeds it by more
// than this, so probabilities stay below 2^8 between rescales.  Any m that is
// at least the true max minus this bound gives the same normalised result.
constexpr float kLazyRescale = 8.f;

// Row sum of 8 probabilities already rounded for the PV product: for bf16,
// v_dot2_f32_bf16 with (1, 1) adds two per instruction, and summing the
// rounded values keeps numerator and denominator of O consistent.
__device__ __forceinline__ float rowsum8(bf16x8 p, float acc)
{
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 pair = {p[2 * i], p[2 * i + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pair, one, acc, false);
    }
    return acc;
}
__device__ __forceinline__ float rowsum8(f32x8 p, float acc)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += p[i];
    return acc;
}

// Per-wave state of the forward pass: QG groups of 32 queries (group g holds
// queries qw + 32 g ..), their Q^T fragments, O^T accumulators, running maxima
// and this lane's share of each row sum.  All groups share the K and V^T
// fragments read from LDS, so LDS traffic per MFMA falls with QG.
template <typename E, int D, int QG, typename L> struct FwdWave {
    typedef typename Frag<E>::type FragE;
    static constexpr int NC = D / 16;
    static constexpr int NMB = D / 32;
    FragE qf[QG][NC];
    f32x16 o[QG][NMB];
    float m[QG], lsum[QG];
    float cs;
    int qw, h, r32, lane;

    __device__ __forceinline__ void load_k(FragE (&a)[NC], const E *tK, int sb) const
    {
#pragma unroll
        for (int c = 0; c < NC; ++c) a[c] = load_row8(L::row8(tK, 32 * sb + r32, 16 * c + 8 * h));
    }

    // S^T of one 32-key sub-block for every query group.
    __device__ __forceinline__ void qk(f32x16 (&s)[QG], const E *tK, int sb) const
    {
        FragE a[NC];
        load_k(a, tK, sb);
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            s[g] = zero16();
#pragma unroll
            for (int c = 0; c < NC; ++c) mma32(s[g], a[c], qf[g][c]);
        }
    }

    // Masks keys above the diagonal or past T in an edge sub-block.
    __device__ __forceinline__ void mask(f32x16 (&s)[QG], int kb, int T, int causal) const
    {
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            const int myq = qw + 32 * g + r32;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = kb + 8 * (j >> 2) + 4 * h + (j & 3);
                if (key >= T || (causal && key > myq)) s[g][j] = -INFINITY;
            }
        }
    }

    // Scaled block max of each group's rows (both wave halves combined).
    __device__ __forceinline__ void block_max(const f32x16 (&s)[QG], float (&mloc)[QG]) const
    {
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            float x = s[g][0];
#pragma unroll
            for (int j = 1; j < 16; ++j) x = fmaxf(x, s[g][j]);
            mloc[g] = half_max(x) * cs;
        }
    }

    // Raises a group's running max when the block max exceeds it by the
    // threshold (rare after the first blocks).  A group whose rows see no key
    // of the block has mloc = -inf and keeps its max; every row sees key 0, so
    // the first block always sets a finite max.
    __device__ __forceinline__ void rescale(const float (&mloc)[QG])
    {
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            if (__any(mloc[g] > m[g] + kLazyRescale)) {
                const float mnew = fmaxf(m[g], mloc[g]);
                const float alpha = fast_exp2(m[g] - mnew);
                m[g] = mnew;
                lsum[g] *= alpha;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[g][mb][j] *= alpha;
            }
        }
    }

    // One straight-line region: softmax of the current sub-block `s` (V rows
    // 32*sbv.. of tV) accumulated into O^T and, when DO_QK, the next
    // sub-block's S^T (K rows 32*sbk.. of tK, masked when EDGE) and its block
    // max, so the next block's MFMAs overlap this block's softmax.
    template <bool DO_QK, bool EDGE>
    __device__ __forceinline__ void phase(f32x16 (&s)[QG], float (&mloc)[QG], const E *tV, int sbv, const E *tK,
                                          int sbk, int kbn, int T, int causal)
    {
        FragE a[NC];
        if constexpr (DO_QK) load_k(a, tK, sbk);
        FragE vt[2][NMB];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
                vt[kk][mb] = L::colA(tV, 32 * sbv + 16 * kk + 4 * h, 32 * mb, lane);
        FragE pf[QG][2];
#pragma unroll
        for (int g = 0; g < QG; ++g)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float p[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) p[t] = fast_exp2(fmaf(s[g][8 * kk + t], cs, -m[g]));
                pf[g][kk] = pack8<E>(p);
                lsum[g] = rowsum8(pf[g][kk], lsum[g]);
            }
        if constexpr (DO_QK) {
#pragma unroll
            for (int g = 0; g < QG; ++g) {
                s[g] = zero16();
#pragma unroll
                for (int c = 0; c < NC; ++c) mma32(s[g], a[c], qf[g][c]);
            }
        }
#pragma unroll
        for (int g = 0; g < QG; ++g)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) mma32(o[g][mb], vt[kk][mb], pf[g][kk]);
        if constexpr (DO_QK) {
            if constexpr (EDGE) mask(s, kbn, T, causal);
            block_max(s, mloc);
        }
    }
};

// K tiles are double-buffered and V tiles triple-buffered: a tile's keys are
// read by QK^T one phase before its values are read by PV.  With NSB 32-key
// sub-blocks per tile, iteration t runs NSB phases; phase i does the softmax
// and PV of sub-block i of tile t and the QK^T of the next sub-block (i + 1 of
// tile t, or 0 of tile t+1).  One barrier per tile, placed before the last
// phase, publishes tile t+1 (stored at the top of iteration t from registers
// loaded one iteration earlier).  Every read of a buffer's previous tile
// precedes the barrier of the iteration before the store that overwrites it.
template <typename E, int D, int NW, int QG, int BN>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(const E *__restrict__ Q, const E *__restrict__ K,
                                                      const E *__restrict__ V, E *__restrict__ O,
                                                      float *__restrict__ LSE, Layout lay, int T, float c_log2,
                                                      int causal, int BH, int nqt, int bins)
{
    typedef typename Frag<E>::type FragE;
    constexpr int NSB = BN / 32;
    constexpr int WQ = 32 * QG;  // queries per wave
    constexpr int BM = WQ * NW;
    constexpr int NT = NW * 64;
    constexpr int STR = Tile<E, D>::kStride;
    constexpr int NC = D / 16;
    constexpr int NMB = D / 32;
    __shared__ __attribute__((aligned(16))) E sK[2][BN * STR];
    __shared__ __attribute__((aligned(16))) E sV[3][BN * STR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int bid = serpentine(blockIdx.x, gridDim.x, bins);
    // heaviest query blocks first (causal work grows with the block index)
    const int qt = causal ? (nqt - 1 - bid / BH) : (bid / BH);
    const int bh = bid % BH;
    const long long qoff = lay.q.at(bh, lay.H), koff = lay.k.at(bh, lay.H);
    const long long voff = lay.v.at(bh, lay.H), ooff = lay.o.at(bh, lay.H);
    const int q0 = qt * BM;
    const int qw = q0 + WQ * w;

    FwdWave<E, D, QG, PadLayout<E, D>> wv;
    wv.lane = lane;
    wv.r32 = lane & 31;
    wv.h = lane >> 5;
    wv.qw = qw;
    // Q^T as the B operand: lane (query r32, half h) holds Q[q][16c + 8h + t].
    // A negative scale is folded into Q so that maxima are taken of positively
    // scaled scores; a zero scale becomes a scale far below the rounding of
    // any score, so masked (-inf) scores still map to zero.
    // (Q rows past T read row T - 1 and are zeroed, and the sign applied, once
    // the first tile's loads have landed, so the prologue waits once.)
    wv.cs = fmaxf(fabsf(c_log2), 1e-30f);
#pragma unroll
    for (int g = 0; g < QG; ++g) {
        const int q = min(qw + 32 * g + wv.r32, T - 1);
#pragma unroll
        for (int c = 0; c < NC; ++c) wv.qf[g][c] = load_row8(Q + qoff + q * lay.q.st + 16 * c + 8 * wv.h);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) wv.o[g][mb] = zero16();
        wv.m[g] = -INFINITY;
        wv.lsum[g] = 0.f;
    }

    const int kv_end = causal ? min(T, q0 + BM) : T;
    const int nkt = (kv_end + BN - 1) / BN;
    // sub-blocks of 32 keys this wave needs: every key block starting at or
    // before its last query (causal), or before T
    const int last_key = causal ? min(qw + WQ - 1, T - 1) : T - 1;
    const int nsb = qw < T ? last_key / 32 + 1 : 0;

    TileRegs<E, D, BN, NT> kr, vr;
    kr.load(K + koff, lay.k.st, 0, T, tid);
    vr.load(V + voff, lay.v.st, 0, T, tid);
    kr.template store<STR>(sK[0], tid);
    vr.template store<STR>(sV[0], tid);
    if (nkt > 1) {
        kr.load(K + koff, lay.k.st, BN, T, tid);
        vr.load(V + voff, lay.v.st, BN, T, tid);
    }
#pragma unroll
    for (int g = 0; g < QG; ++g) {
        const bool live = qw + 32 * g + wv.r32 < T;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const FragE f = live ? wv.qf[g][c] : zero_frag<E>();
            wv.qf[g][c] = c_log2 < 0.f ? neg_frag<E>(f) : f;
        }
    }
    __syncthreads();

    f32x16 s[QG];
    float mloc[QG];
    auto edge = [&](int kb) { return (causal && kb + 31 > qw) || (kb + 32 > T); };
    if (nsb > 0) {
        wv.qk(s, sK[0], 0);
        if (edge(0)) wv.mask(s, 0, T, causal);
        wv.block_max(s, mloc);
        wv.rescale(mloc);
    }
    int vb = 0;  // V buffer of tile kt (kt % 3)
    for (int kt = 0; kt < nkt; ++kt) {
        const int kb = BN * kt;
        const int vb1 = vb == 2 ? 0 : vb + 1;
        if (kt + 1 < nkt) {
            kr.template store<STR>(sK[(kt + 1) & 1], tid);
            vr.template store<STR>(sV[vb1], tid);
        }
        if (kt + 2 < nkt) {
            kr.load(K + koff, lay.k.st, kb + 2 * BN, T, tid);
            vr.load(V + voff, lay.v.st, kb + 2 * BN, T, tid);
        }
#pragma unroll
        for (int i = 0; i < NSB; ++i) {
            const int n = NSB * kt + i;  // sub-block in softmax/PV this phase
            const bool last = i == NSB - 1;
            if (last) __syncthreads();
            const E *tKn = last ? sK[(kt + 1) & 1] : sK[kt & 1];
            const int sbn = last ? 0 : i + 1;
            if (n < nsb) {
                const int kbn = 32 * (n + 1);
                if (n + 1 < nsb) {
                    if (edge(kbn))
                        wv.template phase<true, true>(s, mloc, sV[vb], i, tKn, sbn, kbn, T, causal);
                    else
                        wv.template phase<true, false>(s, mloc, sV[vb], i, tKn, sbn, kbn, T, causal);
                    wv.rescale(mloc);
                } else {
                    wv.template phase<false, false>(s, mloc, sV[vb], i, nullptr, 0, kbn, T, causal);
                }
            }
        }
        vb = vb1;
    }

#pragma unroll
    for (int g = 0; g < QG; ++g) {
        const float ltot = half_sum(wv.lsum[g]);  // both halves hold the same query
        const int q = qw + 32 * g + wv.r32;
        if (q < T) {
            const float inv = 1.f / ltot;
            E *orow = O + ooff + q * lay.o.st;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    const int d0 = 32 * mb + 8 * gg + 4 * wv.h;
#pragma unroll
                    for (int e = 0; e < 4; ++e) orow[d0 + e] = (E)(wv.o[g][mb][4 * gg + e] * inv);
                }
            if (wv.h == 0) LSE[(size_t)bh * T + q] = (wv.m[g] + __builtin_amdgcn_logf(ltot)) * kLn2;
        }
    }
}

// bf16 with d >= 64: a three-stage software pipeline per wave, fed by direct
// HBM -> LDS copies into swizzled tiles.  Phase n issues
//   * on the matrix cores, QK^T of sub-block n+2 and PV of sub-block n (whose
//     probabilities the previous phase formed), and
//   * on the vector ALUs, the softmax of sub-block n+1: block max, lazy
//     rescale, exp2 and bf16 packing (and the mask, which only the wave's
//     last sub-block needs), and the row sum of sub-block n,
// with no dependence between the two streams, so they overlap within a wave.
// Iteration t runs phases 2t and 2t+1, which read V tile t and K tile t+1
// (K runs one tile ahead of V).  Both are requested at the top of iteration
// t-1, right after its barrier, and the barrier at the top of iteration t
// waits for them, so a copy has a whole iteration to land and two buffers of
// each suffice.  The buffers are distinct LDS variables and the loop is
// unrolled by two: every read names its buffer at compile time, which tells
// the compiler it does not depend on the copies in flight into the others
// (an HBM -> LDS copy counts as a pending load that any possibly-aliasing LDS
// read must wait for).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_kernel_pipe(const bf16 *__restrict__ Q, const bf16 *__restrict__ K,
                                                           const bf16 *__restrict__ V, bf16 *__restrict__ O,
                                                           float *__restrict__ LSE, Layout lay, int T, float c_log2,
                                                           int causal, int BH, int nqt, int bins)
{
    typedef SwzLayout<D> L;
    typedef bf16x8 FragE;
    constexpr int BN = 64;
    constexpr int BM = 32 * NW;
    constexpr int NC = D / 16;
    constexpr int NMB = D / 32;
    constexpr int DPW = L::template dma_per_wave<BN, NW>();  // copy instructions per wave per tile
    constexpr bool kEarlyOperands = D <= 64;                  // operand reads before the rescale (see phase)
    __shared__ __attribute__((aligned(16))) bf16 sK0[BN * D];
    __shared__ __attribute__((aligned(16))) bf16 sK1[BN * D];
    __shared__ __attribute__((aligned(16))) bf16 sV0[BN * D];
    __shared__ __attribute__((aligned(16))) bf16 sV1[BN * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int r32 = lane & 31, h = lane >> 5;
    const int bid = serpentine(blockIdx.x, gridDim.x, bins);
    const int qt = causal ? (nqt - 1 - bid / BH) : (bid / BH);
    const int bh = bid % BH;
    const long long qoff = lay.q.at(bh, lay.H), koff = lay.k.at(bh, lay.H);
    const long long voff = lay.v.at(bh, lay.H), ooff = lay.o.at(bh, lay.H);
    const int q0 = qt * BM;
    const int qw = q0 + 32 * w;
    const int myq = qw + r32;
    // A negative scale is folded into Q so that maxima are taken of
    // positively scaled scores; a zero scale becomes one far below the
    // rounding of any score, so masked (-inf) scores still map to zero.
    const float cs = fmaxf(fabsf(c_log2), 1e-30f);

    // Q^T as the B operand: lane (query r32, half h) holds Q[q][16c + 8h + t]
    // (sign applied once the prologue's barrier has waited for the loads).
    FragE qf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        qf[c] = myq < T ? load_row8(Q + qoff + myq * lay.q.st + 16 * c + 8 * h) : zero_frag<bf16>();
    f32x16 o[NMB];  // O^T: lane = query, rows = head dimension
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) o[mb] = zero16();
    float m = -INFINITY, lsum = 0.f;
    // the raw score above which a block raises m: (m + kLazyRescale) / cs
    float thr = -INFINITY;

    const int kv_end = causal ? min(T, q0 + BM) : T;
    const int nkt = (kv_end + BN - 1) / BN;  // >= 1
    // sub-blocks of 32 keys this wave needs; only the last one can hold keys
    // above the diagonal or past T
    const int last_key = causal ? min(qw + 31, T - 1) : T - 1;
    const int nsb = qw < T ? last_key / 32 + 1 : 0;

    SwzFrags<D> F;  // per-lane fragment offsets, shared by all buffers
    F.init(lane);
    // raw S^T of the sub-block the next softmax works on: in s1 before even
    // phases and in s2 before odd ones (each phase's QK^T fills the other)
    f32x16 s1, s2;
    FragE pf[2];  // probabilities of the sub-block the next PV multiplies

    // S^T of one 32-key sub-block: lane (query r32, half h) gets keys
    // 8 (j/4) + 4h + j%4 of it in s[j].
    auto qk = [&](f32x16 &s, const bf16 *tK, int sb) __attribute__((always_inline)) {
        FragE a[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) a[c] = F.row8(tK, sb, c);
        s = zero16();
#pragma unroll
        for (int c = 0; c < NC; ++c) mma32(s, a[c], qf[c]);
    };
    // Row maximum of sub-block kb / 32 (raw scores in s, masked first when
    // `last`) and the lazy rescale: the running max m is only raised (and O,
    // l and, when `pending`, the probabilities whose PV product is still to
    // come rescaled) when the block max exceeds it by more than
    // kLazyRescale; any m at least the true max minus that bound gives the
    // same normalised result.  Every row sees key 0, so the first block sets
    // a finite m.
    auto rescale = [&](f32x16 &s, int kb, bool last, bool pending) __attribute__((always_inline)) {
        if (last) {
            // key kb + 4h + off(j) is visible when off(j) <= lim
            const int lim = (causal ? min(myq, T - 1) : T - 1) - kb - 4 * h;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (8 * (j >> 2) + (j & 3) > lim) s[j] = -INFINITY;
        }
        float x = s[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) x = fmaxf(x, s[j]);
        // a lane whose own 16 scores stay at or below thr needs no rescale;
        // the maximum over both halves of its query is formed only when one
        // does not
        if (__any(x > thr)) {
            const float mloc = half_max(x) * cs;
            const float mnew = fmaxf(m, mloc);
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            thr = (m + kLazyRescale) / cs;
            lsum *= alpha;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[mb][j] *= alpha;
            if (pending) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    float p[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) p[t] = (float)pf[kk][t] * alpha;
                    pf[kk] = pack8<bf16>(p);
                }
            }
        }
    };
    // probabilities of a sub-block relative to the current m
    auto probs = [&](const f32x16 &s, FragE *dst) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            float p[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) p[t] = fast_exp2(fmaf(s[8 * kk + t], cs, -m));
            dst[kk] = pack8<bf16>(p);
        }
    };
    // Phase n: PV of sub-block n (sub-block sbv of tV), QK^T of sub-block n+2
    // (sub-block sbk of tK) into sq when DO_QK, softmax of sub-block n+1 (raw
    // scores in ss) when DO_SM; l accumulates the probabilities a PV product
    // actually uses.  The rescale decision comes first, so that the
    // probabilities of sub-block n+1 and both products form one block of
    // straight-line code the scheduler can interleave (a rescale then also
    // scales the probabilities still waiting for their PV product).  At
    // d <= 64 the LDS operand reads are issued before the decision, so they
    // land during it; at d = 128 that many live operands would leave room
    // for only one wave per SIMD, so they follow it.
    auto phase = [&](auto qk_c, auto sm_c, f32x16 &ss, f32x16 &sq, const bf16 *tV, int sbv, const bf16 *tK, int sbk,
                     int n) __attribute__((always_inline)) {
        constexpr bool DO_QK = decltype(qk_c)::value, DO_SM = decltype(sm_c)::value;
        FragE a[NC], vt[2][NMB], pn[2];
        auto operands = [&]() __attribute__((always_inline)) {
            if constexpr (DO_QK) {
#pragma unroll
                for (int c = 0; c < NC; ++c) a[c] = F.row8(tK, sbk, c);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) vt[kk][mb] = F.colA(tV, sbv, kk, mb);
        };
        if constexpr (kEarlyOperands) operands();
        if constexpr (DO_SM) rescale(ss, 32 * (n + 1), !DO_QK, true);  // sub-block n+1 is the last one when !DO_QK
        if constexpr (!kEarlyOperands) operands();
        if constexpr (DO_SM) probs(ss, pn);
        if constexpr (DO_QK) {
            sq = zero16();
#pragma unroll
            for (int c = 0; c < NC; ++c) mma32(sq, a[c], qf[c]);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) mma32(o[mb], vt[kk][mb], pf[kk]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) lsum = rowsum8(pf[kk], lsum);
        if constexpr (DO_SM) {
            pf[0] = pn[0];
            pf[1] = pn[1];
        }
    };
    const std::integral_constant<bool, true> yes;
    const std::integral_constant<bool, false> no;

    // prologue: K tile 0 for the first two sub-blocks, then V tile 0 and K
    // tile 1 for iteration 0 (always requested: with a single tile the copy
    // reads clamped rows into a buffer nothing reads, which keeps the wait
    // counts the same on every path)
    L::template dma<BN, NW>(sK0, K + koff, lay.k.st, 0, T, w, lane);
    L::template dma<BN, NW>(sV0, V + voff, lay.v.st, 0, T, w, lane);
    L::template dma<BN, NW>(sK1, K + koff, lay.k.st, BN, T, w, lane);
    barrier_vm<2 * DPW>();  // K tile 0 landed (and the older Q loads)
    if (c_log2 < 0.f) {
#pragma unroll
        for (int c = 0; c < NC; ++c) qf[c] = neg_frag<bf16>(qf[c]);
    }
    if (nsb > 0) {
        qk(s1, sK0, 0);
        rescale(s1, 0, nsb == 1, false);
        probs(s1, pf);
    }
    if (nsb > 1) qk(s1, sK0, 1);

    auto iteration = [&](auto b_c, int t) __attribute__((always_inline)) {
        constexpr int B = decltype(b_c)::value;  // t % 2
        const bf16 *tV = B ? sV1 : sV0;          // V tile t
        const bf16 *tK = B ? sK0 : sK1;          // K tile t+1
        bf16 *nK = B ? sK1 : sK0;                // K tile t+2 replaces K tile t
        bf16 *nV = B ? sV0 : sV1;                // V tile t+1 replaces V tile t-1
        barrier_vm<0>();  // V tile t and K tile t+1 landed; K tile t and V tile t-1 no longer read
        F.launder();
        if (t + 2 < nkt) L::template dma<BN, NW>(nK, K + koff, lay.k.st, (t + 2) * BN, T, w, lane);
        if (t + 1 < nkt) L::template dma<BN, NW>(nV, V + voff, lay.v.st, (t + 1) * BN, T, w, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int n = 2 * t + i;
            f32x16 &ss = i == 0 ? s1 : s2;
            f32x16 &sq = i == 0 ? s2 : s1;
            if (n < nsb) {
                if (n + 2 < nsb)
                    phase(yes, yes, ss, sq, tV, i, tK, i, n);
                else if (n + 1 < nsb)
                    phase(no, yes, ss, sq, tV, i, tK, i, n);
                else
                    phase(no, no, ss, sq, tV, i, tK, i, n);
            }
        }
    };
    for (int t = 0;;) {
        iteration(std::integral_constant<int, 0>(), t);
        if (++t >= nkt) break;
        iteration(std::integral_constant<int, 1>(), t);
        if (++t >= nkt) break;
    }

    const float ltot = half_sum(lsum);  // both halves hold the same query
    const float inv = 1.f / ltot;
    // O rows through the K and V buffers (RowStage), once every wave is done
    // with them: two waves' blocks per buffer
    typedef RowStage<bf16, D> RS;
    static_assert(2 * RS::ELEMS <= BN * D, "two output blocks fit one tile buffer");
    bf16 *blk = ((w >> 1) ? sV0 : sK0) + (w & 1) * RS::ELEMS;
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            float o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = o[mb][4 * gg + e] * inv;
            RS::put(blk, r32, 32 * mb + 8 * gg + 4 * h, o4);
        }
    __syncthreads();
    RS::drain(blk, O + ooff, lay.o.st, qw, T, lane);
    if (myq < T && h == 0) LSE[(size_t)bh * T + myq] = (m + __builtin_amdgcn_logf(ltot)) * kLn2;
}

template <typename E, int D>
static hipError_t launch_fwd_t(const void *Q, const void *K, const void *V, void *O, float *LSE, const Layout &lay,
                               int BH, int T, float scale, int causal, hipStream_t stream, const KernelHook &hook)
{
    // One 32-query group per wave (QG = 1): two groups sharing each K and V^T
    // fragment halve the LDS bytes per MFMA but lower occupancy and, with
    // 256-query blocks, worsen the causal load balance; QG = 2 measured slower
    // on every causal workload.
    constexpr int NW = 4;
    constexpr int QG = 1;
    constexpr int BM = 32 * QG * NW;
    // 64-key tiles, except fp32 with d = 128 whose five tile buffers would not fit in LDS
    constexpr int BN = (sizeof(E) == 4 && D == 128) ? 32 : 64;
    const int nqt = (T + BM - 1) / BM;
    const float c_log2 = scale * kLog2e;
    const int grid = nqt * BH;
    if constexpr (sizeof(E) == 2 && D >= 64) {
        constexpr auto kern = fwd_kernel_pipe<D, NW>;
        return launch_kernel(kern, dim3(grid), dim3(NW * 64), stream, hook, "attn_fwd", Q, K, V, O, LSE, lay, T,
                             c_log2, causal, BH, nqt, causal ? serpentine_bins<kern, NW * 64>(grid, hook) : 0);
    }
    constexpr auto kern = fwd_kernel<E, D, NW, QG, BN>;
    return launch_kernel(kern, dim3(grid), dim3(NW * 64), stream, hook, "attn_fwd", Q, K, V, O, LSE, lay, T, c_log2,
                         causal, BH, nqt, causal ? serpentine_bins<kern, NW * 64>(grid, hook) : 0);
}

hipError_t launch_fwd(int dt, int D, const void *Q, const void *K, const void *V, void *O, float *LSE,
                      const Layout &lay, int BH, int T, float scale, int causal, hipStream_t stream,
                      const KernelHook &hook)
{
#define ATTN_FWD_CASE(E, DD) \
    if (D == DD) return launch_fwd_t<E, DD>(Q, K, V, O, LSE, lay, BH, T, scale, causal, stream, hook);
    if (dt == 0) {
        ATTN_FWD_CASE(float, 32) ATTN_FWD_CASE(float, 64) ATTN_FWD_CASE(float, 128)
    } else {
        ATTN_FWD_CASE(bf16, 32) ATTN_FWD_CASE(bf16, 64) ATTN_FWD_CASE(bf16, 128)
    }
#undef ATTN_FWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace attn
