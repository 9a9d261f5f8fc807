// attn_bwd.hip -- fused causal attention backward for gfx950: the three-stage,
// atomic-free structure of Forge (S.-P. Boucher, 2026), section "Ecosystem
// survey" -- a preprocessing kernel for D = rowsum(dO o O) in fp32, a dK/dV
// kernel parallel over key/value rows and a dQ kernel parallel over queries --
// with P recomputed from the saved logsumexp (section "Attention kernel
// design").  Transposed score tiles come from exchanging operand roles, as in
// that section, rather than from moving data:
//   * dK/dV kernel: a wave owns 32 keys and computes S = Q K^T and dP = dO V^T
//     with the keys on the lane axis, so that P and dS feed the matrix cores
//     directly as B operands of dV^T += dO^T P and dK^T += Q^T dS; K and V of
//     the wave stay in registers, the dK^T and dV^T accumulators too
//     (Forge, section "Finding 3": register pressure, not bandwidth, is what
//     bounds this kernel, so its register budget is read from the compiler's
//     resource report); at d = 128 that state does not fit one wave at two
//     waves per SIMD, and a pair of waves shares each 32-key block, one
//     forming S, P and dV, the other dP, dS and dK (bwd_dkdv_pair_kernel);
//   * dQ kernel: a wave owns 32 queries and computes S^T = K Q^T and
//     dP^T = V dO^T with the queries on the lane axis, feeding dS^T as the B
//     operand of dQ^T += K^T dS^T.
// The default path (attn_bwd) is this deterministic pair: the Q-major dQ
// kernel, which also forms D for its queries, then the dK/dV kernel.  The
// measured alternative (attn_bwd_atomic) folds dQ into the dK/dV kernel: the
// workgroup stages its dS tile in LDS, multiplies it by its K tile on the
// matrix cores and adds the partial dQ into an fp32 accumulator with global
// float atomics, which the preprocess zeroes and a final kernel scales and
// rounds.  That drops the dQ pass's recomputation of S and dP (two of its
// three T x T x d products) at the price of a summation order that varies from
// run to run.
#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

// D_i = sum_c dO_ic O_ic in fp32, summed in the same order as the dQ kernel
// does for its queries (so that both backward paths see bitwise the same D):
// two threads per row, thread h accumulating fma(O, dO) over columns
// 16 j + 8 h + t (j ascending, then t), then the two halves added.  With a dQ
// accumulator (atomic path) each thread also zeroes the fp32 elements of its
// columns.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const E *__restrict__ O, const E *__restrict__ dO,
                                                      float *__restrict__ Dout, float *__restrict__ dQacc,
                                                      Layout lay, int T, long long rows)
{
    const long long gtid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long row = gtid >> 1;
    const int h = (int)(gtid & 1);
    float acc = 0.f;
    if (row < rows) {
        const int bh = (int)(row / T), t = (int)(row - (long long)bh * T);
        const E *po = O + lay.o.at(bh, lay.H) + t * lay.o.st + 8 * h;
        const E *pd = dO + lay.dO.at(bh, lay.H) + t * lay.dO.st + 8 * h;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
            const typename Frag<E>::type o8 = load_row8(po + 16 * j), d8 = load_row8(pd + 16 * j);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)o8[e], (float)d8[e], acc);
            if (dQacc) {
                f32x4 *z = reinterpret_cast<f32x4 *>(dQacc + (size_t)row * D + 16 * j + 8 * h);
                z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
                z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    const float other = __shfl_xor(acc, 1, 64);
    if (row < rows && h == 0) Dout[row] = acc + other;
}

// dQ = scale * dQacc, rounded to the element type; 4 elements per thread
// (dQacc is contiguous (B, H, T, d); dQ follows its view).
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float *__restrict__ acc, E *__restrict__ dQ,
                                                             Layout lay, int T, float scale, long long n4)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const f32x4 v = reinterpret_cast<const f32x4 *>(acc)[i];
    const long long row = i / (D / 4);
    const int bh = (int)(row / T), t = (int)(row - (long long)bh * T);
    E *o = dQ + lay.dq.at(bh, lay.H) + t * lay.dq.st + 4 * (int)(i - row * (D / 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (E)(v[e] * scale);
}

// Whether the tile loops are unrolled by two so that each read names its LDS
// buffer at compile time (and reads never wait for the copy into the other
// buffer).  At d = 128 the two loop copies raise register use past what the
// register file holds for these kernels, which costs more than the waits.
template <int D> constexpr bool kStaticBuffers = D <= 64;

// Whether the deterministic backward forms dV and dK with a pair of waves per
// 32-key block (bwd_dkdv_pair_kernel) instead of one wave.  At d = 128 the
// fused kernel holds both 32 x 128 accumulators, K and V fragments and two
// sub-blocks of S and dP: 325 registers, one wave per SIMD.  Forge (section
// "Finding 3") splits its dK/dV kernel in two for the same reason, register
// pressure, there seen as spills; two kernels here (S and dV in one, S, dP and
// dK in the other) ran at two waves per SIMD but formed S twice.  The wave
// pair forms it once: B4 H32 T2048 dV + dK 387 -> 379 us, B8 H16 T1024
// 121.5 -> 107, B1 H3 T1000 56.3 -> 38.3 us, bitwise the same dK and dV.
template <typename E, int D> constexpr bool kPairDkDv = sizeof(E) == 2 && D == 128;

// When the fused dK/dV kernel (bf16, d = 64) runs its general path at three
// waves per SIMD rather than the steady path at two: sequences up to
// kDkDvGeneralMaxT whose grid needs at least two full rounds of the steady
// kernel's resident workgroups.  The steady path keeps two sub-blocks'
// products in flight, which a long chain of query tiles needs; short chains
// gain more from the third wave and the extra workgroups per round, once
// there are rounds to save.  Measured per launch (steady -> general):
// B64 H12 T256 37.3 -> 30.5 us, B64 H6 T512 45.3 -> 40.4, B64 H8 T1024
// 182 -> 172, B8 H16 T1024 (two rounds) 43.0 -> 41.5, B16 H12 T1024 equal;
// B8 H12 T1024 (1.5 rounds) 35.5 -> 35.5, 36.0 -> 36.5 and 36.7 -> 37.8 on
// three boxes; B4 H12 T1536 37.8 -> 45.8, T2048 +7-10%, B2 H12 T4096
// 103 -> 125.
constexpr int kDkDvGeneralMaxT = 1024;
constexpr int kDkDvGeneralMinRounds = 2;

// The wave index as a scalar (uniform branches) where it pays: at d <= 64 it
// makes the dQ kernel faster; at d = 128 it raises register use.
template <int D> __device__ __forceinline__ int bwd_wave() { return kStaticBuffers<D> ? wave_index() : threadIdx.x >> 6; }

// dK/dV (and, when ATOMIC_DQ, the partial dQ) for a block of 32*NW keys.
// Per query tile of BQ rows, iteration t:
//   1. loads of query tile t+1 (direct HBM -> LDS copies, or into registers)
//   2. per 32-query sub-block: S, dP on the matrix cores (Q, dO row fragments
//      from LDS), P and dS in registers; with ATOMIC_DQ, dS^T into LDS
//   3. dV^T += dO^T P, dK^T += Q^T dS (transposed LDS reads)
//   4. registers of tile t+1 into the other Q/dO buffer; barrier
//   5. with ATOMIC_DQ: dQ[tile] += dS K over the block's keys (dS^T and K
//      tiles from LDS), float atomics into dQacc; barrier before dS^T is
//      overwritten
// Both backward paths run the same tile loops and arithmetic, so their dK and
// dV agree bit for bit.  GENERAL runs every tile on the general path (one
// sub-block at a time) in at most 168 registers, three waves per SIMD instead
// of two; it gives bitwise the same dK and dV as the steady path.
template <typename E, int D, int NW, int BQ, bool ATOMIC_DQ, bool ASYNC, bool GENERAL = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(GENERAL ? 3 : 1))) void bwd_dkdv_kernel(
    const E *__restrict__ Q, const E *__restrict__ K, const E *__restrict__ V, const E *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dv, E *__restrict__ dK, E *__restrict__ dV,
    float *__restrict__ dQacc, Layout lay, int T, float scale, float c_log2, int causal, int BH, int nkt, int bins)
{
    typedef typename Frag<E>::type FragE;
    // Q/dO tiles: swizzled and filled by direct HBM -> LDS loads (ASYNC, bf16
    // with d >= 64) or padded and filled through registers
    typedef typename std::conditional<ASYNC, SwzLayout<D>, PadLayout<E, D>>::type L;
    constexpr int BNK = 32 * NW;  // keys per workgroup
    constexpr int NT = NW * 64;
    constexpr int STR = Tile<E, D>::kStride;
    constexpr int SSTR = Tile<E, BQ>::kStride;  // row stride of the staged dS^T tile
    constexpr int NC = D / 16;
    constexpr int NMB = D / 32;
    constexpr int NQB = BQ / 32;
    static_assert(BQ <= NT, "one thread per query row for the LSE/D staging");
    // Two buffers per tile, each its own LDS variable: when the loop is
    // unrolled by two every read names its buffer at compile time, so the
    // compiler can tell that the reads of one buffer do not depend on the copy
    // into the other (an HBM -> LDS copy counts as a pending vector-memory load
    // that any possibly-aliasing LDS read must wait for).
    // Otherwise both buffers share the first variable.
    constexpr int NQE = L::elems(BQ);
    constexpr bool SB = kStaticBuffers<D>;
    __shared__ __attribute__((aligned(16))) E sQ0[SB ? NQE : 2 * NQE];
    __shared__ __attribute__((aligned(16))) E sQ1[SB ? NQE : 1];
    __shared__ __attribute__((aligned(16))) E sdO0[SB ? NQE : 2 * NQE];
    __shared__ __attribute__((aligned(16))) E sdO1[SB ? NQE : 1];
    __shared__ __attribute__((aligned(16))) float sL[2][BQ];  // LSE in base-2 units (+inf past T)
    __shared__ __attribute__((aligned(16))) float sD[2][BQ];
    __shared__ __attribute__((aligned(16))) E sKt[ATOMIC_DQ ? BNK * STR : 1];   // the block's K rows
    __shared__ __attribute__((aligned(16))) E sdS[ATOMIC_DQ ? BNK * SSTR : 1];  // dS^T [key][query]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = bwd_wave<D>();
    const int r32 = lane & 31, h = lane >> 5;
    const int bid = serpentine(blockIdx.x, gridDim.x, bins);
    // causal: key blocks near the start see the most queries; dispatch them first
    const int kt = bid / BH;
    const int bh = bid % BH;
    const long long qoff = lay.q.at(bh, lay.H), koff = lay.k.at(bh, lay.H), voff = lay.v.at(bh, lay.H);
    const long long dooff = lay.dO.at(bh, lay.H), dkoff = lay.dk.at(bh, lay.H), dvoff = lay.dv.at(bh, lay.H);
    const size_t cbase = (size_t)bh * T * D;  // contiguous fp32 dQ accumulator (atomic path)
    const size_t rbase = (size_t)bh * T;
    const int k0 = kt * BNK;
    const int kw = k0 + 32 * w;
    const int mykey = kw + r32;

    // K and V as B operands: lane (key r32, half h) holds row mykey, columns 16c + 8h + t.
    FragE kf[NC], vf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        kf[c] = mykey < T ? load_row8(K + koff + mykey * lay.k.st + 16 * c + 8 * h) : zero_frag<E>();
        vf[c] = mykey < T ? load_row8(V + voff + mykey * lay.v.st + 16 * c + 8 * h) : zero_frag<E>();
    }
    // dK^T and dV^T: lane = key, rows = head dimension
    f32x16 dk[NMB], dv[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        dk[mb] = zero16();
        dv[mb] = zero16();
    }

    const int qt_begin = causal ? k0 / BQ : 0;
    const int nqt = (T + BQ - 1) / BQ;

    TileRegs<E, D, ASYNC ? NT : BQ, NT> qr, dr;  // unused (minimal) when ASYNC
    float lr = INFINITY, drow = 0.f;
    // LSE and D always go through registers (one per thread): queries at or
    // past T get LSE = +inf, so their probabilities are exactly 0 even where
    // the direct loads duplicated row T-1 into the tile.
    auto load_rows = [&](int q0, E *bQ, E *bdO) {
        if constexpr (ASYNC) {
            L::template dma<BQ, NW>(bQ, Q + qoff, lay.q.st, q0, T, w, lane);
            L::template dma<BQ, NW>(bdO, dO + dooff, lay.dO.st, q0, T, w, lane);
        } else {
            qr.load(Q + qoff, lay.q.st, q0, T, tid);
            dr.load(dO + dooff, lay.dO.st, q0, T, tid);
        }
        const int q = q0 + tid;
        if (tid < BQ) {
            lr = q < T ? LSE[rbase + q] : INFINITY;
            drow = q < T ? Dv[rbase + q] : 0.f;
        }
    };
    auto store_rows = [&](int b, E *bQ, E *bdO) {
        if constexpr (!ASYNC) {
            qr.template store<STR>(bQ, tid);
            dr.template store<STR>(bdO, tid);
        }
        if (tid < BQ) {
            sL[b][tid] = lr * kLog2e;  // +inf stays +inf
            sD[b][tid] = -drow;        // negated: it seeds the dP accumulator
        }
    };
    if constexpr (ATOMIC_DQ) {
        TileRegs<E, D, BNK, NT> kt_regs;
        kt_regs.load_zero_past(K + koff, lay.k.st, k0, T, tid);  // dS of keys past T need not be 0
        kt_regs.template store<STR>(sKt, tid);
    }
    if (qt_begin < nqt) {
        load_rows(qt_begin * BQ, sQ0, sdO0);
        store_rows(0, sQ0, sdO0);
    }
    barrier_vm<0>();

    // query tile qt (the (qt - qt_begin)-th) in buffer bsel = (qt - qt_begin) % 2
    // (a compile-time constant when the loop is unrolled), the next tile into
    // the other buffer
    // fragment reads of a staged tile: through the shared per-lane offsets
    // for swizzled tiles, else through the padded layout
    SwzFrags<D> F;
    if constexpr (ASYNC) F.init(lane);
    auto rowA = [&](const E *t, int qb, int c) __attribute__((always_inline)) {
        if constexpr (ASYNC) return F.row8(t, qb, c);
        else return load_row8(L::row8(t, 32 * qb + r32, 16 * c + 8 * h));
    };
    auto colT = [&](const E *t, int qb, int kk, int mb) __attribute__((always_inline)) {
        if constexpr (ASYNC) return F.colA(t, qb, kk, mb);
        else return L::colA(t, 32 * qb + 16 * kk + 4 * h, 32 * mb, lane);
    };
    // -D of the 16 queries a lane's dP accumulator rows hold in sub-block qb
    // (query 32 qb + 8 g + 4 h + e in register 4 g + e): seeding the product
    // with it leaves dP - D in the accumulator, with no subtraction after it
    auto seed_dp = [&](int buf, int qb) __attribute__((always_inline)) {
        f32x16 a;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&sD[buf][32 * qb + 8 * g + 4 * h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[4 * g + e] = d4[e];
        }
        return a;
    };
    constexpr bool kSteadyPath = ASYNC && NQB == 2 && !GENERAL;
    // mode 0: general tile; 1: steady tile; 2: a tile on or before the causal
    // diagonal, run as a steady tile with the causal mask (its keys above a
    // query give P = 0) and skipped when no query of it sees a key of the wave
    auto tile = [&](int qt, auto bsel, auto mode_c) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_c)::value;
        constexpr bool STEADY = MODE != 0, DIAG = MODE == 2;
        const int buf = bsel;
        if constexpr (ASYNC) F.launder();
        const E *tQ, *tdO;
        E *nQ, *ndO;
        if constexpr (SB) {
            tQ = bsel ? sQ1 : sQ0;
            tdO = bsel ? sdO1 : sdO0;
            nQ = bsel ? sQ0 : sQ1;
            ndO = bsel ? sdO0 : sdO1;
        } else {
            tQ = sQ0 + buf * NQE;
            tdO = sdO0 + buf * NQE;
            nQ = sQ0 + (buf ^ 1) * NQE;
            ndO = sdO0 + (buf ^ 1) * NQE;
        }
        const int q0 = qt * BQ;
        const bool more = qt + 1 < nqt;
        if (more) load_rows(q0 + BQ, nQ, ndO);
        // Steady tiles (every sub-block active, none on the causal diagonal)
        // run as straight-line code with both sub-blocks' S and dP issued
        // first: the matrix cores work on sub-block 1 while the vector ALUs
        // form P and dS of sub-block 0, and then on sub-block 0's dV and dK
        // products while sub-block 1's P and dS are formed.
        if constexpr (STEADY) {
          // a diagonal tile is skipped by the waves none of whose keys a query
          // of it sees (or whose keys are all past T)
          if (!DIAG || (kw < T && q0 + BQ - 1 >= kw)) {
            f32x16 s[2], dp[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                s[qb] = zero16();
                dp[qb] = seed_dp(buf, qb);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    mma32(s[qb], rowA(tQ, qb, c), kf[c]);
                    mma32(dp[qb], rowA(tdO, qb, c), vf[c]);
                }
            }
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                FragE pf[2], dsf[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    float p[8], ds[8];
#pragma unroll
                    for (int g2 = 0; g2 < 2; ++g2) {
                        const int g = 2 * kk + g2;
                        const int ql = 32 * qb + 8 * g + 4 * h;
                        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&sL[buf][ql]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) p[4 * g2 + e] = fast_exp2(fmaf(s[qb][4 * g + e], c_log2, -l4[e]));
                        if constexpr (DIAG) {
                            // query q0 + 32qb + 8g + 4h + e sees key mykey when it is not below it
                            const int dlim = mykey - (q0 + 32 * qb) - 4 * h;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (8 * g + e < dlim) p[4 * g2 + e] = 0.f;
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) ds[4 * g2 + e] = p[4 * g2 + e] * dp[qb][4 * g + e];
                    }
                    pf[kk] = pack8<E>(p);
                    dsf[kk] = pack8<E>(ds);
                    if constexpr (ATOMIC_DQ) {
                        // dS^T row = this lane's key, 4 consecutive queries per g
                        E *row = sdS + (32 * w + r32) * SSTR + 32 * qb + 16 * kk + 4 * h;
                        store4(row, ds);
                        store4(row + 8, ds + 4);
                    }
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        mma32(dv[mb], colT(tdO, qb, kk, mb), pf[kk]);
                        mma32(dk[mb], colT(tQ, qb, kk, mb), dsf[kk]);
                    }
            }
          } else if constexpr (ATOMIC_DQ) {
            // a skipped diagonal tile adds dS = 0 to the block's dQ product
            const float z[4] = {0.f, 0.f, 0.f, 0.f};
            E *row = sdS + (32 * w + r32) * SSTR + 4 * h;
#pragma unroll
            for (int g = 0; g < BQ / 8; ++g) store4(row + 8 * g, z);
          }
        } else
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const int qb0 = q0 + 32 * qb;
            // sub-block skipped when past T or entirely before the wave's keys
            const bool active = kw < T && qb0 < T && !(causal && qb0 + 31 < kw);
            float ds[16];
            if (active) {
                f32x16 s = zero16(), dp = seed_dp(buf, qb);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    mma32(s, rowA(tQ, qb, c), kf[c]);
                    mma32(dp, rowA(tdO, qb, c), vf[c]);
                }
                // s[j], dp[j] (dP - D): query 32*qb + 8*(j/4) + 4*h + j%4 of the tile, key mykey
                const bool diag = causal && qb0 + 31 >= kw && qb0 < kw + 32;
                // on the diagonal, query qb0 + 4h + 8g + e is masked when 8g + e < dlim
                const int dlim = diag ? mykey - qb0 - 4 * h : 0;
                float p[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ql = 32 * qb + 8 * g + 4 * h;
                    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&sL[buf][ql]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 4 * g + e;
                        float pv = fast_exp2(fmaf(s[j], c_log2, -l4[e]));
                        if (8 * g + e < dlim) pv = 0.f;
                        p[j] = pv;
                        ds[j] = pv * dp[j];  // dp holds dP - D
                    }
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        mma32(dv[mb], colT(tdO, qb, kk, mb), pack8<E>(p + 8 * kk));
                        mma32(dk[mb], colT(tQ, qb, kk, mb), pack8<E>(ds + 8 * kk));
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) ds[j] = 0.f;
            }
            if constexpr (ATOMIC_DQ) {
                // dS^T row = this lane's key, columns = 4 consecutive queries per g
                E *row = sdS + (32 * w + r32) * SSTR + 32 * qb + 4 * h;
#pragma unroll
                for (int g = 0; g < 4; ++g) store4(row + 8 * g, ds + 4 * g);
            }
        }
        if (more) store_rows(buf ^ 1, nQ, ndO);
        barrier_vm<0>();  // tile qt+1 landed (direct loads included), tile qt no longer read
        if constexpr (ATOMIC_DQ) {
            // dQ tile [BQ x D] += dS [BQ x BNK] K [BNK x D]: NQB*NMB sub-tiles of
            // 32 x 32 spread over the waves; the key assignment of both
            // gathers is key(kk, h, t) within each 16-key chunk.
            for (int st = w; st < NQB * NMB; st += NW) {
                const int qs = st / NMB, db = st % NMB;
                f32x16 acc = zero16();
#pragma unroll
                for (int kc = 0; kc < BNK / 16; ++kc)
                    mma32(acc, ColGather<E, SSTR>::load(sdS, 16 * kc + 4 * h, 32 * qs, lane),
                          ColGather<E, STR>::load(sKt, 16 * kc + 4 * h, 32 * db, lane));
                // acc[j]: query q0 + 32 qs + 8 (j/4) + 4 h + j%4, column 32 db + r32
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int q = q0 + 32 * qs + 8 * (j >> 2) + 4 * h + (j & 3);
                    if (q < T) unsafeAtomicAdd(dQacc + cbase + (size_t)q * D + 32 * db + r32, acc[j]);
                }
            }
            __syncthreads();
        }
    };
    // With static buffers (d <= 64) every tile takes the steady path: a
    // wave's tiles before qs_begin (those with a query below one of its keys,
    // q0 < kw + 32) carry the causal mask, and rows past T have LSE = +inf,
    // so their P is 0.  The diagonal tiles run in a loop of their own before
    // the steady ones, so no two tile paths meet inside a loop iteration:
    // where they did, the compiler reconciled their register assignments
    // with a copy of every dK/dV accumulator per tile (T = 4096: 110 ->
    // 106 us).  With buffers chosen at run time (d = 128) each tile picks the
    // steady or the general path.
    const std::integral_constant<int, 0> b0;
    const std::integral_constant<int, 1> b1;
    const std::integral_constant<int, 0> general;
    const std::integral_constant<int, 1> steady;
    const std::integral_constant<int, 2> diagonal;
    if constexpr (SB && kSteadyPath) {
        // every tile runs the steady path: rows past T have LSE = +inf and so
        // P = 0, and the tiles before qs_begin carry the causal mask
        const int qs_begin = causal ? max(qt_begin, (kw + 32 + BQ - 1) / BQ) : qt_begin;
        int qt = qt_begin;
        for (; qt < min(qs_begin, nqt); ++qt) {
            if ((qt - qt_begin) & 1) tile(qt, b1, diagonal);
            else tile(qt, b0, diagonal);
        }
        if (qt < nqt && ((qt - qt_begin) & 1)) tile(qt++, b1, steady);
        for (; qt + 1 < nqt; qt += 2) {
            tile(qt, b0, steady);
            tile(qt + 1, b1, steady);
        }
        if (qt < nqt) tile(qt++, b0, steady);
    } else if constexpr (SB) {
        for (int qt = qt_begin; qt < nqt;) {
            tile(qt, b0, general);
            if (++qt >= nqt) break;
            tile(qt, b1, general);
            ++qt;
        }
    } else {
        for (int qt = qt_begin; qt < nqt; ++qt) {
            const int q0 = qt * BQ;
            if (kSteadyPath && kw < T && q0 + BQ - 32 < T && !(causal && q0 < kw + 32))
                tile(qt, (qt - qt_begin) & 1, std::integral_constant<int, kSteadyPath ? 1 : 0>());
            else
                tile(qt, (qt - qt_begin) & 1, general);
        }
    }

    // Epilogue: dK and dV rows through the (now unused) tile buffers
    // (RowStage).  Stored directly, the 4-column pieces of the two
    // interleaved outputs had the cache write 33 MB for 24 MB of dK and dV at
    // the bench shape, and the kernel took 40.0 against 37.0 us.
    typedef RowStage<E, D> RS;
    static_assert(2 * RS::ELEMS <= NQE, "two waves' rows fit one tile buffer");
    E *stk = SB ? ((w >> 1) ? sQ1 : sQ0) + (w & 1) * RS::ELEMS : sQ0 + w * RS::ELEMS;
    E *stv = SB ? ((w >> 1) ? sdO1 : sdO0) + (w & 1) * RS::ELEMS : sdO0 + w * RS::ELEMS;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * mb + 8 * g + 4 * h;
            float k4[4], v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                k4[e] = dk[mb][4 * g + e] * scale;
                v4[e] = dv[mb][4 * g + e];
            }
            RS::put(stk, r32, d0, k4);
            RS::put(stv, r32, d0, v4);
        }
    __syncthreads();
    RS::drain(stk, dK + dkoff, lay.dk.st, kw, T, lane);
    RS::drain(stv, dV + dvoff, lay.dv.st, kw, T, lane);
}

// d = 128: dV and dK in one kernel, each 32-key block handled by a pair of
// waves.  Wave 2i forms S = Q K^T, the probabilities P and dV^T += dO^T P;
// wave 2i + 1 forms dP - D = dO V^T - D, reads P from LDS after a barrier,
// and forms dS = P (dP - D) and dK^T += Q^T dS.  S is computed once per block
// (two kernels, one for dV and one for dK, would compute it twice) and each
// wave holds one accumulator and one set of K or V fragments.  Tiles follow
// the general path of bwd_dkdv_kernel (sub-blocks with no visible key
// skipped, the diagonal masked) with the same arithmetic, so dK and dV are
// bitwise those of the one-wave kernel.
template <int D, int NW, int BQ>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv_pair_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V, const bf16 *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dv, bf16 *__restrict__ dK, bf16 *__restrict__ dV,
    Layout lay, int T, float scale, float c_log2, int causal, int BH, int nkt, int bins)
{
    typedef bf16x8 FragE;
    typedef SwzLayout<D> L;
    constexpr int NP = NW / 2;    // wave pairs
    constexpr int BNK = 32 * NP;  // keys per workgroup
    constexpr int NT = NW * 64;
    constexpr int NC = D / 16;
    constexpr int NMB = D / 32;
    constexpr int NQE = L::elems(BQ);
    static_assert(BQ == 64, "two 32-query sub-blocks per tile");
    static_assert(BQ <= NT, "one thread per query row for the LSE/D staging");
    __shared__ __attribute__((aligned(16))) bf16 sQ[2 * NQE];
    __shared__ __attribute__((aligned(16))) bf16 sdO[2 * NQE];
    __shared__ __attribute__((aligned(16))) float sL[2][BQ];  // LSE in base-2 units (+inf past T)
    __shared__ __attribute__((aligned(16))) float sD[2][BQ];  // -D
    // P of each pair's two sub-blocks: float 4 g + e of lane l at ((qb * 4 + g) * 64 + l) * 4 + e
    __shared__ __attribute__((aligned(16))) float sP[NP * 2 * 16 * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_index();
    const int pair = w >> 1, role = w & 1;  // role 0: S, P, dV; role 1: dP, dS, dK
    const int r32 = lane & 31, h = lane >> 5;
    const int bid = serpentine(blockIdx.x, gridDim.x, bins);
    const int kt = bid / BH;
    const int bh = bid % BH;
    const long long qoff = lay.q.at(bh, lay.H), koff = lay.k.at(bh, lay.H), voff = lay.v.at(bh, lay.H);
    const long long dooff = lay.dO.at(bh, lay.H), dkoff = lay.dk.at(bh, lay.H), dvoff = lay.dv.at(bh, lay.H);
    const size_t rbase = (size_t)bh * T;
    const int k0 = kt * BNK;
    const int kw = k0 + 32 * pair;
    const int mykey = kw + r32;

    // K rows (role 0) or V rows (role 1) as B operands: lane (key r32, half h)
    // holds row mykey, columns 16c + 8h + t
    const bf16 *src = role ? V + voff : K + koff;
    const int sst = role ? lay.v.st : lay.k.st;
    FragE kv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) kv[c] = load_row8(src + min(mykey, T - 1) * sst + 16 * c + 8 * h);
    f32x16 acc[NMB];  // dV^T (role 0) or dK^T (role 1): lane = key, rows = head dimension
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[mb] = zero16();

    const int qt_begin = causal ? k0 / BQ : 0;
    const int nqt = (T + BQ - 1) / BQ;
    float lr = INFINITY, drow = 0.f;
    auto load_rows = [&](int q0, bf16 *bQ, bf16 *bdO) {
        L::template dma<BQ, NW>(bQ, Q + qoff, lay.q.st, q0, T, w, lane);
        L::template dma<BQ, NW>(bdO, dO + dooff, lay.dO.st, q0, T, w, lane);
        const int q = q0 + tid;
        if (tid < BQ) {
            lr = q < T ? LSE[rbase + q] : INFINITY;
            drow = q < T ? Dv[rbase + q] : 0.f;
        }
    };
    auto store_rows = [&](int b) {
        if (tid < BQ) {
            sL[b][tid] = lr * kLog2e;  // +inf stays +inf
            sD[b][tid] = -drow;        // negated: it seeds the dP accumulator
        }
    };
    if (qt_begin < nqt) {
        load_rows(qt_begin * BQ, sQ, sdO);
        store_rows(0);
    }
    barrier_vm<0>();

    SwzFrags<D> F;
    F.init(lane);
    float *myP = sP + pair * (2 * 16 * 64);
    // Each role runs its own loop (the same copies and barriers per tile), so
    // the compiler never sees one role's state live in the other's code.
    auto active = [&](int qb0) { return kw < T && qb0 < T && !(causal && qb0 + 31 < kw); };
    auto next = [&](int qt, int buf) {
        const bool more = qt + 1 < nqt;
        if (more) load_rows((qt + 1) * BQ, sQ + (buf ^ 1) * NQE, sdO + (buf ^ 1) * NQE);
        return more;
    };
    if (role == 0) {
        for (int qt = qt_begin; qt < nqt; ++qt) {
            const int buf = (qt - qt_begin) & 1;
            F.launder();
            const bf16 *tQ = sQ + buf * NQE, *tdO = sdO + buf * NQE;
            const int q0 = qt * BQ;
            const bool more = next(qt, buf);
            FragE pf[2][2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int qb0 = q0 + 32 * qb;
                if (!active(qb0)) continue;
                f32x16 sv = zero16();
#pragma unroll
                for (int c = 0; c < NC; ++c) mma32(sv, F.row8(tQ, qb, c), kv[c]);
                const bool diag = causal && qb0 + 31 >= kw && qb0 < kw + 32;
                const int dlim = diag ? mykey - qb0 - 4 * h : 0;
                float p[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&sL[buf][32 * qb + 8 * g + 4 * h]);
                    f32x4 p4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float pv = fast_exp2(fmaf(sv[4 * g + e], c_log2, -l4[e]));
                        if (8 * g + e < dlim) pv = 0.f;
                        p[4 * g + e] = pv;
                        p4[e] = pv;
                    }
                    *reinterpret_cast<f32x4 *>(myP + ((qb * 4 + g) * 64 + lane) * 4) = p4;
                }
                pf[qb][0] = pack8<bf16>(p);
                pf[qb][1] = pack8<bf16>(p + 8);
            }
            barrier_vm<63>();  // P visible to the pair's second wave (LDS only; the copies stay in flight)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                if (!active(q0 + 32 * qb)) continue;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) mma32(acc[mb], F.colA(tdO, qb, kk, mb), pf[qb][kk]);
            }
            if (more) store_rows(buf ^ 1);
            barrier_vm<0>();  // tile qt+1 landed; tile qt and its P no longer read
        }
    } else {
        for (int qt = qt_begin; qt < nqt; ++qt) {
            const int buf = (qt - qt_begin) & 1;
            F.launder();
            const bf16 *tQ = sQ + buf * NQE, *tdO = sdO + buf * NQE;
            const int q0 = qt * BQ;
            const bool more = next(qt, buf);
            f32x16 dpv[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                if (!active(q0 + 32 * qb)) continue;
                f32x16 a;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&sD[buf][32 * qb + 8 * g + 4 * h]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[4 * g + e] = d4[e];
                }
#pragma unroll
                for (int c = 0; c < NC; ++c) mma32(a, F.row8(tdO, qb, c), kv[c]);
                dpv[qb] = a;
            }
            barrier_vm<63>();
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                if (!active(q0 + 32 * qb)) continue;
                float ds[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 p4 = *reinterpret_cast<const f32x4 *>(myP + ((qb * 4 + g) * 64 + lane) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) ds[4 * g + e] = p4[e] * dpv[qb][4 * g + e];  // dpv holds dP - D
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const FragE dsf = pack8<bf16>(ds + 8 * kk);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) mma32(acc[mb], F.colA(tQ, qb, kk, mb), dsf);
                }
            }
            if (more) store_rows(buf ^ 1);
            barrier_vm<0>();
        }
    }

    // dV (role 0) or dK (role 1) rows through the tile buffers (RowStage)
    typedef RowStage<bf16, D> RS;
    static_assert(NW * RS::ELEMS <= 4 * NQE, "every wave's rows fit the tile buffers");
    bf16 *stage = (w < NW / 2 ? sQ + w * RS::ELEMS : sdO + (w - NW / 2) * RS::ELEMS);
    const float f = role ? scale : 1.f;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = acc[mb][4 * g + e] * f;
            RS::put(stage, r32, 32 * mb + 8 * g + 4 * h, v4);
        }
    __syncthreads();
    if (role)
        RS::drain(stage, dK + dkoff, lay.dk.st, kw, T, lane);
    else
        RS::drain(stage, dV + dvoff, lay.dv.st, kw, T, lane);
}


// IL (bf16, d = 64, for long sequences): the steady key tiles of a wave (both
// sub-blocks visible to all its queries and inside T) run in a loop of their
// own with both sub-blocks' S and dP issued first, so the matrix cores work
// on sub-block 1 while dS of sub-block 0 is formed.  The two products in
// flight raise the kernel from three waves per SIMD to two: at T >= 2048 the
// overlap wins (B1 H12 T8192: 174 -> 157 us, B2 H12 T4096: 93 -> 86 us), at
// T = 1024 the lost occupancy mostly does not (B8 H12: 29.8 -> 32.8 us).
template <typename E, int D, int NW, int BN, bool ASYNC, bool COMPUTE_D, bool IL = false>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(const E *__restrict__ Q, const E *__restrict__ K,
                                                         const E *__restrict__ V, const E *__restrict__ O,
                                                         const E *__restrict__ dO, const float *__restrict__ LSE,
                                                         float *__restrict__ Dv, E *__restrict__ dQ, Layout lay,
                                                         int T, float scale, float c_log2, int causal, int BH,
                                                         int nqt, int bins)
{
    typedef typename Frag<E>::type FragE;
    typedef typename std::conditional<ASYNC, SwzLayout<D>, PadLayout<E, D>>::type L;
    constexpr int BM = 32 * NW;
    constexpr int NT = NW * 64;
    constexpr int STR = Tile<E, D>::kStride;
    constexpr int NC = D / 16;
    constexpr int NMB = D / 32;
    constexpr int NSB = BN / 32;
    // two buffers per tile, as in the dK/dV kernel
    constexpr int NKE = L::elems(BN);
    constexpr bool SB = kStaticBuffers<D>;
    __shared__ __attribute__((aligned(16))) E sK0[SB ? NKE : 2 * NKE];
    __shared__ __attribute__((aligned(16))) E sK1[SB ? NKE : 1];
    __shared__ __attribute__((aligned(16))) E sV0[SB ? NKE : 2 * NKE];
    __shared__ __attribute__((aligned(16))) E sV1[SB ? NKE : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = bwd_wave<D>();
    const int r32 = lane & 31, h = lane >> 5;
    const int bid = serpentine(blockIdx.x, gridDim.x, bins);
    const int qt = causal ? (nqt - 1 - bid / BH) : (bid / BH);
    const int bh = bid % BH;
    const long long qoff = lay.q.at(bh, lay.H), koff = lay.k.at(bh, lay.H), voff = lay.v.at(bh, lay.H);
    const long long ooff = lay.o.at(bh, lay.H), dooff = lay.dO.at(bh, lay.H), dqoff = lay.dq.at(bh, lay.H);
    const int q0 = qt * BM;
    const int qw = q0 + 32 * w;
    const int myq = qw + r32;

    // Every operand load of the prologue is issued before any is waited for
    // (rows past T read row T - 1 and are zeroed afterwards), together with
    // the first K/V tile, so the prologue costs one memory round trip.  Loads
    // guarded by the row test and consumed one by one left four round trips
    // in the compiled prologue: a median 15K clocks per wave at B8 H12 T1024,
    // and the kernel 29.8 against 27.5 us.
    const bool live = myq < T;
    const int qr = live ? myq : T - 1;
    FragE qf[NC], df[NC], of[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        qf[c] = load_row8(Q + qoff + qr * lay.q.st + 16 * c + 8 * h);
        df[c] = load_row8(dO + dooff + qr * lay.dO.st + 16 * c + 8 * h);
        if constexpr (COMPUTE_D) of[c] = load_row8(O + ooff + qr * lay.o.st + 16 * c + 8 * h);
    }
    const float lse_row = LSE[(size_t)bh * T + qr];
    const float d_row = COMPUTE_D ? 0.f : Dv[(size_t)bh * T + qr];

    const int kv_end = causal ? min(T, q0 + BM) : T;
    const int nkt = (kv_end + BN - 1) / BN;
    const int wave_last_key = causal ? min(qw + 31, T - 1) : T - 1;

    TileRegs<E, D, ASYNC ? NT : BN, NT> kr, vr;  // unused (minimal) when ASYNC
    auto request = [&](int k0, E *bK, E *bV) {
        if constexpr (ASYNC) {
            L::template dma<BN, NW>(bK, K + koff, lay.k.st, k0, T, w, lane);
            L::template dma<BN, NW>(bV, V + voff, lay.v.st, k0, T, w, lane);
        } else {
            kr.load(K + koff, lay.k.st, k0, T, tid);
            vr.load(V + voff, lay.v.st, k0, T, tid);
        }
    };
    request(0, sK0, sV0);
    if constexpr (!ASYNC) {
        kr.template store<STR>(sK0, tid);
        vr.template store<STR>(sV0, tid);
    }
    barrier_vm<0>();

    if (!live) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qf[c] = zero_frag<E>();
            df[c] = zero_frag<E>();
            if constexpr (COMPUTE_D) of[c] = zero_frag<E>();
        }
    }
    const float lse2 = live ? lse_row * kLog2e : INFINITY;
    float dd;
    if constexpr (COMPUTE_D) {
        // D = rowsum(dO o O) of this lane's query, from the dO and O
        // fragments; published for the dK/dV kernel that runs after this one.
        float dpart = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int t = 0; t < 8; ++t) dpart = fmaf((float)of[c][t], (float)df[c][t], dpart);
        dd = half_sum(dpart);
        if (h == 0 && live) Dv[(size_t)bh * T + myq] = dd;
    } else {
        dd = live ? d_row : 0.f;
    }
    // bf16, D <= 64: -D of this lane's query enters dP^T as one more
    // contraction chunk (its bf16 high and low parts at k = 0, 1 against
    // ones, in the lanes of half 0), so the product leaves dP - D and dS
    // costs one multiply.  At D = 128 the two extra fragments push the
    // kernel past 256 registers and halve its occupancy.
    constexpr bool kFoldD = sizeof(E) == 2 && D <= 64;
    FragE ones = zero_frag<E>(), dneg = zero_frag<E>();
    if constexpr (kFoldD) {
        if (h == 0) {
            const E hi = (E)(-dd);
            ones[0] = (E)1.f;
            ones[1] = (E)1.f;
            dneg[0] = hi;
            dneg[1] = (E)(-dd - (float)hi);
        }
    }
    const float dsub = kFoldD ? 0.f : dd;  // what is left to subtract from the product
    f32x16 dq[NMB];  // dQ^T: lane = query, rows = head dimension
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) dq[mb] = zero16();

    // key tile kt in buffer bsel = kt % 2, the next one into the other buffer
    SwzFrags<D> F;
    if constexpr (ASYNC) F.init(lane);
    auto rowA = [&](const E *t, int sb, int c) __attribute__((always_inline)) {
        if constexpr (ASYNC) return F.row8(t, sb, c);
        else return load_row8(L::row8(t, 32 * sb + r32, 16 * c + 8 * h));
    };
    auto colT = [&](const E *t, int sb, int kk, int mb) __attribute__((always_inline)) {
        if constexpr (ASYNC) return F.colA(t, sb, kk, mb);
        else return L::colA(t, 32 * sb + 16 * kk + 4 * h, 32 * mb, lane);
    };
    // steady_c: a tile with both key sub-blocks visible to every query of the
    // wave and inside T, run with both sub-blocks' S and dP issued first
    auto tile = [&](int kt, auto bsel, auto steady_c) __attribute__((always_inline)) {
        constexpr bool STEADY = decltype(steady_c)::value;
        const int buf = bsel;
        if constexpr (ASYNC) F.launder();
        const E *tK, *tV;
        E *nK, *nV;
        if constexpr (SB) {
            tK = bsel ? sK1 : sK0;
            tV = bsel ? sV1 : sV0;
            nK = bsel ? sK0 : sK1;
            nV = bsel ? sV0 : sV1;
        } else {
            tK = sK0 + buf * NKE;
            tV = sV0 + buf * NKE;
            nK = sK0 + (buf ^ 1) * NKE;
            nV = sV0 + (buf ^ 1) * NKE;
        }
        const int k0 = kt * BN;
        const bool more = kt + 1 < nkt;
        if (more) request(k0 + BN, nK, nV);
        static_assert(!STEADY || (IL && NSB == 2), "steady tiles only in the interleaved variant");
        if constexpr (STEADY) {
            f32x16 s[NSB], dpt[NSB];
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                s[sb] = zero16();
                dpt[sb] = zero16();
                if constexpr (kFoldD) mma32(dpt[sb], ones, dneg);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    mma32(s[sb], rowA(tK, sb, c), qf[c]);
                    mma32(dpt[sb], rowA(tV, sb, c), df[c]);
                }
            }
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                float ds[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) ds[j] = fast_exp2(fmaf(s[sb][j], c_log2, -lse2)) * (dpt[sb][j] - dsub);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const FragE dsf = pack8<E>(ds + 8 * kk);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) mma32(dq[mb], colT(tK, sb, kk, mb), dsf);
                }
            }
        } else if (qw < T && k0 <= wave_last_key) {
            const bool edge = (causal && k0 + BN - 1 > qw) || (k0 + BN > T);
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int kb = k0 + 32 * sb;
                if (kb > wave_last_key) break;
                f32x16 s = zero16(), dpt = zero16();
                if constexpr (kFoldD) mma32(dpt, ones, dneg);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    mma32(s, rowA(tK, sb, c), qf[c]);
                    mma32(dpt, rowA(tV, sb, c), df[c]);
                }
                float ds[16];
                // One uniform branch per sub-block: masking (keys at or past
                // this lane's limit) only on edge tiles, as selects.
                if (edge) {
                    // key kb + 4h + off(j) is visible when off(j) < lim
                    const int lim = (causal ? min(T, myq + 1) : T) - kb - 4 * h;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float pv = fast_exp2(fmaf(s[j], c_log2, -lse2));
                        ds[j] = 8 * (j >> 2) + (j & 3) < lim ? pv * (dpt[j] - dsub) : 0.f;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j) ds[j] = fast_exp2(fmaf(s[j], c_log2, -lse2)) * (dpt[j] - dsub);
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const FragE dsf = pack8<E>(ds + 8 * kk);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
                        mma32(dq[mb], colT(tK, sb, kk, mb), dsf);
                }
            }
        }
        if constexpr (!ASYNC) {
            if (more) {
                kr.template store<STR>(nK, tid);
                vr.template store<STR>(nV, tid);
            }
        }
        barrier_vm<0>();  // tile kt+1 landed (direct loads included), tile kt no longer read
    };
    const std::integral_constant<int, 0> b0;
    const std::integral_constant<int, 1> b1;
    const std::integral_constant<bool, true> yes;
    const std::integral_constant<bool, false> no;
    if constexpr (SB && IL) {
        // the wave's steady tiles [0, ke) (k0 + BN - 1 <= qw when causal,
        // k0 + BN <= T) in a loop of their own, then the edge tiles, so the
        // two tile paths never meet inside a loop iteration
        const int ke = qw < T ? min(min(causal ? (qw + 1) / BN : nkt, T / BN), nkt) : 0;
        int kt = 0;
        for (; kt + 1 < ke; kt += 2) {
            tile(kt, b0, yes);
            tile(kt + 1, b1, yes);
        }
        if (kt < ke) tile(kt++, b0, yes);
        for (; kt < nkt; ++kt) {
            if (kt & 1) tile(kt, b1, no);
            else tile(kt, b0, no);
        }
    } else if constexpr (SB) {
        for (int kt = 0; kt < nkt;) {
            tile(kt, b0, no);
            if (++kt >= nkt) break;
            tile(kt, b1, no);
            ++kt;
        }
    } else {
        for (int kt = 0; kt < nkt; ++kt) tile(kt, kt & 1, no);
    }

    {
        // dQ rows through the K and V buffers (RowStage); the last tile's
        // barrier has passed, so no wave reads them any more
        typedef RowStage<E, D> RS;
        static_assert(2 * RS::ELEMS <= NKE, "two output blocks fit one tile buffer");
        E *blk = SB ? ((w >> 1) ? sV0 : sK0) + (w & 1) * RS::ELEMS : sK0 + w * RS::ELEMS;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float q4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) q4[e] = dq[mb][4 * g + e] * scale;
                RS::put(blk, r32, 32 * mb + 8 * g + 4 * h, q4);
            }
        __syncthreads();
        RS::drain(blk, dQ + dqoff, lay.dq.st, qw, T, lane);
    }
}

template <typename E, int D>
static hipError_t launch_bwd_t(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                               const float *LSE, void *dQ, void *dK, void *dV, float *Dbuf, float *dQacc,
                               const Layout &lay, int BH, int T, float scale, int causal, hipStream_t stream,
                               const KernelHook &hook)
{
    const float c_log2 = scale * kLog2e;
    const long long rows = (long long)BH * T;
    constexpr int NW = 4, BQ = 64, BNK = 32 * NW;
    const int nkt = (T + BNK - 1) / BNK;
    if constexpr (sizeof(E) == 2) {  // the atomic path exists for bf16 only
        if (dQacc) {
            hipError_t e = launch_kernel(bwd_pre_kernel<E, D>, dim3((unsigned)((rows * 2 + 255) / 256)), dim3(256),
                                         stream, hook, "attn_bwd_pre", O, dO, Dbuf, dQacc, lay, T, rows);
            if (e != hipSuccess) return e;
            constexpr auto kern = bwd_dkdv_kernel<E, D, NW, BQ, true, sizeof(E) == 2 && D >= 64>;
            const int grid = nkt * BH;
            e = launch_kernel(kern, dim3(grid), dim3(NW * 64), stream, hook, "attn_bwd_dkdv", Q, K, V, dO, LSE, Dbuf,
                              dK, dV, dQacc, lay, T, scale, c_log2, causal, BH, nkt,
                              causal ? serpentine_bins<kern, NW * 64>(grid, hook) : 0);
            if (e != hipSuccess) return e;
            const long long n4 = rows * D / 4;
            return launch_kernel(bwd_dq_convert_kernel<E, D>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), stream,
                                 hook, "attn_bwd_dq_convert", dQacc, dQ, lay, T, scale, n4);
        }
    }
    constexpr bool ASYNC = sizeof(E) == 2 && D >= 64;  // direct HBM -> LDS staging
    constexpr int BN = 64, BM = 32 * NW;
    const int nqt = (T + BM - 1) / BM;
    // the Q-major dQ kernel also computes D = rowsum(dO o O) for its queries
    // and writes it to Dbuf, which the dK/dV kernel then reads
    constexpr auto kq = bwd_dq_kernel<E, D, NW, BN, ASYNC, true>;
    const int gq = nqt * BH;
    auto dq_pass = [&](auto kern_c) {
        constexpr auto kern = decltype(kern_c)::value;
        return launch_kernel(kern, dim3(gq), dim3(NW * 64), stream, hook, "attn_bwd_dq", Q, K, V, O, dO, LSE, Dbuf,
                             dQ, lay, T, scale, c_log2, causal, BH, nqt,
                             causal ? serpentine_bins<kern, NW * 64>(gq, hook) : 0);
    };
    const std::integral_constant<decltype(kq), kq> plain_dq;
    hipError_t e;
    if constexpr (sizeof(E) == 2 && D == 64) {
        // the interleaved variant for long sequences (see bwd_dq_kernel)
        constexpr auto kqi = bwd_dq_kernel<E, D, NW, BN, ASYNC, true, true>;
        e = T >= 2048 ? dq_pass(std::integral_constant<decltype(kqi), kqi>()) : dq_pass(plain_dq);
    } else {
        e = dq_pass(plain_dq);
    }
    if (e != hipSuccess) return e;
    const int gkv = nkt * BH;
    if constexpr (kPairDkDv<E, D>) {
        // one wave pair per 32-key block (see kPairDkDv); 128 keys per workgroup, as below
        constexpr int PW = 8;
        static_assert(32 * (PW / 2) == BNK, "the pair kernel takes the same key blocks");
        constexpr auto kp = bwd_dkdv_pair_kernel<D, PW, BQ>;
        return launch_kernel(kp, dim3(gkv), dim3(PW * 64), stream, hook, "attn_bwd_dkdv", (const bf16 *)Q,
                             (const bf16 *)K, (const bf16 *)V, (const bf16 *)dO, LSE, (const float *)Dbuf,
                             (bf16 *)dK, (bf16 *)dV, lay, T, scale, c_log2, causal, BH, nkt,
                             causal ? serpentine_bins<kp, PW * 64>(gkv, hook) : 0);
    } else {
        // With the direct HBM -> LDS staging, short sequences with enough
        // workgroups take the three-wave general kernel, the rest the two-wave
        // steady kernel (same results bit for bit; see kDkDvGeneralMaxT)
        constexpr auto kkv = bwd_dkdv_kernel<E, D, NW, BQ, false, ASYNC>;
        if constexpr (ASYNC) {
            constexpr auto kkg = bwd_dkdv_kernel<E, D, NW, BQ, false, ASYNC, true>;
            const long long steady_round = (long long)resident_per_cu<kkv, NW * 64>() * hook.cus;
            if (T <= kDkDvGeneralMaxT && steady_round > 0 && gkv >= kDkDvGeneralMinRounds * steady_round)
                return launch_kernel(kkg, dim3(gkv), dim3(NW * 64), stream, hook, "attn_bwd_dkdv", Q, K, V, dO, LSE,
                                     Dbuf, dK, dV, (float *)nullptr, lay, T, scale, c_log2, causal, BH, nkt,
                                     causal ? serpentine_bins<kkg, NW * 64>(gkv, hook) : 0);
        }
        return launch_kernel(kkv, dim3(gkv), dim3(NW * 64), stream, hook, "attn_bwd_dkdv", Q, K, V, dO, LSE, Dbuf, dK,
                             dV, (float *)nullptr, lay, T, scale, c_log2, causal, BH, nkt,
                             causal ? serpentine_bins<kkv, NW * 64>(gkv, hook) : 0);
    }
}

bool bwd_atomic_supported(int dt, int D) { return dt == 1 && (D == 32 || D == 64 || D == 128); }

hipError_t launch_bwd(int dt, int D, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                      const float *LSE, void *dQ, void *dK, void *dV, float *Dbuf, float *dQacc, const Layout &lay,
                      int BH, int T, float scale, int causal, hipStream_t stream, const KernelHook &hook)
{
#define ATTN_BWD_CASE(E, DD)                                                                                 \
    if (D == DD)                                                                                             \
        return launch_bwd_t<E, DD>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dbuf, dQacc, lay, BH, T, scale, causal, \
                                   stream, hook);
    if (dt == 0) {
        if (dQacc) return hipErrorInvalidValue;  // fp32 always takes the deterministic dQ pass
        ATTN_BWD_CASE(float, 32) ATTN_BWD_CASE(float, 64) ATTN_BWD_CASE(float, 128)
    } else {
        ATTN_BWD_CASE(bf16, 32) ATTN_BWD_CASE(bf16, 64) ATTN_BWD_CASE(bf16, 128)
    }
#undef ATTN_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace attn
