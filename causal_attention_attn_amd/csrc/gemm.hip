// gemm.hip -- the dense layer products around attention in a GPT-2 decoder
// step, bf16 operands with fp32 accumulation on the gfx950 matrix cores:
//   GEMM_NT  C = A B^T   A [M, K], B [N, K]  (forward X W^T, weights [out, in])
//   GEMM_NN  C = A B     A [M, K], B [K, N]  (input gradient dX = dY W)
//   GEMM_TN  C = A^T B   A [K, M], B [K, N]  (weight gradient dW = dY^T X)
// These are the three products Forge times for its MLP ("Forge: Building an
// LLM Training Framework from Scratch in C++ and Metal on Apple Silicon",
// section "Results", GEMM table): the weight gradient has a very long
// contraction (K = B T tokens) and few output tiles, which Forge leaves
// unsplit; here the contraction can be split over workgroups, each writing
// an fp32 partial product that a second kernel sums in a fixed order.
//
// Design (a 128 x 128 output tile per 4-wave workgroup, or 256 x 256 per
// 8-wave workgroup when there are enough such tiles to fill the chip;
// 64-deep contraction tiles):
//   * A and B tiles are staged HBM -> LDS by direct copies
//     (buffer_load_dwordx4 ... lds) into XOR-swizzled tiles, double-buffered,
//     the next contraction tile in flight while the current one is used;
//   * an operand stored contraction-major (row of A or B^T along k) is read
//     as 16-byte row fragments; one stored output-major (k rows) is read with
//     the LDS transpose read, so every layout feeds the same MFMA fragments;
//   * each wave owns a 64 x 64 (128 x 64 in the large tile) part of the tile
//     as 32 x 32 fp32 accumulators and computes its transpose (C^T = B A^T),
//     which leaves four consecutive output columns in each lane for
//     8/16-byte stores; the large tile reads 6 fragments per 8 products
//     instead of 4 per 4;
//   * each XCD takes one contiguous run of output tiles, walked in groups
//     of m-tiles whose size the host picks per shape so that the runs touch
//     the fewest A and B panels (each XCD fills its own L2 with them);
//   * the result leaves through the operand buffers (RowStage), whole rows
//     per store instruction (mlp_fwd 737 -> 832 TFLOP/s, 4096^3 1104 -> 1177).
#include <algorithm>
#include <type_traits>

#include <atomic>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int GBK = 64;  // contraction tile

// Output tile BM x BN over WM x WN waves; each wave holds MB x NB 32 x 32
// accumulators.
template <int BM_, int BN_, int WM_, int WN_> struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NW = WM_ * WN_;
    static constexpr int MB = BM_ / WM_ / 32, NB = BN_ / WN_ / 32;
};
typedef GemmCfg<128, 128, 2, 2> CfgSmall;
typedef GemmCfg<256, 256, 2, 4> CfgLarge;

// Direct HBM -> LDS copy of a [R x W] window of a row-major bf16 matrix
// (leading dimension ld) starting at (row0, col0), into an LDS tile laid out
// as SwzLayout<W>.  Rows at or past nrows read row nrows - 1 and 8-column
// chunks at or past ncols read the last chunk (ncols is a multiple of 8):
// those tile entries only ever meet outputs that are not stored.
template <int R, int W, int NW, bool BUFFER = true>
__device__ __forceinline__ void gemm_dma(bf16 *tile, const bf16 *__restrict__ src, int ld, int row0, int nrows,
                                         int col0, int ncols, int w, int lane)
{
    typedef SwzLayout<W> L;
    constexpr int RPI = 512 / W;  // rows per 1 KB instruction
    constexpr int CPR = W / 8;    // 16-byte chunks per row
    constexpr int NI = R / RPI;
    static_assert(NI % NW == 0, "tile copies must split evenly over the waves");
    const int last_col = ncols - 8;
    // buffer-form copies (see SwzLayout::dma: they leave the waits for LDS
    // reads precise) relative to the window's first row, so that byte offsets
    // stay within R rows of the matrix; the global form where the finer
    // waits let the scheduler keep more fragments live than the registers hold
    const int rbase = min(row0, nrows - 1);
    const bf16 *wsrc = src + (long long)rbase * ld;
    const __amdgpu_buffer_rsrc_t rs = slab_rsrc(wsrc);
#pragma unroll
    for (int i = 0; i < NI / NW; ++i) {
        const int blk = w * (NI / NW) + i;
        const int r = blk * RPI + lane / CPR;
        const int gr = min(row0 + r, nrows - 1) - rbase;
        const int gc = min(col0 + 8 * ((lane % CPR) ^ L::swz(r)), last_col);
        if constexpr (BUFFER)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void __attribute__((address_space(3))) *)(tile + blk * 512),
                                                     16, 2u * (unsigned)(gr * ld + gc), 0, 0, 0);
        else
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(wsrc + (long long)gr * ld + gc),
                (void __attribute__((address_space(3))) *)(tile + blk * 512), 16, 0, 0);
    }
}

// Fragment of a contraction-major tile ([rows x 64 k], SwzLayout<64>): row
// 32 rb + r32, k = 16 kk + 8 h + t.
__device__ __forceinline__ bf16x8 frag_kmajor(const bf16 *t, int rb, int kk, int lane)
{
    const int r32 = lane & 31, h = lane >> 5;
    return load_row8(t + SwzLayout<GBK>::off(32 * rb + r32, 16 * kk + 8 * h));
}

// Fragment of an output-major tile ([64 k x W], SwzLayout<W>): column
// 32 cb + r32, k = 16 kk + 8 h + t, gathered by two transpose reads of four
// rows each (rows 16 kk + 8 h + 0..3, then + 4..7).
template <int W> __device__ __forceinline__ bf16x8 frag_mnmajor(const bf16 *t, int cb, int kk, int lane)
{
    const int L16 = lane & 15, h = lane >> 5;
    const int col = 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (L16 & 3);
    const int r0 = 16 * kk + 8 * h + (L16 >> 2);
    const bf16x4 a = ds_read_tr4(t + SwzLayout<W>::off(r0, col));
    const bf16x4 b = ds_read_tr4(t + SwzLayout<W>::off(r0 + 4, col));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A is contraction-major for NT and NN, B for NT only.
template <int OP> struct GemmOps {
    static constexpr bool kAK = OP != GEMM_KIND_TN;
    static constexpr bool kBK = OP == GEMM_KIND_NT;
};

template <int OP, typename OutT, typename G>
__global__ __launch_bounds__(G::NW * 64) void gemm_kernel(const bf16 *__restrict__ A, const bf16 *__restrict__ B,
                                                          OutT *__restrict__ C, float *__restrict__ part, int M, int N,
                                                          int K, int lda, int ldb, int ldc, int kchunk, int tiles_m,
                                                          int tiles_n, int group_m)
{
    typedef GemmOps<OP> O;
    constexpr int GBM = G::BM, GBN = G::BN, NW = G::NW, MB = G::MB, NB = G::NB;
    __shared__ __attribute__((aligned(16))) bf16 sA0[GBM * GBK];
    __shared__ __attribute__((aligned(16))) bf16 sA1[GBM * GBK];
    __shared__ __attribute__((aligned(16))) bf16 sB0[GBN * GBK];
    __shared__ __attribute__((aligned(16))) bf16 sB1[GBN * GBK];

    const int lane = threadIdx.x & 63;
    const int w = wave_index();
    const int r32 = lane & 31, h = lane >> 5;

    // Work order.  Consecutive workgroups go to different XCDs (round robin
    // over eight), so first undo that interleave: each XCD then takes one
    // contiguous run of (split, tile) items, split-major, so that with a
    // split contraction an XCD works on one or two chunks of K only and
    // streams those slices of A and B through its own L2 once, instead of
    // every XCD reading every chunk.  Inside a split the tiles are walked in
    // groups of group_m m-tiles, m fastest (gemm_walk_group).
    const int tiles = tiles_m * tiles_n;
    int v = blockIdx.x;
    if (gridDim.x % 8 == 0) v = (v % 8) * (gridDim.x / 8) + v / 8;
    const int s = v / tiles;
    int t = v - s * tiles;
    const int gitems = group_m * tiles_n;
    const int group = t / gitems;
    const int first_m = group * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int tm = first_m + (t % gitems) % gsize;
    const int tn = (t % gitems) / gsize;
    const int m0 = tm * GBM, n0 = tn * GBN;
    const int k_begin = s * kchunk;
    const int nkt = (min(K, k_begin + kchunk) - k_begin) / GBK;  // >= 1 (checked on the host)

    // the 256 x 256 tile with both operands output-major spills with the
    // buffer form (256 VGPRs and 20-40 bytes of scratch against 238-242)
    constexpr bool BUF = !(OP == GEMM_KIND_TN && GBM == 256);
    auto request = [&](int kt, bf16 *tA, bf16 *tB) __attribute__((always_inline)) {
        const int k0 = k_begin + kt * GBK;
        if constexpr (O::kAK)
            gemm_dma<GBM, GBK, NW, BUF>(tA, A, lda, m0, M, k0, K, w, lane);
        else
            gemm_dma<GBK, GBM, NW, BUF>(tA, A, lda, k0, K, m0, M, w, lane);
        if constexpr (O::kBK)
            gemm_dma<GBN, GBK, NW, BUF>(tB, B, ldb, n0, N, k0, K, w, lane);
        else
            gemm_dma<GBK, GBN, NW, BUF>(tB, B, ldb, k0, K, n0, N, w, lane);
    };

    // this wave: m 32 MB wm .. +32 MB - 1, n 32 NB wn .. +32 NB - 1 of the tile
    const int wm = w % G::WM, wn = w / G::WM;
    f32x16 acc[NB][MB];  // [n block][m block] of C^T
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = zero16();

    auto compute = [&](const bf16 *tA, const bf16 *tB) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < GBK / 16; ++kk) {
            bf16x8 fa[MB], fb[NB];
#pragma unroll
            for (int j = 0; j < MB; ++j)
                fa[j] = O::kAK ? frag_kmajor(tA, MB * wm + j, kk, lane) : frag_mnmajor<GBM>(tA, MB * wm + j, kk, lane);
#pragma unroll
            for (int i = 0; i < NB; ++i)
                fb[i] = O::kBK ? frag_kmajor(tB, NB * wn + i, kk, lane) : frag_mnmajor<GBN>(tB, NB * wn + i, kk, lane);
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < MB; ++j) mma32(acc[i][j], fb[i], fa[j]);
        }
    };

    request(0, sA0, sB0);
    for (int kt = 0;;) {
        // even tiles in buffers 0, odd tiles in buffers 1: every read names
        // its buffer at compile time (see the attention kernels)
        barrier_vm<0>();  // tile kt landed; tile kt-1 no longer read
        if (kt + 1 < nkt) request(kt + 1, sA1, sB1);
        compute(sA0, sB0);
        if (++kt >= nkt) break;
        barrier_vm<0>();
        if (kt + 1 < nkt) request(kt + 1, sA0, sB0);
        compute(sA1, sB1);
        if (++kt >= nkt) break;
    }

    // acc[i][j][4 g + e]: row n = n0 + 32 (NB wn + i) + 8 g + 4 h + e of C^T,
    // column m = m0 + 32 (MB wm + j) + r32, i.e. C[m][n .. n+3].  Stored
    // through the (now unused) operand buffers, one 32-row block j at a time
    // (RowStage): the wave's 32 x 32 NB block of C, then whole rows.
    auto epilogue = [&](auto *dst, int st, size_t row_base, auto keep) __attribute__((always_inline)) {
        typedef typename std::remove_pointer<decltype(dst)>::type T;
        typedef RowStage<T, 32 * NB> RS;
        constexpr int PER = (int)(sizeof(sA0) / (RS::ELEMS * sizeof(T)));  // wave blocks per buffer
        static_assert(NW <= 2 * PER, "every wave's block fits the A buffers");
        T *blk = reinterpret_cast<T *>(w / PER ? sA1 : sA0) + (w % PER) * RS::ELEMS;
        const int ncols = min(32 * NB, N - (n0 + 32 * NB * wn));
        __syncthreads();  // every wave is done with the operand tiles
#pragma unroll
        for (int j = 0; j < MB; ++j) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
                    RS::put(blk, r32, 32 * i + 8 * g + 4 * h, v);
                }
            __syncthreads();
            RS::template drain<decltype(keep)::value>(blk, dst + row_base + n0 + 32 * NB * wn, st,
                                                       m0 + 32 * (MB * wm + j), M, lane, ncols);
            __syncthreads();  // block drained before the next one is put
        }
    };
    if (part)
        epilogue(part, N, (size_t)s * M * N, std::true_type());  // read back by the reduce kernel
    else
        epilogue(C, ldc, 0, std::false_type());
}

// C = sum over the splits of the fp32 partial products, in split order.
template <typename OutT>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float *__restrict__ part, OutT *__restrict__ C, int M,
                                                          int N, int ldc, int splits)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // group of 4 outputs
    const long long n4 = (long long)M * (N / 4);
    if (i >= n4) return;
    const int m = (int)(i / (N / 4)), n = 4 * (int)(i % (N / 4));
    const size_t plane = (size_t)M * N;
    f32x4 a = *reinterpret_cast<const f32x4 *>(part + (size_t)m * N + n);
    for (int s = 1; s < splits; ++s) a += *reinterpret_cast<const f32x4 *>(part + s * plane + (size_t)m * N + n);
    const float v[4] = {a[0], a[1], a[2], a[3]};
    store4(C + (size_t)m * ldc + n, v);
}

// Whether the 256 x 256 tile is used: only without a split, and when its
// tiles fill every compute unit a whole number of times or at least three
// times over (one such workgroup fits per compute unit).
bool gemm_large_tiles(int M, int N, int used)
{
    const long long t = (long long)((M + 255) / 256) * ((N + 255) / 256);
    return used == 1 && t >= 256 && (t % 256 == 0 || t >= 768);
}

// A and B panels (an m-tile's rows of A, an n-tile's rows of B, per
// contraction chunk) read by the items [a, b) of the work order, the tiles
// of each split walked in groups of g m-tiles, m fastest.  Inside a group
// item u is m-tile u % gs, n-tile u / gs (gs m-tiles in the group): a
// partial group of fewer than gs items touches that many m-tiles, and the
// n-tiles of one group form an interval, the whole range unless the group
// is partial.  Different groups have different m-tiles; only the first and
// the last group of a run can be partial.
long long walk_panels(long long a, long long b, int tiles_m, int tiles_n, int g)
{
    const long long tiles = (long long)tiles_m * tiles_n, gitems = (long long)g * tiles_n;
    long long count = 0;
    while (a < b) {
        const long long s = a / tiles, ta = a - s * tiles, tb = std::min(b - s * tiles, tiles);
        long long m = 0;
        int lo[2] = {0, 0}, hi[2] = {-1, -1}, parts = 0;
        bool all_n = false;
        for (long long gi = ta / gitems; gi <= (tb - 1) / gitems; ++gi) {
            const int gs = std::min(tiles_m - (int)(gi * g), g);
            const long long ua = std::max(ta, gi * gitems) - gi * gitems;
            const long long ub = std::min(tb, gi * gitems + (long long)gs * tiles_n) - gi * gitems;
            m += std::min<long long>(ub - ua, gs);
            const int nl = (int)(ua / gs), nh = (int)((ub - 1) / gs);
            if (nl == 0 && nh == tiles_n - 1)
                all_n = true;
            else if (parts < 2) {
                lo[parts] = nl;
                hi[parts++] = nh;
            }
        }
        long long n = tiles_n;
        if (!all_n) {
            n = hi[0] - lo[0] + 1;
            if (parts == 2) n += hi[1] - lo[1] + 1 - std::max(0, std::min(hi[0], hi[1]) - std::max(lo[0], lo[1]) + 1);
        }
        count += m + n;
        a = s * tiles + tb;
    }
    return count;
}

// Group size of the tile walk: of 1, 2, 4 and 8 (at most tiles_m), the one
// whose eight XCD runs read the fewest panels in total, 8 on a tie or when
// the grid does not split into eight equal runs.  dY^T X for 3072 x 768
// weights, its 8192 tokens in three chunks (24 x 6 tiles per chunk), walks
// row by row: 91-94 MiB read into the L2s against 126 at 8.  Larger groups
// can cost fewer panels but measured worse, the L2 holding fewer of them
// at once (X W1^T, 64 x 24 tiles: 51 MiB at 16 against 48 at 8).
int gemm_walk_group(int tiles_m, int tiles_n, int splits)
{
    const long long items = (long long)tiles_m * tiles_n * splits;
    const int largest = std::min(8, tiles_m);
    if (items % 8 != 0) return largest;
    auto cost = [&](int g) {
        long long c = 0;
        for (int x = 0; x < 8; ++x) c += walk_panels(x * items / 8, (x + 1) * items / 8, tiles_m, tiles_n, g);
        return c;
    };
    int best = largest;
    long long best_cost = cost(best);
    for (int g = 1; g < largest; g *= 2) {
        const long long c = cost(g);
        if (c < best_cost) best = g, best_cost = c;
    }
    return best;
}

template <int OP, typename OutT, typename G>
hipError_t launch_gemm_cfg(const void *A, const void *B, void *C, float *part, int M, int N, int K, int lda, int ldb,
                           int ldc, int kchunk, int used, hipStream_t stream, const KernelHook &hook)
{
    const int tiles_m = (M + G::BM - 1) / G::BM, tiles_n = (N + G::BN - 1) / G::BN;
    return launch_kernel(gemm_kernel<OP, OutT, G>, dim3(tiles_m * tiles_n * used), dim3(G::NW * 64), stream, hook,
                         "gemm", (const bf16 *)A, (const bf16 *)B, (OutT *)C, used > 1 ? part : (float *)nullptr, M, N,
                         K, lda, ldb, ldc, kchunk, tiles_m, tiles_n, gemm_walk_group(tiles_m, tiles_n, used));
}

template <int OP, typename OutT>
hipError_t launch_gemm_t(const void *A, const void *B, void *C, float *part, int M, int N, int K, int lda, int ldb,
                         int ldc, int kchunk, hipStream_t stream, const KernelHook &hook)
{
    const int used = (K + kchunk - 1) / kchunk;  // contraction chunks, each non-empty
    hipError_t e = gemm_large_tiles(M, N, used)
                       ? launch_gemm_cfg<OP, OutT, CfgLarge>(A, B, C, part, M, N, K, lda, ldb, ldc, kchunk, used,
                                                             stream, hook)
                       : launch_gemm_cfg<OP, OutT, CfgSmall>(A, B, C, part, M, N, K, lda, ldb, ldc, kchunk, used,
                                                             stream, hook);
    if (e != hipSuccess || used == 1) return e;
    const long long n4 = (long long)M * (N / 4);
    return launch_kernel(gemm_reduce_kernel<OutT>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), stream, hook,
                         "gemm_reduce", (const float *)part, (OutT *)C, M, N, ldc, used);
}

}  // namespace

int gemm_split_chunk(int K, int splits)
{
    const int kt = K / GBK;
    return ((kt + splits - 1) / splits) * GBK;
}

int gemm_resident_slots()
{
    constexpr int kDefault = 2 * 256;
    static std::atomic<int> slots[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefault;
    int n = slots[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return kDefault;
    // the fewest resident workgroups of any 128 x 128 instantiation
    int occ = 1 << 30;
    auto q = [&](const void *kern) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kern, CfgSmall::NW * 64, 0) == hipSuccess && b > 0)
            occ = b < occ ? b : occ;
    };
    q(reinterpret_cast<const void *>(gemm_kernel<GEMM_KIND_NT, bf16, CfgSmall>));
    q(reinterpret_cast<const void *>(gemm_kernel<GEMM_KIND_NN, bf16, CfgSmall>));
    q(reinterpret_cast<const void *>(gemm_kernel<GEMM_KIND_TN, bf16, CfgSmall>));
    q(reinterpret_cast<const void *>(gemm_kernel<GEMM_KIND_NT, float, CfgSmall>));
    q(reinterpret_cast<const void *>(gemm_kernel<GEMM_KIND_NN, float, CfgSmall>));
    q(reinterpret_cast<const void *>(gemm_kernel<GEMM_KIND_TN, float, CfgSmall>));
    if (occ == (1 << 30)) return kDefault;
    n = cus * occ;
    slots[dev].store(n, std::memory_order_relaxed);
    return n;
}

int gemm_auto_splits(int M, int N, int K)
{
    // The largest split whose workgroups (tiles x splits) are all resident at
    // once -- compute units x workgroups per unit, 256 x 2 on MI355X -- with at
    // least 8 contraction tiles per split.  A second, partly filled round of
    // workgroups, or a reduce that is not needed, costs more than idle slots:
    // dY W1 (8192 x 768 x 3072) takes 48.6 us unsplit against 55.9 us in two
    // splits, dY^T X (3072 x 768 x 8192) 52.9 us in three against 62.9 and
    // 64.2 us in two and four.
    const long long slots = gemm_resident_slots();
    const long long tiles = (long long)((M + CfgSmall::BM - 1) / CfgSmall::BM) * ((N + CfgSmall::BN - 1) / CfgSmall::BN);
    int s = 1;
    while (tiles * (s + 1) <= slots && (K / GBK) / (s + 1) >= 8) ++s;
    return s;
}

hipError_t launch_gemm(int op, int c_f32, const void *A, const void *B, void *C, float *part, int M, int N, int K,
                       int lda, int ldb, int ldc, int kchunk, hipStream_t stream, const KernelHook &hook)
{
#define ATTN_GEMM_CASE(OPV)                                                                                        \
    case OPV:                                                                                                      \
        return c_f32 ? launch_gemm_t<OPV, float>(A, B, C, part, M, N, K, lda, ldb, ldc, kchunk, stream, hook)     \
                     : launch_gemm_t<OPV, bf16>(A, B, C, part, M, N, K, lda, ldb, ldc, kchunk, stream, hook);
    switch (op) {
        ATTN_GEMM_CASE(GEMM_KIND_NT)
        ATTN_GEMM_CASE(GEMM_KIND_NN)
        ATTN_GEMM_CASE(GEMM_KIND_TN)
    }
#undef ATTN_GEMM_CASE
    return hipErrorInvalidValue;
}

}  // namespace attn
