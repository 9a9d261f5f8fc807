// attn_device.h -- gfx950 device building blocks shared by the attention
// kernels: MFMA wrappers, operand-fragment loads from LDS tiles, cooperative
// HBM -> LDS tile staging and small wave-level helpers.
//
// Matrix-core convention used throughout (CDNA3/CDNA4 32x32 MFMA layouts):
//   * an operand fragment is 8 elements of one lane along the contraction
//     index k; lane l = 32*h + r supplies row/column r of its 32-wide matrix
//     and, in a 16-wide k chunk, the elements k = 8h + t (t = 0..7);
//   * the fp32 32x32 accumulator tile holds, in lane l = 32*h + n and
//     register j, the element (row 8*(j/4) + 4*h + j%4, column n).
// bf16 chunks are one v_mfma_f32_32x32x16_bf16; fp32 chunks are eight
// v_mfma_f32_32x32x2_f32 steps, step t pairing element t of both lane halves.
// Only the pairing of A and B elements matters for a contraction, so any
// fixed assignment of contraction indices to (h, t) is valid as long as both
// operands use it.  When an accumulator tile is fed back as a B operand, its
// rows become the contraction index with the assignment
//   key(kk, h, t) = 16*kk + 8*(t/4) + 4*h + t%4          (chunk kk = 0, 1)
// and the matching A operand is gathered with the same assignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename E> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

// Row stride of an LDS tile holding rows of D elements: one 16-byte pad per
// row so that the 16-byte row-fragment reads of 16 consecutive rows fall in
// distinct bank groups.
template <typename E, int D> struct Tile {
    static constexpr int kStride = D + 16 / (int)sizeof(E);
};

__device__ __forceinline__ void mma32(f32x16 &acc, bf16x8 a, bf16x8 b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma32(f32x16 &acc, f32x8 a, f32x8 b)
{
#pragma unroll
    for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16()
{
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// 8 consecutive elements of a row (16-byte aligned for bf16; fp32 rows are
// 16-byte aligned, so two 16-byte reads).
__device__ __forceinline__ bf16x8 load_row8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f32x8 load_row8(const float *p)
{
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[i + 4] = b[i]; }
    return r;
}

template <typename E> __device__ __forceinline__ typename Frag<E>::type zero_frag()
{
    typename Frag<E>::type r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (E)0.f;
    return r;
}

template <typename E> __device__ __forceinline__ typename Frag<E>::type neg_frag(typename Frag<E>::type v)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (E)(-(float)v[i]);
    return v;
}

// A-operand gather for a contraction over tile rows: 8 elements of column
// `col` at rows base + {0,1,2,3, 8,9,10,11} (base = 16*kk + 4*h), the row
// assignment key(kk, h, t) above.
template <typename E, int STR>
__device__ __forceinline__ typename Frag<E>::type load_col8(const E *tile, int base, int col)
{
    typename Frag<E>::type r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = tile[(base + (t & 3) + 8 * (t >> 2)) * STR + col];
    return r;
}

// The same gather from a bf16 tile with the LDS transpose read
// ds_read_b64_tr_b16.  Within each group of 16 lanes the instruction hands
// lane i element e of the 8 bytes loaded by lane 4*e + i/4, element i%4; so
// if lane L of the group loads row r0 + L/4, columns c0 + 4*(L%4) .. +3, lane
// i receives rows r0..r0+3 of column c0 + i.  Two reads (rows +0 and +8)
// give the 8 elements.  `colblock` is the 32-column block (32*mb); lane
// 32*h + r32 receives column colblock + r32.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x4 ds_read_tr4(const bf16 *p)
{
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

template <typename E, int STR> struct ColGather;

template <int STR> struct ColGather<bf16, STR> {
    static __device__ __forceinline__ bf16x8 load(const bf16 *tile, int base, int colblock, int lane)
    {
        const int L = lane & 15;
        const bf16 *p = tile + (base + (L >> 2)) * STR + colblock + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
        const bf16x4 a = ds_read_tr4(p);
        const bf16x4 b = ds_read_tr4(p + 8 * STR);
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

template <int STR> struct ColGather<float, STR> {
    static __device__ __forceinline__ f32x8 load(const float *tile, int base, int colblock, int lane)
    {
        return load_col8<float, STR>(tile, base, colblock + (lane & 31));
    }
};

// Tile layouts.  A layout maps (tile row, column) to LDS elements and provides
// the two operand reads the kernels use: row8 (8 consecutive elements of a
// row, column a multiple of 8) and colA (the transposed A-operand gather).
//
// PadLayout: rows of D elements plus a 16-byte pad, filled by register stores.
template <typename E, int D> struct PadLayout {
    static constexpr int STR = Tile<E, D>::kStride;
    static constexpr int elems(int rows) { return rows * STR; }
    static __device__ __forceinline__ const E *row8(const E *t, int r, int col) { return t + r * STR + col; }
    static __device__ __forceinline__ typename Frag<E>::type colA(const E *t, int base, int colblock, int lane)
    {
        return ColGather<E, STR>::load(t, base, colblock, lane);
    }
};

// Buffer resource for raw (unformatted) loads relative to p: no stride, the
// whole 32-bit record range (no access is ever out of range), and gfx950's
// format word for raw dword access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void *p)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, -1, 0x00020000);
}

// SwzLayout: unpadded bf16 rows (D >= 64) filled by direct HBM -> LDS loads,
// which write each wave's 64 x 16 bytes contiguously and so cannot pad.  The
// 16-byte chunk c of row r sits at chunk position c ^ swz(r).  gfx950's LDS
// serves 256 bytes (sixteen 16-byte bank groups) per cycle, so a 16-byte row
// fragment read is conflict-free when its 16 lanes (16 consecutive rows, one
// chunk) hit 16 different groups, and a transposed read when each 32-lane
// half (4 consecutive rows, 4 adjacent chunks) does:
//   d = 64 (128-byte rows, two per 256 bytes):  swz(r) = 4((r/2)%2) + (r/4)%4
//   d >= 128 (whole 256-byte periods per row):  swz(r) = 4(r%4) + (r/4)%4
// Both depend on r % 16 only.  (An 8-row swizzle, 2(r%4) + (r/4)%2, gave
// two-way conflicts on the row fragments, and at d = 128 on the transposed
// reads too, by the SQ_LDS_BANK_CONFLICT counter.)
template <int D> struct SwzLayout {
    static_assert(D >= 64, "at least eight 16-byte chunks per row");
    static constexpr int elems(int rows) { return rows * D; }
    static __device__ __forceinline__ int swz(int r)
    {
        return D == 64 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 3) : 4 * (r & 3) + ((r >> 2) & 3);
    }
    static __device__ __forceinline__ int off(int r, int col) { return r * D + ((((col >> 3) ^ swz(r)) << 3) | (col & 7)); }
    static __device__ __forceinline__ const bf16 *row8(const bf16 *t, int r, int col) { return t + off(r, col); }
    static __device__ __forceinline__ bf16x8 colA(const bf16 *t, int base, int colblock, int lane)
    {
        const int L = lane & 15;
        const int r = base + (L >> 2);
        const int col = colblock + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
        // both addresses are formed from the tile pointer in one step, which
        // keeps the compiler's knowledge of which LDS variable they read (the
        // kernels that rely on it overlap reads of one buffer with copies
        // into another)
        const bf16x4 a = ds_read_tr4(t + off(r, col));
        const bf16x4 b = ds_read_tr4(t + off(r + 8, col));
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }

    // Direct HBM -> LDS copy of rows [row0, row0 + R) of a [T, D] slab whose
    // rows are `stride` elements apart, by the NW waves of a block: each
    // buffer_load_dwordx4 ... lds moves 1 KB (512 / D rows); lane L fills
    // chunk position L % (D/8) of its row with the global chunk that belongs
    // there.  Rows at or past T are clamped to row T - 1 (finite data that
    // every caller masks or multiplies by zero).  The copies use the buffer
    // form rather than global_load_lds: the compiler counts a global (flat
    // encoded) load into LDS as pending on both the vector-memory and the LDS
    // counter, so while one was in flight every wait for an LDS read waited
    // for all of them (lgkmcnt(0)); with the buffer form each matrix product
    // waits only for its own operands.
    template <int R, int NW>
    static __device__ __forceinline__ void dma(bf16 *tile, const bf16 *__restrict__ src, int stride, int row0,
                                               int T, int w, int lane)
    {
        constexpr int RPI = 512 / D;  // rows per instruction
        constexpr int CPR = D / 8;    // chunks per row
        constexpr int NI = R / RPI;   // instructions per tile
        static_assert(NI % NW == 0, "tile instructions must split evenly over the waves");
        // rows past T read row T-1 (stride >= 0, so clamping the offset clamps the row);
        // base and lim are uniform, r * stride does not change from tile to tile.
        // Byte offsets within the slab fit in 32 bits (element offsets fit in
        // int32, checked on the host), and no offset is out of the record range.
        const __amdgpu_buffer_rsrc_t rs = slab_rsrc(src);
        const int base = row0 * stride, lim = (T - 1) * stride;
#pragma unroll
        for (int i = 0; i < NI / NW; ++i) {
            const int blk = w * (NI / NW) + i;
            const int r = blk * RPI + lane / CPR;
            const int c = (lane % CPR) ^ swz(r);
            const unsigned voff = 2u * (unsigned)(min(base + r * stride, lim) + 8 * c);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void __attribute__((address_space(3))) *)(tile + blk * 512),
                                                     16, voff, 0, 0, 0);
        }
    }
    template <int R, int NW> static constexpr int dma_per_wave() { return (R / (512 / D)) / NW; }
};

// Work item of workgroup `bid` in a grid of `grid` workgroups whose items are
// numbered heaviest first.  When the whole grid is resident at once the
// dispatcher deals it out one workgroup per compute unit per round, so plain
// order gives the first compute units all the heaviest items.  With `bins`
// (the compute-unit count) > 0, odd rounds take their items in reverse, so
// that each compute unit's heavy item of one round meets a light one of the
// next.  The reversal moves whole groups of eight, keeping each item at its
// position modulo 8: consecutive items then keep sharing a cache domain.
__device__ __forceinline__ int serpentine(int bid, int grid, int bins)
{
    if (bins <= 0) return bid;
    const int round = bid / bins;
    if (!(round & 1)) return bid;
    const int first = round * bins;
    const int cnt = min(bins, grid - first);
    const int r = bid - first;
    if ((cnt & 7) == 0) return first + (cnt - 8 - (r & ~7)) + (r & 7);
    return first + cnt - 1 - r;
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: branches on it and on what derives from it stay scalar instead of
// being linearised under execution masks.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// The fragments a wave reads from a swizzled tile (SwzLayout<D>), as
// per-lane element offsets from the start of a 32-row sub-block.  The swizzle
// of row r depends on r % 16 only, so moving by whole sub-blocks or 16-row
// halves of the transposed gathers adds a constant: one register per 16-column
// row fragment and two per 32-column gather block (its rows and the rows 8
// further) serve every buffer and sub-block.  launder() hides their
// values from the compiler once per loop iteration, so that it adds each
// buffer's base where a read is issued (into the instruction's offset field)
// instead of keeping a register per buffer and fragment.  Addresses are
// formed from the tile pointer in one step, which keeps the compiler's
// knowledge of which LDS variable a read touches.
template <int D> struct SwzFrags {
    static constexpr int NC = D / 16;
    static constexpr int NMB = D / 32;
    // byte offsets into a tile, so that an address is one add of the tile base
    int row[NC];   // row fragment: row r32, columns 16c + 8h .. +7
    int tr[NMB];   // transposed gather, rows 4h + (lane%16)/4, columns 32mb + 16((lane/16)%2) + 4(lane%4)
    int tr8[NMB];  // the same columns, rows 8 further
    __device__ __forceinline__ void init(int lane)
    {
        typedef SwzLayout<D> L;
        const int r32 = lane & 31, h = lane >> 5, L16 = lane & 15;
#pragma unroll
        for (int c = 0; c < NC; ++c) row[c] = 2 * L::off(r32, 16 * c + 8 * h);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            const int col = 32 * mb + 16 * ((lane >> 4) & 1) + 4 * (L16 & 3);
            tr[mb] = 2 * L::off(4 * h + (L16 >> 2), col);
            tr8[mb] = 2 * L::off(4 * h + (L16 >> 2) + 8, col);
        }
    }
    __device__ __forceinline__ void launder()
    {
#pragma unroll
        for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(row[c]));
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            asm volatile("" : "+v"(tr[mb]));
            asm volatile("" : "+v"(tr8[mb]));
        }
    }
    static __device__ __forceinline__ const bf16 *at(const bf16 *t, int bytes)
    {
        return reinterpret_cast<const bf16 *>(reinterpret_cast<const char *>(t) + bytes);
    }
    // A-operand row fragment c of row r32 of sub-block sb
    __device__ __forceinline__ bf16x8 row8(const bf16 *t, int sb, int c) const
    {
        return load_row8(at(t + 32 * D * sb, row[c]));
    }
    // A-operand transposed gather: rows 32 sb + 16 kk + (4h + (lane%16)/4 and
    // + 8), column block mb (the layout of SwzLayout<D>::colA)
    __device__ __forceinline__ bf16x8 colA(const bf16 *t, int sb, int kk, int mb) const
    {
        const bf16 *base = t + (32 * sb + 16 * kk) * D;
        const bf16x4 a = ds_read_tr4(at(base, tr[mb]));
        const bf16x4 b = ds_read_tr4(at(base, tr8[mb]));
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// s_waitcnt with vmcnt <= N, lgkmcnt = 0, expcnt untouched (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits 15:14), then a
// workgroup barrier.  Unlike __syncthreads() it leaves the N most recent
// direct-to-LDS loads of this wave in flight.
template <int N> __device__ __forceinline__ void barrier_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
}

// Half-wave reductions: v_permlane32_swap(x, x) leaves (x_l, x_{l+32}) in the
// two results of lane l < 32 and (x_{l-32}, x_l) in lane l >= 32, so both
// halves combine the same pair in the same order.
__device__ __forceinline__ float half_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A tile of R rows x D columns held in registers between its HBM load and its
// LDS store, so the load of the next tile overlaps the math on the current one.
template <typename E, int D, int R, int NT> struct TileRegs {
    static constexpr int kVec = 16 / (int)sizeof(E);
    static constexpr int kCpr = D / kVec;
    static constexpr int kChunks = R * kCpr;
    static constexpr int kIt = kChunks / NT;
    static_assert(kChunks % NT == 0, "tile chunk count must be a multiple of the block size");
    u32x4 v[kIt];

    // rows row0.. of a [T, D] slab whose rows are `stride` elements apart;
    // rows at or past T repeat row T - 1, as the direct-to-LDS copies do
    // (every kernel gives those rows a zero weight: masked scores, LSE = +inf
    // or dS = 0).  The loads are unconditional, so a caller can issue several
    // tiles and operands before its first wait.
    __device__ __forceinline__ void load(const E *__restrict__ src, int stride, int row0, int T, int tid)
    {
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int idx = tid + it * NT;
            const int r = min(row0 + idx / kCpr, T - 1);
            v[it] = *reinterpret_cast<const u32x4 *>(src + r * stride + (idx % kCpr) * kVec);
        }
    }
    // the same, with rows at or past T set to zero (for a tile whose rows
    // past T meet nonzero weights)
    __device__ __forceinline__ void load_zero_past(const E *__restrict__ src, int stride, int row0, int T, int tid)
    {
        load(src, stride, row0, T, tid);
#pragma unroll
        for (int it = 0; it < kIt; ++it)
            if (row0 + (tid + it * NT) / kCpr >= T) v[it] = u32x4{0u, 0u, 0u, 0u};
    }
    template <int STR> __device__ __forceinline__ void store(E *dst, int tid) const
    {
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int idx = tid + it * NT;
            const int r = idx / kCpr, c = (idx % kCpr) * kVec;
            *reinterpret_cast<u32x4 *>(dst + r * STR + c) = v[it];
        }
    }
};

// Four floats rounded to the element type and stored contiguously (8-byte
// aligned for bf16, 16-byte aligned for fp32).
__device__ __forceinline__ void store4(bf16 *dst, const float *v)
{
    *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
__device__ __forceinline__ void store4(float *dst, const float *v)
{
    *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}

// Accumulator registers 8*kk .. 8*kk+7 as a B-operand fragment.
template <typename E> __device__ __forceinline__ typename Frag<E>::type pack8(const float *v)
{
    typename Frag<E>::type r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (E)v[t];
    return r;
}

// Value of `x` held by the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Output rows through LDS.  A wave's 32 x D result block arrives as
// 4-column pieces, lane (row r32, half h) holding columns 32 mb + 8 g + 4 h;
// stored to memory directly, each instruction writes 16 bytes of 32
// different rows and the lines stay partly written until the last piece
// lands (the cache then writes some of them back more than once).  put()
// places the pieces in an LDS block (chunk c of row r at chunk
// c ^ (r % chunks per row), so the 32 rows of a piece spread over the LDS
// banks); after a barrier drain() reads 16-byte chunks and stores whole rows,
// consecutive lanes on consecutive addresses.  The stores are non-temporal
// unless KEEP is set (for data the next kernel reads at once): results kept
// in the XCD's L2 evicted the operand rows the other workgroups there still
// read (dK/dV at B8 H12 T1024 d64 37.0 -> 35.4 us, forward 20.9 -> 19.9 us;
// the product X W1^T with M 8192, N 3072, K 768 read 67 MiB into the L2s,
// 48 with these stores).
template <typename E, int D> struct RowStage {
    static constexpr int VEC = 16 / (int)sizeof(E);  // elements per 16-byte chunk
    static constexpr int CPR = D / VEC;              // chunks per row
    static constexpr int ELEMS = 32 * D;             // LDS elements of one block
    static __device__ __forceinline__ int at(int row, int col)
    {
        return row * D + VEC * ((col / VEC) ^ (row % CPR)) + col % VEC;
    }
    static __device__ __forceinline__ void put(E *blk, int r32, int col, const float *v4)
    {
        store4(blk + at(r32, col), v4);
    }
    // rows row0 .. row0 + 31 of dst (row stride st elements), those below
    // nrows, columns below ncols (a multiple of the chunk width)
    template <bool KEEP = false>
    static __device__ __forceinline__ void drain(const E *blk, E *__restrict__ dst, int st, int row0, int nrows,
                                                 int lane, int ncols = D)
    {
#pragma unroll
        for (int it = 0; it < 32 * CPR / 64; ++it) {
            const int idx = 64 * it + lane;
            const int row = idx / CPR, col = VEC * (idx % CPR);
            if (row0 + row < nrows && col < ncols) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(blk + at(row, col));
                u32x4 *to = reinterpret_cast<u32x4 *>(dst + (size_t)(row0 + row) * st + col);
                if constexpr (KEEP)
                    *to = x;
                else
                    __builtin_nontemporal_store(x, to);
            }
        }
    }
};

// Cooperative copy of rows [row0, row0 + R) of a [T, D] slab into an LDS tile
// (row stride STR); rows at or beyond T are filled with zeros.  NT threads.
template <typename E, int D, int R, int STR, int NT>
__device__ __forceinline__ void stage_tile(E *__restrict__ dst, const E *__restrict__ src, int row0, int T, int tid)
{
    constexpr int kVec = 16 / (int)sizeof(E);   // elements per 16-byte chunk
    constexpr int kCpr = D / kVec;              // chunks per row
    constexpr int kChunks = R * kCpr;
    static_assert(kChunks % NT == 0 || kChunks < NT, "tile chunk count must tile the block");
#pragma unroll
    for (int it = 0; it < (kChunks + NT - 1) / NT; ++it) {
        const int idx = tid + it * NT;
        if (kChunks % NT != 0 && idx >= kChunks) break;
        const int r = idx / kCpr, c = (idx % kCpr) * kVec;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row0 + r < T) v = *reinterpret_cast<const u32x4 *>(src + (size_t)(row0 + r) * D + c);
        *reinterpret_cast<u32x4 *>(dst + r * STR + c) = v;
    }
}

}  // namespace attn
