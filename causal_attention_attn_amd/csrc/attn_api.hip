// attn_api.hip -- the C ABI declared in include/attn.h: host-side argument
// validation (before any HIP call), dispatch to the kernel launchers, and the
// optional event-pair kernel timing.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <utility>
#include <mutex>
#include <vector>

#include "attn.h"
#include "attn_launch.h"
#include "gemm.h"

namespace {

thread_local char g_err[512];

attn_status fail(attn_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

attn_status check_shape(attn_dtype dt, int B, int H, int T, int head_dim, size_t *elems, size_t *rows)
{
    if (dt != ATTN_F32 && dt != ATTN_BF16) return fail(ATTN_EUNSUPPORTED, "unknown dtype %d", (int)dt);
    if (B < 1 || H < 1 || T < 1) return fail(ATTN_EINVAL, "B, H and T must be >= 1 (got %d, %d, %d)", B, H, T);
    if (head_dim != 32 && head_dim != 64 && head_dim != 128)
        return fail(ATTN_EUNSUPPORTED, "head_dim %d not supported (32, 64 or 128)", head_dim);
    // element count and byte size must fit int64; grid and row indices must fit int32
    const unsigned __int128 n = (unsigned __int128)B * H * T * head_dim;
    if (n * 4 > (unsigned __int128)INT64_MAX) return fail(ATTN_EINVAL, "tensor size overflows int64");
    const long long bh = (long long)B * H;
    if (bh * T > INT32_MAX) return fail(ATTN_EINVAL, "B*H*T = %lld exceeds 2^31-1", bh * T);
    *elems = (size_t)n;
    *rows = (size_t)(bh * T);
    return ATTN_OK;
}

// One pointer argument as the host validates it.  A view is a [B, H, T, d]
// tensor of the call's element type with element strides s (batch, head,
// token; the d index has stride 1); anything else is a plain byte range.
struct Arg {
    const char *name;
    uintptr_t p;
    size_t bytes;    // from p to one past the last byte the call may touch
    bool view;
    long long s[3];  // view only; 0 for dimensions of extent 1
};

struct Shape {
    int B, H, T, d;
    size_t eb;  // element bytes
};

// A dimension of an index map: stride (in elements) and extent.
struct Dim {
    long long stride, n;
};

// Whether distinct index tuples always reach distinct elements.  Sufficient
// test: ordered by stride, every stride exceeds the largest offset that the
// dimensions below it reach together (mixed-radix digits then read back
// uniquely).  Dimensions of extent 1 do not count.
bool injective(Dim *dims, int k)
{
    int m = 0;
    for (int i = 0; i < k; ++i)
        if (dims[i].n > 1) dims[m++] = dims[i];
    for (int i = 1; i < m; ++i)  // insertion sort by stride
        for (int j = i; j > 0 && dims[j].stride < dims[j - 1].stride; --j) std::swap(dims[j], dims[j - 1]);
    __int128 reach = 0;
    for (int i = 0; i < m; ++i) {
        if ((__int128)dims[i].stride <= reach) return false;
        reach += (__int128)dims[i].stride * (dims[i].n - 1);
    }
    return true;
}

void view_dims(const Arg &a, const Shape &sh, Dim *out)
{
    out[0] = Dim{1, sh.d};
    out[1] = Dim{a.s[0], sh.B};
    out[2] = Dim{a.s[1], sh.H};
    out[3] = Dim{a.s[2], sh.T};
}

// Validates a view's strides and extent and fills a.bytes; strides of
// dimensions of extent 1 are set to 0 (they only ever multiply index 0).
attn_status make_view(Arg &a, const Shape &sh, const long long *s)
{
    a.view = true;
    const int ext[3] = {sh.B, sh.H, sh.T};
    __int128 last = sh.d - 1;
    for (int i = 0; i < 3; ++i) {
        a.s[i] = ext[i] > 1 ? s[i] : 0;
        if (a.s[i] < 0) return fail(ATTN_EINVAL, "%s has a negative stride (%lld)", a.name, a.s[i]);
        if (((__int128)a.s[i] * sh.eb) % 16)
            return fail(ATTN_EINVAL, "%s stride %lld is not a multiple of 16 bytes", a.name, a.s[i]);
        last += (__int128)a.s[i] * (ext[i] - 1);
    }
    const __int128 bytes = (last + 1) * (__int128)sh.eb;
    if (bytes > (__int128)INT64_MAX || (__int128)a.p + bytes > (__int128)UINTPTR_MAX)
        return fail(ATTN_EINVAL, "%s extent overflows the address space", a.name);
    // the kernels address rows inside one (b, h) slab with 32-bit offsets,
    // including up to 255 rows of tile overhang past T
    if ((__int128)(sh.T + 255) * a.s[2] + sh.d > (__int128)INT32_MAX)
        return fail(ATTN_EUNSUPPORTED, "%s: (T + 255) * token stride + head_dim exceeds 2^31-1 elements", a.name);
    a.bytes = (size_t)bytes;
    return ATTN_OK;
}

Arg range(const char *name, const void *p, size_t bytes) { return Arg{name, (uintptr_t)p, bytes, false, {0, 0, 0}}; }

// Whether output a may share an element with b.  Disjoint byte ranges never
// do.  Two views with the same strides whose bases differ by delta elements
// are disjoint when the view extended by a dimension {delta, 2} is still
// injective (interleaved slices such as the q, k and v parts of a packed
// [B, T, 3, H, d] buffer).  Anything else that overlaps in bytes is refused.
bool may_overlap(const Arg &a, const Arg &b, const Shape &sh)
{
    if (!(a.p < b.p + b.bytes && b.p < a.p + a.bytes)) return false;
    if (!a.view || !b.view || a.s[0] != b.s[0] || a.s[1] != b.s[1] || a.s[2] != b.s[2]) return true;
    const uintptr_t delta = a.p > b.p ? a.p - b.p : b.p - a.p;
    if (delta == 0 || delta % sh.eb) return true;
    Dim dims[5];
    view_dims(a, sh, dims);
    dims[4] = Dim{(long long)(delta / sh.eb), 2};
    return !injective(dims, 5);
}

attn_status check_args(const Arg *in, int nin, const Arg *out, int nout, const Shape &sh)
{
    for (int i = 0; i < nin + nout; ++i) {
        const Arg &r = i < nin ? in[i] : out[i - nin];
        if (r.p == 0) return fail(ATTN_EINVAL, "%s is null", r.name);
        if (r.p % 16) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", r.name);
    }
    for (int i = 0; i < nout; ++i) {
        if (out[i].view) {
            Dim dims[4];
            view_dims(out[i], sh, dims);
            if (!injective(dims, 4))
                return fail(ATTN_EINVAL, "output %s: its strides map several elements to one address", out[i].name);
        }
        for (int j = 0; j < nin; ++j)
            if (may_overlap(out[i], in[j], sh))
                return fail(ATTN_EINVAL, "output %s overlaps input %s", out[i].name, in[j].name);
        for (int j = i + 1; j < nout; ++j)
            if (may_overlap(out[i], out[j], sh))
                return fail(ATTN_EINVAL, "output %s overlaps output %s", out[i].name, out[j].name);
    }
    return ATTN_OK;
}

// Views of n tensors from caller strides (3 per tensor, in argument order),
// or contiguous [B, H, T, d] ones when s is null.
attn_status make_views(Arg *a, const char *const *names, const void *const *ptrs, int n, const long long *s,
                       const Shape &sh)
{
    const long long cs[3] = {(long long)sh.H * sh.T * sh.d, (long long)sh.T * sh.d, sh.d};
    for (int i = 0; i < n; ++i) {
        a[i] = Arg{names[i], (uintptr_t)ptrs[i], 0, true, {0, 0, 0}};
        const attn_status st = make_view(a[i], sh, s ? s + 3 * i : cs);
        if (st != ATTN_OK) return st;
    }
    return ATTN_OK;
}

attn::View kview(const Arg &a) { return attn::View{a.s[0], a.s[1], (int)a.s[2]}; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

attn_status device_ready()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ELAUNCH, "no HIP device: %s", hipGetErrorString(e));
    return ATTN_OK;
}

// ------------------------------------------------- static scratch (no-alloc)
// D of attn_bwd_noalloc lives in this array instead of a caller workspace.
// Each GPU holds its own copy until the process ends.  In host code `scratch`
// is only a stand-in for the symbol: its device address on the current device
// comes from hipGetSymbolAddress (scratch_ptr below) and is what kernels get.
constexpr size_t kScratchFloats = ATTN_NOALLOC_MAX_ROWS;
static __device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_scratch_mu;
std::atomic<float *> g_scratch_ptr[64];

// Device address of `scratch` on the current device, resolved once per device
// (attn_init does it; otherwise the first attn_bwd_noalloc call there).
attn_status scratch_ptr(float **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ELAUNCH, "no HIP device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(ATTN_ELAUNCH, "device index %d beyond the 64 the library tracks", dev);
    float *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *q = nullptr;
            e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !q)
                return fail(ATTN_ELAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                            hipGetErrorString(e));
            p = static_cast<float *>(q);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return ATTN_OK;
}

// ---------------------------------------------------------------- timing hooks
struct Prof {
    std::mutex mu;
    std::vector<hipEvent_t> ev;  // 2 per slot
    std::vector<const char *> name;
    int used = 0;
    std::atomic<int> cap{0};  // written under mu; read without it by current_hook
};
Prof g_prof;

bool prof_acquire(hipEvent_t *e0, hipEvent_t *e1, const char *n)
{
    std::lock_guard<std::mutex> g(g_prof.mu);
    if (g_prof.used >= g_prof.cap.load(std::memory_order_relaxed)) return false;
    *e0 = g_prof.ev[2 * g_prof.used];
    *e1 = g_prof.ev[2 * g_prof.used + 1];
    g_prof.name[g_prof.used] = n;
    ++g_prof.used;
    return true;
}

// Compute units of each device, read once.
std::atomic<int> g_cus[64];

attn::KernelHook current_hook()
{
    attn::KernelHook h;
    if (g_prof.cap.load(std::memory_order_relaxed) > 0) h.acquire = prof_acquire;
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        int n = g_cus[dev].load(std::memory_order_relaxed);
        if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            g_cus[dev].store(n, std::memory_order_relaxed);
        h.cus = n > 0 ? n : 0;
    }
    return h;
}

}  // namespace

extern "C" {

const char *attn_status_str(attn_status s)
{
    switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_EINVAL: return "ATTN_EINVAL";
    case ATTN_EUNSUPPORTED: return "ATTN_EUNSUPPORTED";
    case ATTN_ELAUNCH: return "ATTN_ELAUNCH";
    }
    return "unknown";
}

const char *attn_last_error(void) { return g_err; }

attn_status attn_init(void)
{
    g_err[0] = 0;
    attn_status st = device_ready();
    if (st != ATTN_OK) return st;
    // A dry pass through every launcher (nothing is launched, the pointers
    // are never used) runs each kernel variant's one-time occupancy query;
    // current_hook() reads the compute-unit count.
    attn::KernelHook h = current_hook();
    if (h.cus <= 0) return fail(ATTN_ELAUNCH, "cannot read the compute-unit count of the current device");
    h.acquire = nullptr;
    h.dry = true;
    void *const p = reinterpret_cast<void *>(uintptr_t(1) << 40);
    float *const f = reinterpret_cast<float *>(p);
    attn::Layout lay{};
    lay.H = 1;
    // T >= 2048 selects the long-sequence dQ kernel; T = 1024 over many heads
    // the three-wave dK/dV kernel (chosen by grid size at d = 64)
    const struct {
        int bh, T;
    } shapes[] = {{1, 64}, {1, 4096}, {4 * h.cus, 1024}};
    for (int dt = 0; dt < 2; ++dt)
        for (int d : {32, 64, 128})
            for (const auto &sh : shapes) {
                attn::launch_fwd(dt, d, p, p, p, p, f, lay, sh.bh, sh.T, 1.f, 1, nullptr, h);
                attn::launch_bwd(dt, d, p, p, p, p, p, f, p, p, p, f, nullptr, lay, sh.bh, sh.T, 1.f, 1, nullptr, h);
                if (attn::bwd_atomic_supported(dt, d))
                    attn::launch_bwd(dt, d, p, p, p, p, p, f, p, p, p, f, f, lay, sh.bh, sh.T, 1.f, 1, nullptr, h);
            }
    attn::gemm_resident_slots();
    float *sp = nullptr;
    return scratch_ptr(&sp);
}

static attn_status fwd_common(const char *name, attn_dtype dt, const void *Q, const void *K, const void *V, void *O,
                              float *LSE, const long long *strides, int B, int H, int T, int head_dim, float scale,
                              int causal, hipStream_t stream)
{
    g_err[0] = 0;
    size_t n = 0, rows = 0;
    attn_status st = check_shape(dt, B, H, T, head_dim, &n, &rows);
    if (st != ATTN_OK) return st;
    if (!isfinite(scale)) return fail(ATTN_EINVAL, "scale must be finite");
    const Shape sh{B, H, T, head_dim, (size_t)(dt == ATTN_BF16 ? 2 : 4)};
    static const char *const names[4] = {"Q", "K", "V", "O"};
    const void *const ptrs[4] = {Q, K, V, O};
    Arg v[4];
    st = make_views(v, names, ptrs, 4, strides, sh);
    if (st != ATTN_OK) return st;
    const Arg out[2] = {v[3], range("LSE", LSE, rows * 4)};
    st = check_args(v, 3, out, 2, sh);
    if (st != ATTN_OK) return st;
    st = device_ready();
    if (st != ATTN_OK) return st;
    attn::Layout lay{};
    lay.q = kview(v[0]);
    lay.k = kview(v[1]);
    lay.v = kview(v[2]);
    lay.o = kview(v[3]);
    lay.H = H;
    const hipError_t e = attn::launch_fwd((int)dt, head_dim, Q, K, V, O, LSE, lay, B * H, T, scale, causal ? 1 : 0,
                                          stream, current_hook());
    if (e != hipSuccess) return fail(ATTN_ELAUNCH, "%s launch failed: %s", name, hipGetErrorString(e));
    return ATTN_OK;
}

attn_status attn_fwd(attn_dtype dt, const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H,
                     int T, int head_dim, float scale, int causal, hipStream_t stream)
{
    return fwd_common("attn_fwd", dt, Q, K, V, O, LSE, nullptr, B, H, T, head_dim, scale, causal, stream);
}

attn_status attn_fwd_strided(attn_dtype dt, const void *Q, const void *K, const void *V, void *O, float *LSE,
                             const long long *strides, int B, int H, int T, int head_dim, float scale, int causal,
                             hipStream_t stream)
{
    g_err[0] = 0;
    if (!strides) return fail(ATTN_EINVAL, "strides is null");
    return fwd_common("attn_fwd_strided", dt, Q, K, V, O, LSE, strides, B, H, T, head_dim, scale, causal, stream);
}

size_t attn_bwd_workspace_bytes(attn_dtype dt, int B, int H, int T, int head_dim, int causal)
{
    (void)causal;
    g_err[0] = 0;
    size_t n = 0, rows = 0;
    if (check_shape(dt, B, H, T, head_dim, &n, &rows) != ATTN_OK) return 0;
    return round_up(rows * sizeof(float), 256);  // D = rowsum(dO o O)
}

size_t attn_bwd_atomic_workspace_bytes(attn_dtype dt, int B, int H, int T, int head_dim, int causal)
{
    (void)causal;
    g_err[0] = 0;
    size_t n = 0, rows = 0;
    if (check_shape(dt, B, H, T, head_dim, &n, &rows) != ATTN_OK) return 0;
    if (!attn::bwd_atomic_supported((int)dt, head_dim)) {
        fail(ATTN_EUNSUPPORTED, "the atomic dQ path is bf16 only");
        return 0;
    }
    return round_up(rows * sizeof(float), 256) + n * sizeof(float);  // D, then the fp32 dQ accumulator
}

static attn_status bwd_common(const char *name, bool deterministic, attn_dtype dt, const void *Q, const void *K,
                              const void *V, const void *O, const void *dO, const float *LSE, void *dQ, void *dK,
                              void *dV, void *workspace, size_t workspace_bytes, const long long *strides, int B,
                              int H, int T, int head_dim, float scale, int causal, hipStream_t stream)
{
    g_err[0] = 0;
    size_t n = 0, rows = 0;
    attn_status st = check_shape(dt, B, H, T, head_dim, &n, &rows);
    if (st != ATTN_OK) return st;
    if (!isfinite(scale)) return fail(ATTN_EINVAL, "scale must be finite");
    const bool atomic = !deterministic;
    if (atomic && !attn::bwd_atomic_supported((int)dt, head_dim))
        return fail(ATTN_EUNSUPPORTED, "the atomic dQ path is bf16 only");
    const size_t dbytes = round_up(rows * sizeof(float), 256);
    const size_t need = dbytes + (atomic ? n * sizeof(float) : 0);
    if (workspace_bytes < need)
        return fail(ATTN_EINVAL, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    const Shape sh{B, H, T, head_dim, (size_t)(dt == ATTN_BF16 ? 2 : 4)};
    static const char *const names[8] = {"Q", "K", "V", "O", "dO", "dQ", "dK", "dV"};
    const void *const ptrs[8] = {Q, K, V, O, dO, dQ, dK, dV};
    Arg v[8];
    st = make_views(v, names, ptrs, 8, strides, sh);
    if (st != ATTN_OK) return st;
    const Arg in[6] = {v[0], v[1], v[2], v[3], v[4], range("LSE", LSE, rows * 4)};
    const Arg out[4] = {v[5], v[6], v[7], range("workspace", workspace, need)};
    st = check_args(in, 6, out, 4, sh);
    if (st != ATTN_OK) return st;
    st = device_ready();
    if (st != ATTN_OK) return st;
    attn::Layout lay{};
    lay.q = kview(v[0]);
    lay.k = kview(v[1]);
    lay.v = kview(v[2]);
    lay.o = kview(v[3]);
    lay.dO = kview(v[4]);
    lay.dq = kview(v[5]);
    lay.dk = kview(v[6]);
    lay.dv = kview(v[7]);
    lay.H = H;
    float *Dbuf = (float *)workspace;
    float *dQacc = atomic ? (float *)((char *)workspace + dbytes) : nullptr;
    const hipError_t e = attn::launch_bwd((int)dt, head_dim, Q, K, V, O, dO, LSE, dQ, dK, dV, Dbuf, dQacc, lay,
                                          B * H, T, scale, causal ? 1 : 0, stream, current_hook());
    if (e != hipSuccess) return fail(ATTN_ELAUNCH, "%s launch failed: %s", name, hipGetErrorString(e));
    return ATTN_OK;
}

attn_status attn_bwd(attn_dtype dt, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                     const float *LSE, void *dQ, void *dK, void *dV, void *workspace, size_t workspace_bytes, int B,
                     int H, int T, int head_dim, float scale, int causal, hipStream_t stream)
{
    return bwd_common("attn_bwd", true, dt, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, nullptr, B,
                      H, T, head_dim, scale, causal, stream);
}

attn_status attn_bwd_strided(attn_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                             const void *dO, const float *LSE, void *dQ, void *dK, void *dV, void *workspace,
                             size_t workspace_bytes, const long long *strides, int B, int H, int T, int head_dim,
                             float scale, int causal, hipStream_t stream)
{
    g_err[0] = 0;
    if (!strides) return fail(ATTN_EINVAL, "strides is null");
    return bwd_common("attn_bwd_strided", true, dt, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes,
                      strides, B, H, T, head_dim, scale, causal, stream);
}

attn_status attn_bwd_noalloc(attn_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                             const void *dO, const float *LSE, void *dQ, void *dK, void *dV, int B, int H, int T,
                             int head_dim, float scale, int causal, hipStream_t stream)
{
    g_err[0] = 0;
    size_t n = 0, rows = 0;
    attn_status st = check_shape(dt, B, H, T, head_dim, &n, &rows);
    if (st != ATTN_OK) return st;
    if (rows > kScratchFloats)
        return fail(ATTN_EINVAL, "attn_bwd_noalloc: B*H*T = %zu rows exceed the static scratch of %zu rows", rows,
                    kScratchFloats);
    st = device_ready();
    if (st != ATTN_OK) return st;
    float *sp = nullptr;
    st = scratch_ptr(&sp);
    if (st != ATTN_OK) return st;
    return bwd_common("attn_bwd_noalloc", true, dt, Q, K, V, O, dO, LSE, dQ, dK, dV, sp, kScratchFloats * sizeof(float),
                      nullptr, B, H, T, head_dim, scale, causal, stream);
}

attn_status attn_bwd_atomic(attn_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                            const void *dO, const float *LSE, void *dQ, void *dK, void *dV, void *workspace,
                            size_t workspace_bytes, int B, int H, int T, int head_dim, float scale, int causal,
                            hipStream_t stream)
{
    return bwd_common("attn_bwd_atomic", false, dt, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes,
                      nullptr, B, H, T, head_dim, scale, causal, stream);
}

attn_status attn_bwd_atomic_strided(attn_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                                    const void *dO, const float *LSE, void *dQ, void *dK, void *dV, void *workspace,
                                    size_t workspace_bytes, const long long *strides, int B, int H, int T,
                                    int head_dim, float scale, int causal, hipStream_t stream)
{
    g_err[0] = 0;
    if (!strides) return fail(ATTN_EINVAL, "strides is null");
    return bwd_common("attn_bwd_atomic_strided", false, dt, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace,
                      workspace_bytes, strides, B, H, T, head_dim, scale, causal, stream);
}

// ---------------------------------------------------------------- layer GEMMs
namespace {

struct GemmPlan {
    bool a_kmajor, b_kmajor;
    int kchunk;        // contraction chunk (a multiple of 64)
    int splits;        // chunks, each non-empty
    size_t ws_bytes;   // fp32 partial products (0 when not split)
};

attn_status gemm_plan(gemm_op op, int M, int N, int K, int split_k, GemmPlan *p)
{
    if (op != GEMM_NT && op != GEMM_NN && op != GEMM_TN) return fail(ATTN_EUNSUPPORTED, "unknown gemm_op %d", (int)op);
    if (M < 1 || N < 1 || K < 1) return fail(ATTN_EINVAL, "M, N and K must be >= 1 (got %d, %d, %d)", M, N, K);
    if (K % 64) return fail(ATTN_EUNSUPPORTED, "K = %d is not a multiple of 64", K);
    if (N % 8) return fail(ATTN_EUNSUPPORTED, "N = %d is not a multiple of 8", N);
    if (op == GEMM_TN && M % 8) return fail(ATTN_EUNSUPPORTED, "M = %d is not a multiple of 8 (GEMM_TN)", M);
    if (split_k < 0 || split_k > K / 64)
        return fail(ATTN_EINVAL, "split_k = %d outside 0..%d (K/64)", split_k, K / 64);
    const long long tiles = (long long)((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > INT32_MAX) return fail(ATTN_EINVAL, "too many output tiles");
    p->a_kmajor = op != GEMM_TN;
    p->b_kmajor = op == GEMM_NT;
    const int s = split_k ? split_k : attn::gemm_auto_splits(M, N, K);
    p->kchunk = attn::gemm_split_chunk(K, s);
    p->splits = (K + p->kchunk - 1) / p->kchunk;
    const unsigned __int128 ws = p->splits > 1 ? (unsigned __int128)p->splits * M * N * 4 : 0;
    if (ws > (unsigned __int128)INT64_MAX) return fail(ATTN_EINVAL, "workspace size overflows int64");
    p->ws_bytes = round_up((size_t)ws, 256);
    return ATTN_OK;
}

// bytes spanned by a row-major [rows x cols] matrix with leading dimension ld
attn_status matrix_span(const char *name, int rows, int cols, int ld, size_t eb, size_t *bytes)
{
    if (ld < cols) return fail(ATTN_EINVAL, "%s: leading dimension %d < row length %d", name, ld, cols);
    if (ld % 8) return fail(ATTN_EINVAL, "%s: leading dimension %d is not a multiple of 8", name, ld);
    // the kernels address up to 256 rows of a matrix from one 32-bit byte offset
    if (ld >= (1 << 23)) return fail(ATTN_EINVAL, "%s: leading dimension %d is not below 2^23", name, ld);
    const unsigned __int128 b = ((unsigned __int128)(rows - 1) * ld + cols) * eb;
    if (b > (unsigned __int128)INT64_MAX) return fail(ATTN_EINVAL, "%s: extent overflows int64", name);
    *bytes = (size_t)b;
    return ATTN_OK;
}

}  // namespace

size_t gemm_workspace_bytes(gemm_op op, int M, int N, int K, int split_k)
{
    g_err[0] = 0;
    GemmPlan p;
    if (gemm_plan(op, M, N, K, split_k, &p) != ATTN_OK) return 0;
    return p.ws_bytes;
}

attn_status gemm_bf16(gemm_op op, const void *A, int lda, const void *B, int ldb, void *C, int ldc, attn_dtype c_type,
                      int M, int N, int K, int split_k, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    g_err[0] = 0;
    GemmPlan p;
    attn_status st = gemm_plan(op, M, N, K, split_k, &p);
    if (st != ATTN_OK) return st;
    if (c_type != ATTN_BF16 && c_type != ATTN_F32) return fail(ATTN_EUNSUPPORTED, "unknown output dtype %d", (int)c_type);
    if (workspace_bytes < p.ws_bytes)
        return fail(ATTN_EINVAL, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, p.ws_bytes);
    size_t ba = 0, bb = 0, bc = 0;
    st = p.a_kmajor ? matrix_span("A", M, K, lda, 2, &ba) : matrix_span("A", K, M, lda, 2, &ba);
    if (st != ATTN_OK) return st;
    st = p.b_kmajor ? matrix_span("B", N, K, ldb, 2, &bb) : matrix_span("B", K, N, ldb, 2, &bb);
    if (st != ATTN_OK) return st;
    st = matrix_span("C", M, N, ldc, c_type == ATTN_F32 ? 4 : 2, &bc);
    if (st != ATTN_OK) return st;
    const Shape none{1, 1, 1, 1, 1};  // only byte ranges below
    const Arg in[2] = {range("A", A, ba), range("B", B, bb)};
    if (p.ws_bytes) {
        const Arg out[2] = {range("C", C, bc), range("workspace", workspace, p.ws_bytes)};
        st = check_args(in, 2, out, 2, none);
    } else {
        const Arg out[1] = {range("C", C, bc)};
        st = check_args(in, 2, out, 1, none);
    }
    if (st != ATTN_OK) return st;
    st = device_ready();
    if (st != ATTN_OK) return st;
    const hipError_t e = attn::launch_gemm((int)op, c_type == ATTN_F32, A, B, C, (float *)workspace, M, N, K, lda, ldb,
                                           ldc, p.kchunk, stream, current_hook());
    if (e != hipSuccess) return fail(ATTN_ELAUNCH, "gemm_bf16 launch failed: %s", hipGetErrorString(e));
    return ATTN_OK;
}

attn_status attn_prof_enable(int capacity)
{
    g_err[0] = 0;
    std::lock_guard<std::mutex> g(g_prof.mu);
    for (hipEvent_t e : g_prof.ev) hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.name.clear();
    g_prof.used = 0;
    g_prof.cap.store(0, std::memory_order_relaxed);
    if (capacity <= 0) return ATTN_OK;
    g_prof.ev.resize(2 * (size_t)capacity);
    for (size_t i = 0; i < g_prof.ev.size(); ++i) {
        hipError_t e = hipEventCreate(&g_prof.ev[i]);
        if (e != hipSuccess) {
            for (size_t j = 0; j < i; ++j) hipEventDestroy(g_prof.ev[j]);
            g_prof.ev.clear();
            return fail(ATTN_ELAUNCH, "hipEventCreate failed: %s", hipGetErrorString(e));
        }
    }
    g_prof.name.assign((size_t)capacity, nullptr);
    g_prof.cap.store(capacity, std::memory_order_relaxed);
    return ATTN_OK;
}

int attn_prof_read(attn_kernel_time *out, int max)
{
    std::lock_guard<std::mutex> g(g_prof.mu);
    std::vector<attn_kernel_time> acc;
    for (int i = 0; i < g_prof.used; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess) return -1;
        if (hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) return -1;
        size_t k = 0;
        while (k < acc.size() && strcmp(acc[k].kernel, g_prof.name[i]) != 0) ++k;
        if (k == acc.size()) acc.push_back(attn_kernel_time{g_prof.name[i], 0, 0.0});
        acc[k].launches += 1;
        acc[k].total_ms += ms;
    }
    g_prof.used = 0;
    const int n = (int)acc.size();
    for (int i = 0; i < n && i < max; ++i) out[i] = acc[i];
    return n;
}

}  // extern "C"
