// attn_api.hip -- the C ABI declared in include/attn.h: host-side argument
// validation (before any HIP call), dispatch to the kernel launchers, and the
// optional event-pair kernel timing.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "attn.h"
#include "attn_launch.h"

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

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi; }

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

attn_status check_ptrs(const Range *in, int nin, const Range *out, int nout)
{
    for (int i = 0; i < nin + nout; ++i) {
        const Range &r = i < nin ? in[i] : out[i - nin];
        if (r.lo == 0) return fail(ATTN_EINVAL, "%s is null", r.name);
        if (r.lo % 16) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", r.name);
    }
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(out[i], in[j])) return fail(ATTN_EINVAL, "output %s overlaps input %s", out[i].name, in[j].name);
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j]))
                return fail(ATTN_EINVAL, "output %s overlaps output %s", out[i].name, out[j].name);
    }
    return ATTN_OK;
}

Range rng(const char *name, const void *p, size_t bytes) { return Range{name, (uintptr_t)p, (uintptr_t)p + bytes}; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

attn_status device_ready()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ELAUNCH, "no HIP device: %s", hipGetErrorString(e));
    return ATTN_OK;
}

// ---------------------------------------------------------------- timing hooks
struct Prof {
    std::mutex mu;
    std::vector<hipEvent_t> ev;  // 2 per slot
    std::vector<const char *> name;
    int used = 0;
    int cap = 0;
};
Prof g_prof;

bool prof_acquire(hipEvent_t *e0, hipEvent_t *e1, const char *n)
{
    std::lock_guard<std::mutex> g(g_prof.mu);
    if (g_prof.used >= g_prof.cap) return false;
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
    if (g_prof.cap > 0) h.acquire = prof_acquire;
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

attn_status attn_fwd(attn_dtype dt, const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H,
                     int T, int head_dim, float scale, int causal, hipStream_t stream)
{
    g_err[0] = 0;
    size_t n = 0, rows = 0;
    attn_status st = check_shape(dt, B, H, T, head_dim, &n, &rows);
    if (st != ATTN_OK) return st;
    if (!isfinite(scale)) return fail(ATTN_EINVAL, "scale must be finite");
    const size_t eb = dt == ATTN_BF16 ? 2 : 4;
    const Range in[3] = {rng("Q", Q, n * eb), rng("K", K, n * eb), rng("V", V, n * eb)};
    const Range out[2] = {rng("O", O, n * eb), rng("LSE", LSE, rows * 4)};
    st = check_ptrs(in, 3, out, 2);
    if (st != ATTN_OK) return st;
    st = device_ready();
    if (st != ATTN_OK) return st;
    const hipError_t e = attn::launch_fwd((int)dt, head_dim, Q, K, V, O, LSE, B * H, T, scale, causal ? 1 : 0,
                                          stream, current_hook());
    if (e != hipSuccess) return fail(ATTN_ELAUNCH, "attn_fwd launch failed: %s", hipGetErrorString(e));
    return ATTN_OK;
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
                              void *dV, void *workspace, size_t workspace_bytes, int B, int H, int T, int head_dim,
                              float scale, int causal, hipStream_t stream)
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
    const size_t eb = dt == ATTN_BF16 ? 2 : 4;
    const Range in[6] = {rng("Q", Q, n * eb), rng("K", K, n * eb), rng("V", V, n * eb),
                         rng("O", O, n * eb), rng("dO", dO, n * eb), rng("LSE", LSE, rows * 4)};
    const Range out[4] = {rng("dQ", dQ, n * eb), rng("dK", dK, n * eb), rng("dV", dV, n * eb),
                          rng("workspace", workspace, need)};
    st = check_ptrs(in, 6, out, 4);
    if (st != ATTN_OK) return st;
    st = device_ready();
    if (st != ATTN_OK) return st;
    float *Dbuf = (float *)workspace;
    float *dQacc = atomic ? (float *)((char *)workspace + dbytes) : nullptr;
    const hipError_t e = attn::launch_bwd((int)dt, head_dim, Q, K, V, O, dO, LSE, dQ, dK, dV, Dbuf, dQacc, B * H, T,
                                          scale, causal ? 1 : 0, stream, current_hook());
    if (e != hipSuccess) return fail(ATTN_ELAUNCH, "%s launch failed: %s", name, hipGetErrorString(e));
    return ATTN_OK;
}

attn_status attn_bwd(attn_dtype dt, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                     const float *LSE, void *dQ, void *dK, void *dV, void *workspace, size_t workspace_bytes, int B,
                     int H, int T, int head_dim, float scale, int causal, hipStream_t stream)
{
    return bwd_common("attn_bwd", true, dt, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H, T,
                      head_dim, scale, causal, stream);
}

attn_status attn_bwd_atomic(attn_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                            const void *dO, const float *LSE, void *dQ, void *dK, void *dV, void *workspace,
                            size_t workspace_bytes, int B, int H, int T, int head_dim, float scale, int causal,
                            hipStream_t stream)
{
    return bwd_common("attn_bwd_atomic", false, dt, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace,
                      workspace_bytes, B, H, T, head_dim, scale, causal, stream);
}

attn_status attn_prof_enable(int capacity)
{
    g_err[0] = 0;
    std::lock_guard<std::mutex> g(g_prof.mu);
    for (hipEvent_t e : g_prof.ev) hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.name.clear();
    g_prof.used = 0;
    g_prof.cap = 0;
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
    g_prof.cap = capacity;
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
