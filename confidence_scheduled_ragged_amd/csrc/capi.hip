// capi.hip - the exported C ABI: host-side argument checks, then launches on
// the caller's stream. No allocation, no synchronisation, no per-call state.
#include <atomic>
#include <cmath>
#include <mutex>

#include "common.hpp"

#define DSPARK_API extern "C" __attribute__((visibility("default")))

namespace dspark {

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64) {
        int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4 *p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

__global__ void step_status_kernel(unsigned *flag, int32_t *status) {
    if (threadIdx.x == 0)
        *status = (int32_t)__hip_atomic_exchange(flag, 0u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_step_status(void *ws, int32_t *status, hipStream_t s) {
    unsigned *flag = reinterpret_cast<unsigned *>(static_cast<char *>(ws) + ws_ctrl_offset() +
                                                  kCtrlTimedOutOffset);
    hipLaunchKernelGGL(step_status_kernel, dim3(1), dim3(64), 0, s, flag, status);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *ws, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t g = (n16 + 255) / 256;
    g = g > 1024 ? 1024 : g;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)g), dim3(256), 0, s,
                       static_cast<u32x4 *>(ws), n16);
    return hipGetLastError();
}

}  // namespace dspark

using namespace dspark;

namespace {

constexpr int kMaxD = 1 << 20;
constexpr int kMaxTiers = 4096;

inline bool misaligned(const void *p, size_t a) { return p && ((uintptr_t)p % a) != 0; }

inline dspark_status check_bg(int B, int gamma) {
    if (B < 1 || gamma < 1 || gamma > DSPARK_MAX_GAMMA) return DSPARK_ERR_SHAPE;
    if ((int64_t)B * (gamma + 1) > (int64_t)DSPARK_MAX_ROWS) return DSPARK_ERR_SHAPE;
    return DSPARK_OK;
}

inline bool valid_mode(int mode) {
    return mode == DSPARK_CUT_THRESHOLD || mode == DSPARK_CUT_BUDGET ||
           mode == DSPARK_CUT_STATIC || mode == DSPARK_CUT_COMBINED;
}

inline bool needs_cutoff(int mode) {
    return mode == DSPARK_CUT_THRESHOLD || mode == DSPARK_CUT_COMBINED;
}

inline bool needs_budget(int mode) {
    return mode == DSPARK_CUT_BUDGET || mode == DSPARK_CUT_COMBINED;
}

inline dspark_status launched(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP; }

inline hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

DSPARK_API const char *dspark_status_string(int status) {
    switch (status) {
        case DSPARK_OK: return "ok";
        case DSPARK_ERR_NULL: return "a required pointer is NULL";
        case DSPARK_ERR_SHAPE: return "a size is out of range";
        case DSPARK_ERR_ARG: return "an argument value is invalid";
        case DSPARK_ERR_ALIGN: return "a pointer is misaligned for its element type";
        case DSPARK_ERR_WORKSPACE: return "the workspace is too small";
        case DSPARK_ERR_HIP: return "a HIP kernel launch failed";
        default: return "unknown status";
    }
}

DSPARK_API size_t dspark_workspace_bytes(int B, int gamma, int V) {
    if (check_bg(B, gamma) != DSPARK_OK || V < 1) return 0;
    return ws_total_bytes(B, gamma);
}

DSPARK_API dspark_status dspark_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return DSPARK_ERR_NULL;
    if (misaligned(ws, 16)) return DSPARK_ERR_ALIGN;
    return launched(launch_fill_zero(ws, ws_bytes & ~(size_t)15, as_stream(stream)));
}

DSPARK_API dspark_status dspark_confidence(const dspark_bf16 *hidden, const dspark_bf16 *w,
                                           float bias, const float *temps, int B, int gamma, int d,
                                           float *conf, float *survival, void *stream) {
    if (!hidden || !w || !temps || !conf || !survival) return DSPARK_ERR_NULL;
    if (dspark_status st = check_bg(B, gamma)) return st;
    if (d < 1 || d > kMaxD) return DSPARK_ERR_SHAPE;
    if (!std::isfinite(bias)) return DSPARK_ERR_ARG;
    if (misaligned(hidden, 2) || misaligned(w, 2) || misaligned(temps, 4) || misaligned(conf, 4) ||
        misaligned(survival, 4))
        return DSPARK_ERR_ALIGN;
    return launched(launch_confidence(hidden, w, bias, temps, B, gamma, d, conf, survival,
                                      as_stream(stream)));
}

DSPARK_API dspark_status dspark_schedule(const float *survival, int B, int gamma, int mode,
                                         const float *cutoff, long long budget, int32_t *lengths,
                                         void *stream) {
    if (!survival || !lengths) return DSPARK_ERR_NULL;
    if (needs_cutoff(mode) && !cutoff) return DSPARK_ERR_NULL;
    if (dspark_status st = check_bg(B, gamma)) return st;
    if (!valid_mode(mode)) return DSPARK_ERR_ARG;
    if (needs_budget(mode) && budget < 0) return DSPARK_ERR_ARG;
    if (misaligned(survival, 4) || misaligned(cutoff, 4) || misaligned(lengths, 4))
        return DSPARK_ERR_ALIGN;
    return launched(launch_schedule(survival, B, gamma, mode, cutoff, budget, lengths,
                                    as_stream(stream)));
}

DSPARK_API dspark_status dspark_compact(const int32_t *lengths, const int32_t *tokens, int B,
                                        int gamma, int32_t *cu_seqlens, int32_t *packed_tokens,
                                        int32_t *packed_src_row, const dspark_bf16 *logits, int V,
                                        dspark_bf16 *packed_logits, void *stream) {
    if (!lengths || !tokens || !cu_seqlens || !packed_tokens || !packed_src_row)
        return DSPARK_ERR_NULL;
    if ((logits == nullptr) != (packed_logits == nullptr)) return DSPARK_ERR_NULL;
    if (dspark_status st = check_bg(B, gamma)) return st;
    if (logits && V < 1) return DSPARK_ERR_SHAPE;
    if (misaligned(lengths, 4) || misaligned(tokens, 4) || misaligned(cu_seqlens, 4) ||
        misaligned(packed_tokens, 4) || misaligned(packed_src_row, 4) || misaligned(logits, 2) ||
        misaligned(packed_logits, 2))
        return DSPARK_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    hipError_t e = launch_compact(lengths, tokens, B, gamma, cu_seqlens, packed_tokens,
                                  packed_src_row, s);
    if (e == hipSuccess && logits)
        e = launch_gather_rows(logits, packed_src_row, cu_seqlens, B, gamma, (int64_t)V * 2,
                               packed_logits, s);
    return launched(e);
}

DSPARK_API dspark_status dspark_gather_rows(const void *src, const int32_t *packed_src_row,
                                            const int32_t *cu_seqlens, int B, int gamma,
                                            long long row_bytes, void *dst, void *stream) {
    if (!src || !packed_src_row || !cu_seqlens || !dst) return DSPARK_ERR_NULL;
    if (dspark_status st = check_bg(B, gamma)) return st;
    // the source and destination each span B*(gamma+1) rows: keep their byte size
    // within 2^48 so no offset computation can overflow
    if (row_bytes < 1 || row_bytes > ((long long)1 << 48) / ((long long)B * (gamma + 1)))
        return DSPARK_ERR_SHAPE;
    if (misaligned(packed_src_row, 4) || misaligned(cu_seqlens, 4)) return DSPARK_ERR_ALIGN;
    return launched(launch_gather_rows(src, packed_src_row, cu_seqlens, B, gamma,
                                       (int64_t)row_bytes, dst, as_stream(stream)));
}

DSPARK_API dspark_status dspark_tier_select(const int32_t *cu_seqlens, int B, int gamma,
                                            const int32_t *tiers, int ntiers, int32_t pad_token,
                                            int32_t *padded_total, int32_t *tier_index,
                                            int32_t *packed_tokens, int32_t *packed_src_row,
                                            void *stream) {
    if (!cu_seqlens || !tiers || !padded_total || !tier_index) return DSPARK_ERR_NULL;
    if (dspark_status st = check_bg(B, gamma)) return st;
    if (ntiers < 1 || ntiers > kMaxTiers) return DSPARK_ERR_SHAPE;
    if (misaligned(cu_seqlens, 4) || misaligned(tiers, 4) || misaligned(padded_total, 4) ||
        misaligned(tier_index, 4) || misaligned(packed_tokens, 4) || misaligned(packed_src_row, 4))
        return DSPARK_ERR_ALIGN;
    return launched(launch_tier_select(cu_seqlens, B, gamma, tiers, ntiers, pad_token,
                                       padded_total, tier_index, packed_tokens, packed_src_row,
                                       as_stream(stream)));
}

DSPARK_API dspark_status dspark_cost_cutoff(const float *table, int n, const int32_t *load,
                                            int B, float *cutoff, void *stream) {
    if (!table || !load || !cutoff) return DSPARK_ERR_NULL;
    if (n < 1 || B < 1 || B > DSPARK_MAX_ROWS) return DSPARK_ERR_SHAPE;
    if (misaligned(table, 4) || misaligned(load, 4) || misaligned(cutoff, 4))
        return DSPARK_ERR_ALIGN;
    return launched(launch_cost_cutoff(table, n, load, B, cutoff, as_stream(stream)));
}

DSPARK_API dspark_status dspark_accept(const dspark_bf16 *logits, const int32_t *packed_src_row,
                                       const int32_t *cu_seqlens, const int32_t *tokens, int B,
                                       int gamma, int V, int32_t *packed_argmax, int32_t *accepted,
                                       int32_t *bonus, void *ws, size_t ws_bytes, void *stream) {
    if (!logits || !cu_seqlens || !tokens || !packed_argmax || !accepted || !bonus || !ws)
        return DSPARK_ERR_NULL;
    if (dspark_status st = check_bg(B, gamma)) return st;
    if (V < 1) return DSPARK_ERR_SHAPE;
    if (misaligned(logits, 2) || misaligned(packed_src_row, 4) || misaligned(cu_seqlens, 4) ||
        misaligned(tokens, 4) || misaligned(packed_argmax, 4) || misaligned(accepted, 4) ||
        misaligned(bonus, 4) || misaligned(ws, 16))
        return DSPARK_ERR_ALIGN;
    if (ws_bytes < ws_total_bytes(B, gamma)) return DSPARK_ERR_WORKSPACE;
    return launched(launch_accept(logits, packed_src_row, cu_seqlens, tokens, B, gamma, V,
                                  packed_argmax, accepted, bonus, ws, as_stream(stream)));
}

DSPARK_API dspark_status dspark_cap_accept(const int32_t *packed_argmax_full,
                                           const int32_t *tokens, const int32_t *lengths, int B,
                                           int gamma, int32_t *accepted, int32_t *bonus,
                                           int32_t *accepted_full, long long *sums,
                                           void *stream) {
    if (!packed_argmax_full || !tokens || !lengths || !accepted || !bonus || !accepted_full)
        return DSPARK_ERR_NULL;
    if (dspark_status st = check_bg(B, gamma)) return st;
    if (misaligned(packed_argmax_full, 4) || misaligned(tokens, 4) || misaligned(lengths, 4) ||
        misaligned(accepted, 4) || misaligned(bonus, 4) || misaligned(accepted_full, 4) ||
        misaligned(sums, 8))
        return DSPARK_ERR_ALIGN;
    return launched(launch_cap_accept(packed_argmax_full, tokens, lengths, B, gamma, accepted,
                                      bonus, accepted_full, sums, as_stream(stream)));
}

// Host-side checks of the fused step's arguments (every one but the workspace).
static dspark_status step_check(const dspark_bf16 *hidden, const dspark_bf16 *w, float bias,
                                const float *temps, const int32_t *tokens,
                                const dspark_bf16 *logits, int B, int gamma, int d, int V,
                                int mode, const float *cutoff, long long budget, float *conf,
                                float *survival, int32_t *lengths, int32_t *cu_seqlens,
                                int32_t *packed_tokens, int32_t *packed_src_row,
                                int32_t *packed_argmax, int32_t *accepted, int32_t *bonus,
                                int launches) {
    if (!hidden || !w || !temps || !tokens || !logits || !lengths || !cu_seqlens ||
        !packed_tokens || !packed_src_row || !packed_argmax || !accepted || !bonus)
        return DSPARK_ERR_NULL;
    if (needs_cutoff(mode) && !cutoff) return DSPARK_ERR_NULL;
    if (dspark_status st = check_bg(B, gamma)) return st;
    if (d < 1 || d > kMaxD || V < 1) return DSPARK_ERR_SHAPE;
    if (!valid_mode(mode)) return DSPARK_ERR_ARG;
    if (needs_budget(mode) && budget < 0) return DSPARK_ERR_ARG;
    if (!std::isfinite(bias)) return DSPARK_ERR_ARG;
    if (launches < 0 || launches > 2) return DSPARK_ERR_ARG;
    if (misaligned(hidden, 2) || misaligned(w, 2) || misaligned(temps, 4) ||
        misaligned(tokens, 4) || misaligned(logits, 2) || misaligned(cutoff, 4) ||
        misaligned(conf, 4) || misaligned(survival, 4) || misaligned(lengths, 4) ||
        misaligned(cu_seqlens, 4) || misaligned(packed_tokens, 4) ||
        misaligned(packed_src_row, 4) || misaligned(packed_argmax, 4) ||
        misaligned(accepted, 4) || misaligned(bonus, 4))
        return DSPARK_ERR_ALIGN;
    return DSPARK_OK;
}

// The fused step's launches, after every check has passed.
static dspark_status step_launch(const dspark_bf16 *hidden, const dspark_bf16 *w, float bias,
                                 const float *temps, const int32_t *tokens,
                                 const dspark_bf16 *logits, int B, int gamma, int d, int V,
                                 int mode, const float *cutoff, long long budget, float *conf,
                                 float *survival, int32_t *lengths, int32_t *cu_seqlens,
                                 int32_t *packed_tokens, int32_t *packed_src_row,
                                 int32_t *packed_argmax, int32_t *accepted, int32_t *bonus,
                                 void *ws, hipStream_t s, void *ev_start, void *ev_stop,
                                 int launches, unsigned long long wait_ticks) {
    char *wsb = static_cast<char *>(ws);
    float *surv = survival ? survival : reinterpret_cast<float *>(wsb + ws_surv_offset(B, gamma));
    float *cf = conf ? conf : reinterpret_cast<float *>(wsb + ws_conf_offset(B, gamma));
    hipEvent_t es = static_cast<hipEvent_t>(ev_start), et = static_cast<hipEvent_t>(ev_stop);
    auto fused = fused_slots_fit_32(B, gamma, V, logits) ? slots32::launch_fused_step
                                                         : slots64::launch_fused_step;
    hipError_t e = fused(hidden, w, bias, temps, tokens, logits, B, gamma, d, V, mode, cutoff,
                         budget, cf, surv, lengths, cu_seqlens, packed_tokens, packed_src_row,
                         packed_argmax, accepted, bonus, ws, s, es, et, launches, wait_ticks);
    if (e != hipErrorNotSupported) return launched(e);
    // sizes outside the fused kernels' limits: the same step through the stage kernels
    e = launch_confidence(hidden, w, bias, temps, B, gamma, d, cf, surv, s);
    if (e == hipSuccess) e = launch_schedule(surv, B, gamma, mode, cutoff, budget, lengths, s);
    if (e == hipSuccess)
        e = launch_compact(lengths, tokens, B, gamma, cu_seqlens, packed_tokens, packed_src_row, s);
    if (e == hipSuccess && es) e = hipEventRecord(es, s);
    if (e == hipSuccess)
        e = launch_accept(logits, packed_src_row, cu_seqlens, tokens, B, gamma, V, packed_argmax,
                          accepted, bonus, ws, s);
    if (e == hipSuccess && et) e = hipEventRecord(et, s);
    return launched(e);
}

static dspark_status step_impl(const dspark_bf16 *hidden, const dspark_bf16 *w, float bias,
                               const float *temps, const int32_t *tokens,
                               const dspark_bf16 *logits, int B, int gamma, int d, int V,
                               int mode, const float *cutoff, long long budget, float *conf,
                               float *survival, int32_t *lengths, int32_t *cu_seqlens,
                               int32_t *packed_tokens, int32_t *packed_src_row,
                               int32_t *packed_argmax, int32_t *accepted, int32_t *bonus,
                               void *ws, size_t ws_bytes, void *stream, void *ev_start,
                               void *ev_stop, int launches, unsigned long long wait_ticks) {
    if (dspark_status st = step_check(hidden, w, bias, temps, tokens, logits, B, gamma, d, V, mode,
                                      cutoff, budget, conf, survival, lengths, cu_seqlens,
                                      packed_tokens, packed_src_row, packed_argmax, accepted,
                                      bonus, launches))
        return st;
    if (!ws) return DSPARK_ERR_NULL;
    if (misaligned(ws, 16)) return DSPARK_ERR_ALIGN;
    if (ws_bytes < ws_total_bytes(B, gamma)) return DSPARK_ERR_WORKSPACE;
    return step_launch(hidden, w, bias, temps, tokens, logits, B, gamma, d, V, mode, cutoff,
                       budget, conf, survival, lengths, cu_seqlens, packed_tokens, packed_src_row,
                       packed_argmax, accepted, bonus, ws, as_stream(stream), ev_start, ev_stop,
                       launches, wait_ticks);
}

DSPARK_API dspark_status dspark_step(const dspark_bf16 *hidden, const dspark_bf16 *w, float bias,
                                     const float *temps, const int32_t *tokens,
                                     const dspark_bf16 *logits, int B, int gamma, int d, int V,
                                     int mode, const float *cutoff, long long budget, float *conf,
                                     float *survival, int32_t *lengths, int32_t *cu_seqlens,
                                     int32_t *packed_tokens, int32_t *packed_src_row,
                                     int32_t *packed_argmax, int32_t *accepted, int32_t *bonus,
                                     void *ws, size_t ws_bytes, void *stream) {
    return step_impl(hidden, w, bias, temps, tokens, logits, B, gamma, d, V, mode, cutoff, budget,
                     conf, survival, lengths, cu_seqlens, packed_tokens, packed_src_row,
                     packed_argmax, accepted, bonus, ws, ws_bytes, stream, nullptr, nullptr, 0, 0);
}

DSPARK_API dspark_status dspark_step_ex(
    const dspark_bf16 *hidden, const dspark_bf16 *w, float bias, const float *temps,
    const int32_t *tokens, const dspark_bf16 *logits, int B, int gamma, int d, int V, int mode,
    const float *cutoff, long long budget, float *conf, float *survival, int32_t *lengths,
    int32_t *cu_seqlens, int32_t *packed_tokens, int32_t *packed_src_row, int32_t *packed_argmax,
    int32_t *accepted, int32_t *bonus, void *ws, size_t ws_bytes, void *stream, void *ev_start,
    void *ev_stop, int launches, unsigned long long wait_ticks) {
    return step_impl(hidden, w, bias, temps, tokens, logits, B, gamma, d, V, mode, cutoff, budget,
                     conf, survival, lengths, cu_seqlens, packed_tokens, packed_src_row,
                     packed_argmax, accepted, bonus, ws, ws_bytes, stream, ev_start, ev_stop,
                     launches, wait_ticks);
}

DSPARK_API dspark_status dspark_step_status(void *ws, int32_t *status, void *stream) {
    if (!ws || !status) return DSPARK_ERR_NULL;
    if (misaligned(ws, 16) || misaligned(status, 4)) return DSPARK_ERR_ALIGN;
    return launched(launch_step_status(ws, status, as_stream(stream)));
}

// ------------------------------------------------------------ no allocation

// The workspace of dspark_step_noalloc: one array per device, in the code
// object's own device memory, so the call allocates nothing. In host code the
// name `scratch` is only a stand-in for the symbol; its device address (one per
// device) comes from hipGetSymbolAddress and is the only pointer ever passed to
// a kernel or a fill.
constexpr size_t kNoallocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // device address of `scratch` per device, once set up
}  // namespace

// The current device's scratch address. The first call on a device looks it up
// and zero-fills the array on `s` (the fused step's control words and counters
// must start at zero; every call returns them to zero).
static dspark_status noalloc_scratch(void **out, hipStream_t s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DSPARK_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return DSPARK_ERR_HIP;
        if (launch_fill_zero(p, kNoallocScratchBytes, s) != hipSuccess) return DSPARK_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSPARK_OK;
}

DSPARK_API dspark_status dspark_step_noalloc(
    const dspark_bf16 *hidden, const dspark_bf16 *w, float bias, const float *temps,
    const int32_t *tokens, const dspark_bf16 *logits, int B, int gamma, int d, int V, int mode,
    const float *cutoff, long long budget, float *conf, float *survival, int32_t *lengths,
    int32_t *cu_seqlens, int32_t *packed_tokens, int32_t *packed_src_row, int32_t *packed_argmax,
    int32_t *accepted, int32_t *bonus, int32_t *status, void *stream) {
    if (dspark_status st = step_check(hidden, w, bias, temps, tokens, logits, B, gamma, d, V, mode,
                                      cutoff, budget, conf, survival, lengths, cu_seqlens,
                                      packed_tokens, packed_src_row, packed_argmax, accepted,
                                      bonus, 0))
        return st;
    if (ws_total_bytes(B, gamma) > kNoallocScratchBytes) return DSPARK_ERR_WORKSPACE;
    if (misaligned(status, 4)) return DSPARK_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    void *ws = nullptr;
    if (dspark_status st = noalloc_scratch(&ws, s)) return st;
    dspark_status st = step_launch(hidden, w, bias, temps, tokens, logits, B, gamma, d, V, mode,
                                   cutoff, budget, conf, survival, lengths, cu_seqlens,
                                   packed_tokens, packed_src_row, packed_argmax, accepted, bonus,
                                   ws, s, nullptr, nullptr, 0, 0);
    if (st == DSPARK_OK && status) st = launched(launch_step_status(ws, status, s));
    return st;
}
