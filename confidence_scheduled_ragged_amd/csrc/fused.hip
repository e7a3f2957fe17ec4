// fused.hip - the whole verify step in two launches, with no grid-wide wait.
//
// Launch 1 (front, one workgroup per request): the confidence GEMV of the
// request's gamma hidden rows (one wave per row), the STS sigmoid, the
// sequential survival product and, in threshold mode, the verify length. It
// also zeroes the request's completion counter for launch 2.
//
// Launch 2 (back, a persistent grid sized to be resident at once):
//   * every workgroup derives the whole schedule on its own from launch 1's
//     results (in budget mode a radix select over the batch's survival values)
//     and scans the verify lengths into cu_seqlens in LDS; workgroup k writes
//     the schedule outputs of requests k, k+G, ... ;
//   * the packed rows of all requests, laid end to end, are cut into one
//     contiguous slice per wave; each wave streams its slice and leaves one
//     argmax key per row segment;
//   * when all waves of a workgroup are done, the workgroup adds the number of
//     slots it finished to each request it touched; the workgroup whose
//     addition completes a request computes that request's acceptance and
//     bonus token. No wave ever waits for another workgroup, so the kernel
//     cannot deadlock and needs no co-residency guarantee.
//
// [P1] "DFlash to DSpark in SGLang", sections "DSpark: a sequential head and a
// verify budget" (head, survival, cut), "Ragged verify under full CUDA graphs"
// (front-packed rows and cu_seqlens), "Zero-overhead scheduling and kernels"
// (the schedule and packing fused around the verify) and "Background"
// (greedy acceptance and bonus token).
#include <atomic>

#include "argmax_dev.hpp"
#include "conf_dev.hpp"
#include "sched_dev.hpp"

namespace dspark {

constexpr int kFrontThreads = 1024;
constexpr int kFrontMaxLdsW = 16384;
constexpr int kBackThreads = 512;
constexpr int kBackWaves = kBackThreads / kWave;
constexpr int kBackUnroll = 8;
constexpr int kSelPerThread = 16;                        // budget values per thread
constexpr int kMaxFusedB = 4096;                         // LDS: 8*B + 4 bytes
constexpr int kMaxFusedBudgetN = kSelPerThread * kBackThreads;

// ------------------------------------------------------------------ front

struct FrontParams {
    const uint16_t *hidden, *w;
    const float *temps, *cutoff;
    float bias;
    int gamma, d, mode;
    float *conf, *surv;
    int32_t *lengths;
    unsigned long long *cnt;
};

template <bool kVecH, bool kLdsW>
__global__ __launch_bounds__(kFrontThreads) void step_front_kernel(FrontParams p) {
    extern __shared__ __align__(16) uint16_t w_lds[];
    __shared__ float z_s[DSPARK_MAX_GAMMA], p_s[DSPARK_MAX_GAMMA], s_s[DSPARK_MAX_GAMMA];
    const int b = blockIdx.x;
    const uint16_t *wp = p.w;
    if (kLdsW) {
        stage_w(p.w, p.d, w_lds);
        __syncthreads();
        wp = w_lds;
    }
    request_logits<kVecH>(p.hidden + (size_t)b * p.gamma * p.d, wp, p.bias, p.gamma, p.d, z_s);
    __syncthreads();
    request_survival(z_s, p.temps, p.gamma, p_s, s_s, p.conf + (size_t)b * p.gamma,
                     p.surv + (size_t)b * p.gamma);
    if (threadIdx.x == 0) {
        if (p.mode == DSPARK_CUT_THRESHOLD)
            p.lengths[b] = threshold_length(s_s, p.gamma, p.cutoff[b]);
        p.cnt[b] = 0ull;
    }
}

// ------------------------------------------------------------------- back

struct BackParams {
    const uint16_t *logits;
    const int32_t *tokens;
    const float *surv;
    int B, gamma, V, mode, t_eff, W;
    int32_t *lengths, *cu, *ptok, *psrc, *pam, *acc, *bonus;
    uint64_t *keys;
    unsigned long long *cnt;
};

// Largest b in [0, B] with cu[b] <= r (cu non-decreasing, cu[0] = 0 <= r):
// the request that owns packed row r when r < cu[B].
__device__ __forceinline__ int row_owner(const int *cu, int B, int64_t r) {
    int lo = 0, hi = B;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <bool kVec>
__global__ __launch_bounds__(kBackThreads) void step_back_kernel(BackParams p) {
    extern __shared__ int smem[];
    int *len_s = smem;          // [B]
    int *cu_s = smem + p.B;     // [B + 1]
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh[2];
    __shared__ int scan_lds[17];
    __shared__ int done_s[kBackThreads];
    __shared__ int ndone_s;
    const int B = p.B, g = p.gamma, g1 = p.gamma + 1;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int nw = bd / kWave;

    // 1. verify lengths, derived independently by every workgroup
    if (p.mode == DSPARK_CUT_THRESHOLD) {
        for (int b = tid; b < B; b += bd) {
            const int L = p.lengths[b];
            len_s[b] = L < 0 ? 0 : (L > g ? g : L);
        }
    } else {
        const int N = B * g;
        if (p.t_eff == 0 || p.t_eff == N) {
            for (int b = tid; b < B; b += bd) len_s[b] = p.t_eff == 0 ? 0 : g;
        } else {
            const BudgetCut cut = budget_select_runs<kSelPerThread>(p.surv, N, p.t_eff, hist, sh);
            budget_lengths(p.surv, B, g, cut, len_s, scan_lds);
        }
    }
    __syncthreads();

    // 2. cu_seqlens in LDS
    int carry = 0;
    for (int base = 0; base < B; base += bd) {
        const int b = base + tid;
        const int n = b < B ? len_s[b] + 1 : 0;
        int tot;
        const int st = carry + block_excl_scan(n, &tot, scan_lds);
        if (b < B) cu_s[b] = st;
        carry += tot;
    }
    if (tid == 0) cu_s[B] = carry;
    __syncthreads();
    // schedule outputs: workgroup k writes those of requests k, k+G, ... (a
    // few entries each), so no workgroup starts its slice late
    for (int b = blockIdx.x; b < B; b += gridDim.x) {
        if (tid == 0) {
            p.cu[b + 1] = cu_s[b + 1];
            if (p.mode != DSPARK_CUT_THRESHOLD) p.lengths[b] = len_s[b];
            if (b == 0) p.cu[0] = 0;
        }
        for (int j = tid; j <= len_s[b]; j += bd) {
            p.ptok[cu_s[b] + j] = p.tokens[(size_t)b * g1 + j];
            p.psrc[cu_s[b] + j] = b * g1 + j;
        }
    }

    const int64_t Vv = kVec ? (p.V >> 3) : p.V;
    const int total = cu_s[B];
    const int64_t E = (int64_t)total * Vv;  // slots of all packed rows
    const int64_t Q = partition_q(E, p.W);
    const int64_t w = (int64_t)blockIdx.x * nw + wave;

    // 3. this wave's slice of the packed rows
    int64_t e = w * Q;
    const int64_t e_end = e + Q < E ? e + Q : E;
    int64_t r = e / Vv;
    while (e < e_end) {
        const int64_t row_end = (r + 1) * Vv;
        const int64_t seg_end = e_end < row_end ? e_end : row_end;
        const int b = row_owner(cu_s, B, r);
        const int64_t src = (int64_t)b * g1 + (r - cu_s[b]);
        float best = -INFINITY;
        int bidx = -1;
        lane_row_segment<kVec, kBackUnroll>(p.logits + (size_t)src * (size_t)p.V, e - r * Vv,
                                            seg_end - r * Vv, lane, best, bidx);
        uint64_t key = bidx >= 0 ? argmax_key(best, (uint32_t)bidx) : 0ull;
        key = wave_max_u64(key);
        if (lane == 0) store_key_coherent(p.keys + w + r, key);
        e = seg_end;
        ++r;
    }
    // every key store of this wave is performed before the workgroup counts
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // 4. count this workgroup's finished slots per touched request; the
    //    workgroup that completes a request finishes it
    const int64_t g0 = (int64_t)blockIdx.x * nw * Q;
    int64_t g_end = g0 + (int64_t)nw * Q;
    g_end = g_end < E ? g_end : E;
    if (g0 >= g_end) return;  // no barrier follows
    const int b_first = row_owner(cu_s, B, g0 / Vv);
    const int b_last = row_owner(cu_s, B, (g_end - 1) / Vv);
    for (int base = b_first; base <= b_last; base += bd) {
        if (tid == 0) ndone_s = 0;
        __syncthreads();
        const int b = base + tid;
        if (b <= b_last) {
            const int64_t lo0 = (int64_t)cu_s[b] * Vv;
            const int64_t hi0 = (int64_t)cu_s[b + 1] * Vv;
            const int64_t lo = lo0 > g0 ? lo0 : g0;
            const int64_t hi = hi0 < g_end ? hi0 : g_end;
            if (hi > lo) {
                const unsigned long long mine = (unsigned long long)(hi - lo);
                const unsigned long long old = __hip_atomic_fetch_add(
                    p.cnt + b, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (old + mine == (unsigned long long)(hi0 - lo0)) done_s[atomicAdd(&ndone_s, 1)] = b;
            }
        }
        __syncthreads();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // key loads stay after the counts
        const int nd = ndone_s;
        for (int k = wave; k < nd; k += nw)
            wave_accept_request<true>(p.keys, cu_s, p.tokens, done_s[k], g, total, Vv, Q, p.pam,
                                      p.acc, p.bonus);
        __syncthreads();
    }
}

// ----------------------------------------------------------------- launch

template <bool kVec>
static int back_grid(size_t lds) {
    // resident workgroups of the back kernel for this LDS size, cached per
    // device and 4 KiB LDS bucket
    static std::atomic<int> cache[64][13];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    const int bucket = (int)((lds + 4095) / 4096);
    int gsz = cache[dev][bucket].load(std::memory_order_relaxed);
    if (gsz > 0) return gsz;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, step_back_kernel<kVec>, kBackThreads,
                                                     (size_t)bucket * 4096) != hipSuccess ||
        blocks < 1)
        blocks = 1;
    int64_t gg = (int64_t)blocks * device_cu_count();
    if (gg * kBackWaves > kMaxWaves) gg = kMaxWaves / kBackWaves;
    gsz = (int)gg;
    cache[dev][bucket].store(gsz, std::memory_order_relaxed);
    return gsz;
}

hipError_t launch_fused_step(const uint16_t *hidden, const uint16_t *w, float bias,
                             const float *temps, const int32_t *tokens, const uint16_t *logits,
                             int B, int gamma, int d, int V, int mode, const float *cutoff,
                             long long budget, float *conf, float *surv, int32_t *lengths,
                             int32_t *cu, int32_t *ptok, int32_t *psrc, int32_t *pam,
                             int32_t *acc, int32_t *bonus, void *ws, hipStream_t s) {
    const int N = B * gamma;
    if (B > kMaxFusedB) return hipErrorNotSupported;
    if (mode == DSPARK_CUT_BUDGET && N > kMaxFusedBudgetN) return hipErrorNotSupported;
    char *wsb = static_cast<char *>(ws);
    uint64_t *keys = reinterpret_cast<uint64_t *>(wsb + ws_keys_offset());
    unsigned long long *cnt = reinterpret_cast<unsigned long long *>(wsb + ws_cnt_offset(B, gamma));

    const bool hvec = (d % 8 == 0) && (((uintptr_t)hidden | (uintptr_t)w) % 16 == 0);
    FrontParams fp;
    fp.hidden = hidden;
    fp.w = w;
    fp.temps = temps;
    fp.cutoff = cutoff;
    fp.bias = bias;
    fp.gamma = gamma;
    fp.d = d;
    fp.mode = mode;
    fp.conf = conf;
    fp.surv = surv;
    fp.lengths = lengths;
    fp.cnt = cnt;
    if (hvec && d <= kFrontMaxLdsW)
        hipLaunchKernelGGL((step_front_kernel<true, true>), dim3(B), dim3(kFrontThreads),
                           (size_t)d * 2, s, fp);
    else if (hvec)
        hipLaunchKernelGGL((step_front_kernel<true, false>), dim3(B), dim3(kFrontThreads), 0, s, fp);
    else
        hipLaunchKernelGGL((step_front_kernel<false, false>), dim3(B), dim3(kFrontThreads), 0, s, fp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    const bool vvec = (V % 8 == 0) && ((uintptr_t)logits % 16 == 0);
    const size_t lds = (size_t)(2 * B + 1) * sizeof(int);
    BackParams p;
    p.logits = logits;
    p.tokens = tokens;
    p.surv = surv;
    p.B = B;
    p.gamma = gamma;
    p.V = V;
    p.mode = mode;
    p.t_eff = mode == DSPARK_CUT_BUDGET ? (int)(budget < (long long)N ? budget : N) : 0;
    p.lengths = lengths;
    p.cu = cu;
    p.ptok = ptok;
    p.psrc = psrc;
    p.pam = pam;
    p.acc = acc;
    p.bonus = bonus;
    p.keys = keys;
    p.cnt = cnt;
    if (vvec) {
        const int G = back_grid<true>(lds);
        p.W = G * kBackWaves;
        hipLaunchKernelGGL((step_back_kernel<true>), dim3(G), dim3(kBackThreads), lds, s, p);
    } else {
        const int G = back_grid<false>(lds);
        p.W = G * kBackWaves;
        hipLaunchKernelGGL((step_back_kernel<false>), dim3(G), dim3(kBackThreads), lds, s, p);
    }
    return hipGetLastError();
}

}  // namespace dspark
