// accept.hip - stage kernels for steps 5-6, run after the target forward on the
// verify batch. Up to kMaxFusedB requests: one launch that streams the packed
// rows in one contiguous sub-chunk per wave and finishes each request in the
// wave that completes it (counted on a per-request atomic, no waiting).
// Larger batches: a persistent argmax pass balanced across all waves, then
// one wave per request for acceptance and the bonus token.
#include <atomic>

#include "argmax_dev.hpp"

namespace dspark {

constexpr int kArgmaxThreads = 256;  // 4 waves
constexpr int kArgmaxUnroll = 8;     // 16-byte loads in flight per lane
constexpr int kFinalThreads = 256;

template <bool kVec>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_rows_kernel(
    const uint16_t *__restrict__ logits, const int32_t *__restrict__ psrc,
    const int32_t *__restrict__ cu, int B, int gamma, int V, int W,
    uint64_t *__restrict__ keys) {
    const int cap = B * (gamma + 1);
    const int total = packed_total(cu, B, cap);
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    wave_argmax_share<kVec, kArgmaxUnroll>(logits, psrc, total, cap, V, w, W, keys);
}

template <bool kVec>
__global__ __launch_bounds__(kFinalThreads) void accept_kernel(
    const uint64_t *__restrict__ keys, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ tokens, int B, int gamma, int V, int W,
    int32_t *__restrict__ pam, int32_t *__restrict__ acc, int32_t *__restrict__ bonus) {
    const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const int cap = B * (gamma + 1);
    const int total = packed_total(cu, B, cap);
    const int64_t Vv = kVec ? (V >> 3) : V;
    const int64_t Q = partition_q((int64_t)total * Vv, W);
    wave_accept_request(keys, cu, tokens, b, gamma, total, Vv, Q, pam, acc, bonus);
}

// Waves of the persistent argmax grid: every workgroup must be resident at
// once, or a static balanced partition would run its late workgroups as a
// second round. The count comes from the occupancy of the kernel actually
// launched, times the compute units, capped by the workspace's key slots.
template <bool kVec>
int argmax_wave_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int w = cache[dev].load(std::memory_order_relaxed);
    if (w > 0) return w;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, argmax_rows_kernel<kVec>,
                                                     kArgmaxThreads, 0) != hipSuccess ||
        blocks < 1)
        blocks = 1;
    int64_t waves = (int64_t)blocks * device_cu_count() * (kArgmaxThreads / kWave);
    w = (int)(waves < kMaxWaves ? waves : kMaxWaves);
    w -= w % (kArgmaxThreads / kWave);
    cache[dev].store(w, std::memory_order_relaxed);
    return w;
}

// ------------------------------------------------ one launch (B <= kMaxFusedB)

constexpr int kAcceptThreads = 512;
constexpr int kAcceptWavesPerCU = 16;  // target waves per CU
constexpr int kAcceptUnroll = 2;       // 16-byte loads in flight per lane

struct AcceptParams {
    const uint16_t *logits;
    const int32_t *psrc;   // nullable: packed row r reads row r
    const int32_t *cu, *tokens;
    int B, gamma, V;
    int32_t *pam, *acc, *bonus;
    uint64_t *keys;
    uint64_t *arrivals;    // [B] slots streamed per request, zero between calls
    int target_waves;
};

// Largest b in [0, B) with cu[b] <= r (cu non-decreasing): the request that
// owns packed row r when cu[0] <= r < cu[B].
__device__ __forceinline__ int packed_owner(const int *cu, int B, int64_t r) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Exclusive maximum-scan of one non-negative int per thread across the block
// (0 for thread 0). lds needs 17 ints. Contains barriers: call from every thread.
__device__ __forceinline__ int block_excl_max_scan(int x, int *lds) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    int inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(inc, off, kWave);
        if (lane >= off) inc = y > inc ? y : inc;
    }
    if (lane == kWave - 1) lds[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const int t = lane < nw ? lds[lane] : 0;
        int ti = t;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(ti, off, kWave);
            if (lane >= off) ti = y > ti ? y : ti;
        }
        const int prev = __shfl_up(ti, 1, kWave);  // max over the waves before this one
        if (lane < nw) lds[lane] = lane == 0 ? 0 : prev;
    }
    __syncthreads();
    int before = __shfl_up(inc, 1, kWave);  // max over the earlier lanes of this wave
    if (lane == 0) before = 0;
    const int r = before > lds[wave] ? before : lds[wave];
    __syncthreads();
    return r;
}

template <bool kVec>
__global__ __launch_bounds__(kAcceptThreads) void accept_stream_kernel(AcceptParams p) {
    extern __shared__ int cu_s[];  // [B + 1], made non-decreasing and clamped to the capacity
    __shared__ int scan_lds[17];
    const int B = p.B, g1 = p.gamma + 1;
    const int cap = B * g1;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int lane = tid & (kWave - 1);
    // cu_seqlens, clamped to [0, cap] and made non-decreasing by a running
    // maximum, so every packed row belongs to exactly one request and every
    // request's counter reaches its target: each thread takes a contiguous run
    // of entries, then a block scan carries the maximum across runs
    {
        const int n = B + 1;
        const int per = (n + bd - 1) / bd;
        const int f0 = tid * per;
        int m = 0;
        for (int j = 0; j < per && f0 + j < n; ++j) {
            int c = p.cu[f0 + j];
            c = c < 0 ? 0 : (c > cap ? cap : c);
            m = c > m ? c : m;
            cu_s[f0 + j] = m;
        }
        const int carry = block_excl_max_scan(m, scan_lds);
        for (int j = 0; j < per && f0 + j < n; ++j)
            cu_s[f0 + j] = cu_s[f0 + j] > carry ? cu_s[f0 + j] : carry;
        __syncthreads();
    }

    const int64_t Vv = kVec ? (p.V >> 3) : p.V;
    const int64_t r0 = cu_s[0];
    const int64_t E = ((int64_t)cu_s[B] - r0) * Vv;
    const int64_t K = sub_len(E, p.target_waves);
    const int64_t NS = (E + K - 1) / K;
    const int64_t W = (int64_t)gridDim.x * (bd / kWave);

    auto accept = [&](int b) {
        const int start = cu_s[b];
        wave_accept_rows(
            [&](int j) { return row_argmax<true>(p.keys, start + j - r0, Vv, K); },
            cu_s[b + 1] - start, p.gamma, p.tokens + (size_t)b * g1, p.pam + start, p.acc + b,
            p.bonus + b);
    };
    // requests without rows: accepted 0, bonus -1, by the workgroup that owns them
    if (tid < kWave)
        for (int b = blockIdx.x; b < B; b += gridDim.x)
            if (cu_s[b + 1] == cu_s[b] && lane == 0) {
                p.acc[b] = 0;
                p.bonus[b] = -1;
            }
    auto arrive = [&](int b, int64_t n) {
        __builtin_amdgcn_s_waitcnt(0);  // the key stores are at the coherence point
        unsigned long long old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(p.arrivals + b, (uint64_t)n, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0, kWave);
        if ((int64_t)old + n == (int64_t)(cu_s[b + 1] - cu_s[b]) * Vv) {
            if (lane == 0)  // leave the counter at zero for the next call
                __hip_atomic_store(p.arrivals + b, (uint64_t)0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            accept(b);
        }
    };
    for (int64_t cur = (int64_t)blockIdx.x * (bd / kWave) + tid / kWave; cur < NS; cur += W) {
        int64_t e = cur * K;
        const int64_t e_end = e + K < E ? e + K : E;
        int64_t rr = e / Vv;  // packed row relative to cu[0]
        int cur_b = -1;
        int64_t done = 0;
        while (e < e_end) {
            const int64_t row_end = (rr + 1) * Vv;
            const int64_t seg_end = e_end < row_end ? e_end : row_end;
            const int64_t r = r0 + rr;
            const int b = packed_owner(cu_s, B, r);
            if (b != cur_b) {
                if (cur_b >= 0) arrive(cur_b, done);
                cur_b = b;
                done = 0;
            }
            const int64_t src = p.psrc ? (int64_t)p.psrc[r] : r;
            float best = -INFINITY;
            int bidx = -1;
            if (src >= 0 && src < cap)
                lane_row_segment<kVec, kAcceptUnroll>(p.logits + (size_t)src * (size_t)p.V,
                                                      e - rr * Vv, seg_end - rr * Vv, lane, best,
                                                      bidx);
            uint64_t key = bidx >= 0 ? argmax_key(best, (uint32_t)bidx) : 0ull;
            key = wave_max_u64(key);
            if (lane == 0) store_key_coherent(p.keys + cur + rr, key);
            done += seg_end - e;
            e = seg_end;
            ++rr;
        }
        if (cur_b >= 0) arrive(cur_b, done);
    }
}

template <bool kVec>
static int accept_stream_grid(size_t lds) {
    static std::atomic<int> cache[64][8];  // LDS buckets of 4 KiB: (B+1)*4 <= 16388 bytes
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    const int bucket = (int)((lds + 4095) / 4096);
    int gsz = cache[dev][bucket].load(std::memory_order_relaxed);
    if (gsz > 0) return gsz;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, accept_stream_kernel<kVec>,
                                                     kAcceptThreads, (size_t)bucket * 4096) !=
            hipSuccess ||
        blocks < 1)
        blocks = 1;
    gsz = blocks * device_cu_count();
    cache[dev][bucket].store(gsz, std::memory_order_relaxed);
    return gsz;
}

static hipError_t launch_accept_stream(const uint16_t *logits, const int32_t *psrc,
                                       const int32_t *cu, const int32_t *tokens, int B, int gamma,
                                       int V, int32_t *pam, int32_t *acc, int32_t *bonus,
                                       void *ws, hipStream_t s) {
    const bool vec = (V % 8 == 0) && ((uintptr_t)logits % 16 == 0);
    char *wsb = static_cast<char *>(ws);
    AcceptParams p;
    p.logits = logits;
    p.psrc = psrc;
    p.cu = cu;
    p.tokens = tokens;
    p.B = B;
    p.gamma = gamma;
    p.V = V;
    p.pam = pam;
    p.acc = acc;
    p.bonus = bonus;
    p.keys = reinterpret_cast<uint64_t *>(wsb + ws_keys_offset());
    p.arrivals = reinterpret_cast<uint64_t *>(wsb + ws_acnt_offset());
    const int cus = device_cu_count();
    p.target_waves = kAcceptWavesPerCU * cus < kMaxWaves ? kAcceptWavesPerCU * cus : (int)kMaxWaves;
    const size_t lds = (size_t)(B + 1) * sizeof(int);
    const int64_t Vv = vec ? V / 8 : V;
    const int64_t cap = (int64_t)B * (gamma + 1);
    int need = (p.target_waves + kAcceptThreads / kWave - 1) / (kAcceptThreads / kWave);
    const int64_t max_wgs = ((cap * Vv + kSubMin - 1) / kSubMin + kAcceptThreads / kWave - 1) /
                            (kAcceptThreads / kWave);
    if (max_wgs < need) need = max_wgs < 1 ? 1 : (int)max_wgs;
    int g = vec ? accept_stream_grid<true>(lds) : accept_stream_grid<false>(lds);
    g = g < need ? g : need;
    if (vec)
        hipLaunchKernelGGL((accept_stream_kernel<true>), dim3(g), dim3(kAcceptThreads), lds, s, p);
    else
        hipLaunchKernelGGL((accept_stream_kernel<false>), dim3(g), dim3(kAcceptThreads), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_accept(const uint16_t *logits, const int32_t *psrc, const int32_t *cu,
                         const int32_t *tokens, int B, int gamma, int V, int32_t *pam,
                         int32_t *acc, int32_t *bonus, void *ws, hipStream_t s) {
    if (B <= kMaxFusedB)
        return launch_accept_stream(logits, psrc, cu, tokens, B, gamma, V, pam, acc, bonus, ws, s);
    const bool vec = (V % 8 == 0) && ((uintptr_t)logits % 16 == 0);
    const int W = vec ? argmax_wave_count<true>() : argmax_wave_count<false>();
    uint64_t *keys = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + ws_keys_offset());
    dim3 grid(W / (kArgmaxThreads / kWave)), block(kArgmaxThreads);
    dim3 fgrid((B + kFinalThreads / kWave - 1) / (kFinalThreads / kWave)), fblock(kFinalThreads);
    if (vec) {
        hipLaunchKernelGGL((argmax_rows_kernel<true>), grid, block, 0, s, logits, psrc, cu, B,
                           gamma, V, W, keys);
        hipLaunchKernelGGL((accept_kernel<true>), fgrid, fblock, 0, s, keys, cu, tokens, B, gamma,
                           V, W, pam, acc, bonus);
    } else {
        hipLaunchKernelGGL((argmax_rows_kernel<false>), grid, block, 0, s, logits, psrc, cu, B,
                           gamma, V, W, keys);
        hipLaunchKernelGGL((accept_kernel<false>), fgrid, fblock, 0, s, keys, cu, tokens, B,
                           gamma, V, W, pam, acc, bonus);
    }
    return hipGetLastError();
}

}  // namespace dspark
