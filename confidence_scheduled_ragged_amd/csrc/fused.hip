// fused.hip - the whole verify step as a short chain of launches on one stream.
//
//   front   one workgroup per request: the confidence GEMV of the request's gamma
//           hidden rows (one wave per row), the STS sigmoid, the sequential
//           survival product and, in threshold mode, the verify length.
//   select  (budget mode only) one workgroup: the batch-wide top-T pick over all
//           survival values and each request's verify length.
//   stream  a persistent grid: every workgroup scans the verify lengths into
//           cu_seqlens in LDS and writes the schedule outputs of its own
//           requests; then the packed logit rows of all requests, laid end to
//           end and cut into 16 KiB sub-chunks, are streamed: each wave leaves
//           one argmax key per row segment of each sub-chunk it reads. The
//           sub-chunks are dealt out cyclically over all resident waves.
//   finish  one wave per request: each packed row's argmax from its keys, the
//           longest agreeing prefix and the bonus token.
//
// Small cyclic sub-chunks spread the rows of every request over the whole
// chip. Dynamic hand-out through per-XCD atomic work queues was measured
// slower: one queue serves about one ticket per 11 ns, and even a queue that
// serves only the last fifth of the sub-chunks cost 2-6 us per step. Grid-wide
// waits were measured at 16-76 us each and are not used.
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
constexpr int kStreamThreads = 512;
constexpr int kStreamUnroll = 8;
constexpr int kFinishThreads = 256;
constexpr int kMaxFusedB = 4096;  // LDS of the stream kernel: 8*B + 4 bytes

// ------------------------------------------------------------------ front

struct FrontParams {
    const uint16_t *hidden, *w;
    const float *temps, *cutoff;
    float bias;
    int gamma, d, mode;
    float *conf, *surv;
    int32_t *lengths;
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
    if (threadIdx.x == 0 && p.mode == DSPARK_CUT_THRESHOLD)
        p.lengths[b] = threshold_length(s_s, p.gamma, p.cutoff[b]);
}

// ----------------------------------------------------------------- stream

struct StreamParams {
    const uint16_t *logits;
    const int32_t *tokens;
    const int32_t *lengths;
    int B, gamma, V;
    int32_t *cu, *ptok, *psrc;
    uint64_t *keys;
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
__global__ __launch_bounds__(kStreamThreads) void step_stream_kernel(StreamParams p) {
    extern __shared__ int smem[];
    int *len_s = smem;          // [B]
    int *cu_s = smem + p.B;     // [B + 1]
    __shared__ int scan_lds[17];
    const int B = p.B, g = p.gamma, g1 = p.gamma + 1;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int lane = tid & (kWave - 1);

    // schedule: lengths (clamped), cu_seqlens in LDS, this workgroup's outputs
    for (int b = tid; b < B; b += bd) {
        const int L = p.lengths[b];
        len_s[b] = L < 0 ? 0 : (L > g ? g : L);
    }
    __syncthreads();
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
    for (int b = blockIdx.x; b < B; b += gridDim.x) {
        if (tid == 0) {
            p.cu[b + 1] = cu_s[b + 1];
            if (b == 0) p.cu[0] = 0;
        }
        for (int j = tid; j <= len_s[b]; j += bd) {
            p.ptok[cu_s[b] + j] = p.tokens[(size_t)b * g1 + j];
            p.psrc[cu_s[b] + j] = b * g1 + j;
        }
    }

    // sub-chunks of the packed rows, dealt out cyclically: wave w of W streams
    // sub-chunks w, w + W, w + 2W, ... (no atomics, no waits)
    const int64_t Vv = kVec ? (p.V >> 3) : p.V;
    const int64_t E = (int64_t)cu_s[B] * Vv;
    const int64_t NS = (E + kSubSlots - 1) / kSubSlots;
    const int64_t W = (int64_t)gridDim.x * (bd / kWave);
    for (int64_t cur = (int64_t)blockIdx.x * (bd / kWave) + tid / kWave; cur < NS; cur += W) {
        // stream sub-chunk `cur`: slots [cur*K, min((cur+1)*K, E)), row by row
        int64_t e = cur * kSubSlots;
        const int64_t e_end = e + kSubSlots < E ? e + kSubSlots : E;
        int64_t r = e / Vv;
        while (e < e_end) {
            const int64_t row_end = (r + 1) * Vv;
            const int64_t seg_end = e_end < row_end ? e_end : row_end;
            const int b = row_owner(cu_s, B, r);
            const int64_t src = (int64_t)b * g1 + (r - cu_s[b]);
            float best = -INFINITY;
            int bidx = -1;
            lane_row_segment<kVec, kStreamUnroll>(p.logits + (size_t)src * (size_t)p.V,
                                                  e - r * Vv, seg_end - r * Vv, lane, best, bidx);
            uint64_t key = bidx >= 0 ? argmax_key(best, (uint32_t)bidx) : 0ull;
            key = wave_max_u64(key);
            if (lane == 0) p.keys[cur + r] = key;
            e = seg_end;
            ++r;
        }
    }
}

// ----------------------------------------------------------------- finish

template <bool kVec>
__global__ __launch_bounds__(kFinishThreads) void step_finish_kernel(
    const uint64_t *__restrict__ keys, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ tokens, int B, int gamma, int V, int32_t *__restrict__ pam,
    int32_t *__restrict__ acc, int32_t *__restrict__ bonus) {
    const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const int total = packed_total(cu, B, B * (gamma + 1));
    const int64_t Vv = kVec ? (V >> 3) : V;
    wave_accept_request(keys, cu, tokens, b, gamma, total, Vv, kSubSlots, pam, acc, bonus);
}

// ----------------------------------------------------------------- launch

template <bool kVec>
static int stream_grid(size_t lds) {
    // resident workgroups of the stream kernel for this LDS size, cached per
    // device and 4 KiB LDS bucket
    static std::atomic<int> cache[64][13];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    const int bucket = (int)((lds + 4095) / 4096);
    int gsz = cache[dev][bucket].load(std::memory_order_relaxed);
    if (gsz > 0) return gsz;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, step_stream_kernel<kVec>,
                                                     kStreamThreads, (size_t)bucket * 4096) !=
            hipSuccess ||
        blocks < 1)
        blocks = 1;
    gsz = blocks * device_cu_count();
    cache[dev][bucket].store(gsz, std::memory_order_relaxed);
    return gsz;
}

hipError_t launch_fused_step(const uint16_t *hidden, const uint16_t *w, float bias,
                             const float *temps, const int32_t *tokens, const uint16_t *logits,
                             int B, int gamma, int d, int V, int mode, const float *cutoff,
                             long long budget, float *conf, float *surv, int32_t *lengths,
                             int32_t *cu, int32_t *ptok, int32_t *psrc, int32_t *pam,
                             int32_t *acc, int32_t *bonus, void *ws, hipStream_t s) {
    if (B > kMaxFusedB) return hipErrorNotSupported;
    char *wsb = static_cast<char *>(ws);
    uint64_t *keys = reinterpret_cast<uint64_t *>(wsb + ws_keys_offset());

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
    if (hvec && d <= kFrontMaxLdsW)
        hipLaunchKernelGGL((step_front_kernel<true, true>), dim3(B), dim3(kFrontThreads),
                           (size_t)d * 2, s, fp);
    else if (hvec)
        hipLaunchKernelGGL((step_front_kernel<true, false>), dim3(B), dim3(kFrontThreads), 0, s, fp);
    else
        hipLaunchKernelGGL((step_front_kernel<false, false>), dim3(B), dim3(kFrontThreads), 0, s, fp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    if (mode == DSPARK_CUT_BUDGET) {
        e = launch_schedule(surv, B, gamma, mode, cutoff, budget, lengths, s);
        if (e != hipSuccess) return e;
    }

    const bool vvec = (V % 8 == 0) && ((uintptr_t)logits % 16 == 0);
    const size_t lds = (size_t)(2 * B + 1) * sizeof(int);
    StreamParams p;
    p.logits = logits;
    p.tokens = tokens;
    p.lengths = lengths;
    p.B = B;
    p.gamma = gamma;
    p.V = V;
    p.cu = cu;
    p.ptok = ptok;
    p.psrc = psrc;
    p.keys = keys;
    const dim3 fgrid((B + kFinishThreads / kWave - 1) / (kFinishThreads / kWave));
    if (vvec) {
        hipLaunchKernelGGL((step_stream_kernel<true>), dim3(stream_grid<true>(lds)),
                           dim3(kStreamThreads), lds, s, p);
        hipLaunchKernelGGL((step_finish_kernel<true>), fgrid, dim3(kFinishThreads), 0, s, keys, cu,
                           tokens, B, gamma, V, pam, acc, bonus);
    } else {
        hipLaunchKernelGGL((step_stream_kernel<false>), dim3(stream_grid<false>(lds)),
                           dim3(kStreamThreads), lds, s, p);
        hipLaunchKernelGGL((step_finish_kernel<false>), fgrid, dim3(kFinishThreads), 0, s, keys,
                           cu, tokens, B, gamma, V, pam, acc, bonus);
    }
    return hipGetLastError();
}

}  // namespace dspark
