// fused.hip - the whole verify step as two launches on one stream.
//
//   front   two kinds of workgroup in one grid. Workgroup b < B: the confidence
//           GEMV of request b's gamma hidden rows, the STS sigmoid, the
//           sequential survival product and, in threshold mode, the verify
//           length. The other workgroups stream the root rows (row 0 of every
//           request, verified whatever the cut) while the GEMV runs, and leave
//           argmax keys of their segments. In budget mode the last request
//           workgroup to finish (counted on an atomic arrival counter, no
//           waiting) runs the batch-wide top-T pick and writes every length.
//   stream  every workgroup scans the verify lengths into cu_seqlens in LDS and
//           writes the schedule outputs of its own requests; then the draft
//           rows of all requests, laid end to end, are cut into sub-chunks of
//           about equal length, one contiguous run per wave, and each wave
//           leaves one argmax key per row segment. A per-request atomic counts
//           the draft slots done; the wave that completes a request merges its
//           keys and writes the acceptance and bonus token (no waiting).
//
// Long contiguous runs per wave were measured faster than small interleaved
// sub-chunks (HBM row-buffer locality), and two 16-byte loads in flight per
// lane with full occupancy faster than deeper unrolling with fewer waves.
// Dynamic hand-out through per-XCD atomic work queues was measured slower:
// one queue address serves about one ticket per 11-15 ns. Grid-wide waits
// were measured at 16-76 us each and are not used.
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

constexpr int kFrontThreads = 512;
constexpr int kFrontMaxLdsW = 16384;
constexpr int kFusedSelPer = 8;  // survival values per thread of the in-front select
constexpr int kFusedSelMax = kFusedSelPer * kFrontThreads;
constexpr int kFrontRootWGsPerCU = 1;  // root-row workgroups of the front grid per CU
constexpr int kStreamThreads = 512;
constexpr int kStreamWavesPerCU = 16;  // target waves of the draft-row stream per CU
constexpr int kStreamUnroll = 2;  // 16-byte loads in flight per lane (more waves, fewer bytes each)
// Root rows of the front kernel: four 16-byte loads in flight per lane when
// they are the front's critical path, two when the GEMV-and-pick chain is (the
// last request workgroup runs the batch-wide pick after the slowest GEMV; a
// request's GEMV reads gamma*d bf16, its root row V). Measured per step: the
// mixed workload's threshold arm 111 us with four against 113-115 with two;
// its budget arm (gamma*d = 65536 < V/2) 68.1 against 70.3; the budget
// workload at d = 7168 (gamma*d = 114688 > V/2) 67.7 with two against 69.3.
constexpr int kRootUnrollDeep = 4;
constexpr int kRootUnrollShallow = 2;

// ------------------------------------------------------------------ front

struct FrontParams {
    const uint16_t *hidden, *w, *logits;
    const float *temps, *cutoff;
    float bias;
    int B, gamma, d, V, mode;
    int t;                // budget / combined: number of positions to pick, in [0, B*gamma]
    float *conf, *surv;
    int32_t *lengths;
    uint64_t *rkeys;      // segment keys of the root rows
    uint64_t *req_arrivals;  // [B] the stream kernel's per-request counters, zeroed here
    unsigned *arrivals;   // budget select in the front kernel: arrival counter, else NULL
};

// Root rows (dense row b*(gamma+1) of every request b), laid end to end and
// cut into sub-chunks of about equal length, one per root wave: wave w of
// nwaves streams sub-chunks w, w + nwaves, ... and leaves one key per row
// segment at rkeys[s + b].
template <bool kVec, int kRootUnroll>
__device__ __forceinline__ void front_root_rows(const FrontParams &p, int64_t w, int64_t nwaves) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t Vv = kVec ? (p.V >> 3) : p.V;
    const int64_t E = (int64_t)p.B * Vv;
    const int64_t K = sub_len(E, nwaves);
    const int64_t NS = (E + K - 1) / K;
    const size_t row_stride = (size_t)(p.gamma + 1) * (size_t)p.V;
    for (int64_t cur = w; cur < NS; cur += nwaves) {
        int64_t e = cur * K;
        const int64_t e_end = e + K < E ? e + K : E;
        int64_t r = e / Vv;
        while (e < e_end) {
            const int64_t row_end = (r + 1) * Vv;
            const int64_t seg_end = e_end < row_end ? e_end : row_end;
            float best = -INFINITY;
            int bidx = -1;
            lane_row_segment<kVec, kRootUnroll>(p.logits + (size_t)r * row_stride, e - r * Vv,
                                                  seg_end - r * Vv, lane, best, bidx);
            uint64_t key = bidx >= 0 ? argmax_key(best, (uint32_t)bidx) : 0ull;
            key = wave_max_u64(key);
            if (lane == 0) p.rkeys[cur + r] = key;
            e = seg_end;
            ++r;
        }
    }
}

template <bool kVecH, bool kLdsW, bool kVecV, int kRootUnroll>
__global__ __launch_bounds__(kFrontThreads) void step_front_kernel(FrontParams p) {
    extern __shared__ __align__(16) uint16_t dyn_lds[];
    __shared__ float z_s[DSPARK_MAX_GAMMA], p_s[DSPARK_MAX_GAMMA], s_s[DSPARK_MAX_GAMMA];
    __shared__ uint32_t hist[4 * 256], sh[4];
    __shared__ int scan_lds[17];
    __shared__ int last_s;
    if ((int)blockIdx.x >= p.B) {
        const int nw = blockDim.x / kWave;
        front_root_rows<kVecV, kRootUnroll>(
            p, (int64_t)((int)blockIdx.x - p.B) * nw + threadIdx.x / kWave,
            (int64_t)((int)gridDim.x - p.B) * nw);
        return;
    }
    const int b = blockIdx.x;
    const int tid = threadIdx.x, bd = blockDim.x;
    if (tid == 0)
        __hip_atomic_store(p.req_arrivals + b, (uint64_t)0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    const uint16_t *wp = p.w;
    if (kLdsW) {
        stage_w(p.w, p.d, dyn_lds);
        __syncthreads();
        wp = dyn_lds;
    }
    request_logits<kVecH>(p.hidden + (size_t)b * p.gamma * p.d, wp, p.bias, p.gamma, p.d, z_s);
    __syncthreads();
    request_survival(z_s, p.temps, p.gamma, p_s, s_s, p.conf + (size_t)b * p.gamma, nullptr);
    const bool select_here = p.arrivals != nullptr;
    float *surv_b = p.surv + (size_t)b * p.gamma;
    for (int i = tid; i < p.gamma; i += bd) {
        // the select reads survival from another workgroup of this grid: write
        // it through to the device coherence point
        if (select_here)
            __hip_atomic_store(surv_b + i, s_s[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            surv_b[i] = s_s[i];
    }
    if (p.mode == DSPARK_CUT_THRESHOLD) {
        if (tid == 0) p.lengths[b] = threshold_length(s_s, p.gamma, p.cutoff[b]);
        return;
    }
    if (p.mode == DSPARK_CUT_STATIC) {
        if (tid == 0) p.lengths[b] = p.gamma;
        return;
    }
    if (!select_here) return;

    // budget: count this request as done once its survival stores are complete;
    // the workgroup that counts the last request picks for the whole batch
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(p.arrivals, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        last_s = old == (unsigned)(p.B - 1);
    }
    __syncthreads();
    if (!last_s) return;
    if (tid == 0) __hip_atomic_store(p.arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int N = p.B * p.gamma;
    float *sv = reinterpret_cast<float *>(dyn_lds);  // w is no longer needed
    __syncthreads();
    // combined cut: a position below its request's cutoff ranks below every
    // eligible one, and the budget is capped by the eligible count
    const bool combined = p.mode == DSPARK_CUT_COMBINED;
    // N <= kFusedSelPer * blockDim: every load of a thread is issued before
    // any is waited for (one round trip instead of kFusedSelPer)
    float v[kFusedSelPer], c[kFusedSelPer];
#pragma unroll
    for (int j = 0; j < kFusedSelPer; ++j) {
        const int f = tid + j * bd;
        v[j] = f < N ? __hip_atomic_load(p.surv + f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     : 0.0f;
        c[j] = (combined && f < N) ? p.cutoff[f / p.gamma] : 0.0f;
    }
    int n = 0;
#pragma unroll
    for (int j = 0; j < kFusedSelPer; ++j) {
        const int f = tid + j * bd;
        if (f < N) {
            float x = v[j];
            if (combined && !(x >= c[j])) x = -INFINITY;
            else ++n;
            sv[f] = x;
        }
    }
    int eligible = N;
    if (combined)
        block_excl_scan(n, &eligible, scan_lds);  // contains the barriers sv needs
    else
        __syncthreads();
    const int t = p.t < eligible ? p.t : eligible;
    if (t <= 0 || t >= N) {
        for (int r = tid; r < p.B; r += bd) p.lengths[r] = t <= 0 ? 0 : p.gamma;
        return;
    }
    const BudgetCut cut = budget_select_runs<kFusedSelPer>(sv, N, t, hist, sh);
    budget_lengths(sv, nullptr, p.B, p.gamma, cut, p.lengths, scan_lds);
}

// ----------------------------------------------------------------- stream

struct StreamParams {
    const uint16_t *logits;
    const int32_t *tokens;
    const int32_t *lengths;
    int B, gamma, V;
    int32_t *cu, *ptok, *psrc, *pam, *acc, *bonus;
    uint64_t *keys;
    const uint64_t *rkeys;  // root-row keys from the front kernel
    uint64_t *arrivals;     // [B] draft slots streamed per request, zeroed by the front
    int target_waves;       // sub-chunk length: about one sub-chunk per target wave
    int root_waves;         // waves that streamed the root rows in the front kernel
};

// Largest b in [0, B] with cu[b] - b <= r, i.e. the request that owns draft
// row r (draft rows start at cu[b] - b; requests without drafts own none)
// when r < cu[B] - B.
__device__ __forceinline__ int draft_owner(const int *cu, int B, int64_t r) {
    int lo = 0, hi = B;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)(cu[mid] - mid) <= r) lo = mid; else hi = mid - 1;
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

    // draft rows in sub-chunks of about equal length, one per target wave,
    // dealt out cyclically: wave w of W streams sub-chunks w, w + W, ...
    // Long contiguous runs per wave keep the HBM row buffers better used than
    // many short interleaved ones.
    const int64_t Vv = kVec ? (p.V >> 3) : p.V;
    const int64_t E = (int64_t)(cu_s[B] - B) * Vv;
    const int64_t K = sub_len(E, p.target_waves);
    const int64_t Kr = sub_len((int64_t)B * Vv, p.root_waves);
    const int64_t NS = (E + K - 1) / K;
    const int64_t W = (int64_t)gridDim.x * (bd / kWave);

    // acceptance and bonus of request b by the calling wave: the root row's
    // argmax from the front kernel's keys, the draft rows' from this kernel's
    auto accept = [&](int b) {
        const int start = cu_s[b];
        const int dstart = start - b;  // first draft row of request b
        wave_accept_rows(
            [&](int j) {
                return j == 0 ? row_argmax(p.rkeys, b, Vv, Kr)
                              : row_argmax<true>(p.keys, dstart + j - 1, Vv, K);
            },
            len_s[b] + 1, g, p.tokens + (size_t)b * g1, p.pam + start, p.acc + b, p.bonus + b);
    };
    // requests without draft rows are finished by the workgroup that owns them
    if (tid < kWave)
        for (int b = blockIdx.x; b < B; b += gridDim.x)
            if (len_s[b] == 0) accept(b);
    // `n` more draft slots of request b are done and their keys stored: count
    // them; the wave that completes the request finishes it (no waiting)
    auto arrive = [&](int b, int64_t n) {
        __builtin_amdgcn_s_waitcnt(0);  // the key stores are at the coherence point
        unsigned long long old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(p.arrivals + b, (uint64_t)n, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0, kWave);
        if ((int64_t)old + n == (int64_t)len_s[b] * Vv) accept(b);
    };
    for (int64_t cur = (int64_t)blockIdx.x * (bd / kWave) + tid / kWave; cur < NS; cur += W) {
        // stream sub-chunk `cur`: slots [cur*K, min((cur+1)*K, E)), row by row
        int64_t e = cur * K;
        const int64_t e_end = e + K < E ? e + K : E;
        int64_t r = e / Vv;
        int cur_b = -1;    // request of the rows being streamed
        int64_t done = 0;  // its slots streamed in this sub-chunk
        while (e < e_end) {
            const int64_t row_end = (r + 1) * Vv;
            const int64_t seg_end = e_end < row_end ? e_end : row_end;
            const int b = draft_owner(cu_s, B, r);
            if (b != cur_b) {
                if (cur_b >= 0) arrive(cur_b, done);
                cur_b = b;
                done = 0;
            }
            const int64_t src = (int64_t)b * g1 + 1 + (r - (cu_s[b] - b));
            float best = -INFINITY;
            int bidx = -1;
            lane_row_segment<kVec, kStreamUnroll>(p.logits + (size_t)src * (size_t)p.V,
                                                  e - r * Vv, seg_end - r * Vv, lane, best, bidx);
            uint64_t key = bidx >= 0 ? argmax_key(best, (uint32_t)bidx) : 0ull;
            key = wave_max_u64(key);
            if (lane == 0) store_key_coherent(p.keys + cur + r, key);
            done += seg_end - e;
            e = seg_end;
            ++r;
        }
        if (cur_b >= 0) arrive(cur_b, done);
    }
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

template <bool kVecV, int kRootUnroll>
static void launch_front_u(bool hvec, bool ldsw, const FrontParams &fp, int root_wgs, size_t lds,
                           hipStream_t s) {
    const dim3 grid(fp.B + root_wgs), block(kFrontThreads);
    if (hvec && ldsw)
        hipLaunchKernelGGL((step_front_kernel<true, true, kVecV, kRootUnroll>), grid, block, lds, s,
                           fp);
    else if (hvec)
        hipLaunchKernelGGL((step_front_kernel<true, false, kVecV, kRootUnroll>), grid, block, lds,
                           s, fp);
    else
        hipLaunchKernelGGL((step_front_kernel<false, false, kVecV, kRootUnroll>), grid, block, lds,
                           s, fp);
}

template <bool kVecV>
static void launch_front(bool hvec, bool ldsw, const FrontParams &fp, int root_wgs, size_t lds,
                         hipStream_t s) {
    const bool gemv_critical =
        fp.arrivals != nullptr && (int64_t)fp.gamma * fp.d * 2 > (int64_t)fp.V;
    if (gemv_critical)
        launch_front_u<kVecV, kRootUnrollShallow>(hvec, ldsw, fp, root_wgs, lds, s);
    else
        launch_front_u<kVecV, kRootUnrollDeep>(hvec, ldsw, fp, root_wgs, lds, s);
}

hipError_t launch_fused_step(const uint16_t *hidden, const uint16_t *w, float bias,
                             const float *temps, const int32_t *tokens, const uint16_t *logits,
                             int B, int gamma, int d, int V, int mode, const float *cutoff,
                             long long budget, float *conf, float *surv, int32_t *lengths,
                             int32_t *cu, int32_t *ptok, int32_t *psrc, int32_t *pam,
                             int32_t *acc, int32_t *bonus, void *ws, hipStream_t s,
                             hipEvent_t ev_start, hipEvent_t ev_stop) {
    if (B > kMaxFusedB) return hipErrorNotSupported;
    char *wsb = static_cast<char *>(ws);
    uint64_t *keys = reinterpret_cast<uint64_t *>(wsb + ws_keys_offset());
    uint64_t *rkeys = reinterpret_cast<uint64_t *>(wsb + ws_rkeys_offset(B, gamma));
    uint64_t *rcnt = reinterpret_cast<uint64_t *>(wsb + ws_rcnt_offset());
    unsigned *arrivals = reinterpret_cast<unsigned *>(wsb + ws_ctrl_offset());

    const int N = B * gamma;
    const bool hvec = (d % 8 == 0) && (((uintptr_t)hidden | (uintptr_t)w) % 16 == 0);
    const bool ldsw = hvec && d <= kFrontMaxLdsW;
    const bool select_in_front =
        (mode == DSPARK_CUT_BUDGET || mode == DSPARK_CUT_COMBINED) && N <= kFusedSelMax;
    const bool vvec = (V % 8 == 0) && ((uintptr_t)logits % 16 == 0);
    FrontParams fp;
    fp.hidden = hidden;
    fp.w = w;
    fp.logits = logits;
    fp.temps = temps;
    fp.cutoff = cutoff;
    fp.bias = bias;
    fp.B = B;
    fp.gamma = gamma;
    fp.d = d;
    fp.V = V;
    fp.mode = mode;
    fp.t = (int)(budget < (long long)N ? budget : (long long)N);
    fp.conf = conf;
    fp.surv = surv;
    fp.lengths = lengths;
    fp.rkeys = rkeys;
    fp.req_arrivals = rcnt;
    fp.arrivals = select_in_front ? arrivals : nullptr;
    size_t front_lds = ldsw ? (size_t)d * 2 : 0;
    if (select_in_front && (size_t)N * 4 > front_lds) front_lds = (size_t)N * 4;
    // root-row workgroups: a fixed share of the chip, but no more than the
    // root rows fill with minimum-length sub-chunks
    const int cus = device_cu_count();
    const int64_t Vv = vvec ? V / 8 : V;
    const int64_t root_min_wgs =
        ((int64_t)B * Vv + kSubMin * (kFrontThreads / kWave) - 1) / (kSubMin * (kFrontThreads / kWave));
    int64_t root_wgs = (int64_t)kFrontRootWGsPerCU * cus;
    root_wgs = root_wgs < root_min_wgs ? root_wgs : root_min_wgs;
    if (root_wgs * (kFrontThreads / kWave) > kMaxWaves) root_wgs = kMaxWaves / (kFrontThreads / kWave);
    root_wgs = root_wgs < 1 ? 1 : root_wgs;
    const int root_waves = (int)root_wgs * (kFrontThreads / kWave);
    if (vvec)
        launch_front<true>(hvec, ldsw, fp, (int)root_wgs, front_lds, s);
    else
        launch_front<false>(hvec, ldsw, fp, (int)root_wgs, front_lds, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    if ((mode == DSPARK_CUT_BUDGET || mode == DSPARK_CUT_COMBINED) && !select_in_front) {
        e = launch_schedule(surv, B, gamma, mode, cutoff, budget, lengths, s);
        if (e != hipSuccess) return e;
    }

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
    p.pam = pam;
    p.acc = acc;
    p.bonus = bonus;
    p.keys = keys;
    p.rkeys = rkeys;
    p.arrivals = rcnt;
    p.target_waves = kStreamWavesPerCU * cus < kMaxWaves ? kStreamWavesPerCU * cus : (int)kMaxWaves;
    p.root_waves = root_waves;
    // stream grid: enough workgroups for the target waves, at most the resident
    // ones, and no more than the largest possible draft rows (every request at
    // gamma) fill with minimum-length sub-chunks
    int stream_wgs_needed = (p.target_waves + kStreamThreads / kWave - 1) / (kStreamThreads / kWave);
    const int64_t max_sub = ((int64_t)B * gamma * Vv + kSubMin - 1) / kSubMin;
    const int64_t max_wgs = (max_sub + kStreamThreads / kWave - 1) / (kStreamThreads / kWave);
    if (max_wgs < stream_wgs_needed) stream_wgs_needed = max_wgs < 1 ? 1 : (int)max_wgs;
    int g = vvec ? stream_grid<true>(lds) : stream_grid<false>(lds);
    g = g < stream_wgs_needed ? g : stream_wgs_needed;
    // measurement events bracket the dominant kernel (the draft-row stream)
    if (ev_start && (e = hipEventRecord(ev_start, s)) != hipSuccess) return e;
    if (vvec)
        hipLaunchKernelGGL((step_stream_kernel<true>), dim3(g), dim3(kStreamThreads), lds, s, p);
    else
        hipLaunchKernelGGL((step_stream_kernel<false>), dim3(g), dim3(kStreamThreads), lds, s, p);
    e = hipGetLastError();
    if (e == hipSuccess && ev_stop) e = hipEventRecord(ev_stop, s);
    return e;
}

}  // namespace dspark
