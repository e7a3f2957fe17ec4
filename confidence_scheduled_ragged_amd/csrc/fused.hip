// fused.hip - the whole verify step on one stream, in one launch (threshold
// and static cuts from kOneLaunchMinB requests up) or two (budget and combined
// cuts, whose batch-wide pick must see every request's survival, and smaller
// batches).
//
// One launch: a grid of request workgroups (the confidence GEMV of their
// requests' gamma hidden rows, the STS sigmoid, the sequential survival
// product and the verify length), root workgroups (the root rows, verified
// whatever the cut, streamed while the GEMV runs) and plain stream
// workgroups. The last request workgroup to finish (an atomic arrival count)
// raises a flag; every workgroup waits for it once, scans the lengths into
// cu_seqlens in LDS, writes the schedule outputs of its own requests and
// streams one contiguous sub-chunk of the draft rows. Root-row waves reach
// the drafts later and get shorter sub-chunks. Each row segment leaves its
// argmax key in a slot of its own (zeroed by the request workgroups before
// any is written); per-request atomics count the streamed slots of the root
// row and the drafts, issued without waiting for the key stores; the wave
// that completes a request reads the request's slots (polling any not yet
// landed), its root keys and tokens in one memory round trip and writes the
// acceptance and bonus token.
//
// Two launches:
//   front   request workgroups as above and root workgroups; in budget mode
//           the last request workgroup to finish (counted, no waiting) runs
//           the batch-wide top-T pick and writes every length.
//   stream  every workgroup scans the lengths and writes its schedule
//           outputs; the draft rows are cut into sub-chunks of about equal
//           length (at least 4 KiB), one contiguous run per wave, and the
//           wave that completes a request's draft rows finishes it as above.
//
// Long contiguous runs per wave were measured faster than small interleaved
// sub-chunks (HBM row-buffer locality). Each stream keeps as many bytes in
// flight as fill the memory system and no more (two to four 16-byte loads per
// lane at full occupancy, by stream; deeper pipelines only lengthen every
// round trip).
// Dynamic hand-out through per-XCD atomic work queues was measured slower:
// one queue address serves about one ticket per 11-15 ns. Grid-wide barriers
// were measured at 16-76 us each and are not used; the one-launch form's
// single wait is one-directional (workgroups that never wait raise the flag).
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
#if DSPARK_SLOTS32
namespace slots32 {
#else
namespace slots64 {
#endif

constexpr int kFrontThreads = 512;
constexpr int kFusedSelPer = 8;  // survival values per thread of the in-front select
constexpr int kFusedSelMax = kFusedSelPer * kFrontThreads;
constexpr int kFrontRootWGsPerCU = 1;  // root-row workgroups of the front grid per CU
constexpr int kStreamThreads = 512;
// Stream workgroups of 1024 threads from kOneLaunchMinB requests up (there the
// two-launch form serves batch-wide picks): half as many workgroups scan the
// lengths and write the schedule. Measured with back-to-back steps at B = 256:
// the d = 7168 budget workload 64.4 us per step against 64.9 with 512 (mixed
// traffic's budget and combined arms alike); below kOneLaunchMinB requests 512
// stay (B = 64: 25.4-25.5 us with 1024 against 23.0).
constexpr int kStreamThreadsLarge = 1024;
constexpr int kStreamWavesPerCU = 16;  // target waves of the draft-row stream per CU
// The same target for batches below kOneLaunchMinB requests: fewer waves, each
// with a longer run, and every sub-chunk kStreamUnrollShort loads deep whatever
// its length (half the waves need the deeper pipelines to keep as many bytes in
// flight). Measured with back-to-back two-launch steps (gamma = 16, d = 4096,
// V = 151936, mixed traffic with cutoff 0.25 unless stated), against 16 waves
// per CU: B = 32 26.3 us against 27.9; B = 64 37.9 against 39.0; B = 95 50.0
// against 51.6; B = 64 static 61.2 against 63.5; B = 64 with cutoffs in
// [0.1, 0.5] 22.6 against 24.8; B = 64 under a budget of 2.9 per request 30.9
// against 31.7. Six or eight loads deep: 0.3-1.2 us slower. At B = 256 the
// budget arms are 3.4 us slower with 12 waves per CU than with 16, and 12 us
// slower with 8.
constexpr int kStreamWavesPerCUSmall = 8;
constexpr int kStreamUnroll = 2;  // 16-byte loads in flight per lane (more waves, fewer bytes each)
// Root rows of the front kernel: four 16-byte loads in flight per lane when
// they are the front's critical path, three when the GEMV-and-pick chain is (the
// last request workgroup runs the batch-wide pick after the slowest GEMV; a
// request's GEMV reads gamma*d bf16, its root row V). Measured per step: the
// mixed workload's threshold arm 111 us with four against 113-115 with two;
// its budget arm (gamma*d = 65536 < V/2) 68.1 against 70.3, and 66.1-67.0
// with six or eight against 65.4-65.6 with four; the budget workload at
// d = 7168 (gamma*d = 114688 > V/2) 64.7 with three against 65.2-65.4 with
// two and 65.5 with four.
constexpr int kRootUnrollDeep = 4;
// Smallest batch that takes the one-launch form by default. Below it the
// in-grid wait for the lengths costs more than the second launch it saves
// (measured at gamma = 16, d = 4096, V = 151936 with back-to-back steps: two
// launches 14.5 us against 15.2 at B = 1 and 22.6-23.0 against 25.1-27 at
// B = 64 with cutoffs in [0.1, 0.5]; at the boundary, with cutoff 0.25, two
// launches at B = 95 take 50.0 us and one launch at B = 96 49.9 us; one launch
// faster by a few microseconds from B = 128 up).
constexpr int kOneLaunchMinB = 96;
// The one-launch step: 16-byte loads in flight per lane in the GEMV, the root
// rows and the draft rows (its grid holds four waves per SIMD, so deeper
// unrolling costs no occupancy), and the extra draft slots per early wave, as
// a fraction of a root wave's root-row slots: about the root work left when
// the lengths come out. Measured on the mixed workload's threshold arm: draft
// rows four deep 104.7 us per step, two deep 106.2, six or eight deep
// 107.7-109.5; root rows two or eight deep slower than four; a lead of 0.6 to
// 0.8 alike.
constexpr int kOneGemvUnroll = 4;
constexpr int kOneRootUnroll = 4;
constexpr int kOneStreamUnroll = 4;
// Short sub-chunks (at most kShortSub slots) are streamed with four 16-byte
// loads in flight per lane. Measured with back-to-back steps at B = 256
// (sub-chunks of about 3400 slots): the budget arms take 66.9-67.0 us per step
// (mixed traffic, T = 742) and 66.1 us (d = 7168) with four, against 68.3 and
// 67.7 with eight, 67.5 and 65.9 with three, 68.4 and 66.8 with six; steps at
// B = 1 and B = 64 take as long with four as with eight. Once the waves keep
// the memory system full, more loads in flight per wave only lengthen every
// round trip, the finishing waves' included.
constexpr int kStreamUnrollShort = 4;
constexpr int64_t kShortSub = 4096;
// Minimum sub-chunk of the fused step's root and draft rows: 4 KiB of bf16, one
// load round of a wave at four 16-byte loads per lane. Small steps then spread
// their few rows over many waves, each a single round trip (the finishing
// wave reads a row's segment keys in parallel, so more segments cost no
// extra round trips).
constexpr int64_t kStepSubMin = 256;
__device__ __forceinline__ int64_t step_sub_len(int64_t E, int64_t Wt) {
    const int64_t k = udiv64(E + Wt - 1, Wt);
    return k < kStepSubMin ? kStepSubMin : k;
}
constexpr double kLead = 0.70;
constexpr int kRootUnrollShallow = 3;

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
    uint64_t *keys;       // draft segment keys; the request workgroups zero
    int64_t key_words;    // words [0, key_words) of them before any is written
    uint64_t *req_arrivals;  // [B] the stream kernel's per-request counters, zeroed here
    unsigned *arrivals;   // budget select in the front kernel: arrival counter, else NULL
};

// Root rows (dense row b*(gamma+1) of every request b), laid end to end and
// cut into sub-chunks of about equal length, one per root wave: wave w of
// nwaves streams sub-chunks w, w + nwaves, ... and leaves one key per row
// segment at rkeys[s + b]. kCoherent: the keys are read by other workgroups of
// the same grid.
template <bool kVec, int kRootUnroll, bool kCoherent>
__device__ __forceinline__ void front_root_rows(const FrontParams &p, int64_t w, int64_t nwaves) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t Vv = kVec ? (p.V >> 3) : p.V;
    const int64_t E = (int64_t)p.B * Vv;
    const int64_t K = step_sub_len(E, nwaves);
    const int64_t NS = udiv64(E + K - 1, K);
    const size_t row_stride = (size_t)(p.gamma + 1) * (size_t)p.V;
    for (int64_t cur = w; cur < NS; cur += nwaves) {
        int64_t e = cur * K;
        const int64_t e_end = e + K < E ? e + K : E;
        int64_t r = udiv64(e, Vv);
        while (e < e_end) {
            const int64_t row_end = (r + 1) * Vv;
            const int64_t seg_end = e_end < row_end ? e_end : row_end;
            float best = -INFINITY;
            int bidx = -1;
            lane_row_segment<kVec, kRootUnroll>(p.logits + (size_t)r * row_stride, e - r * Vv,
                                                  seg_end - r * Vv, lane, best, bidx);
            uint64_t key = bidx >= 0 ? argmax_key(best, (uint32_t)bidx) : 0ull;
            key = wave_max_u64(key);
            if (lane == 0) {
                if (kCoherent)
                    store_key_coherent(p.rkeys + cur + r, key);
                else
                    p.rkeys[cur + r] = key;
            }
            e = seg_end;
            ++r;
        }
    }
}

// The row segments of root wave w's sub-chunks (as front_root_rows cuts them):
// f(b, n) for each, n slots of request b's root row.
template <typename F>
__device__ __forceinline__ void root_segments(int64_t E, int64_t K, int64_t Vv, int64_t w,
                                              int64_t nwaves, F f) {
    const int64_t NS = udiv64(E + K - 1, K);
    for (int64_t cur = w; cur < NS; cur += nwaves) {
        int64_t e = cur * K;
        const int64_t e_end = e + K < E ? e + K : E;
        int64_t r = udiv64(e, Vv);
        while (e < e_end) {
            const int64_t row_end = (r + 1) * Vv;
            const int64_t seg_end = e_end < row_end ? e_end : row_end;
            f((int)r, seg_end - e);
            e = seg_end;
            ++r;
        }
    }
}

// Confidence scores, survival curve and (threshold, static) verify length of
// request b by the whole workgroup; w_s is the head (LDS or global).
// coherent_surv / coherent_len: survival / the length are read by other
// workgroups of the same grid, so they are written through to the device
// coherence point.
template <bool kVecH, int kGemvU = kGemvUnroll>
__device__ __forceinline__ void front_request(const FrontParams &p, const uint16_t *w_s, int b,
                                              bool coherent_surv, bool coherent_len, float *z_s,
                                              float *p_s, float *s_s) {
    const int tid = threadIdx.x, bd = blockDim.x;
    request_logits<kVecH, kGemvU>(p.hidden + (size_t)b * p.gamma * p.d, w_s, p.bias, p.gamma, p.d,
                                  z_s);
    __syncthreads();
    request_survival(z_s, p.temps, p.gamma, p_s, s_s, p.conf + (size_t)b * p.gamma, nullptr);
    float *surv_b = p.surv + (size_t)b * p.gamma;
    for (int i = tid; i < p.gamma; i += bd) {
        if (coherent_surv)
            __hip_atomic_store(surv_b + i, s_s[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            surv_b[i] = s_s[i];
    }
    if (tid == 0 && (p.mode == DSPARK_CUT_THRESHOLD || p.mode == DSPARK_CUT_STATIC)) {
        const int L = p.mode == DSPARK_CUT_THRESHOLD ? threshold_length(s_s, p.gamma, p.cutoff[b])
                                                     : p.gamma;
        if (coherent_len)
            __hip_atomic_store(p.lengths + b, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            p.lengths[b] = L;
    }
}

// Arrival counter of request b (b < kMaxFusedB) in the per-request counter
// array: consecutive requests 128 bytes apart, so the atomics of different
// requests do not queue on one cache line (a bijection of [0, 4096)).
__device__ __forceinline__ uint64_t *req_counter(uint64_t *base, int b) {
    static_assert(kMaxFusedB == 4096, "the counter spread assumes 4096 counters");
    return base + ((b & 255) << 4) + (b >> 8);
}

// Part i of n of the draft segment keys set to zero by the calling workgroup.
// The stores are device-coherent: a key written later by another workgroup
// (another XCD) must never be overwritten by a zero left in an L2.
__device__ __forceinline__ void zero_key_part(const FrontParams &p, int i, int n) {
    const int64_t c = udiv64(p.key_words + n - 1, n);
    const int64_t hi = (int64_t)(i + 1) * c < p.key_words ? (int64_t)(i + 1) * c : p.key_words;
    for (int64_t k = (int64_t)i * c + threadIdx.x; k < hi; k += blockDim.x)
        __hip_atomic_store(p.keys + k, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Budget / combined: the batch-wide pick over every request's survival (read
// from the device coherence point: other workgroups wrote it) by one
// workgroup; writes every length. sv: LDS for N = B*gamma floats.
__device__ __forceinline__ void front_pick(const FrontParams &p, float *sv, uint32_t *hist,
                                           uint32_t *sh, int *scan_lds) {
    const int tid = threadIdx.x, bd = blockDim.x;
    const int N = p.B * p.gamma;
    __syncthreads();  // sv may alias LDS the workgroup used before
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

// Request workgroups read the head w from global memory (L2): staging it in LDS
// first, one more round trip before the GEMV, measured 0.7 us slower on the
// budget arm of the mixed traffic workload (B = 256, d = 4096) and no faster
// at d = 7168.
template <bool kVecH, bool kVecV, int kRootUnroll, int kGemvU = kGemvUnroll>
__global__ __launch_bounds__(kFrontThreads) void step_front_kernel(FrontParams p) {
    extern __shared__ __align__(16) uint16_t dyn_lds[];
    __shared__ float z_s[DSPARK_MAX_GAMMA], p_s[DSPARK_MAX_GAMMA], s_s[DSPARK_MAX_GAMMA];
    __shared__ uint32_t hist[kSelHistWords], sh[kSelShWords];
    __shared__ int scan_lds[17];
    __shared__ int last_s;
    if ((int)blockIdx.x >= p.B) {
        const int nw = blockDim.x / kWave;
        front_root_rows<kVecV, kRootUnroll, false>(
            p, (int64_t)((int)blockIdx.x - p.B) * nw + threadIdx.x / kWave,
            (int64_t)((int)gridDim.x - p.B) * nw);
        return;
    }
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid == 0)
        __hip_atomic_store(req_counter(p.req_arrivals, b), (uint64_t)0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    zero_key_part(p, b, p.B);
    // the select reads survival from another workgroup of this grid
    const bool select_here = p.arrivals != nullptr;
    front_request<kVecH, kGemvU>(p, p.w, b, select_here, false, z_s, p_s, s_s);
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
    front_pick(p, reinterpret_cast<float *>(dyn_lds), hist, sh, scan_lds);
}

// ----------------------------------------------------------------- stream

struct StreamParams {
    const uint16_t *logits;
    const int32_t *tokens;
    const int32_t *lengths;
    int B, gamma, V;
    int32_t *cu, *ptok, *psrc, *pam, *acc, *bonus;
    uint64_t *keys;         // draft segment keys, keys[s + r] (zero at the start)
    const uint64_t *rkeys;  // root-row keys
    uint64_t *arrivals;     // [B] streamed slots per request (zero between calls)
    int target_waves;       // sub-chunk length: about one sub-chunk per target wave
    int root_waves;         // waves that streamed the root rows
    int deep;               // 1: every draft sub-chunk kStreamUnrollShort loads deep
    unsigned *timed_out;    // sticky: set when a wait for a key gave up
    unsigned long long wait_ticks;  // bound of such a wait, in 100 MHz clock ticks
};

// Largest b in [0, B] with cu[b] - b <= r, i.e. the request that owns draft
// row r (draft rows start at cu[b] - b, which never falls as b rises;
// requests without drafts own none) when 0 <= r < cu[B] - B. A whole wave
// searches: each round the 64 lanes test 64 evenly spaced candidates of the
// remaining range at once (one LDS read and a ballot), so B = 4096 takes
// three rounds instead of twelve dependent reads.
__device__ __forceinline__ int wave_draft_owner(const int *cu, int B, int64_t r) {
    const int lane = threadIdx.x & (kWave - 1);
    int lo = 0, hi = B;  // cu[lo] - lo <= r holds throughout
    while (true) {
        const int step = (hi - lo + kWave) / kWave;  // ceil((hi - lo + 1) / 64)
        const int idx = lo + lane * step;
        const bool ok = idx <= hi && (int64_t)(cu[idx] - idx) <= r;
        const uint64_t m = __ballot(ok);  // lane 0 always set
        const int at = lo + (63 - __clzll((long long)m)) * step;
        if (step == 1) return at;
        lo = at;
        hi = at + step - 1 < hi ? at + step - 1 : hi;
    }
}

// Verify lengths (clamped to [0, gamma]) and cu_seqlens into LDS. Every thread
// calls it. kCoherent: the lengths were written by other workgroups of this
// same grid.
template <bool kCoherent>
__device__ __forceinline__ void lengths_to_lds(const StreamParams &p, int *len_s, int *cu_s,
                                               int *scan_lds) {
    const int B = p.B, g = p.gamma, tid = threadIdx.x, bd = blockDim.x;
    for (int b = tid; b < B; b += bd) {
        const int L = kCoherent ? __hip_atomic_load(const_cast<int32_t *>(p.lengths + b),
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : p.lengths[b];
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
}

// The schedule outputs (cu_seqlens, packed tokens and source rows) of
// requests wg, wg + nwg, ...
__device__ __forceinline__ void write_schedule(const StreamParams &p, const int *len_s,
                                               const int *cu_s, int wg, int nwg) {
    const int g1 = p.gamma + 1, tid = threadIdx.x, bd = blockDim.x;
    for (int b = wg; b < p.B; b += nwg) {
        if (tid == 0) {
            p.cu[b + 1] = cu_s[b + 1];
            if (b == 0) p.cu[0] = 0;
        }
        for (int j = tid; j <= len_s[b]; j += bd) {
            p.ptok[cu_s[b] + j] = p.tokens[(size_t)b * g1 + j];
            p.psrc[cu_s[b] + j] = b * g1 + j;
        }
    }
}

// Counts n more streamed slots of a request on its arrival counter. True on
// the wave whose count reaches `target` (the request's last contribution);
// that wave also returns the counter to zero for the next call. kAfterStores:
// count only once the calling wave's stores are at the coherence point (root
// keys, which are read without a check); draft segment keys need no wait, as
// the finishing wave polls each until it is set. Called by a whole wave.
template <bool kAfterStores>
__device__ __forceinline__ bool arrive_last(uint64_t *cnt, int64_t n, int64_t target) {
    const int lane = threadIdx.x & (kWave - 1);
    if (kAfterStores) __builtin_amdgcn_s_waitcnt(0);
    unsigned long long old = 0;
    if (lane == 0)
        old = __hip_atomic_fetch_add(cnt, (uint64_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, kWave);
    const bool last = (int64_t)old + n == target;
    if (last && lane == 0)
        __hip_atomic_store(cnt, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return last;
}

// Draft segment key at k, as already loaded (x), polled until it is set: its
// wave stores it before it counts its slots, so once a request's count is
// complete every key of it is on its way. A wait beyond wait_ticks sets the
// sticky time-out flag and gives 0 ("no element").
__device__ __forceinline__ uint64_t settled_key(const StreamParams &p, const uint64_t *k,
                                                uint64_t x) {
    if (x != 0) return x;
    const unsigned long long t0 = wall_clock64();
    while ((x = load_key_coherent(k)) == 0) {
        if (wall_clock64() - t0 > p.wait_ticks) {
            __hip_atomic_store(p.timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return x;
}

constexpr int kFinBatch = 8;  // segment keys in flight per lane in the finisher

// Largest segment key of packed draft row r, whose segments are those of
// sub-chunks sf..sl (sub(e): the sub-chunk of slot e), kept at keys[s + r]; the
// calling lane reads segments t0, t0 + Q, ..., kFinBatch loads at a time.
template <typename Sub>
__device__ __forceinline__ uint64_t draft_row_key(const StreamParams &p, int64_t r, int64_t Vv,
                                                  Sub sub, int t0, int Q) {
    const int64_t sf = sub(r * Vv);
    const int64_t cnt = sub((r + 1) * Vv - 1) - sf + 1;
    const uint64_t *base = p.keys + sf + r;
    uint64_t k = 0;
    for (int64_t t = t0; t < cnt; t += (int64_t)kFinBatch * Q) {
        uint64_t x[kFinBatch];
#pragma unroll
        for (int u = 0; u < kFinBatch; ++u) {
            const int64_t tu = t + (int64_t)u * Q;
            x[u] = load_key_coherent(base + (tu < cnt ? tu : t));  // in range; repeats unused
        }
#pragma unroll
        for (int u = 0; u < kFinBatch; ++u)
            if (t + (int64_t)u * Q < cnt) {
                const uint64_t y = settled_key(p, base + t + (int64_t)u * Q, x[u]);
                k = y > k ? y : k;
            }
    }
    return k;
}

// Acceptance and bonus of request b by the calling wave (a whole wave), once
// all its slots are counted: the root row's argmax from its segment keys
// (sub-chunks of Kr slots; kRootCoherent: written by this same grid), each
// draft row's from its segment keys. For requests of fewer than 64 draft rows
// the draft keys, the root keys and the draft tokens are all loaded before any
// is waited for (one memory round trip): Q lanes per draft row (a power of
// two, Q * L <= 64) read the row's segment keys and reduce them by butterfly
// within their group.
// What the finishing wave of request b needs besides the draft keys, loaded
// when a wave starts on the request so that it has arrived by the time the
// wave may finish it: draft token lane + 1 (lanes below L_b) and, with kRoot
// (the root keys are final: written by an earlier launch), each lane's first
// root segment key. kRootCoherent: the root keys were written by this grid.
struct ReqPre {
    uint64_t xr;
    int32_t tk;
};
template <bool kRoot, bool kRootCoherent>
__device__ __forceinline__ ReqPre prefetch_request(const StreamParams &p, int b, int L, int64_t Vv,
                                                   int64_t Kr) {
    const int lane = threadIdx.x & (kWave - 1);
    ReqPre q;
    q.xr = 0;
    q.tk = 0;
    if (kRoot) {
        const int64_t s = udiv64(b * Vv, Kr) + lane;
        if (s <= udiv64((b + 1) * Vv - 1, Kr))
            q.xr = kRootCoherent ? load_key_coherent(p.rkeys + b + s) : p.rkeys[b + s];
    }
    if (lane < L) q.tk = p.tokens[(size_t)b * (p.gamma + 1) + lane + 1];
    return q;
}

template <bool kRootCoherent, bool kPreRoot, typename Sub>
__device__ __forceinline__ void finish_request(const StreamParams &p, const int *len_s,
                                               const int *cu_s, int b, int64_t Vv, int64_t Kr,
                                               Sub sub, const ReqPre &pre) {
    const int lane = threadIdx.x & (kWave - 1);
    const int L = len_s[b];
    const int64_t r0 = cu_s[b] - b;  // first packed draft row of b
    const int32_t *tok = p.tokens + (size_t)b * (p.gamma + 1);
    int32_t *pam_b = p.pam + cu_s[b];
    // root keys: each lane's first one (prefetched, or loaded now and reduced
    // later), then any further ones
    const int64_t s_lo = udiv64(b * Vv, Kr), s_hi = udiv64((b + 1) * Vv - 1, Kr);
    const uint64_t *rk = p.rkeys + b;
    uint64_t xr = pre.xr;
    if (!kPreRoot && s_lo + lane <= s_hi)
        xr = kRootCoherent ? load_key_coherent(rk + s_lo + lane) : rk[s_lo + lane];
    if (L < kWave) {
        const int32_t tk = pre.tk;
        const int lq = L > 0 ? 31 - __builtin_clz(kWave / L) : 6;  // log2 Q
        const int Q = 1 << lq;
        const int j = lane >> lq;
        uint64_t k = j < L ? draft_row_key(p, r0 + j, Vv, sub, lane & (Q - 1), Q) : 0ull;
        for (int64_t s = s_lo + lane + kWave; s <= s_hi; s += kWave) {
            const uint64_t x = kRootCoherent ? load_key_coherent(rk + s) : rk[s];
            xr = x > xr ? x : xr;
        }
        const int32_t root = key_index(wave_max_u64(xr));
        k = group_max_u64(k, lq);
        // lane j >= 1 takes draft row j - 1's key from the first lane of its group
        const uint64_t dk = __shfl(k, lane >= 1 && lane <= L ? (lane - 1) << lq : 0, kWave);
        wave_accept_rows_t([&](int jj) { return jj == 0 ? root : key_index(dk); },
                           [&](int) { return tk; }, L + 1, p.gamma, pam_b, p.acc + b,
                           p.bonus + b);
    } else {
        for (int64_t s = s_lo + lane + kWave; s <= s_hi; s += kWave) {
            const uint64_t x = kRootCoherent ? load_key_coherent(rk + s) : rk[s];
            xr = x > xr ? x : xr;
        }
        const int32_t root = key_index(wave_max_u64(xr));
        wave_accept_rows(
            [&](int jj) {
                return jj == 0 ? root : key_index(draft_row_key(p, r0 + jj - 1, Vv, sub, 0, 1));
            },
            L + 1, p.gamma, tok, pam_b, p.acc + b, p.bonus + b);
    }
}

// Slots [e, e_end) of the draft rows of all requests laid end to end (Vv
// slots per row), streamed by the calling wave as sub-chunk s: each row
// segment leaves its key at keys[s + r] (s + r rises by one at every sub-chunk
// or row boundary, so no two segments share a key, and a row's segments have
// consecutive keys); arrive(b, n) counts the n slots of request b streamed,
// once at each change of request and at the end, with what the request's
// finishing wave needs (prefetch_request<kPreRoot, kRootCoherent>, root
// sub-chunks of Kr slots), loaded when the wave starts on the request.
template <bool kVec, int kUnroll, bool kPreRoot, bool kRootCoherent, typename Arrive>
__device__ __forceinline__ void stream_draft_span(const StreamParams &p, const int *cu_s,
                                                  int64_t Vv, int64_t Kr, int64_t s, int64_t e,
                                                  int64_t e_end, Arrive arrive) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g1 = p.gamma + 1;
    int64_t r = udiv64(e, Vv);
    int cur_b = -1;    // request of the rows being streamed
    int64_t done = 0;  // its slots streamed in this sub-chunk
    ReqPre pre;
    int b = e < e_end ? wave_draft_owner(cu_s, p.B, r) : 0;
    while (e < e_end) {
        const int64_t row_end = (r + 1) * Vv;
        const int64_t seg_end = e_end < row_end ? e_end : row_end;
        while (b < p.B && (int64_t)(cu_s[b + 1] - (b + 1)) <= r) ++b;
        if (b != cur_b) {
            if (cur_b >= 0) arrive(cur_b, done, pre);
            cur_b = b;
            done = 0;
            pre = prefetch_request<kPreRoot, kRootCoherent>(p, b, cu_s[b + 1] - cu_s[b] - 1, Vv, Kr);
        }
        const int64_t src = (int64_t)b * g1 + 1 + (r - (cu_s[b] - b));
        float best = -INFINITY;
        int bidx = -1;
        lane_row_segment<kVec, kUnroll>(p.logits + (size_t)src * (size_t)p.V, e - r * Vv,
                                        seg_end - r * Vv, lane, best, bidx);
        uint64_t key = bidx >= 0 ? argmax_key(best, (uint32_t)bidx) : 0ull;
        key = wave_max_u64(key);
        if (lane == 0) store_key_coherent(p.keys + s + r, key);
        done += seg_end - e;
        e = seg_end;
        ++r;
    }
    if (cur_b >= 0) arrive(cur_b, done, pre);
}

// The draft rows (E slots) in sub-chunks of K slots dealt cyclically: wave w
// of W streams sub-chunks w, w + W, ... Long contiguous runs per wave keep the
// HBM row buffers better used than many short interleaved ones.
template <bool kVec, typename Arrive>
__device__ __forceinline__ void stream_draft_rows(const StreamParams &p, const int *cu_s,
                                                  int64_t Vv, int64_t Kr, int64_t E, int64_t K,
                                                  int64_t w, int64_t W, Arrive arrive) {
    const int64_t NS = udiv64(E + K - 1, K);
    for (int64_t cur = w; cur < NS; cur += W) {
        const int64_t e0 = cur * K, e1 = cur * K + K < E ? cur * K + K : E;
        if (K <= kShortSub || p.deep)
            stream_draft_span<kVec, kStreamUnrollShort, true, false>(p, cu_s, Vv, Kr, cur, e0, e1,
                                                                     arrive);
        else
            stream_draft_span<kVec, kStreamUnroll, true, false>(p, cu_s, Vv, Kr, cur, e0, e1,
                                                                arrive);
    }
}

template <bool kVec, int kThreads>
__global__ __launch_bounds__(kThreads) void step_stream_kernel(StreamParams p) {
    extern __shared__ int smem[];
    int *len_s = smem;          // [B]
    int *cu_s = smem + p.B;     // [B + 1]
    __shared__ int scan_lds[17];
    const int B = p.B, tid = threadIdx.x, nw = blockDim.x / kWave;

    // schedule: lengths (clamped), cu_seqlens in LDS, this workgroup's outputs
    lengths_to_lds<false>(p, len_s, cu_s, scan_lds);
    write_schedule(p, len_s, cu_s, blockIdx.x, gridDim.x);

    const int64_t Vv = kVec ? (p.V >> 3) : p.V;
    const int64_t E = (int64_t)(cu_s[B] - B) * Vv;
    const int64_t K = step_sub_len(E, p.target_waves);
    const int64_t Kr = step_sub_len((int64_t)B * Vv, p.root_waves);
    auto sub = [&](int64_t e) { return udiv64(e, K); };
    // requests without draft rows are finished first, by the first wave of the
    // workgroup that owns them (finishing them after that wave's stream
    // measured no faster)
    if (tid < kWave)
        for (int b = blockIdx.x; b < B; b += gridDim.x)
            if (len_s[b] == 0)
                finish_request<false, true>(p, len_s, cu_s, b, Vv, Kr, sub,
                                            prefetch_request<true, false>(p, b, 0, Vv, Kr));
    // the wave that completes a request's draft rows finishes it
    stream_draft_rows<kVec>(p, cu_s, Vv, Kr, E, K, (int64_t)blockIdx.x * nw + tid / kWave,
                            (int64_t)gridDim.x * nw, [&](int b, int64_t n, const ReqPre &pre) {
                                if (arrive_last<false>(req_counter(p.arrivals, b), n,
                                                       (int64_t)len_s[b] * Vv))
                                    finish_request<false, true>(p, len_s, cu_s, b, Vv, Kr, sub,
                                                                pre);
                            });
}

// ---------------------------------------------------------------- one launch

// The whole step in one grid (threshold and static cuts, whose lengths need
// no batch-wide pick) of three kinds of workgroup, in this order: request
// workgroups (the GEMV, survival and length of requests g, g + gemv_wgs, ...),
// root workgroups (the root rows, while the GEMV runs) and, when the draft
// stream wants more waves, plain stream workgroups. Once every length is
// final, all of them stream the draft rows. The only wait is for the lengths,
// which only request workgroups write; they come first in the grid and never
// wait before their lengths are out, and the grid is sized to be resident at
// once, so they all run.
//
// The go word: the last request workgroup to finish adds the grid size G to
// it once every length is at the coherence point, and every workgroup takes
// one off exactly once, when it leaves. Before the add the word is at most
// zero; after it, it stays positive until the last workgroup has left, and it
// is zero again at the end of every call. Waiters go on when it is positive.
// The wait is bounded: a workgroup that gives up sets the sticky time-out
// flag, takes its one off and leaves (the outputs of that call are then
// undefined). Each request workgroup also returns its requests' arrival
// counters to zero before it counts itself done, so a call that gave up leaves
// nothing behind that could disturb the next one.
struct OneParams {
    FrontParams f;
    StreamParams s;
    unsigned *gemv_done;  // request workgroups done (zero between calls)
    int *go;              // see above (zero between calls)
    unsigned *timed_out;  // sticky: set when a workgroup gave up waiting for the lengths
    unsigned long long wait_ticks;  // bound of the wait, in 100 MHz clock ticks
    int gemv_wgs, root_wgs;
    int64_t lead;         // draft slots more per early wave than per root wave
};

// The draft rows of the one-launch step, laid end to end (E slots), as one
// sub-chunk per wave in two regions: the first NA sub-chunks, of KA slots, go
// to the early waves (request and plain stream workgroups, free once the
// lengths are final), the others, of KB = KA - lead slots, to the root-row
// waves, which reach the drafts later. When the root waves' share would be
// below the minimum length, the early waves take no more than covers the
// drafts (at least the minimum, at most the minimum plus the lead): a longer
// sub-chunk would only lengthen their chains.
struct SplitLayout {
    int64_t KA, KB, EA, NA, E;
    __device__ __forceinline__ SplitLayout(int64_t E_, int64_t WA, int64_t W, int64_t lead) {
        E = E_;
        const int64_t kb = (E - WA * lead + W - 1) / W;
        if (kb < kStepSubMin) {
            KB = kStepSubMin;
            const int64_t ka = udiv64(E + WA - 1, WA);
            KA = ka < kStepSubMin ? kStepSubMin : (ka > kStepSubMin + lead ? kStepSubMin + lead : ka);
        } else {
            KB = kb;
            KA = KB + lead;
        }
        EA = WA * KA < E ? WA * KA : E;
        NA = udiv64(EA + KA - 1, KA);
    }
    // sub-chunk of slot e < E
    __device__ __forceinline__ int64_t sub(int64_t e) const {
        return e < EA ? udiv64(e, KA) : NA + udiv64(e - EA, KB);
    }
    // slots of sub-chunk s: [*e0, *e1), empty past the end
    __device__ __forceinline__ void span(int64_t s, int64_t *e0, int64_t *e1) const {
        int64_t a, b;
        if (s < NA) {
            a = s * KA;
            b = a + KA < EA ? a + KA : EA;
        } else {
            a = EA + (s - NA) * KB;
            b = a + KB < E ? a + KB : E;
        }
        *e0 = a < E ? a : E;
        *e1 = b;
    }
};

// Default bound of the wait for the lengths in ticks of the 100 MHz constant
// clock (1 s; the lengths normally follow the slowest GEMV by microseconds).
constexpr unsigned long long kWaitTicks = 100000000ull;

// The head w is read from global memory (L2-resident after the first
// workgroups), not staged in LDS: the GEMV then starts without a staging round
// trip and barrier (measured 1-1.5 us faster per step).
template <bool kVecH, bool kVecV>
__global__ __launch_bounds__(kFrontThreads) void step_one_kernel(OneParams q) {
    extern __shared__ __align__(16) uint16_t dyn_lds[];
    __shared__ float z_s[DSPARK_MAX_GAMMA], p_s[DSPARK_MAX_GAMMA], s_s[DSPARK_MAX_GAMMA];
    __shared__ int scan_lds[17];
    __shared__ int last_s, ok_s;
    const FrontParams &p = q.f;
    const StreamParams &sp = q.s;
    const int tid = threadIdx.x, nw = blockDim.x / kWave, wave = tid / kWave;
    const int wg = blockIdx.x, G = gridDim.x, B = p.B;
    const int64_t Vv = kVecV ? (p.V >> 3) : p.V;
    const int64_t root_waves = (int64_t)q.root_wgs * nw;
    const bool is_root = wg >= q.gemv_wgs && wg < q.gemv_wgs + q.root_wgs;
    bool wait = true;
    if (wg < q.gemv_wgs) {
        zero_key_part(p, wg, q.gemv_wgs);
        for (int b = wg; b < B; b += q.gemv_wgs) {
            // the request's arrival counter starts this call at zero (streaming
            // waves only add to it after the go word)
            if (tid == 0)
                __hip_atomic_store(req_counter(sp.arrivals, b), (uint64_t)0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            front_request<kVecH, kOneGemvUnroll>(p, p.w, b, false, true, z_s, p_s, s_s);
            __syncthreads();
        }
        // this workgroup's length, counter and key stores are at the
        // coherence point: count it; the last to count lets every workgroup go
        // on
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const int last = __hip_atomic_fetch_add(q.gemv_done, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT) ==
                             (unsigned)(q.gemv_wgs - 1);
            if (last) {
                __hip_atomic_store(q.gemv_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_add(q.go, G, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            last_s = last;
        }
        __syncthreads();
        wait = !last_s;
    } else if (is_root) {
        front_root_rows<kVecV, kOneRootUnroll, true>(p, (int64_t)(wg - q.gemv_wgs) * nw + wave,
                                                     root_waves);
    }
    if (wait) {
        if (tid == 0) {
            const unsigned long long t0 = wall_clock64();
            int ok = 1;
            while (__hip_atomic_load(q.go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= 0) {
                if (wall_clock64() - t0 > q.wait_ticks) {
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            if (!ok) {
                __hip_atomic_store(q.timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_sub(q.go, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            ok_s = ok;
        }
        __syncthreads();
        if (!ok_s) return;
    }

    // every length is final: the schedule in LDS and this workgroup's outputs
    int *len_s = reinterpret_cast<int *>(dyn_lds);
    int *cu_s = len_s + B;
    lengths_to_lds<true>(sp, len_s, cu_s, scan_lds);
    write_schedule(sp, len_s, cu_s, wg, G);
    // draft waves: the early ones (request and plain stream workgroups) first
    const int64_t WA = (int64_t)(G - q.root_wgs) * nw;
    const int64_t dw = is_root ? WA + (int64_t)(wg - q.gemv_wgs) * nw + wave
                               : (int64_t)(wg < q.gemv_wgs ? wg : wg - q.root_wgs) * nw + wave;
    const SplitLayout lay((int64_t)(cu_s[B] - B) * Vv, WA, (int64_t)G * nw, q.lead);
    const int64_t Kr = step_sub_len((int64_t)B * Vv, root_waves);
    // a request counts its root row and its draft rows; the wave that brings
    // the last of them finishes it: the root row's argmax from the root keys,
    // the draft rows' from the draft keys
    auto sub = [&](int64_t e) { return lay.sub(e); };
    auto arrive_root = [&](int b, int64_t n) {
        if (arrive_last<true>(req_counter(sp.arrivals, b), n, (int64_t)(len_s[b] + 1) * Vv))
            finish_request<true, false>(sp, len_s, cu_s, b, Vv, Kr, sub,
                                        prefetch_request<false, true>(sp, b, len_s[b], Vv, Kr));
    };
    // the root keys are final only once the request's count is complete: the
    // draft waves prefetch the tokens only
    auto arrive = [&](int b, int64_t n, const ReqPre &pre) {
        if (arrive_last<false>(req_counter(sp.arrivals, b), n, (int64_t)(len_s[b] + 1) * Vv))
            finish_request<true, false>(sp, len_s, cu_s, b, Vv, Kr, sub, pre);
    };
    if (is_root)
        root_segments((int64_t)B * Vv, Kr, Vv, (int64_t)(wg - q.gemv_wgs) * nw + wave, root_waves,
                      arrive_root);
    // this wave's sub-chunk: early wave dw < WA takes region A's sub-chunk dw,
    // root wave dw takes region B's sub-chunk dw - WA
    const int64_t s_mine = dw < WA ? (dw < lay.NA ? dw : -1) : lay.NA + (dw - WA);
    if (s_mine >= 0) {
        int64_t e0, e1;
        lay.span(s_mine, &e0, &e1);
        if (e1 - e0 > 0 && e1 - e0 <= kShortSub)
            stream_draft_span<kVecV, kStreamUnrollShort, false, true>(sp, cu_s, Vv, Kr, s_mine, e0,
                                                                      e1, arrive);
        else if (e0 < e1)
            stream_draft_span<kVecV, kOneStreamUnroll, false, true>(sp, cu_s, Vv, Kr, s_mine, e0,
                                                                    e1, arrive);
    }
    // every wave of this workgroup is past the wait: it leaves
    if (tid == 0) __hip_atomic_fetch_sub(q.go, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- launch

template <bool kVec, int kThreads>
static int stream_grid(size_t lds) {
    // resident workgroups of the stream kernel for this LDS size, cached per
    // device and 4 KiB LDS bucket (per instantiation)
    static std::atomic<int> cache[64][13];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    const int bucket = (int)((lds + 4095) / 4096);
    int gsz = cache[dev][bucket].load(std::memory_order_relaxed);
    if (gsz > 0) return gsz;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, step_stream_kernel<kVec, kThreads>,
                                                     kThreads, (size_t)bucket * 4096) !=
            hipSuccess ||
        blocks < 1)
        blocks = 1;
    gsz = blocks * device_cu_count();
    cache[dev][bucket].store(gsz, std::memory_order_relaxed);
    return gsz;
}

// Front grids of at most one workgroup per CU (small batches) take eight
// 16-byte hidden loads in flight per lane: a request's GEMV is then one load
// round per wave. Their occupancy (three waves per SIMD) still holds one
// workgroup per CU.
constexpr int kGemvUnrollSmall = 8;

template <bool kVecV, int kRootUnroll>
static void launch_front_u(bool hvec, const FrontParams &fp, int root_wgs, size_t lds,
                           hipStream_t s) {
    const dim3 grid(fp.B + root_wgs), block(kFrontThreads);
    if (hvec && fp.B + root_wgs <= device_cu_count())
        hipLaunchKernelGGL((step_front_kernel<true, kVecV, kRootUnroll, kGemvUnrollSmall>), grid,
                           block, lds, s, fp);
    else if (hvec)
        hipLaunchKernelGGL((step_front_kernel<true, kVecV, kRootUnroll>), grid, block, lds, s, fp);
    else
        hipLaunchKernelGGL((step_front_kernel<false, kVecV, kRootUnroll>), grid, block, lds, s, fp);
}

template <bool kVecV>
static void launch_front(bool hvec, const FrontParams &fp, int root_wgs, size_t lds,
                         hipStream_t s) {
    const bool gemv_critical =
        fp.arrivals != nullptr && (int64_t)fp.gamma * fp.d * 2 > (int64_t)fp.V;
    if (gemv_critical)
        launch_front_u<kVecV, kRootUnrollShallow>(hvec, fp, root_wgs, lds, s);
    else
        launch_front_u<kVecV, kRootUnrollDeep>(hvec, fp, root_wgs, lds, s);
}

template <bool kVecH, bool kVecV>
static int one_capacity(size_t lds) {
    // workgroups of the one-launch kernel resident at once for this LDS size,
    // cached per device and 4 KiB LDS bucket
    static std::atomic<int> cache[64][16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    const int bucket = (int)((lds + 4095) / 4096);
    if (bucket >= 16) return 0;
    int cap = cache[dev][bucket].load(std::memory_order_relaxed);
    if (cap > 0) return cap;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, step_one_kernel<kVecH, kVecV>,
                                                     kFrontThreads, (size_t)bucket * 4096) !=
            hipSuccess ||
        blocks < 0)
        blocks = 0;
    cap = blocks * device_cu_count();
    if (cap > 0) cache[dev][bucket].store(cap, std::memory_order_relaxed);
    return cap;
}

// Launches the one-launch step when its whole grid fits on the device at once;
// *done tells whether it did.
template <bool kVecH, bool kVecV>
static hipError_t launch_one_v(const OneParams &q, int grid, size_t lds, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop, bool *done) {
    *done = false;
    if (grid > one_capacity<kVecH, kVecV>(lds)) return hipSuccess;
    hipError_t e;
    if (ev_start && (e = hipEventRecord(ev_start, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((step_one_kernel<kVecH, kVecV>), dim3(grid), dim3(kFrontThreads), lds, s,
                       q);
    e = hipGetLastError();
    if (e == hipSuccess && ev_stop) e = hipEventRecord(ev_stop, s);
    *done = e == hipSuccess;
    return e;
}

hipError_t launch_fused_step(const uint16_t *hidden, const uint16_t *w, float bias,
                             const float *temps, const int32_t *tokens, const uint16_t *logits,
                             int B, int gamma, int d, int V, int mode, const float *cutoff,
                             long long budget, float *conf, float *surv, int32_t *lengths,
                             int32_t *cu, int32_t *ptok, int32_t *psrc, int32_t *pam,
                             int32_t *acc, int32_t *bonus, void *ws, hipStream_t s,
                             hipEvent_t ev_start, hipEvent_t ev_stop, int launches,
                             unsigned long long wait_ticks) {
    if (B > kMaxFusedB) return hipErrorNotSupported;
    char *wsb = static_cast<char *>(ws);
    uint64_t *keys = reinterpret_cast<uint64_t *>(wsb + ws_keys_offset());
    uint64_t *rkeys = reinterpret_cast<uint64_t *>(wsb + ws_rkeys_offset(B, gamma));
    uint64_t *rcnt = reinterpret_cast<uint64_t *>(wsb + ws_rcnt_offset());
    unsigned *arrivals = reinterpret_cast<unsigned *>(wsb + ws_ctrl_offset());

    const int N = B * gamma;
    const bool hvec = (d % 8 == 0) && (((uintptr_t)hidden | (uintptr_t)w) % 16 == 0);
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
    fp.keys = keys;
    fp.req_arrivals = rcnt;
    fp.arrivals = select_in_front ? arrivals : nullptr;
    const size_t front_lds = select_in_front ? (size_t)N * 4 : 0;  // the pick's survival values
    // root-row workgroups: a fixed share of the chip, but no more than the
    // root rows fill with minimum-length sub-chunks
    const int cus = device_cu_count();
    const int64_t Vv = vvec ? V / 8 : V;
    const int64_t root_min_wgs =
        ((int64_t)B * Vv + kStepSubMin * (kFrontThreads / kWave) - 1) /
        (kStepSubMin * (kFrontThreads / kWave));
    int64_t root_wgs = (int64_t)kFrontRootWGsPerCU * cus;
    root_wgs = root_wgs < root_min_wgs ? root_wgs : root_min_wgs;
    // small batches keep the whole front grid at one workgroup per CU, where
    // the front takes its small-grid variant
    if (2 * B <= cus && root_wgs > cus - B) root_wgs = cus - B;
    if (root_wgs * (kFrontThreads / kWave) > kMaxWaves) root_wgs = kMaxWaves / (kFrontThreads / kWave);
    root_wgs = root_wgs < 1 ? 1 : root_wgs;
    const int root_waves = (int)root_wgs * (kFrontThreads / kWave);

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
    const int wpc = B < kOneLaunchMinB ? kStreamWavesPerCUSmall : kStreamWavesPerCU;
    p.target_waves = wpc * cus < kMaxWaves ? wpc * cus : (int)kMaxWaves;
    p.root_waves = root_waves;
    p.deep = B < kOneLaunchMinB ? 1 : 0;
    p.timed_out = reinterpret_cast<unsigned *>(wsb + ws_ctrl_offset() + kCtrlTimedOutOffset);
    p.wait_ticks = wait_ticks ? wait_ticks : kWaitTicks;
    // draft segment keys in use: keys[s + r] with s below the sub-chunk count
    // (at most the target waves) and r below the draft rows (B * gamma)
    fp.key_words = (int64_t)p.target_waves + (int64_t)B * gamma;
    // stream workgroups (of `threads`; 512-thread workgroups for the one-launch
    // grid): enough for the target waves, and no more than the largest possible
    // draft rows (every request at gamma) fill with minimum-length sub-chunks
    const int64_t max_sub = ((int64_t)B * gamma * Vv + kStepSubMin - 1) / kStepSubMin;
    auto wgs_needed = [&](int threads) {
        const int wpw = threads / kWave;
        int n = (p.target_waves + wpw - 1) / wpw;
        const int64_t max_wgs = (max_sub + wpw - 1) / wpw;
        if (max_wgs < n) n = max_wgs < 1 ? 1 : (int)max_wgs;
        return n;
    };
    const int stream_wgs_needed = wgs_needed(kFrontThreads);

    // one launch (threshold and static cuts, batches from kOneLaunchMinB):
    // request workgroups (one per CU at most, each looping over its requests),
    // the root workgroups, and plain stream workgroups up to the stream's
    // target, when the whole grid is resident at once and its waves fit the
    // key layout
    if ((mode == DSPARK_CUT_THRESHOLD || mode == DSPARK_CUT_STATIC) && launches != 2 &&
        (B >= kOneLaunchMinB || launches == 1)) {
        OneParams q;
        q.f = fp;
        q.s = p;
        q.gemv_done = arrivals;
        q.go = reinterpret_cast<int *>(wsb + ws_ctrl_offset() + kCtrlGoOffset);
        q.timed_out = reinterpret_cast<unsigned *>(wsb + ws_ctrl_offset() + kCtrlTimedOutOffset);
        q.wait_ticks = wait_ticks ? wait_ticks : kWaitTicks;
        q.gemv_wgs = B < cus ? B : cus;
        q.root_wgs = (int)root_wgs;
        q.lead = (int64_t)(kLead * (double)((int64_t)B * Vv / root_waves));
        int grid = q.gemv_wgs + q.root_wgs;
        if (grid < stream_wgs_needed) grid = stream_wgs_needed;
        // one sub-chunk per wave of the grid
        q.f.key_words = (int64_t)grid * (kFrontThreads / kWave) + (int64_t)B * gamma;
        const size_t lds = (size_t)(2 * B + 1) * 4;
        if ((int64_t)grid * (kFrontThreads / kWave) <= kMaxWaves) {
            bool done = false;
            hipError_t e;
            if (hvec)
                e = vvec ? launch_one_v<true, true>(q, grid, lds, s, ev_start, ev_stop, &done)
                         : launch_one_v<true, false>(q, grid, lds, s, ev_start, ev_stop, &done);
            else
                e = vvec ? launch_one_v<false, true>(q, grid, lds, s, ev_start, ev_stop, &done)
                         : launch_one_v<false, false>(q, grid, lds, s, ev_start, ev_stop, &done);
            if (e != hipSuccess || done) return e;
        }
    }

    if (vvec)
        launch_front<true>(hvec, fp, (int)root_wgs, front_lds, s);
    else
        launch_front<false>(hvec, fp, (int)root_wgs, front_lds, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    if ((mode == DSPARK_CUT_BUDGET || mode == DSPARK_CUT_COMBINED) && !select_in_front) {
        e = launch_schedule(surv, B, gamma, mode, cutoff, budget, lengths, s);
        if (e != hipSuccess) return e;
    }

    const size_t lds = (size_t)(2 * B + 1) * sizeof(int);
    const bool large = B >= kOneLaunchMinB;
    int g = large ? (vvec ? stream_grid<true, kStreamThreadsLarge>(lds)
                          : stream_grid<false, kStreamThreadsLarge>(lds))
                  : (vvec ? stream_grid<true, kStreamThreads>(lds)
                          : stream_grid<false, kStreamThreads>(lds));
    const int g_need = wgs_needed(large ? kStreamThreadsLarge : kStreamThreads);
    g = g < g_need ? g : g_need;
    // measurement events bracket the dominant kernel (the draft-row stream)
    if (ev_start && (e = hipEventRecord(ev_start, s)) != hipSuccess) return e;
    if (large && vvec)
        hipLaunchKernelGGL((step_stream_kernel<true, kStreamThreadsLarge>), dim3(g),
                           dim3(kStreamThreadsLarge), lds, s, p);
    else if (large)
        hipLaunchKernelGGL((step_stream_kernel<false, kStreamThreadsLarge>), dim3(g),
                           dim3(kStreamThreadsLarge), lds, s, p);
    else if (vvec)
        hipLaunchKernelGGL((step_stream_kernel<true, kStreamThreads>), dim3(g),
                           dim3(kStreamThreads), lds, s, p);
    else
        hipLaunchKernelGGL((step_stream_kernel<false, kStreamThreads>), dim3(g),
                           dim3(kStreamThreads), lds, s, p);
    e = hipGetLastError();
    if (e == hipSuccess && ev_stop) e = hipEventRecord(ev_stop, s);
    return e;
}

}  // namespace slots32 / slots64
}  // namespace dspark
