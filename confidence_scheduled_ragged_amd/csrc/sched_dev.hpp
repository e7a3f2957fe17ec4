// sched_dev.hpp - verify-length cut (per-request threshold or batch budget)
// and the block-wide scan used by compaction, as device functions.
//
// [P1] "DFlash to DSpark in SGLang": the per-request cut of section "The
// confidence scheduler and verify modes" (a request's window grows while the
// survival at the next position is worth its per-token cost) and the batch-wide
// verify-length top-k schedule of section "Zero-overhead scheduling and
// kernels"; [P2] contrasts the dynamic budget with a fixed one.
#pragma once

#include "common.hpp"

namespace dspark {

// Order-preserving unsigned image of a float (-0 folded onto +0).
__device__ __forceinline__ uint32_t ordered_f32(float v) { return ordered_bits(v); }

// Exclusive scan of one int per thread across the block (blockDim.x a multiple
// of 64, at most 1024). lds needs 17 ints. Returns the exclusive prefix and
// writes the block total to *total. Contains barriers: call from every thread.
__device__ __forceinline__ int block_excl_scan(int x, int *total, int *lds) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    int inc = wave_incl_scan(x, lane);
    if (lane == kWave - 1) lds[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        int t = lane < nw ? lds[lane] : 0;
        int ti = wave_incl_scan(t, lane);
        if (lane < nw) lds[lane] = ti - t;
        if (lane == nw - 1) lds[16] = ti;
    }
    __syncthreads();
    int r = inc - x + lds[wave];
    *total = lds[16];
    __syncthreads();
    return r;
}

// Survival of flat position f as the budget ranks it. With per-request
// cutoffs (the combined cut) a position below its request's cutoff ranks below
// every eligible one (-inf); without, the survival itself.
__device__ __forceinline__ float ranked_value(const float *__restrict__ surv,
                                              const float *__restrict__ cutoff, int gamma,
                                              int f) {
    const float v = surv[f];
    return (cutoff && !(v >= cutoff[f / gamma])) ? -INFINITY : v;
}

// Number of positions of [0, N) that pass their request's cutoff, summed over
// the block (every thread calls it and gets the total). lds needs 17 ints.
__device__ __forceinline__ int block_count_eligible(const float *__restrict__ surv,
                                                    const float *__restrict__ cutoff, int gamma,
                                                    int N, int *lds) {
    int n = 0;
    for (int f = threadIdx.x; f < N; f += blockDim.x) n += surv[f] >= cutoff[f / gamma] ? 1 : 0;
    int total;
    block_excl_scan(n, &total, lds);
    return total;
}

// Threshold cut of one request: number of positions with survival >= c.
// A NaN c makes every comparison false.
__device__ __forceinline__ int threshold_length(const float *s, int gamma, float c) {
    int n = 0;
    for (int k = 0; k < gamma; ++k) n += (s[k] >= c) ? 1 : 0;
    return n;
}

// Batch budget. Finds the t-th largest survival value tau over all
// N = B*gamma positions (1 <= t < N) by an MSB-first radix select on the
// order-preserving bits, 8 bits per pass, and the number `need` of positions
// equal to tau that fall inside the top t (the ties are taken in flat index
// order, i.e. lower request first, then lower position). Every thread of the
// block calls it; the result is returned to every thread.
struct BudgetCut {
    uint32_t tau;  // ordered bits of the t-th largest value
    int need;      // picks among positions whose value equals tau
};

constexpr int kSelCache = 8;  // values cached per thread between passes

__device__ __forceinline__ BudgetCut budget_select(const float *__restrict__ surv,
                                                   const float *__restrict__ cutoff, int gamma,
                                                   int N, int t, uint32_t *hist /*256*/,
                                                   uint32_t *sh /*2*/) {
    const int tid = threadIdx.x;
    const int bd = blockDim.x;
    const int lane = tid & (kWave - 1);
    uint32_t cache[kSelCache];
#pragma unroll
    for (int j = 0; j < kSelCache; ++j) {
        int f = tid + j * bd;
        cache[j] = f < N ? ordered_f32(ranked_value(surv, cutoff, gamma, f)) : 0u;
    }
    uint32_t prefix = 0, mask = 0;
    uint32_t remaining = (uint32_t)t;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += bd) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSelCache; ++j) {
            int f = tid + j * bd;
            uint32_t u = cache[j];
            if (f < N && (u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        for (int f = tid + kSelCache * bd; f < N; f += bd) {
            uint32_t u = ordered_f32(ranked_value(surv, cutoff, gamma, f));
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l owns digits 255-4l .. 252-4l (descending)
            uint32_t c[4];
            uint32_t tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = hist[255 - 4 * lane - q];
                tot += c[q];
            }
            int inc = wave_incl_scan((int)tot, lane);
            uint32_t cum = (uint32_t)inc - tot;  // count in higher digits
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cum < remaining && remaining <= cum + c[q]) {
                    sh[0] = prefix | ((uint32_t)(255 - 4 * lane - q) << shift);
                    sh[1] = remaining - cum;
                }
                cum += c[q];
            }
        }
        __syncthreads();
        prefix = sh[0];
        remaining = sh[1];
        mask |= 0xFFu << shift;
        __syncthreads();
    }
    (void)lane;
    BudgetCut r;
    r.tau = prefix;
    r.need = (int)remaining;
    return r;
}

// Budget select for the fused step: the same radix select as budget_select,
// but each thread holds a contiguous run of up to kPer flat positions in
// registers (N <= kPer * blockDim.x). Neighbouring positions of one request
// have non-increasing survival, so their digits often repeat; equal digits of
// consecutive positions are counted once per run. Neighbouring threads still
// share digits (most survival values of a batch share their top bits), so each
// pass counts into kSelCopies copies of the histogram, picked by thread index,
// padded to fall in different LDS banks: same-address atomics of one
// instruction drop eightfold. Two histogram buffers alternate between passes;
// a pass clears the one it does not use (last read by the previous pass's
// scan), so a pass needs two barriers: after the counts, and after the digit
// is chosen. Once the chosen digit's bin holds at most kSelDirect values
// (usually after two passes: survival values spread over many binades), they
// are gathered and one wave ranks them directly instead of two more passes.
constexpr int kSelCopies = 8;
constexpr int kSelBinsPad = 257;
constexpr int kSelHistWords = 2 * kSelCopies * kSelBinsPad;
constexpr int kSelDirect = 64;
constexpr int kSelShWords = 8;

template <int kPer>
__device__ __forceinline__ BudgetCut budget_select_runs(const float *__restrict__ surv, int N, int t,
                                                        uint32_t *hist /*kSelHistWords*/,
                                                        uint32_t *sh /*kSelShWords*/) {
    const int tid = threadIdx.x;
    const int bd = blockDim.x;
    const int lane = tid & (kWave - 1);
    const int per = (N + bd - 1) / bd;
    const int f0 = tid * per;
    const int copy = (tid & (kSelCopies - 1)) * kSelBinsPad;
    uint32_t v[kPer];
    int nv = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int f = f0 + j;
        const bool ok = j < per && f < N;
        v[j] = ok ? ordered_f32(surv[f]) : 0u;
        nv += ok ? 1 : 0;
    }
    for (int i = tid; i < kSelHistWords; i += bd) hist[i] = 0;
    __syncthreads();
    uint32_t prefix = 0, mask = 0;
    uint32_t remaining = (uint32_t)t;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        uint32_t *h = hist + (pass & 1) * (kSelCopies * kSelBinsPad);
        if (pass >= 1 && pass < 3) {
            uint32_t *o = hist + ((pass + 1) & 1) * (kSelCopies * kSelBinsPad);
            for (int i = tid; i < kSelCopies * kSelBinsPad; i += bd) o[i] = 0;
        }
        uint32_t cur = 0xFFFFFFFFu, run = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (j < nv && (v[j] & mask) == prefix) {
                const uint32_t dg = (v[j] >> shift) & 255u;
                if (dg == cur) {
                    ++run;
                } else {
                    if (run) atomicAdd(&h[copy + cur], run);
                    cur = dg;
                    run = 1;
                }
            }
        }
        if (run) atomicAdd(&h[copy + cur], run);
        __syncthreads();
        if (tid < kWave) {
            // lane l owns digits 255-4l .. 252-4l (descending), summed over the copies
            uint32_t c[4];
            uint32_t tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int dg = 255 - 4 * lane - q;
                uint32_t n = 0;
#pragma unroll
                for (int k = 0; k < kSelCopies; ++k) n += h[k * kSelBinsPad + dg];
                c[q] = n;
                tot += n;
            }
            const int inc = wave_incl_scan((int)tot, lane);
            uint32_t cum = (uint32_t)inc - tot;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cum < remaining && remaining <= cum + c[q]) {
                    sh[4 * (pass & 1)] = prefix | ((uint32_t)(255 - 4 * lane - q) << shift);
                    sh[4 * (pass & 1) + 1] = remaining - cum;
                    sh[4 * (pass & 1) + 2] = c[q];
                }
                cum += c[q];
            }
        }
        __syncthreads();
        // the choice of this pass sits in its own words, so the next pass may
        // overwrite the other set before every thread has read this one
        prefix = sh[4 * (pass & 1)];
        remaining = sh[4 * (pass & 1) + 1];
        const uint32_t in_bin = sh[4 * (pass & 1) + 2];
        mask |= 0xFFu << shift;
        if (pass < 3 && in_bin <= (uint32_t)kSelDirect) {
            // the values sharing the prefix, gathered into the other (zeroed)
            // histogram buffer: word 0 counts, words 1.. hold them
            uint32_t *o = hist + ((pass + 1) & 1) * (kSelCopies * kSelBinsPad);
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                if (j < nv && (v[j] & mask) == prefix) {
                    const uint32_t at = atomicAdd(&o[0], 1u);
                    if (at < (uint32_t)kSelDirect) o[1 + at] = v[j];
                }
            }
            __syncthreads();
            if (tid < kWave) {
                // lane l ranks candidate l: the remaining-th largest is the value
                // with fewer than `remaining` candidates above it and at least
                // `remaining` at or above it
                const int n = (int)in_bin;
                const uint32_t u = lane < n ? o[1 + lane] : 0u;
                int gt = 0, ge = 0;
                for (int m = 0; m < n; ++m) {
                    const uint32_t w = o[1 + m];
                    gt += w > u ? 1 : 0;
                    ge += w >= u ? 1 : 0;
                }
                if (lane < n && (uint32_t)gt < remaining && remaining <= (uint32_t)ge) {
                    sh[4 * ((pass + 1) & 1)] = u;
                    sh[4 * ((pass + 1) & 1) + 1] = remaining - (uint32_t)gt;
                }
            }
            __syncthreads();
            BudgetCut r;
            r.tau = sh[4 * ((pass + 1) & 1)];
            r.need = (int)sh[4 * ((pass + 1) & 1) + 1];
            return r;
        }
    }
    BudgetCut r;
    r.tau = prefix;
    r.need = (int)remaining;
    return r;
}

// Lengths from a budget cut for requests [0, B): L_b = #{v > tau} + the
// request's share of the `need` tied picks, handed out in request order.
// Values are ranked as budget_select ranks them (cutoff nullable). Every
// thread calls it. lds needs 17 ints.
__device__ __forceinline__ void budget_lengths(const float *__restrict__ surv,
                                               const float *__restrict__ cutoff, int B, int gamma,
                                               BudgetCut cut, int32_t *lengths, int *lds) {
    int carry = 0;
    for (int base = 0; base < B; base += blockDim.x) {
        int b = base + threadIdx.x;
        int gt = 0, eq = 0;
        if (b < B) {
            if (!cutoff && (gamma & 3) == 0 && ((uintptr_t)surv & 15) == 0) {
                // four values per LDS access
                const float4 *s4 = reinterpret_cast<const float4 *>(surv + (size_t)b * gamma);
                for (int k = 0; k < (gamma >> 2); ++k) {
                    const float4 x = s4[k];
                    const uint32_t u0 = ordered_f32(x.x), u1 = ordered_f32(x.y),
                                   u2 = ordered_f32(x.z), u3 = ordered_f32(x.w);
                    gt += (u0 > cut.tau) + (u1 > cut.tau) + (u2 > cut.tau) + (u3 > cut.tau);
                    eq += (u0 == cut.tau) + (u1 == cut.tau) + (u2 == cut.tau) + (u3 == cut.tau);
                }
            } else {
                for (int k = 0; k < gamma; ++k) {
                    uint32_t u = ordered_f32(ranked_value(surv, cutoff, gamma, b * gamma + k));
                    gt += u > cut.tau ? 1 : 0;
                    eq += u == cut.tau ? 1 : 0;
                }
            }
        }
        int tot;
        int before = carry + block_excl_scan(eq, &tot, lds);
        if (b < B) {
            int take = cut.need - before;
            take = take < 0 ? 0 : (take > eq ? eq : take);
            lengths[b] = gt + take;
        }
        carry += tot;
    }
}

}  // namespace dspark
