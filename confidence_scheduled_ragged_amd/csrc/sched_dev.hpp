// sched_dev.hpp - verify-length cut (per-request threshold or batch budget)
// and the block-wide scan used by compaction, as device functions.
//
// [P1] "DFlash to DSpark in SGLang": the per-request cut of section "The
// confidence scheduler and verify modes" (stop walking the survival curve
// where the gain no longer covers the marginal cost) and the batch-wide
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
// consecutive positions are counted once per run, which keeps the LDS
// histogram atomics off the few crowded bins. The four passes use four
// histograms cleared up front, so a pass needs two barriers: after the
// counts, and after the digit is chosen.
template <int kPer>
__device__ __forceinline__ BudgetCut budget_select_runs(const float *__restrict__ surv, int N, int t,
                                                        uint32_t *hist /*4*256*/,
                                                        uint32_t *sh /*2*/) {
    const int tid = threadIdx.x;
    const int bd = blockDim.x;
    const int lane = tid & (kWave - 1);
    const int per = (N + bd - 1) / bd;
    const int f0 = tid * per;
    uint32_t v[kPer];
    int nv = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int f = f0 + j;
        const bool ok = j < per && f < N;
        v[j] = ok ? ordered_f32(surv[f]) : 0u;
        nv += ok ? 1 : 0;
    }
    for (int i = tid; i < 4 * 256; i += bd) hist[i] = 0;
    __syncthreads();
    uint32_t prefix = 0, mask = 0;
    uint32_t remaining = (uint32_t)t;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        uint32_t *h = hist + 256 * pass;
        uint32_t cur = 0xFFFFFFFFu, run = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (j < nv && (v[j] & mask) == prefix) {
                const uint32_t dg = (v[j] >> shift) & 255u;
                if (dg == cur) {
                    ++run;
                } else {
                    if (run) atomicAdd(&h[cur], run);
                    cur = dg;
                    run = 1;
                }
            }
        }
        if (run) atomicAdd(&h[cur], run);
        __syncthreads();
        if (tid < kWave) {
            uint32_t c[4];
            uint32_t tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = h[255 - 4 * lane - q];
                tot += c[q];
            }
            const int inc = wave_incl_scan((int)tot, lane);
            uint32_t cum = (uint32_t)inc - tot;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cum < remaining && remaining <= cum + c[q]) {
                    sh[2 * (pass & 1)] = prefix | ((uint32_t)(255 - 4 * lane - q) << shift);
                    sh[2 * (pass & 1) + 1] = remaining - cum;
                }
                cum += c[q];
            }
        }
        __syncthreads();
        // the choice of this pass sits in its own pair of words, so the next
        // pass may overwrite the other pair before every thread has read this one
        prefix = sh[2 * (pass & 1)];
        remaining = sh[2 * (pass & 1) + 1];
        mask |= 0xFFu << shift;
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
            for (int k = 0; k < gamma; ++k) {
                uint32_t u = ordered_f32(ranked_value(surv, cutoff, gamma, b * gamma + k));
                gt += u > cut.tau ? 1 : 0;
                eq += u == cut.tau ? 1 : 0;
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
