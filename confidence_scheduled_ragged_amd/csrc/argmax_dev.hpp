// argmax_dev.hpp - greedy target choice over packed verify rows, acceptance
// and bonus token, as device functions shared by the stage kernels and the
// fused step kernel.
//
// [P1] "DFlash to DSpark in SGLang", section "Background": the target checks
// the drafted tokens in one forward, the agreeing prefix is committed, and
// the forward yields one extra (bonus) token. Greedy verification takes the
// largest logit of each row, the lowest index among equal maxima.
#pragma once

#include "common.hpp"

namespace dspark {

// Fold eight consecutive bf16 logits (one 16-byte slot starting at element
// `base`) into a lane's running (best, bidx). A slot only replaces the best
// when its maximum is strictly larger, and inside the slot the first element
// equal to that maximum is taken, so each lane keeps the first maximum of the
// elements it has seen in increasing order.
__device__ __forceinline__ void fold_slot(u32x4 a, int base, float &best, int &bidx) {
    const float x0 = bf16_lo(a[0]), x1 = bf16_hi(a[0]), x2 = bf16_lo(a[1]), x3 = bf16_hi(a[1]);
    const float x4 = bf16_lo(a[2]), x5 = bf16_hi(a[2]), x6 = bf16_lo(a[3]), x7 = bf16_hi(a[3]);
    const float m = fmaxf(fmaxf(fmaxf(x0, x1), fmaxf(x2, x3)), fmaxf(fmaxf(x4, x5), fmaxf(x6, x7)));
    if (m > best || bidx < 0) {
        int j = 7;
        j = (x6 == m) ? 6 : j;
        j = (x5 == m) ? 5 : j;
        j = (x4 == m) ? 4 : j;
        j = (x3 == m) ? 3 : j;
        j = (x2 == m) ? 2 : j;
        j = (x1 == m) ? 1 : j;
        j = (x0 == m) ? 0 : j;
        best = m;
        bidx = base + j;
    }
}

// One lane's share of slots [v0, v1) of a row: slots v0+lane, v0+lane+64, ...
// kVec: a slot is 8 bf16 (16-byte aligned row); otherwise a slot is one bf16.
// kUnroll loads are issued before any is consumed. With kUnroll > 2 the last
// partial round is one batch too: its loads past v1 are clamped to slot v1 - 1
// (in the row, and the same cache line) and not folded, so a short segment
// costs one memory round trip instead of one per leftover slot.
template <bool kVec, int kUnroll>
__device__ __forceinline__ void lane_row_segment(const uint16_t *__restrict__ row, int64_t v0,
                                                 int64_t v1, int lane, float &best, int &bidx) {
    if (kVec) {
        const u32x4 *r4 = reinterpret_cast<const u32x4 *>(row);
        int64_t v = v0 + lane;
        for (; v + (int64_t)(kUnroll - 1) * kWave < v1; v += (int64_t)kUnroll * kWave) {
            u32x4 buf[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) buf[u] = __builtin_nontemporal_load(r4 + v + u * kWave);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) fold_slot(buf[u], (int)((v + u * kWave) * 8), best, bidx);
        }
        if (kUnroll > 2) {
            if (v < v1) {
                u32x4 buf[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int64_t x = v + u * kWave;
                    buf[u] = __builtin_nontemporal_load(r4 + (x < v1 ? x : v1 - 1));
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    if (v + u * kWave < v1) fold_slot(buf[u], (int)((v + u * kWave) * 8), best, bidx);
            }
        } else {
            for (; v < v1; v += kWave)
                fold_slot(__builtin_nontemporal_load(r4 + v), (int)(v * 8), best, bidx);
        }
    } else {
        for (int64_t v = v0 + lane; v < v1; v += kWave) {
            const float x = bf16_f32(row[v]);
            if (x > best || bidx < 0) {
                best = x;
                bidx = (int)v;
            }
        }
    }
}

// Packed rows clamped to the capacity of the packed arrays.
__device__ __forceinline__ int packed_total(const int32_t *cu, int B, int cap) {
    int t = cu[B];
    return t < 0 ? 0 : (t > cap ? cap : t);
}

// Argmax work of wave w of W over the packed rows (balanced partition, see
// partition_q). Packed row r reads dense row psrc[r] (or row r when psrc is
// NULL); a source row outside [0, cap) leaves key 0 ("no element").
template <bool kVec, int kUnroll>
__device__ __forceinline__ void wave_argmax_share(const uint16_t *__restrict__ logits,
                                                  const int32_t *__restrict__ psrc, int total,
                                                  int cap, int V, int64_t w, int64_t W,
                                                  uint64_t *__restrict__ keys) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t Vv = kVec ? (V >> 3) : V;
    const int64_t E = (int64_t)total * Vv;
    const int64_t Q = partition_q(E, W);
    int64_t e = w * Q;
    if (e >= E) return;
    const int64_t e_end = e + Q < E ? e + Q : E;
    int64_t r = e / Vv;
    while (e < e_end) {
        const int64_t row_end = (r + 1) * Vv;
        const int64_t seg_end = e_end < row_end ? e_end : row_end;
        const int src = psrc ? psrc[r] : (int)r;
        float best = -INFINITY;
        int bidx = -1;
        if (src >= 0 && src < cap) {
            const uint16_t *row = logits + (size_t)src * (size_t)V;
            lane_row_segment<kVec, kUnroll>(row, e - r * Vv, seg_end - r * Vv, lane, best, bidx);
        }
        uint64_t key = bidx >= 0 ? argmax_key(best, (uint32_t)bidx) : 0ull;
        key = wave_max_u64(key);
        if (lane == 0) keys[w + r] = key;
        e = seg_end;
        ++r;
    }
}

// Keys written and read inside one kernel by different workgroups (possibly on
// different XCDs, each with its own L2) use device-coherent accesses: the
// store writes through to the device coherence point and the load bypasses
// any stale L2 copy. Neither needs an L2-wide write-back or invalidate.
__device__ __forceinline__ void store_key_coherent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_key_coherent(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Index of the largest key among keys[s + r] for s in [s_lo, s_hi]: the
// segment keys of row r left by sub-chunks s_lo..s_hi. kCoherent: the keys were
// written by this same kernel. The loads are issued four at a time, so a row
// costs one memory round trip in the usual case of at most four segments.
template <bool kCoherent = false>
__device__ __forceinline__ int32_t segment_keys_argmax(const uint64_t *__restrict__ keys, int64_t r,
                                                       int64_t s_lo, int64_t s_hi) {
    uint64_t k = 0;
    for (int64_t w = s_lo; w <= s_hi; w += 4) {
        uint64_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = w + u <= s_hi ? w + u + r : s_lo + r;  // in range, repeats are harmless
            x[u] = kCoherent ? load_key_coherent(keys + i) : keys[i];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) k = x[u] > k ? x[u] : k;
    }
    return key_index(k);
}

// The same by the calling wave: lane i reads keys s_lo + i, s_lo + i + 64, ...
// (of row r), so up to 64 segments cost one memory round trip. Called by a
// whole wave; every lane gets the index.
template <bool kCoherent = false>
__device__ __forceinline__ int32_t wave_segment_keys_argmax(const uint64_t *__restrict__ keys,
                                                            int64_t r, int64_t s_lo, int64_t s_hi) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t k = 0;
    for (int64_t s = s_lo + lane; s <= s_hi; s += kWave) {
        const uint64_t x = kCoherent ? load_key_coherent(keys + s + r) : keys[s + r];
        k = x > k ? x : k;
    }
    return key_index(wave_max_u64(k));
}

// Argmax of packed row r from the keys of the waves whose shares (Q slots
// each, Vv slots per row) touch it.
template <bool kCoherent = false>
__device__ __forceinline__ int32_t row_argmax(const uint64_t *__restrict__ keys, int64_t r,
                                              int64_t Vv, int64_t Q) {
    return segment_keys_argmax<kCoherent>(keys, r, (r * Vv) / Q, ((r + 1) * Vv - 1) / Q);
}

// Acceptance and bonus of one request by one wave, from its verified rows'
// argmax: row_am(j) for j in [0, n), n = L_b + 1 rows (root first). Lane j
// handles row j (chunks of 64 rows) and stores it at pam_b[j]. The first row j
// where the target disagrees with draft j+1, or j = L_b, is the accepted
// count; that row's argmax is the bonus. n <= 0 gives accepted 0, bonus -1.
// draft(j) is draft j + 1's token (asked for j < L_b only).
template <typename RowAm, typename Draft>
__device__ __forceinline__ void wave_accept_rows_t(RowAm row_am, Draft draft, int n, int gamma,
                                                   int32_t *__restrict__ pam_b,
                                                   int32_t *__restrict__ acc_b,
                                                   int32_t *__restrict__ bonus_b) {
    const int lane = threadIdx.x & (kWave - 1);
    if (n <= 0) {
        if (lane == 0) {
            *acc_b = 0;
            *bonus_b = -1;
        }
        return;
    }
    const int L = n - 1 < gamma ? n - 1 : gamma;
    int a = -1;
    int32_t bon = -1;
    for (int j0 = 0; j0 < n; j0 += kWave) {
        const int j = j0 + lane;
        int32_t am = -1;
        bool stop = false;
        if (j < n) {
            am = row_am(j);
            pam_b[j] = am;
            stop = (j >= L) || (am != draft(j));
        }
        const uint64_t mask = __ballot(stop);
        if (a < 0 && mask != 0ull) {
            const int first = __ffsll((unsigned long long)mask) - 1;
            a = j0 + first;
            bon = __shfl(am, first, kWave);  // the bonus is that row's argmax
        }
    }
    if (lane == 0) {
        *acc_b = a;
        *bonus_b = bon;
    }
}

// The same with the request's tokens in memory (tok[0] the root token).
template <typename RowAm>
__device__ __forceinline__ void wave_accept_rows(RowAm row_am, int n, int gamma,
                                                 const int32_t *__restrict__ tok,
                                                 int32_t *__restrict__ pam_b,
                                                 int32_t *__restrict__ acc_b,
                                                 int32_t *__restrict__ bonus_b) {
    wave_accept_rows_t(row_am, [&](int j) { return tok[j + 1]; }, n, gamma, pam_b, acc_b, bonus_b);
}

// Acceptance and bonus of request b when every packed row's argmax comes from
// segment keys (packed row r = cu[b] + j).
template <bool kCoherent = false>
__device__ __forceinline__ void wave_accept_request(const uint64_t *__restrict__ keys,
                                                    const int32_t *__restrict__ cu,
                                                    const int32_t *__restrict__ tokens, int b,
                                                    int gamma, int total, int64_t Vv, int64_t Q,
                                                    int32_t *__restrict__ pam,
                                                    int32_t *__restrict__ acc,
                                                    int32_t *__restrict__ bonus) {
    int start = cu[b], end = cu[b + 1];
    start = start < 0 ? 0 : (start > total ? total : start);
    end = end < start ? start : (end > total ? total : end);
    wave_accept_rows([&](int j) { return row_argmax<kCoherent>(keys, start + j, Vv, Q); },
                     end - start, gamma, tokens + (size_t)b * (gamma + 1), pam + start, acc + b,
                     bonus + b);
}

}  // namespace dspark
