// conf_dev.hpp - confidence head (bf16 GEMV, fp32 accumulation, STS, sigmoid)
// and survival product for one request, as device functions shared by the
// stage kernel and the fused step kernel.
//
// [P1] "DFlash to DSpark in SGLang", section "DSpark: a sequential head and a
// verify budget": each drafted position's score is one dot product of the
// drafter's hidden state with a weight vector (plus a bias), divided by that
// block position's temperature and squashed by the logistic function; the
// survival curve multiplies the scores up to each position.
#pragma once

#include "common.hpp"

namespace dspark {

constexpr int kGemvUnroll = 4;  // 16-byte hidden loads in flight per lane

// z[i] = sum_k w[k]*h[b,i,k] + bias for the gamma rows of one request, one
// wave per row. hidden_b points at row 0 of the request. kVec: d % 8 == 0 and
// both pointers 16-byte aligned, so each lane loads 8 bf16 per access. A wave
// takes its rows two at a time (i and i + nwaves) and streams both together:
// twice the hidden-state bytes in flight per wave, and each slice of w read
// once for both rows. w may live in LDS or global memory. Each row's fp32
// accumulation order (per lane, then the butterfly) is fixed and does not
// depend on the pairing, so results are bit-reproducible.
// kUnroll: 16-byte hidden loads in flight per lane and row; each lane still
// accumulates its slots in increasing order, whatever the unrolling.
template <bool kVec, int kUnroll = kGemvUnroll>
__device__ __forceinline__ void request_logits(const uint16_t *__restrict__ hidden_b,
                                               const uint16_t *__restrict__ w, float bias,
                                               int gamma, int d, float *z_lds) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    for (int i0 = wave; i0 < gamma; i0 += 2 * nwaves) {
        const int i1 = i0 + nwaves;
        const bool two = i1 < gamma;
        const uint16_t *h0 = hidden_b + (size_t)i0 * (size_t)d;
        const uint16_t *h1 = hidden_b + (size_t)(two ? i1 : i0) * (size_t)d;
        float acc0 = 0.0f, acc1 = 0.0f;
        if (kVec) {
            const u32x4 *a4 = reinterpret_cast<const u32x4 *>(h0);
            const u32x4 *b4 = reinterpret_cast<const u32x4 *>(h1);
            const u32x4 *w4 = reinterpret_cast<const u32x4 *>(w);
            const int nv = d >> 3;
            int v = lane;
            for (; v + (kUnroll - 1) * kWave < nv; v += kUnroll * kWave) {
                u32x4 av[kUnroll], bv[kUnroll], wv[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    av[u] = __builtin_nontemporal_load(a4 + v + u * kWave);
                    if (two) bv[u] = __builtin_nontemporal_load(b4 + v + u * kWave);
                    wv[u] = w4[v + u * kWave];
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        acc0 = fmaf(bf16_lo(av[u][c]), bf16_lo(wv[u][c]), acc0);
                        acc0 = fmaf(bf16_hi(av[u][c]), bf16_hi(wv[u][c]), acc0);
                        if (two) {
                            acc1 = fmaf(bf16_lo(bv[u][c]), bf16_lo(wv[u][c]), acc1);
                            acc1 = fmaf(bf16_hi(bv[u][c]), bf16_hi(wv[u][c]), acc1);
                        }
                    }
                }
            }
            for (; v < nv; v += kWave) {
                const u32x4 av = __builtin_nontemporal_load(a4 + v);
                const u32x4 bv = two ? __builtin_nontemporal_load(b4 + v) : av;
                const u32x4 wv = w4[v];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    acc0 = fmaf(bf16_lo(av[c]), bf16_lo(wv[c]), acc0);
                    acc0 = fmaf(bf16_hi(av[c]), bf16_hi(wv[c]), acc0);
                    acc1 = fmaf(bf16_lo(bv[c]), bf16_lo(wv[c]), acc1);
                    acc1 = fmaf(bf16_hi(bv[c]), bf16_hi(wv[c]), acc1);
                }
            }
        } else {
            for (int k = lane; k < d; k += kWave) {
                const float wk = bf16_f32(w[k]);
                acc0 = fmaf(bf16_f32(h0[k]), wk, acc0);
                acc1 = fmaf(bf16_f32(h1[k]), wk, acc1);
            }
        }
        acc0 = wave_sum_f32(acc0);
        acc1 = wave_sum_f32(acc1);
        if (lane == 0) {
            z_lds[i0] = acc0 + bias;
            if (two) z_lds[i1] = acc1 + bias;
        }
    }
}

// Scores and survival of one request from its logits in LDS. Every thread of
// the block calls it. p_lds and s_lds receive the scores and the survival
// curve (both in LDS); conf_out / surv_out (global, nullable) get copies.
// Survival is a sequential fp32 product: fl(s*p) <= s for p <= 1, so the
// curve never increases.
__device__ __forceinline__ void request_survival(const float *z_lds, const float *__restrict__ temps,
                                                 int gamma, float *p_lds, float *s_lds,
                                                 float *conf_out, float *surv_out) {
    for (int i = threadIdx.x; i < gamma; i += blockDim.x) {
        float p = 1.0f / (1.0f + expf(-z_lds[i] / temps[i]));
        p_lds[i] = p;
        if (conf_out) conf_out[i] = p;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 1.0f;
        for (int i = 0; i < gamma; ++i) {
            s = s * p_lds[i];
            s_lds[i] = s;
        }
    }
    __syncthreads();
    if (surv_out)
        for (int i = threadIdx.x; i < gamma; i += blockDim.x) surv_out[i] = s_lds[i];
}

// Copy w (d bf16) into LDS with 16-byte accesses (kVec layout).
__device__ __forceinline__ void stage_w(const uint16_t *__restrict__ w, int d, uint16_t *w_lds) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(w);
    u32x4 *dst = reinterpret_cast<u32x4 *>(w_lds);
    for (int v = threadIdx.x; v < (d >> 3); v += blockDim.x) dst[v] = src[v];
}

}  // namespace dspark
