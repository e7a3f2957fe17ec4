// common.hpp - device helpers, workspace layout and internal launch prototypes
// shared by the HIP kernels of the verify hot path (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 lanes
// A 32-bit word holds two bf16 values; the lower half is the lower index.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- argmax keys
// A 64-bit key orders (value, index) pairs so that the larger key has the
// larger value and, on equal values, the lower index: the high word is the
// value's bits mapped to an order-preserving unsigned integer (with -0 folded
// onto +0), the low word is the bitwise complement of the index. Key 0 means
// "no element".
__device__ __forceinline__ uint32_t ordered_bits(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
    return ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ int32_t key_index(uint64_t k) {
    return k == 0 ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)k);
}
// DSPARK_SLOTS32 (set for one of the two builds of the fused step): every
// a / b below has both operands under 2^32, so the 64-bit path is left out.
#ifndef DSPARK_SLOTS32
#define DSPARK_SLOTS32 0
#endif

// a / b for a >= 0, b > 0: one 32-bit division when both fit in 32 bits (the
// usual case for the slot counts and indices of a step), the 64-bit expansion
// otherwise, which is several times longer on the GPU.
__device__ __forceinline__ int64_t udiv64(int64_t a, int64_t b) {
#if DSPARK_SLOTS32
    return (int64_t)((uint32_t)a / (uint32_t)b);
#else
    if ((((uint64_t)a | (uint64_t)b) >> 32) == 0) return (int64_t)((uint32_t)a / (uint32_t)b);
    return (int64_t)((uint64_t)a / (uint64_t)b);
#endif
}

// Largest u64 key over aligned groups of 2^lq lanes (lq <= 6), on every lane
// of the group; the whole wave must be active. Groups of 2 and 4 exchange
// through DPP quad permutes, of 8 and 16 through the half-row and row mirrors
// (lane i of a group meets lane size-1-i, in the other half, once the halves
// hold their own maxima), of 32 and 64 through LDS permutes. Four of the six
// steps of a full wave then stay in the VALU (an LDS permute costs about 120
// cycles).
__device__ __forceinline__ uint64_t dpp_u64(uint64_t k, int ctrl_sel) {
    const int lo = (int)(uint32_t)k, hi = (int)(uint32_t)(k >> 32);
    int l2, h2;
    switch (ctrl_sel) {
    case 0:
        l2 = __builtin_amdgcn_update_dpp(lo, lo, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
        h2 = __builtin_amdgcn_update_dpp(hi, hi, 0xB1, 0xF, 0xF, false);
        break;
    case 1:
        l2 = __builtin_amdgcn_update_dpp(lo, lo, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
        h2 = __builtin_amdgcn_update_dpp(hi, hi, 0x4E, 0xF, 0xF, false);
        break;
    case 2:
        l2 = __builtin_amdgcn_update_dpp(lo, lo, 0x141, 0xF, 0xF, false);  // row_half_mirror
        h2 = __builtin_amdgcn_update_dpp(hi, hi, 0x141, 0xF, 0xF, false);
        break;
    default:
        l2 = __builtin_amdgcn_update_dpp(lo, lo, 0x140, 0xF, 0xF, false);  // row_mirror
        h2 = __builtin_amdgcn_update_dpp(hi, hi, 0x140, 0xF, 0xF, false);
        break;
    }
    return ((uint64_t)(uint32_t)h2 << 32) | (uint64_t)(uint32_t)l2;
}
__device__ __forceinline__ uint64_t group_max_u64(uint64_t k, int lq) {
    uint64_t o;
    if (lq > 0) { o = dpp_u64(k, 0); k = o > k ? o : k; }
    if (lq > 1) { o = dpp_u64(k, 1); k = o > k ? o : k; }
    if (lq > 2) { o = dpp_u64(k, 2); k = o > k ? o : k; }
    if (lq > 3) { o = dpp_u64(k, 3); k = o > k ? o : k; }
    if (lq > 4) { o = __shfl_xor(k, 16, kWave); k = o > k ? o : k; }
    if (lq > 5) { o = __shfl_xor(k, 32, kWave); k = o > k ? o : k; }
    return k;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) { return group_max_u64(k, 6); }
__device__ __forceinline__ float wave_sum_f32(float x) {
    // Butterfly: partners add the same two values, so every lane ends with the
    // same bit pattern and the order is fixed (deterministic).
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Inclusive scan of one int per lane across a wave (every lane active), by
// DPP data movement: shifts by 1, 2, 4 and 8 lanes inside each row of 16, then
// the last lane of row 0 added to row 1, of row 2 to row 3, and of row 1 (by
// then the total of rows 0-1) to rows 2 and 3. A lane whose source falls
// outside its row, or a row outside the row mask, adds 0. Six VALU steps
// instead of six LDS permutes (about 120 cycles each); integer sums, so the
// result is exact whatever the order.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
    (void)lane;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// ---------------------------------------------------- balanced row partition
// The packed logit rows form one virtual array of total*Vv vector slots
// (Vv = slots per row). Wave w of W owns slots [w*Q, min((w+1)*Q, E)),
// E = total*Vv, Q = max(kMinSlotsPerWave, ceil(E/W)). The segment of wave w
// inside packed row r stores its key at keys[w + r]: walking the array, each
// row or wave boundary raises w + r by one, so these indices never collide.
constexpr int64_t kMinSlotsPerWave = 64;

__device__ __forceinline__ int64_t partition_q(int64_t E, int64_t W) {
    int64_t q = (E + W - 1) / W;
    return q < kMinSlotsPerWave ? kMinSlotsPerWave : q;
}

// ---------------------------------------------------- fused-step sub-chunks
// The fused step streams a virtual array of E vector slots (rows laid end to
// end) in sub-chunks of K slots, K = max(kSubMin, ceil(E / Wt)) for a target
// wave count Wt: about one contiguous sub-chunk per wave. The root rows'
// sub-chunk s stores the key of its segment inside row r at rkeys[s + r],
// collision-free as for the balanced partition, with s < Wt <= kMaxWaves; the
// draft rows' segments merge into one key per row by atomic max.
constexpr int64_t kSubMin = 1024;  // 16 KiB of bf16

__device__ __forceinline__ int64_t sub_len(int64_t E, int64_t Wt) {
    const int64_t k = udiv64(E + Wt - 1, Wt);
    return k < kSubMin ? kSubMin : k;
}

// ------------------------------------------------------------ workspace map
// ctrl:  [0, 256)                control words of the fused step (arrival
//                                counters and flags, below); zero between
//                                calls, at the same place for every size, so
//                                one workspace serves calls of any size it is
//                                large enough for
// rcnt:  uint64 [kMaxFusedB]     per-request arrival counters of the fused
//                                step (zero between calls: each request's last
//                                arriver resets its own), spread so that
//                                consecutive requests sit 128 bytes apart
// acnt:  uint64 [kMaxFusedB]     per-request arrival counters of dspark_accept
//                                (zero between calls: each request's last
//                                arriver resets its own)
// keys:  uint64 [kMaxWaves + B*(gamma+1)] argmax segment keys of packed rows
//                                (dspark_accept); in the fused step, one key
//                                per dense draft row (b*(gamma+1) + j), which
//                                the request's front workgroup zeroes
// rkeys: uint64 [kMaxWaves + B]  segment keys of the root rows (fused step)
// surv:  float [B*gamma]         survival scratch (when the caller passes none)
// conf:  float [B*gamma]         score scratch (when the caller passes none)
constexpr int64_t kMaxWaves = 16384;  // bound on waves (or sub-chunks) per pass
constexpr int kMaxFusedB = 4096;      // largest batch of the fused step
constexpr size_t kCtrlBytes = 256;
// Words of the ctrl region: at 0 the arrival counter of the request
// workgroups (both forms of the fused step); on the next 128-byte line the
// one-launch step's go word (positive while the lengths are final and
// workgroups are yet to leave, zero between calls); at 192 the sticky time-out
// flag (set when a workgroup gave up its bounded wait; read and cleared by
// dspark_step_status).
constexpr size_t kCtrlGoOffset = 128;
constexpr size_t kCtrlTimedOutOffset = 192;

inline size_t ws_ctrl_offset() { return 0; }
inline size_t ws_rcnt_offset() { return kCtrlBytes; }
inline size_t ws_acnt_offset() { return kCtrlBytes + (size_t)8 * kMaxFusedB; }
inline size_t ws_keys_offset() { return kCtrlBytes + (size_t)16 * kMaxFusedB; }
inline size_t ws_rkeys_offset(int64_t B, int64_t gamma) {
    return ws_keys_offset() + (size_t)8 * (size_t)(kMaxWaves + B * (gamma + 1));
}
inline size_t ws_surv_offset(int64_t B, int64_t gamma) {
    return ws_rkeys_offset(B, gamma) + (size_t)8 * (size_t)(kMaxWaves + B);
}
inline size_t ws_conf_offset(int64_t B, int64_t gamma) {
    return ws_surv_offset(B, gamma) + (size_t)4 * (size_t)(B * gamma);
}
inline size_t ws_total_bytes(int64_t B, int64_t gamma) {
    const size_t s = ws_conf_offset(B, gamma) + (size_t)4 * (size_t)(B * gamma);
    return (s + 255) & ~(size_t)255;
}

// Number of compute units of the current device (cached per device).
int device_cu_count();

// ------------------------------------------------------ internal launches
hipError_t launch_confidence(const uint16_t *hidden, const uint16_t *w, float bias,
                             const float *temps, int B, int gamma, int d, float *conf,
                             float *surv, hipStream_t s);
hipError_t launch_schedule(const float *surv, int B, int gamma, int mode, const float *cutoff,
                           long long budget, int32_t *lengths, hipStream_t s);
hipError_t launch_compact(const int32_t *lengths, const int32_t *tokens, int B, int gamma,
                          int32_t *cu, int32_t *ptok, int32_t *psrc, hipStream_t s);
hipError_t launch_gather_rows(const void *src, const int32_t *psrc, const int32_t *cu, int B,
                              int gamma, int64_t row_bytes, void *dst, hipStream_t s);
hipError_t launch_accept(const uint16_t *logits, const int32_t *psrc, const int32_t *cu,
                         const int32_t *tokens, int B, int gamma, int V, int32_t *pam,
                         int32_t *acc, int32_t *bonus, void *ws, hipStream_t s);
hipError_t launch_fill_zero(void *ws, size_t bytes, hipStream_t s);

// The fused step in two launches. Returns hipErrorNotSupported (enqueuing
// nothing) when the sizes are outside what it handles; the caller then runs
// the stage kernels instead.
hipError_t launch_cap_accept(const int32_t *pam_full, const int32_t *tokens,
                             const int32_t *lengths, int B, int gamma, int32_t *acc,
                             int32_t *bonus, int32_t *acc_full, long long *sums, hipStream_t s);
hipError_t launch_tier_select(const int32_t *cu, int B, int gamma, const int32_t *tiers,
                              int ntiers, int32_t pad_token, int32_t *padded_total,
                              int32_t *tier_index, int32_t *ptok, int32_t *psrc, hipStream_t s);
hipError_t launch_cost_cutoff(const float *table, int n, const int32_t *load, int B,
                              float *cutoff, hipStream_t s);
// The fused step, built twice: slots32 for steps whose slot counts and indices
// all fit in 32 bits (fused_slots_fit_32), without the 64-bit division paths
// (measured 0.3-0.5 us faster per step at B = 256 under a budget and at B = 1),
// slots64 for any size.
#define DSPARK_FUSED_STEP_DECL                                                                \
    hipError_t launch_fused_step(                                                              \
        const uint16_t *hidden, const uint16_t *w, float bias, const float *temps,            \
        const int32_t *tokens, const uint16_t *logits, int B, int gamma, int d, int V,        \
        int mode, const float *cutoff, long long budget, float *conf, float *surv,            \
        int32_t *lengths, int32_t *cu, int32_t *ptok, int32_t *psrc, int32_t *pam,            \
        int32_t *acc, int32_t *bonus, void *ws, hipStream_t s, hipEvent_t ev_start,           \
        hipEvent_t ev_stop, int launches, unsigned long long wait_ticks);
namespace slots32 {
DSPARK_FUSED_STEP_DECL
}
namespace slots64 {
DSPARK_FUSED_STEP_DECL
}
#undef DSPARK_FUSED_STEP_DECL
// True when the slots32 build serves the step: its largest division operand
// (the rows laid end to end, V or V / 8 slots each, plus a sub-chunk and a
// lead, each at most that much again, plus the wave bound) stays under 2^32.
inline bool fused_slots_fit_32(int B, int gamma, int V, const void *logits) {
    const bool vec = (V % 8 == 0) && ((uintptr_t)logits % 16 == 0);
    const int64_t slots = (int64_t)B * (gamma + 1) * (vec ? V / 8 : V);
    return 4 * slots + 2 * kMaxWaves < ((int64_t)1 << 32);
}
// Reads the fused step's sticky time-out flag of ws into *status and clears it.
hipError_t launch_step_status(void *ws, int32_t *status, hipStream_t s);

}  // namespace dspark
