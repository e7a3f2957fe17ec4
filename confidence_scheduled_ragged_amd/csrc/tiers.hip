// tiers.hip - graph tier of a packed verify batch, picked on the device.
//
// [P1] "DFlash to DSpark in SGLang", section "Ragged verify under full CUDA
// graphs": graphs are captured for a ladder of packed sizes, and a step replays
// the smallest captured size that holds its packed total, so a tighter budget
// replays a smaller graph. The pick and the padding of the packed arrays up to
// that size run on the device, so they can sit in the same stream (or captured
// graph) as the schedule and compaction.
#include "common.hpp"

namespace dspark {

constexpr int kTierThreads = 256;

// Every thread finds the tier itself (the ladder is short and cached); thread
// 0 of block 0 publishes it, and each thread pads its own packed row.
__global__ __launch_bounds__(kTierThreads) void tier_select_kernel(
    const int32_t *__restrict__ cu, int B, int cap, const int32_t *__restrict__ tiers, int ntiers,
    int32_t pad_token, int32_t *__restrict__ padded_total, int32_t *__restrict__ tier_index,
    int32_t *__restrict__ ptok, int32_t *__restrict__ psrc) {
    int total = cu[B];
    total = total < 0 ? 0 : (total > cap ? cap : total);
    int lo = 0, hi = ntiers;  // first tier >= total (binary search, ascending ladder)
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tiers[mid] < total) lo = mid + 1; else hi = mid;
    }
    const int padded = lo < ntiers ? tiers[lo] : total;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *tier_index = lo;
        *padded_total = padded;
    }
    const int end = padded < cap ? padded : cap;
    for (int r = total + blockIdx.x * blockDim.x + threadIdx.x; r < end;
         r += gridDim.x * blockDim.x) {
        if (ptok) ptok[r] = pad_token;
        if (psrc) psrc[r] = -1;
    }
}

hipError_t launch_tier_select(const int32_t *cu, int B, int gamma, const int32_t *tiers,
                              int ntiers, int32_t pad_token, int32_t *padded_total,
                              int32_t *tier_index, int32_t *ptok, int32_t *psrc, hipStream_t s) {
    const int cap = B * (gamma + 1);
    int grid = (cap + kTierThreads - 1) / kTierThreads;
    grid = grid < 1 ? 1 : (grid > 1024 ? 1024 : grid);
    hipLaunchKernelGGL(tier_select_kernel, dim3(grid), dim3(kTierThreads), 0, s, cu, B, cap, tiers,
                       ntiers, pad_token, padded_total, tier_index, ptok, psrc);
    return hipGetLastError();
}

}  // namespace dspark
