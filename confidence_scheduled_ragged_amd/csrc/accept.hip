// accept.hip - stage kernels for steps 5-6: a persistent argmax pass over the
// packed rows (balanced across all waves of the device), then one wave per
// request for acceptance and the bonus token.
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

hipError_t launch_accept(const uint16_t *logits, const int32_t *psrc, const int32_t *cu,
                         const int32_t *tokens, int B, int gamma, int V, int32_t *pam,
                         int32_t *acc, int32_t *bonus, void *ws, hipStream_t s) {
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
