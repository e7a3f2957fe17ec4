// verify_modes.hip - the cap-accept audit arm over a static (full-block)
// verify.
//
// [P1] "DFlash to DSpark in SGLang", section "The confidence scheduler and
// verify modes": cap-accept pays the static verify but commits only the
// scheduled window, so its committed output equals compact's exactly, and it
// logs the acceptance of the whole block beside it; the ratio of the two sums
// is the scheduler's utilisation.
#include "common.hpp"

namespace dspark {

constexpr int kCapThreads = 256;  // 4 waves, one request per wave

__global__ __launch_bounds__(64) void zero_sums_kernel(long long *sums) {
    if (threadIdx.x < 2) sums[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kCapThreads) void cap_accept_kernel(
    const int32_t *__restrict__ pam_full, const int32_t *__restrict__ tokens,
    const int32_t *__restrict__ lengths, int B, int gamma, int32_t *__restrict__ acc,
    int32_t *__restrict__ bonus, int32_t *__restrict__ acc_full, long long *sums) {
    __shared__ long long part[2][kCapThreads / kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int b = blockIdx.x * (kCapThreads / kWave) + wave;
    long long my_a = 0, my_f = 0;
    if (b < B) {
        const int32_t *am = pam_full + (size_t)b * (gamma + 1);
        const int32_t *tok = tokens + (size_t)b * (gamma + 1);
        int L = lengths[b];
        L = L < 0 ? 0 : (L > gamma ? gamma : L);
        // first draft j in [0, gamma) the target disagrees with, else gamma
        int a_full = gamma;
        for (int j0 = 0; j0 < gamma; j0 += kWave) {
            const int j = j0 + lane;
            const bool stop = j < gamma && am[j] != tok[j + 1];
            const uint64_t mask = __ballot(stop);
            if (mask != 0ull) {
                a_full = j0 + __ffsll((unsigned long long)mask) - 1;
                break;
            }
        }
        const int a = a_full < L ? a_full : L;
        if (lane == 0) {
            acc[b] = a;
            acc_full[b] = a_full;
            bonus[b] = am[a];
        }
        my_a = a;
        my_f = a_full;
    }
    if (sums) {
        if (lane == 0) {
            part[0][wave] = my_a;
            part[1][wave] = my_f;
        }
        __syncthreads();
        if (threadIdx.x < 2) {
            long long t = 0;
            for (int i = 0; i < kCapThreads / kWave; ++i) t += part[threadIdx.x][i];
            atomicAdd(reinterpret_cast<unsigned long long *>(sums + threadIdx.x),
                      (unsigned long long)t);
        }
    }
}

hipError_t launch_cap_accept(const int32_t *pam_full, const int32_t *tokens,
                             const int32_t *lengths, int B, int gamma, int32_t *acc,
                             int32_t *bonus, int32_t *acc_full, long long *sums, hipStream_t s) {
    if (sums) hipLaunchKernelGGL(zero_sums_kernel, dim3(1), dim3(64), 0, s, sums);
    const dim3 grid((B + kCapThreads / kWave - 1) / (kCapThreads / kWave));
    hipLaunchKernelGGL(cap_accept_kernel, grid, dim3(kCapThreads), 0, s, pam_full, tokens,
                       lengths, B, gamma, acc, bonus, acc_full, sums);
    return hipGetLastError();
}

}  // namespace dspark
