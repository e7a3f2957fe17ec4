// confidence.hip - stage kernel for steps 1-2: one workgroup per request.
#include "conf_dev.hpp"

namespace dspark {

constexpr int kConfThreads = 1024;
constexpr int kMaxLdsW = 16384;  // w is staged in LDS when d <= this (32 KiB)

template <bool kVec, bool kLdsW>
__global__ __launch_bounds__(kConfThreads) void confidence_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ w, float bias,
    const float *__restrict__ temps, int gamma, int d, float *__restrict__ conf,
    float *__restrict__ surv) {
    extern __shared__ __align__(16) uint16_t w_lds[];
    __shared__ float z_s[DSPARK_MAX_GAMMA], p_s[DSPARK_MAX_GAMMA], s_s[DSPARK_MAX_GAMMA];
    const int b = blockIdx.x;
    const uint16_t *wp = w;
    if (kLdsW) {
        stage_w(w, d, w_lds);
        __syncthreads();
        wp = w_lds;
    }
    request_logits<kVec>(hidden + (size_t)b * gamma * d, wp, bias, gamma, d, z_s);
    __syncthreads();
    request_survival(z_s, temps, gamma, p_s, s_s, conf + (size_t)b * gamma,
                     surv + (size_t)b * gamma);
}

hipError_t launch_confidence(const uint16_t *hidden, const uint16_t *w, float bias,
                             const float *temps, int B, int gamma, int d, float *conf,
                             float *surv, hipStream_t s) {
    const bool vec = (d % 8 == 0) && (((uintptr_t)hidden | (uintptr_t)w) % 16 == 0);
    dim3 grid(B), block(kConfThreads);
    if (vec && d <= kMaxLdsW)
        hipLaunchKernelGGL((confidence_kernel<true, true>), grid, block, (size_t)d * 2, s,
                           hidden, w, bias, temps, gamma, d, conf, surv);
    else if (vec)
        hipLaunchKernelGGL((confidence_kernel<true, false>), grid, block, 0, s, hidden, w,
                           bias, temps, gamma, d, conf, surv);
    else
        hipLaunchKernelGGL((confidence_kernel<false, false>), grid, block, 0, s, hidden, w,
                           bias, temps, gamma, d, conf, surv);
    return hipGetLastError();
}

}  // namespace dspark
