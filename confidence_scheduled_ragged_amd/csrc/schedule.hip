// schedule.hip - stage kernels for step 3 (verify-length cut).
#include "sched_dev.hpp"

namespace dspark {

constexpr int kThreshThreads = 256;
constexpr int kBudgetThreads = 1024;

__global__ __launch_bounds__(kThreshThreads) void schedule_threshold_kernel(
    const float *__restrict__ surv, const float *__restrict__ cutoff, int B, int gamma,
    int32_t *__restrict__ lengths) {
    int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    lengths[b] = threshold_length(surv + (size_t)b * gamma, gamma, cutoff[b]);
}

// Batch budget (cutoff NULL) or the combined cut (the budget over the
// positions that pass their request's cutoff): one workgroup.
__global__ __launch_bounds__(kBudgetThreads) void schedule_budget_kernel(
    const float *__restrict__ surv, const float *__restrict__ cutoff, int B, int gamma,
    long long budget, int32_t *__restrict__ lengths) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh[2];
    __shared__ int scan_lds[17];
    const int N = B * gamma;
    const int eligible = cutoff ? block_count_eligible(surv, cutoff, gamma, N, scan_lds) : N;
    const int t = budget < (long long)eligible ? (int)budget : eligible;
    if (t == 0 || t == N) {
        for (int b = threadIdx.x; b < B; b += blockDim.x) lengths[b] = t == 0 ? 0 : gamma;
        return;
    }
    BudgetCut cut = budget_select(surv, cutoff, gamma, N, t, hist, sh);
    budget_lengths(surv, cutoff, B, gamma, cut, lengths, scan_lds);
}

__global__ __launch_bounds__(kThreshThreads) void schedule_static_kernel(int B, int gamma,
                                                                      int32_t *__restrict__ lengths) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) lengths[b] = gamma;
}

// Cost-table cutoff: every request gets the entry of the step's load level.
__global__ __launch_bounds__(kThreshThreads) void cost_cutoff_kernel(
    const float *__restrict__ table, int n, const int32_t *__restrict__ load, int B,
    float *__restrict__ cutoff) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    int j = *load;
    j = j < 0 ? 0 : (j > n - 1 ? n - 1 : j);
    cutoff[b] = table[j];
}

hipError_t launch_cost_cutoff(const float *table, int n, const int32_t *load, int B,
                              float *cutoff, hipStream_t s) {
    dim3 grid((B + kThreshThreads - 1) / kThreshThreads), block(kThreshThreads);
    hipLaunchKernelGGL(cost_cutoff_kernel, grid, block, 0, s, table, n, load, B, cutoff);
    return hipGetLastError();
}

hipError_t launch_schedule(const float *surv, int B, int gamma, int mode, const float *cutoff,
                           long long budget, int32_t *lengths, hipStream_t s) {
    if (mode == DSPARK_CUT_THRESHOLD) {
        dim3 grid((B + kThreshThreads - 1) / kThreshThreads), block(kThreshThreads);
        hipLaunchKernelGGL(schedule_threshold_kernel, grid, block, 0, s, surv, cutoff, B, gamma,
                           lengths);
    } else if (mode == DSPARK_CUT_STATIC) {
        dim3 grid((B + kThreshThreads - 1) / kThreshThreads), block(kThreshThreads);
        hipLaunchKernelGGL(schedule_static_kernel, grid, block, 0, s, B, gamma, lengths);
    } else {
        hipLaunchKernelGGL(schedule_budget_kernel, dim3(1), dim3(kBudgetThreads), 0, s, surv,
                           mode == DSPARK_CUT_COMBINED ? cutoff : nullptr, B, gamma, budget,
                           lengths);
    }
    return hipGetLastError();
}

}  // namespace dspark
