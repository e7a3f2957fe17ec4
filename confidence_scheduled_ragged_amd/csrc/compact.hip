// compact.hip - stage kernels for step 4 (ragged compaction).
//
// [P1] "DFlash to DSpark in SGLang", section "Ragged verify under full CUDA
// graphs": the scheduled verify rows are front-packed with no padding and a
// cu_seqlens array marks each request's segment; section "Zero-overhead
// scheduling and kernels" fuses the packing into one kernel.
#include "sched_dev.hpp"

namespace dspark {

constexpr int kCompactThreads = 1024;

// One workgroup: scan L_b + 1 over requests in chunks of blockDim requests,
// then write the packed token and source-row entries of that chunk. Reads of
// tokens and writes of the packed arrays walk consecutive addresses.
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(
    const int32_t *__restrict__ lengths, const int32_t *__restrict__ tokens, int B, int gamma,
    int32_t *__restrict__ cu, int32_t *__restrict__ ptok, int32_t *__restrict__ psrc) {
    __shared__ int scan_lds[17];
    __shared__ int start_s[kCompactThreads];
    __shared__ int len_s[kCompactThreads];
    const int g1 = gamma + 1;
    if (threadIdx.x == 0) cu[0] = 0;
    int carry = 0;
    for (int base = 0; base < B; base += blockDim.x) {
        const int b = base + threadIdx.x;
        int L = 0, n = 0;
        if (b < B) {
            L = lengths[b];
            L = L < 0 ? 0 : (L > gamma ? gamma : L);
            n = L + 1;
        }
        int tot;
        int start = carry + block_excl_scan(n, &tot, scan_lds);
        if (b < B) cu[b + 1] = start + n;
        start_s[threadIdx.x] = start;
        len_s[threadIdx.x] = L;
        __syncthreads();
        const int nb = min((int)blockDim.x, B - base);
        for (int q = threadIdx.x; q < nb * g1; q += blockDim.x) {
            const int bl = q / g1, j = q - bl * g1;
            if (j <= len_s[bl]) {
                const int out = start_s[bl] + j;
                const int dense = (base + bl) * g1 + j;
                ptok[out] = tokens[dense];
                psrc[out] = dense;
            }
        }
        carry += tot;
        __syncthreads();
    }
}

// Optional row gather: packed_logits[r, :] = logits[psrc[r], :] for r < cu[B].
// blockIdx.y strides over packed rows, blockIdx.x * blockDim over 16-byte
// slots of a row (or 2-byte elements when rows are not 16-byte aligned).
template <bool kVec>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ logits,
                                                          const int32_t *__restrict__ psrc,
                                                          const int32_t *__restrict__ cu, int B,
                                                          int gamma, int V,
                                                          uint16_t *__restrict__ out) {
    const int cap = B * (gamma + 1);
    int total = cu[B];
    total = total < 0 ? 0 : (total > cap ? cap : total);
    const int64_t slots = kVec ? (V >> 3) : V;
    for (int r = blockIdx.y; r < total; r += gridDim.y) {
        const int src = psrc[r];
        if (src < 0 || src >= cap) continue;
        if (kVec) {
            const u32x4 *in4 = reinterpret_cast<const u32x4 *>(logits + (size_t)src * V);
            u32x4 *o4 = reinterpret_cast<u32x4 *>(out + (size_t)r * V);
            for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < slots;
                 v += (int64_t)gridDim.x * blockDim.x)
                __builtin_nontemporal_store(__builtin_nontemporal_load(in4 + v), o4 + v);
        } else {
            const uint16_t *in = logits + (size_t)src * V;
            uint16_t *o = out + (size_t)r * V;
            for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < slots;
                 v += (int64_t)gridDim.x * blockDim.x)
                o[v] = in[v];
        }
    }
}

hipError_t launch_compact(const int32_t *lengths, const int32_t *tokens, int B, int gamma,
                          int32_t *cu, int32_t *ptok, int32_t *psrc, hipStream_t s) {
    hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(kCompactThreads), 0, s, lengths, tokens, B,
                       gamma, cu, ptok, psrc);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t *logits, const int32_t *psrc, const int32_t *cu,
                              int B, int gamma, int V, uint16_t *out, hipStream_t s) {
    const bool vec = (V % 8 == 0) && (((uintptr_t)logits | (uintptr_t)out) % 16 == 0);
    const int64_t slots = vec ? V / 8 : V;
    const int cap = B * (gamma + 1);
    int gx = (int)((slots + 256 * 4 - 1) / (256 * 4));
    gx = gx < 1 ? 1 : (gx > 64 ? 64 : gx);
    int gy = cap < 4096 ? cap : 4096;
    if (vec)
        hipLaunchKernelGGL((gather_rows_kernel<true>), dim3(gx, gy), dim3(256), 0, s, logits, psrc,
                           cu, B, gamma, V, out);
    else
        hipLaunchKernelGGL((gather_rows_kernel<false>), dim3(gx, gy), dim3(256), 0, s, logits,
                           psrc, cu, B, gamma, V, out);
    return hipGetLastError();
}

}  // namespace dspark
