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

// Row gather through the packed source rows: dst[r, :] = src[psrc[r], :] for
// r < cu[B], rows of `row_elems` elements of type T (16, 4 or 1 bytes).
// blockIdx.y strides over packed rows, blockIdx.x * blockDim over a row's
// elements; each thread has four loads in flight before it stores. A source
// row outside [0, cap) leaves its packed row untouched.
template <typename T>
__global__ __launch_bounds__(256) void gather_rows_kernel(const T *__restrict__ src,
                                                          const int32_t *__restrict__ psrc,
                                                          const int32_t *__restrict__ cu, int B,
                                                          int cap, int64_t row_elems,
                                                          T *__restrict__ dst) {
    constexpr int kUnroll = 4;
    int total = cu[B];
    total = total < 0 ? 0 : (total > cap ? cap : total);
    const int64_t step = (int64_t)gridDim.x * blockDim.x * kUnroll;
    for (int r = blockIdx.y; r < total; r += gridDim.y) {
        const int s = psrc[r];
        if (s < 0 || s >= cap) continue;
        const T *in = src + (size_t)s * (size_t)row_elems;
        T *out = dst + (size_t)r * (size_t)row_elems;
        for (int64_t c0 = (int64_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x; c0 < row_elems;
             c0 += step) {
            T v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t c = c0 + (int64_t)u * blockDim.x;
                if (c < row_elems) v[u] = __builtin_nontemporal_load(in + c);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t c = c0 + (int64_t)u * blockDim.x;
                if (c < row_elems) __builtin_nontemporal_store(v[u], out + c);
            }
        }
    }
}

template <typename T>
static void launch_gather_typed(const void *src, const int32_t *psrc, const int32_t *cu, int B,
                                int gamma, int64_t row_elems, void *dst, hipStream_t s) {
    const int cap = B * (gamma + 1);
    int64_t gx = (row_elems + 256 * 4 - 1) / (256 * 4);
    gx = gx < 1 ? 1 : (gx > 64 ? 64 : gx);
    const int gy = cap < 4096 ? cap : 4096;
    hipLaunchKernelGGL((gather_rows_kernel<T>), dim3((unsigned)gx, gy), dim3(256), 0, s,
                       static_cast<const T *>(src), psrc, cu, B, cap, row_elems,
                       static_cast<T *>(dst));
}

hipError_t launch_compact(const int32_t *lengths, const int32_t *tokens, int B, int gamma,
                          int32_t *cu, int32_t *ptok, int32_t *psrc, hipStream_t s) {
    hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(kCompactThreads), 0, s, lengths, tokens, B,
                       gamma, cu, ptok, psrc);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void *src, const int32_t *psrc, const int32_t *cu, int B,
                              int gamma, int64_t row_bytes, void *dst, hipStream_t s) {
    const uintptr_t al = (uintptr_t)src | (uintptr_t)dst;
    if (row_bytes % 16 == 0 && al % 16 == 0)
        launch_gather_typed<u32x4>(src, psrc, cu, B, gamma, row_bytes / 16, dst, s);
    else if (row_bytes % 4 == 0 && al % 4 == 0)
        launch_gather_typed<uint32_t>(src, psrc, cu, B, gamma, row_bytes / 4, dst, s);
    else
        launch_gather_typed<uint8_t>(src, psrc, cu, B, gamma, row_bytes, dst, s);
    return hipGetLastError();
}

}  // namespace dspark
