// kda_peaks.hip -- measured ceilings of one gfx950 GPU, the second denominator of the
// benchmark's roofline fractions (the first is the vendor's spec sheet): a streaming
// HBM copy and a loop of dense bf16 matrix-core instructions.  Built into its own
// library (libkda_peaks.so); nothing in libkda.so uses it.
//
//   kda_peak_copy  dst[i] = src[i] over `bytes` bytes (multiple of 16), 16-byte
//                  nontemporal loads and stores in a grid-stride loop: the bytes moved
//                  are 2 x bytes (read + write).
//   kda_peak_read  the same read stream alone, reduced to one value per thread group
//                  (written to out so the loads are not removed).
//   kda_peak_mfma  every wave issues `iters` rounds of 8 independent
//                  v_mfma_f32_16x16x32_bf16 accumulations (16 x 16 x 32 x 2 flop each)
//                  on register operands; one float per wave is written to out.
// All three return a hipError_t code (0 = launched) and enqueue on `stream`.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_kernel(const u32x4_t *__restrict__ src, u32x4_t *__restrict__ dst,
                                                  size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
        __builtin_nontemporal_store(a, dst + i);
        __builtin_nontemporal_store(b, dst + i + stride);
        __builtin_nontemporal_store(c, dst + i + 2 * stride);
        __builtin_nontemporal_store(d, dst + i + 3 * stride);
    }
    for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4_t *__restrict__ src, size_t n, uint32_t *out) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
    }
    for (; i < n; i += stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    // one value per 256-thread group; the xor keeps every load live
    acc ^= __shfl_xor(acc, 1);
    if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void mfma_kernel(float *out, int iters) {
    const uint32_t lane = threadIdx.x & 63;
    // operands that the compiler cannot fold: small bf16 values derived from the lane
    u32x4_t ai, bi;
    for (int e = 0; e < 4; ++e) {
        ai[e] = 0x3f803f80u ^ (lane << 3) ^ e;
        bi[e] = 0x3f803f80u ^ (lane << 5) ^ (e << 1);
    }
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ai), b = __builtin_bit_cast(bf16x8_t, bi);
    f32x4_t acc[8];
    for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (lane == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

int kda_peak_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream) {
    if (!src || !dst || bytes % 16 || blocks <= 0) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t *>(src), static_cast<u32x4_t *>(dst), bytes / 16);
    return static_cast<int>(hipGetLastError());
}

int kda_peak_read(const void *src, size_t bytes, uint32_t *out, int blocks, void *stream) {
    if (!src || !out || bytes % 16 || blocks <= 0) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t *>(src), bytes / 16, out);
    return static_cast<int>(hipGetLastError());
}

// out holds blocks * 4 floats
int kda_peak_mfma(float *out, int blocks, int iters, void *stream) {
    if (!out || blocks <= 0 || iters <= 0) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
