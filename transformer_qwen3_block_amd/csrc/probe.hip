// Measurement probes (not part of the forward pass): the attainable HBM read bandwidth and the attainable
// dense f16 MFMA rate of the device, so every roofline fraction can be stated against both the nominal
// peak and what a plain kernel of the same kind reaches on the same box.
#include "common.h"

namespace qw3 {

namespace {

// Streams `n16` 16-byte words with nontemporal loads (grid-stride, 4 loads in flight per lane) and folds
// them into one word per workgroup, so no load can be dropped by the compiler.
__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4 *p, uint64_t n16, uint32_t *out) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = load_nt16(p + i), b = load_nt16(p + i + stride), c = load_nt16(p + i + 2 * stride),
                    d = load_nt16(p + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = load_nt16(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < 256; ++t) r ^= red[t];
        out[blockIdx.x] = r;
    }
}

typedef __attribute__((ext_vector_type(8))) _Float16 h8_t;
typedef __attribute__((ext_vector_type(4))) float f4_t;

// Back-to-back v_mfma_f32_16x16x32_f16 on register operands, kMfmaChains independent accumulators per wave
// (16384 flops per instruction), `iters` rounds of kMfmaChains.  Sixteen chains keep the matrix
// pipeline full (four measured 1.39-1.50 PFLOP/s on 2048-4096 workgroups, sixteen 1.94-1.97).
constexpr int kMfmaChains = 16;
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *out) {
    const int lane = threadIdx.x & 63;
    h8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)(0.001f * (lane + e));
        b[e] = (_Float16)(0.002f * (lane - e));
    }
    f4_t c[kMfmaChains];
#pragma unroll
    for (int i = 0; i < kMfmaChains; ++i) c[i] = f4_t{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int i = 0; i < kMfmaChains; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[i], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMfmaChains; ++i) s += c[i][i & 3];
    if (lane == 0) out[(size_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

}  // namespace qw3

using namespace qw3;

extern "C" {

int32_t qw3_probe_hbm_read(const void *buf_dev, uint64_t bytes, uint32_t *out_dev, int32_t grid, void *stream) {
    if (!buf_dev || !out_dev || bytes < 16 || grid < 1 || grid > 65536 || ((uintptr_t)buf_dev & 15u))
        return QW3_INVALID_ARGUMENT;
    hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint4 *)buf_dev,
                       bytes / 16, out_dev);
    return hipGetLastError() == hipSuccess ? QW3_OK : QW3_DEVICE_ERROR;
}

int32_t qw3_probe_mfma_f16(int32_t iters, int32_t grid, float *out_dev, void *stream) {
    if (!out_dev || iters < 1 || grid < 1 || grid > 65536) return QW3_INVALID_ARGUMENT;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, out_dev);
    return hipGetLastError() == hipSuccess ? QW3_OK : QW3_DEVICE_ERROR;
}

}  // extern "C"
