// FP8 (OCP e4m3) path: per-row activation quantisation (the grouped expert
// GEMMs on fp8 MFMA are in gemm_grouped.hip).  Formats: "DeepSeek V4-Flash architecture Q&A",
// Q7.2 (E4M3, range +-448) and Q7.4 (one scale per output channel).
//
// Row quantiser: amax = max|v|; amax == 0 -> codes 0, scale 1; otherwise
// r = fp32(448 / amax) (IEEE division), code = e4m3(fp32(v * r)), scale =
// fp32(amax / 448).  The row dequantises as code * scale.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kQThreads = 256;

__device__ float block_max(float v, float* lds) {
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    v = lds[0];
    for (int i = 1; i < kQThreads / 64; ++i) v = fmaxf(v, lds[i]);
    __syncthreads();
    return v;
}

// One workgroup per row of bf16 input.
__global__ __launch_bounds__(kQThreads) void k_quant_rows_bf16(const uint16_t* __restrict__ x,
                                                              int cols, uint8_t* __restrict__ q,
                                                              float* __restrict__ s) {
    __shared__ float lds[kQThreads / 64];
    const size_t row = blockIdx.x;
    const uint16_t* xr = x + row * cols;
    float amax = 0.f;
    for (int c = threadIdx.x * 8; c < cols; c += kQThreads * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(__uint_as_float(p[i] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(p[i] & 0xffff0000u)));
        }
    }
    amax = block_max(amax, lds);
    const float r = amax > 0.f ? 448.0f / amax : 0.f;
    for (int c = threadIdx.x * 8; c < cols; c += kQThreads * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t c0 = f32_to_e4m3(__uint_as_float(p[i] << 16) * r);
            const uint32_t c1 = f32_to_e4m3(__uint_as_float(p[i] & 0xffff0000u) * r);
            const uint32_t pair = c0 | (c1 << 8);
            if (i < 2) lo |= pair << (16 * i);
            else hi |= pair << (16 * (i - 2));
        }
        *reinterpret_cast<uint2*>(q + row * cols + c) = make_uint2(lo, hi);
    }
    if (threadIdx.x == 0) s[row] = amax > 0.f ? amax / 448.0f : 1.0f;
}

// h rows (fp32) with their max |h| already reduced into amax (bit patterns):
// the same quantiser as above, one workgroup per row.
__global__ __launch_bounds__(kQThreads) void k_quant_rows_f32(const float* __restrict__ h,
                                                             const uint32_t* __restrict__ amax_bits,
                                                             int cols, uint8_t* __restrict__ q,
                                                             float* __restrict__ s) {
    const size_t row = blockIdx.x;
    const float amax = __uint_as_float(amax_bits[row]);
    const float r = amax > 0.f ? 448.0f / amax : 0.f;
    const float* hr = h + row * cols;
    for (int c = threadIdx.x * 4; c < cols; c += kQThreads * 4) {
        const float4 v = *reinterpret_cast<const float4*>(hr + c);
        const uint32_t packed = static_cast<uint32_t>(f32_to_e4m3(v.x * r)) |
                                (static_cast<uint32_t>(f32_to_e4m3(v.y * r)) << 8) |
                                (static_cast<uint32_t>(f32_to_e4m3(v.z * r)) << 16) |
                                (static_cast<uint32_t>(f32_to_e4m3(v.w * r)) << 24);
        *reinterpret_cast<uint32_t*>(q + row * cols + c) = packed;
    }
    if (threadIdx.x == 0) s[row] = amax > 0.f ? amax / 448.0f : 1.0f;
}

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t v) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * 256)
        p[i] = v;
}

}  // namespace

hipError_t launch_quant_rows_f32(const float* h, const uint32_t* amax_bits, int rows, int cols,
                                 uint8_t* q, float* s, hipStream_t st) {
    hipLaunchKernelGGL(k_quant_rows_f32, dim3(rows), dim3(kQThreads), 0, st, h, amax_bits, cols, q, s);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
    const unsigned blocks = static_cast<unsigned>(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
    hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int rows, int cols, uint8_t* q, float* s,
                             hipStream_t st) {
    hipLaunchKernelGGL(k_quant_rows_bf16, dim3(rows), dim3(kQThreads), 0, st, x, cols, q, s);
    return hipGetLastError();
}

}  // namespace hy3
