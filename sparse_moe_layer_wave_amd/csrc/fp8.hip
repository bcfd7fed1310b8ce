// FP8 (OCP e4m3) path: per-row activation quantisation and the grouped
// expert GEMMs on fp8 MFMA.  Formats: "DeepSeek V4-Flash architecture Q&A",
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

}  // namespace

hipError_t launch_quant_rows(const uint16_t* x, int rows, int cols, uint8_t* q, float* s,
                             hipStream_t st) {
    hipLaunchKernelGGL(k_quant_rows_bf16, dim3(rows), dim3(kQThreads), 0, st, x, cols, q, s);
    return hipGetLastError();
}

}  // namespace hy3
