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

// Four codes of one 8-byte group of bf16 pairs (p = two bf16 values).
__device__ __forceinline__ uint32_t quant_pair2(uint32_t p0, uint32_t p1, float r) {
    return static_cast<uint32_t>(f32_to_e4m3(__uint_as_float(p0 << 16) * r)) |
           (static_cast<uint32_t>(f32_to_e4m3(__uint_as_float(p0 & 0xffff0000u) * r)) << 8) |
           (static_cast<uint32_t>(f32_to_e4m3(__uint_as_float(p1 << 16) * r)) << 16) |
           (static_cast<uint32_t>(f32_to_e4m3(__uint_as_float(p1 & 0xffff0000u) * r)) << 24);
}

__device__ __forceinline__ float amax8(const uint4& v, float m) {
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, fabsf(__uint_as_float(p[i] << 16)));
        m = fmaxf(m, fabsf(__uint_as_float(p[i] & 0xffff0000u)));
    }
    return m;
}

// One workgroup per row of bf16 input; a thread takes 8 values per step of
// kQThreads * 8 columns.  Rows of at most NV steps are read once, into
// registers (NV > 0); longer rows (NV = 0) are read twice, for the max and
// for the codes.  rs, if not NULL, also receives the row's scale at each of
// its k dispatch rows (row_of[row * k + j], skipped where negative), so that
// the grouped gate_up reads a row scale without going through the token.
template <int NV>
__global__ __launch_bounds__(kQThreads) void k_quant_rows_bf16(const uint16_t* __restrict__ x,
                                                              int cols, uint8_t* __restrict__ q,
                                                              float* __restrict__ s,
                                                              const int32_t* __restrict__ row_of, int k,
                                                              float* __restrict__ rs) {
    __shared__ float lds[kQThreads / 64];
    const size_t row = blockIdx.x;
    const uint16_t* xr = x + row * cols;
    uint8_t* qr = q + row * cols;
    float amax = 0.f;
    if constexpr (NV > 0) {
        uint4 v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = (i * kQThreads + threadIdx.x) * 8;
            v[i] = c < cols ? *reinterpret_cast<const uint4*>(xr + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) amax = amax8(v[i], amax);
        amax = block_max(amax, lds);
        const float r = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = (i * kQThreads + threadIdx.x) * 8;
            if (c < cols)
                *reinterpret_cast<uint2*>(qr + c) = make_uint2(quant_pair2(v[i].x, v[i].y, r), quant_pair2(v[i].z, v[i].w, r));
        }
    } else {
        for (int c = threadIdx.x * 8; c < cols; c += kQThreads * 8)
            amax = amax8(*reinterpret_cast<const uint4*>(xr + c), amax);
        amax = block_max(amax, lds);
        const float r = amax > 0.f ? 448.0f / amax : 0.f;
        for (int c = threadIdx.x * 8; c < cols; c += kQThreads * 8) {
            const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
            *reinterpret_cast<uint2*>(qr + c) = make_uint2(quant_pair2(v.x, v.y, r), quant_pair2(v.z, v.w, r));
        }
    }
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    if (threadIdx.x == 0) s[row] = scale;
    if (rs && static_cast<int>(threadIdx.x) < k) {
        const int r = row_of[row * k + threadIdx.x];
        if (r >= 0) rs[r] = scale;
    }
}

// h rows (bf16) with their max |h| already reduced into amax (bit patterns
// of the float), or (amax_bits NULL) given as nblk partial maxima per row,
// hmax[blk * rows + row]: the same quantiser as above, one wave per row
// (kQThreads / 64 rows per workgroup); a lane takes 8 values per step of 512
// columns and keeps up to 8 steps' loads in flight.
constexpr int kRowsPerWg = kQThreads / 64;

__global__ __launch_bounds__(kQThreads) void k_quant_rows_h(const uint16_t* __restrict__ h,
                                                           const uint32_t* __restrict__ amax_bits,
                                                           const float* __restrict__ hmax, int nblk,
                                                           int rows, int cols, uint8_t* __restrict__ q,
                                                           float* __restrict__ s) {
    const size_t row = static_cast<size_t>(blockIdx.x) * kRowsPerWg + (threadIdx.x >> 6);
    if (row >= static_cast<size_t>(rows)) return;
    const int lane = threadIdx.x & 63;
    float amax;
    if (amax_bits) {
        amax = __uint_as_float(amax_bits[row]);
    } else {
        float m = 0.f;
        for (int b = lane; b < nblk; b += 64) m = fmaxf(m, hmax[static_cast<size_t>(b) * rows + row]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        amax = m;
    }
    const float r = amax > 0.f ? 448.0f / amax : 0.f;
    const uint16_t* hr = h + row * cols;
    uint8_t* qr = q + row * cols;
    for (int base = 0; base < cols; base += 8 * 512) {
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = base + (i * 64 + lane) * 8;
            v[i] = c < cols ? *reinterpret_cast<const uint4*>(hr + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = base + (i * 64 + lane) * 8;
            if (c < cols)
                *reinterpret_cast<uint2*>(qr + c) = make_uint2(quant_pair2(v[i].x, v[i].y, r), quant_pair2(v[i].z, v[i].w, r));
        }
    }
    if (lane == 0) s[row] = amax > 0.f ? amax / 448.0f : 1.0f;
}

}  // namespace

hipError_t launch_quant_rows_h(const uint16_t* h, const uint32_t* amax_bits, const float* hmax, int nblk,
                               int rows, int cols, uint8_t* q, float* s, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const unsigned wgs = static_cast<unsigned>((static_cast<long long>(rows) + kRowsPerWg - 1) / kRowsPerWg);
    hipLaunchKernelGGL(k_quant_rows_h, dim3(wgs), dim3(kQThreads), 0, st, h, amax_bits, hmax, nblk, rows, cols,
                       q, s);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int rows, int cols, uint8_t* q, float* s,
                             hipStream_t st, const int32_t* row_of, int k, float* rs) {
    if (rows == 0) return hipSuccess;
    if (k > kQThreads) return hipErrorInvalidValue;
    const int steps = (cols + kQThreads * 8 - 1) / (kQThreads * 8);
#define HY3_QROWS(NV) \
    hipLaunchKernelGGL(k_quant_rows_bf16<NV>, dim3(rows), dim3(kQThreads), 0, st, x, cols, q, s, row_of, k, rs)
    if (steps <= 1) HY3_QROWS(1);
    else if (steps <= 2) HY3_QROWS(2);
    else if (steps <= 4) HY3_QROWS(4);
    else HY3_QROWS(0);
#undef HY3_QROWS
    return hipGetLastError();
}

}  // namespace hy3
