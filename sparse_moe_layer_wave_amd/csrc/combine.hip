// Weighted combine / un-permute in fp32: out[t] = sum_j w[t,j] * y[row_of[t,j]],
// the k terms added in slot order with fp32 fused multiply-adds (bf16 expert
// outputs are widened to fp32 before the sum, as the fp32-combine option of
// the wmrh.cn Hy3 assembly blog, section 2.3, describes; the weighted sum of
// "DeepSeek V4-Flash architecture Q&A", Q8.4).  With the full block's shared
// expert ("Tencent Hy3-Flash Q&A", Q4.7) its output row for the token is
// added last, with weight 1.  Memory-bound: k (+1) bf16 rows in, one fp32 row
// out per token; the k row loads of a column chunk are issued together.
//
// The bf16-output form also ends the decoder layer's residual branch (the
// same blog: the residual add of section 3.2, done as section 2.3 describes
// the fp32 combine): the sum above, then the bf16 residual row widened to
// fp32 and added, and one rounding (nearest even) back to bf16.  The residual is read and the output written by the
// same thread, element for element, so the output may overwrite the residual.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kThreads = 256;

// K: the number of routed slots (compile time, so that all of a column
// chunk's K row loads are in flight before the sums, which keep slot order).
template <bool BF16_OUT, int K>
__global__ __launch_bounds__(kThreads) void k_combine(const uint16_t* __restrict__ y,
                                                     const int32_t* __restrict__ row_of,
                                                     const float* __restrict__ w,
                                                     const uint16_t* resid, void* out, int d,
                                                     int shared_row0) {
    const int t = blockIdx.x;
    __shared__ int s_row[16];
    __shared__ float s_w[16];
    if (static_cast<int>(threadIdx.x) < K) {
        s_row[threadIdx.x] = row_of[static_cast<size_t>(t) * K + threadIdx.x];
        s_w[threadIdx.x] = w[static_cast<size_t>(t) * K + threadIdx.x];
    }
    __syncthreads();
    for (int c = threadIdx.x * 8; c < d; c += kThreads * 8) {
        uint4 v[K];
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = *reinterpret_cast<const uint4*>(y + static_cast<size_t>(s_row[j]) * d + c);
        uint4 vs = make_uint4(0, 0, 0, 0);
        if (shared_row0 >= 0) vs = *reinterpret_cast<const uint4*>(y + (static_cast<size_t>(shared_row0) + t) * d + c);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float wj = s_w[j];
            const uint32_t p[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(wj, __uint_as_float(p[i] << 16), acc[2 * i]);
                acc[2 * i + 1] = fmaf(wj, __uint_as_float(p[i] & 0xffff0000u), acc[2 * i + 1]);
            }
        }
        if (shared_row0 >= 0) {
            const uint32_t p[4] = {vs.x, vs.y, vs.z, vs.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += __uint_as_float(p[i] << 16);
                acc[2 * i + 1] += __uint_as_float(p[i] & 0xffff0000u);
            }
        }
        if constexpr (BF16_OUT) {
            const size_t at = static_cast<size_t>(t) * d + c;
            if (resid) {
                const uint4 r = *reinterpret_cast<const uint4*>(resid + at);
                const uint32_t p[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += __uint_as_float(p[i] << 16);
                    acc[2 * i + 1] += __uint_as_float(p[i] & 0xffff0000u);
                }
            }
            uint32_t q[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                q[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
                       (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + at) = make_uint4(q[0], q[1], q[2], q[3]);
        } else {
            float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + static_cast<size_t>(t) * d + c);
            o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    }
}

template <bool BF16_OUT>
hipError_t launch_k(const uint16_t* y, const int32_t* row_of, const float* w, const uint16_t* resid,
                    void* out, int T, int d, int k, int shared_row0, hipStream_t s) {
    if (T == 0) return hipSuccess;
#define HY3_COMBINE_K(KK)                                                                                    \
    case KK:                                                                                                 \
        hipLaunchKernelGGL((k_combine<BF16_OUT, KK>), dim3(T), dim3(kThreads), 0, s, y, row_of, w, resid, out, d, \
                           shared_row0);                                                                    \
        break;
    switch (k) {
        HY3_COMBINE_K(1) HY3_COMBINE_K(2) HY3_COMBINE_K(3) HY3_COMBINE_K(4) HY3_COMBINE_K(5) HY3_COMBINE_K(6)
        HY3_COMBINE_K(7) HY3_COMBINE_K(8) HY3_COMBINE_K(9) HY3_COMBINE_K(10) HY3_COMBINE_K(11) HY3_COMBINE_K(12)
        HY3_COMBINE_K(13) HY3_COMBINE_K(14) HY3_COMBINE_K(15) HY3_COMBINE_K(16)
        default: return hipErrorInvalidValue;
    }
#undef HY3_COMBINE_K
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, const int32_t* row_of, const float* w, float* out,
                          int T, int d, int k, int shared_row0, hipStream_t s) {
    return launch_k<false>(y, row_of, w, nullptr, static_cast<void*>(out), T, d, k, shared_row0, s);
}

hipError_t launch_combine_bf16(const uint16_t* y, const int32_t* row_of, const float* w,
                               const uint16_t* resid, uint16_t* out, int T, int d, int k,
                               int shared_row0, hipStream_t s) {
    return launch_k<true>(y, row_of, w, resid, static_cast<void*>(out), T, d, k, shared_row0, s);
}

}  // namespace hy3
