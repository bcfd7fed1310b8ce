// Router of the Hy3 MoE layer: fp32 logits, sigmoid scores, top-k selection
// and the renormalised, scaled weights ("Tencent Hy3-295B architecture
// teardown", section 4.1, router flow steps 1, 3, 4 and 5).
//
// Logits.  The gate weight is fp32 and the hidden states are bf16; the pages'
// router casts both to float before the linear map.  Each fp32 weight w is
// split into three bf16 parts by truncation, w = hi + mid + lo exactly (8
// significant bits each), so x.w = x.hi + x.mid + x.lo with every product
// exact in fp32.  That runs on bf16 MFMA with fp32 accumulation and gives an
// fp32-accurate GEMM for three times the bf16 work -- a few microseconds here.
//
// Selection.  Scores lie in [0, 1], so their fp32 bit patterns order like the
// values; key = (score bits << 32) | ~expert makes "largest score, then lowest
// expert index" a plain 64-bit maximum, taken k times across the wavefront.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kScoreTokens = 64;    // tokens per workgroup (4 waves x 16)
constexpr int kScoreExperts = 32;   // experts per workgroup (2 MFMA n-tiles)

__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
    uint32_t u = __float_as_uint(w);
    uint32_t uh = u & 0xffff0000u;
    float r1 = w - __uint_as_float(uh);           // exact: at most 16 significant bits left
    uint32_t um = __float_as_uint(r1) & 0xffff0000u;
    float r2 = r1 - __uint_as_float(um);          // exact: at most 8 significant bits left
    hi = static_cast<uint16_t>(uh >> 16);
    mid = static_cast<uint16_t>(um >> 16);
    lo = static_cast<uint16_t>(__float_as_uint(r2) >> 16);   // r2 fits bf16 exactly
}

union Frag {
    bf16x8_t v;
    uint16_t h[8];
    uint4 q;
};

// scores[t, e] = sigmoid(sum_i x[t,i] W[e,i] + bias[e]) for a 64 x 32 block.
// MFMA 16x16x32: A = 16 tokens x 32 k (lane l: token l%16, k 8*(l/16)..+8),
// B = 32 k x 16 experts (lane l: expert l%16, same k), C lane l: expert l%16,
// tokens 4*(l/16)..+4.
__global__ __launch_bounds__(256) void k_router_scores(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ Wg,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ scores, int T, int d,
                                                       int E) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kScoreTokens + wave * 16;
    const int e0 = blockIdx.y * kScoreExperts;
    const int r = lane & 15;
    const int kg = lane >> 4;

    const int ta = t0 + r;
    const bool va = ta < T;
    const uint16_t* xa = x + static_cast<size_t>(va ? ta : 0) * d + kg * 8;
    const float* wb[2];
    bool vb[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int e = e0 + nt * 16 + r;
        vb[nt] = e < E;
        wb[nt] = Wg + static_cast<size_t>(vb[nt] ? e : 0) * d + kg * 8;
    }

    f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (int kb = 0; kb < d; kb += 32) {
        Frag a;
        a.q = va ? *reinterpret_cast<const uint4*>(xa + kb) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float4 w0 = make_float4(0.f, 0.f, 0.f, 0.f), w1 = w0;
            if (vb[nt]) {
                w0 = *reinterpret_cast<const float4*>(wb[nt] + kb);
                w1 = *reinterpret_cast<const float4*>(wb[nt] + kb + 4);
            }
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            Frag bh, bm, bl;
#pragma unroll
            for (int i = 0; i < 8; ++i) split3(wv[i], bh.h[i], bm.h[i], bl.h[i]);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bh.v, acc[nt], 0, 0, 0);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bm.v, acc[nt], 0, 0, 0);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bl.v, acc[nt], 0, 0, 0);
        }
    }

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int e = e0 + nt * 16 + r;
        if (e >= E) continue;
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + kg * 4 + i;
            if (t < T) {
                const float z = acc[nt][i] + b;
                scores[static_cast<size_t>(t) * E + e] = 1.0f / (1.0f + expf(-z));
            }
        }
    }
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const int lo = __shfl_xor(static_cast<int>(v & 0xffffffffull), off, 64);
        const int hi = __shfl_xor(static_cast<int>(v >> 32), off, 64);
        const unsigned long long o =
            (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |
            static_cast<uint32_t>(lo);
        v = o > v ? o : v;
    }
    return v;
}

// One wavefront per token, 16 tokens per wave, 64 tokens per workgroup (one
// routing block).  Writes idx/w and the block's per-expert pair count.
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ scores, int T,
                                                     int E, int k, float scale,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ wout,
                                                     int32_t* __restrict__ blk_counts, int nb) {
    __shared__ unsigned long long mask[1024];
    for (int e = threadIdx.x; e < E; e += 256) mask[e] = 0ull;
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int i = 0; i < 16; ++i) {
        const int tl = wave * 16 + i;
        const int t = blockIdx.x * kRouteBlock + tl;
        if (t >= T) break;
        const float* srow = scores + static_cast<size_t>(t) * E;
        uint32_t sb[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int e = q * 64 + lane;
            sb[q] = e < E ? __float_as_uint(srow[e]) : 0u;
        }
        uint32_t taken = 0;
        int sel_e[16];
        float sel_s[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j < k) {
                unsigned long long best = 0ull;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int e = q * 64 + lane;
                    if (e < E && !((taken >> q) & 1u)) {
                        const unsigned long long key =
                            (static_cast<unsigned long long>(sb[q]) << 32) |
                            static_cast<uint32_t>(~static_cast<uint32_t>(e));
                        best = key > best ? key : best;
                    }
                }
                best = wave_max_u64(best);
                const int e_win = static_cast<int>(~static_cast<uint32_t>(best & 0xffffffffull));
                if ((e_win & 63) == lane) taken |= 1u << (e_win >> 6);
                sel_e[j] = e_win;
                sel_s[j] = __uint_as_float(static_cast<uint32_t>(best >> 32));
            }
        }
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (j < k) sum += sel_s[j];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j < k && lane == j) {
                idx[static_cast<size_t>(t) * k + j] = sel_e[j];
                wout[static_cast<size_t>(t) * k + j] = scale * (sel_s[j] / sum);
                atomicOr(&mask[sel_e[j]], 1ull << tl);
            }
        }
    }
    __syncthreads();
    if (blk_counts) {
        for (int e = threadIdx.x; e < E; e += 256)
            blk_counts[static_cast<size_t>(e) * nb + blockIdx.x] = __popcll(mask[e]);
    }
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const float* W_gate, const float* bias, int T, int d,
                         int E, int k, float scale, float* scores, int32_t* idx, float* w,
                         int32_t* blk_counts, int nb, hipStream_t s) {
    dim3 g1((T + kScoreTokens - 1) / kScoreTokens, (E + kScoreExperts - 1) / kScoreExperts);
    hipLaunchKernelGGL(k_router_scores, g1, dim3(256), 0, s, x, W_gate, bias, scores, T, d, E);
    hipLaunchKernelGGL(k_router_topk, dim3(nb), dim3(256), 0, s, scores, T, E, k, scale, idx, w,
                       blk_counts, nb);
    return hipGetLastError();
}

}  // namespace hy3
