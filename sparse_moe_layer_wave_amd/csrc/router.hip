// Router of the Hy3 MoE layer: fp32 logits, sigmoid scores, top-k selection
// and the renormalised, scaled weights ("Tencent Hy3-295B architecture
// teardown", section 4.1, router flow steps 1, 3, 4 and 5).
//
// Logits.  The gate weight is fp32 and the hidden states are bf16; the pages'
// router casts both to float before the linear map.  Each fp32 weight w is
// split into three bf16 parts by truncation, w = hi + mid + lo exactly (8
// significant bits each), so x.w = x.hi + x.mid + x.lo with every product
// exact in fp32.  That runs on bf16 MFMA with fp32 accumulation: an
// fp32-accurate GEMM for three times the bf16 work.  Small batches split the
// d-sum into nsplit chunks (partial logits [nsplit, T, E]) so enough
// workgroups stream W_gate; the selection kernel adds the chunks in a fixed
// order, so the result does not depend on scheduling.
//
// Selection.  Scores lie in [0, 1], so their fp32 bit patterns order like the
// values; key = (score bits << 32) | ~expert makes "largest score, then lowest
// expert index" a plain 64-bit maximum.  Sixteen lanes (one DPP row) serve
// one token: each scans every 16th expert for its best untaken key, the row
// takes the maximum with row_ror DPP moves, k times.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kScoreTokens = 64;    // tokens per workgroup (4 waves x 16)
constexpr int kScoreExperts = 32;   // experts per workgroup (2 MFMA n-tiles)
constexpr int kKStep = 32;          // d elements per MFMA
constexpr int kUnroll = 4;          // k-steps whose loads are issued together

__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
    const uint32_t u = __float_as_uint(w);
    const uint32_t uh = u & 0xffff0000u;
    const float r1 = w - __uint_as_float(uh);          // exact: <= 16 significant bits left
    const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(um);          // exact: <= 8 significant bits left
    hi = static_cast<uint16_t>(uh >> 16);
    mid = static_cast<uint16_t>(um >> 16);
    lo = static_cast<uint16_t>(__float_as_uint(r2) >> 16);   // r2 fits bf16 exactly
}

union Frag {
    bf16x8_t v;
    uint16_t h[8];
    uint4 q;
};

// partial[s, t, e] = sum over i in chunk s of x[t,i] W[e,i].
// MFMA 16x16x32: A = 16 tokens x 32 k (lane l: token l%16, k 8*(l/16)..+8),
// B = 32 k x 16 experts (lane l: expert l%16, same k); C lane l holds expert
// l%16 for tokens 4*(l/16)..+4.
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ Wg,
                                                       float* __restrict__ partial, int T, int d,
                                                       int E, int kchunk) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kScoreTokens + wave * 16;
    const int e0 = blockIdx.y * kScoreExperts;
    const int k0 = blockIdx.z * kchunk;
    const int r = lane & 15;
    const int kg = lane >> 4;

    const int ta = t0 + r;
    const bool va = ta < T;
    const uint16_t* xa = x + static_cast<size_t>(va ? ta : 0) * d + k0 + kg * 8;
    const float* wb[2];
    bool vb[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int e = e0 + nt * 16 + r;
        vb[nt] = e < E;
        wb[nt] = Wg + static_cast<size_t>(vb[nt] ? e : 0) * d + k0 + kg * 8;
    }

    f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (int kb = 0; kb < kchunk; kb += kKStep * kUnroll) {
        uint4 av[kUnroll];
        float4 wv[kUnroll][2][2];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int kk = kb + u * kKStep;
            const bool in = kk < kchunk;                   // kchunk is a multiple of 32
            av[u] = va && in ? *reinterpret_cast<const uint4*>(xa + kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                if (vb[nt] && in) {
                    wv[u][nt][0] = *reinterpret_cast<const float4*>(wb[nt] + kk);
                    wv[u][nt][1] = *reinterpret_cast<const float4*>(wb[nt] + kk + 4);
                } else {
                    wv[u][nt][0] = wv[u][nt][1] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (kb + u * kKStep >= kchunk) break;
            Frag a;
            a.q = av[u];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const float w8[8] = {wv[u][nt][0].x, wv[u][nt][0].y, wv[u][nt][0].z,
                                     wv[u][nt][0].w, wv[u][nt][1].x, wv[u][nt][1].y,
                                     wv[u][nt][1].z, wv[u][nt][1].w};
                Frag bh, bm, bl;
#pragma unroll
                for (int i = 0; i < 8; ++i) split3(w8[i], bh.h[i], bm.h[i], bl.h[i]);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bh.v, acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bm.v, acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bl.v, acc[nt], 0, 0, 0);
            }
        }
    }

    float* out = partial + static_cast<size_t>(blockIdx.z) * T * E;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int e = e0 + nt * 16 + r;
        if (e >= E) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + kg * 4 + i;
            if (t < T) out[static_cast<size_t>(t) * E + e] = acc[nt][i];
        }
    }
}

// 64-bit maximum over the 16 lanes of a DPP row (row_ror by 8, 4, 2, 1).
__device__ __forceinline__ unsigned long long row16_max(unsigned long long v) {
#define HY3_ROR_STEP(CTRL)                                                                        \
    {                                                                                             \
        const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(v & 0xffffffffull), CTRL,  \
                                                   0xf, 0xf, false);                              \
        const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(v >> 32), CTRL, 0xf, 0xf,  \
                                                   false);                                        \
        const unsigned long long o =                                                              \
            (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |                  \
            static_cast<uint32_t>(lo);                                                            \
        v = o > v ? o : v;                                                                        \
    }
    HY3_ROR_STEP(0x128)   // row_ror:8
    HY3_ROR_STEP(0x124)   // row_ror:4
    HY3_ROR_STEP(0x122)   // row_ror:2
    HY3_ROR_STEP(0x121)   // row_ror:1
#undef HY3_ROR_STEP
    return v;
}

constexpr int kSelThreads = 1024;   // 16 waves x 4 tokens = 64 tokens (one routing block)

// Sums the partial logits, adds the bias and applies the sigmoid into an LDS
// tile [tb tokens][E + 1] (tb = 64 when E is small; larger E takes the block's
// 64 tokens in sub-batches), then selects k experts per token, 16 lanes each.
// Writes idx/w and, when blk_counts is given, the block's per-expert pair count.
__global__ __launch_bounds__(kSelThreads) void k_router_select(
    const float* __restrict__ partial, int nsplit, const float* __restrict__ bias, int T, int E,
    int k, float scale, int tb, int32_t* __restrict__ idx, float* __restrict__ wout,
    int32_t* __restrict__ blk_counts, int nb) {
    extern __shared__ uint32_t s_score[];              // [tb][E + 1]
    __shared__ unsigned long long mask[1024];
    const int tid = threadIdx.x;
    const int ld = E + 1;
    const size_t plane = static_cast<size_t>(T) * E;
    for (int e = tid; e < E; e += kSelThreads) mask[e] = 0ull;
    const int lane = tid & 63;
    const int j = lane & 15;                              // lane within the token's row
    const int ts = (tid >> 6) * 4 + (lane >> 4);          // token slot within a sub-batch

    for (int sb = 0; sb < kRouteBlock; sb += tb) {
        const int t_first = blockIdx.x * kRouteBlock + sb;
        const int ntok = min(tb, T - t_first);
        if (ntok <= 0) break;
        __syncthreads();
        for (int p = tid; p < ntok * E; p += kSelThreads) {
            const int tl = p / E;
            const int e = p - tl * E;
            const size_t off = static_cast<size_t>(t_first + tl) * E + e;
            float z = 0.f;
            for (int s = 0; s < nsplit; ++s) z += partial[s * plane + off];
            if (bias) z += bias[e];
            s_score[tl * ld + e] = __float_as_uint(1.0f / (1.0f + expf(-z)));
        }
        __syncthreads();

        const bool active = ts < ntok;
        const uint32_t* srow = s_score + (active ? ts : 0) * ld;
        unsigned long long taken = 0ull;                   // bit q: expert j + 16q chosen
        int my_e = 0;
        float my_s = 0.f, sum = 0.f;
        for (int r = 0; r < k; ++r) {
            unsigned long long best = 0ull;
            if (active) {
                for (int q = 0, e = j; e < E; ++q, e += 16) {
                    if (!((taken >> q) & 1ull)) {
                        const unsigned long long key =
                            (static_cast<unsigned long long>(srow[e]) << 32) |
                            static_cast<uint32_t>(~static_cast<uint32_t>(e));
                        best = key > best ? key : best;
                    }
                }
            }
            best = row16_max(best);
            const int e_win = static_cast<int>(~static_cast<uint32_t>(best & 0xffffffffull));
            const float s_win = __uint_as_float(static_cast<uint32_t>(best >> 32));
            if ((e_win & 15) == j) taken |= 1ull << (e_win >> 4);
            if (r == j) {
                my_e = e_win;
                my_s = s_win;
            }
            sum += s_win;                                  // slot order, same in every lane
        }
        if (active && j < k) {
            const size_t pair = static_cast<size_t>(t_first + ts) * k + j;
            idx[pair] = my_e;
            wout[pair] = scale * (my_s / sum);
            atomicOr(&mask[my_e], 1ull << (sb + ts));
        }
    }
    if (blk_counts) {
        __syncthreads();
        for (int e = tid; e < E; e += kSelThreads)
            blk_counts[static_cast<size_t>(e) * nb + blockIdx.x] = __popcll(mask[e]);
    }
}

int select_tokens_per_pass(int E) {
    int tb = kRouteBlock;
    while (tb > 8 && static_cast<size_t>(tb) * (E + 1) * sizeof(uint32_t) > 65536) tb >>= 1;
    return tb;
}

}  // namespace

int router_nsplit(int T, int d, int E) {
    const int wgs = ((T + kScoreTokens - 1) / kScoreTokens) * ((E + kScoreExperts - 1) / kScoreExperts);
    int ns = 1;
    const int chunk_min = kKStep * kUnroll;                  // 128
    while (wgs * ns < 256 && (d % (2 * ns * chunk_min)) == 0 && d / (2 * ns) >= chunk_min) ns *= 2;
    return ns;
}


hipError_t launch_router(const uint16_t* x, const float* W_gate, const float* bias, int T, int d,
                         int E, int k, float scale, float* partial, int nsplit, int32_t* idx,
                         float* w, int32_t* blk_counts, int nb, hipStream_t s) {
    dim3 g1((T + kScoreTokens - 1) / kScoreTokens, (E + kScoreExperts - 1) / kScoreExperts, nsplit);
    hipLaunchKernelGGL(k_router_logits, g1, dim3(256), 0, s, x, W_gate, partial, T, d, E,
                       d / nsplit);
    const int tb = select_tokens_per_pass(E);
    hipLaunchKernelGGL(k_router_select, dim3(nb), dim3(kSelThreads),
                       static_cast<size_t>(tb) * (E + 1) * sizeof(uint32_t), s, partial, nsplit,
                       bias, T, E, k, scale, tb, idx, w, blk_counts, nb);
    return hipGetLastError();
}

}  // namespace hy3
