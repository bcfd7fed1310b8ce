// Expert GEMMs for decode-sized batches: each expert sees a handful of rows,
// so the work is streaming the touched experts' weights from HBM once.
//
// One workgroup = one expert x one slice of weight rows; 4 waves, each owning
// 32 weight rows over the full K and the expert's rows 16 at a time
// (v_mfma_f32_16x16x32_bf16: A = 16 token rows x 32 k, B = 32 k x 16 weight
// rows; lane l holds row l%16 and k 8*(l/16)..+8 of both; C lane l holds
// column l%16, rows 4*(l/16)..+4).  Weights go straight from global memory to
// registers (no reuse, so no LDS): each wave keeps kDepth k-steps of weight
// fragments in flight, 8 KB per k-step group per wave.
//
// gate_up: wave w of block (e, c0) owns gate rows c0+16w..+16 and the matching
//          up rows F+c0+16w..+16, and writes h[r, c] = bf16(SiLU(g) * u)
//          ("DeepSeek V4-Flash architecture Q&A", Q4.5).
// down:    wave w of block (e, n0) owns W_down rows n0+32w..+32 and writes
//          y[r, n] = bf16(h[r] . W_down[e][n]).
// An expert with more than 16 rows is handled in passes of 16 rows.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kDepth = 8;       // k-steps (of 32) loaded before their MFMAs

union Frag {
    bf16x8_t v;
    i32x4_t q;
};

template <bool GATE_UP>
__global__ __launch_bounds__(256) void k_decode_gemm(
    const uint16_t* __restrict__ A,        // gate_up: x [T, K]; down: h [rows, K]
    const int32_t* __restrict__ tok_of,    // gate_up only
    const uint16_t* __restrict__ W,        // gate_up: [E, 2N, K]; down: [E, N, K]
    const int32_t* __restrict__ offsets,
    uint16_t* __restrict__ C,              // gate_up: h [rows, N]; down: y [rows, N]
    int K, int N) {
    const int e = blockIdx.x;
    const int rbeg = offsets[e];
    const int rend = offsets[e + 1];
    if (rbeg == rend) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int kq = (lane >> 4) * 8;

    // this lane's two weight rows (one per n-tile) and its output column(s)
    int wrow0, wrow1, col0, col1;
    if (GATE_UP) {
        const int c = blockIdx.y * 64 + wave * 16 + r16;
        wrow0 = c;
        wrow1 = N + c;
        col0 = blockIdx.y * 64 + wave * 16;
        col1 = col0;
    } else {
        const int n = blockIdx.y * 128 + wave * 32;
        wrow0 = n + r16;
        wrow1 = n + 16 + r16;
        col0 = n;
        col1 = n + 16;
    }
    const size_t wbase = static_cast<size_t>(e) * (GATE_UP ? 2 * N : N) * K;
    const uint16_t* w0 = W + wbase + static_cast<size_t>(wrow0) * K + kq;
    const uint16_t* w1 = W + wbase + static_cast<size_t>(wrow1) * K + kq;

    for (int p0 = rbeg; p0 < rend; p0 += 16) {
        const int prow = p0 + r16;                    // A row this lane loads
        const bool va = prow < rend;
        const uint16_t* a;
        if (GATE_UP) a = A + static_cast<size_t>(va ? tok_of[prow] : 0) * K + kq;
        else a = A + static_cast<size_t>(va ? prow : 0) * K + kq;

        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
        f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < K; kb += 32 * kDepth) {
            i32x4_t b0[kDepth], b1[kDepth], av[kDepth];
#pragma unroll
            for (int u = 0; u < kDepth; ++u) {
                const int kk = kb + 32 * u;
                if (kk < K) {
                    b0[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(w0 + kk));
                    b1[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(w1 + kk));
                    av[u] = va ? *reinterpret_cast<const i32x4_t*>(a + kk) : i32x4_t{0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int u = 0; u < kDepth; ++u) {
                if (kb + 32 * u < K) {
                    Frag fa, f0, f1;
                    fa.q = av[u];
                    f0.q = b0[u];
                    f1.q = b1[u];
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.v, f0.v, acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.v, f1.v, acc1, 0, 0, 0);
                }
            }
        }
        // C lane l: column l%16, rows 4*(l/16)+i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = p0 + (lane >> 4) * 4 + i;
            if (row < rend) {
                if (GATE_UP) {
                    C[static_cast<size_t>(row) * N + col0 + r16] = f32_to_bf16(silu_mul(acc0[i], acc1[i]));
                } else {
                    C[static_cast<size_t>(row) * N + col0 + r16] = f32_to_bf16(acc0[i]);
                    C[static_cast<size_t>(row) * N + col1 + r16] = f32_to_bf16(acc1[i]);
                }
            }
        }
    }
}

}  // namespace

// Decode path while the average expert gets at most 4 rows (so nearly every
// expert fits one 16-row pass); needs d to be a multiple of 128.
bool use_decode_path(int T, int d, int E, int k) {
    return static_cast<long long>(T) * k <= 4LL * E && (d % 128) == 0;
}

hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                                 const int32_t* offsets, uint16_t* h, int E, int d, int F,
                                 hipStream_t s) {
    hipLaunchKernelGGL(k_decode_gemm<true>, dim3(E, F / 64), dim3(256), 0, s, x, tok_of, W_gu,
                       offsets, h, d, F);
    return hipGetLastError();
}

hipError_t launch_down_decode(const uint16_t* h, const uint16_t* W_dn, const int32_t* offsets,
                              uint16_t* y, int E, int d, int F, hipStream_t s) {
    hipLaunchKernelGGL(k_decode_gemm<false>, dim3(E, d / 128), dim3(256), 0, s, h, nullptr, W_dn,
                       offsets, y, F, d);
    return hipGetLastError();
}

}  // namespace hy3
