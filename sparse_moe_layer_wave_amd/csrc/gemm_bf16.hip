// Grouped expert GEMMs with bf16 weights on CDNA4 MFMA (fp32 accumulate).
//
// gate_up: for every M-tile (expert e, rows r0..r1 of the expert-contiguous
//          order) and every block of 64 intermediate columns c0..c0+63:
//          G = X[tok(r)] . Wgu[e][c]^T, U = X[tok(r)] . Wgu[e][F + c]^T,
//          h[r, c] = bf16(SiLU(G) * U).  The A rows are gathered straight from
//          x through token_of; gate and up columns of the same c sit in one
//          tile, so SiLU(gate)*up is formed in registers ("DeepSeek V4-Flash
//          architecture Q&A", Q4.5; fused gate_up layout: "Tencent Hy3-295B
//          architecture teardown", section 2.3).
// down:    y[r, n] = bf16(h[r] . Wdn[e][n]^T).
//
// Tiles: 64 rows x 64 output columns, K step 32, 4 waves in a 2 x 2 grid of
// 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_bf16).  Lane layout of that MFMA:
// A lane l holds row l%32, k 8*(l/32)..+8 of a 16-wide k slice; B lane l holds
// column l%32 and the same k; C lane l holds column l%32, rows
// 8*(j/4) + 4*(l/32) + j%4 for j = 0..15.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int BM = 64;
constexpr int BN = 64;
constexpr int BK = 32;
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements; 80-byte rows spread LDS banks

union Frag {
    bf16x8_t v;
    uint4 q;
};

template <bool GATE_UP>
__global__ __launch_bounds__(256) void k_expert_gemm(
    const uint16_t* __restrict__ A,        // gate_up: x [T, K]; down: h [rows, K]
    const int32_t* __restrict__ tok_of,    // gate_up only
    const uint16_t* __restrict__ W,        // gate_up: [E, 2F, K]; down: [E, N, K]
    const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    const int32_t* __restrict__ offsets,
    uint16_t* __restrict__ C,              // gate_up: h [rows, N=F]; down: y [rows, N=d]
    int K, int N) {
    constexpr int BROWS = GATE_UP ? 2 * BN : BN;   // weight rows per tile
    __shared__ uint16_t As[BM * LDS_STRIDE];
    __shared__ uint16_t Bs[BROWS * LDS_STRIDE];

    if (static_cast<int>(blockIdx.x) >= *ntiles) return;
    const Tile ti = tiles[blockIdx.x];
    const int e = ti.expert;
    const int row0 = ti.row0;
    const int rows = min(BM, offsets[e + 1] - row0);
    const int n0 = blockIdx.y * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;

    // global -> LDS assignment: A row tid/4, 8 k at (tid%4)*8
    const int a_r = tid >> 2;
    const int a_k = (tid & 3) * 8;
    const bool a_valid = a_r < rows;
    const uint16_t* a_src;
    if (GATE_UP) {
        const int t = a_valid ? tok_of[row0 + a_r] : 0;
        a_src = A + static_cast<size_t>(t) * K + a_k;
    } else {
        a_src = A + static_cast<size_t>(a_valid ? row0 + a_r : 0) * K + a_k;
    }
    const size_t wbase = static_cast<size_t>(e) * (GATE_UP ? 2 * N : N) * K;
    const uint16_t* b_src[BROWS / 64];
#pragma unroll
    for (int i = 0; i < BROWS / 64; ++i) {
        const int br = (tid >> 2) + 64 * i;     // 0..BROWS-1
        int wrow;
        if (GATE_UP) wrow = br < BN ? n0 + br : N + n0 + (br - BN);
        else wrow = n0 + br;
        b_src[i] = W + wbase + static_cast<size_t>(wrow) * K + a_k;
    }

    f32x16_t acc0 = {};
    f32x16_t acc1 = {};   // gate_up: the up half

    for (int kb = 0; kb < K; kb += BK) {
        const uint4 av = a_valid ? *reinterpret_cast<const uint4*>(a_src + kb) : make_uint4(0, 0, 0, 0);
        uint4 bv[BROWS / 64];
#pragma unroll
        for (int i = 0; i < BROWS / 64; ++i) bv[i] = *reinterpret_cast<const uint4*>(b_src[i] + kb);
        __syncthreads();
        *reinterpret_cast<uint4*>(&As[a_r * LDS_STRIDE + a_k]) = av;
#pragma unroll
        for (int i = 0; i < BROWS / 64; ++i)
            *reinterpret_cast<uint4*>(&Bs[((tid >> 2) + 64 * i) * LDS_STRIDE + a_k]) = bv[i];
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            const int kk = ks + 8 * (lane >> 5);
            Frag a, b0;
            a.q = *reinterpret_cast<const uint4*>(&As[(32 * wm + (lane & 31)) * LDS_STRIDE + kk]);
            b0.q = *reinterpret_cast<const uint4*>(&Bs[(32 * wn + (lane & 31)) * LDS_STRIDE + kk]);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b0.v, acc0, 0, 0, 0);
            if (GATE_UP) {
                Frag b1;
                b1.q = *reinterpret_cast<const uint4*>(
                    &Bs[(BN + 32 * wn + (lane & 31)) * LDS_STRIDE + kk]);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b1.v, acc1, 0, 0, 0);
            }
        }
    }

    const int col = n0 + 32 * wn + (lane & 31);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int r = 32 * wm + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
        if (r < rows) {
            const float v = GATE_UP ? silu_mul(acc0[j], acc1[j]) : acc0[j];
            C[static_cast<size_t>(row0 + r) * N + col] = f32_to_bf16(v);
        }
    }
}

}  // namespace

int gemm_bm_gate_up(int, int) { return BM; }
int gemm_bm_down(int, int) { return BM; }

hipError_t launch_gate_up_bf16(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                               const Tile* tiles, const int32_t* ntiles, int max_tiles,
                               const int32_t* offsets, uint16_t* h, int T, int d, int F, int k,
                               hipStream_t s) {
    (void)T;
    (void)k;
    dim3 grid(max_tiles, F / BN);
    hipLaunchKernelGGL(k_expert_gemm<true>, grid, dim3(256), 0, s, x, tok_of, W_gu, tiles, ntiles,
                       offsets, h, d, F);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const uint16_t* h, const uint16_t* W_dn, const Tile* tiles,
                            const int32_t* ntiles, int max_tiles, const int32_t* offsets,
                            uint16_t* y, int T, int d, int F, int k, hipStream_t s) {
    (void)T;
    (void)k;
    dim3 grid(max_tiles, d / BN);
    hipLaunchKernelGGL(k_expert_gemm<false>, grid, dim3(256), 0, s, h, nullptr, W_dn, tiles, ntiles,
                       offsets, y, F, d);
    return hipGetLastError();
}

}  // namespace hy3
