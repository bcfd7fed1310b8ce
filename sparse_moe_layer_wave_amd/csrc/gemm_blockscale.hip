// Grouped expert GEMMs for e4m3 weights with one fp32 scale per 128 x 128
// weight block ("DeepSeek V4-Flash architecture Q&A", Q7.2: block-wise
// quantisation, every 128 x 128 block of a weight matrix with its own
// scaling factor), for prefill-sized batches:
//
//   gate_up: h[r, c] = SiLU(sx_t * G) * (sx_t * U), where
//            G = sum over k-blocks kb of Sg[kb] * (xq_t . Wq_gate[c])|kb and U
//            likewise with the up rows; stored as fp32 with the row's max |h|
//            folded into amax[r] for the per-row quantisation that follows;
//   down:    y[r, n] = bf16(sh_r * sum_kb Sd[kb] * (hq_r . Wq_down[n])|kb).
//
// One workgroup computes a tile of 128 rows x 128 weight rows (gate_up: 64 h
// columns, their 64 gate and 64 up weight rows; down: 128 output columns),
// so every k-block of the tile has one scale per weight-row block: one for
// down, one for the gate and one for the up rows of gate_up.  K advances in
// slices of 128 e4m3 values, exactly one k-block: each slice's product is
// accumulated from zero by two v_mfma_scale_f32_32x32x64_f8f6f4 steps (unit
// hardware scales), multiplied by its block scale and added to the fp32
// accumulator.  Four waves in a 2 x 2 grid, each owning 64 rows x 64 weight
// rows (2 x 2 MFMA blocks of 32 x 32): gate_up waves hold the gate and the up
// block of the same 32 h columns, so SiLU(g) * u is formed in registers.
//
// A slice (16 KB of token rows, 16 KB of weight rows) is loaded into
// registers one slice ahead and stored to a 2-slot LDS ring; one barrier per
// slice.  LDS rows are 128 bytes with 16-byte chunk c of row r at c ^ ((r >>
// 1) & 7), so the 16 rows of one fragment read phase hit 16 distinct 4-bank
// groups.  64 KB of LDS per workgroup: two workgroups share a CU.
// MFMA lane layout: A lane l holds row l % 32 and bytes 32 (l / 32)..+32 of a
// 64-wide k step; B the same for a weight row; C lane l holds column l % 32
// and rows 8 (j / 4) + 4 (l / 32) + j % 4, j = 0..15.
//
// Tiles are numbered row block fastest, then column tile; the hardware
// hands workgroup b to XCD b % 8, so tile numbers are remapped to give each
// XCD a contiguous range: the row blocks of one expert that read the same
// weight tile then run on one XCD and share its L2.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kRowB = 128;                       // bytes per LDS row: one slice of one row
constexpr int kTileRows = 128;
constexpr int kSliceB = kTileRows * kRowB;       // 16 KB: one operand of one slice
constexpr int kXcds = 8;

__device__ __forceinline__ int pch(int row, int c) { return c ^ ((row >> 1) & 7); }

struct BlkArgs {
    const uint8_t* A;            // gate_up: xq [T, K]; down: hq [rows, K]
    const int32_t* tok_of;       // gate_up: token of each row
    const uint8_t* W;            // gate_up: [E, 2N, K]; down: [E, N, K] e4m3
    const float* w_scale;        // [E, rows_w / 128, K / 128]
    const float* a_scale;        // gate_up: per token; down: per row
    const int32_t* offsets;      // [E+1] row offsets
    const int32_t* tile_off;     // [E+1] offsets in 128-row blocks
    float* h32;                  // gate_up: h [rows, N] fp32
    uint32_t* amax;              // gate_up: [rows] bits of max |h|
    uint16_t* y;                 // down: [rows, N] bf16
    int K, N, E, nmt, ntiles;    // nmt: row-block slots of the grid; ntiles: nmt * column tiles
};

template <bool GATE_UP>
__global__ __launch_bounds__(256) void k_grouped_blk(BlkArgs g) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 2 * kSliceB];
    __shared__ float s_scale[2][128];
    const int E = g.E, K = g.K, N = g.N;
    const int KB = K >> 7;

    // contiguous range of tiles per XCD
    const int per = (g.ntiles + kXcds - 1) / kXcds;
    const int b = static_cast<int>(blockIdx.x);
    const int lin = (b % kXcds) * per + b / kXcds;
    if (lin >= g.ntiles) return;
    const int mt = lin % g.nmt, nt = lin / g.nmt;
    if (mt >= __builtin_amdgcn_readfirstlane(g.tile_off[E])) return;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (__builtin_amdgcn_readfirstlane(g.tile_off[mid]) <= mt) lo = mid;
        else hi = mid - 1;
    }
    const int e = lo;
    const int r0 = __builtin_amdgcn_readfirstlane(g.offsets[e]) +
                   kTileRows * (mt - __builtin_amdgcn_readfirstlane(g.tile_off[e]));
    const int nrows = min(kTileRows, __builtin_amdgcn_readfirstlane(g.offsets[e + 1]) - r0);
    if (nrows <= 0) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;
    const size_t Nw = GATE_UP ? 2 * static_cast<size_t>(N) : static_cast<size_t>(N);
    const uint8_t* We = g.W + static_cast<size_t>(e) * Nw * K;
    const int c0 = nt * (GATE_UP ? 64 : 128);     // first h column (gate_up) or output column

    // scale rows of this tile: gate_up [gate block, up block]; down [block]
    {
        const float* se = g.w_scale + static_cast<size_t>(e) * (Nw >> 7) * KB;
        const int nb0 = c0 >> 7, nb1 = GATE_UP ? (N + c0) >> 7 : nb0;
        for (int i = tid; i < 2 * 128; i += 256) {
            const int which = i >> 7, kb = i & 127;
            if (kb < KB) s_scale[which][kb] = se[static_cast<size_t>(which ? nb1 : nb0) * KB + kb];
        }
    }

    // loads: thread t copies rows (t >> 3) + 32 j, 16-byte chunk t & 7, of
    // both operands (token rows, weight rows)
    const int lrow = tid >> 3, lch = tid & 7;
    const uint8_t* asrc[4];
    const uint8_t* bsrc[4];
    int ldst[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int R = lrow + 32 * j;
        const int rr = r0 + min(R, nrows - 1);             // padding rows repeat a valid row
        const size_t arow = GATE_UP ? static_cast<size_t>(g.tok_of[rr]) : static_cast<size_t>(rr);
        asrc[j] = g.A + arow * K + lch * 16;
        // weight row R of the tile: gate_up rows 0..63 gate columns c0.., 64..127 the up rows
        const size_t wrow = GATE_UP ? static_cast<size_t>(R < 64 ? c0 + R : N + c0 + (R - 64))
                                    : static_cast<size_t>(c0 + R);
        bsrc[j] = We + wrow * K + lch * 16;
        ldst[j] = R * kRowB + pch(R, lch) * 16;
    }

    // fragment offsets: lane row l32 of a 32-row block, bytes 32 khalf.. of k step s
    const int l32 = lane & 31, khalf = lane >> 5;
    int foff[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) foff[s][h] = l32 * kRowB + pch(l32, 4 * s + 2 * khalf + h) * 16;
    // this wave's 32-row blocks: token rows 64 wr + 32 i; weight rows
    // gate_up: 32 wc (gate) and 64 + 32 wc (up); down: 64 wc + 32 i
    int arow0[2], brow0[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        arow0[i] = (64 * wr + 32 * i) * kRowB;
        brow0[i] = (GATE_UP ? 64 * i + 32 * wc : 64 * wc + 32 * i) * kRowB;
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    i32x4_t ra[4], rb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ra[j] = *reinterpret_cast<const i32x4_t*>(asrc[j]);
        rb[j] = *reinterpret_cast<const i32x4_t*>(bsrc[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<i32x4_t*>(lds + ldst[j]) = ra[j];
        *reinterpret_cast<i32x4_t*>(lds + kSliceB + ldst[j]) = rb[j];
    }
    __syncthreads();

    for (int kt = 0; kt < KB; ++kt) {
        const bool more = kt + 1 < KB;
        if (more) {
            const size_t ko = static_cast<size_t>(kt + 1) * kRowB;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ra[j] = *reinterpret_cast<const i32x4_t*>(asrc[j] + ko);
                rb[j] = *reinterpret_cast<const i32x4_t*>(bsrc[j] + ko);
            }
        }
        const uint8_t* sa = lds + (kt & 1) * 2 * kSliceB;
        const uint8_t* sb = sa + kSliceB;
        f32x16_t t[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            i32x8_t fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const i32x4_t a0 = *reinterpret_cast<const i32x4_t*>(sa + arow0[i] + foff[s][0]);
                const i32x4_t a1 = *reinterpret_cast<const i32x4_t*>(sa + arow0[i] + foff[s][1]);
                const i32x4_t b0 = *reinterpret_cast<const i32x4_t*>(sb + brow0[i] + foff[s][0]);
                const i32x4_t b1 = *reinterpret_cast<const i32x4_t*>(sb + brow0[i] + foff[s][1]);
                fa[i] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                fb[i] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    t[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[i], fb[j], s == 0 ? f32x16_t{} : t[i][j], 0, 0, 0, 127, 0, 127);
        }
        const float s0 = s_scale[0][kt];
        const float s1 = GATE_UP ? s_scale[1][kt] : s0;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                acc[i][0][q] = fmaf(t[i][0][q], s0, acc[i][0][q]);
                acc[i][1][q] = fmaf(t[i][1][q], s1, acc[i][1][q]);
            }
        if (more) {
            uint8_t* da = lds + ((kt + 1) & 1) * 2 * kSliceB;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                *reinterpret_cast<i32x4_t*>(da + ldst[j]) = ra[j];
                *reinterpret_cast<i32x4_t*>(da + kSliceB + ldst[j]) = rb[j];
            }
        }
        __syncthreads();
    }

    // epilogue: C lane layout, column l32, rows 8 (q / 4) + 4 khalf + q % 4
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int R = 64 * wr + 32 * i + 8 * (q >> 2) + 4 * khalf + (q & 3);
            const bool vr = R < nrows;
            const int r = r0 + (vr ? R : 0);
            if constexpr (GATE_UP) {
                const float sx = g.a_scale[g.tok_of[r]];
                const float hv = silu_mul(acc[i][0][q] * sx, acc[i][1][q] * sx);
                const int c = c0 + 32 * wc + l32;
                if (vr) g.h32[static_cast<size_t>(r) * N + c] = hv;
                float m = fabsf(hv);
#pragma unroll
                for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
                if (vr && l32 == 0) atomicMax(&g.amax[r], __float_as_uint(m));
            } else {
                const float sh = g.a_scale[r];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = c0 + 64 * wc + 32 * j + l32;
                    if (vr) g.y[static_cast<size_t>(r) * N + n] = f32_to_bf16(acc[i][j][q] * sh);
                }
            }
        }
    }
}

hipError_t launch_blk(const BlkArgs& a, bool gate_up, int ncol_tiles, hipStream_t s) {
    BlkArgs g = a;
    g.ntiles = g.nmt * ncol_tiles;
    if (g.ntiles == 0) return hipSuccess;
    const int per = (g.ntiles + kXcds - 1) / kXcds;
    const dim3 grid(per * kXcds);
    if (gate_up) hipLaunchKernelGGL(k_grouped_blk<true>, grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL(k_grouped_blk<false>, grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_fp8_block(const uint8_t* xq, const float* xs, const int32_t* tok_of,
                                    const uint8_t* Wq, const float* sb, const int32_t* offsets,
                                    const int32_t* tile_off, int max_mtiles, float* h32,
                                    uint32_t* amax, int E, int d, int F, hipStream_t s) {
    const BlkArgs g{xq, tok_of, Wq, sb, xs, offsets, tile_off, h32, amax, nullptr, d, F, E, max_mtiles, 0};
    return launch_blk(g, true, F / 64, s);
}

hipError_t launch_down_fp8_block(const uint8_t* hq, const float* hs, const uint8_t* Wq,
                                 const float* sb, const int32_t* offsets, const int32_t* tile_off,
                                 int max_mtiles, uint16_t* y, int E, int d, int F, hipStream_t s) {
    const BlkArgs g{hq, nullptr, Wq, sb, hs, offsets, tile_off, nullptr, nullptr, y, F, d, E, max_mtiles, 0};
    return launch_blk(g, false, d / 128, s);
}

}  // namespace hy3
