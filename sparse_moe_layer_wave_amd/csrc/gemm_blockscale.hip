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
// Tiles and work order are those of the grouped GEMMs (grouped_order.h): a
// persistent grid of one workgroup per CU, 256 x 256 square tiles and
// 128 x 512 wide tiles, four waves each owning 128 x 128 outputs (4 x 4
// blocks of 32 x 32).  K advances in slices of 128
// e4m3 values, exactly one k-block, and a wave's weight rows lie in one
// 128-row block (down) or are 64 gate rows and 64 up rows, each in one block
// (gate_up), so every slice has one scale per wave (down) or two (gate_up).
// A block's product over the slice is accumulated from zero by two
// v_mfma_scale_f32_32x32x64_f8f6f4 steps (unit hardware scales) into a
// temporary, which is multiplied by its scale and added to the block's
// accumulator during the next block's MFMAs, so the adds do not wait on
// theirs.  Per slice and wave that is 32 MFMAs and 256 fused multiply-adds.  A lane keeps
// the scales of k-blocks l and 64 + l of each of its wave's row blocks and
// reads the slice's with readlane (K <= 16384).
//
// Copies are global_load_lds_dwordx4 into LDS rings laid out as in the
// grouped GEMMs (square: token rows 2 slots, weight rows 3 slots of 32 KB;
// wide: 2 slots of 80 KB).  Slice schedule: every fragment of slice kt is in
// registers before its first MFMA -- it was read while slice kt - 1 ran.
// While slice kt runs, the fragments of slice kt + 1 take the registers of
// those of slice kt as soon as their last MFMA has issued (the token-row
// fragments after each row of blocks, the weight-row fragments during the
// last row), and the copies of slice kt + 2 (square tiles: token rows; wide
// tiles: everything) and kt + 3 (square tiles: weight rows) refill the slots
// slice kt came from.  One wait and one barrier per slice, at its end: slice
// kt + 2 has landed and every wave is done reading slice kt + 1.
//
// LDS rows are 128 bytes with 16-byte chunk c of row r at c ^ ((r >> 1) & 7).
// MFMA lane layout: A lane l holds row l % 32 and bytes 32 (l / 32)..+32 of
// a 64-wide k step; B the same for a weight row; C lane l holds column l % 32
// and rows 8 (j / 4) + 4 (l / 32) + j % 4, j = 0..15.

#include "grouped_order.h"

namespace hy3 {
namespace {

constexpr int kRowB = 128;                     // bytes per LDS row: one slice of one row
constexpr int kLdsBytes = 160 * 1024;

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
    int K, N, E, npanel;         // K in elements (= bytes per row); npanel: 512-row panels per expert
};

__device__ __forceinline__ f32x16_t mfma_f8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// One tile.  SQUARE: 256 rows x 256 weight rows; else 128 x 512.
template <bool GATE_UP, bool SQUARE>
__device__ __forceinline__ void tile_blk(const BlkArgs& g, uint8_t* lds, const Unit& u, int wave) {
    constexpr int RA = SQUARE ? 256 : 128;         // token rows of a slice
    constexpr int WCOLS = SQUARE ? 128 : 256;      // gate_up: h columns of the tile
    constexpr int NCOLS = SQUARE ? 256 : 512;      // down: output columns of the tile
    constexpr int ROWS = RA + NCOLS;
    constexpr int NPW = SQUARE ? 16 : 20;          // 1 KB copies per wave per slice
    constexpr int kASlot = RA * kRowB;             // square: token ring slot (32 KB)
    constexpr int kBSlot = NCOLS * kRowB;          // square: weight ring slot (32 KB)
    constexpr int kSlotBytes = ROWS * kRowB;       // wide: ring slot (80 KB)
    static_assert(SQUARE ? 2 * kASlot + 3 * kBSlot <= kLdsBytes : 2 * kSlotBytes <= kLdsBytes, "LDS");
    const int N = g.N, K = g.K;
    const int nk = K / kRowB;
    const int lane = lane_id();
    const int tid = wave * 64 + lane;
    const int wm = SQUARE ? (wave & 1) : 0;
    const int wn = SQUARE ? (wave >> 1) : wave;

    // ---- copy sources: a copy fills 8 LDS rows of 128 bytes (lane -> row
    // + lane / 8, physical chunk lane % 8); the lane keeps the 32-bit index
    // of its source row per copy.  Square: copy j < 8 of a wave fills token
    // row group 8 wave + j, copy 8 + j weight row group 8 wave + j; wide:
    // copy j fills row group 20 wave + j of the single ring.
    auto is_a = [&](int j) { return SQUARE ? j < 8 : 8 * (wave * NPW + j) < RA; };
    auto group = [&](int j) { return SQUARE ? 8 * wave + (j & 7) : wave * NPW + j; };
    const uint8_t* We = g.W + static_cast<size_t>(u.e) * (GATE_UP ? 2 * N : N) * K;
    int srow_of[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        const int row = 8 * group(j) + (lane >> 3);
        if (is_a(j)) {
            const int r = min(row, u.rows - 1);                // padding rows repeat a valid row
            srow_of[j] = GATE_UP ? g.tok_of[u.row0 + r] : u.row0 + r;
        } else {
            const int p = SQUARE ? row : row - RA;             // weight panel row
            int wr;
            if (GATE_UP) {
                const int col = u.n * WCOLS + (p >> 7) * 64 + (p & 63);
                wr = col < N ? ((p & 64) ? N + col : col) : 0;
            } else {
                wr = u.n * NCOLS + p;
                wr = wr < N ? wr : 0;
            }
            srow_of[j] = wr;
        }
    }
    int lco[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) lco[q] = ((lane & 7) ^ (4 * q + (lane >> 4))) * 16;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    auto issue_copy = [&](int j, int kt, uint32_t slot) {
        const uint8_t* base = is_a(j) ? g.A : We;
        const uint8_t* src = base + static_cast<size_t>(static_cast<uint32_t>(srow_of[j])) * K +
                             static_cast<size_t>(min(kt, nk - 1)) * kRowB + lco[group(j) & 1];
        copy_to_lds(src, slot + group(j) * 1024);
    };

    // ---- block scales of the wave's weight rows (gate and up row blocks;
    // down: one row block).  A wave whose columns lie past N (a partial
    // panel) gets scale 0 and contributes nothing.
    const int cw = GATE_UP ? u.n * WCOLS + wn * 64 : u.n * NCOLS + wn * 128;
    const int KB = nk;
    const int nrb = (GATE_UP ? 2 * N : N) >> 7;
    const float* se = g.w_scale + static_cast<size_t>(u.e) * nrb * KB;
    const int rb0 = cw >> 7, rb1 = GATE_UP ? (N + cw) >> 7 : rb0;
    float sa_lo = 0.f, sa_hi = 0.f, sb_lo = 0.f, sb_hi = 0.f;
    if (cw < N) {
        if (lane < KB) {
            sa_lo = se[static_cast<size_t>(rb0) * KB + lane];
            sb_lo = se[static_cast<size_t>(rb1) * KB + lane];
        }
        if (64 + lane < KB) {
            sa_hi = se[static_cast<size_t>(rb0) * KB + 64 + lane];
            sb_hi = se[static_cast<size_t>(rb1) * KB + 64 + lane];
        }
    }
    auto scale_of = [&](float lo, float hi, int kt) {
        const float v = kt < 64 ? lo : hi;
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kt & 63));
    };

    // ---- fragments: token rows a0 + 32 mb + l32 and weight rows b0 + 32 nb
    // + l32 of their slots; k step s of a slice is chunks 4 s..4 s + 3, the
    // lane's 32 bytes are chunks 4 s + 2 khalf and 4 s + 2 khalf + 1.
    const int l32 = lane & 31;
    const int khalf = lane >> 5;
    const int a0 = wm * 128;
    const int b0 = (SQUARE ? 0 : RA) + wn * 128;
    int off[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) off[s][h] = l32 * kRowB + pchunk8(l32, 4 * s + 2 * khalf + h) * 16;
    auto frag = [&](const uint8_t* base, int row0, int s) {
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + row0 * kRowB + off[s][0]);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + row0 * kRowB + off[s][1]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16_t{};
    i32x8_t fa[4][2], fb[4][2];                        // [block][k step] of the current slice

    // The 16 blocks of a slice, in row order.  Block b's product goes to
    // P[b % 2]; its scaled add runs during the next block, half after each of
    // that block's two MFMAs (the MFMA it reads issued before them), so the
    // adds share the issue slots with MFMAs in flight.  The adds of a slice's
    // last block run in the first block of the next slice, with the scales
    // it carries (pm_lo, pm_hi).  Fragments of slice kt + 1 are read from
    // (na, nb_) as the current ones retire; copy(b) issues the copies that
    // follow block b.
    f32x16_t P[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) P[i] = f32x16_t{};
    float pm_lo = 0.f, pm_hi = 0.f;                    // scales of the previous slice
    auto add_half = [&](int blk, int half, float lo, float hi) {
        const int pm = blk >> 2, pn = blk & 3;
        const float sc = pn < 2 ? lo : hi;             // gate_up: gate rows, then up rows
#pragma unroll
        for (int q = 8 * half; q < 8 * half + 8; ++q) acc[pm][pn][q] = __builtin_fmaf(P[blk & 1][q], sc, acc[pm][pn][q]);
    };
    auto run_slice = [&](int kt, const uint8_t* na, const uint8_t* nb_, auto copy) {
        const float s_lo = scale_of(sa_lo, sa_hi, kt);           // down; gate_up: gate rows
        const float s_hi = GATE_UP ? scale_of(sb_lo, sb_hi, kt) : s_lo;   // gate_up: up rows
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const int mb = b >> 2, nb = b & 3;
            const int pend = (b + 15) & 15;            // block b - 1 (of this slice or the last)
            P[b & 1] = mfma_f8(fa[mb][0], fb[nb][0], f32x16_t{});
            __builtin_amdgcn_sched_barrier(0);
            add_half(pend, 0, b < 1 ? pm_lo : s_lo, b < 1 ? pm_hi : s_hi);
            __builtin_amdgcn_sched_barrier(0);
            P[b & 1] = mfma_f8(fa[mb][1], fb[nb][1], P[b & 1]);
            __builtin_amdgcn_sched_barrier(0);
            add_half(pend, 1, b < 1 ? pm_lo : s_lo, b < 1 ? pm_hi : s_hi);
            if (nb == 3) {
                fa[mb][0] = frag(na, a0 + 32 * mb, 0);
                fa[mb][1] = frag(na, a0 + 32 * mb, 1);
            }
            if (mb == 3) {
                fb[nb][0] = frag(nb_, b0 + 32 * nb, 0);
                fb[nb][1] = frag(nb_, b0 + 32 * nb, 1);
            }
            copy(b);
            __builtin_amdgcn_sched_barrier(0);
        }
        pm_lo = s_lo;
        pm_hi = s_hi;
    };

    if constexpr (SQUARE) {
        // token ring (2 slots) at 0, weight ring (3 slots) after it.  Issue
        // order per wave: B(0) A(0) B(1) A(1) B(2), then per slice kt: A(kt+2)
        // B(kt+3), so "slice kt+2 landed" is vmcnt(8) at the end of slice kt.
        const uint32_t abase0 = lds0, bbase0 = lds0 + 2 * kASlot;
        const uint8_t* abuf = lds;
        const uint8_t* bbuf = lds + 2 * kASlot;
#pragma unroll
        for (int s = 0; s < 3; ++s) {
#pragma unroll
            for (int j = 8; j < 16; ++j) issue_copy(j, s, bbase0 + s * kBSlot);
            if (s < 2) {
#pragma unroll
                for (int j = 0; j < 8; ++j) issue_copy(j, s, abase0 + s * kASlot);
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(24));     // slice 0 landed
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i][0] = frag(abuf, a0 + 32 * i, 0);
            fa[i][1] = frag(abuf, a0 + 32 * i, 1);
            fb[i][0] = frag(bbuf, b0 + 32 * i, 0);
            fb[i][1] = frag(bbuf, b0 + 32 * i, 1);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));      // slice 1 landed
        lds_barrier();
        for (int kt = 0; kt < nk; ++kt) {
            const uint32_t afill = abase0 + (kt & 1) * kASlot;
            const uint32_t bfill = bbase0 + (kt % 3) * kBSlot;
            run_slice(kt, abuf + ((kt + 1) & 1) * kASlot, bbuf + ((kt + 1) % 3) * kBSlot, [&](int b) {
                if (b < 8) issue_copy(b, kt + 2, afill);
                else issue_copy(b, kt + 3, bfill);
            });
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));  // slice kt + 2 landed
            lds_barrier();                             // and every wave has read slice kt + 1
        }
    } else {
        // one ring of 2 slots; the copies of slice kt + 2 go out over the
        // first 10 blocks of slice kt
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int j = 0; j < NPW; ++j) issue_copy(j, s, lds0 + s * kSlotBytes);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NPW));    // slice 0 landed
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i][0] = frag(lds, a0 + 32 * i, 0);
            fa[i][1] = frag(lds, a0 + 32 * i, 1);
            fb[i][0] = frag(lds, b0 + 32 * i, 0);
            fb[i][1] = frag(lds, b0 + 32 * i, 1);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));      // slice 1 landed
        lds_barrier();
        for (int kt = 0; kt < nk; ++kt) {
            const uint32_t fill = lds0 + (kt & 1) * kSlotBytes;
            const uint8_t* nxt = lds + ((kt + 1) & 1) * kSlotBytes;
            run_slice(kt, nxt, nxt, [&](int b) {
                if (b < NPW / 2) {
                    issue_copy(2 * b, kt + 2, fill);
                    issue_copy(2 * b + 1, kt + 2, fill);
                }
            });
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // slice kt + 2 landed
            lds_barrier();                             // and every wave has read slice kt + 1
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));          // no copy may land after the tile ends
    add_half(15, 0, pm_lo, pm_hi);                     // the last slice's last block
    add_half(15, 1, pm_lo, pm_hi);

    // ---- epilogue: each wave stages its output block in LDS (rows padded
    // by 16 bytes) and stores it as 16-byte chunks, whole rows per group of
    // lanes; the tile's activation row scales are staged in LDS too.
    constexpr int OCOLS = GATE_UP ? 64 : 128;          // output columns per wave
    constexpr int OESZ = GATE_UP ? 4 : 2;              // bytes per output element
    constexpr int OPITCH = OCOLS * OESZ + 16;
    static_assert(4 * 128 * OPITCH + RA * 4 <= kLdsBytes, "LDS");
    uint8_t* ow = lds + wave * (128 * OPITCH);
    float* srow = reinterpret_cast<float*>(lds + 4 * 128 * OPITCH);
    lds_barrier();                                     // every wave is done with the rings
    if (tid < RA) {
        const int r = min(tid, u.rows - 1);
        srow[tid] = GATE_UP ? g.a_scale[g.tok_of[u.row0 + r]] : g.a_scale[u.row0 + r];
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int rl = 32 * mb + 8 * (j >> 2) + 4 * khalf + (j & 3);   // row within the wave's block
            uint8_t* orow = ow + rl * OPITCH;
            const float sr = srow[a0 + rl];
            if constexpr (GATE_UP) {
                float hmax = 0.f;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const float hv = silu_mul(acc[mb][nb][j] * sr, acc[mb][nb + 2][j] * sr);
                    *reinterpret_cast<float*>(orow + (32 * nb + l32) * 4) = hv;
                    hmax = fmaxf(hmax, fabsf(hv));
                }
#pragma unroll
                for (int o = 16; o >= 1; o >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, o, 32));
                if (l32 == 0 && a0 + rl < u.rows && cw < N)
                    atomicMax(&g.amax[u.row0 + a0 + rl], __float_as_uint(hmax));
            } else {
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    *reinterpret_cast<uint16_t*>(orow + (32 * nb + l32) * 2) = f32_to_bf16(acc[mb][nb][j] * sr);
            }
        }
    }
    // a wave's LDS accesses complete in order: it reads its block back
    // without a barrier
    constexpr int CPR = OCOLS * OESZ / 16;             // 16-byte chunks per row
    constexpr int EPC = 16 / OESZ;                     // elements per chunk
#pragma unroll
    for (int it = 0; it < 128 * CPR / 64; ++it) {
        const int q = it * 64 + lane;
        const int rl = q / CPR, cc = q % CPR;
        const int r = a0 + rl;
        const int c = cw + cc * EPC;
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(ow + rl * OPITCH + cc * 16);
        if (r < u.rows && c < N) {
            const size_t grow = static_cast<size_t>(u.row0 + r);
            if constexpr (GATE_UP) *reinterpret_cast<i32x4_t*>(g.h32 + grow * N + c) = v;
            else *reinterpret_cast<i32x4_t*>(g.y + grow * N + c) = v;
        }
    }
}

template <bool GATE_UP>
__global__ __launch_bounds__(256, 1) void k_grouped_blk(BlkArgs g) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
    const int U = g.tile_off[g.E] * g.npanel;
    const int per_wg = gridDim.x / kXcds;          // workgroups per XCD (grid: a multiple of kXcds)
    const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int per_xcd = (U + kXcds - 1) / kXcds;
    int wave;                                      // opaque: not recomputed from the thread index later
    asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(wave) : "v"(static_cast<int>(threadIdx.x) >> 6));
    const int end = min((x + 1) * per_xcd, U);
    for (int L = x * per_xcd + j; L < end; L += per_wg) {
        Unit u;
        bool square;
        if (!unit_of<GATE_UP>(g.tile_off, g.offsets, g.E, g.npanel, g.N, L, u, square)) continue;
        if (square) tile_blk<GATE_UP, true>(g, lds, u, wave);
        else tile_blk<GATE_UP, false>(g, lds, u, wave);
        lds_barrier();                             // every wave has read its staged output back
    }
}

hipError_t launch_blk(BlkArgs g, bool gate_up, int max_blocks, hipStream_t s) {
    g.npanel = gate_up ? (g.N + 255) / 256 : (g.N + 511) / 512;   // 512 weight rows per panel
    const long long units = static_cast<long long>(max_blocks) * g.npanel;
    if (units == 0) return hipSuccess;
    int cus = 0;
    const hipError_t err = device_cu_count(&cus);
    if (err != hipSuccess) return err;
    const dim3 grid(persistent_grid(units, cus));
    if (gate_up) hipLaunchKernelGGL(k_grouped_blk<true>, grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL(k_grouped_blk<false>, grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_fp8_block(const uint8_t* xq, const float* xs, const int32_t* tok_of,
                                    const uint8_t* Wq, const float* sb, const int32_t* offsets,
                                    const int32_t* tile_off, int max_mtiles, float* h32,
                                    uint32_t* amax, int E, int d, int F, hipStream_t s) {
    const BlkArgs g{xq, tok_of, Wq, sb, xs, offsets, tile_off, h32, amax, nullptr, d, F, E, 0};
    return launch_blk(g, true, max_mtiles, s);
}

hipError_t launch_down_fp8_block(const uint8_t* hq, const float* hs, const uint8_t* Wq,
                                 const float* sb, const int32_t* offsets, const int32_t* tile_off,
                                 int max_mtiles, uint16_t* y, int E, int d, int F, hipStream_t s) {
    const BlkArgs g{hq, nullptr, Wq, sb, hs, offsets, tile_off, nullptr, nullptr, y, F, d, E, 0};
    return launch_blk(g, false, max_mtiles, s);
}

}  // namespace hy3
