// Grouped expert GEMMs for prefill-sized batches on CDNA4 MFMA with fp32
// accumulation, on bf16 or e4m3 operands:
//
//   gate_up: h[r, c] = SiLU(x_t . Wg[e][c]) * (x_t . Wu[e][c]) for the rows r
//            of expert e (t = token of r) ("DeepSeek V4-Flash architecture
//            Q&A", Q4.5: SiLU on the gate branch; "Tencent Hy3-295B
//            architecture teardown", section 2.3: the fused gate_up
//            projection, gate rows first).  bf16: h stored as bf16.  e4m3:
//            the two products are rescaled by the token's activation scale
//            and the weights' scales, h is stored as bf16, and each tile
//            stores its rows' max |bf16(h)| over each 128-column block it
//            covers into hmax[block][r], for the per-row quantisation of the
//            bf16 h that follows (which takes the max over the blocks);
//   down:    y[r, n] = h[r] . Wd[e][n] (e4m3: rescaled by the row's and the
//            weights' scales), stored as bf16.
//
// e4m3 weight scales come in two layouts: one per output channel ("DeepSeek
// V4-Flash architecture Q&A", Q7.4), applied in the epilogue, or one per
// 128 x 128 weight block (same page, Q7.2), which varies along K:
//   G = sum over k-blocks kb of Sg[kb] * (xq_t . Wq_gate[c])|kb.
//
// Tiles: an expert's rows are split into 128-row blocks; pairs of blocks run
// as square tiles (256 rows x 256 weight rows) and an odd last block as a
// wide tile (128 rows x 512 weight rows), so no tile carries more than 127
// padding rows and both shapes do the same MFMA work (grouped_order.h: work
// order over a persistent grid, one workgroup per CU).  A workgroup has
// eight waves, two per SIMD (square: 2 x 4, wide: 1 x 8), each owning 128
// token rows x 64 weight rows, 4 x 2 blocks of 32 x 32: 128 fp32
// accumulators per lane, kept in VGPRs (with block scales they are rescaled
// by VALU multiplies between the MFMAs).  A gate_up wave's 64 weight rows are
// 32 gate rows and the 32 up rows of the same h columns, so SiLU(g) * u is
// formed in registers.
//
// K advances in slices of 128 bytes per row (64 bf16, 128 e4m3; for block
// scales exactly one k-block): whole cache lines, so no line is requested
// twice.  A slice is two k steps of 64 bytes; per k step and block one
// v_mfma_scale_f32_32x32x64_f8f6f4 or two v_mfma_f32_32x32x16_bf16.
//
// Copies: a slice of a tile is 64 (square) or 80 (wide) one-kilobyte copies
// of 8 rows, global_load_lds_dwordx4 straight into LDS rings (square: token
// rows 2 slots and weight rows 3 slots of 32 KB; wide: one ring of 2 slots
// of 80 KB); each wave issues its share.  The copies are inline assembly,
// so the compiler does not wait for them before each LDS read; the loop
// waits (s_waitcnt vmcnt) for the slice it needs and meets the other waves
// at a barrier.  A slice runs k step 0 of its 8 blocks, a barrier, then k
// step 1.  Registers hold one k step of token fragments and both k steps of
// weight fragments: during k step 0 the k-step-1 fragments of the same
// slice replace the retiring ones, during k step 1 those of the next slice's
// k step 0.  The barrier marks the slice's slot as read by every wave (and
// the next slice as landed), so the copies of slice kt + 2 go out into it
// during k step 1 (square tiles: token rows; wide tiles: everything); a
// square tile's weight rows of slice kt + 2 go out during k step 0, into
// the third weight slot, freed by the barrier of slice kt - 1.
//
// Block scales: each scale is split as s = m * 2^e with |m| in [1, 2).  The
// MFMAs apply 2^e themselves, through the E8M0 scale of their B operand
// (exact), relative to the largest exponent E of the row block (clamped at
// 2^-127), and accumulate straight into the block's accumulator, which is
// kept divided by the current mantissa: before a slice's MFMAs it is
// multiplied by m_prev / m, and after the last slice by m_last * 2^E.  A
// wave's weight rows lie in one 128-row block (down) or one gate and one up
// block (gate_up), so a slice has one or two scales per wave; a lane keeps
// the scales of k-blocks l and 64 + l and reads the slice's with readlane
// (K <= 16384).
//
// LDS row r keeps logical 16-byte chunk c at physical chunk c ^ ((r >> 1) & 7):
// the 16 lanes of one phase of a fragment read (16 rows at one logical chunk)
// then hit 16 distinct 4-bank groups, all 64 banks once.
// MFMA lane layout: A lane l holds row l % 32 and, per k step, e4m3: 32
// bytes, k 32 (l / 32)..+32 of the 64; bf16: 8 values, k 8 (l / 32)..+8 of
// each 16-wide step; B the same for a weight row; C lane l holds column
// l % 32 and rows 8 (j / 4) + 4 (l / 32) + j % 4, j = 0..15.

#include "grouped_order.h"

namespace hy3 {
namespace {

enum Mode { GU_BF16 = 0, DN_BF16 = 1, GU_FP8 = 2, DN_FP8 = 3, GU_BLK = 4, DN_BLK = 5 };

constexpr int kRowB = 128;                     // bytes per LDS row (one K slice)
constexpr int kLdsBytes = 160 * 1024;          // the whole LDS of a CU
constexpr int kWaves = 8;                      // waves per workgroup (two per SIMD)

struct Args {
    const uint8_t* A;                              // gate_up: x [T, K]; down: h [rows, K]
    const int32_t* tok_of;                         // gate_up: token of each row
    const uint8_t* W;                              // gate_up: [E, 2N, K]; down: [E, N, K]
    const uint8_t* W_last;                         // non-NULL: weights of expert E - 1 (shared)
    const int32_t* offsets;                        // [E+1] row offsets
    const int32_t* tile_off;                       // [E+1] offsets in 128-row blocks
    uint16_t* C;                                   // bf16 out: gate_up h or down y [rows, N]
    const float* a_scale;                          // e4m3: activation scale per row (gate_up: its token's)
    const float* w_scale;                          // per channel: [E, 2N] or [E, N]; block: [E, rows_w/128, K/128]
    float* hmax;                                   // e4m3 gate_up: [N / 128][rows] max |h| per 128-column block
    int rows;                                      // e4m3 gate_up: rows of h (the stride of hmax)
    int* sched;                                    // [kXcds] unit counters, zero at launch
    int K, N, E, npanel;                           // K in elements; npanel: weight panels per expert
};

// The last 64 bytes of LDS: the word through which a claimed unit is
// broadcast (clear of the epilogue's staging).
constexpr int kClaimOff = kLdsBytes - 64;

// e4m3 MFMA whose B operand is scaled by 2^(sb - 127) (an E8M0 exponent,
// exact), A unscaled.
__device__ __forceinline__ f32x16_t mfma_f8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// One k step of bf16: two 32x32x16 MFMAs (the lane's first and second 16 bytes).
__device__ __forceinline__ f32x16_t mfma_bf16(const i32x8_t& a, const i32x8_t& b, f32x16_t c) {
    const i32x4_t a0 = __builtin_shufflevector(a, a, 0, 1, 2, 3), a1 = __builtin_shufflevector(a, a, 4, 5, 6, 7);
    const i32x4_t b0 = __builtin_shufflevector(b, b, 0, 1, 2, 3), b1 = __builtin_shufflevector(b, b, 4, 5, 6, 7);
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0), __builtin_bit_cast(bf16x8_t, b0), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1), __builtin_bit_cast(bf16x8_t, b1), c, 0, 0, 0);
}

// Per-slice block scale of one weight row block, split as s = m * 2^e with
// |m| in [1, 2): sb is the E8M0 byte of 2^(e - E) (E: the largest exponent
// among the block's k-blocks, so the shift is <= 0; clamped at 2^-127), and
// r = m_prev / m the multiplier of the accumulator before this slice's
// products are added.  After the last k-block the accumulator times
// m_last * 2^E is the scaled sum: acc_kb = (1 / m_kb) sum_{j <= kb} m_j
// 2^(e_j - E) P_j.  A zero scale keeps r = 1 and m_prev and gets the
// smallest B scale, 2^-127: its products (at most 2^25 in magnitude) stay
// more than 2^100 below anything they are added to.
struct SliceScale {
    float r;
    int sb;
};

__device__ __forceinline__ SliceScale slice_scale(float s, int E, float& m_prev) {
    int ex;
    const float f = frexpf(s, &ex);            // s = f 2^ex, |f| in [0.5, 1)
    const bool live = s != 0.f;
    const float m = 2.f * f;
    SliceScale o;
    o.r = live ? m_prev / m : 1.f;
    o.sb = live ? max(0, 127 + (ex - 1) - E) : 0;
    if (live) m_prev = m;
    return o;
}

// One tile.  SQUARE: 256 rows x 256 weight rows; else 128 x 512.  claim, if
// not NULL, is a unit counter: thread 0 takes the next unit from it during
// the epilogue and leaves the value in LDS (kClaimOff).
template <int MODE, bool SQUARE>
__device__ __forceinline__ void tile(const Args& g, uint8_t* lds, const Unit& u, int wave, int* claim) {
    constexpr bool GATE_UP = MODE == GU_BF16 || MODE == GU_FP8 || MODE == GU_BLK;
    constexpr bool FP8 = MODE >= GU_FP8;
    constexpr bool BLK = MODE >= GU_BLK;
    constexpr int RA = SQUARE ? 256 : 128;         // token rows of a slice
    constexpr int NB = SQUARE ? 256 : 512;         // weight rows of a slice
    constexpr int WCOLS = NB / 2;                  // gate_up: h columns of the tile
    constexpr int ROWS = RA + NB;
    constexpr int NPW = ROWS / 8 / kWaves;         // 1 KB copies per wave per slice (8; 10)
    constexpr int kASlot = RA * kRowB;             // square: token ring slot (32 KB)
    constexpr int kBSlot = NB * kRowB;             // square: weight ring slot (32 KB)
    constexpr int kSlotBytes = ROWS * kRowB;       // wide: ring slot (80 KB)
    constexpr int WN = SQUARE ? 4 : 8;             // waves along the weight rows
    static_assert(SQUARE ? 2 * kASlot + 3 * kBSlot <= kLdsBytes : 2 * kSlotBytes <= kLdsBytes, "LDS");
    const int N = g.N;
    const size_t rowbytes = static_cast<size_t>(g.K) * (FP8 ? 1 : 2);
    const int nk = static_cast<int>(rowbytes / kRowB);
    const int lane = lane_id();
    const int tid = wave * 64 + lane;
    const int wm = SQUARE ? (wave & 1) : 0;
    const int wn = SQUARE ? (wave >> 1) : wave;

    // ---- copy sources: a copy fills 8 LDS rows of 128 bytes (lane -> row
    // + lane / 8, physical chunk lane % 8), so each row's whole cache line
    // comes from one copy; the lane keeps the 32-bit index of its source row
    // per copy.  Square: copy j < 4 of a wave fills token row group
    // 4 wave + j, copy 4 + j weight row group 4 wave + j; wide: copy j fills
    // row group 10 wave + j of the single ring (token rows first).  Weight
    // panel row p of a gate_up tile is, in groups of 64, 32 gate rows and
    // the 32 up rows of the same h columns.
    auto is_a = [&](int j) { return SQUARE ? j < 4 : NPW * wave + j < RA / 8; };
    auto group = [&](int j) { return SQUARE ? 4 * wave + (j & 3) : NPW * wave + j; };
    const uint8_t* We = (g.W_last && u.e == g.E - 1)
                            ? g.W_last
                            : g.W + static_cast<size_t>(u.e) * (GATE_UP ? 2 * N : N) * rowbytes;
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
                const int col = u.n * WCOLS + (p >> 6) * 32 + (p & 31);
                wr = col < N ? ((p & 32) ? N + col : col) : 0;
            } else {
                wr = u.n * NB + p;
                wr = wr < N ? wr : 0;
            }
            srow_of[j] = wr;
        }
    }
    // logical chunk of the lane: (row >> 1) & 7 = 4 (group & 1) + lane / 16
    int lco[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) lco[q] = ((lane & 7) ^ (4 * q + (lane >> 4))) * 16;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    // slot: LDS address of the ring slot the copy fills; slices past the end
    // re-read the last one into slots nobody reads again
    auto issue_copy = [&](int j, int kt, uint32_t slot) {
        const uint8_t* base = is_a(j) ? g.A : We;
        const uint8_t* src = base + static_cast<size_t>(static_cast<uint32_t>(srow_of[j])) * rowbytes +
                             static_cast<size_t>(min(kt, nk - 1)) * kRowB + lco[group(j) & 1];
        copy_to_lds(src, slot + group(j) * 1024);
    };

    // the wave's first output column (gate_up: h column)
    const int cw = GATE_UP ? u.n * WCOLS + wn * 32 : u.n * NB + wn * 64;

    // e4m3: the epilogue's row scale (thread tid < RA: row tid) and, per
    // channel, the lane's column scales (gate_up: gate, up), loaded before the
    // first copy so that their latency passes under the K loop; the compiler
    // waits for them where the epilogue uses them, after every copy has landed
    float srow_pre = 0.f;
    float cs[2] = {1.f, 1.f};
    if constexpr (FP8) {
        if (tid < RA) srow_pre = g.a_scale[u.row0 + min(tid, u.rows - 1)];
        if constexpr (!BLK) {
            const float* ws_e = g.w_scale + static_cast<size_t>(u.e) * (GATE_UP ? 2 * N : N);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int c = GATE_UP ? cw + (lane & 31) : cw + 32 * nb + (lane & 31);
                cs[nb] = c < N ? ws_e[(GATE_UP && nb) ? N + c : c] : 0.f;
            }
        }
    }

    // ---- block scales of the wave's weight rows (gate and up row blocks;
    // down: one row block).  A wave whose columns lie past N (a partial
    // panel) gets scale 0 and contributes nothing.
    float sa_lo = 0.f, sa_hi = 0.f, sb_lo = 0.f, sb_hi = 0.f;
    int E0 = 0, E1 = 0;
    if constexpr (BLK) {
        const int KB = nk;
        const int nrb = (GATE_UP ? 2 * N : N) >> 7;
        const float* se = g.w_scale + static_cast<size_t>(u.e) * nrb * KB;
        const int rb0 = cw >> 7, rb1 = GATE_UP ? (N + cw) >> 7 : rb0;
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
        // largest exponent among the nonzero scales of each row block (0 if none)
        auto emax = [&](float lo, float hi) {
            int e = -1000, ex;
            if (lo != 0.f) { frexpf(lo, &ex); e = max(e, ex - 1); }
            if (hi != 0.f) { frexpf(hi, &ex); e = max(e, ex - 1); }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) e = max(e, __shfl_xor(e, o));
            return e == -1000 ? 0 : e;
        };
        E0 = emax(sa_lo, sa_hi);
        E1 = GATE_UP ? emax(sb_lo, sb_hi) : E0;
    }
    auto scale_of = [&](float lo, float hi, int kt) {
        const float v = kt < 64 ? lo : hi;
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kt & 63));
    };
    float m0 = 1.f, m1 = 1.f;                          // current mantissas (row block 0, 1)

    // ---- fragments: token rows a0 + 32 mb + l32 and weight rows b0 + 32 nb
    // + l32 of their slots; k step s is chunks 4 s..4 s + 3 of a row, the
    // lane's two 16-byte reads are chunks 4 s + 2 khalf + h (e4m3: its 32
    // bytes) or 4 s + 2 h + khalf (bf16: its 8 values of the step's first
    // and second 16-wide MFMA).
    const int l32 = lane & 31;
    const int khalf = lane >> 5;
    const int a0 = wm * 128;
    const int b0 = (SQUARE ? 0 : RA) + wn * 64;
    int off[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            off[s][h] = l32 * kRowB + pchunk8(l32, FP8 ? 4 * s + 2 * khalf + h : 4 * s + 2 * h + khalf) * 16;
    auto frag = [&](const uint8_t* base, int row0, int s) {
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + row0 * kRowB + off[s][0]);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + row0 * kRowB + off[s][1]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16_t{};
    // token fragments of one k step (they roll from k step 0 to 1 and on to
    // the next slice's k step 0 as they retire), weight fragments of both
    i32x8_t fa[4], fb[2][2];

    // A slice: k step 0 of its 8 blocks (row-major), a barrier, k step 1.
    //  - k step 0 reads slice kt's k-step-1 token fragments (a row's after
    //    its last k-step-0 MFMA) and weight fragments (first thing) from its
    //    slot; the barrier after it (slice kt + 1 has landed, every wave is
    //    done reading slice kt) frees the slot;
    //  - k step 1 reads slice kt + 1's k-step-0 fragments from its slot (the
    //    weight ones first, the token ones as a row retires).
    // copy0(i) / copy1(i) issue the copies that follow block i of k step 0 / 1.
    // Block scales: block b = 2 mb + nb is multiplied by the next slice's
    // ratio after block 2 + b of k step 1 (two blocks after its last MFMA):
    // blocks 0..5 during k step 1 with qn; blocks 6 and 7 after blocks 0 and
    // 1 of the next slice, with that slice's ratio, qc (in slice 0 they are
    // still zero).
    auto rescale = [&](int b, float r) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b >> 1][b & 1][e] *= r;
    };
    auto ratio = [&](int b, const SliceScale& q0, const SliceScale& q1) { return (GATE_UP && (b & 1)) ? q1.r : q0.r; };
    auto mma = [&](int mb, int nb, const i32x8_t& a, const i32x8_t& b, const SliceScale& q0, const SliceScale& q1) {
        if constexpr (BLK) acc[mb][nb] = mfma_f8(a, b, acc[mb][nb], (GATE_UP && nb) ? q1.sb : q0.sb);
        else if constexpr (FP8) acc[mb][nb] = mfma_f8(a, b, acc[mb][nb], 127);
        else acc[mb][nb] = mfma_bf16(a, b, acc[mb][nb]);
    };
    auto run_slice = [&](const SliceScale& qc0, const SliceScale& qc1, const SliceScale& qn0,
                         const SliceScale& qn1, const uint8_t* ca, const uint8_t* cb, const uint8_t* na,
                         const uint8_t* nb_, auto mid_wait, auto copy0, auto copy1) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int mb = p >> 1, nb = p & 1;
            mma(mb, nb, fa[mb], fb[nb][0], qc0, qc1);
            if (p == 0) {
                fb[0][1] = frag(cb, b0, 1);
                fb[1][1] = frag(cb, b0 + 32, 1);
            }
            if (BLK && p < 2) rescale(6 + p, ratio(6 + p, qc0, qc1));
            if (nb == 1) fa[mb] = frag(ca, a0 + 32 * mb, 1);
            copy0(p);
            __builtin_amdgcn_sched_barrier(0);
        }
        mid_wait();
        lds_barrier();
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int mb = p >> 1, nb = p & 1;
            mma(mb, nb, fa[mb], fb[nb][1], qc0, qc1);
            if (p == 0) {
                fb[0][0] = frag(nb_, b0, 0);
                fb[1][0] = frag(nb_, b0 + 32, 0);
            }
            if (BLK && p >= 2) rescale(p - 2, ratio(p - 2, qn0, qn1));
            if (nb == 1) fa[mb] = frag(na, a0 + 32 * mb, 0);
            copy1(p);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // this slice's block scales (kt) and the next one's (kt + 1; none past the last)
    auto scales_of = [&](int kt, SliceScale& q0, SliceScale& q1) {
        if constexpr (BLK) {
            const float s0 = kt < nk ? scale_of(sa_lo, sa_hi, kt) : 0.f;
            q0 = slice_scale(s0, E0, m0);                          // down; gate_up: gate rows
            if (GATE_UP) {
                const float s1 = kt < nk ? scale_of(sb_lo, sb_hi, kt) : 0.f;
                q1 = slice_scale(s1, E1, m1);                      // up rows
            } else {
                q1 = q0;
            }
        } else {
            q0 = q1 = SliceScale{1.f, 127};
        }
    };
    SliceScale qc0, qc1, qn0, qn1;
    scales_of(0, qc0, qc1);
    auto first_frags = [&](const uint8_t* ca, const uint8_t* cb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = frag(ca, a0 + 32 * i, 0);
        fb[0][0] = frag(cb, b0, 0);
        fb[1][0] = frag(cb, b0 + 32, 0);
    };

    if constexpr (SQUARE) {
        // token ring (2 slots) at 0, weight ring (3 slots) after it.  Issue
        // order per wave: B(0) A(0) B(1) A(1), then in slice kt: B(kt+2)
        // during k step 0, into the weight slot slice kt - 1 came from (free
        // since the middle of slice kt - 1), and A(kt+2) during k step 1,
        // into the token slot of slice kt; so "slice kt+1 landed" is vmcnt(4)
        // at the middle of slice kt, and the copies are spread over the slice.
        const uint32_t abase0 = lds0, bbase0 = lds0 + 2 * kASlot;
        const uint8_t* abuf = lds;
        const uint8_t* bbuf = lds + 2 * kASlot;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int j = 4; j < 8; ++j) issue_copy(j, s, bbase0 + s * kBSlot);
#pragma unroll
            for (int j = 0; j < 4; ++j) issue_copy(j, s, abase0 + s * kASlot);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));      // slice 0 landed
        lds_barrier();
        first_frags(abuf, bbuf);
        for (int kt = 0; kt < nk; ++kt) {
            const uint32_t afill = abase0 + (kt & 1) * kASlot;
            const uint32_t bfill = bbase0 + ((kt + 2) % 3) * kBSlot;
            scales_of(kt + 1, qn0, qn1);
            run_slice(qc0, qc1, qn0, qn1, abuf + (kt & 1) * kASlot, bbuf + (kt % 3) * kBSlot,
                      abuf + ((kt + 1) & 1) * kASlot, bbuf + ((kt + 1) % 3) * kBSlot,
                      [&] { __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); },   // slice kt + 1 landed
                      [&](int i) {
                          if (i & 1) issue_copy(4 + (i >> 1), kt + 2, bfill);
                      },
                      [&](int i) {
                          if (i & 1) issue_copy(i >> 1, kt + 2, afill);
                      });
            qc0 = qn0;
            qc1 = qn1;
        }
    } else {
        // one ring of 2 slots; the copies of slice kt + 2 go out in k step 1
        // of slice kt, so "slice kt+1 landed" is vmcnt(0) at its middle
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int j = 0; j < NPW; ++j) issue_copy(j, s, lds0 + s * kSlotBytes);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NPW));    // slice 0 landed
        lds_barrier();
        first_frags(lds, lds);
        for (int kt = 0; kt < nk; ++kt) {
            const uint32_t fill = lds0 + (kt & 1) * kSlotBytes;
            const uint8_t* cur = lds + (kt & 1) * kSlotBytes;
            const uint8_t* nxt = lds + ((kt + 1) & 1) * kSlotBytes;
            scales_of(kt + 1, qn0, qn1);
            run_slice(qc0, qc1, qn0, qn1, cur, cur, nxt, nxt,
                      [&] { __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); },   // slice kt + 1 landed
                      [](int) {},
                      [&](int i) {
                          issue_copy(i, kt + 2, fill);
                          if (i + 8 < NPW) issue_copy(i + 8, kt + 2, fill);
                      });
            qc0 = qn0;
            qc1 = qn1;
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));          // no copy may land after the tile ends

    // ---- epilogue: each wave stages its output block in LDS (rows padded
    // by 16 bytes) and stores it as 16-byte chunks, whole rows per group of
    // lanes: 8x fewer store instructions than storing the MFMA layout (one
    // column per lane) directly.  e4m3: the tile's activation row scales are
    // staged in LDS too (one load per thread, all in flight together), and
    // (gate_up) each wave's per-row max |h|, combined into one max per row
    // and 128-column block of the tile and stored (no atomics: each block of
    // a row belongs to one tile).
    constexpr int OCOLS = GATE_UP ? 32 : 64;           // output columns per wave
    constexpr int OESZ = 2;                            // bytes per output element (bf16)
    constexpr int OPITCH = OCOLS * OESZ + 16;
    static_assert(kWaves * 128 * OPITCH + RA * 4 + RA * WN * 4 <= kClaimOff, "LDS");
    uint8_t* ow = lds + wave * (128 * OPITCH);
    float* srow = reinterpret_cast<float*>(lds + kWaves * 128 * OPITCH);
    float* hm = srow + RA;                             // e4m3 gate_up: [RA][WN] max |h| per wave
    lds_barrier();                                     // every wave is done with the rings
    int claimed = 0;
    if (claim && tid == 0) claimed = atomicAdd(claim, 1);
    if constexpr (FP8) {
        if (tid < RA) srow[tid] = srow_pre;
        __syncthreads();
    }
    // the output's column factors: per channel, the lane's columns' scales
    // (loaded above); block scales: m_last * 2^E of each row block (the
    // accumulators are the sums divided by it)
    if constexpr (BLK) {
        cs[0] = ldexpf(m0, E0);
        cs[1] = GATE_UP ? ldexpf(m1, E1) : cs[0];
    }
    // bf16 down: lanes 2i and 2i + 1 (columns 2i, 2i + 1) swap one value of
    // rows r, r + 1 (adjacent j), so each writes both columns of one row as a
    // dword: half the LDS writes, none of them sub-dword (staging 2.9 -> 2.0
    // us per tile).  The other modes keep one write per value: their staging
    // is bound by the VALU (scales, SiLU), which the swap adds to.
    const bool odd = lane & 1;
    auto put_pair = [&](int rl, int col, float a, float b) {   // a: row rl, b: row rl + 1, column col
        const float send = odd ? a : b;
        const float recv = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
        const f32x2_t lohi = {odd ? recv : a, odd ? b : recv};
        *reinterpret_cast<bf16x2_t*>(ow + (rl + (odd ? 1 : 0)) * OPITCH + (col & ~1) * 2) =
            __builtin_convertvector(lohi, bf16x2_t);
    };
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int rl = 32 * mb + 8 * (j >> 2) + 4 * khalf + (j & 3);   // row within the wave's block
            uint8_t* orow = ow + rl * OPITCH;
            if constexpr (MODE == GU_BF16) {
                *reinterpret_cast<uint16_t*>(orow + l32 * 2) = f32_to_bf16(silu_mul(acc[mb][0][j], acc[mb][1][j]));
            } else if constexpr (MODE == DN_BF16) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    if (j & 1) put_pair(rl - 1, 32 * nb + l32, acc[mb][nb][j - 1], acc[mb][nb][j]);
            } else if constexpr (GATE_UP) {
                const float sr = srow[a0 + rl];
                *reinterpret_cast<uint16_t*>(orow + l32 * 2) =
                    f32_to_bf16(silu_mul(acc[mb][0][j] * cs[0] * sr, acc[mb][1][j] * cs[1] * sr));
            } else {
                const float sr = srow[a0 + rl];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    *reinterpret_cast<uint16_t*>(orow + (32 * nb + l32) * 2) = f32_to_bf16(acc[mb][nb][j] * cs[nb] * sr);
            }
        }
    }
    if constexpr (GATE_UP && FP8) {
        // each row's max |h| over the wave's 32 bf16 columns, read back from
        // the staged block (a wave's LDS accesses complete in order): two
        // rows per lane, instead of a 5-step cross-lane reduction per row
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int rl = lane + 64 * q;
            float m = 0.f;
#pragma unroll
            for (int c = 0; c < 32; c += 8) {
                const uint4 v = *reinterpret_cast<const uint4*>(ow + rl * OPITCH + c * 2);
                const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    m = fmaxf(m, fmaxf(fabsf(__uint_as_float(p[i] << 16)), fabsf(__uint_as_float(p[i] & 0xffff0000u))));
            }
            hm[(a0 + rl) * WN + wn] = cw < N ? m : 0.f;
        }
        // a 128-column block is 4 waves' columns: square tiles have one,
        // wide tiles two (the second may lie past N)
        __syncthreads();
        if (tid < RA && tid < u.rows) {
#pragma unroll
            for (int cb = 0; cb < WN / 4; ++cb) {
                const int blk = u.n * (WCOLS / 128) + cb;
                if (blk * 128 < N) {
                    float m = 0.f;
#pragma unroll
                    for (int w = 4 * cb; w < 4 * cb + 4; ++w) m = fmaxf(m, hm[tid * WN + w]);
                    g.hmax[static_cast<size_t>(blk) * g.rows + u.row0 + tid] = m;
                }
            }
        }
    }
    // a wave's LDS accesses complete in order: it reads its block back
    // without a barrier
    constexpr int CPR = OCOLS * OESZ / 16;             // 16-byte chunks per row (4 or 8)
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
            *reinterpret_cast<i32x4_t*>(g.C + grow * N + c) = v;
        }
    }
    if (claim && tid == 0) *reinterpret_cast<int*>(lds + kClaimOff) = claimed;
}

// Persistent: one workgroup per CU, workgroup b on XCD b % 8 (the dispatcher
// deals workgroups round-robin over the XCDs).  The units are split into 8
// contiguous ranges, one per XCD, so at any time an XCD works on consecutive
// units (one expert's tiles, reading the same weight panels and token rows
// through its L2).  A workgroup takes the unit of its XCD's range at its own
// index, then claims the next ones from the XCD's counter (g.sched[x]),
// each during the epilogue of the tile before, so the claim's latency is
// hidden; once its XCD's range is used up, it claims from the other XCDs'
// counters in turn.  Tile times vary with how much of each tile's data hits
// L2, and claiming keeps the workgroups finishing together (a static
// round-robin left 9-10% of workgroup time idle at the end).
template <int MODE>
__global__ __launch_bounds__(64 * kWaves, 1) void k_grouped(Args g) {
    constexpr bool GATE_UP = MODE == GU_BF16 || MODE == GU_FP8 || MODE == GU_BLK;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
    int* cl = reinterpret_cast<int*>(lds + kClaimOff);
    const int U = g.tile_off[g.E] * g.npanel;
    const int per_wg = gridDim.x / kXcds;          // workgroups per XCD (grid: a multiple of kXcds)
    const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int per_xcd = (U + kXcds - 1) / kXcds;
    int wave;                                      // opaque: not recomputed from the thread index later
    asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(wave) : "v"(static_cast<int>(threadIdx.x) >> 6));
    int src = x;                                   // XCD whose counter the claims go to
    int tried = 0;                                 // ranges found used up
    Unit u;                                        // the unit being decoded (its expert is the next hint)
    u.e = -1;
    bool square = false;
    auto decode = [&](int L) {
        return unit_of<GATE_UP>(g.tile_off, g.offsets, g.E, g.npanel, g.N, L, u, square, u.e);
    };
    // value v taken from counter src -> a unit with work, decoded into u
    // (-1: none left), claiming again while the unit is empty or src's range
    // is used up (uniform control flow: every thread runs the same iterations)
    auto resolve = [&](int v) {
        for (;;) {
            const int L = src * per_xcd + per_wg + v;
            if (L < min((src + 1) * per_xcd, U)) {
                if (decode(L)) return L;
            } else {
                if (++tried >= kXcds) return -1;
                src = (src + 1) % kXcds;
            }
            __syncthreads();                       // every thread has read *cl
            if (threadIdx.x == 0) *cl = atomicAdd(g.sched + src, 1);
            __syncthreads();
            v = __builtin_amdgcn_readfirstlane(*cl);
        }
    };
    int cur = x * per_xcd + j;
    if (!(cur < min((x + 1) * per_xcd, U) && decode(cur))) {
        if (threadIdx.x == 0) *cl = atomicAdd(g.sched + src, 1);
        __syncthreads();
        cur = resolve(__builtin_amdgcn_readfirstlane(*cl));
    }
    while (cur >= 0) {
        int* claim = tried < kXcds ? g.sched + src : nullptr;
        if (square) tile<MODE, true>(g, lds, u, wave, claim);
        else tile<MODE, false>(g, lds, u, wave, claim);
        lds_barrier();                             // staged output read back, *cl written
        cur = claim ? resolve(__builtin_amdgcn_readfirstlane(*cl)) : -1;
    }
}

template <int MODE>
hipError_t launch(Args g, int max_blocks, hipStream_t s) {
    constexpr bool GATE_UP = MODE == GU_BF16 || MODE == GU_FP8 || MODE == GU_BLK;
    g.npanel = GATE_UP ? (g.N + 255) / 256 : (g.N + 511) / 512;   // 512 weight rows per panel
    const long long units = static_cast<long long>(max_blocks) * g.npanel;
    if (units == 0) return hipSuccess;
    int cus = 0;
    const hipError_t err = device_cu_count(&cus);
    if (err != hipSuccess) return err;
    const int grid = persistent_grid(units, cus);
    g.sched += GATE_UP ? 0 : kXcds;                // gate_up and down each have their own counters
    hipLaunchKernelGGL(k_grouped<MODE>, dim3(grid), dim3(64 * kWaves), 0, s, g);
    return hipGetLastError();
}

}  // namespace

int prefill_bm() { return 128; }

hipError_t launch_gate_up_grouped(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                                  const uint16_t* W_last, const int32_t* offsets,
                                  const int32_t* tile_off, int max_blocks, uint16_t* h, int* sched, int E,
                                  int d, int F, hipStream_t s) {
    Args g{reinterpret_cast<const uint8_t*>(x), tok_of, reinterpret_cast<const uint8_t*>(W_gu),
           reinterpret_cast<const uint8_t*>(W_last), offsets, tile_off, h, nullptr, nullptr,
           nullptr, 0, sched, d, F, E, 0};
    return launch<GU_BF16>(g, max_blocks, s);
}

hipError_t launch_down_grouped(const uint16_t* h, const uint16_t* W_dn, const uint16_t* W_last,
                               const int32_t* offsets, const int32_t* tile_off, int max_blocks,
                               uint16_t* y, int* sched, int E, int d, int F, hipStream_t s) {
    Args g{reinterpret_cast<const uint8_t*>(h), nullptr, reinterpret_cast<const uint8_t*>(W_dn),
           reinterpret_cast<const uint8_t*>(W_last), offsets, tile_off, y, nullptr, nullptr,
           nullptr, 0, sched, F, d, E, 0};
    return launch<DN_BF16>(g, max_blocks, s);
}

hipError_t launch_gate_up_fp8(const uint8_t* xq, const float* rs, const int32_t* tok_of,
                              const uint8_t* Wq, const float* ws, const int32_t* offsets,
                              const int32_t* tile_off, int max_blocks, uint16_t* h, float* hmax,
                              int rows, int* sched, int E, int d, int F, hipStream_t s) {
    Args g{xq, tok_of, Wq, nullptr, offsets, tile_off, h, rs, ws, hmax, rows, sched, d, F, E, 0};
    return launch<GU_FP8>(g, max_blocks, s);
}

hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const uint8_t* Wq, const float* ws,
                           const int32_t* offsets, const int32_t* tile_off, int max_blocks,
                           uint16_t* y, int* sched, int E, int d, int F, hipStream_t s) {
    Args g{hq, nullptr, Wq, nullptr, offsets, tile_off, y, hs, ws, nullptr, 0, sched, F, d, E, 0};
    return launch<DN_FP8>(g, max_blocks, s);
}

hipError_t launch_gate_up_fp8_block(const uint8_t* xq, const float* rs, const int32_t* tok_of,
                                    const uint8_t* Wq, const float* sb, const int32_t* offsets,
                                    const int32_t* tile_off, int max_mtiles, uint16_t* h,
                                    float* hmax, int rows, int* sched, int E, int d, int F, hipStream_t s) {
    Args g{xq, tok_of, Wq, nullptr, offsets, tile_off, h, rs, sb, hmax, rows, sched, d, F, E, 0};
    return launch<GU_BLK>(g, max_mtiles, s);
}

hipError_t launch_down_fp8_block(const uint8_t* hq, const float* hs, const uint8_t* Wq,
                                 const float* sb, const int32_t* offsets, const int32_t* tile_off,
                                 int max_mtiles, uint16_t* y, int* sched, int E, int d, int F, hipStream_t s) {
    Args g{hq, nullptr, Wq, nullptr, offsets, tile_off, y, hs, sb, nullptr, 0, sched, F, d, E, 0};
    return launch<DN_BLK>(g, max_mtiles, s);
}

}  // namespace hy3
