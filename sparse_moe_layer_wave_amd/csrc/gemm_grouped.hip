// Grouped expert GEMMs for prefill-sized batches on CDNA4 MFMA with fp32
// accumulation, on bf16 or e4m3 operands:
//
//   gate_up: h[r, c] = SiLU(x_t . Wg[e][c]) * (x_t . Wu[e][c]) for the rows r
//            of expert e (t = token of r) ("DeepSeek V4-Flash architecture
//            Q&A", Q4.5: SiLU on the gate branch; "Tencent Hy3-295B
//            architecture teardown", section 2.3: the fused gate_up
//            projection, gate rows first).  bf16: h stored as bf16.  e4m3:
//            the two products are first rescaled by the token's activation
//            scale and the channel's weight scale ("DeepSeek V4-Flash
//            architecture Q&A", Q7.4: one scale per output channel); h is
//            stored as fp32 and the row's max |h| is folded into amax[r] (an
//            integer atomic max on the bit pattern of |h|) for the per-row
//            quantisation of h that follows;
//   down:    y[r, n] = h[r] . Wd[e][n] (e4m3: rescaled by the row's and the
//            channel's scales), stored as bf16.
//
// Four waves per workgroup, every one both a loader and an MFMA wave, each
// owning a 128 x 128 block of the output tile (4 x 4 blocks of 32 x 32 MFMA
// outputs in AGPRs, so each fragment read from LDS feeds four MFMAs).  Two
// tile shapes share the code:
//   square: 256 rows x 256 weight rows, waves in a 2 x 2 grid;
//   wide:   128 rows x 512 weight rows, waves in a 1 x 4 grid.
// An expert's rows are split into 128-row blocks; pairs of blocks run as
// square tiles and an odd last block as a wide tile, so no tile carries more
// than 127 padding rows and both shapes do the same MFMA work.
//
// K advances in slices of 128 bytes per row (64 bf16 = four steps of
// v_mfma_f32_32x32x16_bf16, or 128 e4m3 = two steps of
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales): whole cache lines, so
// no line is requested twice.  A slice of a tile is 64 or 80 one-kilobyte
// copies (8 rows each), issued as global_load_lds_dwordx4 straight into LDS
// rings; every wave issues its own share.  Square tiles keep token rows and
// weight rows in rings of their own (2 and 3 slots of 32 KB), so the weight
// copies of a slice start a half slice earlier and a barrier never waits for
// the whole queue; wide tiles use one ring of 2 slots of 80 KB.
// The copies are written in inline assembly: the compiler does not see them
// as LDS stores and so does not wait for all of them before each LDS read;
// the loop instead waits (s_waitcnt vmcnt) for the slice it needs and then
// meets the other waves at a barrier.  A slice is consumed in two halves of
// 64 bytes: the fragments of the next half are read from LDS while the
// MFMAs of the current half run, and the copies refilling the ring are
// spread between the MFMAs of the second half, so that neither memory
// queue stalls the wave.
//
// LDS row r keeps logical 16-byte chunk c at physical chunk c ^ ((r >> 1) & 7):
// the 16 lanes of one phase of a fragment read (16 rows at one logical chunk)
// then hit 16 distinct 4-bank groups, all 64 banks once.
// MFMA lane layout: A lane l holds row l%32 and 16 bytes (bf16: k 8*(l/32)..+8
// of a 16-wide step; e4m3: 32 bytes, k 32*(l/32)..+32 of a 64-wide step); B
// the same for a weight row; C lane l holds column l%32 and rows
// 8*(j/4) + 4*(l/32) + j%4, j = 0..15.
//
// Work order: units (expert, chunk of up to 8 row blocks, 512-row weight
// panel, tile) in one sequence; the tiles of one chunk that read the same
// weight panel are adjacent, so the panel streams into L2 once for all of
// them.  The grid is persistent (one workgroup per CU): the sequence is cut
// into 8 contiguous ranges, one per XCD, which that XCD's workgroups take
// round-robin.

#include "grouped_order.h"

namespace hy3 {
namespace {

enum Mode { GU_BF16 = 0, DN_BF16 = 1, GU_FP8 = 2, DN_FP8 = 3 };

constexpr int kRowB = 128;                     // bytes per LDS row (one K slice)
constexpr int kLdsBytes = 160 * 1024;          // the whole LDS of a CU
constexpr int kSlots = 2;                      // LDS ring depth

struct Args {
    const uint8_t* A;                              // gate_up: x [T, K]; down: h [rows, K]
    const int32_t* tok_of;                         // gate_up: token of each row
    const uint8_t* W;                              // gate_up: [E, 2N, K]; down: [E, N, K]
    const uint8_t* W_last;                         // non-NULL: weights of expert E - 1 (shared)
    const int32_t* offsets;                        // [E+1] row offsets
    const int32_t* tile_off;                       // [E+1] offsets in 128-row blocks
    uint16_t* C;                                   // bf16 out: gate_up h (bf16 mode) or y [rows, N]
    const float* a_scale;                          // e4m3: per token (gate_up) or per row (down)
    const float* w_scale;                          // e4m3: [E, 2N] (gate_up) or [E, N] (down)
    float* h32;                                    // e4m3 gate_up: h [rows, N] fp32
    uint32_t* amax;                                // e4m3 gate_up: [rows] bits of max |h|
    int K, N, E, npanel;                           // K in elements; npanel: 512-row panels per expert
};

// One tile.  SQUARE: 256 rows x 256 weight rows; else 128 x 512.
template <int MODE, bool SQUARE>
__device__ __forceinline__ void tile(const Args& g, uint8_t* lds, const Unit& u, int wave) {
    constexpr bool GATE_UP = MODE == GU_BF16 || MODE == GU_FP8;
    constexpr bool FP8 = MODE == GU_FP8 || MODE == DN_FP8;
    constexpr int RA = SQUARE ? 256 : 128;         // A rows per slice
    constexpr int WCOLS = SQUARE ? 128 : 256;      // gate_up: h columns of the tile
    constexpr int NCOLS = SQUARE ? 256 : 512;      // down: output columns of the tile
    constexpr int ROWS = RA + NCOLS;               // LDS rows of a slice
    constexpr int NMFMA = FP8 ? 16 : 32;           // MFMAs per half slice and wave
    const int N = g.N;
    const int lane = lane_id();
    const int tid = wave * 64 + lane;
    const int wm = SQUARE ? (wave & 1) : 0;
    const int wn = SQUARE ? (wave >> 1) : wave;
    const size_t rowbytes = static_cast<size_t>(g.K) * (FP8 ? 1 : 2);
    const int nk = static_cast<int>(rowbytes / kRowB);

    // ---- copy sources.  A copy fills 8 LDS rows of 128 bytes (lane -> row
    // + lane / 8, physical chunk lane % 8), so each row's whole cache line
    // comes from one copy.  Per copy the lane keeps the 32-bit index of its
    // source row (token row or weight row); the address is formed when the
    // copy is issued.
    //   square: token rows and weight rows have rings of their own, 2 and 3
    //     slots of 32 KB; copy j < 8 of a wave fills token row group
    //     8 wave + j, copy 8 + j weight row group 8 wave + j;
    //   wide: one ring of 2 slots of 80 KB (128 token rows, then 512 weight
    //     rows); copy j fills row group 20 wave + j.
    // Whether a copy reads token rows or weight rows depends on (wave, j) only.
    constexpr int NPW = SQUARE ? 16 : 20;          // 1 KB copies per wave per slice
    constexpr int kASlot = RA * kRowB;             // square: token ring slot (32 KB)
    constexpr int kBSlot = NCOLS * kRowB;          // square: weight ring slot (32 KB)
    constexpr int kSlotBytes = ROWS * kRowB;       // wide: ring slot (80 KB)
    static_assert(SQUARE ? 2 * kASlot + 3 * kBSlot <= kLdsBytes : kSlots * kSlotBytes <= kLdsBytes, "LDS");
    auto is_a = [&](int j) { return SQUARE ? j < 8 : 8 * (wave * NPW + j) < RA; };
    auto group = [&](int j) { return SQUARE ? 8 * wave + (j & 7) : wave * NPW + j; };   // within its ring slot
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
                const int col = u.n * WCOLS + (p >> 7) * 64 + (p & 63);
                wr = col < N ? ((p & 64) ? N + col : col) : 0;
            } else {
                wr = u.n * NCOLS + p;
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
    // slot: LDS address of the ring slot the copy fills
    auto issue_copy = [&](int j, int kt, uint32_t slot) {
        const uint8_t* base = is_a(j) ? g.A : We;
        const uint8_t* src = base + static_cast<size_t>(static_cast<uint32_t>(srow_of[j])) * rowbytes +
                             static_cast<size_t>(kt) * kRowB + lco[group(j) & 1];
        copy_to_lds(src, slot + group(j) * 1024);
    };

    // ---- fragment addresses: token rows a0 + 32 mb + l32 and weight rows
    // b0 + 32 nb + l32 of their slots; the physical chunk only depends on l32
    // (block offsets are multiples of 32).  A slice is two halves of 64
    // bytes; half-fragment h of a block in half hs is one 16-byte read:
    // bf16: the lane's 8 values of k step 2 hs + h (chunk 4 hs + 2 h + khalf);
    // e4m3: bytes 16 h.. of the lane's 32 of the k step hs (chunk
    // 4 hs + 2 khalf + h).
    const int l32 = lane & 31;
    const int khalf = lane >> 5;
    const int a0 = wm * 128;
    const int b0 = (SQUARE ? 0 : RA) + wn * 128;
    int off[2][2];
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            off[hs][h] = l32 * kRowB + pchunk8(l32, FP8 ? 4 * hs + 2 * khalf + h : 4 * hs + 2 * h + khalf) * 16;

    f32x16_t acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16_t{};

    // read r of a half slice (16 per half): h = r / 8; r % 8 < 4: A block
    // r % 4 (from abase), else B block r % 4 (from bbase)
    i32x4_t fa[2][2][4], fb[2][2][4];                  // [set][h][block]
    auto read_frag = [&](int set, const uint8_t* abase, const uint8_t* bbase, int hs, int r) {
        const int h = r >> 3, b = r & 3;
        if ((r & 4) == 0) fa[set][h][b] = *reinterpret_cast<const i32x4_t*>(abase + (a0 + 32 * b) * kRowB + off[hs][h]);
        else fb[set][h][b] = *reinterpret_cast<const i32x4_t*>(bbase + (b0 + 32 * b) * kRowB + off[hs][h]);
    };
    auto mfma = [&](int set, int i) {
        if constexpr (FP8) {
            const int mb = i >> 2, nb = i & 3;
            const i32x8_t a = __builtin_shufflevector(fa[set][0][mb], fa[set][1][mb], 0, 1, 2, 3, 4, 5, 6, 7);
            const i32x8_t b = __builtin_shufflevector(fb[set][0][nb], fb[set][1][nb], 0, 1, 2, 3, 4, 5, 6, 7);
            acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[mb][nb], 0, 0, 0, 127, 0, 127);
        } else {
            const int h = i >> 4, mb = (i >> 2) & 3, nb = i & 3;
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, fa[set][h][mb]), __builtin_bit_cast(bf16x8_t, fb[set][h][nb]),
                acc[mb][nb], 0, 0, 0);
        }
    };
    // the 16 reads of a half are spread evenly over its MFMAs
    auto read_at = [&](int set, const uint8_t* abase, const uint8_t* bbase, int hs, int i) {
        if constexpr (FP8) {
            read_frag(set, abase, bbase, hs, i);
        } else {
            if (i & 1) read_frag(set, abase, bbase, hs, i >> 1);
        }
    };

    if constexpr (SQUARE) {
        // ---- square: token ring (2 slots) at 0, weight ring (3 slots) after.
        // Slice kt: first half: MFMAs on its first half (read during slice
        // kt - 1), reading its second half, and the weight copies of slice
        // kt + 2 into the weight slot of slice kt - 1 (read by every wave
        // before the barrier of slice kt - 1).  Barrier: slice kt + 1 landed
        // (only the weight copies of kt + 2 may be in flight) and every read
        // of slice kt done.  Second half: MFMAs on its second half, reading
        // the first half of slice kt + 1, and the token copies of slice kt + 2
        // into the token slot of slice kt.  Slices past the end re-read the
        // last one into slots nobody reads again.  Issue order per wave:
        // B(kt+1), A(kt+1), B(kt+2), so the waits are exact.
        const uint32_t abase0 = lds0, bbase0 = lds0 + 2 * kASlot;
        auto aslot = [&](int kt) { return kt & 1; };
        auto bslot = [&](int kt) { return kt % 3; };
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int kt = min(s, nk - 1);
#pragma unroll
            for (int j = 8; j < 16; ++j) issue_copy(j, kt, bbase0 + s * kBSlot);
#pragma unroll
            for (int j = 0; j < 8; ++j) issue_copy(j, kt, abase0 + s * kASlot);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));     // slice 0 landed
        lds_barrier();
#pragma unroll
        for (int r = 0; r < 16; ++r) read_frag(0, lds, lds + 2 * kASlot, 0, r);

        for (int kt = 0; kt < nk; ++kt) {
            const uint8_t* ca = lds + aslot(kt) * kASlot;
            const uint8_t* cb = lds + 2 * kASlot + bslot(kt) * kBSlot;
            const uint8_t* na = lds + aslot(kt + 1) * kASlot;
            const uint8_t* nb_ = lds + 2 * kASlot + bslot(kt + 1) * kBSlot;
            const int kin = min(kt + 2, nk - 1);
            const uint32_t bfill = bbase0 + bslot(kt + 2) * kBSlot;
#pragma unroll
            for (int i = 0; i < NMFMA; ++i) {
                mfma(0, i);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (i == j * NMFMA / 8) issue_copy(8 + j, kin, bfill);
                read_at(1, ca, cb, 1, i);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
            lds_barrier();                             // slice kt + 1 landed, slice kt read by all
            const uint32_t afill = abase0 + aslot(kt) * kASlot;
#pragma unroll
            for (int i = 0; i < NMFMA; ++i) {
                mfma(1, i);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (i == j * NMFMA / 8) issue_copy(j, kin, afill);
                read_at(0, na, nb_, 0, i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        // ---- wide: one ring of 2 slots.  First half of slice kt: MFMAs on its
        // first half, reading its second half.  Barrier: slice kt + 1 landed,
        // every read of slice kt done.  Second half: MFMAs on its second half,
        // reading the first half of slice kt + 1 and refilling the slot with
        // slice kt + 2.
        const uint32_t my_base = lds0;
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
            const int kt = min(s, nk - 1);
#pragma unroll
            for (int j = 0; j < NPW; ++j) issue_copy(j, kt, my_base + s * kSlotBytes);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NPW));
        lds_barrier();
#pragma unroll
        for (int r = 0; r < 16; ++r) read_frag(0, lds, lds, 0, r);

        for (int kt = 0; kt < nk; ++kt) {
            const uint8_t* cur = lds + (kt & 1) * kSlotBytes;
            const uint8_t* nxt = lds + ((kt + 1) & 1) * kSlotBytes;
#pragma unroll
            for (int i = 0; i < NMFMA; ++i) {
                mfma(0, i);
                read_at(1, cur, cur, 1, i);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            lds_barrier();                             // slice kt + 1 landed, slice kt read by all
            const int kin = min(kt + 2, nk - 1);
            const uint32_t islot = my_base + (kt & 1) * kSlotBytes;
#pragma unroll
            for (int i = 0; i < NMFMA; ++i) {
                mfma(1, i);
#pragma unroll
                for (int j = 0; j < NPW; ++j)
                    if (i == j * NMFMA / NPW) issue_copy(j, kin, islot);
                read_at(0, nxt, nxt, 0, i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));          // no copy may land after the tile ends

    // ---- epilogue.  Each wave stages its output block in LDS (row-major,
    // rows padded by 16 bytes so the two half-waves of a write, 4 rows apart,
    // use different banks) and then stores it as 16-byte chunks, whole rows
    // per group of lanes: 8x fewer store instructions than storing the MFMA
    // layout (one column per lane) directly.  e4m3: the tile's row scales are
    // staged in LDS as well (one load per thread, all in flight together) and
    // the lane's column scales are loaded once, ahead of the loops.
    constexpr int OCOLS = GATE_UP ? 64 : 128;          // output columns per wave
    constexpr int OESZ = MODE == GU_FP8 ? 4 : 2;       // bytes per output element
    constexpr int OPITCH = OCOLS * OESZ + 16;
    static_assert(4 * 128 * OPITCH + RA * 4 <= kLdsBytes, "LDS");
    uint8_t* ow = lds + wave * (128 * OPITCH);
    float* srow = reinterpret_cast<float*>(lds + 4 * 128 * OPITCH);
    lds_barrier();                                     // every wave is done with the ring
    if constexpr (FP8) {
        const int t = tid;
        if (t < RA) {
            const int r = min(t, u.rows - 1);
            srow[t] = GATE_UP ? g.a_scale[g.tok_of[u.row0 + r]] : g.a_scale[u.row0 + r];
        }
        __syncthreads();
    }
    float wsc[4] = {0.f, 0.f, 0.f, 0.f};              // gate_up: gate nb 0,1 then up nb 0,1; down: nb 0..3
    if constexpr (FP8) {
        const float* ws_e = g.w_scale + static_cast<size_t>(u.e) * (GATE_UP ? 2 * N : N);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int c = GATE_UP ? u.n * WCOLS + wn * 64 + 32 * (nb & 1) + l32
                                  : u.n * NCOLS + wn * 128 + 32 * nb + l32;
            if (c < N) wsc[nb] = ws_e[(GATE_UP && nb >= 2) ? N + c : c];
        }
    }
    const int col0 = GATE_UP ? u.n * WCOLS + wn * 64 : u.n * NCOLS + wn * 128;   // the wave's first output column
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int rl = 32 * mb + 8 * (j >> 2) + 4 * khalf + (j & 3);   // row within the wave's block
            uint8_t* orow = ow + rl * OPITCH;
            if constexpr (MODE == GU_BF16) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    *reinterpret_cast<uint16_t*>(orow + (32 * nb + l32) * 2) =
                        f32_to_bf16(silu_mul(acc[mb][nb][j], acc[mb][nb + 2][j]));
            } else if constexpr (MODE == DN_BF16) {
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    *reinterpret_cast<uint16_t*>(orow + (32 * nb + l32) * 2) = f32_to_bf16(acc[mb][nb][j]);
            } else if constexpr (MODE == GU_FP8) {
                const float sx = srow[a0 + rl];
                float hmax = 0.f;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const float gv = acc[mb][nb][j] * sx * wsc[nb];
                    const float uv = acc[mb][nb + 2][j] * sx * wsc[nb + 2];
                    const float hv = silu_mul(gv, uv);             // 0 for columns >= N (zero scales)
                    *reinterpret_cast<float*>(orow + (32 * nb + l32) * 4) = hv;
                    hmax = fmaxf(hmax, fabsf(hv));
                }
                // row max over the 32 lanes that share this row (same khalf)
#pragma unroll
                for (int o = 16; o >= 1; o >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, o, 32));
                if (l32 == 0 && a0 + rl < u.rows) atomicMax(&g.amax[u.row0 + a0 + rl], __float_as_uint(hmax));
            } else {
                const float sh = srow[a0 + rl];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    *reinterpret_cast<uint16_t*>(orow + (32 * nb + l32) * 2) = f32_to_bf16(acc[mb][nb][j] * sh * wsc[nb]);
            }
        }
    }
    // a wave's LDS accesses complete in order, so it can read its block back
    // without a barrier
    constexpr int CPR = OCOLS * OESZ / 16;             // 16-byte chunks per row: 8 or 16
    constexpr int EPC = 16 / OESZ;                     // elements per chunk
#pragma unroll
    for (int it = 0; it < 128 * CPR / 64; ++it) {
        const int q = it * 64 + lane;
        const int rl = q / CPR, cc = q % CPR;
        const int r = a0 + rl;
        const int c = col0 + cc * EPC;
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(ow + rl * OPITCH + cc * 16);
        if (r < u.rows && c < N) {
            const size_t grow = static_cast<size_t>(u.row0 + r);
            if constexpr (MODE == GU_FP8) *reinterpret_cast<i32x4_t*>(g.h32 + grow * N + c) = v;
            else *reinterpret_cast<i32x4_t*>(g.C + grow * N + c) = v;
        }
    }
}

// Persistent: one workgroup per CU, workgroup b on XCD b % 8 (the dispatcher
// deals workgroups round-robin over the XCDs).  The units are split into 8
// contiguous ranges, one per XCD, and the XCD's workgroups take its range
// round-robin, so at any time an XCD works on consecutive units (one
// expert's tiles, reading the same weight panels and token rows through its
// L2).
template <int MODE>
__global__ __launch_bounds__(256, 1) void k_grouped(Args g) {
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
        if (!unit_of<MODE == GU_BF16 || MODE == GU_FP8>(g.tile_off, g.offsets, g.E, g.npanel, g.N, L, u,
                                                        square))
            continue;
        if (square) tile<MODE, true>(g, lds, u, wave);
        else tile<MODE, false>(g, lds, u, wave);
        lds_barrier();                             // every wave has read its staged output back
    }
}

template <int MODE>
hipError_t launch(Args g, int max_blocks, hipStream_t s) {
    constexpr bool GATE_UP = MODE == GU_BF16 || MODE == GU_FP8;
    g.npanel = GATE_UP ? (g.N + 255) / 256 : (g.N + 511) / 512;   // 512 weight rows per panel
    const long long units = static_cast<long long>(max_blocks) * g.npanel;
    if (units == 0) return hipSuccess;
    int cus = 0;
    const hipError_t err = device_cu_count(&cus);
    if (err != hipSuccess) return err;
    const int grid = persistent_grid(units, cus);
    hipLaunchKernelGGL(k_grouped<MODE>, dim3(grid), dim3(256), 0, s, g);
    return hipGetLastError();
}

}  // namespace

int prefill_bm() { return 128; }

hipError_t launch_gate_up_grouped(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                                  const uint16_t* W_last, const int32_t* offsets,
                                  const int32_t* tile_off, int max_blocks, uint16_t* h, int E, int d,
                                  int F, hipStream_t s) {
    Args g{reinterpret_cast<const uint8_t*>(x), tok_of, reinterpret_cast<const uint8_t*>(W_gu),
           reinterpret_cast<const uint8_t*>(W_last), offsets, tile_off, h, nullptr, nullptr, nullptr,
           nullptr, d, F, E, 0};
    return launch<GU_BF16>(g, max_blocks, s);
}

hipError_t launch_down_grouped(const uint16_t* h, const uint16_t* W_dn, const uint16_t* W_last,
                               const int32_t* offsets, const int32_t* tile_off, int max_blocks,
                               uint16_t* y, int E, int d, int F, hipStream_t s) {
    Args g{reinterpret_cast<const uint8_t*>(h), nullptr, reinterpret_cast<const uint8_t*>(W_dn),
           reinterpret_cast<const uint8_t*>(W_last), offsets, tile_off, y, nullptr, nullptr, nullptr,
           nullptr, F, d, E, 0};
    return launch<DN_BF16>(g, max_blocks, s);
}

hipError_t launch_gate_up_fp8(const uint8_t* xq, const float* xs, const int32_t* tok_of,
                              const uint8_t* Wq, const float* ws, const int32_t* offsets,
                              const int32_t* tile_off, int max_blocks, float* h32, uint32_t* amax,
                              int E, int d, int F, hipStream_t s) {
    Args g{xq, tok_of, Wq, nullptr, offsets, tile_off, nullptr, xs, ws, h32, amax, d, F, E, 0};
    return launch<GU_FP8>(g, max_blocks, s);
}

hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const uint8_t* Wq, const float* ws,
                           const int32_t* offsets, const int32_t* tile_off, int max_blocks,
                           uint16_t* y, int E, int d, int F, hipStream_t s) {
    Args g{hq, nullptr, Wq, nullptr, offsets, tile_off, y, hs, ws, nullptr, nullptr, F, d, E, 0};
    return launch<DN_FP8>(g, max_blocks, s);
}

}  // namespace hy3
