// Work order of the persistent grouped GEMMs (gemm_grouped.hip): which tile
// a unit index stands for.
//
// An expert's rows are split into 128-row blocks; pairs of blocks run as
// square tiles (256 rows x 256 weight rows) and an odd last block as a wide
// tile (128 rows x 512 weight rows).  Units are (expert, chunk of up to 8 row
// blocks, 512-row weight panel, tile) in one sequence; the tiles of one chunk
// that read the same weight panel are adjacent, so the panel streams into L2
// once for all of them.  The grid is one workgroup per CU; the sequence is
// cut into 8 contiguous ranges, one per XCD (the dispatcher deals workgroup b
// to XCD b % 8), whose units that XCD's workgroups claim in order.
#pragma once

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kXcds = 8;
constexpr int kChunkBlocks = 8;                // row blocks of 128 per chunk

struct Unit {
    int e, row0, rows, n;                      // n: column tile index of this shape
};

__device__ __forceinline__ int lane_id() {
    // opaque (asm volatile): recomputed where used rather than hoisted out of
    // the persistent unit loop and kept live across the MFMA loop
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    return lane;
}

// LDS rows of one slice are 128 bytes: logical 16-byte chunk c of row r sits
// at physical chunk c ^ ((r >> 1) & 7).  A fragment read phase (16 rows at
// one logical chunk) then touches 16 distinct 4-bank groups.
__device__ __forceinline__ int pchunk8(int row, int c) { return c ^ ((row >> 1) & 7); }

// Unit L -> tile (square or wide).  tile_off: [E+1] row-block offsets,
// offsets: [E+1] row offsets, npanel: 512-row weight panels per expert, N:
// columns of the output (gate_up: h columns).  Returns false for the second
// column tile of a partial last panel (nothing to compute).
template <bool GATE_UP>
__device__ __forceinline__ bool unit_of(const int32_t* tile_off, const int32_t* offsets, int E,
                                        int npanel, int N, int L, Unit& u, bool& square, int hint = -1) {
    // expert: last e with tile_off[e] * npanel <= L; the hint (the expert of
    // the previous unit) is tried first, then the expert after it, with
    // independent loads, before a binary search
    int lo = 0, hi = E - 1;
    if (hint >= 0 && hint + 1 < E) {
        const int a = __builtin_amdgcn_readfirstlane(tile_off[hint]) * npanel;
        const int b = __builtin_amdgcn_readfirstlane(tile_off[hint + 1]) * npanel;
        const int c = hint + 2 <= E ? __builtin_amdgcn_readfirstlane(tile_off[hint + 2]) * npanel : b;
        if (a <= L && L < b) lo = hi = hint;
        else if (b <= L && L < c) lo = hi = hint + 1;
    }
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_off[mid] * npanel <= L) lo = mid;
        else hi = mid - 1;
    }
    u.e = lo;
    // the table values are uniform: kept in scalar registers, so the unit
    // arithmetic below runs on the scalar unit
    const int t0 = __builtin_amdgcn_readfirstlane(tile_off[lo]);
    const int nb_e = __builtin_amdgcn_readfirstlane(tile_off[lo + 1]) - t0;
    int v = L - t0 * npanel;
    // chunks of kChunkBlocks row blocks; a chunk of m blocks has m * npanel
    // units: for each weight panel, its square tiles (two column tiles per
    // panel, pairs of blocks) and then its wide tile (odd last block)
    const int full = nb_e / kChunkBlocks;
    int c, m;
    if (v < full * kChunkBlocks * npanel) {
        c = v / (kChunkBlocks * npanel);
        m = kChunkBlocks;
    } else {
        c = full;
        m = nb_e - full * kChunkBlocks;
    }
    v -= c * kChunkBlocks * npanel;
    const int pairs = m >> 1;
    const int panel = v / m;
    const int w = v - panel * m;
    int blk;
    square = w < 2 * pairs;
    if (square) {
        u.n = 2 * panel + w / pairs;
        blk = c * kChunkBlocks + 2 * (w % pairs);
    } else {
        u.n = panel;
        blk = c * kChunkBlocks + 2 * pairs;
    }
    u.row0 = __builtin_amdgcn_readfirstlane(offsets[lo]) + blk * 128;
    u.rows = min(square ? 256 : 128, __builtin_amdgcn_readfirstlane(offsets[lo + 1]) - u.row0);
    const int cols_sq = GATE_UP ? 128 : 256;   // output columns of a square tile
    return !(square && u.n * cols_sq >= N);
}

// Workgroups per XCD for a launch of `units` units: one workgroup per CU.
inline int persistent_grid(long long units, int cus) {
    const long long cap = cus / kXcds * kXcds > kXcds ? cus / kXcds * kXcds : kXcds;
    const long long want = (units + kXcds - 1) / kXcds * kXcds;
    return static_cast<int>(want < cap ? want : cap);
}

}  // namespace
}  // namespace hy3
