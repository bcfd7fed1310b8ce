// Grouped expert GEMMs for prefill-sized batches on CDNA4 MFMA, fp32
// accumulate, with bf16 or e4m3 operands.  Expert e's rows form M-tiles of 128
// rows; each workgroup computes one M-tile against 256 weight rows:
//
//   gate_up: weight rows = 128 gate rows c0..c0+127 and the matching 128 up
//            rows F+c0..; h[r, c] = SiLU(G) * U for 128 columns ("DeepSeek
//            V4-Flash architecture Q&A", Q4.5: SiLU on the gate branch;
//            "Tencent Hy3-295B architecture teardown", section 2.3: the fused
//            gate_up projection).  bf16: h stored as bf16.  e4m3: G and U are
//            rescaled by the row's activation scale and the channel's weight
//            scale, h is stored as fp32 and the row's max |h| is folded into
//            amax[r] (an integer atomic max on the bit pattern of |h|), for
//            the per-row quantisation of h that follows;
//   down:    weight rows = output columns n0..n0+255; y[r, n] stored as bf16
//            (e4m3: rescaled by the row and channel scales first).
//
// Both formats use 128-byte K-tiles (64 bf16 or 128 e4m3 values per row), so
// the LDS layout and the producers are byte-identical; the consumers issue
// v_mfma_f32_32x32x16_bf16 (4 per K-tile and block) or
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales (2 per K-tile and block).
//
// Eight waves with two roles.  Waves 4-7 are producers: they move K-tiles
// from global memory straight into a 3-stage LDS ring (global_load_lds_dwordx4,
// no register staging, no LDS write instructions), two K-tiles ahead of use.
// Waves 0-3 are consumers in a 2 x 2 grid, each owning 64 rows x 128 weight
// rows = 2 x 4 blocks of v_mfma_f32_32x32x16_bf16, reading fragments from
// LDS.  One barrier per K-tile; it waits on LDS traffic only (never on the
// producers' outstanding global loads).  A K-tile is 64 wide; LDS rows are
// 128 bytes with their eight 16-byte chunks XOR-swizzled (see swz), so the
// rows one fragment read touches fall in distinct banks.
// MFMA lane layout: A lane l holds row l%32, k 8*(l/32)..+8 of a 16-wide k
// slice; B the same for a weight row; C lane l holds column l%32 and rows
// 8*(j/4) + 4*(l/32) + j%4, j = 0..15.
//
// Work order: a 1-D grid over (expert, m-tile group, n-tile, m-tile): the up
// to 8 m-tiles of a group are adjacent for each n-tile, so the weight slice
// they share is fetched once into L2, and a group's A rows (at most 8 MB) are
// reused across all n-tiles before the next group starts.  Workgroups are dealt round-robin over the 8 XCDs, so the
// block index is remapped to give each XCD a contiguous run of that order.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int BM = 128;
constexpr int BNW = 256;                   // weight rows per tile
constexpr int ROWB = 128;                  // bytes of one row of a K-tile
constexpr int TILE_A = BM * ROWB;          // bytes
constexpr int TILE_B = BNW * ROWB;
constexpr int STAGE = TILE_A + TILE_B;     // 48 KB

enum Mode { GU_BF16 = 0, DN_BF16 = 1, GU_FP8 = 2, DN_FP8 = 3 };
constexpr int kStages = 3;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;                 // m-tiles visited together (see the tile order)
constexpr int kChunks = 12;                // 1 KB LDS blocks per producer wave per K-tile

union Frag {
    bf16x8_t v;
    i32x4_t q;
};

union Frag8 {                              // 32 e4m3 values
    i32x8_t v;
    i32x4_t q[2];
};

// Element offset of 16-byte chunk `chunk` of LDS row `row` (64 bf16 = 128 B per
// row).  The chunk is XORed with (row & 7) ^ ((row >> 3) & 1): 16 consecutive
// rows read at one logical chunk then cover all 64 four-byte banks exactly
// once (two 128-byte rows per 64 banks), and so do 8 consecutive rows on a
// 32-bank reading; a row's 8 chunks always land in distinct banks.
__device__ __forceinline__ int lchunk(int row, int chunk) {   // logical <-> physical, an involution
    return chunk ^ (row & 7) ^ ((row >> 3) & 1);
}
__device__ __forceinline__ int swz(int row, int chunk) {   // byte offset
    return row * ROWB + (lchunk(row, chunk) << 4);
}

__device__ __forceinline__ __attribute__((address_space(3))) void* as_lds(uint8_t* p) {
    return reinterpret_cast<__attribute__((address_space(3))) void*>(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}

// s_waitcnt with vmcnt <= kChunks (one K-tile of loads may stay in flight);
// expcnt and lgkmcnt are left at their maxima.
constexpr int kWaitOneTile = (kChunks & 0xF) | ((kChunks >> 4) << 14) | (0x7 << 4) | (0xF << 8);

// Barrier that waits for this wave's LDS accesses only; compiler fences keep
// memory operations from moving across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void k_prefill_gemm(
    const uint8_t* __restrict__ A,         // gate_up: x [T, K]; down: h [rows, K]
    const int32_t* __restrict__ tok_of,    // gate_up only
    const uint8_t* __restrict__ W,         // gate_up: [E, 2N, K]; down: [E, N, K]
    const int32_t* __restrict__ offsets,   // [E+1] row offsets
    const int32_t* __restrict__ tile_off,  // [E+1] M-tile offsets (tiles of BM rows)
    uint16_t* __restrict__ C,              // bf16 out: gate_up h [rows, N] (bf16 mode); y [rows, N]
    const float* __restrict__ a_scale,     // e4m3: per token (gate_up) or per row (down)
    const float* __restrict__ w_scale,     // e4m3: [E, 2N] (gate_up) or [E, N] (down)
    float* __restrict__ h32,               // e4m3 gate_up: h [rows, N] fp32
    uint32_t* __restrict__ amax,           // e4m3 gate_up: [rows] bits of max |h|
    int K, int N, int E, int n_tiles_n) {
    constexpr bool GATE_UP = MODE == GU_BF16 || MODE == GU_FP8;
    constexpr bool FP8 = MODE == GU_FP8 || MODE == DN_FP8;
    constexpr int ESZ = FP8 ? 1 : 2;                // bytes per element
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * STAGE];

    // XCD-aware remap of the block index onto the logical tile order
    const int G = gridDim.x;                       // a multiple of kXcds
    const int per_xcd = G / kXcds;
    const int L = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const int total = tile_off[E] * n_tiles_n;
    if (L >= total) return;
    // expert: last e with tile_off[e] * n_tiles_n <= L
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_off[mid] * n_tiles_n <= L) lo = mid;
        else hi = mid - 1;
    }
    const int e = lo;
    const int mt_e = tile_off[e + 1] - tile_off[e];
    const int local = L - tile_off[e] * n_tiles_n;
    // within the expert: groups of kGroupM m-tiles; each group runs every
    // n-tile with its m-tiles adjacent, so a group's A rows and the weight
    // slice in use both stay in L2 however many rows the expert has
    const int full = mt_e / kGroupM;
    const int span = kGroupM * n_tiles_n;
    int nt, mt;
    if (local < full * span) {
        const int g = local / span;
        const int r = local - g * span;
        nt = r / kGroupM;
        mt = g * kGroupM + (r - nt * kGroupM);
    } else {
        const int rem = mt_e - full * kGroupM;
        const int r = local - full * span;
        nt = r / rem;
        mt = full * kGroupM + (r - nt * rem);
    }
    const int row0 = offsets[e] + mt * BM;
    const int rows = min(BM, offsets[e + 1] - row0);
    const size_t kbytes = static_cast<size_t>(K) * ESZ;   // bytes of one A or weight row
    const int nk = static_cast<int>(kbytes / ROWB);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    if (wave >= 4) {
        // ------------------------------------------------------------ producer
        // A K-tile is 48 blocks of 1 KB of LDS (blocks 0-15: the 128 A rows,
        // 16-47: the 256 weight rows; 8 rows of 128 B per block).  Producer wave
        // p fills blocks 12p..12p+11 with global_load_lds_dwordx4, which writes
        // lane i's 16 bytes at block + 16 i: lane i fetches the logical chunk
        // that the swizzle maps to physical chunk i % 8 of row i / 8.
        const int p = wave - 4;
        const uint8_t* src[kChunks];
#pragma unroll
        for (int j = 0; j < kChunks; ++j) {
            const int b = p * kChunks + j;
            const int pc = lane & 7;
            if (b < 16) {
                const int row = 8 * b + (lane >> 3);
                const int r = min(row, rows - 1);           // rows past the tile end repeat a valid row
                const size_t arow = GATE_UP ? static_cast<size_t>(tok_of[row0 + r]) : static_cast<size_t>(row0 + r);
                src[j] = A + arow * kbytes + (lchunk(row, pc) << 4);
            } else {
                const int row = 8 * (b - 16) + (lane >> 3);  // 0..255
                int wrow;
                if (GATE_UP) {
                    const int c = nt * (BNW / 2) + (row & 127);
                    wrow = c < N ? (row < 128 ? 0 : N) + c : 0;
                } else {
                    wrow = nt * BNW + row;
                    wrow = wrow < N ? wrow : 0;
                }
                src[j] = W + static_cast<size_t>(e) * (GATE_UP ? 2 * N : N) * kbytes +
                         static_cast<size_t>(wrow) * kbytes + (lchunk(row, pc) << 4);
            }
        }
        // Every iteration issues one K-tile (tiles past the end re-read the last
        // one into a stage nobody reads again), so exactly kChunks loads per
        // tile are outstanding and the vmcnt waits below are exact.
#define HY3_ISSUE(KT, STG)                                                                         \
        {                                                                                          \
            const int ko_ = (KT) * ROWB;                                                           \
            uint8_t* stage_ = lds + (STG) * STAGE + p * kChunks * 1024;                            \
            _Pragma("unroll") for (int j = 0; j < kChunks; ++j)                                    \
                __builtin_amdgcn_global_load_lds(src[j] + ko_, as_lds(stage_ + j * 1024), 16, 0, 0); \
        }
        HY3_ISSUE(0, 0);
        HY3_ISSUE(min(1, nk - 1), 1);
        __builtin_amdgcn_s_waitcnt(kWaitOneTile);           // K-tile 0 has landed
        lds_barrier();
        // iteration it: consumers read stage it%3; K-tile it+2 goes into stage
        // (it+2)%3 (read last in iteration it-1); K-tile it+1 must land before
        // the barrier that ends the iteration
#define HY3_PITER(IT, STG2)                                                                        \
        {                                                                                          \
            HY3_ISSUE(min((IT) + 2, nk - 1), STG2);                                                \
            __builtin_amdgcn_s_waitcnt(kWaitOneTile);                                              \
            lds_barrier();                                                                         \
        }
        for (int it = 0; it < nk; it += 3) {
            HY3_PITER(it, 2);
            HY3_PITER(it + 1, 0);
            HY3_PITER(it + 2, 1);
        }
#undef HY3_PITER
#undef HY3_ISSUE
        return;
    }

    // ---------------------------------------------------------------- consumer
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int l32 = lane & 31;
    const int khalf = lane >> 5;
    int a_row[2], b_row[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) a_row[mb] = 64 * wm + 32 * mb + l32;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        if (GATE_UP) b_row[nb] = (nb < 2 ? 0 : 128) + 64 * wn + 32 * (nb & 1) + l32;
        else b_row[nb] = 128 * wn + 32 * nb + l32;
    }
    f32x16_t acc[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16_t{};

    lds_barrier();
    // fragments of k-step ks+1 are read while the MFMAs of step ks run.
    // bf16: 4 k-steps of 16 per K-tile, a lane's 8 values = chunk 2 ks + khalf;
    // e4m3: 2 k-steps of 64, a lane's 32 values = chunks 4 ks + 2 khalf, +1.
    constexpr int KSTEPS = FP8 ? 2 : 4;
    if constexpr (!FP8) {
#define HY3_FRAGS(SET, KS)                                                                         \
    {                                                                                              \
        const int chunk_ = 2 * (KS) + khalf;                                                       \
        _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                           \
            fa[SET][mb].q = *reinterpret_cast<const i32x4_t*>(As + swz(a_row[mb], chunk_));        \
        _Pragma("unroll") for (int nb = 0; nb < 4; ++nb)                                           \
            fb[SET][nb].q = *reinterpret_cast<const i32x4_t*>(Bs + swz(b_row[nb], chunk_));        \
    }
#define HY3_CITER(IT, STG)                                                                         \
    if ((IT) < nk) {                                                                               \
        const uint8_t* As = lds + (STG) * STAGE;                                                   \
        const uint8_t* Bs = As + TILE_A;                                                           \
        Frag fa[2][2], fb[2][4];                                                                   \
        HY3_FRAGS(0, 0);                                                                           \
        _Pragma("unroll") for (int ks = 0; ks < KSTEPS; ++ks) {                                    \
            if (ks + 1 < KSTEPS) HY3_FRAGS((ks + 1) & 1, ks + 1);                                  \
            _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                       \
                _Pragma("unroll") for (int nb = 0; nb < 4; ++nb)                                   \
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                         \
                        fa[ks & 1][mb].v, fb[ks & 1][nb].v, acc[mb][nb], 0, 0, 0);                 \
        }                                                                                          \
    }                                                                                              \
    lds_barrier();
        for (int it = 0; it < nk; it += 3) {   // ceil(nk / 3) * 3 barriers, as the producer
            HY3_CITER(it, 0);
            HY3_CITER(it + 1, 1);
            HY3_CITER(it + 2, 2);
        }
#undef HY3_CITER
#undef HY3_FRAGS
    } else {
#define HY3_FRAGS8(SET, KS)                                                                        \
    {                                                                                              \
        const int chunk_ = 4 * (KS) + 2 * khalf;                                                   \
        _Pragma("unroll") for (int mb = 0; mb < 2; ++mb) {                                         \
            fa[SET][mb].q[0] = *reinterpret_cast<const i32x4_t*>(As + swz(a_row[mb], chunk_));     \
            fa[SET][mb].q[1] = *reinterpret_cast<const i32x4_t*>(As + swz(a_row[mb], chunk_ + 1)); \
        }                                                                                          \
        _Pragma("unroll") for (int nb = 0; nb < 4; ++nb) {                                         \
            fb[SET][nb].q[0] = *reinterpret_cast<const i32x4_t*>(Bs + swz(b_row[nb], chunk_));     \
            fb[SET][nb].q[1] = *reinterpret_cast<const i32x4_t*>(Bs + swz(b_row[nb], chunk_ + 1)); \
        }                                                                                          \
    }
#define HY3_CITER8(IT, STG)                                                                        \
    if ((IT) < nk) {                                                                               \
        const uint8_t* As = lds + (STG) * STAGE;                                                   \
        const uint8_t* Bs = As + TILE_A;                                                           \
        Frag8 fa[2][2], fb[2][4];                                                                  \
        HY3_FRAGS8(0, 0);                                                                          \
        _Pragma("unroll") for (int ks = 0; ks < KSTEPS; ++ks) {                                    \
            if (ks + 1 < KSTEPS) HY3_FRAGS8((ks + 1) & 1, ks + 1);                                 \
            _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                       \
                _Pragma("unroll") for (int nb = 0; nb < 4; ++nb)                                   \
                    acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                 \
                        fa[ks & 1][mb].v, fb[ks & 1][nb].v, acc[mb][nb], 0, 0, 0, 127, 0, 127);    \
        }                                                                                          \
    }                                                                                              \
    lds_barrier();
        for (int it = 0; it < nk; it += 3) {
            HY3_CITER8(it, 0);
            HY3_CITER8(it + 1, 1);
            HY3_CITER8(it + 2, 2);
        }
#undef HY3_CITER8
#undef HY3_FRAGS8
    }

    // epilogue
    const float* ws_e = FP8 ? w_scale + static_cast<size_t>(e) * (GATE_UP ? 2 * N : N) : nullptr;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = 64 * wm + 32 * mb + 8 * (j >> 2) + 4 * khalf + (j & 3);
            if (r >= rows) continue;
            const size_t grow = static_cast<size_t>(row0 + r);
            if constexpr (MODE == GU_BF16) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int c = nt * (BNW / 2) + 64 * wn + 32 * nb + l32;
                    if (c < N) C[grow * N + c] = f32_to_bf16(silu_mul(acc[mb][nb][j], acc[mb][nb + 2][j]));
                }
            } else if constexpr (MODE == DN_BF16) {
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int c = nt * BNW + 128 * wn + 32 * nb + l32;
                    if (c < N) C[grow * N + c] = f32_to_bf16(acc[mb][nb][j]);
                }
            } else if constexpr (MODE == GU_FP8) {
                const float sx = a_scale[tok_of[grow]];
                float hmax = 0.f;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int c = nt * (BNW / 2) + 64 * wn + 32 * nb + l32;
                    if (c < N) {
                        const float g = acc[mb][nb][j] * sx * ws_e[c];
                        const float u = acc[mb][nb + 2][j] * sx * ws_e[N + c];
                        const float hv = silu_mul(g, u);
                        h32[grow * N + c] = hv;
                        hmax = fmaxf(hmax, fabsf(hv));
                    }
                }
                // row max over the 32 lanes that share this row (same khalf)
#pragma unroll
                for (int off = 16; off >= 1; off >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, off, 32));
                if (l32 == 0) atomicMax(&amax[grow], __float_as_uint(hmax));
            } else {
                const float sh = a_scale[grow];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int c = nt * BNW + 128 * wn + 32 * nb + l32;
                    if (c < N) C[grow * N + c] = f32_to_bf16(acc[mb][nb][j] * sh * ws_e[c]);
                }
            }
        }
    }
}

int grid_for(int max_mtiles, int n_tiles_n) {
    const long long g = static_cast<long long>(max_mtiles) * n_tiles_n;
    return static_cast<int>((g + kXcds - 1) / kXcds * kXcds);
}

}  // namespace

int prefill_bm() { return BM; }

hipError_t launch_gate_up_prefill(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                                  const int32_t* offsets, const int32_t* tile_off, int max_mtiles,
                                  uint16_t* h, int E, int d, int F, hipStream_t s) {
    const int ntn = (F + BNW / 2 - 1) / (BNW / 2);
    hipLaunchKernelGGL(k_prefill_gemm<GU_BF16>, dim3(grid_for(max_mtiles, ntn)), dim3(512), 0, s,
                       reinterpret_cast<const uint8_t*>(x), tok_of,
                       reinterpret_cast<const uint8_t*>(W_gu), offsets, tile_off, h, nullptr,
                       nullptr, nullptr, nullptr, d, F, E, ntn);
    return hipGetLastError();
}

hipError_t launch_down_prefill(const uint16_t* h, const uint16_t* W_dn, const int32_t* offsets,
                               const int32_t* tile_off, int max_mtiles, uint16_t* y, int E, int d,
                               int F, hipStream_t s) {
    const int ntn = (d + BNW - 1) / BNW;
    hipLaunchKernelGGL(k_prefill_gemm<DN_BF16>, dim3(grid_for(max_mtiles, ntn)), dim3(512), 0, s,
                       reinterpret_cast<const uint8_t*>(h), nullptr,
                       reinterpret_cast<const uint8_t*>(W_dn), offsets, tile_off, y, nullptr,
                       nullptr, nullptr, nullptr, F, d, E, ntn);
    return hipGetLastError();
}

hipError_t launch_gate_up_fp8(const uint8_t* xq, const float* xs, const int32_t* tok_of,
                              const uint8_t* Wq, const float* ws, const int32_t* offsets,
                              const int32_t* tile_off, int max_mtiles, float* h32, uint32_t* amax,
                              int E, int d, int F, hipStream_t s) {
    const int ntn = (F + BNW / 2 - 1) / (BNW / 2);
    hipLaunchKernelGGL(k_prefill_gemm<GU_FP8>, dim3(grid_for(max_mtiles, ntn)), dim3(512), 0, s, xq,
                       tok_of, Wq, offsets, tile_off, nullptr, xs, ws, h32, amax, d, F, E, ntn);
    return hipGetLastError();
}

hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const uint8_t* Wq, const float* ws,
                           const int32_t* offsets, const int32_t* tile_off, int max_mtiles,
                           uint16_t* y, int E, int d, int F, hipStream_t s) {
    const int ntn = (d + BNW - 1) / BNW;
    hipLaunchKernelGGL(k_prefill_gemm<DN_FP8>, dim3(grid_for(max_mtiles, ntn)), dim3(512), 0, s, hq,
                       nullptr, Wq, offsets, tile_off, y, hs, ws, nullptr, nullptr, F, d, E, ntn);
    return hipGetLastError();
}

}  // namespace hy3
