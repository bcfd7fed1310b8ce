// Expert GEMMs for decode-sized batches: each expert sees a handful of rows,
// so the work is streaming the touched experts' weights from HBM once.
//
// One workgroup = one expert x one slice of weight rows (two slices in turn
// for e4m3); 4 waves, each owning 32 weight rows over the full K and the
// expert's rows 16 at a time.  MFMA:
//   bf16  v_mfma_f32_16x16x32_bf16: A = 16 token rows x 32 k, B = 32 k x 16
//         weight rows; lane l holds row l%16 and k 8*(l/16)..+8 of both;
//   e4m3  v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales): 128 k per step,
//         lane l holds row l%16 and k 32*(l/16)..+32 of both;
// C lane l holds column l%16, rows 4*(l/16)..+4.
//
// Weights are read in the order HBM streams best: each load instruction
// covers 4 weight rows x 256 contiguous bytes (128 bf16 or 256 e4m3 values of
// k), the next batch already in flight in registers while the current one is
// used.  The MFMA wants each lane on a single row, so every batch goes through
// a wave-private 8 KB LDS slab [32 rows][256 bytes] whose 16-byte chunks are
// XOR-swizzled by (row & 15): the 16-row fragment reads then hit 16 different
// bank groups.  Only the owning wave touches its slab, so no barrier is needed.
//
// gate_up: wave w of block (e, c0) owns gate rows c0+16w..+16 and the matching
//          up rows F+c0+16w..+16 ("DeepSeek V4-Flash architecture Q&A", Q4.5:
//          SiLU on the gate branch).  bf16: h[r, c] = bf16(SiLU(g) * u).
//          e4m3: g and u are rescaled by the token's activation scale and the
//          channel's weight scale (Q7.4: one scale per output channel), h is
//          stored as bf16 and the row's max |bf16(h)| folded into amax[r]
//          (integer atomic max on the bit pattern of the float) for the row
//          quantiser that follows.
// down:    wave w of block (e, n0) owns W_down rows n0+32w..+32 and writes
//          y[r, n] = bf16(h[r] . W_down[e][n]) (e4m3: rescaled by the row's
//          and the channel's scales first).
// Every expert's rows are cut into 16-row slices (their offsets come from the
// dispatch run with a 16-row block), one column of workgroups per slice, so
// an expert with many rows streams its weights in parallel columns rather
// than in serial passes.  The shared expert of the full block, when present,
// is the last expert (all T tokens, weights W_last).

#include "internal.h"

namespace hy3 {
namespace {

// FP8B: e4m3 weights with one fp32 scale per 128 x 128 block (below).
enum Mode { GU_BF16 = 0, DN_BF16 = 1, GU_FP8 = 2, DN_FP8 = 3, GU_FP8B = 4, DN_FP8B = 5 };

// Column blocks per workgroup, taken one after the other with the weight
// stream running on across the boundary.  An e4m3 block moves half the bytes
// of a bf16 one, so two of them halve the per-workgroup start and end costs
// (measured at T = 64: gate_up 0.400 -> 0.393 ms, down 0.197 -> 0.186 ms);
// four e4m3 gate_up blocks cost occupancy.  Down blocks (128 rows of d_ff)
// are short: e4m3 takes four per workgroup where d allows (T = 64 down
// 0.191 -> 0.187 ms), bf16 two (0.363 -> 0.355 ms; four gained under 1% and
// lost as much with skewed routing).  The bf16 gate_up keeps one: two gained
// 0.6% at T = 64 but cost 3% with skewed routing, where fewer, longer
// workgroups balance worse.  The e4m3 path needs d and d_ff in whole 256-byte
// batches, so the halved grids divide evenly.
constexpr int kSubsBf16 = 1;
constexpr int kSubsBf16Down = 2;        // where d is a multiple of 256
constexpr int kSubsFp8 = 2;
constexpr int kSubsFp8Down = 4;         // where d is a multiple of 512

constexpr int kBatchB = 256;            // bytes of k per row and batch
constexpr int kSlabB = 32 * kBatchB;    // bytes of one wave's LDS slab (8 KB)

__device__ __forceinline__ int slab_off(int row, int chunk) {   // byte offset, 16 chunks per row
    return row * kBatchB + ((chunk ^ (row & 15)) << 4);
}

struct DecodeArgs {
    const uint8_t* A;                   // gate_up: x (or its e4m3 codes) [T, K]; down: h [rows, K]
    const int32_t* tok_of;              // gate_up only
    const uint8_t* W;                   // gate_up: [E, 2N, K]; down: [E, N, K]
    const uint8_t* W_last;              // non-NULL: weights of expert E - 1 (shared)
    const int32_t* offsets;
    const int32_t* slice_off;           // [E+1] offsets in 16-row slices (one workgroup column each)
    uint16_t* C;                        // bf16 out: gate_up h or down y [rows, N]
    const float* a_scale;               // e4m3: per token (gate_up) or per row (down)
    const float* w_scale;               // e4m3: [E, 2N] (gate_up) or [E, N] (down)
    uint32_t* amax;                     // e4m3 gate_up: [rows] bits of max |h|
    int K, N;                           // K in elements
    int E;                              // experts, the shared one included
};

// Waves per SIMD the register allocation is held to (more waves, more weight
// batches in flight): every one-group kernel fits four (bf16 five, unbounded),
// two groups four (bf16) or three (e4m3 down) without spilling; the e4m3
// gate_up with two groups is left unbounded (two waves).
constexpr int decode_min_waves(int mode, int rg) {
    return rg == 1 ? 4 : mode <= DN_BF16 ? 4 : (mode == DN_FP8 || mode == DN_FP8B) ? 3 : 1;
}

template <int MODE, int SUBS, int RG>
__global__ __launch_bounds__(256, decode_min_waves(MODE, RG)) void k_decode_gemm(DecodeArgs g) {
    constexpr bool GATE_UP = MODE == GU_BF16 || MODE == GU_FP8 || MODE == GU_FP8B;
    constexpr bool BLK = MODE == GU_FP8B || MODE == DN_FP8B;
    constexpr bool FP8 = MODE >= GU_FP8;
    constexpr int ESZ = FP8 ? 1 : 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kSlabB];
    const int E = g.E;
    // Every expert's rows are cut into 16-row slices, one column of workgroups
    // each, so an expert with many rows (a hot expert, or the shared one with
    // all T tokens) streams its weights in parallel columns rather than in
    // serial passes.  Column L: the last expert e with slice_off[e] <= L.
    const int L = static_cast<int>(blockIdx.x);
    if (L >= __builtin_amdgcn_readfirstlane(g.slice_off[E])) return;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (__builtin_amdgcn_readfirstlane(g.slice_off[mid]) <= L) lo = mid;
        else hi = mid - 1;
    }
    const int e = lo;
    const int rbeg = __builtin_amdgcn_readfirstlane(g.offsets[e]) +
                     16 * RG * (L - __builtin_amdgcn_readfirstlane(g.slice_off[e]));
    const int rend = min(rbeg + 16 * RG, __builtin_amdgcn_readfirstlane(g.offsets[e + 1]));
    if (rbeg >= rend) return;
    const int K = g.K, N = g.N;
    const size_t rowbytes = static_cast<size_t>(K) * ESZ;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int r16 = lane & 15;
    const int kq = lane >> 4;                          // quarter of the lane group
    uint8_t* slab = lds + wave * kSlabB;

    // weight row of slab row sr (0..31): n-tile sr/16, row sr%16 of it
    const uint8_t* We = (g.W_last && e == E - 1)
                            ? g.W_last
                            : g.W + static_cast<size_t>(e) * (GATE_UP ? 2 * N : N) * rowbytes;
    constexpr int SUBROWS = GATE_UP ? 64 : 128;        // columns of one block
    auto wrow_of = [&](int sr) -> int {               // block 0 of this workgroup
        if (GATE_UP) return (sr < 16 ? 0 : N) + blockIdx.y * 64 * SUBS + wave * 16 + (sr & 15);
        return blockIdx.y * 128 * SUBS + wave * 32 + sr;
    };
    const int colb = GATE_UP ? blockIdx.y * 64 * SUBS + wave * 16 : blockIdx.y * 128 * SUBS + wave * 32;
    const size_t sub_stride = static_cast<size_t>(SUBROWS) * rowbytes;
    // load instruction i (0..7) of a batch: slab rows 4i + lane/16, bytes
    // (lane%16)*16.  Its address is a wave-uniform base (weight row
    // wrow_of(4i), kept in scalar registers) plus the lane's 32-bit offset.
    const uint8_t* wsrc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wsrc[i] = We + static_cast<size_t>(wrow_of(4 * i)) * rowbytes;
    const uint32_t wlane = static_cast<uint32_t>(kq * rowbytes) + r16 * 16;
    int wdst[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wdst[i] = slab_off(4 * i + kq, r16);

    // e4m3: this lane's column scales per block (column col0 + r16, and + 16 for down)
    float ws0[SUBS], ws1[SUBS];
    // block scales: the wave's acc0 / acc1 weight rows lie in one 128-row
    // block each; lane i keeps that block row's scales of k-blocks i and 64 + i
    int bsc0[SUBS][2], bsc1[SUBS][2];
#pragma unroll
    for (int sb = 0; sb < SUBS; ++sb) {
        ws0[sb] = BLK ? 1.f : 0.f;
        ws1[sb] = BLK ? 1.f : 0.f;
        bsc0[sb][0] = bsc0[sb][1] = bsc1[sb][0] = bsc1[sb][1] = 0;
        if constexpr (BLK) {
            const int KB = K >> 7;
            const float* se = g.w_scale + static_cast<size_t>(e) * ((GATE_UP ? 2 * N : N) >> 7) * KB;
            const int c0 = colb + sb * SUBROWS;
            const int nb0 = c0 >> 7, nb1 = GATE_UP ? (N + c0) >> 7 : (c0 + 16) >> 7;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kk = lane + 64 * h;
                bsc0[sb][h] = kk < KB ? __float_as_int(se[static_cast<size_t>(nb0) * KB + kk]) : 0;
                bsc1[sb][h] = kk < KB ? __float_as_int(se[static_cast<size_t>(nb1) * KB + kk]) : 0;
            }
        } else if constexpr (FP8) {
            const float* ws_e = g.w_scale + static_cast<size_t>(e) * (GATE_UP ? 2 * N : N);
            const int c0 = colb + sb * SUBROWS;
            ws0[sb] = ws_e[c0 + r16];
            ws1[sb] = GATE_UP ? ws_e[N + c0 + r16] : ws_e[c0 + 16 + r16];
        }
    }

    const int nb = static_cast<int>(rowbytes / kBatchB);
    for (int p0 = rbeg; p0 < rend; p0 += 16 * RG) {
        // row group q of the pass: rows p0 + 16 q .. + 16; this lane loads A
        // row p0 + 16 q + r16, or the pass's last row past its end (rows of
        // the MFMA are independent, and those outputs are not stored).  The
        // lane's offset into A is 32-bit (A holds at most a few thousand rows).
        uint32_t a[RG];
#pragma unroll
        for (int q = 0; q < RG; ++q) {
            const int prow = min(p0 + 16 * q + r16, rend - 1);
            const uint32_t arow = static_cast<uint32_t>(GATE_UP ? g.tok_of[prow] : prow);
            // this lane's A bytes within a batch start at kq * (FP8 ? 32 : 16)
            a[q] = arow * static_cast<uint32_t>(rowbytes) + kq * (FP8 ? 32 : 16);
        }

        f32x4_t acc0[RG], acc1[RG];
#pragma unroll
        for (int q = 0; q < RG; ++q) {
            acc0[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc1[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // One weight batch is in flight per wave: batch bt + 1 is loaded into
        // the registers that batch bt leaves once it is in the slab.  Each
        // batch's A fragments are loaded before that (loads return in order,
        // so the wait for them does not include the weight batch behind them).
        i32x4_t wb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) wb[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(wsrc[i] + wlane));
        const int nbt = nb * SUBS;
        for (int bt = 0; bt < nbt; ++bt) {
            const int sb = bt / nb, b = bt - sb * nb;
            const int kb = b * kBatchB;
            const int btn = bt + 1 < nbt ? bt + 1 : bt;      // last batch re-reads itself
            const int sbn = btn / nb;
            const size_t kn = sbn * sub_stride + static_cast<size_t>(btn - sbn * nb) * kBatchB;
            // A: e4m3 2 k-steps of 128, the lane's 32 bytes of step s at
            // 128 s (j = 2 s + half); bf16 4 k-steps of 32, 16 bytes at 64 j
            i32x4_t av[RG][4];
#pragma unroll
            for (int q = 0; q < RG; ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    av[q][j] = *reinterpret_cast<const i32x4_t*>(g.A + kb + a[q] +
                                                                 (FP8 ? 128 * (j >> 1) + 16 * (j & 1) : 64 * j));
#pragma unroll
            for (int i = 0; i < 8; ++i) *reinterpret_cast<i32x4_t*>(slab + wdst[i]) = wb[i];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wb[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(wsrc[i] + kn + wlane));
            __builtin_amdgcn_sched_barrier(0);                // the batch goes out before the MFMAs wait on A
            if constexpr (FP8) {
                // 2 k-steps of 128: lane's 32 bytes = chunks 8 s + 2 kq, +1
                // block scales of this batch's two k-blocks (2b, 2b + 1)
                float sc0[2] = {1.f, 1.f}, sc1[2] = {1.f, 1.f};
                if constexpr (BLK) {
                    int v0[2] = {bsc0[0][0], bsc0[0][1]}, v1[2] = {bsc1[0][0], bsc1[0][1]};
#pragma unroll
                    for (int q = 1; q < SUBS; ++q)
                        if (sb == q) {
                            v0[0] = bsc0[q][0]; v0[1] = bsc0[q][1];
                            v1[0] = bsc1[q][0]; v1[1] = bsc1[q][1];
                        }
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int kblk = 2 * b + s;
                        const bool hi = kblk >= 64;
                        sc0[s] = __int_as_float(__builtin_amdgcn_readlane(hi ? v0[1] : v0[0], kblk & 63));
                        sc1[s] = __int_as_float(__builtin_amdgcn_readlane(hi ? v1[1] : v1[0], kblk & 63));
                    }
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int ch = 8 * s + 2 * kq;
                    const i32x4_t b00 = *reinterpret_cast<const i32x4_t*>(slab + slab_off(r16, ch));
                    const i32x4_t b01 = *reinterpret_cast<const i32x4_t*>(slab + slab_off(r16, ch + 1));
                    const i32x4_t b10 = *reinterpret_cast<const i32x4_t*>(slab + slab_off(16 + r16, ch));
                    const i32x4_t b11 = *reinterpret_cast<const i32x4_t*>(slab + slab_off(16 + r16, ch + 1));
                    const i32x8_t f0 = __builtin_shufflevector(b00, b01, 0, 1, 2, 3, 4, 5, 6, 7);
                    const i32x8_t f1 = __builtin_shufflevector(b10, b11, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int q = 0; q < RG; ++q) {
                        const i32x8_t fa = __builtin_shufflevector(av[q][2 * s], av[q][2 * s + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                        if constexpr (BLK) {
                            // one k-step is one 128-wide k-block: its product
                            // is scaled by the block's scale and added in fp32
                            const f32x4_t z{0.f, 0.f, 0.f, 0.f};
                            const f32x4_t t0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, f0, z, 0, 0, 0, 127, 0, 127);
                            const f32x4_t t1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, f1, z, 0, 0, 0, 127, 0, 127);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                acc0[q][i] = fmaf(t0[i], sc0[s], acc0[q][i]);
                                acc1[q][i] = fmaf(t1[i], sc1[s], acc1[q][i]);
                            }
                        } else {
                            acc0[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, f0, acc0[q], 0, 0, 0, 127, 0, 127);
                            acc1[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, f1, acc1[q], 0, 0, 0, 127, 0, 127);
                        }
                    }
                }
            } else {
                // 4 k-steps of 32: lane's 16 bytes = chunk 4 s + kq
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const i32x4_t f0 = *reinterpret_cast<const i32x4_t*>(slab + slab_off(r16, 4 * s + kq));
                    const i32x4_t f1 = *reinterpret_cast<const i32x4_t*>(slab + slab_off(16 + r16, 4 * s + kq));
#pragma unroll
                    for (int q = 0; q < RG; ++q) {
                        acc0[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[q][s]),
                                                                          __builtin_bit_cast(bf16x8_t, f0), acc0[q], 0, 0, 0);
                        acc1[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[q][s]),
                                                                          __builtin_bit_cast(bf16x8_t, f1), acc1[q], 0, 0, 0);
                    }
                }
            }
            if (b != nb - 1) continue;
            // end of block sb: C lane l: column l%16, rows 4*(l/16)+i of each row group
            const int col0 = colb + sb * SUBROWS;
            float w0 = ws0[0], w1 = ws1[0];
#pragma unroll
            for (int q = 1; q < SUBS; ++q) if (sb == q) { w0 = ws0[q]; w1 = ws1[q]; }
#pragma unroll
            for (int q = 0; q < RG; ++q) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = p0 + 16 * q + kq * 4 + i;
                    const bool vr = row < rend;
                    const size_t crow = static_cast<size_t>(vr ? row : rbeg);
                    if constexpr (MODE == GU_BF16) {
                        if (vr) g.C[crow * N + col0 + r16] = f32_to_bf16(silu_mul(acc0[q][i], acc1[q][i]));
                    } else if constexpr (MODE == DN_BF16) {
                        if (vr) {
                            g.C[crow * N + col0 + r16] = f32_to_bf16(acc0[q][i]);
                            g.C[crow * N + col0 + 16 + r16] = f32_to_bf16(acc1[q][i]);
                        }
                    } else if constexpr (MODE == GU_FP8 || MODE == GU_FP8B) {
                        const float sx = g.a_scale[g.tok_of[crow]];
                        const uint16_t hv = f32_to_bf16(silu_mul(acc0[q][i] * sx * w0, acc1[q][i] * sx * w1));
                        if (vr) g.C[crow * N + col0 + r16] = hv;
                        // row max over the 16 lanes that share this row
                        float m = fabsf(bf16_to_f32(hv));
#pragma unroll
                        for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
                        if (vr && r16 == 0) atomicMax(&g.amax[crow], __float_as_uint(m));
                    } else {
                        const float sh = g.a_scale[crow];
                        if (vr) {
                            g.C[crow * N + col0 + r16] = f32_to_bf16(acc0[q][i] * sh * w0);
                            g.C[crow * N + col0 + 16 + r16] = f32_to_bf16(acc1[q][i] * sh * w1);
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < RG; ++q) {
                acc0[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                acc1[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
}

}  // namespace

// Rows per pass: a workgroup takes up to 16 rows (one MFMA row group) or 32
// (two groups sharing every weight batch).  Two groups stream an expert with
// 17-32 rows once instead of twice, but hold more registers (bf16: four waves
// per SIMD instead of five; e4m3 gate_up: two instead of four).  Measured on
// the whole layer at d = 4096, E = 192, k = 8, d_ff = 1536 (one group / two):
// bf16 T = 64 1.065 / 1.094 ms, T = 96 1.132 / 1.136, T = 128 1.167 / 1.149,
// T = 160 1.191 / 1.170, T = 192 1.260 / 1.183; e4m3 T = 128 0.664 / 0.668,
// T = 160 0.685 / 0.691, T = 192 0.735 / 0.702.  So two groups from 5 rows
// per expert on average with bf16 weights (esz 2), from 8 with e4m3.
int decode_row_groups(int T, int k, int E, int esz, bool shared) {
    (void)shared;
    return static_cast<long long>(T) * k >= (esz == 2 ? 5LL : 8LL) * E ? 2 : 1;
}

// Decode path up to about 11 rows per expert on average with one row group
// and 20 with two; rows of d and d_ff elements of esz bytes must be whole
// 256-byte batches.  Measured on the whole layer at the same dims (this path
// vs the grouped GEMMs): bf16 T = 384 1.302 vs 1.360 ms, T = 448 1.341 vs
// 1.367, T = 512 1.489 vs 1.373; e4m3 T = 384 0.781 vs 0.810, T = 448 0.812
// vs 0.818, T = 512 0.891 vs 0.825.  The full block's shared expert adds T
// rows, counted twice: each of its slices streams a whole expert's weights.
// The kernels address their A operand (x [T, d] or h [rows, d_ff], esz bytes
// per element as the weights) with 32-bit byte offsets, so both must stay
// under 4 GiB.
bool use_decode_path(int T, int d, int F, int E, int k, int esz, bool shared) {
    const long long rows = static_cast<long long>(T) * k + (shared ? 2LL * T : 0);
    const int rg = decode_row_groups(T, k, E, esz, shared);
    const bool a32 = static_cast<long long>(T) * d * esz < (1LL << 32) && rows * F * esz < (1LL << 32);
    return rows <= (rg == 2 ? 20LL : 11LL) * E && (d * esz) % kBatchB == 0 && (F * esz) % kBatchB == 0 && a32;
}

int decode_bm(int rg) { return 16 * rg; }

hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                                 const uint16_t* W_last, const int32_t* offsets,
                                 const int32_t* slice_off, int max_slices, uint16_t* h, int E, int d,
                                 int F, int rg, hipStream_t s) {
    DecodeArgs g{reinterpret_cast<const uint8_t*>(x), tok_of, reinterpret_cast<const uint8_t*>(W_gu),
                 reinterpret_cast<const uint8_t*>(W_last), offsets, slice_off, h, nullptr, nullptr,
                 nullptr, d, F, E};
    if (max_slices == 0) return hipSuccess;
    const dim3 grid(max_slices, F / (64 * kSubsBf16));
    if (rg == 2) hipLaunchKernelGGL((k_decode_gemm<GU_BF16, kSubsBf16, 2>), grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL((k_decode_gemm<GU_BF16, kSubsBf16, 1>), grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_down_decode(const uint16_t* h, const uint16_t* W_dn, const uint16_t* W_last,
                              const int32_t* offsets, const int32_t* slice_off, int max_slices,
                              uint16_t* y, int E, int d, int F, int rg, hipStream_t s) {
    DecodeArgs g{reinterpret_cast<const uint8_t*>(h), nullptr, reinterpret_cast<const uint8_t*>(W_dn),
                 reinterpret_cast<const uint8_t*>(W_last), offsets, slice_off, y, nullptr, nullptr,
                 nullptr, F, d, E};
    if (max_slices == 0) return hipSuccess;
    if (d % (128 * kSubsBf16Down) == 0) {
        const dim3 grid(max_slices, d / (128 * kSubsBf16Down));
        if (rg == 2) hipLaunchKernelGGL((k_decode_gemm<DN_BF16, kSubsBf16Down, 2>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((k_decode_gemm<DN_BF16, kSubsBf16Down, 1>), grid, dim3(256), 0, s, g);
    } else {
        const dim3 grid(max_slices, d / (128 * kSubsBf16));
        if (rg == 2) hipLaunchKernelGGL((k_decode_gemm<DN_BF16, kSubsBf16, 2>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((k_decode_gemm<DN_BF16, kSubsBf16, 1>), grid, dim3(256), 0, s, g);
    }
    return hipGetLastError();
}

hipError_t launch_gate_up_decode_fp8(const uint8_t* xq, const float* xs, const int32_t* tok_of,
                                     const uint8_t* Wq, const float* ws, const int32_t* offsets,
                                     const int32_t* slice_off, int max_slices, uint16_t* h,
                                     uint32_t* amax, int E, int d, int F, int rg, bool block,
                                     hipStream_t s) {
    DecodeArgs g{xq, tok_of, Wq, nullptr, offsets, slice_off, h, xs, ws, amax, d, F, E};
    if (max_slices == 0) return hipSuccess;
    const dim3 grid(max_slices, F / (64 * kSubsFp8));
    if (block) {
        if (rg == 2) hipLaunchKernelGGL((k_decode_gemm<GU_FP8B, kSubsFp8, 2>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((k_decode_gemm<GU_FP8B, kSubsFp8, 1>), grid, dim3(256), 0, s, g);
    } else {
        if (rg == 2) hipLaunchKernelGGL((k_decode_gemm<GU_FP8, kSubsFp8, 2>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((k_decode_gemm<GU_FP8, kSubsFp8, 1>), grid, dim3(256), 0, s, g);
    }
    return hipGetLastError();
}

hipError_t launch_down_decode_fp8(const uint8_t* hq, const float* hs, const uint8_t* Wq,
                                  const float* ws, const int32_t* offsets, const int32_t* slice_off,
                                  int max_slices, uint16_t* y, int E, int d, int F, int rg, bool block,
                                  hipStream_t s) {
    DecodeArgs g{hq, nullptr, Wq, nullptr, offsets, slice_off, y, hs, ws, nullptr, F, d, E};
    if (max_slices == 0) return hipSuccess;
#define HY3_DN_FP8(SUBS)                                                                                   \
    do {                                                                                                   \
        const dim3 grid(max_slices, d / (128 * (SUBS)));                                                   \
        if (block) {                                                                                       \
            if (rg == 2) hipLaunchKernelGGL((k_decode_gemm<DN_FP8B, SUBS, 2>), grid, dim3(256), 0, s, g);  \
            else hipLaunchKernelGGL((k_decode_gemm<DN_FP8B, SUBS, 1>), grid, dim3(256), 0, s, g);          \
        } else {                                                                                           \
            if (rg == 2) hipLaunchKernelGGL((k_decode_gemm<DN_FP8, SUBS, 2>), grid, dim3(256), 0, s, g);   \
            else hipLaunchKernelGGL((k_decode_gemm<DN_FP8, SUBS, 1>), grid, dim3(256), 0, s, g);           \
        }                                                                                                  \
    } while (0)
    if (d % (128 * kSubsFp8Down) == 0) HY3_DN_FP8(kSubsFp8Down);
    else HY3_DN_FP8(kSubsFp8);
#undef HY3_DN_FP8
    return hipGetLastError();
}

}  // namespace hy3
