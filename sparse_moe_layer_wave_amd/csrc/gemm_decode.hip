// Expert GEMMs for decode-sized batches: each expert sees a handful of rows,
// so the work is streaming the touched experts' weights from HBM once.
//
// One workgroup = one expert x one slice of weight rows; 4 waves, each owning
// 32 weight rows over the full K and the expert's rows 16 at a time
// (v_mfma_f32_16x16x32_bf16: A = 16 token rows x 32 k, B = 32 k x 16 weight
// rows; lane l holds row l%16 and k 8*(l/16)..+8 of both; C lane l holds
// column l%16, rows 4*(l/16)..+4).
//
// Weights are read in the order HBM streams best: each load instruction
// covers 4 weight rows x 256 contiguous bytes (a whole-row run of 128 k),
// the next batch already in flight in registers while the current one is
// used.  The MFMA wants each lane on a single row, so every batch goes through
// a wave-private 8 KB LDS slab [32 rows][128 k] whose 16-byte chunks are XOR-
// swizzled by (row & 15): the 16-row fragment reads then hit 16 different
// bank groups.  Only the owning wave touches its slab, so no barrier is needed.
//
// gate_up: wave w of block (e, c0) owns gate rows c0+16w..+16 and the matching
//          up rows F+c0+16w..+16, and writes h[r, c] = bf16(SiLU(g) * u)
//          ("DeepSeek V4-Flash architecture Q&A", Q4.5).
// down:    wave w of block (e, n0) owns W_down rows n0+32w..+32 and writes
//          y[r, n] = bf16(h[r] . W_down[e][n]).
// An expert with more than 16 rows is handled in passes of 16 rows.  The
// shared expert of the full block, when present, is the last expert (all T
// tokens, weights W_last); its workgroups are the longest, so they are
// scheduled first.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kBatchK = 128;            // k per batch (4 MFMA k-steps of 32)
constexpr int kSlab = 32 * kBatchK;     // bf16 elements of one wave's LDS slab (8 KB)

union Frag {
    bf16x8_t v;
    i32x4_t q;
};

__device__ __forceinline__ int slab_off(int row, int chunk) {   // element offset, 16 chunks per row
    return row * kBatchK + ((chunk ^ (row & 15)) << 3);
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) void k_decode_gemm(
    const uint16_t* __restrict__ A,        // gate_up: x [T, K]; down: h [rows, K]
    const int32_t* __restrict__ tok_of,    // gate_up only
    const uint16_t* __restrict__ W,        // gate_up: [E, 2N, K]; down: [E, N, K]
    const uint16_t* __restrict__ W_last,   // non-NULL: weights of expert E - 1 (shared)
    const int32_t* __restrict__ offsets,
    uint16_t* __restrict__ C,              // gate_up: h [rows, N]; down: y [rows, N]
    int K, int N) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kSlab];
    const int E = gridDim.x;
    const int e = W_last ? (blockIdx.x == 0 ? E - 1 : blockIdx.x - 1) : blockIdx.x;
    const int rbeg = offsets[e];
    const int rend = offsets[e + 1];
    if (rbeg == rend) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int kq = (lane >> 4) * 8;
    uint16_t* slab = lds + wave * kSlab;

    // weight row of slab row sr (0..31): n-tile sr/16, row sr%16 of it
    int col0;
    const uint16_t* We = (W_last && e == E - 1) ? W_last : W + static_cast<size_t>(e) * (GATE_UP ? 2 * N : N) * K;
    auto wrow_of = [&](int sr) -> int {
        if (GATE_UP) return (sr < 16 ? 0 : N) + blockIdx.y * 64 + wave * 16 + (sr & 15);
        return blockIdx.y * 128 + wave * 32 + sr;
    };
    col0 = GATE_UP ? blockIdx.y * 64 + wave * 16 : blockIdx.y * 128 + wave * 32;
    // load instruction i (0..7) of a batch: slab rows 4i + lane/16, bytes (lane%16)*16
    const uint16_t* wsrc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        wsrc[i] = We + static_cast<size_t>(wrow_of(4 * i + (lane >> 4))) * K + (lane & 15) * 8;
    int wdst[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wdst[i] = slab_off(4 * i + (lane >> 4), lane & 15);

    const int nb = K / kBatchK;
    for (int p0 = rbeg; p0 < rend; p0 += 16) {
        const int prow = p0 + r16;                    // A row this lane loads
        const bool va = prow < rend;
        const uint16_t* a;
        if (GATE_UP) a = A + static_cast<size_t>(va ? tok_of[prow] : 0) * K + kq;
        else a = A + static_cast<size_t>(va ? prow : 0) * K + kq;

        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
        f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
        i32x4_t cur[8], nxt[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(wsrc[i]));
        for (int b = 0; b < nb; ++b) {
            const int kb = b * kBatchK;
            const int kn = (b + 1 < nb ? b + 1 : b) * kBatchK;   // last batch re-reads itself
#pragma unroll
            for (int i = 0; i < 8; ++i)
                nxt[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(wsrc[i] + kn));
            i32x4_t av[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                av[s] = va ? *reinterpret_cast<const i32x4_t*>(a + kb + 32 * s) : i32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) *reinterpret_cast<i32x4_t*>(slab + wdst[i]) = cur[i];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                // lane l: slab row (nt*16 + l%16), logical chunk 4 s + l/16
                Frag fa, f0, f1;
                fa.q = av[s];
                f0.q = *reinterpret_cast<const i32x4_t*>(slab + slab_off(r16, 4 * s + (lane >> 4)));
                f1.q = *reinterpret_cast<const i32x4_t*>(slab + slab_off(16 + r16, 4 * s + (lane >> 4)));
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.v, f0.v, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.v, f1.v, acc1, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) cur[i] = nxt[i];
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
                    C[static_cast<size_t>(row) * N + col0 + 16 + r16] = f32_to_bf16(acc1[i]);
                }
            }
        }
    }
}

}  // namespace

// Decode path while the average expert gets at most 4 rows (so nearly every
// expert fits one 16-row pass); needs d and d_ff to be multiples of 128.
bool use_decode_path(int T, int d, int F, int E, int k) {
    return static_cast<long long>(T) * k <= 4LL * E && (d % 128) == 0 && (F % 128) == 0;
}

hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                                 const uint16_t* W_last, const int32_t* offsets, uint16_t* h,
                                 int E, int d, int F, hipStream_t s) {
    hipLaunchKernelGGL(k_decode_gemm<true>, dim3(E, F / 64), dim3(256), 0, s, x, tok_of, W_gu,
                       W_last, offsets, h, d, F);
    return hipGetLastError();
}

hipError_t launch_down_decode(const uint16_t* h, const uint16_t* W_dn, const uint16_t* W_last,
                              const int32_t* offsets, uint16_t* y, int E, int d, int F,
                              hipStream_t s) {
    hipLaunchKernelGGL(k_decode_gemm<false>, dim3(E, d / 128), dim3(256), 0, s, h, nullptr, W_dn,
                       W_last, offsets, y, F, d);
    return hipGetLastError();
}

}  // namespace hy3
