// Internal declarations shared by the HIP translation units of libhy3moe.
// Not part of the public ABI (that is include/hy3moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hy3 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Tokens per routing block: one bit per token in a 64-bit LDS mask.
constexpr int kRouteBlock = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (gfx950's v_cvt_pk_bf16_f32; NaN
// stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// SiLU(g) * u = g * u / (1 + e^-g), with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp of fp32 each).  The result is stored as
// bf16 (or quantised to e4m3), 2^-9 relative or coarser, so the fp32 error is
// far below what the stored value keeps.  Limits: g -> -inf gives 0,
// g -> +inf gives g * u.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);   // e^-g
    return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---- LDS staging used by the MFMA kernels (grouped GEMMs, router logits) ----

// LDS rows of 64 bytes keep logical 16-byte chunk c at physical chunk
// c ^ ((row >> 2) & 3): the 16 lanes of one phase of a fragment read (16 rows,
// one logical chunk) then hit 16 distinct 4-bank groups, all 64 banks once.
__device__ __forceinline__ int pchunk(int row, int c) { return c ^ ((row >> 2) & 3); }

// s_waitcnt immediate that waits until at most n vector memory operations of
// the wave are outstanding (lgkmcnt and expcnt not waited for).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// 16 bytes per lane from global memory into LDS: lane i's bytes land at
// lds_base + 16 i (lds_base is wave-uniform, passed in M0; one wait state
// between the M0 write and the copy).  Written in assembly so that the
// compiler does not treat the copy as an LDS store and wait for it before
// every LDS read; the kernels wait for their copies with explicit vmcnt
// counts.  M0 is listed as clobbered although the compiler reserves it: no
// device code of the kernels that use this touches M0 otherwise (the
// compiler sets it only for its own LDS-DMA builtins and for indirect
// register indexing, neither of which they contain).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy_to_lds(const uint8_t* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// Barrier after this wave's LDS reads have completed; copies in flight are
// not waited for.  Compiler fences keep memory operations on their side.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Compute units of the current device.  The count is queried once per device
// and kept for the life of the process (a table of atomics: concurrent first
// calls store the same value), so a launch costs one hipGetDevice.
hipError_t device_cu_count(int* cus);

// Workspace carving, computed identically on the host for every entry point.
struct Layout {
    size_t planes, partial, scores, blk_counts, blk_base, counts, offsets, tile_off, idx, w,
        row_of, tok_of, h, y, xq, xs, hq, hs, amax, xn, sched, total;
    int nb;              // routing blocks
    int nsplit;          // router d-chunks
    int max_mtiles;      // upper bound on row blocks of the grouped GEMMs
    int rows;            // expert rows: T * k, plus T with a shared expert
};

// ---- launchers (each returns hipGetLastError() after enqueueing) ----
// Router scratch: bf16 planes of W_gate [3, E, d], d-split partial logits
// [nsplit, T, E] (nsplit > 1 only), scores [T, E].
struct RouterWork {
    uint16_t* planes;
    float* partial;
    float* scores;
    int nsplit;
};
int router_nsplit(int T, int d, int E);
size_t router_plane_elems(int d, int E);
// score_bias: selection-only bias added to the scores (NULL: none)
hipError_t launch_router(const uint16_t* x, const float* W_gate, const float* bias,
                         const float* score_bias, int T, int d, int E, int k, float scale,
                         const RouterWork& rw, int32_t* idx, float* w, int32_t* blk_counts, int nb,
                         hipStream_t s);
// route_norm: xn = RMSNorm(x) * w as bf16 rows
hipError_t launch_rms_norm(const uint16_t* x, const uint16_t* w, int T, int d, float eps,
                           uint16_t* xn, hipStream_t s);

// shared = 1 appends expert E with every token as its rows (rows T*k + t),
// so offsets and tile_off then hold E + 2 entries.  checked: the routing is
// the caller's; pairs with an expert outside [0, E) or repeated within the
// token's row take no row (row_of = -1) and are counted for no expert.
// zero, nzero: ints the dispatch also sets to 0 for the kernels after it (the
// grouped GEMMs' work counters, the e4m3 decode gate_up's row maxima), or
// NULL, 0; its single-workgroup kernel clears them, so no fill launch is needed.
hipError_t launch_dispatch(const int32_t* idx, int T, int E, int k, int nb,
                           const int32_t* blk_counts, int32_t* blk_base, int32_t* counts,
                           int32_t* offsets, int32_t* tile_off, int bm, int32_t* row_of,
                           int32_t* tok_of, int shared, hipStream_t s, bool checked = false,
                           int32_t* zero = nullptr, int nzero = 0);

// prefill-sized batches: MFMA grouped GEMMs over row blocks of prefill_bm() rows
// (max_blocks bounds the number of row blocks, tile_off[E]).  E counts the
// experts of offsets/tile_off; with W_last non-NULL the last of them is the
// shared expert, whose weights are W_last instead of W[E - 1].  sched: the
// work counters, kSchedInts ints, zero before the gate_up launch (gate_up and
// down use halves of their own).
constexpr int kSchedInts = 16;
int prefill_bm();
hipError_t launch_gate_up_grouped(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                                  const uint16_t* W_last, const int32_t* offsets,
                                  const int32_t* tile_off, int max_blocks, uint16_t* h, int* sched, int E,
                                  int d, int F, hipStream_t s);
hipError_t launch_down_grouped(const uint16_t* h, const uint16_t* W_dn, const uint16_t* W_last,
                               const int32_t* offsets, const int32_t* tile_off, int max_blocks,
                               uint16_t* y, int* sched, int E, int d, int F, hipStream_t s);

// decode-sized batches: weight streaming, one workgroup per (expert, weight
// slice); E and W_last as for the grouped GEMMs
bool use_decode_path(int T, int d, int F, int E, int k, int esz, bool shared);   // esz: bytes per weight
// Decode-sized batches.  rg: 16-row groups a workgroup takes per pass (1 or
// 2, from decode_row_groups); slice_off: [E+1] offsets of the experts' slices
// of decode_bm(rg) rows (the dispatch's block offsets with that block size);
// max_slices: an upper bound on slice_off[E], the grid's column count.
int decode_row_groups(int T, int k, int E, int esz, bool shared);
int decode_bm(int rg);
hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* tok_of, const uint16_t* W_gu,
                                 const uint16_t* W_last, const int32_t* offsets,
                                 const int32_t* slice_off, int max_slices, uint16_t* h, int E, int d,
                                 int F, int rg, hipStream_t s);
hipError_t launch_down_decode(const uint16_t* h, const uint16_t* W_dn, const uint16_t* W_last,
                              const int32_t* offsets, const int32_t* slice_off, int max_slices,
                              uint16_t* y, int E, int d, int F, int rg, hipStream_t s);

// shared_row0 >= 0: row shared_row0 + t of y (the shared expert's output for
// token t) is added with weight 1 after the k routed terms
hipError_t launch_combine(const uint16_t* y, const int32_t* row_of, const float* w, float* out,
                          int T, int d, int k, int shared_row0, hipStream_t s);
// the same sum plus the bf16 residual row (if resid is not null), rounded to
// bf16 into out (which may be resid itself)
hipError_t launch_combine_bf16(const uint16_t* y, const int32_t* row_of, const float* w,
                               const uint16_t* resid, uint16_t* out, int T, int d, int k,
                               int shared_row0, hipStream_t s);

// fp8 path
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
    // OCP E4M3FN, round to nearest even, finite values saturate to +-448.
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(v);
    if (!(a == a)) return static_cast<uint8_t>(sign | 0x7fu);
    if (a >= 448.0f) return static_cast<uint8_t>(sign | 0x7eu);
    if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
        const float m = rintf(a * 512.0f);     // exact scaling, ties to even
        return static_cast<uint8_t>(sign | static_cast<uint32_t>(m));
    }
    uint32_t ua = __float_as_uint(a);          // keep 3 of 23 mantissa bits, ties to even
    ua += 0x7ffffu + ((ua >> 20) & 1u);
    const int e = static_cast<int>(ua >> 23) - 127;
    uint32_t code = (static_cast<uint32_t>(e + 7) << 3) | ((ua >> 20) & 7u);
    if (code > 0x7eu) code = 0x7eu;
    return static_cast<uint8_t>(sign | code);
}

hipError_t launch_block_counts(const int32_t* idx, int T, int E, int k, int nb,
                               int32_t* blk_counts, hipStream_t s);
// rs (optional): each row's scale also written at its k dispatch rows row_of[row * k + j]
hipError_t launch_quant_rows(const uint16_t* x, int rows, int cols, uint8_t* q, float* s,
                             hipStream_t st, const int32_t* row_of = nullptr, int k = 0,
                             float* rs = nullptr);
// bf16 h rows, their max |h|: amax_bits [rows] (bit patterns of the float;
// the weight-streaming gate_up folds them in with atomics), or, with
// amax_bits NULL, the max over the nblk partial maxima hmax[blk * rows + row]
// (the grouped gate_up's).
hipError_t launch_quant_rows_h(const uint16_t* h, const uint32_t* amax_bits, const float* hmax, int nblk,
                               int rows, int cols, uint8_t* q, float* s, hipStream_t st);
// rs: the tokens' activation scales per dispatch row (launch_quant_rows' rs)
hipError_t launch_gate_up_fp8(const uint8_t* xq, const float* rs, const int32_t* tok_of,
                              const uint8_t* Wq, const float* ws, const int32_t* offsets,
                              const int32_t* tile_off, int max_mtiles, uint16_t* h, float* hmax,
                              int rows, int* sched, int E, int d, int F, hipStream_t s);
hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const uint8_t* Wq, const float* ws,
                           const int32_t* offsets, const int32_t* tile_off, int max_mtiles,
                           uint16_t* y, int* sched, int E, int d, int F, hipStream_t s);
// decode-sized batches with e4m3 experts (weight streaming, as the bf16 ones).
// block: ws holds one fp32 scale per 128 x 128 weight block, [E, rows/128,
// K/128] (rows = 2F for gate_up, d for down; K = d, F), instead of one per
// output channel; K <= 16384.
hipError_t launch_gate_up_decode_fp8(const uint8_t* xq, const float* xs, const int32_t* tok_of,
                                     const uint8_t* Wq, const float* ws, const int32_t* offsets,
                                     const int32_t* slice_off, int max_slices, uint16_t* h,
                                     uint32_t* amax, int E, int d, int F, int rg, bool block,
                                     hipStream_t s);
hipError_t launch_down_decode_fp8(const uint8_t* hq, const float* hs, const uint8_t* Wq,
                                  const float* ws, const int32_t* offsets, const int32_t* slice_off,
                                  int max_slices, uint16_t* y, int E, int d, int F, int rg, bool block,
                                  hipStream_t s);

// prefill-sized batches with e4m3 weights in 128 x 128 blocks (one fp32
// scale each, sb [E, rows/128, K/128]); K <= 16384, tile_off in 128-row blocks
hipError_t launch_gate_up_fp8_block(const uint8_t* xq, const float* rs, const int32_t* tok_of,
                                    const uint8_t* Wq, const float* sb, const int32_t* offsets,
                                    const int32_t* tile_off, int max_mtiles, uint16_t* h,
                                    float* hmax, int rows, int* sched, int E, int d, int F, hipStream_t s);
hipError_t launch_down_fp8_block(const uint8_t* hq, const float* hs, const uint8_t* Wq,
                                 const float* sb, const int32_t* offsets, const int32_t* tile_off,
                                 int max_mtiles, uint16_t* y, int* sched, int E, int d, int F, hipStream_t s);

}  // namespace hy3
