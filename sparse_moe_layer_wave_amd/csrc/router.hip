// Router of the Hy3 MoE layer: fp32 logits, sigmoid scores, top-k selection
// and the renormalised, scaled weights ("Tencent Hy3-295B architecture
// teardown", section 4.1, router flow steps 1-5), and route_norm, the RMSNorm
// of the router's input ("Tencent Hy3-Flash Q&A", Q4.9).
//
// Logits.  The gate weight is fp32 and the hidden states are bf16; the pages'
// router casts both to float before the linear map.  Each fp32 weight w is
// split into three bf16 planes by truncation, w = hi + mid + lo exactly (8
// significant bits each), so x.w = x.hi + x.mid + x.lo with every product
// exact in fp32: an fp32-accurate GEMM on bf16 MFMA (fp32 accumulate) for
// three times the bf16 work.  Small batches split in registers as they load
// W; large ones read planes that k_router_prep writes once per call.  Small batches split the d-sum
// over nsplit workgroups, and a second kernel adds the partial sums in the
// fixed order s = 0..nsplit-1, so the result does not depend on scheduling.
// Batches of 4096 tokens or more take k_router_logits_tiled (LDS-staged
// 256-token x 192-expert tiles), which accumulates in the same order.
//
// Selection.  The choice value is the score, or the score plus the
// selection-only e_score_correction_bias (a float32 addition; "Tencent
// Hy3-Flash Q&A", Q4.3; router flow step 2), which may be negative.  Its bit
// pattern is mapped to an unsigned key that orders like the value (sign bit
// set: all bits flipped, else the sign bit set), and key = (value key << 32) |
// ~expert makes "largest value, then lowest expert index" a plain 64-bit
// maximum.  Sixteen lanes (one DPP row) serve one token: each keeps the keys
// of every 16th expert in registers and offers its best untaken one, the row
// takes the maximum with row_ror DPP moves, k times.  The weights use the chosen experts' scores, summed in slot
// order.

#include "internal.h"

namespace hy3 {
namespace {

constexpr int kLogitTokens = 256;   // tokens per workgroup (4 waves x 64)
constexpr int kLogitExperts = 32;   // experts per workgroup (one 32-wide MFMA block)
constexpr int kUnroll = 4;          // k16-steps whose loads are issued together

union Frag {
    bf16x8_t v;
    i32x4_t q;
};

// planes[p][e][i] = part p of W[e][i].
__global__ __launch_bounds__(256) void k_router_prep(const float* __restrict__ W,
                                                     uint16_t* __restrict__ planes, size_t n) {
    const size_t i = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i < n) {
        const float4 w = *reinterpret_cast<const float4*>(W + i);
        const float wv[4] = {w.x, w.y, w.z, w.w};
        uint16_t hi[4], mid[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t uh = __float_as_uint(wv[j]) & 0xffff0000u;
            const float r1 = wv[j] - __uint_as_float(uh);        // exact: <= 16 significant bits
            const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
            const float r2 = r1 - __uint_as_float(um);            // exact: <= 8 significant bits
            hi[j] = static_cast<uint16_t>(uh >> 16);
            mid[j] = static_cast<uint16_t>(um >> 16);
            lo[j] = static_cast<uint16_t>(__float_as_uint(r2) >> 16);
        }
        *reinterpret_cast<uint2*>(planes + i) =
            make_uint2(hi[0] | (uint32_t(hi[1]) << 16), hi[2] | (uint32_t(hi[3]) << 16));
        *reinterpret_cast<uint2*>(planes + n + i) =
            make_uint2(mid[0] | (uint32_t(mid[1]) << 16), mid[2] | (uint32_t(mid[3]) << 16));
        *reinterpret_cast<uint2*>(planes + 2 * n + i) =
            make_uint2(lo[0] | (uint32_t(lo[1]) << 16), lo[2] | (uint32_t(lo[3]) << 16));
    }
}

__device__ __forceinline__ float sigmoid_bias(float z, const float* bias, int e) {
    if (bias) z += bias[e];
    return 1.0f / (1.0f + expf(-z));
}

// Eight fp32 weights -> their hi, mid and lo bf16 planes, two values per
// 32-bit word (element 2 i in the low half), as k_router_prep writes them.
__device__ __forceinline__ void split_planes(float4 a, float4 b, i32x4_t* out) {
    const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t hi[8], mid[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t uh = __float_as_uint(w[j]) & 0xffff0000u;
        const float r1 = w[j] - __uint_as_float(uh);         // exact: <= 16 significant bits
        const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(um);           // exact: <= 8 significant bits
        hi[j] = uh >> 16;
        mid[j] = um >> 16;
        lo[j] = __float_as_uint(r2) >> 16;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        out[0][q] = static_cast<int>(hi[2 * q] | (hi[2 * q + 1] << 16));
        out[1][q] = static_cast<int>(mid[2 * q] | (mid[2 * q + 1] << 16));
        out[2][q] = static_cast<int>(lo[2 * q] | (lo[2 * q + 1] << 16));
    }
}

// Workgroup (tb, eb, s): tokens 256 tb.., experts 32 eb.., d-chunk s; wave w
// owns tokens 64 w..64 w+63 as two 32-row MFMA blocks.
// MFMA 32x32x16: A lane l = token l%32, k 8*(l/32)..+8; B lane l = expert
// l%32, same k; C lane l = expert l%32, tokens 8*(j/4) + 4*(l/32) + j%4.
// nsplit == 1 writes sigmoid scores; otherwise raw partial logits per chunk.
// The weight is read as fp32 and split into its three bf16 planes in
// registers (split_planes, the same arithmetic as k_router_prep), so small
// batches need no separate plane pass.
__global__ __launch_bounds__(256) void k_router_logits(
    const uint16_t* __restrict__ x, const float* __restrict__ W,
    const float* __restrict__ bias, float* __restrict__ partial, float* __restrict__ scores,
    int T, int d, int E, int kchunk, int nsplit) {
    __shared__ f32x16_t red[3][2][64];                // kwaves: waves 1-3's sums
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // One wave of tokens (T <= 64): the four waves take a quarter of the
    // chunk each instead of idling, and their sums are added in wave order.
    const bool kwaves = T <= 64 && kchunk % 64 == 0;
    const int t0 = blockIdx.x * kLogitTokens + (kwaves ? 0 : wave * 64);
    if (t0 >= T) return;                            // whole wave past the batch
    const int e0 = blockIdx.y * kLogitExperts;
    const int k0 = blockIdx.z * kchunk + (kwaves ? wave * (kchunk / 4) : 0);
    const int kc = kwaves ? kchunk / 4 : kchunk;      // this wave's share of the chunk
    const int l32 = lane & 31;
    const int kh = (lane >> 5) * 8;

    const uint16_t* xa[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int ta = min(t0 + 32 * mb + l32, T - 1);   // rows past T repeat a valid row
        xa[mb] = x + static_cast<size_t>(ta) * d + k0 + kh;
    }
    const int eb = min(e0 + l32, E - 1);
    const float* wb = W + static_cast<size_t>(eb) * d + k0 + kh;

    f32x16_t acc[2] = {{}, {}};
    for (int kb = 0; kb < kc; kb += 16 * kUnroll) {
        i32x4_t av[kUnroll][2], bv[kUnroll][3];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int kk = min(kb + 16 * u, kc - 16);      // kc is a multiple of 16
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) av[u][mb] = *reinterpret_cast<const i32x4_t*>(xa[mb] + kk);
            split_planes(*reinterpret_cast<const float4*>(wb + kk), *reinterpret_cast<const float4*>(wb + kk + 4),
                         bv[u]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (kb + 16 * u < kc) {
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    Frag b;
                    b.q = bv[u][p];
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) {
                        Frag a;
                        a.q = av[u][mb];
                        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc[mb], 0, 0, 0);
                    }
                }
            }
        }
    }

    if (kwaves) {
        if (wave > 0) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) red[wave - 1][mb][lane] = acc[mb];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) acc[mb] += red[w][mb][lane];
    }
    const int e = e0 + l32;
    if (e >= E) return;
    float* out = nsplit == 1 ? scores : partial + static_cast<size_t>(blockIdx.z) * T * E;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = t0 + 32 * mb + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            if (t < T) {
                const float v = acc[mb][j];
                out[static_cast<size_t>(t) * E + e] = nsplit == 1 ? sigmoid_bias(v, bias, e) : v;
            }
        }
    }
}

// Large batches.  Workgroup (tt, eg, s): tokens 256 tt.., experts 192 eg..
// with all three planes, d-chunk s.  K advances in slices of 32 values (64
// bytes per row) through a 3-slot LDS ring of 832 rows (256 token rows, then
// the 192 expert rows of each plane), filled with direct-to-LDS copies two
// slices ahead; waves 0-3 each issue 13 of the 52 one-kilobyte copies of a
// slice.  Eight waves, two per SIMD, so that one wave's MFMAs run while the
// other stalls issuing copies or waits: wave (wm, wn) owns tokens 64 wm.. x
// experts 96 wn.. as 2 x 3 blocks of 32 x 32, and a 16-wide k step reads 2
// token and 9 plane fragments and issues 18 MFMAs.  Every accumulator takes
// each step's planes in the order hi, mid, lo, steps in increasing k, as in
// k_router_logits, so both kernels give the same bits for the same
// d-chunks.  A slice's first half runs on fragments read during the previous
// slice; the barrier between the halves (the next slice landed, every read
// of this slice done) frees this slice's slot for the refill issued during
// the second half.
constexpr int kTiledTokens = 256;
constexpr int kTiledExperts = 192;
constexpr int kTiledRows = kTiledTokens + 3 * kTiledExperts;    // 832 LDS rows per slice
constexpr int kTiledSlotB = kTiledRows * 64;                     // 53,248 bytes
constexpr int kTiledSlots = 3;
constexpr int kTiledWaves = 8;
constexpr int kTiledCopyWaves = 4;
constexpr int kTiledNpw = kTiledRows / 16 / kTiledCopyWaves;     // 13 copies per copying wave and slice
constexpr int kTiledFrags = 2 + 9;                               // fragments per k step and wave
constexpr int kTiledMfmas = 2 * 3 * 3;                           // MFMAs per k step and wave
constexpr int kTiledMinT = 4096;                                 // smaller batches: k_router_logits

__global__ __launch_bounds__(64 * kTiledWaves, 1) void k_router_logits_tiled(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes,
    const float* __restrict__ bias, float* __restrict__ partial, float* __restrict__ scores,
    int T, int d, int E, int kchunk, int nsplit) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kTiledSlots * kTiledSlotB];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    const bool copier = wave < kTiledCopyWaves;
    const int t0 = blockIdx.x * kTiledTokens;
    const int e0 = blockIdx.y * kTiledExperts;
    const int k0 = blockIdx.z * kchunk;
    const int nk = kchunk / 32;
    const size_t plane = static_cast<size_t>(E) * d;

    // copy j of copying wave c fills LDS rows 16 (13 c + j) .. +15; lane ->
    // row + lane / 4, physical chunk lane % 4.  Rows past T or E repeat the
    // last valid one.  (The other waves compute the same sources for c =
    // wave - 4 and never use them.)
    const int cw = wave & (kTiledCopyWaves - 1);
    const uint8_t* src[kTiledNpw];
#pragma unroll
    for (int j = 0; j < kTiledNpw; ++j) {
        const int row = 16 * (cw * kTiledNpw + j) + (lane >> 2);
        const int lc = pchunk(row, lane & 3);
        const uint16_t* base;
        if (row < kTiledTokens) {
            base = x + static_cast<size_t>(min(t0 + row, T - 1)) * d;
        } else {
            const int q = row - kTiledTokens;
            const int p = q / kTiledExperts;
            base = planes + p * plane + static_cast<size_t>(min(e0 + q - p * kTiledExperts, E - 1)) * d;
        }
        src[j] = reinterpret_cast<const uint8_t*>(base + k0) + lc * 16;
    }
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    const uint32_t my_copies = lds0 + static_cast<uint32_t>(cw * kTiledNpw) * 1024u;

    // fragment rows: token block mb at 64 wm + 32 mb; plane p, expert block
    // eb at 256 + 192 p + 96 wn + 32 eb; k step h of a slice: chunk 2 h + khalf
    const int l32 = lane & 31;
    const int khalf = lane >> 5;
    int off[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) off[h] = l32 * 64 + pchunk(l32, 2 * h + khalf) * 16;

    f32x16_t acc[2][3];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int eb = 0; eb < 3; ++eb) acc[mb][eb] = f32x16_t{};
    // fragment r of a set: r < 2 token block r; else plane (r - 2) / 3, expert block (r - 2) % 3
    i32x4_t fr[2][kTiledFrags];
    auto read_frag = [&](int set, const uint8_t* base, int h, int r) {
        const int row = r < 2 ? 64 * wm + 32 * r
                              : kTiledTokens + kTiledExperts * ((r - 2) / 3) + 96 * wn + 32 * ((r - 2) % 3);
        fr[set][r] = *reinterpret_cast<const i32x4_t*>(base + row * 64 + off[h]);
    };
    // MFMA i of a k step: plane i / 6, expert block (i / 2) % 3, token block i % 2
    auto mfma = [&](int set, int i) {
        const int p = i / 6, eb = (i >> 1) % 3, mb = i & 1;
        acc[mb][eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, fr[set][mb]), __builtin_bit_cast(bf16x8_t, fr[set][2 + 3 * p + eb]),
            acc[mb][eb], 0, 0, 0);
    };

    if (copier) {
#pragma unroll
        for (int s = 0; s < kTiledSlots; ++s) {
            const int kt = min(s, nk - 1);
#pragma unroll
            for (int j = 0; j < kTiledNpw; ++j) copy_to_lds(src[j] + kt * 64, my_copies + s * kTiledSlotB + j * 1024);
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kTiledSlots - 1) * kTiledNpw));
    lds_barrier();
#pragma unroll
    for (int r = 0; r < kTiledFrags; ++r) read_frag(0, lds, 0, r);

    for (int kt = 0; kt < nk; ++kt) {
        const int sc = kt % kTiledSlots;
        const int sn = (kt + 1) % kTiledSlots;
        const uint8_t* cur = lds + sc * kTiledSlotB;
        const uint8_t* nxt = lds + sn * kTiledSlotB;
        // first half: step 0 of slice kt; read step 1 of slice kt
#pragma unroll
        for (int i = 0; i < kTiledMfmas; ++i) {
            mfma(0, i);
#pragma unroll
            for (int r = 0; r < kTiledFrags; ++r)
                if (i == r * kTiledMfmas / kTiledFrags) read_frag(1, cur, 1, r);
            __builtin_amdgcn_sched_barrier(0);
        }
        // slice kt + 1 landed (at most the copies of kt + 2 in flight), and
        // every wave's reads of slice kt are done: its slot is free
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kTiledNpw));
        lds_barrier();
        const int kin = min(kt + kTiledSlots, nk - 1);
        const uint32_t islot = my_copies + sc * kTiledSlotB;
        // second half: step 1 of slice kt; read step 0 of slice kt + 1;
        // the copying waves refill this slot with slice kt + 3
#pragma unroll
        for (int i = 0; i < kTiledMfmas; ++i) {
            mfma(1, i);
#pragma unroll
            for (int r = 0; r < kTiledFrags; ++r)
                if (i == r * kTiledMfmas / kTiledFrags) read_frag(0, nxt, 0, r);
#pragma unroll
            for (int r = 0; r < kTiledNpw; ++r)
                if (i == r * kTiledMfmas / kTiledNpw && copier) copy_to_lds(src[r] + kin * 64, islot + r * 1024);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));              // no copy may land after the kernel ends

    float* out = nsplit == 1 ? scores : partial + static_cast<size_t>(blockIdx.z) * T * E;
#pragma unroll
    for (int eb = 0; eb < 3; ++eb) {
        const int e = e0 + 96 * wn + 32 * eb + l32;
        if (e >= E) continue;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int t = t0 + 64 * wm + 32 * mb + 8 * (j >> 2) + 4 * khalf + (j & 3);
                if (t < T) {
                    const float v = acc[mb][eb][j];
                    out[static_cast<size_t>(t) * E + e] = nsplit == 1 ? sigmoid_bias(v, bias, e) : v;
                }
            }
        }
    }
}

// scores = sigmoid(sum over s = 0..nsplit-1 of partial[s] + bias), one element
// per thread, the chunks added in that fixed order.
constexpr int kMaxSplit = 32;
__global__ __launch_bounds__(256) void k_router_reduce(const float* __restrict__ partial,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ scores, int T, int E,
                                                       int nsplit) {
    const size_t n = static_cast<size_t>(T) * E;
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    float v[kMaxSplit];
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) v[s] = s < nsplit ? partial[s * n + i] : 0.f;
    float z = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) z += v[s];       // +0.f past nsplit changes nothing
    scores[i] = sigmoid_bias(z, bias, static_cast<int>(i % E));
}

// 64-bit maximum over the 16 lanes of a DPP row (row_ror by 8, 4, 2, 1).
__device__ __forceinline__ unsigned long long row16_max(unsigned long long v) {
#define HY3_ROR_STEP(CTRL)                                                                        \
    {                                                                                             \
        const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(v & 0xffffffffull), CTRL,  \
                                                   0xf, 0xf, false);                              \
        const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(v >> 32), CTRL, 0xf, 0xf,  \
                                                   false);                                        \
        const unsigned long long o =                                                              \
            (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |                  \
            static_cast<uint32_t>(lo);                                                            \
        v = o > v ? o : v;                                                                        \
    }
    HY3_ROR_STEP(0x128)   // row_ror:8
    HY3_ROR_STEP(0x124)   // row_ror:4
    HY3_ROR_STEP(0x122)   // row_ror:2
    HY3_ROR_STEP(0x121)   // row_ror:1
#undef HY3_ROR_STEP
    return v;
}

constexpr int kSelThreads = 1024;   // 16 waves x 4 tokens = 64 tokens (one routing block)

__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The k rounds of one token's top-k: 16 lanes (one DPP row) per token, lane
// j holding the order keys of experts j, j + 16, ... (NQ of them), clamped to
// at least 1 so that 0 can mark "taken or absent".  A round takes each lane's
// largest key (the lowest index among equals), the row's maximum of (key <<
// 32 | ~expert) by DPP, and clears the winner's key.  Returns, in lane j < k,
// the expert of slot j.
template <int NQ>
__device__ __forceinline__ int select_rounds(uint32_t (&key)[NQ], int j, int k) {
    int my_e = 0;
    for (int r = 0; r < k; ++r) {
        uint32_t bk = 0u;
        int bq = 0;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const bool better = key[q] > bk;
            bk = better ? key[q] : bk;
            bq = better ? q : bq;
        }
        unsigned long long best =
            bk ? (static_cast<unsigned long long>(bk) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(j + 16 * bq))
               : 0ull;
        best = row16_max(best);
        const int e_win = static_cast<int>(~static_cast<uint32_t>(best & 0xffffffffull));
        const bool mine = (e_win & 15) == j;
        const int qw = e_win >> 4;
#pragma unroll
        for (int q = 0; q < NQ; ++q) key[q] = (mine && q == qw) ? 0u : key[q];
        if (r == j) my_e = e_win;
    }
    return my_e;
}

// The weights of a token's k slots (lane j < k holds slot j and its score):
// scale * s_j / (sum of the k scores, in slot order).
__device__ __forceinline__ float slot_weight(float my_s, int lane, int k, float scale) {
    float sum = 0.f;
    for (int r = 0; r < k; ++r) sum += __shfl(my_s, (lane & ~15) | r, 64);   // slot order
    return scale * (my_s / sum);
}

// One 64-token routing block per workgroup, 16 lanes (one DPP row) per
// token.  Lane j keeps the order keys of experts j, j + 16, ... (NQ of them)
// in registers, clamped to at least 1 so that 0 can mark "taken or absent".
// A round takes each lane's largest key (the lowest index among equals), the
// row's maximum of (key << 32 | ~expert) by DPP, and clears the winner's key.
// Writes idx/w and, when blk_counts is given, the block's per-expert pair
// count.
template <int NQ>
__global__ __launch_bounds__(kSelThreads) void k_router_select(
    const float* __restrict__ scores, const float* __restrict__ score_bias, int T, int E, int k,
    float scale, int32_t* __restrict__ idx, float* __restrict__ wout,
    int32_t* __restrict__ blk_counts, int nb) {
    __shared__ unsigned long long mask[1024];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kSelThreads) mask[e] = 0ull;
    const int lane = tid & 63;
    const int j = lane & 15;                              // lane within the token's row
    const int ts = (tid >> 6) * 4 + (lane >> 4);          // token slot within the block
    const int t = blockIdx.x * kRouteBlock + ts;
    const bool active = t < T;
    const float* srow = scores + static_cast<size_t>(active ? t : 0) * E;

    uint32_t key[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = j + 16 * q;
        key[q] = 0u;
        if (active && e < E) {
            const float v = score_bias ? srow[e] + score_bias[e] : srow[e];
            key[q] = max(order_key(v), 1u);
        }
    }
    const int my_e = select_rounds<NQ>(key, j, k);
    __syncthreads();                                      // mask cleared
    // lane j < k holds slot j; the weights use the scores themselves
    const float my_s = (active && j < k) ? srow[my_e] : 0.f;
    const float my_w = slot_weight(my_s, lane, k, scale);
    if (active && j < k) {
        const size_t pair = static_cast<size_t>(t) * k + j;
        idx[pair] = my_e;
        wout[pair] = my_w;
        atomicOr(&mask[my_e], 1ull << ts);
    }
    if (blk_counts) {
        __syncthreads();
        for (int e = tid; e < E; e += kSelThreads)
            blk_counts[static_cast<size_t>(e) * nb + blockIdx.x] = __popcll(mask[e]);
    }
}

// A batch of one routing block (T <= 64), whose dispatch (k_dispatch_one)
// rebuilds its token masks from idx and needs no per-block counts: one wave
// per 4 tokens, each wave a workgroup of its own, so the tokens spread over
// as many CUs.  The wave also does k_router_reduce's work for its tokens: the
// d-chunks' partial logits summed in the order s = 0..nsplit-1, then
// sigmoid(z + bias), the same arithmetic and so the same bits (nsplit == 1:
// the logits kernel wrote the scores).  The scores stay in LDS for the
// weights; the selection is k_router_select's.
template <int NQ>
__global__ __launch_bounds__(64) void k_router_select_wave(
    const float* __restrict__ partial, const float* __restrict__ scores, int nsplit,
    const float* __restrict__ bias, const float* __restrict__ score_bias, int T, int E, int k,
    float scale, int32_t* __restrict__ idx, float* __restrict__ wout) {
    __shared__ float s_sc[4][16 * NQ];
    const int lane = threadIdx.x;
    const int j = lane & 15;                              // lane within the token's row
    const int ts = lane >> 4;                             // token of the wave
    const int t = blockIdx.x * 4 + ts;
    const bool active = t < T;
    const size_t n = static_cast<size_t>(T) * E;
    const size_t row = static_cast<size_t>(active ? t : 0) * E;
    // the lane's scores: U d-chunks' partials of all its experts are loaded
    // together, then added chunk by chunk (zeros past nsplit are added last,
    // which changes nothing)
    constexpr int U = NQ <= 12 ? 8 : NQ <= 16 ? 4 : NQ <= 32 ? 2 : 1;
    // the biases first, all in flight with the partials
    float bq[NQ], sbq[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = j + 16 * q;
        bq[q] = (bias && e < E) ? bias[e] : 0.f;
        sbq[q] = (score_bias && e < E) ? score_bias[e] : 0.f;
    }
    float sc[NQ];
    if (nsplit > 1) {
        float z[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) z[q] = 0.f;
        for (int sp0 = 0; sp0 < nsplit; sp0 += U) {
            float pv[U][NQ];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int e = j + 16 * q;
                    pv[u][q] = (active && e < E && sp0 + u < nsplit) ? partial[(sp0 + u) * n + row + e] : 0.f;
                }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < NQ; ++q) z[q] += pv[u][q];
        }
        // sigmoid_bias, with the bias loaded above
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float zb = bias ? z[q] + bq[q] : z[q];
            sc[q] = 1.0f / (1.0f + expf(-zb));
        }
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = j + 16 * q;
            sc[q] = (active && e < E) ? scores[row + e] : 0.f;
        }
    }
    uint32_t key[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = j + 16 * q;
        key[q] = 0u;
        if (active && e < E) {
            const float v = score_bias ? sc[q] + sbq[q] : sc[q];
            key[q] = max(order_key(v), 1u);
        }
        s_sc[ts][e] = sc[q];
    }
    const int my_e = select_rounds<NQ>(key, j, k);
    // a wave's LDS accesses complete in order: the stores above precede this read
    const float my_s = (active && j < k) ? s_sc[ts][my_e] : 0.f;
    const float my_w = slot_weight(my_s, lane, k, scale);
    if (active && j < k) {
        const size_t pair = static_cast<size_t>(t) * k + j;
        idx[pair] = my_e;
        wout[pair] = my_w;
    }
}

// The same for E <= 192 (NQ <= 12) with four waves per 4 tokens: each wave
// loads a quarter of the d-chunks' partials (all its loads in flight at
// once) into LDS, and wave 0 adds them up in the order s = 0..nsplit-1, so
// the scores are bit-identical to the one-wave kernel's.  (One wave alone
// takes two rounds of loads: 16 chunks x 12 experts exceed what a wave keeps
// in flight.)
template <int NQ>
__global__ __launch_bounds__(256) void k_router_select_wave4(
    const float* __restrict__ partial, const float* __restrict__ scores, int nsplit,
    const float* __restrict__ bias, const float* __restrict__ score_bias, int T, int E, int k,
    float scale, int32_t* __restrict__ idx, float* __restrict__ wout) {
    static_assert(NQ <= 12, "LDS holds kMaxSplit x 12 partials per lane");
    __shared__ float s_p[kMaxSplit][NQ][64];
    __shared__ float s_sc[4][16 * NQ];
    const int wv = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int j = lane & 15;                              // lane within the token's row
    const int ts = lane >> 4;                             // token of the workgroup
    const int t = blockIdx.x * 4 + ts;
    const bool active = t < T;
    const size_t n = static_cast<size_t>(T) * E;
    const size_t row = static_cast<size_t>(active ? t : 0) * E;
    // the biases first, in flight with the partials
    float bq[NQ], sbq[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = j + 16 * q;
        bq[q] = (bias && e < E) ? bias[e] : 0.f;
        sbq[q] = (score_bias && e < E) ? score_bias[e] : 0.f;
    }
    float sc[NQ];
    if (nsplit > 1) {
        constexpr int CMAX = kMaxSplit / 4;
        const int c = (nsplit + 3) / 4;                   // chunks per wave
        const int s0 = wv * c;
        float pv[CMAX][NQ];
#pragma unroll
        for (int u = 0; u < CMAX; ++u)
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int e = j + 16 * q;
                const int sp = s0 + u;
                pv[u][q] = (u < c && sp < nsplit && active && e < E) ? partial[sp * n + row + e] : 0.f;
            }
#pragma unroll
        for (int u = 0; u < CMAX; ++u)
            if (u < c && s0 + u < nsplit)
#pragma unroll
                for (int q = 0; q < NQ; ++q) s_p[s0 + u][q][lane] = pv[u][q];
        __syncthreads();
        if (wv != 0) return;
        float z[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) z[q] = 0.f;
        for (int sp = 0; sp < nsplit; ++sp)
#pragma unroll
            for (int q = 0; q < NQ; ++q) z[q] += s_p[sp][q][lane];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float zb = bias ? z[q] + bq[q] : z[q];
            sc[q] = 1.0f / (1.0f + expf(-zb));
        }
    } else {
        if (wv != 0) return;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = j + 16 * q;
            sc[q] = (active && e < E) ? scores[row + e] : 0.f;
        }
    }
    uint32_t key[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = j + 16 * q;
        key[q] = 0u;
        if (active && e < E) {
            const float v = score_bias ? sc[q] + sbq[q] : sc[q];
            key[q] = max(order_key(v), 1u);
        }
        s_sc[ts][e] = sc[q];
    }
    const int my_e = select_rounds<NQ>(key, j, k);
    // a wave's LDS accesses complete in order: the stores above precede this read
    const float my_s = (active && j < k) ? s_sc[ts][my_e] : 0.f;
    const float my_w = slot_weight(my_s, lane, k, scale);
    if (active && j < k) {
        const size_t pair = static_cast<size_t>(t) * k + j;
        idx[pair] = my_e;
        wout[pair] = my_w;
    }
}

}  // namespace

int router_nsplit(int T, int d, int E) {
    const bool tiled = T >= kTiledMinT;
    const int wgs = tiled ? ((T + kTiledTokens - 1) / kTiledTokens) * ((E + kTiledExperts - 1) / kTiledExperts)
                          : ((T + kLogitTokens - 1) / kLogitTokens) * ((E + kLogitExperts - 1) / kLogitExperts);
    const int target = tiled ? 256 : 512;                  // tiled: one workgroup per CU
    const int min_chunk = tiled ? 512 : 256;
    int ns = 1;
    // chunks stay multiples of 32 and at least min_chunk wide
    while (wgs * ns < target && 2 * ns <= kMaxSplit && (d % (2 * ns * 32)) == 0 && d / (2 * ns) >= min_chunk)
        ns *= 2;
    return ns;
}

size_t router_plane_elems(int d, int E) { return static_cast<size_t>(3) * E * d; }

hipError_t launch_router(const uint16_t* x, const float* W_gate, const float* bias,
                         const float* score_bias, int T, int d, int E, int k, float scale,
                         const RouterWork& rw, int32_t* idx, float* w, int32_t* blk_counts, int nb,
                         hipStream_t s) {
    if (T >= kTiledMinT) {
        const size_t n = static_cast<size_t>(E) * d;
        hipLaunchKernelGGL(k_router_prep, dim3(static_cast<unsigned>((n / 4 + 255) / 256)), dim3(256), 0,
                           s, W_gate, rw.planes, n);
        dim3 g1((T + kTiledTokens - 1) / kTiledTokens, (E + kTiledExperts - 1) / kTiledExperts, rw.nsplit);
        hipLaunchKernelGGL(k_router_logits_tiled, g1, dim3(64 * kTiledWaves), 0, s, x, rw.planes, bias, rw.partial,
                           rw.scores, T, d, E, d / rw.nsplit, rw.nsplit);
    } else {
        dim3 g1((T + kLogitTokens - 1) / kLogitTokens, (E + kLogitExperts - 1) / kLogitExperts,
                rw.nsplit);
        hipLaunchKernelGGL(k_router_logits, g1, dim3(256), 0, s, x, W_gate, bias, rw.partial,
                           rw.scores, T, d, E, d / rw.nsplit, rw.nsplit);
    }
    // keys per lane: E / 16 rounded up to a power of two or 12 (E <= 1024)
    const int nq = (E + 15) / 16;
    // one routing block: the wave-per-4-tokens select, which also reduces the
    // d-chunks; more blocks: the reduce, then one workgroup per block, which
    // also counts each block's pairs per expert for the dispatch
    const bool one_block = nb == 1;
    if (!one_block && rw.nsplit > 1) {
        const size_t te = static_cast<size_t>(T) * E;
        hipLaunchKernelGGL(k_router_reduce, dim3(static_cast<unsigned>((te + 255) / 256)), dim3(256),
                           0, s, rw.partial, bias, rw.scores, T, E, rw.nsplit);
    }
#define HY3_SELECT(NQ)                                                                                      \
    do {                                                                                                    \
        if (one_block && (NQ) <= 12)                                                                        \
            hipLaunchKernelGGL(k_router_select_wave4<((NQ) <= 12 ? (NQ) : 12)>,                             \
                               dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, s, rw.partial,       \
                               rw.scores, rw.nsplit, bias, score_bias, T, E, k, scale, idx, w);             \
        else if (one_block)                                                                                 \
            hipLaunchKernelGGL(k_router_select_wave<NQ>, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(64), 0, \
                               s, rw.partial, rw.scores, rw.nsplit, bias, score_bias, T, E, k, scale, idx, w); \
        else                                                                                                \
            hipLaunchKernelGGL(k_router_select<NQ>, dim3(nb), dim3(kSelThreads), 0, s, rw.scores, score_bias, \
                               T, E, k, scale, idx, w, blk_counts, nb);                                     \
    } while (0)
    if (nq <= 1) HY3_SELECT(1);
    else if (nq <= 2) HY3_SELECT(2);
    else if (nq <= 4) HY3_SELECT(4);
    else if (nq <= 8) HY3_SELECT(8);
    else if (nq <= 12) HY3_SELECT(12);                     // E = 192: no empty key slots
    else if (nq <= 16) HY3_SELECT(16);
    else if (nq <= 32) HY3_SELECT(32);
    else HY3_SELECT(64);
#undef HY3_SELECT
    return hipGetLastError();
}

namespace {

constexpr int kNormThreads = 256;

// route_norm: one workgroup per row.  The pages fix neither the precision nor
// eps; this is the usual bf16-model reading: the sum of squares (exact
// products of bf16 values) is accumulated in fp64, r = float(1 / sqrt(sum / d
// + eps)) with the division and square root in fp64, the normalised row is
// cast to bf16 and the bf16 weight is applied with one more bf16 rounding
// (the product of two bf16 values is exact in fp32).
__global__ __launch_bounds__(kNormThreads) void k_rms_norm_bf16(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wgt,
                                                               int d, float eps,
                                                               uint16_t* __restrict__ xn) {
    __shared__ double red[kNormThreads / 64];
    const size_t row = blockIdx.x;
    const uint16_t* xr = x + row * d;
    double ss = 0.0;
    for (int c = threadIdx.x * 8; c < d; c += kNormThreads * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double a = __uint_as_float(p[i] << 16), b = __uint_as_float(p[i] & 0xffff0000u);
            ss += a * a + b * b;                          // exact products (bf16 squares fit fp64)
        }
    }
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int i = 0; i < kNormThreads / 64; ++i) tot += red[i];
    const float r = static_cast<float>(1.0 / sqrt(tot / d + static_cast<double>(eps)));
    for (int c = threadIdx.x * 8; c < d; c += kNormThreads * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
        const uint4 g = *reinterpret_cast<const uint4*>(wgt + c);
        const uint32_t p[4] = {v.x, v.y, v.z, v.w}, q[4] = {g.x, g.y, g.z, g.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a0 = bf16_to_f32(f32_to_bf16(__uint_as_float(p[i] << 16) * r));
            const float a1 = bf16_to_f32(f32_to_bf16(__uint_as_float(p[i] & 0xffff0000u) * r));
            const uint32_t y0 = f32_to_bf16(a0 * __uint_as_float(q[i] << 16));
            const uint32_t y1 = f32_to_bf16(a1 * __uint_as_float(q[i] & 0xffff0000u));
            o[i] = y0 | (y1 << 16);
        }
        *reinterpret_cast<uint4*>(xn + row * d + c) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace

hipError_t launch_rms_norm(const uint16_t* x, const uint16_t* w, int T, int d, float eps,
                           uint16_t* xn, hipStream_t s) {
    hipLaunchKernelGGL(k_rms_norm_bf16, dim3(T), dim3(kNormThreads), 0, s, x, w, d, eps, xn);
    return hipGetLastError();
}

}  // namespace hy3
