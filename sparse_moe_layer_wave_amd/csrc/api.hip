// C ABI of libhy3moe (declared in include/hy3moe.h): argument checks,
// workspace carving and the launch sequence of the layer.  Every check runs on
// the host before anything is enqueued; the library never allocates, frees or
// synchronises.

#include <atomic>

#include "../../include/hy3moe.h"
#include "internal.h"

namespace hy3 {

hipError_t device_cu_count(int* cus) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];   // 0: not yet queried
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < kMaxDevices) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) {
            *cus = v;
            return hipSuccess;
        }
    }
    err = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess && dev >= 0 && dev < kMaxDevices && *cus > 0)
        cache[dev].store(*cus, std::memory_order_relaxed);
    return err;
}

}  // namespace hy3

namespace {

using hy3::Layout;

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Regions used by the routing and permute entries come first, so their needs
// are prefixes of the forward layout and do not depend on d_ff.  shared: the
// block's shared expert adds T expert rows (and one expert to the offsets);
// norm: route_norm's bf16 copy of x.
Layout make_layout(int T, int d, int E, int k, int F, int dtype, bool shared = false,
                   bool norm = false) {
    Layout L{};
    const size_t Tk = static_cast<size_t>(T) * k;
    const size_t R = Tk + (shared ? static_cast<size_t>(T) : 0);   // expert rows
    L.rows = static_cast<int>(R);
    L.nb = (T + hy3::kRouteBlock - 1) / hy3::kRouteBlock;
    L.max_mtiles = static_cast<int>(R / hy3::prefill_bm()) + E + (shared ? 1 : 0);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    L.nsplit = hy3::router_nsplit(T, d, E);
    L.planes = take(hy3::router_plane_elems(d, E) * sizeof(uint16_t));
    L.partial = take(L.nsplit > 1 ? static_cast<size_t>(L.nsplit) * T * E * sizeof(float) : 0);
    L.scores = take(static_cast<size_t>(T) * E * sizeof(float));
    L.xn = take(norm ? static_cast<size_t>(T) * d * sizeof(uint16_t) : 0);
    L.blk_counts = take(static_cast<size_t>(E) * L.nb * sizeof(int32_t));
    L.blk_base = take(static_cast<size_t>(E) * L.nb * sizeof(int32_t));
    L.counts = take(static_cast<size_t>(E) * sizeof(int32_t));
    L.offsets = take(static_cast<size_t>(E + 2) * sizeof(int32_t));
    L.tile_off = take(static_cast<size_t>(E + 2) * sizeof(int32_t));
    L.idx = take(Tk * sizeof(int32_t));
    L.w = take(Tk * sizeof(float));
    L.row_of = take(Tk * sizeof(int32_t));
    L.tok_of = take(R * sizeof(int32_t));
    if (dtype == HY3MOE_WEIGHTS_FP8_E4M3) {
        L.h = take(Tk * F * sizeof(uint16_t));         // bf16 SwiGLU activations
        L.hq = take(Tk * F);                           // their e4m3 codes
        L.hs = take(Tk * sizeof(float));               // per-row scale
        // per-row max |h|: [Tk] bit patterns (weight-streaming gate_up, atomics)
        // or [F / 128][Tk] partial maxima (grouped gate_up)
        L.amax = take(Tk * ((F + 127) / 128) * sizeof(float));
        L.xq = take(static_cast<size_t>(T) * d);
        L.xs = take(static_cast<size_t>(T) * sizeof(float));
    } else {
        L.h = take(R * F * sizeof(uint16_t));
        L.hq = L.hs = L.xq = L.xs = L.amax = 0;
    }
    L.y = take(R * d * sizeof(uint16_t));
    L.sched = take(hy3::kSchedInts * sizeof(int));    // the grouped GEMMs' work counters
    L.total = off;
    return L;
}

size_t route_bytes(const Layout& L) { return L.blk_counts; }

hy3::RouterWork router_work(char* ws, const Layout& L) {
    return hy3::RouterWork{reinterpret_cast<uint16_t*>(ws + L.planes),
                           reinterpret_cast<float*>(ws + L.partial),
                           reinterpret_cast<float*>(ws + L.scores), L.nsplit};
}
size_t permute_bytes(const Layout& L) { return L.idx; }

int check_shape(int T, int d, int E, int k, int F) {
    if (T < 0 || d <= 0 || E <= 0 || F <= 0 || k < 1 || k > E) return HY3MOE_ERR_SHAPE;
    if (k > 16 || E > 1024 || (d % 64) != 0 || (F % 64) != 0 || T > (1 << 24))
        return HY3MOE_ERR_UNSUPPORTED;
    return HY3MOE_OK;
}

// Records stage_events[i] on the stream when the caller supplied it.
hipError_t mark(void* const* ev, int i, hipStream_t s) {
    if (!ev || !ev[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(ev[i]), s);
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return HY3MOE_OK;
    g_last_hip_error = static_cast<int>(e);
    return HY3MOE_ERR_HIP;
}

// ---- the static scratch of hy3moe_forward_noalloc ----
// Device memory of the code object, one copy per GPU, held until the process
// ends.  Host code never uses the array's name as an address (on the host it
// is a stand-in, not device memory): each device's address is fetched once,
// with hipGetSymbolAddress while that device is current, and kept here.
constexpr size_t kScratchBytes = size_t(HY3MOE_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];   // nullptr: not fetched yet

// The scratch array's address on the current device (first call per device:
// hipGetSymbolAddress; concurrent first calls fetch and store the same value).
hipError_t scratch_address(void** addr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *addr = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

int hy3moe_workspace_size(int T, int d, int E, int k, int d_ff, int weight_dtype, size_t* bytes) {
    if (!bytes) return HY3MOE_ERR_NULL;
    const int st = check_shape(T, d, E, k, d_ff);
    if (st != HY3MOE_OK) return st;
    if (weight_dtype != HY3MOE_WEIGHTS_BF16 && weight_dtype != HY3MOE_WEIGHTS_FP8_E4M3)
        return HY3MOE_ERR_UNSUPPORTED;
    *bytes = make_layout(T, d, E, k, d_ff, weight_dtype).total;
    return HY3MOE_OK;
}

int hy3moe_route(const uint16_t* x, const float* W_gate, const float* logit_bias, int T, int d,
                 int E, int k, float scale, int32_t* topk_idx, float* topk_w, void* workspace,
                 size_t workspace_bytes, void* stream) {
    int st = check_shape(T, d, E, k, 64);
    if (st != HY3MOE_OK) return st;
    if (T == 0) return HY3MOE_OK;
    if (!x || !W_gate || !topk_idx || !topk_w || !workspace) return HY3MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(W_gate) || !aligned16(topk_idx) || !aligned16(topk_w) ||
        !aligned16(workspace) || (logit_bias && !aligned16(logit_bias)))
        return HY3MOE_ERR_ALIGN;
    const Layout L = make_layout(T, d, E, k, 64, HY3MOE_WEIGHTS_BF16);
    if (workspace_bytes < route_bytes(L)) return HY3MOE_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    return hip_status(hy3::launch_router(x, W_gate, logit_bias, nullptr, T, d, E, k, scale,
                                         router_work(ws, L), topk_idx, topk_w, nullptr, L.nb,
                                         static_cast<hipStream_t>(stream)));
}

int hy3moe_route_ex(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                    const float* W_gate, const float* logit_bias, const float* score_bias, int T,
                    int d, int E, int k, float scale, int32_t* topk_idx, float* topk_w,
                    void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_shape(T, d, E, k, 64);
    if (st != HY3MOE_OK) return st;
    if (!(norm_eps >= 0.f)) return HY3MOE_ERR_SHAPE;
    if (T == 0) return HY3MOE_OK;
    if (!x || !W_gate || !topk_idx || !topk_w || !workspace) return HY3MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(W_gate) || !aligned16(topk_idx) || !aligned16(topk_w) ||
        !aligned16(workspace) || (logit_bias && !aligned16(logit_bias)) ||
        (score_bias && !aligned16(score_bias)) || (norm_weight && !aligned16(norm_weight)))
        return HY3MOE_ERR_ALIGN;
    const Layout L = make_layout(T, d, E, k, 64, HY3MOE_WEIGHTS_BF16, false, norm_weight != nullptr);
    if (workspace_bytes < route_bytes(L)) return HY3MOE_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xr = x;
    if (norm_weight) {
        uint16_t* xn = reinterpret_cast<uint16_t*>(ws + L.xn);
        const hipError_t e = hy3::launch_rms_norm(x, norm_weight, T, d, norm_eps, xn, s);
        if (e != hipSuccess) return hip_status(e);
        xr = xn;
    }
    return hip_status(hy3::launch_router(xr, W_gate, logit_bias, score_bias, T, d, E, k, scale,
                                         router_work(ws, L), topk_idx, topk_w, nullptr, L.nb, s));
}

int hy3moe_permute(const int32_t* topk_idx, int T, int E, int k, int32_t* counts,
                   int32_t* offsets, int32_t* row_of, int32_t* token_of, void* workspace,
                   size_t workspace_bytes, void* stream) {
    int st = check_shape(T, 64, E, k, 64);
    if (st != HY3MOE_OK) return st;
    if (T == 0) return HY3MOE_OK;
    if (!topk_idx || !counts || !offsets || !row_of || !token_of || !workspace)
        return HY3MOE_ERR_NULL;
    if (!aligned16(topk_idx) || !aligned16(counts) || !aligned16(offsets) || !aligned16(row_of) ||
        !aligned16(token_of) || !aligned16(workspace))
        return HY3MOE_ERR_ALIGN;
    const Layout L = make_layout(T, 64, E, k, 64, HY3MOE_WEIGHTS_BF16);
    if (workspace_bytes < permute_bytes(L)) return HY3MOE_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t* blk_counts = reinterpret_cast<int32_t*>(ws + L.blk_counts);
    hipError_t e = hy3::launch_block_counts(topk_idx, T, E, k, L.nb, blk_counts, s);
    if (e != hipSuccess) return hip_status(e);
    e = hy3::launch_dispatch(topk_idx, T, E, k, L.nb, blk_counts,
                             reinterpret_cast<int32_t*>(ws + L.blk_base), counts, offsets,
                             reinterpret_cast<int32_t*>(ws + L.tile_off), hy3::prefill_bm(), row_of,
                             token_of, 0, s, true);
    return hip_status(e);
}

}  // extern "C"

namespace {

// The bf16 layer, and the full block when any of its extras is given:
// norm_w (route_norm), score_bias (selection-only bias), Ws_gu/Ws_dn (the
// shared expert, both or neither).  With out_bf16 instead of out, the
// output is bf16 with the residual (if any) added in the combine.
// With use_scratch, the workspace is the library's static scratch array
// (hy3moe_forward_noalloc) and the workspace arguments are ignored.
static int forward_bf16(const uint16_t* x, const uint16_t* norm_w, float norm_eps,
                        const float* W_gate, const float* logit_bias, const float* score_bias,
                        const uint16_t* W_gate_up, const uint16_t* W_down, const uint16_t* Ws_gu,
                        const uint16_t* Ws_dn, float* out, int T, int d, int E, int k, int d_ff,
                        float scale, void* stream, int32_t* topk_idx, float* topk_w,
                        void* workspace, size_t workspace_bytes, void* const* ev,
                        const uint16_t* resid = nullptr, uint16_t* out_bf16 = nullptr,
                        bool use_scratch = false) {
    const bool shared = Ws_gu != nullptr;
    int st = check_shape(T, d, E, k, d_ff);
    if (st != HY3MOE_OK) return st;
    if (shared && E > 1023) return HY3MOE_ERR_UNSUPPORTED;
    if (!(norm_eps >= 0.f)) return HY3MOE_ERR_SHAPE;
    if (T == 0) return HY3MOE_OK;
    if (!x || !W_gate || !W_gate_up || !W_down || !(out || out_bf16) || (!workspace && !use_scratch))
        return HY3MOE_ERR_NULL;
    if ((Ws_gu == nullptr) != (Ws_dn == nullptr)) return HY3MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_gate_up) || !aligned16(W_down) ||
        !aligned16(out ? static_cast<const void*>(out) : out_bf16) ||
        (!use_scratch && !aligned16(workspace)) ||
        (resid && !aligned16(resid)) || (logit_bias && !aligned16(logit_bias)) ||
        (score_bias && !aligned16(score_bias)) || (norm_w && !aligned16(norm_w)) ||
        (Ws_gu && !aligned16(Ws_gu)) || (Ws_dn && !aligned16(Ws_dn)) ||
        (topk_idx && !aligned16(topk_idx)) || (topk_w && !aligned16(topk_w)))
        return HY3MOE_ERR_ALIGN;
    const Layout L = make_layout(T, d, E, k, d_ff, HY3MOE_WEIGHTS_BF16, shared, norm_w != nullptr);
    if (use_scratch) {
        if (L.total > kScratchBytes) return HY3MOE_ERR_SCRATCH;
        const hipError_t e = scratch_address(&workspace);
        if (e != hipSuccess) return hip_status(e);
    } else if (workspace_bytes < L.total) {
        return HY3MOE_ERR_WORKSPACE;
    }
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(ws + L.idx);
    float* w = topk_w ? topk_w : reinterpret_cast<float*>(ws + L.w);
    int32_t* blk_counts = reinterpret_cast<int32_t*>(ws + L.blk_counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* tile_off = reinterpret_cast<int32_t*>(ws + L.tile_off);
    int32_t* row_of = reinterpret_cast<int32_t*>(ws + L.row_of);
    int32_t* tok_of = reinterpret_cast<int32_t*>(ws + L.tok_of);
    uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
    uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.y);
    const int Eg = E + (shared ? 1 : 0);           // experts the GEMMs see

    hipError_t e = mark(ev, 0, s);
    const uint16_t* xr = x;                        // the router's input
    if (e == hipSuccess && norm_w) {
        uint16_t* xn = reinterpret_cast<uint16_t*>(ws + L.xn);
        e = hy3::launch_rms_norm(x, norm_w, T, d, norm_eps, xn, s);
        xr = xn;
    }
    if (e == hipSuccess)
        e = hy3::launch_router(xr, W_gate, logit_bias, score_bias, T, d, E, k, scale,
                               router_work(ws, L), idx, w, blk_counts, L.nb, s);
    if (e == hipSuccess) e = mark(ev, 1, s);
    // decode-sized batches: tile_off holds 16-row slice offsets for the
    // weight-streaming kernels, else 128-row block offsets for the grouped GEMMs
    const bool decode = hy3::use_decode_path(T, d, d_ff, E, k, 2, shared);
    const int rg = hy3::decode_row_groups(T, k, E, 2, shared);
    const int max_slices = (L.rows + hy3::decode_bm(rg) - 1) / hy3::decode_bm(rg) + Eg;
    int* sched = reinterpret_cast<int*>(ws + L.sched);
    // the dispatch also zeroes the grouped GEMMs' work counters
    if (e == hipSuccess)
        e = hy3::launch_dispatch(idx, T, E, k, L.nb, blk_counts,
                                 reinterpret_cast<int32_t*>(ws + L.blk_base),
                                 reinterpret_cast<int32_t*>(ws + L.counts), offsets, tile_off,
                                 decode ? hy3::decode_bm(rg) : hy3::prefill_bm(), row_of, tok_of,
                                 shared ? 1 : 0, s, false, decode ? nullptr : sched,
                                 decode ? 0 : hy3::kSchedInts);
    if (e == hipSuccess) e = mark(ev, 2, s);
    if (e == hipSuccess) {
        if (decode)
            e = hy3::launch_gate_up_decode(x, tok_of, W_gate_up, Ws_gu, offsets, tile_off, max_slices,
                                           h, Eg, d, d_ff, rg, s);
        else
            e = hy3::launch_gate_up_grouped(x, tok_of, W_gate_up, Ws_gu, offsets, tile_off,
                                            L.max_mtiles, h, sched, Eg, d, d_ff, s);
    }
    if (e == hipSuccess) e = mark(ev, 3, s);
    if (e == hipSuccess) {
        if (decode)
            e = hy3::launch_down_decode(h, W_down, Ws_dn, offsets, tile_off, max_slices, y, Eg, d,
                                        d_ff, rg, s);
        else
            e = hy3::launch_down_grouped(h, W_down, Ws_dn, offsets, tile_off, L.max_mtiles, y, sched, Eg,
                                         d, d_ff, s);
    }
    if (e == hipSuccess) e = mark(ev, 4, s);
    if (e == hipSuccess) {
        if (out_bf16)
            e = hy3::launch_combine_bf16(y, row_of, w, resid, out_bf16, T, d, k, shared ? T * k : -1, s);
        else
            e = hy3::launch_combine(y, row_of, w, out, T, d, k, shared ? T * k : -1, s);
    }
    if (e == hipSuccess) e = mark(ev, 5, s);
    return hip_status(e);
}

int forward_fp8(const uint16_t* x, const float* W_gate, const uint8_t* Wq_gu, const float* s_gu,
                const uint8_t* Wq_dn, const float* s_dn, float* out, int T, int d, int E, int k,
                int d_ff, float scale, void* stream, const float* logit_bias, int32_t* topk_idx,
                float* topk_w, void* workspace, const Layout& L, void* const* ev, bool block) {
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t Tk = static_cast<size_t>(T) * k;
    int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(ws + L.idx);
    float* w = topk_w ? topk_w : reinterpret_cast<float*>(ws + L.w);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* tile_off = reinterpret_cast<int32_t*>(ws + L.tile_off);
    int32_t* row_of = reinterpret_cast<int32_t*>(ws + L.row_of);
    int32_t* tok_of = reinterpret_cast<int32_t*>(ws + L.tok_of);
    uint16_t* h16 = reinterpret_cast<uint16_t*>(ws + L.h);
    uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
    float* hs = reinterpret_cast<float*>(ws + L.hs);
    uint32_t* amax = reinterpret_cast<uint32_t*>(ws + L.amax);
    uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
    float* xs = reinterpret_cast<float*>(ws + L.xs);
    uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.y);

    hipError_t e = mark(ev, 0, s);
    if (e == hipSuccess)
        e = hy3::launch_router(x, W_gate, logit_bias, nullptr, T, d, E, k, scale, router_work(ws, L),
                               idx, w, reinterpret_cast<int32_t*>(ws + L.blk_counts), L.nb, s);
    if (e == hipSuccess) e = mark(ev, 1, s);
    const bool decode = hy3::use_decode_path(T, d, d_ff, E, k, 1, false);
    const int rg = hy3::decode_row_groups(T, k, E, 1, false);
    const int max_slices = (L.rows + hy3::decode_bm(rg) - 1) / hy3::decode_bm(rg) + E;
    int* sched = reinterpret_cast<int*>(ws + L.sched);
    // the dispatch also zeroes the weight-streaming gate_up's row maxima
    // (decode) or the grouped GEMMs' work counters
    if (e == hipSuccess)
        e = hy3::launch_dispatch(idx, T, E, k, L.nb, reinterpret_cast<int32_t*>(ws + L.blk_counts),
                                 reinterpret_cast<int32_t*>(ws + L.blk_base),
                                 reinterpret_cast<int32_t*>(ws + L.counts), offsets, tile_off,
                                 decode ? hy3::decode_bm(rg) : hy3::prefill_bm(), row_of, tok_of, 0, s,
                                 false, decode ? reinterpret_cast<int32_t*>(amax) : sched,
                                 decode ? static_cast<int>(Tk) : hy3::kSchedInts);
    if (e == hipSuccess) e = mark(ev, 2, s);
    // the grouped gate_up reads its rows' activation scales per dispatch row,
    // from hs, which the h quantiser overwrites after it
    if (e == hipSuccess)
        e = hy3::launch_quant_rows(x, T, d, xq, xs, s, decode ? nullptr : row_of, k, decode ? nullptr : hs);
    float* hmax = reinterpret_cast<float*>(amax);
    const int nblk = (d_ff + 127) / 128;
    if (e == hipSuccess) {
        if (decode)
            e = hy3::launch_gate_up_decode_fp8(xq, xs, tok_of, Wq_gu, s_gu, offsets, tile_off, max_slices,
                                               h16, amax, E, d, d_ff, rg, block, s);
        else if (block)
            e = hy3::launch_gate_up_fp8_block(xq, hs, tok_of, Wq_gu, s_gu, offsets, tile_off,
                                              L.max_mtiles, h16, hmax, static_cast<int>(Tk), sched, E, d, d_ff, s);
        else
            e = hy3::launch_gate_up_fp8(xq, hs, tok_of, Wq_gu, s_gu, offsets, tile_off, L.max_mtiles,
                                        h16, hmax, static_cast<int>(Tk), sched, E, d, d_ff, s);
    }
    if (e == hipSuccess)
        e = hy3::launch_quant_rows_h(h16, decode ? amax : nullptr, decode ? nullptr : hmax, nblk,
                                       static_cast<int>(Tk), d_ff, hq, hs, s);
    if (e == hipSuccess) e = mark(ev, 3, s);
    if (e == hipSuccess) {
        if (decode)
            e = hy3::launch_down_decode_fp8(hq, hs, Wq_dn, s_dn, offsets, tile_off, max_slices, y, E, d,
                                            d_ff, rg, block, s);
        else if (block)
            e = hy3::launch_down_fp8_block(hq, hs, Wq_dn, s_dn, offsets, tile_off, L.max_mtiles, y, sched,
                                           E, d, d_ff, s);
        else
            e = hy3::launch_down_fp8(hq, hs, Wq_dn, s_dn, offsets, tile_off, L.max_mtiles, y, sched, E,
                                     d, d_ff, s);
    }
    if (e == hipSuccess) e = mark(ev, 4, s);
    if (e == hipSuccess) e = hy3::launch_combine(y, row_of, w, out, T, d, k, -1, s);
    if (e == hipSuccess) e = mark(ev, 5, s);
    return hip_status(e);
}

// Argument checks shared by the e4m3 entry points.  Block-scaled weights
// need d and d_ff in whole 256-element batches of the weight-streaming
// kernels and at most 16384 (128 k-blocks per row).
int fp8_entry(const uint16_t* x, const float* W_gate, const uint8_t* Wq_gu, const float* s_gu,
              const uint8_t* Wq_dn, const float* s_dn, float* out, int T, int d, int E, int k,
              int d_ff, float scale, void* stream, const float* logit_bias, int32_t* topk_idx,
              float* topk_w, void* workspace, size_t workspace_bytes, void* const* ev, bool block) {
    int st = check_shape(T, d, E, k, d_ff);
    if (st != HY3MOE_OK) return st;
    if (T == 0) return HY3MOE_OK;
    if (!x || !W_gate || !Wq_gu || !s_gu || !Wq_dn || !s_dn || !out || !workspace)
        return HY3MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(W_gate) || !aligned16(Wq_gu) || !aligned16(s_gu) ||
        !aligned16(Wq_dn) || !aligned16(s_dn) || !aligned16(out) || !aligned16(workspace) ||
        (logit_bias && !aligned16(logit_bias)) || (topk_idx && !aligned16(topk_idx)) ||
        (topk_w && !aligned16(topk_w)))
        return HY3MOE_ERR_ALIGN;
    if ((d % 128) != 0 || (d_ff % 128) != 0) return HY3MOE_ERR_UNSUPPORTED;
    if (block && ((d % 256) != 0 || (d_ff % 256) != 0 || d > 16384 || d_ff > 16384))
        return HY3MOE_ERR_UNSUPPORTED;
    const Layout L = make_layout(T, d, E, k, d_ff, HY3MOE_WEIGHTS_FP8_E4M3);
    if (workspace_bytes < L.total) return HY3MOE_ERR_WORKSPACE;
    return forward_fp8(x, W_gate, Wq_gu, s_gu, Wq_dn, s_dn, out, T, d, E, k, d_ff, scale, stream,
                       logit_bias, topk_idx, topk_w, workspace, L, ev, block);
}

}  // namespace

extern "C" {

int hy3moe_forward(const uint16_t* x, const float* W_gate, const uint16_t* W_gate_up,
                   const uint16_t* W_down, float* out, int T, int d, int E, int k, int d_ff,
                   float scale, void* stream, const float* logit_bias, int32_t* topk_idx,
                   float* topk_w, void* workspace, size_t workspace_bytes) {
    return forward_bf16(x, nullptr, 0.f, W_gate, logit_bias, nullptr, W_gate_up, W_down, nullptr,
                        nullptr, out, T, d, E, k, d_ff, scale, stream, topk_idx, topk_w, workspace,
                        workspace_bytes, nullptr);
}

int hy3moe_forward_timed(const uint16_t* x, const float* W_gate, const uint16_t* W_gate_up,
                         const uint16_t* W_down, float* out, int T, int d, int E, int k, int d_ff,
                         float scale, void* stream, const float* logit_bias, int32_t* topk_idx,
                         float* topk_w, void* workspace, size_t workspace_bytes,
                         void* const* stage_events) {
    return forward_bf16(x, nullptr, 0.f, W_gate, logit_bias, nullptr, W_gate_up, W_down, nullptr,
                        nullptr, out, T, d, E, k, d_ff, scale, stream, topk_idx, topk_w, workspace,
                        workspace_bytes, stage_events);
}

int hy3moe_forward_noalloc(const uint16_t* x, const float* W_gate, const uint16_t* W_gate_up,
                           const uint16_t* W_down, float* out, int T, int d, int E, int k, int d_ff,
                           float scale, void* stream, const float* logit_bias, int32_t* topk_idx,
                           float* topk_w) {
    return forward_bf16(x, nullptr, 0.f, W_gate, logit_bias, nullptr, W_gate_up, W_down, nullptr,
                        nullptr, out, T, d, E, k, d_ff, scale, stream, topk_idx, topk_w, nullptr, 0,
                        nullptr, nullptr, nullptr, true);
}

int hy3moe_block_workspace_size(int T, int d, int E, int k, int d_ff, size_t* bytes) {
    if (!bytes) return HY3MOE_ERR_NULL;
    const int st = check_shape(T, d, E, k, d_ff);
    if (st != HY3MOE_OK) return st;
    if (E > 1023) return HY3MOE_ERR_UNSUPPORTED;
    *bytes = make_layout(T, d, E, k, d_ff, HY3MOE_WEIGHTS_BF16, true, true).total;
    return HY3MOE_OK;
}

int hy3moe_block_forward(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                         const float* W_gate, const float* score_bias, const uint16_t* W_gate_up,
                         const uint16_t* W_down, const uint16_t* Ws_gate_up, const uint16_t* Ws_down,
                         float* out, int T, int d, int E, int k, int d_ff, float scale, void* stream,
                         int32_t* topk_idx, float* topk_w, void* workspace, size_t workspace_bytes) {
    return forward_bf16(x, norm_weight, norm_eps, W_gate, nullptr, score_bias, W_gate_up, W_down,
                        Ws_gate_up, Ws_down, out, T, d, E, k, d_ff, scale, stream, topk_idx, topk_w,
                        workspace, workspace_bytes, nullptr);
}

int hy3moe_block_forward_bf16(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                              const float* W_gate, const float* score_bias,
                              const uint16_t* W_gate_up, const uint16_t* W_down,
                              const uint16_t* Ws_gate_up, const uint16_t* Ws_down,
                              const uint16_t* residual, uint16_t* out, int T, int d, int E, int k,
                              int d_ff, float scale, void* stream, int32_t* topk_idx, float* topk_w,
                              void* workspace, size_t workspace_bytes) {
    return forward_bf16(x, norm_weight, norm_eps, W_gate, nullptr, score_bias, W_gate_up, W_down,
                        Ws_gate_up, Ws_down, nullptr, T, d, E, k, d_ff, scale, stream, topk_idx,
                        topk_w, workspace, workspace_bytes, nullptr, residual, out);
}

int hy3moe_block_forward_bf16_timed(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                                    const float* W_gate, const float* score_bias,
                                    const uint16_t* W_gate_up, const uint16_t* W_down,
                                    const uint16_t* Ws_gate_up, const uint16_t* Ws_down,
                                    const uint16_t* residual, uint16_t* out, int T, int d, int E,
                                    int k, int d_ff, float scale, void* stream, int32_t* topk_idx,
                                    float* topk_w, void* workspace, size_t workspace_bytes,
                                    void* const* stage_events) {
    return forward_bf16(x, norm_weight, norm_eps, W_gate, nullptr, score_bias, W_gate_up, W_down,
                        Ws_gate_up, Ws_down, nullptr, T, d, E, k, d_ff, scale, stream, topk_idx,
                        topk_w, workspace, workspace_bytes, stage_events, residual, out);
}

int hy3moe_block_forward_timed(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                               const float* W_gate, const float* score_bias,
                               const uint16_t* W_gate_up, const uint16_t* W_down,
                               const uint16_t* Ws_gate_up, const uint16_t* Ws_down, float* out, int T,
                               int d, int E, int k, int d_ff, float scale, void* stream,
                               int32_t* topk_idx, float* topk_w, void* workspace,
                               size_t workspace_bytes, void* const* stage_events) {
    return forward_bf16(x, norm_weight, norm_eps, W_gate, nullptr, score_bias, W_gate_up, W_down,
                        Ws_gate_up, Ws_down, out, T, d, E, k, d_ff, scale, stream, topk_idx, topk_w,
                        workspace, workspace_bytes, stage_events);
}



int hy3moe_forward_fp8(const uint16_t* x, const float* W_gate, const uint8_t* Wq_gate_up,
                       const float* s_gate_up, const uint8_t* Wq_down, const float* s_down,
                       float* out, int T, int d, int E, int k, int d_ff, float scale, void* stream,
                       const float* logit_bias, int32_t* topk_idx, float* topk_w, void* workspace,
                       size_t workspace_bytes) {
    return fp8_entry(x, W_gate, Wq_gate_up, s_gate_up, Wq_down, s_down, out, T, d, E, k, d_ff, scale,
                     stream, logit_bias, topk_idx, topk_w, workspace, workspace_bytes, nullptr, false);
}

int hy3moe_forward_fp8_timed(const uint16_t* x, const float* W_gate, const uint8_t* Wq_gate_up,
                             const float* s_gate_up, const uint8_t* Wq_down, const float* s_down,
                             float* out, int T, int d, int E, int k, int d_ff, float scale,
                             void* stream, const float* logit_bias, int32_t* topk_idx,
                             float* topk_w, void* workspace, size_t workspace_bytes,
                             void* const* stage_events) {
    return fp8_entry(x, W_gate, Wq_gate_up, s_gate_up, Wq_down, s_down, out, T, d, E, k, d_ff, scale,
                     stream, logit_bias, topk_idx, topk_w, workspace, workspace_bytes, stage_events,
                     false);
}

int hy3moe_forward_fp8_block128(const uint16_t* x, const float* W_gate, const uint8_t* Wq_gate_up,
                                const float* sb_gate_up, const uint8_t* Wq_down, const float* sb_down,
                                float* out, int T, int d, int E, int k, int d_ff, float scale,
                                void* stream, const float* logit_bias, int32_t* topk_idx,
                                float* topk_w, void* workspace, size_t workspace_bytes) {
    return fp8_entry(x, W_gate, Wq_gate_up, sb_gate_up, Wq_down, sb_down, out, T, d, E, k, d_ff,
                     scale, stream, logit_bias, topk_idx, topk_w, workspace, workspace_bytes, nullptr,
                     true);
}

int hy3moe_forward_fp8_block128_timed(const uint16_t* x, const float* W_gate,
                                      const uint8_t* Wq_gate_up, const float* sb_gate_up,
                                      const uint8_t* Wq_down, const float* sb_down, float* out, int T,
                                      int d, int E, int k, int d_ff, float scale, void* stream,
                                      const float* logit_bias, int32_t* topk_idx, float* topk_w,
                                      void* workspace, size_t workspace_bytes,
                                      void* const* stage_events) {
    return fp8_entry(x, W_gate, Wq_gate_up, sb_gate_up, Wq_down, sb_down, out, T, d, E, k, d_ff,
                     scale, stream, logit_bias, topk_idx, topk_w, workspace, workspace_bytes,
                     stage_events, true);
}

int hy3moe_quantize_rows_e4m3(const uint16_t* x, int rows, int cols, uint8_t* q, float* s,
                              void* stream) {
    if (rows < 0 || cols <= 0) return HY3MOE_ERR_SHAPE;
    if ((cols % 64) != 0 || cols > 65536) return HY3MOE_ERR_UNSUPPORTED;
    if (rows == 0) return HY3MOE_OK;
    if (!x || !q || !s) return HY3MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return HY3MOE_ERR_ALIGN;
    return hip_status(hy3::launch_quant_rows(x, rows, cols, q, s, static_cast<hipStream_t>(stream)));
}

const char* hy3moe_status_string(int status) {
    switch (status) {
        case HY3MOE_OK: return "ok";
        case HY3MOE_ERR_NULL: return "a required pointer is NULL";
        case HY3MOE_ERR_SHAPE: return "invalid shape (T < 0, k < 1, k > E or a non-positive size)";
        case HY3MOE_ERR_UNSUPPORTED:
            return "unsupported shape or dtype (k <= 16, E <= 1024, d and d_ff multiples of 64, "
                   "T <= 2^24)";
        case HY3MOE_ERR_WORKSPACE: return "workspace smaller than hy3moe_workspace_size reports";
        case HY3MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case HY3MOE_ERR_HIP: return "a HIP launch failed (see hy3moe_last_hip_error)";
        case HY3MOE_ERR_SCRATCH:
            return "hy3moe_forward_noalloc: these sizes need more scratch than the library's static "
                   "scratch array holds (HY3MOE_NOALLOC_SCRATCH_BYTES, 64 MiB; use hy3moe_forward "
                   "with a workspace)";
        default: return "unknown status";
    }
}

int hy3moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
