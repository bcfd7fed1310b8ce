/*
 * hy3moe.h -- C ABI of the Hy3 MoE layer forward pass on MI355X (gfx950).
 *
 * The layer (one MoE FFN block of Hy3, routed experts; the full block with
 * the shared expert, route_norm and the selection-only score bias is the
 * hy3moe_block_* group further down):
 *   router   logits = x . W_gate^T (+ per-expert logit bias), computed in fp32;
 *            s = sigmoid(logits); the k experts with the largest s are chosen
 *            (equal scores: lower expert index first; slot j = j-th largest);
 *            w_j = scale * s_j / sum_j s_j
 *            ["Tencent Hy3-295B architecture teardown", section 4.1, router
 *             flow steps 1, 3, 4, 5; "Tencent Hy3-Flash Q&A", Q4.2 and Q6.2]
 *   experts  SwiGLU: h = SiLU(x . Wg^T) * (x . Wu^T), y = h . Wd^T, where the
 *            fused gate_up matrix holds Wg in rows [0, d_ff) and Wu in rows
 *            [d_ff, 2 d_ff)  ["Tencent Hy3-295B architecture teardown",
 *             section 2.3; "DeepSeek V4-Flash architecture Q&A", Q4.5]
 *   combine  out[t] = sum_j w_j * y_{t,j}, accumulated in fp32 in slot order
 *            ["DeepSeek V4-Flash architecture Q&A", Q8.4; wmrh.cn Hy3 assembly
 *             blog, section 2.3 (enable_moe_fp32_combine)]
 *
 * Conventions for every call:
 *   - Every pointer argument is DEVICE memory owned by the caller, except the
 *     size_t* out-parameters of the *_workspace_size calls and the
 *     stage_events arrays of the *_timed calls (host).  The library never
 *     allocates, frees or synchronises; it keeps no state between calls apart
 *     from a thread-local copy of the last HIP error and a per-device cache
 *     of the compute-unit count (queried on a device's first launch; safe to
 *     fill from several threads at once).
 *   - Layouts are dense and row-major.  bf16 = uint16_t bit patterns;
 *     e4m3 = uint8_t codes of the OCP E4M3FN format (bias 7, max 448, no inf).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it; results are ready once the stream has
 *     reached that point.  Device faults surface at the caller's next sync.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     negative status other than HY3MOE_ERR_HIP means nothing was enqueued.
 *     HY3MOE_ERR_HIP means a kernel launch (or a stage event record) failed:
 *     the launches before it may have been enqueued, and the outputs are
 *     undefined.  T == 0 is a successful no-op.  Supported shapes:
 *     1 <= k <= min(E, 16), 1 <= E <= 1024, d and d_ff multiples of 64,
 *     T <= 2^24.  Every pointer must be 16-byte aligned.
 *   - The workspace is scratch device memory of at least the size that
 *     hy3moe_workspace_size reports; its contents on entry do not matter and
 *     are undefined on return.  Calls that share a workspace must not overlap.
 */
#ifndef HY3MOE_H
#define HY3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HY3MOE_OK = 0,
    HY3MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    HY3MOE_ERR_SHAPE = -2,       /* T < 0, k < 1, k > E, or a non-positive size */
    HY3MOE_ERR_UNSUPPORTED = -3, /* outside the supported shapes listed above, or unknown dtype */
    HY3MOE_ERR_WORKSPACE = -4,   /* workspace smaller than required */
    HY3MOE_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
    HY3MOE_ERR_HIP = -6,         /* a HIP launch failed; see hy3moe_last_hip_error() */
    HY3MOE_ERR_SCRATCH = -7      /* hy3moe_forward_noalloc: sizes need more than its static scratch */
} hy3moe_status;

enum { HY3MOE_WEIGHTS_BF16 = 0, HY3MOE_WEIGHTS_FP8_E4M3 = 1 };

/* Bytes of workspace hy3moe_forward (weight_dtype BF16) or hy3moe_forward_fp8
 * (FP8_E4M3) needs for these sizes; it also covers hy3moe_route,
 * hy3moe_route_ex without norm_weight, and hy3moe_permute.  Writes *bytes
 * (host pointer).  Grows monotonically with T. */
int hy3moe_workspace_size(int T, int d, int E, int k, int d_ff, int weight_dtype, size_t* bytes);

/* Router alone ("Tencent Hy3-295B architecture teardown", section 4.1).
 *   x          bf16 [T, d]
 *   W_gate     fp32 [E, d]
 *   logit_bias fp32 [E], added to every token's logits before the sigmoid, or NULL
 *   scale      router_scaling_factor (Hy3: 2.826)
 *   topk_idx   int32 [T, k] out: chosen experts, slot order = descending score,
 *              equal scores by ascending expert index
 *   topk_w     fp32 [T, k] out: scale * s_j / sum of the k chosen scores
 * The logits are fp32 sums of exact products (x is bf16, W_gate is split into
 * three bf16 parts that add up to it exactly); the scores are fp32. */
int hy3moe_route(const uint16_t* x, const float* W_gate, const float* logit_bias,
                 int T, int d, int E, int k, float scale,
                 int32_t* topk_idx, float* topk_w,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Dispatch order alone: a stable counting sort of the T*k (token, slot) pairs by
 * expert, i.e. expert-contiguous rows, ascending token inside an expert (the
 * grouping the per-expert loop of "DeepSeek V4-Flash architecture Q&A", Q8.4,
 * performs, laid out for grouped GEMMs).
 *   topk_idx  int32 [T, k] in: the experts of each token
 *   counts    int32 [E] out: pairs per expert
 *   offsets   int32 [E+1] out: exclusive prefix sum of counts (offsets[E] =
 *             the number of pairs given a row, T*k for a valid routing)
 *   row_of    int32 [T, k] out: row of pair (t, j) in expert-contiguous order
 *   token_of  int32 [T*k] out: token of each row; entries from offsets[E] on
 *             are not written
 * Entries are checked on the device: a pair whose expert is outside [0, E),
 * or repeats an expert listed earlier in the same token's row, is dropped --
 * it is counted for no expert and gets row_of = -1 -- and the other pairs
 * keep the order above.  Nothing is read or written out of bounds. */
int hy3moe_permute(const int32_t* topk_idx, int T, int E, int k,
                   int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of,
                   void* workspace, size_t workspace_bytes, void* stream);

/* The whole layer with bf16 experts.
 *   x          bf16 [T, d];  W_gate fp32 [E, d]
 *   W_gate_up  bf16 [E, 2*d_ff, d] (rows [0,d_ff) gate, [d_ff,2*d_ff) up)
 *   W_down     bf16 [E, d, d_ff]
 *   out        fp32 [T, d] out, overwritten (not accumulated): the routed
 *              experts' weighted sum; shared expert and residual are not added
 *   logit_bias fp32 [E] or NULL (as in hy3moe_route)
 *   topk_idx, topk_w  NULL, or [T, k] outputs receiving the routing
 * Expert products run on bf16 MFMA with fp32 accumulation; SiLU(gate)*up is
 * computed in fp32 and stored as bf16; each expert output row is stored as
 * bf16 and the combine accumulates in fp32 in slot order (deterministic). */
int hy3moe_forward(const uint16_t* x, const float* W_gate,
                   const uint16_t* W_gate_up, const uint16_t* W_down, float* out,
                   int T, int d, int E, int k, int d_ff, float scale, void* stream,
                   const float* logit_bias, int32_t* topk_idx, float* topk_w,
                   void* workspace, size_t workspace_bytes);

/* hy3moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; the scratch is a static device array inside the
 * library, HY3MOE_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU the library
 * runs on, held until the process ends.  The call allocates nothing and
 * enqueues the same kernels as hy3moe_forward, so the results are the same
 * bit for bit.  Sizes whose hy3moe_workspace_size (BF16) exceeds the scratch
 * return HY3MOE_ERR_SCRATCH with nothing enqueued (at the Hy3 sizes d = 4096,
 * E = 192, k = 8, d_ff = 1536 that is T > 603).  All calls on one GPU share
 * its scratch array: calls that may overlap on a GPU (other streams, other
 * threads) race and must be ordered by the caller.  The first call on a
 * device looks the array's address up once (hipGetSymbolAddress); a failure
 * there returns HY3MOE_ERR_HIP.  Other arguments and errors as for
 * hy3moe_forward. */
#define HY3MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int hy3moe_forward_noalloc(const uint16_t* x, const float* W_gate,
                           const uint16_t* W_gate_up, const uint16_t* W_down, float* out,
                           int T, int d, int E, int k, int d_ff, float scale, void* stream,
                           const float* logit_bias, int32_t* topk_idx, float* topk_w);

/* hy3moe_forward with instrumentation: stage_events is a HOST array of 6
 * hipEvent_t handles (any may be NULL) recorded on `stream` before the router,
 * after the router, after the dispatch order, after gate_up, after down and
 * after the combine.  The caller creates the events and reads them with
 * hipEventElapsedTime; the work enqueued is that of hy3moe_forward. */
int hy3moe_forward_timed(const uint16_t* x, const float* W_gate,
                         const uint16_t* W_gate_up, const uint16_t* W_down, float* out,
                         int T, int d, int E, int k, int d_ff, float scale, void* stream,
                         const float* logit_bias, int32_t* topk_idx, float* topk_w,
                         void* workspace, size_t workspace_bytes, void* const* stage_events);

/* The whole layer with e4m3 experts and per-output-channel fp32 scales
 * (formats: "DeepSeek V4-Flash architecture Q&A", Q7.2 and Q7.4).
 *   Wq_gate_up e4m3 [E, 2*d_ff, d], s_gate_up fp32 [E, 2*d_ff]
 *   Wq_down    e4m3 [E, d, d_ff],   s_down    fp32 [E, d]
 * Routing is the fp32 router above.  Each token's x row and each (token, slot)
 * SwiGLU activation row are quantised to e4m3 with one fp32 scale per row, as
 * hy3moe_quantize_rows_e4m3 does (the activation row as stored: rounded to
 * bf16);
 * the products run on fp8 MFMA with fp32 accumulation and are rescaled by row
 * scale * channel scale; expert outputs are stored as bf16 and combined in
 * fp32 as in hy3moe_forward.  d and d_ff must be multiples of 128 here
 * (HY3MOE_ERR_UNSUPPORTED otherwise).  Other arguments as for hy3moe_forward. */
int hy3moe_forward_fp8(const uint16_t* x, const float* W_gate,
                       const uint8_t* Wq_gate_up, const float* s_gate_up,
                       const uint8_t* Wq_down, const float* s_down, float* out,
                       int T, int d, int E, int k, int d_ff, float scale, void* stream,
                       const float* logit_bias, int32_t* topk_idx, float* topk_w,
                       void* workspace, size_t workspace_bytes);

/* hy3moe_forward_fp8 with the six stage events of hy3moe_forward_timed; the
 * e4m3 quantisation of x and of the SwiGLU activations falls in the gate_up
 * stage. */
int hy3moe_forward_fp8_timed(const uint16_t* x, const float* W_gate,
                             const uint8_t* Wq_gate_up, const float* s_gate_up,
                             const uint8_t* Wq_down, const float* s_down, float* out,
                             int T, int d, int E, int k, int d_ff, float scale, void* stream,
                             const float* logit_bias, int32_t* topk_idx, float* topk_w,
                             void* workspace, size_t workspace_bytes, void* const* stage_events);

/* The whole layer with e4m3 experts quantised in 128 x 128 blocks, one fp32
 * scale per block ("DeepSeek V4-Flash architecture Q&A", Q7.2: block-wise
 * quantisation of the weight matrices):
 *   Wq_gate_up e4m3 [E, 2*d_ff, d], sb_gate_up fp32 [E, 2*d_ff/128, d/128]
 *   Wq_down    e4m3 [E, d, d_ff],   sb_down    fp32 [E, d/128, d_ff/128]
 * weight [e, n, i] = e4m3 value * sb[e, n/128, i/128] (row-major scale grids).
 * Activations are quantised per row as in hy3moe_forward_fp8.  Each 128-wide
 * k-block's fp8 MFMA product is scaled by its block's scale and added to the
 * fp32 accumulator, which is rescaled by the row scale at the end.
 * Decode-sized batches run on the weight-streaming kernels; larger ones run on
 * grouped kernels with 128 x 128 tiles, one weight block per tile and k-block.
 * d and d_ff must be multiples of 256 and at most 16384
 * (HY3MOE_ERR_UNSUPPORTED otherwise).  The workspace is
 * hy3moe_workspace_size with HY3MOE_WEIGHTS_FP8_E4M3.  Other arguments as for
 * hy3moe_forward_fp8. */
int hy3moe_forward_fp8_block128(const uint16_t* x, const float* W_gate,
                                const uint8_t* Wq_gate_up, const float* sb_gate_up,
                                const uint8_t* Wq_down, const float* sb_down, float* out,
                                int T, int d, int E, int k, int d_ff, float scale, void* stream,
                                const float* logit_bias, int32_t* topk_idx, float* topk_w,
                                void* workspace, size_t workspace_bytes);

/* hy3moe_forward_fp8_block128 with the six stage events of
 * hy3moe_forward_fp8_timed. */
int hy3moe_forward_fp8_block128_timed(const uint16_t* x, const float* W_gate,
                                      const uint8_t* Wq_gate_up, const float* sb_gate_up,
                                      const uint8_t* Wq_down, const float* sb_down, float* out,
                                      int T, int d, int E, int k, int d_ff, float scale,
                                      void* stream, const float* logit_bias, int32_t* topk_idx,
                                      float* topk_w, void* workspace, size_t workspace_bytes,
                                      void* const* stage_events);

/* ---- the full Hy3 MoE block ("Tencent Hy3-Flash Q&A", Q4.3, Q4.7, Q4.9) ----
 *
 *   block out[t] = Shared(x_t) + sum_j w_j * Expert_idx[t,j](x_t)
 *
 * where Shared is a SwiGLU expert that every token passes through (Q4.7),
 * the router scores route_norm(x) instead of x (Q4.9), and it chooses the k
 * experts with the largest s + score_bias while the weights still use s
 * (e_score_correction_bias, Q4.3; "Tencent Hy3-295B architecture teardown",
 * section 4.1, router flow step 2).  The experts, shared and routed, see x.
 *
 * route_norm: r = fp32(1 / sqrt(sum_i x_i^2 / d + eps)) (sum, division and
 * square root in fp64; the pages fix neither precision nor eps), the row
 * x * r is rounded to bf16 and multiplied by the bf16 weight with one more
 * bf16 rounding.  score_bias: choice value = fp32(s + b) (may be negative);
 * equal values go to the lower expert index. */

/* Bytes of workspace for hy3moe_block_forward at these sizes (with both
 * route_norm and the shared expert); it also covers hy3moe_route_ex.  E <= 1023. */
int hy3moe_block_workspace_size(int T, int d, int E, int k, int d_ff, size_t* bytes);

/* Router of the full block.
 *   norm_weight  bf16 [d] route_norm weight, or NULL for no route_norm
 *   norm_eps     route_norm epsilon (fp32, >= 0; else HY3MOE_ERR_SHAPE)
 *   logit_bias   fp32 [E] added to the logits before the sigmoid, or NULL
 *   score_bias   fp32 [E] selection-only bias (e_score_correction_bias), or NULL
 * Other arguments and outputs as for hy3moe_route; the workspace must hold
 * what hy3moe_block_workspace_size (or, without norm_weight,
 * hy3moe_workspace_size) reports for these sizes. */
int hy3moe_route_ex(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                    const float* W_gate, const float* logit_bias, const float* score_bias,
                    int T, int d, int E, int k, float scale,
                    int32_t* topk_idx, float* topk_w,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The full block with bf16 experts.
 *   norm_weight, norm_eps, score_bias   as for hy3moe_route_ex (each optional)
 *   Ws_gate_up bf16 [2*d_ff, d], Ws_down bf16 [d, d_ff]: the shared expert,
 *              with the routed experts' d_ff; both or neither (NULL)
 *   out        fp32 [T, d] out, overwritten: shared + routed sum, no residual
 * The shared expert runs as expert E of the grouped expert kernels, on every
 * token; its activation and output are bf16 like a routed expert's, and its
 * output row is added to the fp32 combine after the k routed terms with
 * weight 1.  E <= 1023.  Other arguments as for hy3moe_forward. */
int hy3moe_block_forward(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                         const float* W_gate, const float* score_bias,
                         const uint16_t* W_gate_up, const uint16_t* W_down,
                         const uint16_t* Ws_gate_up, const uint16_t* Ws_down, float* out,
                         int T, int d, int E, int k, int d_ff, float scale, void* stream,
                         int32_t* topk_idx, float* topk_w,
                         void* workspace, size_t workspace_bytes);

/* The decoder layer's residual branch ended in the block: hy3moe_block_forward
 * with a bf16 output and the residual added in the fp32 combine (the wmrh.cn
 * Hy3 assembly blog: the residual add of section 3.2, in fp32 as section 2.3
 * describes, rounded back to bf16):
 *   out[t] = bf16( (sum_j w_j * y_j + shared_t) + residual[t] )
 * with the sum in fp32 as for hy3moe_block_forward, the residual widened to
 * fp32 and added last, and one round to nearest even.
 *   residual  bf16 [T, d] in, or NULL for no residual (out is then the block
 *             output rounded to bf16)
 *   out       bf16 [T, d] out, overwritten; it may be the residual buffer
 *             itself (in-place update) and must not overlap any other argument
 * Other arguments, errors and workspace as for hy3moe_block_forward. */
int hy3moe_block_forward_bf16(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                              const float* W_gate, const float* score_bias,
                              const uint16_t* W_gate_up, const uint16_t* W_down,
                              const uint16_t* Ws_gate_up, const uint16_t* Ws_down,
                              const uint16_t* residual, uint16_t* out,
                              int T, int d, int E, int k, int d_ff, float scale, void* stream,
                              int32_t* topk_idx, float* topk_w,
                              void* workspace, size_t workspace_bytes);

/* hy3moe_block_forward_bf16 with the six stage events of hy3moe_forward_timed. */
int hy3moe_block_forward_bf16_timed(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                                    const float* W_gate, const float* score_bias,
                                    const uint16_t* W_gate_up, const uint16_t* W_down,
                                    const uint16_t* Ws_gate_up, const uint16_t* Ws_down,
                                    const uint16_t* residual, uint16_t* out,
                                    int T, int d, int E, int k, int d_ff, float scale, void* stream,
                                    int32_t* topk_idx, float* topk_w,
                                    void* workspace, size_t workspace_bytes,
                                    void* const* stage_events);

/* hy3moe_block_forward with the six stage events of hy3moe_forward_timed
 * (route_norm falls in the router stage). */
int hy3moe_block_forward_timed(const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
                               const float* W_gate, const float* score_bias,
                               const uint16_t* W_gate_up, const uint16_t* W_down,
                               const uint16_t* Ws_gate_up, const uint16_t* Ws_down, float* out,
                               int T, int d, int E, int k, int d_ff, float scale, void* stream,
                               int32_t* topk_idx, float* topk_w,
                               void* workspace, size_t workspace_bytes, void* const* stage_events);

/* Per-row e4m3 quantisation used by hy3moe_forward_fp8 for x ("DeepSeek
 * V4-Flash architecture Q&A", Q7.2: the E4M3 format, range +-448, for forward
 * activations; Q7.4: scaling factors per channel; here one fp32 scale per
 * activation row):
 *   amax = max |x[r, :]|;  amax == 0 -> q = 0, s = 1;  otherwise
 *   r = fp32(448 / amax), q = e4m3(fp32(x * r)) rounded to nearest even and
 *   saturated to +-448, s = fp32(amax / 448); the row dequantises as q * s.
 *   x bf16 [rows, cols] in; q e4m3 [rows, cols] out; s fp32 [rows] out.
 * cols must be a multiple of 64 and at most 65536. */
int hy3moe_quantize_rows_e4m3(const uint16_t* x, int rows, int cols,
                              uint8_t* q, float* s, void* stream);

/* Static text for a status code. */
const char* hy3moe_status_string(int status);

/* hipError_t of the last call on this thread that returned HY3MOE_ERR_HIP (0 if none). */
int hy3moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HY3MOE_H */
