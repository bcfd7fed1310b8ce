"""CPU oracle for one Hy3 MoE layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls, links or
executes this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers, tables
or helpers with the HIP path (``sparse_moe_layer_wave_amd/``) and imports
nothing from it.

What it computes is the plain definition of the layer, in NumPy float64 except
where the pages fix a precision (the router's scores are fp32, the FP8 variant
quantises to OCP e4m3):

* router: logits = x . W_gate^T (fp32 weights), sigmoid scores, top-k with ties
  to the lower expert index, the k scores divided by their sum and multiplied by
  router_scaling_factor -- "Tencent Hy3-295B architecture teardown", section 4.1
  (router flow steps 1, 3, 4, 5) and "Tencent Hy3-Flash Q&A", Q4.2;
* expert: SwiGLU with the fused gate_up projection, SiLU on the gate half --
  "Tencent Hy3-295B architecture teardown", section 2.3 (parameter breakdown)
  and "DeepSeek V4-Flash architecture Q&A", Q4.5;
* full block (``forward_block``): the shared expert's output added to the
  routed sum -- "Tencent Hy3-Flash Q&A", Q4.7; the router fed an RMSNorm'd
  copy of x (route_norm, Q4.9) and choosing with the selection-only
  e_score_correction_bias (Q4.3; "Tencent Hy3-295B architecture teardown",
  section 4.1, router flow step 2);
* residual branch (``forward_block_residual``): the bf16 residual row added to
  the block output in a wider type -- wmrh.cn Hy3 assembly blog, sections 3.2
  (residual add) and 2.3 (fp32 combine);
* combine: per-expert loop adding weight * expert output into the token's row
  -- "DeepSeek V4-Flash architecture Q&A", Q8.4 (the MoE forward sketch and
  the index_add_ note), done in float64 so the fp32-combine requirement
  (wmrh.cn Hy3 assembly blog, section 2.3) is met with margin;
* activation precision: the model's activations are bf16 tensors, and the
  fp32 combine widens bf16 expert outputs before adding them (wmrh.cn Hy3
  assembly blog, section 2.3; "Tencent Hy3-Flash Q&A", Q6.2 describes the
  bf16 sum used when that option is off).  So by default the SwiGLU
  activation h and each expert output y are rounded once to bf16 (from
  float64) where the layer stores them; ``bf16_activations=False`` gives the
  all-float64 expression.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, library routines and brute force.  Parity unpinned: the value 2.826
itself, and anything that would need the real model's weights.
"""

from .codecs import (bf16_bits_to_f64, f32_to_bf16_bits, round_to_bf16, e4m3_bits_to_f64,
                     f32_to_e4m3_bits, E4M3_MAX)
from .moe import (route, expert_swiglu, expert_swiglu_parts, forward, forward_tokens,
                  quant_row_e4m3, quant_row_e4m3_parts, quant_rows_e4m3, dequant_e4m3, forward_fp8,
                  forward_fp8_tokens, rms_norm_bf16, forward_block, forward_block_tokens,
                  forward_block_residual, forward_detail, forward_fp8_detail, Detail,
                  expert_param_count, flops_per_token, NEAR_TIE)

__all__ = [
    "bf16_bits_to_f64", "f32_to_bf16_bits", "round_to_bf16", "e4m3_bits_to_f64", "f32_to_e4m3_bits",
    "E4M3_MAX", "route", "expert_swiglu", "expert_swiglu_parts", "forward", "forward_tokens",
    "quant_row_e4m3", "quant_row_e4m3_parts", "quant_rows_e4m3", "dequant_e4m3", "forward_fp8",
    "forward_fp8_tokens", "rms_norm_bf16", "forward_block", "forward_block_tokens",
    "forward_block_residual", "forward_detail", "forward_fp8_detail", "Detail",
    "expert_param_count", "flops_per_token", "NEAR_TIE",
]
