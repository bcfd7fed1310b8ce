"""Hy3 MoE layer forward pass on MI355X (gfx950): hand-written HIP kernels
behind the C ABI declared in include/hy3moe.h, with a thin ctypes binding
(``sparse_moe_layer_wave_amd.hy3moe``).  ``inputs`` draws the seeded synthetic
workloads."""
