"""Seeded synthetic inputs for the BitDelta path.

This module only draws inputs (base weights, fine-tuned weights, activations,
variant ids).  It holds none of the method's arithmetic: no delta, sign,
packing, scale or product is computed here.  Both the oracle-side tests and
the GPU path take their inputs from it.

Recipe (the page models a fine-tuning delta as Laplace(0, b); section
"Matematiksel temel"):

* W_base ~ N(0, sigma) drawn in float32, rounded to bf16 (RNE);
* Delta ~ Laplace(0, b) by inverse CDF, -b*sgn(u)*ln(1-2|u|) with
  u ~ U(-1/2, 1/2), in float32;
* W_ft = bf16(float32(W_base) + Delta);
* x ~ N(0, 1), rounded to bf16;
* variant ids: truncated Zipf(1.1) over the variants, P(v) ~ (v+1)^-1.1,
  drawn with numpy's Generator.choice;
* checkpoints for a merge: a planted rank-r task vector (Gaussian factors,
  decreasing scales) plus Laplace noise added to the base, rounded to bf16;
  the orthogonal iteration's start ~ N(0, 1) in float32.
"""

from .workloads import (  # noqa: F401
    LAYER_70B,
    WORKLOADS,
    Workload,
    bf16_bits,
    draw_activations,
    draw_base,
    draw_finetuned,
    draw_gaussian,
    draw_layer_bases,
    draw_layer_inputs,
    draw_lowrank_checkpoint,
    draw_stack_bases,
    draw_stack_inputs,
    iter_finetuned,
    iter_stack_finetuned,
    generator,
    laplace_scales,
    small_pair,
    variant_scales,
    zipf_ids,
)
