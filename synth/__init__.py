"""Seeded synthetic inputs for the low-bit quantized MoE expert FFN workloads.

This package only draws random numbers and lays them out in the canonical
input format that both the HIP library and the CPU oracle accept:

* packed codes, row-major ``[E][N][K*bits/8]`` bytes, fields LSB-first along K
  (the packed ``wq`` convention of MLX's ``quantize``, issue "2-bit
  quantized_matmul loses its size advantage over 4-bit at M >= 3", repro);
* per-block scales (and, for affine formats, biases) ``[E][N][K/B]`` as raw
  16-bit patterns of the stated storage dtype;
* activations as raw 16-bit patterns, router logits as float32.

It holds none of the method's arithmetic (no dequantization, routing or
products).  Every value comes from one counter-based generator, SplitMix64
(Steele, Lea, Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014), keyed by (seed, workload, tensor), so that the oracle and the
GPU path see bit-identical inputs on any machine and NumPy version.
"""

from .rng import (  # noqa: F401
    Key,
    raw_u64,
    uniform01,
    normals,
    f32_to_bf16_bits,
    f32_to_f16_bits,
    random_bytes,
    codes_uniform,
    codes_ternary,
    ternary_digits,
    pack_base3,
)
from .workloads import (  # noqa: F401
    MatFmt,
    custom_moe_spec,
    custom_linear_spec,
    FORMATS,
    MoeSpec,
    LinearSpec,
    MOE_WORKLOADS,
    LINEAR_WORKLOADS,
    moe_inputs,
    linear_inputs,
    canonical_matrix_bytes,
    channel_inputs,
)
