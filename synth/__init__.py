"""Seeded synthetic inputs for SketchSSM decode layers.

This module is shared by the CPU oracle (``oracle/``) and by the HIP path
(``ssm_decode_amd``).  It holds input generation only -- shapes, value
distributions, the per-head rank table, the orthonormal bases, the window
phase offsets -- and none of the method's arithmetic.

Every random value comes from one counter-based generator (SplitMix64,
G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014): ``value = mix64(key(seed, stream) + (i+1)*gamma)``
with the published gamma 0x9E3779B97F4A7C15 and finaliser constants.  A
value is addressed by (seed, stream, counter), so the inputs of any decode
step can be regenerated without storing earlier steps.  Uniforms take the
top 53 bits; normals use the Box-Muller transform on two consecutive
uniforms.

The only other source of randomness is the rank draw, which follows the
stated recipe with ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

from .configs import CONFIGS, LayerConfig, sweep_configs, get_config  # noqa: F401
from .gen import (  # noqa: F401
    GAMMA, mix64, stream_key, uniform, normal, round_f32, round_bf16,
    bf16_bits, bf16_bits_to_f32, draw_ranks, rank_offsets, make_basis,
    phase_offsets, LayerInputs, make_layer_inputs, make_step_inputs,
    StepInputs, initial_state, identity_gate, round_to, STREAM,
)
