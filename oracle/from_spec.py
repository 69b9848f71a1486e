"""Build an :class:`OracleLayer` from a synthetic layer description.

The inputs come from the seeded generator module ``synth`` (the only code the
oracle and the GPU path both use); every value is decoded here to float64.
"""
from __future__ import annotations

import numpy as np

import synth

from .moe_oracle import OracleLayer, decode_bf16, decode_f32


def decode_act(spec, a) -> np.ndarray:
    return decode_f32(a) if spec.act == synth.DT_F32 else decode_bf16(a)


def layer_from_spec(spec, router_eh=None, bias=None, cache_size: int = 256) -> OracleLayer:
    if router_eh is None:
        router_eh = synth.router_eh(spec)
    if bias is None:
        bias = synth.router_bias(spec)
    R = decode_act(spec, router_eh).T          # [H][E]
    return OracleLayer(np.ascontiguousarray(R), decode_f32(bias), spec.k,
                       lambda e, which: synth.expert_stored(spec, e, which),
                       cache_size=cache_size)


def tokens_f64(spec, first: int, count: int) -> np.ndarray:
    return decode_act(spec, synth.tokens(spec, first, count))
