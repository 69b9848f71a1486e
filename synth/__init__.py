"""Seeded synthetic inputs for the MoE layer (host side).

This module holds no step of the MoE method itself: it only draws numbers
and encodes them into the storage formats the layer consumes.  Both the
float64 oracle and the GPU path take their inputs from here; the on-device
fill in ``synth/csrc/synth_fill.hip`` implements the very same generator so
that pools too large for host memory (the 77 GB bf16 pool) can be written
straight into HBM, while the host regenerates only the experts it needs.

Generator (one definition, two implementations):

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the constants of Vigna's public-domain
  ``splitmix64.c``), used counter-style: element ``i`` of a tensor stream with
  key ``K`` is ``mix64(K + (i + 1) * GAMMA)`` (the (i+1)-th output of a
  SplitMix64 whose state starts at K).
* Irwin--Hall(4): the four 16-bit fields of that 64-bit word are summed and
  centred, ``S = sum(u_j) - 131070`` (an integer in [-131070, 131070], variance
  4 (2^32 - 1) / 12).  ``value = fp32(S) * fp32(sigma / std(S))`` with one
  IEEE fp32 multiply, then bf16 round-to-nearest-even where the tensor is bf16.
  This is an approximately N(0, sigma) draw, bounded at 3.46 sigma, and is
  integer-exact up to that one correctly rounded multiply, so host and device
  produce identical bits.
* Element index = the linear index in the tensor's logical layout (router
  ``[E][H]``, gate/up ``[E][I][H]``, down ``[E][H][I]``, hidden states
  ``[T][H]``).

4-bit symmetric block format (the layer's quantised expert storage): blocks
of 32 consecutive elements along each row's reduction dimension;
``d = fp16_rne(amax / 7)`` (amax / 7 as an IEEE f64 quotient), ``q =
clamp(rint_half_even(w / d), -7, 7)`` (``q = 0`` when ``d = 0``), nibble
``q + 8``; byte ``j`` of a row holds element ``2j`` in its low nibble and
``2j + 1`` in its high nibble; scales are a separate fp16 array
``[rows][K / 32]``.  Encoding is data preparation; decoding belongs to the
method and is implemented separately by the oracle and by the kernels.

Router bias: ``b_e = fp32(-0.37 * ln(rank_e))`` where ``rank`` is 1 + a
seeded permutation of 0..E-1.  This gives a Zipf(1.1)-shaped expert
popularity (a few thousand distinct experts per 1000 tokens) from the
"Zipf(s=1.1)" wording of the workload description, whose literal readings
route almost every token to the same hundred experts.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
KEY_SALT = 0x5851F42D4C957F2D

# tensor stream tags
TAG_ROUTER, TAG_GATE, TAG_UP, TAG_DOWN, TAG_X, TAG_BIAS = 1, 2, 3, 4, 5, 6

IH_CENTRE = 131070                      # 2 * (2^16 - 1)
IH_STD = math.sqrt((2.0 ** 32 - 1.0) / 3.0)   # std of the 4-field sum

DT_F32, DT_BF16, DT_Q4 = 0, 1, 2
DTYPE_NAMES = {DT_F32: "f32", DT_BF16: "bf16", DT_Q4: "q4"}


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2^64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tag: int) -> int:
    """Key of one tensor stream: mix64(((seed << 16) ^ tag) ^ salt)."""
    return mix64_int(((int(seed) << 16) ^ int(tag)) ^ KEY_SALT)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def raw64(key: int, idx: np.ndarray) -> np.ndarray:
    """Counter-based SplitMix64 words for element indices ``idx`` (uint64)."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GAMMA)
        return _mix64_np(z)


def irwin_hall(key: int, idx: np.ndarray) -> np.ndarray:
    """Centred integer S in [-131070, 131070] (int64) for each index."""
    r = raw64(key, idx)
    m = np.uint64(0xFFFF)
    s = (r & m) + ((r >> np.uint64(16)) & m) + ((r >> np.uint64(32)) & m) + (r >> np.uint64(48))
    return s.astype(np.int64) - IH_CENTRE


def scale_f32(sigma: float) -> np.float32:
    """fp32 multiplier turning S into an approximately N(0, sigma) value."""
    return np.float32(sigma / IH_STD)


def scale_bits(sigma: float) -> int:
    return int(np.array([scale_f32(sigma)], dtype=np.float32).view(np.uint32)[0])


def normal_f32(key: int, idx: np.ndarray, sigma: float) -> np.ndarray:
    """fp32 values fp32(S) * fp32(sigma / std(S)) (one rounded multiply)."""
    s = irwin_hall(key, idx).astype(np.float32)       # exact: |S| < 2^24
    return s * scale_f32(sigma)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, nearest-even, returning the uint16 bit patterns."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(key: int, idx: np.ndarray, sigma: float) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(key, idx, sigma))


# ---------------------------------------------------------------- 4-bit encode
def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of f64 values, as uint16 bits.

    numpy's float64 -> float16 cast rounds the double directly (no detour
    through float32), which is what the device fill does bit by bit.
    """
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def quantize_q4_rows(w_bf16_bits: np.ndarray):
    """Encode bf16 rows [R][K] (K % 32 == 0) into (packed [R][K/2] u8, scales [R][K/32] u16)."""
    w = bf16_bits_to_f32(w_bf16_bits).astype(np.float64)
    R, K = w.shape
    assert K % 32 == 0
    wb = w.reshape(R, K // 32, 32)
    amax = np.abs(wb).max(axis=2)
    d_bits = f64_to_f16_bits(amax / 7.0)
    d = d_bits.view(np.float16).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(wb / d[:, :, None])
    q = np.where(d[:, :, None] == 0.0, 0.0, q)
    q = np.clip(q, -7, 7).astype(np.int64)
    nib = (q + 8).astype(np.uint8).reshape(R, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, d_bits


# ------------------------------------------------------------------ configs
@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shapes and storage of one synthetic MoE layer plus its token stream."""
    name: str
    H: int
    E: int
    k: int
    I: int
    act: int            # DT_F32 or DT_BF16 (router uses the same dtype)
    expert: int         # DT_F32, DT_BF16 or DT_Q4
    bias_alpha: float | None   # None: no bias (all zeros)
    T: int              # tokens per call
    calls: int          # sequential calls in the workload
    weight_seed: int = 1234
    token_seed: int = 42
    sigma_w: float = 0.02
    sigma_x: float = 1.0
    hot: int = 0        # > 0: only the `hot` experts of lowest rank get bias 0, all others -20

    @property
    def router(self) -> int:
        return self.act


CONFIGS = {
    # tiny layer, fp32 everywhere, no bias, 1 token (a 1000-token sweep in tests)
    "tiny_f32": LayerSpec("tiny_f32", 256, 64, 2, 128, DT_F32, DT_F32, None, 1, 1000, token_seed=42),
    # batch-1 decode, bf16 experts
    "decode_bf16": LayerSpec("decode_bf16", 2048, 24576, 10, 256, DT_BF16, DT_BF16, 0.37, 1, 1000, token_seed=43),
    # batch-1 decode, 4-bit experts (decode_bf16's weights quantised)
    "decode_q4": LayerSpec("decode_q4", 2048, 24576, 10, 256, DT_BF16, DT_Q4, 0.37, 1, 1000, token_seed=44),
    # speculative verify: T=5 through decode_q4's layer, 1000 steps
    "verify_q4": LayerSpec("verify_q4", 2048, 24576, 10, 256, DT_BF16, DT_Q4, 0.37, 5, 1000, token_seed=45),
    # prefill chunk: T=2048 through decode_bf16's layer
    "prefill_bf16": LayerSpec("prefill_bf16", 2048, 24576, 10, 256, DT_BF16, DT_BF16, 0.37, 2048, 1, token_seed=46),
    # supplementary (not one of the five workloads): prefill_bf16's weights with the bias
    # concentrated on 64 experts, so each gets about 320 of the 20,480 pairs and the
    # grouped expert kernels become matrix-bound
    "prefill_bf16_hot": LayerSpec("prefill_bf16_hot", 2048, 24576, 10, 256, DT_BF16, DT_BF16, 0.37, 2048, 1,
                                  token_seed=47, hot=64),
}


def small_spec(H=256, E=64, k=2, I=128, act=DT_F32, expert=DT_F32, bias_alpha=None,
               T=1, calls=1, weight_seed=7, token_seed=11, name="small") -> LayerSpec:
    return LayerSpec(name, H, E, k, I, act, expert, bias_alpha, T, calls,
                     weight_seed=weight_seed, token_seed=token_seed)


def _vals(spec: LayerSpec, key: int, idx: np.ndarray, sigma: float, dtype: int) -> np.ndarray:
    if dtype == DT_F32:
        return normal_f32(key, idx, sigma)
    return normal_bf16(key, idx, sigma)


def router_eh(spec: LayerSpec) -> np.ndarray:
    """Router weights stored expert-major [E][H] (fp32 array or bf16 bits)."""
    key = stream_key(spec.weight_seed, TAG_ROUTER)
    out = np.empty((spec.E, spec.H), dtype=np.float32 if spec.act == DT_F32 else np.uint16)
    rows = max(1, (1 << 22) // spec.H)
    for e0 in range(0, spec.E, rows):
        e1 = min(spec.E, e0 + rows)
        idx = np.arange(e0 * spec.H, e1 * spec.H, dtype=np.uint64)
        out[e0:e1] = _vals(spec, key, idx, spec.sigma_w, spec.act).reshape(e1 - e0, spec.H)
    return out


def router_bias(spec: LayerSpec) -> np.ndarray:
    """fp32 [E] logit bias: -alpha * ln(rank), rank = 1 + seeded permutation
    (with ``hot`` > 0: 0 for ranks 1..hot, -20 for the rest)."""
    if spec.bias_alpha is None:
        return np.zeros(spec.E, dtype=np.float32)
    key = stream_key(spec.weight_seed, TAG_BIAS)
    perm = np.argsort(raw64(key, np.arange(spec.E, dtype=np.uint64)), kind="stable")
    rank = np.empty(spec.E, dtype=np.float64)
    rank[perm] = np.arange(1, spec.E + 1, dtype=np.float64)
    if spec.hot > 0:
        return np.where(rank <= spec.hot, 0.0, -20.0).astype(np.float32)
    return (-spec.bias_alpha * np.log(rank)).astype(np.float32)


def tokens(spec: LayerSpec, first: int, count: int) -> np.ndarray:
    """Hidden states of tokens [first, first + count) as [count][H]."""
    key = stream_key(spec.token_seed, TAG_X)
    idx = np.arange(first * spec.H, (first + count) * spec.H, dtype=np.uint64)
    return _vals(spec, key, idx, spec.sigma_x, spec.act).reshape(count, spec.H)


def expert_dense(spec: LayerSpec, e: int, which: str) -> np.ndarray:
    """Unquantised weights of one expert: gate/up [I][H], down [H][I] (fp32 or bf16 bits)."""
    tag = {"gate": TAG_GATE, "up": TAG_UP, "down": TAG_DOWN}[which]
    key = stream_key(spec.weight_seed, tag)
    n = spec.I * spec.H
    idx = np.arange(e * n, (e + 1) * n, dtype=np.uint64)
    dt = DT_F32 if spec.expert == DT_F32 else DT_BF16
    v = _vals(spec, key, idx, spec.sigma_w, dt)
    return v.reshape((spec.I, spec.H) if which != "down" else (spec.H, spec.I))


def expert_stored(spec: LayerSpec, e: int, which: str):
    """One expert's matrix in the layer's storage format.

    Returns ``("f32", array)``, ``("bf16", uint16 bits)`` or
    ``("q4", (packed u8 [rows][K/2], fp16 scale bits [rows][K/32]))``.
    """
    dense = expert_dense(spec, e, which)
    if spec.expert == DT_F32:
        return ("f32", dense)
    if spec.expert == DT_BF16:
        return ("bf16", dense)
    return ("q4", quantize_q4_rows(dense))


def pool_bytes(spec: LayerSpec) -> int:
    n = 3 * spec.E * spec.I * spec.H
    if spec.expert == DT_F32:
        return 4 * n
    if spec.expert == DT_BF16:
        return 2 * n
    return n // 2 + 2 * (n // 32)
