"""Float64 CPU oracle of one sparse MoE layer (test infrastructure only).

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  It shares no code with the HIP
path, and nothing in the product path may call it.

What it computes, per token (each step follows the pages; where the pages
are silent the reading is stated):

1. Router logits ``z_e = sum_h x_h R[h, e] + b_e`` over all E experts.  The
   pages: the engine's routing kernel picks ten of the 24,576 experts for
   every token (pyshine source tour, Understanding the Architecture, the
   paragraph on the residency tiers and the end-to-end paragraph).  Reading: ``z`` is the exact real value (inputs are
   dyadic rationals) rounded once to f64.  A numpy f64 matmul gives every
   logit to within a proved bound; every expert that could still be in the
   top k under that bound is recomputed with ``math.fsum`` (exact, correctly
   rounded), so the values that decide the selection are the correctly
   rounded ones.
2. Selection: the first k experts of the order (z descending, expert index
   ascending) -- ties go to the lower index.
3. Gates: softmax over the k selected logits (equal to a full softmax
   renormalised over the selected experts).
4. Each selected expert is a SwiGLU MLP without biases:
   ``h = silu(G x) * (U x)``, ``y = D h``, ``silu(a) = a / (1 + exp(-a))``.
5. Combine: ``out = sum_j g_j y_j`` in selection order.  The router weight is
   applied here and only here (pyshine source tour, Understanding the
   Architecture, paragraph on the expert hand-off: the expert side leaves the
   router weight to the device-side combine, which does the weighted sum).

The pages' own float64 parity reference for the decode GEMV (hexlives
dispatch, the archived tensor-core benchmark) is the precedent for checking
the GPU path against f64.

Storage decoding (done here, independently of any encoder):
* bf16 bits -> value: the 16 bits are the top half of an IEEE binary32;
* 4-bit blocks: ``w = (nibble - 8) * d`` with ``d`` the block's fp16 scale,
  low nibble = even element; exact in f64.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# --------------------------------------------------------------- decoding
def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def decode_f16(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_q4(packed, scales) -> np.ndarray:
    """4-bit symmetric blocks -> float64 [rows][K].

    ``packed`` is uint8 [rows][K/2] (low nibble = element 2j, high = 2j+1),
    ``scales`` uint16 fp16 bits [rows][K/32]; w = (nibble - 8) * scale.
    """
    p = np.asarray(packed, dtype=np.uint8)
    rows, half = p.shape
    K = 2 * half
    q = np.empty((rows, K), dtype=np.int64)
    q[:, 0::2] = (p & 0x0F).astype(np.int64) - 8
    q[:, 1::2] = (p >> 4).astype(np.int64) - 8
    d = decode_f16(scales)
    assert d.shape == (rows, K // 32)
    return (q.reshape(rows, K // 32, 32) * d[:, :, None]).reshape(rows, K)


def decode_stored(stored) -> np.ndarray:
    kind, payload = stored
    if kind == "f32":
        return decode_f32(payload)
    if kind == "bf16":
        return decode_bf16(payload)
    if kind == "q4":
        return decode_q4(*payload)
    raise ValueError(kind)


# ---------------------------------------------------------------- the layer
class OracleLayer:
    """A layer held as float64 values.

    ``router``: R as the H x E matrix (float64).
    ``bias``:   b [E] float64 (zeros when the layer has none).
    ``expert_fn(e, which)``: the stored matrix of expert e ("gate", "up" or
    "down") as ``(kind, payload)``; decoded here and cached.
    """

    def __init__(self, router_he: np.ndarray, bias: np.ndarray, k: int, expert_fn,
                 cache_size: int = 256):
        self.R = np.ascontiguousarray(router_he, dtype=np.float64)
        self.H, self.E = self.R.shape
        self.b = np.asarray(bias, dtype=np.float64).reshape(self.E)
        self.k = int(k)
        if not (1 <= self.k <= self.E):
            raise ValueError("k must be in [1, E]")
        self._expert_fn = expert_fn
        self._cache: dict[int, tuple] = {}
        self._cache_size = cache_size
        self._absR = None

    def absR(self) -> np.ndarray:
        if self._absR is None:
            self._absR = np.abs(self.R)
        return self._absR

    def expert(self, e: int):
        """(G [I][H], U [I][H], D [H][I]) of expert e in float64."""
        e = int(e)
        hit = self._cache.get(e)
        if hit is not None:
            return hit
        G = decode_stored(self._expert_fn(e, "gate"))
        U = decode_stored(self._expert_fn(e, "up"))
        D = decode_stored(self._expert_fn(e, "down"))
        if len(self._cache) >= self._cache_size:
            self._cache.pop(next(iter(self._cache)))
        self._cache[e] = (G, U, D)
        return G, U, D


# --------------------------------------------------------------- step 1: logits
U64 = 2.0 ** -53            # unit roundoff of binary64


def gamma(n: int) -> float:
    """gamma_n = n u / (1 - n u), the classical bound for n roundings."""
    return n * U64 / (1.0 - n * U64)


def exact_logit(x: np.ndarray, R: np.ndarray, b: np.ndarray, e: int) -> float:
    """Correctly rounded f64 of sum_h x_h R[h,e] + b_e.

    Every product of two bf16 or two fp32 values is exact in f64, and
    ``math.fsum`` returns the correctly rounded sum of its (exact) terms.
    """
    terms = (x * R[:, e]).tolist()
    terms.append(float(b[e]))
    return math.fsum(terms)


def logits_with_bound(X: np.ndarray, layer: OracleLayer):
    """f64 logits for tokens X [T][H] and a per-entry bound on their error.

    Any summation order of H products (the matmul's) plus one bias addition
    has error at most gamma_{H+1} * (sum_h |x_h R_he| + |b_e|); the |.| sum is
    itself computed in f64, so the bound is doubled.
    """
    X = np.atleast_2d(X)
    Z = X @ layer.R + layer.b[None, :]
    A = np.abs(X) @ layer.absR() + np.abs(layer.b)[None, :]
    B = 2.0 * gamma(layer.H + 2) * A + 1e-300
    return Z, B


# ---------------------------------------------------------- step 2: selection
def select_topk(values: np.ndarray, experts: np.ndarray, k: int):
    """First k of (value descending, expert ascending).  Returns positions."""
    order = np.lexsort((experts, -values))
    return order[:k]


def route_token(x: np.ndarray, z_blas: np.ndarray, bound: np.ndarray, layer: OracleLayer):
    """Exact top-k of one token.  Returns (idx int64 [k], z f64 [k]).

    Lower bound on the k-th largest true logit: L = k-th largest (z - B).
    Experts with z + B < L have at least k experts strictly above them and
    cannot be selected; all others are recomputed exactly and ranked.
    """
    k = layer.k
    lo = z_blas - bound
    L = np.partition(lo, layer.E - k)[layer.E - k]        # k-th largest lower bound
    cand = np.nonzero(z_blas + bound >= L)[0]
    zc = np.array([exact_logit(x, layer.R, layer.b, int(e)) for e in cand], dtype=np.float64)
    pos = select_topk(zc, cand, k)
    return cand[pos].astype(np.int64), zc[pos]


# -------------------------------------------------------------- step 3: gates
def softmax_gates(zsel: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits (largest first)."""
    zsel = np.asarray(zsel, dtype=np.float64)
    m = zsel.max()
    w = np.exp(zsel - m)
    return w / w.sum()


# ------------------------------------------------------------- step 4: experts
def silu(a: np.ndarray) -> np.ndarray:
    """a * sigmoid(a), evaluated without overflow for either sign."""
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    pos = a >= 0
    out[pos] = a[pos] / (1.0 + np.exp(-a[pos]))
    ea = np.exp(a[~pos])
    out[~pos] = a[~pos] * ea / (1.0 + ea)
    return out


def expert_swiglu(G: np.ndarray, U: np.ndarray, D: np.ndarray, x: np.ndarray):
    """y = D (silu(G x) * (U x)); returns (y, h)."""
    h = silu(G @ x) * (U @ x)
    return D @ h, h


# ------------------------------------------------------------- step 5: combine
def combine(ys, gates) -> np.ndarray:
    out = np.zeros_like(ys[0])
    for g, y in zip(gates, ys):
        out = out + g * y
    return out


# ------------------------------------------------------------------ drivers
def moe_given(x: np.ndarray, layer: OracleLayer, idx, gates) -> np.ndarray:
    """Layer output for caller-given experts and gates (no routing)."""
    x = np.asarray(x, dtype=np.float64)
    ys = []
    for e in idx:
        G, U, D = layer.expert(int(e))
        ys.append(expert_swiglu(G, U, D, x)[0])
    return combine(ys, np.asarray(gates, dtype=np.float64))


def moe_tokens(X: np.ndarray, layer: OracleLayer, with_output: bool = True):
    """Route and evaluate tokens X [T][H] independently.

    Returns (idx int64 [T][k], gates f64 [T][k], zsel f64 [T][k],
    out f64 [T][H] or None).
    """
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    T = X.shape[0]
    Z, B = logits_with_bound(X, layer)
    idx = np.empty((T, layer.k), dtype=np.int64)
    zs = np.empty((T, layer.k), dtype=np.float64)
    gts = np.empty((T, layer.k), dtype=np.float64)
    out = np.empty((T, layer.H), dtype=np.float64) if with_output else None
    for t in range(T):
        idx[t], zs[t] = route_token(X[t], Z[t], B[t], layer)
        gts[t] = softmax_gates(zs[t])
        if with_output:
            out[t] = moe_given(X[t], layer, idx[t], gts[t])
    return idx, gts, zs, out


# ------------------------------------------------- plain definitions (for pins)
def exact_logits_fraction(x: np.ndarray, R: np.ndarray, b: np.ndarray):
    """All logits as exact rationals (tiny shapes only)."""
    H, E = R.shape
    xf = [Fraction(float(v)) for v in x]
    out = []
    for e in range(E):
        s = Fraction(float(b[e]))
        for h in range(H):
            s += xf[h] * Fraction(float(R[h, e]))
        out.append(s)
    return out


def brute_force_topk(values, k: int):
    """Selected experts by explicit rank counting (O(E^2)), in rank order.

    rank_e = #{e' : v_e' > v_e or (v_e' == v_e and e' < e)}; e is selected iff
    rank_e < k.  Works on any totally ordered values (floats or Fractions).
    """
    E = len(values)
    ranks = []
    for e in range(E):
        r = 0
        for f in range(E):
            if values[f] > values[e] or (values[f] == values[e] and f < e):
                r += 1
        ranks.append(r)
    sel = sorted((r, e) for e, r in enumerate(ranks) if r < k)
    return [e for _, e in sel]
