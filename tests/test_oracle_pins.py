"""Pins of the float64 oracle against things other than itself.

Each test ties one part of the oracle to a definition, a closed form, an
invariant, brute force, or a hand-derived example, so that a plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, a
wrong tie rule) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_layer(R_he, b, k, experts):
    """OracleLayer over in-memory fp32 matrices {e: (G, U, D)}."""
    def fn(e, which):
        G, U, D = experts[e]
        return ("f32", np.asarray({"gate": G, "up": U, "down": D}[which], dtype=np.float32))
    return oracle.OracleLayer(np.asarray(R_he, np.float64), np.asarray(b, np.float64), k, fn)


def random_tiny(seed, H=12, E=16, I=4, k=3, dtype=synth.DT_F32, bias=True):
    spec = synth.small_spec(H=H, E=E, k=k, I=I, act=dtype,
                            expert=dtype if dtype != synth.DT_F32 else synth.DT_F32,
                            bias_alpha=0.37 if bias else None, weight_seed=seed, token_seed=seed + 1)
    L = oracle.layer_from_spec(spec)
    x = oracle.tokens_f64(spec, 0, 1)[0]
    return spec, L, x


# ------------------------------------------------------------ storage decode
def test_decode_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    v = oracle.decode_bf16(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 1.0 + 2.0 ** -7
    assert v[3] == 2.0 ** -133 and v[4] == 0.0 and math.copysign(1, v[4]) < 0
    assert v[5] == 3.140625


def test_decode_q4_by_hand():
    # one row, K=64: block 0 scale 1.0, block 1 scale 0.5
    packed = np.full((1, 32), 0x88, dtype=np.uint8)          # all q = 0
    packed[0, 0] = 0x9F      # element 0: nibble 15 -> +7 ; element 1: nibble 9 -> +1
    packed[0, 16] = 0x01     # element 32: nibble 1 -> -7 ; element 33: nibble 0 -> -8
    scales = np.array([[0x3C00, 0x3800]], dtype=np.uint16)   # fp16 1.0, 0.5
    w = oracle.decode_q4(packed, scales)
    assert w.shape == (1, 64)
    assert w[0, 0] == 7.0 and w[0, 1] == 1.0 and w[0, 2] == 0.0
    assert w[0, 32] == -3.5 and w[0, 33] == -4.0 and w[0, 34] == 0.0


def test_q4_codec_properties():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, size=(6, 128)).astype(np.float32)
    w[1, 32:64] = 0.0                                         # an all-zero block
    bits = synth.f32_to_bf16_bits(w)
    packed, scales = synth.quantize_q4_rows(bits)
    wq = oracle.decode_q4(packed, scales)
    d = oracle.decode_f16(scales)
    wf = oracle.decode_bf16(bits)
    # all-zero block -> scale 0 -> zeros
    assert d[1, 1] == 0.0 and np.all(wq[1, 32:64] == 0.0)
    # error at most half a step, and the amax element lands on +-7 d
    blocks = wf.reshape(6, 4, 32)
    err = np.abs(wq.reshape(6, 4, 32) - blocks)
    assert np.all(err <= 0.5 * d[:, :, None] * (1 + 1e-12) + 1e-300)
    am = np.argmax(np.abs(blocks), axis=2)
    for r in range(6):
        for b in range(4):
            if d[r, b] > 0:
                assert abs(wq.reshape(6, 4, 32)[r, b, am[r, b]]) == 7 * d[r, b]
    # every decoded value is an integer code in [-7, 7] times its block scale
    dd = np.repeat(d, 32, axis=1)
    q = np.divide(wq, dd, out=np.zeros_like(wq), where=dd > 0)
    assert np.array_equal(q, np.rint(q)) and np.abs(q).max() <= 7
    # repacking those codes reproduces the bytes (pack o unpack = identity)
    nib = (q + 8).astype(np.uint8)
    assert np.array_equal(nib[:, 0::2] | (nib[:, 1::2] << 4), packed)


# ------------------------------------------------------------ P1: logits
@pytest.mark.parametrize("dtype", [synth.DT_F32, synth.DT_BF16])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_exact_logits_match_rationals(dtype, seed):
    spec, L, x = random_tiny(seed, dtype=dtype)
    exact = oracle.exact_logits_fraction(x, L.R, L.b)
    Z, B = oracle.logits_with_bound(x[None, :], L)
    for e in range(L.E):
        assert oracle.exact_logit(x, L.R, L.b, e) == float(exact[e])   # correctly rounded
        assert abs(Fraction(float(Z[0, e])) - exact[e]) <= Fraction(float(B[0, e]))


# ------------------------------------------------------------ P2: selection
@pytest.mark.parametrize("k", [1, 2, 5, 16])
@pytest.mark.parametrize("seed", [4, 5, 6])
def test_topk_equals_brute_force(k, seed):
    spec, L, x = random_tiny(seed, k=k, dtype=synth.DT_BF16)
    exact = [float(v) for v in oracle.exact_logits_fraction(x, L.R, L.b)]
    Z, B = oracle.logits_with_bound(x[None, :], L)
    idx, zs = oracle.route_token(x, Z[0], B[0], L)
    assert list(idx) == oracle.brute_force_topk(exact, k)
    assert list(zs) == [exact[e] for e in idx]
    if k == L.E:                                   # full order
        assert sorted(idx) == list(range(L.E))


def test_exact_ties_go_to_lower_index():
    H, E = 8, 6
    rng = np.random.default_rng(0)
    R = rng.normal(0, 1, size=(H, E)).astype(np.float32).astype(np.float64)
    R[:, 4] = R[:, 1]                    # expert 4 duplicates expert 1
    R[:, 5] = R[:, 1]
    R[:, 1] += 0.0
    b = np.zeros(E)
    b[[1, 4, 5]] = 10.0                  # make the three copies the top three
    experts = {e: (np.zeros((1, H)), np.zeros((1, H)), np.zeros((H, 1))) for e in range(E)}
    L = tiny_layer(R, b, 2, experts)
    x = rng.normal(0, 1, size=H).astype(np.float32).astype(np.float64)
    idx, gates, zs, _ = oracle.moe_tokens(x[None, :], L)
    assert list(idx[0]) == [1, 4]
    assert gates[0, 0] == gates[0, 1] == 0.5


def test_refinement_fixes_cancellation_order():
    """Huge cancelling terms hide a 2^-20 difference from a plain f64 sum.

    The exact logits order expert 1 above expert 0; a left-to-right f64 sum
    sees a tie (which would select the lower index, expert 0).
    """
    H = 3
    x = np.array([2.0 ** 40, 2.0 ** 40, 1.0])
    R = np.zeros((H, 3))
    R[:, 0] = [1.0, -1.0, 0.5]
    R[:, 1] = [1.0, -1.0, 0.5 + 2.0 ** -20]
    R[:, 2] = [0.0, 0.0, -1.0]
    experts = {e: (np.zeros((1, H)), np.zeros((1, H)), np.zeros((H, 1))) for e in range(3)}
    L = tiny_layer(R, np.zeros(3), 1, experts)
    naive = [sum(float(x[h] * R[h, e]) + 0.0 for h in [0, 2, 1]) for e in range(3)]
    assert naive[0] == naive[1]          # the plain sum (this order) loses the difference
    idx, _, zs, _ = oracle.moe_tokens(x[None, :], L)
    assert idx[0, 0] == 1 and zs[0, 0] == 0.5 + 2.0 ** -20


def test_sub_resolution_difference_is_a_tie():
    """Exact logits 2^-60 apart round to the same f64: the lower index wins."""
    H = 2
    x = np.array([1.0, 2.0 ** -40])
    R = np.zeros((H, 2))
    R[:, 0] = [1.0, 0.0]
    R[:, 1] = [1.0, 2.0 ** -20]
    experts = {e: (np.zeros((1, H)), np.zeros((1, H)), np.zeros((H, 1))) for e in range(2)}
    L = tiny_layer(R, np.zeros(2), 1, experts)
    idx, _, _, _ = oracle.moe_tokens(x[None, :], L)
    assert idx[0, 0] == 0


# ------------------------------------------------------------ P3: gates
def test_gate_closed_forms():
    z = np.array([1.25, -0.5])
    g = oracle.softmax_gates(z)
    s = 1.0 / (1.0 + math.exp(-(1.25 + 0.5)))
    assert abs(g[0] - s) < 1e-15 and abs(g[1] - (1 - s)) < 1e-15
    g = oracle.softmax_gates(np.full(7, 3.0))
    assert np.all(g == 1.0 / 7)
    rng = np.random.default_rng(1)
    zz = np.sort(rng.normal(size=10))[::-1]
    g = oracle.softmax_gates(zz)
    assert abs(g.sum() - 1.0) < 1e-15 and np.all(np.diff(g) <= 0)
    assert oracle.softmax_gates(np.array([4.0]))[0] == 1.0


# ------------------------------------------------------------ P4: expert MLP
def test_silu_points():
    a = np.array([0.0, 1.0, -1.0, 50.0, -800.0, 800.0])
    s = oracle.silu(a)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(s[2] - (-1.0 / (1.0 + math.exp(1.0)))) < 1e-16
    assert s[3] == 50.0 and s[4] == 0.0 and s[5] == 800.0


def test_single_expert_by_loops():
    rng = np.random.default_rng(2)
    H, I = 5, 3
    G, U, D = rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I))
    x = rng.normal(size=H)
    y, h = oracle.expert_swiglu(G, U, D, x)
    for i in range(I):
        a = sum(G[i, j] * x[j] for j in range(H))
        u = sum(U[i, j] * x[j] for j in range(H))
        assert abs(h[i] - a / (1 + math.exp(-a)) * u) < 1e-12
    for o in range(H):
        assert abs(y[o] - sum(D[o, i] * h[i] for i in range(I))) < 1e-12
    assert np.all(oracle.expert_swiglu(0 * G, U, D, x)[0] == 0)
    assert np.all(oracle.expert_swiglu(G, 0 * U, D, x)[0] == 0)


def test_scalar_layer_closed_form():
    # H = I = 1, E = 2, k = 1: out = D silu(G x) (U x) of the larger-logit expert, gate 1
    experts = {0: (np.array([[2.0]]), np.array([[3.0]]), np.array([[0.5]])),
               1: (np.array([[1.0]]), np.array([[1.0]]), np.array([[1.0]]))}
    L = tiny_layer(np.array([[0.25, 0.5]]), np.array([0.0, -0.5]), 1, experts)
    x = np.array([1.5])        # z = [0.375, 0.25]
    idx, g, zs, out = oracle.moe_tokens(x[None, :], L)
    a = 3.0
    assert idx[0, 0] == 0 and g[0, 0] == 1.0
    assert abs(out[0, 0] - 0.5 * a / (1 + math.exp(-a)) * 4.5) < 1e-15


# ------------------------------------------------------------ P5-P8: invariants
def small_spec_layer(seed=9, expert=synth.DT_BF16, k=4):
    spec = synth.small_spec(H=64, E=24, k=k, I=32, act=synth.DT_BF16, expert=expert,
                            bias_alpha=0.37, weight_seed=seed, token_seed=seed + 5)
    return spec, oracle.layer_from_spec(spec), oracle.tokens_f64(spec, 0, 6)


def test_linearity_in_gates():
    spec, L, X = small_spec_layer()
    idx, g, _, out = oracle.moe_tokens(X[:1], L)
    rng = np.random.default_rng(5)
    g2 = rng.uniform(0, 1, size=g.shape[1])
    o1 = oracle.moe_given(X[0], L, idx[0], g[0])
    assert np.allclose(o1, out[0], rtol=0, atol=0)
    o_a = oracle.moe_given(X[0], L, idx[0], 2.5 * g[0])
    assert np.allclose(o_a, 2.5 * o1, rtol=1e-14, atol=1e-18)
    o_sum = oracle.moe_given(X[0], L, idx[0], g[0] + g2)
    o2 = oracle.moe_given(X[0], L, idx[0], g2)
    assert np.allclose(o_sum, o1 + o2, rtol=1e-13, atol=1e-17)


def test_zeroing_unselected_experts_changes_nothing():
    spec, L, X = small_spec_layer()
    idx, g, _, out = oracle.moe_tokens(X, L)
    used = set(int(e) for e in idx.ravel())

    def fn(e, which):
        st = synth.expert_stored(spec, e, which)
        if e in used:
            return st
        return ("bf16", np.zeros_like(st[1]))
    L0 = oracle.OracleLayer(L.R, L.b, L.k, fn)
    idx0, g0, _, out0 = oracle.moe_tokens(X, L0)
    assert np.array_equal(idx0, idx) and np.array_equal(out0, out)


def test_relabelling_equivariance():
    spec, L, X = small_spec_layer(seed=13)
    idx, g, _, out = oracle.moe_tokens(X, L)
    rng = np.random.default_rng(8)
    pi = rng.permutation(L.E)              # old expert e becomes pi[e]
    inv = np.argsort(pi)
    Rp = np.empty_like(L.R)
    Rp[:, pi] = L.R
    bp = np.empty_like(L.b)
    bp[pi] = L.b
    Lp = oracle.OracleLayer(Rp, bp, L.k, lambda e, w: synth.expert_stored(spec, int(inv[e]), w))
    idxp, gp, _, outp = oracle.moe_tokens(X, Lp)
    assert np.array_equal(idxp, pi[idx]) and np.array_equal(gp, g) and np.array_equal(outp, out)


def test_batch_rows_equal_single_tokens():
    spec, L, X = small_spec_layer(seed=17, expert=synth.DT_Q4)
    idx, g, _, out = oracle.moe_tokens(X, L)
    for t in range(X.shape[0]):
        i1, g1, _, o1 = oracle.moe_tokens(X[t:t + 1], L)
        assert np.array_equal(i1[0], idx[t]) and np.array_equal(g1[0], g[t])
        assert np.array_equal(o1[0], out[t])


# ------------------------------------------------------------ golden example
def test_hand_example():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        ex = json.load(f)
    experts = {int(e): (np.array(v["gate"]), np.array(v["up"]), np.array(v["down"]))
               for e, v in ex["experts"].items()}
    L = tiny_layer(np.array(ex["router_he"]), np.array(ex["bias"]), ex["k"], experts)
    idx, g, zs, out = oracle.moe_tokens(np.array([ex["x"]]), L)
    assert list(idx[0]) == ex["expected_idx"] and list(zs[0]) == ex["expected_logits"]
    s05 = 1.0 / (1.0 + math.exp(-0.5))
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(g[0, 0] - s05) < 1e-15 and abs(g[0, 1] - (1 - s05)) < 1e-15
    h2, h0 = 2.0 * s1, 3.0 * s1
    want = [s05 * h2 + (1 - s05) * 0.5 * h0, -s05 * h2 + (1 - s05) * 2.0 * h0]
    assert np.allclose(out[0], want, rtol=1e-15, atol=0)


# ------------------------------------------------------------ generator pins
def test_splitmix64_published_outputs():
    # the first outputs of SplitMix64 started from state 0
    v = synth.raw64(0, np.arange(3, dtype=np.uint64))
    assert [int(a) for a in v] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_generator_moments_and_rounding():
    key = synth.stream_key(1, synth.TAG_GATE)
    s = synth.irwin_hall(key, np.arange(1 << 18, dtype=np.uint64))
    assert s.min() >= -131070 and s.max() <= 131070
    assert abs(s.mean()) < 3 * synth.IH_STD / 512
    assert abs(s.std() / synth.IH_STD - 1) < 0.01
    v = synth.normal_f32(key, np.arange(1 << 16, dtype=np.uint64), 0.02)
    assert abs(v.std() - 0.02) < 0.0005
    # bf16 rounding is nearest-even on the fp32 bits
    f = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert list(oracle.decode_bf16(synth.f32_to_bf16_bits(f))) == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7]


def test_bias_is_zipf_shaped():
    spec = synth.CONFIGS["decode_bf16"]
    b = synth.router_bias(spec).astype(np.float64)
    r = np.sort(-b)                       # = 0.37 ln(rank), ascending
    assert r[0] == 0.0 and np.allclose(r, 0.37 * np.log(np.arange(1, spec.E + 1)), atol=1e-6)
