"""The host tier's pool (moe_cpu_experts) on the host, no GPU: its outputs
against the float64 oracle for given experts and gates, for 4-bit, bf16 and
fp32 experts; indices outside [0, E) add nothing; any thread count gives
the same bits."""
import numpy as np
import pytest

import oracle
import synth

SPECS = {
    "q4": synth.small_spec(H=256, E=12, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                           bias_alpha=None, weight_seed=61, token_seed=62, name="pool_q4"),
    "q4_wide": synth.small_spec(H=2048, E=6, k=3, I=256, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=None, weight_seed=63, token_seed=64, name="pool_q4_wide"),
    "bf16": synth.small_spec(H=256, E=12, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_BF16,
                             bias_alpha=None, weight_seed=65, token_seed=66, name="pool_bf16"),
    "f32": synth.small_spec(H=96, E=10, k=2, I=40, act=synth.DT_F32, expert=synth.DT_F32,
                            bias_alpha=None, weight_seed=67, token_seed=68, name="pool_f32"),
}


def host_pools(spec):
    """The whole expert pool in the layer's storage layout (host arrays)."""
    out = {}
    for which, name in (("gate", "w_gate"), ("up", "w_up"), ("down", "w_down")):
        st = [synth.expert_stored(spec, e, which) for e in range(spec.E)]
        if st[0][0] == "q4":
            out[name] = np.ascontiguousarray(np.stack([p[1][0] for p in st]).astype(np.uint8))
            out["s" + name[1:]] = np.ascontiguousarray(np.stack([p[1][1] for p in st]).astype(np.uint16))
        elif st[0][0] == "bf16":
            out[name] = np.ascontiguousarray(np.stack([p[1] for p in st]).astype(np.uint16))
        else:
            out[name] = np.ascontiguousarray(np.stack([p[1] for p in st]).astype(np.float32))
    return out


def run_pool(spec, pools, X, idx, gates, n_threads):
    from expert_routing_quantized_amd import binding as B
    T = X.shape[0]
    out = np.full((T, spec.H), np.nan, dtype=np.float32)
    act = B.MOE_F32 if spec.act == synth.DT_F32 else B.MOE_BF16
    ex = {synth.DT_F32: B.MOE_F32, synth.DT_BF16: B.MOE_BF16, synth.DT_Q4: B.MOE_Q4B32}[spec.expert]
    B.cpu_experts(spec.H, spec.E, spec.k, spec.I, act, ex, pools["w_gate"], pools["w_up"], pools["w_down"],
                  np.ascontiguousarray(X), T, np.ascontiguousarray(idx, dtype=np.int32),
                  np.ascontiguousarray(gates, dtype=np.float32), out,
                  s_gate=pools.get("s_gate"), s_up=pools.get("s_up"), s_down=pools.get("s_down"),
                  n_threads=n_threads)
    return out


@pytest.mark.parametrize("name", list(SPECS))
def test_cpu_pool_against_oracle(name):
    spec = SPECS[name]
    pools = host_pools(spec)
    T = 6
    X = synth.tokens(spec, 3, T)
    rng = np.random.default_rng(7)
    idx = np.stack([rng.permutation(spec.E)[:spec.k] for _ in range(T)]).astype(np.int32)
    g = rng.random((T, spec.k)) + 0.1
    gates = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    out = run_pool(spec, pools, X, idx, gates, n_threads=3)
    L = oracle.layer_from_spec(spec)
    Xf = oracle.tokens_f64(spec, 3, T)
    for t in range(T):
        ref = oracle.moe_given(Xf[t], L, idx[t], gates[t].astype(np.float64))
        r = np.linalg.norm(out[t] - ref) / np.linalg.norm(ref)
        assert r <= 1e-5, f"{name} token {t}: rel L2 {r}"
    # the same bits from one thread and from eight
    assert np.array_equal(out.view(np.uint32), run_pool(spec, pools, X, idx, gates, 1).view(np.uint32))
    assert np.array_equal(out.view(np.uint32), run_pool(spec, pools, X, idx, gates, 8).view(np.uint32))


def test_cpu_pool_skips_indices_out_of_range():
    spec = SPECS["q4"]
    pools = host_pools(spec)
    X = synth.tokens(spec, 0, 2)
    idx = np.array([[0, 5, -1, spec.E], [3, spec.E + 7, 1, -5]], dtype=np.int32)
    gates = np.full((2, spec.k), 0.25, dtype=np.float32)
    out = run_pool(spec, pools, X, idx, gates, 2)
    L = oracle.layer_from_spec(spec)
    Xf = oracle.tokens_f64(spec, 0, 2)
    for t, keep in ((0, [0, 5]), (1, [3, 1])):
        ref = oracle.moe_given(Xf[t], L, keep, [0.25, 0.25])
        assert np.linalg.norm(out[t] - ref) / np.linalg.norm(ref) <= 1e-5
    none = run_pool(spec, pools, X, np.full((2, spec.k), -1, dtype=np.int32), gates, 2)
    assert np.all(none == 0.0)


def test_cpu_pool_refusals():
    from expert_routing_quantized_amd import binding as B
    spec = SPECS["q4"]
    pools = host_pools(spec)
    X = synth.tokens(spec, 0, 1)
    out = np.zeros((1, spec.H), dtype=np.float32)
    idx = np.zeros((1, spec.k), dtype=np.int32)
    gates = np.zeros((1, spec.k), dtype=np.float32)
    with pytest.raises(B.MoeError) as e:      # 4-bit experts without scales
        B.cpu_experts(spec.H, spec.E, spec.k, spec.I, B.MOE_BF16, B.MOE_Q4B32, pools["w_gate"], pools["w_up"],
                      pools["w_down"], X, 1, idx, gates, out)
    assert e.value.status == -1
    with pytest.raises(B.MoeError) as e:      # H not a multiple of 32
        B.cpu_experts(100, spec.E, spec.k, spec.I, B.MOE_BF16, B.MOE_Q4B32, pools["w_gate"], pools["w_up"],
                      pools["w_down"], X, 1, idx, gates, out, s_gate=pools["s_gate"], s_up=pools["s_up"],
                      s_down=pools["s_down"])
    assert e.value.status == -2
