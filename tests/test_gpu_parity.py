"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Indices bit-exact (ordered), gates within 1e-6, outputs within a relative
L2 error of 1e-3 per token.  Small layers span several router blocks and
ragged tails; the full-size workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest

import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_f32": synth.CONFIGS["tiny_f32"],
    "tiny_bf16": synth.small_spec(H=256, E=200, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_BF16,
                                  bias_alpha=0.37, weight_seed=21, token_seed=22, name="tiny_bf16"),
    "tiny_q4": synth.small_spec(H=256, E=200, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=23, token_seed=24, name="tiny_q4"),
    "wide_q4": synth.small_spec(H=2048, E=130, k=10, I=256, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=25, token_seed=26, name="wide_q4"),
    "odd_q4": synth.small_spec(H=96, E=70, k=3, I=32, act=synth.DT_BF16, expert=synth.DT_Q4,
                               bias_alpha=None, weight_seed=27, token_seed=28, name="odd_q4"),
    "f32_bf16x": synth.small_spec(H=136, E=65, k=5, I=40, act=synth.DT_F32, expert=synth.DT_BF16,
                                  bias_alpha=0.37, weight_seed=29, token_seed=30, name="f32_bf16x"),
}

_cache = {}


def setup(name):
    if name not in _cache:
        import synth.device as SD
        spec = SMALL[name]
        dl = SD.device_layer(spec)
        _cache[name] = (spec, dl, G.host_oracle(spec))
    return _cache[name]


def test_device_generator_matches_host():
    """Device fill == host generator, bit for bit (every format)."""
    torch = G.torch_mod()
    import synth.device as SD
    for name in ["tiny_f32", "tiny_bf16", "tiny_q4", "odd_q4"]:
        G.note("generator", name)
        spec, dl, _ = setup(name)
        assert np.array_equal(SD.to_numpy_bits(dl.router_eh), synth.router_eh(spec))
        for e in [0, 1, spec.E - 1]:
            for which, t, s in [("gate", dl.w_gate, dl.s_gate), ("up", dl.w_up, dl.s_up),
                                ("down", dl.w_down, dl.s_down)]:
                kind, payload = synth.expert_stored(spec, e, which)
                if kind == "q4":
                    assert np.array_equal(SD.to_numpy_bits(t[e]), payload[0]), (name, e, which)
                    assert np.array_equal(SD.to_numpy_bits(s[e]), payload[1]), (name, e, which)
                else:
                    assert np.array_equal(SD.to_numpy_bits(t[e]), payload), (name, e, which)
        x = SD.device_tokens(spec, 3, 5)
        assert np.array_equal(SD.to_numpy_bits(x), synth.tokens(spec, 3, 5))
    torch.cuda.synchronize()


def test_device_generator_fullsize_rows():
    """Rows of the full-size pools, generated on device by counter offset."""
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.CONFIGS["decode_q4"]
    for e in [0, 7777, spec.E - 1]:
        for which, tag, rows, K in [("gate", synth.TAG_GATE, spec.I, spec.H),
                                    ("down", synth.TAG_DOWN, spec.H, spec.I)]:
            G.note("fullsize rows", e, which)
            codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
            sc = torch.empty((rows, K // 32), dtype=torch.int16, device="cuda")
            SD.fill_q4(codes, sc, synth.stream_key(spec.weight_seed, tag), e * rows, K, spec.sigma_w)
            kind, (hq, hs) = synth.expert_stored(spec, e, which)
            assert np.array_equal(SD.to_numpy_bits(codes), hq)
            assert np.array_equal(SD.to_numpy_bits(sc), hs)
            dense = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
            SD.fill_values(dense, synth.stream_key(spec.weight_seed, tag), e * rows * K, spec.sigma_w)
            assert np.array_equal(SD.to_numpy_bits(dense), synth.expert_dense(spec, e, which))


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("layout", ["EH", "HE"])
def test_decode_parity_small(name, layout):
    import synth.device as SD
    spec, dl, L = setup(name)
    G.note("decode", name, layout)
    layer = SD.make_layer(dl, max_tokens=48, router_layout=layout)
    x = SD.device_tokens(spec, 0, 48)
    idx, gates, out = G.run_route_decode(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 0, 48)
    r = G.compare(idx, gates, out, o_idx, o_g, o_out, f"{name}/{layout}")
    print(f"{name}/{layout}: rel L2 max {r.max():.2e} median {np.median(r):.2e}")
    assert layer.device_error() == 0


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_q4", "wide_q4", "f32_bf16x"])
def test_forced_exact_refinement(name):
    """The integer-accumulator refinement gives the same routing."""
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_FORCE_EXACT_REFINE
    spec, dl, L = setup(name)
    G.note("forced exact", name)
    layer = SD.make_layer(dl, max_tokens=16, flags=MOE_LAYER_FORCE_EXACT_REFINE)
    x = SD.device_tokens(spec, 100, 16)
    idx, gates, out = G.run_route_decode(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 100, 16)
    G.compare(idx, gates, out, o_idx, o_g, o_out, name)
    assert layer.device_error() == 0


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16", "tiny_q4", "wide_q4", "odd_q4", "f32_bf16x"])
@pytest.mark.parametrize("T", [2, 5, 37])
def test_grouped_parity_small(name, T):
    import synth.device as SD
    spec, dl, L = setup(name)
    G.note("grouped", name, T)
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(spec, 200, T)
    idx, gates, out = G.run_grouped(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 200, T)
    G.compare(idx, gates, out, o_idx, o_g, o_out, f"{name}/T={T}")
    assert layer.device_error() == 0


# Batch-1 4-bit decode through moe_grouped_forward: the selection runs inside
# every gate/up block.  fp32 activations, H = 4096 (two quant blocks per lane)
# and the odd shapes of the small layers above.
FUSED_SPECS = {
    "q4_f32x": synth.small_spec(H=256, E=150, k=6, I=96, act=synth.DT_F32, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=81, token_seed=82, name="q4_f32x"),
    "q4_h4096": synth.small_spec(H=4096, E=70, k=8, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                                 bias_alpha=0.37, weight_seed=83, token_seed=84, name="q4_h4096"),
}
SMALL.update(FUSED_SPECS)


@pytest.mark.parametrize("name", ["tiny_q4", "wide_q4", "odd_q4", "q4_f32x", "q4_h4096", "tiny_bf16", "tiny_f32",
                                  "f32_bf16x"])
@pytest.mark.parametrize("exact", [False, True])
def test_fused_decode_single_token(name, exact):
    """moe_grouped_forward at T = 1 against the oracle, and bitwise against
    moe_route + moe_expert_decode on the same tokens one at a time (with
    exact refinement forced, every block runs the exact path)."""
    import torch
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_FORCE_EXACT_REFINE
    spec, dl, L = setup(name)
    G.note("fused decode", name, "exact" if exact else "")
    n = 8 if exact else 24
    layer = SD.make_layer(dl, max_tokens=n, flags=MOE_LAYER_FORCE_EXACT_REFINE if exact else 0)
    x = SD.device_tokens(spec, 300, n)
    rows = [G.run_grouped(layer, x[t:t + 1]) for t in range(n)]
    idx = np.concatenate([r[0] for r in rows])
    gates = np.concatenate([r[1] for r in rows])
    out = np.concatenate([r[2] for r in rows])
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 300, n)
    r = G.compare(idx, gates, out, o_idx, o_g, o_out, f"fused {name}")
    # the reference runs the same router kernel (T = 1): gates are computed
    # from the router's logits, which differ in the last bits between kernels
    srows = [G.run_route_decode(layer, x[t:t + 1]) for t in range(n)]
    s_idx = np.concatenate([r[0] for r in srows])
    s_g = np.concatenate([r[1] for r in srows])
    s_out = np.concatenate([r[2] for r in srows])
    assert np.array_equal(idx, s_idx)
    assert np.array_equal(gates.view(np.uint32), s_g.view(np.uint32))
    assert np.array_equal(out.view(np.uint32), s_out.view(np.uint32))
    print(f"fused {name}: rel L2 max {r.max():.2e}")
    assert layer.device_error() == 0


@pytest.mark.parametrize("name", ["tiny_q4", "odd_q4", "q4_f32x", "q4_h4096"])
@pytest.mark.parametrize("T", [2, 3, 8])
def test_window_internal_routing_matches_given_routing(name, T):
    """Windows of T tokens against the oracle, and bitwise against
    moe_route + moe_grouped_forward with the given routing."""
    import torch
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_ROUTE_GIVEN
    spec, dl, L = setup(name)
    G.note("window routing", name, T)
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(spec, 500, T)
    idx, gates, out = G.run_grouped(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 500, T)
    G.compare(idx, gates, out, o_idx, o_g, o_out, f"window {name} T={T}")
    ws = layer.workspace(T)
    si = torch.empty((T, spec.k), dtype=torch.int32, device=x.device)
    sg = torch.empty((T, spec.k), dtype=torch.float32, device=x.device)
    layer.route(x, T, si, sg, ws)
    s_idx, s_g, s_out = G.run_grouped(layer, x, flags=MOE_ROUTE_GIVEN, idx=si, gates=sg)
    assert np.array_equal(idx, s_idx)
    assert np.array_equal(gates.view(np.uint32), s_g.view(np.uint32))
    assert np.array_equal(out.view(np.uint32), s_out.view(np.uint32))
    assert layer.device_error() == 0


# Grouped MFMA path (bf16 activations and experts, T >= 16): few experts and
# many tokens, so segments span several 32-row tiles with a ragged last one;
# I = 96 and H = 160 leave partial 128-wide channel / output blocks.
MFMA_SPECS = {
    "mfma_multi_tile": synth.small_spec(H=512, E=20, k=4, I=128, act=synth.DT_BF16, expert=synth.DT_BF16,
                                        bias_alpha=0.37, weight_seed=71, token_seed=72, name="mfma_multi_tile"),
    "mfma_ragged": synth.small_spec(H=160, E=37, k=3, I=96, act=synth.DT_BF16, expert=synth.DT_BF16,
                                    bias_alpha=None, weight_seed=73, token_seed=74, name="mfma_ragged"),
    "mfma_wide": synth.small_spec(H=2048, E=300, k=10, I=256, act=synth.DT_BF16, expert=synth.DT_BF16,
                                  bias_alpha=0.37, weight_seed=75, token_seed=76, name="mfma_wide"),
}


@pytest.mark.parametrize("name,T", [("mfma_multi_tile", 300), ("mfma_ragged", 77), ("mfma_wide", 64),
                                    ("mfma_wide", 16), ("mfma_multi_tile", 600), ("mfma_ragged", 530),
                                    ("mfma_multi_tile", 200), ("mfma_wide", 512)])
def test_grouped_mfma_tiles(name, T):
    """Experts with more than 32 tokens go to 64-row tiles (both grouping
    kernels: 800 pairs and more than 1024); T >= 512 also takes the 256 x 256
    router tiles (fp32 accumulation over H) with one expert tile (E = 20, 37)
    and ragged token tiles, or two expert tiles of which the second is
    partial (E = 300, not a multiple of 16, so every tile takes the masked
    epilogue)."""
    import synth.device as SD
    spec = MFMA_SPECS[name]
    G.note("grouped mfma", name, T)
    dl = SD.device_layer(spec)
    L = G.host_oracle(spec)
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(spec, 3, T)
    idx, gates, out = G.run_grouped(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 3, T)
    r = G.compare(idx, gates, out, o_idx, o_g, o_out, f"{name}/T={T}")
    counts = np.bincount(o_idx.ravel(), minlength=spec.E)
    print(f"{name} T={T}: max tokens per expert {counts.max()}, rel L2 max {r.max():.2e}")
    assert layer.device_error() == 0


@pytest.mark.parametrize("name,T", [("tiny_q4", 300), ("tiny_q4", 256), ("odd_q4", 15), ("wide_q4", 10),
                                    ("wide_q4", 25)])
def test_grouped_pair_sort_paths(name, T):
    """P = T k above and at the one-workgroup sort limit (1024 pairs): the
    histogram / scan / scatter sort and the one-block rank sort; at most 256
    pairs go to the deduplicating pair kernels, with h staged in LDS (odd_q4)
    or read from global memory (wide_q4, 100 and 250 pairs over 130 experts,
    so experts repeat across tokens)."""
    import synth.device as SD
    spec, dl, L = setup(name)
    G.note("grouped sort path", name, T)
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(spec, 500, T)
    idx, gates, out = G.run_grouped(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 500, T)
    G.compare(idx, gates, out, o_idx, o_g, o_out, f"{name}/T={T}")
    assert layer.device_error() == 0


@pytest.mark.parametrize("name,T", [("mfma_multi_tile", 7), ("mfma_ragged", 9), ("mfma_wide", 2)])
def test_few_token_router_shapes(name, T):
    """The 16x16 MFMA router at 2 <= T < 16: H = 512 and H = 2048 (row
    quarters transposed through LDS) and H = 160 (generic operand loads),
    with E not a multiple of the 16-expert tile."""
    import synth.device as SD
    spec = MFMA_SPECS[name]
    G.note("few-token router", name, T)
    dl = SD.device_layer(spec)
    L = G.host_oracle(spec)
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(spec, 40, T)
    idx, gates, out = G.run_grouped(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 40, T)
    G.compare(idx, gates, out, o_idx, o_g, o_out, f"{name}/T={T}")
    idx2, gates2, out2 = G.run_route_decode(layer, x)
    G.compare(idx2, gates2, out2, o_idx, o_g, o_out, f"{name}/T={T} route+decode")
    assert layer.device_error() == 0
