"""Edge cases of the selection and of the boundary on the GPU: degenerate
ties (every logit equal), k above the wave count, k = 1, k = E, more
survivors than fit in LDS, and a non-finite hidden state."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def run_case(spec, T, first=0):
    import synth.device as SD
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(spec, first, T)
    L = oracle.layer_from_spec(spec)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, first, T)
    idx, gates, out = G.run_route_decode(layer, x)
    G.compare(idx, gates, out, o_idx, o_g, o_out, spec.name + "/decode")
    idx2, gates2, out2 = G.run_grouped(layer, x)
    G.compare(idx2, gates2, out2, o_idx, o_g, o_out, spec.name + "/grouped")
    assert layer.device_error() == 0
    return dl, layer


def test_all_logits_equal_many_experts():
    """x = 0 and no bias: 3000 equal logits -> experts 0..k-1, gates 1/k, out 0
    (more survivors than the selection keeps in LDS: bisection path)."""
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.small_spec(H=256, E=3000, k=6, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                            bias_alpha=None, weight_seed=51, token_seed=52, name="equal")
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=2)
    x = torch.zeros((2, spec.H), dtype=torch.bfloat16, device="cuda")
    idx, gates, out = G.run_route_decode(layer, x)
    assert np.array_equal(idx, np.tile(np.arange(spec.k), (2, 1)))
    assert np.all(gates == np.float32(1.0 / spec.k))
    assert np.all(out == 0.0)
    assert layer.device_error() == 0


def test_k_above_wave_count():
    spec = synth.small_spec(H=512, E=3000, k=20, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                            bias_alpha=0.37, weight_seed=53, token_seed=54, name="k20")
    run_case(spec, 6)


@pytest.mark.parametrize("k,E", [(1, 500), (8, 8), (16, 2048)])
def test_k_extremes(k, E):
    spec = synth.small_spec(H=256, E=E, k=k, I=32, act=synth.DT_BF16, expert=synth.DT_BF16,
                            bias_alpha=0.37, weight_seed=55 + k, token_seed=56, name=f"k{k}E{E}")
    dl, layer = run_case(spec, 5)
    if k == 1:
        torch = G.torch_mod()
        import synth.device as SD
        x = SD.device_tokens(spec, 0, 5)
        _, gates, _ = G.run_route_decode(layer, x)
        assert np.all(gates == 1.0)


def test_single_survivor_ranges_of_a_large_pool():
    """E = 40,000 (two chunks of the selection's register tile)."""
    spec = synth.small_spec(H=256, E=40000, k=10, I=32, act=synth.DT_BF16, expert=synth.DT_Q4,
                            bias_alpha=0.37, weight_seed=61, token_seed=62, name="E40k")
    run_case(spec, 3)


def test_nan_hidden_state_sets_the_flag():
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.small_spec(H=256, E=300, k=4, I=32, act=synth.DT_BF16, expert=synth.DT_BF16,
                            bias_alpha=0.37, weight_seed=63, token_seed=64, name="nan")
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=3)
    x = SD.device_tokens(spec, 0, 3)
    x[1, 17] = float("nan")
    idx, gates, out = G.run_route_decode(layer, x)
    assert layer.device_error() & 4
    assert np.all(idx[1] == -1) and np.all(np.isnan(gates[1])) and np.all(np.isnan(out[1]))
    L = oracle.layer_from_spec(spec)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 0, 3)
    G.compare(idx[[0, 2]], gates[[0, 2]], out[[0, 2]], o_idx[[0, 2]], o_g[[0, 2]], o_out[[0, 2]], "nan/others")


def test_large_pool_sorted_grouping():
    """E = 40,000 with 1200 pairs: the sorted grouping path (histogram, scan
    over more experts than the scan keeps in registers, scatter)."""
    spec = synth.small_spec(H=256, E=40000, k=10, I=32, act=synth.DT_BF16, expert=synth.DT_Q4,
                            bias_alpha=0.37, weight_seed=65, token_seed=66, name="E40k_sorted")
    import synth.device as SD
    dl = SD.device_layer(spec)
    T = 120
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(spec, 0, T)
    L = oracle.layer_from_spec(spec)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 0, T)
    idx, gates, out = G.run_grouped(layer, x)
    G.compare(idx, gates, out, o_idx, o_g, o_out, "E40k/sorted")
    assert layer.device_error() == 0
