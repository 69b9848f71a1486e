"""Random small layers against the oracle (hypothesis, a fixed sequence of
draws): hidden and intermediate sizes, pool size, top-k, dtype pairs, bias,
the router screen and the number of tokens per call are drawn from the
ranges the fixed-shape tests cover (H and I multiples of 32 up to 512, up to
300 experts, k up to 10, T from 1 to 40: batch 1, verify windows, the
few-token and the grouped MFMA paths).  Indices bit-exact, gates and outputs
within the tolerances."""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

DTYPES = [(synth.DT_F32, synth.DT_F32), (synth.DT_BF16, synth.DT_BF16), (synth.DT_BF16, synth.DT_Q4),
          (synth.DT_F32, synth.DT_BF16), (synth.DT_F32, synth.DT_Q4)]


@settings(max_examples=100, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(data=st.data())
def test_random_small_layers(data):
    G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_ON
    act, expert = data.draw(st.sampled_from(DTYPES), label="dtypes")
    H = 32 * data.draw(st.integers(3, 16), label="H/32")
    I = 32 * data.draw(st.integers(2, 8), label="I/32")
    E = data.draw(st.integers(2, 300), label="E")
    k = data.draw(st.integers(1, min(E, 10)), label="k")
    T = data.draw(st.sampled_from([1, 2, 3, 5, 8, 12, 20, 40]), label="T")
    bias = data.draw(st.sampled_from([None, 0.37]), label="bias")
    screen = act == synth.DT_BF16 and data.draw(st.booleans(), label="screen")
    seed = data.draw(st.integers(1, 10_000), label="seed")
    spec = synth.small_spec(H=H, E=E, k=k, I=I, act=act, expert=expert, bias_alpha=bias,
                            weight_seed=seed, token_seed=seed + 1, name="random")
    G.note("random layer", dict(H=H, I=I, E=E, k=k, T=T, act=act, expert=expert, bias=bias, screen=screen, seed=seed))
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=T, flags=MOE_LAYER_SCREEN_ON if screen else 0)
    x = SD.device_tokens(spec, 0, T)
    fi, fg, fo = G.run_grouped(layer, x)
    L = G.host_oracle(spec)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 0, T)
    G.compare(fi, fg, fo, o_idx, o_g, o_out, f"random H={H} I={I} E={E} k={k} T={T}")
    assert layer.device_error() == 0


@settings(max_examples=20, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(data=st.data())
def test_random_window_layers(data):
    """Verify windows through the int8 window screen at the hidden sizes it
    is built for (H = 1024 and 2048, its 16- and 32-slab kernels, every ring
    depth), 4-bit or bf16 experts, with and without bias."""
    G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_ON
    expert = data.draw(st.sampled_from([synth.DT_Q4, synth.DT_BF16]), label="expert")
    H = data.draw(st.sampled_from([1024, 2048]), label="H")
    I = 32 * data.draw(st.integers(2, 8), label="I/32")
    E = data.draw(st.integers(40, 600), label="E")
    k = data.draw(st.integers(1, 10), label="k")
    T = data.draw(st.integers(2, 8), label="T")
    bias = data.draw(st.sampled_from([None, 0.37]), label="bias")
    seed = data.draw(st.integers(1, 10_000), label="seed")
    spec = synth.small_spec(H=H, E=E, k=k, I=I, act=synth.DT_BF16, expert=expert, bias_alpha=bias,
                            weight_seed=seed, token_seed=seed + 1, name="random_window")
    G.note("random window layer", dict(H=H, I=I, E=E, k=k, T=T, expert=expert, bias=bias, seed=seed))
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=T, flags=MOE_LAYER_SCREEN_ON)
    x = SD.device_tokens(spec, 0, T)
    fi, fg, fo = G.run_grouped(layer, x)
    L = G.host_oracle(spec)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 0, T)
    G.compare(fi, fg, fo, o_idx, o_g, o_out, f"random window H={H} I={I} E={E} k={k} T={T}")
    assert layer.device_error() == 0
