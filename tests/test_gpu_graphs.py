"""HIP graph capture of moe_grouped_forward: each call is captured once and
replayed several times, with eager calls on other inputs (through the same
workspace) between the replays; every replay must reproduce the eager result
bit for bit.  Covers the fused batch-1 decode, a verify window, the pair
deduplication path, the sorted 4-bit grouped path, the MFMA grouped path
(with the 256 x 256 router tiles and their direct-to-LDS loads at T = 600)
and fp32 activations, so no captured path relies on workspace contents
left by an earlier call.
"""
import pytest

import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SPECS = {
    "tiny_q4": synth.small_spec(H=256, E=200, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=23, token_seed=24, name="tiny_q4"),
    "wide_q4": synth.small_spec(H=2048, E=130, k=10, I=256, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=25, token_seed=26, name="wide_q4"),
    "mfma_multi_tile": synth.small_spec(H=512, E=20, k=4, I=128, act=synth.DT_BF16, expert=synth.DT_BF16,
                                        bias_alpha=0.37, weight_seed=71, token_seed=72, name="mfma_multi_tile"),
    "tiny_f32": synth.CONFIGS["tiny_f32"],
}

_layers = {}


def device_layer(name):
    if name not in _layers:
        import synth.device as SD
        _layers[name] = SD.device_layer(SPECS[name])
    return _layers[name]


@pytest.mark.parametrize("name,T", [("wide_q4", 1), ("tiny_q4", 1), ("wide_q4", 5), ("tiny_q4", 37),
                                    ("tiny_q4", 100), ("mfma_multi_tile", 300), ("mfma_multi_tile", 600),
                                    ("tiny_f32", 1)])
def test_graph_replays_match_eager(name, T):
    torch = G.torch_mod()
    import synth.device as SD
    spec = SPECS[name]
    G.note("graph replays", name, T)
    layer = SD.make_layer(device_layer(name), max_tokens=T)
    xa = SD.device_tokens(spec, 0, T)
    xb = SD.device_tokens(spec, 600, T)
    ws = layer.workspace(T)
    dev = xa.device

    def buffers():
        return (torch.empty((T, spec.k), dtype=torch.int32, device=dev),
                torch.empty((T, spec.k), dtype=torch.float32, device=dev),
                torch.empty((T, spec.H), dtype=torch.float32, device=dev))

    ref_i, ref_g, ref_o = buffers()
    layer.grouped_forward(xa, T, ref_i, ref_g, 0, ref_o, ws)
    torch.cuda.synchronize()

    gi, gg, go = buffers()
    bi, bg, bo = buffers()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        layer.grouped_forward(xa, T, gi, gg, 0, go, ws)       # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(graph, stream=s):
            layer.grouped_forward(xa, T, gi, gg, 0, go, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        # other inputs through the same workspace, eagerly, then clobbered outputs
        layer.grouped_forward(xb, T, bi, bg, 0, bo, ws)
        torch.cuda.synchronize()
        gi.fill_(-7)
        gg.fill_(float("nan"))
        go.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gi, ref_i), f"replay {rep}: indices differ"
        assert torch.equal(gg.view(torch.int32), ref_g.view(torch.int32)), f"replay {rep}: gates differ"
        assert torch.equal(go.view(torch.int32), ref_o.view(torch.int32)), f"replay {rep}: outputs differ"
    assert layer.device_error() == 0
