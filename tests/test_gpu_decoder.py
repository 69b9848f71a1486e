"""Batch-1 decode through a stack of layers with one captured graph per layer
(moe_decoder_*): every layer of every step against the float64 oracle on
the input the layer actually read, the residual stream between layers bit
for bit, each layer's results bit for bit against an eager
moe_grouped_forward on the same input, and the doorbells, with the host
either running ahead or waiting for each layer's doorbell."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BASE = synth.small_spec(H=2048, E=130, k=10, I=256, act=synth.DT_BF16, expert=synth.DT_Q4,
                        bias_alpha=0.37, weight_seed=25, token_seed=26, name="wide_q4")
# three distinct layers: the int8 screen on, off, on (the screen's list state
# lives in each layer's own workspace)
SPECS = [dataclasses.replace(BASE, weight_seed=25 + l, name=f"stack{l}") for l in range(3)]


def bf16_bits_to_f64(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_rne(f32):
    """Binary32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.asarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _setup():
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_OFF, MOE_LAYER_SCREEN_ON
    dls = [SD.device_layer(s) for s in SPECS]
    flags = [MOE_LAYER_SCREEN_ON, MOE_LAYER_SCREEN_OFF, MOE_LAYER_SCREEN_ON]
    layers = [SD.make_layer(d, max_tokens=1, flags=f) for d, f in zip(dls, flags)]
    return torch, SD, dls, layers


class _DevArray:
    """n elements of device memory the decoder owns, for torch.as_tensor
    (a zero-copy view through the CUDA array interface)."""

    def __init__(self, addr, n, typestr):
        self.__cuda_array_interface__ = {"shape": (n,), "typestr": typestr, "data": (addr, False),
                                         "version": 3, "strides": None}


def _view(torch, addr, n, typestr):
    return torch.as_tensor(_DevArray(addr, n, typestr), device="cuda")


@pytest.mark.parametrize("wait", [False, True])
def test_decoder_layers_against_oracle(wait):
    torch, SD, dls, layers = _setup()
    from expert_routing_quantized_amd import Decoder
    G.note("decoder", "wait" if wait else "run ahead", [s.name for s in SPECS])
    H, k, n = BASE.H, BASE.k, len(SPECS)
    dec = Decoder(layers)
    oracles = [G.host_oracle(s) for s in SPECS]
    X = SD.device_tokens(BASE, 500, 6).cpu().view(torch.int16).numpy().view(np.uint16)
    slots = [dec.buffers(l) for l in range(n + 1)]
    assert slots[n][1] is None and slots[n][2] is None          # the result slot only
    for l in range(n):
        assert dec.doorbell(l) == 0
    for t in range(X.shape[0]):
        _view(torch, slots[0][0], H, "<i2").copy_(torch.from_numpy(X[t].view(np.int16)))
        torch.cuda.synchronize()
        dec.step(wait_doorbell=wait)
        torch.cuda.synchronize()
        for l in range(n):
            assert dec.doorbell(l) == t + 1, f"layer {l} doorbell {dec.doorbell(l)} after step {t + 1}"
        xs = [_view(torch, slots[l][0], H, "<i2").cpu().numpy().view(np.uint16) for l in range(n + 1)]
        assert np.array_equal(xs[0], X[t])
        for l in range(n):
            out = _view(torch, slots[l][1], H, "<f4").cpu().numpy()
            idx = _view(torch, slots[l][2], k, "<i4").cpu().numpy()
            gates = _view(torch, slots[l][3], k, "<f4").cpu().numpy()
            # the residual stream, bit for bit
            nxt = bf16_rne(bf16_bits_to_f64(xs[l]).astype(np.float32) + out)
            assert np.array_equal(nxt, xs[l + 1]), f"step {t} layer {l}: residual stream differs"
            # the oracle on the input this layer read
            xin = bf16_bits_to_f64(xs[l])[None, :]
            o_idx, o_g, _, o_out = oracle.moe_tokens(xin, oracles[l])
            G.compare(idx[None], gates[None], out[None], o_idx, o_g, o_out, f"decoder step {t} layer {l}")
            # an eager call on the same input: the same bits
            xd = torch.from_numpy(xs[l].view(np.int16)).cuda().view(torch.bfloat16)[None]
            ei, eg, eo = G.run_grouped(layers[l], xd)
            assert np.array_equal(ei[0], idx) and np.array_equal(eg[0].view(np.uint32), gates.view(np.uint32))
            assert np.array_equal(eo[0].view(np.uint32), out.view(np.uint32)), f"step {t} layer {l}: eager differs"
    for L in layers:
        assert L.device_error() == 0
    dec.close()


def test_decoder_refuses_mixed_hidden_sizes():
    torch, SD, dls, layers = _setup()
    from expert_routing_quantized_amd import Decoder, MoeError
    other = dataclasses.replace(BASE, H=1024, name="h1024")
    lo = SD.make_layer(SD.device_layer(other), max_tokens=1)
    with pytest.raises(MoeError) as ei:
        Decoder([layers[0], lo])
    assert ei.value.status == -2
