"""Device-side construction of synthetic layers (uses synth/libmoesynth.so).

The expert pools of the full-size layers (77 GB in bf16, 21.7 GB in 4-bit)
do not fit in host memory, so they are written straight into HBM by the
device implementation of the generator in ``synth/__init__.py``; the router,
its bias and the hidden states are drawn the same way.  Host and device
produce identical bits (checked by the tests on sampled experts).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

from . import (DT_BF16, DT_F32, DT_Q4, TAG_DOWN, TAG_GATE, TAG_ROUTER, TAG_UP, TAG_X, LayerSpec,
               router_bias, scale_bits, stream_key)

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoesynth.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is not built (python expert_routing_quantized_amd/build.py)")
        lib = ctypes.CDLL(LIB)
        lib.synth_fill_values.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                          ctypes.c_void_p]
        lib.synth_fill_values.restype = ctypes.c_int
        lib.synth_fill_q4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                      ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_uint32, ctypes.c_void_p]
        lib.synth_fill_q4.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fill_values(t, key: int, base: int, sigma: float):
    """Fill a contiguous fp32 or bf16 tensor with counters base .. base + numel - 1."""
    import torch
    bf16 = 1 if t.dtype == torch.bfloat16 else 0
    assert t.dtype in (torch.bfloat16, torch.float32) and t.is_contiguous()
    rc = load().synth_fill_values(t.data_ptr(), bf16, key, base, scale_bits(sigma), t.numel(), _stream())
    if rc != 0:
        raise RuntimeError(f"synth_fill_values failed ({rc})")


def fill_q4(codes, scales, key: int, row_base: int, K: int, sigma: float):
    rows = codes.numel() // (K // 2)
    rc = load().synth_fill_q4(codes.data_ptr(), scales.data_ptr(), key, row_base, rows, K,
                              scale_bits(sigma), _stream())
    if rc != 0:
        raise RuntimeError(f"synth_fill_q4 failed ({rc})")


@dataclasses.dataclass
class DeviceLayer:
    spec: LayerSpec
    router_eh: object            # [E][H] act dtype
    bias: object                 # fp32 [E] (None when the layer has no bias)
    w_gate: object
    w_up: object
    w_down: object
    s_gate: object = None
    s_up: object = None
    s_down: object = None

    def nbytes_pool(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.w_gate, self.w_up, self.w_down, self.s_gate, self.s_up, self.s_down)
                   if t is not None)


def _act_torch(dt):
    import torch
    return torch.float32 if dt == DT_F32 else torch.bfloat16


def device_router(spec: LayerSpec, device="cuda"):
    import torch
    r = torch.empty((spec.E, spec.H), dtype=_act_torch(spec.act), device=device)
    fill_values(r, stream_key(spec.weight_seed, TAG_ROUTER), 0, spec.sigma_w)
    return r


def device_layer(spec: LayerSpec, device="cuda") -> DeviceLayer:
    """Router, bias and expert pools of ``spec`` in HBM."""
    import torch
    E, H, I = spec.E, spec.H, spec.I
    router = device_router(spec, device)
    bias = None
    if spec.bias_alpha is not None:
        bias = torch.from_numpy(router_bias(spec)).to(device)
    if spec.expert == DT_Q4:
        def q4(tag, rows, K):
            codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=device)
            sc = torch.empty((rows, K // 32), dtype=torch.int16, device=device)
            fill_q4(codes, sc, stream_key(spec.weight_seed, tag), 0, K, spec.sigma_w)
            return codes, sc
        g, sg = q4(TAG_GATE, E * I, H)
        u, su = q4(TAG_UP, E * I, H)
        d, sd = q4(TAG_DOWN, E * H, I)
        dl = DeviceLayer(spec, router, bias, g.view(E, I, H // 2), u.view(E, I, H // 2),
                         d.view(E, H, I // 2), sg.view(E, I, H // 32), su.view(E, I, H // 32),
                         sd.view(E, H, I // 32))
    else:
        dt = torch.float32 if spec.expert == DT_F32 else torch.bfloat16

        def dense(tag, shape):
            t = torch.empty(shape, dtype=dt, device=device)
            fill_values(t, stream_key(spec.weight_seed, tag), 0, spec.sigma_w)
            return t
        dl = DeviceLayer(spec, router, bias, dense(TAG_GATE, (E, I, H)), dense(TAG_UP, (E, I, H)),
                         dense(TAG_DOWN, (E, H, I)))
    torch.cuda.synchronize()
    return dl


def device_tokens(spec: LayerSpec, first: int, count: int, device="cuda"):
    import torch
    x = torch.empty((count, spec.H), dtype=_act_torch(spec.act), device=device)
    fill_values(x, stream_key(spec.token_seed, TAG_X), first * spec.H, spec.sigma_x)
    return x


def to_numpy_bits(t) -> np.ndarray:
    """Copy a device tensor to host numpy, bf16/fp16 as uint16 bit patterns."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16, torch.int16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make_layer(dl: DeviceLayer, max_tokens: int = 1, router_layout: str = "EH", flags: int = 0,
               router=None):
    """binding.Layer over a DeviceLayer (``router`` overrides the router tensor)."""
    from expert_routing_quantized_amd import binding as B
    spec = dl.spec
    r = dl.router_eh if router is None else router
    layout = B.MOE_ROUTER_EH
    if router_layout == "HE":
        r = r.t().contiguous()
        layout = B.MOE_ROUTER_HE
    act = B.MOE_F32 if spec.act == DT_F32 else B.MOE_BF16
    ex = {DT_F32: B.MOE_F32, DT_BF16: B.MOE_BF16, DT_Q4: B.MOE_Q4B32}[spec.expert]
    return B.Layer(hidden=spec.H, n_experts=spec.E, top_k=spec.k, inter=spec.I,
                   max_tokens=max_tokens, act_dtype=act, expert_dtype=ex, router_w=r,
                   router_bias=dl.bias, w_gate=dl.w_gate, w_up=dl.w_up, w_down=dl.w_down,
                   s_gate=dl.s_gate, s_up=dl.s_up, s_down=dl.s_down, router_layout=layout,
                   flags=flags)
