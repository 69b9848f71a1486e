"""The C ABI without a GPU: the library loads, exports every declared entry
point, and refuses bad arguments with the documented status codes before
touching the HIP runtime."""
import ctypes
import os
import re
import subprocess

import pytest

import expert_routing_quantized_amd as moe
from expert_routing_quantized_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    syms = set(re.findall(r" T (moe_\w+)", out))
    for name in declared_functions():
        assert name in syms, name
        assert getattr(lib, name) is not None
    assert lib.moe_abi_version() == 1


def test_status_strings():
    lib = moe.load_library()
    for code, name in B.STATUS.items():
        assert lib.moe_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.moe_status_string(-99)


def good_desc(**kw):
    base = dict(hidden=256, n_experts=64, top_k=2, inter=128, max_tokens=4,
                act_dtype=B.MOE_BF16, expert_dtype=B.MOE_BF16, router_layout=B.MOE_ROUTER_EH,
                flags=0, router_w=0x10000, router_bias=0, w_gate=0x20000, w_up=0x30000,
                w_down=0x40000, s_gate=0, s_up=0, s_down=0)
    base.update(kw)
    return B.LayerDesc(**base)


def create(desc):
    lib = moe.load_library()
    h = ctypes.c_void_p(0x1234)
    st = lib.moe_layer_create(ctypes.byref(desc) if desc is not None else None, None, ctypes.byref(h))
    return st, h.value, lib.moe_last_error_message().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=250), -2), (dict(hidden=0), -2), (dict(hidden=16384), -2),
    (dict(inter=4), -2), (dict(n_experts=0), -2), (dict(top_k=0), -2),
    (dict(top_k=65), -2), (dict(n_experts=3, top_k=4), -2), (dict(top_k=33, n_experts=64), -2),
    (dict(max_tokens=0), -2), (dict(max_tokens=70000), -2),
    (dict(act_dtype=2), -3), (dict(act_dtype=7), -3), (dict(expert_dtype=9), -3),
    (dict(expert_dtype=B.MOE_F32), -3),                       # fp32 experts with bf16 x
    (dict(router_layout=5), -3), (dict(flags=16), -6),
    (dict(flags=B.MOE_LAYER_SCREEN_ON | B.MOE_LAYER_SCREEN_OFF), -6),
    (dict(flags=B.MOE_LAYER_SCREEN_ON, act_dtype=B.MOE_F32, expert_dtype=B.MOE_F32), -3),   # screen needs bf16 x
    (dict(router_w=0), -1), (dict(w_down=0), -1),
    (dict(expert_dtype=B.MOE_Q4B32), -1),                     # 4-bit without scales
    (dict(expert_dtype=B.MOE_Q4B32, hidden=264, s_gate=8, s_up=8, s_down=8), -2),  # H % 32
    (dict(s_gate=0x50000), -3),                               # scales for bf16 experts
    (dict(w_up=0x30008), -4), (dict(router_w=0x10002), -4),
    (dict(router_bias=0x60001), -4),
])
def test_create_refuses_bad_descriptions(kw, status):
    st, h, msg = create(good_desc(**kw))
    assert st == status and h is None and msg


def test_create_null_arguments():
    lib = moe.load_library()
    assert lib.moe_layer_create(None, None, None) == -1
    st, h, _ = create(None)
    assert st == -1 and h is None


def test_entry_points_refuse_null_layer():
    lib = moe.load_library()
    n = ctypes.c_size_t()
    assert lib.moe_workspace_bytes(None, 1, ctypes.byref(n)) == -1
    assert lib.moe_route(None, 1, 1, 1, 1, 1, 1, None) == -1
    assert lib.moe_expert_decode(None, 1, 1, 1, 1, 1, 1, None) == -1
    assert lib.moe_grouped_forward(None, 1, 1, 1, 1, 0, 1, 1, 1, None) == -1
    assert lib.moe_grouped_forward_noalloc(None, 1, 1, 1, 1, 0, 1, None) == -1
    assert lib.moe_router_screen(None, 1, 1, 1, 1, 1, 1, None) == -1
    code = ctypes.c_int32()
    assert lib.moe_device_error(None, None, ctypes.byref(code)) == -1
    nref = ctypes.c_uint64()
    assert lib.moe_layer_stats(None, None, ctypes.byref(nref)) == -1
    assert lib.moe_layer_destroy(None) == 0


def test_decoder_entry_points_refuse_null_and_range():
    lib = moe.load_library()
    h = ctypes.c_void_p(0x1234)
    assert lib.moe_decoder_create(None, 1, None, ctypes.byref(h)) == -1
    assert h.value is None                                   # cleared on failure
    layers = (ctypes.c_void_p * 1)(None)
    assert lib.moe_decoder_create(layers, 1, None, None) == -1
    assert lib.moe_decoder_create(layers, 1, None, ctypes.byref(h)) == -1    # a NULL layer
    assert lib.moe_decoder_create(layers, 0, None, ctypes.byref(h)) == -6
    assert lib.moe_decoder_create(layers, 65, None, ctypes.byref(h)) == -6
    assert lib.moe_decoder_buffers(None, 0, None, None, None, None) == -1
    assert lib.moe_decoder_step(None, None, 0) == -1
    v = ctypes.c_uint64()
    assert lib.moe_decoder_doorbell(None, 0, ctypes.byref(v)) == -1
    assert lib.moe_decoder_destroy(None) == 0


def test_binding_raises_typed_errors():
    with pytest.raises(B.MoeError) as ei:
        B._check(-2, "where")
    assert ei.value.status == -2


def test_bench_refuses_more_than_one_gpu():
    """The bench runs one GPU's share: --gpus above 1 exits non-zero with a
    message before touching a device."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode != 0
    assert "--gpus above 1 is not supported" in (r.stdout + r.stderr)
