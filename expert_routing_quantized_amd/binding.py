"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP kernels behind the C ABI; this
module turns torch tensors into device pointers and the current HIP stream
into a ``hipStream_t``.  If ``libmoe.so`` has not been built the import
fails loudly -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_Q4B32 = 0, 1, 2
MOE_ROUTER_HE, MOE_ROUTER_EH = 0, 1
MOE_LAYER_FORCE_EXACT_REFINE = 1
MOE_LAYER_SCREEN_ON = 2
MOE_LAYER_SCREEN_OFF = 4
MOE_LAYER_WINDOW_SCREEN_OFF = 8
MOE_ROUTE_INTERNAL, MOE_ROUTE_GIVEN = 0, 1

STATUS = {0: "MOE_OK", -1: "MOE_E_NULL", -2: "MOE_E_GEOMETRY", -3: "MOE_E_DTYPE",
          -4: "MOE_E_ALIGN", -5: "MOE_E_WORKSPACE", -6: "MOE_E_RANGE", -7: "MOE_E_HIP",
          -8: "MOE_E_DEVICE_FLAG"}

EXPORTS = ["moe_layer_create", "moe_layer_destroy", "moe_workspace_bytes", "moe_route",
           "moe_expert_decode", "moe_grouped_forward", "moe_grouped_forward_noalloc", "moe_device_error",
           "moe_router_logits", "moe_router_screen", "moe_layer_stats",
           "moe_decoder_create", "moe_decoder_destroy", "moe_decoder_buffers", "moe_decoder_step",
           "moe_decoder_doorbell", "moe_expert_counts", "moe_layer_set_hot_experts",
           "moe_layer_set_host_experts", "moe_cpu_experts",
           "moe_status_string", "moe_last_error_message", "moe_abi_version"]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
        ("router_layout", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmoe.so and declare its prototypes (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "(python expert_routing_quantized_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    lib.moe_layer_create.argtypes = [ctypes.POINTER(LayerDesc), vp, ctypes.POINTER(vp)]
    lib.moe_layer_destroy.argtypes = [vp]
    lib.moe_workspace_bytes.argtypes = [vp, i32, ctypes.POINTER(sz)]
    lib.moe_route.argtypes = [vp, vp, i32, vp, vp, vp, sz, vp]
    lib.moe_expert_decode.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_router_logits.argtypes = [vp, vp, i32, vp, vp, sz, vp]
    lib.moe_router_screen.argtypes = [vp, vp, i32, vp, vp, vp, sz, vp]
    lib.moe_grouped_forward.argtypes = [vp, vp, i32, vp, vp, u32, vp, vp, sz, vp]
    lib.moe_grouped_forward_noalloc.argtypes = [vp, vp, i32, vp, vp, u32, vp, vp]
    lib.moe_device_error.argtypes = [vp, vp, ctypes.POINTER(i32)]
    lib.moe_layer_stats.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint64)]
    lib.moe_expert_counts.argtypes = [vp, vp, i32, vp, vp]
    lib.moe_layer_set_hot_experts.argtypes = [vp, ctypes.POINTER(i32), i32, vp]
    lib.moe_layer_set_host_experts.argtypes = [vp, ctypes.POINTER(i32), i32, i32, vp]
    lib.moe_cpu_experts.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, vp, vp, vp, i32]
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error_message.argtypes = []
    lib.moe_last_error_message.restype = ctypes.c_char_p
    lib.moe_abi_version.argtypes = []
    lib.moe_decoder_create.argtypes = [ctypes.POINTER(vp), i32, vp, ctypes.POINTER(vp)]
    lib.moe_decoder_destroy.argtypes = [vp]
    lib.moe_decoder_buffers.argtypes = [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                        ctypes.POINTER(vp)]
    lib.moe_decoder_step.argtypes = [vp, vp, i32]
    lib.moe_decoder_doorbell.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_uint64)]
    for name in ["moe_layer_create", "moe_layer_destroy", "moe_workspace_bytes", "moe_route",
                 "moe_expert_decode", "moe_grouped_forward", "moe_grouped_forward_noalloc", "moe_device_error",
                 "moe_router_logits", "moe_router_screen", "moe_layer_stats", "moe_abi_version",
                 "moe_decoder_create", "moe_decoder_destroy", "moe_decoder_buffers", "moe_decoder_step",
                 "moe_decoder_doorbell", "moe_expert_counts", "moe_layer_set_hot_experts",
                 "moe_layer_set_host_experts", "moe_cpu_experts"]:
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _check(st: int, where: str):
    if st != 0:
        detail = load_library().moe_last_error_message().decode()
        raise MoeError(st, where, detail)


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _host_ptr(a):
    """Address of a C-contiguous numpy array (None -> NULL)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def cpu_experts(hidden, n_experts, top_k, inter, act_dtype, expert_dtype, w_gate, w_up, w_down,
                x, T, idx, gates, out, s_gate=None, s_up=None, s_down=None, n_threads=1):
    """moe_cpu_experts on host numpy arrays (the pool's arithmetic, no GPU):
    out [T][H] float32 is written."""
    lib = load_library()
    d = LayerDesc(hidden, n_experts, top_k, inter, max(T, 1), act_dtype, expert_dtype, MOE_ROUTER_EH, 0,
                  None, None, _host_ptr(w_gate), _host_ptr(w_up), _host_ptr(w_down),
                  _host_ptr(s_gate), _host_ptr(s_up), _host_ptr(s_down))
    _check(lib.moe_cpu_experts(ctypes.byref(d), _host_ptr(x), T, _host_ptr(idx), _host_ptr(gates),
                               _host_ptr(out), n_threads), "moe_cpu_experts")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Layer:
    """One MoE layer over caller-owned device tensors.

    The tensors passed here must stay alive and unchanged for the layer's
    lifetime (the object keeps references to them).
    """

    def __init__(self, *, hidden, n_experts, top_k, inter, max_tokens, act_dtype, expert_dtype,
                 router_w, w_gate, w_up, w_down, router_bias=None, s_gate=None, s_up=None,
                 s_down=None, router_layout=MOE_ROUTER_EH, flags=0, stream=None):
        self.lib = load_library()
        self._keep = (router_w, router_bias, w_gate, w_up, w_down, s_gate, s_up, s_down)
        self.desc = LayerDesc(hidden, n_experts, top_k, inter, max_tokens, act_dtype,
                              expert_dtype, router_layout, flags, _ptr(router_w),
                              _ptr(router_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                              _ptr(s_gate), _ptr(s_up), _ptr(s_down))
        self.H, self.E, self.k, self.I = hidden, n_experts, top_k, inter
        self.max_tokens = max_tokens
        h = ctypes.c_void_p()
        _check(self.lib.moe_layer_create(ctypes.byref(self.desc), _stream(stream), ctypes.byref(h)),
               "moe_layer_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            self.lib.moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, T: int) -> int:
        n = ctypes.c_size_t()
        _check(self.lib.moe_workspace_bytes(self.handle, T, ctypes.byref(n)), "moe_workspace_bytes")
        return n.value

    def workspace(self, T: int, device="cuda"):
        import torch
        return torch.empty(max(1, self.workspace_bytes(T)), dtype=torch.uint8, device=device)

    def route(self, x, T, idx, gates, ws, stream=None):
        _check(self.lib.moe_route(self.handle, _ptr(x), T, _ptr(idx), _ptr(gates), _ptr(ws),
                                  ws.numel() if ws is not None else 0, _stream(stream)), "moe_route")

    def router_logits(self, x, T, z, ws, stream=None):
        _check(self.lib.moe_router_logits(self.handle, _ptr(x), T, _ptr(z), _ptr(ws),
                                          ws.numel() if ws is not None else 0, _stream(stream)),
               "moe_router_logits")

    def router_screen(self, x, T, v, bound, ws, stream=None):
        _check(self.lib.moe_router_screen(self.handle, _ptr(x), T, _ptr(v), _ptr(bound), _ptr(ws),
                                          ws.numel() if ws is not None else 0, _stream(stream)),
               "moe_router_screen")

    def expert_decode(self, x, idx, gates, out, ws, stream=None):
        _check(self.lib.moe_expert_decode(self.handle, _ptr(x), _ptr(idx), _ptr(gates), _ptr(out),
                                          _ptr(ws), ws.numel() if ws is not None else 0,
                                          _stream(stream)), "moe_expert_decode")

    def grouped_forward(self, x, T, idx, gates, flags, out, ws, stream=None):
        _check(self.lib.moe_grouped_forward(self.handle, _ptr(x), T, _ptr(idx), _ptr(gates), flags,
                                            _ptr(out), _ptr(ws), ws.numel() if ws is not None else 0,
                                            _stream(stream)), "moe_grouped_forward")

    def grouped_forward_noalloc(self, x, T, idx, gates, flags, out, stream=None):
        _check(self.lib.moe_grouped_forward_noalloc(self.handle, _ptr(x), T, _ptr(idx), _ptr(gates), flags,
                                                    _ptr(out), _stream(stream)), "moe_grouped_forward_noalloc")

    def exact_refinements(self, stream=None) -> int:
        n = ctypes.c_uint64()
        _check(self.lib.moe_layer_stats(self.handle, _stream(stream), ctypes.byref(n)), "moe_layer_stats")
        return n.value

    def expert_counts(self, idx, n, counts, stream=None):
        """counts[e] += 1 (uint32 device tensor [E]) for each of the first n
        indices of the device int32 tensor idx."""
        _check(self.lib.moe_expert_counts(self.handle, _ptr(idx), n, _ptr(counts), _stream(stream)),
               "moe_expert_counts")

    def set_hot_experts(self, ids, stream=None):
        """Copy the listed experts (host sequence of ints) into the layer's hot
        region; an empty sequence removes it."""
        n = len(ids)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(e) for e in ids])
        _check(self.lib.moe_layer_set_hot_experts(self.handle, arr if n else None, n, _stream(stream)),
               "moe_layer_set_hot_experts")

    def set_host_experts(self, ids, n_threads=0, stream=None):
        """Move the listed experts (host sequence of ints) to the host tier;
        an empty sequence removes it."""
        n = len(ids)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(e) for e in ids])
        _check(self.lib.moe_layer_set_host_experts(self.handle, arr if n else None, n, n_threads, _stream(stream)),
               "moe_layer_set_host_experts")

    def device_error(self, stream=None) -> int:
        code = ctypes.c_int32()
        st = self.lib.moe_device_error(self.handle, _stream(stream), ctypes.byref(code))
        if st not in (0, -8):
            _check(st, "moe_device_error")
        return code.value


class Decoder:
    """Batch-1 decode through a stack of layers, one captured graph per layer
    (moe_decoder_*).  Keeps references to the layers, which must outlive it."""

    def __init__(self, layers, stream=None):
        self.lib = load_library()
        self.layers = list(layers)
        arr = (ctypes.c_void_p * len(self.layers))(*[L.handle for L in self.layers])
        h = ctypes.c_void_p()
        _check(self.lib.moe_decoder_create(arr, len(self.layers), _stream(stream), ctypes.byref(h)),
               "moe_decoder_create")
        self.handle = h

    def buffers(self, layer):
        """(x, out, idx, gates) device addresses of `layer` (None where absent)."""
        x, out, idx, gates = (ctypes.c_void_p() for _ in range(4))
        _check(self.lib.moe_decoder_buffers(self.handle, layer, ctypes.byref(x), ctypes.byref(out),
                                            ctypes.byref(idx), ctypes.byref(gates)), "moe_decoder_buffers")
        return x.value, out.value, idx.value, gates.value

    def step(self, wait_doorbell=False, stream=None):
        _check(self.lib.moe_decoder_step(self.handle, _stream(stream), 1 if wait_doorbell else 0),
               "moe_decoder_step")

    def doorbell(self, layer) -> int:
        v = ctypes.c_uint64()
        _check(self.lib.moe_decoder_doorbell(self.handle, layer, ctypes.byref(v)), "moe_decoder_doorbell")
        return v.value

    def close(self):
        if self.handle:
            _check(self.lib.moe_decoder_destroy(self.handle), "moe_decoder_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
