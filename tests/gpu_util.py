"""Helpers for the GPU tests: build device layers, run the C ABI, compare
with the float64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

GATE_TOL = 1e-6      # absolute, per gate
OUT_TOL = 1e-3       # relative L2 per token


def note(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def host_oracle(spec, cache_size=256):
    return oracle.layer_from_spec(spec, cache_size=cache_size)


def run_route_decode(layer, x, ws=None):
    """moe_route for all rows, then moe_expert_decode per row."""
    torch = torch_mod()
    T = x.shape[0]
    idx = torch.empty((T, layer.k), dtype=torch.int32, device=x.device)
    gates = torch.empty((T, layer.k), dtype=torch.float32, device=x.device)
    out = torch.empty((T, layer.H), dtype=torch.float32, device=x.device)
    ws = layer.workspace(T) if ws is None else ws
    layer.route(x, T, idx, gates, ws)
    for t in range(T):
        layer.expert_decode(x[t], idx[t], gates[t], out[t], ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gates.cpu().numpy(), out.cpu().numpy()


def run_grouped(layer, x, flags=0, idx=None, gates=None, ws=None):
    torch = torch_mod()
    T = x.shape[0]
    if idx is None:
        idx = torch.empty((T, layer.k), dtype=torch.int32, device=x.device)
        gates = torch.empty((T, layer.k), dtype=torch.float32, device=x.device)
    out = torch.empty((T, layer.H), dtype=torch.float32, device=x.device)
    ws = layer.workspace(T) if ws is None else ws
    layer.grouped_forward(x, T, idx, gates, flags, out, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gates.cpu().numpy(), out.cpu().numpy()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-300)


def compare(idx, gates, out, o_idx, o_gates, o_out, what=""):
    """Indices bit-exact, gates within GATE_TOL, outputs within OUT_TOL."""
    bad = np.nonzero(np.any(idx != o_idx, axis=1))[0]
    assert bad.size == 0, f"{what}: index mismatch at tokens {bad[:8]}: gpu {idx[bad[:2]]} oracle {o_idx[bad[:2]]}"
    gerr = np.abs(gates.astype(np.float64) - o_gates).max()
    assert gerr <= GATE_TOL, f"{what}: gate error {gerr}"
    if out is not None and o_out is not None:
        r = rel_l2(out, o_out)
        assert np.all(np.isfinite(out)), f"{what}: non-finite output"
        assert r.max() <= OUT_TOL, f"{what}: rel L2 max {r.max()} median {np.median(r)}"
        return r
    return None


def oracle_tokens(spec, L, first, count, with_output=True):
    X = oracle.tokens_f64(spec, first, count)
    return oracle.moe_tokens(X, L, with_output=with_output)
