"""Parity at the full workload sizes, in the launch configuration the
benchmark uses: E = 24,576 experts, H = 2048, top-10, I = 256.

The pools are generated in HBM; the oracle regenerates on the host only the
experts the sampled tokens select.  Routing (indices, gates) is checked on
every token of a call; outputs on samples.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

_state = {}


def host_router():
    """Float64 router/bias shared by every full-size workload (same weights seed)."""
    if "R" not in _state:
        spec = synth.CONFIGS["decode_bf16"]
        L = oracle.layer_from_spec(spec)
        _state["R"] = (L.R, L.b, L.absR())
    return _state["R"]


def oracle_for(spec):
    R, b, absR = host_router()
    L = oracle.OracleLayer(R, b, spec.k, lambda e, w: synth.expert_stored(spec, e, w), cache_size=512)
    L._absR = absR
    return L


def device_for(name):
    """Device layer of a config; frees the other full-size pool first."""
    import torch
    import synth.device as SD
    pool = "q4" if synth.CONFIGS[name].expert == synth.DT_Q4 else "bf16"
    if _state.get("pool_kind") != pool:
        _state.pop("dl", None)
        torch.cuda.empty_cache()
        G.note("generating full-size pool", pool)
        _state["dl"] = SD.device_layer(synth.CONFIGS[name])
        _state["pool_kind"] = pool
    return _state["dl"]


def layer_for(name, T):
    import synth.device as SD
    dl = device_for(name)
    spec = synth.CONFIGS[name]
    # the bf16 workloads share one pool and the 4-bit ones another; tokens differ per workload
    return SD.make_layer(dl, max_tokens=T), spec


@pytest.mark.parametrize("T", [1, 5, 64, 512])
def test_router_logits_within_bound(T):
    """|z_gpu - z_exact| within the documented bound on every logit (the
    selection relies on it): fmaf chains at T = 1, 16x16x32 MFMA tiles folded
    per instruction at T = 5, the MFMA GEMM folding into binary64 every 128
    of H at T = 64, the 256 x 256 tiles accumulating all of H in fp32 at
    T = 512 (GEMM cases checked on sampled expert columns)."""
    import synth.device as SD
    torch = G.torch_mod()
    layer, spec = layer_for("decode_q4", T)
    G.note("router bound", T)
    x = SD.device_tokens(spec, 10, T)
    z = torch.empty((T, spec.E), dtype=torch.float64, device="cuda")
    ws = layer.workspace(T)
    layer.router_logits(x, T, z, ws)
    torch.cuda.synchronize()
    zg = z.cpu().numpy()
    R, b, absR = host_router()
    X = oracle.tokens_f64(spec, 10, T)
    cpl = (spec.H // 8 + 63) // 64
    if T >= 512:
        d32, d64 = 17 * (spec.H // 16), 1
        cols = np.unique(np.concatenate([np.arange(0, spec.E, 131), np.arange(spec.E - 64, spec.E)]))
        R, b, zg = R[:, cols], b[cols], zg[:, cols]
    elif T >= 16:
        d32, d64 = 136, (spec.H + 127) // 128 + 1
        cols = np.unique(np.concatenate([np.arange(0, spec.E, 17), np.arange(spec.E - 64, spec.E)]))
        R, b, zg = R[:, cols], b[cols], zg[:, cols]
    elif T > 1:
        d32, d64 = 33, (spec.H + 127) // 128 + 4
    else:
        d32, d64 = 7, int(np.ceil(np.log2(cpl))) + 7
    gam = d32 * 2.0 ** -23 / (1 - d32 * 2.0 ** -23) + d64 * 2.0 ** -52 / (1 - d64 * 2.0 ** -52)
    nmax = np.sqrt((R * R).sum(axis=0)).max()
    # reference logits in x87 extended precision (64-bit significand): every
    # product is exact and the sum's error (< 1e-14) is far below the bound
    Zo = (X.astype(np.longdouble) @ R.astype(np.longdouble)) + b.astype(np.longdouble)[None, :]
    Bt = gam * np.linalg.norm(X, axis=1)[:, None] * nmax
    B = Bt + 2.0 ** -52 * np.abs(zg) + (d32 + spec.H) * 2.0 ** -125
    ratio = (np.abs(zg.astype(np.longdouble) - Zo) / B).astype(np.float64)
    print(f"T={T}: max |err|/bound = {ratio.max():.3e}, max |err| = {np.abs(zg - Zo).max():.3e}")
    assert ratio.max() < 1.0


def test_decode_q4_decode_parity():
    import synth.device as SD
    layer, spec = layer_for("decode_q4", 16)
    L = oracle_for(spec)
    for first in (0, 500, 984):
        G.note("decode_q4 decode tokens", first)
        x = SD.device_tokens(spec, first, 16)
        idx, gates, out = G.run_route_decode(layer, x)
        o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, first, 16)
        r = G.compare(idx, gates, out, o_idx, o_g, o_out, f"decode_q4@{first}")
        print(f"decode_q4 tokens {first}..: rel L2 max {r.max():.2e} median {np.median(r):.2e}")
    assert layer.device_error() == 0


def test_decode_q4_grouped_single_token_path():
    """moe_grouped_forward at T = 1 (selection fused with gate/up) against
    the oracle on 16 tokens, and bitwise against moe_route +
    moe_expert_decode on all 1000 tokens of the stream (including the ones
    whose order needs exact refinement)."""
    grouped_single_token_path("decode_q4", 1000)


def grouped_single_token_path(name, n):
    import torch
    import synth.device as SD
    layer, spec = layer_for(name, 1)
    L = oracle_for(spec)
    first = 400
    x = SD.device_tokens(spec, first, 16)
    rows = [G.run_grouped(layer, x[t:t + 1]) for t in range(16)]
    idx = np.concatenate([r[0] for r in rows])
    gates = np.concatenate([r[1] for r in rows])
    out = np.concatenate([r[2] for r in rows])
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, first, 16)
    G.compare(idx, gates, out, o_idx, o_g, o_out, f"{name} grouped T=1")
    X = SD.device_tokens(spec, 0, n)
    ws = layer.workspace(1)
    fi = torch.empty((n, spec.k), dtype=torch.int32, device=X.device)
    fg = torch.empty((n, spec.k), dtype=torch.float32, device=X.device)
    fo = torch.empty((n, spec.H), dtype=torch.float32, device=X.device)
    si, sg, so = torch.empty_like(fi), torch.empty_like(fg), torch.empty_like(fo)
    for t in range(n):
        layer.grouped_forward(X[t], 1, fi[t], fg[t], 0, fo[t], ws)
        layer.route(X[t], 1, si[t], sg[t], ws)
        layer.expert_decode(X[t], si[t], sg[t], so[t], ws)
    torch.cuda.synchronize()
    assert torch.equal(fi, si)
    assert torch.equal(fg.view(torch.int32), sg.view(torch.int32))
    assert torch.equal(fo.view(torch.int32), so.view(torch.int32))
    assert layer.device_error() == 0


def test_verify_q4_verify_steps_parity():
    import synth.device as SD
    layer, spec = layer_for("verify_q4", 5)
    L = oracle_for(spec)
    for step in (0, 1, 999):
        G.note("verify_q4 step", step)
        x = SD.device_tokens(spec, 5 * step, 5)
        idx, gates, out = G.run_grouped(layer, x)
        o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 5 * step, 5)
        G.compare(idx, gates, out, o_idx, o_g, o_out, f"verify_q4 step {step}")
    assert layer.device_error() == 0


def test_decode_bf16_decode_parity():
    import synth.device as SD
    layer, spec = layer_for("decode_bf16", 8)
    L = oracle_for(spec)
    G.note("decode_bf16 decode")
    x = SD.device_tokens(spec, 0, 8)
    idx, gates, out = G.run_route_decode(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 0, 8)
    r = G.compare(idx, gates, out, o_idx, o_g, o_out, "decode_bf16")
    print(f"decode_bf16: rel L2 max {r.max():.2e} median {np.median(r):.2e}")
    assert layer.device_error() == 0


def test_decode_bf16_grouped_single_token_path():
    """The same for the bf16 experts (selection fused with the dense gate/up
    rows): oracle on 16 tokens, bitwise against moe_route +
    moe_expert_decode on 300 tokens."""
    grouped_single_token_path("decode_bf16", 300)


def test_prefill_bf16_prefill_chunk_parity():
    """T = 2048: every token's routing, and sampled tokens' outputs."""
    import synth.device as SD
    layer, spec = layer_for("prefill_bf16", 2048)
    G.note("prefill_bf16 grouped forward")
    x = SD.device_tokens(spec, 0, 2048)
    idx, gates, out = G.run_grouped(layer, x)
    assert layer.device_error() == 0
    G.note("prefill_bf16 oracle routing")
    L = oracle_for(spec)
    X = oracle.tokens_f64(spec, 0, 2048)
    Z, B = oracle.logits_with_bound(X, L)
    o_idx = np.empty((2048, spec.k), np.int64)
    o_g = np.empty((2048, spec.k))
    for t in range(2048):
        o_idx[t], zs = oracle.route_token(X[t], Z[t], B[t], L)
        o_g[t] = oracle.softmax_gates(zs)
    G.compare(idx, gates, None, o_idx, o_g, None, "prefill_bf16 routing")
    sample = np.linspace(0, 2047, 12).astype(int)
    o_out = np.stack([oracle.moe_given(X[t], L, o_idx[t], o_g[t]) for t in sample])
    r = G.rel_l2(out[sample], o_out)
    print(f"prefill_bf16 sampled outputs: rel L2 max {r.max():.2e}; distinct experts {len(np.unique(idx))}")
    assert r.max() <= G.OUT_TOL


@pytest.mark.parametrize("T", [2, 3, 4, 6, 8])
def test_verify_window_sizes_parity(T):
    """Verify windows of other sizes through the 4-bit layer (the drafters'
    depths: up to 3 + 1 and 5 + 1 tokens, and the largest independent-pair
    window)."""
    import synth.device as SD
    layer, spec = layer_for("verify_q4", 8)
    L = oracle_for(spec)
    first = 5 * 321 + T
    G.note("verify window T", T)
    x = SD.device_tokens(spec, first, T)
    idx, gates, out = G.run_grouped(layer, x)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, first, T)
    G.compare(idx, gates, out, o_idx, o_g, o_out, f"verify window T={T}")
    assert layer.device_error() == 0


@pytest.mark.parametrize("T", [2, 5, 8])
def test_verify_internal_routing_matches_given_routing(T):
    """Over 200 windows of the verify stream, moe_grouped_forward with
    internal routing gives the same idx, gates and outputs, bit for bit, as
    moe_route followed by moe_grouped_forward with the given routing."""
    import torch
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_ROUTE_GIVEN
    layer, spec = layer_for("verify_q4", 8)
    n = 200
    X = SD.device_tokens(spec, 0, n * T).view(n, T, spec.H)
    ws = layer.workspace(T)
    fi = torch.empty((n, T, spec.k), dtype=torch.int32, device=X.device)
    fg = torch.empty((n, T, spec.k), dtype=torch.float32, device=X.device)
    fo = torch.empty((n, T, spec.H), dtype=torch.float32, device=X.device)
    si, sg, so = torch.empty_like(fi), torch.empty_like(fg), torch.empty_like(fo)
    for w in range(n):
        layer.grouped_forward(X[w], T, fi[w], fg[w], 0, fo[w], ws)
        layer.route(X[w], T, si[w], sg[w], ws)
        layer.grouped_forward(X[w], T, si[w], sg[w], MOE_ROUTE_GIVEN, so[w], ws)
    torch.cuda.synchronize()
    assert torch.equal(fi, si)
    assert torch.equal(fg.view(torch.int32), sg.view(torch.int32))
    assert torch.equal(fo.view(torch.int32), so.view(torch.int32))
    assert layer.device_error() == 0


def _route_sample(spec, L, X, rows):
    Z, B = oracle.logits_with_bound(X[rows], L)
    o_idx = np.empty((len(rows), spec.k), np.int64)
    o_g = np.empty((len(rows), spec.k))
    for i, t in enumerate(rows):
        o_idx[i], zs = oracle.route_token(X[t], Z[i], B[i], L)
        o_g[i] = oracle.softmax_gates(zs)
    return o_idx, o_g


def test_prefill_chunk_8192_sampled_parity():
    """The largest prefill chunk (8,192 tokens): routing on 192 sampled
    tokens, outputs on 8 of them."""
    import synth.device as SD
    layer, spec = layer_for("prefill_bf16", 8192)
    G.note("prefill T=8192 grouped forward")
    x = SD.device_tokens(spec, 0, 8192)
    idx, gates, out = G.run_grouped(layer, x)
    assert layer.device_error() == 0
    L = oracle_for(spec)
    X = oracle.tokens_f64(spec, 0, 8192)
    rows = np.unique(np.concatenate([np.arange(0, 8192, 43), [8191]]))
    o_idx, o_g = _route_sample(spec, L, X, rows)
    G.compare(idx[rows], gates[rows], None, o_idx, o_g, None, "prefill T=8192 routing")
    sel = np.linspace(0, len(rows) - 1, 8).astype(int)
    o_out = np.stack([oracle.moe_given(X[rows[i]], L, o_idx[i], o_g[i]) for i in sel])
    r = G.rel_l2(out[rows[sel]], o_out)
    print(f"prefill T=8192 sampled outputs: rel L2 max {r.max():.2e}")
    assert r.max() <= G.OUT_TOL


def test_prefill_hot_experts_parity():
    """Supplementary: the bias concentrated on 64 experts, so each gets about
    320 pairs and the 64-row MFMA tiles carry nearly all the work."""
    import torch
    import synth.device as SD
    spec = synth.CONFIGS["prefill_bf16_hot"]
    dl0 = device_for("prefill_bf16")
    hot_bias = torch.from_numpy(synth.router_bias(spec)).to(dl0.router_eh.device)
    dl = SD.DeviceLayer(spec, dl0.router_eh, hot_bias, dl0.w_gate, dl0.w_up, dl0.w_down)
    layer = SD.make_layer(dl, max_tokens=2048)
    G.note("prefill hot grouped forward")
    x = SD.device_tokens(spec, 0, 2048)
    idx, gates, out = G.run_grouped(layer, x)
    assert layer.device_error() == 0
    counts = np.bincount(idx.ravel(), minlength=spec.E)
    assert np.count_nonzero(counts) <= 64 and counts.max() > 200
    R, _, absR = host_router()
    L = oracle.OracleLayer(R, synth.router_bias(spec).astype(np.float64), spec.k,
                           lambda e, w: synth.expert_stored(spec, e, w), cache_size=128)
    L._absR = absR
    X = oracle.tokens_f64(spec, 0, 2048)
    rows = np.arange(0, 2048, 7)
    o_idx, o_g = _route_sample(spec, L, X, rows)
    G.compare(idx[rows], gates[rows], None, o_idx, o_g, None, "prefill hot routing")
    sel = np.linspace(0, len(rows) - 1, 10).astype(int)
    o_out = np.stack([oracle.moe_given(X[rows[i]], L, o_idx[i], o_g[i]) for i in sel])
    r = G.rel_l2(out[rows[sel]], o_out)
    print(f"prefill hot sampled outputs: rel L2 max {r.max():.2e}; experts used {np.count_nonzero(counts)}")
    assert r.max() <= G.OUT_TOL
