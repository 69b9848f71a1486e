"""The hot-expert region and the host tier on the GPU.

moe_expert_counts equals a histogram of the routed indices; with the
most-routed experts copied into the layer's region, batch-1 decode, verify
windows and moe_expert_decode give the same outputs as without a region,
bit for bit, and as the oracle's; and the outputs come from the copies:
overwriting the pool's weights of the hot experts afterwards changes
nothing, while the same overwrite changes a layer without a region.
Experts moved to the host tier are computed by the host pool: outputs as
the oracle's, independent of the device pool's copies, the same bits in
graph replays."""
import dataclasses

import numpy as np
import pytest

import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SPECS = {
    "tiny_q4": synth.small_spec(H=256, E=200, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=23, token_seed=24, name="tiny_q4"),
    "tiny_bf16": synth.small_spec(H=256, E=200, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_BF16,
                                  bias_alpha=0.37, weight_seed=21, token_seed=22, name="tiny_bf16"),
    "wide_q4": synth.small_spec(H=2048, E=130, k=10, I=256, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=25, token_seed=26, name="wide_q4"),
}


def cloned(dl):
    """A DeviceLayer whose expert pools are private copies (safe to overwrite)."""
    kw = {f.name: getattr(dl, f.name) for f in dataclasses.fields(dl)}
    for f in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
        if kw[f] is not None:
            kw[f] = kw[f].clone()
    return type(dl)(**kw)


def run_all(layer, x, n1, T, nwin, ws1, wsw):
    """n1 batch-1 calls, then nwin windows of T tokens, then moe_expert_decode
    of the batch-1 routing: (idx, gates, out) of each part, on the host."""
    torch = G.torch_mod()
    dev = x.device
    k, H = layer.k, layer.H
    fi = torch.empty((n1, k), dtype=torch.int32, device=dev)
    fg = torch.empty((n1, k), dtype=torch.float32, device=dev)
    fo = torch.empty((n1, H), dtype=torch.float32, device=dev)
    for t in range(n1):
        layer.grouped_forward(x[t], 1, fi[t], fg[t], 0, fo[t], ws1)
    n = nwin * T
    wi = torch.empty((n, k), dtype=torch.int32, device=dev)
    wg = torch.empty((n, k), dtype=torch.float32, device=dev)
    wo = torch.empty((n, H), dtype=torch.float32, device=dev)
    for w in range(nwin):
        sl = slice(n1 + w * T, n1 + (w + 1) * T)
        dl = slice(w * T, (w + 1) * T)
        layer.grouped_forward(x[sl], T, wi[dl], wg[dl], 0, wo[dl], wsw)
    do = torch.empty((n1, H), dtype=torch.float32, device=dev)
    for t in range(n1):
        layer.expert_decode(x[t], fi[t], fg[t], do[t], ws1)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (fi, fg, fo, wi, wg, wo, do)], fi


def bitwise_equal(a, b):
    for u, v in zip(a, b):
        assert np.array_equal(np.ascontiguousarray(u).view(np.uint32), np.ascontiguousarray(v).view(np.uint32))


@pytest.mark.parametrize("name", list(SPECS))
def test_hot_region_counts_bitwise_and_relocated(name):
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_ON
    spec = SPECS[name]
    G.note("hot region", name)
    dl = cloned(SD.device_layer(spec))
    L = G.host_oracle(spec)
    n1, T, nwin = 24, 5, 3
    first = 300
    x = SD.device_tokens(spec, first, n1 + T * nwin)
    layer = SD.make_layer(dl, max_tokens=8, flags=MOE_LAYER_SCREEN_ON)
    ws1, wsw = layer.workspace(1), layer.workspace(T)
    ref, fi = run_all(layer, x, n1, T, nwin, ws1, wsw)
    # every part against the oracle
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, first, n1 + T * nwin)
    G.compare(ref[0], ref[1], ref[2], o_idx[:n1], o_g[:n1], o_out[:n1], f"{name} batch 1")
    G.compare(ref[3], ref[4], ref[5], o_idx[n1:], o_g[n1:], o_out[n1:], f"{name} windows")
    G.compare(ref[0], ref[1], ref[6], o_idx[:n1], o_g[:n1], o_out[:n1], f"{name} expert_decode")
    # counts: a histogram of the batch-1 indices
    counts = torch.zeros(spec.E, dtype=torch.int32, device="cuda")
    layer.expert_counts(fi, n1 * spec.k, counts)
    torch.cuda.synchronize()
    hist = np.bincount(ref[0].ravel(), minlength=spec.E)
    assert np.array_equal(counts.cpu().numpy(), hist)
    # the hot set: the most-chosen experts (lower index first among equals)
    order = np.lexsort((np.arange(spec.E), -hist))
    hot = [int(e) for e in order[:max(4, spec.E // 10)] if hist[e] > 0]
    assert len(hot) >= 2
    layer.set_hot_experts(hot)
    got, _ = run_all(layer, x, n1, T, nwin, ws1, wsw)
    bitwise_equal(got, ref)
    # the region is what is read: overwrite the pool's hot experts
    hot_t = torch.tensor(hot, dtype=torch.long, device="cuda")
    for f in ("w_gate", "w_up", "w_down"):
        t = getattr(dl, f)
        if t.dtype == torch.uint8:
            t[hot_t] = 0x88 ^ 0x5a                          # other 4-bit codes
        else:
            t[hot_t] = t[hot_t] * 3
    torch.cuda.synchronize()
    got2, _ = run_all(layer, x, n1, T, nwin, ws1, wsw)
    bitwise_equal(got2, ref)
    # control: the same pool without a region gives other outputs
    plain = SD.make_layer(dl, max_tokens=8, flags=MOE_LAYER_SCREEN_ON)
    other, _ = run_all(plain, x, n1, T, nwin, plain.workspace(1), plain.workspace(T))
    used = np.isin(ref[0], hot).any(axis=1)
    assert used.any()
    assert not np.array_equal(other[2][used], ref[2][used])
    # removing the region reads the (overwritten) pool again
    layer.set_hot_experts([])
    got3, _ = run_all(layer, x, n1, T, nwin, ws1, wsw)
    assert np.array_equal(got3[2].view(np.uint32), other[2].view(np.uint32))
    assert layer.device_error() == 0


def test_hot_region_refusals():
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd.binding import MoeError
    spec = SPECS["tiny_q4"]
    layer = SD.make_layer(SD.device_layer(spec), max_tokens=1)
    for ids in ([spec.E], [-1], [3, 3]):
        with pytest.raises(MoeError) as e:
            layer.set_hot_experts(ids)
        assert e.value.status == -6
    with pytest.raises(MoeError) as e:
        layer.set_hot_experts(list(range(spec.E + 1)))
    assert e.value.status == -6
    layer.set_hot_experts(list(range(spec.E)))          # every expert: allowed
    layer.set_hot_experts([])


def test_hot_region_fullsize_decode():
    """The 4-bit decode layer at full size: the region holds the 2,000 most
    chosen experts of 200 tokens; the next tokens' outputs equal those
    without a region bit for bit and the oracle's."""
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.CONFIGS["decode_q4"]
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=1)
    ws = layer.workspace(1)
    calib = SD.device_tokens(spec, 5000, 200)
    idx = torch.empty((200, spec.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((200, spec.k), dtype=torch.float32, device="cuda")
    out = torch.empty((200, spec.H), dtype=torch.float32, device="cuda")
    counts = torch.zeros(spec.E, dtype=torch.int32, device="cuda")
    for t in range(200):
        layer.grouped_forward(calib[t], 1, idx[t], gates[t], 0, out[t], ws)
    layer.expert_counts(idx, 200 * spec.k, counts)
    hist = counts.cpu().numpy()
    hot = [int(e) for e in np.lexsort((np.arange(spec.E), -hist))[:2000]]
    n = 16
    x = SD.device_tokens(spec, 6000, n)
    a = [G.run_grouped(layer, x[t:t + 1], ws=ws) for t in range(n)]
    layer.set_hot_experts(hot)
    b = [G.run_grouped(layer, x[t:t + 1], ws=ws) for t in range(n)]
    for u, v in zip(a, b):
        bitwise_equal(u, v)
    hits = np.isin(np.concatenate([u[0] for u in b]), hot).mean()
    print(f"full size: {100 * hits:.1f} % of the next {n} tokens' experts are in the region")
    G.note("hot region full size: oracle")
    L = G.host_oracle(spec)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 6000, n)
    G.compare(np.concatenate([u[0] for u in b]), np.concatenate([u[1] for u in b]),
              np.concatenate([u[2] for u in b]), o_idx, o_g, o_out, "hot region full size")
    assert layer.device_error() == 0
    del layer, dl


# ---------------------------------------------------------------- host tier
@pytest.mark.parametrize("name", list(SPECS))
def test_host_tier_against_oracle_and_relocated(name):
    """Experts moved to the host tier (the most chosen ones among them, so
    most tokens have host pairs): batch-1 decode, windows and
    moe_expert_decode as the oracle's; overwriting the device pool's copies
    of those experts afterwards changes nothing (the GPU reads zeros in
    their place, the host pool its own copies); with a hot region beside it
    the results are the same bits."""
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_ON
    from expert_routing_quantized_amd.binding import MoeError
    spec = SPECS[name]
    G.note("host tier", name)
    dl = cloned(SD.device_layer(spec))
    L = G.host_oracle(spec)
    n1, T, nwin = 20, 4, 3
    first = 700
    x = SD.device_tokens(spec, first, n1 + T * nwin)
    layer = SD.make_layer(dl, max_tokens=8, flags=MOE_LAYER_SCREEN_ON)
    ws1, wsw = layer.workspace(1), layer.workspace(T)
    ref, fi = run_all(layer, x, n1, T, nwin, ws1, wsw)
    hist = np.bincount(ref[0].ravel(), minlength=spec.E)
    order = np.lexsort((np.arange(spec.E), -hist))
    host = [int(e) for e in order[0:spec.E // 4:2]]          # every other of the most chosen
    hot = [int(e) for e in order[1:spec.E // 4:2]]
    layer.set_host_experts(host, n_threads=4)
    got, _ = run_all(layer, x, n1, T, nwin, ws1, wsw)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, first, n1 + T * nwin)
    G.compare(got[0], got[1], got[2], o_idx[:n1], o_g[:n1], o_out[:n1], f"{name} host tier batch 1")
    G.compare(got[3], got[4], got[5], o_idx[n1:], o_g[n1:], o_out[n1:], f"{name} host tier windows")
    G.compare(got[0], got[1], got[6], o_idx[:n1], o_g[:n1], o_out[:n1], f"{name} host tier expert_decode")
    assert np.isin(got[0], host).any(axis=1).mean() > 0.5
    # the device pool's copies of the host experts are not read any more
    host_t = torch.tensor(host, dtype=torch.long, device="cuda")
    for f in ("w_gate", "w_up", "w_down"):
        t = getattr(dl, f)
        if t.dtype == torch.uint8:
            t[host_t] = 0x77
        else:
            t[host_t] = t[host_t] * 5
    torch.cuda.synchronize()
    got2, _ = run_all(layer, x, n1, T, nwin, ws1, wsw)
    bitwise_equal(got2, got)
    # a hot region beside the host tier (disjoint sets; overlap refused)
    with pytest.raises(MoeError):
        layer.set_hot_experts(host[:1])
    layer.set_hot_experts(hot)
    got3, _ = run_all(layer, x, n1, T, nwin, ws1, wsw)
    bitwise_equal(got3, got)
    with pytest.raises(MoeError) as e:                      # calls above floor(256 / k) tokens
        layer.grouped_forward(x, 256 // spec.k + 1, None, None, 0,
                              torch.empty((1,), device="cuda"), layer.workspace(8))
    assert e.value.status == -6
    layer.set_host_experts([])
    layer.set_hot_experts([])
    assert layer.device_error() == 0


def test_host_tier_graph_replays():
    """Batch-1 calls with host-tier experts captured in a graph (a host node
    on a second stream): every replay, with eager calls in between, gives
    the eager calls' bits."""
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_ON
    spec = SPECS["wide_q4"]
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=1, flags=MOE_LAYER_SCREEN_ON)
    layer.set_host_experts(list(range(0, spec.E, 3)))
    n = 6
    x = SD.device_tokens(spec, 40, n)
    ws = layer.workspace(1)
    idx = torch.empty((n, spec.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((n, spec.k), dtype=torch.float32, device="cuda")
    out = torch.empty((n, spec.H), dtype=torch.float32, device="cuda")
    for t in range(n):
        layer.grouped_forward(x[t], 1, idx[t], gates[t], 0, out[t], ws)
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for t in range(n):
                layer.grouped_forward(x[t], 1, idx[t], gates[t], 0, out[t], ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {rep}"
        eager = G.run_grouped(layer, x[rep:rep + 1], ws=ws)
        assert np.array_equal(eager[2].view(np.uint32), ref[rep:rep + 1].cpu().numpy().view(np.uint32))
    assert layer.device_error() == 0


def test_host_tier_fullsize_decode():
    """The 4-bit decode layer at full size with 300 experts (among them the
    100 most chosen over 200 tokens) on the host: 16 tokens as the oracle's."""
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.CONFIGS["decode_q4"]
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=1)
    ws = layer.workspace(1)
    calib = SD.device_tokens(spec, 5000, 200)
    idx = torch.empty((200, spec.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((200, spec.k), dtype=torch.float32, device="cuda")
    out = torch.empty((200, spec.H), dtype=torch.float32, device="cuda")
    counts = torch.zeros(spec.E, dtype=torch.int32, device="cuda")
    for t in range(200):
        layer.grouped_forward(calib[t], 1, idx[t], gates[t], 0, out[t], ws)
    layer.expert_counts(idx, 200 * spec.k, counts)
    order = np.lexsort((np.arange(spec.E), -counts.cpu().numpy()))
    host = [int(e) for e in order[:100]] + [int(e) for e in order[-200:]]
    layer.set_host_experts(host)
    n = 16
    x = SD.device_tokens(spec, 7000, n)
    b = [G.run_grouped(layer, x[t:t + 1], ws=ws) for t in range(n)]
    gi = np.concatenate([u[0] for u in b])
    print(f"full size: {100 * np.isin(gi, host).any(axis=1).mean():.0f} % of tokens have host pairs")
    G.note("host tier full size: oracle")
    L = G.host_oracle(spec)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 7000, n)
    G.compare(gi, np.concatenate([u[1] for u in b]), np.concatenate([u[2] for u in b]), o_idx, o_g, o_out,
              "host tier full size")
    assert layer.device_error() == 0
    del layer, dl
