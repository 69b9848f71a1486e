"""The router's int8 first pass (screen) on the GPU: its per-expert error
bound holds for every expert, and routing through it gives the oracle's
indices and gates -- at full size, on small layers that force it on, and on
the edge cases (ties, near ties, all-equal logits, tiny and non-finite
hidden states).  The batch-1 fused kernel's output must equal moe_route +
moe_expert_decode bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_q4": synth.small_spec(H=256, E=200, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=23, token_seed=24, name="tiny_q4"),
    "tiny_bf16": synth.small_spec(H=256, E=200, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_BF16,
                                  bias_alpha=0.37, weight_seed=21, token_seed=22, name="tiny_bf16"),
    "wide_q4": synth.small_spec(H=2048, E=130, k=10, I=256, act=synth.DT_BF16, expert=synth.DT_Q4,
                                bias_alpha=0.37, weight_seed=25, token_seed=26, name="wide_q4"),
    "odd_q4": synth.small_spec(H=96, E=70, k=3, I=32, act=synth.DT_BF16, expert=synth.DT_Q4,
                               bias_alpha=None, weight_seed=27, token_seed=28, name="odd_q4"),
    "q4_h4096": synth.small_spec(H=4096, E=70, k=8, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                                 bias_alpha=0.37, weight_seed=83, token_seed=84, name="q4_h4096"),
    "k20_q4": synth.small_spec(H=512, E=3000, k=20, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                               bias_alpha=0.37, weight_seed=53, token_seed=54, name="k20_q4"),
}
_cache = {}


def setup(name):
    if name not in _cache:
        import synth.device as SD
        spec = SMALL[name]
        _cache[name] = (spec, SD.device_layer(spec), G.host_oracle(spec))
    return _cache[name]


def screen_flags(extra=0):
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_ON
    return MOE_LAYER_SCREEN_ON | extra


def per_token(layer, x, n):
    """moe_grouped_forward one token at a time, then moe_route +
    moe_expert_decode one token at a time (both T = 1, the screened path)."""
    torch = G.torch_mod()
    dev = x.device
    ws = layer.workspace(1)
    fi = torch.empty((n, layer.k), dtype=torch.int32, device=dev)
    fg = torch.empty((n, layer.k), dtype=torch.float32, device=dev)
    fo = torch.empty((n, layer.H), dtype=torch.float32, device=dev)
    si, sg, so = torch.empty_like(fi), torch.empty_like(fg), torch.empty_like(fo)
    for t in range(n):
        layer.grouped_forward(x[t], 1, fi[t], fg[t], 0, fo[t], ws)
        layer.route(x[t], 1, si[t], sg[t], ws)
        layer.expert_decode(x[t], si[t], sg[t], so[t], ws)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (fi, fg, fo, si, sg, so)]


def check_bitwise(fi, fg, fo, si, sg, so):
    assert np.array_equal(fi, si)
    assert np.array_equal(fg.view(np.uint32), sg.view(np.uint32))
    assert np.array_equal(fo.view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("exact", [False, True])
def test_screened_decode_small(name, exact):
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_FORCE_EXACT_REFINE
    spec, dl, L = setup(name)
    G.note("screen small", name, exact)
    n = 8 if exact else 24
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags(MOE_LAYER_FORCE_EXACT_REFINE if exact else 0))
    x = SD.device_tokens(spec, 300, n)
    fi, fg, fo, si, sg, so = per_token(layer, x, n)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 300, n)
    G.compare(fi, fg, fo, o_idx, o_g, o_out, f"screen {name}")
    check_bitwise(fi, fg, fo, si, sg, so)
    assert layer.device_error() == 0
    if exact:      # every selection refined its candidates exactly (moe_layer_stats counts them)
        assert layer.exact_refinements() >= 2 * n * spec.k


def _exact_logits(spec, first, n, R=None, b=None):
    X = oracle.tokens_f64(spec, first, n)
    if R is None:
        L = oracle.layer_from_spec(spec)
        R, b = L.R, L.b
    return X, X @ R + b[None, :]


@pytest.mark.parametrize("name", ["tiny_q4", "wide_q4", "odd_q4", "q4_h4096"])
def test_screen_bound_small(name):
    """|v - z| <= bound for every expert of 16 tokens (z: float64, whose own
    error is below 1e-12 here)."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, _ = setup(name)
    layer = SD.make_layer(dl, max_tokens=16, flags=screen_flags())
    x = SD.device_tokens(spec, 40, 16)
    v = torch.empty((16, spec.E), dtype=torch.float32, device="cuda")
    bd = torch.empty_like(v)
    layer.router_screen(x, 16, v, bd, layer.workspace(16))
    torch.cuda.synchronize()
    _, Z = _exact_logits(spec, 40, 16)
    err = np.abs(v.cpu().numpy().astype(np.float64) - Z)
    ratio = err / bd.cpu().numpy()
    print(f"{name}: screen |err|/bound max {ratio.max():.3f}, bound mean {bd.cpu().numpy().mean():.3e}")
    assert ratio.max() < 1.0


def test_screen_bound_fullsize():
    """The 4-bit decode layer at full size: every expert of 6 tokens."""
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.CONFIGS["decode_q4"]
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=6, flags=screen_flags())
    x = SD.device_tokens(spec, 10, 6)
    v = torch.empty((6, spec.E), dtype=torch.float32, device="cuda")
    bd = torch.empty_like(v)
    layer.router_screen(x, 6, v, bd, layer.workspace(6))
    torch.cuda.synchronize()
    G.note("screen bound full size: oracle logits")
    _, Z = _exact_logits(spec, 10, 6)
    vv, bb = v.cpu().numpy().astype(np.float64), bd.cpu().numpy().astype(np.float64)
    err = np.abs(vv - Z)
    ratio = err / bb
    # experts the bound leaves undecided (what the selection recomputes)
    k = spec.k
    lo = np.sort(vv - bb, axis=1)[:, -k]
    ncand = ((vv + bb) >= lo[:, None]).sum(axis=1)
    print(f"full size: |err|/bound max {ratio.max():.3f}; bound mean {bb.mean():.3f}; "
          f"max |err| {err.max():.3e}; experts left undecided per token {ncand.tolist()}")
    assert ratio.max() < 1.0
    assert ncand.max() <= 256
    del layer, dl


def test_screen_ties_and_near_ties():
    """Copies of the rank-1 and rank-k-1 experts (exact ties: lower index
    first) and a row one bf16 ulp from the top expert, routed through the
    screen (their screen values are equal or nearly so, and the recomputed
    logits decide)."""
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.small_spec(H=256, E=96, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_BF16,
                            bias_alpha=None, weight_seed=43, token_seed=44, name="inv_bf16")
    dl = SD.device_layer(spec)
    x = SD.device_tokens(spec, 0, 6)
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    idx0, _, _ = G.run_grouped(layer, x[0:1])
    top = [int(v) for v in idx0[0]]
    R = dl.router_eh.clone()
    used = set(top)
    for src, shift in ((top[1], 9), (top[spec.k - 1], -5)):
        dst = (src + shift) % spec.E
        while dst in used:
            dst = (dst + 1) % spec.E
        R[dst] = R[src]
        used.add(dst)
    near = (top[0] + 3) % spec.E
    while near in used:
        near = (near + 1) % spec.E
    R[near] = R[top[0]]
    R[near].view(torch.int16)[37] += 1
    dl2 = SD.DeviceLayer(spec, R, dl.bias, dl.w_gate, dl.w_up, dl.w_down)
    layer2 = SD.make_layer(dl2, max_tokens=1, flags=screen_flags())
    fi, fg, fo, si, sg, so = per_token(layer2, x, 6)
    Rh = oracle.decode_bf16(SD.to_numpy_bits(R)).T
    L = oracle.OracleLayer(Rh, np.zeros(spec.E), spec.k, lambda e, w: synth.expert_stored(spec, e, w))
    o_idx, o_g, _, o_out = oracle.moe_tokens(oracle.tokens_f64(spec, 0, 6), L)
    G.compare(fi, fg, fo, o_idx, o_g, o_out, "screen ties")
    check_bitwise(fi, fg, fo, si, sg, so)
    assert layer2.device_error() == 0


def test_screen_all_equal_logits():
    """x = 0, no bias: 3000 equal logits -- the screen decides nothing and
    the selection falls back to scanning every screen value."""
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.small_spec(H=256, E=3000, k=6, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                            bias_alpha=None, weight_seed=51, token_seed=52, name="equal")
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    x = torch.zeros((2, spec.H), dtype=torch.bfloat16, device="cuda")
    fi, fg, fo, si, sg, so = per_token(layer, x, 2)
    assert np.array_equal(fi, np.tile(np.arange(spec.k), (2, 1)))
    assert np.all(fg == np.float32(1.0 / spec.k))
    assert np.all(fo == 0.0)
    check_bitwise(fi, fg, fo, si, sg, so)
    assert layer.device_error() == 0


def test_screen_nan_hidden_state():
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, L = setup("tiny_q4")
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    x = SD.device_tokens(spec, 0, 3)
    x[1, 17] = float("nan")
    fi, fg, fo, si, sg, so = per_token(layer, x, 3)
    assert layer.device_error() & 4
    for a in (fi, si):
        assert np.all(a[1] == -1)
    for a in (fg, fo, sg, so):
        assert np.all(np.isnan(a[1]))
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 0, 3)
    G.compare(fi[[0, 2]], fg[[0, 2]], fo[[0, 2]], o_idx[[0, 2]], o_g[[0, 2]], o_out[[0, 2]], "screen nan/others")


def test_screen_tiny_hidden_state():
    """Hidden states scaled by 2^-80 through the screen: routing as the oracle's."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, L = setup("tiny_q4")
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    scale = 2.0 ** -80
    x = (SD.device_tokens(spec, 0, 8).float() * scale).to(torch.bfloat16)
    Xh = oracle.tokens_f64(spec, 0, 8) * scale
    assert np.array_equal(oracle.decode_bf16(SD.to_numpy_bits(x)), Xh)
    fi, fg, fo, si, sg, so = per_token(layer, x, 8)
    o_idx, o_g, _, _ = oracle.moe_tokens(Xh, L)
    G.compare(fi, fg, None, o_idx, o_g, None, "screen tiny x")
    check_bitwise(fi, fg, fo, si, sg, so)
    assert layer.device_error() == 0


def test_screen_off_flag_and_refusals():
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_OFF, MOE_LAYER_SCREEN_ON
    from expert_routing_quantized_amd.binding import MoeError
    spec, dl, L = setup("tiny_q4")
    off = SD.make_layer(dl, max_tokens=1, flags=MOE_LAYER_SCREEN_OFF)
    x = SD.device_tokens(spec, 0, 1)
    v = torch.empty((1, spec.E), dtype=torch.float32, device="cuda")
    with pytest.raises(MoeError) as e:
        off.router_screen(x, 1, v, None, off.workspace(1))
    assert e.value.status == -3
    with pytest.raises(MoeError) as e:
        SD.make_layer(dl, max_tokens=1, flags=MOE_LAYER_SCREEN_ON | MOE_LAYER_SCREEN_OFF)
    assert e.value.status == -6
    f32 = synth.CONFIGS["tiny_f32"]
    with pytest.raises(MoeError) as e:
        SD.make_layer(SD.device_layer(f32), max_tokens=1, flags=MOE_LAYER_SCREEN_ON)
    assert e.value.status == -3


# ---------------------------------------------------------------- the list
HINT_BYTES = 128


def hint_state(ws):
    """The batch-1 list's state at the start of the workspace: call counter,
    calls whose selection took the table, and the ring of recent k-th logits."""
    b = ws[:HINT_BYTES].cpu().numpy()
    return int(b[0:8].view(np.uint64)[0]), int(b[12:16].view(np.uint32)[0]), b[64:128].view(np.float32).copy()


def poison_ring(ws, value):
    torch = G.torch_mod()
    ws[64:128].view(torch.float32).fill_(value)


def grouped_tokens(layer, x, n, ws, before=None):
    torch = G.torch_mod()
    fi = torch.empty((n, layer.k), dtype=torch.int32, device=x.device)
    fg = torch.empty((n, layer.k), dtype=torch.float32, device=x.device)
    fo = torch.empty((n, layer.H), dtype=torch.float32, device=x.device)
    for t in range(n):
        if before is not None:
            before(t)
        layer.grouped_forward(x[t], 1, fi[t], fg[t], 0, fo[t], ws)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (fi, fg, fo)]


@pytest.mark.parametrize("name", ["wide_q4", "k20_q4", "tiny_bf16", "q4_h4096"])
def test_list_taken_and_equal_to_the_full_screen_path(name):
    """Most calls select from the screen's table once the ring has warmed up;
    the results equal, bit for bit, those of calls whose ring is poisoned
    (theta = +inf: no table), and the oracle's."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, L = setup(name)
    G.note("list", name)
    n = 24
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    x = SD.device_tokens(spec, 500, n)
    ws = layer.workspace(1)
    ws.zero_()
    fi, fg, fo = grouped_tokens(layer, x, n, ws)
    ep, listed, ring = hint_state(ws)
    print(f"{name}: {listed} of {n} calls took the table; ring {ring[:4]}")
    assert ep == n and listed >= n // 2
    ws2 = layer.workspace(1)
    ws2.zero_()
    gi, gg, go = grouped_tokens(layer, x, n, ws2, before=lambda t: poison_ring(ws2, float("nan")))
    assert hint_state(ws2)[1] == 0
    check_bitwise(fi, fg, fo, gi, gg, go)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 500, n)
    G.compare(fi, fg, fo, o_idx, o_g, o_out, f"list {name}")
    assert layer.device_error() == 0


def test_list_route_path_and_low_theta():
    """moe_route through the table equals the grouped forward; a ring far
    below the logits lists every expert (table full: the full path)."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, L = setup("k20_q4")
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    x = SD.device_tokens(spec, 900, 12)
    fi, fg, fo, si, sg, so = per_token(layer, x, 12)
    check_bitwise(fi, fg, fo, si, sg, so)
    ws = layer.workspace(1)
    ws.zero_()
    gi, gg, go = grouped_tokens(layer, x, 12, ws, before=lambda t: poison_ring(ws, -1e30))
    assert hint_state(ws)[1] == 0
    check_bitwise(fi, fg, fo, gi, gg, go)


def test_list_counter_not_reset():
    """A list counter that did not start the call at 0 (as a workspace's
    first use may leave it) makes that call select without the list, with
    the same result; the call sets it back, so the next one uses the list."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, L = setup("wide_q4")
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    x = SD.device_tokens(spec, 700, 8)
    ref = grouped_tokens(layer, x, 8, layer.workspace(1))
    ws = layer.workspace(1)
    ws.zero_()
    for t in range(8):
        if t % 2 == 1:
            ws[16:20].view(torch.int32).fill_(3 + t)        # the list's counter
        _, listed0, _ = hint_state(ws)
        r = grouped_tokens(layer, x[t:t + 1], 1, ws)
        check_bitwise(*r, *[a[t:t + 1] for a in ref])
        _, listed1, _ = hint_state(ws)
        assert int(ws[16:20].view(torch.int32).item()) == 0
        if t % 2 == 1:
            assert listed1 == listed0
    assert hint_state(ws)[1] >= 2


def test_list_garbage_workspace():
    """A workspace full of random bytes: correct results from the first call."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, L = setup("tiny_q4")
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    x = SD.device_tokens(spec, 40, 10)
    ws = layer.workspace(1)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=g))
    fi, fg, fo = grouped_tokens(layer, x, 10, ws)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 40, 10)
    G.compare(fi, fg, fo, o_idx, o_g, o_out, "list garbage ws")
    assert layer.device_error() == 0


def test_list_fullsize_decode():
    """The 4-bit decode layer at full size: the table serves most tokens and
    routing equals the oracle's."""
    torch = G.torch_mod()
    import synth.device as SD
    spec = synth.CONFIGS["decode_q4"]
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=1, flags=screen_flags())
    n = 48
    x = SD.device_tokens(spec, 2000, n)
    ws = layer.workspace(1)
    ws.zero_()
    fi, fg, fo = grouped_tokens(layer, x, n, ws)
    ep, listed, ring = hint_state(ws)
    print(f"full size: {listed} of {n} calls took the table; ring min {ring.min():.4f} max {ring.max():.4f}")
    assert listed >= n * 3 // 4
    G.note("list full size: oracle")
    L = G.host_oracle(spec)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 2000, 8)
    G.compare(fi[:8], fg[:8], fo[:8], o_idx, o_g, o_out, "list full size")
    assert layer.device_error() == 0
    del layer, dl


@pytest.mark.parametrize("name", ["tiny_q4", "wide_q4", "odd_q4", "q4_h4096"])
@pytest.mark.parametrize("T", [2, 3, 5, 8])
def test_windows_and_batch1_share_a_screened_workspace(name, T):
    """On a layer with the screen, verify windows (2 <= T <= 8: the window
    screen with its per-token lists, or the bf16 router past H = 2048) and
    batch-1 calls (the screen with its list) alternate through one
    workspace: every window and every single token against the oracle,
    moe_grouped_forward and moe_route."""
    import synth.device as SD
    spec, dl, L = setup(name)
    G.note("screened layer, windows and batch 1", name, T)
    layer = SD.make_layer(dl, max_tokens=8, flags=screen_flags())
    first = 700 + 11 * T
    n = 3 * T + 3
    x = SD.device_tokens(spec, first, n)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, first, n)
    ws = layer.workspace(T)
    pos = 0
    for w in range(3):
        sl = slice(pos, pos + T)
        fi, fg, fo = G.run_grouped(layer, x[sl], ws=ws)
        G.compare(fi, fg, fo, o_idx[sl], o_g[sl], o_out[sl], f"window {name} T={T} w={w}")
        ri, rg, _ = G.run_route_decode(layer, x[sl], ws=ws)
        G.compare(ri, rg, None, o_idx[sl], o_g[sl], None, f"window route {name} T={T} w={w}")
        pos += T
        one = slice(pos, pos + 1)            # then one batch-1 token through the same workspace
        fi, fg, fo = G.run_grouped(layer, x[one], ws=ws)
        G.compare(fi, fg, fo, o_idx[one], o_g[one], o_out[one], f"batch 1 after window {name} T={T} w={w}")
        pos += 1
    assert layer.device_error() == 0


# ---------------------------------------------------------------- windows
WIN_T = [2, 4, 5, 6, 8]   # 4-6: the deeper slab ring at H = 2048
WIN_COUNTS = slice(20, 52)      # the windows' per-token list counters in the hint


def windows(layer, x, T, nwin, ws, before=None):
    """nwin consecutive windows of T tokens through moe_grouped_forward."""
    torch = G.torch_mod()
    n = nwin * T
    fi = torch.empty((n, layer.k), dtype=torch.int32, device=x.device)
    fg = torch.empty((n, layer.k), dtype=torch.float32, device=x.device)
    fo = torch.empty((n, layer.H), dtype=torch.float32, device=x.device)
    for w in range(nwin):
        if before is not None:
            before(w)
        sl = slice(w * T, (w + 1) * T)
        layer.grouped_forward(x[sl], T, fi[sl], fg[sl], 0, fo[sl], ws)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (fi, fg, fo)]


@pytest.mark.parametrize("name", ["tiny_q4", "wide_q4", "odd_q4", "k20_q4"])
@pytest.mark.parametrize("T", WIN_T)
def test_window_screen_values_equal_batch1(name, T):
    """The window screen (all T tokens in one pass, on the matrix cores)
    gives every expert of every token the value the batch-1 screen gives it,
    bit for bit, and its bounds hold against the float64 logits."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, _ = setup(name)
    G.note("window screen values", name, T)
    layer = SD.make_layer(dl, max_tokens=8, flags=screen_flags())
    first = 60 + T
    x = SD.device_tokens(spec, first, T)
    v = torch.empty((T, spec.E), dtype=torch.float32, device="cuda")
    bd = torch.empty_like(v)
    layer.router_screen(x, T, v, bd, layer.workspace(T))
    v1 = torch.empty_like(v)
    b1 = torch.empty_like(v)
    ws1 = layer.workspace(1)
    for t in range(T):
        layer.router_screen(x[t], 1, v1[t], b1[t], ws1)
    torch.cuda.synchronize()
    vw, v1h = v.cpu().numpy(), v1.cpu().numpy()
    assert np.array_equal(vw.view(np.uint32), v1h.view(np.uint32))
    _, Z = _exact_logits(spec, first, T)
    ratio = np.abs(vw.astype(np.float64) - Z) / bd.cpu().numpy()
    print(f"{name} T={T}: window screen |err|/bound max {ratio.max():.3f}")
    assert ratio.max() < 1.0
    assert layer.device_error() == 0


@pytest.mark.parametrize("name", ["tiny_q4", "wide_q4", "k20_q4", "tiny_bf16"])
@pytest.mark.parametrize("T", WIN_T)
def test_window_lists_taken_and_equal_to_the_full_screen_path(name, T):
    """Windows on the screen select from their per-token lists once the ring
    has warmed up; the results equal, bit for bit, those of windows whose
    ring is poisoned (no lists), and the oracle's; each call leaves the
    counters at 0."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, L = setup(name)
    G.note("window lists", name, T)
    nwin = 10
    layer = SD.make_layer(dl, max_tokens=8, flags=screen_flags())
    x = SD.device_tokens(spec, 900, nwin * T)
    ws = layer.workspace(T)
    ws.zero_()
    fi, fg, fo = windows(layer, x, T, nwin, ws)
    ep, listed, ring = hint_state(ws)
    print(f"{name} T={T}: {listed} of {nwin} windows took the lists")
    assert ep == nwin and listed >= nwin // 2
    assert np.all(ws[WIN_COUNTS].cpu().numpy() == 0)
    ws2 = layer.workspace(T)
    ws2.zero_()
    gi, gg, go = windows(layer, x, T, nwin, ws2, before=lambda w: poison_ring(ws2, float("nan")))
    assert hint_state(ws2)[1] == 0
    check_bitwise(fi, fg, fo, gi, gg, go)
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 900, nwin * T)
    G.compare(fi, fg, fo, o_idx, o_g, o_out, f"window lists {name} T={T}")
    assert layer.device_error() == 0


@pytest.mark.parametrize("T", WIN_T)
def test_window_screen_off_flag_same_routing(T):
    """MOE_LAYER_WINDOW_SCREEN_OFF routes windows on the bf16 router: the
    same indices as the window screen, gates within the tolerance."""
    from expert_routing_quantized_amd import MOE_LAYER_WINDOW_SCREEN_OFF
    import synth.device as SD
    spec, dl, L = setup("wide_q4")
    on = SD.make_layer(dl, max_tokens=8, flags=screen_flags())
    off = SD.make_layer(dl, max_tokens=8, flags=screen_flags(MOE_LAYER_WINDOW_SCREEN_OFF))
    x = SD.device_tokens(spec, 1300, 4 * T)
    a = windows(on, x, T, 4, on.workspace(T))
    b = windows(off, x, T, 4, off.workspace(T))
    assert np.array_equal(a[0], b[0])
    o_idx, o_g, _, o_out = G.oracle_tokens(spec, L, 1300, 4 * T)
    G.compare(*a, o_idx, o_g, o_out, f"window screen on T={T}")
    G.compare(*b, o_idx, o_g, o_out, f"window screen off T={T}")


@pytest.mark.parametrize("T", [3, 6])
def test_window_counters_not_reset_and_garbage_workspace(T):
    """Window counters that did not start at 0, and a workspace of random
    bytes: the same results (those calls select without the lists), and
    the window's counters are back at 0 after the calls."""
    torch = G.torch_mod()
    import synth.device as SD
    spec, dl, L = setup("wide_q4")
    G.note("window counters", T)
    layer = SD.make_layer(dl, max_tokens=8, flags=screen_flags())
    nwin = 6
    x = SD.device_tokens(spec, 1700, nwin * T)
    ref = windows(layer, x, T, nwin, layer.workspace(T))
    ws = layer.workspace(T)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=g))

    def bump(w):
        if w % 2 == 1:
            ws[WIN_COUNTS].view(torch.int32).fill_(5 + w)
    r = windows(layer, x, T, nwin, ws, before=bump)
    check_bitwise(*r, *ref)
    # the call clears the counters of its own tokens (those past T keep what they held)
    assert np.all(ws[WIN_COUNTS].view(torch.int32).cpu().numpy()[:T] == 0)
    assert layer.device_error() == 0


@pytest.mark.parametrize("T", [2, 5, 8])
def test_window_screen_edges(T):
    """Windows through the screen: exact ties and a near tie (copied router
    rows), a window of all-zero hidden states (every logit equal), a
    non-finite token inside a window, and hidden states scaled by 2^-80."""
    torch = G.torch_mod()
    import synth.device as SD
    G.note("window edges", T)
    # ties: copies of ranked experts and a row one bf16 ulp from the top one
    spec = synth.small_spec(H=256, E=96, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_BF16,
                            bias_alpha=None, weight_seed=43, token_seed=44, name="inv_bf16")
    dl = SD.device_layer(spec)
    x = SD.device_tokens(spec, 0, T)
    layer = SD.make_layer(dl, max_tokens=8, flags=screen_flags())
    idx0, _, _ = G.run_grouped(layer, x[0:1])
    top = [int(v) for v in idx0[0]]
    R = dl.router_eh.clone()
    used = set(top)
    for src, shift in ((top[1], 9), (top[spec.k - 1], -5)):
        dst = (src + shift) % spec.E
        while dst in used:
            dst = (dst + 1) % spec.E
        R[dst] = R[src]
        used.add(dst)
    near = (top[0] + 3) % spec.E
    while near in used:
        near = (near + 1) % spec.E
    R[near] = R[top[0]]
    R[near].view(torch.int16)[37] += 1
    dl2 = SD.DeviceLayer(spec, R, dl.bias, dl.w_gate, dl.w_up, dl.w_down)
    layer2 = SD.make_layer(dl2, max_tokens=8, flags=screen_flags())
    fi, fg, fo = G.run_grouped(layer2, x)
    Rh = oracle.decode_bf16(SD.to_numpy_bits(R)).T
    L2 = oracle.OracleLayer(Rh, np.zeros(spec.E), spec.k, lambda e, w: synth.expert_stored(spec, e, w))
    o_idx, o_g, _, o_out = oracle.moe_tokens(oracle.tokens_f64(spec, 0, T), L2)
    G.compare(fi, fg, fo, o_idx, o_g, o_out, f"window ties T={T}")
    assert layer2.device_error() == 0
    # all-zero hidden states: every logit equal, the lower indices win
    spec_e = synth.small_spec(H=256, E=3000, k=6, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                              bias_alpha=None, weight_seed=51, token_seed=52, name="equal")
    le = SD.make_layer(SD.device_layer(spec_e), max_tokens=8, flags=screen_flags())
    fi, fg, fo = G.run_grouped(le, torch.zeros((T, spec_e.H), dtype=torch.bfloat16, device="cuda"))
    assert np.array_equal(fi, np.tile(np.arange(spec_e.k), (T, 1)))
    assert np.all(fg == np.float32(1.0 / spec_e.k)) and np.all(fo == 0.0)
    assert le.device_error() == 0
    # a non-finite token inside the window; the others as the oracle's
    spec_t, dl_t, L_t = setup("tiny_q4")
    lt = SD.make_layer(dl_t, max_tokens=8, flags=screen_flags())
    x = SD.device_tokens(spec_t, 0, T)
    bad = T // 2
    x[bad, 17] = float("nan")
    fi, fg, fo = G.run_grouped(lt, x)
    assert lt.device_error() & 4
    assert np.all(fi[bad] == -1) and np.all(np.isnan(fg[bad])) and np.all(np.isnan(fo[bad]))
    keep = [t for t in range(T) if t != bad]
    o_idx, o_g, _, o_out = G.oracle_tokens(spec_t, L_t, 0, T)
    G.compare(fi[keep], fg[keep], fo[keep], o_idx[keep], o_g[keep], o_out[keep], f"window nan/others T={T}")
    # hidden states scaled by 2^-80
    scale = 2.0 ** -80
    x = (SD.device_tokens(spec_t, 0, T).float() * scale).to(torch.bfloat16)
    Xh = oracle.tokens_f64(spec_t, 0, T) * scale
    assert np.array_equal(oracle.decode_bf16(SD.to_numpy_bits(x)), Xh)
    fi, fg, fo = G.run_grouped(lt, x)
    o_idx, o_g, _, _ = oracle.moe_tokens(Xh, L_t)
    G.compare(fi, fg, None, o_idx, o_g, None, f"window tiny x T={T}")
    assert lt.device_error() == 0
