"""Invariants of the GPU path that hold without the oracle, plus the
device-side fault reporting: linearity in the gates, zeroing unselected
experts, relabelling of experts, grouped rows versus single tokens,
determinism, exact ties, and bad caller indices."""
import numpy as np
import pytest

import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SPEC = synth.small_spec(H=512, E=150, k=6, I=64, act=synth.DT_BF16, expert=synth.DT_Q4,
                        bias_alpha=0.37, weight_seed=41, token_seed=42, name="inv_q4")
SPEC_BF = synth.small_spec(H=256, E=96, k=4, I=64, act=synth.DT_BF16, expert=synth.DT_BF16,
                           bias_alpha=None, weight_seed=43, token_seed=44, name="inv_bf16")


def dev(spec):
    import synth.device as SD
    return SD.device_layer(spec)


def test_linearity_in_gates():
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_ROUTE_GIVEN
    dl = dev(SPEC)
    layer = SD.make_layer(dl, max_tokens=8)
    x = SD.device_tokens(SPEC, 0, 8)
    idx, gates, out = G.run_grouped(layer, x)
    it = torch.from_numpy(idx).cuda()
    g1 = torch.from_numpy(gates).cuda()
    g2 = torch.rand_like(g1)
    _, _, o_a = G.run_grouped(layer, x, MOE_ROUTE_GIVEN, it, 2.0 * g1)
    _, _, o_s = G.run_grouped(layer, x, MOE_ROUTE_GIVEN, it, g1 + g2)
    _, _, o_2 = G.run_grouped(layer, x, MOE_ROUTE_GIVEN, it, g2)
    assert np.array_equal(o_a, 2.0 * out)                 # power-of-two scaling is exact
    assert np.all(G.rel_l2(o_s, out + o_2) < 1e-5)


def test_zeroing_unselected_experts_is_bitwise_neutral():
    torch = G.torch_mod()
    import synth.device as SD
    dl = dev(SPEC)
    x = SD.device_tokens(SPEC, 0, 6)
    layer = SD.make_layer(dl, max_tokens=6)
    idx, gates, out = G.run_route_decode(layer, x)
    _, _, out_g = G.run_grouped(layer, x)
    used = np.unique(idx)
    mask = torch.ones(SPEC.E, dtype=torch.bool)
    mask[torch.from_numpy(used).long()] = False
    for t in (dl.w_gate, dl.w_up, dl.w_down):
        t[mask.cuda()] = 0x88 if t.dtype == torch.uint8 else 0
    for t in (dl.s_gate, dl.s_up, dl.s_down):
        t[mask.cuda()] = 0
    layer2 = SD.make_layer(dl, max_tokens=6)
    idx2, gates2, out2 = G.run_route_decode(layer2, x)
    _, _, out2_g = G.run_grouped(layer2, x)
    assert np.array_equal(idx2, idx) and np.array_equal(gates2, gates)
    assert np.array_equal(out2, out) and np.array_equal(out2_g, out_g)


def test_relabelling_experts():
    torch = G.torch_mod()
    import synth.device as SD
    dl = dev(SPEC)
    x = SD.device_tokens(SPEC, 0, 6)
    idx, gates, out = G.run_route_decode(SD.make_layer(dl, max_tokens=6), x)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(SPEC.E)).cuda()
    inv = torch.argsort(perm)
    # new expert perm[e] holds old expert e  ->  new tensor[j] = old[inv[j]]
    dl2 = SD.DeviceLayer(SPEC, dl.router_eh[inv].contiguous(), dl.bias[inv].contiguous(),
                         dl.w_gate[inv].contiguous(), dl.w_up[inv].contiguous(),
                         dl.w_down[inv].contiguous(), dl.s_gate[inv].contiguous(),
                         dl.s_up[inv].contiguous(), dl.s_down[inv].contiguous())
    idx2, gates2, out2 = G.run_route_decode(SD.make_layer(dl2, max_tokens=6), x)
    assert np.array_equal(idx2, perm.cpu().numpy()[idx])
    assert np.array_equal(gates2, gates) and np.array_equal(out2, out)


@pytest.mark.parametrize("spec", [SPEC, SPEC_BF], ids=["q4", "bf16"])
def test_grouped_rows_match_single_tokens_and_determinism(spec):
    import synth.device as SD
    dl = dev(spec)
    T = 29
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(spec, 50, T)
    idx_s, g_s, out_s = G.run_route_decode(layer, x)
    idx_g, g_g, out_g = G.run_grouped(layer, x)
    assert np.array_equal(idx_s, idx_g) and np.array_equal(g_s, g_g)
    assert np.all(G.rel_l2(out_g, out_s) < 1e-5)
    idx_g2, g_g2, out_g2 = G.run_grouped(layer, x)
    assert np.array_equal(idx_g2, idx_g) and np.array_equal(out_g2, out_g)   # bitwise determinism
    _, _, out_s2 = G.run_route_decode(layer, x)
    assert np.array_equal(out_s2, out_s)


def test_exact_ties_and_near_ties_follow_the_oracle():
    """Duplicated router rows (exact ties: lower index first) and rows one
    bf16 ulp apart in one element (near ties decided by the exact logits)."""
    torch = G.torch_mod()
    import oracle
    import synth.device as SD
    spec = SPEC_BF
    dl = dev(spec)
    R = dl.router_eh.clone()
    x = SD.device_tokens(spec, 0, 8)
    # find, for token 0, its top expert and make copies of it at higher and lower indices
    layer = SD.make_layer(dl, max_tokens=8)
    idx0, _, _ = G.run_route_decode(layer, x)
    top = int(idx0[0, 0])
    R[(top + 17) % spec.E] = R[top]
    R[(top + 41) % spec.E] = R[top]
    near = (top + 5) % spec.E
    R[near] = R[top]
    bits = R[near].view(torch.int16)
    bits[100] += 1                      # one ulp in one element: a tiny exact difference
    dl2 = SD.DeviceLayer(spec, R, dl.bias, dl.w_gate, dl.w_up, dl.w_down)
    layer2 = SD.make_layer(dl2, max_tokens=8)
    idx, gates, out = G.run_route_decode(layer2, x)
    Rh = oracle.decode_bf16(SD.to_numpy_bits(R)).T
    L = oracle.OracleLayer(Rh, np.zeros(spec.E), spec.k, lambda e, w: synth.expert_stored(spec, e, w))
    o_idx, o_g, _, o_out = oracle.moe_tokens(oracle.tokens_f64(spec, 0, 8), L)
    G.compare(idx, gates, out, o_idx, o_g, o_out, "ties")
    copies = sorted([top, (top + 17) % spec.E, (top + 41) % spec.E])
    assert set(copies) <= set(idx[0].tolist())


@pytest.mark.parametrize("T", [4, 70])
def test_bad_indices_raise_the_device_flag(T):
    """T = 4: the few-token pair kernels; T = 70 (420 pairs): the sorted
    grouped path."""
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MOE_ROUTE_GIVEN
    dl = dev(SPEC)
    layer = SD.make_layer(dl, max_tokens=T)
    x = SD.device_tokens(SPEC, 0, T)
    idx, gates, out = G.run_grouped(layer, x)
    assert layer.device_error() == 0
    bad = torch.from_numpy(idx).cuda()
    bad[1, 2] = SPEC.E                       # out of range
    g = torch.from_numpy(gates).cuda()
    _, _, o = G.run_grouped(layer, x, MOE_ROUTE_GIVEN, bad, g)
    assert layer.device_error() & 1
    others = [t for t in range(T) if t != 1]
    assert np.all(np.isnan(o[1])) and np.all(np.isfinite(o[others]))
    assert np.array_equal(o[others], out[others])
    dup = torch.from_numpy(idx).cuda()
    dup[2, 1] = dup[2, 0]                    # repeated within token 2
    _, _, o = G.run_grouped(layer, x, MOE_ROUTE_GIVEN, dup, g)
    assert layer.device_error() & 2
    assert np.all(np.isnan(o[2]))
    # single-token path
    o1 = torch.empty(SPEC.H, dtype=torch.float32, device="cuda")
    ws = layer.workspace(1)
    layer.expert_decode(x[1], bad[1], g[1], o1, ws)
    torch.cuda.synchronize()
    assert layer.device_error() & 1 and torch.isnan(o1).all()
    assert layer.device_error() == 0         # the flag clears on read


def test_host_refusals_with_a_live_layer():
    torch = G.torch_mod()
    import synth.device as SD
    from expert_routing_quantized_amd import MoeError
    dl = dev(SPEC)
    layer = SD.make_layer(dl, max_tokens=4)
    x = SD.device_tokens(SPEC, 0, 4)
    ws = layer.workspace(4)
    idx = torch.empty((4, SPEC.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((4, SPEC.k), dtype=torch.float32, device="cuda")
    out = torch.empty((4, SPEC.H), dtype=torch.float32, device="cuda")
    with pytest.raises(MoeError) as e:
        layer.route(x, 5, idx, gates, ws)
    assert e.value.status == -6
    with pytest.raises(MoeError) as e:
        layer.route(x, 4, idx, gates, ws[: ws.numel() // 2])
    assert e.value.status == -5
    with pytest.raises(MoeError) as e:
        layer.route(x.view(-1)[1:], 1, idx, gates, ws)
    assert e.value.status == -4
    with pytest.raises(MoeError) as e:
        layer.grouped_forward(x, 4, None, None, 1, out, ws)
    assert e.value.status == -1
    layer.route(x, 0, idx, gates, ws)        # T = 0 is a no-op
    assert layer.workspace_bytes(0) > 0


@pytest.mark.parametrize("rank,shift,T", [(3, 9, 1), (3, -9, 1), (1, 5, 1), (3, 9, 5), (0, -3, 5)])
def test_ties_at_the_cut_and_inside_the_top(rank, shift, T):
    """A copy of the expert at `rank` of token 0 placed `shift` indices away
    (an exact tie: the lower index ranks first; at rank k-1 the tie decides
    which of the two is selected), plus a row one bf16 ulp away from the
    expert at rank 0 (a near tie decided by the exact logits).  T = 1 routes
    with the batch-1 GEMV bound; T = 5 with the few-token MFMA bound."""
    torch = G.torch_mod()
    import oracle
    import synth.device as SD
    spec = SPEC_BF
    dl = dev(spec)
    R = dl.router_eh.clone()
    x = SD.device_tokens(spec, 0, T)
    layer = SD.make_layer(dl, max_tokens=8)
    idx0, _, _ = G.run_grouped(layer, x)
    top = [int(v) for v in idx0[0]]
    src = top[rank]
    dst = (src + shift) % spec.E
    while dst in top:
        dst = (dst + (1 if shift > 0 else -1)) % spec.E
    R[dst] = R[src]
    near = (top[0] + 2 * shift + 1) % spec.E
    while near in top or near == dst:
        near = (near + 1) % spec.E
    R[near] = R[top[0]]
    bits = R[near].view(torch.int16)
    bits[37] += 1
    dl2 = SD.DeviceLayer(spec, R, dl.bias, dl.w_gate, dl.w_up, dl.w_down)
    layer2 = SD.make_layer(dl2, max_tokens=8)
    idx, gates, out = G.run_grouped(layer2, x)
    Rh = oracle.decode_bf16(SD.to_numpy_bits(R)).T
    L = oracle.OracleLayer(Rh, np.zeros(spec.E), spec.k, lambda e, w: synth.expert_stored(spec, e, w))
    o_idx, o_g, _, o_out = oracle.moe_tokens(oracle.tokens_f64(spec, 0, T), L)
    G.compare(idx, gates, out, o_idx, o_g, o_out, f"ties rank {rank} shift {shift} T {T}")


@pytest.mark.parametrize("T", [1, 5, 20, 600])
def test_tiny_hidden_state_near_ties(T):
    """Hidden states scaled by 2^-80 (their squares underflow binary32) with
    an exact tie and a near tie one bf16 ulp apart in the element where token
    0's |x| is smallest, no bias.  The selection's error bound grows with
    ||x||, so ||x||^2 must not underflow: the routing must still match the
    exact logits.  T = 1, 5, 20 and 600 take the four router kernels."""
    torch = G.torch_mod()
    import oracle
    import synth.device as SD
    spec = SPEC_BF
    dl = dev(spec)
    scale = 2.0 ** -80
    x = (SD.device_tokens(spec, 0, T).float() * scale).to(torch.bfloat16)
    Xh = oracle.tokens_f64(spec, 0, T) * scale
    assert np.array_equal(oracle.decode_bf16(SD.to_numpy_bits(x)), Xh)   # scaling is exact
    layer = SD.make_layer(dl, max_tokens=T)
    idx0, _, _ = G.run_grouped(layer, x)
    top = [int(v) for v in idx0[0]]
    R = dl.router_eh.clone()
    dst = (top[1] + 7) % spec.E
    while dst in top:
        dst = (dst + 1) % spec.E
    R[dst] = R[top[1]]                              # exact tie with rank 1
    near = (top[0] + 3) % spec.E
    while near in top or near == dst:
        near = (near + 1) % spec.E
    R[near] = R[top[0]]
    h = int(np.argmin(np.where(Xh[0] != 0, np.abs(Xh[0]), np.inf)))
    bits = R[near].view(torch.int16)
    bits[h] += 1                                    # near tie: differs by x_h * one ulp
    dl2 = SD.DeviceLayer(spec, R, dl.bias, dl.w_gate, dl.w_up, dl.w_down)
    layer2 = SD.make_layer(dl2, max_tokens=T)
    Rh = oracle.decode_bf16(SD.to_numpy_bits(R)).T
    L = oracle.OracleLayer(Rh, np.zeros(spec.E), spec.k, lambda e, w: synth.expert_stored(spec, e, w))
    o_idx, o_g, _, o_out = oracle.moe_tokens(Xh, L)
    G.note("tiny x", T)
    # The outputs (about 2^-160 here) lie below the binary32 range, in which
    # h and out are kept, so they are zero or subnormal: only the routing is
    # compared with the oracle, the outputs only checked to be finite and tiny.
    assert np.abs(o_out).max() < 2.0 ** -140
    for run in (G.run_grouped, G.run_route_decode):
        idx, gates, out = run(layer2, x)
        G.compare(idx, gates, None, o_idx, o_g, None, f"tiny x T {T}/{run.__name__}")
        assert np.all(np.isfinite(out)) and np.abs(out).max() <= 2.0 ** -120
    assert layer2.device_error() == 0
