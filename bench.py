"""Benchmark of the MoE layer on one MI355X.

Default workload: batch-1 decode through the 4-bit layer (H=2048, E=24,576,
top-10, I=256, 4-bit experts in 32-element blocks with fp16 scales, bf16
router and hidden states, Zipf-shaped router bias), sequential tokens.  One
"step" is one token through the whole path: router GEMV, exact top-k with
softmax gates, expert gate/up GEMV, down GEMV with the weighted combine.

* Inputs are synthetic and seeded, generated straight into HBM before the
  timed region.
* The K timed steps (and the W warm-up steps) are captured into HIP graphs
  and replayed; time = HIP events around the replay on the capture stream.
* Cold router (default): the router is held in 3 bitwise-identical copies
  (302 MB, more than the 256 MB Infinity Cache) and token t reads copy t % 3,
  so each token's router read comes from HBM, as it would with the other
  layers of a model running in between.  ``--mode warm`` uses one copy.
* Roofline of the dominant kernel (the router GEMV, 92% of the bytes): the
  same kernel is launched alone (moe_router_logits) K times in a graph and
  timed with HIP events on its stream.
* CPU baseline: the float64 oracle, timed on a bounded sample of tokens on
  the host's cores; its results also check the GPU outputs of those tokens.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--config", default="decode_q4",
                   choices=["decode_bf16", "decode_q4", "verify_q4", "prefill_bf16", "prefill_bf16_hot"],
                   help="decode_bf16/decode_q4: batch-1 decode (the headline is decode_q4); verify_q4: T=5 verify steps "
                        "through the 4-bit layer; prefill_bf16: T=2048 prefill chunks through the bf16 layer; "
                        "prefill_bf16_hot (supplementary): the same chunk routed to 64 hot experts, so the grouped "
                        "expert kernels are matrix-bound")
    p.add_argument("--sweep", action="store_true",
                   help="cost table of moe_grouped_forward over T: 1-8 tokens through the 4-bit layer, "
                        "16-8192 through the bf16 layer (one JSON line)")
    p.add_argument("--mode", default="cold", choices=["cold", "warm"])
    p.add_argument("--screen", default="on", choices=["on", "off"],
                   help="batch-1 decode through the router's int8 screen (cold: 6 layer copies, "
                        "so the int8 routers too exceed the 256 MB last-level cache)")
    p.add_argument("--cpu-sample", type=int, default=800,
                   help="tokens the oracle is timed on (about 10 s of host work; 0: skip)")
    p.add_argument("--layers", type=int, default=1,
                   help="decode configs: N > 1 stacks N distinct layers (weight seeds base..base+N-1, "
                        "N x 21.7 GB for 4-bit experts) and times every token through all of them "
                        "(one JSON line, per layer-token cost; replaces the router copies)")
    p.add_argument("--parity-stream", action="store_true",
                   help="whole-stream parity against the oracle: 1000 tokens of the tiny fp32 layer and of "
                        "both batch-1 decode layers, 1000 verify steps (T = 5), one 2048-token prefill chunk; "
                        "one JSON line per workload (the exact-refinement counts included)")
    p.add_argument("--hot", type=int, default=0,
                   help="decode configs: copy the N experts most chosen over a 400-token calibration stream "
                        "into the layer's hot region and time the decode stream with it, with a region that "
                        "catches nothing, and without a region")
    p.add_argument("--host", type=int, default=0,
                   help="decode configs: move the N experts least chosen over a calibration stream to the "
                        "host tier (computed by the host's cores) and time the decode stream")
    p.add_argument("--counters", action="store_true",
                   help="hardware-counter run: launch eagerly (no graphs), run the router alone, then "
                        "a plain copy of known size that calibrates the byte counters; prints a summary")
    return p.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "router_gemv_decode_q4_traffic.md")
TRAFFIC_SOURCES = ["expert_routing_quantized_amd/csrc/router.hip", "expert_routing_quantized_amd/csrc/moe_internal.h"]
SCREEN_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "screen_decode_q4_traffic.md")
SCREEN_TRAFFIC_SOURCES = ["expert_routing_quantized_amd/csrc/screen.hip",
                          "expert_routing_quantized_amd/csrc/select_screen.h",
                          "expert_routing_quantized_amd/csrc/moe_internal.h"]
# the whole decode step (screen, fused selection + gate/up, down + combine)
STEP_TRAFFIC_SOURCES = SCREEN_TRAFFIC_SOURCES + ["expert_routing_quantized_amd/csrc/experts.hip",
                                                 "expert_routing_quantized_amd/csrc/select_block.h"]
COPY_CALIBRATION_BYTES = 256 << 20


def median_replay_ms(graph, stream, reps=5):
    """Median over `reps` replays of a captured graph, each bracketed by HIP
    events on the capture stream and a device synchronisation."""
    import statistics
    import torch
    times = []
    for _ in range(reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return statistics.median(times)


def kernel_source_hash(screen=False, step=False) -> str:
    """sha256 over the sources the dominant kernel (the router GEMV, or the
    screen) -- or, with step, every kernel of the screened decode step -- is
    compiled from."""
    import hashlib
    h = hashlib.sha256()
    for rel in (STEP_TRAFFIC_SOURCES if step else SCREEN_TRAFFIC_SOURCES if screen else TRAFFIC_SOURCES):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(screen=False):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is missing or the kernel sources changed since."""
    try:
        fields = {}
        with open(SCREEN_TRAFFIC_PROFILE if screen else TRAFFIC_PROFILE) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].split(": ", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("source_sha256") != kernel_source_hash(screen):
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def measured_step_traffic():
    """HBM bytes of one whole screened decode step (all three kernels) from
    the committed counter summary, or None when missing or stale."""
    try:
        fields = {}
        with open(SCREEN_TRAFFIC_PROFILE) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].split(": ", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("step_source_sha256") != kernel_source_hash(step=True):
            return None
        return float(fields["step_traffic_bytes_per_token"])
    except (OSError, KeyError, ValueError):
        return None


def counters_main(args, spec):
    """Eager launches for rocprofv3 --pmc runs (counter collection does not
    need graphs).  Decode configs: K tokens, K router-only launches, 3
    calibration copies; grouped configs: W + K calls on one batch."""
    import torch

    import synth.device as SD
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup
    dl = SD.device_layer(spec)
    if spec.T > 1:
        # grouped configs: W + K eager moe_grouped_forward calls on one batch
        T = spec.T
        layer = SD.make_layer(dl, max_tokens=T)
        X = SD.device_tokens(spec, 0, T)
        ws = layer.workspace(T)
        idx = torch.empty((T, spec.k), dtype=torch.int32, device=dev)
        gates = torch.empty((T, spec.k), dtype=torch.float32, device=dev)
        out = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
        for _ in range(W + K):
            layer.grouped_forward(X, T, idx, gates, 0, out, ws)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": True, "calls": W + K, "T": T,
                          "router_flops_per_call": 2.0 * T * spec.H * spec.E,
                          "device_errors": layer.device_error()}), flush=True)
        return
    screen = args.screen == "on"
    n_rep = (6 if screen else 3) if args.mode == "cold" else 1
    routers = [dl.router_eh] + [SD.device_router(spec) for _ in range(n_rep - 1)]
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_OFF, MOE_LAYER_SCREEN_ON
    lflags = MOE_LAYER_SCREEN_ON if screen else MOE_LAYER_SCREEN_OFF
    layers = [SD.make_layer(dl, max_tokens=1, router=r, flags=lflags) for r in routers]
    X = SD.device_tokens(spec, 0, W + K)
    ws = layers[0].workspace(1)
    idx = torch.zeros((W + K, spec.k), dtype=torch.int32, device=dev)
    gates = torch.zeros((W + K, spec.k), dtype=torch.float32, device=dev)
    out = torch.zeros((W + K, spec.H), dtype=torch.float32, device=dev)
    zbuf = torch.empty((spec.E,), dtype=torch.float64, device=dev)
    for t in range(W + K):
        layers[t % n_rep].grouped_forward(X[t], 1, idx[t], gates[t], 0, out[t], ws)
    vbuf = torch.empty((spec.E,), dtype=torch.float32, device=dev)
    for t in range(W, W + K):
        if screen:
            layers[t % n_rep].router_screen(X[t], 1, vbuf, None, ws)
        else:
            layers[t % n_rep].router_logits(X[t], 1, zbuf, ws)
    src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": True, "tokens": W + K, "router_launches": K, "screen": screen,
                      "copy_bytes": COPY_CALIBRATION_BYTES, "copies": 3,
                      "dominant_kernel_bytes_per_launch": screen_bytes(spec) if screen else step_bytes(spec)["router"],
                      "source_sha256": kernel_source_hash(screen)}), flush=True)


def screen_bytes(spec) -> int:
    """Bytes one launch of the screen reads: the int8 router, per expert its
    scale, bias and residual norm, and x."""
    act = 2 if spec.act == 1 else 4
    return spec.E * spec.H + 12 * spec.E + spec.H * act


def step_bytes(spec, screen=False, listed=0.0) -> dict:
    """Algorithmic bytes of one decode token (what the method must move);
    with the screen, the int8 pass plus the `listed` bf16 rows recomputed."""
    H, E, k, I = spec.H, spec.E, spec.k, spec.I
    act = 2 if spec.act == 1 else 4
    router = E * H * act + E * 4 + H * act            # weights + bias + x
    if screen:
        router = screen_bytes(spec) + int(round(listed * H * act))
    if spec.expert == 2:
        per_expert = 3 * I * H // 2 + 3 * I * (H // 32) * 2
    else:
        per_expert = 3 * I * H * (2 if spec.expert == 1 else 4)
    experts = k * per_expert
    out = H * 4 + k * 8
    return {"router": router, "experts": experts, "total": router + experts + out}


def cpu_baseline(spec, first, count, gpu_idx, gpu_gates, gpu_out, dl=None):
    """The oracle timed on `count` tokens of the timed stream.  The experts'
    stored bytes come from the seeded input generator: its device copy in
    `dl` when given (bitwise equal to the host generator, and fast to copy),
    else the host generator."""
    import numpy as np

    import oracle
    import synth

    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp:
        threads = min(threads, int(omp))
    log(f"oracle: building float64 router ({spec.E}x{spec.H})")
    L0 = oracle.layer_from_spec(spec)
    X = oracle.tokens_f64(spec, first, count)
    stored = {}

    def from_device(e, which):
        w = {"gate": dl.w_gate, "up": dl.w_up, "down": dl.w_down}[which][e]
        if spec.expert == synth.DT_Q4:
            sc = {"gate": dl.s_gate, "up": dl.s_up, "down": dl.s_down}[which][e]
            return ("q4", (w.cpu().numpy(), sc.cpu().numpy().view(np.uint16)))
        if spec.expert == synth.DT_BF16:
            import torch
            return ("bf16", w.view(torch.int16).cpu().numpy().view(np.uint16))
        return ("f32", w.cpu().numpy())

    def fetch(e, which):
        key = (e, which)
        if key not in stored:
            stored[key] = from_device(e, which) if dl is not None else synth.expert_stored(spec, e, which)
        return stored[key]
    # untimed: the stored bytes of the experts the sample selects (data
    # preparation; any other expert the oracle asks for is fetched on demand)
    for e in np.unique(gpu_idx):
        if 0 <= e < spec.E:
            for which in ("gate", "up", "down"):
                fetch(int(e), which)
    # untimed warm-up over the sample's first tokens (thread pools, caches),
    # then the timed pass: a fresh oracle over the same stored bytes
    Lw = oracle.OracleLayer(L0.R, L0.b, spec.k, fetch)
    Lw._absR = L0.absR()
    oracle.moe_tokens(X[:min(16, count)], Lw)
    Lt = oracle.OracleLayer(L0.R, L0.b, spec.k, fetch)
    Lt._absR = L0.absR()
    t0 = time.perf_counter()
    o_idx, o_g, _, o_out = oracle.moe_tokens(X, Lt)
    dt = time.perf_counter() - t0
    rel = np.linalg.norm(gpu_out.astype(np.float64) - o_out, axis=1) / np.linalg.norm(o_out, axis=1)
    parity = {"tokens": count, "idx_exact": bool(np.array_equal(gpu_idx, o_idx)),
              "gate_max_abs_err": float(np.abs(gpu_gates - o_g).max()),
              "out_rel_l2_max": float(rel.max()), "out_rel_l2_median": float(np.median(rel))}
    base = {"value": count / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{count} tokens (tokens {first}..{first + count - 1} of the timed stream), "
                      f"float64 numpy, {dt:.1f} s; expert bytes pre-generated from the seeded generator"}
    # the same oracle on one thread (BLAS limited to 1), first 50 tokens of the sample
    from threadpoolctl import threadpool_limits
    n1 = min(50, count)
    L1 = oracle.OracleLayer(L0.R, L0.b, spec.k, fetch)
    L1._absR = L0.absR()
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        oracle.moe_tokens(X[:n1], L1)
        d1 = time.perf_counter() - t1
    single = {"value": n1 / d1, "unit": "tokens/s", "cores": 1, "kind": "oracle",
              "sample": f"{n1} tokens (tokens {first}..{first + n1 - 1}), float64 numpy, {d1:.1f} s"}
    if single["value"] > base["value"]:          # report the faster configuration as the baseline
        base, single = single, base
    return base, parity, single


def grouped_main(args, spec):
    """verify_q4 / prefill_bf16: T tokens per call through moe_grouped_forward (one step = one call)."""
    import torch

    import synth.device as SD
    T = spec.T
    K, W = args.steps, args.warmup
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    dl = SD.device_layer(spec)
    layer = SD.make_layer(dl, max_tokens=T)
    nseq = min(K + W, 64)                        # distinct token batches, reused cyclically
    X = SD.device_tokens(spec, 0, nseq * T).view(nseq, T, spec.H)
    ws = layer.workspace(T)
    idx = torch.zeros((nseq, T, spec.k), dtype=torch.int32, device=dev)
    gates = torch.zeros((nseq, T, spec.k), dtype=torch.float32, device=dev)
    out = torch.zeros((nseq, T, spec.H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"layer ready in {time.time() - t0:.1f}s: pool {dl.nbytes_pool() / 1e9:.2f} GB, T={T}")

    from expert_routing_quantized_amd import MOE_ROUTE_GIVEN
    zbuf = torch.empty((T, spec.E), dtype=torch.float64, device=dev)
    # windows of 2-8 tokens on a layer with the router screen (bf16 x, H a
    # multiple of 32 and at most 2048, E >= 4096) route through the window
    # screen: its launch alone is the router's roofline
    win_screen = 2 <= T <= 8 and spec.act == 1 and spec.H % 32 == 0 and spec.H <= 2048 and spec.E >= 4096
    vbuf = torch.empty((T, spec.E), dtype=torch.float32, device=dev)

    def step(i):
        b = i % nseq
        layer.grouped_forward(X[b], T, idx[b], gates[b], 0, out[b], ws)

    def router_only(i):
        if win_screen:
            layer.router_screen(X[i % nseq], T, vbuf, None, ws)
        else:
            layer.router_logits(X[i % nseq], T, zbuf, ws)

    def experts_only(i):
        b = i % nseq
        layer.grouped_forward(X[b], T, idx[b], gates[b], MOE_ROUTE_GIVEN, out[b], ws)

    for i in range(max(min(W, 3), min(nseq, W + K))):
        step(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = {n: torch.cuda.CUDAGraph() for n in ("warm", "main", "router", "experts")}
    with torch.cuda.stream(s):
        with torch.cuda.graph(graphs["warm"], stream=s):
            for i in range(W):
                step(i)
        with torch.cuda.graph(graphs["main"], stream=s):
            for i in range(W, W + K):
                step(i)
        with torch.cuda.graph(graphs["router"], stream=s):
            for i in range(W, W + K):
                router_only(i)
        with torch.cuda.graph(graphs["experts"], stream=s):
            for i in range(W, W + K):
                experts_only(i)
    torch.cuda.synchronize()

    def timed(name):
        return median_replay_ms(graphs[name], s)

    with torch.cuda.stream(s):
        graphs["warm"].replay()
        torch.cuda.synchronize()
        ms = timed("main")
        graphs["router"].replay()
        torch.cuda.synchronize()
        ms_router = timed("router")
        ms_experts = timed("experts")
    err = layer.device_error()
    import numpy as np
    distinct = [len(np.unique(idx[b].cpu().numpy())) for b in range(min(nseq, 8))]
    per_step = ms / 1e3 / K
    router_s = ms_router / 1e3 / K
    experts_s = ms_experts / 1e3 / K
    act = 2 if spec.act == 1 else 4
    if spec.expert == 2:
        per_expert = 3 * spec.I * spec.H // 2 + 3 * spec.I * (spec.H // 32) * 2
    else:
        per_expert = 3 * spec.I * spec.H * (2 if spec.expert == 1 else 4)
    d_mean = float(np.mean(distinct))
    router_bytes = spec.E * spec.H * act + spec.E * 4 + T * spec.H * act
    router_flops = 2.0 * T * spec.H * spec.E
    if router_flops / router_bytes > 312.5:      # above the ridge: MFMA-bound
        kname = ("moe::router_gemm_big_kernel, 256x256 tiles" if T >= 512 else "moe::router_gemm_kernel, 128x128 tiles")
        roof = {"bound": "mfma", "kernel": f"router GEMM ({kname}, bf16 MFMA)",
                "achieved": router_flops / router_s / 1e12, "peak": 2500.0, "unit": "TFLOP/s",
                "frac": router_flops / router_s / 1e12 / 2500.0, "traffic": None,
                "avg_launch_us": router_s * 1e6, "flops_per_launch": router_flops}
    elif win_screen:
        sbytes = screen_bytes(spec) + (T - 1) * spec.H * act
        nbuf = 8 if 4 <= T <= 6 else 4
        roof = {"bound": "hbm", "kernel": (f"window screen (moe::screen_window_kernel<32, 4, {nbuf}>: int8 router on "
                                           "v_mfma_i32_16x16x64_i8, exact integer sums)"),
                "achieved": sbytes / router_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": sbytes / router_s / 1e9 / HBM_PEAK_GBS, "traffic": None,
                "avg_launch_us": router_s * 1e6, "bytes_per_launch": sbytes}
    else:
        roof = {"bound": "hbm", "kernel": "router (moe::router_skinny_lds_kernel, 16x16x32 MFMA tiles)",
                "achieved": router_bytes / router_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": router_bytes / router_s / 1e9 / HBM_PEAK_GBS, "traffic": None,
                "avg_launch_us": router_s * 1e6, "bytes_per_launch": router_bytes}
    experts_bytes = d_mean * per_expert
    # executed expert matrix work: gate, up and down, 2 H I flops each per pair
    experts_flops = 6.0 * T * spec.k * spec.H * spec.I
    res = {
        "metric": f"MoE-layer grouped forward tokens/s ({spec.name}: T={T} per call)",
        "value": T * K / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{spec.name}: T={T} tokens per call, H={spec.H}, E={spec.E}, top-{spec.k}, "
                               f"I={spec.I}, experts {'q4b32' if spec.expert == 2 else 'bf16'}",
                   "us_per_step": per_step * 1e6, "distinct_experts_per_step": distinct,
                   "device_errors": err},
        "roofline": roof,
        "experts_stage": {"us_per_call": experts_s * 1e6, "weight_bytes_per_call": experts_bytes,
                          "weight_gbs": experts_bytes / experts_s / 1e9,
                          "flops_per_call": experts_flops,
                          "tflops": experts_flops / experts_s / 1e12,
                          "mfma_frac": experts_flops / experts_s / 1e12 / 2500.0,
                          "note": "moe_grouped_forward with caller indices: pair grouping, gate/up, down, combine"},
    }
    print(json.dumps(res), flush=True)


def sweep_main(args):
    """Cost of one moe_grouped_forward call over T (graph-captured calls on
    distinct token batches): the table a draft or chunking policy reads."""
    import torch

    import synth
    import synth.device as SD
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows = []
    for name, Ts in (("verify_q4", [1, 2, 3, 4, 5, 6, 8]),
                     ("prefill_bf16", [16, 64, 256, 512, 1024, 2048, 4096, 8192])):
        spec = synth.CONFIGS[name]
        dl = SD.device_layer(spec)
        layer = SD.make_layer(dl, max_tokens=max(Ts))
        for T in Ts:
            reps = max(3, min(200, 200 * 16 // T))
            nb = min(reps, max(1, 16384 // T))             # distinct batches, reused cyclically
            X = SD.device_tokens(spec, 0, nb * T).view(nb, T, spec.H)
            ws = layer.workspace(T)
            idx = torch.empty((T, spec.k), dtype=torch.int32, device=dev)
            gates = torch.empty((T, spec.k), dtype=torch.float32, device=dev)
            out = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
            for i in range(2):
                layer.grouped_forward(X[i % nb], T, idx, gates, 0, out, ws)
            torch.cuda.synchronize()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for i in range(reps):
                        layer.grouped_forward(X[i % nb], T, idx, gates, 0, out, ws)
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                g.replay()
                ms = median_replay_ms(g, s)
            us = ms * 1e3 / reps
            rows.append({"layer": name.split("_")[1], "T": T, "us_per_call": us,
                         "us_per_token": us / T, "tokens_per_s": T / us * 1e6,
                         "device_errors": layer.device_error()})
            log(f"sweep {name} T={T}: {us:.1f} us per call, {T / us * 1e6:.0f} tokens/s")
            del g, X, ws, idx, gates, out
        del layer, dl
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "moe_grouped_forward cost per call over T (cost table)",
                      "unit": "us per call", "n_gpus": 1, "data": "synthetic",
                      "config": {"workload": "T = 1-8 through the 4-bit decode layer, T = 16-8192 through the "
                                             "bf16 layer (H=2048, E=24576, top-10, I=256)"},
                      "sweep": rows}), flush=True)


class _DevArray:
    """A zero-copy torch view (CUDA array interface) of device memory the
    library owns."""

    def __init__(self, addr, n, typestr):
        self.__cuda_array_interface__ = {"shape": (n,), "typestr": typestr, "data": (addr, False),
                                         "version": 3, "strides": None}


def layers_main(args, spec):
    """Batch-1 decode through N distinct layers per token (each with its own
    router, bias, expert pool and workspace), timed three ways over the same
    tokens: (1) one graph of K x N moe_grouped_forward calls, every layer
    taking the token's hidden state; (2) the decoder (moe_decoder_*): one
    captured graph per layer, the layers chained by the residual stream
    (x_{l+1} = bf16(x_l + out_l)), the token written into the input slot
    before each step, the host launching the layers' graphs ahead of the
    device; (3) the same with the host waiting for each layer's doorbell
    before launching the next.  N routers and N pools are far beyond the
    256 MB Infinity Cache, so this is the real cross-layer cache behaviour."""
    import dataclasses
    import statistics

    import torch

    import synth.device as SD
    from expert_routing_quantized_amd import Decoder
    K, W, N = args.steps, args.warmup, args.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    dls, layers = [], []
    for l in range(N):
        sl = dataclasses.replace(spec, weight_seed=spec.weight_seed + l)
        dls.append(SD.device_layer(sl))
        layers.append(SD.make_layer(dls[-1], max_tokens=1))
    X = SD.device_tokens(spec, 0, W + K)
    torch.cuda.synchronize()
    pool = sum(d.nbytes_pool() for d in dls)
    log(f"{N} layers ready in {time.time() - t0:.1f}s: pools {pool / 1e9:.1f} GB")
    wss = [L.workspace(1) for L in layers]
    idx = torch.zeros((W + K, N, spec.k), dtype=torch.int32, device=dev)
    gates = torch.zeros((W + K, N, spec.k), dtype=torch.float32, device=dev)
    out = torch.zeros((W + K, N, spec.H), dtype=torch.float32, device=dev)

    def token(t):
        for l in range(N):
            layers[l].grouped_forward(X[t], 1, idx[t, l], gates[t, l], 0, out[t, l], wss[l])

    for t in range(W):
        token(t)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g_warm, g_main = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g_warm, stream=s):
            for t in range(W):
                token(t)
        with torch.cuda.graph(g_main, stream=s):
            for t in range(W, W + K):
                token(t)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g_warm.replay()
        torch.cuda.synchronize()
        ms = median_replay_ms(g_main, s)
    errs = [L.device_error() for L in layers]
    by = step_bytes(spec)
    per_lt = ms / 1e3 / (K * N)

    # the decoder: one graph per layer, launched by the host per token
    dec = Decoder(layers, stream=s)
    x0 = torch.as_tensor(_DevArray(dec.buffers(0)[0], spec.H, "<i2"), device="cuda")
    Xi = X.view(torch.int16)

    def dec_run(first, count, wait):
        with torch.cuda.stream(s):
            for t in range(first, first + count):
                x0.copy_(Xi[t])
                dec.step(wait_doorbell=wait, stream=s)

    def dec_time(wait):
        dec_run(0, W, wait)
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            dec_run(W, K, wait)
            e1.record(s)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return statistics.median(times)

    ms_dec = dec_time(False)
    ms_bell = dec_time(True)
    dec_bells = [dec.doorbell(l) for l in range(N)]
    dec.close()
    errs_dec = [L.device_error() for L in layers]
    print(json.dumps({
        "metric": "MoE-layer decode layer-tokens/s through N distinct layers (batch-1)",
        "value": 1.0 / per_lt, "unit": "layer-tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.config} batch-1 decode through {N} distinct layers per token "
                               f"(weight seeds {spec.weight_seed}..{spec.weight_seed + N - 1}, "
                               f"{pool / 1e9:.1f} GB of expert pools), {K} tokens, same hidden state into "
                               f"every layer, one graph for the whole stream",
                   "layers": N, "us_per_layer_token": per_lt * 1e6, "us_per_token_all_layers": ms * 1e3 / K,
                   "hbm_gbs": by["total"] / per_lt / 1e9, "device_errors": errs,
                   "per_layer_graphs": {
                       "note": "moe_decoder: one captured graph per layer plus its epilogue (residual stream "
                               "and doorbell), the token copied into the input slot before each step",
                       "us_per_layer_token": ms_dec * 1e3 / (K * N), "us_per_token_all_layers": ms_dec * 1e3 / K,
                       "with_doorbell_wait_us_per_layer_token": ms_bell * 1e3 / (K * N),
                       "doorbells_after": dec_bells, "device_errors": errs_dec}},
    }), flush=True)


def parity_main(args):
    """Every output of whole workloads against the oracle (float64), on the
    seeded synthetic inputs: indices exactly, gates and outputs within the
    tolerances of the parity tests; also the exact-refinement counts and,
    through the screen (batch 1 and verify windows), how many calls selected
    from its list.""" 
    import numpy as np
    import torch

    import oracle
    import synth
    import synth.device as SD
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    from expert_routing_quantized_amd import MOE_LAYER_FORCE_EXACT_REFINE
    # the last three rows force every near-tie logit through the exact
    # refinement (MOE_LAYER_FORCE_EXACT_REFINE), so that path is checked on
    # whole streams at T = 1, 5 and 2048 too
    plan = [("tiny_f32", 1, 1000, 0), ("decode_bf16", 1, 1000, 0), ("decode_q4", 1, 1000, 0),
            ("verify_q4", 5, 1000, 0), ("prefill_bf16", 2048, 1, 0),
            ("decode_q4", 1, 200, MOE_LAYER_FORCE_EXACT_REFINE), ("verify_q4", 5, 200, MOE_LAYER_FORCE_EXACT_REFINE),
            ("prefill_bf16", 2048, 1, MOE_LAYER_FORCE_EXACT_REFINE)]
    for name, T, steps, lflags in plan:
        spec = synth.CONFIGS[name]
        t0 = time.time()
        dl = SD.device_layer(spec)
        layer = SD.make_layer(dl, max_tokens=T, flags=lflags)
        n = T * steps
        X = SD.device_tokens(spec, 0, n)
        ws = layer.workspace(T)
        ws.zero_()
        idx = torch.empty((n, spec.k), dtype=torch.int32, device=dev)
        gates = torch.empty((n, spec.k), dtype=torch.float32, device=dev)
        out = torch.empty((n, spec.H), dtype=torch.float32, device=dev)
        r0 = layer.exact_refinements()
        for st in range(steps):
            a, b = st * T, (st + 1) * T
            layer.grouped_forward(X[a:b], T, idx[a:b], gates[a:b], 0, out[a:b], ws)
        torch.cuda.synchronize()
        nref = layer.exact_refinements() - r0
        # calls whose selection took the screen's list (windows: token 0's list)
        screened = T <= 8 and spec.act == synth.DT_BF16 and spec.E >= 4096 and spec.H % 32 == 0
        listed = int(ws[12:16].view(torch.int32).item()) if screened else None
        errs = layer.device_error()
        gi, gg, go = idx.cpu().numpy(), gates.cpu().numpy(), out.cpu().numpy()
        log(f"{name}: {steps} calls of T={T} on the GPU in {time.time() - t0:.1f} s; oracle ...")

        stored = {}

        def fetch(e, which, dl=dl, spec=spec, stored=stored):
            key = (e, which)
            if key not in stored:
                w = {"gate": dl.w_gate, "up": dl.w_up, "down": dl.w_down}[which][e]
                if spec.expert == synth.DT_Q4:
                    sc = {"gate": dl.s_gate, "up": dl.s_up, "down": dl.s_down}[which][e]
                    stored[key] = ("q4", (w.cpu().numpy(), sc.cpu().numpy().view(np.uint16)))
                elif spec.expert == synth.DT_BF16:
                    stored[key] = ("bf16", w.view(torch.int16).cpu().numpy().view(np.uint16))
                else:
                    stored[key] = ("f32", w.cpu().numpy())
            return stored[key]
        L0 = oracle.layer_from_spec(spec)
        L = oracle.OracleLayer(L0.R, L0.b, spec.k, fetch, cache_size=4096)
        Xh = oracle.tokens_f64(spec, 0, n)
        o_idx = np.empty((n, spec.k), np.int64)
        o_g = np.empty((n, spec.k))
        o_out = np.empty((n, spec.H))
        for c0 in range(0, n, 256):
            c1 = min(n, c0 + 256)
            o_idx[c0:c1], o_g[c0:c1], _, o_out[c0:c1] = oracle.moe_tokens(Xh[c0:c1], L)
            log(f"{name}: oracle {c1}/{n} tokens")
        rel = np.linalg.norm(go.astype(np.float64) - o_out, axis=1) / np.maximum(np.linalg.norm(o_out, axis=1), 1e-300)
        print(json.dumps({
            "workload": name, "T": T, "calls": steps, "tokens": n, "forced_exact_refinement": bool(lflags),
            "idx_mismatched_tokens": int((gi != o_idx).any(axis=1).sum()),
            "gate_max_abs_err": float(np.abs(gg.astype(np.float64) - o_g).max()),
            "out_rel_l2_max": float(rel.max()), "out_rel_l2_median": float(np.median(rel)),
            "exact_refinements": int(nref), "exact_refinements_per_token": nref / n,
            "calls_selected_from_the_screen_list": listed, "device_errors": errs,
            "seconds": round(time.time() - t0, 1)}), flush=True)
        del layer, dl, X, ws, idx, gates, out, L, L0, stored
        torch.cuda.empty_cache()


def hot_main(args, spec):
    """Batch-1 decode with the hot-expert region: calibration counts over a
    separate token stream, the top-N experts copied into the region of every
    layer copy, then the same timed stream three ways (graph replays, cold
    router copies as in the default run): no region (the fused decode
    kernels), the region of the top N, and a region holding one expert that
    the stream never chooses (the same few-token kernels, no hits)."""
    import numpy as np
    import torch

    import synth.device as SD
    K, W, N = args.steps, args.warmup, args.hot
    n_rep = 6 if args.mode == "cold" else 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dl = SD.device_layer(spec)
    routers = [dl.router_eh] + [SD.device_router(spec) for _ in range(n_rep - 1)]
    layers = [SD.make_layer(dl, max_tokens=1, router=r) for r in routers]
    ws = layers[0].workspace(1)
    ncal = 400
    C = SD.device_tokens(spec, 100000, ncal)
    X = SD.device_tokens(spec, 0, W + K)
    idx = torch.zeros((W + K, spec.k), dtype=torch.int32, device=dev)
    gates = torch.zeros((W + K, spec.k), dtype=torch.float32, device=dev)
    out = torch.zeros((W + K, spec.H), dtype=torch.float32, device=dev)
    ci = torch.zeros((ncal, spec.k), dtype=torch.int32, device=dev)
    cg = torch.zeros((ncal, spec.k), dtype=torch.float32, device=dev)
    co = torch.zeros((ncal, spec.H), dtype=torch.float32, device=dev)
    for t in range(ncal):
        layers[0].grouped_forward(C[t], 1, ci[t], cg[t], 0, co[t], ws)
    counts = torch.zeros(spec.E, dtype=torch.int32, device=dev)
    layers[0].expert_counts(ci, ncal * spec.k, counts)
    hist = counts.cpu().numpy()
    order = np.lexsort((np.arange(spec.E), -hist))
    hot = [int(e) for e in order[:N]]

    def run(tag):
        def token(t):
            layers[t % n_rep].grouped_forward(X[t], 1, idx[t], gates[t], 0, out[t], ws)
        for t in range(W):
            token(t)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for t in range(W, W + K):
                    token(t)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
            torch.cuda.synchronize()
            ms = median_replay_ms(g, s)
        res = {"us_per_token": ms * 1e3 / K, "outputs": out[W:W + K].clone(), "idx": idx[W:W + K].cpu().numpy()}
        log(f"{tag}: {res['us_per_token']:.2f} us per token")
        return res

    base = run("no region (fused decode kernels)")
    if args.host > 0:
        host = [int(e) for e in order[spec.E - args.host:]]
        for i, L in enumerate(layers):     # each router copy's layer pins its own host copies
            t1 = time.time()
            L.set_host_experts(host)
            log(f"host tier set on layer {i + 1}/{len(layers)} in {time.time() - t1:.1f}s")
        r = run(f"host tier of the {args.host} least chosen experts")
        for L in layers:
            L.set_host_experts([])
        rows = r["idx"]
        frac = float(np.isin(rows, host).any(axis=1).mean())
        diff = (r["outputs"] - base["outputs"]).double()
        rel = float((diff.norm(dim=1) / base["outputs"].double().norm(dim=1)).max())
        per_expert = 3 * spec.I * spec.H // 2 + 3 * spec.I * (spec.H // 32) * 2
        res = {
            "metric": f"MoE-layer decode us per token with host-tier experts ({spec.name})",
            "value": r["us_per_token"], "unit": "us per token", "n_gpus": 1, "steps": K, "warmup": W,
            "higher_is_better": False, "data": "synthetic",
            "config": {"workload": f"{spec.name}: batch-1 decode, {K} tokens, {n_rep} router copies; the "
                                   f"{args.host} experts least chosen over {ncal} calibration tokens "
                                   f"({args.host * per_expert / 1e9:.2f} GB) on the host tier",
                       "tokens_with_host_pairs": frac,
                       "host_pairs_per_token": float(np.isin(rows, host).sum(axis=1).mean()),
                       "us_per_token_no_host_tier": base["us_per_token"],
                       "max_rel_l2_vs_gpu_only": rel,
                       "device_errors": layers[0].device_error()},
        }
        print(json.dumps(res), flush=True)
        return
    for L in layers:
        L.set_hot_experts(hot)
    with_region = run(f"region of the top {N}")
    cold = [int(order[-1])]
    for L in layers:
        L.set_hot_experts(cold)
    no_hits = run("region with no hits (few-token kernels)")
    for L in layers:
        L.set_hot_experts([])
    same = bool(torch.equal(base["outputs"].view(torch.int32), with_region["outputs"].view(torch.int32)) and
                torch.equal(base["outputs"].view(torch.int32), no_hits["outputs"].view(torch.int32)))
    hit = float(np.isin(with_region["idx"], hot).mean())
    per_expert = 3 * spec.I * spec.H // 2 + 3 * spec.I * (spec.H // 32) * 2 if spec.expert == 2 else \
        3 * spec.I * spec.H * (2 if spec.expert == 1 else 4)
    res = {
        "metric": f"MoE-layer decode us per token with a hot-expert region ({spec.name})",
        "value": with_region["us_per_token"], "unit": "us per token", "n_gpus": 1, "steps": K, "warmup": W,
        "higher_is_better": False, "data": "synthetic",
        "config": {"workload": f"{spec.name}: batch-1 decode, {K} tokens, {n_rep} router copies; region of the "
                               f"{N} experts most chosen over {ncal} calibration tokens "
                               f"({N * per_expert / 1e6:.0f} MB)",
                   "hit_rate": hit,
                   "us_per_token_no_region_fused": base["us_per_token"],
                   "us_per_token_region_no_hits": no_hits["us_per_token"],
                   "outputs_bitwise_equal": same,
                   "device_errors": layers[0].device_error()},
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "single-GPU implementation: --gpus above 1 is not supported "
                                   "(sharding by expert id across GPUs is not implemented)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import synth.device as SD

    if args.sweep:
        return sweep_main(args)
    if args.parity_stream:
        return parity_main(args)
    spec = synth.CONFIGS[args.config]
    if args.counters:
        return counters_main(args, spec)
    if spec.T > 1:
        return grouped_main(args, spec)
    if args.layers > 1:
        return layers_main(args, spec)
    if args.hot > 0 or args.host > 0:
        return hot_main(args, spec)
    K, W = args.steps, args.warmup
    screen = args.screen == "on"
    n_rep = (6 if screen else 3) if args.mode == "cold" else 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    dl = SD.device_layer(spec)
    routers = [dl.router_eh] + [SD.device_router(spec) for _ in range(n_rep - 1)]
    from expert_routing_quantized_amd import MOE_LAYER_SCREEN_OFF, MOE_LAYER_SCREEN_ON
    lflags = MOE_LAYER_SCREEN_ON if screen else MOE_LAYER_SCREEN_OFF
    layers = [SD.make_layer(dl, max_tokens=1, router=r, flags=lflags) for r in routers]
    # tokens: W warm-up, K timed, and as many after them as the oracle's
    # sample needs beyond the timed ones (run eagerly after the timing)
    n_cpu = max(args.cpu_sample, 0)
    NT = W + max(K, n_cpu)
    X = SD.device_tokens(spec, 0, NT)
    torch.cuda.synchronize()
    log(f"layer ready in {time.time() - t0:.1f}s: pool {dl.nbytes_pool() / 1e9:.2f} GB, "
        f"{n_rep} router copies")

    ws = layers[0].workspace(1)
    idx = torch.zeros((NT, spec.k), dtype=torch.int32, device=dev)
    gates = torch.zeros((NT, spec.k), dtype=torch.float32, device=dev)
    out = torch.zeros((NT, spec.H), dtype=torch.float32, device=dev)
    zbuf = torch.empty((spec.E,), dtype=torch.float64, device=dev)
    vbuf = torch.empty((spec.E,), dtype=torch.float32, device=dev)

    def token(t):
        # one moe_grouped_forward call per token (at T = 1 with 4-bit experts
        # the selection runs fused with gate/up)
        layers[t % n_rep].grouped_forward(X[t], 1, idx[t], gates[t], 0, out[t], ws)

    # eager pass over the warm-up tokens (also loads the kernels)
    for t in range(W):
        token(t)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g_warm, g_main, g_router = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g_warm, stream=s):
            for t in range(W):
                token(t)
        with torch.cuda.graph(g_main, stream=s):
            for t in range(W, W + K):
                token(t)
        with torch.cuda.graph(g_router, stream=s):
            for t in range(W, W + K):
                if screen:       # the screen kernel alone (router_screen without bounds)
                    layers[t % n_rep].router_screen(X[t], 1, vbuf, None, ws)
                else:
                    layers[t % n_rep].router_logits(X[t], 1, zbuf, ws)
    torch.cuda.synchronize()

    with torch.cuda.stream(s):
        g_warm.replay()
        torch.cuda.synchronize()
        ms = median_replay_ms(g_main, s)
        # the dominant kernel alone, same launch configuration
        g_router.replay()
        torch.cuda.synchronize()
        ms_router = median_replay_ms(g_router, s)
    # the sample's tokens past the timed ones, eagerly (outputs for the parity check)
    for t in range(W + K, NT):
        token(t)
    listed = 0.0
    if screen:
        # rows the screen recomputed per token (its waves' counts in the
        # workspace), over 32 eager tokens after the timed ones
        from expert_routing_quantized_amd import binding as B
        nw = (spec.E + 23) // 24                   # screen blocks: one count byte each
        cnt = []
        for t in range(W, W + min(32, K)):
            token(t)
            cnt.append(int(ws[256:256 + nw].to(torch.int64).sum().item()))
        listed = sum(cnt) / len(cnt)
    torch.cuda.synchronize()
    errs = [L.device_error() for L in layers]

    per_tok_s = ms / 1e3 / K
    tok_s = K / (ms / 1e3)
    by = step_bytes(spec, screen, listed)
    router_s = ms_router / 1e3 / K
    dom_bytes = screen_bytes(spec) if screen else by["router"]
    router_gbs = dom_bytes / router_s / 1e9
    res = {
        "metric": "MoE-layer decode tokens/s and achieved HBM GB/s (batch-1, 4-bit experts)"
                  if args.config == "decode_q4" else "MoE-layer decode tokens/s and achieved HBM GB/s (batch-1, bf16 experts)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{args.config} batch-1 decode: H={spec.H}, E={spec.E}, top-{spec.k}, I={spec.I}, "
                         + ("4-bit experts (32-blocks, fp16 scales)" if spec.expert == 2 else "bf16 experts")
                         + f", bf16 router and hidden states, {K} sequential tokens, "
                         + f"{args.mode} router ({n_rep} cop{'ies' if n_rep > 1 else 'y'})"
                         + (", routed through the int8 screen" if screen else "")),
            "operands": "x bf16, router bf16" + (" (int8 screen, exact integer dot products, then the listed "
                                                 "rows in bf16)" if screen else "")
                        + ", experts " + ("q4b32" if spec.expert == 2 else "bf16")
                        + ", fp32 accumulation, f64 near-tie refinement",
            "screen_rows_recomputed_per_token": listed if screen else None,
            "bytes_per_token": by["total"],
            "hbm_bytes_per_token_measured": (measured_step_traffic() if screen and args.mode == "cold"
                                             and args.config == "decode_q4" else None),
            "hbm_gbs": by["total"] / per_tok_s / 1e9,
            "us_per_token": per_tok_s * 1e6,
            "device_errors": errs,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("router screen (moe::screen_kernel<6, 4, 2, 1, 2>: int8 router, exact integer dot products)"
                       if screen else "router GEMV (moe::router_kernel<bf16, CPL=4, NT=1>)"),
            "achieved": router_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": router_gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic(screen) if args.mode == "cold" and args.config == "decode_q4" else None,
            "avg_launch_us": router_s * 1e6,
            "bytes_per_launch": dom_bytes,
        },
    }
    if args.cpu_sample > 0:
        n = args.cpu_sample
        gi = idx[W:W + n].cpu().numpy()
        gg = gates[W:W + n].cpu().numpy()
        go = out[W:W + n].cpu().numpy()
        base, parity, single = cpu_baseline(spec, W, n, gi, gg, go, dl)
        res["cpu_baseline"] = base
        res["config"]["parity_sample"] = parity
        res["config"]["oracle_other_threads"] = single
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
