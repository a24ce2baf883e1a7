"""Benchmark: Qwen3-30B-A3B-shaped 48-layer quantized MoE stack, bs=1 greedy
decode, one hipGraph per decode step.

One step = one token through all 48 MoE layers (router GEMV, top-8 routing,
dequant-on-read gate/up GEMV + SiLU*up, down GEMV + weighted combine,
residual + RMSNorm feeding the next layer); the layer-47 output feeds the next
step's layer 0. Weights are seeded synthetic N(0, 0.02) encoded as 4-bit
super-blocks (16.3 GB resident); the input is seeded bf16 N(0, 1).

Prints one JSON line (see the keys below). The default run: warmup 16, 256
timed steps, plus a full-size sampled parity check of step 0 against the CPU
oracle, the dominant kernel's roofline from HIP events, and the CPU oracle
timed on the host as a baseline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-stack decode tok/s at bs=1 + achieved HBM GB/s (% of MI355X peak)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("moe_gemv.hip", "moe_device.h", "moe_internal.h"):
        with open(os.path.join(ROOT, "quantized_moe_decode_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=4, help="passes over all layers for the kernel timing")
    ap.add_argument("--no-batched", action="store_true", help="skip the small-batch / prefill measurements")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the single-step percentiles and the single-layer calls (for counter runs)")
    ap.add_argument("--timeline", action="store_true",
                    help="instead of the benchmark line: per-layer timeline of replayed decode steps from the "
                         "in-kernel stamps of the profiling build (libqmoe_timeline.so)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device copy (reference kernel for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import quantized_moe_decode_gemv_amd as q
    from quantized_moe_decode_gemv_amd import build as qbuild

    if args.timeline:
        if not os.path.exists(qbuild.LIB_TIMELINE):
            sys.exit(f"{qbuild.LIB_TIMELINE} is not built: python -m quantized_moe_decode_gemv_amd.build --timeline")
        q.LIB_PATH = qbuild.LIB_TIMELINE

    S = synth.QWEN3_30B_A3B
    L = args.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 268435456 bytes read, 268435456 bytes written")
        del src, dst
    plan = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=L, max_tokens=1)

    # ------------------------------------------------------------ weights
    t0 = time.time()
    blob = torch.empty(plan.blob_bytes(), dtype=torch.uint8, device=dev)
    blob[: plan.header_bytes()].copy_(torch.from_numpy(plan.pack_header()))
    staging = torch.empty(plan.layer_bytes(), dtype=torch.uint8, pin_memory=True)
    host = staging.numpy()
    for layer in range(L):
        g = synth.layer_experts(S, layer, synth.GATE)
        u = synth.layer_experts(S, layer, synth.UP)
        d = synth.layer_experts(S, layer, synth.DOWN)
        plan.pack_layer(g, u, d, synth.router(S, layer), out=host)
        off = plan.layer_offset(layer)
        blob[off:off + plan.layer_bytes()].copy_(staging)
        if layer % 8 == 7 or layer == L - 1:
            log(f"weights: {layer + 1}/{L} layers generated and uploaded ({time.time() - t0:.0f}s)")
    del g, u, d
    assert plan.blob_check(blob[: plan.header_bytes()].cpu().numpy()) == 0

    # ------------------------------------------------------------ buffers and graph
    H, k = S.hidden, S.top_k
    xs = torch.zeros(L, H, dtype=torch.int16, device=dev)     # bf16 bits: layer inputs (ring)
    ys = torch.zeros(L, H, dtype=torch.float32, device=dev)   # layer outputs
    ids = torch.zeros(L, k, dtype=torch.int32, device=dev)    # routing record of the last step
    ws = torch.zeros(L, k, dtype=torch.float32, device=dev)
    scratch = plan.new_scratch(1, device=dev)
    x0 = synth.x_bf16(S, 3, 0)                                # seeded first token
    stream = torch.cuda.Stream()
    xs[0].copy_(torch.from_numpy(x0[0].view(np.int16)))
    torch.cuda.synchronize()
    if args.timeline:
        # the profiling build takes the layer base as kernel arguments, which
        # the graph keeps from its capture
        timeline_setup(plan, blob, q)
    graph = plan.capture_step(blob, xs, ys, 1, ids, ws, scratch=scratch, stream=stream)
    log("decode step captured as one graph")

    # step 0 from the seeded input; its per-layer results are kept for the
    # oracle leg below (the only place the oracle runs)
    graph.launch(stream)
    torch.cuda.synchronize()
    step0 = dict(xs=xs.cpu().numpy().view(np.uint16).copy(), ys=ys.cpu().numpy().copy(),
                 ids=ids.cpu().numpy().copy(), w=ws.cpu().numpy().copy())

    # ------------------------------------------------------------ timed decode
    for _ in range(args.warmup):
        graph.launch(stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        graph.launch(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps
    tok_s = 1000.0 / ms_per_step
    expert_bytes_per_token = L * S.top_k * S.expert_bytes
    router_bytes_per_token = L * S.n_experts * S.hidden * 4
    gbps = expert_bytes_per_token * tok_s / 1e9
    log(f"decode: {ms_per_step * 1e3:.1f} us/step, {tok_s:.1f} tok/s, expert bytes {gbps:.0f} GB/s")
    finite = bool(torch.isfinite(ys).all().item())
    if args.timeline:
        print(json.dumps(decode_timeline(plan, blob, graph, stream, L, ms_per_step, q, np, torch)), flush=True)
        return
    # spread of single steps (after the timed region, each replay between its own events)
    step_pct = None
    if not args.no_extras:
        step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(64)]
        for a, b in step_evs:
            a.record(stream)
            graph.launch(stream)
            b.record(stream)
        torch.cuda.synchronize()
        st_us = np.array([a.elapsed_time(b) * 1e3 for a, b in step_evs])
        step_pct = {"p10_us": round(float(np.percentile(st_us, 10)), 1),
                    "p50_us": round(float(np.percentile(st_us, 50)), 1),
                    "p90_us": round(float(np.percentile(st_us, 90)), 1), "replays": len(st_us)}
        log(f"single steps: {step_pct}")

    # ------------------------------------------------------------ dominant kernel (gate/up GEMV)
    # same launches as the decode step, with HIP events around the gate/up
    # kernel's execution, rotating over all layers (so no layer's experts are
    # cache-resident from the previous launch)
    gu_bytes = S.top_k * S.inter * 2 * (S.hidden // 256) * 144
    times = gate_up_launch_times(plan, blob, xs, L, args.kernel_reps, scratch, stream, torch)
    gu_us = float(np.mean(times)) * 1e3
    gu_p50 = float(np.median(times)) * 1e3
    gu_gbps = gu_bytes / (gu_us * 1e-6) / 1e9
    log(f"gate/up kernel: {gu_us:.2f} us avg over {len(times)} launches, {gu_gbps:.0f} GB/s")

    single = None
    if not args.no_extras:
        single = single_layer_measurements(S, blob, L, dev, stream, q, np, torch, synth)
        log(f"single layer calls: {json.dumps(single)}")

    mxfp4 = None
    if not args.no_extras:
        mxfp4 = mxfp4_decode(L, dev, stream, args, q, np, torch, synth)
        log(f"mxfp4 decode: {json.dumps(mxfp4)}")

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "gateup_kernel_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = tr.get("hbm_bytes_per_launch")

    # ------------------------------------------------------------ batched workloads on the same layers
    batched = None
    if not args.no_batched:
        batched = batched_measurements(S, blob, L, dev, stream, q, np, torch, synth)
        log(f"batched: {json.dumps(batched)}")

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(S, L, x0, step0)
        log(f"cpu oracle: {cpu}")
        log(f"step-0 parity: {parity}")
        cpu["all_cores"] = cpu_baseline_all_cores(S, L)
        log(f"cpu oracle, all cores: {cpu['all_cores']}")

    result = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) weights encoded as 4-bit super-blocks, bf16 N(0,1) input)",
        "config": {
            "workload": f"Qwen3-30B-A3B-shaped {L}-layer quantized MoE stack, bs=1 greedy decode, hipGraph per step",
            "hidden": S.hidden, "n_experts": S.n_experts, "top_k": S.top_k, "inter": S.inter, "layers": L,
            "global_batch": 1, "seq_len": 1, "parallelism": "single GPU",
        },
        "hbm": {
            "expert_bytes_per_token": expert_bytes_per_token,
            "router_bytes_per_token": router_bytes_per_token,
            "achieved_gbps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "with_router_gbps": round((expert_bytes_per_token + router_bytes_per_token) * tok_s / 1e9, 1),
        },
        "roofline": {
            "kernel": "gateup_kernel (dequant-on-read gate/up GEMV + SiLU*up)",
            "bound": "hbm",
            "achieved": round(gu_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gu_us, 3),
            "median_launch_us": round(gu_p50, 3),
            "launches": len(times),
        },
        "step_time": step_pct,
        "single_layer": single,
        "mxfp4": mxfp4,
        "cpu_baseline": cpu,
        "batched": batched,
        "parity_step0": parity,
        "outputs_finite": finite,
    }
    bad = plausibility(result)
    if bad:
        log(f"implausible figures withheld: {bad}")
    print(json.dumps(result), flush=True)


def plausibility(result):
    """Two-sided plausibility of the reported figures: a bandwidth above the
    HBM peak (any *_gbps, or a roofline's achieved GB/s) or a fraction or
    utilisation above 1 cannot come from a correct measurement. Each such
    figure is replaced by None and its path listed under "implausible";
    returns that list."""
    bad = []

    def walk(d, path):
        for key, v in list(d.items()):
            p = f"{path}.{key}" if path else key
            if isinstance(v, dict):
                walk(v, p)
                continue
            if isinstance(v, bool) or not isinstance(v, (int, float)):
                continue
            if key.endswith("gbps") or (key == "achieved" and d.get("unit") == "GB/s"):
                limit = HBM_PEAK_GBPS
            elif key in ("frac", "frac_of_peak", "mfma_util"):
                limit = 1.0
            else:
                continue
            if not v <= limit:
                d[key] = None
                bad.append(p)

    walk(result, "")
    result["implausible"] = bad
    return bad


def gate_up_launch_times(plan, blob, xs, L, reps, scratch, stream, torch):
    """Durations (ms) of reps x L gate/up launches (router, then gate/up with
    HIP events around it, rotating over the layers so no layer's experts are
    cache-resident from the previous launch), preceded by one pass over the
    layers that is not kept; every launch has events of its own and all
    passes are queued back to back, so the GPU does not idle between them."""
    n = (reps + 1) * L
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:            # torch creates the HIP event on first record
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        l = i % L
        plan.profile_gate_up(blob, l, xs[l], 1, a, b, scratch=scratch, stream=stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs[L:]]


def timeline_setup(plan, blob, q):
    """Hands the profiling build the blob's first layer and the layer size,
    from which its kernels find their layer (before the step is captured)."""
    import ctypes
    lib = q.load()
    lib.moe_timeline_setup.restype = ctypes.c_int
    lib.moe_timeline_setup.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong]
    assert lib.moe_timeline_setup(blob.data_ptr() + plan.layer_offset(0), plan.layer_bytes()) == 0


def decode_timeline(plan, blob, graph, stream, L, ms_per_step, q, np, torch, reps=6, batch=48):
    """Per-layer timeline of the captured decode step from the profiling
    build's s_memrealtime stamps (the tick measured here against the host
    clock): for each layer the router, gate/up
    and down spans (first workgroup start to last wave end) and the gaps
    between consecutive launches, plus two in-kernel marks: the router's norm
    (sum of squares reduced), gate/up's routing (top-k done) and first row's
    dot products, down's row partials (medians over workgroups, from the
    kernel's start). Medians over layers and over `reps` samples, each the
    last of `batch` back-to-back replays. For gate/up and down also the
    10th/50th/90th percentiles over the workgroups of each dispatch group of
    256 (start and end from the kernel's first start, the marks from the
    workgroup's own start), and the spread of the per-XCD medians; both over
    the layers away from the stack's ends."""
    import ctypes
    lib = q.load()
    lib.moe_timeline_reset.restype = ctypes.c_int
    lib.moe_timeline_read.restype = ctypes.c_int
    lib.moe_timeline_read.argtypes = [ctypes.c_void_p]
    assert L <= 64
    rec = np.zeros((256, 1024, 8), dtype=np.uint64)

    # the stamp clock against the host clock: two replays 0.5 s apart, each
    # submitted to an idle GPU; the first router's start stamps differ by the
    # submit interval up to the (small, similar) submit-to-start latencies
    def first_start():
        assert lib.moe_timeline_read(rec.ctypes.data) == 0
        v = rec[0, :, 0]
        return float(v[v > 0].min())
    torch.cuda.synchronize()
    t_a = time.perf_counter()
    graph.launch(stream)
    torch.cuda.synchronize()
    s_a = first_start()
    time.sleep(0.5)
    t_b = time.perf_counter()
    graph.launch(stream)
    torch.cuda.synchronize()
    s_b = first_start()
    tick_mhz = (s_b - s_a) / (t_b - t_a) / 1e6
    us_per_tick = 1.0 / tick_mhz
    rows, step_stamps, batch_step_us = [], [], []
    # per-workgroup distributions of the gate/up and down launches: by
    # dispatch group (workgroups 0-255 take one CU each, the next 256 share
    # CUs with them) and by XCD (workgroup id mod 8)
    wg_kinds = ((1, "gateup", {"routing_known": 5, "row0_dots": 6}), (2, "down", {"row_partials": 6}))
    by_group, by_xcd = {}, {}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    assert lib.moe_timeline_reset() == 0
    for _ in range(reps):
        # the stamps of the last of `batch` back-to-back replays (every
        # workgroup rewrites its record each step), i.e. of a step in the
        # steady state that the timed decode loop runs in
        ev0.record(stream)
        for _ in range(batch):
            graph.launch(stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        batch_step_us.append(ev0.elapsed_time(ev1) * 1e3 / batch)
        assert lib.moe_timeline_read(rec.ctypes.data) == 0
        r = rec.astype(np.float64)

        def span(slot):
            st = r[slot, :, 0]
            en = r[slot, :, 1:5]
            return st[st > 0].min(), en[en > 0].max()

        def mark(slot, field, t0):
            v = r[slot, :, field]
            v = v[v > 0]
            return float(np.median(v) - t0) * us_per_tick if len(v) else None

        base = span(0)[0]
        for l in range(L):
            rs, re_ = span(4 * l)
            gs, ge = span(4 * l + 1)
            ds, de = span(4 * l + 2)
            ns = span(4 * (l + 1))[0] if l + 1 < L else span(3)[0]
            row = {"router": re_ - rs, "gap_router_gateup": gs - re_, "gateup": ge - gs, "gap_gateup_down": ds - ge,
                   "down": de - ds, "gap_down_next": ns - de}
            row = {k2: v * us_per_tick for k2, v in row.items()}
            row["layer_period"] = (ns - rs) * us_per_tick
            if l > 0:
                row["router_norm_mark"] = mark(4 * l, 5, rs)
            row["gateup_topk_mark"] = mark(4 * l + 1, 5, gs)
            row["gateup_row0_mark"] = mark(4 * l + 1, 6, gs)
            row["down_partials_mark"] = mark(4 * l + 2, 6, ds)
            rows.append(row)
            if 2 <= l < L - 2:
                for kind, name, fields in wg_kinds:
                    x = r[4 * l + kind]
                    nwg = int(np.count_nonzero(x[:, 0]))
                    x = x[:nwg]
                    st = x[:, 0]
                    t0 = st.min()
                    series = {"start": st - t0, "end": x[:, 1:5].max(1) - t0}
                    series.update({f: np.where(x[:, i] > 0, x[:, i] - st, np.nan) for f, i in fields.items()})
                    wg = np.arange(nwg)
                    for g in range((nwg + 255) // 256):
                        m = wg // 256 == g
                        for f, v in series.items():
                            by_group.setdefault((name, g, f), []).append(np.nanpercentile(v[m], [10, 50, 90]) * us_per_tick)
                    for xcd in range(8):
                        m = wg % 8 == xcd
                        for f, v in series.items():
                            by_xcd.setdefault((name, xcd, f), []).append(np.nanmedian(v[m]) * us_per_tick)
        step_stamps.append((span(3)[1] - base) * us_per_tick)
    keys = list(rows[-1].keys())
    med = {k2: round(float(np.median([rw[k2] for rw in rows if rw.get(k2) is not None])), 3) for k2 in keys}
    parts = ("router", "gap_router_gateup", "gateup", "gap_gateup_down", "down", "gap_down_next")
    groups = {}
    for (name, g, f), v in by_group.items():
        key = f"{name}_wg{256 * g}-{256 * g + 255}"
        groups.setdefault(key, {})[f] = [round(float(a), 2) for a in np.median(np.array(v), axis=0)]
    xcd_spread = {}
    for _, name, fields in wg_kinds:
        for f in ("start", "end", *fields):
            meds = [float(np.median(by_xcd[(name, xcd, f)])) for xcd in range(8)]
            xcd_spread[f"{name}_{f}"] = round(max(meds) - min(meds), 3)
    return {
        "timeline": {
            "per_layer_median_us": med,
            "sum_of_parts_us": round(sum(med[p] for p in parts), 3),
            "layers": L,
            "samples": reps,
            "replays_per_sample": batch,
            "workgroups_by_dispatch_group_p10_p50_p90_us": groups,
            "xcd_median_spread_us": xcd_spread,
            "step_us_stamps_median": round(float(np.median(step_stamps)), 1),
            "step_us_events_instrumented": round(ms_per_step * 1e3, 1),
            "step_us_events_sampled_batches": round(float(np.median(batch_step_us)), 1),
            "clock": "s_memrealtime",
            "clock_mhz_measured": round(tick_mhz, 3),
        },
        "config": {"workload": f"Qwen3-30B-A3B-shaped {L}-layer quantized MoE stack, bs=1 decode step, hipGraph",
                   "library": "libqmoe_timeline.so (-DQMOE_TIMELINE)"},
    }


MFMA_FP16_PEAK_TFLOPS = 2500.0


def mxfp4_decode(L, dev, stream, args, q, np, torch, synth):
    """The same decode step with MXFP4 expert weights: the L layers'
    Gaussian weights encoded as FP4 E2M1 codes with an E8M0 scale per 32
    (4.25 bits per weight), a blob of their own, the step captured as one
    graph and timed like the main leg; plus the gate/up kernel alone and the
    batched legs on the MXFP4 paths (the grouped path is its 16-pair MFMA
    tiles at every size)."""
    S = synth.QWEN3_30B_A3B_MXFP4
    plan = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=L, max_tokens=1, flags=q.FLAG_WEIGHTS_MXFP4)
    t0 = time.time()
    blob = torch.empty(plan.blob_bytes(), dtype=torch.uint8, device=dev)
    blob[: plan.header_bytes()].copy_(torch.from_numpy(plan.pack_header()))
    staging = torch.empty(plan.layer_bytes(), dtype=torch.uint8, pin_memory=True)
    host = staging.numpy()
    for layer in range(L):
        plan.pack_layer(synth.layer_experts(S, layer, synth.GATE), synth.layer_experts(S, layer, synth.UP),
                        synth.layer_experts(S, layer, synth.DOWN), synth.router(S, layer), out=host)
        off = plan.layer_offset(layer)
        blob[off:off + plan.layer_bytes()].copy_(staging)
        if layer % 16 == 15 or layer == L - 1:
            log(f"mxfp4 weights: {layer + 1}/{L} layers generated and uploaded ({time.time() - t0:.0f}s)")
    H, k = S.hidden, S.top_k
    xs = torch.zeros(L, H, dtype=torch.int16, device=dev)
    ys = torch.zeros(L, H, dtype=torch.float32, device=dev)
    ids = torch.zeros(L, k, dtype=torch.int32, device=dev)
    ws = torch.zeros(L, k, dtype=torch.float32, device=dev)
    scratch = plan.new_scratch(1, device=dev)
    xs[0].copy_(torch.from_numpy(synth.x_bf16(S, 3, 0)[0].view(np.int16)))
    torch.cuda.synchronize()
    graph = plan.capture_step(blob, xs, ys, 1, ids, ws, scratch=scratch, stream=stream)
    for _ in range(args.warmup):
        graph.launch(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        graph.launch(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    finite = bool(torch.isfinite(ys).all().item())
    expert_bytes = L * S.top_k * S.expert_bytes
    # gate/up kernel alone, rotating over the layers
    gu_bytes = S.top_k * S.inter * 2 * S.hidden // 32 * 17
    times = gate_up_launch_times(plan, blob, xs, L, args.kernel_reps, scratch, stream, torch)
    gu_us = float(np.mean(times)) * 1e3
    batched = None
    if not args.no_batched:
        batched = batched_measurements(S, blob, L, dev, stream, q, np, torch, synth, base_flags=q.FLAG_WEIGHTS_MXFP4,
                                       paths={8: ("gemv", "expert_gemv"), 32: ("expert_gemv", "grouped"),
                                              128: ("expert_gemv", "grouped"), 256: ("grouped",)}, with_zipf=True)
    del graph, blob, staging
    torch.cuda.synchronize()
    return {"us_per_step": round(us, 1), "tok_s": round(1e6 / us, 1), "expert_bytes_per_token": expert_bytes,
            "expert_gbps": round(expert_bytes / us * 1e-3, 1), "gateup_us": round(gu_us, 3),
            "gateup_bytes_per_launch": gu_bytes, "gateup_gbps": round(gu_bytes / gu_us * 1e-3, 1),
            "outputs_finite": finite, "batched": batched}


def _graph_us(calls, n_rot, reps, stream, torch):
    """Capture calls(0..n_rot-1) in one CUDA graph on `stream`, replay it, and
    return the average time per call in microseconds (HIP events on `stream`)."""
    with torch.cuda.stream(stream):
        calls(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for l in range(n_rot):
                calls(l)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):          # replay() launches on the current stream
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n_rot)


def single_layer_measurements(S, blob, L, dev, stream, q, np, torch, synth):
    """One token through one layer (router GEMV, top-k, gate/up, down; no
    norm), graph-replayed: the tiny layer (hidden 256, 8 experts, top-2,
    inter 512: 442,368 expert bytes per call) and the Qwen3-30B-A3B-shaped
    layer rotating over 16 layers of the stack (21,233,664 expert bytes per
    call, so no layer's experts are cache-resident from the previous call),
    the latter also with the ReLU2 and SwiGLU-OAI gate activations."""
    res = {}
    T = synth.TINY
    tplan = q.Plan(T.hidden, T.n_experts, T.top_k, T.inter, n_layers=1, max_tokens=1)
    tblob = torch.empty(tplan.blob_bytes(), dtype=torch.uint8, device=dev)
    tblob[: tplan.header_bytes()].copy_(torch.from_numpy(tplan.pack_header()))
    host = np.empty(tplan.layer_bytes(), dtype=np.uint8)
    tplan.pack_layer(synth.layer_experts(T, 0, synth.GATE), synth.layer_experts(T, 0, synth.UP),
                     synth.layer_experts(T, 0, synth.DOWN), synth.router(T, 0), out=host)
    off = tplan.layer_offset(0)
    tblob[off:off + tplan.layer_bytes()].copy_(torch.from_numpy(host))
    tscr = tplan.new_scratch(1, device=dev)
    tx = torch.from_numpy(synth.x_bf16(T, 0, 0).view(np.int16)).to(dev)
    ty = torch.empty(1, T.hidden, dtype=torch.float32, device=dev)
    us = _graph_us(lambda l: tplan.forward(tblob, 0, tx, 1, ty, scratch=tscr, stream=stream), 16, 20, stream, torch)
    res["tiny_layer"] = {"us_per_call": round(us, 2), "expert_bytes": T.top_k * T.expert_bytes}
    plan = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=L, max_tokens=1)
    scr = plan.new_scratch(1, device=dev)
    x = torch.from_numpy(synth.x_bf16(S, 3, 1).view(np.int16)).to(dev)
    y = torch.empty(1, S.hidden, dtype=torch.float32, device=dev)
    n_rot = min(L, 16)
    us = _graph_us(lambda l: plan.forward(blob, l, x, 1, y, scratch=scr, stream=stream), n_rot, 20, stream, torch)
    eb = S.top_k * S.expert_bytes
    res["qwen3_30b_a3b_layer"] = {"us_per_call": round(us, 2), "expert_bytes": eb,
                                 "expert_gbps": round(eb / (us * 1e-6) / 1e9, 1)}
    # the same calls with the other gate activations (epilogue only: same bytes)
    for name, flag in (("relu2", q.FLAG_ACT_RELU2), ("swiglu_oai", q.FLAG_ACT_SWIGLU_OAI)):
        aplan = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=L, max_tokens=1, flags=flag)
        us = _graph_us(lambda l: aplan.forward(blob, l, x, 1, y, scratch=scr, stream=stream), n_rot, 20, stream, torch)
        res["qwen3_30b_a3b_layer"][f"us_per_call_{name}"] = round(us, 2)
    return res


def batched_measurements(S, blob, L, dev, stream, q, np, torch, synth, base_flags=0, paths=None, with_zipf=True):
    """Small-batch decode / short prefill (T = 2 ... 256; N(0,1) logits) on
    the per-token GEMV path, the expert-major GEMV path and the grouped MFMA
    path, and the Zipf-skewed 4096-token chunk on the grouped path. Routing from given logits, expert
    FFN only, each call on a different layer of the stack in turn (so a
    layer's experts are not cache-resident from the previous call); captured
    in a graph, timed with HIP events. Unique expert bytes = experts with at
    least one routed pair x the shape's expert bytes (2,654,208 B; MXFP4
    2,506,752 B). base_flags / paths / with_zipf select the weight encoding
    and the cases."""
    res = {}
    n_rot = min(L, 16)

    def run_case(T, zipf, flag, case):
        plan = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=L, max_tokens=T, flags=flag | base_flags)
        scratch = plan.new_scratch(T, device=dev)
        xb = synth.x_bf16(S, case, T, T=T)
        x = torch.from_numpy(xb.view(np.int16)).to(dev)
        lg = torch.from_numpy(synth.logits_f32(S, case, T, zipf_s=zipf)).to(dev)
        k, E = S.top_k, S.n_experts
        ids = torch.empty(T, k, dtype=torch.int32, device=dev)
        w = torch.empty(T, k, dtype=torch.float32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        pairs = torch.empty(T * k, dtype=torch.int32, device=dev)
        out = torch.empty(T, S.hidden, dtype=torch.float32, device=dev)

        def calls(l):
            plan.route(blob, l, None, lg, T, ids, w, counts, offsets, pairs, scratch=scratch, stream=stream)
            plan.expert_ffn(blob, l, x, T, ids, w, out, counts, offsets, pairs, scratch=scratch, stream=stream)

        with torch.cuda.stream(stream):
            calls(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for l in range(n_rot):
                    calls(l)
        reps = 3 if T >= 1024 else 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):          # replay() launches on the current stream
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * n_rot)
        cnt = counts.cpu().numpy()
        uniq = int((cnt > 0).sum())
        ubytes = uniq * S.expert_bytes
        flops = 2.0 * T * k * 3 * S.hidden * S.inter
        r = {"us": round(us, 2), "unique_experts": uniq, "unique_expert_gbps": round(ubytes / (us * 1e-6) / 1e9, 1),
             "tflops": round(flops / (us * 1e-6) / 1e12, 2)}
        if zipf:
            top = np.sort(cnt)[::-1]
            r["expert_pairs"] = {"largest": [int(v) for v in top[:8]], "experts_ge_88": int((cnt >= 88).sum()),
                                 "empty": int((cnt == 0).sum()), "top8_share": round(float(top[:8].sum() / cnt.sum()), 3)}
        return r

    flags = {"gemv": q.FLAG_FORCE_GEMV, "expert_gemv": q.FLAG_FORCE_EXPERT_GEMV, "grouped": q.FLAG_FORCE_GROUPED}
    if paths is None:
        paths = {2: ("gemv", "expert_gemv"), 8: tuple(flags), 32: tuple(flags), 128: tuple(flags),
                 256: ("expert_gemv", "grouped")}
    for T, names in paths.items():
        res[f"T{T}"] = {name: run_case(T, None, flags[name], 3) for name in names}
    if with_zipf:
        z = run_case(4096, 1.1, q.FLAG_FORCE_GROUPED, 4)
        z["mfma_util"] = round(z["tflops"] / MFMA_FP16_PEAK_TFLOPS, 4)
        res["T4096_zipf"] = z
    res["note"] = "route (given logits) + expert FFN per call; us per call averaged over rotating layers"
    return res


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(S, L, x0, gpu):
    """The CPU oracle, as it stands (plain scalar C, fp64, one thread), run
    over one full decode step of the same stack from the same seeded input.
    Only its arithmetic is timed (router logits, top-k, softmax, expert FFNs,
    weighted sum, RMSNorm); generating the selected experts' encoded blocks is
    not. The oracle's own trajectory is also compared with the GPU's step 0:
    a layer whose GPU input is bitwise the oracle's must match its routing
    ids (near-tie rule), y within max|err| <= 2e-3 * max|ref| and x_next
    within one bf16 step or that tolerance; after bf16 rounding flips have put
    the inputs apart the trajectories are followed while they still agree."""
    import numpy as np
    import oracle
    import synth

    tau, tol = 1e-4, 2e-3
    src = oracle.ExpertSource(S, max_cached=16)
    x = x0[0]
    t_oracle = 0.0
    worst, flips, compared, exact, stopped, same = 0.0, 0, 0, 0, None, True
    for l in range(L):
        wr = synth.router(S, l)
        t = time.perf_counter()
        lg = oracle.router_logits(wr, x)
        rid, rw, gap = oracle.route(lg, S.top_k)
        t_oracle += time.perf_counter() - t
        bl = [src.blocks(l, e) for e in rid]
        t = time.perf_counter()
        y = oracle.moe_token([b[0] for b in bl], [b[1] for b in bl], [b[2] for b in bl], rw, x)
        _, xn = oracle.resid_rmsnorm(x, y)
        t_oracle += time.perf_counter() - t
        if stopped is None:
            g_next = gpu["xs"][(l + 1) % L]
            err = np.abs(gpu["ys"][l] - y).max() / np.abs(y).max()
            g = oracle.bf16_array(g_next)
            r = oracle.bf16_array(xn)
            step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126))) - 7)
            near = bool(np.all(np.abs(g - r) <= np.maximum(step, tol * np.abs(r).max())))
            if set(gpu["ids"][l].tolist()) != set(rid.tolist()):
                if same and gap > tau:
                    raise AssertionError(f"layer {l}: GPU ids {gpu['ids'][l]} vs oracle {rid} (gap {gap:.2e})")
                stopped = f"routing parted at layer {l} (gap {gap:.1e})"
            elif err > tol or not near:
                if same:
                    raise AssertionError(f"layer {l}: max|err|/max|ref| = {err:.3e}, x_next within bound: {near}")
                stopped = f"trajectories parted at layer {l}"
            else:
                worst = max(worst, err)
                flips += int(np.count_nonzero(g != r))
                compared += 1
                exact += int(same)
                same = bool(np.array_equal(g_next, xn))
        x = xn
    cpu = {
        "value": round(1.0 / t_oracle, 5),
        "unit": "tok/s",
        "cores": 1,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"one full decode step ({L} layers, 1 token) from the same seeded input; "
                  f"oracle arithmetic timed ({t_oracle:.1f} s), expert block generation excluded",
    }
    parity = {"layers_compared": compared, "layers_on_identical_inputs": exact,
              "worst_rel_err": float(f"{worst:.3e}"), "x_next_bf16_differences": flips, "tolerance": tol,
              "stopped": stopped}
    return cpu, parity


def cpu_baseline_all_cores(S, L):
    """The same oracle, unchanged, on every usable host core at once (up to
    16): one thread per core, each taking independent tokens (its own seeded input)
    through layers 0-7 of the stack (router, top-k, softmax, expert FFNs,
    weighted sum, RMSNorm; the oracle's C routines release the interpreter
    lock). Expert blocks are generated beforehand and not timed. tok/s is the
    number of (token, layer) items finished per second of wall time divided by
    the stack's layer count (the items are run four times over)."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    import synth

    cores = min(len(os.sched_getaffinity(0)), 16)    # the process's CPU share, at most 16 threads
    layers = list(range(8))
    src = oracle.ExpertSource(S, max_cached=4 * S.n_experts)
    items = []
    for l in layers:
        wr = synth.router(S, l)
        for i in range(cores):
            x = synth.x_bf16(S, 5, i)[0]
            rid, rw, _ = oracle.route(oracle.router_logits(wr, x), S.top_k)
            items.append((wr, x, [src.blocks(l, e) for e in rid]))

    def run(item):
        wr, x, bl = item
        rid, rw, _ = oracle.route(oracle.router_logits(wr, x), S.top_k)
        y = oracle.moe_token([b[0] for b in bl], [b[1] for b in bl], [b[2] for b in bl], rw, x)
        return oracle.resid_rmsnorm(x, y)[1]

    reps = 4
    t = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        list(ex.map(run, items * reps))
    wall = time.perf_counter() - t
    return {"value": round(reps * len(items) / wall / L, 5), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} x {len(items)} (token, layer) items ({cores} independent tokens x layers 0-7), "
                      f"{wall:.2f} s wall; tok/s = items per second / {L} layers"}


if __name__ == "__main__":
    main()
