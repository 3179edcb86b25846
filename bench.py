#!/usr/bin/env python3
"""Throughput of the MoE decode layer on one MI355X.

A step is one call of moe_decode_layer (or moe_decode_stack for the stack
workload): RMSNorm, router over all experts, softmax + top-k +
renormalisation, gathered SwiGLU experts, the shared expert, the weighted
combine and the residual, for one batch of B tokens, in one kernel launch.

Inputs are seeded and synthetic (synth/): weights ~N(0, 0.02), tokens
~N(0, 1), all 896 experts drawn on the device. So that no step finds the
previous step's weights in the 256 MB memory-side cache, the timed loop
rotates over `--copies` layer instances that each hold their own router,
shared expert and RMSNorm gain (drawn as layers 0..copies-1 of the
workload's seed) and their own token batch; the routed-expert tensor is
common to them (the routing of different instances picks nearly disjoint
experts).

With --unfused a step is one call of moe_decode_layer_unfused instead (of
moe_decode_stack_unfused for the stack workload): the same layer as eleven
kernel launches with every intermediate in device memory, the baseline the
fused kernel is measured against. --side shared|prefetch|both moves the shared
expert and / or a next-layer weight prefetch of that path to a second stream
(moe_decode_stack_unfused's flags).

`value` is tokens per second (B / step time). The roofline object gives the
weight bytes the step must touch (router + shared + gain + every distinct
selected expert, each counted once per step) over the measured kernel time,
against the 8 TB/s HBM peak. The CPU baseline times the plain oracle on a
few tokens of the same workload on the host.
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

WORKLOAD_NOTES = {
    "tiny_f32": "tiny fp32 MoE layer H=256 E=32 k=4 I=Is=128",
    "k3_b1": "K3-scale layer share H=7168 E=896 k=16 I=1024 Is=2048, bf16 experts/shared, fp32 router",
    "k3_b8": "K3-scale layer share at B=8",
    "k3_b64_zipf": "K3-scale layer share at B=64 with log-Zipf(1.1) router bias",
    "k3_stack4_fp8": "4-layer K3-scale stack, fp8 e4m3 experts (bf16 scale per 128 rows), bf16 router/shared",
    "k3_spec_verify": "K3-scale layer share, speculative-decoding verify step: requests of 1 base + 7 draft tokens "
                      "(drafts = base + 0.5 N(0,1))",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="k3_b1",
                    choices=["tiny_f32", "k3_b1", "k3_b8", "k3_b64_zipf", "k3_stack4_fp8", "k3_spec_verify"])
    ap.add_argument("--batch", type=int, default=None, help="tokens per step (default: the workload's first)")
    ap.add_argument("--copies", type=int, default=8, help="layer instances the timed loop rotates over")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="time the multi-launch path (moe_decode_layer_unfused) instead of the fused kernel")
    ap.add_argument("--side", choices=["none", "shared", "prefetch", "both"], default="none",
                    help="with --unfused: work on a second stream (the shared expert, the next layer's prefetch)")
    return ap.parse_args()


def cpu_baseline(w, B, budget_s):
    """The oracle (single-threaded plain C) on tokens of the same workload,
    until about budget_s seconds of oracle time have run, on one core: the
    calling thread pins itself to the last core it may use (Linux applies
    sched_setaffinity(0) to the calling thread only) and restores its
    affinity afterwards."""
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[-1]
    os.sched_setaffinity(0, {core})
    try:
        return _cpu_baseline_pinned(w, B, budget_s, core, len(allowed))
    finally:
        os.sched_setaffinity(0, allowed)


def _cpu_baseline_pinned(w, B, budget_s, core, ncores):
    import numpy as np

    import oracle
    import synth
    d = oracle.desc_of(w)
    layers = []
    for l in range(w.layers):
        L = oracle.Layer(gamma=synth.gamma(w, layer=l), router_w=synth.router_w(w, l),
                         router_bias=synth.router_bias(w, l), gate_up={}, down={},
                         shared_gate_up=synth.shared_gate_up(w, l), shared_down=synth.shared_down(w, l))
        layers.append(L)

    def need_experts(xt):
        # materialise the experts each layer of this token selects (generation is not timed)
        cur = xt
        for l, L in enumerate(layers):
            xhat, _ = oracle.rmsnorm(d, cur[0], L.gamma)
            idx, _ = oracle.route(d, oracle.router_logits(d, L, xhat))
            for e in idx:
                e = int(e)
                if e not in L.gate_up:
                    L.gate_up[e], s1 = synth.expert_gate_up(w, e, l)
                    L.down[e], s2 = synth.expert_down(w, e, l)
                    if s1 is not None:
                        L.gate_up_scale[e], L.down_scale[e] = s1, s2
            if l + 1 < len(layers):
                cur, _, _, _ = oracle.layer(d, L, cur)

    x = synth.x_tokens(w, max(B, 1))
    spent, ntok, t = 0.0, 0, 0
    while spent < budget_s and ntok < 4096:
        xt = np.ascontiguousarray(x[t % x.shape[0]][None, :])
        need_experts(xt)
        t0 = time.perf_counter()
        if w.layers == 1:
            oracle.layer(d, layers[0], xt)
        else:
            oracle.stack(d, layers, xt)
        spent += time.perf_counter() - t0
        ntok += 1
        t += 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": ntok / spent, "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"{ntok} token(s) of {w.name}, one at a time, {spent:.1f} s of single-threaded oracle time",
            "s_per_step": B * spent / ntok, "cpu_model": model, "host_cores": os.cpu_count(),
            "pinned_core": core, "cores_allowed": ncores}


# launch shapes of the streaming probe: (256-thread workgroups per CU, 16-byte
# loads in flight per lane), i.e. workgroups x loads x 4 KB in flight per CU
# (as far as the workgroups are resident): "wide" fills every wave slot,
# "tuned" keeps 32 KB per CU, where a 4 GiB read sweep peaked on MI355X (more
# in flight lowers the rate)
PROBE_SHAPES = {"wide": (16, 8), "tuned": (4, 2)}


def stream_probe(torch, md, dev, stream, gib=4, reps=5):
    """HBM read rate (GB/s) of a plain 16-byte streaming kernel over `gib` GiB
    for each probe shape: the practical ceiling of a weight-streaming step."""
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    lib = md.probe_lib()
    out = {}
    for name, (wg_per_cu, loads) in PROBE_SHAPES.items():
        best = 0.0
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = lib.moe_probe_stream_read_u(buf.data_ptr(), n, sink.data_ptr(), cus * wg_per_cu, loads,
                                             stream.cuda_stream)
            b.record(stream)
            if rc != 0:
                raise RuntimeError(f"moe_probe_stream_read_u failed: hip error {rc}")
            torch.cuda.synchronize()
            best = max(best, n / (a.elapsed_time(b) * 1e-3) / 1e9)
        out[name] = best
    del buf
    return out


def calibration_copy(torch, md, dev, stream):
    """One plain copy of a known size (1 GiB), whose FETCH_SIZE / WRITE_SIZE
    counters calibrate those of the decode kernel in a --pmc profile."""
    from moe_decode_02_amd.profiling import COPY_BYTES
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(3)
    grid = torch.cuda.get_device_properties(dev).multi_processor_count * 16
    rc = md.probe_lib().moe_probe_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, grid, stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"moe_probe_copy failed: hip error {rc}")
    torch.cuda.synchronize()
    del src, dst


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding of the layer is a design, not code)", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import moe_decode_02_amd as md
    import synth
    from synth.device import DeviceLayer, act_tensor, desc_of, to_device, workspace

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    md.lib()  # fails loudly when the HIP library is not built
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    B = args.batch or w.B
    L = w.layers
    C = max(1, args.copies)
    d = desc_of(w)
    log(f"bench: {w.name} B={B} layers={L} copies={C} on {torch.cuda.get_device_name(0)}")

    # layer instances: instance c, layer l uses generator layer index c*L + l for its
    # router / shared / gain; routed experts of layer l are shared by all instances
    t0 = time.time()
    base = [DeviceLayer(w, layer=l, device=dev) for l in range(L)]
    insts = []
    for c in range(C):
        layers = []
        for l in range(L):
            if c == 0:
                layers.append(base[l])
                continue
            li = DeviceLayer.__new__(DeviceLayer)
            li.__dict__.update(base[l].__dict__)
            gl = c * L + l
            li.gamma = to_device(synth.gamma(w, layer=gl), dev)
            li.router_w = to_device(synth.router_w(w, gl), dev)
            b = synth.router_bias(w, gl)
            li.router_bias = to_device(b, dev) if b is not None else None
            if w.Is > 0:
                li.sgu = torch.empty_like(base[l].sgu)
                li.sd = torch.empty_like(base[l].sd)
                synth.fill_device(li.sgu, synth.key(w.seed, gl, synth.T_SHARED_GU), w.shared, synth.WEIGHT_SIGMA)
                synth.fill_device(li.sd, synth.key(w.seed, gl, synth.T_SHARED_D), w.shared, synth.WEIGHT_SIGMA)
            li.weights = li._struct()
            layers.append(li)
        insts.append(layers)
    xs = []
    for c in range(C):
        xs.append(to_device(synth.x_tokens(w, B, layer=100 + c), dev))
    ys = [act_tensor(w, B, dev) for _ in range(C)]
    idx = [torch.zeros((L, B, w.k), dtype=torch.int32, device=dev) for _ in range(C)]
    wts = [torch.zeros((L, B, w.k), dtype=torch.float32, device=dev) for _ in range(C)]
    ws = workspace(d, B, L, dev)
    flags = {"none": 0, "shared": md.MOE_UF_SHARED_SIDE, "prefetch": md.MOE_UF_PREFETCH_SIDE,
             "both": md.MOE_UF_SHARED_SIDE | md.MOE_UF_PREFETCH_SIDE}[args.side]
    if flags and not args.unfused:
        log("bench: --side applies to the multi-launch path (--unfused)")
        return 2
    side = torch.cuda.Stream(device=dev) if flags else None  # default priority
    if args.unfused:
        ws_unf = torch.empty(md.moe_unfused_stack_workspace_bytes(d, B, L), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"bench: inputs ready in {time.time() - t0:.1f} s, {torch.cuda.memory_allocated() / 2**30:.1f} GiB on the GPU")

    stream = torch.cuda.current_stream(dev)

    def step(i):
        c = i % C
        if args.unfused and L == 1 and not flags:
            md.moe_decode_layer_unfused(d, insts[c][0].weights, xs[c], ys[c], B, idx[c], wts[c], ws_unf,
                                        stream=stream)
        elif args.unfused:
            md.moe_decode_stack_unfused(d, [li.weights for li in insts[c]], xs[c], ys[c], B, idx[c], wts[c], ws_unf,
                                        stream=stream, side_stream=side, flags=flags)
        elif L == 1:
            md.moe_decode_layer(d, insts[c][0].weights, xs[c], ys[c], B, idx[c], wts[c], ws, stream=stream)
        else:
            md.moe_decode_stack(d, [li.weights for li in insts[c]], xs[c], ys[c], B, idx[c], wts[c], ws,
                                stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if md.moe_check_workspace(ws) != md.MOE_OK:
        log("bench: a warm-up launch hit its barrier watchdog")
        return 1

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    if md.moe_check_workspace(ws) != md.MOE_OK:
        log("bench: a timed launch hit its barrier watchdog")
        return 1
    ms_step = ms_total / args.steps
    # algorithmic bytes of each instance that the timed steps ran (its routing
    # as its last call left it): weights touched, each counted once per step
    per_inst = {}
    for c in sorted({i % C for i in range(args.steps)}):
        sel = idx[c].cpu().numpy()
        per_inst[c] = sum(insts[c][l].touched_bytes(sel[l]) for l in range(L))
    nbytes = sum(per_inst[i % C] for i in range(args.steps)) / args.steps
    distinct = [float(np.mean([len(np.unique(idx[c].cpu().numpy()[l])) for l in range(L)])) for c in per_inst]
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    for c in range(C):
        if not torch.isfinite(ys[c].float()).all():
            log(f"bench: non-finite output in instance {c}")
            return 1

    # per-launch spread (events around single launches, after the timed region)
    per = []
    for i in range(min(args.steps, 200)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(i)
        b.record(stream)
        per.append((a, b))
    torch.cuda.synchronize()
    lat = np.array([a.elapsed_time(b) * 1e3 for a, b in per])
    log(f"bench: {ms_step * 1e3:.1f} us/step over {args.steps} steps (wall {wall / args.steps * 1e6:.1f} us), "
        f"single-launch median {np.median(lat):.1f} p95 {np.percentile(lat, 95):.1f} min {lat.min():.1f} us, "
        f"{nbytes / 1e6:.1f} MB/step -> {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of 8 TB/s)")

    calibration_copy(torch, md, dev, stream)
    probes = stream_probe(torch, md, dev, stream)
    probe = max(probes.values())
    log("bench: streaming-read probe " + ", ".join(f"{k} {v:.0f} GB/s" for k, v in probes.items()) +
        f"; the step reaches {gbs / probe:.1%} of the best")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, B, args.cpu_seconds)
        log(f"bench: cpu baseline {cpu}")

    # HBM bytes per launch measured by the committed FETCH_SIZE / WRITE_SIZE
    # profile of this workload, if it was taken on the current kernel source
    from moe_decode_02_amd.profiling import read_traffic
    tr = None if args.unfused else read_traffic(os.path.join(ROOT, "profiles", f"moe_kernel_{w.name}_B{B}_traffic.txt"))
    hbm_bytes = None if tr is None else tr["read"] + tr["write"]
    traffic = None if tr is None else hbm_bytes / (ms_step * 1e-3) / 1e9

    out = {
        "metric": "MoE decode layer us/step + tok/s (B=1-64); achieved HBM GB/s vs peak",
        "value": B / (ms_step * 1e-3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "us_per_step": ms_step * 1e3,
        "us_per_step_single_launch": {"median": float(np.median(lat)), "p95": float(np.percentile(lat, 95)),
                                      "min": float(lat.min())},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {synth.F32: "f32", synth.BF16: "bf16", synth.FP8: "fp8e4m3"}[w.expert],
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {WORKLOAD_NOTES[w.name]}", "batch": B, "layers": L,
                   "rotated_instances": C,
                   "path": ("unfused" + ("" if not flags else f", side stream: {args.side}")) if args.unfused
                   else "fused",
                   "kernel_launches_per_step": L * (11 if w.Is > 0 else 8) + (L - 1) * bool(flags & 2)
                   if args.unfused else 1,
                   "distinct_experts_per_layer": round(float(np.mean(distinct)), 1)},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": nbytes, "hbm_bytes_per_launch": hbm_bytes},
        "cpu_baseline": cpu,
        "stream_probe_GBs": {k: round(v, 1) for k, v in probes.items()},
        "stream_probe_shapes": {k: {"workgroups_per_cu": s[0], "loads_per_lane": s[1],
                                    "kb_in_flight_per_cu": s[0] * 256 * s[1] * 16 // 1024}
                                for k, s in PROBE_SHAPES.items()},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
