#!/usr/bin/env python3
"""Benchmark of the MoE decode layer (output-neuron-centric "warp decode"
form) on one MI355X.

One step = one pass of the whole layer (gate/up kernel, then down kernel) over
one decode batch: B tokens of the Qwen-3-style layer (128 experts, top-8,
hidden 2048, intermediate 768) with MXFP8 expert weights, BF16 activations.
The headline line is the B = 1 workload; the same line carries the B = 32
workload under "b32".  All inputs are seeded synthetic data resident in HBM
before timing starts.

Timing hygiene: the layer's weights are replicated into R distinct device
copies and step s runs on copy s % R with its own routing, so consecutive
steps never find their expert rows in the 256 MB last-level cache.

  value            tokens/s: B / the median per-step time over >= 100 replays
                   (and >= 0.2 s) of one HIP graph of >= 200 layer steps (a
                   multiple of --steps, cycling the --steps batches), each
                   replay timed by HIP events
  roofline         the dominant kernel (gate/up): algorithmic bytes per launch
                   (unique routed experts x gate/up codes + E8M0 scales) divided
                   by its mean execution time from HIP events recorded by its
                   own dispatch; under graph_node the same bytes over its time
                   per node in a graph of that kernel alone
  hbm_read_peak    best-of-10 contiguous-read bandwidth of a 16-byte-load
                   kernel over a 4 GiB buffer, measured in the same run
  cpu_baseline     the CPU oracle on this host's cores on a bounded sample
  stack48          a 48-layer decode step (chained layers, per-layer routing
                   from the router kernel) at B in {1, 2, 4, 8, 16, 32, 64}
  large            the 128-expert / top-8 / H 4096 / I 1536 layer with Zipf(1.2)
                   expert popularity at B in {1, 8, 32}
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E, published
GRAPH_MIN_STEPS = 200          # layer steps per timed graph (at least)
MIN_REPLAYS = 100              # timed replays per graph (at least)


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("wd.hip", "wd_device.h", "wd_kernels.h"):
        with open(os.path.join(ROOT, "moe_decode_gate_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from the
    committed rocprofv3 counter summary, if it was taken on the current kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_layer_kernels.txt")
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    for line in lines:
        f = line.split()
        if len(f) >= 2 and f[0] == "traffic" and f[1] == name:
            kv = dict(x.split("=", 1) for x in f[2:])
            if kv.get("kernel_source_digest") == kernel_source_digest():
                return float(kv["hbm_bytes_per_launch"])
    return None


def expert_bytes(spec):
    """Algorithmic bytes one routed expert costs each kernel: its MXFP8 codes
    plus one E8M0 byte per 32 codes (gate/up: 2I rows of H; down: H rows of I)."""
    gate_up = 2 * spec.I * spec.H + 2 * spec.I * (spec.H // 32)
    down = spec.H * spec.I + spec.H * (spec.I // 32)
    return gate_up, down


class Workload:
    """R device copies of one layer plus per-step routing and activations."""

    def __init__(self, torch, wd, gen, L, B, steps, copies, seed, routing="softmax"):
        spec = L.spec
        self.spec, self.B = spec, B
        dev = "cuda"
        base = [torch.from_numpy(a).to(dev) for a in (L.wgu, L.sgu, L.wd, L.sd)]
        self.copies = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
        torch.cuda.synchronize()
        self.steps = steps
        xs, ids, ws = [], [], []
        for s in range(steps):
            t = gen.make_tokens(gen.LayerSpec(E=spec.E, K=spec.K, H=spec.H, I=spec.I, seed=seed), B,
                                routing=routing, step=s)
            xs.append(t.x); ids.append(t.ids); ws.append(t.w)
        self.host_x, self.host_ids, self.host_w = np.stack(xs), np.stack(ids), np.stack(ws)
        self.x = torch.from_numpy(self.host_x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.ids = torch.from_numpy(self.host_ids).to(dev)
        self.w = torch.from_numpy(self.host_w).to(dev)
        self.act = torch.empty((steps, B, spec.K, spec.I), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((steps, B, spec.H), dtype=torch.bfloat16, device=dev)
        # the down kernel's expert-split scratch (zeroed once; every call leaves it zero); the
        # library's default launch configuration decides whether it is used
        self.dscr = wd.down_scratch(B, spec.H)
        self.dn_default = {"down_scratch": self.dscr}
        self.unique = np.array([np.unique(self.host_ids[s]).size for s in range(steps)])
        self.wd = wd
        self.gen = gen

    def step(self, j, which="both", cfg_gu=None, cfg_dn=None, batch=None):
        """Layer step j on weight copy j % R with batch `batch` (default j)."""
        s = j if batch is None else batch
        wgu, sgu, wdn, sdn = self.copies[j % len(self.copies)]
        if which in ("both", "gate_up"):
            self.wd.gate_up(self.x[s], self.ids[s], wgu, sgu, act=self.act[s], cfg=cfg_gu)
        if which in ("both", "down"):
            self.wd.down(self.act[s], self.ids[s], self.w[s], wdn, sdn, out=self.out[s],
                         cfg=self.dn_default if cfg_dn is None else cfg_dn)


def capture(torch, fn):
    """One HIP graph of everything fn() launches (on a side stream, as torch's
    capture requires)."""
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            fn()
    torch.cuda.synchronize()
    return g


def time_replays(torch, wd, g, warm=20, min_replays=None, min_seconds=0.2, max_replays=4000, chunk=50):
    """Replays of one captured graph, each bracketed by HIP events on the stream
    that launches it: `warm` untimed replays, then at least `min_replays` and at
    least `min_seconds` of timed ones.  The replays are queued in chunks behind a
    sleeping wave, so the host is ahead of the GPU and each event pair measures
    the GPU's time for that replay (its nodes and the gaps between them).
    Returns the per-replay durations in microseconds."""
    if min_replays is None:
        min_replays = MIN_REPLAYS
    min_replays = min(min_replays, MIN_REPLAYS)
    if MIN_REPLAYS < 100:                    # a profiling run: no time floor, no long warm-up
        min_seconds, warm = 0.0, min(warm, 2)
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(); g.replay(); e1.record()
    torch.cuda.synchronize()
    est_s = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
    n = int(min(max_replays, max(min_replays, -(-min_seconds // est_s))))
    us = []
    sleep_units = 20000                 # ~70 ms before the first chunk; then twice the measured enqueue time
    while len(us) < n:
        m = min(chunk, n - len(us))
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(m + 1)]
        wd.gpu_sleep(sleep_units)
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(m):
            g.replay()
            evs[i + 1].record()
        host_s = time.perf_counter() - t0
        torch.cuda.synchronize()
        us += [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(m)]
        # one sleep unit is 8192 shader clocks, about 3.4 us
        sleep_units = int(min(40000, 600 + 2 * host_s / 3.4e-6))
    return np.array(us)


def spread(per_step_us):
    q = np.percentile(per_step_us, [0, 10, 50, 90, 100])
    return dict(min=float(q[0]), p10=float(q[1]), median=float(q[2]), p90=float(q[3]), max=float(q[4]))


def measure(torch, wd, work: Workload, steps: int, warmup: int, gu_cfg=None, dn_cfg=None):
    """Step time and per-kernel durations of one workload.

    Headline: G layer steps captured in one HIP graph (G = the smallest
    multiple of `steps` that is at least 200; step j runs batch j % steps on
    weight copy j % R), replayed at least 100 times (and for at least 0.2 s)
    after 20 warm-up replays; each replay is timed by HIP events; the per-step
    time is the median replay time divided by G.  Holding G at 200 or more
    keeps the graph's own start-up (a few microseconds per replay) below 0.1%
    of the replay, so the result does not depend on `steps`.

    Per kernel, two figures: (1) the kernel's execution time, from HIP events
    recorded by its own dispatch (hipExtLaunchKernelGGL) over at least 200
    eager launches queued behind a sleeping wave (mean, after one untimed
    pass); (2) its time per node in a graph of that kernel alone (G launches,
    replayed as above), which adds the dispatch gap between consecutive
    nodes, the regime the headline runs in.  The two graph figures add up to
    the step time."""
    spec = work.spec
    # warmup (eager), also initialises the library's device check outside capture
    for s in range(warmup):
        work.step(s % work.steps, cfg_gu=gu_cfg, cfg_dn=dn_cfg)
    torch.cuda.synchronize()

    G = -(-GRAPH_MIN_STEPS // steps) * steps          # graph steps: a multiple of `steps`, >= 200

    # --- timed region: the layer graph
    g = capture(torch, lambda: [work.step(j, cfg_gu=gu_cfg, cfg_dn=dn_cfg, batch=j % steps) for j in range(G)])
    rep_us = time_replays(torch, wd, g)
    per_step = rep_us / G
    us_per_step = float(np.median(per_step))
    del g

    # --- per-kernel time per node in single-kernel graphs (same replay timing)
    node_us = {}
    for which, cfg in (("gate_up", gu_cfg), ("down", dn_cfg)):
        kw = {"cfg_gu" if which == "gate_up" else "cfg_dn": cfg}
        g = capture(torch, lambda: [work.step(j, which, batch=j % steps, **kw) for j in range(G)])
        node_us[which] = float(np.median(time_replays(torch, wd, g, min_replays=50))) / G
        del g

    # --- per-kernel execution time from HIP events that the kernels' own
    # dispatches record (hipExtLaunchKernelGGL) on the launch stream: one
    # untimed pass over the batches, then G timed launches of each kernel
    for s in range(steps):
        work.step(s, cfg_gu=gu_cfg, cfg_dn=dn_cfg)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(G)]
    for row in evs:
        for e in row:
            e.record()                          # materialise the hipEvent_t
    torch.cuda.synchronize()
    wd.gpu_sleep(20000)                         # ~70 ms: lets the host queue the launches ahead
    for j in range(G):
        work.step(j, "gate_up", batch=j % steps,
                  cfg_gu=dict(start_event=evs[j][0].cuda_event, stop_event=evs[j][1].cuda_event, **(gu_cfg or {})))
        work.step(j, "down", batch=j % steps,
                  cfg_dn=dict(start_event=evs[j][2].cuda_event, stop_event=evs[j][3].cuda_event,
                              **(work.dn_default if dn_cfg is None else dn_cfg)))
    torch.cuda.synchronize()
    gu_ms = np.array([evs[j][0].elapsed_time(evs[j][1]) for j in range(G)])
    dn_ms = np.array([evs[j][2].elapsed_time(evs[j][3]) for j in range(G)])

    u = work.unique[:steps].astype(np.float64)
    per_expert_gu, per_expert_dn = expert_bytes(spec)
    gu_bytes = float(np.mean(u * per_expert_gu))
    dn_bytes = float(np.mean(u * per_expert_dn))
    B = work.B
    res = dict(
        B=B, steps=steps, graph_steps=G, replays=int(rep_us.size), us_per_step=us_per_step,
        ms_per_step=us_per_step * 1e-3,
        tokens_per_s=B / (us_per_step * 1e-6), step_us_spread=spread(per_step),
        unique_experts_mean=float(u.mean()),
        unique_weight_bytes_mean=gu_bytes + dn_bytes,
        layer_GBps_graph=(gu_bytes + dn_bytes) / (us_per_step * 1e-6) / 1e9,
        gate_up_us=float(gu_ms.mean() * 1e3), down_us=float(dn_ms.mean() * 1e3),
        gate_up_graph_node_us=node_us["gate_up"], down_graph_node_us=node_us["down"],
        gate_up_bytes=gu_bytes, down_bytes=dn_bytes,
        gate_up_GBps=gu_bytes / (gu_ms.mean() * 1e-3) / 1e9,
        down_GBps=dn_bytes / (dn_ms.mean() * 1e-3) / 1e9,
        gate_up_graph_node_GBps=gu_bytes / (node_us["gate_up"] * 1e-6) / 1e9,
        down_graph_node_GBps=dn_bytes / (node_us["down"] * 1e-6) / 1e9,
        kernels_GBps=(gu_bytes + dn_bytes) / ((gu_ms.mean() + dn_ms.mean()) * 1e-3) / 1e9,
    )
    return res


def roofline(r, kernel, traffic_name):
    """The roofline object of one kernel: `achieved` from its execution time
    (kernel-own events); the same bytes over its time per graph node (execution
    plus the dispatch gap) under `graph_node`."""
    a = r[f"{kernel}_GBps"]
    gn = r[f"{kernel}_graph_node_GBps"]
    return {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": a / PEAK_HBM_GBPS,
            "traffic": load_traffic(traffic_name), "kernel": kernel,
            "algorithmic_bytes_per_launch": r[f"{kernel}_bytes"], "duration_us": r[f"{kernel}_us"],
            "graph_node": {"achieved": gn, "frac": gn / PEAK_HBM_GBPS, "duration_us": r[f"{kernel}_graph_node_us"]}}


def measure_large(torch, wd, gen, oracle, read_peak, batches=(1, 8, 32), steps=40, warmup=10):
    """The larger layer (128 experts, top-8, H 4096, I 1536) with Zipf(1.2)
    expert popularity at B in {1, 8, 32}: step time from one HIP graph and
    per-kernel durations, as for the headline workload, with four distinct
    weight copies cycled (10 GB; consecutive steps never share a copy, and a
    copy comes back only after three other steps' rows, at least 470 MB, have
    passed through the 256 MB last-level cache), plus sampled parity against
    the oracle."""
    cfg = gen.CONFIGS["large"]
    spec = cfg["spec"]
    t0 = time.time()
    L = gen.make_layer(spec, threads=16)
    eprint(f"[bench] large layer generated in {time.time() - t0:.1f} s")
    out = []
    for B in batches:
        w = Workload(torch, wd, gen, L, B, max(steps, warmup), 4, seed=spec.seed, routing=cfg["routing"])
        r = measure(torch, wd, w, steps, warmup)
        cos, err, ymax = sampled_parity(oracle, L, w, [0, steps - 1])
        r.update(parity_cos_min=cos, parity_max_abs_err=err, parity_max_abs_y=ymax,
                 frac_of_measured_read_peak=r["layer_GBps_graph"] / read_peak,
                 roofline=roofline(r, "gate_up", f"gate_up_large_b{B}"),
                 roofline_down=roofline(r, "down", f"down_large_b{B}"))
        eprint(f"[bench] large B={B}: {json.dumps(r)}")
        out.append(r)
        del w
        torch.cuda.empty_cache()
    return dict(workload="E=128 top-8 H=4096 I=1536, Zipf(1.2) routing", weight_copies=4, per_B=out)


def one_shot_read(torch, wd, nbytes, copies=16, reps=16):
    """The shortest kernel-own time (HIP events from the dispatch) to read nbytes
    once, over one-pass launch shapes of the stream-read kernel (every lane's
    loads issued together, no grid-stride loop), each launch on its own buffer
    copy so that none finds the bytes in the MALL: the floor a kernel that
    streams nbytes in one launch can reach on this GPU."""
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(wd.stream_blocks(), dtype=torch.int32, device="cuda")
    best, best_cfg = float("inf"), None
    for unroll in (1, 2, 4, 8):
        blocks = -(-(nbytes // 16) // (256 * unroll))
        if blocks > wd.stream_blocks():
            continue
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in evs:
            for x in e:
                x.record()
        torch.cuda.synchronize()
        wd.gpu_sleep(20000)
        for r in range(reps):
            wd.stream_read(bufs[r % copies], sink, blocks=blocks, unroll=unroll,
                           start_event=evs[r][0].cuda_event, stop_event=evs[r][1].cuda_event)
        torch.cuda.synchronize()
        us = float(np.median([evs[r][0].elapsed_time(evs[r][1]) for r in range(2, reps)])) * 1e3
        if us < best:
            best, best_cfg = us, (unroll, blocks)
    del bufs
    return best, best_cfg


def unit_shift(m: float) -> int:
    """Integer k with m * 2^k in [0.5, 1) (0 for m = 0)."""
    return 0 if m == 0.0 else -int(np.floor(np.log2(m))) - 1


def measure_stack(torch, wd, gen, L, read_peak, batches=(1, 2, 4, 8, 16, 32, 64), layers=48):
    """A decode step through `layers` MoE layers of the layer's shape: distinct
    device copies of the weights (about 30 GB for 48 layers), per-layer routing
    from the router kernel on per-layer seeded logits, each layer's output
    feeding the next layer's input, all layers captured in one HIP graph per
    batch size and replayed (>= 100 replays, each timed by HIP events).

    Each layer's down-projection E8M0 bytes are shifted by the integer that
    brings that layer's largest |output| into [0.5, 1) on this batch (an exact
    power-of-two rescale, standing in for the normalisation a model applies
    between layers), so every layer carries unit-scale activations; without it
    the chained outputs shrink about quadratically per layer and reach zero
    within a few layers."""
    spec = L.spec
    base = [torch.from_numpy(a).to("cuda") for a in (L.wgu, L.sgu, L.wd, L.sd)]
    copies = [base] + [[t.clone() for t in base] for _ in range(layers - 1)]
    sd0 = base[3].clone()
    per_expert = gen.expert_bytes(spec)
    out = []
    for B in batches:
        ids, ws, uniq = [], [], 0
        for l in range(layers):
            lspec = gen.LayerSpec(E=spec.E, K=spec.K, H=spec.H, I=spec.I, seed=gen.CONFIGS["stack"]["spec"].seed + l)
            logits = torch.from_numpy(gen.make_logits(lspec, B)).to("cuda")
            i, w = wd.route(logits, spec.K)
            ids.append(i); ws.append(w)
        torch.cuda.synchronize()
        for i in ids:
            uniq += int(torch.unique(i).numel())
        x0 = torch.from_numpy(gen.make_tokens(spec, B).x.view(np.int16)).to("cuda").view(torch.bfloat16)
        xs = [x0.clone(), torch.empty_like(x0)]
        act = torch.empty((B, spec.K, spec.I), dtype=torch.bfloat16, device="cuda")
        dcfg = {"down_scratch": wd.down_scratch(B, spec.H)}

        # per-layer unit-scale shifts for this batch (eager, before capture)
        shifts = []
        src, dst = xs
        for l in range(layers):
            c = copies[l]
            c[3].copy_(sd0)
            wd.gate_up(src, ids[l], c[0], c[1], act=act)
            wd.down(act, ids[l], ws[l], c[2], c[3], out=dst, cfg=dcfg)
            k = unit_shift(float(dst.float().abs().max().item()))
            if k:
                c[3].copy_((sd0.to(torch.int16) + k).to(torch.uint8))
                wd.down(act, ids[l], ws[l], c[2], c[3], out=dst, cfg=dcfg)
            shifts.append(k)
            src, dst = dst, src
        last_max = float(src.float().abs().max().item())
        xs[0].copy_(x0)

        def step():
            src, dst = xs
            for l in range(layers):
                c = copies[l]
                wd.gate_up(src, ids[l], c[0], c[1], act=act)
                wd.down(act, ids[l], ws[l], c[2], c[3], out=dst, cfg=dcfg)
                src, dst = dst, src

        step()                                   # eager once (warm-up, device checks)
        torch.cuda.synchronize()
        g = capture(torch, step)
        rep = time_replays(torch, wd, g, min_replays=50)
        us = float(np.median(rep))
        gbps = uniq * per_expert / (us * 1e-6) / 1e9
        out.append(dict(B=B, step_us=us, step_us_spread=spread(rep), replays=int(rep.size),
                        tokens_per_s=B / (us * 1e-6), unique_experts=uniq,
                        GBps=gbps, frac_of_measured_read_peak=gbps / read_peak,
                        down_scale_shifts=shifts, last_layer_max_abs_out=last_max))
        eprint(f"[bench] stack B={B}: {out[-1]}")
        del g
    del copies, base
    torch.cuda.empty_cache()
    best = max(out, key=lambda r: r["GBps"])
    return dict(layers=layers, per_B=out, peak_bandwidth_B=best["B"],
                note="distinct weight copies per layer, per-layer routing, chained activations kept at unit scale "
                     "by per-layer E8M0 shifts of the down projection, one HIP graph")


def measure_comparison(torch, wd, gen, L, batches=(1, 2, 4, 8, 16, 32, 64), steps=20, copies=16):
    """Warp decode against the expert-centric path on the same inputs: for each
    batch size, `steps` layer steps (fresh routing and x per step, weight copies
    cycled so that consecutive steps do not hit the same cached weights)
    captured in one HIP graph per path and replayed (median of >= 30 replays,
    each timed by HIP events); plus the expert-centric stages' own kernel
    durations from HIP events.  Above 64 tokens warp decode runs its defaults
    there (gate/up on the matrix cores, down in the token form)."""
    spec = L.spec
    base = [torch.from_numpy(a).to("cuda") for a in (L.wgu, L.sgu, L.wd, L.sd)]
    cps = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    stage_names = ("align", "gather", "gate_up", "down", "combine")
    out = []
    for B in batches:
        xs, ids, ws = [], [], []
        for s in range(steps):
            t = gen.make_tokens(gen.LayerSpec(E=spec.E, K=spec.K, H=spec.H, I=spec.I, seed=spec.seed + 7), B, step=s)
            xs.append(torch.from_numpy(t.x.view(np.int16)).to("cuda").view(torch.bfloat16))
            ids.append(torch.from_numpy(t.ids).to("cuda")); ws.append(torch.from_numpy(t.w).to("cuda"))
        act = torch.empty((B, spec.K, spec.I), dtype=torch.bfloat16, device="cuda")
        y_wd = torch.empty((steps, B, spec.H), dtype=torch.bfloat16, device="cuda")
        y_ec = torch.empty_like(y_wd)
        wsp = torch.empty(wd.ec_workspace_bytes(B, spec.K, spec.E, spec.H, spec.I), dtype=torch.uint8, device="cuda")

        dcfg = {"down_scratch": wd.down_scratch(B, spec.H)}

        def run_wd(s, stream=None):
            c = cps[s % copies]
            wd.gate_up(xs[s], ids[s], c[0], c[1], act=act, stream=stream)
            wd.down(act, ids[s], ws[s], c[2], c[3], out=y_wd[s], cfg=dcfg, stream=stream)

        def run_ec(s, stream=None, cfg=None):
            c = cps[s % copies]
            wd.ec_moe_decode(xs[s], ids[s], ws[s], c[0], c[1], c[2], c[3], out=y_ec[s], workspace=wsp, cfg=cfg,
                             stream=stream)

        res = dict(B=B)
        for name, fn in (("warp_decode", run_wd), ("expert_centric", run_ec)):
            for s in range(steps):
                fn(s)                                 # eager pass: warm-up and device checks
            torch.cuda.synchronize()
            g = capture(torch, lambda: [fn(s, stream=torch.cuda.current_stream()) for s in range(steps)])
            rep = time_replays(torch, wd, g, min_replays=30, min_seconds=0.1)
            res[f"{name}_us_per_step"] = float(np.median(rep)) / steps
            del g
        # stage kernel durations of the expert-centric path
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(10)] for _ in range(steps)]
        for row in evs:
            for e in row:
                e.record()
        torch.cuda.synchronize()
        wd.gpu_sleep(20000)
        for s in range(steps):
            cfg = wd.ECLaunch()
            for i in range(5):
                cfg.start_event[i] = evs[s][2 * i].cuda_event
                cfg.stop_event[i] = evs[s][2 * i + 1].cuda_event
            run_ec(s, cfg=cfg)
        torch.cuda.synchronize()
        res["expert_centric_stage_us"] = {
            n: float(np.mean([evs[s][2 * i].elapsed_time(evs[s][2 * i + 1]) for s in range(steps)]) * 1e3)
            for i, n in enumerate(stage_names)}
        res["speedup_warp_decode"] = res["expert_centric_us_per_step"] / res["warp_decode_us_per_step"]
        # both paths computed the same layer: their outputs agree to the conventional path's rounding
        a, b = y_wd.float(), y_ec.float()
        res["outputs_cos"] = float((a * b).sum() / (a.norm() * b.norm()))
        eprint(f"[bench] compare B={B}: {json.dumps(res)}")
        out.append(res)
        del xs, ids, ws, act, y_wd, y_ec, wsp
    del cps, base
    torch.cuda.empty_cache()
    faster = [r["B"] for r in out if r["speedup_warp_decode"] < 1.0]
    return dict(per_B=out, steps=steps, weight_copies=copies,
                crossover_B=min(faster) if faster else None,
                largest_B_measured=max(r["B"] for r in out),
                note="both paths graph-replayed on the same inputs; speedup = expert-centric time / warp-decode "
                     "time; crossover_B = smallest measured B where the expert-centric path is faster")


def hbm_read_peak(torch, wd, nbytes=4 << 30, reps=5):
    """Best contiguous-read bandwidth over launch shapes (GB/s), and the copy
    bandwidth of 1 GiB (read + write bytes / time)."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(wd.stream_blocks(), dtype=torch.int32, device="cuda")
    best, best_cfg = 0.0, None
    for unroll in (1, 4, 8):
        for blocks in (1024, 2048, 4096, wd.stream_blocks()):
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                wd.stream_read(buf, sink, blocks=blocks, unroll=unroll)
                e1.record()
                torch.cuda.synchronize()
                bw = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
                if bw > best:
                    best, best_cfg = bw, (unroll, blocks)
    # 1 GiB copy: a kernel of known traffic (1 GiB read + 1 GiB written)
    half = 1 << 30
    src, dst = buf[:half], buf[half:2 * half]
    copy_best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        wd.stream_copy(dst, src)
        e1.record()
        torch.cuda.synchronize()
        copy_best = max(copy_best, 2 * half / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, src, dst
    return best, best_cfg, copy_best


def sampled_parity(oracle, L, work: Workload, steps_to_check):
    """Cosine and max |err| of GPU outputs against the oracle on a few steps,
    and the largest |output| of the oracle there (the scale of that error:
    the BF16 output's half-ulp is 2^-9 of its binade)."""
    cos_min, err_max, ymax = 1.0, 0.0, 0.0
    for s in steps_to_check:
        y64, _ = oracle.moe_decode(work.host_x[s], work.host_ids[s], work.host_w[s],
                                   L.wgu, L.sgu, L.wd, L.sd)
        got = work.out[s].float().cpu().numpy().astype(np.float64)
        cos = float(got.ravel() @ y64.ravel() / (np.linalg.norm(got) * np.linalg.norm(y64)))
        cos_min = min(cos_min, cos)
        err_max = max(err_max, float(np.abs(got - y64).max()))
        ymax = max(ymax, float(np.abs(y64).max()))
    return cos_min, err_max, ymax


def accuracy(oracle, L, work: Workload, steps_to_check):
    """Errors against the FP64 layer with unrounded activations of: the GPU
    warp-decode output; the oracle's conventional-path numerics (x and the
    intermediate rounded through MXFP8, per-expert outputs in BF16); and the
    GPU expert-centric path, which adds its matrix instruction's arithmetic."""
    import torch
    wd = work.wd
    spec = work.spec
    ws = torch.empty(wd.ec_workspace_bytes(work.B, spec.K, spec.E, spec.H, spec.I), dtype=torch.uint8, device="cuda")
    e_wd, e_cv, e_ec, ref_sq, m_wd, m_cv = 0.0, 0.0, 0.0, 0.0, 0.0, 0.0
    for s in steps_to_check:
        args = (work.host_x[s], work.host_ids[s], work.host_w[s], L.wgu, L.sgu, L.wd, L.sd)
        gt = oracle.moe_decode_exact(*args)
        cv = oracle.moe_decode_conventional(*args)
        got = work.out[s].float().cpu().numpy().astype(np.float64)
        c = work.copies[0]
        ec = wd.ec_moe_decode(work.x[s], work.ids[s], work.w[s], c[0], c[1], c[2], c[3], workspace=ws)
        ec = ec.float().cpu().numpy().astype(np.float64)
        e_wd += float(((got - gt) ** 2).sum()); e_cv += float(((cv - gt) ** 2).sum())
        e_ec += float(((ec - gt) ** 2).sum())
        ref_sq += float((gt ** 2).sum())
        m_wd += float(np.abs(got - gt).mean()); m_cv += float(np.abs(cv - gt).mean())
    rel_wd, rel_cv, rel_ec = (e_wd / ref_sq) ** 0.5, (e_cv / ref_sq) ** 0.5, (e_ec / ref_sq) ** 0.5
    # against the layer with the weights as drawn, before MXFP8 quantization (the
    # checked steps' tokens in one batch: every token's result is its own)
    xs = np.concatenate([work.host_x[s] for s in steps_to_check])
    ids = np.concatenate([work.host_ids[s] for s in steps_to_check])
    wts = np.concatenate([work.host_w[s] for s in steps_to_check])
    drawn = {}

    def weights(e, part):
        if e not in drawn:
            drawn.clear()
            drawn[e] = work.gen.expert_weights_fp32(spec, e)
        return drawn[e][part]

    full = oracle.moe_decode_dense_weights(xs, ids, wts, lambda e: weights(e, 0), lambda e: weights(e, 1))
    outs = {"warp_decode_gpu": np.concatenate([work.out[s].float().cpu().numpy() for s in steps_to_check]),
            "conventional": np.concatenate([oracle.moe_decode_conventional(
                work.host_x[s], work.host_ids[s], work.host_w[s], L.wgu, L.sgu, L.wd, L.sd)
                for s in steps_to_check]),
            "mxfp8_exact": np.concatenate([oracle.moe_decode_exact(
                work.host_x[s], work.host_ids[s], work.host_w[s], L.wgu, L.sgu, L.wd, L.sd)
                for s in steps_to_check])}
    fsq = float((full ** 2).sum())
    vs_full = {k: (float(((v.astype(np.float64) - full) ** 2).sum()) / fsq) ** 0.5 for k, v in outs.items()}
    return dict(rel_l2_warp_decode_gpu=rel_wd, rel_l2_conventional=rel_cv, rel_l2_ratio=rel_cv / rel_wd,
                rel_l2_expert_centric_gpu=rel_ec, rel_l2_ratio_gpu_paths=rel_ec / rel_wd,
                mean_abs_ratio=m_cv / m_wd, steps=len(steps_to_check),
                reference="FP64 layer, exact MXFP8 weights, unrounded intermediate and output",
                vs_unquantized_weights=dict(
                    {f"rel_l2_{k}": v for k, v in vs_full.items()},
                    rel_l2_ratio=vs_full["conventional"] / vs_full["warp_decode_gpu"],
                    reference="FP64 layer with the FP32 weights as drawn before MXFP8 quantization"))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo) and its logical CPU count."""
    name = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"{name} ({os.cpu_count()} logical CPUs visible)"


def cpu_baseline(oracle, L, gen, B, seconds=12.0, single_seconds=4.0):
    """The oracle as it stands, on every host core, over fresh seeded batches
    of the same workload until about `seconds` of CPU work have run; and the
    same on one thread for about `single_seconds`."""
    spec = L.spec

    def run(nthreads, budget, first_step):
        n_tok, t_used, s = 0, 0.0, 0
        while t_used < budget:
            t = gen.make_tokens(spec, B, step=first_step + s)
            t0 = time.perf_counter()
            oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd, nthreads=nthreads)
            t_used += time.perf_counter() - t0
            n_tok += B
            s += 1
        return n_tok, t_used, s

    cores = oracle.max_threads()            # the oracle's thread count persists per call: set it each time
    n1, t1, _ = run(1, single_seconds, 20_000)
    n_tok, t_used, s = run(cores, seconds, 10_000)
    from oracle import build as ob
    return dict(value=n_tok / t_used, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{n_tok} tokens in {s} batches of B={B} on the same layer, {t_used:.1f} s",
                cpu_model=cpu_model(), compiler_flags=" ".join(ob.CFLAGS),
                single_thread=dict(value=n1 / t1, unit="tokens/s", cores=1,
                                   sample=f"{n1} tokens in batches of B={B}, {t1:.1f} s"))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=0, help="distinct weight copies (0 = auto)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-b32", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-large", action="store_true", help="skip the H 4096 / I 1536 layer")
    ap.add_argument("--no-compare", action="store_true", help="skip the expert-centric comparison")
    ap.add_argument("--only-compare", action="store_true",
                    help="run only the expert-centric comparison and print its JSON object (for profiling)")
    ap.add_argument("--replays", type=int, default=100,
                    help="minimum timed replays of each graph (fewer only for profiling runs)")
    ap.add_argument("--graph-min-steps", type=int, default=200,
                    help="layer steps per timed graph, at least (fewer only for profiling runs)")
    ap.add_argument("--compare-batches", default="1,2,4,8,16,32,64,96,128,192,256,384,512",
                    help="batch sizes of the comparison")
    args = ap.parse_args()
    global GRAPH_MIN_STEPS, MIN_REPLAYS
    GRAPH_MIN_STEPS, MIN_REPLAYS = args.graph_min_steps, args.replays
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer runs on a single "
              "MI355X; there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from moe_decode_gate_amd import binding as wd
    from moe_decode_gate_amd import inputs as gen
    torch.cuda.set_device(0)

    spec = gen.CONFIGS["qwen3"]["spec"]
    t0 = time.time()
    L = gen.make_layer(spec, threads=16)
    eprint(f"[bench] layer generated in {time.time() - t0:.1f} s")
    compare_batches = tuple(int(b) for b in args.compare_batches.split(","))
    if args.only_compare:
        print(json.dumps({"vs_expert_centric": measure_comparison(torch, wd, gen, L, compare_batches)}), flush=True)
        return

    peak, peak_cfg, copy_bw = hbm_read_peak(torch, wd)
    eprint(f"[bench] contiguous-read peak {peak:.0f} GB/s (unroll, blocks = {peak_cfg}); copy {copy_bw:.0f} GB/s")
    gu_b1_bytes, dn_b1_bytes = (8 * n for n in expert_bytes(spec))   # each kernel's bytes of 8 experts
    floor_us, floor_cfg = one_shot_read(torch, wd, gu_b1_bytes)
    floor_dn_us, floor_dn_cfg = one_shot_read(torch, wd, dn_b1_bytes)
    eprint(f"[bench] one-shot read of {gu_b1_bytes} B: {floor_us:.2f} us (unroll, blocks = {floor_cfg}); "
           f"of {dn_b1_bytes} B: {floor_dn_us:.2f} us ({floor_dn_cfg})")

    steps, warmup = args.steps, args.warmup
    copies1 = args.copies or 16
    w1 = Workload(torch, wd, gen, L, 1, max(steps, warmup), copies1, seed=spec.seed)
    r1 = measure(torch, wd, w1, steps, warmup)
    eprint(f"[bench] B=1: {json.dumps(r1)}")
    import oracle
    cos1, err1, ymax1 = sampled_parity(oracle, L, w1, [0, steps // 2, steps - 1])
    r1.update(parity_cos_min=cos1, parity_max_abs_err=err1, parity_max_abs_y=ymax1,
              gate_up_over_one_shot_read=r1["gate_up_us"] / floor_us,
              down_over_one_shot_read=r1["down_us"] / floor_dn_us,
              roofline_down=roofline(r1, "down", "down_qwen3_b1"))
    del w1
    torch.cuda.empty_cache()

    r32 = None
    if not args.no_b32:
        w32 = Workload(torch, wd, gen, L, 32, max(steps, warmup), args.copies or 4, seed=gen.CONFIGS["qwen3_b32"]["spec"].seed)
        r32 = measure(torch, wd, w32, steps, warmup)
        cos32, err32, ymax32 = sampled_parity(oracle, L, w32, [0, steps - 1])
        r32.update(parity_cos_min=cos32, parity_max_abs_err=err32, parity_max_abs_y=ymax32,
                   frac_of_measured_read_peak=r32["layer_GBps_graph"] / peak,
                   accuracy=accuracy(oracle, L, w32, [0, steps - 1]),
                   roofline=roofline(r32, "gate_up", "gate_up_qwen3_b32"),
                   roofline_down=roofline(r32, "down", "down_qwen3_b32"))
        eprint(f"[bench] B=32: {json.dumps(r32)}")
        # the same workload with both kernels in their token forms (one wave per (token, slot,
        # rows) for gate/up, one per (token, outputs) for down: no matrix cores, no LDS)
        tf = measure(torch, wd, w32, steps, warmup, gu_cfg=dict(form=1), dn_cfg=dict(form=1))
        cos_t, err_t, ymax_t = sampled_parity(oracle, L, w32, [0, steps - 1])
        tf.update(parity_cos_min=cos_t, parity_max_abs_err=err_t, parity_max_abs_y=ymax_t,
                  frac_of_measured_read_peak=tf["layer_GBps_graph"] / peak,
                  roofline=roofline(tf, "gate_up", "gate_up_token_form_qwen3_b32"),
                  launch={"gate_up": {"form": 1}, "down": {"form": 1}})
        r32["token_form"] = tf
        eprint(f"[bench] B=32 token form: {json.dumps(tf)}")
        del w32
        torch.cuda.empty_cache()

    stack = None if args.no_stack else measure_stack(torch, wd, gen, L, peak)

    large = None if args.no_large else measure_large(torch, wd, gen, oracle, peak)

    compare = None if args.no_compare else measure_comparison(torch, wd, gen, L, compare_batches)

    cpu = None if args.no_cpu else cpu_baseline(oracle, L, gen, 1)

    line = {
        "metric": "MoE-layer decode tokens/s and achieved HBM TB/s (% of 8 TB/s) at B=1 and 32",
        "value": r1["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": r1["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp8-e4m3/bf16/fp32",
        "data": "synthetic: seeded N(0,0.02) weights quantized to MXFP8, N(0,1) bf16 x, softmax top-8 routing",
        "config": {"workload": "Qwen-3-style MoE decode layer E=128 top-8 H=2048 I=768, B=1",
                   "global_batch": 1, "parallelism": "single GPU", "weight_copies": copies1},
        "roofline": roofline(r1, "gate_up", "gate_up_qwen3_b1"),
        "timing": "value = B / median per-step time over >= 100 replays (and >= 0.2 s) of one HIP graph of "
                  "`steps` layer steps, each replay timed by HIP events; roofline.achieved = the kernel's "
                  "algorithmic bytes / its mean execution time from HIP events recorded by its own dispatch; "
                  "roofline.graph_node = the same bytes / its time per node in a graph of that kernel alone "
                  "(execution plus the dispatch gap between nodes)",
        "hbm_read_peak_GBps": peak,
        "one_shot_read": {"gate_up_bytes": gu_b1_bytes, "gate_up_us": floor_us,
                          "gate_up_GBps": gu_b1_bytes / (floor_us * 1e-6) / 1e9, "gate_up_unroll_blocks": floor_cfg,
                          "down_bytes": dn_b1_bytes, "down_us": floor_dn_us,
                          "down_GBps": dn_b1_bytes / (floor_dn_us * 1e-6) / 1e9, "down_unroll_blocks": floor_dn_cfg,
                          "note": "a plain read of the B=1 kernels' bytes in one launch (kernel-own events, "
                                  "distinct buffers): the floor for a one-launch stream of that size"},
        "hbm_copy_GBps": copy_bw,
        "layer_GBps": r1["layer_GBps_graph"],
        "frac_of_8TBps": r1["layer_GBps_graph"] / PEAK_HBM_GBPS,
        "frac_of_measured_read_peak": r1["layer_GBps_graph"] / peak,
        "b1": r1,
        "b32": r32,
        "stack48": stack,
        "large": large,
        "vs_expert_centric": compare,
        "cpu_baseline": cpu,
        "kernel_source_digest": kernel_source_digest(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
