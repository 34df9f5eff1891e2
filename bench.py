"""Benchmark: SeKV mixed-resolution decode attention on one MI355X.

Workload (default): 32 layers x 32 heads, d=128, n=131072 tokens, bf16 K/V,
batch 1, synthetic inputs (seeded surprisal with spikes, planted low-rank span
structure, per-(layer, head) zoom rates 0.5-20%, retrieval-head needles).
Every layer is built on the GPU (segmentation, summaries, anchors, truncated
SVD of every span into a device-resident basis store), then decode steps are
timed: one step = one decode-attention pass over all 32 layers.

Reported metric: key positions per second per layer-step (B*n / t_layer_step),
plus achieved HBM bandwidth of one layer-step (the planned decode kernel, which
does the work, and the small combine kernel) from the algorithmic bytes of each
layer-step (anchors, summaries, zoomed spans' bases, q/out/mask), timed with
HIP events around a graph replay of every step.

Secondary measures in the same JSON line (skip with --no-secondary): the same
workload with the bases in pinned host memory (read in place, through the
device basis cache, and the staged copy of the zoomed spans), the GQA batch-8
workload at 1/5/15/30% zoom, the 32K single layer, and the prefill builder on
its stress workload.  The CPU baseline is the oracle on the host's cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --home host ...          # headline with bases in pinned host memory, read in place
    python bench.py --copy-calibration ...   # also runs a 1 GiB device copy (counter scaling)
    python bench.py --traffic-from FETCH_DIR WRITE_DIR   # rocprofv3 --pmc runs -> profiles/decode_traffic.json
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "decode-attn key-positions/s per layer-step at 128K ctx; achieved HBM GB/s %peak"
# the oracle's process pool: at most the host's cores, and no more than one GPU's share of them
CPU_POOL_MAX = 16


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=128)
    p.add_argument("--warmup", type=int, default=4)
    p.add_argument("--config", default="layers32_128k")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the workload's)")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true", help="headline only")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="timed window of the oracle pool")
    p.add_argument("--calib-steps", type=int, default=8)
    p.add_argument("--home", choices=("device", "host", "host_staged"), default="device")
    p.add_argument("--cache-gb", type=float, default=0.0,
                   help="device cache of host-resident bases (--home host), GiB over all layers")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "sekv_device.h", "sekv_internal.h"):
        with open(os.path.join(ROOT, "hierarchical_kv_cache_surprisal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic of the decode kernels measured with rocprofv3 counters, if the
    stored figure was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(workload)
    if not e or e.get("kernel_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


COPY_BYTES = 1 << 30


def decode_kernel(name: str):
    """The decode kernels of a device-resident layer-step: the planned decode
    kernel and the combine kernel."""
    if "k_planned<" in name:
        return "k_planned"
    if "k_combine<" in name:
        return "k_combine"
    return None


def _pmc_rows(d, counter):
    """(kernel name, counter value) per dispatch from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def traffic_from(fetch_dir, write_dir):
    """HBM bytes per layer-step of the decode kernels from two rocprofv3 --pmc
    runs of `bench.py --no-graph --copy-calibration` (FETCH_SIZE, then
    WRITE_SIZE, in KiB per dispatch), each scaled by what the same counter reads
    for the 1 GiB device copy (read once, written once).  Writes
    profiles/decode_traffic.json keyed by workload, with the kernel-source hash."""
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        copy = [v for k, v in rows if "elementwise" in k.lower()]
        if not copy:
            raise SystemExit(f"no copy-kernel dispatch with {counter} in {d}")
        kib_copy = max(copy)  # the 1 GiB copy is the largest copy dispatch
        scale = COPY_BYTES / (kib_copy * 1024.0)
        per = {}
        for k, v in rows:
            name = decode_kernel(k)
            if name:
                per.setdefault(name, []).append(v * 1024.0 * scale)
        res[counter] = {"scale": scale, "copy_kib": kib_copy,
                        "kernels": {n: {"dispatches": len(v), "bytes_mean": sum(v) / len(v)} for n, v in per.items()}}
    fetch = sum(e["bytes_mean"] for e in res["FETCH_SIZE"]["kernels"].values())
    write = sum(e["bytes_mean"] for e in res["WRITE_SIZE"]["kernels"].values())
    out = {"kernel_hash": kernel_source_hash(), "bytes_per_launch": fetch + write,
           "fetch_bytes": fetch, "write_bytes": write, "detail": res,
           "note": "one launch = one layer-step (k_planned + k_combine): mean over dispatches"}
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    try:
        with open(path) as f:
            allw = json.load(f)
    except (OSError, ValueError):
        allw = {}
    allw["layers32_128k"] = out
    with open(path, "w") as f:
        json.dump(allw, f, indent=1)
    print(json.dumps(out, indent=1))


# ============================================================================ decode runs

class DecodeRun:
    """One workload on one context: build every layer, calibrate per-head
    thresholds at the target zoom rates from the GPU's routing scores, count
    the algorithmic bytes of a layer-step, and time decode steps."""

    def __init__(self, s, home, dev, stream, log_build=True):
        import torch

        import synth
        from hierarchical_kv_cache_surprisal_amd import sekv
        self.s, self.home, self.dev, self.stream = s, home, dev, stream
        self.ctx = sekv.Context(s.L, s.B, s.n, s.Hq, s.Hkv, s.d, s.kv_dtype, s.w, home)
        self.H = torch.from_numpy(synth.surprisal_batch(s)).to(dev)
        self.t_gen = self.t_build = 0.0
        for l in range(s.L):
            t0 = time.perf_counter()
            K, V = synth.kv_layer(s, l, device=dev)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            self.ctx.build(l, self.H, K, V, s.alpha, s.rank_choices, s.rank_seed)
            torch.cuda.synchronize()
            t2 = time.perf_counter()
            self.t_gen += t1 - t0
            self.t_build += t2 - t1
            del K, V
            if log_build and (l == 0 or (l + 1) % 8 == 0):
                log(f"{s.name} [{home}]: built layer {l + 1}/{s.L} (gen {t1 - t0:.2f}s build {t2 - t1:.2f}s)")
        torch.cuda.empty_cache()
        self.spans = [self.ctx.spans(b) for b in range(s.B)]
        self.m_max = self.spans[0][3]
        self.m_tot = sum(len(sp[0]) for sp in self.spans)
        self.n_a = sum(len(sp[2]) for sp in self.spans)
        self.out = torch.empty(s.B, s.Hq, s.d, device=dev)
        self.mask = torch.zeros(s.L, s.B, s.Hq, self.m_max, dtype=torch.uint8, device=dev)
        self.qs = None
        self.taus = None

    def close(self):
        import torch
        self.ctx.close()
        self.qs = self.mask = self.out = None
        torch.cuda.empty_cache()

    def make_queries(self, steps):
        import torch

        import synth
        s = self.s
        self.qs = torch.stack([torch.stack([synth.queries(s, l, t, device=self.dev) for t in range(steps)])
                               for l in range(s.L)])  # [L][steps][B][Hq][d]

    def calibrate(self, rates_of_layer, calib_steps):
        """tau per (layer, query head) at the quantile of the GPU's routing scores
        (calibration queries, not the timed ones) that gives the target zoom rate."""
        import numpy as np
        import torch

        import synth
        s = self.s
        scores = torch.empty(s.B, s.Hq, self.m_max, device=self.dev)
        taus = np.zeros((s.L, s.Hq), np.float32)
        for l in range(s.L):
            rates = rates_of_layer(l)
            pooled = [[] for _ in range(s.Hq)]
            for t in range(calib_steps):
                q = synth.queries(s, l, 10_000 + t, device=self.dev)
                self.ctx.route_scores(l, q, scores)
                for b in range(s.B):
                    m_b = len(self.spans[b][0])
                    for h in range(s.Hq):
                        pooled[h].append(scores[b, h, :m_b].clone())
            for h in range(s.Hq):
                allsc = torch.cat(pooled[h]).double()
                th = float(torch.quantile(allsc, 1.0 - float(rates[h])))
                taus[l, h] = np.float32(1.0 / (1.0 + math.exp(-th)))
        self.taus = taus

    def step(self, t, stream=None, noalloc=False):
        st = stream if stream is not None else self.stream
        for l in range(self.s.L):
            self.ctx.decode_attn(l, self.qs[l, t], self.taus[l], self.out, self.mask[l], st, noalloc=noalloc)

    def algorithmic_bytes(self, steps):
        """Bytes a layer-step must move at the least, averaged over sampled steps:
        anchors K and V, every span's kbar, vbar of the spans no head of the group
        zoomed, the bases of the spans some head zoomed, ln|S|, q, out, tau and the
        mask.  Also returns the mean zoom rate and the zoomed bases' bytes alone."""
        import numpy as np
        import torch
        s, dev = self.s, self.dev
        L, B, Hkv, d, m_max = s.L, s.B, s.Hkv, s.d, self.m_max
        esz = 2 if s.kv_dtype == "bf16" else 4
        rank_t = torch.zeros(L, B, Hkv, m_max, dtype=torch.float64, device=dev)
        cnt_t = torch.zeros(B, m_max, dtype=torch.float64, device=dev)
        valid = torch.zeros(B, m_max, dtype=torch.bool, device=dev)
        for b in range(B):
            mcb = self.spans[b][1]
            cnt_t[b, :len(mcb)] = torch.from_numpy(mcb.astype(np.float64)).to(dev)
            valid[b, :len(mcb)] = True
            for l in range(L):
                for g in range(Hkv):
                    rk, _, _ = self.ctx.bases_layout(l, b, g)
                    rank_t[l, b, g, :len(rk)] = torch.from_numpy(rk.astype(np.float64)).to(dev)
        fixed = (Hkv * self.n_a * 2 * d * esz        # anchors K and V
                 + Hkv * self.m_tot * d * esz        # kbar
                 + Hkv * self.m_tot * 4              # ln|S|
                 + B * s.Hq * d * 8 + s.Hq * 4       # q in, out, tau
                 + s.Hq * self.m_tot)                # mask
        sample = list(range(0, steps, max(1, steps // 8)))
        zoom_rates = []
        per_layer = np.zeros(L)
        basis_layer = np.zeros(L)
        for t in sample:
            self.step(t)
            torch.cuda.synchronize()
            mv = self.mask.view(L, B, Hkv, s.G, m_max)
            z = mv.amax(dim=3).to(torch.bool) & valid[None, :, None, :]
            zall = mv.amin(dim=3).to(torch.bool) & valid[None, :, None, :]
            basis = (2.0 * (cnt_t[None, :, None, :] + d) * rank_t * esz * z).sum(dim=(1, 2, 3))
            vbar = (Hkv * self.m_tot - zall.sum(dim=(1, 2, 3)).double()) * d * esz
            per_layer += (basis + vbar).cpu().numpy() + fixed
            basis_layer += basis.cpu().numpy()
            zoom_rates.append(float(self.mask.float().sum() / (L * s.Hq * self.m_tot)))
        per_layer /= len(sample)
        basis_layer /= len(sample)
        return per_layer, float(np.mean(zoom_rates)), float(basis_layer.mean())

    def capture(self, steps, noalloc=False):
        """One HIP graph of `steps` decode steps (every layer), captured on a side
        stream after eager warm-up calls have sized the work schedules."""
        import torch
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(self.stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for t in range(steps):
                    self.step(t, cap, noalloc=noalloc)
        self.stream.wait_stream(cap)
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        return g

    def time_steps(self, steps, graph):
        """ms for `steps` decode steps (graph replay, or eager launches), with HIP
        events on the stream the kernels run on."""
        import torch
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        # eager launches allocate small Python objects on every call: keep the
        # collector out of the timed region
        gc.collect()
        gc.disable()
        torch.cuda.synchronize()
        ev0.record(self.stream)
        if graph is not None:
            graph.replay()
        else:
            for t in range(steps):
                self.step(t)
        ev1.record(self.stream)
        torch.cuda.synchronize()
        gc.enable()
        return ev0.elapsed_time(ev1)


def _layer_step_entry(s, t_ms, launches, bytes_ls, zoom):
    t_ls = t_ms * 1e-3 / launches
    gbs = bytes_ls / t_ls / 1e9
    return {"t_layer_step_us": t_ls * 1e6, "key_positions_per_s": s.B * s.n / t_ls,
            "algorithmic_bytes_per_layer_step": bytes_ls, "GB/s": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
            "mean_zoom_rate": zoom}


# ============================================================================ main

def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              f"(the decode path runs on one GPU; multi-GPU execution is not implemented).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from hierarchical_kv_cache_surprisal_amd import sekv

    sekv.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    s = synth.spec(args.config)
    if args.layers:
        s = s.replace(L=args.layers)
    L, B, n, Hq, Hkv, d = s.L, s.B, s.n, s.Hq, s.Hkv, s.d
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------------ headline workload
    run = DecodeRun(s, args.home, dev, stream)
    st = run.ctx.stats()
    log(f"spans m={run.m_tot} anchors={run.n_a}; device-resident {st['device_resident_bytes']/1e9:.2f} GB "
        f"vs full KV {st['full_kv_bytes']/1e9:.1f} GB")
    run.make_queries(args.steps)
    run.calibrate(lambda l: synth.zoom_targets(s, l), args.calib_steps)
    log("thresholds calibrated")
    if args.cache_gb > 0:
        run.ctx.set_basis_cache(int(args.cache_gb * (1 << 30)))
        log(f"device basis cache: {args.cache_gb} GiB over {L} layers (eager launches: the cache plans on the host)")
    for t in range(args.warmup):
        run.step(t % args.steps)
    torch.cuda.synchronize()
    per_layer, zoom_rate, _ = run.algorithmic_bytes(args.steps)
    bytes_per_ls = float(per_layer.mean())
    log(f"algorithmic bytes per layer-step {bytes_per_ls/1e6:.2f} MB (min {per_layer.min()/1e6:.1f}, "
        f"max {per_layer.max()/1e6:.1f}); mean zoom rate {zoom_rate:.4f}")
    graph = None
    # staged bases sync each call, the basis cache plans on the host: no graph for either
    if not args.no_graph and args.home != "host_staged" and args.cache_gb <= 0:
        graph = run.capture(args.steps)
    w0 = time.perf_counter()
    t_ms = run.time_steps(args.steps, graph)
    wall = time.perf_counter() - w0
    graph = None
    launches = args.steps * L
    t_ls = t_ms * 1e-3 / launches
    kps = B * n / t_ls
    gbs = bytes_per_ls / t_ls / 1e9
    log(f"timed {args.steps} steps x {L} layers: {t_ms:.3f} ms (wall {wall*1e3:.1f} ms), "
        f"t_layer_step {t_ls*1e6:.2f} us, {kps:.3e} KP/s, {gbs:.0f} GB/s = {100*gbs/PEAK_HBM_GBS:.1f}% of peak")
    st2 = run.ctx.stats()
    taus_head = run.taus.copy()
    build_head = {"layers": L, "seconds": run.t_build, "tokens_per_s": L * B * n / run.t_build,
                  "kv_head_rows_per_s": L * B * Hkv * n / run.t_build, "gen_seconds": run.t_gen}
    memory = {"device_resident_bytes": st["device_resident_bytes"], "full_kv_bytes": st["full_kv_bytes"]}
    cache_stats = ({k: st2[k] for k in ("cache_zoomed", "cache_hits", "cache_spans_fetched", "cache_bytes_fetched")}
                   if args.cache_gb > 0 else None)
    m_tot, n_a = run.m_tot, run.n_a

    if args.copy_calibration:
        # a device copy of known size, for scaling the HBM byte counters
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # an elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 x {COPY_BYTES >> 20} MiB device copy")
    run.close()
    del run

    read_ref = read_reference(dev, stream, [int(bytes_per_ls), 1 << 30])

    # ------------------------------------------------------------------ secondary workloads
    secondary = None
    if not args.no_secondary and args.config == "layers32_128k" and not args.layers and args.home == "device":
        secondary = {}
        for name, fn in (("host_home", lambda: host_home_runs(s, dev, stream, args)),
                         ("gqa_zoom_sweep", lambda: gqa_sweep(dev, stream, args)),
                         ("single_layer_32k", lambda: single_layer(dev, stream, args)),
                         ("builder_prefill_128k", lambda: builder_runs(dev, stream))):
            t0 = time.perf_counter()
            secondary[name] = fn()
            log(f"secondary {name}: {time.perf_counter() - t0:.1f}s")

    # ------------------------------------------------------------------ CPU baseline (the oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(s, taus_head, args.cpu_seconds)

    traffic = load_traffic(s.name)
    res = {
        "metric": METRIC,
        "value": kps,
        "unit": "key-positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.kv_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{s.name}: {L} layers x {Hq} q-heads / {Hkv} kv-heads, d={d}, n={n}, "
                               f"{s.kv_dtype} KV, batch {B}, {args.steps} decode steps, zoom 0.5-20% per head, "
                               f"bases {args.home}-resident"
                               + (" (the workload's host-pinned home is under secondary.host_home)"
                                  if args.home == "device" else ""),
                   "layers": L, "q_heads": Hq, "kv_heads": Hkv, "d_head": d, "ctx": n, "batch": B,
                   "spans": m_tot, "anchors": n_a, "graph": not args.no_graph and args.home != "host_staged"
                   and args.cache_gb <= 0, "bases": args.home,
                   **({"basis_cache_gib": args.cache_gb} if args.cache_gb > 0 else {})},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS,
                     "traffic": traffic if args.home == "device" else None,
                     "kernel": "one layer-step: k_planned (the work) + k_combine, HIP events around the "
                               "graph replay of every timed step"},
        "cpu_baseline": cpu,
        "read_reference": read_ref,
        "t_layer_step_us": t_ls * 1e6,
        "algorithmic_bytes_per_layer_step": bytes_per_ls,
        "head_positions_per_s": B * Hq * n / t_ls,
        "mean_zoom_rate": zoom_rate,
        "builder": build_head,
        "memory": memory,
        **({"basis_cache": cache_stats} if cache_stats else {}),
        **({"secondary": secondary} if secondary is not None else {}),
    }
    print(json.dumps(res), flush=True)


# ============================================================================ secondary workloads

def pinned_copy_rate(dev, stream, nbytes=256 << 20, reps=10):
    """Host-to-device copy rate of a pinned buffer (the link's measured rate)."""
    import torch
    h = torch.ones(nbytes // 4, dtype=torch.float32).pin_memory()
    dv = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    with torch.cuda.stream(stream):
        dv.copy_(h, non_blocking=True)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            dv.copy_(h, non_blocking=True)
        e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    return nbytes / t / 1e9


def host_home_runs(s, dev, stream, args, steps=32, staged_layers=4, staged_steps=4):
    """The headline workload with the bases in pinned host memory (its stated
    home): through a 4 GiB device basis cache with prefetch (eager launches),
    then read in place by the decode kernel (graph replay), then the staged
    copy of each step's zoomed spans on a 4-layer slice.  Times include the
    transfers; link GB/s counts the basis bytes that cross the link."""
    import torch

    import synth
    out = {"pinned_h2d_GBs": pinned_copy_rate(dev, stream)}
    run = DecodeRun(s, "host", dev, stream, log_build=False)
    run.make_queries(steps)
    run.calibrate(lambda l: synth.zoom_targets(s, l), args.calib_steps)
    # the device basis cache: 4 GiB over the layers, eager launches; the cache
    # fills over the first calls of each layer
    run.ctx.set_basis_cache(4 << 30)
    for t in range(max(8, args.warmup)):
        run.step(t % steps)
    per_layer, zoom, basis = run.algorithmic_bytes(steps)
    torch.cuda.synchronize()
    c0 = run.ctx.stats()
    t_ms = run.time_steps(steps, None)
    c1 = run.ctx.stats()
    e = _layer_step_entry(s, t_ms, steps * s.L, float(per_layer.mean()), zoom)
    z = c1["cache_zoomed"] - c0["cache_zoomed"]
    hits = c1["cache_hits"] - c0["cache_hits"]
    pref = (c1["cache_bytes_fetched"] - c0["cache_bytes_fetched"]) / (steps * s.L)
    miss = basis * (1.0 - hits / z) if z else 0.0
    e.update({"cache_gib": 4, "cache_hit_rate": hits / z if z else None,
              "prefetch_bytes_per_layer_step": pref, "miss_bytes_per_layer_step_est": miss,
              "link_GB/s": (pref + miss) / (e["t_layer_step_us"] * 1e-6) / 1e9,
              "mode": "device basis cache with prefetch on a side stream, eager launches"})
    out["cache"] = e
    log(f"host home + cache: {e['t_layer_step_us']:.1f} us per layer-step, hit rate {e['cache_hit_rate']}")
    # in place: no cache, every zoomed span read over the link by the decode kernel
    run.ctx.set_basis_cache(0)
    for t in range(args.warmup):
        run.step(t % steps)
    g = run.capture(steps)
    t_ms = run.time_steps(steps, g)
    g = None
    e = _layer_step_entry(s, t_ms, steps * s.L, float(per_layer.mean()), zoom)
    e["link_bytes_per_layer_step"] = basis
    e["link_GB/s"] = basis / (e["t_layer_step_us"] * 1e-6) / 1e9
    e["mode"] = "bases read in place from pinned host memory, graph replay"
    out["in_place"] = e
    log(f"host home in place: {e['t_layer_step_us']:.1f} us per layer-step, link {e['link_GB/s']:.1f} GB/s")
    run.close()
    # the pages' literal path: zoomed spans copied to device staging every step
    s4 = s.replace(L=staged_layers)
    run = DecodeRun(s4, "host_staged", dev, stream, log_build=False)
    run.make_queries(staged_steps)
    run.calibrate(lambda l: synth.zoom_targets(s, l), args.calib_steps)
    run.step(0)
    per_layer, zoom, basis = run.algorithmic_bytes(staged_steps)
    c0 = run.ctx.stats()
    t_ms = run.time_steps(staged_steps, None)
    c1 = run.ctx.stats()
    e = _layer_step_entry(s4, t_ms, staged_steps * s4.L, float(per_layer.mean()), zoom)
    fb = (c1["bytes_fetched"] - c0["bytes_fetched"]) / (staged_steps * s4.L)
    e.update({"layers": staged_layers, "fetched_bytes_per_layer_step": fb,
              "copy_launches_per_layer_step": (c1["memcpy_calls"] - c0["memcpy_calls"]) / (staged_steps * s4.L),
              "link_GB/s": fb / (e["t_layer_step_us"] * 1e-6) / 1e9,
              "mode": "route, host sync, one copy kernel of the zoomed spans to staging, attend (eager)"})
    out["staged"] = e
    log(f"host staged: {e['t_layer_step_us']:.1f} us per layer-step")
    run.close()
    return out


def gqa_sweep(dev, stream, args, steps=16, rates=(0.01, 0.05, 0.15, 0.30)):
    """GQA batch-8 workload (groups of four query heads, ranks 8..64) at each
    zoom rate: thresholds re-calibrated per rate, graph replay."""
    import synth
    s = synth.spec("gqa_batch8_128k")
    run = DecodeRun(s, "device", dev, stream, log_build=False)
    run.make_queries(steps)
    out = {}
    for r in rates:
        run.calibrate(lambda l: [r] * s.Hq, args.calib_steps)
        for t in range(6):  # the work schedule follows the new zoom rates
            run.step(t % steps)
        per_layer, zoom, _ = run.algorithmic_bytes(steps)
        for t in range(4):
            run.step(t % steps)
        g = run.capture(steps)
        t_ms = run.time_steps(steps, g)
        g = None
        out[f"{int(round(r * 100))}%"] = _layer_step_entry(s, t_ms, steps * s.L, float(per_layer.mean()), zoom)
        log(f"gqa {r:.2f}: {out[f'{int(round(r * 100))}%']['t_layer_step_us']:.1f} us")
    run.close()
    return out


def single_layer(dev, stream, args, steps=64):
    """The 32K single layer (32 heads, ~5% zoom), graph replay of 64 steps."""
    import synth
    s = synth.spec("single_layer_32k")
    run = DecodeRun(s, "device", dev, stream, log_build=False)
    run.make_queries(steps)
    run.calibrate(lambda l: synth.zoom_targets(s, l), args.calib_steps)
    for t in range(args.warmup):
        run.step(t % steps)
    per_layer, zoom, _ = run.algorithmic_bytes(steps)
    g = run.capture(steps)
    t_ms = run.time_steps(steps, g)
    g = None
    e = _layer_step_entry(s, t_ms, steps * s.L, float(per_layer.mean()), zoom)
    run.close()
    return e


# one-sided Jacobi sweeps per span matrix under the plain stopping rule (a sweep
# with no rotation), measured in a diagnostic build of the builder (mean over every
# span of the 128K workload at the bf16 rotation threshold).  The builder stops
# earlier where the kept rank is below the span's size, so the FLOP rate below is
# the plain rule's work over the measured time (an equivalent rate).
JACOBI_SWEEPS = 8.6


def builder_runs(dev, stream, alphas=(0.5, 1.0, 2.0), ranks=(8, 16, 32)):
    """The prefill builder on its stress workload (131072 tokens x 32 kv heads,
    bases in pinned host memory) over alpha x rank budget: seconds per build
    (segmentation, summaries, anchors, the SVD of every span of K and V, the
    copy into the pinned store) and nominal Jacobi FLOP/s."""
    import numpy as np
    import torch

    import synth
    from hierarchical_kv_cache_surprisal_amd import sekv
    s = synth.spec("prefill_builder_128k")
    H = torch.from_numpy(synth.surprisal_batch(s)).to(dev)
    K, V = synth.kv_layer(s, 0, device=dev)
    torch.cuda.synchronize()
    out = {}
    for a in alphas:
        # a context's span table belongs to one (surprisal, alpha)
        ctx = sekv.Context(1, s.B, s.n, s.Hq, s.Hkv, s.d, s.kv_dtype, s.w, "host")
        for r in ranks:
            ctx.build(0, H, K, V, a, (r,), s.rank_seed)  # warm (allocations of this alpha)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ctx.build(0, H, K, V, a, (r,), s.rank_seed)
            torch.cuda.synchronize()
            t = time.perf_counter() - t0
            mc = np.asarray(ctx.spans(0)[1], np.float64)
            q = np.minimum(mc, 128.0)
            per_sweep = 6.0 * 128.0 * q * (q - 1.0) / 2.0
            gram = np.where(mc > 128, 2.0 * mc * s.d * s.d, 0.0)
            flops = 2 * s.Hkv * float((JACOBI_SWEEPS * per_sweep + gram).sum())
            out[f"alpha{a}_rank{r}"] = {"seconds": t, "tokens_per_s": s.n / t, "spans": int(mc.size),
                                        "mean_span": float(mc.mean()), "nominal_tflops": flops / t / 1e12}
            log(f"builder alpha {a} rank {r}: {t * 1e3:.1f} ms, {mc.size} spans")
        ctx.close()
    del K, V
    torch.cuda.empty_cache()
    out["note"] = (f"one build of 131072 tokens x {s.Hkv} kv heads (K and V), bases in pinned host memory; "
                   f"nominal FLOP = {JACOBI_SWEEPS} sweeps (the plain stopping rule's mean; the builder stops earlier "
                   f"for ranks below the span size) x 6pq(q-1)/2 per span matrix (p = 128, q = min(c, 128)) "
                   f"plus 2cd^2 for the Gram of spans longer than 128")
    return out


# ============================================================================ read reference

def read_reference(dev, stream, sizes, reps=20):
    """What a plain streaming read reaches on this GPU: a hand-written kernel of
    16-byte loads (libsekv_bench.so), each workgroup reading a contiguous slice,
    over a small sweep of grid sizes and loads in flight; the best per size.
    Sizes: one layer-step's algorithmic bytes, and 1 GiB."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "hierarchical_kv_cache_surprisal_amd", "libsekv_bench.so"))
    lib.sekv_bench_read.restype = ctypes.c_int
    lib.sekv_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    sink_len = 1 << 16
    sink = torch.zeros(sink_len, dtype=torch.int32, device=dev)
    out = []
    for nbytes in sizes:
        nbytes = max(16, nbytes // 16 * 16)
        x = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        best = None
        for grid in (1024, 2048, 4096, 8192):
            for unroll in (4, 8):
                def launch():
                    rc = lib.sekv_bench_read(x.data_ptr(), nbytes, sink.data_ptr(), sink_len, grid, unroll,
                                             stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"sekv_bench_read: {rc}")
                for _ in range(3):
                    launch()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    launch()
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) * 1e-3 / reps
                if best is None or t < best[0]:
                    best = (t, grid, unroll)
        t, grid, unroll = best
        out.append({"bytes": nbytes, "us": t * 1e6, "GB/s": nbytes / t / 1e9,
                    "frac_of_peak": nbytes / t / 1e9 / PEAK_HBM_GBS, "grid": grid, "loads_in_flight": unroll})
        del x
    log("read reference: " + ", ".join(f"{o['bytes'] / 1e6:.1f} MB {o['GB/s']:.0f} GB/s" for o in out))
    return {"kernel": "hand-written 16-byte streaming read (libsekv_bench.so), back-to-back launches, "
                      "best of grid {1024..8192} x {4, 8} loads in flight", "runs": out}


# ============================================================================ CPU baseline

def _oracle_worker(wid, spec_name, layer, g, taus_group, n_q, t_solo, t_all, solo, q_out, go_solo, go_all):
    """One process of the oracle pool: build the oracle's artefacts of kv head g
    of `layer` (not timed), then decode head-steps for a fixed window: alone
    (solo workers, one at a time), then with every worker at once."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import sekv_oracle as O
    torch.set_num_threads(1)
    with threadpool_limits(limits=1):
        s = synth.spec(spec_name)
        H = synth.surprisal_batch(s)
        K, V = synth.kv_layer(s, layer, device="cpu", heads=[g])
        Kh = K.float().numpy().astype(np.float64)
        Vh = V.float().numpy().astype(np.float64)
        del K, V
        _, arts = O.build_layer(H, Kh, Vh, s.alpha, s.w, layer, s.rank_choices, s.rank_seed, s.kv_dtype,
                                heads=[g])
        del Kh, Vh
        qs = [synth.queries(s, layer, t).numpy().astype(np.float64) for t in range(n_q)]
        heads = [(b, h) for b in range(s.B) for h in range(g * s.G, (g + 1) * s.G)]
        q_out.put(("built", wid))

        def window(seconds):
            n = 0
            t0 = time.perf_counter()
            while True:
                q = qs[n % n_q]
                for (b, h) in heads:
                    O.decode_head(q[b, h], float(taus_group[h - g * s.G]), arts[(b, g)])
                n += 1
                t = time.perf_counter() - t0
                if t >= seconds:
                    return n * len(heads), t

        if solo:
            go_solo.wait()
            q_out.put(("solo", wid) + window(t_solo))
        go_all.wait()
        q_out.put(("all", wid) + window(t_all))


def cpu_baseline(s, taus, seconds):
    """The oracle (numpy fp64, untuned) on a bounded sample of the workload, on
    the host's cores: one process per core (at most CPU_POOL_MAX), half of them
    on kv heads of layer 0 (streaming heads, low zoom) and half on kv heads of
    the layer with the highest zoom rates (retrieval heads).  Each process builds
    its head's artefacts (not timed), then decodes head-steps for `seconds` with
    every process running; two of them first run alone for a 1-thread figure.
    A layer-step is every query head of the layer: with P cores working at once
    it takes (mean time per head-step) x H_q / P."""
    import multiprocessing as mp

    import numpy as np

    import synth
    P = max(2, min(CPU_POOL_MAX, len(os.sched_getaffinity(0))))
    lz = [float(np.mean(synth.zoom_targets(s, l))) for l in range(s.L)]
    lr = int(np.argmax(lz))
    half = P // 2
    tasks = []
    for i in range(P):
        layer = 0 if i < half else lr
        k = i if i < half else i - half
        cnt = half if i < half else P - half
        g = (k * s.Hkv) // cnt
        tasks.append((layer, g))
    mpc = mp.get_context("spawn")
    q_out = mpc.Queue()
    go_all = mpc.Event()
    solo_ids = [0, half]
    go_solo = {w: mpc.Event() for w in solo_ids}
    t_solo = max(2.0, seconds / 3)
    procs = []
    t0 = time.perf_counter()
    for i, (layer, g) in enumerate(tasks):
        tg = [float(taus[layer, h]) for h in range(g * s.G, (g + 1) * s.G)]
        p = mpc.Process(target=_oracle_worker,
                        args=(i, s.name, layer, g, tg, 16, t_solo, seconds, i in go_solo, q_out,
                              go_solo.get(i, go_all), go_all))
        p.start()
        procs.append(p)
    try:
        built = 0
        while built < P:
            msg = q_out.get(timeout=600)
            built += msg[0] == "built"
        t_build = time.perf_counter() - t0
        solo = {}
        for w in solo_ids:
            go_solo[w].set()
            msg = q_out.get(timeout=600)
            solo[msg[1]] = (msg[2], msg[3])
        go_all.set()
        res = {}
        while len(res) < P:
            msg = q_out.get(timeout=600)
            if msg[0] == "all":
                res[msg[1]] = (msg[2], msg[3])
    finally:
        for p in procs:
            p.join(timeout=60)
            if p.is_alive():
                p.kill()
    # per-head-step time of each sampled head with every process running
    t_head = np.array([res[i][1] / res[i][0] for i in range(P)])
    t_ls_all = float(t_head.mean()) * s.Hq / P
    t_solo_head = np.array([solo[w][1] / solo[w][0] for w in solo_ids])
    t_ls_one = float(t_solo_head.mean()) * s.Hq
    kps = s.B * s.n / t_ls_all
    kps1 = s.B * s.n / t_ls_one
    log(f"cpu oracle: {P} processes, {sum(r[0] for r in res.values())} head-steps in {seconds:.0f}s -> {kps:.3e} KP/s; "
        f"1 thread {kps1:.3e} KP/s (artefacts built in {t_build:.1f}s, not timed)")
    return {"value": kps, "unit": "key-positions/s", "cores": P, "kind": "oracle",
            "one_thread_value": kps1,
            "sample": f"numpy fp64 oracle, {P} processes of 1 thread: kv heads "
                      f"{sorted(set(g for l, g in tasks if l == 0))} of layer 0 (streaming heads) and "
                      f"{sorted(set(g for l, g in tasks if l == lr))} of layer {lr} (the layer with the highest zoom "
                      f"rates), each decoding its head for {seconds:.0f}s at the benchmark's thresholds while every "
                      f"process runs; layer-step = mean head-step time x {s.Hq} heads / {P} processes.  "
                      f"one_thread_value: heads {tasks[0][1]} (layer 0) and {tasks[half][1]} (layer {lr}) alone for "
                      f"{t_solo:.0f}s each, x {s.Hq} heads.  Artefact builds of the sample ({t_build:.0f}s) not timed",
            "per_layer_head_step_ms": {"layer0": float(t_head[:half].mean() * 1e3),
                                       f"layer{lr}": float(t_head[half:].mean() * 1e3)}}


if __name__ == "__main__":
    main()
