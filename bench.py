"""Benchmark: SeKV mixed-resolution decode attention on one MI355X.

Workload (default): 32 layers x 32 heads, d=128, n=131072 tokens, bf16 K/V,
batch 1, synthetic inputs (seeded surprisal with spikes, planted low-rank span
structure, per-(layer, head) zoom rates 0.5-20%, retrieval-head needles).
Every layer is built on the GPU (segmentation, summaries, anchors, truncated
SVD of every span into a device-resident basis store), then decode steps are
timed: one step = one decode-attention pass over all 32 layers.

Reported metric: key positions per second per layer-step (B*n / t_layer_step),
plus achieved HBM bandwidth of one layer-step (the route kernel, which does the
work, and the small combine kernel) from the algorithmic bytes of each
layer-step (anchors, summaries, zoomed spans' bases, q/out/mask), timed with
HIP events around a graph replay of every step.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --home host ...          # bases in pinned host memory, read in place: PCIe-inclusive rate
    python bench.py --home host_staged ...   # bases in pinned host memory, zoomed spans copied to staging per step
    python bench.py --copy-calibration ...   # also runs a 1 GiB device copy (counter scaling)
    python bench.py --traffic-from FETCH_DIR WRITE_DIR   # rocprofv3 --pmc runs -> profiles/decode_traffic.json
"""
from __future__ import annotations

import argparse
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
    p.add_argument("--cpu-heads", type=int, default=4, help="kv heads in the CPU-baseline sample")
    p.add_argument("--cpu-steps", type=int, default=160, help="decode steps in the CPU-baseline sample")
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
    """HBM traffic of the decode kernel measured with rocprofv3 counters, if the
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
    """The decode kernels of a device-resident layer-step: the route kernel in
    its decode mode (mode template argument 0, before the routing-projection
    flag; mode 2 is the routing-scores pass used to calibrate thresholds) and
    the combine kernel."""
    import re
    if re.search(r"k_route<[^>]*,\s*0,\s*(false|true)>", name):
        return "k_route"
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
           "note": "one launch = one layer-step (k_route + k_combine): mean over dispatches"}
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
    esz = 2 if s.kv_dtype == "bf16" else 4
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------------ build every layer
    ctx = sekv.Context(L, B, n, Hq, Hkv, d, s.kv_dtype, s.w, args.home)
    H = torch.from_numpy(synth.surprisal_batch(s)).to(dev)
    t_gen = t_build = 0.0
    for l in range(L):
        t0 = time.perf_counter()
        K, V = synth.kv_layer(s, l, device=dev)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ctx.build(l, H, K, V, s.alpha, s.rank_choices, s.rank_seed)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        t_gen += t1 - t0
        t_build += t2 - t1
        del K, V
        if l == 0 or (l + 1) % 8 == 0:
            log(f"built layer {l + 1}/{L} (gen {t1 - t0:.2f}s build {t2 - t1:.2f}s)")
    torch.cuda.empty_cache()
    mstart, mcount, anchors, m_max = ctx.spans(0)
    ms_all = [ctx.spans(b) for b in range(B)]
    st = ctx.stats()
    log(f"spans m={len(mstart)} anchors={len(anchors)}; device-resident {st['device_resident_bytes']/1e9:.2f} GB "
        f"vs full KV {st['full_kv_bytes']/1e9:.1f} GB")

    # ------------------------------------------------------------------ queries and thresholds
    qs = torch.stack([torch.stack([synth.queries(s, l, t, device=dev) for t in range(args.steps)])
                      for l in range(L)])  # [L][steps][B][Hq][d]
    scores = torch.empty(B, Hq, m_max, device=dev)
    taus = np.zeros((L, Hq), np.float32)
    for l in range(L):
        rates = synth.zoom_targets(s, l)
        pooled = [[] for _ in range(Hq)]
        for t in range(args.calib_steps):
            q = synth.queries(s, l, 10_000 + t, device=dev)
            ctx.route_scores(l, q, scores)
            for b in range(B):
                m_b = len(ms_all[b][0])
                for h in range(Hq):
                    pooled[h].append(scores[b, h, :m_b].clone())
        for h in range(Hq):
            allsc = torch.cat(pooled[h]).double()
            th = float(torch.quantile(allsc, 1.0 - float(rates[h])))
            taus[l, h] = np.float32(1.0 / (1.0 + math.exp(-th)))
    log("thresholds calibrated")

    out = torch.empty(B, Hq, d, device=dev)
    mask = torch.zeros(L, B, Hq, m_max, dtype=torch.uint8, device=dev)

    if args.cache_gb > 0:
        ctx.set_basis_cache(int(args.cache_gb * (1 << 30)))
        log(f"device basis cache: {args.cache_gb} GiB over {L} layers (eager launches: the cache plans on the host)")

    def step(t):
        for l in range(L):
            ctx.decode_attn(l, qs[l, t], taus[l], out, mask[l], stream)

    # ------------------------------------------------------------------ warmup + algorithmic bytes
    for t in range(args.warmup):
        step(t % args.steps)
    torch.cuda.synchronize()

    # per-(layer, b, g, span) basis bytes and fixed bytes per layer-step
    lay_bytes = []  # algorithmic bytes of each layer-step, averaged over the sampled steps
    rank_t = torch.zeros(L, B, Hkv, m_max, dtype=torch.float64, device=dev)
    cnt_t = torch.zeros(B, m_max, dtype=torch.float64, device=dev)
    valid = torch.zeros(B, m_max, dtype=torch.bool, device=dev)
    for b in range(B):
        mcb = ms_all[b][1]
        cnt_t[b, :len(mcb)] = torch.from_numpy(mcb.astype(np.float64)).to(dev)
        valid[b, :len(mcb)] = True
        for l in range(L):
            for g in range(Hkv):
                rk, _, _ = ctx.bases_layout(l, b, g)
                rank_t[l, b, g, :len(rk)] = torch.from_numpy(rk.astype(np.float64)).to(dev)
    n_a = sum(len(ms_all[b][2]) for b in range(B))
    m_tot = sum(len(ms_all[b][0]) for b in range(B))
    fixed = (Hkv * n_a * 2 * d * esz          # anchors K and V
             + Hkv * m_tot * d * esz          # kbar
             + Hkv * m_tot * 4                # ln|S|
             + B * Hq * d * 8 + Hq * 4        # q in, out, tau
             + Hq * m_tot)                    # mask
    sample_steps = list(range(0, args.steps, max(1, args.steps // 8)))
    zoom_rates = []
    per_layer = np.zeros(L)
    for t in sample_steps:
        step(t)
        torch.cuda.synchronize()
        z = mask.view(L, B, Hkv, s.G, m_max).amax(dim=3).to(torch.bool) & valid[None, :, None, :]
        zall = mask.view(L, B, Hkv, s.G, m_max).amin(dim=3).to(torch.bool) & valid[None, :, None, :]
        basis = (2.0 * (cnt_t[None, :, None, :] + d) * rank_t * esz * z).sum(dim=(1, 2, 3))
        vbar = (Hkv * m_tot - zall.sum(dim=(1, 2, 3)).double()) * d * esz
        per_layer += (basis + vbar).cpu().numpy() + fixed
        zoom_rates.append(float(mask.float().sum() / (L * Hq * m_tot)))
    per_layer /= len(sample_steps)
    bytes_per_ls = float(per_layer.mean())
    log(f"algorithmic bytes per layer-step {bytes_per_ls/1e6:.2f} MB (min {per_layer.min()/1e6:.1f}, "
        f"max {per_layer.max()/1e6:.1f}); mean zoom rate {np.mean(zoom_rates):.4f}")

    # ------------------------------------------------------------------ timed region
    graph = None
    # staged bases sync each call, the basis cache plans on the host: no graph for either
    if not args.no_graph and args.home != "host_staged" and args.cache_gb <= 0:
        try:
            g = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    for t in range(args.steps):
                        for l in range(L):
                            ctx.decode_attn(l, qs[l, t], taus[l], out, mask[l], cap)
            stream.wait_stream(cap)
            torch.cuda.synchronize()
            for _ in range(2):  # replay warmup
                g.replay()
            torch.cuda.synchronize()
            graph = g
        except Exception as e:  # pragma: no cover
            log(f"graph capture failed ({e}); timing eager launches")
            graph = None
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    # eager launches allocate small Python objects on every call: a full
    # collection of the calibration leftovers inside the timed region would stall
    # the launch loop for milliseconds, so collect now and pause the collector
    pooled = None
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for t in range(args.steps):
            step(t)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gc.enable()
    t_ms = ev0.elapsed_time(ev1)
    launches = args.steps * L
    t_ls = t_ms * 1e-3 / launches
    kps = B * n / t_ls
    gbs = bytes_per_ls / t_ls / 1e9
    log(f"timed {args.steps} steps x {L} layers: {t_ms:.3f} ms (wall {wall*1e3:.1f} ms), "
        f"t_layer_step {t_ls*1e6:.2f} us, {kps:.3e} KP/s, {gbs:.0f} GB/s = {100*gbs/PEAK_HBM_GBS:.1f}% of peak")

    read_ref = read_reference(dev, stream, [int(bytes_per_ls), 1 << 30])

    if args.copy_calibration:
        # a device copy of known size, for scaling the HBM byte counters
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # an elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 x {COPY_BYTES >> 20} MiB device copy")

    # ------------------------------------------------------------------ CPU baseline (the oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(s, ctx, H, taus, args.cpu_heads, args.cpu_steps)

    st2 = ctx.stats()
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
                               f"bases {args.home}-resident",
                   "layers": L, "q_heads": Hq, "kv_heads": Hkv, "d_head": d, "ctx": n, "batch": B,
                   "spans": m_tot, "anchors": n_a, "graph": graph is not None, "bases": args.home,
                   **({"basis_cache_gib": args.cache_gb} if args.cache_gb > 0 else {})},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS,
                     "traffic": traffic if args.home == "device" else None,
                     "kernel": "one layer-step: k_route (the work) + k_combine"},
        "cpu_baseline": cpu,
        "read_reference": read_ref,
        "t_layer_step_us": t_ls * 1e6,
        "algorithmic_bytes_per_layer_step": bytes_per_ls,
        "head_positions_per_s": B * Hq * n / t_ls,
        "mean_zoom_rate": float(np.mean(zoom_rates)),
        "builder": {"layers": L, "seconds": t_build, "tokens_per_s": L * B * n / t_build,
                    "kv_head_rows_per_s": L * B * Hkv * n / t_build, "gen_seconds": t_gen},
        "memory": {"device_resident_bytes": st["device_resident_bytes"], "full_kv_bytes": st["full_kv_bytes"]},
        **({"basis_cache": {k: st2[k] for k in ("cache_zoomed", "cache_hits", "cache_spans_fetched",
                                                 "cache_bytes_fetched")}} if args.cache_gb > 0 else {}),
    }
    print(json.dumps(res), flush=True)


def read_reference(dev, stream, sizes, reps=40):
    """What a plain library read achieves on this GPU: torch.sum over a float32
    tensor of each size (one layer-step's algorithmic bytes, and 1 GiB), launched
    back to back on the timing stream.  Context for the roofline fraction: the
    decode step is one short launch, which a streaming read of the same size
    does not fill at the spec peak either."""
    import torch

    out = []
    for nbytes in sizes:
        x = torch.ones(max(1, nbytes // 4), dtype=torch.float32, device=dev)
        r = torch.empty((), dtype=torch.float32, device=dev)
        with torch.cuda.stream(stream):
            for _ in range(3):
                torch.sum(x, dim=0, out=r)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                torch.sum(x, dim=0, out=r)
            e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        out.append({"bytes": int(x.numel() * 4), "us": t * 1e6, "GB/s": x.numel() * 4 / t / 1e9,
                    "frac_of_peak": x.numel() * 4 / t / 1e9 / PEAK_HBM_GBS})
        del x, r
    log("read reference (torch.sum): " + ", ".join(f"{o['bytes'] / 1e6:.1f} MB {o['GB/s']:.0f} GB/s" for o in out))
    return {"kernel": "torch.sum over float32, back-to-back launches", "runs": out}


def cpu_baseline(s, ctx, H, taus, n_heads, steps):
    """The oracle (numpy fp64, untuned) on a bounded sample: build the artefacts
    of `n_heads` kv heads of layer 0 (not timed), then time the decode of those
    heads for `steps` queries (about 10 s), scaled to one full layer-step."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import sekv_oracle as O

    heads = list(range(n_heads))
    K, V = synth.kv_layer(s, 0, device="cuda", heads=heads)
    Kh = K.float().cpu().numpy().astype(np.float64)
    Vh = V.float().cpu().numpy().astype(np.float64)
    del K, V
    Hn = H.cpu().numpy()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        segs, arts = O.build_layer(Hn, Kh, Vh, s.alpha, s.w, 0, s.rank_choices, s.rank_seed, s.kv_dtype,
                                   heads=heads)
        t_build = time.perf_counter() - t0
        qh = [synth.queries(s, 0, t).numpy().astype(np.float64) for t in range(steps)]
        t0 = time.perf_counter()
        for t in range(steps):
            for b in range(s.B):
                for g in heads:
                    for h in range(g * s.G, (g + 1) * s.G):
                        O.decode_head(qh[t][b, h], float(taus[0, h]), arts[(b, g)])
        t_dec = time.perf_counter() - t0
    per_head = t_dec / (steps * s.B * len(heads) * s.G)
    t_ls = per_head * s.Hq * s.B  # one layer-step: every query head of every sequence
    kps = s.B * s.n / t_ls
    log(f"cpu oracle: {t_dec:.1f}s for {steps * s.B * len(heads) * s.G} head-steps, {per_head*1e3:.1f} ms per "
        f"head-step -> {kps:.3e} KP/s (artefact build of the sample {t_build:.1f}s, not timed)")
    return {"value": kps, "unit": "key-positions/s", "cores": 1, "kind": "oracle",
            "sample": f"numpy fp64 oracle, 1 thread: decode of {len(heads)} kv heads x {s.G} q-heads of layer 0 "
                      f"for {steps} steps ({t_dec:.1f}s) at the same thresholds, scaled to a {s.Hq}-head layer-step "
                      f"(oracle artefact build of the sample: {t_build:.1f}s, not timed)",
            # the oracle's build of the same sample (segmentation, summaries, LAPACK SVD), for
            # the builder's own comparison; not part of the decode figure above
            "builder_kv_head_rows_per_s": s.B * len(heads) * s.n / t_build}


if __name__ == "__main__":
    main()
