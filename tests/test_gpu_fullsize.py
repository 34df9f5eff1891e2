"""GPU parity at the workloads' full sizes, on sampled outputs.

The oracle cannot decode or build every head of a 128K-token, 32-head layer in
seconds, so these tests build the whole layer on the GPU and compare sampled
heads, one by one, with the oracle:

* decode: the GPU's own artefacts of the sampled heads are exported and decoded
  by the oracle (identical inputs), so the zoom masks must match bit for bit
  and the outputs within 1e-4 relative (fp32 accumulation against fp64);
* build: the span table and anchors bit-exact, the summaries and the SVD of
  sampled spans (always including the longest) against the oracle's build of
  the same heads.

The decode runs in the configuration the benchmark times: device-resident
bases, every step replayed from a captured HIP graph.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import sekv_oracle as O
from tests import sekv_testlib as T
from tests.test_gpu_parity import DEV, _check_build, _check_margins, _ctx, _lib

pytestmark = pytest.mark.gpu


def gpu_artefacts(ctx, s, layer, b, g, seg) -> O.HeadArtifacts:
    """The GPU-built artefacts of (layer, b, g), upcast to float64, as the oracle's type."""
    kb, vb, KA, VA, rank, bases = ctx.export_head(layer, b, g)
    AK, BKt, AV, BVt = T.unpack_bases(bases, seg.mcount, rank, s.kv_dtype, s.d)
    f = lambda x: T.from_storage(x, s.kv_dtype)
    return O.HeadArtifacts(kv_dtype=s.kv_dtype, mstart=seg.mstart.copy(), mcount=seg.mcount.copy(),
                           anchors=seg.anchors.copy(), kbar=f(kb), vbar=f(vb), KA=f(KA), VA=f(VA),
                           rank=np.asarray(rank, np.int64), AK=AK, BKt=BKt, AV=AV, BVt=BVt)


class SpanTable:
    """The GPU's span table of one sequence (the decode reads counts and anchors only;
    the table itself is checked bit-exact against the oracle's segmentation)."""

    def __init__(self, ctx, b):
        ms, mc, an, _ = ctx.spans(b)
        self.mstart = np.asarray(ms, np.int64)
        self.mcount = np.asarray(mc, np.int64)
        self.anchors = np.asarray(an, np.int64)


def gpu_segmentation(ctx, b) -> SpanTable:
    return SpanTable(ctx, b)


def taus_for_workload(s, ctx, layer, q_steps_dev, rates, sampled_arts, q_steps_np):
    """Per query head tau at the workload's zoom rate.  Heads that are compared
    (keys of sampled_arts: (b, g)) get tau in the widest score gap near the
    target rate, clear of the fp32 tie band; the others get the GPU scores'
    quantile (their outputs are not compared)."""
    m_max = ctx.m_max()
    taus = np.zeros(s.Hq, np.float32)
    compared = {h for (b, g) in sampled_arts for h in range(g * s.G, (g + 1) * s.G)}
    pooled = [[] for _ in range(s.Hq)]
    if len(compared) < s.Hq:
        scores = torch.empty(s.B, s.Hq, m_max, device=DEV)
        for t in range(len(q_steps_dev)):
            ctx.route_scores(layer, q_steps_dev[t], scores)
            for b in range(s.B):
                m_b = len(ctx.spans(b)[0])
                for h in range(s.Hq):
                    pooled[h].append(scores[b, h, :m_b].double().clone())
    for h in range(s.Hq):
        if h in compared:
            sc, bands = [], []
            for (b, g), a in sampled_arts.items():
                if h // s.G != g:
                    continue
                for t in range(q_steps_np.shape[0]):
                    sc.append(O.route_scores(q_steps_np[t, b, h], a.kbar, a.mcount))
                    bands.append(T.route_band(q_steps_np[t, b, h], a.kbar, a.mcount))
            taus[h] = T.tau_from_theta(T.place_theta(np.concatenate(sc), float(rates[h]),
                                                     float(np.concatenate(bands).max())))
        else:
            th = float(torch.quantile(torch.cat(pooled[h]), 1.0 - float(rates[h])))
            taus[h] = np.float32(1.0 / (1.0 + math.exp(-th)))
    return taus


def graph_decode(ctx, layer, q_steps_dev, taus, out_steps, mask_steps):
    """Eager warm-up (sizes the work schedule), then every step from one captured graph."""
    stream = torch.cuda.current_stream()
    for t in range(len(q_steps_dev)):
        ctx.decode_attn(layer, q_steps_dev[t], taus, out_steps[t], mask_steps[t], stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for t in range(len(q_steps_dev)):
                ctx.decode_attn(layer, q_steps_dev[t], taus, out_steps[t], mask_steps[t], cap)
    stream.wait_stream(cap)
    for o in out_steps:
        o.zero_()
    for m in mask_steps:
        m.fill_(7)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()


def compare_sampled(s, q_steps_np, taus, arts, out_steps, mask_steps, tol=1e-4):
    """Masks bit-exact and outputs within tol for every query head of the sampled (b, g)."""
    worst, nz = 0.0, 0
    for t in range(q_steps_np.shape[0]):
        out_h = out_steps[t].cpu().numpy().astype(np.float64)
        mask_h = mask_steps[t].cpu().numpy()
        for (b, g), a in arts.items():
            for h in range(g * s.G, (g + 1) * s.G):
                T.assert_no_ties(q_steps_np[t, b, h], float(taus[h]), a)
                o_ref, z_ref, _ = O.decode_head(q_steps_np[t, b, h], float(taus[h]), a)
                assert np.array_equal(mask_h[b, h, :a.m].astype(bool), z_ref), f"mask differs: step {t} b {b} h {h}"
                assert np.all(mask_h[b, h, a.m:] == 7), "mask written beyond m"
                e = T.rel_err(out_h[b, h], o_ref)
                worst = max(worst, e)
                nz += int(z_ref.sum())
                assert e <= tol, f"step {t} b {b} h {h}: rel err {e}"
    return worst, nz


def build_gpu_layer(s, home="device", layer=0, alpha=None, ranks=None):
    ctx = _ctx(s, home, L=1)
    H = synth.surprisal_batch(s)
    K, V = synth.kv_layer(s, layer, device=DEV)
    ctx.build(0, torch.from_numpy(H).to(DEV), K, V, s.alpha if alpha is None else alpha,
              s.rank_choices if ranks is None else ranks, s.rank_seed)
    torch.cuda.synchronize()
    return ctx, H, K, V


def check_build_sampled(s, ctx, H, K, V, heads, alpha=None, ranks=None, span_sample=24, with_arts=False):
    """Span tables of every sequence bit-exact; summaries and sampled spans' SVD of `heads`.
    Returns the oracle's segmentation (and, with_arts, its artefacts without bases)."""
    Ks = K[:, heads].float().cpu()
    Vs = V[:, heads].float().cpu()
    segs, arts = O.build_layer(H, Ks.numpy().astype(np.float64), Vs.numpy().astype(np.float64),
                               s.alpha if alpha is None else alpha, s.w, 0,
                               s.rank_choices if ranks is None else ranks, s.rank_seed, s.kv_dtype,
                               heads=heads, with_bases=False)
    _check_margins(s, H, segs)
    # the GPU's bases of sampled spans against the Eckart-Young optimum of their member rows
    _check_build(s, ctx, segs, arts, 0, H, Ks, Vs, heads=heads, span_sample=span_sample)
    return (segs, arts) if with_arts else segs


# ============================================================================ workloads

def test_single_layer_32k_all_heads_decode_and_build():
    """32 heads, n = 32768, bf16, ~5% zoom, needle every fourth head: every head
    decoded on the GPU's artefacts and compared with the oracle."""
    s = synth.spec("single_layer_32k")
    ctx, H, K, V = build_gpu_layer(s)
    segs = check_build_sampled(s, ctx, H, K, V, heads=[0, 13, 31])
    seg = gpu_segmentation(ctx, 0)
    arts = {(0, g): gpu_artefacts(ctx, s, 0, 0, g, seg) for g in range(s.Hkv)}
    steps = 3
    q_np = np.stack([synth.queries(s, 0, t).numpy().astype(np.float64) for t in range(steps)])
    q_dev = [torch.from_numpy(q_np[t].astype(np.float32)).to(DEV) for t in range(steps)]
    rates = synth.zoom_targets(s, 0)
    taus = taus_for_workload(s, ctx, 0, q_dev, rates, arts, q_np)
    m_max = ctx.m_max()
    outs = [torch.zeros(s.B, s.Hq, s.d, device=DEV) for _ in range(steps)]
    masks = [torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV) for _ in range(steps)]
    graph_decode(ctx, 0, q_dev, taus, outs, masks)
    worst, nz = compare_sampled(s, q_np, taus, arts, outs, masks)
    assert nz > 0


def test_layer_128k_sampled_heads_graph_replay():
    """The benchmark's layer shape: 32 heads, n = 131072, bf16, per-head zoom rates of a
    retrieval-heavy layer; sampled heads compared, decode from a captured graph."""
    s = synth.spec("layers32_128k")
    layer = 12  # a layer with retrieval heads
    ctx = _ctx(s, "device", L=1)
    H = synth.surprisal_batch(s)
    K, V = synth.kv_layer(s, layer, device=DEV)
    ctx.build(0, torch.from_numpy(H).to(DEV), K, V, s.alpha, s.rank_choices, s.rank_seed)
    torch.cuda.synchronize()
    rates = synth.zoom_targets(s, layer)
    heads = sorted({0, int(np.argmax(rates)), s.Hkv - 1})
    # build parity on the sampled heads (the oracle's layer index must match the GPU's: 0)
    _, own = check_build_sampled(s, ctx, H, K, V, heads=heads, with_arts=True)
    seg = gpu_segmentation(ctx, 0)
    arts = {(0, g): gpu_artefacts(ctx, s, 0, 0, g, seg) for g in heads}
    steps = 3
    q_np = np.stack([synth.queries(s, layer, t).numpy().astype(np.float64) for t in range(steps)])
    q_dev = [torch.from_numpy(q_np[t].astype(np.float32)).to(DEV) for t in range(steps)]
    taus = taus_for_workload(s, ctx, 0, q_dev, rates, arts, q_np)
    m_max = ctx.m_max()
    outs = [torch.zeros(s.B, s.Hq, s.d, device=DEV) for _ in range(steps)]
    masks = [torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV) for _ in range(steps)]
    graph_decode(ctx, 0, q_dev, taus, outs, masks)
    worst, nz = compare_sampled(s, q_np, taus, arts, outs, masks)
    assert nz > 0
    # the zoom decisions against the oracle's own summaries (its build of the same
    # heads, which may differ from the GPU's by one bf16 ulp of an element): a
    # decision may differ only where the two summaries' scores fall on either side
    # of the threshold, i.e. within their distance (plus the fp32 band) of it
    flips = total = 0
    for t in range(steps):
        mask_h = masks[t].cpu().numpy()
        for g in heads:
            q = q_np[t, 0, g]
            th = O.logit_threshold(float(taus[g]))
            sc_own = O.head_route_scores(q, own[(0, g)])
            sc_gpu = O.head_route_scores(q, arts[(0, g)])
            m_g = own[(0, g)].m
            flip = mask_h[0, g, :m_g].astype(bool) != (sc_own > th)
            near = np.abs(sc_own - th) <= np.abs(sc_own - sc_gpu) + T.route_band(q, own[(0, g)].kbar,
                                                                                 own[(0, g)].mcount)
            assert np.all(near[flip]), (t, g, np.flatnonzero(flip & ~near))
            flips += int(flip.sum())
            total += m_g
    assert flips <= max(1, total // 1000), (flips, total)
    # every head (compared or not) produced finite outputs and a mask only of 0/1 below m
    m = len(seg.mcount)
    for t in range(steps):
        assert torch.isfinite(outs[t]).all()
        assert int(masks[t][:, :, :m].max()) <= 1


def eager_decode(ctx, layer, q_steps_dev, taus, out_steps, mask_steps):
    stream = torch.cuda.current_stream()
    for o in out_steps:
        o.zero_()
    for m in mask_steps:
        m.fill_(7)
    for t in range(len(q_steps_dev)):
        ctx.decode_attn(layer, q_steps_dev[t], taus, out_steps[t], mask_steps[t], stream)
    torch.cuda.synchronize()


def test_layer_128k_host_bases_in_place_and_cached():
    """The benchmark's layer with its bases in pinned host memory (the pages' CPU
    tier): zoomed spans read in place over the host link (decode replayed from a
    captured graph), then through a device basis cache with prefetch (eager,
    repeated so that cached and uncached spans are both read).  Sampled heads
    compared with the oracle on the GPU's own artefacts."""
    s = synth.spec("layers32_128k")
    layer = 12
    ctx = _ctx(s, "host", L=1)
    H = synth.surprisal_batch(s)
    K, V = synth.kv_layer(s, layer, device=DEV)
    ctx.build(0, torch.from_numpy(H).to(DEV), K, V, s.alpha, s.rank_choices, s.rank_seed)
    torch.cuda.synchronize()
    del K, V
    rates = synth.zoom_targets(s, layer)
    heads = sorted({int(np.argmax(rates)), 5})
    seg = gpu_segmentation(ctx, 0)
    arts = {(0, g): gpu_artefacts(ctx, s, 0, 0, g, seg) for g in heads}
    steps = 3
    q_np = np.stack([synth.queries(s, layer, t).numpy().astype(np.float64) for t in range(steps)])
    q_dev = [torch.from_numpy(q_np[t].astype(np.float32)).to(DEV) for t in range(steps)]
    taus = taus_for_workload(s, ctx, 0, q_dev, rates, arts, q_np)
    m_max = ctx.m_max()
    outs = [torch.zeros(s.B, s.Hq, s.d, device=DEV) for _ in range(steps)]
    masks = [torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV) for _ in range(steps)]
    graph_decode(ctx, 0, q_dev, taus, outs, masks)
    worst, nz = compare_sampled(s, q_np, taus, arts, outs, masks)
    assert nz > 0
    ctx.set_basis_cache(256 << 20)
    for rep in range(3):
        eager_decode(ctx, 0, q_dev, taus, outs, masks)
        compare_sampled(s, q_np, taus, arts, outs, masks)
    st = ctx.stats()
    assert st["cache_zoomed"] > 0 and st["cache_hits"] > 0, st


@pytest.mark.parametrize("rate", [0.01, 0.05, 0.15, 0.30])
def test_gqa_batch8_128k_zoom_sweep(rate, _gqa_layer):
    """32 query heads on 8 kv heads, batch 8 at n = 131072, ranks 8..64: sampled
    (sequence, kv head) pairs and all their query heads, zoom rates 1-30%."""
    s, ctx, segs_gpu, arts = _gqa_layer
    steps = 2
    q_np = np.stack([synth.queries(s, 0, 100 + t).numpy().astype(np.float64) for t in range(steps)])
    q_dev = [torch.from_numpy(q_np[t].astype(np.float32)).to(DEV) for t in range(steps)]
    rates = np.full(s.Hq, rate)
    taus = taus_for_workload(s, ctx, 0, q_dev, rates, arts, q_np)
    m_max = ctx.m_max()
    outs = [torch.zeros(s.B, s.Hq, s.d, device=DEV) for _ in range(steps)]
    masks = [torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV) for _ in range(steps)]
    graph_decode(ctx, 0, q_dev, taus, outs, masks)
    worst, nz = compare_sampled(s, q_np, taus, arts, outs, masks)
    assert nz > 0


def test_gqa_plan_floor_above_the_workgroup_target(_gqa_layer, monkeypatch):
    """A workgroup target below what the per-share limits allow: 64 workgroups,
    against at least 448 shares for 64 (sequence, kv head) rows of about 3500 spans
    each (at most 512 span rows per share).  The planner settles for the smallest
    plan the limits allow (a second wave of workgroups) instead of searching for a
    budget that does not exist, and the decode matches the oracle on the sampled
    heads.  The context reads the target when it is created."""
    s, _, _, arts = _gqa_layer
    monkeypatch.setenv("SEKV_FILL_TASKS", "64")
    ctx, H, K, V = build_gpu_layer(s)
    del K, V
    torch.cuda.empty_cache()
    steps = 2
    q_np = np.stack([synth.queries(s, 0, 200 + t).numpy().astype(np.float64) for t in range(steps)])
    q_dev = [torch.from_numpy(q_np[t].astype(np.float32)).to(DEV) for t in range(steps)]
    taus = taus_for_workload(s, ctx, 0, q_dev, np.full(s.Hq, 0.05), arts, q_np)
    m_max = ctx.m_max()
    outs = [torch.zeros(s.B, s.Hq, s.d, device=DEV) for _ in range(steps)]
    masks = [torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV) for _ in range(steps)]
    eager_decode(ctx, 0, q_dev, taus, outs, masks)
    worst, nz = compare_sampled(s, q_np, taus, arts, outs, masks)
    assert nz > 0
    ctx.close()


@pytest.fixture(scope="module")
def _gqa_layer():
    s = synth.spec("gqa_batch8_128k")
    ctx, H, K, V = build_gpu_layer(s)
    # build parity of two kv heads of every sequence (span tables of all sequences)
    check_build_sampled(s, ctx, H, K, V, heads=[0, 5], span_sample=12)
    sampled = [(0, 0), (3, 5), (7, 7), (5, 2)]
    arts = {}
    for b, g in sampled:
        seg = gpu_segmentation(ctx, b)
        arts[(b, g)] = gpu_artefacts(ctx, s, 0, b, g, seg)
    del K, V
    torch.cuda.empty_cache()
    yield s, ctx, None, arts
    del ctx


@pytest.mark.parametrize("alpha", [0.5, 1.0, 2.0])
@pytest.mark.parametrize("rank", [8, 16, 32])
def test_prefill_builder_128k(alpha, rank):
    """Builder stress: 32 kv heads x 131072 tokens, three-level surprisal spikes, planted
    rank 6-24 span structure; alpha in {0.5, 1, 2} and rank budgets {8, 16, 32}."""
    s = synth.spec("prefill_builder_128k")
    ctx, H, K, V = build_gpu_layer(s, alpha=alpha, ranks=(rank,))
    segs = check_build_sampled(s, ctx, H, K, V, heads=[0, 21], alpha=alpha, ranks=(rank,), span_sample=16)
    m = segs[0].m
    assert m > 0
    st = ctx.stats()
    assert st["device_resident_bytes"] > 0


# ============================================================================ extremes

def test_largest_group_and_head_count():
    """H_q = 64 query heads on 8 kv heads (G = 8, the largest group), bf16, ragged
    batch of 2 with different contexts' spans; every head compared."""
    s = synth.spec("single_layer_32k").replace(B=2, n=6144, Hq=64, Hkv=8, steps=2)
    ctx, H, K, V = build_gpu_layer(s)
    arts = {}
    for b in range(s.B):
        seg = gpu_segmentation(ctx, b)
        for g in range(s.Hkv):
            arts[(b, g)] = gpu_artefacts(ctx, s, 0, b, g, seg)
    steps = 2
    q_np = np.stack([synth.queries(s, 0, t).numpy().astype(np.float64) for t in range(steps)])
    q_dev = [torch.from_numpy(q_np[t].astype(np.float32)).to(DEV) for t in range(steps)]
    rates = np.linspace(0.0, 0.5, s.Hq)
    rates[0] = 0.02
    taus = taus_for_workload(s, ctx, 0, q_dev, rates, arts, q_np)
    m_max = ctx.m_max()
    outs = [torch.zeros(s.B, s.Hq, s.d, device=DEV) for _ in range(steps)]
    masks = [torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV) for _ in range(steps)]
    graph_decode(ctx, 0, q_dev, taus, outs, masks)
    worst, nz = compare_sampled(s, q_np, taus, arts, outs, masks)
    assert nz > 0


def test_single_layer_32k_routing_projection_budget_append():
    """The routing projection (d' = 32), a zoom budget per head and decode-time
    appends at full size: 32 heads, n = 32768.  The GPU builds the layer with the
    projection; every head's artefacts (routing summaries included) are exported
    and decoded by the oracle with the same budgets and appended tokens."""
    from tests.test_gpu_parity import _cut_ok, _ranked
    s = synth.spec("single_layer_32k")
    dr = 32
    rng = np.random.default_rng(17)
    W = (rng.standard_normal((s.Hkv, dr, s.d)) / math.sqrt(s.d)).astype(np.float32).astype(np.float64)
    ctx = _ctx(s, "device", L=1)
    ctx.set_routing(0, dr, W)
    H = synth.surprisal_batch(s)
    K, V = synth.kv_layer(s, 0, device=DEV)
    ctx.build(0, torch.from_numpy(H).to(DEV), K, V, s.alpha, s.rank_choices, s.rank_seed)
    torch.cuda.synchronize()
    seg = gpu_segmentation(ctx, 0)
    arts = {}
    for g in range(s.Hkv):
        a = gpu_artefacts(ctx, s, 0, 0, g, seg)
        a.W = W[g]
        a.Kr = T.from_storage(ctx.export_route_summary(0, 0, g, dr), s.kv_dtype)
        arts[(0, g)] = a
    # the routing summaries against eq. (3) on the GPU's own unrounded inputs, two heads
    segs_o = O.segment(H[0], s.alpha, s.w)
    for g in (0, s.Hkv - 1):
        a = arts[(0, g)]
        Kg = K[0, g].float().cpu().numpy().astype(np.float64)
        for k in range(0, a.m, max(1, a.m // 40)):
            ref = O.routing_summary(H[0], Kg, segs_o.members[k], W[g])
            assert np.all(np.abs(a.Kr[k] - ref) <= 2.0 ** -7 * np.max(np.abs(ref)) + 1e-30), (g, k)
    steps = 3
    q_np = np.stack([synth.queries(s, 0, t).numpy().astype(np.float64) for t in range(steps)])
    taus = T.thresholds_for(q_np, arts, s.G, np.full(s.Hq, 0.08), s.B)
    m_max = ctx.m_max()
    gen = torch.Generator().manual_seed(9)
    for t in range(steps):
        q = q_np[t]
        budgets = np.full(s.Hq, -1, np.int32)
        for h in range(s.Hq):
            a = arts[(0, h)]
            sc = O.head_route_scores(q[0, h], a)
            band = T.head_band(q[0, h], a)
            order = _ranked(sc, O.logit_threshold(float(taus[h])))
            ks = [k for k in range(1, len(order)) if _cut_ok(sc, band, order, k, set())]
            if h % 4 != 3 and ks:
                budgets[h] = min(ks, key=lambda k: abs(k - len(order) // 2))
        out = torch.zeros(s.B, s.Hq, s.d, device=DEV)
        mask = torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV)
        ctx.decode_attn(0, torch.from_numpy(q.astype(np.float32)).to(DEV), taus, out, mask, budget=budgets)
        torch.cuda.synchronize()
        out_h = out.cpu().numpy().astype(np.float64)
        mask_h = mask.cpu().numpy()
        capped = 0
        for h in range(s.Hq):
            a = arts[(0, h)]
            T.assert_no_ties(q[0, h], float(taus[h]), a)
            bud = int(budgets[h])
            o_ref, z_ref, _ = O.decode_head(q[0, h], float(taus[h]), a, bud)
            assert np.array_equal(mask_h[0, h, :a.m].astype(bool), z_ref), f"mask differs: step {t} h {h}"
            assert T.rel_err(out_h[0, h], o_ref) <= 1e-4, f"step {t} h {h}"
            capped += int(bud >= 0)
        assert capped > s.Hq // 2
        # a few decoded tokens join the window before the next step
        Kn = torch.randn(s.B, s.Hkv, 3, s.d, generator=gen).to(torch.bfloat16)
        Vn = torch.randn(s.B, s.Hkv, 3, s.d, generator=gen).to(torch.bfloat16)
        ctx.append_tokens(0, Kn.to(DEV).contiguous(), Vn.to(DEV).contiguous())
        for g in range(s.Hkv):
            arts[(0, g)] = O.append_tokens(arts[(0, g)], Kn[0, g].float().numpy().astype(np.float64),
                                           Vn[0, g].float().numpy().astype(np.float64))
