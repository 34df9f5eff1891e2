"""The decode entry point that allocates nothing (sekv_decode_attn_noalloc),
through the C ABI, against sekv_decode_attn on the same context and queries.

Both run the same kernels on the same work schedule, so the zoom masks must
match bit for bit and the outputs within 1e-4 relative (the decode parity
bar against the oracle); the scratch array is shared by every call on the
GPU, so two calls in a row, the second on a smaller context, must both be
right.  The entry point is also replayed from a captured HIP graph, with eager
work between the replays, each replay checked against the eager result.
"""
import numpy as np
import pytest
import torch

import synth
from tests import sekv_testlib as T
from tests.test_gpu_parity import DEV, _ctx, _inputs, _lib

pytestmark = pytest.mark.gpu


def _taus(s, ctx, layer, qd, rates):
    """Per query head tau at the given zoom rate (quantile of the GPU's routing scores)."""
    m_max = ctx.m_max()
    scores = torch.empty(s.B, s.Hq, m_max, device=DEV)
    ctx.route_scores(layer, qd, scores)
    taus = np.zeros(s.Hq, np.float32)
    for h in range(s.Hq):
        pool = torch.cat([scores[b, h, :len(ctx.spans(b)[0])].double() for b in range(s.B)])
        th = float(torch.quantile(pool, 1.0 - float(rates[h % len(rates)])))
        taus[h] = np.float32(1.0 / (1.0 + np.exp(-th)))
    return taus


def _built(s, home):
    H, K, V = _inputs(s)
    ctx = _ctx(s, home)
    ctx.build(0, torch.from_numpy(H).to(DEV), K.to(DEV), V.to(DEV), s.alpha, s.rank_choices, s.rank_seed)
    torch.cuda.synchronize()
    return ctx


def _compare(s, ctx, qd, taus, with_mask):
    """sekv_decode_attn, then sekv_decode_attn_noalloc on the same query; masks
    bit-exact, outputs within 1e-4 relative."""
    m_max = ctx.m_max()
    out_ref = torch.zeros(s.B, s.Hq, s.d, device=DEV)
    mask_ref = torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV)
    ctx.decode_attn(0, qd, taus, out_ref, mask_ref)
    out = torch.full((s.B, s.Hq, s.d), float("nan"), device=DEV)
    mask = torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV) if with_mask else None
    ctx.decode_attn(0, qd, taus, out, mask, noalloc=True)
    torch.cuda.synchronize()
    if with_mask:
        assert torch.equal(mask, mask_ref), "zoom masks differ"
    ref = out_ref.cpu().numpy().astype(np.float64)
    got = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in range(s.B):
        for h in range(s.Hq):
            worst = max(worst, T.rel_err(got[b, h], ref[b, h]))
    assert worst <= 1e-4, f"worst relative error {worst:.3e}"
    zoomed = int((mask_ref[:, :, :] == 1).sum().item())
    return worst, zoomed


def test_noalloc_matches_decode_two_calls_second_smaller():
    _lib()
    # first: a ragged GQA batch, DEVICE bases, the zoom mask into the scratch array
    s1 = synth.spec("gqa_batch8_128k").replace(B=3, Hq=8, Hkv=2, n=6000, steps=2)
    c1 = _built(s1, "device")
    # second: one sequence, one query head per kv head, bases read in place from host memory
    s2 = synth.spec("single_layer_32k").replace(n=2048, Hq=4, Hkv=4, steps=2)
    c2 = _built(s2, "host")
    sekv = _lib()
    # no work schedule before the first sekv_decode_attn of the layer
    q2 = synth.queries(s2, 0, 0).to(DEV)
    with pytest.raises(sekv.SekvError, match="STATE"):
        c2.decode_attn(0, q2, np.full(s2.Hq, 0.5, np.float32), torch.zeros_like(q2), noalloc=True)
    for t in range(s1.steps):
        q1 = synth.queries(s1, 0, t).to(DEV)
        taus1 = _taus(s1, c1, 0, q1, [0.02, 0.1, 0.3, 0.6])
        _, z1 = _compare(s1, c1, q1, taus1, with_mask=False)
        # the smaller input right after, on the same scratch array
        q2 = synth.queries(s2, 0, t).to(DEV)
        taus2 = _taus(s2, c2, 0, q2, [0.05, 0.5, 0.15, 1.0])
        _, z2 = _compare(s2, c2, q2, taus2, with_mask=True)
        assert z1 > 0 and z2 > 0


def test_noalloc_refuses_staged_bases():
    s = synth.spec("single_layer_32k").replace(n=2048, Hq=2, Hkv=2, steps=1)
    ctx = _built(s, "host_staged")
    q = synth.queries(s, 0, 0).to(DEV)
    out = torch.zeros_like(q)
    ctx.decode_attn(0, q, np.full(s.Hq, 0.9, np.float32), out)
    sekv = _lib()
    with pytest.raises(sekv.SekvError, match="STATE"):
        ctx.decode_attn(0, q, np.full(s.Hq, 0.9, np.float32), out, noalloc=True)


def test_noalloc_graph_replays_match_eager():
    s = synth.spec("gqa_batch8_128k").replace(B=2, Hq=8, Hkv=2, n=5000, steps=3)
    ctx = _built(s, "device")
    qs = [synth.queries(s, 0, t).to(DEV) for t in range(s.steps)]
    taus = _taus(s, ctx, 0, qs[0], [0.05, 0.2])
    m_max = ctx.m_max()
    stream = torch.cuda.current_stream()
    # ordinary decodes size the work schedule; from here on only the entry point
    # that allocates nothing runs, and it leaves the schedule as it is
    for q in qs:
        ctx.decode_attn(0, q, taus, torch.zeros(s.B, s.Hq, s.d, device=DEV), None, stream)
    eager_out, eager_mask = [], []
    for q in qs:
        o = torch.zeros(s.B, s.Hq, s.d, device=DEV)
        m = torch.full((s.B, s.Hq, m_max), 7, dtype=torch.uint8, device=DEV)
        ctx.decode_attn(0, q, taus, o, m, stream, noalloc=True)
        eager_out.append(o)
        eager_mask.append(m)
    torch.cuda.synchronize()
    assert sum(int((m == 1).sum().item()) for m in eager_mask) > 0
    outs = [torch.zeros_like(o) for o in eager_out]
    masks = [torch.zeros_like(m) for m in eager_mask]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for t, q in enumerate(qs):
                ctx.decode_attn(0, q, taus, outs[t], masks[t], cap, noalloc=True)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        for m in masks:
            m.fill_(7)
        # eager work between the replays: a decode of another query on the same scratch
        scratch_out = torch.zeros(s.B, s.Hq, s.d, device=DEV)
        ctx.decode_attn(0, qs[(rep + 1) % len(qs)], taus, scratch_out, None, stream, noalloc=True)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in range(len(qs)):
            assert torch.equal(masks[t], eager_mask[t]), f"replay {rep} step {t}: masks differ"
            assert torch.equal(outs[t], eager_out[t]), f"replay {rep} step {t}: outputs differ"
