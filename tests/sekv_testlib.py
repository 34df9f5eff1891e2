"""Shared test helpers: marshal oracle artefacts into the C ABI's packed layout,
place zoom thresholds away from ties, and compare results.

Test infrastructure (may use the oracle); never imported by the product path.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

from oracle import sekv_oracle as O


def pad8(x: int) -> int:
    return (x + 7) & ~7


def storage(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """float64 values exactly representable in the KV dtype -> storage array."""
    if kv_dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return O.bf16_bits(x)


def from_storage(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    return O.bf16_from_bits(x)


def pack_bases(art: O.HeadArtifacts, kv_dtype: str, d: int) -> np.ndarray:
    """The packed layout documented at sekv_get_bases_layout: per span
    [A_K^T (r x c8) | B_K^T (r x d) | A_V^T (r x c8) | B_V^T (r x d)],
    c8 = c rounded up to 8, A stored transposed with zero columns c..c8-1."""
    parts = []
    for k in range(art.m):
        c, r = int(art.mcount[k]), int(art.rank[k])
        c8 = pad8(c)
        for A, Bt in ((art.AK[k], art.BKt[k]), (art.AV[k], art.BVt[k])):
            at = np.zeros((r, c8))
            at[:, :c] = np.asarray(A, dtype=np.float64).T
            parts.append(at.reshape(-1))
            parts.append(np.asarray(Bt, dtype=np.float64).reshape(-1))
    flat = np.concatenate(parts) if parts else np.zeros(0)
    return storage(flat, kv_dtype)


def unpack_bases(flat_storage: np.ndarray, mcount, rank, kv_dtype: str, d: int):
    """Inverse of pack_bases: lists AK (c x r), BKt (r x d), AV, BVt (float64)."""
    flat = from_storage(flat_storage, kv_dtype)
    AK, BKt, AV, BVt = [], [], [], []
    pos = 0
    for c, r in zip(mcount, rank):
        c, r = int(c), int(r)
        c8 = pad8(c)
        out = []
        for _ in range(2):
            at = flat[pos:pos + r * c8].reshape(r, c8)
            pos += r * c8
            bt = flat[pos:pos + r * d].reshape(r, d)
            pos += r * d
            out += [at[:, :c].T.copy(), bt]
        AK.append(out[0]); BKt.append(out[1]); AV.append(out[2]); BVt.append(out[3])
    return AK, BKt, AV, BVt


def import_oracle_layer(ctx, layer: int, segs: Sequence[O.Segmentation],
                        arts: Dict[Tuple[int, int], O.HeadArtifacts], B: int, Hkv: int, d: int,
                        kv_dtype: str, set_spans: bool = True, set_layout: bool = True):
    """Install the oracle's artefacts of one layer into a library context."""
    if set_spans:
        for b in range(B):
            ctx.import_spans(b, segs[b].mstart, segs[b].mcount, segs[b].anchors)
    m_max = ctx.m_max()  # the row stride of the context's per-span arrays (spare rows included)
    if set_layout:
        rank = np.ones((B, Hkv, m_max), np.int32)
        for (b, g), a in arts.items():
            rank[b, g, :a.m] = a.rank
        ctx.import_layout(layer, rank)
    for (b, g), a in arts.items():
        ctx.import_head(layer, b, g, storage(a.kbar, kv_dtype), storage(a.vbar, kv_dtype),
                        storage(a.KA, kv_dtype), storage(a.VA, kv_dtype), a.rank.astype(np.int32),
                        pack_bases(a, kv_dtype, d))
        if a.Kr is not None:  # routed layer (the context's routing projection is already set)
            ctx.import_route_summary(layer, b, g, storage(a.Kr, kv_dtype))


# ----------------------------------------------------------------------------- thresholds

def route_band(q: np.ndarray, kbar: np.ndarray, mcount: np.ndarray) -> np.ndarray:
    """Half-width of the region around a routing score inside which fp32
    evaluation on the GPU may decide differently from the fp64 oracle:
    4 * gamma_d * (sum_i |q_i kbar_i| / (|kbar| sqrt(d)) + ln|S|), with
    gamma_d = d u / (1 - d u), u = 2^-24 (a standard dot-product error bound),
    plus a few ulps for the norm, the square root and the final add."""
    d = q.size
    u = 2.0 ** -24
    gam = d * u / (1 - d * u)
    nrm = np.sqrt(np.einsum("ij,ij->i", kbar, kbar))
    mag = np.abs(kbar) @ np.abs(q)
    cos_mag = np.where(nrm > 0, mag / np.maximum(nrm, 1e-300) / math.sqrt(d), 0.0)
    return 4 * gam * (cos_mag + np.log(mcount)) + 16 * u * (cos_mag + np.log(mcount) + 1)


def route_band_projected(q: np.ndarray, W: np.ndarray, Kr: np.ndarray, mcount: np.ndarray) -> np.ndarray:
    """Tie band of the projected routing score (W q).Kr/sqrt(d') + ln|S| in fp32:
    the error of each q'_j = W_j.q (d terms) carried through the dot with Kr,
    plus the dot over d' terms, with the same gamma bound as route_band."""
    d = q.size
    dr = W.shape[0]
    u = 2.0 ** -24
    gd = d * u / (1 - d * u)
    gr = dr * u / (1 - dr * u)
    qp = W @ q
    qerr = gd * (np.abs(W) @ np.abs(q))
    mag = np.abs(Kr) @ np.abs(qp)
    term = (gr * mag + np.abs(Kr) @ qerr) / math.sqrt(dr)
    return 4 * term + 16 * u * (mag / math.sqrt(dr) + np.log(mcount) + 1)


def head_band(q: np.ndarray, a: O.HeadArtifacts) -> np.ndarray:
    if a.W is not None:
        return route_band_projected(q, a.W, a.Kr, a.mcount)
    return route_band(q, a.kbar, a.mcount)


def place_theta(scores: np.ndarray, rate: float, band_max: float) -> float:
    """theta at the midpoint of the widest gap between sorted scores near the
    target zoom quantile (scores: all steps pooled); the gap must clear the band."""
    s = np.sort(scores.reshape(-1))[::-1]
    N = s.size
    target = rate * N
    lo = max(1, int(target * 0.6))
    hi = min(N - 1, max(lo + 1, int(math.ceil(target * 1.4)) + 1))
    gaps = s[lo - 1:hi - 1] - s[lo:hi]
    i = int(np.argmax(gaps))
    th = 0.5 * (s[lo - 1 + i] + s[lo + i])
    assert gaps[i] > 8 * band_max, f"no gap wide enough near the target rate: {gaps[i]} vs band {band_max}"
    return th


def tau_from_theta(theta: float) -> float:
    """float32 tau whose logit is within rounding of theta."""
    if theta == -math.inf:
        return 0.0
    if theta == math.inf:
        return 1.0
    return float(np.float32(1.0 / (1.0 + math.exp(-theta))))


def thresholds_for(q_steps: np.ndarray, arts, G: int, rates: np.ndarray, B: int) -> np.ndarray:
    """Per query head tau (float32) such that no decision of any step falls in the tie band."""
    steps, _, Hq, d = q_steps.shape
    taus = np.zeros(Hq, np.float32)
    for h in range(Hq):
        if rates[h] >= 1.0:
            taus[h] = 0.0
            continue
        sc, bands = [], []
        for b in range(B):
            a = arts[(b, h // G)]
            for t in range(steps):
                sc.append(O.head_route_scores(q_steps[t, b, h], a))
                bands.append(head_band(q_steps[t, b, h], a))
        sc = np.concatenate(sc)
        bm = float(np.concatenate(bands).max())
        taus[h] = tau_from_theta(place_theta(sc, rates[h], bm))
    return taus


def assert_no_ties(q: np.ndarray, tau: float, a: O.HeadArtifacts):
    th = O.logit_threshold(tau)
    if not math.isfinite(th):
        return
    s = O.head_route_scores(q, a)
    bd = head_band(q, a)
    close = np.abs(s - th) <= bd
    assert not close.any(), f"{close.sum()} routing decisions inside the fp32 tie band"


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """||o - o_ref||_inf / max(||o_ref||_inf, 1e-6)."""
    return float(np.max(np.abs(out - ref)) / max(float(np.max(np.abs(ref))), 1e-6))
