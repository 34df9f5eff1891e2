"""CPU oracle for SeKV's prefill builder and mixed-resolution decode attention.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, step-by-step
statement of what the method computes, in numpy float64.  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the
product path (the HIP library and its binding) never does, and shares no
code, table or helper with it.

Sources (cited by page title, section and equation):
  [Summary] "SeKV：面向长上下文推理的分辨率自适应 KV Cache 与层级语义记忆"
            (long-form summary page), sections 2.1-2.3, eqs. (1), (2), (3),
            (5), (6), (9), the budget rule after eq. (9), Figure 2.
  [Review]  "SeKV：支持分层语义记忆的分辨率自适应KV缓存，用于长上下文大语言模型推理"
            (review page), workflow paragraph: weighted-mean summaries with a
            log|S| pre-softmax correction sharing one softmax with the
            reconstructed tokens.

Readings taken where the pages are silent or cut (each is also listed in the
design notes):
  * mu, sigma are the population mean / std of H over the whole sequence, fp64.
  * both threshold rules use a strict ">".
  * anchors = every boundary token, plus the last w positions (local window).
  * the members of a span are its positions minus anchors; empty spans are
    dropped; |S| is the member count; log is the natural log.
  * the routing projection W is the identity (no trained weights), so the
    routing summary of eq. (3) is kbar / ||kbar|| and sqrt(d') = sqrt(d);
    when a projection is given it is one d' x d matrix per (layer, kv head),
    applied to the keys (eq. 3) and to every query head reading that kv head
    (eq. 5).
  * soft rank gates (eq. 6) are given per stored component and scale the
    stored factor A = U_r Sigma_r, rounded once to the storage type.
  * the zoom rule sigmoid(s) > tau is evaluated as s > logit(tau); tau <= 0
    zooms everything, tau >= 1 nothing.
  * the trained rank gate of eq. (6) is replaced by a hard rank r_S drawn by
    a splitmix64 hash from a list of choices; r_eff = min(r_S, |S|, d).
  * a zoomed span contributes only its reconstructed tokens; a non-zoomed
    span contributes one summary entry with logit q.kbar/sqrt(d) + ln|S|.
  * budget cap: a budget counts zoomed spans per (sequence, query head);
    equal scores are ranked by span index, lower first.
  * decode-time append: appended tokens join the full-resolution window;
    re-segmentation (resegment_window) moves rows older than the last w
    positions out of it, with the prefill's threshold.
  * stored artefacts (summaries, SVD factors) are rounded to the KV dtype
    with round-to-nearest-even; everything else is fp64.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
(closed forms, hand-worked segmentation fixtures, brute force, LAPACK
identities).  No function is "parity unpinned".
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; below
    2**-126 the quantum stays 2**-133 (subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    y = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, y), y)
    return np.where(x == 0, x, y)


def round_to(x, kv_dtype: str) -> np.ndarray:
    """Storage rounding of an artefact; "f64" (oracle-only, for exact pins) keeps float64."""
    if kv_dtype == "f64":
        return np.asarray(x, dtype=np.float64).copy()
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return round_bf16(x)
    raise ValueError(kv_dtype)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of values that are already exactly bfloat16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(u) -> np.ndarray:
    u = np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# build, step 1: entropy-guided span segmentation   [Summary 2.1, eq. (1)]
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Segmentation:
    mu: float
    sigma: float
    theta: float                 # mu + alpha * sigma
    starts: np.ndarray           # int64 [m0]  span starts before empty spans are dropped
    anchors: np.ndarray          # int64 [n_a] ascending
    mstart: np.ndarray           # int64 [m]   first member position of each kept span
    mcount: np.ndarray           # int64 [m]   member count |S|
    members: List[np.ndarray]    # member positions of each kept span

    @property
    def m(self) -> int:
        return int(self.mcount.size)


def segment(H, alpha: float, w: int) -> Segmentation:
    """Cut one sequence into spans where surprisal exceeds mu + alpha * sigma.

    [Summary 2.1]: a token whose surprisal H_t exceeds the in-context mean
    plus alpha standard deviations is a span boundary, and these
    high-surprisal boundary tokens are kept as full-resolution anchors.
    Figure 2 and the memory model (eq. 17) add a local window of the last w
    tokens at full resolution.
    """
    H = np.asarray(H, dtype=np.float64)
    n = H.size
    if n == 0:
        raise ValueError("empty sequence")
    if not np.all(np.isfinite(H)) or np.any(H < 0):
        raise ValueError("surprisal must be finite and non-negative")
    mu = float(np.mean(H))
    sigma = float(np.sqrt(np.mean((H - mu) ** 2)))
    theta = mu + alpha * sigma
    flag = H > theta
    starts = np.concatenate([[0], np.flatnonzero(flag)]).astype(np.int64)
    starts = np.unique(starts)
    is_anchor = flag.copy()
    if w > 0:
        is_anchor[max(0, n - w):] = True
    anchors = np.flatnonzero(is_anchor).astype(np.int64)
    ends = np.concatenate([starts[1:], [n]])
    members, mstart, mcount = [], [], []
    for s, e in zip(starts, ends):
        mem = np.arange(s, e)[~is_anchor[s:e]]
        if mem.size == 0:
            continue
        members.append(mem)
        mstart.append(int(mem[0]))
        mcount.append(int(mem.size))
    return Segmentation(mu=mu, sigma=sigma, theta=theta, starts=starts, anchors=anchors,
                        mstart=np.asarray(mstart, dtype=np.int64),
                        mcount=np.asarray(mcount, dtype=np.int64), members=members)


# ----------------------------------------------------------------------------
# build, step 2: surprisal-weighted summaries   [Summary 2.2, eq. (2); Review]
# ----------------------------------------------------------------------------

def span_weights(H, members: np.ndarray) -> np.ndarray:
    """w_t = H_t / sum_{k in S} H_k over the span's members (uniform if that sum is 0)."""
    h = np.asarray(H, dtype=np.float64)[members]
    tot = h.sum()
    if tot == 0.0:
        return np.full(h.size, 1.0 / h.size)
    return h / tot


def weighted_mean(H, X, members: np.ndarray) -> np.ndarray:
    """kbar_S = sum_t w_t X_t / sum_t w_t (the Review's weighted mean; sum w = 1)."""
    wt = span_weights(H, members)
    return (wt[:, None] * np.asarray(X, dtype=np.float64)[members]).sum(axis=0) / wt.sum()


def routing_summary(H, K, members: np.ndarray, W) -> np.ndarray:
    """Kbar_S = sum_t w_t W K_t / || sum_t w_t W K_t ||_2   [Summary 2.2, eq. (3)].

    W is the (layer, head) routing projection, d' x d; every member key is
    projected, the projections are averaged with the surprisal weights of
    eq. (2) and the result is scaled to unit length (left at zero when the
    sum is the zero vector).
    """
    wt = span_weights(H, members)
    W = np.asarray(W, dtype=np.float64)
    acc = np.zeros(W.shape[0])
    for t, w in zip(members, wt):
        acc += w * (W @ np.asarray(K[t], dtype=np.float64))
    nrm = math.sqrt(float(acc @ acc))
    return acc / nrm if nrm > 0.0 else acc


# ----------------------------------------------------------------------------
# build, step 3: per-span rank and truncated SVD   [Summary 2.2, eq. (6)]
# ----------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """One output of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) for state x:
    advance by the golden gamma, then the two xor-shift-multiply finalisers."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def span_rank(seed: int, layer: int, g: int, k: int, choices: Sequence[int]) -> int:
    """Hard rank of span k in (layer, kv head g), standing in for the trained gate of eq. (6)."""
    key = (seed ^ (layer << 40) ^ (g << 32) ^ k) & _M64
    return int(choices[splitmix64(key) % len(choices)])


def apply_rank_gates(A, gates, kv_dtype: str) -> np.ndarray:
    """Soft rank gate of eq. (6) on a stored factor A = U_r Sigma_r (|S| x r):
    component i is scaled by its gate m_i, so that A' Bt = sum_i m_i sigma_i u_i v_i^T.
    The exact product of the stored value and the gate is rounded once to the
    storage type (round to nearest, ties to even)."""
    A = np.asarray(A, dtype=np.float64)
    m = np.asarray(gates, dtype=np.float64)[:A.shape[1]]
    return round_to(A * m[None, :], kv_dtype)


def truncated_svd(X, r: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rank-r truncation of the SVD of X (rows = tokens): A = U_r Sigma_r, Bt = V_r^T,
    so that A @ Bt = sum_{i<r} sigma_i u_i v_i^T as in eq. (6) with every gate on."""
    X = np.asarray(X, dtype=np.float64)
    U, s, Vt = np.linalg.svd(X, full_matrices=False)
    return U[:, :r] * s[:r], Vt[:r]


# ----------------------------------------------------------------------------
# build for one (sequence, layer, kv head)
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class HeadArtifacts:
    kv_dtype: str
    mstart: np.ndarray
    mcount: np.ndarray
    anchors: np.ndarray
    kbar: np.ndarray      # [m, d] stored (rounded) values
    vbar: np.ndarray
    KA: np.ndarray        # [n_a, d]
    VA: np.ndarray
    rank: np.ndarray      # [m] r_eff
    AK: List[np.ndarray]  # per span [|S|, r]
    BKt: List[np.ndarray]  # per span [r, d]
    AV: List[np.ndarray]
    BVt: List[np.ndarray]
    W: Optional[np.ndarray] = None   # routing projection [d', d] (None: identity)
    Kr: Optional[np.ndarray] = None  # routing summaries [m, d'] (stored values), with W

    @property
    def m(self) -> int:
        return int(self.mcount.size)

    @property
    def d(self) -> int:
        return int(self.kbar.shape[1]) if self.kbar.size else int(self.KA.shape[1])


def build_head(H, K, V, seg: Segmentation, layer: int, g: int, choices: Sequence[int],
               seed: int, kv_dtype: str, with_bases: bool = True, W=None) -> HeadArtifacts:
    """Everything the decode step of one (sequence, layer, kv head) reads.
    W: the head's routing projection [d', d], or None for the identity."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = K.shape[1]
    kbar = np.zeros((seg.m, d))
    vbar = np.zeros((seg.m, d))
    rank = np.zeros(seg.m, dtype=np.int64)
    AK, BKt, AV, BVt = [], [], [], []
    for k, mem in enumerate(seg.members):
        kbar[k] = weighted_mean(H, K, mem)
        vbar[k] = weighted_mean(H, V, mem)
        r = min(span_rank(seed, layer, g, k, choices), mem.size, d)
        rank[k] = r
        if with_bases:
            a, bt = truncated_svd(K[mem], r)
            AK.append(round_to(a, kv_dtype))
            BKt.append(round_to(bt, kv_dtype))
            a, bt = truncated_svd(V[mem], r)
            AV.append(round_to(a, kv_dtype))
            BVt.append(round_to(bt, kv_dtype))
    Kr = None
    if W is not None:
        W = np.asarray(W, dtype=np.float64)
        Kr = np.zeros((seg.m, W.shape[0]))
        for k, mem in enumerate(seg.members):
            Kr[k] = routing_summary(H, K, mem, W)
        Kr = round_to(Kr, kv_dtype)
    return HeadArtifacts(kv_dtype=kv_dtype, mstart=seg.mstart.copy(), mcount=seg.mcount.copy(),
                         anchors=seg.anchors.copy(), kbar=round_to(kbar, kv_dtype),
                         vbar=round_to(vbar, kv_dtype), KA=K[seg.anchors].copy(),
                         VA=V[seg.anchors].copy(), rank=rank, AK=AK, BKt=BKt, AV=AV, BVt=BVt, W=W, Kr=Kr)


# ----------------------------------------------------------------------------
# decode: stage 1 routing   [Summary 2.3, eqs. (3), (5), (9)]
# ----------------------------------------------------------------------------

def logit_threshold(tau: float) -> float:
    """theta = ln(tau) - ln(1 - tau), so that sigmoid(s) > tau  <=>  s > theta."""
    tau = float(tau)
    if math.isnan(tau):
        raise ValueError("tau is NaN")
    if tau <= 0.0:
        return -math.inf
    if tau >= 1.0:
        return math.inf
    return math.log(tau) - math.log1p(-tau)


def route_scores_projected(q, W, Kr, mcount) -> np.ndarray:
    """s_S = (W q) . Kbar_S / sqrt(d') + ln|S|   [Summary 2.3, eq. (5)]: the query
    is projected into the routing space by the same W as the keys of eq. (3)."""
    qp = np.asarray(W, dtype=np.float64) @ np.asarray(q, dtype=np.float64)
    dr = qp.size
    out = np.empty(len(mcount))
    for k in range(len(mcount)):
        out[k] = float(qp @ np.asarray(Kr[k], dtype=np.float64)) / math.sqrt(dr) + math.log(int(mcount[k]))
    return out


def head_route_scores(q, art: "HeadArtifacts") -> np.ndarray:
    """The routing scores of one head: with its projection W if it has one, else eq. (5) with W = I."""
    if art.W is not None:
        return route_scores_projected(q, art.W, art.Kr, art.mcount)
    return route_scores(q, art.kbar, art.mcount)


def route_scores(q, kbar, mcount) -> np.ndarray:
    """s_S = q . kbar_S / (||kbar_S|| sqrt(d)) + ln|S|  (eq. 5 with W = I)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.size
    out = np.empty(len(mcount))
    for k in range(len(mcount)):
        nrm = float(np.sqrt(np.dot(kbar[k], kbar[k])))
        cos = 0.0 if nrm == 0.0 else float(np.dot(q, kbar[k])) / (nrm * math.sqrt(d))
        out[k] = cos + math.log(int(mcount[k]))
    return out


def zoom_decisions(scores, theta: float) -> np.ndarray:
    """z_S = 1[sigmoid(s_S) > tau]  evaluated as  s_S > theta  (eq. 9)."""
    return np.asarray(scores) > theta


def capped_decisions(scores, theta: float, budget: Optional[int]) -> np.ndarray:
    """Zoom decisions under a budget of at most `budget` spans  [Summary 2.3, after eq. (9)].

    The spans that pass the threshold are ranked by their gate sigma(s_S),
    highest first; if there are more of them than the budget, only the first
    `budget` are zoomed.  sigma is increasing, so ranking by s_S is the same
    order.  Reading: equal scores are ranked by span index, lower first; a
    budget of None or below 0 means no cap.
    """
    z = zoom_decisions(scores, theta)
    if budget is None or budget < 0 or int(z.sum()) <= budget:
        return z
    s = np.asarray(scores, dtype=np.float64)
    cand = [k for k in range(s.size) if z[k]]
    ranked = sorted(cand, key=lambda k: (-s[k], k))
    out = np.zeros(s.size, dtype=bool)
    out[ranked[:budget]] = True
    return out


# ----------------------------------------------------------------------------
# decode: stage 2 mixed-resolution attention in one softmax   [Review; Summary Fig. 2, eq. (6)]
# ----------------------------------------------------------------------------

def mixed_entries(q, art: HeadArtifacts, zoom) -> Tuple[np.ndarray, np.ndarray]:
    """The (logit, value) list of the shared softmax for one query head."""
    q = np.asarray(q, dtype=np.float64)
    d = q.size
    sc = 1.0 / math.sqrt(d)
    logits = [art.KA @ q * sc]
    values = [art.VA]
    for k in range(art.m):
        if zoom[k]:
            Khat = art.AK[k] @ art.BKt[k]
            Vhat = art.AV[k] @ art.BVt[k]
            logits.append(Khat @ q * sc)
            values.append(Vhat)
        else:
            logits.append(np.array([float(art.kbar[k] @ q) * sc + math.log(int(art.mcount[k]))]))
            values.append(art.vbar[k][None, :])
    return np.concatenate(logits), np.concatenate(values, axis=0)


def softmax_attend(logits, values) -> np.ndarray:
    logits = np.asarray(logits, dtype=np.float64)
    p = np.exp(logits - logits.max())
    return (p @ np.asarray(values, dtype=np.float64)) / p.sum()


def decode_head(q, tau: float, art: HeadArtifacts, budget: Optional[int] = None
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One decode step of one query head: (output [d], zoom mask [m], scores [m]).
    `budget` caps the zoomed spans (capped_decisions); None: no cap."""
    theta = logit_threshold(tau)
    s = head_route_scores(q, art)
    z = capped_decisions(s, theta, budget)
    logits, values = mixed_entries(q, art, z)
    return softmax_attend(logits, values), z, s


def dense_attention(q, K, V) -> np.ndarray:
    """softmax(K q / sqrt(d)) V over every token: the full-KV reference."""
    q = np.asarray(q, dtype=np.float64)
    return softmax_attend(np.asarray(K, dtype=np.float64) @ q / math.sqrt(q.size), V)


# ----------------------------------------------------------------------------
# decode-time append   [Summary Figure 2, eq. (17): the recent tokens stay at full resolution]
# ----------------------------------------------------------------------------

def append_tokens(art: HeadArtifacts, K_new, V_new) -> HeadArtifacts:
    """New tokens join the full-resolution local window: later decode steps see
    them as exact entries of the shared softmax, like the anchors.  Reading:
    they are not re-segmented into spans (no summary, no basis)."""
    K_new = np.asarray(K_new, dtype=np.float64).reshape(-1, art.KA.shape[1])
    V_new = np.asarray(V_new, dtype=np.float64).reshape(-1, art.VA.shape[1])
    return dataclasses.replace(art, KA=np.concatenate([art.KA, K_new]), VA=np.concatenate([art.VA, V_new]))


def resegment_window(art: HeadArtifacts, positions, H_all, theta: float, w: int, n_total: int,
                     layer: int, g: int, choices: Sequence[int], seed: int) -> HeadArtifacts:
    """Streaming re-segmentation of the full-resolution window  [Summary 2.1 and Figure 2,
    applied to decoded tokens].

    positions: the context position of every row of art.KA / art.VA.  H_all: the
    surprisal of every position so far (prefill and decoded tokens); theta: the
    prefill's mu + alpha * sigma; n_total: positions so far.  The window keeps the
    last w positions; an older row leaves it when it is not itself a boundary
    (H_t <= theta: a row above theta stays a full-resolution anchor).  Readings:
      * the threshold stays the prefill's (earlier cuts never move);
      * every maximal run of consecutive leaving positions becomes a new span; a
        run next to the last span before the window starts a span of its own,
        since that span's members are no longer held at full resolution;
      * new spans follow the existing ones (span index m_old, m_old + 1, ...), with
        summaries, routing summaries, hard ranks and truncated SVD bases built as
        in the prefill from the stored rows.
    Returns the new artefacts; the positions of the remaining rows are
    [p for p in positions if p is not leaving], in their order.
    """
    H_all = np.asarray(H_all, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    leave = (positions < n_total - w) & (H_all[positions] <= theta)
    order = np.argsort(positions[leave], kind="stable")
    rows = np.flatnonzero(leave)[order]
    runs: List[np.ndarray] = []
    for r in rows:
        if runs and positions[r] == positions[runs[-1][-1]] + 1:
            runs[-1] = np.append(runs[-1], r)
        else:
            runs.append(np.array([r]))
    KA = np.asarray(art.KA, dtype=np.float64)
    VA = np.asarray(art.VA, dtype=np.float64)
    d = KA.shape[1]
    mstart, mcount = list(art.mstart), list(art.mcount)
    kbar, vbar, rank = list(art.kbar), list(art.vbar), list(art.rank)
    AK, BKt, AV, BVt = list(art.AK), list(art.BKt), list(art.AV), list(art.BVt)
    Kr = None if art.Kr is None else list(art.Kr)
    m_old = art.m
    for j, run in enumerate(runs):
        k = m_old + j
        mem = np.arange(run.size)                    # members, in the gathered rows
        Hm = H_all[positions[run]]
        Kmem, Vmem = KA[run], VA[run]
        mstart.append(int(positions[run[0]]))
        mcount.append(int(run.size))
        kbar.append(round_to(weighted_mean(Hm, Kmem, mem), art.kv_dtype))
        vbar.append(round_to(weighted_mean(Hm, Vmem, mem), art.kv_dtype))
        if Kr is not None:
            Kr.append(round_to(routing_summary(Hm, Kmem, mem, art.W), art.kv_dtype))
        r = min(span_rank(seed, layer, g, k, choices), run.size, d)
        rank.append(r)
        a, bt = truncated_svd(Kmem, r)
        AK.append(round_to(a, art.kv_dtype))
        BKt.append(round_to(bt, art.kv_dtype))
        a, bt = truncated_svd(Vmem, r)
        AV.append(round_to(a, art.kv_dtype))
        BVt.append(round_to(bt, art.kv_dtype))
    keep = ~leave
    dm = lambda lst: np.asarray(lst, dtype=np.float64).reshape(-1, d) if lst else np.zeros((0, d))
    return dataclasses.replace(
        art, mstart=np.asarray(mstart, dtype=np.int64), mcount=np.asarray(mcount, dtype=np.int64),
        anchors=positions[keep].copy(), kbar=dm(kbar), vbar=dm(vbar), KA=KA[keep].copy(), VA=VA[keep].copy(),
        rank=np.asarray(rank, dtype=np.int64), AK=AK, BKt=BKt, AV=AV, BVt=BVt,
        Kr=None if Kr is None else np.asarray(Kr, dtype=np.float64).reshape(len(Kr), -1))


# ----------------------------------------------------------------------------
# whole-layer conveniences (loops over sequences and heads)
# ----------------------------------------------------------------------------

def build_layer(H, K, V, alpha: float, w: int, layer: int, choices: Sequence[int], seed: int,
                kv_dtype: str, heads: Optional[Sequence[int]] = None, with_bases: bool = True,
                W=None) -> Tuple[List[Segmentation], Dict[Tuple[int, int], HeadArtifacts]]:
    """H [B][n]; K, V [B][Hkv'][n][d] (Hkv' = len(heads)); W None or [Hkv][d'][d]
    (indexed by kv head); returns segmentations per sequence and artefacts keyed
    by (b, kv head)."""
    H = np.asarray(H, dtype=np.float64)
    B = H.shape[0]
    heads = list(range(np.asarray(K).shape[1])) if heads is None else list(heads)
    segs = [segment(H[b], alpha, w) for b in range(B)]
    arts = {}
    for b in range(B):
        for i, g in enumerate(heads):
            arts[(b, g)] = build_head(H[b], K[b][i], V[b][i], segs[b], layer, g, choices, seed,
                                      kv_dtype, with_bases=with_bases,
                                      W=None if W is None else W[g])
    return segs, arts


def decode_layer(q, tau, arts: Dict[Tuple[int, int], HeadArtifacts], G: int,
                 heads: Optional[Sequence[int]] = None, budget=None):
    """q [B][Hq][d], tau [Hq], budget None or [Hq]; query head h reads kv head h // G.
    Returns dicts keyed by (b, h): output, zoom mask, scores."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    out, zm, sc = {}, {}, {}
    for b in range(B):
        for h in range(Hq):
            if heads is not None and h not in heads:
                continue
            key = (b, h // G)
            if key not in arts:
                continue
            cap = None if budget is None else int(budget[h])
            out[(b, h)], zm[(b, h)], sc[(b, h)] = decode_head(q[b, h], float(tau[h]), arts[key], cap)
    return out, zm, sc
