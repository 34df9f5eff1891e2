"""Seeded synthetic workloads for the SeKV decode path and its prefill builder.

This module only draws random numbers and plants structure; it computes
nothing that the method computes (no statistics of the surprisal, no
segmentation, no summaries, no scores).  Both the CPU oracle and the HIP
path consume what it returns, so the two always see identical inputs.

Shapes of the inputs follow the SeKV pages (Liu Zhao's long-form summary,
sections 2.1-2.3): a per-token surprisal H_t (eq. 1) whose spikes mark topic
shifts, per-(layer, head) keys and values with low-rank structure inside each
semantic span (the premise of eqs. 6-8), and decode queries.  The real
workloads of the pages (LongBench, RULER, InfiniteBench, NIAH) are not used:
a 128K context stands in for RULER/InfiniteBench lengths and a planted
"needle" span aligned with the query stands in for NIAH (section 3.3).

Random streams
  * surprisal: numpy PCG64 seeded with SeedSequence([cfg_id, 0, b, 11]) -- host.
  * keys/values/queries: torch.Generator on the requested device, seeded from
    SeedSequence([cfg_id, layer, b, head, stream]).  The same seed on a
    different device type gives a different (equally valid) draw, so a test
    draws once and hands copies to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    cfg_id: int
    L: int               # layers
    B: int               # independent sequences
    Hq: int              # query heads
    Hkv: int             # key/value heads
    d: int               # head dimension
    n: int               # context length
    kv_dtype: str        # "f32" or "bf16"
    alpha: float         # boundary sensitivity of the span rule
    w: int               # local window kept at full resolution
    steps: int           # decode steps
    s0: float            # lognormal sigma of the base surprisal
    spikes: Tuple[Tuple[float, float], ...]   # (rate, multiplier) per level
    plant_level: int     # spikes of this level or higher start a planted segment
    rho: Tuple[int, int]  # planted rank range (inclusive)
    noise: float         # std of the isotropic noise added to K and V
    rank_choices: Tuple[int, ...]
    rank_seed: int
    zoom: str            # "all", "rate", "stream_retrieval"
    zoom_rate: float = 0.05
    needle: str = "none"  # "none", "every4", "retrieval"
    needle_beta: float = 1.5   # query gain along the needle direction, in units of sqrt(d)
    needle_shift: float = 2.0  # shift of the needle span's mean, in units of sqrt(d)
    needle_min_len: int = 24

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


def _spec_table() -> Dict[str, Spec]:
    tiny = Spec(name="tiny", cfg_id=1, L=1, B=1, Hq=1, Hkv=1, d=64, n=2048, kv_dtype="f32",
                alpha=1.0, w=0, steps=16, s0=0.5, spikes=((0.03, 4.0),), plant_level=1,
                rho=(4, 4), noise=0.05, rank_choices=(8,), rank_seed=0x5EC1, zoom="all")
    cfg2 = Spec(name="single_layer_32k", cfg_id=2, L=1, B=1, Hq=32, Hkv=32, d=128, n=32768,
                kv_dtype="bf16", alpha=1.5, w=512, steps=64, s0=0.25, spikes=((0.014, 6.0),),
                plant_level=1, rho=(4, 4), noise=0.05, rank_choices=(4, 8, 16, 32),
                rank_seed=0x5EC2, zoom="rate", zoom_rate=0.05, needle="every4")
    cfg3 = cfg2.replace(name="layers32_128k", cfg_id=3, L=32, n=131072, steps=128,
                        rank_seed=0x5EC3, zoom="stream_retrieval", needle="retrieval")
    cfg4 = Spec(name="gqa_batch8_128k", cfg_id=4, L=1, B=8, Hq=32, Hkv=8, d=128, n=131072,
                kv_dtype="bf16", alpha=1.0, w=512, steps=64, s0=0.25, spikes=((0.026, 6.0),),
                plant_level=1, rho=(4, 4), noise=0.05, rank_choices=tuple(range(8, 65)),
                rank_seed=0x5EC4, zoom="rate", zoom_rate=0.05)
    cfg5 = Spec(name="prefill_builder_128k", cfg_id=5, L=1, B=1, Hq=32, Hkv=32, d=128, n=131072,
                kv_dtype="bf16", alpha=1.0, w=512, steps=0, s0=0.1,
                spikes=((3 / 64, 10.0), (7 / 512, 18.0), (1 / 512, 256.0)), plant_level=2,
                rho=(6, 24), noise=0.02, rank_choices=(16,), rank_seed=0x5EC5, zoom="rate")
    return {s.name: s for s in (tiny, cfg2, cfg3, cfg4, cfg5)}


SPECS: Dict[str, Spec] = _spec_table()


def spec(name: str, **overrides) -> Spec:
    s = SPECS[name]
    return s.replace(**overrides) if overrides else s


def seed_for(*keys: int) -> int:
    """A 63-bit seed derived from a tuple of non-negative integers."""
    st = np.random.SeedSequence([int(k) for k in keys]).generate_state(2, dtype=np.uint64)
    return int(st[0] >> np.uint64(1))


def _torch_gen(device, *keys: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*keys))
    return g


def torch_dtype(kv_dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[kv_dtype]


# ----------------------------------------------------------------------------
# surprisal
# ----------------------------------------------------------------------------

def spike_levels(s: Spec, b: int) -> np.ndarray:
    """int8 [n]: 0 for an ordinary token, i for a spike of level i (1-based).

    Levels occupy disjoint positions; level i covers round(rate_i * n) of them.
    """
    rng = np.random.Generator(np.random.PCG64(seed_for(s.cfg_id, 0, b, 12)))
    perm = rng.permutation(s.n)
    lev = np.zeros(s.n, dtype=np.int8)
    pos = 0
    for i, (rate, _mult) in enumerate(s.spikes, start=1):
        cnt = int(round(rate * s.n))
        lev[perm[pos:pos + cnt]] = i
        pos += cnt
    return lev


def surprisal(s: Spec, b: int) -> np.ndarray:
    """float32 [n]: lognormal(0, s0) base times the spike multiplier of each level."""
    rng = np.random.Generator(np.random.PCG64(seed_for(s.cfg_id, 0, b, 11)))
    base = rng.lognormal(mean=0.0, sigma=s.s0, size=s.n)
    lev = spike_levels(s, b)
    mult = np.ones(s.n)
    for i, (_rate, m) in enumerate(s.spikes, start=1):
        mult[lev == i] = m
    return (base * mult).astype(np.float32)


def surprisal_batch(s: Spec) -> np.ndarray:
    return np.stack([surprisal(s, b) for b in range(s.B)])


def planted_starts(s: Spec, b: int) -> np.ndarray:
    """Start positions of the generator's own planted segments (position 0 included)."""
    lev = spike_levels(s, b)
    starts = np.flatnonzero(lev >= s.plant_level)
    return np.unique(np.concatenate([[0], starts])).astype(np.int64)


# ----------------------------------------------------------------------------
# keys, values
# ----------------------------------------------------------------------------

def _needle_heads(s: Spec, layer: int) -> List[int]:
    """KV heads of this layer that carry a needle span."""
    if s.needle == "none":
        return []
    if s.needle == "every4":
        return [g for g in range(s.Hkv) if g % 4 == 0]
    if s.needle == "retrieval":
        ret = retrieval_heads(s)
        return sorted({h // s.G for (l, h) in ret if l == layer})
    raise ValueError(s.needle)


def needle_segment(s: Spec, layer: int, b: int) -> Tuple[int, int]:
    """(start, end) of the planted segment that holds the needle for (layer, b)."""
    st = planted_starts(s, b)
    ends = np.concatenate([st[1:], [s.n]])
    rng = np.random.Generator(np.random.PCG64(seed_for(s.cfg_id, layer, b, 13)))
    depth = int(rng.uniform(0.1, 0.9) * (s.n - s.w))
    ok = np.flatnonzero((ends - st >= s.needle_min_len) & (st >= depth) & (ends <= s.n - s.w))
    if ok.size == 0:
        ok = np.flatnonzero((ends - st >= s.needle_min_len) & (ends <= s.n - s.w))
    i = int(ok[0])
    return int(st[i]), int(ends[i])


def needle_direction(s: Spec, layer: int, b: int, g: int, device="cpu") -> torch.Tensor:
    gen = _torch_gen(device, s.cfg_id, layer, b, g, 14)
    u = torch.randn(s.d, generator=gen, device=device, dtype=torch.float32)
    return u / u.norm()


def _planted(s: Spec, seg: torch.Tensor, nseg: int, gen: torch.Generator, device) -> torch.Tensor:
    d, n = s.d, s.n
    mu = torch.randn(nseg, d, generator=gen, device=device, dtype=torch.float32)
    rlo, rhi = s.rho
    rho = torch.randint(rlo, rhi + 1, (nseg,), generator=gen, device=device)
    X = mu[seg]
    F = torch.randn(nseg, d, rhi, generator=gen, device=device, dtype=torch.float32)
    F = F / rho.to(torch.float32).sqrt()[:, None, None]
    F = F * (torch.arange(rhi, device=device)[None, None, :] < rho[:, None, None])
    c = torch.randn(n, rhi, generator=gen, device=device, dtype=torch.float32)
    for j in range(rhi):
        X += F[:, :, j][seg] * c[:, j:j + 1]
    X += s.noise * torch.randn(n, d, generator=gen, device=device, dtype=torch.float32)
    return X, mu


def kv_head(s: Spec, layer: int, b: int, g: int, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Keys and values [n][d] of one (layer, sequence, kv head), rounded to the KV dtype."""
    st = torch.as_tensor(planted_starts(s, b), device=device)
    flag = torch.zeros(s.n, dtype=torch.int64, device=device)
    flag[st[1:]] = 1
    seg = torch.cumsum(flag, 0)
    nseg = int(st.numel())
    out = []
    for which in (0, 1):
        gen = _torch_gen(device, s.cfg_id, layer, b, g, 20 + which)
        X, _mu = _planted(s, seg, nseg, gen, device)
        if which == 0 and g in _needle_heads(s, layer):
            a, e = needle_segment(s, layer, b)
            u = needle_direction(s, layer, b, g, device)
            X[a:e] += (s.needle_shift * math.sqrt(s.d)) * u
        out.append(X.to(torch_dtype(s.kv_dtype)))
    return out[0], out[1]


def kv_layer(s: Spec, layer: int, device="cpu", heads: Optional[Sequence[int]] = None):
    """Keys and values [B][Hkv][n][d] for one layer (optionally a subset of kv heads)."""
    heads = list(range(s.Hkv)) if heads is None else list(heads)
    dt = torch_dtype(s.kv_dtype)
    K = torch.empty(s.B, len(heads), s.n, s.d, dtype=dt, device=device)
    V = torch.empty_like(K)
    for b in range(s.B):
        for i, g in enumerate(heads):
            K[b, i], V[b, i] = kv_head(s, layer, b, g, device)
    return K, V


# ----------------------------------------------------------------------------
# queries and zoom-rate targets
# ----------------------------------------------------------------------------

def queries(s: Spec, layer: int, step: int, device="cpu") -> torch.Tensor:
    """float32 [B][Hq][d]: standard normal, plus a gain along the needle direction
    for the query heads whose kv head carries a needle."""
    gen = _torch_gen(device, s.cfg_id, layer, step, 0, 30)
    q = torch.randn(s.B, s.Hq, s.d, generator=gen, device=device, dtype=torch.float32)
    nh = _needle_heads(s, layer)
    for b in range(s.B):
        for g in nh:
            u = needle_direction(s, layer, b, g, device)
            q[b, g * s.G:(g + 1) * s.G] += (s.needle_beta * math.sqrt(s.d)) * u
    return q


def retrieval_heads(s: Spec) -> List[Tuple[int, int]]:
    """(layer, query head) pairs that behave like retrieval heads: 20% of all
    pairs, drawn only from the middle-to-late layers 8..27 (the zoom-rate
    heat-maps of the pages' section 3.4 are bright in a few mid/late layers)."""
    if s.zoom != "stream_retrieval":
        return []
    rng = np.random.Generator(np.random.PCG64(seed_for(s.cfg_id, 0, 0, 40)))
    lo, hi = (8, 27) if s.L >= 28 else (0, s.L - 1)
    cand = [(l, h) for l in range(lo, hi + 1) for h in range(s.Hq)]
    k = int(round(0.2 * s.L * s.Hq))
    k = min(k, len(cand))
    pick = rng.choice(len(cand), size=k, replace=False)
    return sorted(cand[i] for i in pick)


def zoom_targets(s: Spec, layer: int) -> np.ndarray:
    """float64 [Hq]: the fraction of spans each query head of this layer should zoom.

    "all" means every span (tau = 0); other modes return rates in (0, 1).
    """
    if s.zoom == "all":
        return np.ones(s.Hq)
    if s.zoom == "rate":
        return np.full(s.Hq, s.zoom_rate)
    if s.zoom == "stream_retrieval":
        rng = np.random.Generator(np.random.PCG64(seed_for(s.cfg_id, layer, 0, 41)))
        stream = np.exp(rng.uniform(np.log(0.005), np.log(0.01), size=s.Hq))
        retr = np.exp(rng.uniform(np.log(0.02), np.log(0.20), size=s.Hq))
        ret = {h for (l, h) in retrieval_heads(s) if l == layer}
        return np.array([retr[h] if h in ret else stream[h] for h in range(s.Hq)])
    raise ValueError(s.zoom)
