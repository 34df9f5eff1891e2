"""The host planner of the planned decode kernel (csrc/plan.cpp), on the CPU.

The planner cuts a layer-step's work, the sequence "span rows of (b, g), anchor
rows of (b, g)" over the (sequence, kv head) pairs in order, into shares of at
most NS segments and 512 span rows.  These tests check its contract on
synthetic span tables (lengths, ranks and zoom frequencies of the shapes the
decode workloads have): every row in exactly one segment and in order, the
per-share limits, consecutive partial slots per pair, the charged cost within
the budget (or one oversized row), the share target met when the limits allow
it, and the bounded search when they do not."""
import ctypes
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_kv_cache_surprisal_amd", "csrc")

_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    out = str(tmp_path_factory.mktemp("plan") / "libplan_harness.so")
    subprocess.run([gxx, "-O2", "-std=c++17", "-shared", "-fPIC", f"-I{CSRC}",
                    os.path.join(ROOT, "tests", "plan_harness.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", out],
                   check=True, capture_output=True, text=True)
    L = ctypes.CDLL(out)
    L.harness_plan.restype = ctypes.c_int
    L.harness_plan.argtypes = [ctypes.c_int] * 8 + [_i32p, _i32p, _i32p, _i32p, _f32p, _f32p] + \
        [ctypes.c_double] * 4 + [ctypes.c_int, _i32p, ctypes.c_int, _i32p, ctypes.POINTER(ctypes.c_double)]
    L.harness_expected_bytes.restype = ctypes.c_double
    L.harness_expected_bytes.argtypes = [ctypes.c_int] * 5 + [_i32p, _i32p, _i32p, _f32p]
    return L


def _p(a, t):
    return a.ctypes.data_as(t) if a is not None else None


class Table:
    """A synthetic layer: B sequences, Hkv kv heads, spans of 1..max_count tokens
    (a few long ones), ranks 1..32, zoom frequencies with most rows never zoomed."""

    def __init__(self, seed, B=2, Hkv=3, d=128, esz=2, m_hi=700, na_hi=1500, max_count=4096):
        rng = np.random.default_rng(seed)
        self.B, self.Hkv, self.d, self.esz = B, Hkv, d, esz
        self.m = rng.integers(1, m_hi, size=B).astype(np.int32)
        self.na = rng.integers(0, na_hi, size=B).astype(np.int32)
        self.m_max = int(self.m.max())
        cnt = np.minimum(rng.geometric(1 / 48, size=(B, self.m_max)), max_count)
        cnt[rng.random((B, self.m_max)) < 0.02] = max_count
        self.count = cnt.astype(np.int32)
        BH = B * Hkv
        self.rank = rng.integers(1, 33, size=(BH, self.m_max)).astype(np.int32)
        z = rng.random((BH, self.m_max)).astype(np.float32)
        z[rng.random((BH, self.m_max)) < 0.8] = 0.0
        self.zprob = z
        self.zunits = np.array([sum(float(z[bg, k]) * math.ceil(self.count[bg // Hkv, k] / d)
                                    for k in range(self.m[bg // Hkv])) for bg in range(BH)], dtype=np.float32)

    def plan(self, lib, NS=4, max_rows=512, max_parts=512, span_cost=2.0, unit_cost=12288.0, zdev=1.5,
             budget=0.0, target=0):
        BH = self.B * self.Hkv
        cap = 4 * 200000
        segs = np.zeros(cap, dtype=np.int32)
        parts = np.zeros(BH, dtype=np.int32)
        bout = ctypes.c_double(0.0)
        n = lib.harness_plan(self.B, self.Hkv, self.d, self.esz, self.m_max, NS, max_rows, max_parts,
                             _p(self.m, _i32p), _p(self.na, _i32p), _p(self.count, _i32p), _p(self.rank, _i32p),
                             _p(self.zprob, _f32p), _p(self.zunits, _f32p), span_cost, unit_cost, zdev,
                             budget, target, _p(segs, _i32p), cap, _p(parts, _i32p), ctypes.byref(bout))
        assert n >= 0
        return n, segs[: 4 * n * NS].reshape(n, NS, 4), parts, bout.value

    def count_only(self, lib, budget, NS=4, max_rows=512, max_parts=512):
        bout = ctypes.c_double(0.0)
        return lib.harness_plan(self.B, self.Hkv, self.d, self.esz, self.m_max, NS, max_rows, max_parts,
                                _p(self.m, _i32p), _p(self.na, _i32p), _p(self.count, _i32p),
                                _p(self.rank, _i32p), _p(self.zprob, _f32p), _p(self.zunits, _f32p),
                                2.0, 12288.0, 1.5, budget, 0, None, 0, None, ctypes.byref(bout))


def _check_structure(t, n, segs, parts, NS, max_rows):
    """Every row once, in the canonical order; per-share limits; slots."""
    BH = t.B * t.Hkv
    expect = []  # canonical sequence of (bg, is_anchor, row)
    for bg in range(BH):
        b = bg // t.Hkv
        expect += [(bg, 0, k) for k in range(t.m[b])]
        expect += [(bg, 1, r) for r in range(t.na[b])]
    got = []
    seen_slots = [[] for _ in range(BH)]
    for s in range(n):
        rows = [tuple(x) for x in segs[s]]
        used = [x for x in rows if x[2] > 0]
        assert 1 <= len(used) <= NS
        # the list ends at the first segment with no rows
        assert all(x == (0, 0, 0, 0) for x in rows[len(used):])
        span_rows = 0
        for (x, first, cnt, slot) in used:
            bg = x & 0x7FFFFFFF
            anchor = 1 if x < 0 else 0
            assert 0 <= bg < BH
            got += [(bg, anchor, first + i) for i in range(cnt)]
            if not anchor:
                span_rows += cnt
            seen_slots[bg].append(slot)
        assert span_rows <= max_rows
    assert got == expect
    for bg in range(BH):
        assert seen_slots[bg] == list(range(len(seen_slots[bg])))
        assert parts[bg] == len(seen_slots[bg])


def _share_costs(t, share, span_cost, unit_cost, zdev):
    """Charged cost of the share, and of the share without its last row."""
    row = 2.0 * t.d * t.esz
    items = []
    for (x, first, cnt, _slot) in share:
        if cnt == 0:
            continue
        bg = x & 0x7FFFFFFF
        b = bg // t.Hkv
        for k in range(first, first + cnt):
            if x < 0:
                items.append((row, 0.0))
                continue
            pz = float(t.zprob[bg, k])
            c = int(t.count[b, k])
            w = 2.0 * (((c + 7) // 8) * 8 + t.d) * int(t.rank[bg, k]) * t.esz + ((c + t.d - 1) // t.d) * unit_cost
            items.append((row * span_cost + pz * w, pz * (1 - pz) * w * w))
    def charged(it):
        return sum(m for m, _ in it) + zdev * math.sqrt(sum(v for _, v in it))
    return charged(items), charged(items[:-1])


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("NS,max_rows", [(4, 512), (2, 512), (1, 64)])
def test_cut_covers_every_row_once_within_the_limits(lib, seed, NS, max_rows):
    t = Table(seed)
    total = lib.harness_expected_bytes(t.B, t.Hkv, t.d, t.esz, t.m_max, _p(t.m, _i32p), _p(t.na, _i32p),
                                       _p(t.count, _i32p), _p(t.zunits, _f32p))
    for budget in (total / 700, total / 97, total / 5, 10 * total):
        n, segs, parts, _ = t.plan(lib, NS=NS, max_rows=max_rows, budget=budget)
        _check_structure(t, n, segs, parts, NS, max_rows)
        # the count-only pass agrees with the committed cut
        assert t.count_only(lib, budget, NS=NS, max_rows=max_rows) == n


@pytest.mark.parametrize("seed", [4, 5])
def test_cut_keeps_each_share_within_its_budget(lib, seed):
    t = Table(seed)
    total = lib.harness_expected_bytes(t.B, t.Hkv, t.d, t.esz, t.m_max, _p(t.m, _i32p), _p(t.na, _i32p),
                                       _p(t.count, _i32p), _p(t.zunits, _f32p))
    for budget in (total / 400, total / 60):
        n, segs, parts, _ = t.plan(lib, budget=budget)
        over = 0
        for s in range(n):
            full, head = _share_costs(t, segs[s], 2.0, 12288.0, 1.5)
            if full > budget * (1 + 1e-9):
                # only a row taken while the share was at most half full may overrun
                assert head <= 0.5 * budget * (1 + 1e-9)
                over += 1
        assert over < n


def test_expected_bytes_counts_rows_and_units(lib):
    t = Table(6)
    row = 2.0 * t.d * t.esz
    want = sum(t.m[bg // t.Hkv] * 2 * row + t.na[bg // t.Hkv] * row + float(t.zunits[bg]) * 16384.0
               for bg in range(t.B * t.Hkv))
    got = lib.harness_expected_bytes(t.B, t.Hkv, t.d, t.esz, t.m_max, _p(t.m, _i32p), _p(t.na, _i32p),
                                     _p(t.count, _i32p), _p(t.zunits, _f32p))
    assert got == pytest.approx(want, rel=1e-12)
    # before any zoom mask: rows only
    got0 = lib.harness_expected_bytes(t.B, t.Hkv, t.d, t.esz, t.m_max, _p(t.m, _i32p), _p(t.na, _i32p),
                                      _p(t.count, _i32p), None)
    assert got0 == pytest.approx(sum(t.m[bg // t.Hkv] * 2 * row + t.na[bg // t.Hkv] * row
                                     for bg in range(t.B * t.Hkv)), rel=1e-12)


@pytest.mark.parametrize("target", [8, 48, 200, 768])
def test_share_target_is_met_when_the_limits_allow(lib, target):
    t = Table(7, B=4, Hkv=2)
    n, segs, parts, budget = t.plan(lib, target=target)
    _check_structure(t, n, segs, parts, 4, 512)
    # the floor: the fewest shares that the segment and row limits allow
    floor = t.count_only(lib, 1e30)
    assert n <= max(target, floor)
    if floor <= target:
        assert n <= target


def test_target_below_the_floor_ends_with_the_floor(lib):
    """One share per workgroup cannot hold more than 512 span rows: a target of
    one share for thousands of span rows is out of reach, and the bounded
    budget search ends with the floor instead of growing the budget forever."""
    t = Table(8, B=2, Hkv=4, m_hi=3000)
    floor = t.count_only(lib, 1e30)
    assert floor > 1
    n, segs, parts, budget = t.plan(lib, target=1)
    assert n == floor
    _check_structure(t, n, segs, parts, 4, 512)


def test_empty_layer_and_anchor_only_layer(lib):
    t = Table(9, B=1, Hkv=2)
    t.m[:] = 0
    t.zunits[:] = 0
    n, segs, parts, _ = t.plan(lib, target=16)
    _check_structure(t, n, segs, parts, 4, 512)
    assert all(x < 0 for s in range(n) for (x, _f, c, _w) in segs[s] if c > 0)  # anchors only
    t.na[:] = 0
    n, segs, parts, _ = t.plan(lib, target=16)
    assert n == 0 and list(parts) == [0, 0]
