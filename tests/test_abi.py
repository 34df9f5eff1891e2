"""The C ABI library builds, loads and exports every symbol declared in include/sekv.h.
Host-only checks: no kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sekv.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sekv_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("sekv_create", "sekv_destroy", "sekv_build", "sekv_zoom_fetch", "sekv_decode_attn",
                 "sekv_route_scores", "sekv_import_spans", "sekv_import_layout", "sekv_import_head",
                 "sekv_export_head", "sekv_get_spans", "sekv_get_bases_layout", "sekv_get_stats",
                 "sekv_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    from hierarchical_kv_cache_surprisal_amd import sekv
    lib = sekv.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(sekv.EXPORTED) == _declared()


def test_struct_layouts_match_header():
    from hierarchical_kv_cache_surprisal_amd import sekv
    assert ctypes.sizeof(sekv.sekv_config) == 10 * 4
    assert ctypes.sizeof(sekv.sekv_stats) == 13 * 8


def test_create_rejects_bad_configs_without_touching_a_device():
    from hierarchical_kv_cache_surprisal_amd import sekv
    bad = [
        dict(n_layers=0),
        dict(n_q_heads=6, n_kv_heads=4),
        dict(n_q_heads=48, n_kv_heads=3),   # G = 16
        dict(d_head=96),
        dict(kv_dtype=7),
        dict(local_window=-1),
        dict(basis_home=9),
        dict(n_q_heads=128, n_kv_heads=128),
    ]
    base = dict(n_layers=1, batch=1, n_ctx=64, n_q_heads=4, n_kv_heads=4, d_head=64, kv_dtype=0,
                local_window=0, basis_home=1, device=0)
    for over in bad:
        kw = dict(base, **over)
        with pytest.raises(sekv.SekvError) as ei:
            sekv.sekv_create(**kw)
        assert ei.value.status == sekv.SEKV_ERR_INVALID, over


def test_null_context_calls_fail_cleanly():
    from hierarchical_kv_cache_surprisal_amd import sekv
    lib = sekv.load_library()
    assert lib.sekv_decode_attn(None, 0, None, None, None, None, None) == sekv.SEKV_ERR_INVALID
    assert lib.sekv_build(None, 0, None, None, None, 1.0, None, 0, 0, None) == sekv.SEKV_ERR_INVALID
    st = sekv.sekv_stats()
    assert lib.sekv_get_stats(None, ctypes.byref(st)) == sekv.SEKV_ERR_INVALID
    lib.sekv_destroy(None)
    # every other entry point that takes a context refuses a NULL one before any HIP call
    for name in _declared():
        f = getattr(lib, name)
        if name in ("sekv_create", "sekv_destroy", "sekv_last_error") or not f.argtypes:
            continue
        args = []
        for t in f.argtypes:
            if t in (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64):
                args.append(0)
            elif t is ctypes.c_double:
                args.append(1.0)
            else:
                args.append(None)
        assert f(*args) == sekv.SEKV_ERR_INVALID, name


def test_pack_unpack_roundtrip():
    """The test-side packer follows the header's layout rule (blocks padded to 8)."""
    from tests.sekv_testlib import pack_bases, unpack_bases, pad8
    from oracle import sekv_oracle as O
    rng = np.random.default_rng(0)
    H = rng.lognormal(0, 0.5, 200)
    K = rng.normal(size=(200, 64))
    V = rng.normal(size=(200, 64))
    seg = O.segment(H, 1.0, 10)
    art = O.build_head(H, K, V, seg, 0, 0, (3, 5, 8), 1, "f32")
    flat = pack_bases(art, "f32", 64)
    want = sum(2 * r * (pad8(c) + 64) for c, r in zip(art.mcount, art.rank))
    assert flat.size == want
    AK, BKt, AV, BVt = unpack_bases(flat, art.mcount, art.rank, "f32", 64)
    for k in range(art.m):
        assert np.array_equal(AK[k], art.AK[k]) and np.array_equal(BVt[k], art.BVt[k])


def test_binding_rejects_bad_tensors_before_the_library():
    """The Context wrapper checks dtype, device and size of every device buffer the
    library would read or write through a raw pointer, and the host arrays'
    lengths, and raises ValueError before any call into the library."""
    import torch
    from hierarchical_kv_cache_surprisal_amd import sekv
    ctx = object.__new__(sekv.Context)  # no library context: the checks come first
    ctx.B, ctx.Hq, ctx.Hkv, ctx.L, ctx.n, ctx.d, ctx.kv_dtype, ctx.device = 1, 4, 2, 1, 64, 64, "bf16", 0
    ctx.ptr = None
    cpu_q = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError, match="cuda"):
        ctx.decode_attn(0, cpu_q, np.zeros(4, np.float32), cpu_q)
    with pytest.raises(ValueError, match="cuda"):
        ctx.build(0, torch.zeros(1, 64), torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16),
                  torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16), 1.0, (8,), 1)
    with pytest.raises(ValueError, match="K_new"):
        ctx.append_tokens(0, torch.zeros(3), torch.zeros(3))
    with pytest.raises(ValueError, match="torch tensor"):
        sekv._check_tensor(np.zeros(4), "x", torch.float32, 4, 0)
    with pytest.raises(ValueError, match="entries"):
        sekv._check_host(np.zeros(3), "tau", 4)
