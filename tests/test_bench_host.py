"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the
counter-file reduction behind `roofline.traffic`, and the streaming-read
reference library's argument checks."""
import csv
import ctypes
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_from_scales_by_the_copy_and_averages_dispatches(tmp_path, monkeypatch):
    """FETCH_SIZE of the 1 GiB copy reads half (scale 2), WRITE_SIZE reads exactly:
    the decode kernels' per-dispatch means are scaled and summed per layer-step."""
    planned = "void sekv::k_planned<128, unsigned short, 1, false, false>(sekv::DecodeArgs)"
    combine = "void sekv::k_combine<128>(sekv::DecodeArgs)"
    copy = "void at::native::vectorized_elementwise_kernel<4, MulFunctor>"
    kib = 1 << 20  # 1 GiB in KiB
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE",
                    [(copy, kib / 2), (copy, 100.0), (planned, 50000.0), (planned, 52000.0), (combine, 400.0)])
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE",
                    [(copy, kib), (planned, 300.0), (planned, 500.0), (combine, 16.0)])
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    csrc = root / "hierarchical_kv_cache_surprisal_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("decode.hip", "sekv_device.h", "sekv_internal.h"):
        (csrc / f).write_text(f)
    monkeypatch.setattr(bench, "ROOT", str(root))
    bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))
    out = json.loads((root / "profiles" / "decode_traffic.json").read_text())["layers32_128k"]
    fetch = (51000.0 + 400.0) * 1024 * 2.0
    write = (400.0 + 16.0) * 1024 * 1.0
    assert out["fetch_bytes"] == pytest.approx(fetch)
    assert out["write_bytes"] == pytest.approx(write)
    assert out["bytes_per_launch"] == pytest.approx(fetch + write)
    assert out["kernel_hash"] == bench.kernel_source_hash()
    # the stored figure is used only while the kernel sources hash the same
    assert bench.load_traffic("layers32_128k") == pytest.approx(fetch + write)
    (csrc / "decode.hip").write_text("changed")
    assert bench.load_traffic("layers32_128k") is None


def test_decode_kernel_names():
    assert bench.decode_kernel("void sekv::(anonymous namespace)::k_planned<128, unsigned short, 4, true, false>"
                               "(sekv::DecodeArgs)") == "k_planned"
    assert bench.decode_kernel("void sekv::(anonymous namespace)::k_combine<64>(sekv::DecodeArgs)") == "k_combine"
    assert bench.decode_kernel("void sekv::(anonymous namespace)::k_route<128, unsigned short, 1, 2, false>") is None


def test_read_reference_library_rejects_bad_arguments_without_launching():
    path = os.path.join(ROOT, "hierarchical_kv_cache_surprisal_amd", "libsekv_bench.so")
    if not os.path.exists(path):
        pytest.skip("libsekv_bench.so is not built")
    lib = ctypes.CDLL(path)
    f = lib.sekv_bench_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_void_p]
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    assert f(None, 16, p, 8, 1, 4, None) == -1          # no source
    assert f(p, 0, p, 8, 1, 4, None) == -1              # no bytes
    assert f(p, 24, p, 8, 1, 4, None) == -1             # not a multiple of 16
    assert f(p, 16, p, 8, 9, 4, None) == -1             # grid beyond the sink
    assert f(p, 16, p, 8, 1, 3, None) == -1             # unsupported unroll
