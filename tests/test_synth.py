"""Checks of the seeded workload generators: determinism and the statistics each
workload is meant to have (span lengths, anchor share, planted rank)."""
import numpy as np
import pytest
import torch

import synth
from oracle import sekv_oracle as O


def test_surprisal_deterministic_and_positive():
    s = synth.spec("single_layer_32k")
    a, b = synth.surprisal(s, 0), synth.surprisal(s, 0)
    assert a.dtype == np.float32 and np.array_equal(a, b)
    assert np.all(a > 0)
    assert not np.array_equal(a, synth.surprisal(s.replace(cfg_id=4), 0))


@pytest.mark.parametrize("name,alpha,mean_lo,mean_hi,anc_lo,anc_hi", [
    ("tiny", 1.0, 8, 16, 0.05, 0.12),
    ("single_layer_32k", 1.5, 50, 80, 0.02, 0.04),
    ("layers32_128k", 1.5, 50, 80, 0.015, 0.025),
    ("gqa_batch8_128k", 1.0, 28, 45, 0.025, 0.04),
    ("prefill_builder_128k", 0.5, 12, 20, 0.05, 0.08),
    ("prefill_builder_128k", 1.0, 50, 80, 0.015, 0.025),
    ("prefill_builder_128k", 2.0, 400, 650, 0.004, 0.008),
])
def test_span_statistics(name, alpha, mean_lo, mean_hi, anc_lo, anc_hi):
    s = synth.spec(name)
    seg = O.segment(synth.surprisal(s, 0), alpha, s.w)
    assert mean_lo <= seg.mcount.mean() <= mean_hi
    assert anc_lo <= seg.anchors.size / s.n <= anc_hi


def test_gqa_sequences_differ():
    s = synth.spec("gqa_batch8_128k")
    H = synth.surprisal_batch(s)
    assert H.shape == (8, s.n)
    assert len({H[b].tobytes() for b in range(8)}) == 8


def test_kv_planted_low_rank_and_deterministic():
    s = synth.spec("tiny")
    K, V = synth.kv_head(s, 0, 0, 0)
    K2, _ = synth.kv_head(s, 0, 0, 0)
    assert K.dtype == torch.float32 and torch.equal(K, K2)
    st = synth.planted_starts(s, 0)
    ends = np.concatenate([st[1:], [s.n]])
    i = int(np.argmax(ends - st))
    X = K[st[i]:ends[i]].double().numpy()
    sv = np.linalg.svd(X - X.mean(0), compute_uv=False)
    # planted rank rho = 4 plus isotropic noise of std 0.05
    assert sv[3] > 20 * sv[4]
    assert sv[4] < 0.05 * np.sqrt(X.shape[0]) * 3


def test_bf16_and_needle():
    s = synth.spec("single_layer_32k", n=4096, w=128)
    K, V = synth.kv_head(s, 0, 0, 0)
    assert K.dtype == torch.bfloat16 and K.shape == (4096, 128)
    a, e = synth.needle_segment(s, 0, 0)
    assert e - a >= s.needle_min_len and e <= s.n - s.w
    q = synth.queries(s, 0, 0)
    assert q.shape == (1, 32, 128) and q.dtype == torch.float32
    u = synth.workloads.needle_direction(s, 0, 0, 0)
    # needle heads (g % 4 == 0) get a large component along u; others do not
    assert float(q[0, 0] @ u) > 8.0
    assert abs(float(q[0, 1] @ synth.workloads.needle_direction(s, 0, 0, 1))) < 5.0


def test_zoom_targets():
    s = synth.spec("layers32_128k")
    ret = synth.retrieval_heads(s)
    assert len(ret) == round(0.2 * 32 * 32)
    assert all(8 <= l <= 27 for l, _ in ret)
    rates = np.stack([synth.zoom_targets(s, l) for l in range(s.L)])
    assert rates.min() >= 0.005 - 1e-12 and rates.max() <= 0.2 + 1e-12
    assert 0.01 < rates.mean() < 0.04
