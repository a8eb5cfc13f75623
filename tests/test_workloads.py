"""Host-side checks of the synthetic workload recipes (workloads.py) and of the
bench's traffic-record lookup.  CPU only."""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import workloads as W  # noqa: E402


def test_streams_are_seeded_and_independent():
    a = W.normal("prefill", W.T_ACT, (64,), seed=0)
    assert np.array_equal(a, W.normal("prefill", W.T_ACT, (64,), seed=0))
    assert not np.array_equal(a, W.normal("prefill", W.T_WEIGHT, (64,), seed=0))
    assert not np.array_equal(a, W.normal("long", W.T_ACT, (64,), seed=0))
    assert not np.array_equal(a, W.normal("prefill", W.T_ACT, (64,), seed=1))


def test_router_draws_distinct_experts_per_token():
    m = W.MOE
    ids = W.topk_ids(m.tokens, m.top_k, m.experts)
    assert ids.shape == (m.tokens, m.top_k) and ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < m.experts
    assert all(len(set(row)) == m.top_k for row in ids)
    counts = np.bincount(ids.ravel(), minlength=m.experts)
    # every expert is routed to; rows per expert ~ Binomial(947, 1/16):
    # mean 59.2, sd 7.45, so 40 .. 85 holds with wide margin at this seed
    assert counts.sum() == m.tokens * m.top_k and counts.min() > 0
    assert 40 <= counts.min() and counts.max() <= 85
    assert np.array_equal(ids, W.topk_ids(m.tokens, m.top_k, m.experts))


def test_long_prefill_outlier_columns():
    k = W.LONG.k
    cols = W.outlier_columns(k)
    assert len(cols) == k // 100 == 51 and len(set(cols)) == 51
    assert cols.min() >= 0 and cols.max() < k and np.all(np.diff(cols) > 0)
    a = W.activations("long", 256, k)
    scale = np.median(np.abs(a), axis=0)
    others = np.setdiff1d(np.arange(k), cols)
    # the scaled columns sit ~20x above the rest (Student-t(3) medians)
    assert np.median(scale[cols]) > 15 * np.median(scale[others])


def test_random_scales_are_normal_range_fp16():
    d = W.random_scales(0, 1, (4096,))
    f = d.view(np.float16).astype(np.float64)
    assert np.all(np.isfinite(f)) and np.all(f > 0)
    assert f.min() >= 2.0 ** -12 and f.max() < 2.0 ** -2 * 2
    assert np.all((d & 0x7C00) != 0)  # no subnormals


def test_traffic_record_goes_stale_with_its_sources(tmp_path, monkeypatch):
    import bench
    key = "k_example decode"
    files = ["quantize.hip"]
    rec = {"hbm_bytes_per_launch": 12345, "sources": files,
           "sources_sha256": bench.sources_sha256(files)}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({key: rec}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic(key) == 12345
    assert bench.traffic("absent key") is None
    rec["sources_sha256"] = "0" * 64
    path.write_text(json.dumps({key: rec}))
    assert bench.traffic(key) is None
