"""Host-side logic of bench.py (CPU only): the CPU-oracle lines, run on
scaled-down shapes, come out under exactly the workload names that the GPU
lines carry (the oracle's figures attach to the GPU lines by name), each with
a positive figure and the thread count the oracle splits its rows over."""
import types

import workloads as W

import bench


def small_workloads():
    G, M = W.GemmShape, W.MoeShape
    fake = types.SimpleNamespace()
    fake.SMALL = G("small", 16, 256, 512)
    fake.DECODE = [G("decode_m%d" % m, m, 512, 256) for m in (1, 4, 16)]
    fake.PREFILL = G("prefill", 64, 512, 256)
    fake.PREFILL_SHORT = G("prefill_short", 32, 512, 256)
    fake.LONG = G("long", 128, 512, 256)
    fake.MOE = M("moe", 120, 8, 16, 256, 64)
    for f in ("activations", "weights", "topk_ids", "random_w4_codes", "random_int8",
              "random_scales", "outlier_columns"):
        setattr(fake, f, getattr(W, f))
    return fake


def test_cpu_oracle_lines_match_gpu_line_names():
    fw = small_workloads()
    legs = bench.cpu_oracle_lines(fw, time_scale=0.01)
    m = fw.MOE
    want = {bench.name_small(fw.SMALL)}
    want |= {bench.name_decode(s) for s in fw.DECODE[1:]}
    want |= {bench.name_gemm(n, s) for n, s in (("prefill", fw.PREFILL),
                                                 ("prefill_short", fw.PREFILL_SHORT),
                                                 ("long", fw.LONG))}
    want.add(bench.name_moe(m))
    for T in (1, 4, 16):
        active = len(set(W.topk_ids(T, m.top_k, m.experts, seed=T).ravel().tolist()))
        want.add(bench.name_moe_decode(m, T, active))
    assert set(legs) == want
    for name, rec in legs.items():
        assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["cores"] >= 1, name
        assert rec["sample"], name
