"""The host-CPU integer-SIMD W4A8 path (qgemm_w4a8_grouped_host) against the
CPU oracle: it needs no GPU, so these run with the CPU suite."""
import numpy as np
import pytest

import block_quantized_integer_amd as bqi
import oracle
import workloads as W
from helpers import assert_within_bound


def _avx2():
    try:
        flags = open("/proc/cpuinfo").read()
    except OSError:
        return False
    return " avx2" in flags and " fma" in flags


pytestmark = pytest.mark.skipif(not _avx2(), reason="host CPU without AVX2/FMA")


@pytest.mark.parametrize("T,tk,E,K,N", [(1, 8, 128, 2048, 768), (4, 8, 16, 256, 130),
                                        (37, 4, 8, 128, 96), (3, 2, 5, 96, 33)])
def test_host_w4a8_matches_oracle(T, tk, E, K, N):
    g = np.random.default_rng(T * 100 + K)
    qa = W.random_int8("moe", 720, (T, K), seed=K)
    da = W.random_scales("moe", 721, (T, K // 32), seed=K)
    ids = W.topk_ids(T, tk, E, seed=T)
    packed = g.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    wsc = W.random_scales("moe", 722, (E, N, K // 32), seed=K)
    y = bqi.qgemm_w4a8_grouped_host(qa, da, ids, packed, wsc)
    yr, asum = oracle.qgemm_w4a8_grouped(qa, da, ids, packed, wsc, nthreads=4)
    assert_within_bound(y, yr, asum, K // 32, "host T=%d" % T)


def test_host_w4a8_exact_block_dots_and_thread_independence():
    """Power-of-two scales and one nonzero block per activation row make every
    output exactly 2^e * P, so the int32 block dots are checked bit for bit;
    the result must not depend on the thread count."""
    g = np.random.default_rng(5)
    T, tk, E, K, N = 6, 3, 4, 128, 20
    qa = np.zeros((T, K), np.int8)
    for t in range(T):
        b = t % (K // 32)
        qa[t, 32 * b: 32 * b + 32] = g.integers(-128, 128, 32)
    da = np.full((T, K // 32), 0x3c00, np.uint16)          # 1.0
    wsc = np.full((E, N, K // 32), 0x4400, np.uint16)      # 4.0
    packed = g.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    ids = g.integers(0, E, (T, tk)).astype(np.int32)
    ids[1, 2] = -1
    y1 = bqi.qgemm_w4a8_grouped_host(qa, da, ids, packed, wsc, nthreads=1)
    y7 = bqi.qgemm_w4a8_grouped_host(qa, da, ids, packed, wsc, nthreads=7)
    assert np.array_equal(y1.view(np.uint32), y7.view(np.uint32))
    codes = oracle.unpack_w4(packed).astype(np.int64) - 8
    for t in range(T):
        for j in range(tk):
            e = ids[t, j]
            if e < 0:
                assert np.all(y1[t, j] == 0)
                continue
            P = codes[e] @ qa[t].astype(np.int64)
            assert np.array_equal(y1[t, j], (4.0 * P).astype(np.float32))
