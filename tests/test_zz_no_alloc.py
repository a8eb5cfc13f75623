"""The allocation-free grouped W4A8 entry point (qgemm_w4a8_grouped_noalloc,
called through the C ABI) against the workspace entry point
(qgemm_w4a8_grouped) on the same inputs: bit-identical outputs, on two calls
in a row, the second with a smaller input, so that the second runs over what
the first left in the library's array (the last pair past 8192 routed rows,
where the routing pass works through its ids in chunks).  Also the decode size
(no workspace used) and a problem the array cannot hold (rejected, nothing
written)."""
import ctypes as C

import numpy as np
import pytest

import workloads as W
from helpers import dev_tensor, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_quantized_integer_amd as bqi  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bqi.lib()
    yield
    torch.cuda.synchronize()


def inputs(T, top_k, E, K, N, seed):
    qa = dev_tensor(W.random_int8("moe", 750, (T, K), seed=seed))
    da = dev_tensor(W.random_scales("moe", 751, (T, K // 32), seed=seed))
    ids_np = W.topk_ids(T, top_k, E, seed=seed)
    ids_np[::97, 0] = -1          # a few invalid ids: zero rows
    ids = dev_tensor(ids_np)
    packed, wsc = W.random_w4_codes(E, N, K, seed=seed)
    return qa, da, ids, dev_tensor(packed), dev_tensor(wsc)


def noalloc_call(qa, da, ids, wq4, wd, y):
    """Straight through the C ABI (ctypes), on the current stream."""
    T, K = qa.shape
    top_k = ids.shape[1]
    E, N, _ = wq4.shape
    P = C.c_void_p
    return bqi.lib().qgemm_w4a8_grouped_noalloc(
        P(qa.data_ptr()), P(da.data_ptr()), T, P(ids.data_ptr()), top_k, P(wq4.data_ptr()),
        P(wd.data_ptr()), E, N, K, P(y.data_ptr()),
        P(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("first,second", [
    ((947, 8, 128, 2048, 768), (300, 8, 128, 2048, 768)),   # the MoE workload, then fewer tokens
    ((600, 4, 16, 512, 200), (150, 2, 16, 512, 200)),       # fewer slots, ragged N
    # past 8192 routed rows: the routing pass in chunks of ids
    ((1300, 8, 64, 256, 96), (1100, 8, 64, 256, 96))])
def test_noalloc_matches_workspace_entry_point(first, second):
    for i, shape in enumerate((first, second)):
        T, top_k, E, K, N = shape
        log("noalloc call %d: T=%d top_k=%d E=%d K=%d N=%d" % (i, T, top_k, E, K, N))
        qa, da, ids, wq4, wd = inputs(T, top_k, E, K, N, seed=31 + i)
        y_ref = bqi.qgemm_w4a8_grouped(qa, da, ids, wq4, wd)
        y = torch.full((T, top_k, N), float("nan"), device="cuda:0")
        assert noalloc_call(qa, da, ids, wq4, wd, y) == bqi.BQI_OK
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), "call %d differs" % i


def test_noalloc_decode_size_and_rejection():
    # 16 tokens x top-8: the GEMV path, which needs no workspace
    qa, da, ids, wq4, wd = inputs(16, 8, 128, 2048, 768, seed=41)
    y_ref = bqi.qgemm_w4a8_grouped(qa, da, ids, wq4, wd)
    y = torch.empty_like(y_ref)
    assert noalloc_call(qa, da, ids, wq4, wd, y) == bqi.BQI_OK
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    # a workspace larger than the array (4 bytes per routed row: 2^22 routed
    # rows): rejected before any launch, y untouched
    T, top_k, E, K, N = 1 << 19, 8, 4, 32, 1
    need = bqi.workspace_size(T, top_k, E, K)
    assert need > bqi.NOALLOC_SCRATCH_BYTES
    qa = torch.zeros((T, K), dtype=torch.int8, device="cuda:0")
    da = torch.zeros((T, K // 32), dtype=torch.int16, device="cuda:0")
    ids = torch.zeros((T, top_k), dtype=torch.int32, device="cuda:0")
    wq4 = torch.zeros((E, N, K // 2), dtype=torch.uint8, device="cuda:0")
    wd = torch.zeros((E, N, K // 32), dtype=torch.int16, device="cuda:0")
    y = torch.full((T, top_k, N), 3.0, device="cuda:0")
    assert noalloc_call(qa, da, ids, wq4, wd, y) == bqi.BQI_ESHAPE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
