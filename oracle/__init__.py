"""Plain CPU reference ("oracle") for block-quantized integer GEMM/GEMV.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The library (``block_quantized_integer_amd``) never imports, links or
executes anything here, and this package imports nothing from it.

The arithmetic lives in ``bq_oracle.c`` (plain C11, gcc, no fast-math); this
module only loads ``liboracle.so`` and marshals numpy arrays.  What each
function computes, and which page passage it follows, is documented in
``bq_oracle.h``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
QK = 32

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, IEEE arithmetic)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    src = os.path.join(_HERE, "bq_oracle.c")
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O3", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    I64 = C.c_int64
    sig = {
        "orc_f32_to_f16": (C.c_uint16, [C.c_float]),
        "orc_f16_to_f32": (C.c_float, [C.c_uint16]),
        "orc_f32_to_f16_array": (None, [P, I64, P]),
        "orc_f16_to_f32_array": (None, [P, I64, P]),
        "orc_quantize_q8_0_f32": (None, [P, I64, I64, I64, P, P]),
        "orc_quantize_q8_0_f16": (None, [P, I64, I64, I64, P, P]),
        "orc_quantize_w4": (None, [P, I64, I64, P, P]),
        "orc_unpack_w4": (None, [P, I64, I64, P]),
        "orc_pack_w4": (None, [P, I64, I64, P]),
        "orc_block_dots": (None, [P, I64, P, I64, I64, P]),
        "orc_qgemm_q8_0": (None, [P, P, I64, P, P, I64, I64, P, P, C.c_int]),
        "orc_qgemm_q8_0_at": (None, [P, P, I64, P, P, I64, I64, P, P, I64, P, P]),
        "orc_route_topk": (I64, [P, I64, I64, I64, P, P, P]),
        "orc_qgemm_w4a8_grouped": (None, [P, P, I64, P, I64, P, P, I64, I64, I64,
                                          P, P, C.c_int]),
        "orc_qgemm_w4a8_grouped_at": (None, [P, P, I64, P, I64, P, P, I64, I64,
                                             I64, P, P, I64, P, P]),
        "orc_moe_combine": (None, [P, P, I64, I64, I64, P, P]),
        "orc_gguf_q8_0_to_planar": (None, [P, I64, I64, P, P]),
        "orc_gguf_q4_0_to_planar": (None, [P, I64, I64, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return a


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# ---- fp16 -------------------------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    """fp32 -> fp16 bits, round to nearest even (oracle's own routine)."""
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_f16_array(_p(x), x.size, _p(out))
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(np.asarray(h, dtype=np.uint16), np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().orc_f16_to_f32_array(_p(h), h.size, _p(out))
    return out


# ---- quantizers ---------------------------------------------------------------

def quantize_q8_0(x: np.ndarray, k: int | None = None):
    """Q8_0 quantize rows of x (fp32, or fp16 given as np.float16).

    Returns (q int8 [rows][k], d uint16 fp16-bits [rows][k/32]).  ``k`` may be
    smaller than the row length (the remaining columns are padding, like ldx).
    """
    x = np.ascontiguousarray(x)
    rows, ldx = x.shape
    k = ldx if k is None else k
    assert k % QK == 0 and k <= ldx
    q = np.empty((rows, k), np.int8)
    d = np.empty((rows, k // QK), np.uint16)
    lib = _load()
    if x.dtype == np.float32:
        lib.orc_quantize_q8_0_f32(_p(x), rows, k, ldx, _p(q), _p(d))
    elif x.dtype == np.float16:
        xb = x.view(np.uint16)
        lib.orc_quantize_q8_0_f16(_p(xb), rows, k, ldx, _p(q), _p(d))
    else:
        raise TypeError(x.dtype)
    return q, d


def quantize_w4(w: np.ndarray):
    """4-bit group quantize (test data): returns (packed uint8 [rows][k/2], d)."""
    w = _c(w, np.float32)
    rows, k = w.shape
    assert k % QK == 0
    p = np.empty((rows, k // 2), np.uint8)
    d = np.empty((rows, k // QK), np.uint16)
    _load().orc_quantize_w4(_p(w), rows, k, _p(p), _p(d))
    return p, d


def unpack_w4(packed: np.ndarray) -> np.ndarray:
    packed = _c(packed, np.uint8)
    shp = packed.shape
    rows = int(np.prod(shp[:-1]))
    k = shp[-1] * 2
    codes = np.empty(shp[:-1] + (k,), np.uint8)
    _load().orc_unpack_w4(_p(packed), rows, k, _p(codes))
    return codes


def pack_w4(codes: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    shp = codes.shape
    rows = int(np.prod(shp[:-1]))
    k = shp[-1]
    packed = np.empty(shp[:-1] + (k // 2,), np.uint8)
    _load().orc_pack_w4(_p(codes), rows, k, _p(packed))
    return packed


# ---- block dots / GEMMs ----------------------------------------------------------

def block_dots(aq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    aq = _c(aq, np.int8)
    wq = _c(wq, np.int8)
    m, k = aq.shape
    n, k2 = wq.shape
    assert k == k2 and k % QK == 0
    P = np.empty((m, n, k // QK), np.int32)
    _load().orc_block_dots(_p(aq), m, _p(wq), n, k, _p(P))
    return P


def qgemm_q8_0(aq, ad, wq, wd, nthreads: int = 1):
    """Returns (y fp64 [m][n], asum fp64 [m][n])."""
    aq = _c(aq, np.int8)
    ad = _c(ad, np.uint16)
    wq = _c(wq, np.int8)
    wd = _c(wd, np.uint16)
    m, k = aq.shape
    n = wq.shape[0]
    assert wq.shape[1] == k and ad.shape == (m, k // QK) and wd.shape == (n, k // QK)
    y = np.empty((m, n), np.float64)
    a = np.empty((m, n), np.float64)
    _load().orc_qgemm_q8_0(_p(aq), _p(ad), m, _p(wq), _p(wd), n, k, _p(y), _p(a),
                           int(nthreads))
    return y, a


def qgemm_q8_0_at(aq, ad, wq, wd, mi, nj):
    aq = _c(aq, np.int8)
    ad = _c(ad, np.uint16)
    wq = _c(wq, np.int8)
    wd = _c(wd, np.uint16)
    m, k = aq.shape
    n = wq.shape[0]
    mi = _c(np.asarray(mi, np.int64), np.int64)
    nj = _c(np.asarray(nj, np.int64), np.int64)
    assert mi.shape == nj.shape
    assert (mi >= 0).all() and (mi < m).all() and (nj >= 0).all() and (nj < n).all()
    y = np.empty(mi.shape, np.float64)
    a = np.empty(mi.shape, np.float64)
    _load().orc_qgemm_q8_0_at(_p(aq), _p(ad), m, _p(wq), _p(wd), n, k, _p(mi),
                              _p(nj), mi.size, _p(y), _p(a))
    return y, a


def route_topk(ids: np.ndarray, n_experts: int):
    """Returns (counts int32 [E], offsets int32 [E+1], rows int32 [valid], n_invalid)."""
    ids = _c(ids, np.int32)
    T, top_k = ids.shape
    counts = np.empty(n_experts, np.int32)
    offsets = np.empty(n_experts + 1, np.int32)
    rows = np.empty(T * top_k, np.int32)
    inv = _load().orc_route_topk(_p(ids), T, top_k, n_experts, _p(counts),
                                 _p(offsets), _p(rows))
    return counts, offsets, rows[: T * top_k - inv].copy(), int(inv)


def qgemm_w4a8_grouped(aq, ad, ids, wq4, wd, nthreads: int = 1):
    """Returns (y fp64 [T][top_k][n], asum fp64 [T][top_k][n])."""
    aq = _c(aq, np.int8)
    ad = _c(ad, np.uint16)
    ids = _c(ids, np.int32)
    wq4 = _c(wq4, np.uint8)
    wd = _c(wd, np.uint16)
    T, k = aq.shape
    top_k = ids.shape[1]
    E, n, kh = wq4.shape
    assert kh * 2 == k and ids.shape[0] == T and wd.shape == (E, n, k // QK)
    y = np.empty((T, top_k, n), np.float64)
    a = np.empty((T, top_k, n), np.float64)
    _load().orc_qgemm_w4a8_grouped(_p(aq), _p(ad), T, _p(ids), top_k, _p(wq4),
                                   _p(wd), E, n, k, _p(y), _p(a), int(nthreads))
    return y, a


def qgemm_w4a8_grouped_at(aq, ad, ids, wq4, wd, ri, cj):
    aq = _c(aq, np.int8)
    ad = _c(ad, np.uint16)
    ids = _c(ids, np.int32)
    wq4 = _c(wq4, np.uint8)
    wd = _c(wd, np.uint16)
    T, k = aq.shape
    top_k = ids.shape[1]
    E, n, _ = wq4.shape
    ri = _c(np.asarray(ri, np.int64), np.int64)
    cj = _c(np.asarray(cj, np.int64), np.int64)
    assert (ri >= 0).all() and (ri < T * top_k).all() and (cj >= 0).all() and (cj < n).all()
    y = np.empty(ri.shape, np.float64)
    a = np.empty(ri.shape, np.float64)
    _load().orc_qgemm_w4a8_grouped_at(_p(aq), _p(ad), T, _p(ids), top_k, _p(wq4),
                                      _p(wd), E, n, k, _p(ri), _p(cj), ri.size,
                                      _p(y), _p(a))
    return y, a


def moe_combine(y: np.ndarray, p: np.ndarray):
    """out[t][c] = sum_j p[t][j] * y[t][j][c] in fp64 (exact products, slot
    order), with the tolerance scale sum_j |p y|.  y fp32 [T][top_k][n], p fp32
    [T][top_k].  Returns (out, asum) fp64 [T][n].  See bq_oracle.h."""
    y = np.ascontiguousarray(y, np.float32)
    p = np.ascontiguousarray(p, np.float32)
    T, top_k, n = y.shape
    assert p.shape == (T, top_k)
    out = np.empty((T, n), np.float64)
    asum = np.empty((T, n), np.float64)
    _load().orc_moe_combine(_p(y), _p(p), T, top_k, n, _p(out), _p(asum))
    return out, asum


def gguf_q8_0_to_planar(blocks: np.ndarray, rows: int, k: int):
    """Split a GGUF Q8_0 block array (uint8, rows*k/32*34 bytes) into codes
    int8 [rows][k] and scale bits uint16 [rows][k/32]."""
    blocks = np.ascontiguousarray(blocks, np.uint8)
    assert k % QK == 0 and blocks.size == rows * (k // QK) * 34
    q = np.empty((rows, k), np.int8)
    d = np.empty((rows, k // QK), np.uint16)
    _load().orc_gguf_q8_0_to_planar(_p(blocks), rows, k, _p(q), _p(d))
    return q, d


def gguf_q4_0_to_planar(blocks: np.ndarray, rows: int, k: int):
    """Split a GGUF Q4_0 block array (uint8, rows*k/32*18 bytes) into packed
    codes uint8 [rows][k/2] and scale bits uint16 [rows][k/32]."""
    blocks = np.ascontiguousarray(blocks, np.uint8)
    assert k % QK == 0 and blocks.size == rows * (k // QK) * 18
    packed = np.empty((rows, k // 2), np.uint8)
    d = np.empty((rows, k // QK), np.uint16)
    _load().orc_gguf_q4_0_to_planar(_p(blocks), rows, k, _p(packed), _p(d))
    return packed, d
