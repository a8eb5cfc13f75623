"""block_quantized_integer_amd -- block-quantized integer GEMM/GEMV on MI355X.

Thin Python binding over the C ABI of ``libbqi.so`` (``include/bqi.h``).  The
functions here only check tensor dtypes/shapes/devices and pass raw pointers
and the current HIP stream; every step of the computation runs in the
library's gfx950 kernels.  There is no CPU fallback: if ``libbqi.so`` is
missing, importing the library functions raises.

Entry points (same names as the C ABI):
  quantize_q8_0(x)                       -> (q int8 [R][K], d uint16-as-int16 fp16 bits [R][K/32])
  qgemm_q8_0(aq, ad, wq, wd)             -> y fp32 [M][N] = A W^T
  quantize_qgemm_q8_0(x, wq, wd)         -> (y, q, d): both of the above, fused for decode
  route_topk(topk_ids, n_experts)        -> (counts, offsets, rows)
  qgemm_w4a8_grouped(aq, ad, topk_ids, wq4, wd) -> y fp32 [T][top_k][N]

fp16 scale bit patterns travel as torch.int16 tensors (torch has no uint16
arithmetic on GPU); only their bits matter.

Every wrapper takes an optional `stream` (a torch.cuda.Stream or a raw
hipStream_t handle); without one it uses the current stream.  Outputs and
workspaces that a wrapper allocates are allocated on that same stream.
"""
from __future__ import annotations

import ctypes as C
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libbqi.so")

BQI_OK, BQI_EINVAL, BQI_ESHAPE, BQI_EALIGN, BQI_EHIP, BQI_ENOTSUP = 0, -1, -2, -3, -4, -5
BQI_F32, BQI_F16 = 0, 1

SYMBOLS = ("bqi_status_string", "bqi_abi_version", "quantize_q8_0", "qgemm_q8_0",
           "quantize_qgemm_q8_0", "route_topk", "qgemm_w4a8_grouped_workspace_size",
           "qgemm_w4a8_grouped", "moe_combine_f32", "gguf_q8_0_to_planar",
           "gguf_q4_0_to_planar", "qgemm_w4a8_grouped_host", "qgemm_w4a8_grouped_noalloc")

_lib = None


class BqiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, lib().bqi_status_string(status).decode()))


def lib() -> C.CDLL:
    """Load libbqi.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbqi.so not found at %s; build it with "
                          "`python -m block_quantized_integer_amd.build`" % LIB_PATH)
    L = C.CDLL(LIB_PATH)
    P, I64, I32 = C.c_void_p, C.c_int64, C.c_int
    L.bqi_status_string.restype = C.c_char_p
    L.bqi_status_string.argtypes = [I32]
    L.bqi_abi_version.restype = I32
    L.bqi_abi_version.argtypes = []
    L.quantize_q8_0.restype = I32
    L.quantize_q8_0.argtypes = [P, I32, I64, I64, I64, P, P, P]
    L.qgemm_q8_0.restype = I32
    L.qgemm_q8_0.argtypes = [P, P, I64, P, P, I64, I64, P, P]
    L.quantize_qgemm_q8_0.restype = I32
    L.quantize_qgemm_q8_0.argtypes = [P, I32, I64, I64, I64, P, P, I64, P, P, P, P]
    L.moe_combine_f32.restype = I32
    L.moe_combine_f32.argtypes = [P, P, I64, I64, I64, P, P]
    L.gguf_q8_0_to_planar.restype = I32
    L.gguf_q8_0_to_planar.argtypes = [P, I64, I64, P, P, P]
    L.gguf_q4_0_to_planar.restype = I32
    L.gguf_q4_0_to_planar.argtypes = [P, I64, I64, P, P, P]
    L.qgemm_w4a8_grouped_host.restype = I32
    L.qgemm_w4a8_grouped_host.argtypes = [P, P, I64, P, I64, P, P, I64, I64, I64, P, I32]
    L.route_topk.restype = I32
    L.route_topk.argtypes = [P, I64, I64, I64, P, P, P, P]
    L.qgemm_w4a8_grouped_workspace_size.restype = C.c_size_t
    L.qgemm_w4a8_grouped_workspace_size.argtypes = [I64, I64, I64, I64]
    L.qgemm_w4a8_grouped.restype = I32
    L.qgemm_w4a8_grouped.argtypes = [P, P, I64, P, I64, P, P, I64, I64, I64, P, P,
                                     C.c_size_t, P]
    L.qgemm_w4a8_grouped_noalloc.restype = I32
    L.qgemm_w4a8_grouped_noalloc.argtypes = [P, P, I64, P, I64, P, P, I64, I64, I64, P, P]
    _lib = L
    return L


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _on(stream, device):
    """Context in which the wrappers allocate their outputs and workspaces:
    the caller's stream when one is given, so that torch's caching allocator
    ties those blocks to the stream the kernels run on (a block freed when a
    wrapper returns is then reused only by work ordered after the kernels).
    A raw hipStream_t handle is wrapped as an external stream of `device`."""
    torch = _torch()
    if stream is None:
        import contextlib
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        stream = torch.cuda.ExternalStream(handle, device=device)
    return torch.cuda.stream(stream)


def _check(t, dtype, ndim, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %d" % (name, ndim, t.dim()))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else C.c_void_p(0)


def _raise(st, where):
    if st != BQI_OK:
        raise BqiError(st, where)


def quantize_q8_0(x, q=None, d=None, stream=None):
    """Q8_0-quantize the rows of x (fp32 or fp16, [R][ldx] with row stride
    ldx >= K; pass a column slice x[:, :K] of a contiguous tensor to quantize
    only the first K columns).  Returns (q int8 [R][K], d int16 [R][K/32])."""
    torch = _torch()
    if x.dtype not in (torch.float32, torch.float16):
        raise TypeError("x must be float32 or float16")
    if x.dim() != 2 or x.stride(1) != 1 or not x.is_cuda:
        raise ValueError("x must be a 2-D GPU tensor with unit column stride")
    R, K = x.shape
    ldx = x.stride(0) if R > 1 else K
    with _on(stream, x.device):
        if q is None:
            q = torch.empty((R, K), dtype=torch.int8, device=x.device)
        if d is None:
            d = torch.empty((R, K // 32), dtype=torch.int16, device=x.device)
    _check(q, torch.int8, 2, "q")
    _check(d, torch.int16, 2, "d")
    dt = BQI_F32 if x.dtype == torch.float32 else BQI_F16
    st = lib().quantize_q8_0(_ptr(x), dt, R, K, ldx, _ptr(q), _ptr(d), _stream(stream))
    _raise(st, "quantize_q8_0")
    return q, d


def qgemm_q8_0(aq, ad, wq, wd, y=None, stream=None):
    """y[M][N] = A W^T for Q8_0 activations (aq, ad) and Q8_0 weights (wq, wd)."""
    torch = _torch()
    _check(aq, torch.int8, 2, "aq")
    _check(ad, torch.int16, 2, "ad")
    _check(wq, torch.int8, 2, "wq")
    _check(wd, torch.int16, 2, "wd")
    M, K = aq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or tuple(ad.shape) != (M, K // 32) or tuple(wd.shape) != (N, K // 32):
        raise ValueError("shape mismatch: aq %s ad %s wq %s wd %s" % (
            tuple(aq.shape), tuple(ad.shape), tuple(wq.shape), tuple(wd.shape)))
    if y is None:
        with _on(stream, aq.device):
            y = torch.empty((M, N), dtype=torch.float32, device=aq.device)
    _check(y, torch.float32, 2, "y")
    st = lib().qgemm_q8_0(_ptr(aq), _ptr(ad), M, _ptr(wq), _ptr(wd), N, K, _ptr(y),
                          _stream(stream))
    _raise(st, "qgemm_q8_0")
    return y


def quantize_qgemm_q8_0(x, wq, wd, y=None, q=None, d=None, stream=None):
    """Quantize the rows of x (fp32 or fp16, unit column stride) to Q8_0 and
    multiply by the Q8_0 weights: returns (y fp32 [M][N], q int8 [M][K],
    d int16 [M][K/32]), identical to quantize_q8_0 followed by qgemm_q8_0 (one
    launch for decode-sized M)."""
    torch = _torch()
    if x.dtype not in (torch.float32, torch.float16):
        raise TypeError("x must be float32 or float16")
    if x.dim() != 2 or x.stride(1) != 1 or not x.is_cuda:
        raise ValueError("x must be a 2-D GPU tensor with unit column stride")
    _check(wq, torch.int8, 2, "wq")
    _check(wd, torch.int16, 2, "wd")
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K or tuple(wd.shape) != (N, K // 32):
        raise ValueError("shape mismatch: x %s wq %s wd %s" % (
            tuple(x.shape), tuple(wq.shape), tuple(wd.shape)))
    ldx = x.stride(0) if M > 1 else K
    with _on(stream, x.device):
        if y is None:
            y = torch.empty((M, N), dtype=torch.float32, device=x.device)
        if q is None:
            q = torch.empty((M, K), dtype=torch.int8, device=x.device)
        if d is None:
            d = torch.empty((M, K // 32), dtype=torch.int16, device=x.device)
    _check(y, torch.float32, 2, "y")
    _check(q, torch.int8, 2, "q")
    _check(d, torch.int16, 2, "d")
    dt = BQI_F32 if x.dtype == torch.float32 else BQI_F16
    st = lib().quantize_qgemm_q8_0(_ptr(x), dt, M, K, ldx, _ptr(wq), _ptr(wd), N, _ptr(y),
                                   _ptr(q), _ptr(d), _stream(stream))
    _raise(st, "quantize_qgemm_q8_0")
    return y, q, d


def route_topk(topk_ids, n_experts, counts=None, offsets=None, rows=None, stream=None):
    """Group routed rows by expert.  Returns (counts [E], offsets [E+1], rows [T*top_k])."""
    torch = _torch()
    _check(topk_ids, torch.int32, 2, "topk_ids")
    T, top_k = topk_ids.shape
    dev = topk_ids.device
    with _on(stream, dev):
        if counts is None:
            counts = torch.empty(n_experts, dtype=torch.int32, device=dev)
        if offsets is None:
            offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
        if rows is None:
            rows = torch.empty(max(1, T * top_k), dtype=torch.int32, device=dev)
    st = lib().route_topk(_ptr(topk_ids), T, top_k, n_experts, _ptr(counts), _ptr(offsets),
                          _ptr(rows), _stream(stream))
    _raise(st, "route_topk")
    return counts, offsets, rows


def workspace_size(n_tokens, top_k, n_experts, k) -> int:
    return int(lib().qgemm_w4a8_grouped_workspace_size(n_tokens, top_k, n_experts, k))


def qgemm_w4a8_grouped(aq, ad, topk_ids, wq4, wd, y=None, workspace=None, stream=None):
    """Grouped W4A8: y[T][top_k][N] for 4-bit expert weights wq4 [E][N][K/2]
    (uint8), wd [E][N][K/32] (int16 fp16 bits) and Q8_0 activations."""
    torch = _torch()
    _check(aq, torch.int8, 2, "aq")
    _check(ad, torch.int16, 2, "ad")
    _check(topk_ids, torch.int32, 2, "topk_ids")
    _check(wq4, torch.uint8, 3, "wq4")
    _check(wd, torch.int16, 3, "wd")
    T, K = aq.shape
    top_k = topk_ids.shape[1]
    E, N, KH = wq4.shape
    if KH * 2 != K or tuple(ad.shape) != (T, K // 32) or topk_ids.shape[0] != T \
            or tuple(wd.shape) != (E, N, K // 32):
        raise ValueError("shape mismatch")
    need = workspace_size(T, top_k, E, K)
    with _on(stream, aq.device):
        # the workspace is freed when this function returns: allocated on the
        # kernels' stream, it is not handed out again before they finish
        if y is None:
            y = torch.empty((T, top_k, N), dtype=torch.float32, device=aq.device)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=aq.device)
    _check(y, torch.float32, 3, "y")
    if workspace.numel() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    st = lib().qgemm_w4a8_grouped(_ptr(aq), _ptr(ad), T, _ptr(topk_ids), top_k, _ptr(wq4),
                                  _ptr(wd), E, N, K, _ptr(y), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    _raise(st, "qgemm_w4a8_grouped")
    return y


NOALLOC_SCRATCH_BYTES = 16 << 20  # BQI_NOALLOC_SCRATCH_BYTES


def qgemm_w4a8_grouped_noalloc(aq, ad, topk_ids, wq4, wd, y, stream=None):
    """qgemm_w4a8_grouped with the library's own per-GPU workspace array: the
    library allocates nothing (y must be given).  Calls that overlap on one GPU
    race on that array."""
    torch = _torch()
    _check(aq, torch.int8, 2, "aq")
    _check(ad, torch.int16, 2, "ad")
    _check(topk_ids, torch.int32, 2, "topk_ids")
    _check(wq4, torch.uint8, 3, "wq4")
    _check(wd, torch.int16, 3, "wd")
    _check(y, torch.float32, 3, "y")
    T, K = aq.shape
    top_k = topk_ids.shape[1]
    E, N, KH = wq4.shape
    if KH * 2 != K or tuple(ad.shape) != (T, K // 32) or topk_ids.shape[0] != T \
            or tuple(wd.shape) != (E, N, K // 32) or tuple(y.shape) != (T, top_k, N):
        raise ValueError("shape mismatch")
    st = lib().qgemm_w4a8_grouped_noalloc(_ptr(aq), _ptr(ad), T, _ptr(topk_ids), top_k,
                                          _ptr(wq4), _ptr(wd), E, N, K, _ptr(y),
                                          _stream(stream))
    _raise(st, "qgemm_w4a8_grouped_noalloc")
    return y


def moe_combine_f32(y, p, out=None, stream=None):
    """out[t][c] = sum_j p[t][j] * y[t][j][c] for y fp32 [T][top_k][N] and
    router probabilities p fp32 [T][top_k].  Returns out fp32 [T][N]."""
    torch = _torch()
    _check(y, torch.float32, 3, "y")
    _check(p, torch.float32, 2, "p")
    T, top_k, N = y.shape
    if tuple(p.shape) != (T, top_k):
        raise ValueError("shape mismatch: y %s p %s" % (tuple(y.shape), tuple(p.shape)))
    if out is None:
        with _on(stream, y.device):
            out = torch.empty((T, N), dtype=torch.float32, device=y.device)
    _check(out, torch.float32, 2, "out")
    st = lib().moe_combine_f32(_ptr(y), _ptr(p), T, top_k, N, _ptr(out), _stream(stream))
    _raise(st, "moe_combine_f32")
    return out


def _gguf(fmt, blocks, rows, k, codes, scales, stream):
    torch = _torch()
    _check(blocks, torch.uint8, 1, "blocks")
    per = 34 if fmt == "q8_0" else 18
    if k % 32 or blocks.numel() != rows * (k // 32) * per:
        raise ValueError("blocks must hold rows * k/32 GGUF %s blocks" % fmt)
    with _on(stream, blocks.device):
        if codes is None:
            codes = torch.empty((rows, k) if fmt == "q8_0" else (rows, k // 2),
                                dtype=torch.int8 if fmt == "q8_0" else torch.uint8,
                                device=blocks.device)
        if scales is None:
            scales = torch.empty((rows, k // 32), dtype=torch.int16, device=blocks.device)
    _check(codes, torch.int8 if fmt == "q8_0" else torch.uint8, 2, "codes")
    _check(scales, torch.int16, 2, "scales")
    f = lib().gguf_q8_0_to_planar if fmt == "q8_0" else lib().gguf_q4_0_to_planar
    st = f(_ptr(blocks), rows, k, _ptr(codes), _ptr(scales), _stream(stream))
    _raise(st, "gguf_%s_to_planar" % fmt)
    return codes, scales


def gguf_q8_0_to_planar(blocks, rows, k, q=None, d=None, stream=None):
    """Split a GGUF Q8_0 block array (uint8 [rows*k/32*34]) into codes int8
    [rows][k] and scale bits int16 [rows][k/32]."""
    return _gguf("q8_0", blocks, rows, k, q, d, stream)


def gguf_q4_0_to_planar(blocks, rows, k, wq4=None, wd=None, stream=None):
    """Split a GGUF Q4_0 block array (uint8 [rows*k/32*18]) into packed codes
    uint8 [rows][k/2] and scale bits int16 [rows][k/32]."""
    return _gguf("q4_0", blocks, rows, k, wq4, wd, stream)


def qgemm_w4a8_grouped_host(aq, ad, topk_ids, wq4, wd, nthreads=0):
    """The grouped W4A8 GEMM on the host CPU (AVX2 integer SIMD) for numpy
    arrays: aq int8 [T][K], ad uint16 [T][K/32], topk_ids int32 [T][top_k],
    wq4 uint8 [E][N][K/2], wd uint16 [E][N][K/32].  Returns y float32
    [T][top_k][N].  Synchronous; no GPU involved."""
    import numpy as np
    aq = np.ascontiguousarray(aq, np.int8)
    ad = np.ascontiguousarray(ad).view(np.uint16)
    ids = np.ascontiguousarray(topk_ids, np.int32)
    wq4 = np.ascontiguousarray(wq4, np.uint8)
    wd = np.ascontiguousarray(wd).view(np.uint16)
    T, K = aq.shape
    top_k = ids.shape[1]
    E, N, KH = wq4.shape
    if KH * 2 != K or ad.shape != (T, K // 32) or ids.shape[0] != T or wd.shape != (E, N, K // 32):
        raise ValueError("shape mismatch")
    y = np.empty((T, top_k, N), np.float32)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    st = lib().qgemm_w4a8_grouped_host(p(aq), p(ad), T, p(ids), top_k, p(wq4), p(wd), E, N, K,
                                       p(y), int(nthreads))
    _raise(st, "qgemm_w4a8_grouped_host")
    return y
