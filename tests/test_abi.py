"""C-ABI checks that need no GPU: the library loads, exports exactly the
symbols include/bqi.h declares, and rejects bad arguments with the documented
status codes before touching HIP (fake, never-dereferenced pointers)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import block_quantized_integer_amd as bqi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bqi.h")

OK, EINVAL, ESHAPE, EALIGN = bqi.BQI_OK, bqi.BQI_EINVAL, bqi.BQI_ESHAPE, bqi.BQI_EALIGN
FAKE = 0x10000          # 64 KiB: aligned to everything, never dereferenced
P = C.c_void_p


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"BQI_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ("quantize_q8_0", "qgemm_q8_0", "qgemm_w4a8_grouped", "route_topk",
                 "qgemm_w4a8_grouped_workspace_size", "bqi_status_string", "bqi_abi_version"):
        assert name in syms
    assert sorted(bqi.SYMBOLS) == syms


def test_library_exports_exactly_the_header_symbols():
    L = bqi.lib()
    for s in declared_symbols():
        assert hasattr(L, s)
    out = subprocess.run(["nm", "-D", "--defined-only", bqi.LIB_PATH], check=True,
                         stdout=subprocess.PIPE, text=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == declared_symbols()


def test_status_strings():
    L = bqi.lib()
    assert L.bqi_abi_version() == 240
    for st in (OK, EINVAL, ESHAPE, EALIGN, bqi.BQI_EHIP):
        assert L.bqi_status_string(st).decode().startswith("BQI_")
    assert L.bqi_status_string(12345)


def q(x, dt, rows, k, ldx, qp, dp):
    return bqi.lib().quantize_q8_0(P(x), dt, rows, k, ldx, P(qp), P(dp), P(0))


def test_quantize_validation():
    assert q(FAKE, 7, 4, 32, 32, FAKE, FAKE) == EINVAL            # bad dtype
    assert q(FAKE, 0, -1, 32, 32, FAKE, FAKE) == ESHAPE           # negative rows
    assert q(FAKE, 0, 4, 48, 48, FAKE, FAKE) == ESHAPE            # k % 32
    assert q(FAKE, 0, 4, 64, 32, FAKE, FAKE) == ESHAPE            # ldx < k
    assert q(0, 0, 4, 32, 32, FAKE, FAKE) == EINVAL               # null x
    assert q(FAKE, 0, 4, 32, 32, 0, FAKE) == EINVAL               # null q
    assert q(FAKE, 0, 4, 32, 32, FAKE, 0) == EINVAL               # null d
    assert q(FAKE + 4, 0, 4, 32, 32, FAKE, FAKE) == EALIGN        # x misaligned
    assert q(FAKE, 0, 4, 32, 33, FAKE, FAKE) == EALIGN            # fp32 row stride
    assert q(FAKE, 1, 4, 32, 34, FAKE, FAKE) == EALIGN            # fp16 row stride
    assert q(FAKE, 0, 4, 32, 32, FAKE + 8, FAKE) == EALIGN        # q misaligned
    assert q(FAKE, 0, 4, 32, 32, FAKE, FAKE + 1) == EALIGN        # d misaligned
    assert q(FAKE, 0, 0, 32, 32, 0, 0) == OK                      # empty: no launch
    assert q(FAKE, 0, 4, 0, 0, 0, 0) == OK
    assert q(FAKE, 0, 1 << 31, 32, 32, FAKE, FAKE) == ESHAPE      # too many rows


def g(aq, ad, m, wq, wd, n, k, y):
    return bqi.lib().qgemm_q8_0(P(aq), P(ad), m, P(wq), P(wd), n, k, P(y), P(0))


def test_qgemm_validation():
    assert g(FAKE, FAKE, -1, FAKE, FAKE, 8, 32, FAKE) == ESHAPE
    assert g(FAKE, FAKE, 8, FAKE, FAKE, -2, 32, FAKE) == ESHAPE
    assert g(FAKE, FAKE, 8, FAKE, FAKE, 8, 33, FAKE) == ESHAPE
    assert g(FAKE, FAKE, 8, FAKE, FAKE, 8, 32, 0) == EINVAL
    assert g(0, FAKE, 8, FAKE, FAKE, 8, 32, FAKE) == EINVAL
    assert g(FAKE, FAKE, 8, FAKE, 0, 8, 32, FAKE) == EINVAL
    assert g(FAKE + 2, FAKE, 8, FAKE, FAKE, 8, 32, FAKE) == EALIGN
    assert g(FAKE, FAKE, 8, FAKE + 8, FAKE, 8, 32, FAKE) == EALIGN
    assert g(FAKE, FAKE + 1, 8, FAKE, FAKE, 8, 32, FAKE) == EALIGN
    assert g(FAKE, FAKE, 8, FAKE, FAKE, 8, 32, FAKE + 2) == EALIGN
    assert g(0, 0, 0, 0, 0, 8, 32, 0) == OK
    assert g(0, 0, 8, 0, 0, 0, 32, 0) == OK
    assert g(FAKE, FAKE, 1 << 31, FAKE, FAKE, 8, 32, FAKE) == ESHAPE


def fq(x=FAKE, dt=0, m=1, k=64, ldx=64, wq=FAKE, wd=FAKE, n=8, y=FAKE, qp=FAKE, dp=FAKE):
    return bqi.lib().quantize_qgemm_q8_0(P(x), dt, m, k, ldx, P(wq), P(wd), n, P(y), P(qp),
                                         P(dp), P(0))


def test_fused_quantize_qgemm_validation():
    assert fq(dt=5) == EINVAL
    assert fq(m=-1) == ESHAPE
    assert fq(k=48, ldx=48) == ESHAPE
    assert fq(ldx=32) == ESHAPE
    assert fq(x=0) == EINVAL
    assert fq(qp=0) == EINVAL
    assert fq(dp=0) == EINVAL
    assert fq(wq=0) == EINVAL
    assert fq(y=0) == EINVAL
    assert fq(x=FAKE + 4) == EALIGN
    assert fq(ldx=66) == EALIGN           # fp32 rows must stay 16-byte aligned
    assert fq(qp=FAKE + 8) == EALIGN
    assert fq(wq=FAKE + 8) == EALIGN
    assert fq(y=FAKE + 2) == EALIGN
    assert fq(m=0) == OK
    assert fq(m=1 << 31) == ESHAPE


def test_moe_combine_validation():
    L = bqi.lib()
    c = lambda y=FAKE, p=FAKE, T=4, tk=8, n=16, out=FAKE: L.moe_combine_f32(
        P(y), P(p), T, tk, n, P(out), P(0))
    assert c(T=-1) == ESHAPE
    assert c(tk=-1) == ESHAPE
    assert c(n=-1) == ESHAPE
    assert c(out=0) == EINVAL
    assert c(y=0) == EINVAL
    assert c(p=0) == EINVAL
    assert c(y=FAKE + 2) == EALIGN
    assert c(out=FAKE + 1) == EALIGN
    assert c(T=0) == OK
    assert c(n=0) == OK


def test_gguf_validation():
    L = bqi.lib()
    for f in (L.gguf_q8_0_to_planar, L.gguf_q4_0_to_planar):
        g = lambda b=FAKE, rows=4, k=64, c=FAKE, d=FAKE: f(P(b), rows, k, P(c), P(d), P(0))
        assert g(k=48) == ESHAPE
        assert g(rows=-1) == ESHAPE
        assert g(b=0) == EINVAL
        assert g(c=0) == EINVAL
        assert g(d=0) == EINVAL
        assert g(b=FAKE + 2) == EALIGN
        assert g(c=FAKE + 8) == EALIGN
        assert g(d=FAKE + 1) == EALIGN
        assert g(rows=0) == OK
        assert g(k=0) == OK


def test_route_validation():
    L = bqi.lib()
    r = lambda ids, T, tk, E, c, o, rows: L.route_topk(P(ids), T, tk, E, P(c), P(o), P(rows), P(0))
    assert r(FAKE, -1, 8, 4, FAKE, FAKE, FAKE) == ESHAPE
    assert r(FAKE, 4, 8, 65537, FAKE, FAKE, FAKE) == ESHAPE
    assert r(FAKE, 1 << 28, 8, 4, FAKE, FAKE, FAKE) == ESHAPE     # rows > 2^30
    assert r(FAKE, 4, 8, 4, 0, FAKE, FAKE) == EINVAL
    assert r(0, 4, 8, 4, FAKE, FAKE, FAKE) == EINVAL
    assert r(FAKE, 4, 8, 4, FAKE, FAKE + 2, FAKE) == EALIGN
    assert r(0, 0, 0, 0, 0, 0, 0) == OK


def test_grouped_validation_and_workspace():
    L = bqi.lib()
    ws = L.qgemm_w4a8_grouped_workspace_size(947, 8, 128, 2048)
    assert ws >= 4 * (128 + 129 + 947 * 8) and ws % 256 == 0
    assert L.qgemm_w4a8_grouped_workspace_size(-1, 8, 128, 2048) == 0
    assert L.qgemm_w4a8_grouped_workspace_size(947, 8, 128, 48) == 0
    assert L.qgemm_w4a8_grouped_workspace_size(1 << 28, 8, 128, 2048) == 0

    def w(aq=FAKE, ad=FAKE, T=4, ids=FAKE, tk=2, wq=FAKE, wd=FAKE, E=3, n=16, k=64,
          y=FAKE, ws_ptr=FAKE, ws_bytes=1 << 20):
        return L.qgemm_w4a8_grouped(P(aq), P(ad), T, P(ids), tk, P(wq), P(wd), E, n, k, P(y),
                                    P(ws_ptr), ws_bytes, P(0))
    assert w(k=48) == ESHAPE
    assert w(T=-1) == ESHAPE
    assert w(E=65537) == ESHAPE
    assert w(y=0) == EINVAL
    assert w(ids=0) == EINVAL
    assert w(aq=0) == EINVAL
    assert w(wq=0) == EINVAL
    assert w(ws_ptr=0) == EINVAL
    assert w(ws_bytes=16) == EINVAL
    assert w(ws_ptr=FAKE + 128) == EALIGN
    assert w(aq=FAKE + 4) == EALIGN
    assert w(wq=FAKE + 8) == EALIGN
    assert w(y=FAKE + 1) == EALIGN
    assert w(T=0) == OK
    assert w(n=0) == OK


def test_grouped_noalloc_validation():
    """The allocation-free grouped entry point checks its arguments like the
    workspace one, and rejects a problem whose workspace exceeds the library's
    array before any HIP call (so these run without a GPU)."""
    L = bqi.lib()

    def w(aq=FAKE, ad=FAKE, T=4, ids=FAKE, tk=2, wq=FAKE, wd=FAKE, E=3, n=16, k=64, y=FAKE):
        return L.qgemm_w4a8_grouped_noalloc(P(aq), P(ad), T, P(ids), tk, P(wq), P(wd), E, n, k,
                                            P(y), P(0))
    assert w(k=48) == ESHAPE
    assert w(T=-1) == ESHAPE
    assert w(E=65537) == ESHAPE
    assert w(y=0) == EINVAL
    assert w(ids=0) == EINVAL
    assert w(aq=0) == EINVAL
    assert w(wq=0) == EINVAL
    assert w(aq=FAKE + 4) == EALIGN
    assert w(y=FAKE + 1) == EALIGN
    assert w(T=0) == OK
    assert w(n=0) == OK
    limit = bqi.NOALLOC_SCRATCH_BYTES
    # the routing tables take 4 bytes per routed row: 2^22 routed rows (plus
    # the per-expert tables) no longer fit; 2^21 do
    assert L.qgemm_w4a8_grouped_workspace_size(1 << 21, 1, 128, 32) <= limit
    assert L.qgemm_w4a8_grouped_workspace_size(1 << 22, 1, 128, 32) > limit
    assert w(T=1 << 22, tk=1, E=128, n=768, k=32) == ESHAPE
    assert w(T=1 << 19, tk=8, E=4, n=1, k=32) == ESHAPE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bqi, "_lib", None)
    monkeypatch.setattr(bqi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        bqi.lib()


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "block_quantized_integer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                for needle in ("import oracle", "from oracle", "liboracle", "bq_oracle", "orc_"):
                    assert needle not in text, (f, needle)
