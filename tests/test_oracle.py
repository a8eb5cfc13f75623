"""Pins for the CPU oracle: checks against what the format's definition and
the mathematics fix, independently of the oracle's own code.

The pages print no worked numeric example, so every pin here is a closed form,
an invariant, exact rational arithmetic (fractions), a library routine on a
special case (numpy fp16 conversion, numpy float64 matmul, numpy stable
argsort), or brute force on tiny inputs.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8_0_closed_forms.txt")


# ---------------------------------------------------------------------------
# independent helpers (exact rational arithmetic; numpy)
# ---------------------------------------------------------------------------

def f16_value(bits):
    return float(np.array(bits, np.uint16).view(np.float16))


def rne_fp16_exact(v: Fraction) -> float:
    """Round a non-negative rational to the nearest fp16 value, ties to even,
    by exact search over the fp16 grid (no floating point involved)."""
    assert v >= 0
    if v == 0:
        return 0.0
    if v >= Fraction(65520):
        return float("inf")
    # exponent of the binade containing v (fp16 normal: 2^-14 .. 2^15)
    e = -14
    while e < 15 and v >= Fraction(2) ** (e + 1):
        e += 1
    ulp = Fraction(2) ** (e - 10)  # also the subnormal spacing when e == -14
    n = v / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return float(fl * ulp)


def rhaz(v: Fraction) -> int:
    """Round half away from zero, exactly."""
    a = abs(v)
    fl = a.numerator // a.denominator
    if a - fl >= Fraction(1, 2):
        fl += 1
    return fl if v >= 0 else -fl


def quantize_exact(x):
    """Q8_0 of one 32-block by exact rational arithmetic."""
    amax = max(abs(Fraction(float(v))) for v in x)
    d = rne_fp16_exact(amax / 127)
    if d == 0.0:
        return 0.0, [0] * len(x)
    dq = Fraction(d)
    return d, [max(-127, min(127, rhaz(Fraction(float(v)) / dq))) for v in x]


def parse_golden():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition(" ") if line.startswith("case") else line.partition(":")
        if key == "case":
            cur = {"name": val.strip()}
            cases.append(cur)
        elif key == "x":
            cur["x"] = [float(t) for t in val.split()]
        elif key == "d":
            cur["d"] = int(val.strip(), 16)
        elif key == "q":
            cur["q"] = [int(t) for t in val.split()]
    return cases


# ---------------------------------------------------------------------------
# fp16 conversion
# ---------------------------------------------------------------------------

def _check_f16_against_numpy(bits_u32):
    x = bits_u32.view(np.float32)
    got = oracle.f32_to_f16_bits(x)
    with np.errstate(all="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.isnan(got[nan].view(np.float16)).all()


def test_f16_rne_stratified_vs_numpy():
    """Every sign and fp32 exponent, with the mantissa patterns that decide
    rounding (all low-13-bit patterns around the fp16 tie for a spread of
    high mantissas), against numpy's IEEE conversion."""
    hi = np.arange(0, 1 << 10, 37, dtype=np.uint32)        # fp16-kept mantissa bits
    lo = np.concatenate([np.arange(0, 64), np.arange(0x1000 - 64, 0x1000 + 64),
                         np.arange(0x2000 - 64, 0x2000)]).astype(np.uint32)
    man = (hi[:, None] << 13 | lo[None, :]).ravel()
    ex = np.arange(256, dtype=np.uint32)
    sign = np.array([0, 1], np.uint32)
    bits = (sign[:, None, None] << 31 | ex[None, :, None] << 23 | man[None, None, :]).ravel()
    _check_f16_against_numpy(bits)


def test_f16_rne_random_vs_numpy():
    g = np.random.default_rng(1)
    _check_f16_against_numpy(g.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32))


@pytest.mark.slow
def test_f16_rne_exhaustive_vs_numpy():
    """All 2^32 fp32 bit patterns (several minutes)."""
    base = np.arange(0, 1 << 26, dtype=np.uint32)
    for c in range(64):
        _check_f16_against_numpy(base + np.uint32(c << 26))


def test_f16_to_f32_exhaustive_vs_numpy():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(got[nan]).all()


# ---------------------------------------------------------------------------
# Q8_0 quantizer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", parse_golden(), ids=lambda c: c["name"])
def test_quantize_golden_closed_forms(case):
    x = np.zeros((1, 32), np.float32)
    x[0, : len(case["x"])] = np.array(case["x"], np.float32)
    q, d = oracle.quantize_q8_0(x)
    assert int(d[0, 0]) == case["d"], hex(int(d[0, 0]))
    want = np.zeros(32, np.int64)
    want[: len(case["q"])] = case["q"]
    assert np.array_equal(q[0].astype(np.int64), want)


def test_scale_matches_exact_rational_rne():
    """d = fp16_rne(amax/127) computed exactly with fractions, over amax
    spanning every fp32 binade that matters (subnormal d .. overflow edge)."""
    g = np.random.default_rng(2)
    vals = []
    for e in range(-40, 24):
        m = g.integers(1 << 23, 1 << 24, size=12)
        vals += [float(v) * 2.0 ** (e - 23) for v in m]
    # amax whose quotient sits on an fp16 rounding midpoint (ties)
    for s in range(1024, 2048, 61):
        for e in (-20, -5, 0, 3):
            vals.append((s + 0.5) * 127 * 2.0 ** (e - 10))
    vals = np.array(vals, np.float32)
    vals = vals[np.isfinite(vals)]
    x = np.zeros((len(vals), 32), np.float32)
    x[:, 0] = vals
    _, d = oracle.quantize_q8_0(x)
    for i, v in enumerate(vals):
        want = rne_fp16_exact(Fraction(float(v)) / 127)
        got = f16_value(d[i, 0])
        assert got == want or (np.isinf(want) and np.isinf(got)), (v, got, want)


def test_codes_match_exact_rational_rounding():
    """Codes equal round_half_away(x/d) computed with fractions, for random
    blocks of several distributions, including values placed on and one ulp
    around every rounding tie k+1/2."""
    g = np.random.default_rng(3)
    blocks = [g.standard_normal(32).astype(np.float32) for _ in range(40)]
    blocks += [(g.standard_t(3, 32) * 20).astype(np.float32) for _ in range(20)]
    blocks += [(g.standard_normal(32) * 1e-6).astype(np.float32) for _ in range(10)]
    # near-tie blocks: amax = 127 * d exactly for a chosen fp16 d, others at (k+1/2) d +- 1 ulp
    for dbits in (0x3C00, 0x2008, 0x1A3F, 0x4B21, 0x0400, 0x3555):
        dv = np.float32(f16_value(dbits))
        ks = g.integers(0, 127, size=31)
        t = ((ks + 0.5) * dv).astype(np.float32)
        sgn = g.choice([-1, 0, 1], size=31)
        t = np.array([np.nextafter(v, np.float32(np.inf) * s) if s else v for v, s in zip(t, sgn)],
                     np.float32) * g.choice([-1, 1], size=31).astype(np.float32)
        blocks.append(np.concatenate([[np.float32(127) * dv], t]).astype(np.float32))
    x = np.stack(blocks)
    q, d = oracle.quantize_q8_0(x)
    for i, blk in enumerate(blocks):
        dw, qw = quantize_exact(blk)
        assert f16_value(d[i, 0]) == dw
        assert list(q[i].astype(int)) == qw, i


def test_quantize_invariants():
    g = np.random.default_rng(4)
    x = np.concatenate([g.standard_normal((64, 256)),
                        g.standard_t(3, (64, 256)) * 50,
                        g.uniform(-0.05, 0.05, (64, 256))]).astype(np.float32)
    q, d = oracle.quantize_q8_0(x)
    dv = d.view(np.float16).astype(np.float64)
    qb = q.reshape(len(x), -1, 32).astype(np.float64)
    xb = x.reshape(len(x), -1, 32).astype(np.float64)
    normal = dv >= 2.0 ** -14
    assert normal.all()
    # quantization error bound |x - q d| <= d/2
    err = np.abs(xb - qb * dv[..., None])
    assert (err <= dv[..., None] / 2).all()
    # every nonzero block with a normal scale reaches |q| = 127
    assert (np.abs(qb).max(axis=-1) == 127).all()
    # odd symmetry: quantize(-x) = (-q, d)
    qn, dn = oracle.quantize_q8_0(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)
    # power-of-two scaling leaves codes unchanged and scales d by the power
    for s in (2.0 ** -1, 2.0 ** 4):  # stays inside the fp16 normal range
        qs, ds = oracle.quantize_q8_0((x * np.float32(s)).astype(np.float32))
        assert np.array_equal(qs, q)
        assert np.array_equal(ds.view(np.float16).astype(np.float64), dv * s)
    # subnormal scales: the bound holds wherever the code is not clamped
    xs = (g.standard_normal((64, 64)) * 1e-4).astype(np.float32)
    q, d = oracle.quantize_q8_0(xs)
    dv = d.view(np.float16).astype(np.float64)[..., None]
    assert (dv < 2.0 ** -14).all()
    qb = q.reshape(64, -1, 32).astype(np.float64)
    xb = xs.reshape(64, -1, 32).astype(np.float64)
    unclamped = np.abs(qb) < 127
    assert (np.abs(xb - qb * dv)[unclamped] <= (dv / 2 + 0 * xb)[unclamped]).all()
    assert (np.abs(xb / dv)[~unclamped] >= 126.5).all()


def test_quantize_ldx_and_f16_input():
    g = np.random.default_rng(5)
    x = g.standard_normal((7, 100)).astype(np.float32)
    q, d = oracle.quantize_q8_0(x, k=96)
    q2, d2 = oracle.quantize_q8_0(np.ascontiguousarray(x[:, :96]))
    assert np.array_equal(q, q2) and np.array_equal(d, d2)
    # fp16 input: widened exactly to fp32 first
    xh = x.astype(np.float16)
    qh, dh = oracle.quantize_q8_0(xh, k=96)
    qf, df = oracle.quantize_q8_0(np.ascontiguousarray(xh.astype(np.float32)[:, :96]))
    assert np.array_equal(qh, qf) and np.array_equal(dh, df)


# ---------------------------------------------------------------------------
# block dots and the Q8_0 GEMM
# ---------------------------------------------------------------------------

def test_block_dots_bruteforce_and_extremes():
    g = np.random.default_rng(6)
    a = g.integers(-128, 128, (5, 96), dtype=np.int8)
    w = g.integers(-128, 128, (7, 96), dtype=np.int8)
    P = oracle.block_dots(a, w)
    ref = np.einsum("mbi,nbi->mnb", a.reshape(5, 3, 32).astype(np.int64),
                    w.reshape(7, 3, 32).astype(np.int64))
    assert np.array_equal(P.astype(np.int64), ref)
    full = np.full((1, 32), 127, np.int8)
    assert oracle.block_dots(full, full)[0, 0, 0] == 32 * 127 * 127 == 516128
    neg = np.full((1, 32), -128, np.int8)
    assert oracle.block_dots(neg, neg)[0, 0, 0] == 32 * 128 * 128 == 524288
    assert oracle.block_dots(neg, full)[0, 0, 0] == -32 * 128 * 127


def _dequant(q, d):
    return (q.reshape(q.shape[0], -1, 32).astype(np.float64)
            * d.view(np.float16).astype(np.float64)[..., None]).reshape(q.shape)


def test_gemm_matches_numpy_dequant_matmul():
    g = np.random.default_rng(7)
    for (m, n, k) in [(3, 5, 32), (4, 9, 96), (16, 33, 256)]:
        aq = g.integers(-128, 128, (m, k), dtype=np.int8)
        wq = g.integers(-128, 128, (n, k), dtype=np.int8)
        ad = W.random_scales(0, 90 + m, (m, k // 32))
        wd = W.random_scales(0, 91 + n, (n, k // 32))
        y, a = oracle.qgemm_q8_0(aq, ad, wq, wd)
        ref = _dequant(aq, ad) @ _dequant(wq, wd).T
        assert (np.abs(y - ref) <= 1e-12 * a).all()
        # asum is sum_b |term_b|: compare with numpy per-block terms
        P = np.einsum("mbi,nbi->mnb", aq.reshape(m, -1, 32).astype(np.int64),
                      wq.reshape(n, -1, 32).astype(np.int64)).astype(np.float64)
        S = ad.view(np.float16).astype(np.float64)[:, None, :] * wd.view(np.float16).astype(np.float64)[None, :, :]
        assert np.allclose(a, np.abs(P * S).sum(-1), rtol=1e-14, atol=0)
        # threaded driver gives bit-identical results
        y4, a4 = oracle.qgemm_q8_0(aq, ad, wq, wd, nthreads=4)
        assert np.array_equal(y4, y) and np.array_equal(a4, a)
        # sampled form gives the same values
        mi = g.integers(0, m, 20)
        nj = g.integers(0, n, 20)
        ys, as_ = oracle.qgemm_q8_0_at(aq, ad, wq, wd, mi, nj)
        assert np.array_equal(ys, y[mi, nj]) and np.array_equal(as_, a[mi, nj])


def test_gemm_exact_rational_tiny():
    g = np.random.default_rng(8)
    m, n, k = 2, 3, 64
    aq = g.integers(-128, 128, (m, k), dtype=np.int8)
    wq = g.integers(-128, 128, (n, k), dtype=np.int8)
    ad = W.random_scales(0, 80, (m, 2))
    wd = W.random_scales(0, 81, (n, 2))
    y, _ = oracle.qgemm_q8_0(aq, ad, wq, wd)
    for i in range(m):
        for j in range(n):
            ex = sum(Fraction(f16_value(ad[i, t // 32])) * Fraction(f16_value(wd[j, t // 32]))
                     * int(aq[i, t]) * int(wq[j, t]) for t in range(k))
            assert abs(Fraction(y[i, j]) - ex) <= abs(ex) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_gemm_closed_forms():
    k = 256
    one = np.full((1, k // 32), 0x3C00, np.uint16)  # d = 1.0
    full = np.full((1, k), 127, np.int8)
    y, a = oracle.qgemm_q8_0(full, one, full, one)
    assert y[0, 0] == k * 16129 == 4129024 and a[0, 0] == y[0, 0]
    # one-hot weight rows pick out dequantized activations
    g = np.random.default_rng(9)
    aq = g.integers(-127, 128, (4, k), dtype=np.int8)
    ad = W.random_scales(0, 70, (4, k // 32))
    n = 40
    wq = np.zeros((n, k), np.int8)
    idx = g.choice(k, n, replace=False)
    wq[np.arange(n), idx] = 1
    wd = np.full((n, k // 32), 0x3C00, np.uint16)
    y, _ = oracle.qgemm_q8_0(aq, ad, wq, wd)
    assert np.array_equal(y, _dequant(aq, ad)[:, idx])
    # negating the activations negates y exactly; swapping operand roles transposes y
    wq2 = g.integers(-128, 128, (6, k), dtype=np.int8)
    wd2 = W.random_scales(0, 71, (6, k // 32))
    y1, _ = oracle.qgemm_q8_0(aq, ad, wq2, wd2)
    y2, _ = oracle.qgemm_q8_0(-aq, ad, wq2, wd2)
    assert np.array_equal(y2, -y1)
    y3, _ = oracle.qgemm_q8_0(wq2, wd2, aq, ad)
    assert np.array_equal(y3, y1.T)


def test_gemm_scale_index_sensitivity():
    """A transposed or shifted scale index changes the result: per-block
    scales must line up with their own block."""
    g = np.random.default_rng(10)
    aq = g.integers(-127, 128, (2, 128), dtype=np.int8)
    wq = g.integers(-127, 128, (3, 128), dtype=np.int8)
    ad = W.random_scales(0, 60, (2, 4))
    wd = W.random_scales(0, 61, (3, 4))
    y, _ = oracle.qgemm_q8_0(aq, ad, wq, wd)
    y_shift, _ = oracle.qgemm_q8_0(aq, np.roll(ad, 1, axis=1), wq, wd)
    assert not np.allclose(y, y_shift)
    ref = _dequant(aq, ad) @ _dequant(wq, wd).T
    assert np.allclose(y, ref, rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
# 4-bit weights, routing, grouped W4A8
# ---------------------------------------------------------------------------

def test_w4_pack_layout_and_roundtrip():
    g = np.random.default_rng(11)
    codes = g.integers(0, 16, (3, 64), dtype=np.uint8)
    p = oracle.pack_w4(codes)
    # stated layout: byte j of a 32-group = element j (low nibble) | element j+16 (high nibble)
    want = np.empty((3, 32), np.uint8)
    for grp in range(2):
        c = codes[:, 32 * grp: 32 * grp + 32]
        want[:, 16 * grp: 16 * grp + 16] = c[:, :16] | (c[:, 16:] << 4)
    assert np.array_equal(p, want)
    assert np.array_equal(oracle.unpack_w4(p), codes)


def test_w4_quantizer_bounds():
    g = np.random.default_rng(12)
    w = (g.standard_normal((16, 128)) * 0.02).astype(np.float32)
    p, d = oracle.quantize_w4(w)
    c = oracle.unpack_w4(p).astype(np.int64)
    assert c.min() >= 1 and c.max() <= 15
    dv = d.view(np.float16).astype(np.float64)
    q = (c - 8).reshape(16, -1, 32)
    err = np.abs(w.reshape(16, -1, 32) - q * dv[..., None])
    assert (err <= dv[..., None] / 2).all()
    assert (np.abs(q).max(-1) == 7).all()
    for blk in range(3):
        dq = rne_fp16_exact(max(abs(Fraction(float(v))) for v in w[blk, :32]) / 7)
        assert f16_value(d[blk, 0]) == dq


def test_w4_quantizer_ties_closed_form():
    """Round half away from zero in the 4-bit quantizer, from closed forms:
    element 0 of each group is 7 d, which makes the group's scale exactly d
    (7 d and d are exact in fp32, and 7 d / 7 = d has no rounding); every
    other element is +-(k + 1/2) d (k = 0..6, exact: at most 4 + 11
    significant bits) or its fp32 neighbour toward or away from zero.  The
    code is 8 +- (k + 1) at and beyond the midpoint, 8 +- k below it.  A
    round-to-even quantizer differs at k = 0, 2, 4, 6."""
    g = np.random.default_rng(13)
    dbits = np.arange(0x0800, 0x7000, 53, dtype=np.uint16)      # normal fp16 scales
    d = dbits.view(np.float16).astype(np.float32)
    ng = d.size
    k = g.integers(0, 7, size=(ng, 31))
    side = g.integers(0, 3, size=(ng, 31))                       # 0 toward zero, 1 tie, 2 away
    sign = g.choice(np.array([-1.0, 1.0], np.float32), size=(ng, 31))
    mid = ((k + 0.5) * d[:, None]).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (k + 0.5) * d[:, None].astype(np.float64))
    x = np.where(side == 0, np.nextafter(mid, np.float32(0)),
                 np.where(side == 2, np.nextafter(mid, np.float32(np.inf)), mid))
    w = np.concatenate([(np.float32(7) * d)[:, None], (x * sign).astype(np.float32)], 1)
    p, dq = oracle.quantize_w4(w.astype(np.float32))
    assert np.array_equal(dq.reshape(-1), dbits)
    c = oracle.unpack_w4(p).astype(np.int64)
    want = 8 + np.where(side == 0, k, k + 1) * sign.astype(np.int64)
    assert (c[:, 0] == 15).all()
    assert np.array_equal(c[:, 1:], want)
    # the ties alone: 8 +- (k + 1), never the even neighbour
    tie = side == 1
    assert np.array_equal(np.abs(c[:, 1:][tie] - 8), (k + 1)[tie])


def test_route_topk_properties():
    ids = W.topk_ids(97, 8, 16, seed=3)
    ids[5, 2] = -1
    ids[9, 0] = 16
    counts, offsets, rows, inv = oracle.route_topk(ids, 16)
    assert inv == 2
    flat = ids.ravel()
    assert counts.sum() == flat.size - 2
    assert np.array_equal(np.diff(offsets), counts) and offsets[0] == 0
    valid = (flat >= 0) & (flat < 16)
    order = np.argsort(np.where(valid, flat, 99), kind="stable")[: valid.sum()]
    assert np.array_equal(rows, order.astype(np.int32))
    for e in range(16):
        seg = rows[offsets[e]: offsets[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


def test_w4a8_reduces_to_q8_gemm_and_numpy():
    g = np.random.default_rng(13)
    T, top_k, E, n, k = 11, 3, 5, 40, 96
    aq = g.integers(-128, 128, (T, k), dtype=np.int8)
    ad = W.random_scales(0, 50, (T, k // 32))
    packed = g.integers(0, 256, (E, n, k // 2), dtype=np.uint8)
    wd = W.random_scales(0, 51, (E, n, k // 32))
    ids = g.integers(0, E, (T, top_k)).astype(np.int32)
    ids[4, 1] = E + 3          # invalid -> zero row
    ids[7, 2] = ids[7, 0]      # duplicate expert within a token is legal
    y, a = oracle.qgemm_w4a8_grouped(aq, ad, ids, packed, wd)
    codes = oracle.unpack_w4(packed).astype(np.int16) - 8
    for t in range(T):
        for j in range(top_k):
            e = ids[t, j]
            if not (0 <= e < E):
                assert (y[t, j] == 0).all() and (a[t, j] == 0).all()
                continue
            yq, aq8 = oracle.qgemm_q8_0(aq[t:t + 1], ad[t:t + 1], codes[e].astype(np.int8), wd[e])
            assert np.array_equal(y[t, j], yq[0]) and np.array_equal(a[t, j], aq8[0])
            ref = _dequant(aq[t:t + 1], ad[t:t + 1]) @ _dequant(codes[e].astype(np.int8), wd[e]).T
            assert (np.abs(y[t, j] - ref[0]) <= 1e-12 * a[t, j]).all()
    # threaded driver and sampled form agree
    y2, _ = oracle.qgemm_w4a8_grouped(aq, ad, ids, packed, wd, nthreads=3)
    assert np.array_equal(y2, y)
    ri = g.integers(0, T * top_k, 30)
    cj = g.integers(0, n, 30)
    ys, _ = oracle.qgemm_w4a8_grouped_at(aq, ad, ids, packed, wd, ri, cj)
    assert np.array_equal(ys, y.reshape(T * top_k, n)[ri, cj])
    # permuting tokens permutes output rows
    perm = g.permutation(T)
    yp, _ = oracle.qgemm_w4a8_grouped(aq[perm], ad[perm], ids[perm], packed, wd)
    assert np.array_equal(yp, y[perm])


def test_w4a8_single_expert_is_plain_gemm():
    g = np.random.default_rng(14)
    T, n, k = 9, 24, 64
    aq = g.integers(-128, 128, (T, k), dtype=np.int8)
    ad = W.random_scales(0, 40, (T, 2))
    codes = g.integers(0, 16, (1, n, k), dtype=np.uint8)
    wd = W.random_scales(0, 41, (1, n, 2))
    y, _ = oracle.qgemm_w4a8_grouped(aq, ad, np.zeros((T, 1), np.int32), oracle.pack_w4(codes), wd)
    ref = _dequant(aq, ad) @ _dequant((codes[0].astype(np.int16) - 8).astype(np.int8), wd[0]).T
    assert np.allclose(y[:, 0, :], ref, rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------------------
# MoE combine (the step after the grouped GEMM)
# ---------------------------------------------------------------------------

def test_moe_combine_exact_rational_tiny():
    g = np.random.default_rng(21)
    T, top_k, n = 3, 4, 5
    y = (g.standard_normal((T, top_k, n)) * 10).astype(np.float32)
    p = g.random((T, top_k)).astype(np.float32)
    out, asum = oracle.moe_combine(y, p)
    for t in range(T):
        for c in range(n):
            terms = [Fraction(float(p[t, j])) * Fraction(float(y[t, j, c])) for j in range(top_k)]
            exact = sum(terms)
            a = sum(abs(x) for x in terms)
            # fp64 sum of exact products: top_k roundings at most
            assert abs(Fraction(out[t, c]) - exact) <= Fraction(top_k, 2 ** 52) * a
            assert asum[t, c] == float(a) or abs(Fraction(asum[t, c]) - a) <= Fraction(top_k, 2 ** 52) * a


def test_moe_combine_closed_forms_and_numpy():
    g = np.random.default_rng(22)
    T, top_k, n = 7, 8, 33
    y = g.standard_normal((T, top_k, n)).astype(np.float32)
    # one-hot weights pick one slot exactly
    p = np.zeros((T, top_k), np.float32)
    pick = g.integers(0, top_k, T)
    p[np.arange(T), pick] = 1.0
    out, _ = oracle.moe_combine(y, p)
    assert np.array_equal(out, y[np.arange(T), pick].astype(np.float64))
    # equal slots with power-of-two weights summing to 1 reproduce the slot
    y_eq = np.repeat(y[:, :1, :], top_k, axis=1)
    out, _ = oracle.moe_combine(y_eq, np.full((T, top_k), 1.0 / top_k, np.float32))
    assert np.array_equal(out, y_eq[:, 0, :].astype(np.float64))
    # numpy einsum in fp64
    p = g.random((T, top_k)).astype(np.float32)
    out, asum = oracle.moe_combine(y, p)
    ref = np.einsum("tj,tjc->tc", p.astype(np.float64), y.astype(np.float64))
    assert np.all(np.abs(out - ref) <= 1e-13 * asum)
    # a transposed slot index would not match
    bad = np.einsum("tj,tjc->tc", p.astype(np.float64)[:, ::-1], y.astype(np.float64))
    assert not np.allclose(out, bad)


# ---------------------------------------------------------------------------
# GGUF block import
# ---------------------------------------------------------------------------

def parse_gguf_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "gguf_blocks.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition(" ") if line.startswith("block") else line.partition(":")
        if key == "block":
            fmt, name = val.split()
            cur = {"fmt": fmt, "name": name}
            cases.append(cur)
        elif key == "bytes":
            cur["bytes"] = np.array([int(v, 16) for v in val.split()], np.uint8)
        elif key == "d":
            cur["d"] = int(val.strip(), 16)
        elif key == "codes":
            cur["codes"] = [int(v, 0) for v in val.split()]
        elif key == "values":
            cur["values"] = [float(v) for v in val.split()]
    return cases


@pytest.mark.parametrize("case", parse_gguf_golden(), ids=lambda c: c["name"])
def test_gguf_golden_blocks(case):
    raw = case["bytes"]
    if case["fmt"] == "q8_0":
        assert raw.size == 34
        q, d = oracle.gguf_q8_0_to_planar(raw, 1, 32)
        assert d[0, 0] == case["d"]
        assert q[0].tolist() == case["codes"]
        vals = q[0].astype(np.float64) * oracle.f16_bits_to_f32(d)[0, 0]
    else:
        assert raw.size == 18
        packed, d = oracle.gguf_q4_0_to_planar(raw, 1, 32)
        assert d[0, 0] == case["d"]
        assert packed[0].tolist() == case["codes"]
        vals = (oracle.unpack_w4(packed)[0].astype(np.float64) - 8) * oracle.f16_bits_to_f32(d)[0, 0]
    assert vals.tolist() == case["values"]


def test_gguf_matches_numpy_structured_dtype_and_roundtrips():
    g = np.random.default_rng(23)
    rows, k = 5, 160
    nb = k // 32
    q8 = np.dtype([("d", "<u2"), ("qs", "i1", 32)])
    q4 = np.dtype([("d", "<u2"), ("qs", "u1", 16)])
    assert q8.itemsize == 34 and q4.itemsize == 18
    a = np.zeros(rows * nb, q8)
    a["d"] = g.integers(0, 1 << 16, rows * nb)
    a["qs"] = g.integers(-128, 128, (rows * nb, 32))
    q, d = oracle.gguf_q8_0_to_planar(a.view(np.uint8), rows, k)
    assert np.array_equal(d.reshape(-1), a["d"])
    assert np.array_equal(q.reshape(rows, nb, 32).reshape(-1, 32), a["qs"])
    back = np.zeros(rows * nb, q8)
    back["d"], back["qs"] = d.reshape(-1), q.reshape(-1, 32)
    assert np.array_equal(back.view(np.uint8), a.view(np.uint8))
    b = np.zeros(rows * nb, q4)
    b["d"] = g.integers(0, 1 << 16, rows * nb)
    b["qs"] = g.integers(0, 256, (rows * nb, 16))
    packed, d4 = oracle.gguf_q4_0_to_planar(b.view(np.uint8), rows, k)
    assert np.array_equal(d4.reshape(-1), b["d"])
    assert np.array_equal(packed.reshape(-1, 16), b["qs"])
    # the codes of block 1 start at byte 34 + 2: a reader that forgot the
    # 2-byte scale (stride 32) would take bytes 32 + 2 .. 65 and misread them
    flat = a.view(np.uint8).reshape(-1)
    assert np.array_equal(flat[36:68].view(np.int8), q[0, 32:64])
    assert not np.array_equal(flat[34:66].view(np.int8), q[0, 32:64])
