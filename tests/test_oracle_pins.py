"""Pins for the fp64 oracle against values that do not come from the oracle.

Each test fixes the oracle to something independent of its own code: the
hand-derived worked examples under tests/golden/, exact rational arithmetic
(fractions.Fraction over independently decoded fp16/bf16 bit patterns), closed
forms evaluated with the decimal module, invariants, and brute-force loops.
The cases are chosen so that a dropped scale, a wrong block index, a
transposed operand, a wrong sign or offset, a missing softcap factor or a
wrong tie-break each fail at least one of them.
"""
import decimal
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# -------------------------------------------------- independent decoders --
def f16_exact(bits: int) -> Fraction:
    """fp16 bit pattern -> exact rational, decoded by struct (not numpy)."""
    return Fraction(struct.unpack("<e", struct.pack("<H", int(bits)))[0])


def bf16_exact(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0])


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def rn32(fr: Fraction) -> float:
    """Exact round-half-even of a rational to fp32 (normal range)."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    m = a * (1 << 23)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(Fraction(fl, 1 << 23) * Fraction(2) ** e)


def exact_gemv(codes, sbits, xbits):
    n, k = codes.shape
    xs = [bf16_exact(b) for b in xbits]
    y, a = [], []
    for r in range(n):
        acc = Fraction(0)
        mag = Fraction(0)
        for b in range(k // 32):
            d = f16_exact(sbits[r, b])
            for j in range(32):
                t = int(codes[r, 32 * b + j]) * d * xs[32 * b + j]
                acc += t
                mag += abs(t)
        y.append(acc)
        a.append(mag)
    return y, a


def fp16_bits(v: float) -> int:
    return struct.unpack("<H", struct.pack("<e", v))[0]


def bf16_bits(v: float) -> int:
    b = f32_bits(v)
    assert b & 0xFFFF == 0, "value must be exactly representable in bf16"
    return b >> 16


# ---------------------------------------------------------- worked example --
def _worked_inputs():
    codes = np.zeros((2, 32), dtype=np.int8)
    codes[0] = [(j % 16) - 8 for j in range(32)]
    codes[1] = 7
    scales = np.array([[fp16_bits(0.5)], [fp16_bits(0.25)]], dtype=np.uint16)
    assert scales[0, 0] == 0x3800 and scales[1, 0] == 0x3400
    xs = {
        "ramp": [float(j) for j in range(32)],
        "alt": [(-1.0) ** j for j in range(32)],
        "e5": [1.0 if j == 5 else 0.0 for j in range(32)],
        "e21": [1.0 if j == 21 else 0.0 for j in range(32)],
    }
    return codes, scales, {k: np.array([bf16_bits(v) for v in vals], dtype=np.uint16)
                           for k, vals in xs.items()}


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_worked_example_2x32():
    codes, scales, xs = _worked_inputs()
    rows = _golden_rows("gemv_worked_2x32.txt")
    assert len(rows) == 4
    for case, y0, y1, a0, a1 in rows:
        y, a = oracle.gemv(codes, scales, xs[case])
        assert y.tolist() == [float(y0), float(y1)], case
        assert a.tolist() == [float(a0), float(a1)], case
    head = oracle.lmhead(codes, scales, xs["ramp"])
    assert head["idx"] == 1


def test_nibble_convention():
    # stored unsigned nibble minus the midpoint 8
    assert oracle.codes_from_nibbles([0, 8, 15]).tolist() == [-8, 0, 7]
    allc = np.arange(-8, 8)
    assert oracle.codes_from_nibbles(oracle.nibbles_from_codes(allc)).tolist() == allc.tolist()
    with pytest.raises(ValueError):
        oracle.nibbles_from_codes([8])
    with pytest.raises(ValueError):
        oracle.codes_from_nibbles([16])


# ----------------------------------------------------- exact arithmetic --
def test_dequant_exact_rational():
    rng = np.random.default_rng(11)
    codes, sb = synth.q4_weights(rng, 3, 96)
    w = oracle.dequant(codes, sb)
    for r in range(3):
        for k in range(96):
            assert Fraction(w[r, k]) == int(codes[r, k]) * f16_exact(sb[r, k // 32])


def test_gemv_bruteforce_fraction_nonsquare():
    # 5 x 96: non-square so a transposed operand cannot pass; three blocks
    # with different scales so a wrong block index cannot pass.
    rng = np.random.default_rng(3)
    codes, sb = synth.q4_weights(rng, 5, 96)
    x = synth.bf16_normal(rng, 96)
    y, a = oracle.gemv(codes, sb, x)
    ye, ae = exact_gemv(codes, sb, x)
    for r in range(5):
        assert abs(Fraction(y[r]) - ye[r]) <= Fraction(1, 10 ** 12) * ae[r]
        assert abs(Fraction(a[r]) - ae[r]) <= Fraction(1, 10 ** 12) * ae[r]


def test_gemv_integer_inputs_exact():
    # power-of-two scales and integer x: every partial sum is an exact
    # multiple of 2^-8, so the fp64 oracle must equal the integer result.
    rng = np.random.default_rng(5)
    n, k = 24, 512
    codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    pw = rng.integers(6, 9, size=(n, k // 32))
    sb = np.vectorize(lambda p: fp16_bits(2.0 ** -int(p)))(pw).astype(np.uint16)
    xi = rng.integers(-8, 9, size=k)
    xb = np.array([bf16_bits(float(v)) for v in xi], dtype=np.uint16)
    y, _ = oracle.gemv(codes, sb, xb)
    for r in range(n):
        tot = 0
        for kk in range(k):
            tot += int(codes[r, kk]) * int(xi[kk]) * (1 << (8 - int(pw[r, kk // 32])))
        assert y[r] == tot / 256.0


def test_gemv_onehot_selects_column():
    rng = np.random.default_rng(7)
    n, k = 6, 128
    codes, sb = synth.q4_weights(rng, n, k)
    for kk in range(k):
        x = np.zeros(k, dtype=np.uint16)
        x[kk] = bf16_bits(1.0)
        y, _ = oracle.gemv(codes, sb, x)
        for r in range(n):
            assert Fraction(y[r]) == int(codes[r, kk]) * f16_exact(sb[r, kk // 32])


def test_gemv_zero_codes_and_zero_x():
    rng = np.random.default_rng(8)
    codes, sb = synth.q4_weights(rng, 4, 64)
    x = synth.bf16_normal(rng, 64)
    y, a = oracle.gemv(np.zeros_like(codes), sb, x)
    assert (y == 0).all() and (a == 0).all()
    y, a = oracle.gemv(codes, sb, np.zeros(64, dtype=np.uint16))
    assert (y == 0).all() and (a == 0).all()


def test_gemm_bruteforce_fraction():
    rng = np.random.default_rng(9)
    s, n, k = 3, 4, 64
    codes, sb = synth.q4_weights(rng, n, k)
    xs = synth.bf16_normal(rng, (s, k))
    y, a = oracle.gemm(codes, sb, xs)
    assert y.shape == (s, n)
    for t in range(s):
        ye, ae = exact_gemv(codes, sb, xs[t])
        for r in range(n):
            assert abs(Fraction(y[t, r]) - ye[r]) <= Fraction(1, 10 ** 12) * ae[r]
            assert abs(Fraction(a[t, r]) - ae[r]) <= Fraction(1, 10 ** 12) * ae[r]


def test_gemm_rows_equal_gemv():
    rng = np.random.default_rng(10)
    codes, sb = synth.q4_weights(rng, 33, 160)
    xs = synth.bf16_normal(rng, (5, 160))
    y, _ = oracle.gemm(codes, sb, xs)
    for t in range(5):
        yv, _ = oracle.gemv(codes, sb, xs[t])
        np.testing.assert_allclose(y[t], yv, rtol=1e-13, atol=0)


# ----------------------------------------------------------------- softcap --
def _tanh_decimal(u: Fraction) -> decimal.Decimal:
    with decimal.localcontext() as ctx:
        ctx.prec = 40
        e = (decimal.Decimal(u.numerator) / decimal.Decimal(u.denominator) * 2).exp()
        return (e - 1) / (e + 1)


def test_softcap_closed_forms():
    assert oracle.softcap(0.0) == 0.0
    z = np.linspace(-300, 300, 1201)
    c = oracle.softcap(z)
    np.testing.assert_array_equal(oracle.softcap(-z), -c)  # odd
    assert (np.abs(c) <= 30.0).all() and (np.diff(c) > 0)[np.abs(z[1:]) < 200].all()
    for zz in (10, 216, 1, -7.5):
        ref = float(30 * _tanh_decimal(Fraction(zz) / 30))
        assert abs(float(oracle.softcap(float(zz))) - ref) <= 1e-14 * 30
    assert abs(float(oracle.softcap(10.0)) - 9.64538212594903) < 1e-13
    assert float(oracle.softcap(868.0)) == 30.0
    # slope 1 at the origin: the cap divides then multiplies by 30
    assert abs(float(oracle.softcap(1e-6)) - 1e-6) < 1e-18
    # cap <= 0 disables
    assert oracle.softcap(123.0, cap=0).item() == 123.0
    # another cap value scales both sides
    assert abs(float(oracle.softcap(10.0, cap=15.0)) - float(15 * _tanh_decimal(Fraction(10, 15)))) < 1e-13


# ------------------------------------------------------------------ argmax --
def _brute_argmax(v):
    best, bi = None, -1
    for i, x in enumerate(v):
        if best is None or x > best:
            best, bi = x, i
    return bi


def test_argmax_and_margin_bruteforce():
    rng = np.random.default_rng(12)
    for trial in range(20):
        v = rng.standard_normal(4096)
        if trial % 4 == 1:
            v[0] = v.max() + 1.0
        if trial % 4 == 2:
            v[-1] = v.max() + 1.0
        if trial % 4 == 3:
            m = v.max() + 0.5
            v[[17, 1000, 4095]] = m
        i = oracle.first_argmax(v)
        assert i == _brute_argmax(v.tolist())
        srt = sorted(v.tolist(), reverse=True)
        assert oracle.top2_margin(v) == srt[0] - srt[1]


def test_lmhead_exact_ties_take_lowest_index():
    # integer inputs make rows 5, 77 and 299 produce exactly equal logits
    rng = np.random.default_rng(13)
    v, k = 300, 64
    codes = rng.integers(-2, 3, size=(v, k), dtype=np.int8)
    sb = np.full((v, k // 32), fp16_bits(2.0 ** -7), dtype=np.uint16)
    xi = rng.integers(-3, 4, size=k)
    x = np.array([bf16_bits(float(t)) for t in xi], dtype=np.uint16)
    planted = np.where(xi > 0, 7, np.where(xi < 0, -8, 0)).astype(np.int8)
    for r in (5, 77, 299):
        codes[r] = planted
    out = oracle.lmhead(codes, sb, x)
    assert out["idx"] == 5
    assert out["margin"] == 0.0
    exact = sum(int(planted[j]) * int(xi[j]) for j in range(k)) * Fraction(1, 128)
    assert Fraction(out["z"][5]) == exact
    assert abs(out["val"] - float(30 * _tanh_decimal(exact / 30))) < 1e-13


# -------------------------------------------------------------------- PLE --
def test_ple_golden_bits():
    q = np.array([[-127, -1, 0, 1, 127]], dtype=np.int8)
    rows = _golden_rows("ple_bits.txt")
    assert len(rows) == 3
    for row in rows:
        s = struct.unpack("<f", struct.pack("<I", int(row[0], 16)))[0]
        out, err = oracle.ple_gather(q, np.array([s], dtype=np.float32),
                                     np.array([0], dtype=np.int32), 16.0)
        assert err == 0
        got = ["%08x" % v for v in out.view(np.uint32)[0]]
        assert got == row[1:]


def test_ple_bruteforce_general_multiplier():
    # multiplier fp32(sqrt(1536)): the token-embedding normaliser quoted on
    # the mixed-bit page; the exact product needs up to 56 bits.
    rng = np.random.default_rng(14)
    table, scale, _ = synth.ple_inputs(rng, 50, 40, 1)
    ids = np.array([0, 49, 7, 7], dtype=np.int32)
    for mult in (16.0, float(np.float32(math.sqrt(1536))), 0.3):
        out, err = oracle.ple_gather(table, scale, ids, mult)
        assert err == 0
        m = Fraction(float(np.float32(mult)))
        for t, i in enumerate(ids):
            for j in range(40):
                ref = rn32(int(table[i, j]) * Fraction(float(scale[i])) * m)
                assert f32_bits(float(out[t, j])) == f32_bits(ref), (mult, t, j)


def test_ple_out_of_range_ids():
    rng = np.random.default_rng(15)
    table, scale, _ = synth.ple_inputs(rng, 10, 16, 1)
    out, err = oracle.ple_gather(table, scale, np.array([3, -1, 10, 9], dtype=np.int32))
    assert err == 1
    assert (out[1] == 0).all() and (out[2] == 0).all()
    assert (out[0] != 0).any() or (table[3] == 0).all()


def test_page_shape_constants():
    # sidecar file sizes on the Core AI card equal V x row bytes exactly
    assert synth.VOCAB * synth.SHAPES["ple_e2b"]["dim"] == 2_348_810_240
    assert synth.VOCAB * 4 == 1_048_576
    assert synth.SHAPES["ple_e2b"]["dim"] == 8960
    # the mixed-bit PLE table: 35 layer-major 128-byte INT4 blocks per row
    # (4480 bytes) hold the same 35 x 256 values per token
    assert 35 * 128 == 4480 and 4480 * 2 == synth.SHAPES["ple_e2b"]["dim"] == 35 * 256
    assert synth.SHAPES["ple_e4b"]["dim"] == 10752
    assert 16.0 == math.sqrt(256)
    assert f"{np.float32(math.sqrt(1536)):.6f}" == "39.191837"
    # E4B decode step weight bytes at 0.5625 B per weight
    mats = synth.stack_e4b_matrices()
    assert len(mats) == 42 * 4 + 1
    total = sum(n * k // 2 + n * (k // 32) * 2 for _, n, k in mats)
    assert total == 2_545_090_560


# ------------------------------------------------------------------- GELU --
def test_gelu_tanh_identities():
    import torch

    g = np.linspace(-12, 12, 4001, dtype=np.float32)
    f = oracle.gelu_tanh_f32(g)
    assert f[np.argmin(np.abs(g))] == 0.0
    # gelu(x) - gelu(-x) = x for the tanh form (tanh is odd)
    np.testing.assert_allclose(f - oracle.gelu_tanh_f32(-g), g, atol=2e-6, rtol=1e-6)
    ref = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy()
    np.testing.assert_allclose(f, ref, atol=2e-6, rtol=2e-6)
    # sanity of the bf16 host rounding used for the down GEMV input
    bits = oracle.ffn_down_input_bits(np.array([1.0], np.float32), np.array([2.0], np.float32))
    gel1 = float(oracle.gelu_tanh_f32(np.array([1.0], np.float32))[0])
    assert float(oracle.bf16_bits_to_f64(bits)[0]) == float(
        torch.tensor(gel1 * 2.0, dtype=torch.float32).to(torch.bfloat16).float())


def _bf16_rne_fraction(v: float) -> int:
    """bf16 bit pattern nearest to the finite float v, ties to an even last
    significand bit, found in exact rational arithmetic: the two bf16 values
    around v are the upper half of v's fp32 pattern and the next one away
    from zero; compare |v - lo| with |hi - v| as fractions."""
    from fractions import Fraction

    u = struct.unpack("<I", struct.pack("<f", v))[0]
    lo_bits = u >> 16
    hi_bits = lo_bits + 1  # one bf16 step further from zero (same sign)

    def val(b16: int) -> Fraction:
        return Fraction(struct.unpack("<f", struct.pack("<I", b16 << 16))[0])

    fv, lo, hi = Fraction(v), val(lo_bits), val(hi_bits)
    dlo, dhi = abs(fv - lo), abs(hi - fv)
    if dlo < dhi:
        return lo_bits
    if dhi < dlo:
        return hi_bits
    return lo_bits if lo_bits % 2 == 0 else hi_bits


def test_ffn_down_input_bits_round_half_even():
    """The down GEMV's input is the fp32 product gelu(g) * u rounded to bf16
    by round-to-nearest-even (mixed-bit page, fused gate/up kernel: fp32 GELU
    in the epilogue; the bf16 activation format of the configs). Pinned
    against an exact-rational rounding, on random products and on products
    planted exactly half-way between two bf16 values with even and with odd
    lower neighbours, both signs, plus values that are bf16 already."""
    rng = np.random.default_rng(77)
    g = rng.normal(0, 2.5, size=4000).astype(np.float32)
    u = rng.normal(0, 1.0, size=4000).astype(np.float32)
    # For g >= 16 the fp32 tanh of the GELU's argument is exactly 1, so
    # gelu(g) = g exactly and g * 1 = g: plant exact ties and exact values.
    ties = []
    for hi16 in (0x4180, 0x4181, 0x4203, 0x4204, 0x4400, 0x43FF):
        ties.append(struct.unpack("<f", struct.pack("<I", (hi16 << 16) | 0x8000))[0])  # half-way
        ties.append(struct.unpack("<f", struct.pack("<I", (hi16 << 16) | 0x7FFF))[0])  # just below
        ties.append(struct.unpack("<f", struct.pack("<I", (hi16 << 16) | 0x8001))[0])  # just above
        ties.append(struct.unpack("<f", struct.pack("<I", hi16 << 16))[0])             # exact
    gt = np.array(ties * 2, dtype=np.float32)
    ut = np.array([1.0] * len(ties) + [-1.0] * len(ties), dtype=np.float32)
    assert (oracle.gelu_tanh_f32(gt) == gt).all()
    g = np.concatenate([g, gt])
    u = np.concatenate([u, ut])
    bits = oracle.ffn_down_input_bits(g, u)
    prod = oracle.gelu_tanh_f32(g) * u  # numpy fp32 product
    want = np.array([_bf16_rne_fraction(float(p)) for p in prod], dtype=np.uint16)
    assert np.array_equal(bits, want)
    # the half-way products (every fourth planted value) land on even bf16
    # patterns, the lower neighbour for 0x4180 and the upper one for 0x4181
    n_t = len(ties)
    assert {int(b) & 1 for b in want[4000:4000 + n_t:4]} == {0}
    assert want[4000] == 0x4180 and want[4004] == 0x4182


def test_decoders_exact():
    for v in (0.0, 1.0, -2.5, 65504.0, 2.0 ** -24, 6.1e-5):
        b = fp16_bits(v)
        assert oracle.f16_bits_to_f64(np.array([b], np.uint16))[0] == float(f16_exact(b))
    rng = np.random.default_rng(16)
    xb = synth.bf16_normal(rng, 1000)
    got = oracle.bf16_bits_to_f64(xb)
    for i in range(0, 1000, 37):
        assert got[i] == float(bf16_exact(xb[i]))


# ------------------------------------------------ fused gate/up + GELU --
def _decimal_gelu(g: float) -> decimal.Decimal:
    """tanh-form GELU at 40 digits: tanh from exp (decimal module), the
    constant sqrt(2/pi) from decimal's sqrt and a 40-digit pi."""
    with decimal.localcontext() as ctx:
        ctx.prec = 40
        pi = decimal.Decimal("3.141592653589793238462643383279502884197")
        gd = decimal.Decimal(g)
        z = (decimal.Decimal(2) / pi).sqrt() * (gd + decimal.Decimal("0.044715") * gd ** 3)
        e2 = (2 * z).exp()
        return decimal.Decimal("0.5") * gd * (1 + (e2 - 1) / (e2 + 1))


def test_gelu_f64_against_decimal():
    for g in (-7.5, -3.0, -1.5, -0.25, 1e-3, 0.5, 1.0, 1.5, 2.75, 6.0):
        ref = _decimal_gelu(g)
        got = oracle.gelu_tanh_f64(np.array([g]))[0]
        # 1 + tanh cancels for negative g: the fp64 form is accurate to a few
        # ulps of |g| in absolute terms, not relative to a tiny result
        bound = abs(ref) * decimal.Decimal("1e-14") + decimal.Decimal(4 * 2.0 ** -52 * abs(g))
        assert abs(decimal.Decimal(got) - ref) <= bound, g
    # 0.5 * g * (1 + tanh(...)): an odd tanh gives gelu(g) - gelu(-g) = g
    g = np.linspace(-30, 30, 6001)
    np.testing.assert_allclose(oracle.gelu_tanh_f64(g) - oracle.gelu_tanh_f64(-g), g, rtol=0, atol=1e-12)


def test_gelu_slope_bound():
    # central differences of the decimal GELU on a grid over [-12, 12]; the
    # oracle's slope bound must cover them and not be loose by more than 10%
    h = decimal.Decimal("1e-12")
    slopes = []
    for g in np.linspace(-12, 12, 241):
        gd = float(g)
        with decimal.localcontext() as ctx:
            ctx.prec = 40
            d = (_decimal_gelu(gd + 1e-6) - _decimal_gelu(gd - 1e-6)) / decimal.Decimal(2e-6)
        slopes.append(float(d))
    assert max(abs(s) for s in slopes) <= oracle.GELU_SLOPE_MAX
    assert max(slopes) > oracle.GELU_SLOPE_MAX / 1.1
    assert min(slopes) < -0.1  # the tanh form dips below zero near g = -1.5
    del h


def test_gelu_mul_pairs_gate_and_up_rows():
    # 2h rows: g from rows 0..h-1, u from rows h..2h-1, each checked against a
    # Fraction brute-force dot product; a = gelu(g) * u at fp64 accuracy
    rng = np.random.default_rng(21)
    h, k = 3, 64
    codes, sb = synth.q4_weights(rng, 2 * h, k)
    x = synth.bf16_normal(rng, k)
    a, g, u, ag, au = oracle.gelu_mul(codes, sb, x)
    ye, ae = exact_gemv(codes, sb, x)
    for j in range(h):
        assert abs(Fraction(g[j]) - ye[j]) <= Fraction(1, 10 ** 12) * ae[j]
        assert abs(Fraction(u[j]) - ye[h + j]) <= Fraction(1, 10 ** 12) * ae[h + j]
        assert abs(Fraction(ag[j]) - ae[j]) <= Fraction(1, 10 ** 12) * ae[j]
        ref = _decimal_gelu(float(ye[j])) * decimal.Decimal(float(ye[h + j]))
        assert abs(decimal.Decimal(a[j]) - ref) <= abs(ref) * decimal.Decimal("1e-12") + decimal.Decimal("1e-200")
    with pytest.raises(ValueError):
        oracle.gelu_mul(codes[:5], sb[:5], x)


def test_gelu_mul_tolerance_covers_rounding_and_catches_swaps():
    rng = np.random.default_rng(22)
    h, k = 400, 1536
    codes, sb = synth.q4_weights(rng, 2 * h, k)
    x = synth.bf16_normal(rng, k)
    a, g, u, ag, au = oracle.gelu_mul(codes, sb, x)
    tol = oracle.gelu_mul_tolerance(g, u, ag, au)
    # the bf16 rounding of the exact value (half an ulp) is inside the bound
    import torch
    rb = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.all(np.abs(rb - a) <= tol)
    # a gate/up swap or a dropped GELU falls outside it for most outputs (the
    # GELU is close to the identity for large positive g, so not for all)
    swapped = oracle.gelu_tanh_f64(u) * g
    no_gelu = g * u
    assert np.mean(np.abs(swapped - a) > tol) > 0.85
    assert np.mean(np.abs(no_gelu - a) > tol) > 0.7
    # the bound is a few percent of the values it guards: it inherits the
    # GEMV bar 1e-4 * sum|w x|, which is loose next to |sum w x| itself
    big = np.abs(a) > 1e-3
    assert np.median(tol[big] / np.abs(a[big])) < 5e-2


# -------------------------------------------------------------- quantiser --
def _rne_int(fr: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    f = fr.numerator // fr.denominator
    rem = fr - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def _f16_rne(fr: Fraction) -> int:
    """fp16 bits of a rational, round half to even (struct's 'e' packing of
    the correctly rounded double, valid here because the doubles involved
    are exact: m / -8 or a single fp32 quotient)."""
    return struct.unpack("<H", struct.pack("<e", float(fr)))[0]


def _quantize_block_exact(xbits, rule):
    xs = [bf16_exact(b) for b in xbits]
    mags = [abs(v) for v in xs]
    j = mags.index(max(mags))  # first index of the largest magnitude
    if rule == oracle.QUANT_Q4_0:
        d = xs[j] / -8
        lo = -8
    else:
        d = Fraction(float(np.float32(float(mags[j])) / np.float32(7.0)))  # fp32 quotient, correctly rounded
        lo = -7
    dbits = _f16_rne(d)
    d16 = f16_exact(dbits)
    codes = [0] * 32 if d16 == 0 else [max(lo, min(7, _rne_int(v / d16))) for v in xs]
    return codes, dbits


@pytest.mark.parametrize("rule", [0, 1])
def test_quantize_bruteforce_fraction(rule):
    # exact rational quotients and ties-to-even against the oracle's fp32
    # division + rint; 8 x 96 random blocks plus blocks with planted ties
    rng = np.random.default_rng(40 + rule)
    x = synth.bf16_normal(rng, 8 * 96).reshape(8, 96)
    # planted: a block of exact half-way quotients (x = (i + 1/2) * d) and a
    # block whose largest magnitude appears twice with opposite signs
    half = [struct.unpack("<I", struct.pack("<f", (i - 7.5) * 0.25))[0] >> 16 for i in range(16)]
    x[0, :32] = np.array(half + half, dtype=np.uint16)
    x[1, 32:64] = 0
    x[1, 40] = struct.unpack("<I", struct.pack("<f", 3.0))[0] >> 16
    x[1, 50] = struct.unpack("<I", struct.pack("<f", -3.0))[0] >> 16
    codes, sbits, flags = oracle.q4_quantize(x, rule)
    assert not flags.any()
    for r in range(8):
        for b in range(3):
            ec, ed = _quantize_block_exact(x[r, 32 * b:32 * b + 32], rule)
            assert int(sbits[r, b]) == ed, (r, b)
            assert codes[r, 32 * b:32 * b + 32].tolist() == ec, (r, b)
    if rule == oracle.QUANT_Q4_0:
        # first of +3 / -3 wins: d = -3/8, +3 -> -8, -3 -> +8 clamped to 7
        assert codes[1, 40] == -8 and codes[1, 50] == 7


def test_quantize_invariants():
    rng = np.random.default_rng(44)
    x = synth.bf16_normal(rng, 64 * 256).reshape(64, 256)
    xf = oracle.bf16_bits_to_f64(x).reshape(64, 8, 32)
    c, s, f = oracle.q4_quantize(x, oracle.QUANT_Q4_0)
    d = oracle.f16_bits_to_f64(s)
    cb = c.reshape(64, 8, 32).astype(np.float64)
    jmax = np.argmax(np.abs(xf), axis=2)
    # the largest magnitude lands on -8 exactly (m / -8 is exact in fp16 here)
    assert np.all(np.take_along_axis(cb, jmax[..., None], axis=2) == -8)
    assert np.all(d == np.take_along_axis(xf, jmax[..., None], axis=2)[..., 0] / -8)
    # reconstruction error at most half a scale step, except where the q4_0
    # grid's missing +8 clamps a value of the other sign (quotient in
    # (7.5, 8]): there at most one step
    err = np.abs(cb * d[..., None] - xf)
    clamped = xf / d[..., None] > 7.5
    dd = np.broadcast_to(np.abs(d)[..., None], err.shape)
    assert np.all(err[~clamped] <= dd[~clamped] / 2)
    assert np.all(err[clamped] <= dd[clamped]) and np.all(cb[clamped] == 7)
    # the symmetric rule is odd: negating x negates the codes, keeps the scale
    c7, s7, _ = oracle.q4_quantize(x, oracle.QUANT_ABSMAX7)
    c7n, s7n, _ = oracle.q4_quantize(x ^ np.uint16(0x8000), oracle.QUANT_ABSMAX7)
    assert np.array_equal(c7n, -c7) and np.array_equal(s7n, s7)
    assert c7.min() >= -7 and c7.max() <= 7


def test_quantize_special_blocks():
    x = np.zeros((1, 128), dtype=np.uint16)  # block 0: all zero
    x[0, 32] = 0x7FC0                         # block 1: NaN
    x[0, 64] = 0x7F00                         # block 2: 2^127 -> scale overflows fp16
    x[0, 96:128] = 0x3F80                     # block 3: all 1.0
    c, s, f = oracle.q4_quantize(x)
    assert f.tolist() == [[False, True, True, False]]
    assert s[0, 0] == 0 and not c[0, :32].any()
    assert not c[0, 64:96].any()
    assert oracle.f16_bits_to_f64(s[0, 3:4])[0] == -0.125 and np.all(c[0, 96:] == -8)


# ------------------------------------------------ per-row INT4 / INT2 --
def test_rowq_unpack_bytes_follow_the_stated_convention():
    # INT2: 4 codes per byte, first code in bits [1:0], two's complement
    # 0xE4 = 0b11_10_01_00 -> 0, 1, -2, -1 ; 0x1B = 0b00_01_10_11 -> -1, -2, 1, 0
    b = np.array([[0xE4, 0x1B]], dtype=np.uint8)
    assert oracle.rowq_unpack(b, 1, 8, 2).tolist() == [[0, 1, -2, -1, -1, -2, 1, 0]]
    # INT4: low nibble first, two's complement: 0x8F -> -1, -8 ; 0x70 -> 0, 7
    b = np.array([[0x8F, 0x70]], dtype=np.uint8)
    assert oracle.rowq_unpack(b, 1, 4, 4).tolist() == [[-1, -8, 0, 7]]
    # INT8: signed bytes: 0x80 -> -128, 0x7F -> 127, 0xFF -> -1
    b = np.array([[0x80, 0x7F, 0xFF, 0x01]], dtype=np.uint8)
    assert oracle.rowq_unpack(b, 1, 4, 8).tolist() == [[-128, 127, -1, 1]]
    rng = np.random.default_rng(70)
    for bits in (2, 4, 8):
        c = rng.integers(-(1 << (bits - 1)), 1 << (bits - 1), size=(3, 64)).astype(np.int8)
        assert np.array_equal(oracle.rowq_unpack(oracle.rowq_pack(c, bits), 3, 64, bits), c)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_rowq_gemv_bruteforce_fraction(bits):
    rng = np.random.default_rng(71 + bits)
    n, k = 5, 128
    w = rng.integers(0, 256, size=(n, k * bits // 8), dtype=np.uint8)
    sc = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
    x = synth.bf16_normal(rng, k)
    y, a = oracle.rowq_gemv(w, sc, bits, x)
    # independent decode: walk the bytes bit by bit
    for r in range(n):
        codes = []
        for byte in w[r].tolist():
            for i in range(8 // bits):
                u = (byte >> (i * bits)) & ((1 << bits) - 1)
                codes.append(u - (1 << bits) if u >= (1 << (bits - 1)) else u)
        xs = [bf16_exact(v) for v in x]
        ye = Fraction(float(sc[r])) * sum(Fraction(c) * v for c, v in zip(codes, xs))
        ae = abs(Fraction(float(sc[r]))) * sum(abs(Fraction(c) * v) for c, v in zip(codes, xs))
        assert abs(Fraction(y[r]) - ye) <= Fraction(1, 10 ** 12) * ae
        assert abs(Fraction(a[r]) - ae) <= Fraction(1, 10 ** 12) * ae


def test_rowq_lmhead_planted_rows_and_ties():
    # INT2, k = 64, x = +1 on the first 32 elements and -1 on the rest. Row
    # codes: 1 on the +1 half and -2 on the -1 half give 32 + 64 = 96 per unit
    # scale, the row maximum. Rows 3 and 6 hold it with scale 1 (a tie: the
    # lower, 3, wins); row 5 holds it with scale 0.5 (48); the other rows are
    # zero codes. cap 0 gives the raw value; cap 30 gives 30 tanh(96 / 30).
    n, k = 8, 64
    best = np.array([1] * 32 + [-2] * 32, dtype=np.int8)
    codes = np.zeros((n, k), dtype=np.int8)
    codes[3] = codes[5] = codes[6] = best
    w = oracle.rowq_pack(codes, 2)
    sc = np.array([1, 1, 1, 1, 1, 0.5, 1, 1], dtype=np.float32)
    x = np.array([0x3F80] * 32 + [0xBF80] * 32, dtype=np.uint16)  # bf16 +1, -1
    r = oracle.rowq_lmhead(w, sc, 2, x, 0.0)
    assert r["idx"] == 3 and r["val"] == 96.0 and r["margin"] == 0.0
    r = oracle.rowq_lmhead(w, sc, 2, x, 30.0)
    assert r["idx"] == 3 and abs(r["val"] - 30.0 * math.tanh(96.0 / 30.0)) < 1e-12
    assert r["z"].tolist() == [0, 0, 0, 96, 0, 48, 96, 0]


def test_rowq_gather_hand_decoded_rows():
    # INT2 row 0xE4 -> codes 0, 1, -2, -1; scale 0.5, multiplier 2 -> the codes
    w = np.array([[0xE4], [0x1B]], dtype=np.uint8)
    out, err = oracle.rowq_gather(w, np.array([[0.5], [3.0]], dtype=np.float32), 2, 4, [0, 1, 0], 2.0)
    assert err == 0
    assert out.tolist() == [[0, 1, -2, -1], [-6, -12, 6, 0], [0, 1, -2, -1]]
    # INT4, two groups of two codes: 0x8F 0x70 -> -1, -8 | 0, 7 with scales
    # 0.25 and 4 per group, multiplier 1
    w = np.array([[0x8F, 0x70]], dtype=np.uint8)
    out, err = oracle.rowq_gather(w, np.array([[0.25, 4.0]], dtype=np.float32), 4, 2, [0], 1.0)
    assert err == 0 and out.tolist() == [[-0.25, -2.0, 0.0, 28.0]]
    # an id outside the table: zero row and the flag
    out, err = oracle.rowq_gather(w, np.array([[0.25, 4.0]], dtype=np.float32), 4, 2, [1, 0, -1], 1.0)
    assert err == 1 and out[0].tolist() == [0, 0, 0, 0] and out[2].tolist() == [0, 0, 0, 0]
    assert out[1].tolist() == [-0.25, -2.0, 0.0, 28.0]


@pytest.mark.parametrize("bits,group", [(2, 64), (2, 256), (4, 32), (4, 128)])
def test_rowq_gather_bruteforce_fraction(bits, group):
    # bytes decoded bit by bit, the product rounded from the exact rational;
    # multipliers 16 (PLE), fp32(sqrt(1536)) (token embedding) and 0.3
    rng = np.random.default_rng(75 + bits + group)
    v, dim = 6, 256
    w = rng.integers(0, 256, size=(v, dim * bits // 8), dtype=np.uint8)
    sc = rng.uniform(1e-3, 1e-2, size=(v, dim // group)).astype(np.float32)
    ids = np.array([5, 0, 3, 3], dtype=np.int32)
    for mult in (16.0, float(np.float32(math.sqrt(1536))), 0.3):
        out, err = oracle.rowq_gather(w, sc, bits, group, ids, mult)
        assert err == 0
        m = Fraction(float(np.float32(mult)))
        for t, r in enumerate(ids.tolist()):
            codes = []
            for byte in w[r].tolist():
                for i in range(8 // bits):
                    u = (byte >> (i * bits)) & ((1 << bits) - 1)
                    codes.append(u - (1 << bits) if u >= (1 << (bits - 1)) else u)
            for j in range(dim):
                ref = rn32(codes[j] * Fraction(float(sc[r, j // group])) * m)
                assert f32_bits(float(out[t, j])) == f32_bits(ref), (bits, group, mult, t, j)


def test_rowq_gelu_mul_pairs_gate_row_j_with_up_row_h_plus_j():
    # INT4, k = 32, rows [gate0, gate1, up0, up1] with constant codes 1, 0, 2, 3,
    # x = 1 and unit scales: g = (32, 0), u = (64, 96); gelu(32) = 32 to
    # double precision and gelu(0) = 0, so a = (2048, 0). Pairing row j with
    # row j + 1 instead (interleaved gate/up) would give a = (0, gelu(64) * 96).
    w = np.array([[0x11] * 16, [0x00] * 16, [0x22] * 16, [0x33] * 16], dtype=np.uint8)
    sc = np.ones(4, dtype=np.float32)
    x = np.full(32, 0x3F80, dtype=np.uint16)  # bf16 1.0
    a, g, u, ag, au = oracle.rowq_gelu_mul(w, sc, 4, x)
    assert g.tolist() == [32.0, 0.0] and u.tolist() == [64.0, 96.0]
    assert a.tolist() == [2048.0, 0.0]
    assert ag.tolist() == [32.0, 0.0] and au.tolist() == [64.0, 96.0]
    with pytest.raises(ValueError):
        oracle.rowq_gelu_mul(w[:3], sc[:3], 4, x)
