"""Activations whose values span more binades than a scaled fp16 copy holds.

The S=1 q4_0 and per-row kernels stage bf16 activations as fp16 scaled by
one power of two per group (a 32-wide block for the S=1 GEMV, the fused GELU,
the heads and the per-row formats). The S=64 GEMM, its head and the
multi-vector GEMV and head feed the activations to the matrix cores as
stored, so for them the same inputs check that nothing on that path narrows
the range (a staged copy per token or per vector would fail them). A value more than 31
binades below its group's largest (fewer on the per-row formats, whose staged
values carry an extra field shift of 2^-8 for INT2 and 2^-4 for INT4) would
lose significand bits there. On the q4_0 kernels such a group sends the
launch down the exact path, which reads x as stored; the per-row kernels
stage such a block as stored and sum it on its own in fp32, beside the
packed dot of the other blocks. These cases are built so that the scaled path
would miss the GEMV bar |y - y_ref| <= 1e-4 sum|w x| + 1e-6: an outlier whose
code is zero on every row (the rows' sums then come from values the scaled
copy flushes), and a value exactly one binade past the limit whose last
significand bit carries the row (checked beside the same value at the limit,
which the scaled path holds exactly).
"""
import struct

import numpy as np
import pytest
import torch

import int4_weight_only_block_amd as q4
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
# one binade past this span (largest minus smallest exponent field of a
# group's nonzero values) takes the exact path (the per-row formats: the
# block's own exact sum); per-row formats subtract their largest field shift
SPAN = 31
ROWQ_SPAN = {2: 23, 4: 27, 8: 31}


def d(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def bf16(v: float) -> int:
    b = struct.unpack("<I", struct.pack("<f", float(v)))[0]
    assert b & 0xFFFF == 0, f"{v} is not a bf16 value"
    return b >> 16


def fp16_bits(v: float) -> int:
    return struct.unpack("<H", struct.pack("<e", v))[0]


def within(y_gpu, y_ref, a_ref, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    tol = oracle.gemv_tolerance(a_ref)
    bad = np.nonzero(~(err <= tol))
    assert bad[0].size == 0, (f"{what}: {bad[0].size} outputs over the bar, first at {[b[:3] for b in bad]}, "
                              f"worst err/tol {float(np.max(err / tol)):.3g}")


def outlier_x(rng, shape, pos, value=2.0 ** 40):
    """bf16 N(0,1) activations with x[..., pos] = value."""
    x = synth.bf16_normal(rng, shape)
    x[..., pos] = bf16(value)
    return x


def threshold_x(rng, k, s):
    """x[0] = 2^60, x[1] = 2^(60 - s) * (1 + 127/128) (every significand bit
    set, so the last one sits s + 7 binades below 2^60), every other value
    +-U[2^39, 2^41) rounded to bf16 (within 21 binades of 2^60)."""
    mag = 2.0 ** rng.uniform(39, 41, size=k)
    sign = rng.choice([-1.0, 1.0], size=k)
    x = synth.f32_to_bf16_bits((mag * sign).astype(np.float32))
    x[0] = bf16(2.0 ** 60)
    x[1] = bf16(2.0 ** (60 - s) * (1 + 127 / 128))
    return x


def threshold_codes(rng, n, k):
    """q4_0 codes whose first half of the rows is zero except at k = 1, so
    those rows' sums are d * c * x[1] alone; the other rows random."""
    codes, sb = synth.q4_weights(rng, n, k)
    h = n // 2
    codes[:h] = 0
    codes[:h, 1] = rng.choice([-8, -5, -1, 3, 7], size=h)
    return codes, sb


# ------------------------------------------------------------ S=1 GEMV --
@pytest.mark.parametrize("n,k", [(300, 2560), (1536, 1536), (77, 10240), (64, 32)])
def test_gemv_outlier_with_zero_codes(n, k):
    rng = synth.rng_for(600, n, k)
    codes, sb = synth.q4_weights(rng, n, k)
    pos = min(k - 1, 3 * 32 + 5)
    x = outlier_x(rng, k, pos)
    codes[:, pos] = 0
    codes[::3, pos] = 5  # every third row sees the outlier
    y = q4.q4_gemv(q4.q4_pack(d(codes), d(sb)), n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemv(codes, sb, x)
    within(y, yr, a, f"gemv outlier {n}x{k}")


def test_gemv_outlier_integer_exact():
    """Power-of-two scales and integer activations beside a 2^40 outlier
    whose code is zero on every row: the exact path's sums are exact in fp32,
    so the result equals the oracle bit for bit."""
    n, k = 301, 2560
    rng = np.random.default_rng(601)
    codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    p = rng.integers(6, 9, size=(n, k // 32))
    sb = np.vectorize(lambda e: fp16_bits(2.0 ** -int(e)))(p).astype(np.uint16)
    xi = rng.integers(-8, 9, size=k).astype(np.float64)
    x = np.array([bf16(v) for v in xi], dtype=np.uint16)
    for pos in (0, 31, 1000, k - 1):
        x[pos] = bf16(2.0 ** 40)
        codes[:, pos] = 0
    y = q4.q4_gemv(q4.q4_pack(d(codes), d(sb)), n, k, d(x)).cpu().numpy()
    yr, _ = oracle.gemv(codes, sb, x)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("extra", [0, 1])
@pytest.mark.parametrize("n,k", [(256, 2560), (100, 1536)])
def test_gemv_span_threshold(n, k, extra):
    """A value whose last significand bit lies SPAN + 7 binades below the
    block maximum is held exactly by the scaled path; one binade further it
    would round there, so the exact path must take it. Half the rows carry
    only that value."""
    rng = synth.rng_for(602, n, k, extra)
    codes, sb = threshold_codes(rng, n, k)
    x = threshold_x(rng, k, SPAN + extra)
    y = q4.q4_gemv(q4.q4_pack(d(codes), d(sb)), n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemv(codes, sb, x)
    within(y, yr, a, f"gemv span {SPAN + extra}")


def test_gelu_mul_outlier():
    h, k = 600, 2560
    rng = synth.rng_for(603)
    codes, sb = synth.q4_weights(rng, 2 * h, k)
    pos = 700
    x = outlier_x(rng, k, pos)
    codes[:, pos] = 0
    got = q4.q4_gemv_gelu_mul(q4.q4_pack(d(codes), d(sb)), 2 * h, k, d(x)).cpu().numpy().view(np.uint16)
    a, g, u, ag, au = oracle.gelu_mul(codes, sb, x)
    tol = oracle.gelu_mul_tolerance(g, u, ag, au)
    err = np.abs(oracle.bf16_bits_to_f64(got) - a)
    assert (err <= tol).all(), f"{int((err > tol).sum())} outputs over the bound"


@pytest.mark.parametrize("vocab,k", [(20000, 1536), (9000, 2560)])
def test_lmhead_outlier(vocab, k):
    rng = synth.rng_for(604, vocab, k)
    codes, sb = synth.q4_weights(rng, vocab, k)
    pos = 40
    x = outlier_x(rng, k, pos)
    codes[:, pos] = 0
    ref = oracle.lmhead(codes, sb, x, 30.0)
    i, v = q4.lmhead_softcap_argmax(q4.q4_pack(d(codes), d(sb)), vocab, k, d(x), 30.0)
    assert ref["margin"] >= 1e-3
    assert int(i.item()) == ref["idx"]
    assert abs(float(v.item()) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6


# ----------------------------------------------------- multi-vector GEMV --
@pytest.mark.parametrize("m", [2, 4, 8])
def test_gemv_multi_outlier_in_one_vector(m):
    """One vector holds a 2^40 outlier with code zero on every row: a staged
    copy with one power of two per vector would flush its other values."""
    n, k = 500, 2560
    rng = synth.rng_for(605, m)
    codes, sb = synth.q4_weights(rng, n, k)
    x = synth.bf16_normal(rng, (m, k))
    x[m - 1, 1234] = bf16(2.0 ** 40)
    codes[:, 1234] = 0
    y = q4.q4_gemv_multi(q4.q4_pack(d(codes), d(sb)), n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemm(codes, sb, x)
    within(y, yr, a, f"multi m={m} outlier")


@pytest.mark.parametrize("extra", [0, 1])
def test_gemv_multi_span_threshold(extra):
    n, k, m = 256, 2560, 4
    rng = synth.rng_for(606, extra)
    codes, sb = threshold_codes(rng, n, k)
    x = np.stack([threshold_x(rng, k, SPAN + extra) for _ in range(m)])
    y = q4.q4_gemv_multi(q4.q4_pack(d(codes), d(sb)), n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemm(codes, sb, x)
    within(y, yr, a, f"multi span {SPAN + extra}")


def test_lmhead_multi_outlier():
    vocab, k, m = 12000, 2560, 4
    rng = synth.rng_for(607)
    codes, sb = synth.q4_weights(rng, vocab, k)
    x = synth.bf16_normal(rng, (m, k))
    x[2, 99] = bf16(2.0 ** 40)
    codes[:, 99] = 0
    i, v = q4.lmhead_softcap_argmax_multi(q4.q4_pack(d(codes), d(sb)), vocab, k, d(x), 30.0)
    i, v = i.cpu().numpy(), v.cpu().numpy()
    for r in range(m):
        ref = oracle.lmhead(codes, sb, x[r], 30.0)
        assert ref["margin"] >= 1e-3
        assert int(i[r]) == ref["idx"], r
        assert abs(float(v[r]) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6


# --------------------------------------------------------- S=64 GEMM --
@pytest.mark.parametrize("n,k,n_tok", [(3072, 2560, 64), (2560, 2048, 64), (20480, 2560, 17), (300, 1536, 5)])
def test_gemm_s64_outlier_in_one_token(n, k, n_tok):
    """A token with a 2^40 outlier whose code is zero on every row: a copy
    scaled by one power of two per token would flush its other values. Covers
    split-K shapes (QKV, O) and an unsplit one (gate+up)."""
    rng = synth.rng_for(608, n, k, n_tok)
    codes, sb = synth.q4_weights(rng, n, k)
    x = synth.bf16_normal(rng, (n_tok, k))
    x[n_tok // 2, 777] = bf16(2.0 ** 40)
    codes[:, 777] = 0
    y = q4.q4_gemm_s64(q4.q4_pack(d(codes), d(sb)), n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemm(codes, sb, x)
    within(y, yr, a, f"gemm outlier {n}x{k} s={n_tok}")


@pytest.mark.parametrize("extra", [0, 1])
def test_gemm_s64_span_threshold(extra):
    n, k, n_tok = 512, 2560, 64
    rng = synth.rng_for(609, extra)
    codes, sb = threshold_codes(rng, n, k)
    x = np.stack([threshold_x(rng, k, SPAN + extra) for _ in range(n_tok)])
    y = q4.q4_gemm_s64(q4.q4_pack(d(codes), d(sb)), n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemm(codes, sb, x)
    within(y, yr, a, f"gemm span {SPAN + extra}")


def test_lmhead_s64_outlier():
    vocab, k, n_tok = 8192, 2560, 9
    rng = synth.rng_for(610)
    codes, sb = synth.q4_weights(rng, vocab, k)
    x = synth.bf16_normal(rng, (n_tok, k))
    x[4, 2000] = bf16(2.0 ** 40)
    codes[:, 2000] = 0
    i, v = q4.lmhead_softcap_argmax_s64(q4.q4_pack(d(codes), d(sb)), vocab, k, d(x), 30.0)
    i, v = i.cpu().numpy(), v.cpu().numpy()
    for r in range(n_tok):
        ref = oracle.lmhead(codes, sb, x[r], 30.0)
        if ref["margin"] >= 1e-3:
            assert int(i[r]) == ref["idx"], r
        assert abs(float(v[r]) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6


# ------------------------------------------------------ per-row formats --
def _rowq(rng, n, k, bits):
    w = rng.integers(0, 256, size=(n, k * bits // 8), dtype=np.uint8)
    sc = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
    return w, sc


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_rowq_outlier_with_zero_codes(bits):
    n, k = 400, 3072
    rng = synth.rng_for(611, bits)
    w, sc = _rowq(rng, n, k, bits)
    codes = oracle.rowq_unpack(w, n, k, bits)
    pos = 517
    codes[:, pos] = 0
    w = oracle.rowq_pack(codes, bits)
    x = outlier_x(rng, k, pos)
    y = q4.rowq_gemv(d(w), d(sc), n, k, bits, d(x)).cpu().numpy()
    yr, a = oracle.rowq_gemv(w, sc, bits, x)
    within(y, yr, a, f"rowq int{bits} outlier")
    ref = oracle.rowq_lmhead(w, sc, bits, x, 30.0)
    i, v = q4.rowq_softcap_argmax(d(w), d(sc), n, k, bits, d(x), 30.0)
    if ref["margin"] >= 1e-3:
        assert int(i.item()) == ref["idx"]
    assert abs(float(v.item()) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6
    got = q4.rowq_gemv_gelu_mul(d(w), d(sc), n, k, bits, d(x)).cpu().numpy().view(np.uint16)
    a_ref, g, u, ag, au = oracle.rowq_gelu_mul(w, sc, bits, x)
    tol = oracle.gelu_mul_tolerance(g, u, ag, au)
    assert (np.abs(oracle.bf16_bits_to_f64(got) - a_ref) <= tol).all()


@pytest.mark.parametrize("extra", [0, 1])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_rowq_span_threshold(bits, extra):
    """The per-row formats' limit is SPAN minus the largest field shift."""
    n, k = 256, 1536
    s = ROWQ_SPAN[bits] + extra
    rng = synth.rng_for(612, bits, extra)
    w, sc = _rowq(rng, n, k, bits)
    codes = oracle.rowq_unpack(w, n, k, bits)
    h = n // 2
    codes[:h] = 0
    lim = (1 << (bits - 1)) - 1
    codes[:h, 1] = rng.choice([-lim - 1, -1, 1, lim], size=h)
    w = oracle.rowq_pack(codes, bits)
    x = threshold_x(rng, k, s)
    y = q4.rowq_gemv(d(w), d(sc), n, k, bits, d(x)).cpu().numpy()
    yr, a = oracle.rowq_gemv(w, sc, bits, x)
    within(y, yr, a, f"rowq int{bits} span {s}")


@pytest.mark.parametrize("pattern", ["all", "alternate"])
@pytest.mark.parametrize("bits,k", [(2, 3072), (2, 2112), (4, 2080), (8, 2080)])
def test_rowq_many_wide_blocks(bits, k, pattern):
    """Wide blocks are summed one by one beside the packed dot: every block
    (or every other one) carries an outlier of 2^40 whose code is zero on
    every row, so lanes hold several wide blocks, both blocks of an INT2
    chunk are wide, and k leaves a ragged last round of chunks."""
    n = 300
    rng = synth.rng_for(613, bits, k, pattern == "all")
    w, sc = _rowq(rng, n, k, bits)
    codes = oracle.rowq_unpack(w, n, k, bits)
    blocks = range(0, k // 32, 1 if pattern == "all" else 2)
    pos = [32 * b + int(rng.integers(0, 32)) for b in blocks]
    codes[:, pos] = 0
    w = oracle.rowq_pack(codes, bits)
    x = synth.bf16_normal(rng, k)
    x[pos] = bf16(2.0 ** 40)
    y = q4.rowq_gemv(d(w), d(sc), n, k, bits, d(x)).cpu().numpy()
    yr, a = oracle.rowq_gemv(w, sc, bits, x)
    within(y, yr, a, f"rowq int{bits} k={k} {pattern} wide")
    ref = oracle.rowq_lmhead(w, sc, bits, x, 30.0)
    i, v = q4.rowq_softcap_argmax(d(w), d(sc), n, k, bits, d(x), 30.0)
    if ref["margin"] >= 1e-3:
        assert int(i.item()) == ref["idx"]
    assert abs(float(v.item()) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6
    got = q4.rowq_gemv_gelu_mul(d(w), d(sc), n, k, bits, d(x)).cpu().numpy().view(np.uint16)
    a_ref, g, u, ag, au = oracle.rowq_gelu_mul(w, sc, bits, x)
    tol = oracle.gelu_mul_tolerance(g, u, ag, au)
    assert (np.abs(oracle.bf16_bits_to_f64(got) - a_ref) <= tol).all()
