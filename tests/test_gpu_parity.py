"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: bit-exact for packing (one-hot column sweep), integer-exact GEMV cases
and the PLE gather; |y - y_ref| <= 1e-4 * sum|w x| + 1e-6 for fp32-accumulated
GEMV outputs; exact argmax indices when the top-2 margin of the capped logits
is >= 1e-3 (smaller margins are excluded and counted), capped value within the
GEMV tolerance of the winning row.
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


def d(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def fp16_bits(v: float) -> int:
    return struct.unpack("<H", struct.pack("<e", v))[0]


def bf16_bits_of_ints(vals) -> np.ndarray:
    out = np.array([struct.unpack("<I", struct.pack("<f", float(v)))[0] >> 16 for v in vals], dtype=np.uint16)
    return out


def pack(codes, sb):
    return q4.q4_pack(d(codes), d(sb))


def assert_within_tol(y_gpu, y_ref, a_ref, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    tol = oracle.gemv_tolerance(a_ref)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, (f"{what}: {bad.size} outputs over tolerance, first {bad[:5]}, "
                           f"err/tol {float(np.max(err / tol)):.3g}")
    return float(np.max(err / tol))


# K values covering every (lanes per row, blocks per lane) kernel variant,
# including ragged block counts
K_VARIANTS = [32, 64, 96, 160, 1536, 2048, 2560, 3072, 4096, 5120, 6144, 8192, 10240, 12288, 14336, 16384]


@pytest.mark.parametrize("k", K_VARIANTS)
def test_gemv_integer_exact(k):
    """Power-of-two scales and integer activations: every partial sum is
    exact in fp32 in any order, so the GPU must equal the oracle bit-exactly."""
    rng = np.random.default_rng(100 + k)
    n = 77 if k > 4096 else 301  # ragged row counts: not a multiple of any row-group size
    codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    p = rng.integers(6, 9, size=(n, k // 32))
    sb = np.vectorize(lambda e: fp16_bits(2.0 ** -int(e)))(p).astype(np.uint16)
    x = bf16_bits_of_ints(rng.integers(-8, 9, size=k))
    y = q4.q4_gemv(pack(codes, sb), n, k, d(x)).cpu().numpy()
    yr, _ = oracle.gemv(codes, sb, x)
    assert np.array_equal(y.astype(np.float64), yr)


def test_degenerate_inputs_all_q4_paths():
    """All-zero codes and all-zero activations through the multi-vector GEMV,
    the S=64 GEMM, the fused GELU and the three heads: every sum is exactly
    zero, so outputs are exact zeros, GELU(0) * 0 is +0 in bf16, and each
    head returns row 0 (the lowest of equal maxima) with value 0. Extreme
    codes -8 / 7 stay within the GEMV bar on the matrix-core paths."""
    rng = synth.rng_for(2)
    n, k = 300, 2560
    codes, sb = synth.q4_weights(rng, n, k)
    zero_w = pack(np.zeros_like(codes), sb)
    packed = pack(codes, sb)
    xs = synth.bf16_normal(rng, (64, k))
    zx = np.zeros((64, k), np.uint16)
    for w, x in ((zero_w, xs), (packed, zx)):
        for m in (2, 4, 8):
            assert (q4.q4_gemv_multi(w, n, k, d(x[:m])).cpu().numpy() == 0).all(), m
        for t in (1, 17, 64):
            assert (q4.q4_gemm_s64(w, n, k, d(x[:t])).cpu().numpy() == 0).all(), t
        a = q4.q4_gemv_gelu_mul(w, n, k, d(x[0])).cpu().numpy().view(np.uint16)
        assert (a == 0).all()
        i, v = q4.lmhead_softcap_argmax(w, n, k, d(x[0]), 30.0)
        assert int(i.item()) == 0 and float(v.item()) == 0.0
        i, v = q4.lmhead_softcap_argmax_multi(w, n, k, d(x[:5]), 30.0)
        assert (i.cpu().numpy() == 0).all() and (v.cpu().numpy() == 0).all()
        i, v = q4.lmhead_softcap_argmax_s64(w, n, k, d(x[:33]), 30.0)
        assert (i.cpu().numpy() == 0).all() and (v.cpu().numpy() == 0).all()
    for c in (-8, 7):
        cc = np.full_like(codes, c)
        w = pack(cc, sb)
        yr, a = oracle.gemm(cc, sb, xs[:4])
        y = q4.q4_gemv_multi(w, n, k, d(xs[:4])).cpu().numpy()
        for r in range(4):
            assert_within_tol(y[r], yr[r], a[r], f"multi codes {c}")
        y = q4.q4_gemm_s64(w, n, k, d(xs[:4])).cpu().numpy()
        for r in range(4):
            assert_within_tol(y[r], yr[r], a[r], f"gemm codes {c}")


@pytest.mark.parametrize("n,k", [(1536, 1536), (1, 1536), (3, 32), (1000, 2560), (513, 10240), (64, 16384)])
def test_gemv_random_tolerance(n, k):
    rng = synth.rng_for(0, n, k)
    codes, sb = synth.q4_weights(rng, n, k)
    x = synth.bf16_normal(rng, k)
    y = q4.q4_gemv(pack(codes, sb), n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemv(codes, sb, x)
    assert_within_tol(y, yr, a, f"gemv {n}x{k}")


def test_pack_layout_onehot_full_sweep():
    """x = e_k for every k of the 1536 x 1536 matrix returns column k exactly:
    a complete pin of the packed layout, the nibble offset and scale indexing."""
    n = k = 1536
    rng = synth.rng_for(0)
    codes, sb = synth.q4_weights(rng, n, k)
    packed = pack(codes, sb)
    eye = np.zeros((k, k), dtype=np.uint16)
    eye[np.arange(k), np.arange(k)] = 0x3F80  # bf16 1.0
    xs = d(eye)
    out = torch.empty((k, n), dtype=torch.float32, device=DEV)
    for kk in range(k):
        q4.q4_gemv(packed, n, k, xs[kk], out[kk])
    got = out.cpu().numpy().T.astype(np.float64)
    assert np.array_equal(got, oracle.dequant(codes, sb))


def test_gemv_degenerate_inputs():
    rng = synth.rng_for(1)
    n, k = 300, 2560
    codes, sb = synth.q4_weights(rng, n, k)
    x = synth.bf16_normal(rng, k)
    # all-zero codes: exactly zero
    y = q4.q4_gemv(pack(np.zeros_like(codes), sb), n, k, d(x)).cpu().numpy()
    assert (y == 0).all()
    # all-zero activations: exactly zero
    packed = pack(codes, sb)
    y = q4.q4_gemv(packed, n, k, d(np.zeros(k, np.uint16))).cpu().numpy()
    assert (y == 0).all()
    # extreme codes -8 / 7
    for c in (-8, 7):
        cc = np.full_like(codes, c)
        y = q4.q4_gemv(pack(cc, sb), n, k, d(x)).cpu().numpy()
        yr, a = oracle.gemv(cc, sb, x)
        assert_within_tol(y, yr, a, f"codes {c}")
    # wide dynamic range of activations inside one block and across blocks
    xf = rng.standard_normal(k).astype(np.float32)
    xf[::7] *= 1e20
    xf[3::11] *= 1e-25
    xf[64:96] *= 1e-30
    xw = synth.f32_to_bf16_bits(xf)
    y = q4.q4_gemv(packed, n, k, d(xw)).cpu().numpy()
    yr, a = oracle.gemv(codes, sb, xw)
    assert_within_tol(y, yr, a, "wide range")


def test_pack_err_flag():
    codes = np.zeros((4, 64), dtype=np.int8)
    sb = np.full((4, 2), fp16_bits(1.0), dtype=np.uint16)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    q4.q4_pack(d(codes), d(sb), err_flag=flag)
    assert int(flag.item()) == 0
    codes[2, 5] = 9
    q4.q4_pack(d(codes), d(sb), err_flag=flag)
    assert int(flag.item()) == 1


def test_ffn_pair():
    """E2B FFN: fused gate+up GEMV [2*6144, 1536], host fp32 GELU-tanh * up
    rounded to bf16, down GEMV [1536, 6144]. The oracle's bf16 product feeds
    both sides so each GEMV is checked on its own."""
    s = synth.SHAPES["ffn_e2b"]
    rng = synth.rng_for(0, 2)
    gu_codes, gu_sb = synth.q4_weights(rng, *s["gate_up"])
    dn_codes, dn_sb = synth.q4_weights(rng, *s["down"])
    x = synth.bf16_normal(rng, s["gate_up"][1])
    gu = q4.q4_gemv(pack(gu_codes, gu_sb), *s["gate_up"], d(x)).cpu().numpy()
    gur, gua = oracle.gemv(gu_codes, gu_sb, x)
    assert_within_tol(gu, gur, gua, "gate_up")
    inter = s["inter"]
    a_bits = oracle.ffn_down_input_bits(gur[:inter].astype(np.float32), gur[inter:].astype(np.float32))
    y = q4.q4_gemv(pack(dn_codes, dn_sb), *s["down"], d(a_bits)).cpu().numpy()
    yr, ya = oracle.gemv(dn_codes, dn_sb, a_bits)
    assert_within_tol(y, yr, ya, "down")


# ------------------------------------------------- multi-vector GEMV --
@pytest.mark.parametrize("m,n,k", [(2, 1536, 1536), (3, 777, 96), (4, 3072, 2560), (4, 2560, 10240),
                                   (8, 2560, 2048), (5, 5, 32), (4, 20480, 2560), (7, 1000, 6144),
                                   (2, 300, 16384)])
def test_gemv_multi_tolerance(m, n, k):
    rng = synth.rng_for(60, m, n, k)
    codes, sb = synth.q4_weights(rng, n, k)
    xs = synth.bf16_normal(rng, m * k).reshape(m, k)
    y = q4.q4_gemv_multi(pack(codes, sb), n, k, d(xs)).cpu().numpy()
    yr, a = oracle.gemm(codes, sb, xs)
    assert_within_tol(y.ravel(), yr.ravel(), a.ravel(), f"multi m={m}")


@pytest.mark.parametrize("k", [64, 1536, 2560, 10240])
def test_gemv_multi_integer_exact(k):
    n, m = 515, 4
    rng = synth.rng_for(61, k)
    codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    sb = np.full((n, k // 32), fp16_bits(2.0 ** -6), dtype=np.uint16)
    xi = rng.integers(-4, 5, size=(m, k))
    xs = np.stack([bf16_bits_of_ints(r) for r in xi])
    y = q4.q4_gemv_multi(pack(codes, sb), n, k, d(xs)).cpu().numpy()
    want = (codes.astype(np.int64) @ xi.T.astype(np.int64)).T / 64.0
    assert np.array_equal(y.astype(np.float64), want)


def test_gemv_multi_lds_limit_and_m1():
    n, k = 64, 16384
    rng = synth.rng_for(62)
    codes, sb = synth.q4_weights(rng, n, k)
    packed = pack(codes, sb)
    xs = synth.bf16_normal(rng, 8 * k).reshape(8, k)
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_gemv_multi(packed, n, k, d(xs))
    assert e.value.code == q4.ERR_UNSUPPORTED
    y1 = q4.q4_gemv_multi(packed, n, k, d(xs[:1])).cpu().numpy()
    y0 = q4.q4_gemv(packed, n, k, d(xs[0])).cpu().numpy()
    assert np.array_equal(y1[0], y0)


# ---------------------------------------------- per-row INT4 / INT2 GEMV --
def _rowq_inputs(rng, n, k, bits):
    w = rng.integers(0, 256, size=(n, k * bits // 8), dtype=np.uint8)  # uniform codes
    sc = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
    x = synth.bf16_normal(rng, k)
    return w, sc, x


# the mixed-bit E2B decode shapes (INT2 FFN L15-34 and the INT2 head, INT4 FFN
# L0-14 and attention q/o), ragged row counts, and every lane split
@pytest.mark.parametrize("bits,n,k", [(2, 12288, 1536), (2, 1536, 12288), (2, 262144, 1536), (4, 6144, 1536),
                                      (4, 1536, 6144), (4, 2048, 1536), (4, 1536, 2048), (2, 77, 64), (4, 301, 32),
                                      (2, 515, 4096), (4, 1000, 16384), (2, 33, 16384), (4, 129, 960),
                                      # INT8: PLE gate [256, 1536], projection [1536, 256] and the
                                      # per-layer model projection [8960, 1536]; ragged and wide
                                      (8, 256, 1536), (8, 1536, 256), (8, 8960, 1536), (8, 77, 32), (8, 301, 96),
                                      (8, 1000, 16384), (8, 3000, 5120)])
def test_rowq_gemv_tolerance(bits, n, k):
    rng = synth.rng_for(80, bits, n, k)
    w, sc, x = _rowq_inputs(rng, n, k, bits)
    y = q4.rowq_gemv(d(w), d(sc), n, k, bits, d(x)).cpu().numpy()
    yr, a = oracle.rowq_gemv(w, sc, bits, x)
    assert_within_tol(y, yr, a, f"rowq int{bits}")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_rowq_gemv_integer_exact(bits):
    n, k = 700, 3072
    rng = synth.rng_for(81, bits)
    w = rng.integers(0, 256, size=(n, k * bits // 8), dtype=np.uint8)
    sc = np.full(n, 2.0 ** -5, dtype=np.float32)
    xi = rng.integers(-4, 5, size=k)
    y = q4.rowq_gemv(d(w), d(sc), n, k, bits, d(bf16_bits_of_ints(xi))).cpu().numpy()
    codes = oracle.rowq_unpack(w, n, k, bits).astype(np.int64)
    assert np.array_equal(y.astype(np.float64), (codes @ xi) / 32.0)


@pytest.mark.parametrize("bits,n,k", [(2, 1536, 1536), (2, 12288, 1536), (2, 1536, 12288), (4, 2048, 1536),
                                      (4, 1536, 6144), (8, 256, 1536), (8, 8960, 1536)])
def test_rowq_gemv_degenerate_rows(bits, n, k):
    """Rows whose codes are all zero (and rows with a single nonzero code)
    among random rows, with N(0,1) activations: every output, the zero rows'
    included, must meet the GEMV bar, whose floor is 1e-6 where sum|w x| is
    zero; zero activations give exactly zero."""
    rng = synth.rng_for(88, bits, n, k)
    w, sc, x = _rowq_inputs(rng, n, k, bits)
    w[::3] = 0
    one = np.arange(1, n, 7)
    w[one] = 0
    w[one, rng.integers(0, w.shape[1], size=one.size)] = 1  # one code of 1 per row
    y = q4.rowq_gemv(d(w), d(sc), n, k, bits, d(x)).cpu().numpy()
    yr, a = oracle.rowq_gemv(w, sc, bits, x)
    assert_within_tol(y, yr, a, f"rowq int{bits} degenerate rows")
    zx = d(np.zeros(k, np.uint16))
    y0 = q4.rowq_gemv(d(w), d(sc), n, k, bits, zx).cpu().numpy()
    assert (y0 == 0).all()
    # the head and the fused GELU on the same rows: all logits 0 -> row 0, value 0
    i, v = q4.rowq_softcap_argmax(d(w), d(sc), n, k, bits, zx, 30.0)
    assert int(i.item()) == 0 and float(v.item()) == 0.0
    if n % 2 == 0 and k <= q4.GELU_MAX_K:
        a = q4.rowq_gemv_gelu_mul(d(w), d(sc), n, k, bits, zx).cpu().numpy().view(np.uint16)
        assert (a == 0).all()
    # degenerate rows through the head: the winner is the oracle's when clear
    ref = oracle.rowq_lmhead(w, sc, bits, x, 30.0)
    i, v = q4.rowq_softcap_argmax(d(w), d(sc), n, k, bits, d(x), 30.0)
    if ref["margin"] >= 1e-3:
        assert int(i.item()) == ref["idx"]
    assert abs(float(v.item()) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6


# fused [gate; up] GELU on the per-row formats: the E2B INT2 and INT4 FFN
# halves, ragged output counts, and the widest supported k
@pytest.mark.parametrize("bits,h,k", [(2, 12288, 1536), (4, 6144, 1536), (2, 77, 64), (4, 301, 32),
                                      (2, 515, 6144), (4, 1000, 6144), (2, 33, 4096), (4, 129, 960),
                                      (8, 256, 1536), (8, 77, 96), (8, 1000, 6144)])
def test_rowq_gelu_mul_tolerance(bits, h, k):
    rng = synth.rng_for(82, bits, h, k)
    w, sc, x = _rowq_inputs(rng, 2 * h, k, bits)
    bits_out = q4.rowq_gemv_gelu_mul(d(w), d(sc), 2 * h, k, bits, d(x)).cpu().numpy().view(np.uint16)
    got = oracle.bf16_bits_to_f64(bits_out)
    a, g, u, ag, au = oracle.rowq_gelu_mul(w, sc, bits, x)
    tol = oracle.gelu_mul_tolerance(g, u, ag, au)
    bad = np.nonzero(~(np.abs(got - a) <= tol))[0]
    assert bad.size == 0, (f"{bad.size} of {h} over the bound, first {bad[:5]}, "
                           f"got {got[bad[:3]]} want {a[bad[:3]]} tol {tol[bad[:3]]}")


@pytest.mark.parametrize("bits", [2, 4])
def test_rowq_gelu_mul_integer_inputs_match_host_epilogue(bits):
    """Power-of-two row scales and x in {-1, 0, 1}: g and u are exact in fp32
    on both sides, so the result may differ from the host fp32 GELU-tanh
    product rounded to bf16 only through the two tanh implementations. The
    scale 2^-8 keeps |g| below about 3: far down the negative tail (g near
    -10) fp32's 1 + tanh cancels to a few bits and two correct fp32 GELUs
    part by many ulps, which the tolerance test above covers instead."""
    h, k = 4096, 1536
    rng = synth.rng_for(83, bits)
    w = rng.integers(0, 256, size=(2 * h, k * bits // 8), dtype=np.uint8)
    sc = np.full(2 * h, 2.0 ** -8, dtype=np.float32)
    x = bf16_bits_of_ints(rng.integers(-1, 2, size=k))
    got = q4.rowq_gemv_gelu_mul(d(w), d(sc), 2 * h, k, bits, d(x)).cpu().numpy().view(np.uint16)
    _, g, u, _, _ = oracle.rowq_gelu_mul(w, sc, bits, x)
    assert np.all(g.astype(np.float32) == g) and np.all(u.astype(np.float32) == u)
    want = oracle.ffn_down_input_bits(g.astype(np.float32), u.astype(np.float32))
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    same_sign = (got >> 15) == (want >> 15)
    assert np.all(same_sign | (diff == 0) | (np.abs(oracle.bf16_bits_to_f64(want)) < 1e-30))
    assert diff.max() <= 1, diff.max()
    assert np.mean(diff == 0) > 0.99


def test_rowq_int2_ffn_chain():
    """One E2B INT2 FFN layer (gate and up [12288, 1536], down [1536, 12288])
    as the fused launch plus the down GEMV on its bf16 output; the down GEMV
    is checked against the oracle fed the GPU's own a."""
    rng = synth.rng_for(84)
    w_gu, sc_gu, x = _rowq_inputs(rng, 2 * 12288, 1536, 2)
    w_dn = rng.integers(0, 256, size=(1536, 12288 // 4), dtype=np.uint8)
    sc_dn = rng.uniform(1e-3, 1e-2, size=1536).astype(np.float32)
    a_gpu = q4.rowq_gemv_gelu_mul(d(w_gu), d(sc_gu), 2 * 12288, 1536, 2, d(x))
    y = q4.rowq_gemv(d(w_dn), d(sc_dn), 1536, 12288, 2, a_gpu).cpu().numpy()
    a_bits = a_gpu.cpu().numpy().view(np.uint16)
    a, g, u, ag, au = oracle.rowq_gelu_mul(w_gu, sc_gu, 2, x)
    assert np.all(np.abs(oracle.bf16_bits_to_f64(a_bits) - a) <= oracle.gelu_mul_tolerance(g, u, ag, au))
    yr, am = oracle.rowq_gemv(w_dn, sc_dn, 2, a_bits)
    assert_within_tol(y, yr, am, "rowq int2 down")


# the tied per-row head: softcap + argmax fused over the rowq logits
def _check_rowq_head(w, sc, bits, x, cap=30.0, ws=None):
    vocab = w.shape[0]
    k = x.size
    i, v = q4.rowq_softcap_argmax(d(w), d(sc), vocab, k, bits, d(x), cap, ws)
    gi, gv = int(i.item()), float(v.item())
    ref = oracle.rowq_lmhead(w, sc, bits, x, cap)
    c, ri = ref["capped"], ref["idx"]
    if ref["margin"] >= 1e-3:
        assert gi == ri, (vocab, k, bits, gi, ri, ref["margin"])
    else:
        _, am = oracle.rowq_gemv(w, sc, bits, x)  # the GEMV bar's sum of |terms| per row
        assert 0 <= gi < vocab and c[ri] - c[gi] < 1e-3 + 1e-4 * am[gi] + 1e-6
    assert abs(gv - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6, (gv, ref["val"])
    return ref["margin"] < 1e-3


def test_rowq_head_e2b_int2_tied_head():
    """The INT2 [262144, 1536] embedding used as the head, four vectors."""
    rng = synth.rng_for(85)
    w, sc, _ = _rowq_inputs(rng, 262144, 1536, 2)
    ws = torch.zeros(q4.rowq_head_workspace_bytes(262144, 1536, 2), dtype=torch.uint8, device=DEV)
    excluded = sum(_check_rowq_head(w, sc, 2, synth.bf16_normal(rng, 1536), ws=ws) for _ in range(4))
    assert excluded <= 1


@pytest.mark.parametrize("bits,vocab,k", [(2, 1, 64), (2, 3, 128), (2, 1000, 1536), (2, 70001, 2048),
                                          (2, 4099, 12288), (4, 1, 32), (4, 777, 1536), (4, 70001, 2560),
                                          (4, 3000, 16384), (8, 5, 32), (8, 20001, 1536), (8, 999, 10240)])
def test_rowq_head_shapes(bits, vocab, k):
    rng = synth.rng_for(86, bits, vocab, k)
    w, sc, x = _rowq_inputs(rng, vocab, k, bits)
    _check_rowq_head(w, sc, bits, x)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_rowq_head_planted_ties_and_raw_values(bits):
    """Integer activations and a power-of-two scale make every logit exact:
    rows planted with the sign pattern of x hold the unique maximum, the
    lowest planted row must win across and within workgroups, and cap <= 0
    returns the exact raw logit."""
    vocab, k = (262144, 1536) if bits == 2 else (40000, 1536)
    rng = synth.rng_for(87, bits)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    w0 = rng.integers(0, 256, size=(vocab, k * bits // 8), dtype=np.uint8)
    w0[:, 0] &= np.uint8((0xFF << bits) & 0xFF)  # code 0 of every row is 0 ...
    xi = rng.integers(-3, 4, size=k)
    xi[0] = 4  # ... so no random row reaches the planted sum
    planted = np.where(xi > 0, hi, np.where(xi < 0, lo, 0)).astype(np.int8)
    prow = oracle.rowq_pack(planted[None, :], bits)[0]
    sc = np.full(vocab, 2.0 ** -9, dtype=np.float32)
    scd = d(sc)
    x = d(bf16_bits_of_ints(xi))
    zr = float(int(planted.astype(np.int64) @ xi)) * 2.0 ** -9
    last = vocab - 1
    for rows, expect in [((5, 77777 % vocab, last), 5), ((last,), last), ((0, last), 0),
                         ((1023, 1024, 4096), 1023), ((64, 63), 63)]:
        ww = w0.copy()
        for r in rows:
            ww[r] = prow
        w = d(ww)
        i, v = q4.rowq_softcap_argmax(w, scd, vocab, k, bits, x, 30.0)
        assert int(i.item()) == expect, rows
        assert abs(float(v.item()) - float(oracle.softcap(zr))) <= 1e-6 + 1e-4 * abs(zr)
        i, v = q4.rowq_softcap_argmax(w, scd, vocab, k, bits, x, 0.0)
        assert int(i.item()) == expect and float(v.item()) == zr


# -------------------------------------------------------------- quantiser --
def _quantize_gpu(x, rule):
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    c, sc = q4.q4_quantize(d(x), rule, err_flag=err)
    return c.cpu().numpy(), sc.cpu().numpy().view(np.uint16), int(err.item())


@pytest.mark.parametrize("rule", [q4.QUANT_Q4_0, q4.QUANT_ABSMAX7])
@pytest.mark.parametrize("n,k", [(12288, 1536), (3, 32), (777, 96), (64, 16384)])
def test_quantize_bit_exact(rule, n, k):
    rng = synth.rng_for(50, n, k, rule)
    x = synth.bf16_normal(rng, n * k).reshape(n, k)
    c, sc, err = _quantize_gpu(x, rule)
    rc, rs, rf = oracle.q4_quantize(x, rule)
    assert np.array_equal(sc, rs)
    assert np.array_equal(c, rc)
    assert err == int(rf.any()) == 0


@pytest.mark.parametrize("rule", [q4.QUANT_Q4_0, q4.QUANT_ABSMAX7])
def test_quantize_special_blocks(rule):
    def b(v):
        return struct.unpack("<I", struct.pack("<f", v))[0] >> 16
    x = np.zeros((4, 256), dtype=np.uint16)
    x[0, 32:64] = [b((i - 15.5) * 0.25) for i in range(32)]         # half-way quotients
    x[0, 64:96] = 0x8000                                              # -0 block
    x[0, 100], x[0, 110] = b(3.0), b(-3.0)                            # equal magnitudes, both signs
    x[0, 128:160] = b(2.0 ** -130)                        # bf16 denormals
    x[1, :32] = np.arange(32, dtype=np.uint16) | 0x0100               # tiny normals
    x[2, :] = synth.bf16_normal(synth.rng_for(51), 256)
    x[2, 40] = b(1e5)                                                 # one outlier in a block
    x[3, 0:32] = b(1.0)
    x[3, 33] = 0x7FC0                                                 # NaN in block 1
    x[3, 64] = 0x7F70                                                 # scale overflows fp16
    # exact ties x / d16 = j + 1/2 with d16 = 31/64, whose reciprocal is not
    # exact (x * RN(1/d) lands a few ulps off the half): block 2 of row 1 has
    # q4_0's scale (largest magnitude -3.875), block 3 the absmax/7 one
    # (largest 217/64)
    halves = [s * (2 * j + 1) * 31 / 128 for j in range(4) for s in (1, -1)]
    x[1, 64] = b(-3.875)
    x[1, 65:73] = [b(v) for v in halves]
    x[1, 96] = b(217 / 64)
    x[1, 97:105] = [b(v) for v in halves]
    c, sc, err = _quantize_gpu(x, rule)
    rc, rs, rf = oracle.q4_quantize(x, rule)
    assert np.array_equal(sc, rs)
    assert np.array_equal(c, rc)
    assert err == 1 and rf[3, 1] and rf[3, 2] and not rf[:3].any()


@pytest.mark.parametrize("rule", [q4.QUANT_Q4_0, q4.QUANT_ABSMAX7])
def test_quantize_pack_gemv_gemm_head_chain(rule):
    """Quantise on the GPU, pack, then GEMV, S=64 GEMM and the head on the
    result: q4_0 scales come out negative for blocks whose largest value is
    positive, which the synthetic scale distribution never produces."""
    n, k = 3000, 1536
    rng = synth.rng_for(52, rule)
    w = synth.bf16_normal(rng, n * k).reshape(n, k)
    c, sc, _ = _quantize_gpu(w, rule)
    if rule == q4.QUANT_Q4_0:
        assert (oracle.f16_bits_to_f64(sc) < 0).mean() > 0.3
    packed = pack(c, sc)
    x = synth.bf16_normal(rng, k)
    y = q4.q4_gemv(packed, n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemv(c, sc, x)
    assert_within_tol(y, yr, a, "gemv on quantised weights")
    xs = synth.bf16_normal(rng, 64 * k).reshape(64, k)
    ws = torch.empty(q4.q4_gemm_workspace_bytes(n, k), dtype=torch.uint8, device=DEV)
    out = torch.empty((64, n), dtype=torch.float32, device=DEV)
    q4.q4_gemm_s64(packed, n, k, d(xs), out, ws)
    yg, ag = oracle.gemm(c, sc, xs)
    assert_within_tol(out.cpu().numpy().ravel(), yg.ravel(), ag.ravel(), "gemm on quantised weights")
    excluded = _check_head_batch(c, sc, [x, xs[0], xs[1]])
    assert excluded <= 1


# ------------------------------------------------ fused gate/up + GELU --
def _gelu_mul_gpu(codes, sb, x):
    n, k = codes.shape
    bits = q4.q4_gemv_gelu_mul(pack(codes, sb), n, k, d(x)).cpu().numpy().view(np.uint16)
    return bits


# E2B and E4B FFN shapes, ragged pair counts, and every lane split the fused
# kernel has (16 lanes x 1..5 blocks, 32 lanes x 2..6 blocks, ragged blocks)
@pytest.mark.parametrize("h,k", [(6144, 1536), (10240, 2560), (37, 96), (300, 4096), (129, 6144),
                                 (1, 32), (1000, 2048), (77, 5120), (513, 160)])
def test_gelu_mul_tolerance(h, k):
    rng = synth.rng_for(31, h, k)
    codes, sb = synth.q4_weights(rng, 2 * h, k)
    x = synth.bf16_normal(rng, k)
    got = oracle.bf16_bits_to_f64(_gelu_mul_gpu(codes, sb, x))
    a, g, u, ag, au = oracle.gelu_mul(codes, sb, x)
    tol = oracle.gelu_mul_tolerance(g, u, ag, au)
    bad = np.nonzero(~(np.abs(got - a) <= tol))[0]
    assert bad.size == 0, (f"{bad.size} of {h} over the bound, first {bad[:5]}, "
                           f"got {got[bad[:3]]} want {a[bad[:3]]} tol {tol[bad[:3]]}")


def test_gelu_mul_integer_inputs_match_host_epilogue():
    """Power-of-two scales and x in {-1, 0, 1}: g and u are exact in fp32 on
    both sides, so the GPU result may differ from the host fp32 GELU-tanh
    product rounded to bf16 only through the two tanh implementations: at
    most one bf16 ulp, and rarely."""
    h, k = 6144, 1536
    rng = synth.rng_for(32)
    codes = rng.integers(-8, 8, size=(2 * h, k), dtype=np.int8)
    sb = np.full((2 * h, k // 32), fp16_bits(2.0 ** -8), dtype=np.uint16)
    xi = rng.integers(-1, 2, size=k)
    x = bf16_bits_of_ints(xi)
    got = _gelu_mul_gpu(codes, sb, x)
    _, g, u, _, _ = oracle.gelu_mul(codes, sb, x)
    assert np.all(g.astype(np.float32) == g) and np.all(u.astype(np.float32) == u)
    want = oracle.ffn_down_input_bits(g.astype(np.float32), u.astype(np.float32))
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    same_sign = (got >> 15) == (want >> 15)
    assert np.all(same_sign | (diff == 0) | (np.abs(oracle.bf16_bits_to_f64(want)) < 1e-30))
    assert diff.max() <= 1, diff.max()
    assert np.mean(diff == 0) > 0.99


def test_ffn_chain_fused():
    """E2B FFN as one fused launch plus the down GEMV on its bf16 output; the
    down GEMV is checked against the oracle fed the GPU's own a."""
    s = synth.SHAPES["ffn_e2b"]
    rng = synth.rng_for(0, 2)
    gu_codes, gu_sb = synth.q4_weights(rng, *s["gate_up"])
    dn_codes, dn_sb = synth.q4_weights(rng, *s["down"])
    x = synth.bf16_normal(rng, s["gate_up"][1])
    a_gpu = q4.q4_gemv_gelu_mul(pack(gu_codes, gu_sb), *s["gate_up"], d(x))
    a_bits = a_gpu.cpu().numpy().view(np.uint16)
    a, g, u, ag, au = oracle.gelu_mul(gu_codes, gu_sb, x)
    assert np.all(np.abs(oracle.bf16_bits_to_f64(a_bits) - a) <= oracle.gelu_mul_tolerance(g, u, ag, au))
    y = q4.q4_gemv(pack(dn_codes, dn_sb), *s["down"], a_gpu).cpu().numpy()
    yr, ya = oracle.gemv(dn_codes, dn_sb, a_bits)
    assert_within_tol(y, yr, ya, "down after fused gate/up")


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_gemv_e4b_layer_shapes(name):
    shapes = {"qkv": (3072, 2560), "o": (2560, 2048), "gate_up": (20480, 2560), "down": (2560, 10240)}
    n, k = shapes[name]
    rng = synth.rng_for(5, list(shapes).index(name))
    codes, sb = synth.q4_weights(rng, n, k)
    x = synth.bf16_normal(rng, k)
    y = q4.q4_gemv(pack(codes, sb), n, k, d(x)).cpu().numpy()
    yr, a = oracle.gemv(codes, sb, x)
    assert_within_tol(y, yr, a, name)


# ------------------------------------------------------------------- head --
def _check_head_batch(codes, sb, xs, cap=30.0):
    vocab, k = codes.shape
    packed = pack(codes, sb)
    ws = torch.zeros(q4.lmhead_workspace_bytes(vocab, k), dtype=torch.uint8, device=DEV)
    got = []
    for x in xs:
        i, v = q4.lmhead_softcap_argmax(packed, vocab, k, d(x), cap, ws)
        got.append((int(i.item()), float(v.item())))
    return _check_head_results(codes, sb, xs, got, cap)


def _check_head_results(codes, sb, xs, got, cap=30.0):
    """got[s] = (idx, val) for xs[s]: the index must be the oracle's wherever
    the top-2 margin of the capped logits is at least 1e-3, the value within
    the GEMV bar of the oracle's maximum. Returns the excluded count."""
    z, a = oracle.gemm(codes, sb, np.stack(xs))
    excluded = 0
    for s, (gi, gv) in enumerate(got):
        c = oracle.softcap(z[s], cap)
        ri = oracle.first_argmax(c)
        m = oracle.top2_margin(c)
        if m >= 1e-3:
            assert gi == ri, (s, gi, ri, m)
        else:
            excluded += 1
            assert c[ri] - c[gi] < 1e-3 + 1e-4 * a[s, gi] + 1e-6
        assert abs(gv - c[ri]) <= 1e-4 * a[s, ri] + 1e-6, (s, gv, c[ri])
    return excluded


def test_lmhead_e2b_full_100_vectors():
    s = synth.SHAPES["head_e2b"]
    rng = synth.rng_for(0, 3)
    codes, sb = synth.q4_weights(rng, s["vocab"], s["k"])
    xs = [synth.bf16_normal(rng, s["k"]) for _ in range(s["n_vectors"])]
    excluded = _check_head_batch(codes, sb, xs)
    print(f"head: {excluded} of {len(xs)} vectors excluded (top-2 margin < 1e-3)")
    assert excluded <= 5


def test_lmhead_planted_ties_and_boundaries():
    vocab, k = 262144, 1536
    rng = synth.rng_for(7)
    codes = rng.integers(-2, 3, size=(vocab, k), dtype=np.int8)
    sb = np.full((vocab, k // 32), fp16_bits(2.0 ** -7), dtype=np.uint16)
    xi = rng.integers(-3, 4, size=k)
    x = bf16_bits_of_ints(xi)
    planted = np.where(xi > 0, 7, np.where(xi < 0, -8, 0)).astype(np.int8)
    packed_rows = {}
    for rows, expect in [((5, 77777, 262143), 5), ((262143,), 262143), ((0, 262143), 0),
                         ((1023, 1024, 4096), 1023)]:
        cc = codes.copy()
        for r in rows:
            cc[r] = planted
        packed = pack(cc, sb)
        i, v = q4.lmhead_softcap_argmax(packed, vocab, k, d(x), 30.0)
        assert int(i.item()) == expect, rows
        zr = float(sum(int(planted[j]) * int(xi[j]) for j in range(k))) / 128.0
        assert abs(float(v.item()) - float(oracle.softcap(zr))) <= 1e-6 + 1e-4 * abs(zr)
        packed_rows[rows] = packed
    # cap <= 0 returns the raw logit (exact for integer inputs)
    i, v = q4.lmhead_softcap_argmax(packed_rows[(262143,)], vocab, k, d(x), 0.0)
    assert int(i.item()) == 262143
    assert float(v.item()) == float(sum(int(planted[j]) * int(xi[j]) for j in range(k))) / 128.0


def test_lmhead_small_vocab_ragged():
    for vocab, k in [(1, 64), (3, 32), (1000, 1536), (4099, 2560), (777, 10240)]:
        rng = synth.rng_for(11, vocab, k)
        codes, sb = synth.q4_weights(rng, vocab, k)
        xs = [synth.bf16_normal(rng, k) for _ in range(3)]
        _check_head_batch(codes, sb, xs)


def test_lmhead_e4b_head_shape():
    rng = synth.rng_for(0, 4)
    codes, sb = synth.q4_weights(rng, 262144, 2560)
    xs = [synth.bf16_normal(rng, 2560) for _ in range(4)]
    _check_head_batch(codes, sb, xs)


def _multi_head(packed, vocab, k, xs, cap=30.0, ws=None):
    i, v = q4.lmhead_softcap_argmax_multi(packed, vocab, k, d(np.stack(xs)), cap, ws)
    return list(zip(i.cpu().numpy().tolist(), v.cpu().numpy().tolist()))


def test_lmhead_multi_e2b_full_100_vectors():
    """The verify head: the E2B head with the 100 vectors in batches of 8, 4,
    3 and 2 (both matrix-core chains, ragged batches)."""
    s = synth.SHAPES["head_e2b"]
    rng = synth.rng_for(0, 3)
    codes, sb = synth.q4_weights(rng, s["vocab"], s["k"])
    xs = [synth.bf16_normal(rng, s["k"]) for _ in range(s["n_vectors"])]
    packed = pack(codes, sb)
    ws = torch.zeros(q4.lmhead_multi_workspace_bytes(s["vocab"], s["k"], 8), dtype=torch.uint8, device=DEV)
    got, i = [], 0
    for m in [8] * 11 + [4, 3, 2, 3]:
        got += _multi_head(packed, s["vocab"], s["k"], xs[i:i + m], ws=ws)
        i += m
    assert i == len(xs)
    excluded = _check_head_results(codes, sb, xs, got)
    assert excluded <= 5


def test_lmhead_multi_e4b_and_ragged_vocab():
    for vocab, k, m in [(262144, 2560, 4), (1, 64, 2), (3, 32, 8), (1000, 1536, 5), (4099, 2560, 7),
                        (777, 10240, 4), (70001, 2048, 6)]:
        rng = synth.rng_for(14, vocab, k, m)
        codes, sb = synth.q4_weights(rng, vocab, k)
        xs = [synth.bf16_normal(rng, k) for _ in range(m)]
        got = _multi_head(pack(codes, sb), vocab, k, xs)
        _check_head_results(codes, sb, xs, got)


def test_lmhead_multi_planted_ties_per_vector():
    """Equal maxima in several rows: each vector's lowest winning row, with
    vectors that pick different rows (x and -x) in one call; cap <= 0 gives
    the raw maxima, exact for integer inputs."""
    vocab, k = 262144, 1536
    rng = synth.rng_for(15)
    codes = rng.integers(-2, 3, size=(vocab, k), dtype=np.int8)
    sb = np.full((vocab, k // 32), fp16_bits(2.0 ** -7), dtype=np.uint16)
    xi = rng.integers(-3, 4, size=k)
    up = np.where(xi > 0, 7, np.where(xi < 0, -8, 0)).astype(np.int8)    # the maximum for x
    down = np.where(xi > 0, -8, np.where(xi < 0, 7, 0)).astype(np.int8)  # the maximum for -x
    for r in (70000, 5, 262143):
        codes[r] = up
    for r in (262143, 1024, 1023):
        codes[r] = down
    packed = pack(codes, sb)
    x, xn = bf16_bits_of_ints(xi), bf16_bits_of_ints(-xi)
    got = _multi_head(packed, vocab, k, [x, xn, x], cap=0.0)
    zu = float(sum(int(up[j]) * int(xi[j]) for j in range(k))) / 128.0
    zd = float(sum(int(down[j]) * int(-xi[j]) for j in range(k))) / 128.0
    assert got == [(5, zu), (1023, zd), (5, zu)]
    got = _multi_head(packed, vocab, k, [xn, x], cap=30.0)
    assert [g[0] for g in got] == [1023, 5]
    assert abs(got[1][1] - float(oracle.softcap(zu))) <= 1e-6 + 1e-4 * abs(zu)


# ------------------------------------------------ head over 64 tokens --
@pytest.mark.parametrize("vocab,k,n_tok", [(40000, 1536, 64), (40000, 1536, 17), (3001, 2560, 1),
                                           (130, 10240, 64)])
def test_lmhead_s64_against_oracle(vocab, k, n_tok):
    rng = synth.rng_for(90, vocab, k, n_tok)
    codes, sb = synth.q4_weights(rng, vocab, k)
    xs = synth.bf16_normal(rng, n_tok * k).reshape(n_tok, k)
    i, v = q4.lmhead_softcap_argmax_s64(pack(codes, sb), vocab, k, d(xs), 30.0)
    got = list(zip(i.cpu().tolist(), v.cpu().tolist()))
    excluded = _check_head_results(codes, sb, list(xs), got)
    assert excluded <= max(2, n_tok // 10)


def test_lmhead_s64_planted_ties_and_raw_values():
    """Integer inputs, so every logit is exact: rows 5, 77 and 9999 hold the
    same maximum for x (the lowest, 5, must win), row 1023 holds the maximum
    for -x, and tokens alternate between x and -x in one call; cap <= 0 gives
    the raw logits exactly."""
    vocab, k, n_tok = 10000, 1536, 64
    rng = synth.rng_for(91)
    codes = rng.integers(-2, 3, size=(vocab, k), dtype=np.int8)
    sb = np.full((vocab, k // 32), fp16_bits(2.0 ** -7), dtype=np.uint16)
    xi = rng.integers(-3, 4, size=k)
    up = np.where(xi > 0, 7, np.where(xi < 0, -8, 0)).astype(np.int8)
    down = np.where(xi > 0, -8, np.where(xi < 0, 7, 0)).astype(np.int8)
    for r in (5, 77, 9999):
        codes[r] = up
    codes[1023] = down
    packed = pack(codes, sb)
    xs = np.stack([bf16_bits_of_ints(xi if t % 2 == 0 else -xi) for t in range(n_tok)])
    zu = float(np.dot(up.astype(np.int64), xi)) / 128.0
    zd = float(np.dot(down.astype(np.int64), -xi)) / 128.0
    i, v = q4.lmhead_softcap_argmax_s64(packed, vocab, k, d(xs), 0.0)
    assert i.cpu().tolist() == [5 if t % 2 == 0 else 1023 for t in range(n_tok)]
    assert v.cpu().tolist() == [zu if t % 2 == 0 else zd for t in range(n_tok)]
    i, v = q4.lmhead_softcap_argmax_s64(packed, vocab, k, d(xs), 30.0)
    assert i.cpu().tolist() == [5 if t % 2 == 0 else 1023 for t in range(n_tok)]
    assert abs(float(v[0].item()) - float(oracle.softcap(zu))) <= 1e-6 + 1e-4 * abs(zu)


def test_lmhead_s64_e4b_head_sampled_tokens():
    """The E4B head [262144, 2560] for a 64-token chunk. Four tokens are
    checked against the whole oracle head. For every token, the value must
    match the oracle's logit of the returned row, and that row must match the
    single-token head's row or hold an exact logit within both error bars of
    it."""
    vocab, k, n_tok = 262144, 2560, 64
    rng = synth.rng_for(92)
    codes, sb = synth.q4_weights(rng, vocab, k)
    packed = pack(codes, sb)
    xs = synth.bf16_normal(rng, n_tok * k).reshape(n_tok, k)
    i, v = q4.lmhead_softcap_argmax_s64(packed, vocab, k, d(xs), 30.0)
    idx, val = i.cpu().tolist(), v.cpu().tolist()
    for t in (0, 21, 42, 63):
        ref = oracle.lmhead(codes, sb, xs[t])
        if ref["margin"] >= 1e-3:
            assert idx[t] == ref["idx"], (t, idx[t], ref["idx"])
        assert abs(val[t] - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6
    ws = torch.zeros(q4.lmhead_workspace_bytes(vocab, k), dtype=torch.uint8, device=DEV)
    for t in range(n_tok):
        r = idx[t]
        z, a = oracle.gemv(codes[r:r + 1], sb[r:r + 1], xs[t])
        assert abs(val[t] - float(oracle.softcap(z[0]))) <= 1e-4 * a[0] + 1e-6, t
        i1, _ = q4.lmhead_softcap_argmax(packed, vocab, k, d(xs[t]), 30.0, ws)
        r1 = int(i1.item())
        if r1 != r:
            z1, a1 = oracle.gemv(codes[r1:r1 + 1], sb[r1:r1 + 1], xs[t])
            assert abs(z1[0] - z[0]) <= 1e-4 * (a[0] + a1[0]) + 2e-6, (t, r, r1)


def test_lmhead_shared_workspace_and_graph_replays():
    """One workspace serves calls of different sizes back to back and the
    replays of a captured call; every call writes a fresh result (outputs are
    preset to a sentinel before each call), and every call leaves the arrival
    counter in the workspace's last 256 bytes at zero."""
    ws = torch.zeros(q4.lmhead_workspace_bytes(262144, 2560), dtype=torch.uint8, device=DEV)
    idx = torch.empty(1, dtype=torch.int32, device=DEV)
    val = torch.empty(1, dtype=torch.float32, device=DEV)
    cases = []
    for vocab, k in [(262144, 1536), (4099, 2560), (1, 64), (70000, 2560)]:
        rng = synth.rng_for(12, vocab, k)
        codes, sb = synth.q4_weights(rng, vocab, k)
        cases.append((vocab, k, codes, sb, pack(codes, sb)))
    for vocab, k, codes, sb, packed in cases + cases[::-1]:
        rng = synth.rng_for(13, vocab, k)
        x = synth.bf16_normal(rng, k)
        idx.fill_(-7)
        val.fill_(float("nan"))
        q4.lmhead_softcap_argmax(packed, vocab, k, d(x), 30.0, ws, idx, val)
        z, a = oracle.gemm(codes, sb, x[None, :])
        c = oracle.softcap(z[0])
        ri = oracle.first_argmax(c)
        gi = int(idx.item())
        assert gi != -7, (vocab, k)
        if oracle.top2_margin(c) >= 1e-3:
            assert gi == ri, (vocab, k, gi, ri)
        assert abs(float(val.item()) - c[ri]) <= 1e-4 * a[0, ri] + 1e-6

    vocab, k, codes, sb, packed = cases[3]
    xbuf = torch.zeros(k, dtype=torch.int16, device=DEV)
    q4.lmhead_softcap_argmax(packed, vocab, k, xbuf, 30.0, ws, idx, val)  # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        q4.lmhead_softcap_argmax(packed, vocab, k, xbuf, 30.0, ws, idx, val)
    for rep in range(4):
        x = synth.bf16_normal(synth.rng_for(14, rep), k)
        xbuf.copy_(d(x))
        idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        z, a = oracle.gemm(codes, sb, x[None, :])
        c = oracle.softcap(z[0])
        ri = oracle.first_argmax(c)
        gi = int(idx.item())
        assert gi != -7, rep
        if oracle.top2_margin(c) >= 1e-3:
            assert gi == ri, (rep, gi, ri)
        assert abs(float(val.item()) - c[ri]) <= 1e-4 * a[0, ri] + 1e-6
    torch.cuda.synchronize()
    assert int(ws[-256:].count_nonzero().item()) == 0


# -------------------------------------------------------------------- PLE --
@pytest.mark.parametrize("dim", [8960, 10752])
def test_ple_gather_full_tables(dim):
    vocab = synth.VOCAB
    g = torch.Generator(device=DEV)
    g.manual_seed(1234 + dim)
    table = torch.randint(-127, 128, (vocab, dim), dtype=torch.int8, device=DEV, generator=g)
    scale = torch.empty(vocab, dtype=torch.float32, device=DEV).uniform_(1e-3, 1e-2, generator=g)
    rng = synth.rng_for(0, dim)
    for n_ids in (1, 64):
        ids = synth.ple_ids(rng, vocab, n_ids)
        if n_ids == 64:
            ids[:4] = [0, vocab - 1, ids[10], ids[10]]  # boundaries and duplicates
        idt = d(ids)
        out = q4.ple_gather(table, scale, idt, 16.0).cpu().numpy()
        rows = table[idt.long()].cpu().numpy()
        rsc = scale[idt.long()].cpu().numpy()
        ref, err = oracle.ple_gather(rows, rsc, np.arange(n_ids, dtype=np.int32), 16.0)
        assert err == 0
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_token_embedding_gather_full_table():
    """The E2B token embedding: int8 [262144, 1536] with a per-row scale,
    gathered rows multiplied by sqrt(1536) (the model card's 39.191837)."""
    vocab, dim = synth.VOCAB, 1536
    g = torch.Generator(device=DEV)
    g.manual_seed(4321)
    table = torch.randint(-127, 128, (vocab, dim), dtype=torch.int8, device=DEV, generator=g)
    scale = torch.empty(vocab, dtype=torch.float32, device=DEV).uniform_(1e-3, 1e-2, generator=g)
    ids = synth.ple_ids(synth.rng_for(5), vocab, 64)
    ids[:3] = [0, vocab - 1, ids[7]]
    idt = d(ids)
    out = q4.ple_gather(table, scale, idt, 39.191837).cpu().numpy()
    ref, err = oracle.ple_gather(table[idt.long()].cpu().numpy(), scale[idt.long()].cpu().numpy(),
                                 np.arange(64, dtype=np.int32), 39.191837)
    assert err == 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_ple_gather_general_multiplier_and_ragged_dim():
    rng = synth.rng_for(3)
    for dim in (8960, 100, 7, 4096 + 3):
        table, scale, ids = synth.ple_inputs(rng, 5000, dim, 37)
        for mult in (16.0, float(np.float32(np.sqrt(1536.0))), 0.3):
            out = q4.ple_gather(d(table), d(scale), d(ids), mult).cpu().numpy()
            ref, _ = oracle.ple_gather(table, scale, ids, mult)
            assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), (dim, mult)


def test_ple_gather_out_of_range_ids():
    rng = synth.rng_for(4)
    table, scale, _ = synth.ple_inputs(rng, 100, 256, 1)
    ids = np.array([3, -1, 100, 99], dtype=np.int32)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = q4.ple_gather(d(table), d(scale), d(ids), 16.0, err_flag=flag).cpu().numpy()
    ref, err = oracle.ple_gather(table, scale, ids, 16.0)
    assert int(flag.item()) == 1 and err == 1
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    flag.zero_()
    q4.ple_gather(d(table), d(scale), d(np.array([0, 99], np.int32)), 16.0, err_flag=flag)
    assert int(flag.item()) == 0


# ------------------------------------ mixed-bit INT2 / INT4 row gathers --
@pytest.mark.parametrize("bits,dim,group,mult", [(2, 1536, 1536, 39.191837),  # INT2 token embedding
                                                 (4, 8960, 256, 16.0)])       # INT4 PLE table
def test_rowq_gather_full_tables(bits, dim, group, mult):
    """The mixed-bit recipe's tables at full size: the INT2 input embedding
    [262144, 1536] with a per-row scale and sqrt(1536), and the INT4 PLE table
    [262144, 35 x 256] with one scale per row and layer and 16.0; 1 and 64 ids
    with the first and last rows and a duplicate. Bit-exact."""
    vocab = synth.VOCAB
    g = torch.Generator(device=DEV)
    g.manual_seed(77 + bits)
    w = torch.randint(0, 256, (vocab, dim * bits // 8), dtype=torch.uint8, device=DEV, generator=g)
    sc = torch.empty((vocab, dim // group), dtype=torch.float32, device=DEV).uniform_(1e-3, 1e-2, generator=g)
    rng = synth.rng_for(78, bits)
    for n_ids in (1, 64):
        ids = synth.ple_ids(rng, vocab, n_ids)
        if n_ids == 64:
            ids[:4] = [0, vocab - 1, ids[10], ids[10]]
        idt = d(ids)
        out = q4.rowq_gather(w, sc, bits, group, idt, mult).cpu().numpy()
        ref, err = oracle.rowq_gather(w[idt.long()].cpu().numpy(), sc[idt.long()].cpu().numpy(), bits, group,
                                      np.arange(n_ids, dtype=np.int32), mult)
        assert err == 0
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), (bits, n_ids)


@pytest.mark.parametrize("bits,dim,group", [(2, 64, 64), (2, 4096, 128), (2, 1536, 64), (4, 32, 32),
                                            (4, 96, 32), (4, 4096, 2048), (4, 8960, 256)])
def test_rowq_gather_shapes_and_multipliers(bits, dim, group):
    rng = synth.rng_for(79, bits, dim, group)
    vocab = 3000
    w = rng.integers(0, 256, size=(vocab, dim * bits // 8), dtype=np.uint8)
    sc = rng.uniform(1e-3, 1e-2, size=(vocab, dim // group)).astype(np.float32)
    ids = synth.ple_ids(rng, vocab, 37)
    for mult in (16.0, float(np.float32(np.sqrt(1536.0))), 0.3):
        out = q4.rowq_gather(d(w), d(sc), bits, group, d(ids), mult).cpu().numpy()
        ref, _ = oracle.rowq_gather(w, sc, bits, group, ids, mult)
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), (bits, dim, group, mult)


def test_rowq_gather_int2_extreme_scales():
    """INT2 scales near the top of the fp32 range (where code * scale alone
    would overflow but the product with mult < 1 is finite), at the bottom
    (subnormal) and around 2^126, with multipliers below and above one."""
    rng = synth.rng_for(81)
    w = rng.integers(0, 256, size=(8, 16), dtype=np.uint8)   # INT2, dim 64
    sc = np.array([[3.0e38], [2.0 ** 126], [2.0 ** 126 * 0.999], [1.0e-40], [1.5e-45], [-3.0e38], [1.0], [0.0]],
                  dtype=np.float32)
    ids = np.arange(8, dtype=np.int32)
    for mult in (0.3, 16.0, float(np.float32(np.sqrt(1536.0)))):
        out = q4.rowq_gather(d(w), d(sc), 2, 64, d(ids), mult).cpu().numpy()
        ref, _ = oracle.rowq_gather(w, sc, 2, 64, ids, mult)
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), mult


def test_rowq_gather_out_of_range_ids():
    rng = synth.rng_for(80)
    w = rng.integers(0, 256, size=(50, 128), dtype=np.uint8)   # INT4, dim 256
    sc = rng.uniform(1e-3, 1e-2, size=(50, 2)).astype(np.float32)
    ids = np.array([3, -1, 50, 49], dtype=np.int32)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = q4.rowq_gather(d(w), d(sc), 4, 128, d(ids), 16.0, err_flag=flag).cpu().numpy()
    ref, err = oracle.rowq_gather(w, sc, 4, 128, ids, 16.0)
    assert int(flag.item()) == 1 and err == 1
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    flag.zero_()
    q4.rowq_gather(d(w), d(sc), 4, 128, d(np.array([0, 49], np.int32)), 16.0, err_flag=flag)
    assert int(flag.item()) == 0


# ------------------------------------------------------- graph replays --
def test_every_entry_point_replays_in_a_graph():
    """One call of every entry point captured in a HIP graph, replayed four
    times with fresh inputs and eager work between replays; each replay must
    equal an eager run of the same calls bit for bit (nothing in the library
    records a memset or depends on state left by a previous call)."""
    rng = synth.rng_for(95)
    n, k, m = 1000, 2560, 4
    codes, sb = synth.q4_weights(rng, 2 * n, k)
    packed = pack(codes, sb)
    w2 = d(rng.integers(0, 256, size=(n, k // 4), dtype=np.uint8))
    s2 = d(rng.uniform(1e-3, 1e-2, size=n).astype(np.float32))
    table, scale, _ = synth.ple_inputs(rng, 5000, 256, 1)
    table, scale = d(table), d(scale)
    x = torch.zeros(k, dtype=torch.int16, device=DEV)
    xm = torch.zeros((m, k), dtype=torch.int16, device=DEV)
    x64 = torch.zeros((64, k), dtype=torch.int16, device=DEV)
    ids = torch.zeros(8, dtype=torch.int32, device=DEV)
    xb = torch.zeros((1, k), dtype=torch.int16, device=DEV)
    outs = {
        "y": torch.empty(2 * n, dtype=torch.float32, device=DEV),
        "a": torch.empty(n, dtype=torch.int16, device=DEV),
        "ym": torch.empty((m, 2 * n), dtype=torch.float32, device=DEV),
        "yg": torch.empty((64, 2 * n), dtype=torch.float32, device=DEV),
        "yr": torch.empty(n, dtype=torch.float32, device=DEV),
        "hi": torch.empty(1, dtype=torch.int32, device=DEV), "hv": torch.empty(1, dtype=torch.float32, device=DEV),
        "mi": torch.empty(m, dtype=torch.int32, device=DEV), "mv": torch.empty(m, dtype=torch.float32, device=DEV),
        "si": torch.empty(64, dtype=torch.int32, device=DEV), "sv": torch.empty(64, dtype=torch.float32, device=DEV),
        "ri": torch.empty(1, dtype=torch.int32, device=DEV), "rv": torch.empty(1, dtype=torch.float32, device=DEV),
        "ra": torch.empty(n // 2, dtype=torch.int16, device=DEV),
        "pg": torch.empty((8, 256), dtype=torch.float32, device=DEV),
        "rg": torch.empty((8, k), dtype=torch.float32, device=DEV),
        "qc": torch.empty((1, k), dtype=torch.int8, device=DEV),
        "qs": torch.empty((1, k // 32), dtype=torch.int16, device=DEV),
        "pk": torch.empty(q4.q4_packed_bytes(64, k), dtype=torch.uint8, device=DEV),
    }
    pack_codes = torch.zeros((64, k), dtype=torch.int8, device=DEV)
    pack_scales = torch.zeros((64, k // 32), dtype=torch.int16, device=DEV)
    ws_g = torch.empty(q4.q4_gemm_workspace_bytes(2 * n, k), dtype=torch.uint8, device=DEV)
    ws_h = torch.zeros(q4.lmhead_workspace_bytes(2 * n, k), dtype=torch.uint8, device=DEV)
    ws_m = torch.empty(q4.lmhead_multi_workspace_bytes(2 * n, k, m), dtype=torch.uint8, device=DEV)
    ws_s = torch.empty(q4.lmhead_s64_workspace_bytes(2 * n, k), dtype=torch.uint8, device=DEV)
    ws_r = torch.empty(q4.rowq_head_workspace_bytes(n, k, 2), dtype=torch.uint8, device=DEV)
    w_int2_rows = d(rng.integers(0, 256, size=(5000, k // 4), dtype=np.uint8))
    s_int2_rows = d(rng.uniform(1e-3, 1e-2, size=(5000, 1)).astype(np.float32))

    def calls():
        q4.q4_gemv(packed, 2 * n, k, x, outs["y"])
        q4.q4_gemv_gelu_mul(packed, 2 * n, k, x, outs["a"])
        q4.q4_gemv_multi(packed, 2 * n, k, xm, outs["ym"])
        q4.q4_gemm_s64(packed, 2 * n, k, x64, outs["yg"], ws_g)
        q4.rowq_gemv(w2, s2, n, k, 2, x, outs["yr"])
        q4.rowq_gemv_gelu_mul(w2, s2, n, k, 2, x, outs["ra"])
        q4.rowq_softcap_argmax(w2, s2, n, k, 2, x, 30.0, ws_r, outs["ri"], outs["rv"])
        q4.lmhead_softcap_argmax(packed, 2 * n, k, x, 30.0, ws_h, outs["hi"], outs["hv"])
        q4.lmhead_softcap_argmax_multi(packed, 2 * n, k, xm, 30.0, ws_m, outs["mi"], outs["mv"])
        q4.lmhead_softcap_argmax_s64(packed, 2 * n, k, x64, 30.0, ws_s, outs["si"], outs["sv"])
        q4.ple_gather(table, scale, ids, 16.0, out=outs["pg"])
        q4.rowq_gather(w_int2_rows, s_int2_rows, 2, k, ids, 39.191837, out=outs["rg"])
        q4.q4_quantize(xb, q4.QUANT_Q4_0, codes=outs["qc"], scales=outs["qs"])
        q4.q4_pack(pack_codes, pack_scales, packed=outs["pk"])

    def fresh_inputs(rep):
        r = synth.rng_for(96, rep)
        x.copy_(d(synth.bf16_normal(r, k)))
        xm.copy_(d(synth.bf16_normal(r, (m, k))))
        x64.copy_(d(synth.bf16_normal(r, (64, k))))
        xb.copy_(d(synth.bf16_normal(r, (1, k))))
        ids.copy_(d(synth.ple_ids(r, 5000, 8)))
        c, sc = synth.q4_weights(r, 64, k)
        pack_codes.copy_(d(c))
        pack_scales.copy_(d(sc))

    fresh_inputs(0)
    calls()  # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(1, 5):
        fresh_inputs(rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {name: t.clone() for name, t in outs.items()}
        q4.q4_gemv(packed, 2 * n, k, x64[0], outs["y"])  # unrelated eager work between replays
        calls()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(got[name], t), (rep, name)


# ----------------------------------------------------------- S=64 GEMM --
@pytest.mark.parametrize("n,k,n_tok", [(1536, 1536, 64), (64, 32, 64), (100, 96, 1), (300, 2560, 37),
                                       # the four E4B layer shapes: QKV, O, down (split K) ...
                                       (3072, 2560, 64), (2560, 2048, 64), (2560, 10240, 64), (77, 16384, 5),
                                       # many row tiles: one K slice, no reduce (E4B gate+up; a
                                       # ragged last tile; k not a multiple of 256)
                                       (20480, 2560, 64), (16400, 512, 17),
                                       # 80-row workgroups whose shared fifth tile is ragged
                                       (19990, 512, 64), (20470, 2560, 3)])
def test_gemm_s64_tolerance(n, k, n_tok):
    rng = synth.rng_for(20, n, k, n_tok)
    codes, sb = synth.q4_weights(rng, n, k)
    xs = synth.bf16_normal(rng, (n_tok, k))
    y = q4.q4_gemm_s64(pack(codes, sb), n, k, d(xs)).cpu().numpy()
    yr, a = oracle.gemm(codes, sb, xs)
    assert_within_tol(y.ravel(), yr.ravel(), a.ravel(), f"gemm {n}x{k} s={n_tok}")


@pytest.mark.parametrize("n,k", [(300, 1536), (64, 4096), (1000, 2048)])
def test_gemm_s64_integer_exact(n, k):
    """Integer activations and power-of-two scales: exact in fp32 in any order."""
    rng = np.random.default_rng(300 + k)
    codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    p = rng.integers(6, 9, size=(n, k // 32))
    sb = np.vectorize(lambda e: fp16_bits(2.0 ** -int(e)))(p).astype(np.uint16)
    xi = rng.integers(-8, 9, size=(64, k))
    xs = bf16_bits_of_ints(xi.ravel()).reshape(64, k)
    y = q4.q4_gemm_s64(pack(codes, sb), n, k, d(xs)).cpu().numpy()
    yr, _ = oracle.gemm(codes, sb, xs)
    assert np.array_equal(y.astype(np.float64), yr)


def test_gemm_rows_match_gemv_and_are_deterministic():
    n, k = 2560, 2048
    rng = synth.rng_for(21)
    codes, sb = synth.q4_weights(rng, n, k)
    xs = synth.bf16_normal(rng, (64, k))
    packed = pack(codes, sb)
    xd = d(xs)
    y1 = q4.q4_gemm_s64(packed, n, k, xd).cpu().numpy()
    y2 = q4.q4_gemm_s64(packed, n, k, xd).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    _, a = oracle.gemm(codes, sb, xs)
    for s in (0, 31, 63):
        yv = q4.q4_gemv(packed, n, k, xd[s]).cpu().numpy()
        assert (np.abs(y1[s].astype(np.float64) - yv) <= 2 * oracle.gemv_tolerance(a[s])).all()
    # a chunk shorter than 64 returns the same rows as the full chunk
    y5 = q4.q4_gemm_s64(packed, n, k, xd[:5].contiguous()).cpu().numpy()
    assert (np.abs(y5.astype(np.float64) - y1[:5]) <= 2 * oracle.gemv_tolerance(a[:5])).all()


def test_gemm_s64_shared_workspace_across_shapes():
    """One workspace serves a sequence of split-K calls of different shapes
    and token counts (the prefill step's pattern), twice over: no call may
    read what an earlier one left in it."""
    shapes = [(3072, 2560, 64), (2560, 2048, 64), (2560, 10240, 64), (300, 2560, 37), (2560, 2048, 7)]
    need = max(q4.q4_gemm_workspace_bytes(n, k) for n, k, _ in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    rng = synth.rng_for(23)
    for rep in range(2):
        for n, k, t in shapes:
            codes, sb = synth.q4_weights(rng, n, k)
            xs = synth.bf16_normal(rng, (t, k))
            y = torch.empty((t, n), dtype=torch.float32, device=DEV)
            q4.q4_gemm_s64(pack(codes, sb), n, k, d(xs), y, ws)
            yr, a = oracle.gemm(codes, sb, xs)
            assert_within_tol(y.cpu().numpy().ravel(), yr.ravel(), a.ravel(), f"shared ws {n}x{k} s={t} rep {rep}")


def test_gemm_s64_scale_range():
    """Scales across the fp16 range, rows of only large scales and subnormal
    scales: the fp32 fold of each block's MFMA sum must keep them all."""
    n, k = 256, 1024
    rng = synth.rng_for(22)
    codes, _ = synth.q4_weights(rng, n, k)
    e = rng.uniform(-24, 15.9, size=(n, k // 32))
    sb = np.float16(2.0 ** e).view(np.uint16).copy()
    sb[:8] = np.float16(3.0e4).view(np.uint16)      # rows of only large scales
    sb[8:16, ::2] = np.float16(2.0 ** -20).view(np.uint16)  # subnormal scales
    xs = synth.bf16_normal(rng, (64, k))
    y = q4.q4_gemm_s64(pack(codes, sb), n, k, d(xs)).cpu().numpy()
    yr, a = oracle.gemm(codes, sb, xs)
    assert np.isfinite(y[:, :8]).all()
    assert_within_tol(y.ravel(), yr.ravel(), a.ravel(), "gemm scale range")
