"""Sweeps over the launch plans of the GEMV-family kernels, through the C ABI.

Each kernel family picks a lane split, a per-lane block count, a full or
ragged variant and a row walk from (n, k). These tests step k through every
block count the planners map to a distinct kernel, and n through a short
matrix (partial last row group) and a tall one (waves that walk several
rows). The inputs are exact: codes, integer activations in [-4, 4] and scales
that are powers of two drawn per block (per row for the per-row formats), so
every partial sum is exact in fp32 in any order and the GPU result must equal
the fp64 oracle bit for bit. The head uses the same inputs; its logits are
then exact, ties included, and the index must be the oracle's lowest winning
row. The fused gate/up GELU is checked against its tolerance bound.
"""
import numpy as np
import pytest
import torch

import int4_weight_only_block_amd as q4
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# block counts (k / 32): every (lanes per row, blocks per lane) pair the q4_0
# planner can choose, with full and ragged last lanes, up to k = 16384
BLOCKS = [1, 2, 3, 5, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 79, 80, 81, 96, 97, 128, 129, 160, 191,
          192, 193, 224, 255, 256, 257, 320, 383, 384, 385, 448, 511, 512]
# a short matrix, and a tall one for the k values whose plans walk rows
SHORT_N = 45
TALL = {1: 41000, 80: 41000, 81: 21000, 192: 21000, 193: 3000, 320: 3000, 512: 3000}


def d(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def int_bf16(xi) -> np.ndarray:
    """bf16 bit patterns of small integers (exact)."""
    return (np.asarray(xi, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def pow2_f16_bits(rng, shape, lo=-8, hi=-5) -> np.ndarray:
    """fp16 bit patterns of 2^e, e uniform in [lo, hi]."""
    e = rng.integers(lo, hi + 1, size=shape)
    return ((e + 15) << 10).astype(np.uint16)


def exact_q4_inputs(rng, n, k, m=None):
    codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    sb = pow2_f16_bits(rng, (n, k // 32))
    shape = k if m is None else (m, k)
    return codes, sb, int_bf16(rng.integers(-4, 5, size=shape))


def cases(tall=True):
    out = [(SHORT_N, b) for b in BLOCKS]
    if tall:
        out += [(n, b) for b, n in TALL.items()]
    return out


@pytest.mark.parametrize("n,blocks", cases())
def test_gemv_plans_exact(n, blocks):
    k = 32 * blocks
    rng = synth.rng_for(400, n, blocks)
    codes, sb, x = exact_q4_inputs(rng, n, k)
    y = q4.q4_gemv(q4.q4_pack(d(codes), d(sb)), n, k, d(x)).cpu().numpy()
    yr, _ = oracle.gemv(codes, sb, x)
    bad = np.nonzero(y.astype(np.float64) != yr)[0]
    assert bad.size == 0, (n, k, bad[:5], y[bad[:3]], yr[bad[:3]])


# (8 vectors of k = 10240 would not fit one workgroup's LDS)
@pytest.mark.parametrize("m,blocks", [(m, b) for m in (2, 5, 8) for b in (1, 3, 16, 17, 48, 80, 81, 160, 191)]
                         + [(2, 320), (4, 320), (3, 512)])
def test_gemv_multi_plans_exact(m, blocks):
    k = 32 * blocks
    n = 1203
    rng = synth.rng_for(401, m, blocks)
    codes, sb, xs = exact_q4_inputs(rng, n, k, m)
    y = q4.q4_gemv_multi(q4.q4_pack(d(codes), d(sb)), n, k, d(xs)).cpu().numpy()
    yr, _ = oracle.gemm(codes, sb, xs)
    assert np.array_equal(y.astype(np.float64), yr), (m, k)


@pytest.mark.parametrize("vocab,blocks", [(1, 1), (63, 48), (70001, 1), (70001, 5), (70001, 48), (70001, 80),
                                          (70001, 81), (20001, 192), (20001, 320), (9000, 512)])
def test_head_plans_exact(vocab, blocks):
    k = 32 * blocks
    rng = synth.rng_for(402, vocab, blocks)
    codes, sb, x = exact_q4_inputs(rng, vocab, k)
    i, v = q4.lmhead_softcap_argmax(q4.q4_pack(d(codes), d(sb)), vocab, k, d(x), 30.0)
    ref = oracle.lmhead(codes, sb, x)
    # exact logits: the lowest row among equal maxima, no margin exclusion
    assert int(i.item()) == ref["idx"], (vocab, k, int(i.item()), ref["idx"])
    assert abs(float(v.item()) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6


@pytest.mark.parametrize("h,blocks", [(19, b) for b in [1, 2, 3, 5, 16, 17, 31, 32, 33, 64, 65, 80, 81, 96,
                                                           128, 160, 191, 192]] + [(10300, 80), (5200, 192)])
def test_gelu_plans_within_bound(h, blocks):
    k = 32 * blocks
    rng = synth.rng_for(403, h, blocks)
    codes, sb = synth.q4_weights(rng, 2 * h, k)
    x = synth.bf16_normal(rng, k)
    a_out = torch.empty(h, dtype=torch.int16, device=DEV)
    q4.q4_gemv_gelu_mul(q4.q4_pack(d(codes), d(sb)), 2 * h, k, d(x), a_out)
    got = oracle.bf16_bits_to_f64(a_out.cpu().numpy().view(np.uint16))
    a, g, u, ag, au = oracle.gelu_mul(codes, sb, x)
    tol = oracle.gelu_mul_tolerance(g, u, ag, au)
    bad = np.nonzero(~(np.abs(got - a) <= tol))[0]
    assert bad.size == 0, (h, k, bad[:5])


# per-row formats: k in steps of one chunk (64 INT2, 32 INT4 or 32 INT8 codes)
# through every lane split and chunk count, short and tall matrices
ROWQ = ([(2, 23, c) for c in [1, 2, 3, 4, 5, 8, 9, 16, 17, 24, 25, 32, 33, 48, 49, 64, 96, 128, 129, 192, 256]]
        + [(4, 23, c) for c in [1, 2, 3, 5, 6, 8, 9, 16, 17, 24, 48, 49, 96, 97, 192, 193, 256, 320, 384, 448, 512]]
        + [(8, 23, c) for c in [1, 2, 3, 5, 6, 8, 9, 16, 17, 24, 48, 49, 96, 97, 192, 193, 256, 320, 384, 448, 512]]
        + [(2, 30000, 24), (2, 3000, 192), (4, 30000, 48), (4, 3000, 512), (8, 30000, 48), (8, 3000, 512)])


@pytest.mark.parametrize("bits,n,chunks", ROWQ)
def test_rowq_plans_exact(bits, n, chunks):
    k = chunks * (64 if bits == 2 else 32)  # codes per chunk: 16 bytes of INT2 / INT4, 32 bytes of INT8
    rng = synth.rng_for(404, bits, n, chunks)
    w = rng.integers(0, 256, size=(n, k * bits // 8), dtype=np.uint8)
    sc = (2.0 ** rng.integers(-6, -2, size=n)).astype(np.float32)
    x = int_bf16(rng.integers(-4, 5, size=k))
    y = q4.rowq_gemv(d(w), d(sc), n, k, bits, d(x)).cpu().numpy()
    yr, _ = oracle.rowq_gemv(w, sc, bits, x)
    bad = np.nonzero(y.astype(np.float64) != yr)[0]
    assert bad.size == 0, (bits, n, k, bad[:5], y[bad[:3]], yr[bad[:3]])


# the per-row head through the same plans; with exact logits and no cap the
# index is the oracle's lowest winning row (ties are common at these sizes)
# and the value its raw maximum, bit for bit
@pytest.mark.parametrize("bits,n,chunks", [c for c in ROWQ if c[2] in (1, 3, 16, 17, 48, 96, 192, 256, 512)])
def test_rowq_head_plans_exact(bits, n, chunks):
    k = chunks * (64 if bits == 2 else 32)
    rng = synth.rng_for(405, bits, n, chunks)
    w = rng.integers(0, 256, size=(n, k * bits // 8), dtype=np.uint8)
    sc = (2.0 ** rng.integers(-6, -2, size=n)).astype(np.float32)
    x = int_bf16(rng.integers(-4, 5, size=k))
    i, v = q4.rowq_softcap_argmax(d(w), d(sc), n, k, bits, d(x), 0.0)
    ref = oracle.rowq_lmhead(w, sc, bits, x, 0.0)
    assert int(i.item()) == ref["idx"], (bits, n, k, int(i.item()), ref["idx"])
    assert float(v.item()) == ref["val"]
