"""q4_gemv_chain on the GPU against the fp64 oracle, through the C ABI.

A chain runs several GEMV / fused-GELU links and an optional head in one
persistent launch. Its outputs are held to the bars of the single-matrix
calls: |y - y_ref| <= 1e-4 sum|w x| + 1e-6 for GEMV links, the GELU product
bound for GELU links, the exact index (margin >= 1e-3) and the value bar for
the head. Data-dependent links (a GELU link writing the bf16 input a later
link reads) are checked against the oracle applied to what the GELU link
wrote, with every output poisoned first, so a link that read its input
before the writer had finished fails.
"""
import numpy as np
import pytest
import torch

import int4_weight_only_block_amd as q4
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def d(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def within(y_gpu, y_ref, a_ref, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    tol = oracle.gemv_tolerance(a_ref)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, f"{what}: {bad.size} over the bar, first {bad[:5]}, worst {float(np.max(err / tol)):.3g}"


class Mat:
    def __init__(self, rng, n, k):
        self.n, self.k = n, k
        self.codes, self.sb = synth.q4_weights(rng, n, k)
        self.packed = q4.q4_pack(d(self.codes), d(self.sb))


def _ffn_chain(rng, h=6144, k=1536, vocab=50000):
    """GELU gate+up [2h, k] -> down [k, h] reading its output -> a GEMV on
    its own input -> head [vocab, k]."""
    gu, dn, qkv, head = Mat(rng, 2 * h, k), Mat(rng, k, h), Mat(rng, 3 * k, k), Mat(rng, vocab, k)
    x0, x2, x3 = (synth.bf16_normal(rng, k) for _ in range(3))
    a = torch.full((h,), 0x7FC0, dtype=torch.int16, device=DEV)  # NaN until written
    y1 = torch.full((k,), float("nan"), device=DEV)
    y2 = torch.full((3 * k,), float("nan"), device=DEV)
    links = [q4.chain_link(gu.packed, 2 * h, k, d(x0), a, q4.LINK_GELU),
             q4.chain_link(dn.packed, k, h, a, y1, q4.LINK_GEMV, wait=True),
             q4.chain_link(qkv.packed, 3 * k, k, d(x2), y2, q4.LINK_GEMV, wait=True),
             q4.chain_link(head.packed, vocab, k, d(x3), None, q4.LINK_HEAD, wait=True)]
    return links, (gu, dn, qkv, head), (x0, x2, x3), (a, y1, y2)


def _check_ffn(mats, xs, outs, idx, val):
    gu, dn, qkv, head = mats
    x0, x2, x3 = xs
    a, y1, y2 = outs
    a_bits = a.cpu().numpy().view(np.uint16)
    ar, g, u, ag, au = oracle.gelu_mul(gu.codes, gu.sb, x0)
    tol = oracle.gelu_mul_tolerance(g, u, ag, au)
    assert (np.abs(oracle.bf16_bits_to_f64(a_bits) - ar) <= tol).all()
    yr, am = oracle.gemv(dn.codes, dn.sb, a_bits)  # the down link's input is what the GELU link wrote
    within(y1.cpu().numpy(), yr, am, "down reading the GELU output")
    yr, am = oracle.gemv(qkv.codes, qkv.sb, x2)
    within(y2.cpu().numpy(), yr, am, "third link")
    ref = oracle.lmhead(head.codes, head.sb, x3, 30.0)
    if ref["margin"] >= 1e-3:
        assert int(idx.item()) == ref["idx"]
    assert abs(float(val.item()) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6


def test_chain_dependent_links_and_head():
    torch.cuda.set_device(DEV)
    links, mats, xs, outs = _ffn_chain(synth.rng_for(800))
    ch = q4.q4_chain_build(links, cap=30.0)
    for rep in range(3):  # counters must come back clear after every call
        for o in outs:
            o.fill_(-1)  # bf16 / fp32 patterns no link writes by chance
        idx, val = q4.q4_gemv_chain(ch)
        torch.cuda.synchronize()
        assert ch.err() == 0
        _check_ffn(mats, xs, outs, idx, val)


def test_chain_in_a_graph():
    torch.cuda.set_device(DEV)
    links, mats, xs, outs = _ffn_chain(synth.rng_for(801), h=2048, k=1536, vocab=20000)
    ch = q4.q4_chain_build(links)
    idx = torch.empty(1, dtype=torch.int32, device=DEV)
    val = torch.empty(1, dtype=torch.float32, device=DEV)
    q4.q4_gemv_chain(ch, idx, val)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q4.q4_gemv_chain(ch, idx, val)
    for _ in range(4):
        for o in outs:
            o.fill_(-1)
        idx.fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        assert ch.err() == 0
        _check_ffn(mats, xs, outs, idx, val)


@pytest.mark.parametrize("wait", [True, False])
def test_chain_integer_exact_every_split(wait):
    """Power-of-two scales and integer activations: each link's sums are exact
    in fp32 in any order, so the chain equals the oracle bit for bit, for k
    covering every lane split (16, 32 and 64 lanes per row, ragged blocks)
    and ragged row counts."""
    torch.cuda.set_device(DEV)
    rng = np.random.default_rng(802)
    ks = [32, 96, 512, 1536, 2048, 2560, 3072, 5120, 6144, 8192, 10240]
    links, refs = [], []
    for i, k in enumerate(ks):
        n = int(rng.integers(1, 700))
        codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
        p = rng.integers(6, 9, size=(n, k // 32))
        sb = (2.0 ** -p).astype(np.float16).view(np.uint16)
        xi = rng.integers(-8, 9, size=k).astype(np.float32)
        x = synth.f32_to_bf16_bits(xi)
        y = torch.full((n,), float("nan"), device=DEV)
        links.append(q4.chain_link(q4.q4_pack(d(codes), d(sb)), n, k, d(x), y, q4.LINK_GEMV, wait=wait))
        refs.append(oracle.gemv(codes, sb, x)[0])
    ch = q4.q4_chain_build(links)
    q4.q4_gemv_chain(ch)
    torch.cuda.synchronize()
    assert ch.err() == 0
    for l, yr, k in zip(links, refs, ks):
        assert np.array_equal(l["out"].cpu().numpy().astype(np.float64), yr), k


def test_chain_independent_gemvs():
    """Links that read no earlier output need no wait: 48 [1536, 1536] GEMVs."""
    torch.cuda.set_device(DEV)
    rng = synth.rng_for(803)
    mats = [Mat(rng, 1536, 1536) for _ in range(48)]
    xs = [synth.bf16_normal(rng, 1536) for _ in range(48)]
    ys = [torch.full((1536,), float("nan"), device=DEV) for _ in range(48)]
    ch = q4.q4_chain_build([q4.chain_link(m.packed, 1536, 1536, d(x), y, wait=False)
                            for m, x, y in zip(mats, xs, ys)])
    q4.q4_gemv_chain(ch)
    torch.cuda.synchronize()
    assert ch.err() == 0
    for m, x, y in zip(mats, xs, ys):
        yr, a = oracle.gemv(m.codes, m.sb, x)
        within(y.cpu().numpy(), yr, a, "independent link")


def test_chain_wide_activations():
    """A link whose input holds a 2^40 outlier with zero codes on every row
    takes the exact path inside the chain."""
    torch.cuda.set_device(DEV)
    rng = synth.rng_for(804)
    m1, m2 = Mat(rng, 3072, 2560), Mat(rng, 2560, 10240)
    x1 = synth.bf16_normal(rng, 2560)
    x2 = synth.bf16_normal(rng, 10240)
    x2[333] = 0x5380  # bf16 2^40
    m2.codes[:, 333] = 0
    m2.packed = q4.q4_pack(d(m2.codes), d(m2.sb))
    y1 = torch.empty(3072, device=DEV)
    y2 = torch.empty(2560, device=DEV)
    ch = q4.q4_chain_build([q4.chain_link(m1.packed, 3072, 2560, d(x1), y1),
                            q4.chain_link(m2.packed, 2560, 10240, d(x2), y2, wait=True)])
    q4.q4_gemv_chain(ch)
    torch.cuda.synchronize()
    assert ch.err() == 0
    for m, x, y in ((m1, x1, y1), (m2, x2, y2)):
        yr, a = oracle.gemv(m.codes, m.sb, x)
        within(y.cpu().numpy(), yr, a, "wide")


def test_chain_wait_timeout_sets_error_and_recovers():
    """A 1 us bound on every wait: workgroups that reach a wait before the
    others have arrived give up, set the error word and leave (every wave
    exits normally). While the word is set a call does nothing; zeroing the
    workspace clears it, after which the same chain with the default bound
    is correct."""
    torch.cuda.set_device(DEV)
    rng = synth.rng_for(805)
    mats = [Mat(rng, 2560, 2560) for _ in range(6)]
    xs = [synth.bf16_normal(rng, 2560) for _ in range(6)]
    ys = [torch.empty(2560, device=DEV) for _ in range(6)]
    links = [q4.chain_link(m.packed, 2560, 2560, d(x), y, wait=True) for m, x, y in zip(mats, xs, ys)]
    tight = q4.q4_chain_build(links, spin_us=1)
    normal = q4.q4_chain_build(links)
    normal.ws = tight.ws  # one workspace for both
    q4.q4_gemv_chain(tight)
    torch.cuda.synchronize()
    e = tight.err()
    assert e in (0, 1)
    if e:
        for y in ys:
            y.fill_(float("nan"))
        q4.q4_gemv_chain(normal)  # refused by the kernel: outputs stay NaN
        torch.cuda.synchronize()
        assert all(torch.isnan(y).all() for y in ys)
        tight.clear()
    q4.q4_gemv_chain(normal)
    torch.cuda.synchronize()
    assert normal.err() == 0
    for m, x, y in zip(mats, xs, ys):
        yr, a = oracle.gemv(m.codes, m.sb, x)
        within(y.cpu().numpy(), yr, a, "after recovery")
