"""lmhead_softcap_argmax_noalloc against lmhead_softcap_argmax, through the C ABI.

The allocation-free head keeps its per-workgroup partials in the library's
own device array instead of a caller workspace; it runs the same kernels, so
its (index, value) must equal the workspace entry point's bit for bit. Two
calls in a row, the second on a smaller head (fewer partials than the first
left in the array), then a third call captured in a HIP graph and replayed.
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


def _head(seed, vocab, k, nvec):
    rng = synth.rng_for(seed, vocab, k)
    codes, sb = synth.q4_weights(rng, vocab, k)
    xs = synth.bf16_normal(rng, (nvec, k))
    return codes, sb, xs


def _same(a, b):
    ia, va = a
    ib, vb = b
    assert int(ia.item()) == int(ib.item())
    assert np.array_equal(va.cpu().numpy().view(np.uint32), vb.cpu().numpy().view(np.uint32))


def test_noalloc_head_matches_workspace_head_two_calls():
    torch.cuda.set_device(DEV)
    # first call: the E2B-shaped head (the most partials); second: a smaller one
    for seed, vocab, k in ((700, 262144, 1536), (701, 5003, 2560)):
        codes, sb, xs = _head(seed, vocab, k, 3)
        packed = q4.q4_pack(d(codes), d(sb))
        for r in range(xs.shape[0]):
            x = d(xs[r])
            got = q4.lmhead_softcap_argmax_noalloc(packed, vocab, k, x, 30.0)
            want = q4.lmhead_softcap_argmax(packed, vocab, k, x, 30.0)
            torch.cuda.synchronize()
            _same(got, want)
            # and both against the oracle (index when the margin is clear)
            if r == 0:
                ref = oracle.lmhead(codes, sb, xs[r], 30.0)
                if ref["margin"] >= 1e-3:
                    assert int(got[0].item()) == ref["idx"]
                assert abs(float(got[1].item()) - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6


def test_noalloc_head_in_a_graph():
    torch.cuda.set_device(DEV)
    vocab, k = 40000, 2560
    codes, sb, xs = _head(702, vocab, k, 4)
    packed = q4.q4_pack(d(codes), d(sb))
    x = torch.empty(k, dtype=torch.int16, device=DEV)
    idx = torch.empty(1, dtype=torch.int32, device=DEV)
    val = torch.empty(1, dtype=torch.float32, device=DEV)
    x.copy_(d(xs[0]))
    q4.lmhead_softcap_argmax_noalloc(packed, vocab, k, x, 30.0, idx, val)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q4.lmhead_softcap_argmax_noalloc(packed, vocab, k, x, 30.0, idx, val)
    for r in range(4):
        x.copy_(d(xs[r]))
        g.replay()
        want = q4.lmhead_softcap_argmax(packed, vocab, k, x, 30.0)
        torch.cuda.synchronize()
        _same((idx, val), want)
