"""The decode step exactly as the benchmark times it, checked against the oracle.

bench.py captures one E4B-shaped S=1 decode step (PLE gather, 42 layers of
QKV / O / gate+up / down GEMVs, the LM head with softcap and argmax) in one
HIP graph and replays it. Here the same Workload is built on a fixed seed,
keeping the codes and scales of a few matrices, the graph is captured with
the same helper and replayed, and the outputs it wrote are compared with the
fp64 oracle: the head's index exactly (when the top-2 margin of the capped
logits is >= 1e-3) and its value, sampled layer GEMVs element by element
within the GEMV bar, and the PLE row bit for bit.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth

pytestmark = pytest.mark.gpu


def test_decode_step_graph_against_oracle():
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mats = synth.stack_e4b_matrices()
    head = len(mats) - 1
    # layer 0 QKV, gate+up and down, layer 20 O, layer 41 down, the head
    keep = {0, 2, 3, 4 * 20 + 1, 4 * 41 + 3, head}
    wl = bench.Workload(dev, seed=7, keep=keep)
    graph = bench.capture_step(torch, wl)
    # poison what the step writes, so only the replays can produce it
    for i in keep - {head}:
        wl.ys[i].fill_(float("nan"))
    wl.idx.fill_(-7)
    wl.val.fill_(float("nan"))
    wl.ple_out.fill_(float("nan"))
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()

    for i in sorted(keep):
        name, n, k = mats[i]
        codes, scales = wl.kept[i]
        c = codes.cpu().numpy()
        sb = scales.cpu().numpy().view(np.uint16)
        x = wl.xs[i].cpu().numpy().view(np.uint16)
        if i == head:
            ref = oracle.lmhead(c, sb, x, 30.0)
            got_i, got_v = int(wl.idx.item()), float(wl.val.item())
            if ref["margin"] >= 1e-3:
                assert got_i == ref["idx"], (got_i, ref["idx"], ref["margin"])
            assert abs(got_v - ref["val"]) <= 1e-4 * ref["a_idx"] + 1e-6, (got_v, ref["val"])
        else:
            yr, a = oracle.gemv(c, sb, x)
            y = wl.ys[i].cpu().numpy().astype(np.float64)
            err = np.abs(y - yr)
            tol = oracle.gemv_tolerance(a)
            assert (err <= tol).all(), f"{name}: {int((~(err <= tol)).sum())} of {n} over the bar"

    tok = int(wl.ids.item())
    row = wl.table[tok:tok + 1].cpu().numpy()
    sc = wl.scale[tok:tok + 1].cpu().numpy()
    ref, err = oracle.ple_gather(row, sc, np.array([0], np.int32), 16.0)
    assert err == 0
    got = wl.ple_out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
