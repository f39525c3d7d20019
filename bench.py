"""Benchmark: one E4B-shaped S=1 decode step of the q4_0 hot path on one GPU.

A step is one pass of the whole hot path over one token:
  PLE gather (one id, E4B table [262144, 10752] int8, x16.0)
  -> 42 layers x {QKV [3072, 2560], O [2560, 2048], gate+up [20480, 2560],
                  down [2560, 10240]} q4_0 GEMVs
  -> LM head [262144, 2560] GEMV + softcap 30 + argmax.
Each GEMV reads its own resident bf16 N(0,1) activation vector; the kernels
run in dependency order on one stream, captured once in a HIP graph and
replayed. Weight bytes per step: 2,545,090,560 (0.5625 B per weight).

Prints ONE JSON line: value = decode-step weight bytes / step time (GB/s),
plus the roofline of the kernel that takes the most time per step (per-launch
durations from back-to-back HIP event pairs on the launch stream), the LM head
roofline, the S=64 prefill step when the GEMM is available, and the fp64
oracle timed on a bounded sample on the host cores.

Only one GPU is used; --gpus N with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "q4_0 GEMV/LM-head achieved HBM GB/s (% of peak); decode-step weight bytes/s"
HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "int4_weight_only_block_amd", "csrc", f)
                  for f in ("q4_gemv.hip", "ple_gather.hip", "q4dec_internal.h")]


def q4_bytes(n: int, k: int) -> int:
    """Algorithmic bytes of one q4_0 GEMV launch: nibbles + fp16 scales +
    bf16 activations + fp32 outputs."""
    return n * k // 2 + n * (k // 32) * 2 + 2 * k + 4 * n


def weight_bytes(n: int, k: int) -> int:
    return n * k // 2 + n * (k // 32) * 2


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip per-kernel event timing")
    ap.add_argument("--no-prefill", action="store_true", help="skip the S=64 prefill step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--verify-pass", action="store_true",
                    help="build the decode workload and run one 4-token verify pass eagerly, untimed "
                         "(for counter runs)")
    ap.add_argument("--heads-once", action="store_true",
                    help="run the single-vector LM head once on an E2B- and once on an E4B-shaped matrix, "
                         "untimed (for counter runs)")
    ap.add_argument("--gemm-shapes", metavar="NxK[,NxK...]",
                    help="run only q4_gemm_s64 on 64 tokens for each shape (4 distinct matrices, one "
                         "HIP graph per shape) and print us per launch (for counter runs)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="no GPU work: per-shape launch durations of every complete decode step in the "
                         "rocprofv3 kernel trace csv under DIR/ktr/, with the algorithmic bytes and the "
                         "rate and fraction of the HBM peak they give (one JSON line)")
    ap.add_argument("--counters-summary", metavar="DIR",
                    help="no GPU work: turn the rocprofv3 FETCH_SIZE / WRITE_SIZE csv output under DIR "
                         "(pmc_FETCH_SIZE/, pmc_WRITE_SIZE/ over one decode step, cal_FETCH_SIZE/, "
                         "cal_WRITE_SIZE/ over --copy-calibration) into profiles/hbm_counters.json")
    return ap.parse_args()


class Workload:
    """Resident inputs of one decode step (drawn on the GPU, seeded).

    ``keep`` names matrix indices (into ``mats``) whose unpacked codes and
    scales stay resident in ``kept`` so a test can check the step's outputs
    against the oracle."""

    def __init__(self, dev, seed: int, keep=()):
        import torch

        import int4_weight_only_block_amd as q4
        import synth

        self.q4 = q4
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        self.mats = synth.stack_e4b_matrices()
        self.packed, self.xs, self.ys = [], [], []
        self.kept = {}
        for i, (_, n, k) in enumerate(self.mats):
            codes, scales = synth.torch_q4_weights(g, n, k, dev)
            self.packed.append(q4.q4_pack(codes, scales))
            if i in keep:
                self.kept[i] = (codes, scales)
            del codes, scales
            self.xs.append(synth.torch_bf16_normal(g, k, dev))
            self.ys.append(torch.empty(n, dtype=torch.float32, device=dev))
        s = synth.SHAPES["ple_e4b"]
        self.vocab = s["vocab"]
        self.ple_dim = s["dim"]
        self.table = torch.randint(-127, 128, (s["vocab"], s["dim"]), dtype=torch.int8, device=dev,
                                   generator=g)
        self.scale = torch.empty(s["vocab"], dtype=torch.float32, device=dev).uniform_(1e-3, 1e-2, generator=g)
        self.ids = torch.randint(0, s["vocab"], (1,), dtype=torch.int32, device=dev, generator=g)
        self.ple_out = torch.empty((1, s["dim"]), dtype=torch.float32, device=dev)
        hn, hk = self.mats[-1][1], self.mats[-1][2]
        self.head_nk = (hn, hk)
        self.ws = torch.zeros(q4.lmhead_workspace_bytes(hn, hk), dtype=torch.uint8, device=dev)
        self.idx = torch.empty(1, dtype=torch.int32, device=dev)
        self.val = torch.empty(1, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    # one kernel-enqueuing callable per launch, in step order
    def launches(self):
        q4 = self.q4
        out = [("ple", lambda: q4.ple_gather(self.table, self.scale, self.ids, 16.0, out=self.ple_out))]
        for i, (name, n, k) in enumerate(self.mats[:-1]):
            out.append((name.split(".")[1], (lambda i=i, n=n, k=k: q4.q4_gemv(self.packed[i], n, k, self.xs[i],
                                                                               self.ys[i]))))
        hn, hk = self.head_nk
        out.append(("head", lambda: q4.lmhead_softcap_argmax(self.packed[-1], hn, hk, self.xs[-1], 30.0, self.ws,
                                                             self.idx, self.val)))
        return out

    def step(self):
        for _, fn in self.launches():
            fn()

    def gelu_launches(self):
        """The gate+up GEMVs as fused launches with the GELU-tanh * up
        epilogue (bf16 output for the down projection); timed on their own,
        not part of the step."""
        import torch

        q4 = self.q4
        if not hasattr(self, "_a_out"):
            self._a_out = {i: torch.empty(n // 2, dtype=torch.int16, device=self.xs[i].device)
                           for i, (name, n, k) in enumerate(self.mats[:-1]) if name.endswith("gate_up")}
        return [lambda i=i, n=n, k=k: q4.q4_gemv_gelu_mul(self.packed[i], n, k, self.xs[i], self._a_out[i])
                for i, (name, n, k) in enumerate(self.mats[:-1]) if name.endswith("gate_up")]

    def head_copies_launches(self):
        """Head launches over the resident head and two more copies of it
        (1.1 GB in rotation), for timing the head kernel on its own."""
        import torch

        if not hasattr(self, "_head_copies"):
            self._head_copies = [self.packed[-1]] + [self.packed[-1].clone() for _ in range(2)]
            torch.cuda.synchronize()
        q4, (hn, hk) = self.q4, self.head_nk
        return [lambda p=p: q4.lmhead_softcap_argmax(p, hn, hk, self.xs[-1], 30.0, self.ws, self.idx, self.val)
                for p in self._head_copies]

    def weight_bytes(self) -> int:
        return sum(weight_bytes(n, k) for _, n, k in self.mats)

    # ------------------------------------------------------ S=64 prefill step
    def prefill_setup(self, gen):
        """64-token activations per GEMM (bf16 N(0,1)), fp32 outputs and one
        shared workspace (the GEMMs run one after another on one stream)."""
        import synth
        import torch

        dev = self.xs[0].device
        self.pxs, self.pys = [], []
        ws_need = 0
        for _, n, k in self.mats[:-1]:
            self.pxs.append(synth.torch_bf16_normal(gen, (64, k), dev))
            self.pys.append(torch.empty((64, n), dtype=torch.float32, device=dev))
            ws_need = max(ws_need, self.q4.q4_gemm_workspace_bytes(n, k))
        self.pws = torch.empty(ws_need, dtype=torch.uint8, device=dev)
        self.p_head_x = synth.torch_bf16_normal(gen, (64, self.head_nk[1]), dev)
        torch.cuda.synchronize()

    def prefill_step(self):
        """PLE gather for 64 ids, 42 x 4 S=64 GEMMs, head on the chunk's last
        row (the only row a decoder samples from)."""
        q4 = self.q4
        q4.ple_gather(self.table, self.scale, self.p_ids, 16.0, out=self.p_ple_out)
        for i, (_, n, k) in enumerate(self.mats[:-1]):
            q4.q4_gemm_s64(self.packed[i], n, k, self.pxs[i], self.pys[i], self.pws)
        hn, hk = self.head_nk
        q4.lmhead_softcap_argmax(self.packed[-1], hn, hk, self.p_head_x[63], 30.0, self.ws, self.idx, self.val)

    def prefill_flops(self) -> int:
        return sum(2 * 64 * n * k for _, n, k in self.mats[:-1]) + 2 * self.head_nk[0] * self.head_nk[1]


def capture_step(torch, wl: Workload):
    """One eager pass (lazy initialisation), then the decode step captured
    in a HIP graph on the current stream."""
    wl.step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wl.step()
    return graph


def probe_kernels(torch, wl: Workload, reps: int = 20):
    """Average per-launch duration (ms) of each launch kind: the launches of
    one kind (42 distinct matrices per GEMV kind; three distinct copies of the
    head so consecutive launches cannot hit the infinity cache), repeated to
    at least 24 launches so the graph's own replay cost is amortised, are
    captured in their own HIP graph and replayed between HIP events on the
    launch stream."""
    launches = wl.launches() + [("gate_up_gelu", fn) for fn in wl.gelu_launches()]
    kinds = []
    for kind, _ in launches:
        if kind not in kinds:
            kinds.append(kind)
    out = {}
    for kind in kinds:
        fns = [fn for kk, fn in launches if kk == kind]
        if kind == "head":
            fns = wl.head_copies_launches()
        fns = fns * max(1, -(-24 // len(fns)))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for fn in fns:
                fn()
        graph.replay()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        out[kind] = e0.elapsed_time(e1) / (reps * len(fns))
        del graph
    return out


def probe_chain(torch, wl: Workload, graph, reps: int = 10):
    """The same decode step as one persistent chain launch (q4_gemv_chain:
    the 168 layer GEMVs and the head as links, each waiting for the one
    before) after the PLE gather, timed in a HIP graph and eagerly, beside
    the eager sequence of the step's 171 launches and the graph of it (the
    timed step). Eager timings include the host's launch cost."""
    q4 = wl.q4
    hn, hk = wl.head_nk
    links = [q4.chain_link(wl.packed[i], n, k, wl.xs[i], wl.ys[i], q4.LINK_GEMV, wait=True)
             for i, (_, n, k) in enumerate(wl.mats[:-1])]
    links.append(q4.chain_link(wl.packed[-1], hn, hk, wl.xs[-1], None, q4.LINK_HEAD, wait=True))
    ch = q4.q4_chain_build(links, cap=30.0)

    def chain_step():
        q4.ple_gather(wl.table, wl.scale, wl.ids, 16.0, out=wl.ple_out)
        q4.q4_gemv_chain(ch, wl.idx, wl.val)

    def timed(fn, r):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(r):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / r

    chain_step()
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        chain_step()
    cg.replay()
    out = {"links": len(links), "launches_per_step": 2,
           "graph_ms": round(timed(cg.replay, reps), 4),
           "eager_ms": round(timed(chain_step, reps), 4),
           "launch_sequence_eager_ms": round(timed(wl.step, reps), 4),
           "launch_sequence_graph_ms": round(timed(graph.replay, reps), 4),
           "err_word": ch.err()}
    del cg
    return out


def probe_verify_m4(torch, wl: Workload, seed: int, reps: int = 10, once: bool = False):
    """A 4-token verify pass: the 168 layer GEMVs with m = 4 activation
    vectors each (q4_gemv_multi: every weight read once for the 4 tokens)
    and the head for the same 4 vectors with softcap and per-vector argmax
    (lmhead_softcap_argmax_multi), one HIP graph; reported as ms per pass,
    the head alone in us, and weight bytes/s. Not part of the decode step.
    With once, the pass runs one time, eagerly, and nothing is timed (for
    counter runs, which then see each of its launches once)."""
    import int4_weight_only_block_amd as q4
    import synth

    dev = wl.xs[0].device
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 3)
    mats = wl.mats[:-1]
    _, vocab, kh = wl.mats[-1]
    xs4 = [synth.torch_bf16_normal(g, (4, k), dev) for _, n, k in mats]
    ys4 = [torch.empty((4, n), dtype=torch.float32, device=dev) for _, n, k in mats]
    xh4 = synth.torch_bf16_normal(g, (4, kh), dev)
    ws = torch.empty(q4.lmhead_multi_workspace_bytes(vocab, kh, 4), dtype=torch.uint8, device=dev)
    idx = torch.empty(4, dtype=torch.int32, device=dev)
    val = torch.empty(4, dtype=torch.float32, device=dev)

    def head():
        q4.lmhead_softcap_argmax_multi(wl.packed[-1], vocab, kh, xh4, 30.0, ws, idx, val)

    def run():
        for i, (_, n, k) in enumerate(mats):
            q4.q4_gemv_multi(wl.packed[i], n, k, xs4[i], ys4[i])
        head()

    def time_graph(fn, r):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(r):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / r

    if once:
        run()
        torch.cuda.synchronize()
        return {"verify_pass_launches": len(mats) + 2}
    ms = time_graph(run, reps)
    head_us = time_graph(head, 10 * reps) * 1e3
    wb = sum(weight_bytes(n, k) for _, n, k in mats) + weight_bytes(vocab, kh)
    hb = weight_bytes(vocab, kh)
    return {"m": 4, "launches": len(mats) + 2, "ms_per_pass": round(ms, 4), "weight_bytes": wb,
            "weight_GBs": round(wb / (ms * 1e-3) / 1e9, 1), "frac_of_hbm_peak": round(wb / (ms * 1e-3) / 8e12, 4),
            "head_4_vectors_us": round(head_us, 2), "head_weight_GBs": round(hb / head_us / 1e3, 1)}


def probe_head_s64(torch, wl: Workload, reps: int = 10):
    """The head for every row of a 64-token prefill chunk
    (lmhead_softcap_argmax_s64: the S=64 MFMA kernel with a per-token argmax
    epilogue) on the E4B head, rotating over three copies of it so no call
    finds its weights in the infinity cache; reported per call (64 tokens)."""
    q4 = wl.q4
    hn, hk = wl.head_nk
    wl.head_copies_launches()  # makes the three copies of the head
    ws = torch.zeros(q4.lmhead_s64_workspace_bytes(hn, hk), dtype=torch.uint8, device=wl.p_head_x.device)
    idx = torch.empty(64, dtype=torch.int32, device=ws.device)
    val = torch.empty(64, dtype=torch.float32, device=ws.device)

    def run():
        for p in wl._head_copies:
            q4.lmhead_softcap_argmax_s64(p, hn, hk, wl.p_head_x, 30.0, ws, idx, val)

    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(wl._head_copies))
    del graph
    wb = weight_bytes(hn, hk)
    flops = 2 * 64 * hn * hk
    return {"shape": [hn, hk], "tokens": 64, "avg_call_us": round(us, 2),
            "weight_GBs": round(wb / us / 1e3, 1), "TFLOPs": round(flops / us / 1e6, 1),
            "us_per_token": round(us / 64, 3)}


def probe_quantize(torch, dev, seed: int, reps: int = 20):
    """q4_quantize on an E4B gate+up sized bf16 matrix [20480, 2560] (the
    export step, not part of a decode step): bf16 read + int8 codes + fp16
    scales written, four distinct matrices in rotation."""
    import int4_weight_only_block_amd as q4
    import synth

    g = torch.Generator(device=dev)
    g.manual_seed(seed + 2)
    n, k = 20480, 2560
    xs = [synth.torch_bf16_normal(g, (n, k), dev) for _ in range(4)]
    codes = torch.empty((n, k), dtype=torch.int8, device=dev)
    scales = torch.empty((n, k // 32), dtype=torch.int16, device=dev)
    q4.q4_quantize(xs[0], q4.QUANT_Q4_0, codes, scales)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x in xs:
            q4.q4_quantize(x, q4.QUANT_Q4_0, codes, scales)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(xs))
    b = n * k * 2 + n * k + n * (k // 32) * 2
    return {"shape": [n, k], "rule": "q4_0", "avg_launch_us": round(us, 3), "bytes_per_launch": b,
            "achieved_GBs": round(b / us / 1e3, 1), "frac_of_hbm_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}


def probe_pack(torch, dev, seed: int, reps: int = 20):
    """q4_pack on an E4B gate+up sized matrix [20480, 2560] (load time, not
    part of a decode step): int8 codes and fp16 scales read, the packed
    nibble and scale planes written, four distinct inputs in rotation; one
    kernel per call."""
    import int4_weight_only_block_amd as q4
    import synth

    g = torch.Generator(device=dev)
    g.manual_seed(seed + 6)
    n, k = 20480, 2560
    ins = [synth.torch_q4_weights(g, n, k, dev) for _ in range(4)]
    packed = torch.empty(q4.q4_packed_bytes(n, k), dtype=torch.uint8, device=dev)
    q4.q4_pack(ins[0][0], ins[0][1], packed)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c, sc in ins:
            q4.q4_pack(c, sc, packed)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(ins))
    b = n * k + n * (k // 32) * 2 + weight_bytes(n, k)
    return {"shape": [n, k], "avg_call_us": round(us, 3), "bytes_per_call": b,
            "achieved_GBs": round(b / us / 1e3, 1), "frac_of_hbm_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}


def probe_rowq(torch, dev, seed: int, reps: int = 20):
    """Per-row symmetric INT2 GEMVs on the mobile mixed-bit kernel-probe
    workload: six INT2 FFNs (gate and up [12288, 1536], down [1536, 12288])
    and the INT2 262,144-row head [262144, 1536], 185 MB of codes per run,
    one HIP graph. Each FFN runs as the fused gate/up GELU launch plus the
    down GEMV (13 launches); the unfused run (gate, up and down as separate
    GEMVs, 19 launches) and a run whose head is the fused softcap + argmax
    (no logits written; 14 launches) are timed too. Not part of the q4_0 decode step. Bytes
    counted: packed codes + fp32 row scales + bf16 x + the outputs."""
    import int4_weight_only_block_amd as q4

    g = torch.Generator(device=dev)
    g.manual_seed(seed + 4)
    H, D, V = 12288, 1536, 262144

    def codes(n, k):
        return torch.randint(0, 256, (n, k // 4), dtype=torch.uint8, device=dev, generator=g)

    def scales(n):
        return torch.empty(n, dtype=torch.float32, device=dev).uniform_(1e-3, 1e-2, generator=g)

    ffn = [(codes(2 * H, D), scales(2 * H), codes(D, H), scales(D)) for _ in range(6)]
    head, head_sc = codes(V, D), scales(V)
    x = torch.randn(D, device=dev, generator=g).to(torch.bfloat16)
    a = torch.empty(H, dtype=torch.int16, device=dev)
    gu = torch.empty(2 * H, dtype=torch.float32, device=dev)
    y = torch.empty(D, dtype=torch.float32, device=dev)
    logits = torch.empty(V, dtype=torch.float32, device=dev)

    def run_fused():
        for w_gu, s_gu, w_dn, s_dn in ffn:
            q4.rowq_gemv_gelu_mul(w_gu, s_gu, 2 * H, D, 2, x, a)
            q4.rowq_gemv(w_dn, s_dn, D, H, 2, a, y)
        q4.rowq_gemv(head, head_sc, V, D, 2, x, logits)

    ws = torch.empty(q4.rowq_head_workspace_bytes(V, D, 2), dtype=torch.uint8, device=dev)
    hi = torch.empty(1, dtype=torch.int32, device=dev)
    hv = torch.empty(1, dtype=torch.float32, device=dev)

    def run_argmax():
        for w_gu, s_gu, w_dn, s_dn in ffn:
            q4.rowq_gemv_gelu_mul(w_gu, s_gu, 2 * H, D, 2, x, a)
            q4.rowq_gemv(w_dn, s_dn, D, H, 2, a, y)
        q4.rowq_softcap_argmax(head, head_sc, V, D, 2, x, 30.0, ws, hi, hv)

    def run_unfused():
        for w_gu, s_gu, w_dn, s_dn in ffn:
            q4.rowq_gemv(w_gu[:H], s_gu[:H], H, D, 2, x, gu[:H])
            q4.rowq_gemv(w_gu[H:], s_gu[H:], H, D, 2, x, gu[H:])
            q4.rowq_gemv(w_dn, s_dn, D, H, 2, a, y)
        q4.rowq_gemv(head, head_sc, V, D, 2, x, logits)

    def time_graph(fn):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = time_graph(run_fused)
    ms_unfused = time_graph(run_unfused)
    ms_argmax = time_graph(run_argmax)
    code_bytes = 6 * (2 * H * D + D * H) // 4 + V * D // 4
    b = (code_bytes + 4 * (6 * (2 * H + D) + V) + 2 * (6 * (D + H) + D)
         + 6 * (2 * H + 4 * D) + 4 * V)
    return {"workload": "int2_kprobe_6ffn_plus_head", "launches": 13, "ms_per_run": round(ms, 4),
            "ms_per_run_unfused_19_launches": round(ms_unfused, 4),
            "ms_per_run_head_fused_argmax_14_launches": round(ms_argmax, 4), "code_bytes": code_bytes,
            "bytes_per_run": b, "achieved_GBs": round(b / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def probe_configs(torch, dev, wl: Workload, seed: int, reps: int = 10):
    """The smaller workloads, each in its own HIP graph over distinct copies
    so no launch finds its weights in the infinity cache:

    * gemv_1536: 768 distinct q4_0 [1536, 1536] matrices (1.02 GB) back to
      back, plus the latency of one launch alone (one-launch graph replayed,
      and an eager launch between two events, median of 100);
    * ffn_e2b: 64 distinct E2B FFN pairs, the fused gate/up GELU launch
      [12288, 1536] then the down GEMV [1536, 6144] on its bf16 output;
    * head_e2b: the E2B-shaped head [262144, 1536] with softcap + argmax,
      100 activation vectors over 3 copies of the head, one vector per call,
      and the same 100 vectors 8 per call (13 calls of the multi-vector head);
    * ple: the E2B table [262144, 8960] for 1 and 64 ids, the E4B table
      [262144, 10752] for 64 ids;
    * rowq_gather: the mixed-bit INT2 token embedding [262144, 1536] and the
      INT4 PLE table [262144, 35 x 256], for 1 and 64 ids;
    * rowq_int8: the mixed-bit INT8 per-row GEMVs (PLE gate [256, 1536],
      projection [1536, 256], model projection [8960, 1536]);
    * rowq_head_int2: the tied INT2 head [262144, 1536] with softcap + argmax,
      100 vectors over 3 copies, and its logits-only GEMV."""
    import int4_weight_only_block_amd as q4
    import synth

    g = torch.Generator(device=dev)
    g.manual_seed(seed + 5)

    def packed(n, k):
        codes, scales = synth.torch_q4_weights(g, n, k, dev)
        return q4.q4_pack(codes, scales)

    def time_graph(fn, r=reps):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(r):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) / r * 1e3  # us per replay

    def rate(b, us):
        return {"achieved_GBs": round(b / us / 1e3, 1), "frac_of_hbm_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}

    out = {}
    # --- one small GEMV
    n = k = 1536
    mats = [packed(n, k) for _ in range(768)]
    x = synth.torch_bf16_normal(g, k, dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)

    def run_gemv():
        for p in mats:
            q4.q4_gemv(p, n, k, x, y)

    us = time_graph(run_gemv) / len(mats)
    one_graph_us = time_graph(lambda: q4.q4_gemv(mats[0], n, k, x, y), 200)
    eager = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(100):
        e0.record()
        q4.q4_gemv(mats[i], n, k, x, y)
        e1.record()
        torch.cuda.synchronize()
        eager.append(e0.elapsed_time(e1) * 1e3)
    eager.sort()
    out["gemv_1536"] = {"shape": [n, k], "matrices": len(mats), "avg_launch_us": round(us, 3),
                        "bytes_per_launch": q4_bytes(n, k), **rate(q4_bytes(n, k), us),
                        "single_launch_graph_us": round(one_graph_us, 3),
                        "single_launch_eager_us_median": round(eager[len(eager) // 2], 3)}
    del mats
    # --- E2B FFN pair
    H, D = 6144, 1536
    pairs = [(packed(2 * H, D), packed(D, H)) for _ in range(64)]
    a = torch.empty(H, dtype=torch.int16, device=dev)

    def run_ffn():
        for gu, dn in pairs:
            q4.q4_gemv_gelu_mul(gu, 2 * H, D, x, a)
            q4.q4_gemv(dn, D, H, a, y)

    us = time_graph(run_ffn) / len(pairs)
    b = weight_bytes(2 * H, D) + 2 * D + 2 * H + weight_bytes(D, H) + 2 * H + 4 * D
    out["ffn_e2b"] = {"gate_up": [2 * H, D], "down": [D, H], "pairs": len(pairs), "launches_per_pair": 2,
                      "avg_pair_us": round(us, 3), "bytes_per_pair": b, **rate(b, us)}
    del pairs
    # --- E2B-shaped head, 100 vectors
    V = 262144
    heads = [packed(V, D) for _ in range(3)]
    xs = synth.torch_bf16_normal(g, (100, D), dev)
    ws = torch.zeros(q4.lmhead_workspace_bytes(V, D), dtype=torch.uint8, device=dev)
    idx = torch.empty(100, dtype=torch.int32, device=dev)
    val = torch.empty(100, dtype=torch.float32, device=dev)

    def run_head():
        for i in range(100):
            q4.lmhead_softcap_argmax(heads[i % 3], V, D, xs[i], 30.0, ws, idx[i:i + 1], val[i:i + 1])

    us = time_graph(run_head, 3) / 100
    b = weight_bytes(V, D) + 2 * D + 8
    wsm = torch.zeros(q4.lmhead_multi_workspace_bytes(V, D, 8), dtype=torch.uint8, device=dev)
    batches = [(s, min(8, 100 - s)) for s in range(0, 100, 8)]

    def run_head_multi():
        for j, (s, m) in enumerate(batches):
            q4.lmhead_softcap_argmax_multi(heads[j % 3], V, D, xs[s:s + m], 30.0, wsm, idx[s:s + m], val[s:s + m])

    us_m = time_graph(run_head_multi, 3)
    out["head_e2b"] = {"shape": [V, D], "vectors": 100, "copies": 3, "avg_call_us": round(us, 3),
                       "bytes_per_call": b, **rate(b, us),
                       "multi_8_per_call_us_for_100": round(us_m, 2), "multi_calls": len(batches)}
    del heads
    # --- PLE gathers
    s2 = synth.SHAPES["ple_e2b"]
    t2 = torch.randint(-127, 128, (s2["vocab"], s2["dim"]), dtype=torch.int8, device=dev, generator=g)
    sc2 = torch.empty(s2["vocab"], dtype=torch.float32, device=dev).uniform_(1e-3, 1e-2, generator=g)
    ple = {}
    for name, table, scale in (("e2b", t2, sc2), ("e4b", wl.table, wl.scale)):
        vocab, dim = table.shape
        for T in ((1, 64) if name == "e2b" else (64,)):
            ids = torch.randint(0, vocab, (32, T), dtype=torch.int32, device=dev, generator=g)
            o = torch.empty((T, dim), dtype=torch.float32, device=dev)

            def run_ple(table=table, scale=scale, ids=ids, o=o):
                for r in range(ids.shape[0]):
                    q4.ple_gather(table, scale, ids[r], 16.0, out=o)

            us = time_graph(run_ple) / ids.shape[0]
            b = T * (dim + 4 + 4 * dim + 4)
            ple[f"{name}_T{T}"] = {"table": [vocab, dim], "ids": T, "avg_launch_us": round(us, 3),
                                   "bytes_per_launch": b, "achieved_GBs": round(b / us / 1e3, 1)}
    out["ple"] = ple
    del t2, sc2
    # --- mixed-bit tables: INT2 token embedding, INT4 PLE table
    rg = {}
    for name, bits, dim, group, mult in (("int2_embed", 2, 1536, 1536, 39.191837), ("int4_ple", 4, 8960, 256, 16.0)):
        V = synth.VOCAB
        w = torch.randint(0, 256, (V, dim * bits // 8), dtype=torch.uint8, device=dev, generator=g)
        sc = torch.empty((V, dim // group), dtype=torch.float32, device=dev).uniform_(1e-3, 1e-2, generator=g)
        for T in (1, 64):
            ids = torch.randint(0, V, (32, T), dtype=torch.int32, device=dev, generator=g)
            o = torch.empty((T, dim), dtype=torch.float32, device=dev)

            def run_rg(w=w, sc=sc, ids=ids, o=o, bits=bits, group=group, mult=mult):
                for r in range(ids.shape[0]):
                    q4.rowq_gather(w, sc, bits, group, ids[r], mult, out=o)

            us = time_graph(run_rg) / ids.shape[0]
            b = T * (dim * bits // 8 + 4 * (dim // group) + 4 + 4 * dim)
            rg[f"{name}_T{T}"] = {"table": [V, dim], "bits": bits, "group": group, "ids": T,
                                  "avg_launch_us": round(us, 3), "bytes_per_launch": b,
                                  "achieved_GBs": round(b / us / 1e3, 1)}
        del w, sc
    out["rowq_gather"] = rg
    # --- INT8 per-row GEMVs of the mixed-bit recipe (PLE gate, PLE projection,
    # per-layer model projection), 35 distinct copies each (one per layer)
    r8 = {}
    for name, n, k in (("ple_gate", 256, 1536), ("ple_proj", 1536, 256), ("model_proj", 8960, 1536)):
        ws8 = [torch.randint(0, 256, (n, k), dtype=torch.uint8, device=dev, generator=g) for _ in range(35)]
        sc8 = torch.empty(n, dtype=torch.float32, device=dev).uniform_(1e-3, 1e-2, generator=g)
        x8 = synth.torch_bf16_normal(g, k, dev)
        y8 = torch.empty(n, dtype=torch.float32, device=dev)

        def run_r8(ws8=ws8, sc8=sc8, x8=x8, y8=y8, n=n, k=k):
            for w8 in ws8:
                q4.rowq_gemv(w8, sc8, n, k, 8, x8, y8)

        us = time_graph(run_r8) / len(ws8)
        b = n * k + 4 * n + 2 * k + 4 * n
        r8[name] = {"shape": [n, k], "avg_launch_us": round(us, 3), "bytes_per_launch": b,
                    "achieved_GBs": round(b / us / 1e3, 1)}
        del ws8
    out["rowq_int8"] = r8
    # --- the tied INT2 head [262144, 1536] with softcap + argmax, 100 vectors
    # over 3 copies, one vector per call; the logits-only GEMV beside it
    V = synth.VOCAB
    h2 = [torch.randint(0, 256, (V, D // 4), dtype=torch.uint8, device=dev, generator=g) for _ in range(3)]
    hs2 = torch.empty(V, dtype=torch.float32, device=dev).uniform_(1e-3, 1e-2, generator=g)
    wsr = torch.zeros(q4.rowq_head_workspace_bytes(V, D, 2), dtype=torch.uint8, device=dev)
    lg = torch.empty(V, dtype=torch.float32, device=dev)

    def run_rhead():
        for i in range(100):
            q4.rowq_softcap_argmax(h2[i % 3], hs2, V, D, 2, xs[i], 30.0, wsr, idx[i:i + 1], val[i:i + 1])

    def run_rlogits():
        for i in range(100):
            q4.rowq_gemv(h2[i % 3], hs2, V, D, 2, xs[i], lg)

    us = time_graph(run_rhead, 3) / 100
    us_l = time_graph(run_rlogits, 3) / 100
    b = V * D // 4 + 4 * V + 2 * D + 8
    out["rowq_head_int2"] = {"shape": [V, D], "vectors": 100, "copies": 3, "launches_per_call": 2,
                             "avg_call_us": round(us, 3), "bytes_per_call": b, **rate(b, us),
                             "logits_only_gemv_us": round(us_l, 3)}
    del h2
    torch.cuda.synchronize()
    return out


def cpu_baseline(seconds: float):
    """fp64 oracle on a bounded sample of the decode step: whole matrices of
    layer 0 (QKV, O, gate+up, down) and then row slices of the head until the
    time budget is spent. Returns weight-GB/s on the host cores."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import synth

    rng = synth.rng_for(0, 99)
    sample = [("qkv", 3072, 2560), ("o", 2560, 2048), ("gate_up", 20480, 2560), ("down", 2560, 10240)]
    mats = []
    for name, n, k in sample:
        codes, sb = synth.q4_weights(rng, n, k)
        mats.append((name, codes, sb, synth.bf16_normal(rng, k)))
    head_rows = 16384
    hc, hs = synth.q4_weights(rng, head_rows, 2560)
    hx = synth.bf16_normal(rng, 2560)
    done_bytes = 0
    parts = []
    t0 = time.perf_counter()
    for name, codes, sb, x in mats:
        oracle.gemv(codes, sb, x)
        done_bytes += weight_bytes(*codes.shape)
        parts.append(name)
    n_head = 0
    while time.perf_counter() - t0 < seconds:
        out = oracle.lmhead(hc, hs, hx)
        assert out["idx"] >= 0
        done_bytes += weight_bytes(head_rows, 2560)
        n_head += head_rows
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": round(done_bytes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle: E4B layer-0 {'/'.join(parts)} GEMVs plus {n_head} head rows "
                   f"[{head_rows}-row slices of 262144x2560 with softcap+argmax]; "
                   f"{done_bytes / 1e9:.3f} GB of q4_0 weights in {dt:.1f} s"),
        "host_cpus": os.cpu_count(),
        "host_cpu_model": host_cpu_model(),
    }


def host_cpu_model() -> str:
    """The host CPU's model name (as lscpu reports it, read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_configs():
    """The fp64 oracle on each smaller workload, one call each (wall time on
    the host cores): the [1536, 1536] GEMV, the E2B FFN pair (gate/up GEMV
    with the GELU product, then the down GEMV), the E2B-shaped head for one
    vector, and the PLE gather of 64 ids from an E2B-wide table (4096 rows:
    the gather's work depends on the ids and the row width, not the row
    count)."""
    import oracle
    import synth

    rng = synth.rng_for(0, 98)
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    c, sb = synth.q4_weights(rng, 1536, 1536)
    x = synth.bf16_normal(rng, 1536)
    dt = min(timed(lambda: oracle.gemv(c, sb, x)) for _ in range(3))
    out["gemv_1536"] = {"seconds": round(dt, 5), "GBs": round(q4_bytes(1536, 1536) / dt / 1e9, 3)}
    H, D = 6144, 1536
    cg, sg = synth.q4_weights(rng, 2 * H, D)
    cd, sd = synth.q4_weights(rng, D, H)

    def ffn():
        _, g, u, _, _ = oracle.gelu_mul(cg, sg, x)
        oracle.gemv(cd, sd, oracle.ffn_down_input_bits(g, u))

    dt = min(timed(ffn) for _ in range(2))
    b = weight_bytes(2 * H, D) + weight_bytes(D, H)
    out["ffn_e2b"] = {"seconds": round(dt, 4), "GBs": round(b / dt / 1e9, 3)}
    del cg, sg, cd, sd
    ch, shb = synth.q4_weights(rng, synth.VOCAB, D)
    dt = timed(lambda: oracle.lmhead(ch, shb, x))
    out["head_e2b"] = {"seconds": round(dt, 3), "GBs": round(weight_bytes(synth.VOCAB, D) / dt / 1e9, 3)}
    del ch, shb
    dim = synth.SHAPES["ple_e2b"]["dim"]
    table, scale, ids = synth.ple_inputs(rng, 4096, dim, 64)
    dt = min(timed(lambda: oracle.ple_gather(table, scale, ids)) for _ in range(3))
    out["ple_e2b_T64"] = {"seconds": round(dt, 5), "GBs": round(64 * (dim + 4 + 4 * dim + 4) / dt / 1e9, 3)}
    return out


def load_traffic(shape: str):
    """HBM bytes per launch of one launch shape, from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summaries scaled by the copy-kernel calibration;
    None when absent or when the kernel source changed since the counters
    were taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    with open(COUNTERS_FILE) as f:
        c = json.load(f)
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = c.get("shapes", {}).get(shape)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


def counters_summary(d: str) -> dict:
    """HBM bytes per launch of every decode-step launch shape from rocprofv3
    counter csv files: the last complete step's dispatches (PLE gather, then
    42 x {QKV, O, gate+up, down}, then the head) are matched to the shapes by
    their order, FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by
    what the same counters read for a plain copy of known size, and each
    shape's launches are averaged."""
    import csv

    import synth

    def rows(sub):
        files = [f for f in os.listdir(os.path.join(d, sub)) if f.endswith("counter_collection.csv")]
        if len(files) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {sub}, found {files}")
        with open(os.path.join(d, sub, files[0])) as f:
            return list(csv.DictReader(f))

    def step(sub):
        rs = [r for r in rows(sub) if "q4dec::" in r["Kernel_Name"]
              and ("q4_rows_kernel" in r["Kernel_Name"] or "ple_gather" in r["Kernel_Name"])]
        starts = [i for i, r in enumerate(rs) if "ple_gather" in r["Kernel_Name"]]
        mats = synth.stack_e4b_matrices()
        for s0 in reversed(starts):
            seq = rs[s0:s0 + 1 + len(mats)]
            if len(seq) == 1 + len(mats) and ", 1, " in seq[-1]["Kernel_Name"]:  # ends in the head kernel
                names = ["ple"] + [nm.split(".")[-1] for nm, _, _ in mats]
                return [(nm, float(r["Counter_Value"])) for nm, r in zip(names, seq)]
        raise SystemExit(f"no complete decode step under {sub}")

    def copy_kib(sub):
        vals = [float(r["Counter_Value"]) for r in rows(sub) if "copyBuffer" in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no copy dispatch under {sub}")
        return sum(vals) / len(vals)

    gib_kib = float(1 << 20)
    fetch_scale = gib_kib / copy_kib("cal_FETCH_SIZE")
    write_scale = gib_kib / copy_kib("cal_WRITE_SIZE")
    fetch, write = step("pmc_FETCH_SIZE"), step("pmc_WRITE_SIZE")
    shapes = {}
    for (nm, fv), (nm2, wv) in zip(fetch, write):
        assert nm == nm2
        e = shapes.setdefault(nm, {"fetch_kib": [], "write_kib": []})
        e["fetch_kib"].append(fv)
        e["write_kib"].append(wv)
    out = {}
    for nm, e in shapes.items():
        f = sum(e["fetch_kib"]) / len(e["fetch_kib"])
        w = sum(e["write_kib"]) / len(e["write_kib"])
        out[nm] = {"launches": len(e["fetch_kib"]), "fetch_kib_raw": round(f, 3), "write_kib_raw": round(w, 3),
                   "hbm_bytes_per_launch": int(round((f * fetch_scale + w * write_scale) * 1024))}
    return {"kernel_source_hash": kernel_source_hash(), "fetch_scale": round(fetch_scale, 6),
            "write_scale": round(write_scale, 6),
            "calibration": f"plain 1 GiB device copy: FETCH_SIZE {copy_kib('cal_FETCH_SIZE'):.1f} KiB, "
                           f"WRITE_SIZE {copy_kib('cal_WRITE_SIZE'):.1f} KiB per dispatch",
            "shapes": out}


def trace_summary(d: str) -> dict:
    """Per-shape durations (End - Start of each dispatch) of every complete
    decode step in a rocprofv3 kernel trace: a PLE gather followed by the
    step's 169 q4_0 launches in order (42 x {QKV, O, gate+up, down}, then the
    head), matched to the shapes by that order."""
    import csv
    import statistics

    import synth

    sub = os.path.join(d, "ktr")
    files = [f for f in os.listdir(sub) if f.endswith("kernel_trace.csv")]
    if len(files) != 1:
        raise SystemExit(f"expected one kernel_trace.csv under {sub}, found {files}")
    with open(os.path.join(sub, files[0])) as f:
        rs = [r for r in csv.DictReader(f) if "q4dec::" in r["Kernel_Name"]]
    rs.sort(key=lambda r: int(r["Start_Timestamp"]))
    mats = synth.stack_e4b_matrices()
    kinds = ["ple"] + [nm.split(".")[-1] for nm, _, _ in mats]
    durs = {kd: [] for kd in dict.fromkeys(kinds)}
    steps, i = 0, 0
    while i < len(rs):
        seq = rs[i:i + len(kinds)]
        ok = (len(seq) == len(kinds) and "ple_gather" in seq[0]["Kernel_Name"]
              and all("q4_rows_kernel" in r["Kernel_Name"] for r in seq[1:])
              and ", 1, " in seq[-1]["Kernel_Name"])  # the head mode
        if not ok:
            i += 1
            continue
        for kd, r in zip(kinds, seq):
            durs[kd].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        steps += 1
        i += len(kinds)
    if not steps:
        raise SystemExit(f"no complete decode step in {files[0]}")
    shapes = {}
    for nm, n, k in mats:
        shapes.setdefault(nm.split(".")[-1], (n, k))
    out = {}
    for kd, v in durs.items():
        e = {"launches": len(v), "mean_us": round(statistics.fmean(v), 3),
             "median_us": round(statistics.median(v), 3)}
        if kd != "ple":
            n, k = shapes[kd]
            b = weight_bytes(n, k) + 2 * k + 8 if kd == "head" else q4_bytes(n, k)
            gbs = b / (e["mean_us"] * 1e-6) / 1e9
            e.update({"shape": [n, k], "bytes_per_launch": b, "achieved_GBs": round(gbs, 1),
                      "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        out[kd] = e
    return {"kernel_source_hash": kernel_source_hash(), "trace": files[0], "decode_steps": steps,
            "shapes": out}


def heads_once(torch, dev, seed: int) -> dict:
    """The single-vector LM head (softcap + argmax, one launch) once on an
    E2B-shaped [262144, 1536] and once on an E4B-shaped [262144, 2560] matrix,
    eagerly and untimed (for counter runs, which then see each launch once)."""
    import int4_weight_only_block_amd as q4
    import synth

    g = torch.Generator(device=dev)
    g.manual_seed(seed + 13)
    out = {}
    for vocab, k in ((262144, 1536), (262144, 2560)):
        packed = q4.q4_pack(*synth.torch_q4_weights(g, vocab, k, dev))
        x = synth.torch_bf16_normal(g, k, dev)
        ws = torch.zeros(q4.lmhead_workspace_bytes(vocab, k), dtype=torch.uint8, device=dev)
        idx, val = q4.lmhead_softcap_argmax(packed, vocab, k, x, 30.0, ws)
        torch.cuda.synchronize()
        out[f"{vocab}x{k}"] = {"idx": int(idx.item()), "val": float(val.item())}
        del packed
    return {"heads_once": out}


def gemm_shapes_only(torch, dev, spec: str, seed: int) -> dict:
    """q4_gemm_s64 alone on 64 bf16 tokens for each NxK shape in spec: 4
    distinct packed matrices, their 4 launches captured in one HIP graph and
    replayed 5 times between HIP events; us per launch."""
    import int4_weight_only_block_amd as q4
    import synth

    g = torch.Generator(device=dev)
    g.manual_seed(seed + 11)
    out = {}
    for item in spec.split(","):
        n, k = (int(v) for v in item.lower().split("x"))
        mats = [q4.q4_pack(*synth.torch_q4_weights(g, n, k, dev)) for _ in range(4)]
        x = synth.torch_bf16_normal(g, (64, k), dev)
        y = torch.empty((64, n), dtype=torch.float32, device=dev)
        ws = torch.zeros(q4.q4_gemm_workspace_bytes(n, k), dtype=torch.uint8, device=dev)

        def run():
            for m in mats:
                q4.q4_gemm_s64(m, n, k, x, y, ws)

        run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        out[f"{n}x{k}"] = round(e0.elapsed_time(e1) * 1e3 / (5 * len(mats)), 3)
        del graph, mats
    return {"gemm_s64_us_per_launch": out}


def main():
    args = parse()
    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary)))
        return
    if args.counters_summary:
        c = counters_summary(args.counters_summary)
        with open(COUNTERS_FILE, "w") as f:
            json.dump(c, f, indent=1)
            f.write("\n")
        print(json.dumps(c))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path is built and measured on one GPU's share)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "copies": 3}))
        return

    if args.gemm_shapes:
        print(json.dumps(gemm_shapes_only(torch, dev, args.gemm_shapes, args.seed)))
        return
    if args.heads_once:
        print(json.dumps(heads_once(torch, dev, args.seed)))
        return

    wl = Workload(dev, args.seed)
    if args.verify_pass:
        print(json.dumps(probe_verify_m4(torch, wl, args.seed, once=True)))
        return
    graph = capture_step(torch, wl)
    for _ in range(max(args.warmup, 0)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    wbytes = wl.weight_bytes()
    value = wbytes / (ms_step * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16*f16->f32",
        "data": "synthetic (seeded on-device draws: codes U[-8,7], fp16 scales U[1e-3,2e-2], bf16 N(0,1))",
        "config": {
            "workload": "e4b_decode_step_s1",
            "layers": 42, "hidden": 2560, "intermediate": 10240, "q_heads": 8, "kv_heads": 2,
            "head_dim": 256, "vocab": 262144, "ple_dim": 10752, "softcap": 30.0,
            "weight_bytes_per_step": wbytes, "launches_per_step": 1 + 168 + 2,
            "graph": "hip graph, one stream",
        },
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "timed_wall_s": round(wall, 3),
    }

    if not args.no_probe:
        per_kind = probe_kernels(torch, wl)
        shapes = {name.split(".")[-1] if "." in name else name: (n, k) for name, n, k in wl.mats}
        step_kinds = [kk for kk, _ in wl.launches()]
        kernels = {}
        for kind, mean_ms in per_kind.items():
            if kind == "ple":
                b = 4 + 4 + wl.ple_dim * (1 + 4)
                desc = f"ple_gather_kernel, 1 id, table [{wl.vocab}, {wl.ple_dim}] int8"
            elif kind == "gate_up_gelu":
                n, k = shapes["gate_up"]
                b = weight_bytes(n, k) + 2 * k + 2 * (n // 2)
                desc = f"q4_rows_kernel GELU mode [{n}, {k}] (fused gate/up GELU, not in the step)"
            elif kind == "head":
                n, k = wl.head_nk
                # weights and x; the last workgroup reduces the partials and
                # the call returns (index, value)
                b = weight_bytes(n, k) + 2 * k + 8
                desc = f"q4_rows_kernel head mode [{n}, {k}] (both passes, one launch)"
            else:
                n, k = shapes[kind]
                b = q4_bytes(n, k)
                desc = f"q4_rows_kernel GEMV [{n}, {k}]"
            per_step = step_kinds.count(kind)
            ach = b / (mean_ms * 1e-3) / 1e9
            kernels[kind] = {
                "kernel": desc,
                "launches_per_step": per_step,
                "avg_launch_us": round(mean_ms * 1e3, 3),
                "ms_per_step": round(mean_ms * per_step, 4),
                "bytes_per_launch": b,
                "achieved_GBs": round(ach, 1),
                "frac_of_hbm_peak": round(ach / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(kind),
            }
        gelu = kernels.pop("gate_up_gelu", None)
        if gelu:
            gelu.pop("ms_per_step", None)
            result["fused_gate_up_gelu"] = gelu
        result["kernels"] = kernels
        result["kernel_timing"] = ("per launch shape: the step's launches of that shape (42 distinct matrices; "
                                   "the head over 3 distinct copies), repeated to >= 24, captured in one HIP "
                                   "graph and replayed between HIP events on the launch stream")
        dominant = max((kk for kk in kernels if kk != "ple"), key=lambda kk: kernels[kk]["ms_per_step"])
        kd = kernels[dominant]
        result["roofline"] = {
            "kernel": f"{dominant}: {kd['kernel']}",
            "bound": "hbm",
            "achieved": kd["achieved_GBs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": kd["frac_of_hbm_peak"],
            "traffic": kd["traffic"],
            "avg_launch_us": kd["avg_launch_us"],
            "bytes_per_launch": kd["bytes_per_launch"],
        }
        result["roofline_by_shape"] = {kk: {"achieved": v["achieved_GBs"], "frac": v["frac_of_hbm_peak"],
                                            "avg_launch_us": v["avg_launch_us"], "ms_per_step": v["ms_per_step"]}
                                       for kk, v in kernels.items()}
        kh = kernels["head"]
        result["roofline_lmhead"] = {
            "bound": "hbm", "achieved": kh["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kh["frac_of_hbm_peak"], "traffic": kh["traffic"],
            "avg_launch_us": kh["avg_launch_us"], "bytes_per_launch": kh["bytes_per_launch"],
        }
        result["kernel_time_sum_ms"] = round(sum(v["ms_per_step"] for v in kernels.values()), 4)
        result["launch_gap_ms_per_step"] = round(ms_step - result["kernel_time_sum_ms"], 4)
        result["decode_step_chain"] = probe_chain(torch, wl, graph)

    if not args.no_prefill:
        g2 = torch.Generator(device=dev)
        g2.manual_seed(args.seed + 1)
        wl.prefill_setup(g2)
        wl.p_ids = torch.randint(0, wl.vocab, (64,), dtype=torch.int32, device=dev, generator=g2)
        wl.p_ple_out = torch.empty((64, wl.ple_dim), dtype=torch.float32, device=dev)
        wl.prefill_step()
        torch.cuda.synchronize()
        pgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pgraph):
            wl.prefill_step()
        for _ in range(3):
            pgraph.replay()
        torch.cuda.synchronize()
        reps = max(5, args.steps // 10)
        e0.record()
        for _ in range(reps):
            pgraph.replay()
        e1.record()
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / reps
        flops = wl.prefill_flops()
        result["prefill_s64"] = {
            "workload": "e4b_prefill_step_s64",
            "ms_per_step": round(pms, 4),
            "tokens_per_s": round(64 / (pms * 1e-3), 1),
            "weight_GBs": round(wbytes / (pms * 1e-3) / 1e9, 1),
            "TFLOPs": round(flops / (pms * 1e-3) / 1e12, 1),
            "flops_per_step": flops,
            "steps": reps,
            "roofline": {"bound": "hbm", "floor_ms_at_8TBs": round(wbytes / 8e12 * 1e3, 4),
                         "mfma_fp16_floor_ms": round(flops / 2.5e15 * 1e3, 4)},
        }
        del pgraph
        if not args.no_probe:
            result["prefill_s64"]["head_all_64_rows"] = probe_head_s64(torch, wl)

    if not args.no_probe:
        result["verify_m4"] = probe_verify_m4(torch, wl, args.seed)
        result["quantize_e4b_gate_up"] = probe_quantize(torch, dev, args.seed)
        result["pack_e4b_gate_up"] = probe_pack(torch, dev, args.seed)
        result["rowq_int2_kprobe"] = probe_rowq(torch, dev, args.seed)
        result["configs"] = probe_configs(torch, dev, wl, args.seed)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        result["cpu_oracle_configs"] = cpu_oracle_configs()

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
