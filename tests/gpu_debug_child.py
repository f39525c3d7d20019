"""Child process of test_gpu_debug_checks.py (run with Q4DEC_LIB pointing at
libq4dec_debug.so): calls every kernel family of the debug build over the
model shapes and ragged ones, then reports the launch-contract words as one
JSON line. Not collected by pytest (no test_ prefix)."""
import json
import sys

import numpy as np
import torch

import int4_weight_only_block_amd as q4
import oracle
import synth

dev = torch.device("cuda:0")
out = {"lib": q4.LIB_PATH}
out["start"] = list(q4.debug_status())
rng = synth.rng_for(31)
gen = torch.Generator(device=dev)
gen.manual_seed(31)


def bf(*shape):
    return synth.torch_bf16_normal(gen, shape, dev)


def packed(n, k):
    codes = torch.randint(-8, 8, (n, k), dtype=torch.int8, device=dev, generator=gen)
    sc = (torch.rand((n, k // 32), device=dev, generator=gen) * 0.02 + 1e-3).to(torch.float16).view(torch.int16)
    return q4.q4_pack(codes, sc)


print("case gemv", flush=True)
for n, k in [(1536, 1536), (3072, 2560), (2560, 2048), (20480, 2560), (2560, 10240), (300, 2560), (77, 10240),
             (64, 32), (1000, 1536), (6144, 16384)]:
    q4.q4_gemv(packed(n, k), n, k, bf(k))
for n, k in [(12288, 1536), (20480, 2560), (200, 96)]:
    q4.q4_gemv_gelu_mul(packed(n, k), n, k, bf(k))
print("case heads", flush=True)
for v, k in [(65536, 1536), (262144, 2560), (1000, 96)]:
    p = packed(v, k)
    q4.lmhead_softcap_argmax(p, v, k, bf(k), 30.0, torch.zeros(q4.lmhead_workspace_bytes(v, k), dtype=torch.uint8,
                                                                 device=dev))
    q4.lmhead_softcap_argmax_multi(p, v, k, bf(4, k))
    q4.lmhead_softcap_argmax_s64(p, v, k, bf(64, k))
print("case multi", flush=True)
for n, k, m in [(3072, 2560, 4), (2560, 10240, 4), (300, 96, 8), (20480, 2560, 2)]:
    q4.q4_gemv_multi(packed(n, k), n, k, bf(m, k))
print("case gemm", flush=True)
for n, k, t in [(3072, 2560, 64), (2560, 2048, 64), (20480, 2560, 64), (2560, 10240, 64), (300, 2560, 37),
                (16400, 512, 17), (77, 16384, 5), (100, 96, 1)]:
    q4.q4_gemm_s64(packed(n, k), n, k, bf(t, k))
print("case rowq", flush=True)
for bits, n, k in [(2, 1536, 12288), (2, 24576, 1536), (4, 1536, 1536), (4, 2560, 10240), (8, 8960, 1536),
                   (8, 256, 1536), (2, 300, 3008)]:
    w = torch.randint(0, 256, (n, k * bits // 8), dtype=torch.uint8, device=dev, generator=gen)
    s = torch.rand(n, device=dev, generator=gen) * 0.01 + 1e-3
    x = bf(k)
    q4.rowq_gemv(w, s, n, k, bits, x)
    try:  # the fused GELU form takes k up to a per-format limit
        q4.rowq_gemv_gelu_mul(w, s, n, k, bits, x)
    except q4.Q4Error as e:
        if e.code != q4.ERR_UNSUPPORTED:
            raise
    q4.rowq_softcap_argmax(w, s, n, k, bits, x, 30.0)
print("case gather, pack, quantize", flush=True)
table = torch.randint(-128, 128, (4096, 8960), dtype=torch.int8, device=dev, generator=gen)
tsc = torch.rand(4096, device=dev, generator=gen) + 0.5
ids = torch.randint(0, 4096, (64,), dtype=torch.int32, device=dev, generator=gen)
q4.ple_gather(table, tsc, ids, 16.0)
q4.ple_gather(table, tsc, ids[:1], 16.0)
for bits, dim, group in [(2, 1536, 1536), (4, 8960, 256)]:
    w = torch.randint(0, 256, (4096, dim * bits // 8), dtype=torch.uint8, device=dev, generator=gen)
    gs = torch.rand((4096, dim // group), device=dev, generator=gen) + 0.5
    q4.rowq_gather(w, gs, bits, group, ids, 16.0)
q4.q4_quantize(bf(2048, 2560))
q4.q4_quantize(bf(3, 96))
torch.cuda.synchronize()
out["after_calls"] = list(q4.debug_status())

# the debug build computes what the release build does: one GEMV against
# the oracle
n, k = 1000, 1536
codes, sb = synth.q4_weights(rng, n, k)
xh = synth.bf16_normal(rng, k)
pk = q4.q4_pack(torch.from_numpy(codes).to(dev), torch.from_numpy(sb.view(np.int16)).to(dev))
y = q4.q4_gemv(pk, n, k, torch.from_numpy(xh.view(np.int16)).to(dev)).cpu().numpy().astype(np.float64)
yr, a = oracle.gemv(codes, sb, xh)
out["gemv_within_bar"] = bool((np.abs(y - yr) <= oracle.gemv_tolerance(a)).all())

rc_self = q4.debug_selftest()
torch.cuda.synchronize()
out["selftest"] = [rc_self, *q4.debug_status()]
out["cleared"] = list(q4.debug_status())
print(json.dumps(out), flush=True)
sys.exit(0)
