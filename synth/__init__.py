"""Seeded synthetic inputs for the q4_0 decode hot path.

This module is shared by the oracle side and the GPU side. It draws random
numbers and stores them in the interchange formats; it holds none of the
method's arithmetic (no dequantisation, no dot product, no softcap, no gather).

Interchange formats (what both sides receive):

* q4_0 weights: ``codes`` int8 ``[N, K]`` with values in ``[-8, 7]`` and
  ``scales`` uint16 ``[N, K/32]`` holding IEEE fp16 bit patterns, one scale per
  32 consecutive weights along K. This is the per-block-32 symmetric int4 grid
  described on the Gemma-4-E2B Core AI model card (Provenance table, "Weight
  format") and the model-zoo E2B card ("QAT weights" section).
* activations: uint16 arrays of bf16 bit patterns (the upper half of an fp32),
  obtained from fp32 normal draws by round-to-nearest-even.
* PLE table: int8 ``[V, D]`` uniform in ``[-127, 127]``, fp32 row scales ``[V]``
  and int32 token ids, as in the sidecar listing of the Core AI model card
  ("The PLE gather-table sidecar" section).

Workload shapes (``SHAPES``) restate the E2B / E4B dimensions the pages give:
vocabulary 262,144, E2B hidden 1536 with per-layer-embedding width
35 x 256 = 8960, E4B hidden 2560 with 42 layers, intermediate 10,240 and a
per-layer-embedding width 42 x 256 = 10,752 (model-zoo E4B card, architecture
paragraph).
"""
from __future__ import annotations

import numpy as np

VOCAB = 262_144

SHAPES = {
    # one q4_0 GEMV, batch 1
    "gemv_1536": dict(n=1536, k=1536),
    # E2B-shaped FFN pair: gate+up fused by rows [gate; up], then down
    "ffn_e2b": dict(gate_up=(2 * 6144, 1536), down=(1536, 6144), inter=6144),
    # LM head, E2B-shaped
    "head_e2b": dict(vocab=VOCAB, k=1536, n_vectors=100),
    # per-layer-embedding tables
    "ple_e2b": dict(vocab=VOCAB, dim=35 * 256),
    "ple_e4b": dict(vocab=VOCAB, dim=42 * 256),
    # E4B-shaped linear stack: per layer QKV fused [8*256 + 2*256 + 2*256, 2560],
    # O [2560, 8*256], gate+up fused [2*10240, 2560], down [2560, 10240];
    # head [262144, 2560]
    "stack_e4b": dict(
        layers=42,
        hidden=2560,
        inter=10240,
        q_heads=8,
        kv_heads=2,
        head_dim=256,
        vocab=VOCAB,
    ),
}


def stack_e4b_matrices():
    """(name, n, k) of every q4_0 matrix in one E4B-shaped decode step, in
    execution order: per layer QKV, O, gate+up, down; then the head."""
    s = SHAPES["stack_e4b"]
    h, hd = s["hidden"], s["head_dim"]
    qkv_rows = (s["q_heads"] + 2 * s["kv_heads"]) * hd
    out = []
    for layer in range(s["layers"]):
        out.append((f"l{layer}.qkv", qkv_rows, h))
        out.append((f"l{layer}.o", h, s["q_heads"] * hd))
        out.append((f"l{layer}.gate_up", 2 * s["inter"], h))
        out.append((f"l{layer}.down", h, s["inter"]))
    out.append(("head", s["vocab"], h))
    return out


def rng_for(seed: int, *key: int) -> np.random.Generator:
    """PCG64 generator; ``key`` spawns an independent child stream per
    (layer, matrix) so large workloads can be drawn in any order."""
    ss = np.random.SeedSequence(seed)
    for k in key:
        ss = ss.spawn(k + 1)[k]
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (input formatting)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def q4_weights(rng: np.random.Generator, n: int, k: int,
               scale_lo: float = 1e-3, scale_hi: float = 2e-2):
    """codes int8 [n, k] uniform in [-8, 7]; fp16 scale bits uint16 [n, k/32]
    uniform in [scale_lo, scale_hi] before fp16 rounding."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    scales = rng.uniform(scale_lo, scale_hi, size=(n, k // 32)).astype(np.float16)
    return codes, scales.view(np.uint16)


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """bf16 bit patterns of standard-normal fp32 draws."""
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def ple_inputs(rng: np.random.Generator, vocab: int, dim: int, n_ids: int,
               scale_lo: float = 1e-3, scale_hi: float = 1e-2):
    """int8 table [vocab, dim] uniform in [-127, 127], fp32 row scales [vocab]
    and int32 ids [n_ids] uniform in [0, vocab)."""
    table = rng.integers(-127, 128, size=(vocab, dim), dtype=np.int8)
    scale = rng.uniform(scale_lo, scale_hi, size=vocab).astype(np.float32)
    ids = rng.integers(0, vocab, size=n_ids, dtype=np.int32)
    return table, scale, ids


def ple_ids(rng: np.random.Generator, vocab: int, n_ids: int) -> np.ndarray:
    return rng.integers(0, vocab, size=n_ids, dtype=np.int32)


# ---------------------------------------------------------------------------
# Device-side drawing for the multi-gigabyte decode-step workload. Uses torch's
# seeded Philox generator on the GPU; values follow the same distributions as
# the numpy draws above. Only called by bench.py and GPU tests.
# ---------------------------------------------------------------------------
def torch_q4_weights(gen, n: int, k: int, device,
                     scale_lo: float = 1e-3, scale_hi: float = 2e-2):
    import torch

    codes = torch.randint(-8, 8, (n, k), dtype=torch.int8, device=device,
                          generator=gen)
    scales = torch.empty((n, k // 32), dtype=torch.float32, device=device)
    scales.uniform_(scale_lo, scale_hi, generator=gen)
    return codes, scales.to(torch.float16).view(torch.int16)


def torch_bf16_normal(gen, shape, device):
    import torch

    x = torch.randn(shape, dtype=torch.float32, device=device, generator=gen)
    return x.to(torch.bfloat16).view(torch.int16)
