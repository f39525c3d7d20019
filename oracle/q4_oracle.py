"""CPU fp64 oracle for the q4_0 decode hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module;
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with the HIP library: it reads the
interchange formats produced by ``synth`` (int8 codes, fp16 / bf16 bit
patterns, int8 tables, int32 ids) and evaluates the plain definitions in fp64.

Sources (titles of the pages, with the section each function follows):

* [CARD] "visible-cx/gemma-4-E2B-CoreAI" model card: Provenance table (weight
  format: int4 per-block-32, the ggml q4_0 grid), the PLE gather-table sidecar
  section (int8 table, fp32 per-row scale, multiplier 16.0 = sqrt(256)) and the
  engine contract (int32 ids, int8 table, fp32 scale).
* [E2B] "Gemma 4 E2B (text decoder) - Core AI" model-zoo card: signature
  features (final logit softcap tanh(z/30)*30), "QAT weights" section (q4_0 is
  per-block-32 absmax symmetric int4), "What it took" (fused head with an
  in-kernel argmax returning (value, index)).
* [E4B] "Gemma 4 E4B" model-zoo card: architecture paragraph (softcap 30,
  vocabulary 262,144).
* [MIX] "Gemma-4 E2B mobile mixed-bit QAT weights" knowledge page: P6 section
  (official packing stores the UNSIGNED code minus the midpoint, -8 for int4)
  and the receiving-end design (q_u = q_s + 8; the fused gate/up kernel uses a
  precise fp32 tanh GELU).

Every function is pinned by ``tests/test_oracle_pins.py`` to values that do
not come from this file: hand-derived worked examples, exact rational
arithmetic, closed forms, invariants and brute force. No function here is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

# Rows of the weight matrix processed per numpy call; bounds peak memory of the
# fp64 dequantised slab (ROW_CHUNK * K * 8 bytes).
ROW_CHUNK = 8192


# ---------------------------------------------------------------- decoding --
def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> fp64, exactly (bf16 is the upper half of fp32)."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits) -> np.ndarray:
    """fp16 bit patterns -> fp64, exactly."""
    return np.ascontiguousarray(bits).view(np.uint16).view(np.float16).astype(np.float64)


def codes_from_nibbles(nibbles) -> np.ndarray:
    """Stored unsigned nibble -> signed code: c = n - 8, so c is in [-8, 7].

    [MIX] P6 section: the official int4 packing is the unsigned code minus the
    midpoint 8; the receiving-end design maps q_u = q_s + 8.
    """
    n = np.asarray(nibbles).astype(np.int16)
    if ((n < 0) | (n > 15)).any():
        raise ValueError("nibbles must be in [0, 15]")
    return (n - 8).astype(np.int8)


def nibbles_from_codes(codes) -> np.ndarray:
    """Signed code -> stored unsigned nibble n = c + 8 ([MIX] P6 section)."""
    c = np.asarray(codes).astype(np.int16)
    if ((c < -8) | (c > 7)).any():
        raise ValueError("codes must be in [-8, 7]")
    return (c + 8).astype(np.uint8)


# ----------------------------------------------------------------- dequant --
def dequant(codes, scale_bits) -> np.ndarray:
    """q4_0 dequantisation in fp64: w[n, k] = c[n, k] * d[n, k // 32].

    [CARD] Provenance table: int4 weights, one scale per block of 32 along the
    input dimension; [E2B] "QAT weights": per-block-32 absmax symmetric int4.
    Exact in fp64 (a 4-bit integer times an 11-bit fp16 significand).
    """
    codes = np.asarray(codes)
    n, k = codes.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    d = f16_bits_to_f64(scale_bits).reshape(n, k // 32)
    return codes.astype(np.float64) * np.repeat(d, 32, axis=1)


# ---------------------------------------------- per-row INT4 / INT2 GEMV --
def rowq_unpack(w_bytes, n: int, k: int, bits: int) -> np.ndarray:
    """Dense-packed per-row symmetric codes -> int8 [n, k] ([MIX] decode
    recipe: per-channel symmetric linear, all zero points 0, bytes = elements *
    bits / 8; packing convention: INT2 holds 4 codes per byte with the first
    code in bits [1:0], two's complement in [-2, 1]; INT4 is the same with
    nibbles, low nibble first, in [-8, 7]; the INT8 PLE gate / projection
    matrices are plain signed bytes, [-128, 127])."""
    if bits == 8:
        return np.ascontiguousarray(w_bytes).view(np.int8).reshape(n, k).copy()
    if bits not in (2, 4):
        raise ValueError("bits must be 2, 4 or 8")
    per = 8 // bits
    b = np.ascontiguousarray(w_bytes).view(np.uint8).reshape(n, k // per)
    shifts = np.arange(per, dtype=np.uint8) * bits
    u = (b[..., None] >> shifts) & ((1 << bits) - 1)         # [n, k/per, per], first code lowest
    c = u.astype(np.int16) - ((u >> (bits - 1)) << bits)     # two's complement
    return c.reshape(n, k).astype(np.int8)


def rowq_pack(codes, bits: int) -> np.ndarray:
    """int8 codes [n, k] in range -> the dense bytes rowq_unpack reads."""
    c = np.asarray(codes).astype(np.int16)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    if ((c < lo) | (c > hi)).any():
        raise ValueError("codes out of range")
    if bits == 8:
        return c.astype(np.int8).view(np.uint8)
    per = 8 // bits
    n, k = c.shape
    u = (c & ((1 << bits) - 1)).astype(np.uint8).reshape(n, k // per, per)
    out = np.zeros((n, k // per), dtype=np.uint8)
    for i in range(per):
        out |= (u[..., i] << (i * bits)).astype(np.uint8)
    return out


def rowq_gemv(w_bytes, row_scale, bits: int, x_bits):
    """y[r] = scale[r] * sum_k c[r, k] x[k] in fp64 ([MIX] receiving-end
    design: per-row scale, the raw integer-weighted sum is scaled once per
    row), plus A[r] = |scale[r]| * sum_k |c[r, k] x[k]| for the GEMV bar."""
    x = bf16_bits_to_f64(x_bits)
    k = x.size
    sc = np.asarray(row_scale, dtype=np.float32).astype(np.float64)
    n = sc.size
    w = np.ascontiguousarray(w_bytes).view(np.uint8).reshape(n, k * bits // 8)
    y = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    ax = np.abs(x)
    for r0 in range(0, n, ROW_CHUNK):
        c = rowq_unpack(w[r0:r0 + ROW_CHUNK], min(ROW_CHUNK, n - r0), k, bits).astype(np.float64)
        y[r0:r0 + len(c)] = sc[r0:r0 + len(c)] * (c @ x)
        a[r0:r0 + len(c)] = np.abs(sc[r0:r0 + len(c)]) * (np.abs(c) @ ax)
    return y, a


def rowq_lmhead(w_bytes, row_scale, bits: int, x_bits, cap: float = 30.0):
    """The head on the per-row formats ([MIX] mixed-bit map: the INT2
    [262144, 1536] input embedding is tied with the head): logits from
    rowq_gemv, the softcap and the first argmax of the capped logits, as in
    lmhead. Returns dict(idx, val, margin, a_idx, z, capped)."""
    z, a = rowq_gemv(w_bytes, row_scale, bits, x_bits)
    c = softcap(z, cap)
    i = first_argmax(c)
    return dict(idx=i, val=float(c[i]), margin=top2_margin(c), a_idx=float(a[i]), z=z, capped=c)


# --------------------------------------------------------------- quantiser --
QUANT_Q4_0 = 0     # q4_0 grid: d = m / -8, m the block's largest-magnitude value
QUANT_ABSMAX7 = 1  # symmetric: d = max|x| / 7, codes in [-7, 7]


def q4_quantize(x_bits, rule: int = QUANT_Q4_0):
    """bf16 weights [n, k] -> q4_0 codes (int8 [n, k]) and fp16 scale bits
    (uint16 [n, k/32]), plus a per-block flag for blocks the format cannot
    hold (a NaN input, or a scale beyond the fp16 range).

    [E2B] "QAT weights": q4_0 is per-block-32 absmax symmetric int4 (the ggml
    q4_0 grid); the plain absmax variant (--lin-sym) is the literal grid.
    [CARD] Provenance: the int4 rounding happens at export. The pages give no
    formula, so this is the plain reading, every step in fp32:
      m   = the block value of largest magnitude (lowest index on ties),
      d   = m / -8 (rule QUANT_Q4_0; exact) or max|x| / 7 (QUANT_ABSMAX7,
            correctly rounded), stored as fp16 (round to nearest even),
      c_j = clamp(rint(x_j / d16), lo, 7), the quotient a correctly rounded
            fp32 division, rint to nearest even, lo = -8 (q4_0) or -7;
            c_j = 0 when d16 is zero or not finite; a zero scale is +0.
    With the q4_0 rule the largest-magnitude value gets the code -8 exactly
    unless its fp16 scale rounds away from m / -8.
    """
    x = (np.ascontiguousarray(x_bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    n, k = x.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(n, k // 32, 32)
    ax = np.abs(xb)
    nan_blk = np.isnan(xb).any(axis=2)
    ax = np.where(np.isnan(ax), np.float32(-1.0), ax)
    jmax = np.argmax(ax, axis=2)  # first index of the largest magnitude
    m = np.take_along_axis(xb, jmax[..., None], axis=2)[..., 0]
    if rule == QUANT_Q4_0:
        d = m / np.float32(-8.0)
        lo = -8
    elif rule == QUANT_ABSMAX7:
        d = np.abs(m) / np.float32(7.0)
        lo = -7
    else:
        raise ValueError("unknown rule")
    with np.errstate(over="ignore"):
        d16 = d.astype(np.float16)
    d16 = np.where(d16 == 0, np.float16(0.0), d16)  # a zero block stores +0, not -0
    d32 = d16.astype(np.float32)
    usable = np.isfinite(d32) & (d32 != 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(xb / np.where(usable, d32, np.float32(1.0))[..., None])
    q = np.where(usable[..., None] & ~np.isnan(q), np.clip(q, lo, 7), 0).astype(np.int8)
    flags = nan_blk | ~np.isfinite(d32)
    return q.reshape(n, k), d16.view(np.uint16), flags


# -------------------------------------------------------------------- GEMV --
def gemv(codes, scale_bits, x_bits):
    """y[n] = sum_k w[n, k] * x[k] in fp64, plus A[n] = sum_k |w[n, k] x[k]|.

    A is the magnitude sum the tolerance |y_gpu - y| <= 1e-4 * A + 1e-6 is
    measured against. Row-chunked so large heads fit in memory.
    """
    codes = np.asarray(codes)
    n, k = codes.shape
    x = bf16_bits_to_f64(x_bits).reshape(k)
    ax = np.abs(x)
    y = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, ROW_CHUNK):
        w = dequant(codes[r0:r0 + ROW_CHUNK], np.asarray(scale_bits)[r0:r0 + ROW_CHUNK])
        y[r0:r0 + len(w)] = w @ x
        a[r0:r0 + len(w)] = np.abs(w) @ ax
    return y, a


def gemm(codes, scale_bits, x_bits):
    """Y[s, n] = sum_k w[n, k] * X[s, k] in fp64 (X rows are tokens of one
    prefill chunk, [CARD] "prefill (S=64 chunked prefill)"), plus the
    magnitude sums A[s, n] = sum_k |w[n, k] X[s, k]|."""
    codes = np.asarray(codes)
    n, k = codes.shape
    xs = bf16_bits_to_f64(x_bits).reshape(-1, k)
    s = xs.shape[0]
    axs = np.abs(xs)
    y = np.empty((s, n), dtype=np.float64)
    a = np.empty((s, n), dtype=np.float64)
    for r0 in range(0, n, ROW_CHUNK):
        w = dequant(codes[r0:r0 + ROW_CHUNK], np.asarray(scale_bits)[r0:r0 + ROW_CHUNK])
        y[:, r0:r0 + len(w)] = xs @ w.T
        a[:, r0:r0 + len(w)] = axs @ np.abs(w).T
    return y, a


# ----------------------------------------------------------------- LM head --
def softcap(z, cap: float = 30.0):
    """Final logit softcap cap * tanh(z / cap) in fp64 ([E2B] signature
    features: tanh(z/30)*30; [E4B] softcap 30). cap <= 0 disables it."""
    z = np.asarray(z, dtype=np.float64)
    if cap <= 0:
        return z.copy()
    return cap * np.tanh(z / cap)


def first_argmax(v) -> int:
    """Index of the maximum; among equal maxima the lowest index wins."""
    v = np.asarray(v)
    return int(np.argmax(v))


def top2_margin(v) -> float:
    """Largest value minus the largest value at any other index."""
    v = np.asarray(v, dtype=np.float64)
    if v.size < 2:
        return float("inf")
    i = int(np.argmax(v))
    rest = np.delete(v, i)
    return float(v[i] - rest.max())


def lmhead(codes, scale_bits, x_bits, cap: float = 30.0):
    """Head GEMV, softcap, then argmax over the capped logits ([E2B] "What it
    took": fused head with a two-level argmax that returns (value, index);
    signature features: softcap).

    Returns dict(idx, val, margin, a_idx, z, capped) where ``margin`` is the
    top-2 margin of the capped logits and ``a_idx`` the magnitude sum of the
    winning row (for the value tolerance).
    """
    z, a = gemv(codes, scale_bits, x_bits)
    c = softcap(z, cap)
    i = first_argmax(c)
    return dict(idx=i, val=float(c[i]), margin=top2_margin(c), a_idx=float(a[i]),
                z=z, capped=c)


# -------------------------------------------------------------- PLE gather --
def ple_gather(table, row_scale, ids, mult: float = 16.0):
    """Per-Layer-Embedding gather: out[t, j] = RN_fp32(q[id_t, j] * s[id_t] * mult).

    [CARD] sidecar section: int8 table [V, L*ld], fp32 per-row scale [V],
    multiplier embed_scale_pl 16.0. The product of the int8 code, the fp32
    scale and the fp32 multiplier is formed exactly in 80-bit extended
    precision (at most 8 + 24 + 24 = 56 significant bits) and rounded once to
    fp32. Ids outside [0, V) give a zero row and set the returned error flag.
    Returns (out float32 [T, D], err int).
    """
    table = np.asarray(table)
    v, dim = table.shape
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    out = np.zeros((ids.size, dim), dtype=np.float32)
    ok = (ids >= 0) & (ids < v)
    err = int((~ok).any())
    if ok.any():
        rows = ids[ok]
        q = table[rows].astype(np.longdouble)
        s = np.asarray(row_scale, dtype=np.float32)[rows].astype(np.longdouble)
        m = np.longdouble(np.float32(mult))
        out[ok] = (q * s[:, None] * m).astype(np.float32)
    return out, err


def rowq_gather(w_bytes, scales, bits: int, group: int, ids, mult: float = 16.0):
    """Row gather on the dense per-row formats: out[t, j] = RN_fp32(c[id_t, j]
    * s[id_t, j // group] * mult). [MIX] bundle table and mixed-bit map: the
    input embedding (tied with the head) is INT2 [262144, 1536] with one scale
    per row, and the PLE table stores each row as 35 layer-major 128-byte INT4
    blocks with one scale per (row, layer); the codes follow rowq_unpack.
    ``scales`` is fp32 [V, dim / group]. The product of a code, an fp32 scale
    and the fp32 multiplier is exact in 80-bit extended precision (at most
    4 + 24 + 24 significant bits) and is rounded once to fp32. Ids outside
    [0, V) give a zero row and set the returned error flag. Returns
    (out float32 [T, dim], err int)."""
    sc = np.asarray(scales, dtype=np.float32)
    v, ng = sc.shape
    dim = ng * group
    w = np.ascontiguousarray(w_bytes).view(np.uint8).reshape(v, dim * bits // 8)
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    out = np.zeros((ids.size, dim), dtype=np.float32)
    ok = (ids >= 0) & (ids < v)
    err = int((~ok).any())
    if ok.any():
        rows = ids[ok]
        c = rowq_unpack(w[rows], rows.size, dim, bits).astype(np.longdouble)
        s = np.repeat(sc[rows].astype(np.longdouble), group, axis=1)
        m = np.longdouble(np.float32(mult))
        out[ok] = (c * s * m).astype(np.float32)
    return out, err


# --------------------------------------------------------- FFN host glue --
def gelu_tanh_f32(g):
    """tanh-approximation GELU evaluated in fp32 ([MIX] fused gate/up kernel:
    precise fp32 tanh GELU in the epilogue):
    0.5 * g * (1 + tanh(sqrt(2/pi) * (g + 0.044715 * g^3)))."""
    g = np.asarray(g, dtype=np.float32)
    k0 = np.float32(np.sqrt(2.0 / np.pi))
    k1 = np.float32(0.044715)
    inner = k0 * (g + k1 * g * g * g)
    return (np.float32(0.5) * g * (np.float32(1.0) + np.tanh(inner))).astype(np.float32)


def ffn_down_input_bits(g, u):
    """Host step between the fused gate+up GEMV and the down GEMV:
    a = gelu_tanh(g) * u in fp32, rounded to bf16 (torch's round to nearest
    even). Returns uint16 bf16 bit patterns."""
    import torch

    a = gelu_tanh_f32(np.asarray(g, dtype=np.float32)) * np.asarray(u, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def gelu_tanh_f64(g):
    """tanh-form GELU in fp64: 0.5 * g * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3)))."""
    g = np.asarray(g, dtype=np.float64)
    return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))


# Bound on |d gelu_tanh / dg| over the reals (the maximum, about 1.129, sits
# near g = 1.5; the minimum, about -0.17, near g = -1.5); checked on a grid
# in the pins.
GELU_SLOPE_MAX = 1.2


def gelu_mul(codes, scale_bits, x_bits):
    """Fused gate/up with the GELU epilogue ([MIX] fused gate/up kernels:
    one pass over the concatenated [gate; up] rows, fp32 tanh GELU in the
    epilogue). With h = n / 2: g = W[:h] x, u = W[h:] x (exact, fp64) and
    a = gelu_tanh(g) * u in fp64. Returns (a, g, u, A_g, A_u), where A_* are
    the magnitude sums of the two GEMVs."""
    codes = np.asarray(codes)
    n = codes.shape[0]
    if n % 2:
        raise ValueError("gelu_mul needs an even number of rows ([gate; up])")
    y, a_mag = gemv(codes, scale_bits, x_bits)
    h = n // 2
    g, u = y[:h], y[h:]
    return gelu_tanh_f64(g) * u, g, u, a_mag[:h], a_mag[h:]


def rowq_gelu_mul(w_bytes, row_scale, bits: int, x_bits):
    """gelu_mul on the per-row INT4 / INT2 formats ([MIX] fused gate/up
    kernels for the int2 / int4 symmetric layouts): the n rows are [gate; up],
    g = rowq_gemv of rows 0 .. h-1, u = rowq_gemv of rows h .. n-1 (each with
    its own row scale), a = gelu_tanh(g) * u in fp64. Returns (a, g, u, A_g,
    A_u) like gelu_mul."""
    y, a_mag = rowq_gemv(w_bytes, row_scale, bits, x_bits)
    n = y.size
    if n % 2:
        raise ValueError("rowq_gelu_mul needs an even number of rows ([gate; up])")
    h = n // 2
    g, u = y[:h], y[h:]
    return gelu_tanh_f64(g) * u, g, u, a_mag[:h], a_mag[h:]


def gelu_mul_tolerance(g, u, a_g, a_u):
    """Per-output bound for a bf16 result of gelu_mul computed from fp32
    GEMV sums. Each sum is within t = 1e-4 * A + 1e-6 of the exact value
    (the GEMV bar); the GELU's slope is at most GELU_SLOPE_MAX; fp32
    evaluation of the GELU adds at most 1e-6 * (|g| + 1); the fp32 product
    and the final rounding to bf16 add at most 2^-8 relative (half a bf16
    ulp) plus 2^-23. Returns the bound on |a_gpu - a_exact|."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    tg = gemv_tolerance(a_g)
    tu = gemv_tolerance(a_u)
    gel = np.abs(gelu_tanh_f64(g))
    e = np.abs(u) * (GELU_SLOPE_MAX * tg + 1e-6 * (np.abs(g) + 1.0)) + (gel + GELU_SLOPE_MAX * tg) * tu
    a = gel * np.abs(u)
    return (2.0 ** -8 + 2.0 ** -23) * (a + e) + e + 1e-30


# ------------------------------------------------------------- tolerances --
def gemv_tolerance(a):
    """Per-output tolerance for fp32-accumulated GEMV results:
    1e-4 * sum_k |w x| + 1e-6."""
    return 1e-4 * np.asarray(a, dtype=np.float64) + 1e-6
