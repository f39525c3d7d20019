"""Python binding of libq4dec (q4_0 decode hot path on MI355X / gfx950).

Argument marshalling only: every function checks that its torch tensors have
the dtype, device and contiguity the C ABI expects, passes raw device pointers
and the current HIP stream to the library, and raises ``Q4Error`` with the
library's error text on a non-zero status. All compute runs in the HIP
kernels of libq4dec.so; there is no other code path. If the shared library has
not been built the import of any call fails loudly.

The C declarations and their meaning are in include/q4dec.h.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# Q4DEC_LIB selects another build of the same library (libq4dec_asan.so, the
# host-sanitizer build, for CPU runs of the host paths)
LIB_PATH = os.environ.get("Q4DEC_LIB") or os.path.join(HERE, "libq4dec.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "q4dec.h")

ABI_VERSION = 2
OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_ALIGN = -3
ERR_WORKSPACE = -4
ERR_UNSUPPORTED = -5
ERR_HIP = -6
MAX_K = 16384
GELU_MAX_K = 6144
QUANT_Q4_0 = 0
QUANT_ABSMAX7 = 1

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_SIGNATURES = {
    "q4dec_abi_version": (ctypes.c_int32, []),
    "q4dec_last_error": (ctypes.c_char_p, []),
    "q4dec_debug_status": (ctypes.c_int, [_c_p]),
    "q4dec_debug_selftest": (ctypes.c_int, [_c_p]),
    "q4_packed_bytes": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "q4_pack": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "q4_quantize": (ctypes.c_int, [_c_p, _c_i64, _c_i64, ctypes.c_int32, _c_p, _c_p, _c_p, _c_p]),
    "q4_gemv": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "q4_gemv_gelu_mul": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "q4_gemv_multi": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p]),
    "rowq_gemv": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, ctypes.c_int32, _c_p, _c_p, _c_p]),
    "rowq_gemv_gelu_mul": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, ctypes.c_int32, _c_p, _c_p, _c_p]),
    "rowq_head_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, ctypes.c_int32]),
    "rowq_softcap_argmax": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, ctypes.c_int32, _c_p, ctypes.c_float, _c_p,
                                           ctypes.c_size_t, _c_p, _c_p, _c_p]),
    "q4_gemm_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "q4_gemm_s64": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "lmhead_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "lmhead_multi_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "lmhead_softcap_argmax_multi": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, ctypes.c_float, _c_p,
                                                   ctypes.c_size_t, _c_p, _c_p, _c_p]),
    "lmhead_softcap_argmax": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, ctypes.c_float, _c_p,
                                             ctypes.c_size_t, _c_p, _c_p, _c_p]),
    "lmhead_softcap_argmax_noalloc": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, ctypes.c_float, _c_p, _c_p,
                                                     _c_p]),
    "lmhead_s64_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "lmhead_softcap_argmax_s64": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, ctypes.c_float, _c_p,
                                                 ctypes.c_size_t, _c_p, _c_p, _c_p]),
    "ple_gather": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_i64, ctypes.c_float, _c_p,
                                  _c_p, _c_p]),
    "rowq_gather": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, ctypes.c_int32, _c_i64, _c_p, _c_i64,
                                   ctypes.c_float, _c_p, _c_p, _c_p]),
}



class ChainLink(ctypes.Structure):
    """q4_chain_link of include/q4dec.h."""
    _fields_ = [("packed", ctypes.c_void_p), ("x", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("mode", ctypes.c_int32), ("wait", ctypes.c_int32)]


_SIGNATURES.update({
    "q4_chain_table_bytes": (ctypes.c_size_t, [_c_i64]),
    "q4_chain_workspace_bytes": (ctypes.c_size_t, []),
    "q4_chain_build": (ctypes.c_int, [_c_p, _c_i64, ctypes.c_float, _c_i64, _c_p, ctypes.c_size_t]),
    "q4_gemv_chain": (ctypes.c_int, [_c_p, _c_p, _c_p, ctypes.c_size_t, _c_p, _c_p, _c_p]),
})

_lib = None


class Q4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libq4dec error {code}: {msg}")
        self.code = code


def lib():
    """Load libq4dec.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libq4dec.so not found at {LIB_PATH}; build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        if h.q4dec_abi_version() != ABI_VERSION:
            raise RuntimeError("libq4dec.so ABI version mismatch; rebuild it")
        _lib = h
    return _lib


def header_functions():
    """Names of the functions include/q4dec.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"defined"})


def _check(rc: int):
    if rc != OK:
        raise Q4Error(rc, lib().q4dec_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


_U16 = (torch.int16, torch.uint16, torch.bfloat16, torch.float16)
_I8 = (torch.int8,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_BYTES = (torch.uint8, torch.int8)


def _check_packed(packed: torch.Tensor, n: int, k: int):
    need = q4_packed_bytes(n, k)
    if need and packed.numel() * packed.element_size() < need:
        raise ValueError(f"packed buffer holds {packed.numel() * packed.element_size()} bytes, "
                         f"[{n}, {k}] needs {need}")


def q4dec_abi_version() -> int:
    return int(lib().q4dec_abi_version())


def q4dec_last_error() -> str:
    return lib().q4dec_last_error().decode()


def debug_status() -> tuple[int, int]:
    """(return code, word): the launch-contract bits set since the last call
    (a debug build of the library), cleared by the call; a release build
    returns ERR_UNSUPPORTED and 0."""
    w = ctypes.c_uint32(0)
    rc = int(lib().q4dec_debug_status(ctypes.byref(w)))
    return rc, int(w.value)


def debug_selftest(stream=None) -> int:
    """Launch the debug build's always-failing check (bit 31)."""
    import torch

    st = stream if stream is not None else torch.cuda.current_stream()
    return int(lib().q4dec_debug_selftest(ctypes.c_void_p(st.cuda_stream)))


def q4_packed_bytes(n: int, k: int) -> int:
    return int(lib().q4_packed_bytes(n, k))


def q4_pack(codes: torch.Tensor, scales: torch.Tensor, packed: torch.Tensor | None = None,
            err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """int8 codes [n, k] in [-8, 7] and fp16 scale bits [n, k/32] -> packed bytes."""
    n, k = codes.shape
    pc = _dev(codes, "codes", _I8)
    ps = _dev(scales, "scales", _U16, n * (k // 32) if k % 32 == 0 else None)
    nbytes = q4_packed_bytes(n, k)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=codes.device)
    pp = _dev(packed, "packed", _BYTES)
    if packed.numel() * packed.element_size() < nbytes:
        raise ValueError("packed buffer too small")
    pe = _dev(err_flag, "err_flag", _I32, 1) if err_flag is not None else None
    _check(lib().q4_pack(pc, ps, n, k, pp, pe, _stream(codes)))
    return packed


def q4_quantize(x: torch.Tensor, rule: int = QUANT_Q4_0, codes: torch.Tensor | None = None,
                scales: torch.Tensor | None = None, err_flag: torch.Tensor | None = None):
    """bf16 [n, k] -> (int8 codes [n, k], fp16 scale bits int16 [n, k/32])."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [n, k]")
    n, k = x.shape
    px = _dev(x, "x", _U16)
    if codes is None:
        codes = torch.empty((n, k), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((n, max(k // 32, 1)), dtype=torch.int16, device=x.device)
    pc = _dev(codes, "codes", _I8, n * k)
    ps = _dev(scales, "scales", _U16, n * max(k // 32, 1))
    pe = _dev(err_flag, "err_flag", _I32, 1) if err_flag is not None else None
    _check(lib().q4_quantize(px, n, k, int(rule), pc, ps, pe, _stream(x)))
    return codes, scales


def q4_gemv(packed: torch.Tensor, n: int, k: int, x: torch.Tensor,
            y: torch.Tensor | None = None) -> torch.Tensor:
    """y[n] fp32 = dequant(W) @ x for bf16 x[k]."""
    pp = _dev(packed, "packed", _BYTES)
    _check_packed(packed, n, k)
    px = _dev(x, "x", _U16, k)
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=x.device)
    py = _dev(y, "y", _F32, n)
    _check(lib().q4_gemv(pp, n, k, px, py, _stream(x)))
    return y


def q4_gemv_multi(packed: torch.Tensor, n: int, k: int, x: torch.Tensor,
                  y: torch.Tensor | None = None) -> torch.Tensor:
    """y fp32 [m, n] = W x[v] for the m <= 8 bf16 rows of x [m, k], the
    weights read once."""
    m = x.shape[0] if x.dim() == 2 else 1
    pp = _dev(packed, "packed", _BYTES)
    _check_packed(packed, n, k)
    px = _dev(x, "x", _U16, m * k)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    py = _dev(y, "y", _F32, m * n)
    _check(lib().q4_gemv_multi(pp, n, k, px, m, py, _stream(x)))
    return y


def rowq_gemv(w: torch.Tensor, row_scale: torch.Tensor, n: int, k: int, bits: int, x: torch.Tensor,
              y: torch.Tensor | None = None) -> torch.Tensor:
    """y fp32 [n] = row_scale * (codes @ x) for dense-packed per-row INT2 /
    INT4 / INT8 codes w [n, k * bits / 8] (uint8)."""
    pw = _dev(w, "w", _BYTES, n * k * bits // 8)
    ps = _dev(row_scale, "row_scale", _F32, n)
    px = _dev(x, "x", _U16, k)
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=x.device)
    py = _dev(y, "y", _F32, n)
    _check(lib().rowq_gemv(pw, ps, n, k, int(bits), px, py, _stream(x)))
    return y


def rowq_gemv_gelu_mul(w: torch.Tensor, row_scale: torch.Tensor, n: int, k: int, bits: int, x: torch.Tensor,
                       a: torch.Tensor | None = None) -> torch.Tensor:
    """a[j] = bf16(gelu_tanh(g_j) * u_j) for per-row INT2 / INT4 / INT8 [gate; up]
    rows (g = rows 0 .. n/2-1, u = rows n/2 .. n-1, each scaled by its own
    row scale); returns bf16 bits (int16)."""
    pw = _dev(w, "w", _BYTES, n * k * bits // 8)
    ps = _dev(row_scale, "row_scale", _F32, n)
    px = _dev(x, "x", _U16, k)
    if a is None:
        a = torch.empty(max(n // 2, 1), dtype=torch.int16, device=x.device)
    pa = _dev(a, "a", _U16, max(n // 2, 1))
    _check(lib().rowq_gemv_gelu_mul(pw, ps, n, k, int(bits), px, pa, _stream(x)))
    return a


def rowq_head_workspace_bytes(vocab: int, k: int, bits: int) -> int:
    return int(lib().rowq_head_workspace_bytes(vocab, k, int(bits)))


def rowq_softcap_argmax(w: torch.Tensor, row_scale: torch.Tensor, vocab: int, k: int, bits: int,
                        x: torch.Tensor, cap: float = 30.0, ws: torch.Tensor | None = None,
                        idx_out: torch.Tensor | None = None, val_out: torch.Tensor | None = None):
    """(idx int32 [1], val fp32 [1]): the softcapped maximum of the per-row
    INT2 / INT4 / INT8 head logits row_scale * (codes @ x), lowest index on
    ties."""
    pw = _dev(w, "w", _BYTES, vocab * k * bits // 8)
    ps = _dev(row_scale, "row_scale", _F32, vocab)
    px = _dev(x, "x", _U16, k)
    if ws is None:
        ws = torch.empty(rowq_head_workspace_bytes(vocab, k, bits), dtype=torch.uint8, device=x.device)
    pws = _dev(ws, "ws", _BYTES)
    if idx_out is None:
        idx_out = torch.empty(1, dtype=torch.int32, device=x.device)
    if val_out is None:
        val_out = torch.empty(1, dtype=torch.float32, device=x.device)
    pi = _dev(idx_out, "idx_out", _I32, 1)
    pv = _dev(val_out, "val_out", _F32, 1)
    _check(lib().rowq_softcap_argmax(pw, ps, vocab, k, int(bits), px, float(cap), pws,
                                     ws.numel() * ws.element_size(), pi, pv, _stream(x)))
    return idx_out, val_out


def q4_gemv_gelu_mul(packed: torch.Tensor, n: int, k: int, x: torch.Tensor,
                     a: torch.Tensor | None = None) -> torch.Tensor:
    """a[j] = bf16(gelu_tanh(g_j) * u_j) for the [gate; up] matrix of n rows
    (g = rows 0 .. n/2-1, u = rows n/2 .. n-1); returns bf16 bits (int16)."""
    pp = _dev(packed, "packed", _BYTES)
    _check_packed(packed, n, k)
    px = _dev(x, "x", _U16, k)
    if a is None:
        a = torch.empty(max(n // 2, 1), dtype=torch.int16, device=x.device)
    pa = _dev(a, "a", _U16, max(n // 2, 1))
    _check(lib().q4_gemv_gelu_mul(pp, n, k, px, pa, _stream(x)))
    return a


def q4_gemm_workspace_bytes(n: int, k: int) -> int:
    return int(lib().q4_gemm_workspace_bytes(n, k))


def q4_gemm_s64(packed: torch.Tensor, n: int, k: int, x: torch.Tensor,
                y: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y[s, n] fp32 = X @ dequant(W)^T for bf16 X[s, k], 1 <= s <= 64."""
    s = x.shape[0] if x.dim() == 2 else 1
    pp = _dev(packed, "packed", _BYTES)
    _check_packed(packed, n, k)
    px = _dev(x, "x", _U16, s * k)
    if y is None:
        y = torch.empty((s, n), dtype=torch.float32, device=x.device)
    py = _dev(y, "y", _F32, s * n)
    need = q4_gemm_workspace_bytes(n, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    pw = _dev(ws, "ws", _BYTES)
    _check(lib().q4_gemm_s64(pp, n, k, px, s, py, pw, ws.numel() * ws.element_size(), _stream(x)))
    return y


def lmhead_workspace_bytes(vocab: int, k: int) -> int:
    return int(lib().lmhead_workspace_bytes(vocab, k))


def lmhead_softcap_argmax(packed: torch.Tensor, vocab: int, k: int, x: torch.Tensor,
                          cap: float = 30.0, ws: torch.Tensor | None = None,
                          idx_out: torch.Tensor | None = None,
                          val_out: torch.Tensor | None = None):
    """(idx int32 [1], val fp32 [1]) of the softcapped head logits' maximum."""
    pp = _dev(packed, "packed", _BYTES)
    _check_packed(packed, vocab, k)
    px = _dev(x, "x", _U16, k)
    need = lmhead_workspace_bytes(vocab, k)
    if ws is None:
        ws = torch.zeros(need, dtype=torch.uint8, device=x.device)  # the arrival counter starts at zero
    pw = _dev(ws, "ws", _BYTES)
    if idx_out is None:
        idx_out = torch.empty(1, dtype=torch.int32, device=x.device)
    if val_out is None:
        val_out = torch.empty(1, dtype=torch.float32, device=x.device)
    pi = _dev(idx_out, "idx_out", _I32, 1)
    pv = _dev(val_out, "val_out", _F32, 1)
    _check(lib().lmhead_softcap_argmax(pp, vocab, k, px, float(cap), pw,
                                       ws.numel() * ws.element_size(), pi, pv, _stream(x)))
    return idx_out, val_out


def lmhead_softcap_argmax_noalloc(packed: torch.Tensor, vocab: int, k: int, x: torch.Tensor,
                                  cap: float = 30.0, idx_out: torch.Tensor | None = None,
                                  val_out: torch.Tensor | None = None):
    """lmhead_softcap_argmax with the library's own partials array (no
    workspace). Calls that overlap on one GPU race."""
    pp = _dev(packed, "packed", _BYTES)
    _check_packed(packed, vocab, k)
    px = _dev(x, "x", _U16, k)
    if idx_out is None:
        idx_out = torch.empty(1, dtype=torch.int32, device=x.device)
    if val_out is None:
        val_out = torch.empty(1, dtype=torch.float32, device=x.device)
    pi = _dev(idx_out, "idx_out", _I32, 1)
    pv = _dev(val_out, "val_out", _F32, 1)
    _check(lib().lmhead_softcap_argmax_noalloc(pp, vocab, k, px, float(cap), pi, pv, _stream(x)))
    return idx_out, val_out


def lmhead_multi_workspace_bytes(vocab: int, k: int, m: int) -> int:
    return int(lib().lmhead_multi_workspace_bytes(vocab, k, m))


def lmhead_softcap_argmax_multi(packed: torch.Tensor, vocab: int, k: int, x: torch.Tensor,
                                cap: float = 30.0, ws: torch.Tensor | None = None,
                                idx_out: torch.Tensor | None = None,
                                val_out: torch.Tensor | None = None):
    """(idx int32 [m], val fp32 [m]): the softcapped head maximum for each of
    the m <= 8 bf16 vectors x [m, k], with the head read once."""
    m = x.shape[0] if x.dim() == 2 else 1
    pp = _dev(packed, "packed", _BYTES)
    _check_packed(packed, vocab, k)
    px = _dev(x, "x", _U16, m * k)
    need = lmhead_multi_workspace_bytes(vocab, k, m)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    pw = _dev(ws, "ws", _BYTES)
    if idx_out is None:
        idx_out = torch.empty(m, dtype=torch.int32, device=x.device)
    if val_out is None:
        val_out = torch.empty(m, dtype=torch.float32, device=x.device)
    pi = _dev(idx_out, "idx_out", _I32, m)
    pv = _dev(val_out, "val_out", _F32, m)
    _check(lib().lmhead_softcap_argmax_multi(pp, vocab, k, px, m, float(cap), pw,
                                             ws.numel() * ws.element_size(), pi, pv, _stream(x)))
    return idx_out, val_out


def lmhead_s64_workspace_bytes(vocab: int, k: int) -> int:
    return int(lib().lmhead_s64_workspace_bytes(vocab, k))


def lmhead_softcap_argmax_s64(packed: torch.Tensor, vocab: int, k: int, x: torch.Tensor,
                              cap: float = 30.0, ws: torch.Tensor | None = None,
                              idx_out: torch.Tensor | None = None,
                              val_out: torch.Tensor | None = None):
    """(idx int32 [s], val fp32 [s]): the softcapped head maximum for each of
    the s <= 64 bf16 token rows x [s, k] of a prefill chunk."""
    n_tok = x.shape[0] if x.dim() == 2 else 1
    pp = _dev(packed, "packed", _BYTES)
    _check_packed(packed, vocab, k)
    px = _dev(x, "x", _U16, n_tok * k)
    need = lmhead_s64_workspace_bytes(vocab, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    pw = _dev(ws, "ws", _BYTES)
    if idx_out is None:
        idx_out = torch.empty(n_tok, dtype=torch.int32, device=x.device)
    if val_out is None:
        val_out = torch.empty(n_tok, dtype=torch.float32, device=x.device)
    pi = _dev(idx_out, "idx_out", _I32, n_tok)
    pv = _dev(val_out, "val_out", _F32, n_tok)
    _check(lib().lmhead_softcap_argmax_s64(pp, vocab, k, px, n_tok, float(cap), pw,
                                           ws.numel() * ws.element_size(), pi, pv, _stream(x)))
    return idx_out, val_out


def ple_gather(table: torch.Tensor, row_scale: torch.Tensor, ids: torch.Tensor,
               mult: float = 16.0, out: torch.Tensor | None = None,
               err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """out[t, :] fp32 = table[ids[t]] * row_scale[ids[t]] * mult, rounded once."""
    vocab, dim = table.shape
    pt = _dev(table, "table", _I8)
    psc = _dev(row_scale, "row_scale", _F32, vocab)
    pi = _dev(ids, "ids", _I32)
    n_ids = ids.numel()
    if out is None:
        out = torch.empty((n_ids, dim), dtype=torch.float32, device=table.device)
    po = _dev(out, "out", _F32, n_ids * dim)
    pe = _dev(err_flag, "err_flag", _I32, 1) if err_flag is not None else None
    _check(lib().ple_gather(pt, psc, vocab, dim, pi, n_ids, float(mult), po, pe, _stream(table)))
    return out


def rowq_gather(w: torch.Tensor, scales: torch.Tensor, bits: int, group: int, ids: torch.Tensor,
                mult: float = 16.0, out: torch.Tensor | None = None,
                err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """out[t, :] fp32 = codes[ids[t]] * scales[ids[t], j // group] * mult,
    rounded once; w holds the dense INT2 / INT4 rows, scales is fp32
    [vocab, dim / group]."""
    vocab, ngroups = scales.shape
    dim = ngroups * group
    pw = _dev(w, "w", _BYTES, vocab * dim * bits // 8)
    ps = _dev(scales, "scales", _F32)
    pi = _dev(ids, "ids", _I32)
    n_ids = ids.numel()
    if out is None:
        out = torch.empty((n_ids, dim), dtype=torch.float32, device=w.device)
    po = _dev(out, "out", _F32, n_ids * dim)
    pe = _dev(err_flag, "err_flag", _I32, 1) if err_flag is not None else None
    _check(lib().rowq_gather(pw, ps, vocab, dim, bits, group, pi, n_ids, float(mult), po, pe, _stream(w)))
    return out


# ------------------------------------------------------------- GEMV chain
LINK_GEMV, LINK_GELU, LINK_HEAD = 0, 1, 2
CHAIN_MAX_K = 10240
CHAIN_GELU_MAX_K = 5120


class Chain:
    """A chain built by q4_chain_build: the host table, its device copy, the
    workspace (zeroed), and references that keep every link's tensors alive.
    ``err()`` reads the workspace's error word (synchronises)."""

    def __init__(self, table_host, table_dev, ws, keep, head):
        self.table_host, self.table_dev, self.ws, self._keep, self.head = table_host, table_dev, ws, keep, head

    def err(self) -> int:
        return int(self.ws[:4].view(torch.int32).item())

    def clear(self):
        self.ws.zero_()


def chain_link(packed: torch.Tensor, n: int, k: int, x: torch.Tensor, out: torch.Tensor | None = None,
               mode: int = LINK_GEMV, wait: bool = True) -> dict:
    """One link: GEMV (out fp32 [n]), GELU (out bf16 [n/2]) or HEAD (last link, no out)."""
    return dict(packed=packed, n=n, k=k, x=x, out=out, mode=mode, wait=wait)


def q4_chain_build(links, cap: float = 30.0, spin_us: int = 0) -> Chain:
    arr = (ChainLink * len(links))()
    keep = []
    for i, l in enumerate(links):
        n, k, mode = int(l["n"]), int(l["k"]), int(l["mode"])
        pp = _dev(l["packed"], f"links[{i}].packed", _BYTES)
        _check_packed(l["packed"], n, k)
        px = _dev(l["x"], f"links[{i}].x", _U16, k)
        po = 0
        if mode == LINK_GEMV:
            po = _dev(l["out"], f"links[{i}].out", _F32, n)
        elif mode == LINK_GELU:
            po = _dev(l["out"], f"links[{i}].out", _U16, n // 2)
        arr[i] = ChainLink(pp, px, po, n, k, mode, 1 if l.get("wait", True) else 0)
        keep += [l["packed"], l["x"], l["out"]]
    nb = int(lib().q4_chain_table_bytes(len(links)))
    if nb == 0:
        raise ValueError(f"chain of {len(links)} links out of range")
    host = np.zeros((nb + 7) // 8, dtype=np.uint64)
    _check(lib().q4_chain_build(ctypes.cast(arr, ctypes.c_void_p), len(links), float(cap), int(spin_us),
                                host.ctypes.data, host.nbytes))
    dev = links[0]["x"].device
    table_dev = torch.from_numpy(host.view(np.uint8)).to(dev)
    ws = torch.zeros(int(lib().q4_chain_workspace_bytes()), dtype=torch.uint8, device=dev)
    return Chain(host, table_dev, ws, keep, head=int(links[-1]["mode"]) == LINK_HEAD)


def q4_gemv_chain(chain: Chain, idx_out: torch.Tensor | None = None, val_out: torch.Tensor | None = None):
    """Run a built chain (one launch on the current stream). Returns (idx,
    val) for a chain ending in a head, else None."""
    dev = chain.table_dev.device
    pi = pv = 0
    if chain.head:
        if idx_out is None:
            idx_out = torch.empty(1, dtype=torch.int32, device=dev)
        if val_out is None:
            val_out = torch.empty(1, dtype=torch.float32, device=dev)
        pi = _dev(idx_out, "idx_out", _I32, 1)
        pv = _dev(val_out, "val_out", _F32, 1)
    _check(lib().q4_gemv_chain(chain.table_host.ctypes.data, chain.table_dev.data_ptr(), chain.ws.data_ptr(),
                               chain.ws.numel(), pi, pv, _stream(chain.table_dev)))
    return (idx_out, val_out) if chain.head else None
