"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before touching the
GPU (no compute call is made here)."""
import ctypes
import os

import pytest

import int4_weight_only_block_amd as q4

pytestmark = pytest.mark.skipif(not os.path.exists(q4.LIB_PATH), reason="libq4dec.so not built")

EXPECTED = {
    "q4dec_abi_version", "q4dec_last_error", "q4dec_debug_status", "q4dec_debug_selftest", "q4_packed_bytes", "q4_pack", "q4_quantize", "q4_gemv", "q4_gemv_gelu_mul", "q4_gemv_multi", "rowq_gemv", "rowq_gemv_gelu_mul",
    "rowq_head_workspace_bytes", "rowq_softcap_argmax",
    "q4_gemm_s64", "q4_gemm_workspace_bytes", "lmhead_workspace_bytes", "lmhead_softcap_argmax", "lmhead_softcap_argmax_noalloc", "lmhead_multi_workspace_bytes",
    "q4_chain_table_bytes", "q4_chain_workspace_bytes", "q4_chain_build", "q4_gemv_chain", "lmhead_softcap_argmax_multi", "lmhead_s64_workspace_bytes", "lmhead_softcap_argmax_s64", "ple_gather", "rowq_gather",
}


def test_header_declares_expected_functions():
    assert set(q4.header_functions()) == EXPECTED


def test_library_exports_every_header_symbol():
    h = ctypes.CDLL(q4.LIB_PATH)
    for name in q4.header_functions():
        assert hasattr(h, name), name
    assert q4.q4dec_abi_version() == q4.ABI_VERSION


def test_packed_bytes():
    assert q4.q4_packed_bytes(1536, 1536) == 1536 * 768 + 1536 * 48 * 2
    assert q4.q4_packed_bytes(262144, 1536) == 226_492_416
    assert q4.q4_packed_bytes(3, 32) == 256 + 256  # each plane padded to 256 B
    assert q4.q4_packed_bytes(4, 33) == 0
    assert q4.q4_packed_bytes(0, 32) == 0
    assert q4.q4_packed_bytes(-1, 32) == 0
    assert q4.lmhead_workspace_bytes(262144, 1536) >= 8


FAKE = 0x10000  # 64 KiB-aligned non-NULL address; never dereferenced


def _rc_and_msg(rc):
    return rc, q4.q4dec_last_error()


def test_gemv_validation():
    L = q4.lib()
    rc, msg = _rc_and_msg(L.q4_gemv(None, 16, 32, FAKE, FAKE, None))
    assert rc == q4.ERR_NULL and "packed" in msg
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE, 16, 32, None, FAKE, None))
    assert rc == q4.ERR_NULL and "x" in msg
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE, 16, 32, FAKE, None, None))
    assert rc == q4.ERR_NULL and "y" in msg
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE, 0, 32, FAKE, FAKE, None))
    assert rc == q4.ERR_SHAPE and "n" in msg
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE, 16, 48, FAKE, FAKE, None))
    assert rc == q4.ERR_SHAPE and "k" in msg
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE, 16, q4.MAX_K + 32, FAKE, FAKE, None))
    assert rc == q4.ERR_UNSUPPORTED
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE + 4, 16, 32, FAKE, FAKE, None))
    assert rc == q4.ERR_ALIGN and "packed" in msg
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE, 16, 32, FAKE + 2, FAKE, None))
    assert rc == q4.ERR_ALIGN and "x" in msg
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE, 16, 32, FAKE, FAKE + 2, None))
    assert rc == q4.ERR_ALIGN and "y" in msg
    rc, msg = _rc_and_msg(L.q4_gemv(FAKE, 1 << 31, 32, FAKE, FAKE, None))
    assert rc == q4.ERR_SHAPE


def test_gemv_gelu_mul_validation():
    L = q4.lib()
    rc, msg = _rc_and_msg(L.q4_gemv_gelu_mul(None, 16, 32, FAKE, FAKE, None))
    assert rc == q4.ERR_NULL and "packed" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_gelu_mul(FAKE, 16, 32, FAKE, None, None))
    assert rc == q4.ERR_NULL and "a" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_gelu_mul(FAKE, 15, 32, FAKE, FAKE, None))
    assert rc == q4.ERR_SHAPE and "even" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_gelu_mul(FAKE, 16, 40, FAKE, FAKE, None))
    assert rc == q4.ERR_SHAPE and "k" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_gelu_mul(FAKE, 16, q4.GELU_MAX_K + 32, FAKE, FAKE, None))
    assert rc == q4.ERR_UNSUPPORTED and "k" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_gelu_mul(FAKE, 16, 32, FAKE, FAKE + 1, None))
    assert rc == q4.ERR_ALIGN and "a" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_gelu_mul(FAKE, 16, 32, FAKE + 8, FAKE, None))
    assert rc == q4.ERR_ALIGN and "x" in msg


def test_quantize_validation():
    L = q4.lib()
    ok = [FAKE, 16, 64, 0, FAKE, FAKE, None, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return _rc_and_msg(L.q4_quantize(*a))

    assert call(0, None)[0] == q4.ERR_NULL
    rc, msg = call(4, None)
    assert rc == q4.ERR_NULL and "codes" in msg
    rc, msg = call(5, None)
    assert rc == q4.ERR_NULL and "scales" in msg
    assert call(1, 0)[0] == q4.ERR_SHAPE
    assert call(2, 48)[0] == q4.ERR_SHAPE
    rc, msg = call(3, 2)
    assert rc == q4.ERR_SHAPE and "rule" in msg
    assert call(0, FAKE + 2)[0] == q4.ERR_ALIGN
    assert call(4, FAKE + 8)[0] == q4.ERR_ALIGN
    assert call(5, FAKE + 1)[0] == q4.ERR_ALIGN


def test_gemv_multi_validation():
    L = q4.lib()
    rc, msg = _rc_and_msg(L.q4_gemv_multi(FAKE, 16, 32, FAKE, 0, FAKE, None))
    assert rc == q4.ERR_SHAPE and "m" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_multi(FAKE, 16, 32, FAKE, 9, FAKE, None))
    assert rc == q4.ERR_SHAPE
    rc, msg = _rc_and_msg(L.q4_gemv_multi(FAKE, 16, 32, FAKE, 4, None, None))
    assert rc == q4.ERR_NULL and "y" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_multi(FAKE, 16, 32, FAKE, 4, FAKE + 2, None))
    assert rc == q4.ERR_ALIGN and "y" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_multi(FAKE, 16, 48, FAKE, 4, FAKE, None))
    assert rc == q4.ERR_SHAPE and "k" in msg
    rc, msg = _rc_and_msg(L.q4_gemv_multi(None, 16, 32, FAKE, 4, FAKE, None))
    assert rc == q4.ERR_NULL and "packed" in msg


def test_rowq_gemv_validation():
    L = q4.lib()
    ok = [FAKE, FAKE, 16, 128, 2, FAKE, FAKE, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return _rc_and_msg(L.rowq_gemv(*a))

    for i, name in [(0, "w"), (1, "row_scale"), (5, "x"), (6, "y")]:
        rc, msg = call(i, None)
        assert rc == q4.ERR_NULL and name in msg
    rc, msg = call(4, 3)
    assert rc == q4.ERR_SHAPE and "bits" in msg
    rc, msg = call(3, 96)
    assert rc == q4.ERR_SHAPE and "64" in msg  # INT2 codes come in 64-wide 16-byte chunks
    a = list(ok); a[3] = 48; a[4] = 4
    rc, msg = _rc_and_msg(L.rowq_gemv(*a))
    assert rc == q4.ERR_SHAPE and "32" in msg  # INT4 in 32-wide ones
    a[4] = 8
    rc, msg = _rc_and_msg(L.rowq_gemv(*a))
    assert rc == q4.ERR_SHAPE and "32" in msg  # INT8 in 32-wide 32-byte ones
    assert call(4, 16)[0] == q4.ERR_SHAPE
    assert call(2, 0)[0] == q4.ERR_SHAPE
    assert call(3, q4.MAX_K + 64)[0] == q4.ERR_UNSUPPORTED
    assert call(0, FAKE + 8)[0] == q4.ERR_ALIGN
    assert call(5, FAKE + 2)[0] == q4.ERR_ALIGN
    assert call(6, FAKE + 2)[0] == q4.ERR_ALIGN


def test_rowq_gemv_gelu_mul_validation():
    L = q4.lib()
    ok = [FAKE, FAKE, 16, 128, 2, FAKE, FAKE, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return _rc_and_msg(L.rowq_gemv_gelu_mul(*a))

    for i, name in [(0, "w"), (1, "row_scale"), (5, "x"), (6, "a")]:
        rc, msg = call(i, None)
        assert rc == q4.ERR_NULL and name in msg
    rc, msg = call(2, 15)
    assert rc == q4.ERR_SHAPE and "even" in msg
    rc, msg = call(3, q4.GELU_MAX_K + 64)
    assert rc == q4.ERR_UNSUPPORTED and str(q4.GELU_MAX_K) in msg
    assert call(4, 16)[0] == q4.ERR_SHAPE and "bits" in call(4, 16)[1]
    assert call(3, 96)[0] == q4.ERR_SHAPE
    assert call(6, FAKE + 1)[0] == q4.ERR_ALIGN
    assert call(1, FAKE + 2)[0] == q4.ERR_ALIGN


def test_lmhead_multi_validation():
    L = q4.lib()
    need = L.lmhead_multi_workspace_bytes(262144, 1536, 4)
    assert need >= 8 * 8 * 1024
    ok = [FAKE, 1000, 1536, FAKE, 4, 30.0, FAKE, need, FAKE, FAKE, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return _rc_and_msg(L.lmhead_softcap_argmax_multi(*a))

    for i, name in [(0, "packed"), (3, "x"), (6, "ws"), (8, "idx_out"), (9, "val_out")]:
        rc, msg = call(i, None)
        assert rc == q4.ERR_NULL and name in msg
    rc, msg = call(4, 9)
    assert rc == q4.ERR_SHAPE and "m" in msg
    assert call(4, 0)[0] == q4.ERR_SHAPE
    assert call(1, 0)[0] == q4.ERR_SHAPE
    assert call(2, 48)[0] == q4.ERR_SHAPE
    assert call(2, q4.MAX_K + 32)[0] == q4.ERR_UNSUPPORTED
    rc, msg = call(7, need - 8)
    assert rc == q4.ERR_WORKSPACE and "ws_bytes" in msg
    assert call(6, FAKE + 4)[0] == q4.ERR_ALIGN
    assert call(3, FAKE + 8)[0] == q4.ERR_ALIGN
    assert call(8, FAKE + 2)[0] == q4.ERR_ALIGN


def test_pack_validation():
    L = q4.lib()
    assert L.q4_pack(None, FAKE, 4, 32, FAKE, None, None) == q4.ERR_NULL
    assert L.q4_pack(FAKE, None, 4, 32, FAKE, None, None) == q4.ERR_NULL
    assert L.q4_pack(FAKE, FAKE, 4, 32, None, None, None) == q4.ERR_NULL
    assert L.q4_pack(FAKE, FAKE, 4, 31, FAKE, None, None) == q4.ERR_SHAPE
    assert L.q4_pack(FAKE, FAKE, -4, 32, FAKE, None, None) == q4.ERR_SHAPE
    assert L.q4_pack(FAKE, FAKE, 4, 32, FAKE + 8, None, None) == q4.ERR_ALIGN
    assert "packed" in q4.q4dec_last_error()


def test_lmhead_validation():
    L = q4.lib()
    need = q4.lmhead_workspace_bytes(1024, 64)
    args = [FAKE, 1024, 64, FAKE, 30.0, FAKE, need, FAKE, FAKE, None]

    def call(**kw):
        a = list(args)
        names = ["packed", "vocab", "k", "x", "cap", "ws", "ws_bytes", "idx", "val", "stream"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return L.lmhead_softcap_argmax(*a)

    assert call(ws=None) == q4.ERR_NULL and "ws" in q4.q4dec_last_error()
    assert call(idx=None) == q4.ERR_NULL
    assert call(val=None) == q4.ERR_NULL
    assert call(ws_bytes=need - 1) == q4.ERR_WORKSPACE
    assert call(vocab=0) == q4.ERR_SHAPE and "vocab" in q4.q4dec_last_error()
    assert call(k=40) == q4.ERR_SHAPE
    assert call(ws=FAKE + 4) == q4.ERR_ALIGN
    assert call(idx=FAKE + 2) == q4.ERR_ALIGN


def test_lmhead_noalloc_validation():
    """Argument errors return before the scratch lookup or any launch."""
    L = q4.lib()
    args = [FAKE, 1024, 64, FAKE, 30.0, FAKE, FAKE, None]

    def call(**kw):
        a = list(args)
        names = ["packed", "vocab", "k", "x", "cap", "idx", "val", "stream"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return L.lmhead_softcap_argmax_noalloc(*a)

    assert call(packed=None) == q4.ERR_NULL and "packed" in q4.q4dec_last_error()
    assert call(x=None) == q4.ERR_NULL
    assert call(idx=None) == q4.ERR_NULL and "idx_out" in q4.q4dec_last_error()
    assert call(val=None) == q4.ERR_NULL
    assert call(vocab=0) == q4.ERR_SHAPE and "vocab" in q4.q4dec_last_error()
    assert call(vocab=1 << 31) == q4.ERR_SHAPE
    assert call(k=40) == q4.ERR_SHAPE
    assert call(k=q4.MAX_K + 32) == q4.ERR_UNSUPPORTED
    assert call(packed=FAKE + 8) == q4.ERR_ALIGN
    assert call(idx=FAKE + 2) == q4.ERR_ALIGN
    assert "lmhead_softcap_argmax_noalloc" in q4.q4dec_last_error()


def test_gemm_validation():
    L = q4.lib()
    need = q4.q4_gemm_workspace_bytes(64, 64)
    assert need > 0 and q4.q4_gemm_workspace_bytes(64, 40) == 0
    ok = [FAKE, 64, 64, FAKE, 64, FAKE, FAKE, need, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return L.q4_gemm_s64(*a)

    assert call(4, 0) == q4.ERR_SHAPE and "n_tok" in q4.q4dec_last_error()
    assert call(4, 65) == q4.ERR_SHAPE
    assert call(0, None) == q4.ERR_NULL
    assert call(6, None) == q4.ERR_NULL and "ws" in q4.q4dec_last_error()
    assert call(2, 48) == q4.ERR_SHAPE
    assert call(2, q4.MAX_K + 32) == q4.ERR_UNSUPPORTED
    assert call(7, need - 1) == q4.ERR_WORKSPACE
    assert call(6, FAKE + 16) == q4.ERR_ALIGN
    assert call(0, FAKE + 8) == q4.ERR_ALIGN


def test_head_s64_validation():
    L = q4.lib()
    need = q4.lmhead_s64_workspace_bytes(1000, 64)
    assert need > 0 and q4.lmhead_s64_workspace_bytes(1000, 40) == 0
    assert q4.lmhead_s64_workspace_bytes(0, 64) == 0
    # packed, vocab, k, x, n_tok, cap, ws, ws_bytes, idx_out, val_out, stream
    ok = [FAKE, 1000, 64, FAKE, 64, 30.0, FAKE, need, FAKE, FAKE, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return L.lmhead_softcap_argmax_s64(*a)

    for i, name in [(0, "packed"), (3, "x"), (6, "ws"), (8, "idx_out"), (9, "val_out")]:
        assert call(i, None) == q4.ERR_NULL and name in q4.q4dec_last_error()
    assert call(4, 0) == q4.ERR_SHAPE and "n_tok" in q4.q4dec_last_error()
    assert call(4, 65) == q4.ERR_SHAPE
    assert call(1, 0) == q4.ERR_SHAPE and "vocab" in q4.q4dec_last_error()
    assert call(2, 48) == q4.ERR_SHAPE
    assert call(2, q4.MAX_K + 32) == q4.ERR_UNSUPPORTED
    assert call(7, need - 1) == q4.ERR_WORKSPACE
    assert call(6, FAKE + 16) == q4.ERR_ALIGN
    assert call(0, FAKE + 8) == q4.ERR_ALIGN
    assert call(3, FAKE + 8) == q4.ERR_ALIGN
    assert call(8, FAKE + 2) == q4.ERR_ALIGN


def test_rowq_head_validation():
    L = q4.lib()
    need = q4.rowq_head_workspace_bytes(262144, 1536, 2)
    assert need == 8192 * 8
    # w, row_scale, vocab, k, bits, x, cap, ws, ws_bytes, idx_out, val_out, stream
    ok = [FAKE, FAKE, 262144, 1536, 2, FAKE, 30.0, FAKE, need, FAKE, FAKE, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return L.rowq_softcap_argmax(*a)

    for i, name in [(0, "w"), (1, "row_scale"), (5, "x"), (7, "ws"), (9, "idx_out"), (10, "val_out")]:
        assert call(i, None) == q4.ERR_NULL and name in q4.q4dec_last_error()
    assert call(4, 3) == q4.ERR_SHAPE and "bits" in q4.q4dec_last_error()
    assert call(4, 16) == q4.ERR_SHAPE
    assert call(2, 0) == q4.ERR_SHAPE and "n" in q4.q4dec_last_error()
    assert call(3, 32) == q4.ERR_SHAPE  # INT2 chunks hold 64 codes
    assert call(3, q4.MAX_K + 64) == q4.ERR_UNSUPPORTED
    assert call(8, need - 1) == q4.ERR_WORKSPACE
    assert call(7, FAKE + 4) == q4.ERR_ALIGN
    assert call(0, FAKE + 8) == q4.ERR_ALIGN
    assert call(5, FAKE + 8) == q4.ERR_ALIGN
    assert call(9, FAKE + 2) == q4.ERR_ALIGN
    assert call(10, FAKE + 1) == q4.ERR_ALIGN


def test_rowq_gather_validation():
    L = q4.lib()
    # w, scales, vocab, dim, bits, group, ids, n_ids, mult, out, err_flag, stream
    ok = [FAKE, FAKE, 100, 1536, 2, 1536, FAKE, 4, 39.19, FAKE, None, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return L.rowq_gather(*a)

    for i, name in [(0, "w"), (1, "scales"), (6, "ids"), (9, "out")]:
        assert call(i, None) == q4.ERR_NULL and name in q4.q4dec_last_error()
    assert call(4, 8) == q4.ERR_SHAPE and "bits" in q4.q4dec_last_error()
    assert call(2, 0) == q4.ERR_SHAPE and "vocab" in q4.q4dec_last_error()
    assert call(3, 1504) == q4.ERR_SHAPE and "dim" in q4.q4dec_last_error()   # not a multiple of 64
    assert call(5, 96) == q4.ERR_SHAPE and "group" in q4.q4dec_last_error()   # INT2 groups of 64
    assert call(5, 1000) == q4.ERR_SHAPE                                       # does not divide dim
    assert call(7, -1) == q4.ERR_SHAPE and "n_ids" in q4.q4dec_last_error()
    assert call(7, 0) == q4.OK                                                 # no-op
    assert call(0, FAKE + 8) == q4.ERR_ALIGN
    assert call(9, FAKE + 4) == q4.ERR_ALIGN
    a = list(ok)
    a[4], a[3], a[5] = 4, 8960, 256   # the INT4 PLE layout is accepted
    a[7] = 0
    assert L.rowq_gather(*a) == q4.OK


def test_ple_validation():
    L = q4.lib()
    ok = [FAKE, FAKE, 100, 64, FAKE, 4, 16.0, FAKE, None, None]
    assert L.ple_gather(None, *ok[1:]) == q4.ERR_NULL
    a = list(ok); a[2] = 0
    assert L.ple_gather(*a) == q4.ERR_SHAPE and "vocab" in q4.q4dec_last_error()
    a = list(ok); a[3] = -1
    assert L.ple_gather(*a) == q4.ERR_SHAPE and "dim" in q4.q4dec_last_error()
    a = list(ok); a[5] = -1
    assert L.ple_gather(*a) == q4.ERR_SHAPE
    a = list(ok); a[5] = 0  # empty gather is a no-op and touches nothing
    assert L.ple_gather(*a) == q4.OK
    a = list(ok); a[7] = FAKE + 2
    assert L.ple_gather(*a) == q4.ERR_ALIGN


def test_binding_rejects_host_tensors():
    import torch

    with pytest.raises(ValueError):
        q4.q4_gemv(torch.zeros(100, dtype=torch.uint8), 2, 32, torch.zeros(32, dtype=torch.int16))


def test_chain_build_validation():
    """q4_chain_build is host-only; every rejection below returns before any
    device query (fake, never dereferenced addresses)."""
    import numpy as np

    L = q4.lib()
    MB = 1 << 20

    def link(i, **kw):
        d = dict(packed=FAKE + (10 + 4 * i) * MB, x=FAKE + (11 + 4 * i) * MB, out=FAKE + (12 + 4 * i) * MB,
                 n=256, k=2560, mode=q4.LINK_GEMV, wait=1)
        d.update(kw)
        return q4.ChainLink(d["packed"], d["x"], d["out"], d["n"], d["k"], d["mode"], d["wait"])

    def build(links, table_bytes=None, n=None):
        arr = (q4.ChainLink * len(links))(*links)
        nl = len(links) if n is None else n
        tb = int(L.q4_chain_table_bytes(max(nl, 1))) if table_bytes is None else table_bytes
        host = np.zeros(max(tb, 8) // 8 + 1, dtype=np.uint64)
        return L.q4_chain_build(arr, nl, 30.0, 0, host.ctypes.data, tb)

    assert L.q4_chain_table_bytes(0) == 0 and L.q4_chain_table_bytes(169) == 64 + 169 * 64
    assert L.q4_chain_workspace_bytes() >= 256 + 16 * 256
    assert build([link(0)], n=0) == q4.ERR_SHAPE
    assert build([link(0)], table_bytes=64) == q4.ERR_WORKSPACE
    assert build([link(0, k=40)]) == q4.ERR_SHAPE and "k must be" in q4.q4dec_last_error()
    assert build([link(0, k=q4.CHAIN_MAX_K + 32)]) == q4.ERR_UNSUPPORTED
    assert build([link(0, n=0)]) == q4.ERR_SHAPE
    assert build([link(0, mode=7)]) == q4.ERR_SHAPE
    assert build([link(0, mode=q4.LINK_HEAD), link(1)]) == q4.ERR_SHAPE and "last" in q4.q4dec_last_error()
    assert build([link(0, mode=q4.LINK_GELU, n=255)]) == q4.ERR_SHAPE
    assert build([link(0, mode=q4.LINK_GELU, k=q4.CHAIN_GELU_MAX_K + 32)]) == q4.ERR_SHAPE
    assert build([link(0, packed=FAKE + 10 * MB + 8)]) == q4.ERR_ALIGN
    assert build([link(0, out=0)]) == q4.ERR_NULL
    # an output in a line its own link reads
    assert build([link(0, out=FAKE + 11 * MB + 4096)]) == q4.ERR_SHAPE and "line" in q4.q4dec_last_error()
    # an output in a line an earlier link reads
    assert build([link(0), link(1, out=FAKE + 11 * MB)]) == q4.ERR_SHAPE
    # two outputs sharing a line
    assert build([link(0), link(1, out=FAKE + 12 * MB + 128)]) == q4.ERR_SHAPE
    # a later link reading an earlier output without a wait in between
    assert build([link(0), link(1, x=FAKE + 12 * MB, wait=0)]) == q4.ERR_SHAPE and "wait" in q4.q4dec_last_error()


def test_chain_run_validation():
    import numpy as np

    L = q4.lib()
    host = np.zeros(64, dtype=np.uint64)
    ws_bytes = int(L.q4_chain_workspace_bytes())
    assert L.q4_gemv_chain(None, FAKE, FAKE, ws_bytes, FAKE, FAKE, None) == q4.ERR_NULL
    assert L.q4_gemv_chain(host.ctypes.data, FAKE, FAKE, ws_bytes - 1, FAKE, FAKE, None) == q4.ERR_WORKSPACE
    assert L.q4_gemv_chain(host.ctypes.data, FAKE, FAKE + 64, ws_bytes, FAKE, FAKE, None) == q4.ERR_ALIGN
    # a table that q4_chain_build did not write
    assert L.q4_gemv_chain(host.ctypes.data, FAKE, FAKE, ws_bytes, FAKE, FAKE, None) == q4.ERR_SHAPE


def test_debug_status_in_a_release_build():
    """Only a build with Q4DEC_DEBUG=1 carries the launch-contract checks; a
    release build says so (no GPU call is made)."""
    if os.path.basename(q4.LIB_PATH) != "libq4dec.so":
        pytest.skip("not the release library")
    rc, word = q4.debug_status()
    assert rc == q4.ERR_UNSUPPORTED and word == 0
    assert "Q4DEC_DEBUG" in q4.q4dec_last_error()
    assert q4.lib().q4dec_debug_status(None) == q4.ERR_NULL
