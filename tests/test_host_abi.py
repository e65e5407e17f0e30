"""Host-side tests of libqlr.so: it loads, exports every declared symbol, and its
host logic (codebook, size queries, argument validation) behaves.  No kernel is
launched here: every call below either is host-only or fails validation before
any HIP call."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from quantized_base_fine_amd import qlr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "qlr.h")).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(qlr_\w+)\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ["qlr_quantize", "qlr_dequantize", "qlr_linear_fwd", "qlr_linear_fwd_mixed",
                 "qlr_codebook", "qlr_qweight_sizes", "qlr_workspace_bytes"]:
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = qlr.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert name in qlr.EXPORTS, name  # the binding knows its signature


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_codebook_bit_equal_to_oracle(bits):
    got = np.array(qlr.codebook(bits), dtype=np.float32)
    ref = oracle.quantile_codebook(bits)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape", [(1, 1), (1, 64), (37, 101), (256, 256), (4096, 11008), (22016, 8192)])
def test_sizes_match_oracle(bits, shape):
    assert qlr.qweight_sizes(shape[0], shape[1], bits) == oracle.qweight_sizes(shape[0], shape[1], bits)


def test_workspace_sizes():
    assert qlr.workspace_bytes(qlr.OP_QUANTIZE) == 256
    assert qlr.workspace_bytes(qlr.OP_LINEAR, 0, 4096, 4096, 16) == 0
    assert qlr.workspace_bytes(qlr.OP_LINEAR, 7, 4096, 4096, 0) == 0
    # float32 partial sums of x A^T over the adapter product's K splits, rounded
    # to 256 bytes: one pass (no split) for M > 16; 32 splits at M=1, K=4096; 1 at K=64
    assert qlr.workspace_bytes(qlr.OP_LINEAR, 2048, 4096, 4096, 16) == 2048 * 16 * 4  # M > 16: one K pass
    assert qlr.workspace_bytes(qlr.OP_LINEAR, 1, 4096, 4096, 16) == 32 * 16 * 4
    assert qlr.workspace_bytes(qlr.OP_LINEAR, 3, 10, 64, 5) == 256
    # splits x M x r <= 4096 (a decode workgroup prefetches every partial sum at once)
    assert qlr.workspace_bytes(qlr.OP_LINEAR, 16, 4096, 11008, 64) == 4 * 16 * 64 * 4
    assert qlr.workspace_bytes(qlr.OP_LINEAR, 1, 22016, 8192, 64) == 64 * 64 * 4


def _status(fn, *args):
    return qlr.STATUS[fn(*args)]


def test_status_strings_and_last_error():
    lib = qlr.lib()
    for code in qlr.STATUS:
        assert lib.qlr_status_string(code)
    assert lib.qlr_codebook(5, (C.c_float * 32)()) == 4
    assert b"bits 5" in lib.qlr_last_error()


def test_size_query_errors():
    lib = qlr.lib()
    a = C.c_size_t()
    assert _status(lib.qlr_qweight_sizes, 4, 4, 5, 64, C.byref(a), C.byref(a), C.byref(a)) == "QLR_ERR_BITS"
    assert _status(lib.qlr_qweight_sizes, 4, 4, 4, 32, C.byref(a), C.byref(a), C.byref(a)) == "QLR_ERR_BLOCK"
    assert _status(lib.qlr_qweight_sizes, -1, 4, 4, 64, C.byref(a), C.byref(a), C.byref(a)) == "QLR_ERR_SHAPE"
    assert _status(lib.qlr_qweight_sizes, 4, 4, 4, 64, None, C.byref(a), C.byref(a)) == "QLR_ERR_NULL"
    assert _status(lib.qlr_codebook, 4, None) == "QLR_ERR_NULL"
    assert _status(lib.qlr_force_path, 9) == "QLR_ERR_PATH"


FAKE = 0x10000  # a 16-byte-aligned address that validation never dereferences


def _qw(bits=4, rows=64, cols=128, ver=1, block=64, group=256, codes=FAKE, q8=FAKE, c=FAKE):
    return qlr.CQWeight(ver, bits, block, group, rows, cols, codes, q8, c)


def _lin(w, x=FAKE, xdt=qlr.QLR_BF16, M=4, A=FAKE, B=FAKE, abdt=qlr.QLR_BF16, r=4, y=FAKE,
         ydt=qlr.QLR_F32, ws=FAKE, wsb=1 << 20):
    lib = qlr.lib()
    return qlr.STATUS[lib.qlr_linear_fwd(x, xdt, M, C.byref(w), A, B, abdt, r, 1.0, y, ydt, ws, wsb, None)]


def test_linear_validation_errors():
    assert _lin(_qw(bits=5)) == "QLR_ERR_BITS"
    assert _lin(_qw(ver=2)) == "QLR_ERR_FORMAT"
    assert _lin(_qw(block=32)) == "QLR_ERR_BLOCK"
    assert _lin(_qw(group=128)) == "QLR_ERR_BLOCK"
    assert _lin(_qw(cols=100)) == "QLR_ERR_SHAPE"
    assert _lin(_qw(codes=0)) == "QLR_ERR_NULL"
    assert _lin(_qw(q8=FAKE + 8)) == "QLR_ERR_ALIGN"
    assert _lin(_qw(), x=0) == "QLR_ERR_NULL"
    assert _lin(_qw(), x=FAKE + 2) == "QLR_ERR_ALIGN"
    assert _lin(_qw(), A=0) == "QLR_ERR_NULL"
    assert _lin(_qw(), M=-1) == "QLR_ERR_SHAPE"
    assert _lin(_qw(), r=-1) == "QLR_ERR_SHAPE"
    assert _lin(_qw(), xdt=qlr.QLR_F16) == "QLR_ERR_DTYPE"
    assert _lin(_qw(), ydt=7) == "QLR_ERR_DTYPE"
    assert _lin(_qw(), ws=0) == "QLR_ERR_WORKSPACE"
    assert _lin(_qw(), wsb=16) == "QLR_ERR_WORKSPACE"
    assert _lin(_qw(), M=0, x=0, y=0) == "QLR_OK"  # nothing to do, nothing launched


def test_forced_path_errors():
    lib = qlr.lib()
    try:
        lib.qlr_force_path(qlr.PATH_GEMV)
        assert _lin(_qw(), M=17) == "QLR_ERR_PATH"
        assert _lin(_qw(), xdt=qlr.QLR_F32) == "QLR_ERR_PATH"
        lib.qlr_force_path(qlr.PATH_GEMM)
        assert _lin(_qw(), abdt=qlr.QLR_F32) == "QLR_ERR_PATH"
    finally:
        lib.qlr_force_path(qlr.PATH_AUTO)


def _quant(W=FAKE, wdt=qlr.QLR_F16, rows=64, cols=128, bits=4, block=64, out=None, ws=FAKE, wsb=256):
    out = out or _qw(bits=bits, rows=rows, cols=cols)
    return qlr.STATUS[qlr.lib().qlr_quantize(W, wdt, rows, cols, bits, block, C.byref(out), ws, wsb, None)]


def test_quantize_validation_errors():
    assert _quant(W=0) == "QLR_ERR_NULL"
    assert _quant(wdt=9) == "QLR_ERR_DTYPE"
    assert _quant(bits=5) == "QLR_ERR_BITS"
    assert _quant(block=128) == "QLR_ERR_BLOCK"
    assert _quant(rows=0) == "QLR_ERR_SHAPE"
    assert _quant(out=_qw(rows=65, cols=128)) == "QLR_ERR_SHAPE"
    assert _quant(W=FAKE + 4) == "QLR_ERR_ALIGN"
    assert _quant(ws=0) == "QLR_ERR_WORKSPACE"
    assert _quant(wsb=64) == "QLR_ERR_WORKSPACE"


def test_mixed_alias_detection():
    lib = qlr.lib()
    w = _qw(rows=64, cols=128)
    arr = (qlr.CLayer * 2)()
    arr[0] = qlr.CLayer(C.pointer(w), 0x100000, 0, 0, 0, 0.0, 0x200000)
    arr[1] = qlr.CLayer(C.pointer(w), 0x300000, 0, 0, 0, 0.0, 0x200000 + 64)  # overlaps y0
    assert qlr.STATUS[lib.qlr_linear_fwd_mixed(arr, 2, 4, qlr.QLR_BF16, qlr.QLR_BF16, qlr.QLR_F32,
                                               None, 0, None)] == "QLR_ERR_ALIAS"
    arr[1] = qlr.CLayer(C.pointer(w), 0x200000 + 16, 0, 0, 0, 0.0, 0x400000)  # x1 inside y0
    assert qlr.STATUS[lib.qlr_linear_fwd_mixed(arr, 2, 4, qlr.QLR_BF16, qlr.QLR_BF16, qlr.QLR_F32,
                                               None, 0, None)] == "QLR_ERR_ALIAS"
    arr[1] = qlr.CLayer(C.pointer(_qw(bits=7)), 0x300000, 0, 0, 0, 0.0, 0x500000)
    assert qlr.STATUS[lib.qlr_linear_fwd_mixed(arr, 2, 4, qlr.QLR_BF16, qlr.QLR_BF16, qlr.QLR_F32,
                                               None, 0, None)] == "QLR_ERR_BITS"


def _bwd(w, dy=0x100000, dydt=qlr.QLR_BF16, x=0x200000, xdt=qlr.QLR_BF16, M=4, A=0x300000, B=0x400000,
         abdt=qlr.QLR_BF16, r=4, dx=0x500000, dxdt=qlr.QLR_F32, dA=0x600000, dB=0x700000, ws=0x800000,
         wsb=1 << 20):
    lib = qlr.lib()
    return qlr.STATUS[lib.qlr_linear_bwd(dy, dydt, x, xdt, M, C.byref(w), A, B, abdt, r, 1.0, dx, dxdt,
                                         dA, dB, ws, wsb, None)]


def test_backward_validation_errors():
    assert _bwd(_qw(bits=5)) == "QLR_ERR_BITS"
    assert _bwd(_qw(cols=100)) == "QLR_ERR_SHAPE"
    assert _bwd(_qw(), M=-1) == "QLR_ERR_SHAPE"
    assert _bwd(_qw(), dy=0) == "QLR_ERR_NULL"
    assert _bwd(_qw(), x=0) == "QLR_ERR_NULL"
    assert _bwd(_qw(), dA=0) == "QLR_ERR_NULL"
    assert _bwd(_qw(), B=0) == "QLR_ERR_NULL"
    assert _bwd(_qw(), dx=0x500008) == "QLR_ERR_ALIGN"
    assert _bwd(_qw(), dydt=qlr.QLR_F16) == "QLR_ERR_DTYPE"
    assert _bwd(_qw(), xdt=qlr.QLR_F32) == "QLR_ERR_DTYPE"  # x and dy must share a dtype
    assert _bwd(_qw(), dxdt=9) == "QLR_ERR_DTYPE"
    assert _bwd(_qw(), dA=0x100000) == "QLR_ERR_ALIAS"  # dA on top of dy
    assert _bwd(_qw(), dB=0x600000 + 256) == "QLR_ERR_ALIAS"  # dB inside dA
    assert _bwd(_qw(), dx=0x200000) == "QLR_ERR_ALIAS"  # dx on top of x
    assert _bwd(_qw(), ws=0) == "QLR_ERR_WORKSPACE"
    assert _bwd(_qw(), wsb=64) == "QLR_ERR_WORKSPACE"
    # no adapter: x is not read and no workspace is needed; M = 0 with r = 0 launches nothing
    assert _bwd(_qw(), M=0, r=0, x=0, dy=0, dx=0, A=0, B=0, dA=0, dB=0, ws=0) == "QLR_OK"
    lib = qlr.lib()
    try:
        lib.qlr_force_path(qlr.PATH_GEMM)
        assert _bwd(_qw(rows=65)) == "QLR_ERR_PATH"  # the MFMA backward takes whole 64-row steps
        assert _bwd(_qw(), abdt=qlr.QLR_F32) == "QLR_ERR_PATH"
    finally:
        lib.qlr_force_path(qlr.PATH_AUTO)


def test_backward_workspace_sizes():
    assert qlr.workspace_bytes(qlr.OP_LINEAR_BWD, 2048, 4096, 4096, 0) == 0
    small = qlr.workspace_bytes(qlr.OP_LINEAR_BWD, 3, 64, 128, 4)
    # t and u (one split each), B transposed (r x N float32-sized), no gradient partials at M = 3
    assert small == 256 + 256 + 1024
    big = qlr.workspace_bytes(qlr.OP_LINEAR_BWD, 2048, 4096, 4096, 16)
    assert big >= 2 * 2048 * 16 * 4 + 16 * 4096 * 4
    assert big % 256 == 0


def test_dba_validation_and_workspace():
    lib = qlr.lib()
    w = _qw(rows=64, cols=128)
    good = qlr.CDba(16, 1, 0x100000, 0x200000, 0x300000, 0x400000, 0x500000)

    def call(ad, ws=0x900000, wsb=1 << 20, M=4, x=0x600000, y=0x700000):
        return qlr.STATUS[lib.qlr_linear_fwd_dba(x, qlr.QLR_BF16, M, C.byref(w), C.byref(ad) if ad else None, y,
                                                 qlr.QLR_F32, ws, wsb, None)]
    assert call(None) == "QLR_ERR_NULL"
    assert call(qlr.CDba(0, 1, 0x100000, 0x200000, 0x300000, 0x400000, 0x500000)) == "QLR_ERR_SHAPE"
    assert call(qlr.CDba(16, 0, 0x100000, 0x200000, 0x300000, 0x400000, 0x500000)) == "QLR_ERR_SHAPE"
    assert call(qlr.CDba(16, 1, 0, 0x200000, 0x300000, 0x400000, 0x500000)) == "QLR_ERR_NULL"
    assert call(qlr.CDba(16, 1, 0x100004, 0x200000, 0x300000, 0x400000, 0x500000)) == "QLR_ERR_ALIGN"
    assert call(good, ws=0) == "QLR_ERR_WORKSPACE"
    assert call(good, wsb=64) == "QLR_ERR_WORKSPACE"
    # workspace: [t' | t'] float32 splits x M x 2 l R, then the alpha-signed factor N x 2 l R bf16
    need = qlr.workspace_bytes(qlr.OP_LINEAR_DBA, 2048, 4096, 4096, 16)
    assert need == 2 * 2048 * 32 * 4 + 4096 * 32 * 2  # two K splits of the first stage at M = 2048
    assert qlr.workspace_bytes(qlr.OP_LINEAR_DBA, 0, 64, 128, 16) == 64 * 32 * 2


def test_outlier_validation_and_workspace():
    lib = qlr.lib()
    w = _qw(rows=64, cols=128)

    def quant(k=10, sp=None, W=0x100000, wdt=qlr.QLR_F16, rows=64, cols=128, ws=0x900000, wsb=1 << 24, out=None):
        sp = sp if sp is not None else qlr.CSparse(rows, cols, k, 0x200000, 0x300000, 0x400000)
        out = out or _qw(rows=rows, cols=cols)
        return qlr.STATUS[lib.qlr_quantize_outliers(W, wdt, rows, cols, 4, 64, k, C.byref(out), C.byref(sp), ws,
                                                    wsb, None)]
    assert quant(W=0) == "QLR_ERR_NULL"
    assert quant(wdt=9) == "QLR_ERR_DTYPE"
    assert quant(k=-1) == "QLR_ERR_SHAPE"
    assert quant(k=64 * 128 + 1) == "QLR_ERR_SHAPE"
    assert quant(rows=1 << 16, cols=1 << 15) == "QLR_ERR_SHAPE"  # flat indices must fit int32
    assert quant(sp=qlr.CSparse(64, 128, 11, 0x200000, 0x300000, 0x400000)) == "QLR_ERR_SHAPE"  # nnz != k
    assert quant(sp=qlr.CSparse(64, 128, 10, 0x200000, 0, 0x400000)) == "QLR_ERR_NULL"
    assert quant(sp=qlr.CSparse(64, 128, 10, 0x200004, 0x300000, 0x400000)) == "QLR_ERR_ALIGN"
    assert quant(ws=0) == "QLR_ERR_WORKSPACE"
    assert quant(wsb=1024) == "QLR_ERR_WORKSPACE"
    # workspace: flag, selection state, histogram, per-4096-element counts and plan, the k
    # (index, value) pairs, and a dense float32-sized copy of the weight (256-byte aligned pieces)
    up = lambda b: (b + 255) // 256 * 256
    nel, k = 4096 * 4096, 16777
    nblk = -(-nel // 4096)
    assert qlr.workspace_bytes(qlr.OP_QUANTIZE_OUTLIERS, k, 4096, 4096) == (
        256 + 256 + 2048 * 4 + 2 * up(8 * nblk) + 2 * up(4 * k) + 4 * nel)

    def fwd(sp, M=4, ws=0x900000, wsb=1 << 24):
        return qlr.STATUS[lib.qlr_linear_fwd_outliers(0x600000, qlr.QLR_BF16, M, C.byref(w),
                                                      C.byref(sp) if sp else None, 0x500000, 0x500000,
                                                      qlr.QLR_BF16, 4, 1.0, 0x700000, qlr.QLR_F32, ws, wsb, None)]
    good = qlr.CSparse(64, 128, 10, 0x200000, 0x300000, 0x400000)
    assert fwd(None) == "QLR_ERR_NULL"
    assert fwd(qlr.CSparse(65, 128, 10, 0x200000, 0x300000, 0x400000)) == "QLR_ERR_SHAPE"
    assert fwd(qlr.CSparse(64, 128, -1, 0x200000, 0x300000, 0x400000)) == "QLR_ERR_SHAPE"
    assert fwd(qlr.CSparse(64, 128, 10, 0, 0x300000, 0x400000)) == "QLR_ERR_NULL"
    assert fwd(qlr.CSparse(64, 128, 10, 0x200000, 0x300008, 0x400000)) == "QLR_ERR_ALIGN"
    assert fwd(good, ws=0) == "QLR_ERR_WORKSPACE"
    assert fwd(good, wsb=64) == "QLR_ERR_WORKSPACE"
    assert fwd(good, M=0, ws=0, wsb=0) == "QLR_OK"
    # the linear workspace, then the M x N float32 sparse term
    assert qlr.workspace_bytes(qlr.OP_LINEAR_OUTLIERS, 2048, 4096, 4096, 16) == (
        qlr.workspace_bytes(qlr.OP_LINEAR, 2048, 4096, 4096, 16) + 2048 * 4096 * 4)


def test_wha_validation_and_workspace():
    lib = qlr.lib()
    w = _qw(rows=64, cols=128)
    good = qlr.CSparse(64, 128, 10, 0x200000, 0x300000, 0x400000)

    def call(F, hb=128, M=4, ws=0x900000, wsb=1 << 24):
        return qlr.STATUS[lib.qlr_linear_fwd_wha(0x600000, qlr.QLR_BF16, M, C.byref(w), C.byref(F) if F else None, hb,
                                                 0x700000, qlr.QLR_F32, ws, wsb, None)]
    assert call(None) == "QLR_ERR_NULL"
    for hb in (0, 3, 96, 256):  # not a power of two, or not dividing cols
        assert call(good, hb=hb) == "QLR_ERR_SHAPE"
    assert call(qlr.CSparse(64, 64, 10, 0x200000, 0x300000, 0x400000)) == "QLR_ERR_SHAPE"
    assert call(qlr.CSparse(64, 128, 10, 0x200000, 0, 0x400000)) == "QLR_ERR_NULL"
    assert call(qlr.CSparse(64, 128, 10, 0x200000, 0x300000, 0x400004)) == "QLR_ERR_ALIGN"
    assert call(good, ws=0) == "QLR_ERR_WORKSPACE"
    assert call(good, wsb=256) == "QLR_ERR_WORKSPACE"
    assert call(good, M=0, ws=0, wsb=0) == "QLR_OK"
    wide = _qw(rows=64, cols=65536)
    assert qlr.STATUS[lib.qlr_linear_fwd_wha(0x600000, qlr.QLR_BF16, 4, C.byref(wide), C.byref(
        qlr.CSparse(64, 65536, 10, 0x200000, 0x300000, 0x400000)), 65536, 0x700000, qlr.QLR_F32, 0x900000, 1 << 24,
        None)] == "QLR_ERR_SHAPE"  # the transform holds x rows in LDS: cols <= 32768
    # workspace: the M x N float32 branch term
    assert qlr.workspace_bytes(qlr.OP_LINEAR_WHA, 2048, 4096, 4096) == 2048 * 4096 * 4
    assert qlr.workspace_bytes(qlr.OP_LINEAR_WHA, 1, 4096, 4096) == 4096 * 4


def test_static_forward_rejects_oversized_calls():
    """qlr_linear_fwd_static refuses, before touching a device, a call whose scratch exceeds its static
    area (the pointers are never dereferenced: the size check comes first)."""
    lib = qlr.lib()
    fake = 1 << 20  # a 16-byte aligned non-null address
    cw = qlr.CQWeight(qlr.FORMAT_VERSION, 4, qlr.BLOCK, qlr.GROUP, 4096, 4096, fake, fake, fake)
    M, r = 20000, 128
    assert qlr.workspace_bytes(qlr.OP_LINEAR, M, 4096, 4096, r) > qlr.STATIC_SCRATCH_BYTES
    st = lib.qlr_linear_fwd_static(fake, qlr.QLR_BF16, M, C.byref(cw), fake, fake, qlr.QLR_BF16, r, 0.125, fake,
                                   qlr.QLR_BF16, None)
    assert qlr.STATUS[st] == "QLR_ERR_WORKSPACE"
    assert b"static area" in lib.qlr_last_error()
