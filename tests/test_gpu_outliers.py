"""GPU parity of the hybrid outlier split (qlr_quantize_outliers, qlr_linear_fwd_outliers).

Quantize: the dense part's codes, 8-bit scale codes and float32 group steps, and
the CSR side channel (row offsets, columns, float32 residuals) are compared bit
for bit with the oracle.  Forward: per element |y - y_ref| <= rel S + 1e-5
(plus half a bf16 ulp for bf16 y), S the magnitude sum of the base and sparse
terms (the scale the other forward tests use, plus the outliers), rel the
kernel family's bound: 1e-3 for the decode and float32 families, 5e-3 for the
prefill GEMM family, whose bf16 weights (outliers added, with 2- and 4-bit
codes) are rounded once more.  Calls go through the C ABI via the binding.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import dev, f32_of
from oracle import outliers as ool

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from quantized_base_fine_amd import qlr  # noqa: E402

PATHS = {"gemv": qlr.PATH_GEMV, "gemm": qlr.PATH_GEMM, "f32": qlr.PATH_F32, "auto": qlr.PATH_AUTO}
GEMM_REL = 5e-3


def _rel(path, M):
    """The bound's relative term of the kernel family a call runs on (auto: M > 16 is the prefill GEMM)."""
    return GEMM_REL if path == qlr.PATH_GEMM or (path == qlr.PATH_AUTO and M > 16) else 1e-3


def _gpu_split(W, wdtype, bits, k):
    print(f"outlier split {W.shape} {wdtype} bits={bits} k={k}", flush=True)
    qw, sp = qlr.quantize_outliers(dev(W, wdtype), bits, k)
    torch.cuda.synchronize()
    return qw, sp


def _check_split(W, wdtype, bits, k, qw, sp):
    rows, cols = W.shape
    q, (row_ptr, col, val) = ool.quantize_with_outliers(W, wdtype, bits, rows, cols, k)
    assert np.array_equal(qw.codes.cpu().numpy(), q.codes), "dense codes differ"
    assert np.array_equal(qw.absmax_q8.cpu().numpy(), q.absmax_q8), "scale codes differ"
    assert np.array_equal(qw.absmax_c.cpu().numpy().view(np.uint32), q.absmax_c.view(np.uint32)), "steps differ"
    assert np.array_equal(sp.row_ptr.cpu().numpy(), row_ptr), "row offsets differ"
    assert np.array_equal(sp.col.cpu().numpy()[:k], col), "columns differ"
    assert np.array_equal(sp.val.cpu().numpy()[:k].view(np.uint32), val.view(np.uint32)), "residuals differ"
    assert sp.max_group_nnz == _max_group_nnz(row_ptr), "largest 128-row group count differs"
    return q, (row_ptr, col, val)


def _max_group_nnz(row_ptr):
    """The largest entry count of the row groups [128 g, 128 g + 128) of a CSR (host)."""
    rows = len(row_ptr) - 1
    edges = np.append(np.arange(0, rows, 128), rows)
    return int(np.max(np.diff(row_ptr[edges]))) if rows > 0 else 0


def _ties(seed, rows, cols, dtype):
    """Weights in {-1.5, -1, ..., 1.5}: |w| has four classes, so the k-th largest key
    is shared by thousands of entries spread over every 4096-element block."""
    rng = np.random.default_rng(seed)
    w = (rng.integers(-3, 4, size=(rows, cols)) * 0.5).astype(np.float32)
    return workloads.store(w, dtype)


@pytest.mark.parametrize("k", [0, 1, 5, 1000, 37 * 111])
def test_split_small_every_k(k):
    """37 x 111 float32 (a ragged last 64-block and a ragged 4096-element block), k up to every entry."""
    W = workloads.make_weight(300, 37, 111, 0.02, "f32", outlier_frac=0.01)
    _check_split(W, "f32", 4, k, *_gpu_split(W, "f32", 4, k))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("wdtype", ["f16", "bf16"])
def test_split_bits_and_dtypes(bits, wdtype):
    """300 x 1000 with 1 % planted x20 outliers and k = that count (74 selection blocks)."""
    W = workloads.make_weight(301, 300, 1000, 0.02, wdtype, outlier_frac=0.01)
    k = int(round(0.01 * W.size))
    _check_split(W, wdtype, bits, k, *_gpu_split(W, wdtype, bits, k))


@pytest.mark.parametrize("k", [17000, 20000, 34000, 60000])
def test_split_ties_across_blocks(k):
    """200 x 300 with four |w| classes: ties at the threshold are taken in flat index order."""
    W = _ties(5, 200, 300, "f32")
    n15 = int(np.sum(np.abs(W) == 1.5))
    for kk in (k, n15):  # also a k that ends exactly at a class boundary
        _check_split(W, "f32", 4, kk, *_gpu_split(W, "f32", 4, kk))


def test_split_attn_full():
    """4096 x 4096 fp16 attention weight, k = its 0.1 % planted outliers: every byte."""
    lin = workloads.attn(1)
    k = int(round(0.001 * lin.W.size))
    _check_split(lin.W, lin.wdtype, 4, k, *_gpu_split(lin.W, lin.wdtype, 4, k))


def test_split_zero_k_equals_plain_quantize_and_is_deterministic():
    W = workloads.make_weight(302, 96, 640, 0.02, "f16", outlier_frac=0.01)
    qa, sa = _gpu_split(W, "f16", 4, 0)
    qp = qlr.quantize(dev(W, "f16"), 4)
    torch.cuda.synchronize()
    assert torch.equal(qa.codes, qp.codes) and torch.equal(qa.absmax_q8, qp.absmax_q8)
    assert torch.equal(qa.absmax_c, qp.absmax_c) and not sa.row_ptr.any()
    k = 700
    a, b = _gpu_split(W, "f16", 4, k), _gpu_split(W, "f16", 4, k)
    for x, y in ((a[0].codes, b[0].codes), (a[1].row_ptr, b[1].row_ptr), (a[1].col[:k], b[1].col[:k]),
                 (a[1].val[:k], b[1].val[:k])):
        assert torch.equal(x, y)


def test_split_nonfinite_is_an_error():
    W = workloads.make_weight(303, 64, 128, 0.02, "f32")
    W[3, 5] = np.nan
    with pytest.raises(qlr.QlrError) as e:
        _gpu_split(W, "f32", 4, 10)
    assert e.value.name == "QLR_ERR_NONFINITE"


# ---------------------------------------------------------------- forward


def _layer(N, K, M, r, seed, xdtype="bf16", abdtype="bf16", frac=0.01):
    lin = workloads.make_linear(f"o{seed}", 310 + seed, N, K, M, sigma=0.02, wdtype="f16", bits=4, r=r,
                                alpha=16.0, abdtype=abdtype, xdtype=xdtype, outlier_frac=frac)
    return lin, int(round(frac * N * K))


def _run(lin, qw, sp, ydt="f32", path=qlr.PATH_AUTO, x=None):
    x = lin.x if x is None else x
    xd = dev(x, lin.xdtype)
    A = dev(lin.A, lin.abdtype) if lin.r > 0 else None
    B = dev(lin.B, lin.abdtype) if lin.r > 0 else None
    print(f"outliers fwd {lin.name} N={lin.N} K={lin.K} M={x.shape[0]} r={lin.r} nnz={sp.nnz} path={path} "
          f"y={ydt}", flush=True)
    with qlr.path(path):
        y = qlr.linear_outliers(xd, qw, sp, A, B, lin.scale,
                                out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    return f32_of(y)


def _check_fwd(y, lin, q, csr, ydt="f32", x=None, rel=1e-3):
    x = lin.x if x is None else x
    wd = oracle.dequantize(q.codes, q.absmax_q8, q.absmax_c, lin.bits, lin.W.size).reshape(lin.W.shape)
    A, B = (lin.A, lin.B) if lin.r > 0 else (None, None)
    ref = ool.linear_outliers(x, lin.xdtype, wd, csr, A, B, lin.abdtype, lin.scale)
    S = ool.linear_outliers_tolerance(x, lin.xdtype, wd, csr)
    bound = rel * S + 1e-5 + (np.abs(ref) * 2.0 ** -8 if ydt == "bf16" else 0.0)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(np.isfinite(y))
    assert np.all(err <= bound), f"max err/bound {float(np.max(err / bound)):.3f}"


@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 5), ("gemv", 16), ("gemm", 40), ("gemm", 300),
                                    ("f32", 3), ("f32", 20), ("auto", 2)])
@pytest.mark.parametrize("r", [0, 16])
def test_fwd_paths_small(path, M, r):
    """320 x 576 (5 row steps, a partial 128-column tile), 1 % outliers, every path."""
    lin, k = _layer(320, 576, M, r, seed=M + r)
    qw, sp = _gpu_split(lin.W, lin.wdtype, lin.bits, k)
    q, csr = ool.quantize_with_outliers(lin.W, lin.wdtype, lin.bits, lin.N, lin.K, k)
    for ydt in ("f32", "bf16"):
        _check_fwd(_run(lin, qw, sp, ydt, PATHS[path]), lin, q, csr, ydt, rel=_rel(PATHS[path], M))


@pytest.mark.parametrize("path,M", [("gemm", 3), ("f32", 2), ("gemv", 1)])
def test_fwd_long_rows(path, M):
    """K = 33280: rows of x too long to stage in LDS (the sparse term reads x from memory)."""
    lin, k = _layer(64, 33280, M, 8, seed=40 + M)
    qw, sp = _gpu_split(lin.W, lin.wdtype, lin.bits, k)
    q, csr = ool.quantize_with_outliers(lin.W, lin.wdtype, lin.bits, lin.N, lin.K, k)
    _check_fwd(_run(lin, qw, sp, "f32", PATHS[path]), lin, q, csr, rel=_rel(PATHS[path], M))


@pytest.mark.parametrize("r", [0, 16])
def test_fwd_decode_two_tiles_per_workgroup(r):
    """N = 8192, K = 512, M = 1: 512 row tiles of the decode kernel on 256 workgroups (the side
    channel of a workgroup's second tile is loaded at its end); 1 % outliers, so many rows hold
    more than 4."""
    lin, k = _layer(8192, 512, 1, r, seed=70 + r)
    qw, sp = _gpu_split(lin.W, lin.wdtype, lin.bits, k)
    q, csr = ool.quantize_with_outliers(lin.W, lin.wdtype, lin.bits, lin.N, lin.K, k)
    assert np.max(np.diff(csr[0])) > 4
    for ydt in ("f32", "bf16"):
        _check_fwd(_run(lin, qw, sp, ydt, qlr.PATH_GEMV), lin, q, csr, ydt)


@pytest.mark.parametrize("M", [40, 300])
def test_fwd_gemm_ragged_columns(M):
    """N = 330 (output rows not a multiple of 4: the scalar stores of the prefill kernel)."""
    lin, k = _layer(330, 576, M, 16, seed=80 + M)
    qw, sp = _gpu_split(lin.W, lin.wdtype, lin.bits, k)
    q, csr = ool.quantize_with_outliers(lin.W, lin.wdtype, lin.bits, lin.N, lin.K, k)
    for ydt in ("f32", "bf16"):
        _check_fwd(_run(lin, qw, sp, ydt, qlr.PATH_GEMM), lin, q, csr, ydt, rel=GEMM_REL)


def test_fwd_f32_inputs():
    """float32 x and adapters (the float32 family) with outliers."""
    lin, k = _layer(128, 256, 7, 4, seed=50, xdtype="f32", abdtype="f32")
    qw, sp = _gpu_split(lin.W, lin.wdtype, lin.bits, k)
    q, csr = ool.quantize_with_outliers(lin.W, lin.wdtype, lin.bits, lin.N, lin.K, k)
    _check_fwd(_run(lin, qw, sp), lin, q, csr)


def test_fwd_attn_full():
    """4096 x 4096, r16, k = the 0.1 % planted outliers: M = 2048 and M = 1, every output."""
    base = workloads.attn(1)
    k = int(round(0.001 * base.W.size))
    qw, sp = _gpu_split(base.W, base.wdtype, base.bits, k)
    q, csr = ool.quantize_with_outliers(base.W, base.wdtype, base.bits, base.N, base.K, k)
    for M in (2048, 1):
        lin = workloads.attn(M, W=base.W)
        _check_fwd(_run(lin, qw, sp, "bf16"), lin, q, csr, "bf16", rel=_rel(qlr.PATH_AUTO, M))


def test_fwd_zero_nnz_equals_plain_and_empty_batch():
    lin, _ = _layer(192, 512, 40, 16, seed=60)
    qw, sp = _gpu_split(lin.W, lin.wdtype, lin.bits, 0)
    x, A, B = dev(lin.x, "bf16"), dev(lin.A, "bf16"), dev(lin.B, "bf16")
    for p in (qlr.PATH_GEMM, qlr.PATH_F32):
        with qlr.path(p):
            y0 = qlr.linear_outliers(x, qw, sp, A, B, lin.scale, out_dtype=torch.float32)
            yp = qlr.linear(x, qw, A, B, lin.scale, out_dtype=torch.float32)
            e = qlr.linear_outliers(x[:0], qw, sp, A, B, lin.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y0, yp) and e.shape == (0, 192)


def test_fwd_graph_replays_match_eager():
    """The forward with outliers captured in a HIP graph, replayed with eager work between replays."""
    lin, k = _layer(256, 512, 300, 16, seed=61)
    qw, sp = _gpu_split(lin.W, lin.wdtype, lin.bits, k)
    x, A, B = dev(lin.x, "bf16"), dev(lin.A, "bf16"), dev(lin.B, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call = qlr.OutliersCall(x, qw, sp, A, B, lin.scale, out_dtype=torch.float32)
        ref = call().clone()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call()
    for i in range(4):
        call.y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.y, ref), i
        _ = (x.float() * 2).sum().item()


@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 5), ("gemm", 40), ("f32", 3)])
def test_fwd_wide_rows(path, M):
    """K = 11008 (the 7B-class down projection's width), 1 % outliers."""
    lin, k = _layer(256, 11008, M, 16, seed=120 + M)
    qw, sp = _gpu_split(lin.W, lin.wdtype, lin.bits, k)
    q, csr = ool.quantize_with_outliers(lin.W, lin.wdtype, lin.bits, lin.N, lin.K, k)
    _check_fwd(_run(lin, qw, sp, "f32", PATHS[path]), lin, q, csr, rel=_rel(PATHS[path], M))


def _csr_per_tile(N, K, counts, seed):
    """CSR (row_ptr, col, val) with counts[t] entries in rows [128 t, 128 t + 128), spread over the rows,
    columns distinct and ascending within a row, residuals ~ N(0, 0.2^2)."""
    rng = np.random.default_rng(seed)
    per_row = np.zeros(N, dtype=np.int64)
    for t, c in enumerate(counts):
        rows = np.arange(128 * t, min(N, 128 * t + 128))
        per_row[rows] = c // len(rows)
        per_row[rows[: c % len(rows)]] += 1
    row_ptr = np.concatenate([[0], np.cumsum(per_row)]).astype(np.int32)
    col = np.concatenate([np.sort(rng.choice(K, size=int(n), replace=False)) for n in per_row]).astype(np.int32)
    val = (rng.standard_normal(int(row_ptr[-1])) * 0.2).astype(np.float32)
    return row_ptr, col, val


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_fwd_gemm_tiles_fused_and_not(bits):
    """Prefill GEMM, 384 x 576, M = 300, r 16: the first 128-row tile holds 3000 entries (more than the
    kernel adds to its weights itself: the float32 term covers it), the second 400 (added to the
    weights with 2- and 4-bit codes), the third none; every output against the oracle."""
    N, K, M = 384, 576, 300
    lin = workloads.make_linear("otile", 390 + bits, N, K, M, sigma=0.02, wdtype="f16", bits=bits, r=16,
                                alpha=16.0, abdtype="bf16", xdtype="bf16")
    csr = _csr_per_tile(N, K, [3000, 400, 0], seed=bits)
    qw = qlr.quantize(dev(lin.W, "f16"), bits)
    sp = qlr.sparse_from_csr(N, K, *csr, "cuda")
    q = oracle.quantize(lin.W.reshape(-1), "f16", bits)
    for ydt in ("f32", "bf16"):
        _check_fwd(_run(lin, qw, sp, ydt, qlr.PATH_GEMM), lin, q, csr, ydt, rel=GEMM_REL)


@pytest.mark.parametrize("counts", [[400, 300, 0], [3000, 400, 0]])
def test_fwd_gemm_group_count_skips_addend(counts):
    """Prefill GEMM with 4-bit codes, 384 x 576, M = 300, r 16: with sp.max_group_nnz exact the addend
    kernel is skipped when every 128-row tile's entries fit (400 here) and launched when one does not
    (3000); both agree bit for bit with the same call with the count unknown (-1, the addend kernel
    always launched), and with the oracle."""
    N, K, M = 384, 576, 300
    lin = workloads.make_linear("ogrp", 420 + counts[0], N, K, M, sigma=0.02, wdtype="f16", bits=4, r=16,
                                alpha=16.0, abdtype="bf16", xdtype="bf16")
    csr = _csr_per_tile(N, K, counts, seed=counts[0])
    qw = qlr.quantize(dev(lin.W, "f16"), 4)
    q = oracle.quantize(lin.W.reshape(-1), "f16", 4)
    sp = qlr.sparse_from_csr(N, K, *csr, "cuda")
    assert sp.max_group_nnz == -1
    y_unknown = _run(lin, qw, sp, "f32", qlr.PATH_GEMM)
    sp.max_group_nnz = _max_group_nnz(csr[0])
    assert sp.max_group_nnz == max(counts)
    y_known = _run(lin, qw, sp, "f32", qlr.PATH_GEMM)
    assert np.array_equal(y_known.view(np.uint32), y_unknown.view(np.uint32))
    _check_fwd(y_known, lin, q, csr, rel=GEMM_REL)


def test_split_group_count_on_the_attn_split():
    """The split of the 4096 x 4096 attention weight (k = 16,777): its group count is exact, fits the
    GEMM's tiles (so the prefill forward launches no addend kernel), and the forward agrees bit for bit
    with the same call with the count unknown."""
    base = workloads.attn(1)
    k = int(round(0.001 * base.W.size))
    qw, sp = _gpu_split(base.W, "f16", 4, k)
    row_ptr = sp.row_ptr.cpu().numpy()
    assert sp.max_group_nnz == _max_group_nnz(row_ptr)
    assert 0 < sp.max_group_nnz <= 1982
    lin = workloads.attn(300, W=base.W)
    y_known = _run(lin, qw, sp, "bf16", qlr.PATH_GEMM)
    sp.max_group_nnz = -1
    y_unknown = _run(lin, qw, sp, "bf16", qlr.PATH_GEMM)
    assert np.array_equal(y_known.view(np.uint32), y_unknown.view(np.uint32))
