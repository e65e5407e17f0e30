"""GPU parity of the Walsh-Hadamard adapter branch (qlr_linear_fwd_wha) against the oracle.

Per element |y - y_ref| <= rel S + 1e-5 (plus half a bf16 ulp for bf16 y), S the
magnitude sum of the base terms and of every product c_j x_k H[k][j] / P that
defines the branch (oracle.wha.linear_wht_tolerance): rel = 1e-3 on the decode
and float32 families, and on the prefill GEMM family (bf16 x, M > 16) the 5e-3
that family states for its bf16 weights, which there hold W' + F H / P rounded
to bf16.  Calls go through the C ABI.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import dev, f32_of
from oracle import wha as owha

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from quantized_base_fine_amd import qlr  # noqa: E402

PATHS = {"gemv": qlr.PATH_GEMV, "gemm": qlr.PATH_GEMM, "f32": qlr.PATH_F32, "auto": qlr.PATH_AUTO}
GEMM_REL = 5e-3


def _rel(path, M, xdtype="bf16"):
    """The bound's relative term for the kernel family a call runs on."""
    gemm = path == qlr.PATH_GEMM or (path == qlr.PATH_AUTO and M > 16 and xdtype == "bf16")
    return GEMM_REL if gemm else 1e-3


def _wdeq(lin):
    q = oracle.quantize(lin.W.reshape(-1), lin.wdtype, lin.bits)
    return oracle.dequantize(q.codes, q.absmax_q8, q.absmax_c, lin.bits, lin.W.size).reshape(lin.W.shape)


def _layer(N, K, M, seed, bits=4, xdtype="bf16"):
    return workloads.make_linear(f"h{seed}", 400 + seed, N, K, M, sigma=0.02, wdtype="f16", bits=bits, r=0,
                                 alpha=16.0, abdtype="bf16", xdtype=xdtype)


def _coeffs(lin, per_row, floor, seed):
    return workloads.wha_coefficients(lin.N, lin.K, per_row * lin.N, cfg=410 + seed, floor=floor)


def _run(lin, qw, F, P, ydt="f32", path=qlr.PATH_AUTO, x=None):
    x = lin.x if x is None else x
    print(f"wha {lin.name} N={lin.N} K={lin.K} M={x.shape[0]} bits={lin.bits} P={P} nnz={F.nnz} path={path} "
          f"y={ydt}", flush=True)
    with qlr.path(path):
        y = qlr.linear_wha(dev(x, lin.xdtype), qw, F, P,
                           out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    return f32_of(y)


def _check(y, lin, wd, csr, P, ydt="f32", x=None, path=qlr.PATH_AUTO):
    """path: the one y was computed on (it sets the bound's relative term)."""
    x = lin.x if x is None else x
    rel = _rel(path, x.shape[0], lin.xdtype)
    ref = owha.linear_wht(x, lin.xdtype, wd, csr, P)
    S = owha.linear_wht_tolerance(x, lin.xdtype, wd, csr, P)
    bound = rel * S + 1e-5 + (np.abs(ref) * 2.0 ** -8 if ydt == "bf16" else 0.0)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(np.isfinite(y))
    assert np.all(err <= bound), f"max err/bound {float(np.max(err / bound)):.3f}"


def _prep(lin, per_row=32, floor=8, seed=0):
    qw = qlr.quantize(dev(lin.W, lin.wdtype), lin.bits)
    csr = _coeffs(lin, per_row, floor, seed)
    F = qlr.sparse_from_csr(lin.N, lin.K, *csr, "cuda")
    torch.cuda.synchronize()
    return qw, csr, F


@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 5), ("gemv", 16), ("gemm", 40), ("gemm", 300),
                                    ("f32", 3), ("f32", 20), ("auto", 2)])
@pytest.mark.parametrize("P", [512, 64, 1])
def test_wha_paths_small(path, M, P):
    """N = 320, K = 512; P = the full width, blocks of 64, and the degenerate P = 1 (z = x)."""
    lin = _layer(320, 512, M, seed=M + P)
    qw, csr, F = _prep(lin, seed=M)
    wd = _wdeq(lin)
    for ydt in ("f32", "bf16"):
        _check(_run(lin, qw, F, P, ydt, PATHS[path]), lin, wd, csr, P, ydt, path=PATHS[path])


@pytest.mark.parametrize("bits", [2, 3, 8])
@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemm", 100)])
def test_wha_bits(bits, path, M):
    """The other code widths, K = 576 = 64 x 9 (blocks of 64)."""
    lin = _layer(192, 576, M, seed=20 + bits + M, bits=bits)
    qw, csr, F = _prep(lin, seed=bits)
    _check(_run(lin, qw, F, 64, "f32", PATHS[path]), lin, _wdeq(lin), csr, 64, path=PATHS[path])


@pytest.mark.parametrize("M", [1, 9])
def test_wha_f32_inputs_and_uneven_rows(M):
    """float32 x (the float32 family); a skewed allocation (floor 1, some rows with hundreds)."""
    lin = _layer(256, 1024, M, seed=30 + M, xdtype="f32")
    qw, csr, F = _prep(lin, per_row=48, floor=1, seed=3)
    assert np.diff(csr[0]).max() > 4 * 48
    _check(_run(lin, qw, F, 1024), lin, _wdeq(lin), csr, 1024)


def test_wha_attn_full():
    """4096 x 4096, P = 4096, 131072 coefficients (the parameter count of a rank-16 adapter):
    M = 2048 and M = 1, every output."""
    base = workloads.attn(1)
    qw = qlr.quantize(dev(base.W, base.wdtype), base.bits)
    csr = workloads.wha_coefficients(4096, 4096, 16 * (4096 + 4096), cfg=2, floor=8)
    F = qlr.sparse_from_csr(4096, 4096, *csr, "cuda")
    wd = _wdeq(base)
    for M in (2048, 1):
        lin = workloads.attn(M, W=base.W)
        _check(_run(lin, qw, F, 4096, "bf16"), lin, wd, csr, 4096, "bf16")


def test_wha_edge_cases():
    lin = _layer(128, 256, 40, seed=50)
    qw, csr, F = _prep(lin, per_row=8, floor=2, seed=5)
    empty = qlr.sparse_from_csr(128, 256, np.zeros(129, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32),
                                "cuda")
    x = dev(lin.x, "bf16")
    for p in (qlr.PATH_GEMM, qlr.PATH_F32):
        with qlr.path(p):
            y0 = qlr.linear_wha(x, qw, empty, 256, out_dtype=torch.float32)      # no coefficients
            yp = qlr.linear(x, qw, out_dtype=torch.float32)
            a = qlr.linear_wha(x, qw, F, 256, out_dtype=torch.float32)
            b = qlr.linear_wha(x, qw, F, 256, out_dtype=torch.float32)
            e = qlr.linear_wha(x[:0], qw, F, 256, out_dtype=torch.float32)      # M = 0
        torch.cuda.synchronize()
        assert torch.equal(y0, yp) and torch.equal(a, b) and e.shape == (0, 128)
    with pytest.raises(qlr.QlrError):
        qlr.linear_wha(x, qw, F, 96)  # not a power of two


def test_wha_graph_replays_match_eager():
    lin = _layer(256, 512, 300, seed=60)
    qw, csr, F = _prep(lin, seed=6)
    x = dev(lin.x, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call = qlr.WhaCall(x, qw, F, 512, out_dtype=torch.float32)
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
def test_wha_wide_blocked(path, M):
    """K = 11008 = 2^8 x 43 with blocks of 256 (three x pieces per thread on the decode kernel)."""
    lin = _layer(256, 11008, M, seed=90 + M)
    qw, csr, F = _prep(lin, per_row=64, floor=8, seed=9)
    _check(_run(lin, qw, F, 256, "f32", PATHS[path]), lin, _wdeq(lin), csr, 256, path=PATHS[path])


@pytest.mark.parametrize("K,M", [(8192, 1), (8192, 40), (16384, 1)])
def test_wha_wide_full_transform(K, M):
    """One full transform over K = 8192 (two LDS rounds for bits 9-12 on the decode kernel) and
    K = 16384 (no room for the transform beside the decode kernel's tables: the separate kernel)."""
    lin = _layer(192, K, M, seed=100 + M + K // 1024)
    qw, csr, F = _prep(lin, per_row=48, floor=8, seed=10)
    _check(_run(lin, qw, F, K, "f32"), lin, _wdeq(lin), csr, K)


@pytest.mark.parametrize("nnz", [1, 3, 4, 5, 37])
def test_wha_few_coefficients(nnz):
    """A handful of coefficients in the last rows: fewer than 4 (one 4-byte load each), exactly 4 and just
    above (16-byte loads clamped to the array's end, elements before the lane's own skipped)."""
    lin = _layer(96, 256, 24, seed=70 + nnz)
    qw = qlr.quantize(dev(lin.W, lin.wdtype), lin.bits)
    rng = np.random.default_rng(700 + nnz)
    rows = np.sort(rng.choice(np.arange(90, 96), size=nnz))
    row_ptr = np.searchsorted(rows, np.arange(97)).astype(np.int32)
    col = rng.integers(0, 256, nnz).astype(np.int32)
    val = rng.standard_normal(nnz).astype(np.float32)
    csr = (row_ptr, col, val)
    F = qlr.sparse_from_csr(96, 256, *csr, "cuda")
    wd = _wdeq(lin)
    for path in ("gemm", "f32"):
        _check(_run(lin, qw, F, 64, "f32", PATHS[path]), lin, wd, csr, 64, path=PATHS[path])


@pytest.mark.parametrize("N,K,P,M", [(200, 32768, 32768, 40), (130, 4096, 16, 257), (136, 1024, 1024, 17)])
def test_wha_prefill_merged_weight(N, K, P, M):
    """The prefill GEMM with the branch merged into a bf16 copy of the weight: the widest rows (K = 32768,
    one transform over all of them), short blocks (P = 16: one butterfly pass of four stages), weight
    rows that end inside a 128-row tile, M just past the decode sizes and one row past a 256-row tile;
    rows with repeated columns add their coefficients."""
    lin = _layer(N, K, M, seed=110 + P)
    qw = qlr.quantize(dev(lin.W, lin.wdtype), lin.bits)
    row_ptr, col, val = _coeffs(lin, 24, 4, seed=11)
    col = col.copy()
    col[1] = col[0]  # a repeated column in row 0
    csr = (row_ptr, col, val)
    F = qlr.sparse_from_csr(N, K, *csr, "cuda")
    wd = _wdeq(lin)
    for ydt in ("f32", "bf16"):
        _check(_run(lin, qw, F, P, ydt, qlr.PATH_GEMM), lin, wd, csr, P, ydt, path=qlr.PATH_GEMM)
