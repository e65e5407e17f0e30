"""GPU parity of the double-binary adapter branch (qlr_linear_fwd_dba) against the oracle.

Per element |y - y_ref| <= 1e-3 S + 1e-5 (plus half a bf16 ulp for bf16 y), S the
magnitude sum of the base and the branch terms (oracle.dba.linear_dba_tolerance).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import dev, f32_of
from oracle import dba as odba

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from quantized_base_fine_amd import qlr  # noqa: E402

PATHS = {"gemv": qlr.PATH_GEMV, "gemm": qlr.PATH_GEMM, "f32": qlr.PATH_F32, "auto": qlr.PATH_AUTO}


def _wdeq(lin):
    q = oracle.quantize(lin.W.reshape(-1), lin.wdtype, lin.bits)
    return oracle.dequantize(q.codes, q.absmax_q8, q.absmax_c, lin.bits, lin.W.size).reshape(lin.W.shape)


def _run(lin, ad, qw, ydt="f32", path=qlr.PATH_AUTO):
    x = dev(lin.x, lin.xdtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to("cuda")
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    print(f"dba {lin.name} N={lin.N} K={lin.K} M={lin.M} bits={lin.bits} R={ad.R} l={ad.ell} path={path} y={ydt}",
          flush=True)
    with qlr.path(path):
        y = qlr.linear_dba(x, qw, t(ad.b1), t(ad.b2), h(ad.alpha), h(ad.beta), h(ad.gamma),
                           out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    return f32_of(y)


def _check(y, lin, ad, wd, ydt="f32", ms=None):
    x = lin.x if ms is None else lin.x[ms]
    args = (ad.alpha.astype(np.float64), ad.beta.astype(np.float64), ad.gamma.astype(np.float64), ad.b1, ad.b2)
    ref = odba.linear_dba(x, lin.xdtype, wd, *args)
    S = odba.linear_dba_tolerance(x, lin.xdtype, wd, *args)
    bound = 1e-3 * S + 1e-5 + (np.abs(ref) * 2.0 ** -8 if ydt == "bf16" else 0.0)
    got = (y if ms is None else y[ms]).astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"max err/bound {float(np.max(err / bound)):.3f}"


def _small(N, K, M, bits, seed, xdtype="bf16"):
    return workloads.make_linear(f"d{seed}", 90 + seed, N, K, M, sigma=0.02, wdtype="f16", bits=bits, r=0,
                                 alpha=16.0, abdtype="bf16", xdtype=xdtype)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 5), ("gemm", 40), ("gemm", 300), ("f32", 3)])
@pytest.mark.parametrize("R,ell", [(16, 1), (8, 2), (5, 1), (64, 1)])
def test_dba_paths_small(bits, path, M, R, ell):
    """Ragged N = 333, K = 640, every kernel family, bits, rank and envelope rank."""
    lin = _small(333, 640, M, bits, seed=bits + M + R + ell)
    ad = workloads.dba_adapter(lin.N, lin.K, R, ell, cfg=90, sub=bits + M)
    qw = qlr.quantize(dev(lin.W, "f16"), bits)
    wd = _wdeq(lin)
    for ydt in ("f32", "bf16"):
        _check(_run(lin, ad, qw, ydt, PATHS[path]), lin, ad, wd, ydt)


def test_dba_tiny_fp32():
    lin = workloads.tiny()
    ad = workloads.dba_adapter(lin.N, lin.K, 16, 1, cfg=1)
    qw = qlr.quantize(dev(lin.W, "f32"), 4)
    _check(_run(lin, ad, qw), lin, ad, _wdeq(lin))


def test_dba_attn_full():
    """4096x4096 with outliers, R = 16, l = 1: M = 1 (decode) and M = 2048 (prefill), every output."""
    base = workloads.attn(1)
    ad = workloads.dba_adapter(4096, 4096, 16, 1, cfg=2)
    qw = qlr.quantize(dev(base.W, "f16"), 4)
    wd = _wdeq(base)
    for M in (1, 2048):
        lin = workloads.attn(M, W=base.W)
        _check(_run(lin, ad, qw, "bf16"), lin, ad, wd, "bf16")


def test_dba_zero_alpha_is_the_base_and_repeats_are_identical():
    lin = _small(128, 256, 20, 4, seed=3)
    ad = workloads.dba_adapter(lin.N, lin.K, 16, 1, cfg=93)
    qw = qlr.quantize(dev(lin.W, "f16"), 4)
    x = dev(lin.x, "bf16")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to("cuda")
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    for p in (qlr.PATH_GEMV, qlr.PATH_GEMM, qlr.PATH_F32):
        with qlr.path(p):
            xx = x[:1] if p == qlr.PATH_GEMV else x
            base = qlr.linear(xx, qw, out_dtype=torch.float32)
            z = qlr.linear_dba(xx, qw, t(ad.b1), t(ad.b2), torch.zeros_like(h(ad.alpha)), h(ad.beta), h(ad.gamma),
                               out_dtype=torch.float32)
            y1 = qlr.linear_dba(xx, qw, t(ad.b1), t(ad.b2), h(ad.alpha), h(ad.beta), h(ad.gamma),
                                out_dtype=torch.float32)
            y2 = qlr.linear_dba(xx, qw, t(ad.b1), t(ad.b2), h(ad.alpha), h(ad.beta), h(ad.gamma),
                                out_dtype=torch.float32)
            e = qlr.linear_dba(x[:0], qw, t(ad.b1), t(ad.b2), h(ad.alpha), h(ad.beta), h(ad.gamma),
                               out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(base, z)
        assert torch.equal(y1, y2)
        assert e.shape == (0, 128)
