"""GPU parity of the backward (adapter training): dx, dA, dB against the CPU oracle.

Per element |g - g_ref| <= 1e-3 S + 1e-5 with S the magnitude sum of the terms
that define g (plus half a bf16 ulp for a bf16 dx).  Calls go through the C ABI
(qlr_linear_bwd) via the binding.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import check_backward, dev, f32_of

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from quantized_base_fine_amd import qlr  # noqa: E402

BITS = [2, 3, 4, 8]
PATHS = {"gemm": qlr.PATH_GEMM, "f32": qlr.PATH_F32, "auto": qlr.PATH_AUTO}


def _quant(lin):
    Wd = dev(lin.W, lin.wdtype)
    qw = qlr.quantize(Wd, lin.bits)
    torch.cuda.synchronize()
    return qw


def _wdeq(lin, cols=None):
    q = oracle.quantize(lin.W.reshape(-1), lin.wdtype, lin.bits)
    w = oracle.dequantize(q.codes, q.absmax_q8, q.absmax_c, lin.bits, lin.W.size).reshape(lin.W.shape)
    return w if cols is None else np.ascontiguousarray(w[:, cols])


def _run_bwd(lin, qw, dy, dxdt="f32", path=qlr.PATH_AUTO, need_dx=True):
    x = dev(lin.x, lin.xdtype)
    g = dev(dy, lin.xdtype)
    A = dev(lin.A, lin.abdtype) if lin.r > 0 else None
    B = dev(lin.B, lin.abdtype) if lin.r > 0 else None
    odt = torch.float32 if dxdt == "f32" else torch.bfloat16
    print(f"bwd {lin.name} N={lin.N} K={lin.K} M={lin.M} bits={lin.bits} r={lin.r} path={path} dx={dxdt}",
          flush=True)
    with qlr.path(path):
        dx, dA, dB = qlr.linear_bwd(g, x, qw, A, B, lin.scale, dx_dtype=odt, need_dx=need_dx)
    torch.cuda.synchronize()
    return (None if dx is None else f32_of(dx), None if dA is None else f32_of(dA),
            None if dB is None else f32_of(dB))


def _small(N, K, M, bits, r, seed, xdtype="bf16", abdtype="bf16"):
    return workloads.make_linear(f"b{seed}", 70 + seed, N, K, M, sigma=0.02, wdtype="f16", bits=bits,
                                 r=r, alpha=16.0, abdtype=abdtype, xdtype=xdtype)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("path,M", [("gemm", 1), ("gemm", 5), ("gemm", 100), ("gemm", 300), ("f32", 3),
                                    ("f32", 20)])
@pytest.mark.parametrize("r", [0, 4, 16, 72])
def test_bwd_paths_small(bits, path, M, r):
    """N = 320 (5 row steps), K = 576 (a partial 128-column tile), every path, bits and rank."""
    lin = _small(320, 576, M, bits, r, seed=bits + M + r)
    qw = _quant(lin)
    dy = workloads.upstream_grad(lin)
    wd = _wdeq(lin)
    for dxdt in ("f32", "bf16"):
        check_backward(_run_bwd(lin, qw, dy, dxdt, PATHS[path]), lin, dy, wd, dxdt=dxdt)


@pytest.mark.parametrize("M", [2, 40])
def test_bwd_f32_ragged_rows(M):
    """Rows not a multiple of 64 (the float32 family takes any N), bf16 operands."""
    lin = _small(333, 640, M, 4, 8, seed=11 + M)
    qw = _quant(lin)
    dy = workloads.upstream_grad(lin)
    check_backward(_run_bwd(lin, qw, dy), lin, dy, _wdeq(lin))


@pytest.mark.parametrize("path,M", [("gemm", 130), ("gemm", 1), ("f32", 7)])
def test_bwd_long_contraction(path, M):
    """N = 11008 (172 row steps of the transposed GEMM) with K = 256."""
    lin = _small(11008, 256, M, 4, 64, seed=5)
    qw = _quant(lin)
    dy = workloads.upstream_grad(lin)
    check_backward(_run_bwd(lin, qw, dy, "f32", PATHS[path]), lin, dy, _wdeq(lin))


def test_bwd_tiny_config():
    """256x256 fp32 weights, rank-4 fp32 adapters, fp32 x and dy (float32 family)."""
    lin = workloads.tiny()
    qw = _quant(lin)
    dy = workloads.upstream_grad(lin)
    check_backward(_run_bwd(lin, qw, dy), lin, dy, _wdeq(lin))


def test_bwd_attn_full():
    """4096x4096 with outliers, r16: M = 2048 and M = 1, every element of dx, dA, dB."""
    base = workloads.attn(1)
    qw = _quant(base)
    wd = _wdeq(base)
    for M in (2048, 1):
        lin = workloads.attn(M, W=base.W)
        dy = workloads.upstream_grad(lin)
        check_backward(_run_bwd(lin, qw, dy, "bf16"), lin, dy, wd, dxdt="bf16")


@pytest.mark.parametrize("which", ["up", "down"])
def test_bwd_mlp_sampled(which):
    """7B-class MLP projections, r64, M = 2048: sampled dx and dA columns, all of dB."""
    base = workloads.mlp(which, 1)
    qw = _quant(base)
    rng = np.random.default_rng(4)
    ks = sorted(set([0, base.K - 1] + rng.choice(base.K, size=40, replace=False).tolist()))
    wd = _wdeq(base, ks)
    lin = workloads.mlp(which, 2048, W=base.W)
    dy = workloads.upstream_grad(lin)
    check_backward(_run_bwd(lin, qw, dy, "bf16"), lin, dy, wd, ks=ks, dxdt="bf16")


def test_bwd_big65_sampled():
    """65B-class 22016x8192, r64, M = 4096: sampled dx and dA columns, all of dB."""
    base = workloads.big65(1)
    qw = _quant(base)
    rng = np.random.default_rng(6)
    ks = sorted(set([0, base.K - 1] + rng.choice(base.K, size=24, replace=False).tolist()))
    wd = _wdeq(base, ks)
    lin = workloads.big65(4096, W=base.W)
    dy = workloads.upstream_grad(lin)
    check_backward(_run_bwd(lin, qw, dy, "bf16"), lin, dy, wd, ks=ks, dxdt="bf16")


def test_bwd_edge_cases():
    lin = _small(128, 256, 40, 4, 8, seed=9)
    qw = _quant(lin)
    dy = dev(workloads.upstream_grad(lin), "bf16")
    x = dev(lin.x, "bf16")
    A, B = dev(lin.A, "bf16"), dev(lin.B, "bf16")
    for p in (qlr.PATH_GEMM, qlr.PATH_F32):
        with qlr.path(p):
            dx0, _, _ = qlr.linear_bwd(dy, x, qw, dx_dtype=torch.float32)                 # r = 0
            dxb, dAb, dBb = qlr.linear_bwd(dy, x, qw, A, torch.zeros_like(B), 2.0,     # B = 0
                                           dx_dtype=torch.float32)
            g1 = qlr.linear_bwd(dy, x, qw, A, B, lin.scale, dx_dtype=torch.float32)
            g2 = qlr.linear_bwd(dy, x, qw, A, B, lin.scale, dx_dtype=torch.float32)
            nd = qlr.linear_bwd(dy, x, qw, A, B, lin.scale, need_dx=False)             # no dx
            e = qlr.linear_bwd(dy[:0], x[:0], qw, A, B, lin.scale, dx_dtype=torch.float32)  # M = 0
            xz = qlr.linear_bwd(dy, None, qw, dx_dtype=torch.float32)                  # r = 0: x unused
        torch.cuda.synchronize()
        assert torch.equal(dx0, dxb) and torch.equal(dx0, xz[0])
        assert not dAb.any() and dBb.any()
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)  # deterministic: fixed reduction orders, no atomics
        assert nd[0] is None and torch.equal(nd[1], g1[1]) and torch.equal(nd[2], g1[2])
        assert e[0].shape == (0, 256) and not e[1].any() and not e[2].any()


def test_bwd_graph_replays_match_eager():
    """The backward captured in a HIP graph, replayed with eager work and syncs between replays."""
    lin = _small(256, 512, 300, 4, 16, seed=12)
    qw = _quant(lin)
    dy = dev(workloads.upstream_grad(lin), "bf16")
    x = dev(lin.x, "bf16")
    A, B = dev(lin.A, "bf16"), dev(lin.B, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call = qlr.LinearBwdCall(dy, x, qw, A, B, lin.scale, dx_dtype=torch.float32)
        ref = [t.clone() for t in call()]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call()
    for i in range(4):
        for t in (call.dx, call.dA, call.dB):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((call.dx, call.dA, call.dB), ref):
            assert torch.equal(a, b), i
        _ = (x.float() * 2).sum().item()  # eager work between replays
