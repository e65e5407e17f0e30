"""GPU parity of the single-row decode path on x rows at the edges of its fp16 form.

At M = 1 every wave takes a slice of K and, when the slice is exactly
representable that way, multiplies fp16 levels with the slice as fp16 numbers
scaled by a power of two (largest |x| into [2^14, 2^15)); a slice that is not
(a range wider than fp16 holds, a largest |x| below 2^-126, Inf or NaN) is
summed in float32 instead.  These rows put one wave's slice on each side of
that line, and the results must meet the same per-element bound as on any
input: |y - y_ref| <= 1e-3 S + 1e-5 (S = sum_k |x w'|), and for the rows whose
outputs are far below 1e-5, the same bound with 1e-40 in place of 1e-5.
Non-finite x gives the oracle's non-finite outputs.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import dev, f32_of, oracle_rows_dequant

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from quantized_base_fine_amd import qlr  # noqa: E402

N, K = 80, 4096           # 8 waves x 512 columns; N not a multiple of 16
SLICE = K // 8


def _bf16(a):
    return workloads.to_bf16_bits(np.asarray(a, dtype=np.float32))


def x_rows(seed):
    """name -> float32 x row (values exactly bf16)."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal(K).astype(np.float32)
    rows = {}
    rows["normal"] = base.copy()
    w = base.copy()
    w[3] = np.float32(2.0 ** -30)        # wave 0: 2^-30 next to values near 1: below the fp16 range once scaled
    rows["wide"] = w
    # wave 1: values +-1 (scaled by 2^14) and one 2^-28, the smallest that stays a normal fp16 number
    # once scaled; then 2^-29, the largest below
    for name, v in (("edge", 2.0 ** -28), ("edge_below", 2.0 ** -29)):
        w = base.copy()
        w[SLICE:2 * SLICE] = np.where(base[SLICE:2 * SLICE] < 0, -1.0, 1.0)
        w[SLICE + 5] = np.float32(v)
        w[SLICE + 6] = -np.float32(v)
        rows[name] = w
    w = base.copy()
    w[2 * SLICE + 9] = np.float32(3.0e38)  # wave 2: near the top of the bf16 range
    rows["huge"] = w
    rows["tiny"] = (base * np.float32(1e-30)).astype(np.float32)
    w = (base * np.float32(1e-38)).astype(np.float32)   # bf16 subnormals among normal values
    rows["subnormal_mix"] = w
    w = np.zeros(K, dtype=np.float32)
    w[4 * SLICE: 5 * SLICE] = base[:SLICE] * np.float32(2.0 ** -130)  # wave 4: only subnormals
    w[:SLICE] = base[:SLICE]
    rows["subnormal_slice"] = w
    rows["zeros"] = np.zeros(K, dtype=np.float32)
    w = base.copy()
    w[7 * SLICE:] = np.float32(0.0)
    w[7 * SLICE + 1] = -np.float32(0.0)
    rows["zero_slice"] = w
    return {k: oracle.widen(_bf16(v), "bf16").astype(np.float32) for k, v in rows.items()}


def _lin(bits, r, seed):
    return workloads.make_linear(f"xr{bits}", 70 + bits, N, K, 1, sigma=0.02, wdtype="f16", bits=bits, r=r,
                                 alpha=16.0, abdtype="bf16", xdtype="bf16", seed=seed)


def _check(y, x_bf16, lin, wd, name):
    yref = oracle.linear(x_bf16, "bf16", wd, lin.A, lin.B, lin.abdtype, lin.scale)
    S = oracle.linear_tolerance(x_bf16, "bf16", wd)
    y = y.astype(np.float64)
    assert np.all(np.isfinite(y)), name
    err = np.abs(y - yref)
    assert np.all(err <= 1e-3 * S + 1e-5), (name, float(np.max(err / (1e-3 * S + 1e-5))))
    if np.max(np.abs(yref)) < 1e-20:
        assert np.all(err <= 1e-3 * S + 1e-40), (name, float(np.max(err / (1e-3 * S + 1e-40))))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("r", [0, 16, 64])
def test_single_row_x_edges(bits, r):
    """Single-row kernel (r 16: adapter product fused, the fp16 row in its own copy; r 64: prefetched
    partial sums, the row converted in place; r 0: no adapter)."""
    lin = _lin(bits, r, seed=bits + r)
    qw = qlr.quantize(dev(lin.W, "f16"), bits)
    rows = list(range(N))
    wd = oracle_rows_dequant(lin.W, "f16", bits, rows)
    A = dev(lin.A, "bf16") if r else None
    B = dev(lin.B, "bf16") if r else None
    for name, xr in x_rows(bits + 100 * r).items():
        xb = _bf16(xr)[None, :]
        with qlr.path(qlr.PATH_GEMV):
            y = qlr.linear(dev(xb, "bf16"), qw, A, B, lin.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check(f32_of(y), xb, lin, wd, name)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_grouped_decode_x_edges(bits):
    """The grouped single-row launch of a mixed call at M = 1 (3-bit codes as 12-byte pieces), one
    linear per x row kind, in one call."""
    names = list(x_rows(0).keys())
    lins, entries = [], []
    for i, name in enumerate(names):
        lin = _lin(bits, 8, seed=300 + i)
        xb = _bf16(x_rows(i)[name])[None, :]
        lin.x = xb
        qw = qlr.quantize(dev(lin.W, "f16"), bits)
        lins.append((lin, qw, name))
        entries.append(dict(x=dev(xb, "bf16"), qw=qw, A=dev(lin.A, "bf16"), B=dev(lin.B, "bf16"), scale=lin.scale))
    ys = qlr.linear_mixed(entries, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = list(range(N))
    for (lin, _, name), y in zip(lins, ys):
        _check(f32_of(y), lin.x, lin, oracle_rows_dequant(lin.W, "f16", bits, rows), name)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_single_row_nonfinite_x(bits):
    """An Inf in x makes every output +-Inf by the sign of its weight column (no adapter); a NaN makes
    every output NaN; as the oracle."""
    lin = _lin(bits, 0, seed=bits)
    qw = qlr.quantize(dev(lin.W, "f16"), bits)
    rows = list(range(N))
    wd = oracle_rows_dequant(lin.W, "f16", bits, rows)
    base = x_rows(1)["normal"]
    for k, v in ((5, np.inf), (SLICE * 3 + 7, -np.inf), (SLICE * 6 + 1, np.nan)):
        xr = base.copy()
        xr[k] = v
        xb = _bf16(xr)[None, :]
        with qlr.path(qlr.PATH_GEMV):
            y = f32_of(qlr.linear(dev(xb, "bf16"), qw, out_dtype=torch.float32))
        torch.cuda.synchronize()
        with np.errstate(invalid="ignore"):
            yref = oracle.linear(xb, "bf16", wd, None, None, "bf16", 0.0)
        assert np.array_equal(np.isnan(y), np.isnan(yref)), k
        fin = ~np.isnan(yref)
        assert np.array_equal(y[fin], yref[fin].astype(np.float32)), k
