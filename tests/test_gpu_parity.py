"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Codes, 8-bit absmax codes, group steps and dequantized float32 weights must be
bit-exact; linear outputs must satisfy |y - y_ref| <= 1e-3 sum_k |x w'| + 1e-5
per element (plus half a bf16 ulp for bf16 outputs).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import check_linear, dev, f32_of, host, oracle_groups, oracle_rows_dequant

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from quantized_base_fine_amd import qlr  # noqa: E402

BITS = [2, 3, 4, 8]


def _gpu_quant(W, wdtype, bits):
    Wd = dev(W, wdtype)
    qw = qlr.quantize(Wd if Wd.dim() == 2 else Wd.reshape(1, -1), bits)
    torch.cuda.synchronize()
    return qw


def _assert_qweight_equal(qw, ref, groups=None):
    codes, q8, cst = host(qw.codes), host(qw.absmax_q8), host(qw.absmax_c)
    if groups is None:
        assert np.array_equal(codes[: ref.codes.size], ref.codes)
        assert np.array_equal(q8[: ref.absmax_q8.size], ref.absmax_q8)
        assert np.array_equal(cst[: ref.absmax_c.size].view(np.uint32), ref.absmax_c.view(np.uint32))
        return
    for g, rq in groups.items():
        cb = 8 * qw.bits * 256
        assert np.array_equal(codes[g * cb:(g + 1) * cb], rq.codes), g
        assert np.array_equal(q8[g * 256:(g + 1) * 256], rq.absmax_q8), g
        assert cst[g].view(np.uint32) == rq.absmax_c[0].view(np.uint32), g


def _rand_w(shape, dtype, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(shape) * scale).astype(np.float32)
    return workloads.store(w, dtype)


# ---------------------------------------------------------------- quantize / dequantize

@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("wdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(256, 256), (37, 101), (3, 2 * 16384 + 64 * 5 + 3)])
def test_quantize_bitexact(bits, wdtype, shape):
    W = _rand_w(shape, wdtype, seed=bits * 100 + len(wdtype) + shape[0])
    qw = _gpu_quant(W, wdtype, bits)
    ref = oracle.quantize(W.reshape(-1), wdtype, bits)
    _assert_qweight_equal(qw, ref)


@pytest.mark.parametrize("bits", BITS)
def test_quantize_special_values(bits):
    """Zero blocks, +-0, exact ties at level midpoints, absmax on both signs."""
    L = oracle.quantile_codebook(bits)
    n = L.size
    w = np.zeros((8, 64), dtype=np.float32)
    w[1, 0], w[1, 1], w[1, 2], w[1, 3] = 0.5, -0.0, 0.0, -0.5
    w[2, :] = -3.0
    mids = [(float(L[i]) + float(L[i + 1])) for i in range(n - 1)]
    k = 0
    for i, m in enumerate(mids):  # exact midpoints for absmax 2.0 (tie -> lower)
        if float(np.float32(m)) == m and abs(m) <= 2.0 and k < 63:
            w[3, 1 + k] = m
            k += 1
    w[3, 0] = 2.0
    w[4, :] = np.float32(1e-40)  # subnormal absmax
    w[5, ::2] = 1e-30
    w[6, 5] = -7.0
    qw = _gpu_quant(w.reshape(1, -1), "f32", bits)
    ref = oracle.quantize(w.reshape(-1), "f32", bits)
    _assert_qweight_equal(qw, ref)
    back = host(qlr.dequantize(qw, torch.float32)).reshape(-1)
    refd = oracle.dequantize(ref.codes, ref.absmax_q8, ref.absmax_c, bits, w.size)
    assert np.array_equal(back.view(np.uint32), refd.view(np.uint32))


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("shape", [(256, 256), (37, 101), (300, 1000)])
def test_dequantize_bitexact(bits, shape):
    W = _rand_w(shape, "f16", seed=7 + bits)
    qw = _gpu_quant(W, "f16", bits)
    ref = oracle.quantize(W.reshape(-1), "f16", bits)
    refd = oracle.dequantize(ref.codes, ref.absmax_q8, ref.absmax_c, bits, W.size)
    got = host(qlr.dequantize(qw, torch.float32)).reshape(-1)
    assert np.array_equal(got.view(np.uint32), refd.view(np.uint32))  # signed zeros included
    gotb = host(qlr.dequantize(qw, torch.bfloat16)).reshape(-1)
    assert np.array_equal(gotb, workloads.to_bf16_bits(refd))


def test_quantize_nonfinite_rejected():
    W = _rand_w((64, 128), "f16", seed=1)
    W[10, 77] = np.float16(np.inf)
    with pytest.raises(qlr.QlrError) as ei:
        _gpu_quant(W, "f16", 4)
    assert ei.value.name == "QLR_ERR_NONFINITE"
    W[10, 77] = np.float16(np.nan)
    Wd = dev(W, "f16")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    qlr.quantize(Wd, 4, ws=ws, blocking=False)
    torch.cuda.synchronize()
    assert host(ws)[:4].view(np.uint32)[0] != 0


def test_quantize_attn_full():
    """7B-class attention projection, 4096 x 4096 fp16 with 0.1% x20 outliers: every code."""
    lin = workloads.attn(1)
    qw = _gpu_quant(lin.W, "f16", 4)
    ref = oracle.quantize(lin.W.reshape(-1), "f16", 4)
    _assert_qweight_equal(qw, ref)
    got = host(qlr.dequantize(qw, torch.float32)).reshape(-1)
    refd = oracle.dequantize(ref.codes, ref.absmax_q8, ref.absmax_c, 4, lin.W.size)
    assert np.array_equal(got.view(np.uint32), refd.view(np.uint32))


# ---------------------------------------------------------------- linear forward

def _run_linear(lin, qw, ydt="f32", path=qlr.PATH_AUTO):
    x = dev(lin.x, lin.xdtype)
    A = dev(lin.A, lin.abdtype) if lin.r > 0 else None
    B = dev(lin.B, lin.abdtype) if lin.r > 0 else None
    with qlr.path(path):
        y = qlr.linear(x, qw, A, B, lin.scale, out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    return f32_of(y)


def _small_linear(N, K, M, bits, r, seed, xdtype="bf16", abdtype="bf16"):
    return workloads.make_linear(f"s{seed}", 50 + seed, N, K, M, sigma=0.02, wdtype="f16", bits=bits,
                                 r=r, alpha=16.0, abdtype=abdtype, xdtype=xdtype)


PATHS = {"gemv": qlr.PATH_GEMV, "gemm": qlr.PATH_GEMM, "f32": qlr.PATH_F32}


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 5), ("gemv", 16), ("gemm", 1), ("gemm", 100),
                                    ("gemm", 300), ("f32", 3), ("f32", 20)])
@pytest.mark.parametrize("r", [0, 4, 16, 72])
def test_linear_paths_small(bits, path, M, r):
    """Ragged N (not a multiple of 16 or 128), K of 10 blocks, every path, bits and rank."""
    lin = _small_linear(333, 640, M, bits, r, seed=bits + M + r)
    qw = _gpu_quant(lin.W, "f16", bits)
    rows = list(range(lin.N))
    wd = oracle_rows_dequant(lin.W, "f16", bits, rows)
    for ydt in ("f32", "bf16"):
        y = _run_linear(lin, qw, ydt, PATHS[path])
        check_linear(y, lin, wd, rows, ydt)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K", [2496, 2560, 3200, 4096])
@pytest.mark.parametrize("M,r", [(2, 0), (16, 16), (5, 64)])
def test_decode_mfma_x_in_registers(bits, K, M, r):
    """The MFMA decode path around its x-in-registers case (x over the 32 KB that is staged in LDS and
    40..64 blocks per row, every wave's K range two chunks: M = 16 at K >= 2560 and M = 5 at K = 4096;
    K = 2496 has 39 blocks and keeps x riding with the chunks; M = 2 and the narrower M = 5 rows stage x
    in LDS): ragged N (1049 rows: 66 tiles), every code width, with and without the adapter; every output
    against the oracle, float32 and bf16 y."""
    lin = _small_linear(1049, K, M, bits, r, seed=K + M + r + bits)
    qw = _gpu_quant(lin.W, "f16", bits)
    rows = list(range(lin.N))
    wd = oracle_rows_dequant(lin.W, "f16", bits, rows)
    for ydt in ("f32", "bf16"):
        check_linear(_run_linear(lin, qw, ydt, qlr.PATH_GEMV), lin, wd, rows, ydt)


@pytest.mark.parametrize("K", [2560, 4096])
def test_decode_3bit_single_row_mfma(K):
    """3-bit codes at M = 1 take the MFMA path (x staged in LDS): every output."""
    lin = _small_linear(777, K, 1, 3, 16, seed=K // 64)
    qw = _gpu_quant(lin.W, "f16", 3)
    rows = list(range(lin.N))
    wd = oracle_rows_dequant(lin.W, "f16", 3, rows)
    for ydt in ("f32", "bf16"):
        check_linear(_run_linear(lin, qw, ydt, qlr.PATH_GEMV), lin, wd, rows, ydt)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("r", [80, 128])
@pytest.mark.parametrize("M", [1, 8])
def test_decode_adapter_many_tiles(bits, r, M):
    """20487 rows (1281 tiles of 16: 5 or 6 per workgroup on a 256-CU grid): the B rows of all of a
    workgroup's tiles go to LDS up front when they are at most 1024 16-byte pieces (r 80: 960), else the
    epilogue reads them from global memory (r 128: 1536); both against the oracle, every output."""
    lin = _small_linear(20487, 256, M, bits, r, seed=11 + r + M)
    qw = _gpu_quant(lin.W, "f16", bits)
    rows = list(range(lin.N))
    wd = oracle_rows_dequant(lin.W, "f16", bits, rows)
    for ydt in ("f32", "bf16"):
        check_linear(_run_linear(lin, qw, ydt, qlr.PATH_GEMV), lin, wd, rows, ydt)


@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 7), ("gemm", 130), ("f32", 7)])
def test_linear_long_k_tail(path, M):
    """K = 11008 (172 blocks: DQ groups straddle rows, waves get partial chunks), N = 100, every path."""
    lin = _small_linear(100, 11008, M, 4, 64, seed=3)
    qw = _gpu_quant(lin.W, "f16", 4)
    rows = list(range(lin.N))
    wd = oracle_rows_dequant(lin.W, "f16", 4, rows)
    check_linear(_run_linear(lin, qw, "f32", PATHS[path]), lin, wd, rows)


def test_linear_tiny_config():
    """256x256 fp32 weights, rank-4 fp32 adapters, 8x256 fp32 x (float32 path)."""
    lin = workloads.tiny()
    qw = _gpu_quant(lin.W, "f32", 4)
    rows = list(range(lin.N))
    wd = oracle_rows_dequant(lin.W, "f32", 4, rows)
    check_linear(_run_linear(lin, qw), lin, wd, rows)


def test_linear_attn_full():
    """4096x4096 with outliers, r16: M=1 (decode) and M=2048 (prefill), every output."""
    base = workloads.attn(1)
    qw = _gpu_quant(base.W, "f16", 4)
    rows = list(range(base.N))
    ref = oracle.quantize(base.W.reshape(-1), "f16", 4)
    wd = oracle.dequantize(ref.codes, ref.absmax_q8, ref.absmax_c, 4, base.W.size).reshape(base.W.shape)
    for M in (1, 2048):
        lin = workloads.attn(M, W=base.W)
        check_linear(_run_linear(lin, qw, "bf16"), lin, wd, rows, "bf16")
        check_linear(_run_linear(lin, qw, "f32"), lin, wd, rows, "f32")


@pytest.mark.parametrize("which", ["up", "down"])
def test_linear_mlp_sampled(which):
    """7B-class MLP projections, r64: M = 1, 16, 2048 on sampled output columns."""
    base = workloads.mlp(which, 1)
    qw = _gpu_quant(base.W, "f16", 4)
    rng = np.random.default_rng(2)
    rows = sorted(set([0, base.N - 1] + rng.choice(base.N, size=30, replace=False).tolist()))
    wd = oracle_rows_dequant(base.W, "f16", 4, rows)
    for M in (1, 16, 2048):
        lin = workloads.mlp(which, M, W=base.W)
        check_linear(_run_linear(lin, qw, "bf16"), lin, wd, rows, "bf16")
        check_linear(_run_linear(lin, qw, "f32"), lin, wd, rows, "f32")


def test_linear_big65_sampled():
    """65B-class 22016x8192, r64: M = 1 and 4096 on sampled rows and columns."""
    base = workloads.big65(1)
    qw = _gpu_quant(base.W, "f16", 4)
    rng = np.random.default_rng(3)
    rows = sorted(set([0, base.N - 1] + rng.choice(base.N, size=24, replace=False).tolist()))
    wd = oracle_rows_dequant(base.W, "f16", 4, rows)
    for M in (1, 4096):
        lin = workloads.big65(M, W=base.W)
        ms = sorted(set([0, M - 1] + rng.choice(M, size=min(M, 40), replace=False).tolist()))
        check_linear(_run_linear(lin, qw, "bf16"), lin, wd, rows, "bf16", ms=ms)
        check_linear(_run_linear(lin, qw, "f32"), lin, wd, rows, "f32", ms=ms)


def test_linear_edge_cases():
    lin = _small_linear(96, 256, 4, 4, 8, seed=9)
    qw = _gpu_quant(lin.W, "f16", 4)
    x = dev(lin.x, "bf16")
    A, B = dev(lin.A, "bf16"), dev(lin.B, "bf16")
    for p in (qlr.PATH_GEMV, qlr.PATH_GEMM, qlr.PATH_F32):
        with qlr.path(p):
            y0 = qlr.linear(x, qw, out_dtype=torch.float32)                  # r = 0
            yb = qlr.linear(x, qw, A, torch.zeros_like(B), 2.0, out_dtype=torch.float32)  # B = 0
            y1 = qlr.linear(x, qw, A, B, lin.scale, out_dtype=torch.float32)
            y2 = qlr.linear(x, qw, A, B, lin.scale, out_dtype=torch.float32)
            e = qlr.linear(x[:0], qw, A, B, lin.scale, out_dtype=torch.float32)  # M = 0
        torch.cuda.synchronize()
        assert torch.equal(y0, yb)
        assert torch.equal(y1, y2)  # deterministic: no atomics on the output path
        assert e.shape == (0, 96)


# ---------------------------------------------------------------- mixed stack

def test_mixed_small():
    """Per-layer (bits, rank) drawn as for the mixed stack, shrunk shapes, M = 48, 8 and 1 (at M = 1 the
    2-, 4- and 8-bit layers run as grouped decode launches: blocks per row 6 and 7, so waves hold 0 or 1
    blocks; ragged rows)."""
    plan = workloads.mixed_plan()
    for M in (48, 8, 1):
        lins = [workloads.mixed_linear(i, M=M, plan=plan, shape_override=(200 + 16 * (i % 3), 384 + 64 * (i % 2)))
                for i in range(10)]
        entries, qws = [], []
        for lin in lins:
            qw = _gpu_quant(lin.W, "f16", lin.bits)
            qws.append(qw)
            entries.append(dict(x=dev(lin.x, "bf16"), qw=qw, A=dev(lin.A, "bf16"), B=dev(lin.B, "bf16"),
                                scale=lin.scale))
        ys = qlr.linear_mixed(entries, out_dtype=torch.float32)
        torch.cuda.synchronize()
        for lin, y in zip(lins, ys):
            rows = list(range(lin.N))
            check_linear(f32_of(y), lin, oracle_rows_dequant(lin.W, "f16", lin.bits, rows), rows)


def test_mixed_grouped_equals_single():
    """Grouped launches of the mixed call (one code width and adapter flag per group,
    more layers than one launch holds) equal the single-layer calls bit for bit."""
    # the first 18 layers share one code width (two launches of it), the rest keep their draw
    plan = [(n, k, 4 if i < 18 else b, r) for i, (n, k, b, r) in enumerate(workloads.mixed_plan())]
    M = 300
    entries, singles = [], []
    for i in range(24):
        lin = workloads.mixed_linear(i, M=M, plan=plan, shape_override=(144 + 16 * (i % 4), 320 + 64 * (i % 3)))
        qw = _gpu_quant(lin.W, "f16", lin.bits)
        x = dev(lin.x, "bf16")
        if i % 5 == 4:  # some layers without an adapter
            e = dict(x=x, qw=qw, scale=0.0)
        else:
            e = dict(x=x, qw=qw, A=dev(lin.A, "bf16"), B=dev(lin.B, "bf16"), scale=lin.scale)
        entries.append(e)
        with qlr.path(qlr.PATH_GEMM):
            singles.append(qlr.linear(x, qw, e.get("A"), e.get("B"), e["scale"], out_dtype=torch.float32))
    ys = qlr.linear_mixed(entries, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for i, (y, y1) in enumerate(zip(ys, singles)):
        assert torch.equal(y, y1), f"layer {i}"


# ---------------------------------------------------------------- decode repeats and graph replays

def test_decode_repeats_bit_identical():
    """Back-to-back decode calls on one (uninitialised) workspace agree bit for bit."""
    lin = workloads.mlp("down", 1)
    qw = _gpu_quant(lin.W, "f16", 4)
    x, A, B = dev(lin.x, "bf16"), dev(lin.A, "bf16"), dev(lin.B, "bf16")
    ws = torch.full((qlr.workspace_bytes(qlr.OP_LINEAR, 1, lin.N, lin.K, lin.r),), 0xA5, dtype=torch.uint8,
                    device="cuda")
    ys = [qlr.linear(x, qw, A, B, lin.scale, out_dtype=torch.float32, ws=ws) for _ in range(4)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    rows = list(range(0, lin.N, 97))
    check_linear(f32_of(ys[0]), lin, oracle_rows_dequant(lin.W, "f16", 4, rows), rows)


def test_decode_graph_replays_match_eager():
    """Decode calls captured in a HIP graph: every replay equals the eager result."""
    lin = workloads.attn(1)
    qw = _gpu_quant(lin.W, "f16", 4)
    x, A, B = dev(lin.x, "bf16"), dev(lin.A, "bf16"), dev(lin.B, "bf16")
    ws = torch.zeros(qlr.workspace_bytes(qlr.OP_LINEAR, 1, lin.N, lin.K, lin.r), dtype=torch.uint8, device="cuda")
    y = torch.empty((1, lin.N), dtype=torch.bfloat16, device="cuda")
    qlr.linear(x, qw, A, B, lin.scale, out=y, ws=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qlr.linear(x, qw, A, B, lin.scale, out=y, ws=ws)
        qlr.linear(x, qw, A, B, lin.scale, out=y, ws=ws)
    for i in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), i
        _ = (x.float() * 2).sum().item()  # unrelated eager work between replays


def test_linear_rows_past_32bit_offsets():
    """M = 262,400 rows of K = 4096 (x above 2 GiB): the GEMM runs as two row ranges (261,888 rows, then 512),
    each addressed with 32-bit buffer offsets from its own base.  x repeats one 512-row block, so every row's
    reference is that block's; rows on both sides of the split and at the ends are checked."""
    import types
    base = _small_linear(256, 4096, 512, 4, 16, seed=40)
    qw = _gpu_quant(base.W, "f16", 4)
    rows = list(range(256))
    wd = oracle_rows_dequant(base.W, "f16", 4, rows)
    M = 262400
    xs = dev(base.x, "bf16")
    x = xs.repeat((M + 511) // 512, 1)[:M].contiguous()
    A, B = dev(base.A, "bf16"), dev(base.B, "bf16")
    print(f"linear M={M} K=4096 N=256 r=16 (two row ranges)", flush=True)
    y = qlr.linear(x, qw, A, B, base.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ms = [0, 1, 261887, 261888, 261889, 262143, 262144, M - 1] + \
        np.random.default_rng(40).choice(M, size=8, replace=False).tolist()
    got = f32_of(y[torch.tensor(ms, device=y.device)])
    ref = types.SimpleNamespace(x=base.x[[m % 512 for m in ms]], xdtype="bf16", A=base.A, B=base.B,
                                abdtype="bf16", scale=base.scale)
    check_linear(got, ref, wd, rows, "f32")
    del x, y
    torch.cuda.empty_cache()
