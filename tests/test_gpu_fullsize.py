"""GPU parity at the full sizes of the 7B MLP, 65B and mixed-stack workloads.

  * MLP up/down (11008 x 4096, 4096 x 11008) and 65B-class (22016 x 8192)
    weights: every double-quantization group's codes, 8-bit absmax codes and
    steps, and every float32 dequantized weight, bit-exact against the oracle
    (run group chunk by group chunk).
  * The mixed stack: all 224 linears of 32 layers x 7 Llama-7B shapes with the
    drawn (bits, rank) per linear, through one qlr_linear_fwd_mixed call at
    M = 512 (the workload's size) and at decode sizes M = 1 and 16; every layer
    checked against the oracle on all x rows and sampled weight rows (codes of
    the groups covering them bit-exact).  Its inputs are drawn on the GPU by a
    seeded generator (the host draw of 6.5 G weights takes minutes); the groups
    and rows the oracle needs are copied back before anything else touches them.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import GROUP, BLOCK, check_linear, dev, f32_of, groups_covering, host, rows_from_groups

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from quantized_base_fine_amd import qlr  # noqa: E402

PER = BLOCK * GROUP  # elements per double-quantization group


@pytest.mark.parametrize("which", ["up", "down", "big65"])
def test_quantize_full_all_groups(which):
    """Every group of the full weight: codes, absmax codes, steps and float32 W' bit-exact."""
    lin = workloads.big65(1) if which == "big65" else workloads.mlp(which, 1)
    print(f"quantize {which} {lin.W.shape}", flush=True)
    qw = qlr.quantize(dev(lin.W, "f16"), 4)
    wdq = qlr.dequantize(qw, torch.float32).reshape(-1)
    torch.cuda.synchronize()
    codes, q8, cst = host(qw.codes), host(qw.absmax_q8), host(qw.absmax_c)
    flat = lin.W.reshape(-1)
    ngroups = flat.size // PER
    assert ngroups * PER == flat.size
    chunk = 128  # groups per oracle call
    cb = 8 * 4 * GROUP  # code bytes per group
    for g0 in range(0, ngroups, chunk):
        g1 = min(ngroups, g0 + chunk)
        ref = oracle.quantize(flat[g0 * PER:g1 * PER], "f16", 4)
        assert np.array_equal(codes[g0 * cb:g1 * cb], ref.codes), g0
        assert np.array_equal(q8[g0 * GROUP:g1 * GROUP], ref.absmax_q8), g0
        assert np.array_equal(cst[g0:g1].view(np.uint32), ref.absmax_c.view(np.uint32)), g0
        refd = oracle.dequantize(ref.codes, ref.absmax_q8, ref.absmax_c, 4, ref.numel)
        got = host(wdq[g0 * PER:g1 * PER])
        assert np.array_equal(got.view(np.uint32), refd.view(np.uint32)), g0


class _Lin:
    """The fields check_linear reads."""

    def __init__(self, x, A, B, scale):
        self.x, self.xdtype, self.A, self.B, self.abdtype, self.scale = x, "bf16", A, B, "bf16", scale


def test_mixed_full_stack():
    """All 224 linears of the mixed stack at M = 512 (one mixed call), and at M = 1 and 16."""
    dv = torch.device("cuda")
    plan = workloads.mixed_plan()
    M = 512
    rng = np.random.default_rng(44)
    entries, keep = [], []
    for i in range(len(plan)):
        N, K, bits, r, alpha, W, x, A, B = workloads.device_mixed_linear(i, M, dv, plan)
        qw = qlr.quantize(W, bits)
        rows = sorted({0, N - 1, int(rng.integers(1, N - 1))})
        flat = W.reshape(-1)
        wg = {g: host(flat[g * PER:(g + 1) * PER]) for g in groups_covering(K, rows, N * K)}
        del W, flat
        entries.append(dict(x=x, qw=qw, A=A, B=B, scale=alpha / r))
        keep.append((bits, rows, wg))
    torch.cuda.synchronize()
    print(f"stack of {len(entries)} linears quantized", flush=True)
    refs = []
    for (bits, rows, wg), e in zip(keep, entries):
        qw = e["qw"]
        qg = {g: oracle.quantize(w, "f16", bits) for g, w in wg.items()}
        codes, q8, cst = host(qw.codes), host(qw.absmax_q8), host(qw.absmax_c)
        cb = 8 * bits * GROUP
        for g, rq in qg.items():
            assert np.array_equal(codes[g * cb:(g + 1) * cb], rq.codes), (bits, g)
            assert np.array_equal(q8[g * GROUP:(g + 1) * GROUP], rq.absmax_q8), (bits, g)
            assert cst[g].view(np.uint32) == rq.absmax_c[0].view(np.uint32), (bits, g)
        refs.append(rows_from_groups(qg, qw.cols, bits, rows))
    for Mr in (M, 1, 16):
        sub = [dict(e, x=e["x"][:Mr]) for e in entries]
        ys = qlr.linear_mixed(sub, out_dtype=torch.float32)
        torch.cuda.synchronize()
        print(f"mixed call at M={Mr} done", flush=True)
        worst = 0.0
        for (bits, rows, wg), e, y, wd in zip(keep, sub, ys, refs):
            lin = _Lin(host(e["x"]), host(e["A"]), host(e["B"]), e["scale"])
            worst = max(worst, check_linear(f32_of(y), lin, wd, rows, "f32"))
        print(f"M={Mr}: worst err/bound over the stack {worst:.3f}", flush=True)
        del ys
