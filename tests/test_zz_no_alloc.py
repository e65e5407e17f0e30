"""The allocation-free forward (qlr_linear_fwd_static, for callers that cannot allocate) against the
workspace forward qlr_linear_fwd, through the C ABI: two calls in a row on each kernel family, the second
with a smaller input, each equal bit for bit to the workspace call (same kernels, same partial sums)."""
import numpy as np
import pytest

import workloads
from gpu_util import dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from quantized_base_fine_amd import qlr  # noqa: E402


def _layer(N, K, M, r, bits, seed):
    lin = workloads.make_linear(f"na{seed}", 70 + seed, N, K, M, sigma=0.02, wdtype="f16", bits=bits, r=r,
                                alpha=16.0, abdtype="bf16", xdtype="bf16")
    qw = qlr.quantize(dev(lin.W, "f16"), bits)
    return lin, qw, dev(lin.x, "bf16"), dev(lin.A, "bf16"), dev(lin.B, "bf16")


@pytest.mark.parametrize("path,M1,M2", [(qlr.PATH_AUTO, 16, 1), (qlr.PATH_GEMV, 16, 5), (qlr.PATH_GEMM, 300, 40),
                                        (qlr.PATH_F32, 20, 3), (qlr.PATH_AUTO, 600, 16)])
@pytest.mark.parametrize("bits", [3, 4])
def test_static_equals_workspace_call(path, M1, M2, bits):
    lin, qw, x, A, B = _layer(512, 4096, max(M1, M2), 64, bits, seed=bits)
    print(f"static forward path={path} M={M1} then {M2} bits={bits}", flush=True)
    for M in (M1, M2):
        xs = x[:M]
        with qlr.path(path):
            ref = qlr.linear(xs, qw, A, B, lin.scale, out_dtype=torch.float32)
            got = qlr.linear_static(xs, qw, A, B, lin.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (path, M)


def test_static_without_adapter_and_repeat():
    """r = 0 (no scratch used), then a call with the adapter on the same stream: both equal the workspace calls."""
    lin, qw, x, A, B = _layer(300, 1024, 8, 16, 4, seed=9)
    with qlr.path(qlr.PATH_GEMV):
        r0 = qlr.linear(x, qw, out_dtype=torch.float32)
        g0 = qlr.linear_static(x, qw, out_dtype=torch.float32)
        r1 = qlr.linear(x, qw, A, B, lin.scale, out_dtype=torch.float32)
        g1 = qlr.linear_static(x, qw, A, B, lin.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(g0, r0) and torch.equal(g1, r1)
