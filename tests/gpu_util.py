"""Helpers for the GPU parity tests (host <-> device marshalling, oracle on sampled rows)."""
import numpy as np

import oracle

BLOCK, GROUP = 64, 256


def dev(arr, dtype, device="cuda"):
    """numpy storage array -> torch device tensor ('bf16' arrays are uint16 bit patterns)."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def host(t):
    """torch device tensor -> numpy (bf16 returned as uint16 bits)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32_of(t):
    import torch
    return t.detach().float().cpu().numpy()


def groups_covering(K, rows, numel):
    """Sorted DQ-group indices that contain the blocks of the given weight rows."""
    nb = K // BLOCK
    gs = set()
    for n in rows:
        gs.update(range((n * nb) // GROUP, ((n + 1) * nb - 1) // GROUP + 1))
    return sorted(gs)


def oracle_groups(W, wdtype, bits, groups):
    """Oracle quantization of the listed DQ groups of a weight (flattened).

    Returns {group: QuantizedWeight of that group's 16384 elements}.  Groups are
    independent, so quantizing a group alone gives the same codes and scales as
    quantizing the whole weight.
    """
    flat = W.reshape(-1)
    out = {}
    per = BLOCK * GROUP
    for g in groups:
        out[g] = oracle.quantize(flat[g * per:(g + 1) * per], wdtype, bits)
    return out


def oracle_rows_dequant(W, wdtype, bits, rows):
    """float32 dequantized rows (len(rows), K) computed by the oracle alone."""
    N, K = W.shape
    qg = oracle_groups(W, wdtype, bits, groups_covering(K, rows, W.size))
    return rows_from_groups(qg, K, bits, rows)


def rows_from_groups(qg, K, bits, rows):
    """float32 dequantized weight rows from the oracle's per-group quantization ``qg``
    ({group: QuantizedWeight}) of the groups covering them."""
    per = BLOCK * GROUP
    out = np.empty((len(rows), K), dtype=np.float32)
    for i, n in enumerate(rows):
        e0, e1 = n * K, (n + 1) * K
        seg = []
        g = e0 // per
        while g * per < e1:
            q = qg[g]
            d = oracle.dequantize(q.codes, q.absmax_q8, q.absmax_c, bits, q.numel)
            lo, hi = max(e0, g * per) - g * per, min(e1, (g + 1) * per) - g * per
            seg.append(d[lo:hi])
            g += 1
        out[i] = np.concatenate(seg)
    return out


# Rounding a float32 value y to bf16 moves it by at most half a bf16 ulp, which is at most 2^-8 |y|.
BF16_HALF_ULP_REL = 2.0 ** -8


def check_linear(y_gpu, lin, wdeq_rows, rows, ydt="f32", ms=None, rel=1e-3):
    """Per-element bound |y - y_ref| <= rel * S + 1e-5 (+ half a bf16 ulp for bf16 y).

    ``wdeq_rows``: oracle-dequantized rows ``rows`` of W'; ``ms``: x rows to check;
    ``rel``: 1e-3 (the layer's bound), or the bf16-weight GEMM family's wider one.
    Returns the worst ratio error / bound.
    """
    x = lin.x if ms is None else lin.x[ms]
    A, B = lin.A, (None if lin.B is None else lin.B[rows])
    yref = oracle.linear(x, lin.xdtype, wdeq_rows, A, B, lin.abdtype, lin.scale)
    S = oracle.linear_tolerance(x, lin.xdtype, wdeq_rows)
    bound = rel * S + 1e-5
    if ydt == "bf16":
        bound = bound + np.abs(yref) * BF16_HALF_ULP_REL
    got = y_gpu if ms is None else y_gpu[ms]
    got = got[:, rows].astype(np.float64)
    err = np.abs(got - yref)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"max err/bound {ratio:.3f}"
    return ratio


def check_backward(got, lin, dy, wdeq, ks=None, dxdt="f32"):
    """Per-element bound 1e-3 * S + 1e-5 on dx, dA and dB (+ half a bf16 ulp for a bf16 dx).

    ``got`` = (dx, dA, dB) as float32 numpy arrays (dA, dB None when r == 0);
    ``wdeq``: the oracle's dequantized W' (all rows), restricted to the columns
    ``ks`` when given (dx and dA are then checked on those columns only, dB in
    full).  Returns the worst ratio error / bound of each gradient.
    """
    dx, dA, dB = got
    cols = slice(None) if ks is None else ks
    xs = lin.x[:, cols]
    As = None if lin.r == 0 else lin.A[:, cols]
    ref = oracle.linear_backward(dy, lin.xdtype, xs, lin.xdtype, wdeq, As, lin.B, lin.abdtype, lin.scale)
    S = oracle.linear_backward_tolerance(dy, lin.xdtype, xs, lin.xdtype, wdeq, As, lin.B, lin.abdtype, lin.scale)
    ratios = []

    def one(g, r_, s_, extra=0.0):
        bound = 1e-3 * s_ + 1e-5 + extra * np.abs(r_)
        g = g.astype(np.float64)
        assert g.shape == r_.shape
        assert np.all(np.isfinite(g))
        err = np.abs(g - r_)
        ratio = float(np.max(err / bound)) if err.size else 0.0
        assert np.all(err <= bound), f"max err/bound {ratio:.3f}"
        ratios.append(ratio)

    if dx is not None:
        one(dx[:, cols], ref[0], S[0], BF16_HALF_ULP_REL if dxdt == "bf16" else 0.0)
    if lin.r > 0:
        one(dA[:, cols], ref[1], S[1])
        if ks is None:
            one(dB, ref[2], S[2])
        else:
            rA, rB = oracle.adapter_grads(dy, lin.xdtype, lin.x, lin.xdtype, lin.A, lin.B, lin.abdtype, lin.scale)
            sA, sB = oracle.adapter_grads_tolerance(dy, lin.xdtype, lin.x, lin.xdtype, lin.A, lin.B,
                                                    lin.abdtype, lin.scale)
            one(dB, rB, sB)
    return ratios
