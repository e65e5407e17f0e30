"""Benchmark of the quantized-base + low-rank-adapter linear layer on one MI355X.

Workload: a 7B-class attention projection, W 4096 x 4096 fp16 ~ N(0, 0.02^2)
with 0.1% of entries x20 (outliers), 4-bit quantile codebook, blocks of 64,
double quantization in groups of 256; adapter rank 16, alpha 16, bf16;
x bf16 ~ N(0, 1) at M = 1 (decode) and M = 2048 (prefill).  Synthetic data
from the seeded generators in ``workloads``.

One step is one pass of the whole path over a stack of R distinct copies of
the layer (R chosen so the packed weights exceed twice the 256 MB last-level
cache, so the decode figure is HBM bandwidth, not cache bandwidth):
  quantize      all R weights (codes, 8-bit absmax codes, group steps)
  dequantize    one weight to float32 (export path)
  prefill       y = x W'^T + s (x A^T) B^T at M = 2048 for all R layers
  prefill base  the same without the adapter (one GEMM kernel per call)
  decode        y = x W'^T + s (x A^T) B^T at M = 1 for all R layers
  decode base   the same without the adapter (one GEMV kernel per call)
  backward      dx = dy W' + s (dy B) A, dA = s (dy B)^T x, dB = s dy^T (x A^T)
                at M = 2048 for all R layers (dy bf16 ~ N(0, 1), dx bf16, dA/dB fp32)
  backward base dx = dy W' alone (one transposed GEMM kernel per call)
  dba decode / dba prefill   the forward with a double-binary adapter branch
                (R = 16, l = 1) in place of the fp16 adapter, at M = 1 (graph) and M = 2048
  outliers decode / prefill  the forward with the weight's 0.1 % largest-|w| entries
                split off into a float32 CSR side channel (k = 16777) and the dense
                rest quantized, with the fp16 adapter, at M = 1 (graph) and M = 2048
  wha decode / wha prefill   the forward with a Walsh-Hadamard adapter in place of
                the fp16 one: 131072 coefficients per layer (the parameter count of the
                rank-16 adapter), one full transform over K = 4096, at M = 1 (graph) and
                M = 2048
The outlier split itself (qlr_quantize_outliers, blocking) is timed outside the
step, on one layer.
Each phase is bracketed by HIP events on the stream its calls run on (events
between the calls of a phase would add a queue barrier per call).  Calls are
prepared (marshalled once); the prefill phases are GPU-bound and issued eagerly,
the launch-bound decode phases replay HIP graphs of their R calls (checked
against the eager outputs first).  A phase is its calls back to back, and its
time / R is the average launch duration (kernel time plus the dispatch gap
between back-to-back kernels, about 1.8 us on this GPU).

value          = decode effective GB/s (algorithmic bytes of all decode calls /
                 decode phase time); bytes = codes + absmax codes + group steps
                 + A + B + x + y.
value_prefill  = prefill TFLOP/s with 2MNK + 2Mr(K+N) flops per call.
roofline       = the decode GEMV kernel (base calls: one kernel per call).
roofline_prefill = the prefill GEMM kernel (base calls).
backward       = backward TFLOP/s with 2MNK + 2Mr(3K + 2N) flops per call;
                 its roofline is the transposed GEMM kernel (base calls).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NF4+LoRA linear: weight GB/s at M=1, TFLOP/s at M=2048 (% roofline)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
N_, K_, BITS, R_, ALPHA = 4096, 4096, 4, 16, 16.0
M_DECODE, M_PREFILL = 1, 2048
MALL_BYTES = 256 << 20


def decode_bytes(M=M_DECODE, N=N_, K=K_, b=BITS, r=R_):
    numel = N * K
    return numel * b // 8 + numel // 64 + 4 * (numel // 16384) + 2 * r * K + 2 * N * r + 2 * M * K + 2 * M * N


def prefill_flops(M=M_PREFILL, N=N_, K=K_, r=R_):
    return 2 * M * N * K + 2 * M * r * (K + N)


def backward_flops(M=M_PREFILL, N=N_, K=K_, r=R_):
    # dx = dy W' (2MNK) + u A (2MrK); u = dy B (2MNr); t = x A^T (2MKr); dA (2MrK); dB (2MNr)
    return 2 * M * N * K + 2 * M * r * (3 * K + 2 * N)


def dba_bytes(M=M_DECODE, N=N_, K=K_, b=BITS, R=R_, ell=1):
    # codes + absmax codes + group steps + sign words (N R + R K bits) + fp16 scales + x + y
    numel = N * K
    return (numel * b // 8 + numel // 64 + 4 * (numel // 16384) + (N * R + R * K) // 8 + 2 * ell * (N + R + K)
            + 2 * M * K + 2 * M * N)


def dba_flops(M=M_PREFILL, N=N_, K=K_, R=R_, ell=1):
    return 2 * M * N * K + 2 * M * ell * R * (K + N)


NNZ = int(round(0.001 * N_ * K_))  # the attention weight's planted outliers


def outlier_bytes(M=M_DECODE, nnz=NNZ):
    # the decode bytes plus the CSR side channel (row offsets, columns, float32 values)
    return decode_bytes(M) + 4 * (N_ + 1) + 8 * nnz


def outlier_flops(M=M_PREFILL, nnz=NNZ):
    return prefill_flops(M) + 2 * M * nnz


WHA_NNZ = R_ * (N_ + K_)  # coefficients of the Walsh-Hadamard adapter: the rank-16 adapter's parameter count


def wha_bytes(M=M_DECODE, nnz=WHA_NNZ):
    # the base's bytes, the coefficients (CSR: offsets, columns, float32 values), x and y
    numel = N_ * K_
    return numel * BITS // 8 + numel // 64 + 4 * (numel // 16384) + 4 * (N_ + 1) + 8 * nnz + 2 * M * K_ + 2 * M * N_


def wha_flops(M=M_PREFILL, nnz=WHA_NNZ):
    # base product, the transform's additions (K log2 K per row) and the sparse product
    return 2 * M * N_ * K_ + M * K_ * 12 + 2 * M * nnz


def quantize_bytes(N=N_, K=K_, b=BITS):
    numel = N * K
    return 2 * numel + numel * b // 8 + numel // 64 + 4 * (numel // 16384)


def traffic_from_profile(kernel_key: str):
    """HBM bytes per launch from the committed counter summary, if it is current."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sha256"]:
        return None  # the kernel changed since the counters were taken
    return rec["bytes_per_launch"]


# Kernels whose HBM traffic the counter runs measure, with the sources they are
# built from (the stored figure is dropped when any of them changes).
_CSRC = "quantized_base_fine_amd/csrc/"
TRAFFIC_KERNELS = {
    "decode": ("k_gemv<4, 2, true, false, 2, true, false, 0, false, false>",
               [_CSRC + f for f in ("qlr_gemv.hip", "qlr_lut.h", "qlr_device.h", "qlr_internal.h")]),
    "prefill": ("k_gemm<4, 2, false, false, false>",
                [_CSRC + f for f in ("qlr_gemm.hip", "qlr_lut.h", "qlr_device.h", "qlr_internal.h")]),
    "backward": ("k_gemm<4, 2, false, true, false>",
                 [_CSRC + f for f in ("qlr_gemm.hip", "qlr_lut.h", "qlr_device.h", "qlr_internal.h")]),
}
COPY_BYTES = 256 << 20  # the calibration copy reads and writes this many bytes


def traffic_from_counters(fetch_dir: str, write_dir: str, out_path: str = ""):
    """profiles/traffic.json (or out_path) from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE in KiB per dispatch) of `bench.py --eager --copy-calibration`: the mean per
    launch of each kernel, scaled by what the counter reads for the calibration copy of
    known size.  Every kernel of TRAFFIC_KERNELS must appear in both runs."""
    import csv
    import glob
    import hashlib

    def load(d, counter):
        per = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if row["Counter_Name"] == counter:
                        per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return per

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")

    def copy_kib(per):
        vals = [v for k, vs in per.items() if "elementwise" in k for v in vs]
        return max(vals) if vals else None

    cf, cw = copy_kib(fetch), copy_kib(write)
    if not cf or not cw:
        raise SystemExit("no calibration copy in the counter runs (run bench.py with --copy-calibration)")
    scale_f, scale_w = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    out = {}
    for key, (kname, sources) in TRAFFIC_KERNELS.items():
        fv = [v for k, vs in fetch.items() if kname in k for v in vs]
        wv = [v for k, vs in write.items() if kname in k for v in vs]
        if not fv or not wv:
            raise SystemExit(f"no counter rows for {kname} (kernel renamed? update TRAFFIC_KERNELS)")
        h = hashlib.sha256()
        for src in sources:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        out[key] = {"kernel": kname, "sources": sources, "sha256": h.hexdigest(),
                    "launches": len(fv), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                    "calibration": {"copy_fetch_kib": cf, "copy_write_kib": cw,
                                    "fetch_scale": round(scale_f, 4), "write_scale": round(scale_w, 4)},
                    "bytes_per_launch": int(round(fk * 1024 * scale_f + wk * 1024 * scale_w))}
    with open(out_path or os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


MIXED_M = 512


def decode_by_bits(torch, qlr, W, x1, A0, B0, scale, dev, reps=5):
    """Decode GEMV (M = 1) of the same 4096x4096 layer at the other code widths, without
    and with the r16 adapter: per-call time (HIP graph of R distinct copies, R sized to
    exceed twice the last-level cache) and effective GB/s of each call's algorithmic bytes."""
    out = {}
    for b in (2, 3, 8):
        cb, qb, kb = qlr.qweight_sizes(N_, K_, b)
        R = (2 * MALL_BYTES) // (cb + qb + kb) + 1
        qws = torch.empty(qlr.workspace_bytes(qlr.OP_QUANTIZE), dtype=torch.uint8, device=dev)
        ws = torch.empty(max(qlr.workspace_bytes(qlr.OP_LINEAR, 1, N_, K_, R_), 16), dtype=torch.uint8, device=dev)
        y = torch.empty((1, N_), dtype=torch.bfloat16, device=dev)
        layers = [qlr.quantize(W, b, ws=qws) for _ in range(R)]
        rec = {}
        for name, mk in (("base", lambda q: qlr.LinearCall(x1, q, out=y)),
                         ("adapter", lambda q: qlr.LinearCall(x1, q, A0, B0, scale, out=y, ws=ws))):
            calls = [mk(q) for q in layers]
            for c in calls:
                c()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.current_stream(dev)):
                for c in calls:
                    c()
            g.replay()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                g.replay()
            e.record()
            torch.cuda.synchronize()
            us = s.elapsed_time(e) * 1e3 / (reps * R)
            nbytes = decode_bytes(b=b, r=R_ if name == "adapter" else 0)
            rec[name] = {"us_per_call": round(us, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "bytes_per_call": nbytes}
        rec["layers"] = R
        out[str(b)] = rec
        del layers
    return out



class _YCall:
    """A prepared mixed call seen as one call with one output tensor (its outputs concatenated
    for the graph-replay check)."""

    def __init__(self, mc):
        self.mc = mc
        self.y = None

    def __call__(self):
        ys = self.mc()
        if self.y is None:
            self.y = _Cat(ys)
        return ys


class _Cat:
    def __init__(self, ys):
        self.ys = ys

    def clone(self):
        return [y.clone() for y in self.ys]

    def zero_(self):
        for y in self.ys:
            y.zero_()

    def equal(self, ref):
        import torch
        return all(torch.equal(a, b) for a, b in zip(self.ys, ref))


def time_sequence(torch, calls, stream, graph: bool, reps: int = 5):
    """Median over reps of the time of the calls back to back (a HIP graph of them when
    `graph`, checked against the eager outputs first), per call, in us."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    run = None
    if graph:
        ref = [c.y.clone() for c in calls]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in calls:
                c()
        for c in calls:
            c.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert all((c.y.equal(r0) if isinstance(c.y, _Cat) else torch.equal(c.y, r0))
                   for c, r0 in zip(calls, ref)), "graph replay differs from eager"
        run = g.replay
    else:
        def run():
            for c in calls:
                c()
    run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / len(calls))
    ts.sort()
    return ts[len(ts) // 2]


# The other single-linear workloads: 7B MLP projections (r64) and a 65B-class MLP projection (r64).
CONFIGS = {
    "mlp_up_11008x4096": ("up", (1, 16), 2048),
    "mlp_down_4096x11008": ("down", (1, 16), 2048),
    "big65_22016x8192": ("big65", (1,), 4096),
}


def bench_configs(torch, qlr, workloads, dev, stream, only=None, graph=True):
    """Decode and prefill of each workload in CONFIGS over R distinct copies of its quantized
    weight (R sized so the copies exceed twice the 256 MB last-level cache), with and without
    the adapter: per-call time, effective GB/s (decode) or TFLOP/s (prefill) and the roofline
    fraction of the adapter-free call (one GEMV / GEMM kernel)."""
    import numpy as np

    def to_dev(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    out = {}
    for name, (which, m_dec, m_pre) in CONFIGS.items():
        if only and name != only:
            continue
        lin = workloads.big65(1) if which == "big65" else workloads.mlp(which, 1)
        N, K, r = lin.N, lin.K, lin.r
        W = to_dev(lin.W, "f16")
        A, B = to_dev(lin.A, "bf16"), to_dev(lin.B, "bf16")
        cb, qb, kb = qlr.qweight_sizes(N, K, BITS)
        R = (2 * MALL_BYTES) // (cb + qb + kb) + 1
        qws = torch.empty(qlr.workspace_bytes(qlr.OP_QUANTIZE), dtype=torch.uint8, device=dev)
        layers = [qlr.quantize(W, BITS, ws=qws) for _ in range(R)]
        del W
        rec = {"N": N, "K": K, "bits": BITS, "rank": r, "layers": R}
        for M in tuple(m_dec) + (m_pre,):
            gen = torch.Generator(device=dev)
            gen.manual_seed(1000 + M)
            x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(qlr.workspace_bytes(qlr.OP_LINEAR, M, N, K, r), 16), dtype=torch.uint8, device=dev)
            decode = M <= 16
            for tag, adp in (("adapter", True), ("base", False)):
                calls = [qlr.LinearCall(x, q, A, B, lin.scale, out=y, ws=ws) if adp else qlr.LinearCall(x, q, out=y)
                         for q in layers]
                us = time_sequence(torch, calls, stream, graph=graph and decode)
                rr = r if adp else 0
                key = f"M{M}_{tag}"
                if decode:
                    nbytes = decode_bytes(M=M, N=N, K=K, r=rr)
                    gbs = nbytes / (us * 1e-6) / 1e9
                    rec[key] = {"us_per_call": round(us, 3), "gbs": round(gbs, 1), "bytes_per_call": nbytes,
                                "frac": round(gbs / HBM_PEAK_GBS, 4)}
                else:
                    fl = prefill_flops(M=M, N=N, K=K, r=rr)
                    tfs = fl / (us * 1e-6) / 1e12
                    rec[key] = {"us_per_call": round(us, 3), "tflops": round(tfs, 1), "flops_per_call": fl,
                                "frac": round(tfs / BF16_PEAK_TFLOPS, 4)}
                del calls
            del x, y, ws
        del layers
        torch.cuda.empty_cache()
        out[name] = rec
    return out


def build_mixed(torch, qlr, workloads, dev):
    """The mixed stack at full size: 32 layers x 7 independent linears with per-linear
    (bits, rank) drawn by the stack's seed, M = 512, inputs drawn on the GPU by the seeded
    generator the full-size parity test uses (W N(0, 0.02^2) fp16, A N(0, 1/K),
    B N(0, 0.01^2) bf16, x N(0, 1) bf16), quantized once.  Returns the prepared M = 512
    call, its flops, the prepared decode call (the same layers at M = 1: each x's first
    row) and its algorithmic bytes."""
    qws = torch.empty(qlr.workspace_bytes(qlr.OP_QUANTIZE), dtype=torch.uint8, device=dev)
    plan = workloads.mixed_plan()
    entries, flops, dbytes = [], 0, 0
    for i, (N, K, b, r) in enumerate(plan):
        N, K, b, r, alpha, W, x, A, B = workloads.device_mixed_linear(i, MIXED_M, dev, plan)
        qw = qlr.quantize(W, b, ws=qws)
        del W
        entries.append(dict(x=x, qw=qw, A=A, B=B, scale=alpha / r))
        flops += 2 * MIXED_M * N * K + 2 * MIXED_M * r * (K + N)
        dbytes += decode_bytes(M=1, N=N, K=K, b=b, r=r)
    dec = qlr.MixedCall([dict(e, x=e["x"][:1]) for e in entries], out_dtype=torch.bfloat16)
    return qlr.MixedCall(entries, out_dtype=torch.bfloat16), flops, len(entries), dec, dbytes


def single_call_latency(torch, layer, stream, reps: int = 25):
    """One call at a time (synchronized before and after, HIP events around it): the
    latency a lone call sees, median and min over reps, us."""
    res = {}
    for ph in ("decode", "decode_base", "prefill", "prefill_base"):
        call = layer[ph]
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(1e3 * e0.elapsed_time(e1))
        ts.sort()
        res[ph] = {"median_us": round(ts[len(ts) // 2], 3), "min_us": round(ts[0], 3)}
    return res


def device_copy(torch, dev, stream, decode_gbs, reps: int = 10):
    """A 1 GiB device-to-device copy (read + write counted), the bandwidth a plain
    streaming kernel reaches here; the decode figure is set against it."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    ts.sort()
    gbs = 2 * n / ts[len(ts) // 2] / 1e9
    del src, dst
    return {"bytes": 2 * n, "gbs": round(gbs, 1), "decode_vs_copy": round(decode_gbs / gbs, 4)}


def cpu_baseline(budget_s: float = 12.0):
    """The oracle (numpy float64) on the host cores, on a bounded sample."""
    import numpy as np
    import threadpoolctl

    import oracle
    import workloads

    lin = workloads.attn(M_DECODE)
    t0 = time.perf_counter()
    qw = oracle.quantize(lin.W.reshape(-1), "f16", BITS)
    t_quant = time.perf_counter() - t0
    reps, t_dec = 0, 0.0
    while t_dec < budget_s / 2 or reps == 0:
        t0 = time.perf_counter()
        wd = oracle.dequantize(qw.codes, qw.absmax_q8, qw.absmax_c, BITS, lin.W.size).reshape(N_, K_)
        oracle.linear(lin.x, "bf16", wd, lin.A, lin.B, "bf16", lin.scale)
        t_dec += time.perf_counter() - t0
        reps += 1
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    gbs = reps * decode_bytes() / t_dec / 1e9
    return {
        "value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
        "sample": f"one 4096x4096 4-bit r16 layer at M=1: oracle dequantize + float64 forward, "
                  f"{reps} reps ({t_dec:.1f} s); oracle quantize of that layer took {t_quant:.1f} s",
        "quantize_s": round(t_quant, 3),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=0, help="distinct layer copies (default: > 2x MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed-stack phase")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one elementwise copy of 256 MiB (counter calibration)")
    ap.add_argument("--counter-phases", action="store_true",
                    help="time only the fp16-adapter and base phases (one launch per layer of each roofline "
                         "kernel) and print their per-call times: for the counter runs")
    ap.add_argument("--eager", action="store_true",
                    help="no HIP graphs (every launch visible to per-dispatch counter collection)")
    ap.add_argument("--no-configs", action="store_true", help="skip the MLP and 65B workloads")
    ap.add_argument("--mixed-only", action="store_true",
                    help="time only the mixed stack (M = 512 eagerly, then M = 1 as a graph unless --eager) and exit")
    ap.add_argument("--config-only", choices=sorted(CONFIGS),
                    help="time only this workload (decode and prefill; eager when --eager) and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: write profiles/traffic.json from two rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from_counters(*args.traffic_from)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sharding is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from quantized_base_fine_amd import qlr

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # One stream of our own carries every call; prepared calls bind to it and the
    # graphs are captured on it.
    torch.cuda.set_stream(torch.cuda.Stream(dev))
    if args.mixed_only:
        st = torch.cuda.current_stream(dev)
        mc, fl, n, dec, dbytes = build_mixed(torch, qlr, workloads, dev)
        res = {"linears": n}
        for name, call, graph in (("M512", mc, False), ("M1", dec, not args.eager)):
            us = time_sequence(torch, [_YCall(call)], st, graph=graph, reps=3)
            res[name] = {"us_per_call": round(us, 2)}
            if name == "M512":
                res[name]["tflops"] = round(fl / (us * 1e-6) / 1e12, 1)
            else:
                res[name]["gbs"] = round(dbytes / (us * 1e-6) / 1e9, 1)
        print(json.dumps(res))
        return
    if args.config_only:
        if args.copy_calibration:
            src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
            torch.add(src, 0.0, out=torch.empty_like(src))
            torch.cuda.synchronize()
            del src
        res = bench_configs(torch, qlr, workloads, dev, torch.cuda.current_stream(dev), only=args.config_only,
                            graph=not args.eager)
        print(json.dumps(res))
        return
    cb, qb, kb = qlr.qweight_sizes(N_, K_, BITS)
    R = args.layers or (2 * MALL_BYTES) // (cb + qb + kb) + 1

    def to_dev(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    lin1 = workloads.attn(M_DECODE)
    linp = workloads.attn(M_PREFILL, W=lin1.W)
    W = to_dev(lin1.W, "f16")
    x1, xp = to_dev(lin1.x, "bf16"), to_dev(linp.x, "bf16")
    A0, B0 = to_dev(lin1.A, "bf16"), to_dev(lin1.B, "bf16")
    qws = torch.empty(qlr.workspace_bytes(qlr.OP_QUANTIZE), dtype=torch.uint8, device=dev)
    ws1 = torch.empty(max(qlr.workspace_bytes(qlr.OP_LINEAR, M_DECODE, N_, K_, R_), 16), dtype=torch.uint8, device=dev)
    wsp = torch.empty(max(qlr.workspace_bytes(qlr.OP_LINEAR, M_PREFILL, N_, K_, R_), 16), dtype=torch.uint8, device=dev)
    wdeq = torch.empty((N_, K_), dtype=torch.float32, device=dev)
    dyp = to_dev(workloads.upstream_grad(linp), "bf16")
    wsb = torch.empty(max(qlr.workspace_bytes(qlr.OP_LINEAR_BWD, M_PREFILL, N_, K_, R_), 16), dtype=torch.uint8,
                      device=dev)
    dxp = torch.empty((M_PREFILL, K_), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((R_, K_), dtype=torch.float32, device=dev)
    dB = torch.empty((N_, R_), dtype=torch.float32, device=dev)
    ad = workloads.dba_adapter(N_, K_, R_, 1, cfg=2)
    dba_t = [torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev) for a in (ad.b1, ad.b2)]
    dba_t += [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (ad.alpha, ad.beta, ad.gamma)]
    ws_d1 = torch.empty(qlr.workspace_bytes(qlr.OP_LINEAR_DBA, M_DECODE, N_, K_, R_), dtype=torch.uint8, device=dev)
    ws_dp = torch.empty(qlr.workspace_bytes(qlr.OP_LINEAR_DBA, M_PREFILL, N_, K_, R_), dtype=torch.uint8, device=dev)
    ws_o1 = torch.empty(max(qlr.workspace_bytes(qlr.OP_LINEAR_OUTLIERS, M_DECODE, N_, K_, R_), 16), dtype=torch.uint8,
                        device=dev)
    ws_op = torch.empty(qlr.workspace_bytes(qlr.OP_LINEAR_OUTLIERS, M_PREFILL, N_, K_, R_), dtype=torch.uint8,
                        device=dev)
    ws_os = torch.empty(qlr.workspace_bytes(qlr.OP_QUANTIZE_OUTLIERS, NNZ, N_, K_), dtype=torch.uint8, device=dev)
    ws_h1 = torch.empty(qlr.workspace_bytes(qlr.OP_LINEAR_WHA, M_DECODE, N_, K_), dtype=torch.uint8, device=dev)
    ws_hp = torch.empty(qlr.workspace_bytes(qlr.OP_LINEAR_WHA, M_PREFILL, N_, K_), dtype=torch.uint8, device=dev)
    wha_csr = workloads.wha_coefficients(N_, K_, WHA_NNZ, cfg=2, floor=8)
    F0 = qlr.sparse_from_csr(N_, K_, *wha_csr, dev)
    layers = []
    for _ in range(R):
        qw = qlr.QWeight.empty(N_, K_, BITS, dev)
        qo, so = qlr.quantize_outliers(W, BITS, NNZ, ws=ws_os)
        A, B = A0.clone(), B0.clone()
        y1 = torch.empty((M_DECODE, N_), dtype=torch.bfloat16, device=dev)
        yp = torch.empty((M_PREFILL, N_), dtype=torch.bfloat16, device=dev)
        layers.append(dict(
            qw=qw, qo=qo, so=so,
            wha_decode=None, wha_prefill=None,
            prefill=qlr.LinearCall(xp, qw, A, B, linp.scale, out=yp, ws=wsp),
            prefill_base=qlr.LinearCall(xp, qw, out=yp),
            decode=qlr.LinearCall(x1, qw, A, B, lin1.scale, out=y1, ws=ws1),
            decode_base=qlr.LinearCall(x1, qw, out=y1),
            backward=qlr.LinearBwdCall(dyp, xp, qw, A, B, linp.scale, dx=dxp, dA=dA, dB=dB, ws=wsb),
            backward_base=qlr.LinearBwdCall(dyp, xp, qw, dx=dxp),
            dba_decode=qlr.DbaCall(x1, qw, *dba_t, out=y1, ws=ws_d1),
            dba_prefill=qlr.DbaCall(xp, qw, *dba_t, out=yp, ws=ws_dp),
            ol_decode=qlr.OutliersCall(x1, qo, so, A, B, lin1.scale, out=y1, ws=ws_o1),
            ol_prefill=qlr.OutliersCall(xp, qo, so, A, B, linp.scale, out=yp, ws=ws_op)))
        # each layer has its own coefficient arrays (a copy of one draw), like its own weight
        F = qlr.Sparse(N_, K_, F0.nnz, F0.row_ptr.clone(), F0.col.clone(), F0.val.clone())
        layers[-1]["wha_decode"] = qlr.WhaCall(x1, qw, F, K_, out=y1, ws=ws_h1)
        layers[-1]["wha_prefill"] = qlr.WhaCall(xp, qw, F, K_, out=yp, ws=ws_hp)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for L in layers:  # correctness of the inputs does not depend on the timed loop
        qlr.quantize(W, BITS, out=L["qw"], ws=qws)
    stream = torch.cuda.current_stream(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def qlr_deq(qw, out):
        import ctypes as C
        cw = qw.c_struct()
        qlr.check(qlr.lib().qlr_dequantize(C.byref(cw), out.data_ptr(), qlr.QLR_F32,
                                           C.c_void_p(stream.cuda_stream)))

    def quantize_all():
        for L in layers:
            qlr.quantize(W, BITS, out=L["qw"], ws=qws, blocking=False)

    # The quantize phase runs as a HIP graph (launch-bound: two short kernels per
    # layer); it is checked against the eager result before timing.
    g_quant = None
    if not args.eager:
        ref_codes = layers[-1]["qw"].codes.clone()
        quantize_all()
        torch.cuda.synchronize()
        g_quant = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_quant, stream=stream):
            quantize_all()
        for _ in range(2):
            layers[-1]["qw"].codes.zero_()
            g_quant.replay()
            torch.cuda.synchronize()
            assert torch.equal(layers[-1]["qw"].codes, ref_codes), "graph replay differs from eager quantize"

    PHASES = ("prefill", "prefill_base", "decode", "decode_base", "backward", "backward_base", "dba_decode",
              "dba_prefill", "ol_decode", "ol_prefill", "wha_decode", "wha_prefill")
    if args.counter_phases:
        PHASES = PHASES[:6]
    mixed = None
    if not args.no_mixed:
        mixed, mixed_flops, mixed_n, mixed_dec, mixed_dec_bytes = build_mixed(torch, qlr, workloads, dev)
        mixed()
        torch.cuda.synchronize()

    # The decode phases (short, launch-bound calls) also run as HIP graphs of the
    # R prepared calls; every replay is checked against the eager outputs first.
    graphs = {}
    for ph in (() if args.eager else tuple(p for p in ("decode", "decode_base", "dba_decode", "ol_decode", "wha_decode")
                                            if p in PHASES)):
        for L in layers:
            L[ph]()
        torch.cuda.synchronize()
        ref = [L[ph].y.clone() for L in layers]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for L in layers:
                L[ph]()
        for _ in range(2):
            for L in layers:
                L[ph].y.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert all(torch.equal(L[ph].y, r0) for L, r0 in zip(layers, ref)), f"{ph}: graph replay differs"
        graphs[ph] = g

    def run_step(marks):
        """quantize (graph) -> dequantize -> the four linear phases, marks on `stream`."""
        marks[0].record(stream)
        if g_quant is not None:
            g_quant.replay()
        else:
            quantize_all()
        marks[1].record(stream)
        qlr_deq(layers[0]["qw"], wdeq)
        marks[2].record(stream)
        for i, ph in enumerate(PHASES):
            if ph in graphs:
                graphs[ph].replay()
            else:
                for L in layers:
                    L[ph]()
            marks[3 + i].record(stream)
        if mixed is not None:
            mixed()
            marks[3 + len(PHASES)].record(stream)

    # the outlier split of one layer (blocking: it reads the non-finite flags), timed on its own
    for _ in range(2):
        qlr.quantize_outliers(W, BITS, NNZ, out=layers[0]["qo"], sparse=layers[0]["so"], ws=ws_os)
    split_ms = []
    for _ in range(5):
        e0, e1 = ev(), ev()
        e0.record(stream)
        qlr.quantize_outliers(W, BITS, NNZ, out=layers[0]["qo"], sparse=layers[0]["so"], ws=ws_os)
        e1.record(stream)
        torch.cuda.synchronize()
        split_ms.append(e0.elapsed_time(e1))

    nmarks = 4 + len(PHASES)
    for _ in range(args.warmup):
        run_step([ev() for _ in range(nmarks)])
    recs = [[ev() for _ in range(nmarks)] for _ in range(args.steps)]  # created before timing
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start, end = ev(), ev()
    start.record(stream)
    for marks in recs:
        run_step(marks)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    total_ms = start.elapsed_time(end)

    phase_ms = {k: 0.0 for k in ("quantize", "dequantize") + PHASES + (("mixed",) if mixed else ())}
    for marks in recs:
        phase_ms["quantize"] += marks[0].elapsed_time(marks[1])
        phase_ms["dequantize"] += marks[1].elapsed_time(marks[2])
        for i, ph in enumerate(PHASES):
            phase_ms[ph] += marks[2 + i].elapsed_time(marks[3 + i])
        if mixed is not None:
            phase_ms["mixed"] += marks[2 + len(PHASES)].elapsed_time(marks[3 + len(PHASES)])
    S = args.steps
    mean = {p: 1e3 * phase_ms[p] / (S * R) for p in PHASES}  # average launch duration, us
    if args.counter_phases:
        print(json.dumps({"call_us": {p: round(v, 3) for p, v in mean.items()}}))
        return
    dec_gbs = S * R * decode_bytes() / (phase_ms["decode"] / 1e3) / 1e9
    pre_tfs = S * R * prefill_flops() / (phase_ms["prefill"] / 1e3) / 1e12
    q_gbs = S * R * quantize_bytes() / (phase_ms["quantize"] / 1e3) / 1e9
    deq_gbs = S * (N_ * K_ * (4 + BITS / 8) + N_ * K_ / 64) / (phase_ms["dequantize"] / 1e3) / 1e9
    q_us = 1e3 * phase_ms["quantize"] / (S * R)
    gemv_bytes = decode_bytes(r=0)
    gemm_flops = prefill_flops(r=0)
    gemv_ach = gemv_bytes / (mean["decode_base"] * 1e-6) / 1e9
    gemm_ach = gemm_flops / (mean["prefill_base"] * 1e-6) / 1e12
    bwd_tfs = S * R * backward_flops() / (phase_ms["backward"] / 1e3) / 1e12
    dx_flops = backward_flops(r=0)
    dx_ach = dx_flops / (mean["backward_base"] * 1e-6) / 1e12

    out = {
        "metric": METRIC,
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / S, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attn_proj_4096x4096_nf4_dq_r16", "N": N_, "K": K_, "bits": BITS,
                   "block": 64, "group": 256, "rank": R_, "alpha": ALPHA, "M_decode": M_DECODE,
                   "M_prefill": M_PREFILL, "layers_per_step": R, "w_dtype": "f16",
                   "x_dtype": "bf16", "y_dtype": "bf16", "outliers": "0.1% x20"},
        "value_prefill": round(pre_tfs, 2),
        "unit_prefill": "TFLOP/s",
        "call_us": {p: round(v, 3) for p, v in mean.items()},
        "phases_ms_per_step": {k: round(v / S, 4) for k, v in phase_ms.items()},
        "quantize_gbs": round(q_gbs, 1),
        "dequantize_gbs": round(deq_gbs, 1),
        "roofline": {
            "bound": "hbm", "kernel": "k_gemv (decode dequant GEMV, M=1, no adapter: one kernel per call)",
            "achieved": round(gemv_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gemv_ach / HBM_PEAK_GBS, 4), "launch_us": round(mean["decode_base"], 3),
            "bytes_per_launch": gemv_bytes, "traffic": traffic_from_profile("decode"),
        },
        "roofline_prefill": {
            "bound": "mfma", "kernel": "k_gemm (prefill dequant GEMM, M=2048, no adapter: one kernel per call)",
            "achieved": round(gemm_ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(gemm_ach / BF16_PEAK_TFLOPS, 4), "launch_us": round(mean["prefill_base"], 3),
            "flops_per_launch": gemm_flops, "traffic": traffic_from_profile("prefill"),
        },
        "roofline_quantize": {
            "bound": "hbm", "kernel": "quantize (flag clear + quantize, graph replay, per layer)",
            "achieved": round(quantize_bytes() / (q_us * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "launch_us": round(q_us, 3),
            "bytes_per_launch": quantize_bytes(),
        },
        "backward": {
            "workload": "attn_proj_4096x4096_nf4_dq_r16 backward at M=2048 (dy bf16, dx bf16, dA/dB fp32)",
            "flops_per_call": backward_flops(), "us_per_call": round(mean["backward"], 3),
            "value": round(bwd_tfs, 2), "unit": "TFLOP/s",
            "roofline": {
                "bound": "mfma", "kernel": "k_gemm TR (input gradient dy W', M=2048, no adapter: one kernel per call)",
                "achieved": round(dx_ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dx_ach / BF16_PEAK_TFLOPS, 4), "launch_us": round(mean["backward_base"], 3),
                "flops_per_launch": dx_flops, "traffic": traffic_from_profile("backward"),
            },
        },
        "dba": {
            "workload": "attn_proj_4096x4096_nf4_dq with a double-binary adapter (R=16, l=1) instead of the fp16 one",
            "decode_us": round(mean["dba_decode"], 3),
            "decode_gbs": round(dba_bytes() / (mean["dba_decode"] * 1e-6) / 1e9, 1),
            "decode_bytes_per_call": dba_bytes(),
            "prefill_us": round(mean["dba_prefill"], 3),
            "prefill_tflops": round(dba_flops() / (mean["dba_prefill"] * 1e-6) / 1e12, 1),
            "adapter_bytes": (N_ * R_ + R_ * K_) // 8 + 2 * (N_ + R_ + K_),
            "fp16_adapter_bytes": 2 * R_ * (N_ + K_),
        },
        "outliers": {
            "workload": "attn_proj_4096x4096_nf4_dq_r16 with its 0.1% largest-|w| entries (k=16777) in a float32 "
                        "CSR side channel",
            "decode_us": round(mean["ol_decode"], 3),
            "decode_gbs": round(outlier_bytes() / (mean["ol_decode"] * 1e-6) / 1e9, 1),
            "decode_bytes_per_call": outlier_bytes(),
            "prefill_us": round(mean["ol_prefill"], 3),
            "prefill_tflops": round(outlier_flops() / (mean["ol_prefill"] * 1e-6) / 1e12, 1),
            "split_us": round(1e3 * sorted(split_ms)[len(split_ms) // 2], 1),
            "split_note": "qlr_quantize_outliers on one layer, median of 5, includes its flag read and sync",
        },
        "wha": {
            "workload": "attn_proj_4096x4096_nf4_dq with a Walsh-Hadamard adapter (one 4096-point transform, "
                        "131072 coefficients) instead of the fp16 one",
            "decode_us": round(mean["wha_decode"], 3),
            "decode_gbs": round(wha_bytes() / (mean["wha_decode"] * 1e-6) / 1e9, 1),
            "decode_bytes_per_call": wha_bytes(),
            "prefill_us": round(mean["wha_prefill"], 3),
            "prefill_tflops": round(wha_flops() / (mean["wha_prefill"] * 1e-6) / 1e12, 1),
            "adapter_bytes": 4 * (N_ + 1) + 8 * WHA_NNZ,
        },
        "wall_s": round(wall, 3),
    }
    if not args.eager:
        out["decode_by_bits"] = decode_by_bits(torch, qlr, W, x1, A0, B0, lin1.scale, dev)
    if not args.no_configs and not args.eager:
        out["configs"] = bench_configs(torch, qlr, workloads, dev, stream)
    if mixed is not None and not args.eager:
        # the stack at decode size: one mixed call per replay of a HIP graph, checked against eager first
        dec_us = time_sequence(torch, [_YCall(mixed_dec)], stream, graph=True)
        out["mixed_decode"] = {
            "workload": "the mixed stack at M=1 (each linear's first x row), one qlr_linear_fwd_mixed call",
            "bytes_per_call": mixed_dec_bytes, "us_per_call": round(dec_us, 2),
            "gbs": round(mixed_dec_bytes / (dec_us * 1e-6) / 1e9, 1),
            "frac": round(mixed_dec_bytes / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        }
    if mixed is not None:
        mixed_ms = phase_ms["mixed"] / S
        mixed_tfs = mixed_flops / (mixed_ms * 1e-3) / 1e12
        out["mixed"] = {
            "workload": f"mixed stack: 32 layers x 7 linears (4096x4096 x4, 11008x4096 x2, 4096x11008), "
                        f"bits and ranks by seed, M={MIXED_M}",
            "linears": mixed_n, "flops_per_call": mixed_flops, "ms_per_call": round(mixed_ms, 4),
            "value": round(mixed_tfs, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(mixed_tfs, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(mixed_tfs / BF16_PEAK_TFLOPS, 4)},
        }
    out["single_call"] = single_call_latency(torch, layers[0], stream)
    out["device_copy"] = device_copy(torch, dev, stream, out["value"])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
