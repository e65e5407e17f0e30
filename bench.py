"""Benchmark of the quantized-base + low-rank-adapter linear layer on one MI355X.

Workload: a 7B-class attention projection, W 4096 x 4096 fp16 ~ N(0, 0.02^2)
with 0.1% of entries x20 (outliers), 4-bit quantile codebook, blocks of 64,
double quantization in groups of 256; adapter rank 16, alpha 16, bf16;
x bf16 ~ N(0, 1) at M = 1 (decode) and M = 2048 (prefill).  Synthetic data
from the seeded generators in ``workloads``.

One step is one pass of the whole path over a stack of R distinct copies of
the layer (R chosen so the packed weights exceed twice the 256 MB last-level
cache, so the decode figure is HBM bandwidth, not cache bandwidth):
  quantize   all R weights (codes, 8-bit absmax codes, group steps)
  dequantize one weight to float32 (export path)
  decode     y = x W'^T + s (x A^T) B^T at M = 1 for all R layers
  prefill    the same at M = 2048 for all R layers
Each phase is timed with HIP events on the stream the kernels run on.

value       = decode effective GB/s (algorithmic bytes of all decode calls /
              decode phase time); bytes = codes + absmax codes + group steps
              + A + B + x + y.
value_prefill = prefill TFLOP/s with 2MNK + 2Mr(K+N) flops per call.
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one elementwise copy of 256 MiB (counter calibration)")
    args = ap.parse_args()
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
    layers = []
    for _ in range(R):
        layers.append(dict(qw=qlr.QWeight.empty(N_, K_, BITS, dev), A=A0.clone(), B=B0.clone(),
                           y1=torch.empty((M_DECODE, N_), dtype=torch.bfloat16, device=dev),
                           yp=torch.empty((M_PREFILL, N_), dtype=torch.bfloat16, device=dev)))
    qws = torch.empty(qlr.workspace_bytes(qlr.OP_QUANTIZE), dtype=torch.uint8, device=dev)
    # linear workspaces are zero-filled once before their first use
    ws1 = torch.zeros(max(qlr.workspace_bytes(qlr.OP_LINEAR, M_DECODE, N_, K_, R_), 16), dtype=torch.uint8, device=dev)
    wsp = torch.zeros(max(qlr.workspace_bytes(qlr.OP_LINEAR, M_PREFILL, N_, K_, R_), 16), dtype=torch.uint8, device=dev)
    wdeq = torch.empty((N_, K_), dtype=torch.float32, device=dev)
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
    ref_codes = layers[-1]["qw"].codes.clone()
    quantize_all()
    torch.cuda.synchronize()
    g_quant = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_quant):
        quantize_all()
    for _ in range(2):
        layers[-1]["qw"].codes.zero_()
        g_quant.replay()
        torch.cuda.synchronize()
        assert torch.equal(layers[-1]["qw"].codes, ref_codes), "graph replay differs from eager quantize"

    def run_step(record):
        """quantize (graph) -> dequantize -> prefill -> decode, phase marks on `stream`.

        Prefill is GPU-bound and queued before decode, so the host is far ahead
        of the GPU when the short decode calls run: the per-call events bracket
        GPU work only, with no host gaps between calls.
        """
        marks = [ev() for _ in range(5)]
        per = {"decode": [], "prefill": []}
        marks[0].record(stream)
        g_quant.replay()
        marks[1].record(stream)
        qlr_deq(layers[0]["qw"], wdeq)
        marks[2].record(stream)
        for L in layers:
            if record:
                a, b = ev(), ev()
                a.record(stream)
            qlr.linear(xp, L["qw"], L["A"], L["B"], linp.scale, out=L["yp"], ws=wsp)
            if record:
                b.record(stream)
                per["prefill"].append((a, b))
        marks[3].record(stream)
        for L in layers:
            if record:
                a, b = ev(), ev()
                a.record(stream)
            qlr.linear(x1, L["qw"], L["A"], L["B"], lin1.scale, out=L["y1"], ws=ws1)
            if record:
                b.record(stream)
                per["decode"].append((a, b))
        marks[4].record(stream)
        return marks, per

    for _ in range(args.warmup):
        run_step(False)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start, end = ev(), ev()
    start.record(stream)
    recs = [run_step(True) for _ in range(args.steps)]
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    total_ms = start.elapsed_time(end)

    phase_ms = {"quantize": 0.0, "dequantize": 0.0, "prefill": 0.0, "decode": 0.0}
    kern_ms = {"decode": [], "prefill": []}
    for marks, per in recs:
        phase_ms["quantize"] += marks[0].elapsed_time(marks[1])
        phase_ms["dequantize"] += marks[1].elapsed_time(marks[2])
        phase_ms["prefill"] += marks[2].elapsed_time(marks[3])
        phase_ms["decode"] += marks[3].elapsed_time(marks[4])
        for k, pairs in per.items():
            kern_ms[k] += [a.elapsed_time(b) for a, b in pairs]
    S = args.steps
    dec_gbs = S * R * decode_bytes() / (phase_ms["decode"] / 1e3) / 1e9
    pre_tfs = S * R * prefill_flops() / (phase_ms["prefill"] / 1e3) / 1e12
    q_gbs = S * R * quantize_bytes() / (phase_ms["quantize"] / 1e3) / 1e9
    deq_gbs = S * (N_ * K_ * (4 + BITS / 8) + N_ * K_ / 64) / (phase_ms["dequantize"] / 1e3) / 1e9
    dec_us = 1e3 * float(np.mean(kern_ms["decode"]))
    pre_us = 1e3 * float(np.mean(kern_ms["prefill"]))
    q_us = 1e3 * phase_ms["quantize"] / (S * R)
    dec_ach = decode_bytes() / (dec_us * 1e-6) / 1e9
    pre_ach = prefill_flops() / (pre_us * 1e-6) / 1e12

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
        "phases_ms_per_step": {k: round(v / S, 4) for k, v in phase_ms.items()},
        "quantize_gbs": round(q_gbs, 1),
        "dequantize_gbs": round(deq_gbs, 1),
        "roofline": {
            "bound": "hbm", "kernel": "decode linear M=1 (adapter product + fused dequant GEMV)",
            "achieved": round(dec_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dec_ach / HBM_PEAK_GBS, 4), "launch_us": round(dec_us, 3),
            "bytes_per_launch": decode_bytes(), "traffic": traffic_from_profile("decode"),
        },
        "roofline_prefill": {
            "bound": "mfma", "kernel": "prefill linear M=2048 (adapter product + fused dequant GEMM)",
            "achieved": round(pre_ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre_ach / BF16_PEAK_TFLOPS, 4), "launch_us": round(pre_us, 3),
            "flops_per_launch": prefill_flops(), "traffic": traffic_from_profile("prefill"),
        },
        "roofline_quantize": {
            "bound": "hbm", "kernel": "quantize (flag clear + quantize, graph replay, per layer)",
            "achieved": round(quantize_bytes() / (q_us * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "launch_us": round(q_us, 3),
            "bytes_per_launch": quantize_bytes(),
        },
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
