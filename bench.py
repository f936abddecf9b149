"""Benchmark of the 2:4 decode-shaped SpMM hot path on one MI355X.

Workload (the shape the headline metric is quoted on): A 4096 x 4096 fp16 ~ N(0, 0.02),
pruned 2:4 along K; B 4096 x N fp16 ~ N(0, 1) for N in {8, 16, 32}; fp32 accumulation,
fp16 output. One step = 2:4 prune/encode of A followed by the SpMM with each of the
three B. By default A is encoded into the operand-major layout (snm_prune_encode_nm_tiled
/ snm_spmm_nm_tiled) and B is stored as decode activations X[N][K] (column-major B);
--a-layout canonical and --b-layout row select the other paths.
Inputs rotate over 32 independent copies (> 1.5 GiB) so that the 256 MiB last-level cache
cannot serve them: every step streams its operands from HBM.

Prints one JSON line. `value` is dense-equivalent TFLOP/s of the whole step (2*R*K*N
summed over the three products, divided by the step time, encode included). The
`roofline` object is that of the SpMM kernel: algorithmic HBM bytes of its launches
(values + metadata + B + Y) over their total duration measured with HIP events on the
launch stream, against 8 TB/s. `cpu_baseline` times the float64 NumPy oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_SPARSE_PEAK_TFLOPS = 5000.0
METRIC = "N:M SpMM dense-equiv TFLOP/s + HBM GB/s vs roofline, fp16, 1 MI355X"

R, K, NS = 4096, 4096, (8, 16, 32)
NROT = 32


def spmm_bytes(n: int) -> int:
    return R * (K // 2) * 2 + R * (K // 8) + K * n * 2 + R * n * 2


ENCODE_BYTES = R * K * 2 + R * (K // 2) * 2 + R * (K // 8)


def cpu_baseline(min_seconds: float = 10.0) -> dict:
    """The oracle as it stands, on the host cores: full-size encode + the three products,
    repeated until at least `min_seconds` have passed."""
    import platform
    import numpy as np
    import oracle
    import workloads
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    A, Bs = workloads.weight_and_activations(workloads.WORKLOADS["nm_decode"])
    flops = sum(2 * R * K * n for n in NS)
    t0 = time.perf_counter()
    reps = 0
    while True:
        v, m = oracle.prune_encode_nm(A)
        for B in Bs:
            oracle.spmm_nm(v, m, B)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full step(s) of the workload (prune/encode 4096x4096 + float64 "
                      f"products with N=8,16,32), {dt:.2f} s per step; BLAS threads={threads}; "
                      f"host {platform.processor() or platform.machine()}"}


def run_gpu(steps: int, warmup: int, layout: str = "col", a_layout: str = "tiled"):
    import numpy as np
    import torch
    import structured_sparse_matrix_amd as snm
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A0, Bs0 = workloads.weight_and_activations(workloads.WORKLOADS["nm_decode"])
    A0d = torch.from_numpy(A0).to(dev)
    B0d = [torch.from_numpy(b).to(dev) for b in Bs0]
    # 32 resident copies at distinct addresses
    As = [A0d.clone() for _ in range(NROT)]
    Bs = [[b.clone() for b in B0d] for _ in range(NROT)]
    # the same activations stored as X[N][K] (B column-major), the decode layout
    Xs = [[b.t().contiguous().t() for b in B0d] for _ in range(NROT)]
    if a_layout == "tiled":
        nv, nm = snm.nm_tiled_sizes(R, K)
        vals = [torch.empty((nv,), dtype=torch.float16, device=dev) for _ in range(NROT)]
        metas = [torch.empty((nm,), dtype=torch.uint8, device=dev) for _ in range(NROT)]
    else:
        vals = [torch.empty((R, K // 2), dtype=torch.float16, device=dev) for _ in range(NROT)]
        metas = [torch.empty((R, K // 8), dtype=torch.uint8, device=dev) for _ in range(NROT)]
    Ys = [[torch.empty((R, n), dtype=torch.float16, device=dev) for n in NS] for _ in range(NROT)]
    del A0d, B0d

    Bsel = Xs if layout == "col" else Bs

    def step(i, ev=None):
        j = i % NROT
        if ev is not None:
            ev[0].record()
        if a_layout == "tiled":
            snm.prune_encode_nm_tiled(As[j], vals[j], metas[j])
        else:
            snm.prune_encode_nm(As[j], vals[j], metas[j])
        if ev is not None:
            ev[1].record()
        for t in range(len(NS)):
            if a_layout == "tiled":
                snm.spmm_nm_tiled(vals[j], metas[j], R, Bsel[j][t], out=Ys[j][t])
            else:
                snm.spmm_nm(vals[j], metas[j], Bsel[j][t], out=Ys[j][t])
            if ev is not None:
                ev[2 + t].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + len(NS))] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(warmup + i, events[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    enc_ms = [e[0].elapsed_time(e[1]) for e in events]
    spmm_ms = [[e[1 + t].elapsed_time(e[2 + t]) for e in events] for t in range(len(NS))]
    return total_ms, wall, enc_ms, spmm_ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--b-layout", choices=("col", "row"), default="col",
                    help="B stored column-major (activations X[N][K], default) or row-major")
    ap.add_argument("--a-layout", choices=("tiled", "canonical"), default="tiled",
                    help="compressed A in the operand-major layout (default) or the canonical one")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np

    total_ms, wall, enc_ms, spmm_ms = run_gpu(args.steps, args.warmup, args.b_layout, args.a_layout)
    ms_per_step = total_ms / args.steps
    flops_step = sum(2 * R * K * n for n in NS)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    spmm_total_bytes = sum(spmm_bytes(n) for n in NS)
    spmm_avg_ms = [float(np.mean(x)) for x in spmm_ms]
    spmm_sum_ms = sum(spmm_avg_ms)
    achieved = spmm_total_bytes / (spmm_sum_ms * 1e-3) / 1e9
    enc_avg = float(np.mean(enc_ms))
    kernels = {
        "prune_encode_nm": {"avg_us": enc_avg * 1e3, "bytes": ENCODE_BYTES,
                            "GB/s": ENCODE_BYTES / (enc_avg * 1e-3) / 1e9,
                            "hbm_frac": ENCODE_BYTES / (enc_avg * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    for n, t in zip(NS, spmm_avg_ms):
        gbs = spmm_bytes(n) / (t * 1e-3) / 1e9
        kernels[f"spmm_nm_N{n}"] = {"avg_us": t * 1e3, "bytes": spmm_bytes(n), "GB/s": gbs,
                                    "hbm_frac": gbs / HBM_PEAK_GBS,
                                    "dense_equiv_TFLOP/s": 2 * R * K * n / (t * 1e-3) / 1e12}
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "2:4 SpMM decode-shaped: A 4096x4096 fp16 N(0,0.02) pruned 2:4 along K, "
                               "B 4096xN fp16 N(0,1), N in {8,16,32}; step = prune_encode_nm + 3 spmm_nm; "
                               "32 rotating input copies",
                   "R": R, "K": K, "N": list(NS), "rotating_copies": NROT,
                   "B_storage": "column-major (X[N][K])" if args.b_layout == "col" else "row-major (K x N)",
                   "A_storage": "operand-major (tiled)" if args.a_layout == "tiled" else "canonical"},
        "roofline": {"bound": "hbm", "kernel": "spmm_nm_tiled" if args.a_layout == "tiled" else "spmm_nm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "kernels": kernels,
        "wall_s_timed_region": wall,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
