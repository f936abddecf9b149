"""Benchmark of the 2:4 decode-shaped SpMM hot path on one MI355X.

Workload (the shape the headline metric is quoted on): A 4096 x 4096 fp16 ~ N(0, 0.02),
pruned 2:4 along K; B 4096 x N fp16 ~ N(0, 1) for N in {8, 16, 32}; fp32 accumulation,
fp16 output. One step = 2:4 prune/encode of A followed by the SpMM with each of the
three B. By default A is encoded into the operand-major layout (snm_prune_encode_nm_tiled
/ snm_spmm_nm_tiled) and B is stored as decode activations X[N][K] (column-major B);
--a-layout canonical and --b-layout row select the other paths. Inputs rotate over 32
independent copies (> 1.5 GiB) so that the 256 MiB last-level cache cannot serve them:
every step streams its operands from HBM.

Timed regions, each bracketed by synchronisation and one HIP event pair on the launch
stream:
  1. K whole steps -> ms_per_step and `value` (dense-equivalent TFLOP/s of the whole
     step: 2*R*K*N summed over the three products / step time, encode included). Steps
     are independent, so step i runs on stream i % S (--streams, default 2): two steps
     in flight hide one kernel's launch ramp and tail behind the other's work;
  2. for each kernel of the step, K back-to-back launches of that kernel alone over the
     same rotating inputs -> its average launch duration (an event between every launch
     would drain the queue and add a gap of its own). `roofline` is the SpMM kernel's:
     algorithmic HBM bytes of its three launches (values + metadata + B + Y) over their
     summed average durations, against 8 TB/s.
`roofline.traffic` is read from the committed counter summary in profiles/ when it was
taken on the current kernel source, else null. `cpu_baseline` times the float64 NumPy
oracle on the host.
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
METRIC = "N:M SpMM dense-equiv TFLOP/s + HBM GB/s vs roofline, fp16, 1 MI355X"

R, K, NS = 4096, 4096, (8, 16, 32)
NROT = 32
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_spmm_nm_tiled_decode_4096.json")
CALIBRATION_BYTES = 256 << 20


def spmm_bytes(n: int) -> int:
    return R * (K // 2) * 2 + R * (K // 8) + K * n * 2 + R * n * 2


ENCODE_BYTES = R * K * 2 + R * (K // 2) * 2 + R * (K // 8)


MFMA_SUMMARY = os.path.join(ROOT, "profiles", "mfma_spmm_vnm_128_2_16_8192x8192x4096.json")


def measured_mfma():
    """Matrix-core counters of the V:2:16 product from the committed rocprofv3 summary, or
    None if it is missing or was taken on a different kernel source."""
    try:
        with open(MFMA_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    from structured_sparse_matrix_amd.profiling import kernel_source_hash, WIDE_KERNEL_SOURCES
    if s.get("kernel_source_hash") != kernel_source_hash(WIDE_KERNEL_SOURCES):
        return None
    return {g.get("label", str(i)): {"mfma_busy_frac": g["mfma_busy_frac"],
                                     "fp16_matrix_ops": g["fp16_matrix_ops"]}
            for i, g in enumerate(s["groups"])}


def measured_traffic():
    """HBM bytes per SpMM launch from the committed rocprofv3 counter summary, or None if
    the summary is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    from structured_sparse_matrix_amd.profiling import kernel_source_hash
    if s.get("kernel_source_hash") != kernel_source_hash():
        return None
    return s.get("bytes_per_launch_avg")


def cpu_baseline(min_seconds: float = 10.0) -> dict:
    """The oracle as it stands, on the host cores: full-size encode + the three products,
    repeated until at least `min_seconds` have passed."""
    import platform
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads") or 1) for i in info) if info else 1
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
            "sample": f"{reps} full step(s) of the workload (2:4 prune/encode of 4096x4096 + float64 "
                      f"products with N=8,16,32 over the decoded matrix), {dt:.2f} s per step; "
                      f"BLAS threads={threads}; host {platform.processor() or platform.machine()}"}


def run_gpu(steps: int, warmup: int, b_layout: str, a_layout: str, calibration_copy: bool,
            nstreams: int = 2, submit: str = "eager"):
    import torch
    import structured_sparse_matrix_amd as snm
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if calibration_copy:
        # a plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.empty(CALIBRATION_BYTES // 2, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    A0, Bs0 = workloads.weight_and_activations(workloads.WORKLOADS["nm_decode"])
    A0d = torch.from_numpy(A0).to(dev)
    B0d = [torch.from_numpy(b).to(dev) for b in Bs0]
    # NROT resident copies at distinct addresses
    As = [A0d.clone() for _ in range(NROT)]
    if b_layout == "col":   # the same activations stored as X[N][K]
        Bsel = [[b.t().contiguous().t() for b in B0d] for _ in range(NROT)]
    else:
        Bsel = [[b.clone() for b in B0d] for _ in range(NROT)]
    if a_layout == "tiled":
        nv, nm = snm.nm_tiled_sizes(R, K)
        vals = [torch.empty((nv,), dtype=torch.float16, device=dev) for _ in range(NROT)]
        metas = [torch.empty((nm,), dtype=torch.uint8, device=dev) for _ in range(NROT)]
    else:
        vals = [torch.empty((R, K // 2), dtype=torch.float16, device=dev) for _ in range(NROT)]
        metas = [torch.empty((R, K // 8), dtype=torch.uint8, device=dev) for _ in range(NROT)]
    Ys = [[torch.empty((R, n), dtype=torch.float16, device=dev) for n in NS] for _ in range(NROT)]
    del A0d, B0d

    # The timed loops call the C entry points with their arguments bound once (checked
    # here, outside the timed region): the Python binding's per-call marshalling costs a
    # few microseconds of host time, as long as a decode-sized kernel, and would otherwise
    # leave the GPU waiting between back-to-back launches.
    from structured_sparse_matrix_amd._lib import load as load_lib, check
    lib = load_lib()
    # Steps are independent (each has its own rotating copy), so step i is enqueued on
    # stream i % nstreams: two steps in flight overlap one kernel's ramp and tail with the
    # other's work. A copy is reused every NROT steps, always on the same stream.
    assert NROT % nstreams == 0
    main_stream = torch.cuda.current_stream()
    streams = [main_stream] + [torch.cuda.Stream() for _ in range(nstreams - 1)]

    def bind(name, *args):
        fn = getattr(lib, name)
        check(name, fn(*args))
        return lambda: fn(*args)

    def bind_steps(strms):
        """The step's calls for every rotating copy j, bound to stream j % nstreams of strms."""
        enc_calls, mm_calls = [], []
        for j in range(NROT):
            stream = strms[j % nstreams].cuda_stream
            if a_layout == "tiled":
                enc_calls.append(bind("snm_prune_encode_nm_tiled", As[j].data_ptr(), R, K, K,
                                      vals[j].data_ptr(), metas[j].data_ptr(), stream))
            else:
                enc_calls.append(bind("snm_prune_encode_nm", As[j].data_ptr(), R, K, K,
                                      vals[j].data_ptr(), metas[j].data_ptr(), stream))
            row = []
            for t in range(len(NS)):
                B, Y = Bsel[j][t], Ys[j][t]
                lay = 1 if b_layout == "col" else 0
                ldb = B.stride(1) if lay == 1 else B.stride(0)
                if a_layout == "tiled":
                    row.append(bind("snm_spmm_nm_tiled", vals[j].data_ptr(), metas[j].data_ptr(), R, K,
                                    B.data_ptr(), NS[t], ldb, lay, Y.data_ptr(), NS[t], stream))
                else:
                    row.append(bind("snm_spmm_nm", vals[j].data_ptr(), metas[j].data_ptr(), R, K,
                                    B.data_ptr(), NS[t], ldb, lay, Y.data_ptr(), NS[t], 1, 0, 0, 0, 0, stream))
            mm_calls.append(row)

        def step(i):
            j = i % NROT
            enc_calls[j]()
            for t in range(len(NS)):
                mm_calls[j][t]()
        return enc_calls, mm_calls, step

    enc_calls, mm_calls, step = bind_steps(streams)

    def timed_steps():
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(main_stream)
        for st in streams[1:]:
            st.wait_stream(main_stream)
        for i in range(steps):
            step(warmup + i)
        for st in streams[1:]:
            main_stream.wait_stream(st)
        stop.record(main_stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop), time.perf_counter() - t0

    def timed_kernel(launch):
        """K back-to-back launches of one kernel over the rotating copies of the main stream,
        one event pair on that stream: an event between every launch would drain the queue
        and add its own gap."""
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(main_stream)
        for i in range(steps):
            launch((i * nstreams) % NROT)
        stop.record(main_stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    def encode(j):
        enc_calls[j]()

    def spmm(t):
        def launch(j):
            mm_calls[j][t]()
        return launch

    def timed_graph():
        """The K steps captured once into a HIP graph (the same streams, fork and join) and
        replayed: the timed region then holds no host launch cost, which otherwise (four
        launches of a few microseconds each per step of about 30 us) can leave the GPU
        waiting on a slow host. The graph holds only our kernels and stream waits."""
        cap = torch.cuda.Stream()
        gstreams = [cap] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
        _, _, gstep = bind_steps(gstreams)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for st in gstreams[1:]:
                st.wait_stream(cap)
            for i in range(steps):
                gstep(warmup + i)
            for st in gstreams[1:]:
                cap.wait_stream(st)
        g.replay()   # untimed first replay
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(main_stream)
        g.replay()
        stop.record(main_stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop), time.perf_counter() - t0

    for i in range(warmup):
        step(i)
    eager_ms, eager_wall = timed_steps()
    if submit == "graph":
        total_ms, wall = timed_graph()
    else:
        total_ms, wall = eager_ms, eager_wall
    enc_ms = timed_kernel(encode)
    spmm_ms = [timed_kernel(spmm(t)) for t in range(len(NS))]
    return total_ms, wall, enc_ms, spmm_ms, eager_ms


def bench_other(workload: str, steps: int, warmup: int) -> dict:
    """Per-kernel timings of the other workloads (not the headline line): each kernel is
    timed over K back-to-back launches with one HIP event pair."""
    import numpy as np
    import torch
    import structured_sparse_matrix_amd as snm
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[workload]
    nrot = 4

    def timed(launch):
        for i in range(warmup):
            launch(i % nrot)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            launch(i % nrot)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps * 1e-3   # seconds per launch

    out = {"workload": workload, "kernels": {}}
    if w.kind == "vnm":
        A, (B,) = workloads.weight_and_activations(w)
        Ad = [torch.from_numpy(A).to(dev) for _ in range(nrot)]
        Bd = [torch.from_numpy(B).to(dev) for _ in range(nrot)]
        enc = [snm.prune_encode_vnm(a, w.V, w.M) for a in Ad]
        Ys = [torch.empty((w.R, B.shape[1]), dtype=torch.float16, device=dev) for _ in range(nrot)]
        # encoders timed through the C entry points into outputs allocated once (the binding
        # allocates the three arrays on every call)
        from structured_sparse_matrix_amd._lib import load as load_lib, check
        lib = load_lib()
        stream = torch.cuda.current_stream().cuda_stream

        def enc_args(j, e):
            return (Ad[j].data_ptr(), w.R, w.K, w.K, w.V, w.M, e[0].data_ptr(), e[1].data_ptr(),
                    e[2].data_ptr(), stream)
        for j in range(nrot):
            check("snm_prune_encode_vnm", lib.snm_prune_encode_vnm(*enc_args(j, enc[j])))
        t_enc = timed(lambda j: lib.snm_prune_encode_vnm(*enc_args(j, enc[j])))
        t_mm = timed(lambda j: snm.spmm_vnm(*enc[j], Bd[j], w.V, w.M, out=Ys[j]))
        C = B.shape[1]
        Kp = 4 * (w.K // w.M)
        bytes_mm = w.R * (2 * w.K // w.M) * 2 + w.R * (w.K // w.M) // 2 + (w.R // w.V) * (w.K // w.M) * 4 \
            + w.K * C * 2 + w.R * C * 2
        bytes_enc = w.R * w.K * 2 + w.R * (2 * w.K // w.M) * 2 + w.R * (w.K // w.M) // 2 + (w.R // w.V) * (w.K // w.M) * 4
        out["kernels"]["prune_encode_vnm"] = {"avg_us": t_enc * 1e6, "GB/s": bytes_enc / t_enc / 1e9}
        def mm_stats(t):
            return {"avg_us": t * 1e6, "GB/s": bytes_mm / t / 1e9,
                    "dense_equiv_TFLOP/s": 2 * w.R * w.K * C / t / 1e12,
                    "smfmac_TFLOP/s": 2 * w.R * Kp * C / t / 1e12,
                    "sparse_mfma_frac": 2 * w.R * Kp * C / t / 1e12 / 5000.0,
                    "hbm_frac": bytes_mm / t / 1e9 / HBM_PEAK_GBS}
        out["kernels"]["spmm_vnm"] = mm_stats(t_mm)
        # the same arrays in the row-group interleaved storage (whole-line copies of A)
        enc_t = [snm.prune_encode_vnm_tiled(a, w.V, w.M) for a in Ad]
        t_enc_t = timed(lambda j: lib.snm_prune_encode_vnm_tiled(*enc_args(j, enc_t[j])))
        t_mm_t = timed(lambda j: snm.spmm_vnm_tiled(*enc_t[j], Bd[j], w.V, w.M, out=Ys[j]))
        out["kernels"]["prune_encode_vnm_tiled"] = {"avg_us": t_enc_t * 1e6, "GB/s": bytes_enc / t_enc_t / 1e9}
        out["kernels"]["spmm_vnm_tiled"] = mm_stats(t_mm_t)
        if workload == "vnm_128_2_16":
            # rocprofv3 counters of the same kernels (profiles/), None if the source changed
            out["counters"] = measured_mfma()
    elif w.kind == "attention":
        Q, Km, V = workloads.attention_qkv(w)
        Qd, Kd, Vd = (torch.from_numpy(x).to(dev) for x in (Q, Km, V))
        nb, L, d = Q.shape
        vals, meta = snm.sddmm_prune_nm(Qd, Kd, 1.0 / np.sqrt(d))
        O = torch.empty((nb, L, d), dtype=torch.float16, device=dev)
        nrot = 1
        # the SDDMMs are timed through the C entry points with their outputs allocated once
        # (the binding allocates 1.125 GiB per call, which the timed loop should not see)
        from structured_sparse_matrix_amd._lib import load as load_lib, check
        lib = load_lib()
        stream = torch.cuda.current_stream().cuda_stream
        sd_args = (Qd.data_ptr(), Kd.data_ptr(), nb, L, L, d, float(1.0 / np.sqrt(d)), vals.data_ptr(),
                   meta.data_ptr(), None, stream)
        check("snm_sddmm_prune_nm", lib.snm_sddmm_prune_nm(*sd_args))
        t_sd = timed(lambda j: lib.snm_sddmm_prune_nm(*sd_args))
        t_sm = timed(lambda j: snm.softmax_nm_rows(vals))
        t_pv = timed(lambda j: snm.spmm_nm(vals, meta, Vd, out=O))
        vbytes = nb * L * (L // 2) * 2
        mbytes = nb * L * (L // 8)
        out["kernels"]["sddmm_prune_nm"] = {"avg_us": t_sd * 1e6, "GB/s": (vbytes + mbytes + 2 * nb * L * d * 2) / t_sd / 1e9,
                                            "dense_TFLOP/s": 2 * nb * L * L * d / t_sd / 1e12}
        out["kernels"]["softmax_nm_rows"] = {"avg_us": t_sm * 1e6, "GB/s": 2 * vbytes / t_sm / 1e9}
        out["kernels"]["spmm_nm_PV"] = {"avg_us": t_pv * 1e6, "GB/s": (vbytes + mbytes + 2 * nb * L * d * 2) / t_pv / 1e9,
                                        "smfmac_TFLOP/s": 2 * nb * L * L * d / t_pv / 1e12}
        out["attention_total_us"] = (t_sd + t_sm + t_pv) * 1e6
        # fused-softmax variant: the SDDMM also writes each row's largest kept score, the
        # SpMM exponentiates and normalises on the fly (no separate pass over the scores)
        vals2, meta2, rmax = snm.sddmm_prune_nm_rowmax(Qd, Kd, 1.0 / np.sqrt(d))
        sdr_args = (Qd.data_ptr(), Kd.data_ptr(), nb, L, L, d, float(1.0 / np.sqrt(d)), vals2.data_ptr(),
                    meta2.data_ptr(), rmax.data_ptr(), stream)
        t_sdr = timed(lambda j: lib.snm_sddmm_prune_nm_rowmax(*sdr_args))
        t_pvs = timed(lambda j: snm.spmm_nm_softmax(vals2, meta2, rmax, Vd, out=O))
        out["kernels"]["sddmm_prune_nm_rowmax"] = {
            "avg_us": t_sdr * 1e6, "GB/s": (vbytes + mbytes + 4 * nb * L + 2 * nb * L * d * 2) / t_sdr / 1e9}
        out["kernels"]["spmm_nm_softmax_PV"] = {
            "avg_us": t_pvs * 1e6, "GB/s": (vbytes + mbytes + 4 * nb * L + 2 * nb * L * d * 2) / t_pvs / 1e9}
        out["attention_fused_total_us"] = (t_sdr + t_pvs) * 1e6
    return out


FP32_MFMA_PEAK_TFLOPS = 157.3


def bench_attention_variant(variant: str, steps: int, warmup: int) -> dict:
    """Per-kernel timings of the attention workload (batch 4 x 16 heads, seq 4096, head_dim 64)
    in bf16 with 2:4, or in fp32 with 1:2: unfused (SDDMM-prune, softmax, P.V) and fused
    (SDDMM with row maxima, P.V with the softmax inside). Each kernel: K back-to-back
    launches between one HIP event pair."""
    import numpy as np
    import torch
    import structured_sparse_matrix_amd as snm
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS["attention_2_4"]
    bf = variant == "attention_2_4_bf16"
    Q, Km, V = workloads.attention_qkv_typed(w, "bf16" if bf else "f32")
    if bf:
        Qd, Kd, Vd = (torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) for x in (Q, Km, V))
    else:
        Qd, Kd, Vd = (torch.from_numpy(x).to(dev) for x in (Q, Km, V))
    nb, L, d = Q.shape
    scale = 1.0 / np.sqrt(d)

    def timed(launch):
        for _ in range(warmup):
            launch()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            launch()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps * 1e-3

    esz = 2 if bf else 4
    vbytes = nb * L * (L // 2) * esz
    mbytes = nb * L * (L // 8 if bf else L // 4)
    qkv = nb * L * d * esz
    flops = 2 * nb * L * L * d
    out = {"workload": variant, "shape": "batch 4 x 16 heads, seq 4096, head_dim 64",
           "dtype": "bf16" if bf else "f32", "pattern": "2:4" if bf else "1:2", "kernels": {}}
    O = torch.empty((nb, L, d), dtype=Qd.dtype, device=dev)
    if bf:
        sddmm = lambda: snm.sddmm_prune_nm_bf16(Qd, Kd, scale)
        sddmm_r = lambda: snm.sddmm_prune_nm_bf16(Qd, Kd, scale, return_rowmax=True)
        vals, meta = sddmm()
        v2, m2, rmax = sddmm_r()
        soft = lambda: snm.softmax_nm_rows_bf16(vals)
        pv = lambda: snm.spmm_nm_bf16(vals, meta, Vd, out=O)
        pvs = lambda: snm.spmm_nm_softmax_bf16(v2, m2, rmax, Vd, out=O)
        peak, unit = 2500.0, "bf16 dense / sparse MFMA 2.5 / 5.0 PF/s"
    else:
        sddmm = lambda: snm.sddmm_prune_1of2_f32(Qd, Kd, scale)
        sddmm_r = lambda: snm.sddmm_prune_1of2_f32(Qd, Kd, scale, return_rowmax=True)
        vals, meta = sddmm()
        v2, m2, rmax = sddmm_r()
        soft = lambda: snm.softmax_nm_rows_f32(vals)
        pv = lambda: snm.spmm_1of2_f32(vals, meta, Vd, out=O)
        pvs = lambda: snm.spmm_1of2_f32(v2, m2, Vd, row_max=rmax, out=O)
        peak, unit = FP32_MFMA_PEAK_TFLOPS, "fp32 MFMA 157.3 TF/s"
    # the timed SDDMMs go through the C entry point with their outputs allocated once (the
    # binding allocates the score arrays on every call, which the timed loop should not see)
    from structured_sparse_matrix_amd._lib import load as load_lib, check
    lib = load_lib()
    entry = "snm_sddmm_prune_nm_bf16" if bf else "snm_sddmm_prune_1of2_f32"
    stream = torch.cuda.current_stream().cuda_stream
    fn = getattr(lib, entry)
    a_plain = (Qd.data_ptr(), Kd.data_ptr(), nb, L, L, d, float(scale), vals.data_ptr(), meta.data_ptr(),
               None, None, stream)
    a_rmax = (Qd.data_ptr(), Kd.data_ptr(), nb, L, L, d, float(scale), v2.data_ptr(), m2.data_ptr(),
              None, rmax.data_ptr(), stream)
    check(entry, fn(*a_plain))
    check(entry, fn(*a_rmax))
    t = {"sddmm": timed(lambda: fn(*a_plain)), "softmax": timed(soft), "pv": timed(pv),
         "sddmm_rowmax": timed(lambda: fn(*a_rmax)), "pv_softmax": timed(pvs)}
    io = vbytes + mbytes + 2 * qkv
    for name, byt, fl in (("sddmm", io, flops), ("softmax", 2 * vbytes, 0), ("pv", io, flops),
                          ("sddmm_rowmax", io + 4 * nb * L, flops), ("pv_softmax", io + 4 * nb * L, flops)):
        k = {"avg_us": t[name] * 1e6, "GB/s": byt / t[name] / 1e9, "hbm_frac": byt / t[name] / 1e9 / HBM_PEAK_GBS}
        if fl:
            k["TFLOP/s"] = fl / t[name] / 1e12
            k["mfma_frac"] = fl / t[name] / 1e12 / (peak if not bf else (2500.0 if "sddmm" in name else 5000.0))
        out["kernels"][name] = k
    out["mfma_peak"] = unit
    out["attention_total_us"] = (t["sddmm"] + t["softmax"] + t["pv"]) * 1e6
    out["attention_fused_total_us"] = (t["sddmm_rowmax"] + t["pv_softmax"]) * 1e6
    return out


def bench_sweep(steps: int, warmup: int, families=None) -> dict:
    """The general V:N:M sweep (VENOM, Sec. 4, Fig. 9 and Fig. 10 shapes, plus the GPT-3
    layer): per point, the V:2:M encode and the SpMM, each timed over K back-to-back
    launches of its C entry point with one event pair, and the dense fp16 product of the
    same shape (torch.matmul) for the speedup the pages report. Timing only: parity of
    every (V, M) is covered by the GPU tests. Inputs are drawn on the device from a seeded
    torch generator (A ~ N(0, 0.02), B ~ N(0, 1), fp16); they stay cache-warm between
    launches, as in the pages' microbenchmarks."""
    import torch
    import workloads
    from structured_sparse_matrix_amd import vnm_sizes
    from structured_sparse_matrix_amd._lib import load as load_lib, check

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = load_lib()
    stream = torch.cuda.current_stream().cuda_stream

    def bind(name, *args):
        fn = getattr(lib, name)
        check(name, fn(*args))
        return lambda: fn(*args)

    def timed(launch):
        for _ in range(warmup):
            launch()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            launch()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps * 1e-3

    gen = torch.Generator(device=dev)
    points = []
    for idx, (fam, R, K, C, V, M) in enumerate(workloads.vnm_sweep()):
        if families and fam not in families:
            continue
        gen.manual_seed(1000 + idx)
        lda = -(-K // 8) * 8
        Abuf = torch.zeros((R, lda), dtype=torch.float16, device=dev)
        Abuf[:, :K] = (torch.randn((R, K), generator=gen, device=dev) * 0.02).half()
        B = torch.randn((K, C), generator=gen, device=dev).half()
        nv, nmi, ncl = vnm_sizes(R, K, V, M)
        values = torch.empty((nv,), dtype=torch.float16, device=dev)
        midx = torch.empty((nmi,), dtype=torch.uint8, device=dev)
        colloc = torch.empty((ncl,), dtype=torch.uint8, device=dev)
        Y = torch.empty((R, C), dtype=torch.float16, device=dev)
        enc = bind("snm_prune_encode_vnm", Abuf.data_ptr(), R, K, lda, V, M, values.data_ptr(),
                   midx.data_ptr(), colloc.data_ptr(), stream)
        mm = bind("snm_spmm_vnm", values.data_ptr(), midx.data_ptr(), colloc.data_ptr(), R, K, V, M,
                  B.data_ptr(), C, C, Y.data_ptr(), C, stream)
        t_enc = timed(enc)
        t_mm = timed(mm)
        Ad = Abuf[:, :K].contiguous()
        Yd = torch.empty((R, C), dtype=torch.float16, device=dev)
        t_dense = timed(lambda: torch.matmul(Ad, B, out=Yd))
        Kc = 4 * (K // M)
        mm_bytes = R * (2 * K // M) * 2 + R * (K // M) // 2 + (R // V) * (K // M) * 4 + K * C * 2 + R * C * 2
        enc_bytes = R * K * 2 + R * (2 * K // M) * 2 + R * (K // M) // 2 + (R // V) * (K // M) * 4
        smf = 2 * R * Kc * C / t_mm / 1e12
        points.append({
            "family": fam, "R": R, "K": K, "C": C, "V": V, "M": M,
            "spmm_us": round(t_mm * 1e6, 2), "encode_us": round(t_enc * 1e6, 2),
            "dense_gemm_us": round(t_dense * 1e6, 2),
            "smfmac_TFLOP/s": round(smf, 1), "sparse_mfma_frac": round(smf / 5000.0, 4),
            "dense_equiv_TFLOP/s": round(2 * R * K * C / t_mm / 1e12, 1),
            "spmm_GB/s": round(mm_bytes / t_mm / 1e9, 1), "encode_GB/s": round(enc_bytes / t_enc / 1e9, 1),
            "speedup_vs_dense": round(t_dense / t_mm, 2), "ideal_speedup": M / 2})
        print(f"{fam:6s} {R:6d}x{K:6d}x{C:5d} V{V:<4d}M{M:<4d} spmm {t_mm * 1e6:8.1f} us  "
              f"{smf:7.1f} TF/s smfmac  dense {t_dense * 1e6:8.1f} us  x{t_dense / t_mm:5.2f} "
              f"(ideal {M / 2:g})  encode {t_enc * 1e6:7.1f} us", file=sys.stderr, flush=True)
        del Abuf, Ad, B, Y, Yd, values, midx, colloc
    return {"workload": "vnm_sweep", "points": points}


def bench_decode_ws(steps: int, warmup: int) -> dict:
    """The decode product with the split reduction (snm_spmm_nm_tiled_ws) beside the unsplit
    one (snm_spmm_nm_tiled) on 4096 x 4096 and on 4096 x 14336 (a feed-forward down
    projection), N = 8 / 16 / 32, B as X[N][K]. Each entry point is timed over K
    back-to-back launches with one event pair, twice in alternating order (the first heavy
    loop of a process runs slower); the minimum is reported. The compressed A rotates over
    copies of > 512 MiB so that the last-level cache cannot hold it."""
    import torch
    import structured_sparse_matrix_amd as snm
    from structured_sparse_matrix_amd._lib import load as load_lib, check

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = load_lib()
    stream = torch.cuda.current_stream().cuda_stream

    def timed(launch, nrot):
        for i in range(warmup):
            launch(i % nrot)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            launch(i % nrot)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps * 1e-3

    gen = torch.Generator(device=dev)
    points = []
    for (r, k) in ((4096, 4096), (4096, 14336)):
        gen.manual_seed(r + k)
        A = (torch.randn((r, k), generator=gen, device=dev) * 0.02).half()
        vt0, mt0 = snm.prune_encode_nm_tiled(A)
        del A
        nrot = max(2, -(-(512 << 20) // (vt0.numel() * 2 + mt0.numel())))
        vts = [vt0.clone() for _ in range(nrot)]
        mts = [mt0.clone() for _ in range(nrot)]
        for n in NS:
            X = torch.randn((n, k), generator=gen, device=dev).half()
            Y = torch.empty((r, n), dtype=torch.float16, device=dev)
            nb = snm.spmm_nm_tiled_ws_bytes(r, k, n)
            ws = torch.zeros((max(nb, 16),), dtype=torch.uint8, device=dev)

            def unsplit(i):
                check("snm_spmm_nm_tiled", lib.snm_spmm_nm_tiled(vts[i].data_ptr(), mts[i].data_ptr(), r, k,
                                                                 X.data_ptr(), n, k, 1, Y.data_ptr(), n, stream))

            def split(i):
                check("snm_spmm_nm_tiled_ws", lib.snm_spmm_nm_tiled_ws(
                    vts[i].data_ptr(), mts[i].data_ptr(), r, k, X.data_ptr(), n, k, Y.data_ptr(), n,
                    ws.data_ptr(), nb, stream))

            t = {"unsplit": [], "ws": []}
            for order in (("unsplit", "ws"), ("ws", "unsplit")):
                for name in order:
                    t[name].append(timed(unsplit if name == "unsplit" else split, nrot))
            by = r * (k // 2) * 2 + r * (k // 8) + k * n * 2 + r * n * 2
            pt = {"R": r, "K": k, "N": n, "workspace_bytes": nb, "split": nb > 0, "algorithmic_bytes": by}
            for name, ts in t.items():
                sec = min(ts)
                pt[name] = {"avg_us": sec * 1e6, "GB/s": by / sec / 1e9, "hbm_frac": by / sec / 1e9 / HBM_PEAK_GBS,
                            "dense_equiv_TFLOP/s": 2 * r * k * n / sec / 1e12}
            pt["speedup_ws_vs_unsplit"] = min(t["unsplit"]) / min(t["ws"])
            points.append(pt)
        del vts, mts
        torch.cuda.empty_cache()
    return {"workload": "nm_decode_long_k", "dtype": "fp16", "data": "synthetic",
            "config": {"workload": "2:4 decode SpMM, A R x K fp16 N(0,0.02) in the operand-major "
                                   "layout, X[N][K] fp16 N(0,1); split reduction vs unsplit"},
            "steps": steps, "warmup": warmup, "points": points}


def bench_bitmap(steps: int, warmup: int) -> dict:
    """Unstructured sparsity in the bitmap format (Coruscant, Sec. 3 and 5.2): OPT-30B /
    OPT-66B weight shapes (7168 and 9216 square) at 30 / 50 / 70 % sparsity, activations
    N = 8 / 16 / 32 stored column-major. Per point: the encoder (count + values), the
    SpMM, and the dense fp16 product of the same shape (torch.matmul, the pages' dense
    baseline), each over K back-to-back launches with one event pair. Inputs rotate over
    enough copies (> 256 MiB) that the last-level cache cannot hold them. A is drawn on the
    device (N(0, 0.02), seeded) and its smallest magnitudes are zeroed."""
    import torch
    from structured_sparse_matrix_amd import bitmap_sizes
    from structured_sparse_matrix_amd._lib import load as load_lib, check

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = load_lib()
    stream = torch.cuda.current_stream().cuda_stream

    def timed(launch, nrot):
        for i in range(warmup):
            launch(i % nrot)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            launch(i % nrot)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps * 1e-3

    gen = torch.Generator(device=dev)
    points = []
    for n in (7168, 9216):
        for sp in (0.3, 0.5, 0.7):
            gen.manual_seed(int(n + 100 * sp))
            A = (torch.randn((n, n), generator=gen, device=dev) * 0.02).half()
            mag = A.float().abs().flatten()
            k = int(sp * mag.numel())
            thr = mag.kthvalue(k).values if k > 0 else torch.tensor(-1.0, device=dev)
            A[A.float().abs() <= thr] = 0
            del mag
            nt, no = bitmap_sizes(n, n)
            bm = torch.empty((nt,), dtype=torch.int64, device=dev)
            off = torch.empty((no,), dtype=torch.int32, device=dev)
            check("snm_bitmap_count", lib.snm_bitmap_count(A.data_ptr(), n, n, n, bm.data_ptr(), off.data_ptr(), stream))
            nv = int(off[-1].item())
            fmt_bytes = nv * 2 + nt * 8 + no * 4
            nrot = max(2, -(-(300 << 20) // fmt_bytes))
            copies = []
            for _ in range(nrot):
                vals = torch.empty((nv,), dtype=torch.float16, device=dev)
                check("snm_bitmap_encode", lib.snm_bitmap_encode(A.data_ptr(), n, n, n, bm.data_ptr(),
                                                                 off.data_ptr(), vals.data_ptr(), stream))
                copies.append((bm.clone(), off.clone(), vals))
            enc = [(A.data_ptr(), bm.data_ptr(), off.data_ptr(), copies[0][2].data_ptr())]
            t_enc = timed(lambda j: (lib.snm_bitmap_count(enc[0][0], n, n, n, enc[0][1], enc[0][2], stream),
                                     lib.snm_bitmap_encode(enc[0][0], n, n, n, enc[0][1], enc[0][2], enc[0][3], stream)), 1)
            point = {"n": n, "sparsity": sp, "values": nv,
                     "format_bytes": fmt_bytes, "compression": fmt_bytes / (n * n * 2),
                     "encode_us": t_enc * 1e6, "N": {}}
            for N in (8, 16, 32):
                X = [torch.randn((N, n), generator=gen, device=dev).half() for _ in range(nrot)]
                Y = torch.empty((n, N), dtype=torch.float16, device=dev)
                args = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr(), n, n, X[j].data_ptr(), N, n, 1,
                         Y.data_ptr(), N, stream) for j, c in enumerate(copies)]
                check("snm_spmm_bitmap", lib.snm_spmm_bitmap(*args[0]))
                t_mm = timed(lambda j: lib.snm_spmm_bitmap(*args[j]), nrot)
                Ad = [A] + [A.clone() for _ in range(min(nrot, 3) - 1)]
                Yd = torch.empty((n, N), dtype=torch.float16, device=dev)
                t_dense = timed(lambda j: torch.matmul(Ad[j % len(Ad)], X[j].t(), out=Yd), nrot)
                byts = fmt_bytes + n * N * 2 + n * N * 2
                point["N"][str(N)] = {"spmm_us": t_mm * 1e6, "GB/s": byts / t_mm / 1e9,
                                      "hbm_frac": byts / t_mm / 1e9 / HBM_PEAK_GBS,
                                      "dense_gemm_us": t_dense * 1e6, "speedup_vs_dense": t_dense / t_mm}
                print(f"bitmap {n}x{n} s={sp} N={N}: spmm {t_mm * 1e6:7.1f} us {byts / t_mm / 1e9:7.0f} GB/s  "
                      f"dense {t_dense * 1e6:7.1f} us  x{t_dense / t_mm:4.2f}  (compression {fmt_bytes / (n * n * 2):.3f})",
                      file=sys.stderr, flush=True)
                del Ad, X
            points.append(point)
            del A, copies
            torch.cuda.empty_cache()
    return {"workload": "bitmap", "points": points}


def bench_energy(steps: int, warmup: int) -> dict:
    """Energy of the V:2:M encodings the GPU produces (VENOM, Sec. 5, Fig. 11): a 768 x 768
    Gaussian weight (seed 5; the size of the page's BERT-base query weight), V in
    {1, 16, 32, 64, 128}, N:M in {2:4, 2:5, 2:8, 2:10, 2:20, 2:40}, K zero-padded to a
    multiple of 4M. energy = sum |kept| / sum |A| in float64 on the host, from the
    encoder's output; each encode is also timed."""
    import numpy as np
    import torch
    import workloads
    from structured_sparse_matrix_amd import vnm_sizes
    from structured_sparse_matrix_amd._lib import load as load_lib, check

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = load_lib()
    stream = torch.cuda.current_stream().cuda_stream
    A = workloads.normal_f16(np.random.default_rng(5), (768, 768))
    total = float(np.abs(A.astype(np.float64)).sum())
    points = []
    for V in (1, 16, 32, 64, 128):
        for M in (4, 5, 8, 10, 20, 40):
            K = -(-768 // (4 * M)) * (4 * M)
            lda = -(-K // 8) * 8
            buf = torch.zeros((768, lda), dtype=torch.float16, device=dev)
            buf[:, :768] = torch.from_numpy(A).to(dev)
            nv, nmi, ncl = vnm_sizes(768, K, V, M)
            values = torch.empty((nv,), dtype=torch.float16, device=dev)
            midx = torch.empty((nmi,), dtype=torch.uint8, device=dev)
            colloc = torch.empty((ncl,), dtype=torch.uint8, device=dev)
            args = (buf.data_ptr(), 768, K, lda, V, M, values.data_ptr(), midx.data_ptr(),
                    colloc.data_ptr(), stream)
            check("snm_prune_encode_vnm", lib.snm_prune_encode_vnm(*args))
            for _ in range(warmup):
                lib.snm_prune_encode_vnm(*args)
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for _ in range(steps):
                lib.snm_prune_encode_vnm(*args)
            stop.record()
            torch.cuda.synchronize()
            kept = values.cpu().numpy().astype(np.float64)
            points.append({"V": V, "M": M, "sparsity": 1.0 - 2.0 / M,
                           "energy": float(np.abs(kept).sum()) / total,
                           "encode_us": start.elapsed_time(stop) / steps * 1e3})
    return {"workload": "energy", "matrix": "768x768 fp16 N(0,1), seed 5", "points": points}


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
    ap.add_argument("--calibration-copy", action="store_true",
                    help=f"copy {CALIBRATION_BYTES >> 20} MiB once before timing (counter calibration)")
    ap.add_argument("--workload", default="nm_decode",
                    help="nm_decode (the headline line) or vnm_64_2_8 / vnm_128_2_16 / attention_2_4 "
                         "(per-kernel timings only) or vnm_sweep (the general V:N:M sweep) or energy "
                         "(energy of the GPU's V:2:M encodings) or bitmap (unstructured sparsity, "
                         "bitmap format) or attention_2_4_bf16 / attention_1_2_f32 (the attention "
                         "workload in bf16 with 2:4, in fp32 with 1:2) or nm_decode_long_k (the decode "
                         "product with and without the split reduction, 4096 x 4096 and 4096 x 14336)")
    ap.add_argument("--streams", type=int, default=2,
                    help="decode steps in flight (step i on stream i %% S); kernel timings use one")
    ap.add_argument("--submit", choices=("eager", "graph"), default="eager",
                    help="timed decode steps launched one by one from the host (default) or "
                         "replayed from one captured HIP graph")
    ap.add_argument("--families", default="",
                    help="with --workload vnm_sweep: comma-separated subset of fig9,fig10,gpt3")
    args = ap.parse_args()
    if args.streams < 1 or NROT % args.streams != 0:
        ap.error(f"--streams must divide the {NROT} rotating input copies")
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.workload in ("attention_2_4_bf16", "attention_1_2_f32"):
        print(json.dumps(bench_attention_variant(args.workload, args.steps, args.warmup)))
        return
    if args.workload == "nm_decode_long_k":
        print(json.dumps(bench_decode_ws(args.steps, args.warmup)))
        return
    if args.workload == "bitmap":
        print(json.dumps(bench_bitmap(args.steps, args.warmup)))
        return
    if args.workload == "energy":
        print(json.dumps(bench_energy(args.steps, args.warmup)))
        return
    if args.workload == "vnm_sweep":
        fams = args.families.split(",") if args.families else None
        print(json.dumps(bench_sweep(args.steps, args.warmup, fams)))
        return
    if args.workload != "nm_decode":
        print(json.dumps(bench_other(args.workload, args.steps, args.warmup)))
        return
    import numpy as np

    total_ms, wall, enc_ms, spmm_ms, eager_ms = run_gpu(args.steps, args.warmup, args.b_layout,
                                                        args.a_layout, args.calibration_copy,
                                                        args.streams, args.submit)
    ms_per_step = total_ms / args.steps
    flops_step = sum(2 * R * K * n for n in NS)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    spmm_total_bytes = sum(spmm_bytes(n) for n in NS)
    spmm_avg_ms = list(spmm_ms)
    achieved = spmm_total_bytes / (sum(spmm_avg_ms) * 1e-3) / 1e9
    enc_avg = enc_ms
    enc_name = "prune_encode_nm_tiled" if args.a_layout == "tiled" else "prune_encode_nm"
    spmm_name = "spmm_nm_tiled" if args.a_layout == "tiled" else "spmm_nm"
    kernels = {
        enc_name: {"avg_us": enc_avg * 1e3, "bytes": ENCODE_BYTES,
                   "GB/s": ENCODE_BYTES / (enc_avg * 1e-3) / 1e9,
                   "hbm_frac": ENCODE_BYTES / (enc_avg * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    for n, t in zip(NS, spmm_avg_ms):
        gbs = spmm_bytes(n) / (t * 1e-3) / 1e9
        kernels[f"{spmm_name}_N{n}"] = {"avg_us": t * 1e3, "bytes": spmm_bytes(n), "GB/s": gbs,
                                        "hbm_frac": gbs / HBM_PEAK_GBS,
                                        "dense_equiv_TFLOP/s": 2 * R * K * n / (t * 1e-3) / 1e12}
    traffic = measured_traffic() if (args.a_layout, args.b_layout) == ("tiled", "col") else None
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
                               "B 4096xN fp16 N(0,1), N in {8,16,32}; step = 2:4 prune/encode + 3 SpMM; "
                               "32 rotating input copies",
                   "R": R, "K": K, "N": list(NS), "rotating_copies": NROT,
                   "streams": args.streams,
                   "submission": "one HIP graph of the K steps" if args.submit == "graph"
                                 else "eager launches",
                   "B_storage": "column-major (X[N][K])" if args.b_layout == "col" else "row-major (K x N)",
                   "A_storage": "operand-major (tiled)" if args.a_layout == "tiled" else "canonical"},
        "roofline": {"bound": "hbm", "kernel": spmm_name, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "basis": "algorithmic bytes of the three SpMM launches / their summed average "
                              "durations (HIP events around K back-to-back launches of each)"},
        "kernels": kernels,
        "wall_s_timed_region": wall,
        "eager_ms_per_step": eager_ms / args.steps,   # equals ms_per_step unless --submit graph
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
