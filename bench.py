"""Benchmark of the Q8_0 matmul hot path on one MI355X.

Default workload (``--workload decode``): one decode step of a
Llama-3.2-1B-shaped model at batch 1 -- 16 layers of fused QKV [3072x2048],
O [2048x2048], fused gate||up [16384x2048], down [2048x8192], then the LM head
[128256x2048]; every distinct input is an fp32 N(0,1) row that is quantized
(q8_quantize_rows) right before the GEMV(s) that read it (q8_matmul).  Weights
are N(0, 0.02) fp32, quantized and repacked on the device before timing.  The
1.31 GB weight set exceeds every on-chip cache, so each step streams it from
HBM.  A step is captured once into a HIP graph and replayed.

Other workloads (same JSON line format): ``single`` (one 2048x2048 GEMV),
``batched`` (the decode step at m = 1..8 rows), ``prefill`` (the MFMA GEMM
shapes), ``moe`` (the routed-expert GEMVs).

Output: one JSON line with the metric, the roofline of the dominant kernel
(its average launch duration measured with HIP events on its own stream) and
the CPU oracle timed on the host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOPS


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode", "single", "batched", "prefill", "moe"])
    ap.add_argument("--m", type=int, default=1, help="rows per GEMV for --workload batched")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 1))
    return ap.parse_args()


def _sync():
    import torch
    torch.cuda.synchronize()


class Timer:
    """HIP events on one stream."""

    def __init__(self, stream):
        import torch
        self.stream = stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record(self.stream)

    def stop(self):
        self.b.record(self.stream)

    def ms(self):
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


# --------------------------------------------------------------------------
# decode step (and its batched variant)
# --------------------------------------------------------------------------

class DecodeStep:
    def __init__(self, m: int, threads: int, keep_host_rows: bool):
        import torch

        import oracle
        import workloads as wl
        from decode_q8_amd import q8

        self.torch, self.q8, self.wl = torch, q8, wl
        self.m = m
        self.mats = wl.decode_matrices()
        dev = torch.device("cuda", 0)
        self.w_packed, self.host_rows = [], []
        # weights: host fp32 (threaded generation) -> device -> quantize -> repack
        chunk = 8
        for c0 in range(0, len(self.mats), chunk):
            group = self.mats[c0:c0 + chunk]
            ws = wl.many(lambda mt: wl.weight(wl.BATCHED if m > 1 else wl.DECODE, mt.index, mt.n, mt.k,
                                              group=mt.layer), [(mt,) for mt in group], threads)
            for mt, w in zip(group, ws):
                wt = torch.from_numpy(w).to(dev)
                wr = q8.quantize(wt, q8.Q8_LAYOUT_ROWS)
                self.w_packed.append(q8.repack(wr, mt.n, mt.k))
                del wt, wr
                if keep_host_rows:
                    self.host_rows.append(_oracle_quantize(w, threads))
            del ws
        # activations: one fp32 input per distinct input, resident on the device
        self.inputs = []   # (fp32 device [m][k], quantized device buffer)
        self.host_x = []
        for layer in range(wl.LLAMA_LAYERS + 1):
            mats = [mt for mt in self.mats if mt.layer == layer]
            for mt in mats:
                x = wl.activation(wl.BATCHED if m > 1 else wl.DECODE, mt.act, m, mt.k, group=layer)
                xt = torch.from_numpy(x).to(dev)
                qb = torch.empty(q8.q8_quantized_bytes(m, mt.k), dtype=torch.uint8, device=dev)
                self.inputs.append((xt, qb))
                self.host_x.append(x)
        self.y = [torch.empty((m, mt.n), dtype=torch.float32, device=dev) for mt in self.mats]
        need = max(q8.q8_matmul_workspace_bytes(m, mt.n, mt.k) for mt in self.mats)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        self.weight_bytes = sum(mt.n * (mt.k // 32) * 34 for mt in self.mats)
        self.act_bytes = sum(m * (mt.k // 32) * 34 for mt in self.mats)
        self.out_bytes = sum(4 * m * mt.n for mt in self.mats)

    def run(self, stream, gemv_timers=None):
        q8 = self.q8
        s = stream.cuda_stream
        for i, mt in enumerate(self.mats):
            xt, qb = self.inputs[i]
            q8.q8_quantize_rows(xt, mt.k, self.m, mt.k, q8.Q8_LAYOUT_ACT, qb, s)
            if gemv_timers is not None:
                gemv_timers[i].start()
            q8.q8_matmul(qb, self.m, self.w_packed[i], q8.Q8_LAYOUT_PACKED, mt.n, mt.k, self.y[i], mt.n,
                         self.ws, self.ws.numel(), s)
            if gemv_timers is not None:
                gemv_timers[i].stop()

    def gemv_bytes(self, i):
        mt = self.mats[i]
        return mt.n * (mt.k // 32) * 34 + self.m * (mt.k // 32) * 34 + 4 * self.m * mt.n


def _oracle_quantize(w: np.ndarray, threads: int) -> np.ndarray:
    """Oracle quantization of a weight matrix into ROWS layout, split over row
    chunks on a thread pool (the C call releases the GIL)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    n, k = w.shape
    out = np.empty(n * (k // 32) * 34, np.uint8)
    step = max(1, (n + threads - 1) // threads)

    def part(r0):
        r1 = min(n, r0 + step)
        out[r0 * (k // 32) * 34: r1 * (k // 32) * 34] = oracle.quantize_rows(w[r0:r1], oracle.LAYOUT_ROWS)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(part, range(0, n, step)))
    return out


def bench_decode(args):
    import torch
    m = args.m if args.workload == "batched" else 1
    t0 = time.time()
    step = DecodeStep(m, args.threads, keep_host_rows=not args.no_cpu_baseline)
    prep_s = time.time() - t0
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    # eager reference outputs
    with torch.cuda.stream(stream):
        step.run(stream)
    torch.cuda.synchronize()
    eager = [y.clone() for y in step.y]

    # capture one step into a graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step.run(stream)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t = Timer(torch.cuda.current_stream())
    t.start()
    for _ in range(args.steps):
        g.replay()
    t.stop()
    total_ms = t.ms()
    torch.cuda.synchronize()
    ms_per_step = total_ms / args.steps
    # every replay wrote the same bits as the eager step
    for i, y in enumerate(step.y):
        if not torch.equal(y.view(torch.int32), eager[i].view(torch.int32)):
            raise RuntimeError(f"graph replay output {i} differs from the eager step")

    # dominant kernel: the GEMV, timed per launch with events on its stream
    timers = [Timer(stream) for _ in step.mats]
    gemv_ms = np.zeros(len(step.mats))
    reps = max(1, min(args.steps, 5))
    for _ in range(reps):
        with torch.cuda.stream(stream):
            step.run(stream, timers)
        torch.cuda.synchronize()
        gemv_ms += np.array([tm.ms() for tm in timers])
    gemv_ms /= reps
    gemv_bytes = np.array([step.gemv_bytes(i) for i in range(len(step.mats))], dtype=np.float64)
    avg_ms = float(gemv_ms.mean())
    achieved = float(gemv_bytes.mean() / (avg_ms * 1e-3) / 1e9)

    value = step.weight_bytes / (ms_per_step * 1e-3) / 1e9
    per_mat = {}
    for i, mt in enumerate(step.mats):
        key = mt.name
        b, ms = per_mat.get(key, (0.0, 0.0))
        per_mat[key] = (b + gemv_bytes[i], ms + gemv_ms[i])
    per_shape = {k: round(b / (ms * 1e-3) / 1e9, 1) for k, (b, ms) in per_mat.items()}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_decode(step, args.threads)

    out = {
        "metric": "Q8_0 matmul weight GB/s (%HBM peak) at M=1" if m == 1 else f"Q8_0 matmul weight GB/s at M={m}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xint8->int32, fp32 scale/sum",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": {
            "workload": f"Llama-3.2-1B-shaped decode step, batch {m}: 16 x (QKV 3072x2048, O 2048x2048, "
                        "gate||up 16384x2048, down 2048x8192) + LM head 128256x2048, Q8_0 packed",
            "m": m,
            "weight_bytes": step.weight_bytes,
            "launches_per_step": "%d quantize + %d GEMV (+ chain passes)" % (len(step.mats), len(step.mats)),
            "hip_graph": True,
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
            "gemv_GBs_by_matrix": per_shape,
            "prep_seconds": round(prep_s, 1),
        },
        "roofline": {
            "kernel": f"q8k::gemv_kernel<{m}, packed>",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_launch_us": round(avg_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": int(gemv_bytes.mean()),
        },
        "cpu_baseline": cpu,
    }
    return out


def cpu_baseline_decode(step, threads):
    """The oracle (quantize each input, then its matmul with fp64
    accumulation) over the whole decode step on the host cores."""
    import oracle
    t0 = time.time()
    for i, mt in enumerate(step.mats):
        xa = oracle.quantize_rows(step.host_x[i], oracle.LAYOUT_ACT)
        oracle.matmul(xa, step.m, step.host_rows[i], mt.n, mt.k, threads=threads)
    dt = time.time() - t0
    return {
        "value": round(step.weight_bytes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "one whole decode step (all 65 matrices, quantize + matmul), %.2f s" % dt,
    }


# --------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "only one GPU is measured: the row-sharded multi-GPU path is not built, "
                                   "so --gpus must be 1"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    if args.workload in ("decode", "batched"):
        out = bench_decode(args)
    else:
        raise SystemExit(f"workload {args.workload} not implemented yet")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
