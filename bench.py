"""Benchmark of the Q8_0 matmul hot path on one MI355X.

Default workload (``--workload decode``): one decode step of a
Llama-3.2-1B-shaped model at batch 1 -- 16 layers of fused QKV [3072x2048],
O [2048x2048], fused gate||up [16384x2048], down [2048x8192], then the LM head
[128256x2048].  Every distinct input is an fp32 N(0,1) row.  The whole step
is one q8_quantize_matmul_sequence launch (the 65 GEMVs in dependency order,
activation quantization fused into each, every output bit-identical to its own
q8_quantize_matmul launch, which the bench checks).  ``--per-matrix`` runs one
q8_quantize_matmul launch per matrix instead, ``--unfused`` separate
q8_quantize_rows and q8_matmul launches.  Weights are N(0, 0.02) fp32, quantized
(q8_quantize_rows) and repacked (q8_repack_weights) on the device before
timing.  The 1.31 GB weight set is larger than every on-chip cache, so each
step streams it from HBM.  A step is captured once into a HIP graph and
replayed.

Other workloads (same JSON line format): ``single`` (one 2048x2048 GEMV),
``batched`` (the decode step with ``--m`` rows per GEMV), ``prefill`` (the
int8-MFMA GEMM at M in {188, 752, 2048} x (N, K) in {(2048, 2048),
(8192, 2048), (2048, 8192)}), ``moe`` (a mixture-of-experts layer on the
device: router over 256 experts, top-8 of 16 tokens, fused gate||up and down
routed GEMVs, SwiGLU, weighted combine), ``norm`` (the fused residual + RMSNorm +
Q8_0 quantize producer at the prefill row counts, hidden 2048), ``kv`` (a
decode step's attention over a Q8 KV cache: 16 layers, 16 sequences x 4096
positions), ``copy`` (a device copy of 1 GiB, used to calibrate rocprofv3's
byte counters), ``read`` (the streaming-read ceiling, q8_stream_read over
1 GiB and over the decode step's, the LM head's and single matrices' sizes),
``quantize`` (weight quantization and repack of the LM head matrix, activation
quantization of 2048 prefill rows).

The JSON line carries the metric, the roofline of the dominant kernel (its
average launch duration measured with HIP events on the stream it runs on),
the 10th/50th/90th percentile of the per-replay times, and the CPU oracle
timed on the host on a bounded sample of the same workload.  The decode step's
line also carries the streaming-read ceiling measured in the same run on a
buffer of the step's weight bytes, and the step's fraction of it (the pages'
own yardstick for weight-streaming decode).
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
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "single", "batched", "prefill", "moe", "norm", "kv", "copy", "read",
                             "quantize"])
    ap.add_argument("--m", type=int, default=1, help="rows per GEMV for --workload batched")
    ap.add_argument("--unfused", action="store_true", help="decode: separate quantize and GEMV launches")
    ap.add_argument("--per-matrix", action="store_true",
                    help="decode: one fused quantize+GEMV launch per matrix instead of one launch per step")
    ap.add_argument("--layout", choices=["packed", "rows"], default="packed",
                    help="decode/batched: weight layout; rows (row-contiguous Q8_0) implies one launch per matrix")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ramp-seconds", type=float, default=0.3,
                    help="replays of each captured step before timing, by wall time, on top of --warmup: "
                         "the clocks ramp up over the first ~0.2 s of work")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode: leave out the prefill GEMM half of the metric")
    ap.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 1))
    return ap.parse_args()


class Timer:
    """A pair of HIP events recorded on one stream."""

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


def base_record(args, metric, value, unit, ms_per_step, dtype, config, roofline, cpu):
    return {
        "metric": metric,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_p10_p50_p90": [STEP_SPREAD.get(k) for k in ("p10", "p50", "p90")],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "clock_ramp": {"seconds": RAMP["seconds"], "replays": RAMP["replays"]},
    }


def hbm_roofline(kernel, bytes_per_launch, avg_ms):
    achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    return {
        "kernel": kernel,
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": None,
        "avg_launch_us": round(avg_ms * 1e3, 3),
        "algorithmic_bytes_per_launch": int(bytes_per_launch),
    }


# Kernel sources whose sha256 a committed profile summary must match before its
# counter-derived traffic is reported.
SEQ_SOURCES = ["decode_q8_amd/csrc/gemv_seq.hip", "decode_q8_amd/csrc/gemv_core.hpp", "decode_q8_amd/csrc/layout.hpp",
               "decode_q8_amd/csrc/device.hpp"]
GEMV_SOURCES = ["decode_q8_amd/csrc/gemv.hip", "decode_q8_amd/csrc/gemv_core.hpp", "decode_q8_amd/csrc/layout.hpp",
                "decode_q8_amd/csrc/device.hpp"]
GEMM_SOURCES = ["decode_q8_amd/csrc/gemm.hip", "decode_q8_amd/csrc/gemm_loop.inc", "decode_q8_amd/csrc/gemm_strip.inc"]
READ_SOURCES = ["decode_q8_amd/csrc/measure.hip", "decode_q8_amd/csrc/device.hpp"]

# Spread of the per-replay times of the most recent graph_time call (ms at the
# 10th, 50th and 90th percentile), reported beside the mean in every record.
STEP_SPREAD = {}
# Wall time of replays every graph_time call runs after its warm-up and before
# timing (set from --ramp-seconds), and how many replays that took last time.
RAMP = {"seconds": 0.3, "replays": 0}


def graph_time(run, stream, steps, warmup):
    """Capture run(stream) into a graph, replay warmup + steps times; returns
    (ms per replay, graph).  The mean comes from one event pair around the
    `steps` timed replays.  A second pass of `steps` replays, with an event
    between consecutive replays, gives the per-replay times whose percentiles
    go to STEP_SPREAD (the events themselves add a little time, so that pass
    is not the mean)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run(stream)
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    # clock ramp: keep replaying for RAMP["seconds"] of wall time, whatever
    # --warmup asked for, so the timed pass does not start on rising clocks
    t_ramp, ramp = time.time(), 0
    while time.time() - t_ramp < RAMP["seconds"]:
        for _ in range(16):
            g.replay()
        ramp += 16
        torch.cuda.synchronize()
    RAMP["replays"] = ramp
    t = Timer(torch.cuda.current_stream())
    t.start()
    for _ in range(steps):
        g.replay()
    t.stop()
    ms = t.ms() / steps
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(cur)
    for i in range(steps):
        g.replay()
        marks[i + 1].record(cur)
    marks[-1].synchronize()
    each = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
    STEP_SPREAD.clear()
    STEP_SPREAD.update({f"p{q}": round(float(np.percentile(each, q)), 5) for q in (10, 50, 90)})
    torch.cuda.synchronize()
    return ms, g


def replay_ms(graph, steps):
    """Mean ms per replay of an already captured graph over `steps` replays
    (one event pair on the current stream): an identical-control repeat of a
    timed configuration, taken later in the same run."""
    import torch
    t = Timer(torch.cuda.current_stream())
    t.start()
    for _ in range(steps):
        graph.replay()
    t.stop()
    ms = t.ms() / steps
    torch.cuda.synchronize()
    return ms


def read_ceiling_gbs(nbytes, steps=20, warmup=3):
    """The streaming-read ceiling: q8_stream_read over a fresh device buffer of
    nbytes (rounded down to 16), graph-replayed; GB/s by the mean replay."""
    import torch

    from decode_q8_amd import q8
    n = nbytes // 16 * 16
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    saved = dict(STEP_SPREAD)
    ms, _ = graph_time(lambda s: q8.q8_stream_read(buf, n, sink, s.cuda_stream), stream, steps, warmup)
    STEP_SPREAD.clear()
    STEP_SPREAD.update(saved)
    del buf
    torch.cuda.synchronize()
    return n / (ms * 1e-3) / 1e9


def per_launch_ms(run, count, stream, g_filler, reps):
    """Average duration of each of the `count` timed launches of run(stream,
    timers), measured with HIP events on `stream`.  Before each eager pass the
    stream is kept busy with replays of the captured step, so that the host
    has queued every event and launch of the pass before the GPU reaches them:
    the events then bracket the kernels alone, not host launch latency."""
    import torch
    total = np.zeros(count)
    for _ in range(reps):
        timers = [Timer(stream) for _ in range(count)]
        with torch.cuda.stream(stream):
            for _ in range(8):
                g_filler.replay()
            run(stream, timers)
        torch.cuda.synchronize()
        total += np.array([t.ms() for t in timers])
    return total / reps


def profiled_field(profile: str, source, key: str):
    """Field `key` of profiles/<profile> if that summary was taken from the
    current kernel source (sha256 of the source file, or of the listed files
    concatenated, matches); otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, val = line.split(":", 1)
            fields[k.strip()] = val.strip()
    h = hashlib.sha256()
    for src in ([source] if isinstance(source, str) else list(source)):
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if fields.get("source_sha256") != h.hexdigest() or key not in fields:
        return None
    return float(fields[key])


def profiled_traffic(profile: str, source, key: str = "traffic_bytes_per_launch"):
    """HBM bytes per launch recorded in profiles/<profile> (field `key`) by the
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if that summary was taken from the
    current kernel source (the sha256 of the source file, or of the listed
    files concatenated, matches); otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            name, val = line.split(":", 1)
            fields[name.strip()] = val.strip()
    sources = [source] if isinstance(source, str) else list(source)
    h = hashlib.sha256()
    for src in sources:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    sha = h.hexdigest()
    if fields.get("source_sha256") != sha or key not in fields:
        return None
    return int(fields[key])


def sequence_ms(run, stream, g_filler, reps):
    """Duration of one eager run(stream) measured by one event pair on
    `stream`, queued behind replays of the captured step (see per_launch_ms)."""
    import torch
    total = 0.0
    for _ in range(reps):
        t = Timer(stream)
        with torch.cuda.stream(stream):
            for _ in range(8):
                g_filler.replay()
            t.start()
            run(stream)
            t.stop()
        torch.cuda.synchronize()
        total += t.ms()
    return total / reps


def oracle_rows(w: np.ndarray, threads: int) -> np.ndarray:
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


def outputs_sha256(tensors) -> str:
    """sha256 of the outputs' bytes, in order (the Ember post's trial method
    records a hash of each mode's outputs next to its timing)."""
    import hashlib
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.detach().contiguous().cpu().numpy().tobytes())
    return h.hexdigest()


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the CPU baseline."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed_repeat(fn, min_seconds=10.0, max_reps=100000):
    """Run fn until min_seconds have passed (the CPU baseline's bounded sample:
    about 10 s of oracle work); returns (seconds per call, calls)."""
    reps, t0 = 0, time.time()
    while True:
        fn()
        reps += 1
        dt = time.time() - t0
        if dt >= min_seconds or reps >= max_reps:
            return dt / reps, reps


# --------------------------------------------------------------------------
# decode step (batch m) and the single GEMV
# --------------------------------------------------------------------------

class DecodeStep:
    """The matrices of a decode step and three ways to run them: "sequence"
    (one q8_quantize_matmul_sequence launch for the whole step), "fused" (one
    q8_quantize_matmul launch per matrix) and "unfused" (q8_quantize_rows then
    q8_matmul per matrix)."""

    def __init__(self, mats, workload, m, threads, keep_host_rows, mode, rows_layout=False):
        import torch

        import workloads as wl
        from decode_q8_amd import q8

        self.q8, self.m, self.mats, self.mode = q8, m, mats, mode
        self.fused = mode != "unfused"
        self.layout = q8.Q8_LAYOUT_ROWS if rows_layout else q8.Q8_LAYOUT_PACKED
        dev = torch.device("cuda", 0)
        self.w_packed, self.host_rows = [], []
        chunk = 8
        for c0 in range(0, len(mats), chunk):
            group = mats[c0:c0 + chunk]
            ws = wl.many(lambda mt: wl.weight(workload, mt.index, mt.n, mt.k, group=mt.layer),
                         [(mt,) for mt in group], threads)
            for mt, w in zip(group, ws):
                wt = torch.from_numpy(w).to(dev)
                wr = q8.quantize(wt, q8.Q8_LAYOUT_ROWS)
                self.w_packed.append(wr if rows_layout else q8.repack(wr, mt.n, mt.k))
                del wt, wr
                if keep_host_rows:
                    self.host_rows.append(oracle_rows(w, threads))
            del ws
        self.inputs, self.host_x = [], []
        for mt in mats:
            x = wl.activation(workload, mt.act, m, mt.k, group=mt.layer)
            xt = torch.from_numpy(x).to(dev)
            qb = torch.empty(q8.q8_quantized_bytes(m, mt.k), dtype=torch.uint8, device=dev)
            self.inputs.append((xt, qb))
            self.host_x.append(x)
        self.y = [torch.empty((m, mt.n), dtype=torch.float32, device=dev) for mt in mats]
        need = max(q8.q8_matmul_workspace_bytes(m, mt.n, mt.k) for mt in mats)
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        self.steps = [(self.inputs[i][0], mt.k, self.w_packed[i], mt.n, mt.k, self.y[i], mt.n)
                      for i, mt in enumerate(mats)]
        if mode == "sequence":
            need = q8.q8_sequence_workspace_bytes(self.steps, m)
            self.seq_ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        self.weight_bytes = sum(mt.n * (mt.k // 32) * 34 for mt in mats)
        torch.cuda.synchronize()

    def run(self, stream, gemv_timers=None):
        if self.mode == "sequence":
            self.q8.q8_quantize_matmul_sequence(self.steps, self.m, self.seq_ws, self.seq_ws.numel(),
                                                stream.cuda_stream)
        else:
            self.run_per_matrix(stream, gemv_timers)

    def run_per_matrix(self, stream, gemv_timers=None):
        q8 = self.q8
        s = stream.cuda_stream
        for i, mt in enumerate(self.mats):
            xt, qb = self.inputs[i]
            if not self.fused:
                q8.q8_quantize_rows(xt, mt.k, self.m, mt.k, q8.Q8_LAYOUT_ACT, qb, s)
            if gemv_timers is not None:
                gemv_timers[i].start()
            if self.fused:
                q8.q8_quantize_matmul(xt, mt.k, self.m, self.w_packed[i], self.layout, mt.n, mt.k,
                                      self.y[i], mt.n, self.ws, self.ws.numel(), s)
            else:
                q8.q8_matmul(qb, self.m, self.w_packed[i], self.layout, mt.n, mt.k, self.y[i], mt.n,
                             self.ws, self.ws.numel(), s)
            if gemv_timers is not None:
                gemv_timers[i].stop()

    def gemv_bytes(self, i):
        """Algorithmic bytes of matrix i's GEMV launch: weights once, the
        activation once (fp32 when quantized inside the kernel, Q8_0 bytes
        otherwise), the outputs once."""
        mt = self.mats[i]
        act = 4 * self.m * mt.k if self.fused else self.m * (mt.k // 32) * 34
        return mt.n * (mt.k // 32) * 34 + act + 4 * self.m * mt.n

    def oracle_step(self, threads):
        import oracle
        for i, mt in enumerate(self.mats):
            xa = oracle.quantize_rows(self.host_x[i], oracle.LAYOUT_ACT)
            oracle.matmul(xa, self.m, self.host_rows[i], mt.n, mt.k, threads=threads)


def bench_gemv_workload(args, mats, workload, m, label, allow_sequence=True):
    import torch

    from decode_q8_amd import q8
    t0 = time.time()
    rows = args.layout == "rows"
    mode = ("unfused" if args.unfused else
            ("fused" if args.per_matrix or rows or not allow_sequence else "sequence"))
    step = DecodeStep(mats, workload, m, args.threads, keep_host_rows=not args.no_cpu_baseline, mode=mode,
                      rows_layout=rows)
    prep_s = time.time() - t0
    stream = torch.cuda.Stream()

    with torch.cuda.stream(stream):
        step.run(stream)
    torch.cuda.synchronize()
    eager = [y.clone() for y in step.y]
    eager_sha = outputs_sha256(eager)
    ms_per_step, graph = graph_time(step.run, stream, args.steps, args.warmup)
    for i, y in enumerate(step.y):
        if not torch.equal(y.view(torch.int32), eager[i].view(torch.int32)):
            raise RuntimeError(f"graph replay output {i} differs from the eager step")
    if mode == "sequence":
        # a non-zero status word means a wait timed out: the outputs are undefined
        status = q8.sequence_status(step.seq_ws)
        if status != 0:
            raise RuntimeError(f"sequence status word {status}: a wait timed out, outputs undefined")
        # the one-launch step must equal the per-matrix launches bit for bit
        step.run_per_matrix(stream)
        torch.cuda.synchronize()
        for i, y in enumerate(step.y):
            if not torch.equal(y.view(torch.int32), eager[i].view(torch.int32)):
                raise RuntimeError(f"sequence output {i} differs from its own launch")

    # per-matrix breakdown (one launch per matrix, each bracketed by its own
    # events queued behind replays of the captured step)
    gemv_ms = per_launch_ms(step.run_per_matrix, len(step.mats), stream, g_filler=graph,
                            reps=max(1, min(args.steps, 10)))
    gemv_bytes = np.array([step.gemv_bytes(i) for i in range(len(step.mats))], dtype=np.float64)
    ctrl_ms = replay_ms(graph, args.steps)
    # the dominant kernel's average launch duration: one event pair around the
    # queued-ahead launches of one step, divided by the number of launches
    seq_ms = None
    if mode == "sequence":
        seq_ms = sequence_ms(step.run, stream, graph, reps=max(1, min(args.steps, 10)))
    elif mode == "fused":
        seq_ms = sequence_ms(step.run, stream, graph, reps=max(1, min(args.steps, 10))) / len(step.mats)

    value = step.weight_bytes / (ms_per_step * 1e-3) / 1e9
    per = {}
    for i, mt in enumerate(step.mats):
        b, ms = per.get(mt.name, (0.0, 0.0))
        per[mt.name] = (b + gemv_bytes[i], ms + gemv_ms[i])
    per_matrix = {k: round(b / (ms * 1e-3) / 1e9, 1) for k, (b, ms) in per.items()}

    cpu = None
    if not args.no_cpu_baseline:
        sec, reps_c = timed_repeat(lambda: step.oracle_step(args.threads), min_seconds=8.0)
        sec1, reps_1 = timed_repeat(lambda: step.oracle_step(1), min_seconds=6.0)
        cpu = {"value": round(step.weight_bytes / sec / 1e9, 3), "unit": "GB/s", "cores": args.threads,
               "kind": "oracle",
               "sample": f"the whole {label} ({len(mats)} matrices, quantize + matmul), {reps_c} runs, "
                         f"{sec:.3f} s each",
               "value_1_core": round(step.weight_bytes / sec1 / 1e9, 3),
               "sample_1_core": f"the same step on one thread, {reps_1} runs, {sec1:.3f} s each",
               "cpu_model": cpu_model()}

    launches = {"sequence": f"1 (q8_quantize_matmul_sequence over {len(mats)} fused quantize+GEMV steps)",
                "fused": f"{len(mats)} fused quantize+GEMV",
                "unfused": f"{len(mats)} quantize + {len(mats)} GEMV"}[mode]
    config = {
        "workload": label if not rows else label.replace("Q8_0 packed", "Q8_0 row-contiguous"),
        "m": m,
        "layout": args.layout,
        "weight_bytes": step.weight_bytes,
        "launches_per_step": launches,
        "hip_graph": True,
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "per_matrix_launch_GBs": per_matrix,
        "per_matrix_launch_us": {mt.name: round(float(gemv_ms[i]) * 1e3, 2) for i, mt in enumerate(step.mats)
                                 if mt.layer == 0 or mt.name == "lm_head"},
        "prep_seconds": round(prep_s, 1),
    }
    if len(mats) > 1:
        # the pages' yardstick: a pure streaming read of the same number of bytes
        ceiling = read_ceiling_gbs(step.weight_bytes)
        config["stream_read_ceiling_GBs"] = round(ceiling, 1)
        config["frac_of_stream_read_ceiling"] = round(value / ceiling, 4)
    # identical-control repeats of the timed step, after the other measurements
    # of this run (per-launch breakdown, oracle, read ceiling) ran in between;
    # a spread above 2% flags the run as unstable
    controls = [ms_per_step, ctrl_ms, replay_ms(graph, args.steps)]
    torch.cuda.synchronize()
    final_sha = outputs_sha256(step.y)
    if final_sha != eager_sha:
        raise RuntimeError("the step's outputs after the timed replays differ from the first eager pass")
    config["output_sha256"] = eager_sha
    spread = 100.0 * (max(controls) - min(controls)) / min(controls)
    config["control_ms_per_step"] = [round(c, 5) for c in controls]
    config["control_spread_pct"] = round(spread, 2)
    config["control_spread_over_2pct"] = bool(spread > 2.0)
    metric = ("Q8_0 matmul weight GB/s (%HBM peak) at M=1" if m == 1 else f"Q8_0 matmul weight GB/s at M={m}")
    if mode == "sequence":
        kname = "q8k::gemv_sequence_kernel<%d>" % m
        roof = hbm_roofline(kname, float(gemv_bytes.sum()), seq_ms)
        roof["timing"] = "one event pair around the step's single launch, queued ahead"
        if m == 1 and len(mats) == 65:
            roof["traffic"] = profiled_traffic("gemv_sequence_decode_step_llama1b.txt", SEQ_SOURCES)
    else:
        kname = "q8k::gemv_kernel<%d, %s, %s>" % (m, args.layout, "fp32 in" if step.fused else "int8 in")
        avg_ms = seq_ms if seq_ms is not None else float(gemv_ms.mean())
        roof = hbm_roofline(kname, float(gemv_bytes.mean()), avg_ms)
        roof["timing"] = ("one event pair around all launches of the step, queued ahead; per launch = total / "
                          "launches" if seq_ms is not None else "one event pair per launch, queued ahead")
        if step.fused and m == 1 and len(mats) == 65 and not rows:
            roof["traffic"] = profiled_traffic("gemv_decode_step_llama1b.txt", GEMV_SOURCES)
    return base_record(args, metric, value, "GB/s", ms_per_step, "int8xint8->int32, fp32 scale/sum", config,
                       roof, cpu)


HEADLINE_METRIC = "Q8_0 matmul weight GB/s (%HBM peak) at M=1; int8 TOPS (%MFMA peak) prefill"


def bench_decode(args):
    import workloads as wl
    m = args.m if args.workload == "batched" else 1
    label = (f"Llama-3.2-1B-shaped decode step, batch {m}: 16 x (QKV 3072x2048, O 2048x2048, "
             "gate||up 16384x2048, down 2048x8192) + LM head 128256x2048, Q8_0 packed")
    rec = bench_gemv_workload(args, wl.decode_matrices(), wl.BATCHED if m > 1 else wl.DECODE, m, label)
    if args.workload == "decode" and not args.no_prefill and not args.per_matrix and not args.unfused \
            and args.layout == "packed":
        # the metric's second half: the prefill GEMM, measured in the same run
        p = prefill_measure(args)
        rec["metric"] = HEADLINE_METRIC
        rec["prefill"] = p
        c = rec["config"]
        c["prefill_int8_TOPS"] = p["value"]
        c["prefill_frac_of_int8_peak"] = p["frac_of_int8_peak"]
        c["prefill_ms_per_step"] = p["ms_per_step"]
        for kname, r in p["rooflines"].items():
            key = "tiled" if kname.startswith("gemm_kernel") else "strip"
            c[f"prefill_{key}_kernel_TOPS"] = r["achieved"]
            c[f"prefill_{key}_kernel_frac"] = r["frac"]
        c["prefill_mfma_busy_pct"] = p["mfma_busy_pct"]
        if p["cpu_baseline"]:
            c["prefill_cpu_baseline_TOPS"] = p["cpu_baseline"]["value"]
    return rec


def bench_single(args):
    import workloads as wl
    mats = [wl.Matrix("w", 2048, 2048, 0, 0, 0)]
    return bench_gemv_workload(args, mats, wl.SINGLE, 1, "single Q8_0 GEMV, W 2048x2048, one activation row",
                               allow_sequence=False)


# --------------------------------------------------------------------------
# prefill GEMM
# --------------------------------------------------------------------------

def gemm_kernel_for(m: int, n: int) -> str:
    """The GEMM kernel libq8 runs for an m x n output (its rule: 128 x 128
    workgroup tiles when there are at least 256 of them, else 32 x 64 strips
    with k split across the waves)."""
    return "gemm_kernel" if ((m + 127) // 128) * ((n + 127) // 128) >= 256 else "gemm_strip_kernel"


PREFILL_ORDER_SEED = 20261202


def prefill_measure(args):
    """The nine prefill GEMM shapes (M in {188, 752, 2048} x (N, K) in
    {(2048, 2048), (8192, 2048), (2048, 8192)}): 256 sampled outputs of every
    shape checked against the oracle first, then the shapes captured in one
    graph in a seeded shuffled order and timed; per-launch durations by HIP
    events on the launch stream give the two kernels' rooflines."""
    import torch

    import oracle
    import workloads as wl
    from decode_q8_amd import q8
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream()
    cases = []
    for (n, k) in wl.PREFILL_NK:
        w = wl.weight(wl.PREFILL, n + k, n, k)
        wr = q8.quantize(torch.from_numpy(w).to(dev), q8.Q8_LAYOUT_ROWS)
        wp = q8.repack(wr, n, k)
        host_rows = oracle_rows(w, args.threads)
        for m in wl.PREFILL_M:
            x = wl.activation(wl.PREFILL, m, m, k, outliers=True)
            xq = q8.quantize(torch.from_numpy(x).to(dev), q8.Q8_LAYOUT_ACT)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            cases.append(dict(m=m, n=n, k=k, xq=xq, wp=wp, y=y, x=x, rows=host_rows))
    order = np.random.default_rng(PREFILL_ORDER_SEED).permutation(len(cases))
    cases = [cases[i] for i in order]
    torch.cuda.synchronize()

    def run(s, timers=None):
        for i, c in enumerate(cases):
            if timers is not None:
                timers[i].start()
            q8.q8_matmul(c["xq"], c["m"], c["wp"], q8.Q8_LAYOUT_PACKED, c["n"], c["k"], c["y"], c["n"], None, 0,
                         s.cuda_stream)
            if timers is not None:
                timers[i].stop()

    # parity first: sampled outputs of every shape against the oracle
    with torch.cuda.stream(stream):
        run(stream)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    pts = []
    for c in cases:
        xa = oracle.quantize_rows(c["x"], oracle.LAYOUT_ACT)
        mi, ni = rng.integers(0, c["m"], 256), rng.integers(0, c["n"], 256)
        y_ref, S = oracle.matmul_points(xa, c["m"], c["rows"], c["n"], c["k"], mi, ni)
        got = c["y"].cpu().numpy()[mi, ni].astype(np.float64)
        if np.any(np.abs(got - y_ref) > 1e-5 * S):
            raise RuntimeError(f"prefill M={c['m']} N={c['n']} K={c['k']}: outputs outside 1e-5*S of the oracle")
        pts.append((c, xa))

    first_sha = outputs_sha256([c["y"] for c in cases])
    ms_per_step, graph = graph_time(run, stream, args.steps, args.warmup)
    ms = per_launch_ms(run, len(cases), stream, graph, reps=max(1, min(args.steps, 10)))
    torch.cuda.synchronize()
    if outputs_sha256([c["y"] for c in cases]) != first_sha:
        raise RuntimeError("prefill outputs after the timed replays differ from the checked pass")
    ops = np.array([2.0 * c["m"] * c["n"] * c["k"] for c in cases])
    value = ops.sum() / (ms_per_step * 1e-3) / 1e12
    tops_by_case = {f"M{c['m']}_N{c['n']}_K{c['k']}": round(ops[i] / (ms[i] * 1e-3) / 1e12, 1)
                    for i, c in enumerate(cases)}
    kernels = {}
    for i, c in enumerate(cases):
        kname = gemm_kernel_for(c["m"], c["n"])
        o, t, names = kernels.get(kname, (0.0, 0.0, []))
        kernels[kname] = (o + ops[i], t + ms[i], names + [f"M{c['m']}_N{c['n']}_K{c['k']}"])
    mfma_busy = profiled_field("gemm_prefill_counters.txt", GEMM_SOURCES, "mfma_busy_pct")
    rooflines = {}
    for kname, (o, t, names) in kernels.items():
        achieved = o / (t * 1e-3) / 1e12
        tkey = "traffic_bytes_per_launch_" + ("tiled" if kname.startswith("gemm_kernel") else "strip")
        rooflines[kname] = {"kernel": "q8k::" + kname, "bound": "mfma", "achieved": round(achieved, 1),
                            "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                            "traffic": profiled_traffic("gemm_prefill.txt", GEMM_SOURCES, tkey),
                            "avg_launch_us": round(t / len(names) * 1e3, 3),
                            "algorithmic_ops_per_launch": int(o / len(names)), "shapes": names,
                            "timing": "one event pair per launch on the launch stream, queued ahead; "
                                      "achieved = total ops / total duration over its shapes"}
    cpu = None
    if not args.no_cpu_baseline:
        # bounded sample: 2048 outputs of every case, computed one by one
        rng = np.random.default_rng(0)
        sample = [(c, xa, rng.integers(0, c["m"], 2048), rng.integers(0, c["n"], 2048)) for c, xa in pts]

        def one_pass():
            for c, xa, mi, ni in sample:
                oracle.matmul_points(xa, c["m"], c["rows"], c["n"], c["k"], mi, ni)

        dt, reps = timed_repeat(one_pass, min_seconds=6.0)
        cpu_ops = sum(2.0 * 2048 * c["k"] for c in cases)
        cpu = {"value": round(cpu_ops / dt / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
               "sample": f"2048 outputs of each of the 9 prefill shapes, single-threaded, {reps} repetitions, "
                         f"{dt * reps:.1f} s", "cpu_model": cpu_model()}
    return {
        "metric": "Q8_0 prefill GEMM int8 TOPS (%MFMA peak)",
        "value": round(value, 3), "unit": "TOPS", "frac_of_int8_peak": round(value / INT8_PEAK_TOPS, 4),
        "ms_per_step": round(ms_per_step, 5), "ops_per_step": int(ops.sum()),
        "workload": "prefill GEMM: M in {188, 752, 2048} x (N, K) in {(2048, 2048), (8192, 2048), (2048, 8192)}, "
                    "Q8_0 packed weights, activations with 1% outlier channels x20",
        "oracle_check": "256 sampled outputs per shape within 1e-5 * sum|block terms|",
        "output_sha256": first_sha,
        "order": [f"M{c['m']}_N{c['n']}_K{c['k']}" for c in cases], "order_seed": PREFILL_ORDER_SEED,
        "tops_by_case": tops_by_case, "rooflines": rooflines, "mfma_busy_pct": mfma_busy,
        "cpu_baseline": cpu, "step_spread_ms_p10_p50_p90": [STEP_SPREAD.get(q) for q in ("p10", "p50", "p90")],
    }


def bench_prefill(args):
    p = prefill_measure(args)
    tiled = p["rooflines"].get("gemm_kernel")
    roof = dict(tiled) if tiled else dict(next(iter(p["rooflines"].values())))
    roof["mfma_busy_pct"] = p["mfma_busy_pct"]
    config = {"workload": p["workload"], "ops_per_step": p["ops_per_step"],
              "frac_of_int8_peak": p["frac_of_int8_peak"], "tops_by_case": p["tops_by_case"],
              "rooflines_by_kernel": p["rooflines"], "order": p["order"], "output_sha256": p["output_sha256"],
              "hip_graph": True}
    return base_record(args, p["metric"], p["value"], "TOPS", p["ms_per_step"],
                       "int8xint8->int32 (MFMA), fp32 scale/sum", config, roof, p["cpu_baseline"])


# --------------------------------------------------------------------------
# routed experts
# --------------------------------------------------------------------------

def bench_moe(args):
    """One mixture-of-experts layer on the device: router -> fused gate||up
    routed GEMV -> SwiGLU + quantize -> down routed GEMV -> weighted combine."""
    import torch

    import oracle
    import workloads as wl
    from decode_q8_amd import q8
    dev = torch.device("cuda", 0)
    E, T, K8, H, F = wl.MOE_EXPERTS, wl.MOE_TOKENS, wl.MOE_TOPK, wl.MOE_HIDDEN, wl.MOE_FFN
    P = T * K8
    logits = wl.router_logits(wl.MOE, T, E)
    ids_h = wl.routing(wl.MOE, T, E, K8)  # the same selection the device router makes (tested)
    used = sorted(set(int(e) for e in np.unique(ids_h)))
    s_gu, s_d = q8.q8_quantized_bytes(2 * F, H), q8.q8_quantized_bytes(H, F)
    # every expert has its place in HBM; only the routed ones are generated
    # (the kernels read nothing else)
    gu = torch.zeros(E * s_gu, dtype=torch.uint8, device=dev)
    dn = torch.zeros(E * s_d, dtype=torch.uint8, device=dev)
    host = {}
    for e0 in range(0, len(used), 8):
        es = used[e0:e0 + 8]
        gen = wl.many(lambda e: (wl.weight(wl.MOE, e, F, H, group=0), wl.weight(wl.MOE, e, F, H, group=1),
                                 wl.weight(wl.MOE, e, H, F, group=2)), [(e,) for e in es], args.threads)
        for e, (wg, wu, wd) in zip(es, gen):
            w_gu = np.concatenate([wg, wu])
            q8.q8_repack_weights(q8.quantize(torch.from_numpy(w_gu).to(dev), q8.Q8_LAYOUT_ROWS), 2 * F, H,
                                 gu[e * s_gu:(e + 1) * s_gu])
            q8.q8_repack_weights(q8.quantize(torch.from_numpy(wd).to(dev), q8.Q8_LAYOUT_ROWS), H, F,
                                 dn[e * s_d:(e + 1) * s_d])
            if not args.no_cpu_baseline and e in used[:2]:
                host[e] = (oracle_rows(w_gu, args.threads), oracle_rows(wd, args.threads))
        del gen
    x = wl.activation(wl.MOE, 100, T, H)
    xq = q8.quantize(torch.from_numpy(x).to(dev), q8.Q8_LAYOUT_ACT)
    lg = torch.from_numpy(logits).to(dev)
    ids = torch.empty((T, K8), dtype=torch.int32, device=dev)
    wts = torch.empty((T, K8), dtype=torch.float32, device=dev)
    y_gu = torch.empty((P, 2 * F), dtype=torch.float32, device=dev)
    hq = torch.empty(q8.q8_quantized_bytes(P, F), dtype=torch.uint8, device=dev)
    y_d = torch.empty((P, H), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    need = max(q8.q8_grouped_workspace_bytes(T, K8, E, 2 * F, H), q8.q8_grouped_workspace_bytes(T, K8, E, H, F))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stages = ["route", "gate_up", "swiglu", "down", "combine"]

    def run(s, timers=None):
        st = s.cuda_stream
        calls = [lambda: q8.q8_moe_route(lg, T, E, K8, True, ids, wts, st),
                 lambda: q8.q8_grouped_matmul(xq, T, 0, ids, T, K8, gu, E, s_gu, 2 * F, H, y_gu, ws, need, st),
                 lambda: q8.q8_swiglu_quantize(y_gu, 2 * F, y_gu[:, F:], 2 * F, P, F, hq, st),
                 lambda: q8.q8_grouped_matmul(hq, P, 1, ids, T, K8, dn, E, s_d, H, F, y_d, ws, need, st),
                 lambda: q8.q8_moe_combine(y_d, H, wts, T, K8, H, out, H, st)]
        for i, c in enumerate(calls):
            if timers is not None:
                timers[i].start()
            c()
            if timers is not None:
                timers[i].stop()

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run(stream)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_h), "device router disagrees with the host routing"
    assert int(ws[:4].view(torch.int32).cpu()[0]) == 0, "an expert id was out of range"
    ms_per_step, graph = graph_time(run, stream, args.steps, args.warmup)
    ms = per_launch_ms(run, len(stages), stream, graph, reps=max(1, min(args.steps, 10)))
    U = len(used)
    w_gu_bytes, w_d_bytes = float(U * s_gu), float(U * s_d)
    wbytes = w_gu_bytes + w_d_bytes
    value = wbytes / (ms_per_step * 1e-3) / 1e9
    # the dominant launch: the fused gate||up routed GEMV (weights, token rows, outputs)
    gu_bytes = w_gu_bytes + T * (H // 32) * 34 + 4 * P * 2 * F
    cpu = None
    if not args.no_cpu_baseline:
        # bounded sample: the whole layer for the pairs routed to the first two
        # experts, repeated for a few seconds
        sample = [(p, e) for e in host for p in range(P) if ids_h.reshape(-1)[p] == e]

        def oracle_sample():
            for p, e in sample:
                rows_gu, rows_d = host[e]
                xa = oracle.quantize_rows(x[p // K8:p // K8 + 1], oracle.LAYOUT_ACT)
                yg, _ = oracle.matmul(xa, 1, rows_gu, 2 * F, H, threads=args.threads)
                hq1 = oracle.swiglu_quantize(yg[:, :F], yg[:, F:])
                oracle.matmul(hq1, 1, rows_d, H, F, threads=args.threads)

        sec, reps = timed_repeat(oracle_sample)
        nb = len(sample) * (s_gu + s_d)
        cpu = {"value": round(nb / sec / 1e9, 3), "unit": "GB/s", "cores": args.threads, "kind": "oracle",
               "sample": f"gate||up, SwiGLU and down of the {len(sample)} pairs routed to 2 experts, "
                         f"{reps} repetitions"}
    config = {
        "workload": "MoE layer: router over 256 experts (top-8, softmax over the selected), fused gate||up "
                    "(2x 2048x7168) and down (7168x2048) routed GEMVs per expert, SwiGLU, weighted combine; "
                    "16 tokens, hidden 7168",
        "distinct_experts": U,
        "expected_distinct_experts": round(256 * (1 - (1 - 8 / 256) ** 16), 2),
        "weight_bytes_per_step": int(wbytes),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "us_by_stage": {name: round(float(ms[i]) * 1e3, 2) for i, name in enumerate(stages)},
        "GBs_by_gemv": {"gate_up": round(w_gu_bytes / (ms[1] * 1e-3) / 1e9, 1),
                        "down": round(w_d_bytes / (ms[3] * 1e-3) / 1e9, 1)},
        "hip_graph": True,
    }
    roof = hbm_roofline("q8k::grouped_gemv_kernel", gu_bytes, float(ms[1]))
    roof["traffic"] = profiled_traffic("grouped_gemv_moe.txt", GEMV_SOURCES)
    roof["note"] = ("the fused gate||up launch; its time includes the expert-grouping kernel that precedes the "
                    "GEMV in each call")
    return base_record(args, "Q8_0 routed-expert GEMV weight GB/s (%HBM peak)", value, "GB/s", ms_per_step,
                       "int8xint8->int32, fp32 scale/sum", config, roof, cpu)


# --------------------------------------------------------------------------
# fused residual + RMSNorm + quantization producer
# --------------------------------------------------------------------------

def norm_bytes(rows: int, k: int) -> int:
    """Algorithmic HBM bytes of one q8_rmsnorm_quantize launch: x, residual in
    and residual out (fp32), the int8 codes and fp16 scales, the fp32 gain."""
    return rows * k * (4 + 4 + 4 + 1) + rows * (k // 32) * 2 + 4 * k


def bench_norm(args):
    import torch

    import oracle
    import workloads as wl
    from decode_q8_amd import q8
    dev = torch.device("cuda", 0)
    k = wl.LLAMA_HIDDEN
    cases = []
    for rows in wl.NORM_ROWS:
        x, res, gain = wl.norm_inputs(wl.NORM, rows, rows, k)
        c = dict(rows=rows, k=k, x=x, res=res, gain=gain, xt=torch.from_numpy(x).to(dev),
                 rt=torch.from_numpy(res).to(dev), gt=torch.from_numpy(gain).to(dev),
                 ro=torch.empty((rows, k), dtype=torch.float32, device=dev),
                 q=torch.empty(q8.q8_quantized_bytes(rows, k), dtype=torch.uint8, device=dev))
        cases.append(c)
    torch.cuda.synchronize()
    # the producer is checked against the oracle before it is timed (full rows)
    for c in cases:
        q8.q8_rmsnorm_quantize(c["xt"], c["rt"], c["ro"], c["gt"], c["rows"], k, wl.NORM_EPS, c["q"])
        ro_ref, q_ref = oracle.rmsnorm_quantize(c["x"], c["res"], c["gain"], wl.NORM_EPS)
        torch.cuda.synchronize()
        assert np.array_equal(c["q"].cpu().numpy(), q_ref), f"rows={c['rows']}: codes differ from the oracle"
        assert np.array_equal(c["ro"].cpu().numpy().view(np.uint32), ro_ref.view(np.uint32))
    stream = torch.cuda.Stream()
    timed = cases[1:]  # the prefill launches; the decode row (cases[0]) is latency only
    assert cases[0]["rows"] == 1 and all(c["rows"] > 1 for c in timed)
    nbytes = np.array([norm_bytes(c["rows"], k) for c in timed], dtype=np.float64)
    # Every timed pass works on its own copy of the buffers, enough copies that
    # their footprint (>= 1 GiB) exceeds the GPU's caches (4 MB L2 per XCD,
    # 256 MB Infinity Cache): each launch reads its inputs from HBM, as a
    # producer reading a freshly written residual stream of a large model would
    # at worst.
    copies = max(2, int(np.ceil((1 << 30) / nbytes.sum())))
    sets = [[dict(c, xt=c["xt"].clone(), rt=c["rt"].clone(), ro=torch.empty_like(c["ro"]),
                  q=torch.empty_like(c["q"])) for c in cases] for _ in range(copies)]
    torch.cuda.synchronize()

    def run_cases(sel):
        def run(s, timers=None):
            for i, c in enumerate(sel):
                if timers is not None:
                    timers[i].start()
                q8.q8_rmsnorm_quantize(c["xt"], c["rt"], c["ro"], c["gt"], c["rows"], k, wl.NORM_EPS, c["q"],
                                       s.cuda_stream)
                if timers is not None:
                    timers[i].stop()
        return run

    # a step: the three prefill launches; one graph holds a step on every copy
    ms_all, graph = graph_time(run_cases([c for st in sets for c in st if c["rows"] > 1]), stream, args.steps,
                               args.warmup)
    ms_per_step = ms_all / copies
    # per-launch durations: one launch size over every copy, back to back in a
    # graph of its own (a launch of a few microseconds is shorter than the
    # overhead of an event pair around it)
    ms = np.array([graph_time(run_cases([st[i + 1] for st in sets]), stream, args.steps, 2)[0] / copies
                   for i in range(len(timed))])
    ms_row1 = graph_time(run_cases([st[0] for st in sets]), stream, args.steps, 2)[0] / copies
    value = nbytes.sum() / (ms_per_step * 1e-3) / 1e9
    big = int(np.argmax(nbytes))
    cpu = None
    if not args.no_cpu_baseline:
        c = timed[big]
        sec, reps = timed_repeat(lambda: oracle.rmsnorm_quantize(c["x"], c["res"], c["gain"], wl.NORM_EPS))
        cpu = {"value": round(norm_bytes(c["rows"], k) / sec / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the {c['rows']}-row launch, {reps} repetitions, single-threaded, {sec * reps:.1f} s"}
    config = {
        "workload": f"fused residual + RMSNorm + Q8_0 quantize: rows in {{188, 752, 2048}} x hidden {k} "
                    "(Llama-3.2-1B prefill tokens), residual stream with 1% outlier channels x20",
        "bytes_per_step": int(nbytes.sum()),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "GBs_by_rows": {str(c["rows"]): round(nbytes[i] / (ms[i] * 1e-3) / 1e9, 1) for i, c in enumerate(timed)},
        "decode_row_launch_us": round(float(ms_row1) * 1e3, 3),
        "buffer_copies": copies,
        "hip_graph": True,
    }
    roof = hbm_roofline("q8k::rmsnorm_quantize_kernel", float(nbytes[big]), float(ms[big]))
    roof["traffic"] = profiled_traffic("rmsnorm_quantize_prefill.txt", "decode_q8_amd/csrc/norm.hip")
    roof["note"] = f"the {timed[big]['rows']}-row launch (the largest of the step)"
    return base_record(args, "fused residual+RMSNorm+Q8_0 quantize HBM GB/s (%HBM peak)", value, "GB/s",
                       ms_per_step, "f32 (fp64 sum of squares), int8 out", config, roof, cpu)


# --------------------------------------------------------------------------
# Q8 KV cache: cache write + decode attention
# --------------------------------------------------------------------------

def attention_bytes(S: int, Hk: int, hd: int, L: int, H: int) -> int:
    """Algorithmic HBM bytes of one q8_attention_decode call: the K and V codes
    and fp32 block scales of every cached position once, the queries and the
    outputs."""
    return S * Hk * L * (2 * hd + 2 * (hd // 32) * 4) + 2 * S * H * hd * 4


def bench_kv(args):
    """One decode step's attention for Llama-3.2-1B: per layer (16, each with
    its own cache of 16 sequences x 4096 positions) the new token's fused
    norm + rope + cache write, then decode attention over the cache."""
    import torch

    import oracle
    import workloads as wl
    from decode_q8_amd import q8
    dev = torch.device("cuda", 0)
    S, H, Hk, hd, L = wl.KV_SEQS, wl.LLAMA_HEADS, wl.LLAMA_KV_HEADS, wl.LLAMA_HEAD_DIM, wl.KV_CONTEXT
    layers = wl.LLAMA_LAYERS
    n_slots = S * L
    cos_t, sin_t = wl.rope_tables(L, hd)
    cos_d, sin_d = torch.from_numpy(cos_t).to(dev), torch.from_numpy(sin_t).to(dev)
    # the step's new token of each sequence sits at position L - 1 (its slot
    # was filled with the rest of the cache; the write refreshes it)
    pos = torch.full((S,), L - 1, dtype=torch.int32, device=dev)
    slots = torch.arange(S, dtype=torch.int32, device=dev) * L + (L - 1)
    base = torch.arange(S, dtype=torch.int32, device=dev) * L
    lens = torch.full((S,), L, dtype=torch.int32, device=dev)
    need = q8.q8_attention_workspace_bytes(S, H, Hk, hd, L)
    per_layer, host0 = [], None
    caches = []
    for l0 in range(0, layers, 8):
        caches += wl.many(lambda layer: wl.kv_cache(wl.KV, layer, Hk, n_slots, hd),
                          [(layer,) for layer in range(l0, min(layers, l0 + 8))], args.threads)
    for layer in range(layers):
        kc, ks, vc, vs = caches[layer]
        caches[layer] = None
        qkv, qg, kg = wl.kv_inputs(wl.KV, 3000 + layer, S, H, Hk, hd)
        c = dict(kc=torch.from_numpy(kc).to(dev), ks=torch.from_numpy(ks).to(dev), vc=torch.from_numpy(vc).to(dev),
                 vs=torch.from_numpy(vs).to(dev), qkv=torch.from_numpy(qkv).to(dev), qg=torch.from_numpy(qg).to(dev),
                 kg=torch.from_numpy(kg).to(dev), q=torch.empty((S, H, hd), dtype=torch.float32, device=dev),
                 out=torch.empty((S, H, hd), dtype=torch.float32, device=dev),
                 ws=torch.zeros(need, dtype=torch.uint8, device=dev))
        if layer == 0:
            host0 = (kc, ks, vc, vs, qkv, qg, kg)
        per_layer.append(c)
        del kc, ks, vc, vs
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(hd)

    def write(c, st):
        q8.q8_kv_write(c["qkv"], S, H, Hk, hd, pos, L, cos_d, sin_d, c["qg"], c["kg"], 1e-5, slots, n_slots, c["q"],
                       c["kc"], c["ks"], c["vc"], c["vs"], None, st)

    def attend(c, st):
        q8.q8_attention_decode(c["q"], S, H, Hk, hd, c["kc"], c["ks"], c["vc"], c["vs"], n_slots, base, lens, L,
                               scale, c["out"], c["ws"], need, st)

    def run(s, timers=None):
        for i, c in enumerate(per_layer):
            write(c, s.cuda_stream)
            if timers is not None:
                timers[i].start()
            attend(c, s.cuda_stream)
            if timers is not None:
                timers[i].stop()

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run(stream)
    torch.cuda.synchronize()
    # check layer 0 against the oracle chain on two sequences before timing
    kc, ks, vc, vs, qkv, qg, kg = host0
    sl = np.arange(S, dtype=np.int32) * L + (L - 1)
    q_ref, kc1, ks1, vc1, vs1 = oracle.kv_write(qkv, H, Hk, hd, np.full(S, L - 1, np.int32), cos_t, sin_t, qg, kg,
                                                1e-5, np.arange(S, dtype=np.int32), S)
    assert np.array_equal(per_layer[0]["q"].cpu().numpy().view(np.uint32), q_ref.view(np.uint32)), "rotated queries"
    kc[:, sl], ks[:, sl], vc[:, sl], vs[:, sl] = kc1, ks1, vc1, vs1
    two = np.array([0, S - 1])
    out_ref, bound = oracle.attention_decode(q_ref[two], kc, ks, vc, vs, (two * L).astype(np.int32),
                                             np.full(2, L, np.int32), scale)
    out0 = per_layer[0]["out"].cpu().numpy()[two]
    assert np.all(np.abs(out0.astype(np.float64) - out_ref) <= bound), "attention outside the oracle's budget"
    assert int(per_layer[0]["ws"][:4].view(torch.int32).cpu()[0]) == 0
    ms_per_step, graph = graph_time(run, stream, args.steps, args.warmup)
    ms = per_launch_ms(run, layers, stream, graph, reps=max(1, min(args.steps, 10)))
    abytes = attention_bytes(S, Hk, hd, L, H)
    kv_bytes = S * Hk * L * (2 * hd + 2 * (hd // 32) * 4) * layers
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        q1 = q_ref[:1]
        sec, reps = timed_repeat(lambda: oracle.attention_decode(q1, kc, ks, vc, vs, np.zeros(1, np.int32),
                                                                 np.full(1, L, np.int32), scale))
        cpu = {"value": round(abytes / S / sec / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"attention of one sequence (32 heads x 4096 positions) of one layer, {reps} repetitions, "
                         f"{sec * reps:.1f} s"}
    config = {
        "workload": "Llama-3.2-1B decode-step attention over a Q8 KV cache: 16 layers, 16 sequences x 4096 cached "
                    "positions, 32 query / 8 KV heads of 64; per layer the new tokens' fused norm + rope + cache "
                    "write, then decode attention",
        "kv_bytes_per_step": int(kv_bytes),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "attention_call_us": round(float(ms.mean()) * 1e3, 2),
        "hip_graph": True,
    }
    roof = hbm_roofline("q8k::attn_partial_kernel + attn_combine_kernel", float(abytes), float(ms.mean()))
    roof["traffic"] = profiled_traffic("attention_decode_kv.txt",
                                       ["decode_q8_amd/csrc/kv.hip", "decode_q8_amd/csrc/device.hpp"])
    roof["note"] = "one attention call (the partial kernel and its small combine kernel), averaged over the 16 layers"
    return base_record(args, "Q8 KV-cache decode attention HBM GB/s (%HBM peak)", value, "GB/s", ms_per_step,
                       "int8 KV, fp32 softmax/accumulation", config, roof, cpu)


# --------------------------------------------------------------------------

def bench_quantize(args):
    """The preparation rows on their own: weight quantization (q8_quantize_rows
    to the row-contiguous layout) and repack (q8_repack_weights) of the LM head
    matrix 128256x2048 (1.05 GB of fp32 in), and activation quantization (the
    ACT layout) of 2048 prefill rows of 2048.  Checked against the oracle on
    the first and last 64 rows before timing."""
    import torch

    import oracle
    import workloads as wl
    from decode_q8_amd import q8
    dev = torch.device("cuda", 0)
    n, k = wl.LLAMA_VOCAB, wl.LLAMA_HIDDEN
    w = wl.weight(wl.DECODE, 0, n, k, group=wl.LLAMA_LAYERS)  # the decode step's LM head weights
    wt = torch.from_numpy(w).to(dev)
    qb = q8.q8_quantized_bytes(n, k)
    wr = torch.empty(qb, dtype=torch.uint8, device=dev)
    wp = torch.empty(qb, dtype=torch.uint8, device=dev)
    xm = 2048
    x = wl.activation(wl.PREFILL, xm, xm, k, outliers=True)
    xt = torch.from_numpy(x).to(dev)
    xq = torch.empty(q8.q8_quantized_bytes(xm, k), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    run_q = lambda s: q8.q8_quantize_rows(wt, k, n, k, q8.Q8_LAYOUT_ROWS, wr, s.cuda_stream)
    run_r = lambda s: q8.q8_repack_weights(wr, n, k, wp, s.cuda_stream)
    run_a = lambda s: q8.q8_quantize_rows(xt, k, xm, k, q8.Q8_LAYOUT_ACT, xq, s.cuda_stream)
    for f in (run_q, run_r, run_a):
        with torch.cuda.stream(stream):
            f(stream)
    torch.cuda.synchronize()
    row_b = (k // 32) * 34
    wr_h = wr.cpu().numpy()
    for r0 in (0, n - 64):
        ref = oracle.quantize_rows(w[r0:r0 + 64], oracle.LAYOUT_ROWS)
        if not np.array_equal(wr_h[r0 * row_b:(r0 + 64) * row_b], ref):
            raise RuntimeError(f"weight quantization differs from the oracle at rows {r0}..{r0 + 63}")
        if not np.array_equal(wp[r0 * row_b:(r0 + 64) * row_b].cpu().numpy(), oracle.pack(ref, 64, k)):
            raise RuntimeError(f"repacked tile at rows {r0}..{r0 + 63} differs from the oracle's packing")
    if not np.array_equal(xq.cpu().numpy(), oracle.quantize_rows(x, oracle.LAYOUT_ACT)):
        raise RuntimeError("activation quantization differs from the oracle")

    ms_q, _ = graph_time(run_q, stream, args.steps, args.warmup)
    spread = dict(STEP_SPREAD)
    ms_r, _ = graph_time(run_r, stream, args.steps, args.warmup)
    ms_a, _ = graph_time(run_a, stream, args.steps, args.warmup)
    STEP_SPREAD.clear()
    STEP_SPREAD.update(spread)
    bytes_q = 4 * n * k + qb       # fp32 in, Q8_0 out
    bytes_r = 2 * qb               # Q8_0 in, the same bytes reordered out
    bytes_a = 4 * xm * k + q8.q8_quantized_bytes(xm, k)
    value = bytes_q / (ms_q * 1e-3) / 1e9
    roof = hbm_roofline("q8k::quantize_kernel (row-contiguous weights)", float(bytes_q), ms_q)
    roof["timing"] = "one event pair around the graph replays of the single launch"
    roof["traffic"] = profiled_traffic("quantize_repack_lm_head.txt",
                                       ["decode_q8_amd/csrc/quantize.hip", "decode_q8_amd/csrc/repack.hip",
                                        "decode_q8_amd/csrc/device.hpp"])
    cpu = None
    if not args.no_cpu_baseline:
        rows = 4096
        sec, reps_c = timed_repeat(lambda: oracle.quantize_rows(w[:rows], oracle.LAYOUT_ROWS))
        cpu = {"value": round((4 * rows * k + rows * row_b) / sec / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"weight quantization of the first {rows} of the {n} rows, {reps_c} runs, {sec:.3f} s each"}
    config = {"workload": "Q8_0 weight quantization of the LM head matrix 128256x2048 (fp32 in, row-contiguous "
                          "Q8_0 out), then repack to the packed layout; activation quantization of 2048 prefill "
                          "rows of 2048",
              "weight_quantize_GBs": round(value, 1), "weight_quantize_us": round(ms_q * 1e3, 2),
              "repack_GBs": round(bytes_r / (ms_r * 1e-3) / 1e9, 1), "repack_us": round(ms_r * 1e3, 2),
              "activation_quantize_GBs": round(bytes_a / (ms_a * 1e-3) / 1e9, 1),
              "activation_quantize_us": round(ms_a * 1e3, 2),
              "activation_note": "per graph replay of one short launch, so host replay overhead dominates; the "
                                 "2048-row activation (16.8 MB) stays in the Infinity Cache between replays (warm)"}
    return base_record(args, "Q8_0 weight quantization GB/s (fp32 in + Q8_0 out)", value, "GB/s", ms_q, "f32->q8_0",
                       config, roof, cpu)


def bench_copy(args):
    """1 GiB device-to-device copy: known bytes for calibrating byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    stream = torch.cuda.Stream()
    ms_per_step, _ = graph_time(lambda s: b.copy_(a), stream, args.steps, args.warmup)
    value = 2.0 * n / (ms_per_step * 1e-3) / 1e9
    return base_record(args, "device copy GB/s (read + write)", value, "GB/s", ms_per_step, "u8",
                       {"workload": "copy 1 GiB", "bytes_read": n, "bytes_written": n}, None, None)


def bench_read(args):
    """The streaming-read ceiling (q8_stream_read) at 1 GiB, with the sizes of
    the decode step's weights, the LM head and one gate||up matrix beside it."""
    from decode_q8_amd import q8
    import torch
    n = 1 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    ms_per_step, _ = graph_time(lambda s: q8.q8_stream_read(buf, n, sink, s.cuda_stream), stream, args.steps,
                                args.warmup)
    spread = dict(STEP_SPREAD)
    del buf
    torch.cuda.synchronize()
    value = n / (ms_per_step * 1e-3) / 1e9
    sizes = {"decode_step_weights_1313MB": 1312980992, "lm_head_279MB": 128256 * 64 * 34,
             "gate_up_35.7MB": 16384 * 64 * 34, "qkv_6.7MB": 3072 * 64 * 34}
    others = {k: round(read_ceiling_gbs(b), 1) for k, b in sizes.items()}
    STEP_SPREAD.clear()
    STEP_SPREAD.update(spread)
    roof = hbm_roofline("q8k::stream_read_kernel", float(n), ms_per_step)
    roof["traffic"] = profiled_traffic("stream_read_ceiling.txt", READ_SOURCES)
    return base_record(args, "streaming-read GB/s", value, "GB/s", ms_per_step, "u8",
                       {"workload": "plain streaming read of 1 GiB (each byte once, 16-byte loads)",
                        "bytes_read": n, "other_sizes_GBs": others}, roof, None)


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
    RAMP["seconds"] = args.ramp_seconds
    fn = {"decode": bench_decode, "batched": bench_decode, "single": bench_single, "prefill": bench_prefill,
          "moe": bench_moe, "norm": bench_norm, "kv": bench_kv, "copy": bench_copy,
          "read": bench_read, "quantize": bench_quantize}[args.workload]
    print(json.dumps(fn(args)), flush=True)


if __name__ == "__main__":
    main()
