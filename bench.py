#!/usr/bin/env python3
"""Throughput of the bit-exact block-scaled int8 GEMM path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mlp|head|step|layer|w1]
                    [--b-format int8|pow2|int4|int4-pow2] [--requant]

One step is one pass of the whole path over one batch: per GEMM, the
quantize pass of each operand (per row, or per column with the transposed
int8 output) and the int8 GEMM with its fused epilogue and output hash.  The
default workload is the GPT-2-small MLP (batch 8 x sequence 1024 = 8192
token rows): the up-projection 8192x768 @ 768x3072 with ReLU, then the
down-projection 8192x3072 @ 3072x768 on its output.  Inputs are seeded
synthetic f32 tensors, resident in HBM before timing starts.

Prints ONE JSON line: value = int8 GEMM operations (2MNK summed over the
step's GEMMs) per second of the whole step, in TOPS, from HIP events around
K steps, replays of HIP graphs that hold ten steps each (--steps-per-graph;
--eager: launched call by call); `kernels` = every call of the step with its
device duration (HIP events around a batch of back-to-back launches: warm)
and, unless --no-cold, its duration when a 512 MiB scrub write precedes each
launch (cold: inputs evicted from the 256 MB last-level cache); `roofline`
for the step's dominant kernel; `lm_head` (MLP workload only, unless
--no-head) = the LM-head GEMMs measured in the same run (forward
8192x50304x768, weight gradient 768x50304x8192: per-GEMM durations, TOPS,
roofline fractions, warm and cold); `cpu_baseline` = the CPU oracle timed on
this host; `parity` = whether output_hash of every stored output, read back
from device memory, equals the oracle's hash (and the fused hash).
--b-format stores every B operand in one of the presk page's "Integer
weights" formats (the headline line uses the default int8 / absmax).
--requant lets a GEMM whose output is the next GEMM's per-row quantized
operand write those codes and scales itself (gemm_i8_requant).
"""
import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA, tera-ops/s
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
RIDGE = PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # ops per byte


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# workloads: lists of GEMMs (name, A-source, B-source, relu); the GPU step and
# the oracle step walk the same list
# ---------------------------------------------------------------------------
def make_workload(name):
    """Returns (description, host tensors, GEMMs); a GEMM is (name, A source,
    A mode, B source, B mode, relu, output name or None).  Mode 'rows' = the
    source is quantized per row (it is A, or B transposed), 'cols' = per
    column (it is B, or A transposed)."""
    from synth import inputs as S
    if name == "mlp":
        X, Wu, Wd = S.w2_inputs()
        desc = ("GPT-2-small MLP: up 8192x768 @ 768x3072 (ReLU), then down "
                "8192x3072 @ 3072x768 on the up output; quantize passes included")
        gemms = [("up", "X", "rows", "Wu", "cols", True, "H"),
                 ("down", "H", "rows", "Wd", "cols", False, None)]
        return desc, {"X": X, "Wu": Wu, "Wd": Wd}, gemms
    if name == "head":
        X, Wh = S.w3_fwd_inputs()
        _, dY = S.w3_wgrad_inputs()
        desc = ("GPT-2-small LM head: forward 8192x768 @ 768x50304 and weight "
                "gradient X^T (768x8192) @ dY (8192x50304); quantize passes included")
        gemms = [("head_fwd", "X", "rows", "Wh", "cols", False, None),
                 ("head_wgrad", "X", "cols", "dY", "cols", False, None)]
        return desc, {"X": X, "Wh": Wh, "dY": dY}, gemms
    if name == "step":
        tensors, gemms = {}, []
        for gm in S.step_gemms():
            a, am, b, bm = gm.operands
            for src in (a, b):
                key = f"{gm.linear}.{src}"
                if key not in tensors:
                    tensors[key] = S.step_tensor(gm.linear, src, gm.d_in, gm.d_out)
            gemms.append((f"{gm.linear}.{gm.kind}", f"{gm.linear}.{a}", am, f"{gm.linear}.{b}", bm,
                          False, None))
        desc = ("GPT-2-small training step: the 147 GEMMs of 12 layers x (QKV, attention "
                "out, MLP up, MLP down) forward, dgrad and wgrad plus the LM head "
                "(8192 token rows); quantize passes included")
        return desc, tensors, gemms
    if name == "layer":
        tensors, gemms = {}, []
        for gm in S.step_gemms():
            if not gm.linear.startswith("L0."):
                continue
            a, am, b, bm = gm.operands
            for src in (a, b):
                key = f"{gm.linear}.{src}"
                if key not in tensors:
                    tensors[key] = S.step_tensor(gm.linear, src, gm.d_in, gm.d_out)
            gemms.append((f"{gm.linear}.{gm.kind}", f"{gm.linear}.{a}", am, f"{gm.linear}.{b}", bm,
                          False, None))
        desc = ("GPT-2-small layer: the 12 GEMMs of layer 0 of the training step (QKV, attention "
                "out, MLP fc, MLP proj; forward, dgrad and wgrad each; 8192 token rows); quantize "
                "passes included")
        return desc, tensors, gemms
    if name == "w1":
        A, B = S.w1_inputs()
        return ("single 256x256x256 GEMM", {"A": A, "B": B},
                [("w1", "A", "rows", "B", "cols", False, None)])
    raise SystemExit(f"unknown workload {name}")


def gemm_mnk(shapes, a_src, a_mode, b_src, b_mode):
    """(M, N, K) of a GEMM from its operands' shapes and modes."""
    M, K = shapes[a_src] if a_mode == "rows" else shapes[a_src][::-1]
    K2, N = shapes[b_src] if b_mode == "cols" else shapes[b_src][::-1]
    assert K == K2, (a_src, b_src)
    return M, N, K


# ---------------------------------------------------------------------------
# GPU step with preallocated buffers and direct C-ABI calls
# ---------------------------------------------------------------------------
# storage formats of the B operands (presk page, "Integer weights"): flag bits
# of quantize_*_fmt (1 = power-of-two scales, 2 = int4 values two per byte)
B_FORMATS = {"int8": 0, "pow2": 1, "int4": 2, "int4-pow2": 3}


def int4_line_bytes(n):
    return 16 * ((n + 31) // 32)


class GpuStep:
    def __init__(self, g, torch, tensors, gemms, fmt_b=0, requant=False):
        self.g, self.torch, self.lib = g, torch, g.load()
        dev = torch.device("cuda:0")
        self.dev = dev
        self.stream = torch.cuda.current_stream(dev)
        self.sp = self.stream.cuda_stream
        self.t = {k: torch.from_numpy(v).to(dev) for k, v in tensors.items()}
        self.gemms = []
        self.fmt_b = fmt_b
        ws_bytes = 256
        shapes = {k: tuple(v.shape) for k, v in tensors.items()}
        for (name, a_src, a_mode, b_src, b_mode, relu, out_name) in gemms:
            M, N, K = gemm_mnk(shapes, a_src, a_mode, b_src, b_mode)
            shapes[out_name or name] = (M, N)
            ld = (K + 15) // 16 * 16
            ldb = int4_line_bytes(K) if fmt_b & 2 else ld
            e = dict(name=name, M=M, N=N, K=K, relu=relu, a_mode=a_mode, a_key=a_src, ldb=ldb,
                     b_mode=b_mode, b_key=b_src, out=out_name or name,
                     QA=torch.empty((M, ld), dtype=torch.int8, device=dev),
                     sA=torch.empty(M, dtype=torch.float32, device=dev),
                     QB=torch.empty((N, ldb), dtype=torch.int8, device=dev),
                     sB=torch.empty(N, dtype=torch.float32, device=dev),
                     C=torch.empty((M, N), dtype=torch.float32, device=dev),
                     h=torch.zeros(1, dtype=torch.int64, device=dev), ld=ld)
            self.t[e["out"]] = e["C"]
            ws_bytes = max(ws_bytes, g.workspace_bytes(M, N, K, 8 if fmt_b & 2 else 0))
            self.gemms.append(e)
        # requantizing epilogue: a GEMM whose output is the per-row quantized A
        # operand of a later GEMM writes that GEMM's codes and scales itself
        # (gemm_i8_requant) and the later GEMM skips its quantize_A
        for e in self.gemms:
            e["requant_into"] = None
            e["skip_qa"] = False
        if requant:
            for i, e in enumerate(self.gemms):
                for e2 in self.gemms[i + 1:]:
                    if e2["a_key"] == e["out"] and e2["a_mode"] == "rows":
                        e["requant_into"] = e2
                        e2["skip_qa"] = True
                        ws_bytes = max(ws_bytes, int(self.lib.gemm_i8_requant_workspace_bytes(
                            e["M"], e["N"], e["K"])))
                        break
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        # the quantize passes of input tensors (not of a GEMM's output) depend
        # on nothing in the step: they go first, together, as one
        # quantize_batch call
        self.inputs = set(tensors)
        specs, self.batched = [], []
        for e in self.gemms:
            if not e["skip_qa"] and e["a_key"] in self.inputs:
                specs.append((self.t[e["a_key"]], e["a_mode"] == "cols", 0, e["QA"], e["ld"], e["sA"]))
                self.batched.append((e["name"], "quantize_A"))
            if e["b_key"] in self.inputs:
                specs.append((self.t[e["b_key"]], e["b_mode"] == "cols", self.fmt_b, e["QB"], e["ldb"], e["sB"]))
                self.batched.append((e["name"], "quantize_B"))
        self.jobs = (g.QuantizeJob * max(1, len(specs)))()
        for i, (X, by_col, fmt, Q, ldq, s) in enumerate(specs):
            rows, cols = X.shape
            self.jobs[i] = g.QuantizeJob(X.data_ptr(), rows, cols, X.stride(0), Q.data_ptr(), ldq,
                                         s.data_ptr(), 1 if by_col else 0, fmt)
        self.njobs = len(specs)

    def _q(self, mode, X, Q, s, ld, fmt=0):
        rows, cols = X.shape
        fn = self.lib.quantize_rows_fmt if mode == "rows" else self.lib.quantize_cols_fmt
        rc = fn(X.data_ptr(), rows, cols, X.stride(0), Q.data_ptr(), ld, s.data_ptr(), fmt, self.sp)
        if rc:
            raise RuntimeError(self.lib.i8g_status_string(rc).decode())

    def _gemm(self, e):
        flags = (1 if e["relu"] else 0) | 2 | (8 if self.fmt_b & 2 else 0)
        rc = self.lib.gemm_i8_blockscaled(e["QA"].data_ptr(), e["ld"], e["sA"].data_ptr(),
                                          e["QB"].data_ptr(), e["ldb"], e["sB"].data_ptr(),
                                          e["M"], e["N"], e["K"], e["C"].data_ptr(), e["N"], flags,
                                          e["h"].data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                                          self.sp)
        if rc:
            raise RuntimeError(self.lib.i8g_status_string(rc).decode())

    def _requant(self, e):
        e2 = e["requant_into"]
        flags = (1 if e["relu"] else 0) | 2
        rc = self.lib.gemm_i8_requant(e["QA"].data_ptr(), e["ld"], e["sA"].data_ptr(),
                                      e["QB"].data_ptr(), e["ldb"], e["sB"].data_ptr(),
                                      e["M"], e["N"], e["K"], e2["QA"].data_ptr(), e2["ld"],
                                      e2["sA"].data_ptr(), flags, e["h"].data_ptr(),
                                      self.ws.data_ptr(), self.ws.numel(), self.sp)
        if rc:
            raise RuntimeError(self.lib.i8g_status_string(rc).decode())

    def _batch(self):
        rc = self.lib.quantize_batch(self.jobs, self.njobs, self.sp)
        if rc:
            raise RuntimeError(self.lib.i8g_status_string(rc).decode())

    def calls(self, e, batched=False):
        """The calls of one GEMM of the step, as (label, function); with
        batched=True the input quantize passes, which quantize_batch makes,
        are left out."""
        out = []
        skip = set(lab for name, lab in self.batched if name == e["name"]) if batched else set()
        if not e["skip_qa"] and "quantize_A" not in skip:
            out.append(("quantize_A", lambda: self._q(e["a_mode"], self.t[e["a_key"]], e["QA"], e["sA"], e["ld"])))
        if "quantize_B" not in skip:
            out.append(("quantize_B", lambda: self._q(e["b_mode"], self.t[e["b_key"]], e["QB"], e["sB"],
                                                      e["ldb"], self.fmt_b)))
        if e["requant_into"] is not None:
            out.append(("requant", lambda: self._requant(e)))
        else:
            out.append(("gemm", lambda: self._gemm(e)))
        return out

    def run(self):
        """Enqueue one step on torch's current stream (a graph capture switches
        it, so it is read at every call)."""
        self.stream = self.torch.cuda.current_stream(self.dev)
        self.sp = self.stream.cuda_stream
        if self.njobs:
            self._batch()
        for e in self.gemms:
            for _, fn in self.calls(e, batched=True):
                fn()

    def hashes(self):
        """The hashes the GEMM kernels fused into their epilogues."""
        return [self.g.hash_value(e["h"]) for e in self.gemms]

    def stored_hashes(self):
        """output_hash of every stored output, read back from device memory
        (None for a requantized output, which is not stored)."""
        out = []
        for e in self.gemms:
            if e["requant_into"] is not None:
                out.append(None)
                continue
            out.append(self.g.hash_value(self.g.output_hash(e["C"])))
        self.torch.cuda.synchronize()
        return out


# ---------------------------------------------------------------------------
# CPU oracle step (the cpu_baseline leg)
# ---------------------------------------------------------------------------
def oracle_step(tensors, gemms, budget_s=None, fmt_b=0):
    """The CPU oracle over the GEMMs in order; with a time budget it stops
    after the GEMM that crosses it.  Returns (hashes, int8 ops done)."""
    from oracle import formats, hashref, ref
    t = dict(tensors)
    shapes = {k: tuple(v.shape) for k, v in t.items()}
    hashes, ops = [], 0.0
    t0 = time.perf_counter()
    for (name, a_src, a_mode, b_src, b_mode, relu, out_name) in gemms:
        M, N, K = gemm_mnk(shapes, a_src, a_mode, b_src, b_mode)
        q = {"rows": ref.quantize_rows, "cols": ref.quantize_cols}
        QA, sA = q[a_mode](t[a_src])
        if fmt_b:
            qf = formats.quantize_cols if b_mode == "cols" else formats.quantize_rows
            QB, sB = qf(t[b_src], fmt_b)
        else:
            QB, sB = q["cols" if b_mode == "cols" else "rows"](t[b_src])
        C = ref.gemm_i8_blockscaled(QA, sA, QB, sB, relu)
        t[out_name or name] = C
        shapes[out_name or name] = C.shape
        hashes.append(hashref.output_hash(C))
        ops += 2.0 * M * N * K
        del QA, QB
        if budget_s is not None and time.perf_counter() - t0 >= budget_s:
            break
    return hashes, ops


def cpu_baseline(tensors, gemms, ops, budget_s=10.0, fmt_b=0):
    """The oracle timed on this host: whole steps (one to three, about
    budget_s of work) when a step is short, else the leading GEMMs of one
    step up to the budget.  Returns (record, oracle hashes of the GEMMs it ran)."""
    from threadpoolctl import threadpool_info
    blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
    threads = max([d.get("num_threads", 1) for d in blas] or [1])
    host = {"cpu_model": cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
            "blas_threads": threads}
    t0 = time.perf_counter()
    hashes, done = oracle_step(tensors, gemms, budget_s, fmt_b)
    first = time.perf_counter() - t0
    if len(hashes) < len(gemms):
        return {"value": done / first / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
                **host, "sample": f"the first {len(hashes)} of the step's {len(gemms)} GEMMs "
                          f"({done / 1e9:.1f} GOP) in {first:.1f} s; numpy float32 per-op "
                          f"quantize/epilogue (1 thread), float64 BLAS contraction "
                          f"({threads} threads), numpy uint64 hash"}, hashes
    times = [first]
    while time.perf_counter() - t0 < budget_s and len(times) < 3:
        t1 = time.perf_counter()
        oracle_step(tensors, gemms, None, fmt_b)
        times.append(time.perf_counter() - t1)
    sec = statistics.median(times)
    return {"value": ops / sec / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle", **host,
            "sample": f"{len(times)} full step(s) of the same workload, median {sec:.2f} s; "
                      f"numpy float32 per-op quantize/epilogue (1 thread), float64 BLAS "
                      f"contraction ({threads} threads), numpy uint64 hash"}, hashes


# ---------------------------------------------------------------------------
# traffic from committed PMC summaries (null unless the kernels are unchanged)
# ---------------------------------------------------------------------------
def code_digest_text(text):
    """Source text without comments and with whitespace collapsed: edits to
    comments or layout leave the digest unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha():
    """Digest of the code the timed kernels and their planner are built
    from (api.hip holds the host-side argument checks and verify.hip the
    self-checks; neither changes a kernel).  Comments do not count."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int8_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f in ("verify.hip", "api.hip"):
            continue
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + code_digest_text(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel_key):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_sha") != kernel_source_sha():
        return None
    ent = data.get("kernels", {}).get(kernel_key)
    return None if ent is None else ent.get("bytes_per_launch")


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def capture_graphs(torch, step, steps, spg, ref_hashes):
    """HIP graphs of one step and (when at least spg steps are timed) of spg
    steps.  The library allocates nothing, launches only kernels on the given
    stream and leaves its workspace header zero, so a replay repeats the step
    exactly; every replay below, with eager steps between them, must
    reproduce the eager hashes.  With one step per graph the kernel trace
    shows the GPU idle ~8 us between consecutive replays, none between the
    kernels inside one: hence several steps per graph."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    torch.cuda.synchronize()
    graphs, graph_s = [graph], None
    if spg > 1 and steps >= spg:
        graph_s = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_s):
            for _ in range(spg):
                step.run()
        torch.cuda.synchronize()
        graphs.append(graph_s)
    for gr in graphs:
        for _ in range(3):
            for e in step.gemms:
                e["h"].zero_()
            gr.replay()
            torch.cuda.synchronize()
            if step.hashes() != ref_hashes:
                raise SystemExit("graph replay changed the output hashes")
            step.run()
            torch.cuda.synchronize()
            if step.hashes() != ref_hashes:
                raise SystemExit("eager step after a replay changed the output hashes")
    return graph, graph_s


def time_steps(torch, step, steps, warmup, spg, eager, ref_hashes):
    """Device time of exactly `steps` steps (HIP events on the step's
    stream), as graph replays or eager launches.  Returns (ms per step,
    wall ms per step, launch description)."""
    graph = graph_s = None
    if not eager:
        graph, graph_s = capture_graphs(torch, step, steps, spg, ref_hashes)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
    n_s = steps // spg if graph_s is not None else 0
    n_1 = steps - n_s * spg
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    start.record(stream)
    if graph is None:
        for _ in range(steps):
            step.run()
    else:
        for _ in range(n_s):
            graph_s.replay()
        for _ in range(n_1):
            graph.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if step.hashes() != ref_hashes:
        raise SystemExit("timed steps changed the output hashes")
    launch = "eager" if graph is None else f"hip graph replays ({n_s} x {spg} steps + {n_1} x 1 step)"
    return start.elapsed_time(stop) / steps, wall * 1e3 / steps, launch


def time_call(torch, step, fn, reps, scrub=None):
    """Average device time of one call in microseconds.
    Warm (scrub is None): the call launched `reps` times back to back on the
    step's stream, behind a short sleep kernel so that the host runs ahead of
    the GPU, one event pair around the batch; its inputs stay in the caches.
    Cold: before each launch the 512 MiB `scrub` buffer is overwritten (more
    than the 256 MB last-level cache), so the call starts from HBM; each
    launch has its own event pair."""
    torch.cuda.synchronize()
    if scrub is None:
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(2_000_000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(step.stream)
        for _ in range(reps):
            fn()
        e1.record(step.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps
    ev = []
    for r in range(reps):
        scrub.fill_(r & 0x7F)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(step.stream)
        fn()
        e1.record(step.stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return statistics.mean(a.elapsed_time(b) for a, b in ev) * 1e3


def call_record(step, e, label, avg, cold, fmt_b):
    """Algorithmic bytes / ops of one call of the step and its rates."""
    M, N, K = e["M"], e["N"], e["K"]
    if label in ("gemm", "requant"):
        gops = 2.0 * M * N * K
        b_bytes = N * int4_line_bytes(K) if fmt_b & 2 else N * K
        out_bytes = 4 * M * N if label == "gemm" else M * N + 4 * M   # f32, or int8 + scales
        nbytes = M * K + b_bytes + 4 * M + 4 * N + out_bytes + 8
        bound = "mfma" if gops / nbytes >= RIDGE else "hbm"
        shape = f"{M}x{N}x{K}"
    else:
        # the quantized source tensor and the direction of its scales
        mode = e["a_mode"] if label == "quantize_A" else e["b_mode"]
        rows, cols = step.t[e["a_key"] if label == "quantize_A" else e["b_key"]].shape
        nscale = rows if mode == "rows" else cols
        nlines, length = (rows, cols) if mode == "rows" else (cols, rows)
        qbytes = nlines * int4_line_bytes(length) if (label == "quantize_B" and fmt_b & 2) else rows * cols
        gops, nbytes, bound = 0.0, 4 * rows * cols + qbytes + 4 * nscale, "hbm"
        shape = f"{rows}x{cols} ({mode})"

    def rate(us):
        if bound == "mfma":
            return gops / (us * 1e-6) / 1e12, PEAK_INT8_TOPS, "TFLOP/s"
        return nbytes / (us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s"

    ach, peak, unit = rate(avg)
    rec = {"call": f"{e['name']}.{label}", "shape": shape, "avg_us": round(avg, 2),
           "total_us_per_step": round(avg, 2), "bound": bound,
           "achieved": round(ach, 1), "peak": peak, "unit": unit,
           "frac": round(ach / peak, 4), "algorithmic_bytes": nbytes, "int8_ops": gops,
           "tops": round(gops / (avg * 1e-6) / 1e12, 1) if gops else None}
    if gops:
        rec["pct_of_int8_peak"] = round(100.0 * gops / (avg * 1e-6) / 1e12 / PEAK_INT8_TOPS, 2)
    if cold is not None:
        cach, _, _ = rate(cold)
        rec["cold_avg_us"] = round(cold, 2)
        rec["cold_frac"] = round(cach / peak, 4)
        if gops:
            rec["cold_tops"] = round(gops / (cold * 1e-6) / 1e12, 1)
    return rec


def measure_calls(torch, step, reps, cold_reps, scrub, fmt_b):
    """Per-call device durations (warm, and cold when scrub is given) of
    every call of the step, and of the batched input passes as the step
    issues them.  Returns (records, batch record or None)."""
    kernels = []
    for e in step.gemms:
        for label, fn in step.calls(e):
            avg = time_call(torch, step, fn, reps)
            cold = time_call(torch, step, fn, cold_reps, scrub) if scrub is not None else None
            kernels.append(call_record(step, e, label, avg, cold, fmt_b))
    batch = None
    if step.njobs:
        # the batch runs the input passes timed one by one above; its bytes
        # are theirs (it is not a single kernel, so it is not a roofline candidate)
        us = time_call(torch, step, step._batch, reps)
        cold = time_call(torch, step, step._batch, cold_reps, scrub) if scrub is not None else None
        parts = [k for k in kernels if tuple(k["call"].rsplit(".", 1)) in set(step.batched)]
        nbytes = sum(k["algorithmic_bytes"] for k in parts)
        batch = {"call": "inputs.quantize_batch", "passes": len(parts), "avg_us": round(us, 2),
                 "sum_of_single_calls_us": round(sum(k["avg_us"] for k in parts), 2),
                 "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "unit": "GB/s",
                 "algorithmic_bytes": nbytes}
        if cold is not None:
            batch["cold_avg_us"] = round(cold, 2)
            batch["cold_achieved"] = round(nbytes / (cold * 1e-6) / 1e9, 1)
    return kernels, batch


def golden_head_hashes():
    """The oracle's output hashes of the LM-head GEMMs (forward, weight
    gradient), written by tests/golden/make_step_golden.py from oracle/."""
    path = os.path.join(ROOT, "tests", "golden", "step_golden.json")
    with open(path) as f:
        gh = json.load(f)["head"]
    return [int(gh["fwd"]["hash"], 16), int(gh["wgrad"]["hash"], 16)]


def lm_head_record(g, torch, args, scrub):
    """The LM-head GEMMs (forward 8192x50304x768, weight gradient
    768x50304x8192) measured in the same run as the headline: the whole
    LM-head step (its quantize passes and both GEMMs), and per call warm and
    cold durations with TOPS and roofline fractions.  Parity: output_hash of
    the stored outputs against the oracle's hashes."""
    desc, tensors, gemms = make_workload("head")
    step = GpuStep(g, torch, tensors, gemms)
    del tensors
    step.run()
    torch.cuda.synchronize()
    fused = step.hashes()
    stored = step.stored_hashes()
    want = golden_head_hashes()
    steps = max(2, min(args.steps, 10))
    ms, _, launch = time_steps(torch, step, steps, 1, max(1, min(args.steps_per_graph, steps)), args.eager, fused)
    reps = max(3, min(args.steps, 10))
    kernels, batch = measure_calls(torch, step, reps, 3, scrub, 0)
    if step.hashes() != fused:
        raise SystemExit("LM head: repeated calls changed the output hashes")
    ops = sum(2.0 * e["M"] * e["N"] * e["K"] for e in step.gemms)
    rec = {"workload": desc, "steps": steps, "ms_per_step": round(ms, 4),
           "tops": round(ops / (ms * 1e-3) / 1e12, 1),
           "pct_of_int8_peak": round(100.0 * ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
           "launch": launch,
           "gemms": [dict(k, traffic=traffic_for(k["call"])) for k in kernels if k["call"].endswith(".gemm")],
           "quantize": [k for k in kernels if not k["call"].endswith(".gemm")],
           "quantize_batch": batch,
           "parity": stored == want and fused == want,
           "gpu_hashes": [f"{h:#018x}" for h in stored]}
    del step
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mlp", choices=["mlp", "head", "step", "layer", "w1"])
    ap.add_argument("--b-format", default="int8", choices=list(B_FORMATS),
                    help="storage format of every B operand (int4: two values per byte; "
                         "pow2: power-of-two scales); A operands stay int8 with absmax scales")
    ap.add_argument("--requant", action="store_true",
                    help="a GEMM whose output feeds the next GEMM's per-row quantize writes int8 "
                         "codes and scales directly (gemm_i8_requant; the f32 output is not stored)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-head", action="store_true",
                    help="leave out the LM-head sub-record of the MLP workload's line")
    ap.add_argument("--no-cold", action="store_true",
                    help="leave out the cold-cache (512 MiB scrub before each launch) timings")
    ap.add_argument("--steps-per-graph", type=int, default=10, metavar="S",
                    help="steps captured in one HIP graph; the K timed steps are K // S replays of "
                         "it and K % S replays of a one-step graph")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of the step captured in a HIP graph")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="also run one plain device copy of MB MiB (a reference for HBM "
                         "byte counters collected by a profiler around this run)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(its sharding is described in DESIGN.md); rerun with --gpus 1", flush=True)
        sys.exit(2)

    import torch
    import int8_gemm_amd as g

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"[bench] workload {a.workload}: generating inputs")
    desc, tensors, gemms = make_workload(a.workload)
    fmt_b = B_FORMATS[a.b_format]
    step = GpuStep(g, torch, tensors, gemms, fmt_b, a.requant)
    if a.copy_probe > 0:
        src = torch.ones(a.copy_probe << 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {a.copy_probe} MiB read + {a.copy_probe} MiB written")
        del src, dst
    ops = sum(2.0 * e["M"] * e["N"] * e["K"] for e in step.gemms)
    log(f"[bench] {len(step.gemms)} GEMMs, {ops / 1e9:.2f} GOP per step; warmup {a.warmup}")
    for _ in range(a.warmup):
        step.run()
    torch.cuda.synchronize()
    gpu_hashes = step.hashes()

    # timed region: exactly K steps (graph replays, or eager launches)
    spg = max(1, a.steps_per_graph)
    log(f"[bench] timing {a.steps} steps")
    ms_per_step, wall_ms, launch = time_steps(torch, step, a.steps, a.warmup, spg, a.eager, gpu_hashes)
    value = ops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] {ms_per_step:.4f} ms/step (wall {wall_ms:.4f} ms/step, {launch}), {value:.1f} TOPS")

    # per-call device durations, warm and cold
    scrub = None if a.no_cold else torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    reps = max(5, min(a.steps, 50))
    kernels, batch_entry = measure_calls(torch, step, reps, max(3, min(a.steps, 20)), scrub, fmt_b)
    if step.hashes() != gpu_hashes:
        raise SystemExit("repeated calls changed the output hashes")
    # parity is judged on the stored outputs: output_hash reads every output
    # back from device memory (outside the timed region)
    stored_hashes = step.stored_hashes()
    dom = max(kernels, key=lambda k: k["avg_us"])
    roof = {"bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
            "unit": dom["unit"], "frac": dom["frac"], "traffic": traffic_for(dom["call"]),
            "kernel": dom["call"], "shape": dom["shape"], "avg_us": dom["avg_us"]}
    if "cold_avg_us" in dom:
        roof["cold_avg_us"] = dom["cold_avg_us"]
        roof["cold_frac"] = dom["cold_frac"]

    head = None
    if a.workload == "mlp" and not a.no_head and fmt_b == 0 and not a.requant:
        log("[bench] LM-head GEMMs (sub-record)")
        head = lm_head_record(g, torch, a, scrub)
        log(f"[bench] LM head {head['ms_per_step']:.3f} ms/step, {head['tops']:.1f} TOPS, parity {head['parity']}")
    del scrub

    cpu = None
    parity = None
    if not a.no_cpu_baseline:
        log("[bench] cpu_baseline: oracle on the host")
        cpu, cpu_hashes = cpu_baseline(tensors, gemms, ops, fmt_b=fmt_b)
        n = len(cpu_hashes)
        parity = (cpu_hashes == stored_hashes[:n] and
                  all(s is None or s == f for s, f in zip(stored_hashes, gpu_hashes)))
        log(f"[bench] oracle {cpu['value']:.4f} TOPS, parity {parity}")

    out = {
        "metric": "bit-exact block-scaled int8 GEMM TOPS (% of int8 MFMA peak), GPT-2-small shapes",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": desc, "name": a.workload, "b_format": a.b_format, "requant": a.requant,
                   "gemms": [f"{e['M']}x{e['N']}x{e['K']}{' relu' if e['relu'] else ''}"
                             for e in step.gemms],
                   "int8_ops_per_step": ops, "batch": 8, "seq_len": 1024, "tokens": 8192},
        "pct_of_int8_peak": round(100.0 * value / PEAK_INT8_TOPS, 2),
        "roofline": roof,
        "kernels": kernels,
        "quantize_batch": batch_entry,
        "lm_head": head,
        "cpu_baseline": cpu,
        "parity": parity,
        "parity_basis": "output_hash of every stored output (read back from device memory) "
                        "against the CPU oracle's hashes, plus the fused hashes equal to those",
        "gpu_hashes": [f"{h:#018x}" for h in gpu_hashes],
        "launch": launch,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
