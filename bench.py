#!/usr/bin/env python3
"""Benchmark of the few-row block-quantized GEMV on one MI355X.

Headline step: the LM-head projection W 128256 x 4096 in the Q8_0 lane at 1, 8
and 16 activation rows -- three calls of qgemv_q8_0, each streaming the whole
558,170,112-byte weight image once (the rows the metric is quoted at).  Two
weight copies alternate, so no call finds its image in the 256 MB Infinity
Cache.  `value` is the weight bytes of the step over its time.

Beside it, on the same line:
  * roofline      -- per row count, the GEMV kernel's average launch duration
                     (HIP events on its stream) against its algorithmic bytes,
                     and their sum over the step; HBM bytes from the committed
                     rocprofv3 counter summaries when they match the source;
  * read_ceiling  -- a plain streaming read of the same bytes (qg_read_probe),
                     the achievable-read figure the GEMVs are also read against;
  * secondary     -- the other workloads at their listed rows, each with its
                     kernel's roofline: the Llama-3.2-1B-shaped Q8_0 layer (1
                     row), the Llama-3.2-3B-shaped layer in Q4_0 and in Q4_K
                     (1/2/4/8 rows),
                     the LM head in the f16 lane and in Q4_0 (1/8/16), the
                     1024 x 1024 Q8_0 GEMV (1 row), the routed MoE step
                     (1/8/9/16 rows);
  * cpu_baseline  -- the C oracle on a bounded slice of the headline workload,
                     all cores and one core, median of five reps;
  * sweep         -- (unless --no-sweep) every workload at 1/2/4/8/9/16 rows.
Every timed form runs five reps; the median rep is reported with the slowest.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-sweep] [--no-cpu-baseline]
"""
import argparse
import ctypes as C
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "weight GB/s and % HBM roofline for Q8_0/Q4_0 GEMV at 1/8/16 rows"
REPS = 5

LM_N, LM_K = 128256, 4096
HEAD_ROWS = (1, 8, 16)
LAYER_1B = [("wq", 2048, 2048), ("wk", 512, 2048), ("wv", 512, 2048), ("wo", 2048, 2048), ("gate", 8192, 2048),
            ("up", 8192, 2048), ("down", 2048, 8192)]
LAYER_3B = [("wq", 3072, 3072), ("wk", 1024, 3072), ("wv", 1024, 3072), ("wo", 3072, 3072), ("gate", 8192, 3072),
            ("up", 8192, 3072), ("down", 3072, 8192)]
# which of the three input rows (block input, attention output, FFN hidden) feeds each projection
LAYER_SRC = {"wo": 1, "down": 2}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=60)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--out", default=None, help="also write the JSON line to this file")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run a plain elementwise kernel over 256 MiB (reads 256 MiB, writes 256 MiB) five "
                        "times, the known-size reference for the HBM byte counters")
    p.add_argument("--profile", default=None, metavar="WORKLOAD:ROWS",
                   help="time one workload (lm-head-q8, lm-head-q8-prepared, lm-head-q4, lm-head-q4-prepared, "
                        "lm-head-f16, lm-head-fp8, layer-1b, layer-3b, layer-1b-prepared, layer-3b-prepared, moe, "
                        "moe-fp8, read-probe) at ROWS rows for --steps calls after a short warm-up, print it, and exit: a "
                        "short program for rocprofv3")
    p.add_argument("--traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL", "WORKLOAD"), default=None,
                   help="reduce two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then WRITE_SIZE) of a "
                        "--calibrate-copy --profile run into the HBM bytes per launch of KERNEL, stored in "
                        "profiles/traffic.json under KERNEL|WORKLOAD, then exit")
    p.add_argument("--counters", nargs=3, metavar=("CSV", "KERNEL", "WORKLOAD"), default=None,
                   help="reduce a rocprofv3 --pmc counter_collection.csv of a --profile run into the per-dispatch "
                        "averages of its counters for KERNEL, stored in profiles/counters.json under "
                        "KERNEL|WORKLOAD, then exit")
    return p.parse_args()


class Timer:
    """Times enqueued work with HIP events on torch's current stream.

    A bounded sleep kernel holds the stream while the host enqueues, so the
    measured interval is GPU time, not host launch time."""

    def __init__(self, torch):
        self.torch = torch
        self.cycles_per_ms = self._calibrate()

    def _calibrate(self):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda._sleep(1000)
        a.record()
        t.cuda._sleep(2_000_000)
        b.record()
        t.cuda.synchronize()
        ms = a.elapsed_time(b)
        return 2_000_000 / max(ms, 1e-3)

    def hold(self, ms):
        self.torch.cuda._sleep(int(self.cycles_per_ms * ms))


def ctypes_arr(struct, items):
    arr = (struct * len(items))()
    for i, it in enumerate(items):
        arr[i] = it
    return arr


# ------------------------------------------------------------ profiles ---
PROFILED_SOURCES = {
    "rl_set_kernel": ("qg_q8.hip", "qg_device.h", "qg_layout.h"),
    "mp_set_kernel": ("qg_q8.hip", "qg_device.h", "qg_layout.h"),
    "gemv_f16_kernel": ("qg_f16.hip", "qg_device.h", "qg_layout.h"),
    "gemv_fp8_kernel": ("qg_fp8.hip", "qg_device.h", "qg_layout.h"),
    "read_probe_kernel": ("qg_probe.hip", "qg_device.h"),
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in PROFILED_SOURCES.get(kernel, ("qg_q8.hip", "qg_device.h", "qg_layout.h")):
        with open(os.path.join(ROOT, "block_quantized_few_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


COPY_BYTES = 256 << 20


def calibrate_copy(torch):
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def pmc_per_dispatch(path, counter):
    """{kernel name: [value per dispatch]} of one counter from a rocprofv3 counter_collection.csv."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def _pick(d, pat, big=False):
    vals = [v for name, vs in d.items() if pat in name for v in vs]
    if big:
        vals = [v for v in vals if v * 1024 > COPY_BYTES / 2]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel named like {pat!r} in the counter file")
    return sum(vals) / len(vals), len(vals)


def _update_json(name, key, rec):
    path = os.path.join(ROOT, "profiles", name)
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[key] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")


def reduce_traffic(fetch_csv, write_csv, kernel, workload):
    """HBM bytes per launch of `kernel`, from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the
    factor that maps the same counter to the known bytes of the calibration kernel."""
    fetch = pmc_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = pmc_per_dispatch(write_csv, "WRITE_SIZE")
    cf, _ = _pick(fetch, "neg", big=True)
    cw, _ = _pick(write, "neg", big=True)
    kf, nf = _pick(fetch, kernel)
    kw, nw = _pick(write, kernel)
    ff, fw = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    rec = {"hbm_bytes_per_launch": round(kf * 1024 * ff + kw * 1024 * fw),
           "fetch_kib_per_dispatch": round(kf, 1), "write_kib_per_dispatch": round(kw, 1), "dispatches": [nf, nw],
           "calibration": {"kernel": "torch.neg over 256 MiB fp32", "known_bytes_each_way": COPY_BYTES,
                           "fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                           "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)},
           "source_hash": kernel_source_hash(kernel)}
    _update_json("traffic.json", f"{kernel}|{workload}", rec)
    print(json.dumps(rec))


def reduce_counters(csv_path, kernel, workload):
    """Per-dispatch averages of every counter in a --pmc run, for the dispatches of `kernel`."""
    import csv
    names = set()
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            names.add(r["Counter_Name"])
    avg = {}
    for c in sorted(names):
        v, n = _pick(pmc_per_dispatch(csv_path, c), kernel)
        avg[c] = round(v, 1)
    rec = {"avg_per_dispatch": avg, "dispatches": n, "source_hash": kernel_source_hash(kernel)}
    _update_json("counters.json", f"{kernel}|{workload}", rec)
    print(json.dumps(rec))


def _read_profile(name, kernel, workload):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        e = json.load(f).get(f"{kernel}|{workload}")
    if not e or e.get("source_hash") != kernel_source_hash(kernel):
        return None
    return e


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed PMC summary, if taken on this kernel source."""
    e = _read_profile("traffic.json", kernel, workload)
    return None if e is None else e.get("hbm_bytes_per_launch")


def read_busy(kernel, workload):
    """VALU-busy and MFMA-busy % from the committed counter summary, if taken on this kernel source: the
    counters' per-dispatch averages as rocprofv3 reported them (its derived busy metrics when collected)."""
    e = _read_profile("counters.json", kernel, workload)
    return None if e is None else e["avg_per_dispatch"]


# --------------------------------------------------------------- timing ---
def time_reps(torch, timer, stream, fn, iters, reps=REPS):
    """Per-rep average ms of `iters` back-to-back calls (HIP events on `stream`), `reps` reps after a warm-up."""
    for i in range(min(iters, 5)):
        fn(i)
    torch.cuda.synchronize()
    out = []
    for rep in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        timer.hold(max(5.0, iters * 0.05))
        a.record(stream)
        for i in range(iters):
            fn(rep * iters + i)
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / iters)
    return out


def summarize(ms_reps):
    return {"median_us": round(statistics.median(ms_reps) * 1e3, 3), "slowest_us": round(max(ms_reps) * 1e3, 3)}


def roofline_entry(kernel, alg_bytes, ms_reps, traffic=None, ceiling=None, busy=None):
    avg_ms = statistics.median(ms_reps)
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    e = {"kernel": kernel, "bound": "hbm", "alg_bytes_per_launch": int(alg_bytes),
         "avg_launch_us": round(avg_ms * 1e3, 3), "slowest_rep_us": round(max(ms_reps) * 1e3, 3),
         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}
    if ceiling:
        e["pct_of_read_ceiling"] = round(100.0 * achieved / ceiling, 1)
    if busy:
        e["counters"] = busy
    return e


# ------------------------------------------------------------------ layers ---
class LayerSet:
    """A decode layer's projections in one lane with rotating weight copies."""

    def __init__(self, torch, q, synth, layer, fmt, workload, rows, copies=None):
        self.torch, self.q = torch, q
        self.layer, self.fmt, self.rows = layer, fmt, rows
        self.wbytes = sum(q.image_bytes(fmt, n, k) for _, n, k in layer)
        self.copies = copies or max(2, math.ceil((1 << 30) / self.wbytes))
        self.imgs = []
        for c in range(self.copies):
            row = []
            for i, (_, n, k) in enumerate(layer):
                w = synth.gaussian((n, k), 0.02, synth.tensor_seed(workload, i, c), device="cuda")
                row.append(q.quantize_weights(fmt, w))
                del w
            self.imgs.append(row)
        self.set_rows(rows, synth, workload)

    def set_rows(self, rows, synth, workload):
        q, torch = self.q, self.torch
        self.rows = rows
        k_in, k_dn = self.layer[0][2], self.layer[6][2]
        seeds = [(32 + rows, k_in), (48 + rows, k_in), (64 + rows, k_dn)]
        self.xs = [synth.gaussian((rows, k), 1.0, synth.tensor_seed(workload, tid), device="cuda") for tid, k in seeds]
        self.wss = [q.empty_ws(rows, x.shape[1]) for x in self.xs]
        self.ys = [torch.empty((rows, n), dtype=torch.float32, device="cuda") for _, n, _ in self.layer]
        self.projs = []
        for c in range(self.copies):
            items = []
            for i, (name, n, k) in enumerate(self.layer):
                j = LAYER_SRC.get(name, 0)
                items.append(q._ProjRows(self.imgs[c][i].data_ptr(), n, k, self.xs[j].data_ptr(),
                                         self.wss[j].data_ptr(), self.wss[j].numel(), self.ys[i].data_ptr()))
            self.projs.append(ctypes_arr(q._ProjRows, items))
        # the GEMV launch alone, on rows quantized once beforehand (as a model's fused norm step leaves them)
        self.prepared = [ctypes_arr(q._Proj, [q._Proj(self.imgs[c][i].data_ptr(), n, k,
                                                      self.wss[LAYER_SRC.get(nm, 0)].data_ptr(),
                                                      self.wss[LAYER_SRC.get(nm, 0)].numel(), self.ys[i].data_ptr())
                                              for i, (nm, n, k) in enumerate(self.layer)])
                         for c in range(self.copies)]
        # launches of one step: the GEMV set, plus one quantize launch where the set does not quantize inside
        self.launches = 1 if q.set_fuses(self.fmt, rows) else 2

    def prepare(self, L, sh):
        acts = ctypes_arr(self.q._Act, [self.q._Act(x.data_ptr(), x.shape[1], w.data_ptr(), w.numel())
                                        for x, w in zip(self.xs, self.wss)])
        L.qg_prepare_rows_set(acts, len(self.xs), self.rows, sh)

    def alg_bytes_gemv(self):
        """Algorithmic bytes of the GEMV launch: weights + activations + fp32 outputs.

        Quantizing inside (set_fuses): each distinct fp32 activation set is read once.  Otherwise the launch
        reads q8 rows (codes + fp32 scales, + int32 code sums for Q4_0) per projection."""
        out = sum(self.rows * n * 4 for _, n, _k in self.layer)
        if self.q.set_fuses(self.fmt, self.rows):
            srcs = {}
            for name, _n, k in self.layer:
                srcs[LAYER_SRC.get(name, 0)] = k
            return self.wbytes + out + sum(self.rows * k * 4 for k in srcs.values())
        act = 1.0 + 4.0 / 32 + (4.0 / 32 if self.fmt in (self.q.Q4_0, self.q.Q4_K) else 0.0)
        return self.wbytes + out + sum(self.rows * k * act for _, _n, k in self.layer)


def q8_alg_bytes(q, fmt, n, k, rows, fused):
    """Algorithmic bytes of one q8-lane GEMV launch: the image, the activation rows (fp32 when quantized inside
    the launch, else q8 codes + fp32 scales (+ int32 code sums for Q4_0)), the fp32 outputs."""
    act = 4.0 if fused else 1.0 + 4.0 / 32 + (4.0 / 32 if fmt in (q.Q4_0, q.Q4_K) else 0.0)
    return q.image_bytes(fmt, n, k) + rows * k * act + rows * n * 4


class LmHead:
    """The LM head 128256 x 4096 in one lane: two weight copies, activation rows, prepared workspaces."""

    def __init__(self, torch, q, synth, lane):
        self.torch, self.q, self.lane = torch, q, lane
        self.fmt = {"q8_0": q.Q8_0, "q4_0": q.Q4_0, "q4_k": q.Q4_K, "f16": q.F16, "fp8": q.FP8}[lane]
        self.imgs = []
        for c in range(2):
            w = synth.gaussian((LM_N, LM_K), 0.02, synth.tensor_seed(4, 0, c), device="cuda")
            self.imgs.append(q.f16_image(w.half()) if lane == "f16" else q.quantize_weights(self.fmt, w))
            del w
        self.ptrs = [t.data_ptr() for t in self.imgs]
        self.wbytes = 2 * LM_N * LM_K if lane == "f16" else q.image_bytes(self.fmt, LM_N, LM_K)
        self.rows = {}
        self.keep = []

    def at(self, synth, rows):
        """(x, y, ws) for `rows` rows; ws is prepared (q8 pair/row order or FP8 groups) for the kernel-alone form."""
        if rows not in self.rows:
            torch, q = self.torch, self.q
            x = synth.gaussian((rows, LM_K), 1.0, synth.tensor_seed(4, 32 + rows), device="cuda")
            y = torch.empty((rows, LM_N), device="cuda")
            if self.fmt == q.FP8:
                ws = q.prepare_fp8(x)
            elif self.fmt in (q.Q8_0, q.Q4_0, q.Q4_K):
                ws = q.prepare_rows(x)
            else:
                ws = None
            self.rows[rows] = (x, y, ws)
        return self.rows[rows]

    def call(self, L, sh, synth, rows):
        """The public entry point at `rows` rows (fp32 rows in; quantization included)."""
        x, y, _ = self.at(synth, rows)
        q, p = self.q, self.ptrs
        xp, yp = x.data_ptr(), y.data_ptr()
        if self.fmt == q.F16:
            return lambda i: L.gemv_f16(p[i % 2], LM_N, LM_K, xp, rows, yp, sh)
        nb = q.fp8_workspace_bytes(rows, LM_K) if self.fmt == q.FP8 else q.workspace_bytes(rows, LM_K)
        ws = self.torch.empty(max(1, nb), dtype=self.torch.uint8, device="cuda")
        self.keep.append(ws)
        wp, wn = ws.data_ptr(), ws.numel()
        if self.fmt == q.FP8:
            return lambda i: L.qgemv_fp8(p[i % 2], LM_N, LM_K, xp, rows, yp, wp, wn, sh)
        fn = {q.Q8_0: L.qgemv_q8_0, q.Q4_0: L.qgemv_q4_0, q.Q4_K: L.qgemv_q4_k}[self.fmt]
        return lambda i: fn(p[i % 2], LM_N, LM_K, xp, rows, yp, wp, wn, sh)

    def kernel_alone(self, L, sh, synth, rows):
        """(fn, kernel name, algorithmic bytes): one GEMV launch per call.  At rows the library quantizes inside
        the launch (q8 lane, 1-2 rows), and in the f16 lane, that is the entry point itself; otherwise the GEMV
        on rows prepared once."""
        q = self.q
        x, y, ws = self.at(synth, rows)
        p, yp = self.ptrs, y.data_ptr()
        if self.fmt == q.F16:
            return (self.call(L, sh, synth, rows), "gemv_f16_kernel",
                    2 * LM_N * LM_K + rows * LM_K * 4 + rows * LM_N * 4)
        if self.fmt == q.FP8:
            wp, wn = ws.data_ptr(), ws.numel()
            alg = self.wbytes + rows * LM_K * (1 + 4 / 128) + rows * LM_N * 4
            return (lambda i: L.qgemv_fp8_prepared(p[i % 2], LM_N, LM_K, wp, wn, rows, yp, sh)), "gemv_fp8_kernel", alg
        if rows <= q.FUSED_ROWS:
            return self.call(L, sh, synth, rows), "rl_set_kernel", q8_alg_bytes(q, self.fmt, LM_N, LM_K, rows, True)
        wp, wn = ws.data_ptr(), ws.numel()
        return ((lambda i: L.qgemv_prepared(self.fmt, p[i % 2], LM_N, LM_K, wp, wn, rows, yp, sh)), "mp_set_kernel",
                q8_alg_bytes(q, self.fmt, LM_N, LM_K, rows, False))


# ---------------------------------------------------------- read ceiling ---
def read_ceiling(torch, L, sh, stream, timer, sizes):
    """Best bare-read bandwidth (qg_read_probe) for each byte count, over grids and loads in flight; sizes smaller
    than 1 GiB rotate through slices of a 1 GiB buffer so that they stream from HBM."""
    buf = torch.empty(max(1 << 30, 2 * max(sizes)) + 4096, dtype=torch.uint8, device="cuda")
    base = (buf.data_ptr() + 255) // 256 * 256
    sink = torch.empty(65536 * 8, dtype=torch.int32, device="cuda")
    sp = sink.data_ptr()
    out = []
    for nbytes in sizes:
        nb = nbytes // 256 * 256
        slices = max(1, (buf.numel() - 4096) // nb)
        cands = []
        for grid in (256, 512, 1024, 2048, 4096):
            for la in (2, 4, 8):
                fn = lambda i, g=grid, la=la: L.qg_read_probe(C.c_void_p(base + (i % slices) * nb), nb, g, la, sp, sh)
                ms = time_reps(torch, timer, stream, fn, 20, reps=1)[0]
                cands.append((ms, grid, la))
        _, grid, la = min(cands)
        fn = lambda i: L.qg_read_probe(C.c_void_p(base + (i % slices) * nb), nb, grid, la, sp, sh)
        reps = time_reps(torch, timer, stream, fn, 40)
        med = statistics.median(reps)
        out.append({"bytes": int(nb), "best_gbps": round(nb / (med * 1e-3) / 1e9, 1),
                    "pct_hbm": round(100 * nb / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1), "grid": grid,
                    "loads_in_flight": la, **summarize(reps), "rotating_slices": int(slices)})
    del buf, sink
    return {"kernel": "read_probe_kernel (qg_read_probe): 16-byte non-temporal loads, one contiguous range per "
                      "512-thread workgroup; best of grids 256-4096 x 2/4/8 loads in flight", "sizes": out}


def ceiling_for(rc, nbytes):
    """The probe figure measured on the nearest byte count."""
    if not rc:
        return None
    best = min(rc["sizes"], key=lambda e: abs(math.log(e["bytes"] / nbytes)))
    return best["best_gbps"]


# -------------------------------------------------------------------- main ---
def main():
    args = parse()
    if args.traffic:
        reduce_traffic(*args.traffic)
        return
    if args.counters:
        reduce_counters(*args.counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU: the GEMV path runs on a single MI355X and has no multi-GPU "
              "path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    from block_quantized_few_amd import qgemv as q
    from block_quantized_few_amd import synth

    torch.cuda.set_device(0)
    L = q.lib()
    stream = torch.cuda.current_stream()
    sh = C.c_void_p(stream.cuda_stream)
    timer = Timer(torch)
    if args.calibrate_copy:
        calibrate_copy(torch)
    if args.profile:
        profile_one(args, torch, q, synth, L, sh, stream, timer)
        return
    t_start = time.time()

    def note(msg):
        print(f"[bench {time.time() - t_start:6.1f}s] {msg}", file=sys.stderr, flush=True)

    # ---------------------------------------------------------- ceilings ---
    rc = read_ceiling(torch, L, sh, stream, timer,
                      [q.image_bytes(q.Q8_0, LM_N, LM_K), sum(q.image_bytes(q.Q8_0, n, k) for _, n, k in LAYER_1B),
                       sum(q.image_bytes(q.Q4_0, n, k) for _, n, k in LAYER_3B)])
    note(f"read ceiling {[(e['bytes'], e['best_gbps']) for e in rc['sizes']]}")

    # ------------------------------------------------------------ headline ---
    head = LmHead(torch, q, synth, "q8_0")
    calls = {r: head.call(L, sh, synth, r) for r in HEAD_ROWS}
    torch.cuda.synchronize()
    note("LM head Q8_0 ready")

    def step(i):
        for j, r in enumerate(HEAD_ROWS):
            calls[r](3 * i + j)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timer.hold(max(20.0, K * 0.4))
    start.record(stream)
    h0 = time.perf_counter()
    for i in range(K):
        step(i)
    host_ms = (time.perf_counter() - h0) * 1e3
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K
    for r in HEAD_ROWS:
        assert bool(torch.isfinite(head.at(synth, r)[1]).all()), f"non-finite LM-head output at rows={r}"
    step_bytes = head.wbytes * len(HEAD_ROWS)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    note(f"headline step {ms_per_step * 1e3:.1f} us")

    # the step in five reps (median, slowest), and each row count's GEMV kernel alone
    step_reps = time_reps(torch, timer, stream, step, max(10, K // 3))
    ceil_lm = ceiling_for(rc, head.wbytes)
    by_rows, alg_sum, us_sum = [], 0.0, 0.0
    for r in HEAD_ROWS:
        fn, kname, alg = head.kernel_alone(L, sh, synth, r)
        reps = time_reps(torch, timer, stream, fn, 40)
        wl = f"lm-head-q8_0-rows{r}"
        e = {"rows": r, **roofline_entry(kname, alg, reps, read_traffic(kname, wl), ceil_lm, read_busy(kname, wl))}
        e["weight_gbps"] = round(head.wbytes / (statistics.median(reps) * 1e-3) / 1e9, 1)
        e["pct_hbm_weight"] = round(100 * e["weight_gbps"] / HBM_PEAK_GBPS, 1)
        e["entry_point_us"] = summarize(time_reps(torch, timer, stream, calls[r], 40))
        by_rows.append(e)
        alg_sum += alg
        us_sum += statistics.median(reps) * 1e3
    note("headline rooflines done")
    achieved = alg_sum / (us_sum * 1e-6) / 1e9
    traffic = sum(e["traffic"] for e in by_rows) if all(e["traffic"] for e in by_rows) else None
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "pct_hbm_roofline": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "step_reps": summarize(step_reps),
        "config": {"workload": "lm head 128256x4096, Q8_0 weights, q8 activations, at 1, 8 and 16 rows",
                   "rows": list(HEAD_ROWS), "calls_per_step": len(HEAD_ROWS),
                   "weight_bytes_per_call": head.wbytes, "weight_bytes_per_step": step_bytes,
                   "rotation_copies": 2, "entry_point": "qgemv_q8_0 (fp32 rows in, quantization included)",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "rl_set_kernel (1 row, quantization fused) + mp_set_kernel (8 and 16 rows, on "
                               "prepared rows): the step's GEMV launches",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "alg_bytes_per_step": int(alg_sum), "kernel_us_per_step": round(us_sum, 3),
                     "pct_of_read_ceiling": round(100 * achieved / ceil_lm, 1) if ceil_lm else None,
                     "by_rows": by_rows},
        "read_ceiling": rc,
        "host_enqueue_ms": round(host_ms, 3),
    }
    del calls

    # --------------------------------------------------------- secondary ---
    result["secondary"] = secondary(torch, q, synth, L, sh, stream, timer, rc, note)
    del head

    # ---------------------------------------------------------- CPU oracle ---
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth)
        note("cpu baseline done")

    # --------------------------------------------------------------- sweep ---
    if not args.no_sweep:
        result["sweep"] = sweep(torch, q, synth, L, sh, stream, timer)
        note("sweep done")

    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


# ------------------------------------------------------------ secondary ---
def secondary(torch, q, synth, L, sh, stream, timer, rc, note):
    out = []

    # Llama-3.2-1B-shaped Q8_0 layer at one row (one launch: quantization fused)
    ls = LayerSet(torch, q, synth, LAYER_1B, q.Q8_0, 1, 1)
    out.append(layer_entry(torch, q, L, sh, stream, timer, rc, ls, "llama-3.2-1b-shaped decode layer", "q8_0", 1,
                           "llama1b-layer-q8_0"))
    del ls
    note("1B layer done")

    # Llama-3.2-3B-shaped layer at 1/2/4/8 rows: Q4_0, and Q4_K (the K-quant superblock form)
    for fmt, lane in ((q.Q4_0, "q4_0"), (q.Q4_K, "q4_k")):
        ls = LayerSet(torch, q, synth, LAYER_3B, fmt, 2 if fmt == q.Q4_0 else 5, 1)
        for rows in (1, 2, 4, 8):
            ls.set_rows(rows, synth, 2 if fmt == q.Q4_0 else 5)
            out.append(layer_entry(torch, q, L, sh, stream, timer, rc, ls, "llama-3.2-3b-shaped decode layer", lane,
                                   rows, f"llama3b-layer-{lane}"))
        del ls
        note(f"3B layer {lane} done")

    # LM head, the other lanes at 1/8/16 rows (f16: the workload's second lane; Q4_0: the metric's other format)
    for lane in ("f16", "q4_0"):
        h = LmHead(torch, q, synth, lane)
        for rows in HEAD_ROWS:
            fn, kname, alg = h.kernel_alone(L, sh, synth, rows)
            reps = time_reps(torch, timer, stream, fn, 20)
            wl = f"lm-head-{lane}-rows{rows}"
            e = {"workload": "lm head 128256x4096", "lane": lane, "rows": rows, "weight_bytes": int(h.wbytes),
                 "weight_gbps": round(h.wbytes / (statistics.median(reps) * 1e-3) / 1e9, 1),
                 "roofline": roofline_entry(kname, alg, reps, read_traffic(kname, wl), ceiling_for(rc, h.wbytes),
                                            read_busy(kname, wl))}
            e["pct_hbm_weight"] = round(100 * e["weight_gbps"] / HBM_PEAK_GBPS, 1)
            if lane != "f16" and rows > q.FUSED_ROWS:
                e["entry_point_us"] = summarize(time_reps(torch, timer, stream, h.call(L, sh, synth, rows), 20))
            out.append(e)
        del h
        note(f"LM head {lane} done")

    # Q8_0 1024 x 1024 at one row (launch-bound: 1.1 MB), rotating copies of >= 1 GiB
    n = k = 1024
    wb = q.image_bytes(q.Q8_0, n, k)
    copies = math.ceil((1 << 30) / wb)
    big = synth.gaussian((copies * n, k), 0.02, synth.tensor_seed(0, 0), device="cuda")
    imgs = [q.quantize_weights(q.Q8_0, big[c * n:(c + 1) * n]) for c in range(copies)]
    del big
    x = synth.gaussian((1, k), 1.0, synth.tensor_seed(0, 33), device="cuda")
    y = torch.empty((1, n), device="cuda")
    ws = q.empty_ws(1, k)
    ptrs = [im.data_ptr() for im in imgs]
    reps = time_reps(torch, timer, stream,
                     lambda i: L.qgemv_q8_0(ptrs[i % copies], n, k, x.data_ptr(), 1, y.data_ptr(), ws.data_ptr(),
                                            ws.numel(), sh), 200)
    out.append({"workload": "q8_0 gemv 1024x1024", "lane": "q8_0", "rows": 1, "weight_bytes": int(wb),
                "launches": 1, **summarize(reps),
                "weight_gbps": round(wb / (statistics.median(reps) * 1e-3) / 1e9, 1),
                "roofline": roofline_entry("rl_set_kernel", q8_alg_bytes(q, q.Q8_0, n, k, 1, True), reps),
                "note": "1.1 MB per call: a launch-bound size, timed back to back"})
    del imgs
    note("1024x1024 done")

    # routed MoE step at 1/8/9/16 rows (three launches at 1-2 rows, four up to 8 rows, six beyond)
    W = moe_weights(torch, q, synth)
    for rows in (1, 8, 9, 16):
        one, expert = moe_call(torch, q, synth, L, sh, W, rows)
        reps = time_reps(torch, timer, stream, one, 64)
        u = moe_unique(torch, one, expert)
        wb = 2 * MOE_E * MOE_HIDDEN + u * (W["gu_b"] + W["dn_b"])
        med = statistics.median(reps)
        out.append({"workload": "routed moe step (256 experts top-8 + shared, hidden 2048, ffn 512)",
                    "lane": "q8_0 + f16 router", "rows": rows, "launches": 3 if rows <= 2 else 4 if rows <= 8 else 6,
                    "unique_experts": round(u, 2), "weight_bytes": int(wb), **summarize(reps),
                    "weight_gbps": round(wb / (med * 1e-3) / 1e9, 1),
                    "pct_hbm_weight": round(100 * wb / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)})
    del W
    note("moe done")
    return out


def layer_entry(torch, q, L, sh, stream, timer, rc, ls, name, lane, rows, wl_key):
    """A decode layer's seven projections at `rows` rows: the set (ms per projection set, quantization
    included) and its GEMV kernel's roofline (the set launch itself where it quantizes inside; otherwise the GEMV
    on rows prepared once)."""
    set_reps = time_reps(torch, timer, stream,
                         lambda i: L.qgemv_set_rows(ls.fmt, ls.projs[i % ls.copies], 7, rows, sh), 100)
    if q.set_fuses(ls.fmt, rows):
        kreps, kname = set_reps, "rl_set_kernel"
    else:
        ls.prepare(L, sh)
        kreps = time_reps(torch, timer, stream,
                          lambda i: L.qgemv_set(ls.fmt, ls.prepared[i % ls.copies], 7, rows, sh), 100)
        kname = "rl_set_kernel" if rows <= q.FUSED_ROWS else "mp_set_kernel"
    wl = f"{wl_key}-rows{rows}"
    med = statistics.median(set_reps)
    return {"workload": f"{name} (7 projections)", "lane": lane, "rows": rows, "weight_bytes": int(ls.wbytes),
            "launches": ls.launches, "ms_per_set": round(med, 5), "set_reps": summarize(set_reps),
            "weight_gbps": round(ls.wbytes / (med * 1e-3) / 1e9, 1),
            "pct_hbm_weight": round(100 * ls.wbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
            "rotation_copies": ls.copies,
            "roofline": roofline_entry(kname, ls.alg_bytes_gemv(), kreps, read_traffic(kname, wl),
                                       ceiling_for(rc, ls.wbytes), read_busy(kname, wl))}


# ----------------------------------------------------------------- oracle ---
def cpu_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, os.cpu_count() or 1, avail


def cpu_baseline(synth):
    """The C oracle on a bounded slice of the headline workload: the first 32768 of the LM head's 128256 output
    rows (4096 columns, Q8_0 blocks from the oracle's own quantizer) at 1, 8 and 16 activation rows, the three
    calls as one step; five reps on all the cores this process may use (at most 16, the host share of one GPU)
    and five on one core.  GB/s counts the slice's weight bytes, as the GPU figure counts the whole image's."""
    import numpy as np

    import oracle as O

    model, nproc, avail = cpu_info()
    threads = max(1, min(16, avail))
    ns = 32768
    w = synth.gaussian((ns, LM_K), 0.02, synth.tensor_seed(4, 0, 0)).numpy()
    blocks = O.quantize_weights(O.Q8_0, w)
    del w
    xs = {r: synth.gaussian((r, LM_K), 1.0, synth.tensor_seed(4, 32 + r)).numpy() for r in HEAD_ROWS}
    sbytes = ns * LM_K // 32 * 34

    def run(th):
        reps = []
        for _ in range(REPS):
            t0 = time.perf_counter()
            for r in HEAD_ROWS:
                O.gemv_q(O.Q8_0, blocks, ns, LM_K, xs[r], threads=th)
            reps.append(time.perf_counter() - t0)
        med = statistics.median(reps)
        return {"value": round(len(HEAD_ROWS) * sbytes / med / 1e9, 3), "unit": "GB/s", "cores": th,
                "ms_per_step": round(med * 1e3, 2), "slowest_ms": round(max(reps) * 1e3, 2)}

    allc = run(threads)
    one = run(1)
    assert np.isfinite(O.gemv_q(O.Q8_0, blocks, ns, LM_K, xs[1], threads=threads)).all()
    return {**allc, "kind": "oracle",
            "sample": f"LM head rows 0..{ns - 1} of {LM_N} (x 4096, Q8_0, {sbytes} weight bytes) at rows 1, 8 and 16 "
                      f"per step; median of {REPS} reps",
            "single_core": one, "cpu_model": model, "nproc": nproc, "cores_available": avail}


# ------------------------------------------------------------------ sweep ---
def entry(workload, lane, rows, wbytes, ms_reps, launches):
    ms = statistics.median(ms_reps)
    gbps = wbytes / (ms * 1e-3) / 1e9
    return {"workload": workload, "lane": lane, "rows": rows, "weight_bytes": int(wbytes), "launches": launches,
            "us_per_call": round(ms * 1e3, 3), "slowest_rep_us": round(max(ms_reps) * 1e3, 3),
            "weight_gbps": round(gbps, 1), "pct_hbm": round(100 * gbps / HBM_PEAK_GBPS, 1)}


def sweep(torch, q, synth, L, sh, stream, timer):
    out = []
    ROWSW = [1, 2, 4, 8, 9, 16]
    # decode layers (set launch): 1B Q8_0 and 3B Q4_0
    for lname, lay, fmt, wl, lane in (("llama-3.2-1b layer", LAYER_1B, q.Q8_0, 1, "q8_0"),
                                      ("llama-3.2-3b layer", LAYER_3B, q.Q4_0, 2, "q4_0"),
                                      ("llama-3.2-3b layer", LAYER_3B, q.Q4_K, 5, "q4_k")):
        ls = LayerSet(torch, q, synth, lay, fmt, wl, 1)
        for rows in ROWSW:
            ls.set_rows(rows, synth, wl)
            reps = time_reps(torch, timer, stream,
                             lambda i: L.qgemv_set_rows(fmt, ls.projs[i % ls.copies], 7, rows, sh), 100)
            out.append(entry(f"{lname} (7 projections)", lane, rows, ls.wbytes, reps, ls.launches))
            ls.prepare(L, sh)
            reps = time_reps(torch, timer, stream,
                             lambda i: L.qgemv_set(fmt, ls.prepared[i % ls.copies], 7, rows, sh), 100)
            out.append(entry(f"{lname} (7 projections), prepared rows", lane, rows, ls.wbytes, reps, 1))
        del ls
    # LM head in every lane
    for lane in ("q8_0", "q4_0", "q4_k", "f16", "fp8"):
        h = LmHead(torch, q, synth, lane)
        for rows in ROWSW:
            reps = time_reps(torch, timer, stream, h.call(L, sh, synth, rows), 20)
            launches = 1 if lane == "f16" or (lane in ("q8_0", "q4_0", "q4_k") and rows <= q.FUSED_ROWS) else 2
            out.append(entry("lm head 128256x4096", lane, rows, h.wbytes, reps, launches))
            if launches == 2:
                fn, _, _ = h.kernel_alone(L, sh, synth, rows)
                out.append(entry("lm head 128256x4096, prepared rows", lane, rows, h.wbytes,
                                 time_reps(torch, timer, stream, fn, 20), 1))
        del h
    out.extend(moe_sweep(torch, q, synth, L, sh, stream, timer))
    out.extend(grouped_sweep(torch, q, synth, L, sh, stream, timer))
    return out


MOE_HIDDEN, MOE_FFN, MOE_E, MOE_TOPK = 2048, 512, 256, 8


def moe_weights(torch, q, synth, copies=2, fmt=None):
    """Two copies of the routed MoE's 256 experts (Q8_0, or fmt) plus the shared one (index 256), stacked, and
    the f16 router image.  Each copy's gate/up and down weights are drawn as one tall matrix each (one
    generator call), then quantized expert by expert into the stacked images."""
    hidden, ffn, E = MOE_HIDDEN, MOE_FFN, MOE_E
    fmt = q.Q8_0 if fmt is None else fmt
    nimg = E + 1
    gu_b = q.image_bytes(fmt, 2 * ffn, hidden)
    dn_b = q.image_bytes(fmt, hidden, ffn)
    gus, dns = [], []
    for c in range(copies):
        gu = torch.empty(nimg * gu_b, dtype=torch.uint8, device="cuda")
        dn = torch.empty(nimg * dn_b, dtype=torch.uint8, device="cuda")
        w = synth.gaussian((nimg * 2 * ffn, hidden), 0.02, synth.tensor_seed(3, 1, c), device="cuda")
        for e in range(nimg):
            q.quantize_weights(fmt, w[e * 2 * ffn:(e + 1) * 2 * ffn], gu[e * gu_b:(e + 1) * gu_b])
        w = synth.gaussian((nimg * hidden, ffn), 0.02, synth.tensor_seed(3, 3, c), device="cuda")
        for e in range(nimg):
            q.quantize_weights(fmt, w[e * hidden:(e + 1) * hidden], dn[e * dn_b:(e + 1) * dn_b])
        del w
        gus.append(gu)
        dns.append(dn)
    router = q.f16_image(synth.gaussian((E, hidden), 0.02, synth.tensor_seed(3, 0), device="cuda").half())
    return {"router": router, "gu": gus, "dn": dns, "gu_b": gu_b, "dn_b": dn_b, "fmt": fmt}


def moe_call(torch, q, synth, L, sh, W, rows, nx=64):
    """One qg_moe_step call per index i (weight copy i % copies, input i % nx) and the routed experts."""
    hidden, ffn, E, topk = MOE_HIDDEN, MOE_FFN, MOE_E, MOE_TOPK
    m = rows * (topk + 1)
    xs = [synth.gaussian((rows, hidden), 1.0, synth.tensor_seed(3, 32 + rows, s), device="cuda") for s in range(nx)]
    logits = torch.empty((rows, E), device="cuda")
    expert = torch.empty(m, dtype=torch.int32, device="cuda")
    wgt = torch.empty(m, device="cuda")
    y = torch.empty((rows, hidden), device="cuda")
    fp8 = W["fmt"] == q.FP8
    wsb = (q.moe_fp8_workspace_bytes if fp8 else q.moe_workspace_bytes)(rows, E, hidden, ffn, topk, True)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    P = lambda t: t.data_ptr()
    xps = [P(x) for x in xs]
    copies = len(W["gu"])
    step = L.qg_moe_step_fp8 if fp8 else L.qg_moe_step

    def one(i):
        c = i % copies
        step(P(W["router"]), E, hidden, ffn, topk, 1, P(W["gu"][c]), P(W["dn"][c]), xps[i % nx], rows, P(y),
             P(logits), P(expert), P(wgt), P(ws), ws.numel(), sh)

    # keep the inputs alive with the closure's owner
    one.keep = (xs, logits, expert, wgt, y, ws)
    one.nx = nx
    return one, expert


def moe_unique(torch, one, expert):
    """Average count of distinct experts (the shared one included) that a call touches, over the inputs."""
    uniq = []
    for s in range(one.nx):
        one(s)
        torch.cuda.synchronize()
        uniq.append(len(set(expert.cpu().tolist())))
    return sum(uniq) / len(uniq)


def moe_sweep(torch, q, synth, L, sh, stream, timer):
    """Routed MoE step (qg_moe_step) in the Q8_0 and FP8 lanes at 1/8/9/16 rows."""
    out = []
    for fmt, lane in ((q.Q8_0, "q8_0 + f16 router"), (q.FP8, "fp8 + f16 router")):
        W = moe_weights(torch, q, synth, fmt=fmt)
        for rows in (1, 8, 9, 16):
            one, expert = moe_call(torch, q, synth, L, sh, W, rows)
            reps = time_reps(torch, timer, stream, one, 64)
            u = moe_unique(torch, one, expert)
            wb = 2 * MOE_E * MOE_HIDDEN + u * (W["gu_b"] + W["dn_b"])
            launches = ((4 if rows == 1 else 5 if rows <= 8 else 6) if fmt == q.FP8 else
                        (3 if rows <= 2 else 4 if rows <= 8 else 6))
            e = entry("routed moe step (256 experts top-8 + shared)", lane, rows, wb, reps, launches)
            e["unique_experts"] = round(u, 2)
            out.append(e)
        del W
    return out


def grouped_sweep(torch, q, synth, L, sh, stream, timer):
    """Grouped routed-expert GEMV alone at the MoE's gate/up shape (257 experts of 1024 x 2048: top-8 of 256 plus
    a shared one per row), Q8_0 and FP8 lanes, 16 seeded routings and two weight copies in rotation; weight
    bytes are those of the experts each call touches."""
    import numpy as np

    n, k, E, topk, nx = 2 * MOE_FFN, MOE_HIDDEN, MOE_E, MOE_TOPK, 16
    out = []
    for lane, fmt in (("q8_0", q.Q8_0), ("fp8", q.FP8)):
        eb = q.image_bytes(fmt, n, k)
        imgs = []
        for c in range(2):
            buf = torch.empty((E + 1) * eb, dtype=torch.uint8, device="cuda")
            w = synth.gaussian(((E + 1) * n, k), 0.02, synth.tensor_seed(8, 0, c), device="cuda")
            for e in range(E + 1):
                q.quantize_weights(fmt, w[e * n:(e + 1) * n], buf[e * eb:(e + 1) * eb])
            del w
            imgs.append(buf)
        for rows in (1, 8, 16):
            m = rows * (topk + 1)
            rng = np.random.default_rng(1000 + rows)
            routes = []
            for _ in range(nx):
                ex = np.concatenate([np.concatenate([rng.choice(E, topk, replace=False), [E]]) for _ in range(rows)])
                routes.append(torch.from_numpy(ex.astype(np.int32)).cuda())
            xi = torch.from_numpy(np.repeat(np.arange(rows), topk + 1).astype(np.int32)).cuda()
            x = synth.gaussian((rows, k), 1.0, synth.tensor_seed(8, 300 + rows), device="cuda")
            y = torch.empty((m, n), device="cuda")
            if fmt == q.FP8:
                ws = torch.empty(q.fp8_grouped_workspace_bytes(rows, k, m), dtype=torch.uint8, device="cuda")
                call = L.qgemv_fp8_grouped
            else:
                ws = torch.empty(q.grouped_workspace_bytes(rows, k, m), dtype=torch.uint8, device="cuda")
                call = L.qgemv_q8_0_grouped
            ip = [t.data_ptr() for t in imgs]
            rp = [t.data_ptr() for t in routes]

            def one(i, call=call, ip=ip, rp=rp, x=x, xi=xi, y=y, ws=ws, rows=rows, m=m):
                call(ip[i % 2], E + 1, n, k, x.data_ptr(), rows, rp[i % nx], xi.data_ptr(), m, y.data_ptr(),
                     ws.data_ptr(), ws.numel(), sh)

            reps = time_reps(torch, timer, stream, one, 64)
            u = sum(len(set(t.cpu().tolist())) for t in routes) / nx
            e_ = entry("grouped gate/up 1024x2048, 256 experts top-8 + shared", lane, rows, u * eb, reps, 2)
            e_["unique_experts"] = round(u, 2)
            out.append(e_)
        del imgs
    return out


def profile_one(args, torch, q, synth, L, sh, stream, timer):
    """--profile WORKLOAD:ROWS: one workload, a short warm-up then --steps timed calls, for a per-kernel profile
    (rocprofv3 --kernel-trace --stats, or one --pmc counter set per run)."""
    wl, rows = args.profile.split(":")
    rows = int(rows)
    if wl.startswith("lm-head-"):
        lane = wl[len("lm-head-"):]
        prepared = lane.endswith("-prepared")
        lane = {"q8": "q8_0", "q4": "q4_0", "q4k": "q4_k"}.get(lane.replace("-prepared", ""),
                                                             lane.replace("-prepared", ""))
        h = LmHead(torch, q, synth, lane)
        fn = h.kernel_alone(L, sh, synth, rows)[0] if prepared else h.call(L, sh, synth, rows)
        wbytes = h.wbytes
    elif wl in ("layer-1b", "layer-3b", "layer-1b-prepared", "layer-3b-prepared", "layer-3b-q4k",
                "layer-3b-q4k-prepared"):
        lay, fmt, wid = ((LAYER_1B, q.Q8_0, 1) if wl.startswith("layer-1b") else
                         (LAYER_3B, q.Q4_K, 5) if wl.startswith("layer-3b-q4k") else (LAYER_3B, q.Q4_0, 2))
        ls = LayerSet(torch, q, synth, lay, fmt, wid, rows)
        if wl.endswith("-prepared"):
            ls.prepare(L, sh)
            fn = lambda i: L.qgemv_set(fmt, ls.prepared[i % ls.copies], 7, rows, sh)
        else:
            fn = lambda i: L.qgemv_set_rows(fmt, ls.projs[i % ls.copies], 7, rows, sh)
        wbytes = ls.wbytes
    elif wl in ("moe", "moe-fp8"):
        W = moe_weights(torch, q, synth, fmt=q.FP8 if wl == "moe-fp8" else None)
        fn, _ = moe_call(torch, q, synth, L, sh, W, rows)
        wbytes = None
    elif wl == "read-probe":
        nb = q.image_bytes(q.Q8_0, LM_N, LM_K)
        buf = torch.empty(2 * nb + 512, dtype=torch.uint8, device="cuda")
        base = (buf.data_ptr() + 255) // 256 * 256
        sink = torch.empty(65536 * 8, dtype=torch.int32, device="cuda")
        fn = lambda i: L.qg_read_probe(C.c_void_p(base + (i % 2) * nb), nb, 1024, 4, sink.data_ptr(), sh)
        wbytes = nb
    else:
        raise SystemExit(f"--profile: unknown workload {wl!r}")
    ms = statistics.median(time_reps(torch, timer, stream, fn, args.steps, reps=1))
    line = {"profile": wl, "rows": rows, "steps": args.steps, "us_per_call": round(ms * 1e3, 3)}
    if wbytes:
        line["weight_bytes"] = int(wbytes)
        line["weight_gbps"] = round(wbytes / (ms * 1e-3) / 1e9, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
