#!/usr/bin/env python3
"""Benchmark of the few-row block-quantized GEMV on one MI355X.

Headline step: one decode layer of a Llama-3.2-1B-shaped model in the Q8_0
lane at one activation row -- the seven projections Wq 2048x2048, Wk/Wv
512x2048, Wo 2048x2048, gate/up 8192x2048, down 2048x8192 (64,618,496 weight
bytes) with the q8 quantization of their three fp32 input rows, all in one
launch.  The weights rotate through enough distinct copies (>= 1 GiB) that every
step streams them from HBM, not from the 256 MB Infinity Cache.

Prints one JSON line: weight GB/s of the step (value), the roofline of the
GEMV kernel measured with HIP events on its own stream, the CPU oracle timed on
a bounded sample, and (unless --no-sweep) the other workloads at 1..16 rows.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-sweep] [--no-cpu-baseline]
"""
import argparse
import ctypes as C
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "weight GB/s and % HBM roofline for Q8_0/Q4_0 GEMV at 1/8/16 rows"

LAYER_1B = [("wq", 2048, 2048), ("wk", 512, 2048), ("wv", 512, 2048), ("wo", 2048, 2048), ("gate", 8192, 2048),
            ("up", 8192, 2048), ("down", 2048, 8192)]
LAYER_3B = [("wq", 3072, 3072), ("wk", 1024, 3072), ("wv", 1024, 3072), ("wo", 3072, 3072), ("gate", 8192, 3072),
            ("up", 8192, 3072), ("down", 3072, 8192)]
# which of the three input rows (block input, attention output, FFN hidden) feeds each projection
LAYER_SRC = {"wo": 1, "down": 2}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--out", default=None, help="also write the JSON line (with the sweep) to this file")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run a plain elementwise kernel over 256 MiB (reads 256 MiB, writes 256 MiB) five "
                        "times, the known-size reference for the HBM byte counters")
    p.add_argument("--profile", default=None, metavar="WORKLOAD:ROWS",
                   help="time one sweep workload (lm-head-q8, lm-head-f16, lm-head-fp8, layer-1b, layer-3b, moe) at "
                        "ROWS activation rows for --steps calls after warm-up, print it, and exit: a short program "
                        "for rocprofv3")
    p.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                   help="reduce two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then WRITE_SIZE) "
                        "of a --calibrate-copy run into profiles/traffic.json, then exit")
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


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("qg_q8.hip", "qg_device.h", "qg_layout.h"):
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


def reduce_traffic(fetch_csv, write_csv):
    """HBM bytes per launch of the headline kernel, from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by the factor that maps the same counter to the known bytes of the calibration kernel."""
    fetch = pmc_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = pmc_per_dispatch(write_csv, "WRITE_SIZE")

    def pick(d, pat, big=False):
        vals = [v for name, vs in d.items() if pat in name for v in vs]
        if big:
            vals = [v for v in vals if v * 1024 > COPY_BYTES / 2]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel named like {pat!r} in the counter file")
        return sum(vals) / len(vals), len(vals)

    cf, _ = pick(fetch, "neg", big=True)
    cw, _ = pick(write, "neg", big=True)
    kf, nf = pick(fetch, "rl_set_kernel")
    kw, nw = pick(write, "rl_set_kernel")
    ff, fw = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    rec = {"rl_set_kernel|llama1b-layer-q8_0-rows1": {
        "hbm_bytes_per_launch": round(kf * 1024 * ff + kw * 1024 * fw),
        "fetch_kib_per_dispatch": round(kf, 1), "write_kib_per_dispatch": round(kw, 1), "dispatches": [nf, nw],
        "calibration": {"kernel": "torch.neg over 256 MiB fp32", "known_bytes_each_way": COPY_BYTES,
                        "fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                        "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)},
        "source_hash": kernel_source_hash()}}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed PMC summary, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(f"{kernel}|{workload}")
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


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
        # launches of one step: the GEMV set, plus one quantize launch above the fused row count
        self.launches = 1 if rows <= q.FUSED_ROWS else 2

    def alg_bytes_gemv(self):
        """Algorithmic bytes of the GEMV launch: weights + activations + fp32 outputs.

        Fused (rows <= FUSED_ROWS): each distinct fp32 activation set is read once.  Otherwise the launch
        reads q8 rows (codes + fp32 scales, + int32 code sums for Q4_0) per projection."""
        out = sum(self.rows * n * 4 for _, n, _k in self.layer)
        if self.rows <= self.q.FUSED_ROWS:
            srcs = {}
            for name, _n, k in self.layer:
                srcs[LAYER_SRC.get(name, 0)] = k
            return self.wbytes + out + sum(self.rows * k * 4 for k in srcs.values())
        act = 1.0 + 4.0 / 32 + (4.0 / 32 if self.fmt == self.q.Q4_0 else 0.0)
        return self.wbytes + out + sum(self.rows * k * act for _, _n, k in self.layer)


def main():
    args = parse()
    if args.traffic:
        reduce_traffic(*args.traffic)
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

    # ------------------------------------------------------------ headline ---
    rows = 1
    t_setup = time.time()
    layer = LayerSet(torch, q, synth, LAYER_1B, q.Q8_0, 1, rows)
    torch.cuda.synchronize()
    print(f"[bench] 1B layer Q8_0: {layer.copies} copies x {layer.wbytes} B ready in {time.time() - t_setup:.1f}s",
          file=sys.stderr, flush=True)

    def step(i):
        L.qgemv_set_rows(q.Q8_0, layer.projs[i % layer.copies], 7, rows, sh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    timer.hold(max(20.0, K * 0.08))
    start.record(stream)
    h0 = time.perf_counter()
    for i in range(K):
        step(i)
    host_ms = (time.perf_counter() - h0) * 1e3
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K
    # At one row the step is one launch of the GEMV kernel (quantization fused), so the events around the
    # K back-to-back steps on the kernel's own stream also give its average launch duration.
    assert layer.launches == 1
    gemv_avg_ms = ms_per_step
    # a host-side check that the layer outputs are finite (no silent garbage)
    assert all(bool(torch.isfinite(y).all()) for y in layer.ys)

    value = layer.wbytes / (ms_per_step * 1e-3) / 1e9
    alg = layer.alg_bytes_gemv()
    achieved = alg / (gemv_avg_ms * 1e-3) / 1e9
    kname = "rl_set_kernel<Q8_0, rows 1, fused quantization>"
    traffic = read_traffic("rl_set_kernel", "llama1b-layer-q8_0-rows1")
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
        "config": {"workload": "llama-3.2-1b-shaped decode layer, Q8_0 weights, q8 activations",
                   "rows": rows, "projections": [f"{nm} {n}x{k}" for nm, n, k in LAYER_1B],
                   "weight_bytes_per_step": layer.wbytes, "rotation_copies": layer.copies,
                   "launches_per_step": layer.launches, "parallelism": "single GPU"},
        "roofline": {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": int(alg), "avg_launch_us": round(gemv_avg_ms * 1e3, 3)},
        "host_enqueue_ms": round(host_ms, 3),
    }

    # ---------------------------------------------------------- CPU oracle ---
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(torch, synth, layer)

    # --------------------------------------------------------------- sweep ---
    if not args.no_sweep:
        result["sweep"] = sweep(torch, q, synth, L, sh, stream, timer, layer)

    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


# ----------------------------------------------------------------- oracle ---
def cpu_baseline(torch, synth, layer):
    """The C oracle on the headline layer (copy 0, same rows), on the host's cores, for about 10 s."""
    import oracle as O

    threads = max(1, min(16, os.cpu_count() or 1))
    blocks = []
    for i, (_, n, k) in enumerate(LAYER_1B):
        w = synth.gaussian((n, k), 0.02, synth.tensor_seed(1, i, 0), device="cuda").cpu().numpy()
        blocks.append(O.quantize_weights(O.Q8_0, w))
    xs = [x.cpu().numpy() for x in layer.xs]
    reps, t0 = 0, time.perf_counter()
    while True:
        for i, (name, n, k) in enumerate(LAYER_1B):
            O.gemv_q(O.Q8_0, blocks[i], n, k, xs[LAYER_SRC.get(name, 0)], threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0:
            break
    return {"value": round(layer.wbytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "ms_per_step": round(el / reps * 1e3, 3),
            "sample": f"the headline layer's 7 Q8_0 projections at rows={layer.rows}, {reps} reps in {el:.1f}s"}


# ------------------------------------------------------------------ sweep ---
def time_calls(torch, timer, stream, fn, iters):
    for i in range(min(iters, 5)):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timer.hold(max(10.0, iters * 0.1))
    a.record(stream)
    for i in range(iters):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def entry(workload, lane, rows, wbytes, ms, launches):
    gbps = wbytes / (ms * 1e-3) / 1e9
    return {"workload": workload, "lane": lane, "rows": rows, "weight_bytes": int(wbytes), "launches": launches,
            "us_per_call": round(ms * 1e3, 3), "weight_gbps": round(gbps, 1),
            "pct_hbm": round(100 * gbps / HBM_PEAK_GBPS, 1)}


def sweep(torch, q, synth, L, sh, stream, timer, layer1b):
    out = []
    ROWSW = [1, 2, 4, 8, 9, 16]
    t0 = time.time()

    # Q8_0 1024x1024, one GEMV (quantize + GEMV launches)
    n = k = 1024
    wb = q.image_bytes(q.Q8_0, n, k)
    copies = math.ceil((1 << 30) / wb)
    big = synth.gaussian((copies * n, k), 0.02, synth.tensor_seed(0, 0), device="cuda")
    imgs = [q.quantize_weights(q.Q8_0, big[c * n:(c + 1) * n]) for c in range(copies)]
    del big
    for rows in ROWSW:
        x = synth.gaussian((rows, k), 1.0, synth.tensor_seed(0, 32 + rows), device="cuda")
        y = torch.empty((rows, n), device="cuda")
        ws = q.empty_ws(rows, k)
        xp, yp, wp, wn = x.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel()
        ptrs = [im.data_ptr() for im in imgs]
        ms = time_calls(torch, timer, stream, lambda i: L.qgemv_q8_0(ptrs[i % copies], n, k, xp, rows, yp, wp, wn, sh),
                        400)
        out.append(entry("q8_0 1024x1024", "q8_0", rows, wb, ms, 1 if rows <= q.FUSED_ROWS else 2))
    del imgs
    print(f"[bench] sweep 1024x1024 done {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # residual add + RMS norm + A1 in one launch (qg_add_rmsnorm_prepare), next to A1 alone (qg_prepare_rows)
    # of the same rows; bytes: x, residual and gamma read, h and the workspace written
    for k in (2048, 8192):
        gamma = (1.0 + synth.gaussian((k,), 0.1, synth.tensor_seed(6, 2), device="cuda")).contiguous()
        for rows in (1, 8, 16):
            x = synth.gaussian((rows, k), 1.0, synth.tensor_seed(6, 32 + rows), device="cuda")
            res = synth.gaussian((rows, k), 0.5, synth.tensor_seed(6, 48 + rows), device="cuda")
            h = torch.empty_like(x)
            ws = q.empty_ws(rows, k)
            xp, rp, gp, hp, wp, wn = x.data_ptr(), res.data_ptr(), gamma.data_ptr(), h.data_ptr(), ws.data_ptr(), ws.numel()
            nb = 4 * rows * k * 3 + 4 * k + q.workspace_bytes(rows, k)
            ms = time_calls(torch, timer, stream,
                            lambda i: L.qg_add_rmsnorm_prepare(xp, rp, gp, 1e-5, rows, k, hp, None, wp, wn, sh), 400)
            e = entry(f"add + rmsnorm + q8 prepare, k={k}", "fp32 -> q8", rows, nb, ms, 1)
            e["note"] = "weight_bytes here: activation bytes moved"
            out.append(e)
            ms = time_calls(torch, timer, stream, lambda i: L.qg_prepare_rows(xp, rows, k, wp, wn, sh), 400)
            e = entry(f"q8 prepare alone, k={k}", "fp32 -> q8", rows, 4 * rows * k + q.workspace_bytes(rows, k), ms, 1)
            e["note"] = "weight_bytes here: activation bytes moved"
            out.append(e)
    print(f"[bench] sweep norm done {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # decode layers (set launch): 1B Q8_0 and 3B Q4_0
    for lname, lay, fmt, wl, lane, obj in (("llama-3.2-1b layer", LAYER_1B, q.Q8_0, 1, "q8_0", layer1b),
                                           ("llama-3.2-3b layer", LAYER_3B, q.Q4_0, 2, "q4_0", None)):
        ls = obj or LayerSet(torch, q, synth, lay, fmt, wl, 1)
        for rows in ROWSW:
            ls.set_rows(rows, synth, wl)

            def one(i, ls=ls, rows=rows, fmt=fmt):
                L.qgemv_set_rows(fmt, ls.projs[i % ls.copies], 7, rows, sh)

            ms = time_calls(torch, timer, stream, one, 200)
            out.append(entry(f"{lname} (7 projections)", lane, rows, ls.wbytes, ms, ls.launches))
            if rows > q.FUSED_ROWS:
                # the GEMV launch alone, on rows quantized once beforehand
                acts = ctypes_arr(q._Act, [q._Act(x.data_ptr(), x.shape[1], w.data_ptr(), w.numel())
                                           for x, w in zip(ls.xs, ls.wss)])
                L.qg_prepare_rows_set(acts, len(ls.xs), rows, sh)
                pre = [ctypes_arr(q._Proj, [q._Proj(ls.imgs[c][i].data_ptr(), n_, k_,
                                                    ls.wss[LAYER_SRC.get(nm, 0)].data_ptr(),
                                                    ls.wss[LAYER_SRC.get(nm, 0)].numel(), ls.ys[i].data_ptr())
                                            for i, (nm, n_, k_) in enumerate(ls.layer)]) for c in range(ls.copies)]

                def gemv(i, pre=pre, rows=rows, fmt=fmt):
                    L.qgemv_set(fmt, pre[i % len(pre)], 7, rows, sh)

                ms = time_calls(torch, timer, stream, gemv, 200)
                out.append(entry(f"{lname} (7 projections), prepared rows", lane, rows, ls.wbytes, ms, 1))
        del ls
        print(f"[bench] sweep {lname} done {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    layer1b.set_rows(1, synth, 1)

    # LM head 128256 x 4096, f16, Q8_0 and FP8 (block-FP8 weights, 1 x 128 activation groups), two copies each
    n, k = 128256, 4096
    w16 = []
    q8 = []
    f8 = []
    for c in range(2):
        w = synth.gaussian((n, k), 0.02, synth.tensor_seed(4, 0, c), device="cuda")
        w16.append(q.f16_image(w.half()))
        q8.append(q.quantize_weights(q.Q8_0, w))
        f8.append(q.quantize_weights(q.FP8, w))
        del w
    f8b = q.image_bytes(q.FP8, n, k)
    for rows in (1, 2, 4, 8, 9, 16):
        x = synth.gaussian((rows, k), 1.0, synth.tensor_seed(4, 32 + rows), device="cuda")
        y = torch.empty((rows, n), device="cuda")
        ws = q.empty_ws(rows, k)
        xp, yp, wp, wn = x.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel()
        p16 = [t.data_ptr() for t in w16]
        p8 = [t.data_ptr() for t in q8]
        pf = [t.data_ptr() for t in f8]
        ms = time_calls(torch, timer, stream, lambda i: L.gemv_f16(p16[i % 2], n, k, xp, rows, yp, sh), 40)
        out.append(entry("lm head 128256x4096", "f16", rows, 2 * n * k, ms, 1))
        ms = time_calls(torch, timer, stream, lambda i: L.qgemv_q8_0(p8[i % 2], n, k, xp, rows, yp, wp, wn, sh), 40)
        out.append(entry("lm head 128256x4096", "q8_0", rows, q.image_bytes(q.Q8_0, n, k), ms,
                         1 if rows <= q.FUSED_ROWS else 2))
        wsf = q.prepare_fp8(x)
        fp, fn = wsf.data_ptr(), wsf.numel()
        ms = time_calls(torch, timer, stream, lambda i: L.qgemv_fp8(pf[i % 2], n, k, xp, rows, yp, fp, fn, sh), 40)
        out.append(entry("lm head 128256x4096", "fp8", rows, f8b, ms, 2))
        ms = time_calls(torch, timer, stream, lambda i: L.qgemv_fp8_prepared(pf[i % 2], n, k, fp, fn, rows, yp, sh), 40)
        out.append(entry("lm head 128256x4096, prepared rows", "fp8", rows, f8b, ms, 1))
    del w16, q8, f8
    print(f"[bench] sweep lm head done {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    out.extend(moe_sweep(torch, q, synth, L, sh, stream, timer))
    print(f"[bench] sweep moe done {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    out.extend(grouped_sweep(torch, q, synth, L, sh, stream, timer))
    print(f"[bench] sweep grouped done {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    return out


MOE_HIDDEN, MOE_FFN, MOE_E, MOE_TOPK = 2048, 512, 256, 8


def moe_weights(torch, q, synth, copies=2, fmt=None):
    """Two copies of the routed MoE's 256 experts (Q8_0, or fmt) plus the shared one (index 256), stacked, and
    the f16 router image."""
    hidden, ffn, E = MOE_HIDDEN, MOE_FFN, MOE_E
    fmt = q.Q8_0 if fmt is None else fmt
    nimg = E + 1
    gu_b = q.image_bytes(fmt, 2 * ffn, hidden)
    dn_b = q.image_bytes(fmt, hidden, ffn)
    gus, dns = [], []
    for c in range(copies):
        gu = torch.empty(nimg * gu_b, dtype=torch.uint8, device="cuda")
        dn = torch.empty(nimg * dn_b, dtype=torch.uint8, device="cuda")
        for e in range(nimg):
            w = synth.gaussian((2 * ffn, hidden), 0.02, synth.tensor_seed(3, 1 + 3 * e, c), device="cuda")
            q.quantize_weights(fmt, w, gu[e * gu_b:(e + 1) * gu_b])
            w = synth.gaussian((hidden, ffn), 0.02, synth.tensor_seed(3, 3 + 3 * e, c), device="cuda")
            q.quantize_weights(fmt, w, dn[e * dn_b:(e + 1) * dn_b])
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
    return one, expert


def moe_sweep(torch, q, synth, L, sh, stream, timer):
    """Routed MoE step (qg_moe_step): router f16 GEMV, top-8 routing + plan, grouped gate/up, SwiGLU + q8,
    grouped down, combine -- six launches, five at 1-2 rows (SwiGLU + q8 inside the down launch)."""
    out = []
    for fmt, lane in ((q.Q8_0, "q8_0 + f16 router"), (q.FP8, "fp8 + f16 router")):
        W = moe_weights(torch, q, synth, fmt=fmt)
        for rows in (1, 8, 9, 16):
            nx = 64
            one, expert = moe_call(torch, q, synth, L, sh, W, rows, nx)
            ms = time_calls(torch, timer, stream, one, 128)
            # weight bytes actually streamed: router + every touched expert (the shared one included)
            uniq = []
            for s in range(nx):
                one(s)
                torch.cuda.synchronize()
                uniq.append(len(set(expert.cpu().tolist())))
            u = sum(uniq) / nx
            wb = 2 * MOE_E * MOE_HIDDEN + u * (W["gu_b"] + W["dn_b"])
            launches = 6 if fmt == q.FP8 else (5 if rows <= 2 else 6)
            e = entry("routed moe step (256 experts top-8 + shared)", lane, rows, wb, ms, launches)
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
            for e in range(E + 1):
                w = synth.gaussian((n, k), 0.02, synth.tensor_seed(8, e, c), device="cuda")
                q.quantize_weights(fmt, w, buf[e * eb:(e + 1) * eb])
            imgs.append(buf)
        for rows in (1, 8, 16):
            m = rows * (topk + 1)
            rng = np.random.default_rng(1000 + rows)
            routes = []
            for r_ in range(nx):
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

            ms = time_calls(torch, timer, stream, one, 64)
            u = sum(len(set(t.cpu().tolist())) for t in routes) / nx
            e_ = entry("grouped gate/up 1024x2048, 256 experts top-8 + shared", lane, rows, u * eb, ms,
                       3)
            e_["unique_experts"] = round(u, 2)
            out.append(e_)
        del imgs
    return out


def profile_one(args, torch, q, synth, L, sh, stream, timer):
    """--profile WORKLOAD:ROWS: one workload of the sweep, --warmup untimed then --steps timed calls, for a
    per-kernel profile (rocprofv3 --kernel-trace --stats, or one --pmc counter per run)."""
    wl, rows = args.profile.split(":")
    rows = int(rows)
    n, k = 128256, 4096
    if wl in ("lm-head-q8", "lm-head-f16", "lm-head-fp8"):
        lane = wl[len("lm-head-"):]
        imgs = []
        for c in range(2):
            w = synth.gaussian((n, k), 0.02, synth.tensor_seed(4, 0, c), device="cuda")
            imgs.append(q.f16_image(w.half()) if lane == "f16" else
                        q.quantize_weights(q.Q8_0 if lane == "q8" else q.FP8, w))
            del w
        x = synth.gaussian((rows, k), 1.0, synth.tensor_seed(4, 32 + rows), device="cuda")
        y = torch.empty((rows, n), device="cuda")
        p = [t.data_ptr() for t in imgs]
        xp, yp = x.data_ptr(), y.data_ptr()
        if lane == "q8":
            ws = q.empty_ws(rows, k)
            fn = lambda i: L.qgemv_q8_0(p[i % 2], n, k, xp, rows, yp, ws.data_ptr(), ws.numel(), sh)
            wbytes = q.image_bytes(q.Q8_0, n, k)
        elif lane == "f16":
            fn = lambda i: L.gemv_f16(p[i % 2], n, k, xp, rows, yp, sh)
            wbytes = 2 * n * k
        else:
            ws = q.prepare_fp8(x)
            fn = lambda i: L.qgemv_fp8_prepared(p[i % 2], n, k, ws.data_ptr(), ws.numel(), rows, yp, sh)
            wbytes = q.image_bytes(q.FP8, n, k)
    elif wl in ("layer-1b", "layer-3b"):
        lay, fmt, wid = (LAYER_1B, q.Q8_0, 1) if wl == "layer-1b" else (LAYER_3B, q.Q4_0, 2)
        ls = LayerSet(torch, q, synth, lay, fmt, wid, rows)
        fn = lambda i: L.qgemv_set_rows(fmt, ls.projs[i % ls.copies], 7, rows, sh)
        wbytes = ls.wbytes
    elif wl == "moe":
        W = moe_weights(torch, q, synth)
        fn, _ = moe_call(torch, q, synth, L, sh, W, rows)
        wbytes = None
    else:
        raise SystemExit(f"--profile: unknown workload {wl!r}")
    ms = time_calls(torch, timer, stream, fn, args.steps)
    line = {"profile": wl, "rows": rows, "steps": args.steps, "us_per_call": round(ms * 1e3, 3)}
    if wbytes:
        line["weight_bytes"] = int(wbytes)
        line["weight_gbps"] = round(wbytes / (ms * 1e-3) / 1e9, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
