"""Benchmark: weight-stream GB/s of the batch-1 quantized SwiGLU FFN on one MI355X.

Workload (one step): the 27B-class dense FFN, Q4_0, d_model 5120, ffn 17408,
one token, one swiglu_ffn call: h = silu(Wg x) * (Wu x) (the fused gate/up
GEMV kernel, which also clears out), then out = Wd h (the GEMV kernel over
the two column halves of Wd, each adding its half-row sums into out).
Synthetic seeded weights and activations (synth.CFG5), repacked once at load.
Enough packed copies of the three matrices rotate through the steps that the
working set is >= 1 GiB (over 4x the 256 MB Infinity Cache), so each step
streams its weights from HBM.

value = algorithmic weight bytes per step (150,405,120 B: 18 B per 32 weights)
        / time per step: the K steps (one swiglu_ffn call each, over the
        rotating copies) captured once in a HIP graph and uploaded; the W
        warm-up steps; then the graph launched once between two device
        synchronizations, timed by HIP events recorded on the stream right
        before and after the launch (the K steps' device time; the wall
        clock across the launch and the closing synchronization, which adds
        the launch latency, is detail.value_wall_clock).  It follows the per-kernel passes below, so the
        device runs the step in its steady state (its first milliseconds of
        work after an idle spell run slower); the read ceiling is measured
        after it.  The same K steps launched one call at a time through the C
        ABI, just before, are reported beside it (detail.value_eager_launches).
roofline: the dominant kernel (fused gate/up, 100,270,080 B per launch) timed
with HIP events on the stream it runs on, against 8 TB/s HBM: the K steps
run with each launch carrying its own start/stop events (two pairs queued
with qgemv_time_next_launch before each swiglu_ffn call: the library
launches both kernels with hipExtLaunchKernel), so the events hold each
dispatch's own start and end -- the durations rocprofv3's kernel trace
reports.  Timed launches leave gaps between the kernels (as hipEventRecord
pairs do), hence a pass of their own.
Also reported: back to back (HIP graphs of 32 launches over the rotating
copies) the gate/up product alone (swiglu_gate_up, the same kernel) and the
whole block (swiglu_ffn), whose difference is the down product's share as the
step runs it; and the read ceiling -- what a plain
16-byte grid-stride read kernel (qgemv_read_probe) streams over 1 GiB and,
back to back, over rotating slices of each product's size -- with each
kernel's fraction of it.
cpu_baseline: the CPU oracle (scalar C, binary64) on the same workload.

Per-case records (a separate mode, not part of the default run): --records
FILE writes one JSON line per case -- every matrix of every configuration at
one token, the 27B-class matrices at 8 and 128 tokens and the others at 128
-- with the product's graph-replay time and rate, its fraction of HBM peak
and of a plain read of the same size, the cache-resident rate, the largest
error in units of the bound and bit-exact dequantization on 64 sampled rows
against the oracle, and the oracle's time on one and on all host threads
(scaled from a block of rows).  The counter fields (HBM bytes fetched, VALU
and LDS instructions, matrix-core utilisation) come from rocprofv3 --pmc runs
of --counter-pass (each case's product once, 3 ms apart), given with
--records-counters DIR,...

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--warm", action="store_true", help="also report a cache-resident (single copy) rate")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload report")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with a plain 256 MiB device copy (known bytes, for scaling HBM counters)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the read-ceiling probe and the back-to-back graph passes (short profiled runs)")
    ap.add_argument("--records", default="",
                    help="write one JSON line per case (every matrix of every config, one token and batched) "
                         "to this file, then exit")
    ap.add_argument("--records-counters", default="",
                    help="with --records: comma-separated rocprofv3 output directories of --counter-pass runs "
                         "whose counters fill the records' counter fields")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run each case's product once, 3 ms apart, then a 256 MiB copy (for rocprofv3 --pmc), "
                         "then exit")
    ap.add_argument("--workloads", default="",
                    help="comma-separated keys of the per-workload report to run (e.g. cfg5_n8,cfg5_n128; "
                         "'extras': the FFN block, Q8_0-activation and head-plus-sampling steps); default: all")
    return ap.parse_args()


class TimingEvents:
    """HIP events for kernel timing, handed to the library's launch hook (the
    dispatch records them).  Uses the HIP runtime torch already loaded (same
    soname)."""

    def __init__(self, n):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreateWithFlags(ctypes.byref(e), 0) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i, stream_ptr):
        if self.lib.hipEventRecord(self.ev[i], ctypes.c_void_p(stream_ptr)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i, j):
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for e in self.ev:
            self.lib.hipEventDestroy(e)
        self.ev = []


GEMV_SOURCES = ("dequant_matrix_vector_amd/csrc/gemv_impl.h", "dequant_matrix_vector_amd/csrc/gemv_xs.h",
                "dequant_matrix_vector_amd/csrc/gemv_xs.hip", "dequant_matrix_vector_amd/csrc/gemv.hip")
TRAFFIC_PROFILE = "profiles/gemv_q4_0_27b_ffn_hbm_counters.md"


def measured_traffic():
    """HBM bytes per launch of the fused gate/up kernel from the committed
    rocprofv3 counter summary, or None if the kernel sources changed since the
    counters were taken."""
    import hashlib
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("gemv_source_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return int(fields["traffic_gate_up_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def read_ceiling(qg, torch, dev, launch_bytes=(100270080, 50135040)):
    """Streaming-read rate of a plain kernel (qgemv_read_probe: 16-byte loads,
    grid-stride), best over a few launch shapes: over 1 GiB in one launch, and
    back to back over rotating slices of each product's size (a launch of the
    products' length pays the same ramp-up and drain)."""
    pool = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    pool.random_(0, 255)
    out = torch.zeros(256 * 64, dtype=torch.int32, device=dev)
    sptr = torch.cuda.current_stream().cuda_stream
    probe = qg.lib.qgemv_read_probe
    res = {}

    def run(nbytes, nslice, wpc, u, iters):
        def launch(i):
            if probe(pool.data_ptr() + (i % nslice) * nbytes, nbytes, wpc, u, out.data_ptr(), sptr) != 0:
                raise RuntimeError("qgemv_read_probe failed")
        for i in range(3):
            launch(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            launch(i)
        e1.record()
        torch.cuda.synchronize()
        return nbytes / (e0.elapsed_time(e1) * 1e-3 / iters) / 1e9

    shapes = [(4, 2), (4, 8), (16, 8), (8, 4)]
    res["GBs_1GiB"] = round(max(run(1 << 30, 1, w, u, 10) for w, u in shapes), 1)
    for nb in launch_bytes:
        nslice = (1 << 30) // nb
        res[f"GBs_{nb}_per_launch"] = round(max(run(nb, nslice, w, u, 60) for w, u in shapes), 1)
    del pool
    torch.cuda.empty_cache()
    return res


def upload_graph(graph, stream_ptr):
    """hipGraphUpload of a captured torch graph's executable on the stream, so
    that its first launch carries no upload; a no-op if the runtime or torch
    does not offer it."""
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        exe = int(graph.raw_cuda_graph_exec())
    except (OSError, AttributeError, RuntimeError, TypeError, ValueError):
        return False
    hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipGraphUpload.restype = ctypes.c_int
    return hip.hipGraphUpload(ctypes.c_void_p(exe), ctypes.c_void_p(stream_ptr)) == 0


def back_to_back_us(torch, launch, n=32, reps=5):
    """Device microseconds per launch of launch(i, stream) when n of them run
    back to back (a HIP graph of n launches over the rotating copies,
    replayed)."""
    s = torch.cuda.current_stream().cuda_stream
    for i in range(3):
        launch(i, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for i in range(n):
            launch(i, cs)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n)


def cpu_baseline(tens, x, w, min_seconds):
    """The oracle (scalar binary64 C) on the full FFN: one thread, then the rows
    of each product split over the host's cores (at most 16, the host share of
    one GPU) with the oracle itself unchanged (ctypes releases the GIL in the
    C calls; every row is summed in the same order, so the results agree)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    wb = sum(t.weight_bytes for t in tens)
    half = min_seconds / 2

    reps, t0 = 0, time.perf_counter()
    while True:
        r1 = oracle.swiglu("q4_0", tens[0].raw, tens[1].raw, tens[2].raw, x, w.d_model, w.ffn)
        reps += 1
        el1 = time.perf_counter() - t0
        if el1 >= half:
            break
    per1 = el1 / reps

    threads = max(1, min(16, os.cpu_count() or 1))

    def product(pool, t, xin, rows, cols):
        cuts = np.linspace(0, rows, threads + 1).astype(int)
        parts = pool.map(lambda ab: oracle.gemv("q4_0", t.raw, xin, rows, cols, row_begin=int(ab[0]),
                                                row_end=int(ab[1]))[0], zip(cuts[:-1], cuts[1:]))
        return np.concatenate(list(parts), axis=-1)

    def ffn(pool):
        g = product(pool, tens[0], x, w.ffn, w.d_model)
        u = product(pool, tens[1], x, w.ffn, w.d_model)
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        return product(pool, tens[2], h, w.d_model, w.ffn)

    with ThreadPoolExecutor(threads) as pool:
        out = ffn(pool)
        assert np.allclose(out, r1["out"], rtol=1e-4, atol=1e-6)   # the binary32 h differs in the last bits
        repm, t0 = 0, time.perf_counter()
        while True:
            ffn(pool)
            repm += 1
            elm = time.perf_counter() - t0
            if elm >= half:
                break
    perm = elm / repm
    return {"value": round(wb / perm / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "value_1_thread": round(wb / per1 / 1e9, 4), "cpu_model": cpu_model(),
            "sample": f"full FFN (gate, up, down): {repm} runs with the rows of each product split over "
                      f"{threads} threads ({perm * 1e3:.1f} ms per FFN) and {reps} runs on 1 thread "
                      f"({per1 * 1e3:.0f} ms per FFN), binary64 scalar C"}


def workload_report(qg, synth, torch, np, dev, graph_iters=20, only=()):
    """Device time per step of every workload, from HIP graph replays.

    A step is the workload's whole hot path: the FFN (gate/up + down) for the
    FFN workloads, every listed GEMV for the layer workloads (their gate/up
    pair through the fused gate/up kernel).  Packed copies rotate across the
    graph's steps; when the copies reach 1 GiB the weights stream from HBM
    ("hbm"), otherwise they may sit in the 256 MB Infinity Cache ("cache")."""
    rep = {}
    plans = [(synth.CFG1, 1), (synth.CFG2, 1), (synth.CFG3, 1), (synth.CFG4, 1),
             (synth.CFG5, 8), (synth.CFG5, 128), (synth.CFG6, 1), (synth.CFG3, 128), (synth.CFG6, 128),
             (synth.CFG2, 128), (synth.CFG4, 128)]
    for w, n_tok in plans:
        key = f"cfg{w.cfg_id}" + (f"_n{n_tok}" if (w.n_tok != (1,) or n_tok != 1) else "")
        if only and key not in only:
            continue
        tens = synth.gen_workload(w)
        wbytes = sum(t.weight_bytes for t in tens)
        ncopy = int(min(graph_iters, max(1, -(-ROTATE_BYTES // wbytes))))
        raws = [(torch.from_numpy(t.raw).to(dev),
                 None if t.row_scale is None else torch.from_numpy(t.row_scale).to(dev)) for t in tens]
        copies = [[qg.repack(t.fmt, r, t.rows, t.cols, row_scale=rs) for (r, rs), t in zip(raws, tens)]
                  for _ in range(ncopy)]
        del raws
        names = [t.name for t in tens]
        xs = {c: torch.randn((n_tok, c), device=dev) for c in {t.cols for t in tens}}
        outs = {t.name: torch.empty((n_tok, t.rows), device=dev) for t in tens}
        ffn_names = ("gate", "up", "down")
        is_ffn = all(n in names for n in ffn_names)
        gi, ui, di = (names.index(n) for n in ffn_names) if is_ffn else (None, None, None)
        # the FFN through swiglu_ffn, with the scratch that lets the matrix-core
        # path split K (h is the scratch's first n_tok*ffn floats)
        scratch = (torch.empty(qg.swiglu_ffn_scratch_elems(tens[gi].fmt, w.d_model, w.ffn, n_tok), device=dev)
                   if is_ffn else None)

        def step(i):
            pk = copies[i % ncopy]
            if is_ffn:
                # stream=None: the binding takes torch's current stream, which is the
                # capture stream inside the graph
                qg.swiglu_ffn(tens[gi].fmt, pk[gi], pk[ui], pk[di], xs[w.d_model], w.d_model, w.ffn,
                              out=outs["down"], h_scratch=scratch)
            for j, t in enumerate(tens):
                if is_ffn and t.name in ffn_names:   # already run by swiglu_ffn
                    continue
                qg.qgemv(t.fmt, pk[j], xs[t.cols], t.rows, t.cols, y=outs[t.name])

        for i in range(3):
            step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(graph_iters):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * graph_iters)
        rep[key] = {"workload": w.name, "n_tok": n_tok, "us_per_step": round(us, 2),
                    "weight_bytes": wbytes, "GBs": round(wbytes / us / 1e3, 1),
                    "pct_hbm_peak": round(100 * wbytes / us / 1e3 / HBM_PEAK_GBS, 1),
                    "resident": "hbm" if ncopy * wbytes >= ROTATE_BYTES else "cache",
                    "path": "matrix cores (bf16 MFMA)" if n_tok > 1 else "GEMV"}
        if n_tok > 1:
            flops = 2 * n_tok * sum(t.rows * t.cols for t in tens)
            rep[key]["TFLOPs"] = round(flops / us / 1e6, 2)
            rep[key]["pct_bf16_mfma_peak"] = round(100 * flops / us / 1e6 / BF16_MFMA_PEAK_TFLOPS, 1)
        del copies, g
        torch.cuda.empty_cache()
    if not only or "extras" in only:
        rep.update(extra_report(qg, synth, torch, np, dev, graph_iters))
    return rep


def _graph_us(torch, step, graph_iters):
    """Device microseconds per step of `step(i)` replayed from a HIP graph."""
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(graph_iters):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (5 * graph_iters)


def extra_report(qg, synth, torch, np, dev, graph_iters=20):
    """The steps around the FFN and the head: the 27B-class FFN block with
    RMSNorm in and the residual add out (against the bare FFN), and the vocab
    heads followed by greedy sampling on the device."""
    rep = {}
    w = synth.CFG5
    tens = synth.gen_workload(w)
    wbytes = sum(t.weight_bytes for t in tens)
    ncopy = int(min(graph_iters, max(1, -(-ROTATE_BYTES // wbytes))))
    raws = [torch.from_numpy(t.raw).to(dev) for t in tens]
    copies = [[qg.repack("q4_0", r, t.rows, t.cols) for r, t in zip(raws, tens)] for _ in range(ncopy)]
    del raws
    gamma = torch.rand(w.d_model, device=dev) + 0.5
    for n_tok in (1, 8):
        x = torch.randn((n_tok, w.d_model), device=dev)
        out = torch.empty_like(x)
        sb = torch.empty(qg.swiglu_ffn_block_scratch_elems("q4_0", w.d_model, w.ffn, n_tok), device=dev)
        sf = torch.empty(qg.swiglu_ffn_scratch_elems("q4_0", w.d_model, w.ffn, n_tok), device=dev)

        def block(i):
            c = copies[i % ncopy]
            qg.swiglu_ffn_block("q4_0", c[0], c[1], c[2], gamma, 1e-5, x, w.d_model, w.ffn, out=out, h_scratch=sb)

        def bare(i):
            c = copies[i % ncopy]
            qg.swiglu_ffn("q4_0", c[0], c[1], c[2], x, w.d_model, w.ffn, out=out, h_scratch=sf)

        ub, uf = _graph_us(torch, block, graph_iters), _graph_us(torch, bare, graph_iters)
        rep[f"cfg5_block_n{n_tok}"] = {"workload": w.name + " + RMSNorm in, residual out", "n_tok": n_tok,
                                       "us_per_step": round(ub, 2), "ffn_alone_us_per_step": round(uf, 2),
                                       "GBs": round(wbytes / ub / 1e3, 1)}
        if n_tok == 1:
            hq = torch.empty(w.ffn, device=dev)

            def q8act(i):
                c = copies[i % ncopy]
                qg.swiglu_ffn_q8act("q4_0", c[0], c[1], c[2], x, w.d_model, w.ffn, out=out, h_scratch=hq)

            uq = _graph_us(torch, q8act, graph_iters)
            rep["cfg5_ffn_q8act"] = {"workload": w.name + ", x and h quantized to Q8_0 (integer dot products)",
                                     "n_tok": 1, "us_per_step": round(uq, 2), "ffn_f32_us_per_step": round(uf, 2),
                                     "GBs": round(wbytes / uq / 1e3, 1)}
    # several tokens with x and h quantized to Q8_0: the batched launches
    # (quantize, gate/up, reduce, quantize, down, reduce)
    for n_tok in (8, 128):
        x = torch.randn((n_tok, w.d_model), device=dev)
        out = torch.empty_like(x)
        hq = torch.empty(qg.swiglu_ffn_q8act_scratch_elems("q4_0", w.d_model, w.ffn, n_tok), device=dev)

        def q8b(i):
            c = copies[i % ncopy]
            qg.swiglu_ffn_q8act("q4_0", c[0], c[1], c[2], x, w.d_model, w.ffn, out=out, h_scratch=hq)

        uq = _graph_us(torch, q8b, graph_iters)
        rep[f"cfg5_ffn_q8act_n{n_tok}"] = {
            "workload": w.name + f", x and h quantized to Q8_0, {n_tok} tokens (matrix cores, exact block sums)",
            "n_tok": n_tok, "us_per_step": round(uq, 2), "GBs": round(wbytes / uq / 1e3, 1),
            "TOPs": round(2 * n_tok * (wbytes * 32 // 18) / uq / 1e6, 1)}
    del copies
    torch.cuda.empty_cache()
    for w, idx in ((synth.CFG2, 7), (synth.CFG4, 3)):
        t = synth.gen_tensor(w, idx)
        raw = torch.from_numpy(t.raw).to(dev)
        rs = None if t.row_scale is None else torch.from_numpy(t.row_scale).to(dev)
        ncopy = int(min(graph_iters, max(1, -(-ROTATE_BYTES // t.weight_bytes))))
        hc = [qg.repack(t.fmt, raw, t.rows, t.cols, row_scale=rs) for _ in range(ncopy)]
        del raw
        x = torch.randn((1, t.cols), device=dev)
        logits = torch.empty((1, t.rows), device=dev)
        tok = torch.empty(1, dtype=torch.int32, device=dev)
        ws = torch.zeros(qg.head_argmax_workspace_bytes(t.fmt, t.rows, t.cols), dtype=torch.uint8, device=dev)

        def head(i):   # the argmax fused into the product (candidates), then the combine launch
            qg.qgemv_head_argmax(t.fmt, hc[i % ncopy], x, t.rows, t.cols, logits=logits, token=tok, workspace=ws,
                                 fused=True)

        def head_two(i):   # the product, then the argmax launch
            qg.qgemv_head_argmax(t.fmt, hc[i % ncopy], x, t.rows, t.cols, logits=logits, token=tok, fused=False)

        def head_only(i):
            qg.qgemv(t.fmt, hc[i % ncopy], x, t.rows, t.cols, y=logits)

        uh, u2 = _graph_us(torch, head, graph_iters), _graph_us(torch, head_two, graph_iters)
        uo = _graph_us(torch, head_only, graph_iters)
        rep[f"cfg{w.cfg_id}_head_argmax"] = {"workload": f"{w.name}: {t.fmt} head [{t.rows}][{t.cols}] + argmax",
                                            "us_per_step": round(min(uh, u2), 2), "fused_us_per_step": round(uh, 2),
                                            "two_launches_us_per_step": round(u2, 2),
                                            "head_alone_us_per_step": round(uo, 2),
                                            "GBs": round(t.weight_bytes / min(uh, u2) / 1e3, 1)}
        del hc
        torch.cuda.empty_cache()
    return rep


# ----------------------------------------------------------- per-case records --
# One JSON line per case (cfg, matrix, n_tok): device time and rate of the
# product alone, against HBM peak, a plain read of the same size and the
# cache-resident rate; the largest error against the oracle in units of the
# bound and whether the device dequantizes bit-exactly, both on sampled rows;
# the oracle's time; and, from rocprofv3 counter runs of --counter-pass, the
# HBM bytes fetched, VALU and LDS instructions and matrix-core utilisation.

RECORD_SEED = 0
RECORD_SAMPLE_ROWS = 64
COUNTER_GAP_S = 0.003


def record_cases(synth):
    """(workload, matrix index, n_tok) of every case, in a fixed order."""
    ws = (synth.CFG1, synth.CFG2, synth.CFG3, synth.CFG4, synth.CFG5, synth.CFG6)
    cases = [(w, i, 1) for w in ws for i in range(len(w.tensors))]
    cases += [(synth.CFG5, i, n) for n in (8, 128) for i in range(len(synth.CFG5.tensors))]
    cases += [(w, i, 128) for w in (synth.CFG2, synth.CFG3, synth.CFG4, synth.CFG6) for i in range(len(w.tensors))]
    return cases


def _case_inputs(qg, synth, torch, dev, w, i, n_tok, ncopy):
    t = synth.gen_tensor(w, i, seed=RECORD_SEED)
    raw = torch.from_numpy(t.raw).to(dev)
    rs = None if t.row_scale is None else torch.from_numpy(t.row_scale).to(dev)
    copies = [qg.repack(t.fmt, raw, t.rows, t.cols, row_scale=rs) for _ in range(ncopy)]
    x = synth.gen_x(w, t.cols, n_tok, seed=RECORD_SEED, which=100 + i)
    return t, copies, x


def counter_pass(qg, synth, torch, np, dev):
    """Each case's product once, after an idle gap, in record_cases order
    (every input prepared first), then a 256 MiB copy whose bytes scale the
    HBM counters."""
    prepared = []
    for w, i, n_tok in record_cases(synth):
        t, copies, x = _case_inputs(qg, synth, torch, dev, w, i, n_tok, 1)
        xd = torch.from_numpy(x).to(dev)
        y = torch.empty((n_tok, t.rows), device=dev)
        prepared.append((t, copies[0], xd, y))
    torch.cuda.synchronize()
    for t, pk, xd, y in prepared:
        time.sleep(COUNTER_GAP_S)
        qg.qgemv(t.fmt, pk, xd, t.rows, t.cols, y=y)
        torch.cuda.synchronize()
    time.sleep(COUNTER_GAP_S)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def counters_by_case(dirs, ncases):
    """{counter: [per-case sums]} from rocprofv3 counter CSVs of --counter-pass
    runs: the library's product dispatches grouped by the idle gaps between
    cases; FETCH_SIZE scaled to bytes by the closing 256 MiB copy."""
    import csv
    out = {}
    for d in dirs:
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        disp = {}
        for r in rows:
            key = int(r["Dispatch_Id"])
            e = disp.setdefault(key, {"name": r["Kernel_Name"], "t0": int(r["Start_Timestamp"]), "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        seq = sorted(disp.values(), key=lambda e: e["t0"])
        copy = [e for e in seq if "copyBuffer" in e["name"]]
        prod = [e for e in seq if "qg::" in e["name"] and "repack" not in e["name"] and "dequant" not in e["name"]]
        groups, last = [], None
        for e in prod:
            if last is None or e["t0"] - last > COUNTER_GAP_S * 1e9 / 3:
                groups.append({})
            for k, v in e["c"].items():
                groups[-1][k] = groups[-1].get(k, 0.0) + v
            last = e["t0"]
        if len(groups) != ncases:
            raise RuntimeError(f"{d}: {len(groups)} dispatch groups for {ncases} cases")
        for k in groups[0]:
            vals = [g.get(k, 0.0) for g in groups]
            if k == "FETCH_SIZE":
                if not copy:
                    raise RuntimeError(f"{d}: no calibration copy")
                f = (256 << 10) / copy[-1]["c"]["FETCH_SIZE"]   # KiB read by the copy / KiB it reports
                vals = [v * 1024 * f for v in vals]
            out[k] = vals
    return out


def write_records(qg, synth, torch, np, dev, path, counter_dirs=()):
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    cases = record_cases(synth)
    cnt = counters_by_case(counter_dirs, len(cases)) if counter_dirs else {}
    pool = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    pool.random_(0, 255)
    pout = torch.zeros(256 * 64, dtype=torch.int32, device=dev)
    threads = max(1, min(16, os.cpu_count() or 1))
    cpu = cpu_model()
    ex = ThreadPoolExecutor(threads)   # one pool for every case (its start-up is not the oracle's time)
    list(ex.map(lambda k: k, range(threads)))

    def ceiling(nb):
        # a plain read of nb bytes per launch, back to back over rotating slices
        nb = max(16, nb // 16 * 16)
        nslice = max(1, (1 << 30) // nb)
        best = 0.0
        for wpc, u in ((16, 8), (8, 4), (4, 2)):
            def launch(k):
                cs = torch.cuda.current_stream().cuda_stream   # the capture stream inside the graph
                if qg.lib.qgemv_read_probe(pool.data_ptr() + (k % nslice) * nb, nb, wpc, u, pout.data_ptr(), cs):
                    raise RuntimeError("qgemv_read_probe failed")
            best = max(best, nb / _graph_us(torch, lambda k: launch(k), 20) / 1e3)
        return best

    with open(path, "w") as f:
        for ci, (w, i, n_tok) in enumerate(cases):
            wb = synth.algorithmic_bytes(*w.tensors[i][1:])
            ncopy = int(min(20, max(1, -(-ROTATE_BYTES // wb))))
            t, copies, x = _case_inputs(qg, synth, torch, dev, w, i, n_tok, ncopy)
            xd = torch.from_numpy(x).to(dev)
            y = torch.empty((n_tok, t.rows), device=dev)
            us = _graph_us(torch, lambda k: qg.qgemv(t.fmt, copies[k % ncopy], xd, t.rows, t.cols, y=y), 20)
            warm_us = _graph_us(torch, lambda k: qg.qgemv(t.fmt, copies[0], xd, t.rows, t.cols, y=y), 20)
            qg.qgemv(t.fmt, copies[0], xd, t.rows, t.cols, y=y)
            wd = qg.qdequant(t.fmt, copies[0], t.rows, t.cols)
            torch.cuda.synchronize()
            # sampled rows: evenly spaced, the last row included
            sel = np.unique(np.linspace(0, t.rows - 1, min(t.rows, RECORD_SAMPLE_ROWS)).astype(np.int64))
            ygpu = y.cpu().numpy()[:, sel].astype(np.float64)
            wgpu = wd[torch.from_numpy(sel).to(dev)].cpu().numpy()
            del wd
            rsel = None if t.row_scale is None else t.row_scale[sel]
            wref = oracle.dequant(t.fmt, np.ascontiguousarray(t.raw[sel]), len(sel), t.cols, rsel)
            bitexact = bool(np.array_equal(wgpu.view(np.uint32), wref.view(np.uint32)))
            yref, S = oracle.gemv(t.fmt, np.ascontiguousarray(t.raw[sel]), x, len(sel), t.cols, rsel)
            rel = 2e-5 if n_tok == 1 else 8e-3
            err = float(np.max(np.abs(ygpu - yref) / (rel * S + 1e-7)))
            # the oracle's time: a block of rows on one thread, then blocks on
            # every thread at once, scaled to all rows
            blk = min(t.rows, max(1, int(2e7 // (t.cols * n_tok))))
            t0 = time.perf_counter()
            oracle.gemv(t.fmt, t.raw, x, t.rows, t.cols, t.row_scale, 0, blk)
            one = (time.perf_counter() - t0) * t.rows / blk
            nb_mt = min(t.rows, blk * threads)
            cuts = np.linspace(0, nb_mt, threads + 1).astype(int)
            t0 = time.perf_counter()
            list(ex.map(lambda ab: oracle.gemv(t.fmt, t.raw, x, t.rows, t.cols, t.row_scale, int(ab[0]),
                                               int(ab[1])), zip(cuts[:-1], cuts[1:])))
            mt = (time.perf_counter() - t0) * t.rows / nb_mt
            gbps = wb / us / 1e3
            ceil = ceiling(wb)
            rec = {"cfg": w.name, "matrix": t.name, "fmt": t.fmt, "rows": t.rows, "cols": t.cols, "n_tok": n_tok,
                   "weight_bytes": wb, "kernel_us": round(us, 2), "gbps": round(gbps, 1),
                   "pct_peak": round(100 * gbps / HBM_PEAK_GBS, 2),
                   "pct_measured_ceiling": round(100 * gbps / ceil, 2), "measured_ceiling_gbps": round(ceil, 1),
                   "resident": "hbm" if ncopy * wb >= ROTATE_BYTES else "cache",
                   "path": "GEMV" if n_tok == 1 else "matrix cores",
                   "fetch_bytes": round(cnt["FETCH_SIZE"][ci]) if "FETCH_SIZE" in cnt else None,
                   "valu_insts": round(cnt["SQ_INSTS_VALU"][ci]) if "SQ_INSTS_VALU" in cnt else None,
                   "lds_insts": round(cnt["SQ_INSTS_LDS"][ci]) if "SQ_INSTS_LDS" in cnt else None,
                   "mfma_util": (round(cnt["SQ_VALU_MFMA_BUSY_CYCLES"][ci] /
                                       (cnt["GRBM_GUI_ACTIVE"][ci] / 8 * 1024), 4)
                                 if "SQ_VALU_MFMA_BUSY_CYCLES" in cnt and cnt["GRBM_GUI_ACTIVE"][ci] > 0 else None),
                   "warm_gbps": round(wb / warm_us / 1e3, 1),
                   "oracle_us_1t": round(one * 1e6, 1), "oracle_us_mt": round(mt * 1e6, 1),
                   "host_cores": threads, "cpu_model": cpu, "max_err_ratio": round(err, 4),
                   "dequant_bitexact": bitexact, "sample_rows": int(len(sel)), "seed": RECORD_SEED}
            f.write(json.dumps(rec) + "\n")
            f.flush()
            print(f"record {ci + 1}/{len(cases)}: {w.name} {t.name} n_tok={n_tok} {us:.2f} us "
                  f"err {err:.3g} bitexact {bitexact}", file=sys.stderr, flush=True)
            del copies
            torch.cuda.empty_cache()
    ex.shutdown()


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported "
              "(the path shards by rows across GPUs; the benchmark runs and reports one GPU)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import dequant_matrix_vector_amd as qg
    import synth

    dev = torch.device("cuda:0")
    if a.counter_pass:
        counter_pass(qg, synth, torch, np, dev)
        return
    if a.records:
        write_records(qg, synth, torch, np, dev, a.records,
                      tuple(d for d in a.records_counters.split(",") if d))
        return
    w = synth.CFG5
    d_model, ffn = w.d_model, w.ffn
    tens = synth.gen_workload(w)
    x = synth.gen_x(w, d_model, 1)
    step_bytes = sum(t.weight_bytes for t in tens)
    gu_bytes = tens[0].weight_bytes + tens[1].weight_bytes
    ncopy = max(1, -(-ROTATE_BYTES // step_bytes))

    raws = [torch.from_numpy(t.raw).to(dev) for t in tens]
    copies = []
    for _ in range(ncopy):
        copies.append([qg.repack("q4_0", r, t.rows, t.cols) for r, t in zip(raws, tens)])
    del raws
    xd = torch.from_numpy(x).to(dev)
    h = torch.empty((1, ffn), dtype=torch.float32, device=dev)
    out = torch.empty((1, d_model), dtype=torch.float32, device=dev)
    scratch_elems = qg.swiglu_ffn_scratch_elems("q4_0", d_model, ffn, 1)
    hs = torch.empty(scratch_elems, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    # The timed loop calls the C ABI directly with its arguments marshalled
    # beforehand (the binding's per-call checks cost more host time than a
    # step's kernels take, which would leave the GPU idle between launches).
    fq = qg.FORMATS["q4_0"]
    gu_args = [(fq, g.data_ptr(), u.data_ptr(), xd.data_ptr(), h.data_ptr(), d_model, ffn, 1, sptr)
               for g, u, _ in copies]
    ffn_args = [(fq, g.data_ptr(), u.data_ptr(), dn.data_ptr(), xd.data_ptr(), out.data_ptr(), hs.data_ptr(),
                 scratch_elems, d_model, ffn, 1, sptr) for g, u, dn in copies]
    gate_up_call, ffn_call = qg.lib.swiglu_gate_up, qg.lib.swiglu_ffn
    evs = TimingEvents(4 * a.steps)
    time_next, ev_handles = qg.lib.qgemv_time_next_launch, evs.ev

    def step(i, timed=False):
        # timed: the call's gate/up launch takes the first pair, its down
        # launch the second
        if timed and (time_next(ev_handles[4 * i], ev_handles[4 * i + 1]) != 0 or
                      time_next(ev_handles[4 * i + 2], ev_handles[4 * i + 3]) != 0):
            raise RuntimeError("qgemv_time_next_launch failed")
        if ffn_call(*ffn_args[i % ncopy]) != 0:
            raise RuntimeError("swiglu_ffn failed")

    # Order of the passes: the K steps are captured in one HIP graph first
    # (capturing leaves the device idle for milliseconds); then the per-kernel
    # passes; then the K steps launched one call at a time; then the W warm-up
    # steps and, right after them, the timed launch of the graph (value), so
    # that the device is in the steady state the step runs in (after an idle
    # spell its first milliseconds of work run slower).  The read ceiling
    # comes after: its tens of milliseconds of full-rate reads leave the next
    # few milliseconds of kernels 3-5% slower.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream().cuda_stream
        for i in range(a.steps):
            if ffn_call(*ffn_args[i % ncopy][:-1], cs) != 0:
                raise RuntimeError("swiglu_ffn failed")
    uploaded = upload_graph(graph, sptr)

    # roofline: the K steps with each launch carrying its own events (the
    # timed launch path leaves the GPU idle between kernels, so this pass
    # gives kernel durations, not the step rate)
    for i in range(a.steps):
        step(i, True)
    torch.cuda.synchronize()
    gu_ms = [evs.ms(4 * i, 4 * i + 1) for i in range(a.steps)]
    dn_ms = [evs.ms(4 * i + 2, 4 * i + 3) for i in range(a.steps)]
    evs.close()
    gu_avg = float(np.mean(gu_ms))
    dn_avg = float(np.mean(dn_ms))
    achieved = gu_bytes / (gu_avg * 1e-3) / 1e9

    # back to back (no events between them): HIP graphs of 32 gate/up
    # launches and of 32 blocks over the rotating copies; the down product's
    # share is their difference
    def gu_launch(i, s):
        a = gu_args[i % ncopy]
        if gate_up_call(*a[:-1], s) != 0:
            raise RuntimeError("swiglu_gate_up failed")

    def ffn_launch(i, s):
        a = ffn_args[i % ncopy]
        if ffn_call(*a[:-1], s) != 0:
            raise RuntimeError("swiglu_ffn failed")

    gu_b2b = dn_b2b = ffn_b2b = float("nan")
    ceil = None
    if not a.no_extras:
        gu_b2b = back_to_back_us(torch, gu_launch)
        ffn_b2b = back_to_back_us(torch, ffn_launch)
        dn_b2b = ffn_b2b - gu_b2b

    # the K steps as launches from the host, one call at a time (no events
    # between the kernels, which run back to back)
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    # value: the W warm-up steps, then the K steps' graph, between two device
    # synchronizations; timed by events on the stream right around the
    # graph's launch (the K steps' device time), and by the wall clock across
    # the launch and the closing synchronization (reported beside it)
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_graph = time.perf_counter() - t0
    wall = ev0.elapsed_time(ev1) * 1e-3
    del graph
    if not a.no_extras:
        ceil = read_ceiling(qg, torch, dev, (gu_bytes, tens[2].weight_bytes))
        torch.cuda.empty_cache()
    ms_per_step = wall * 1e3 / a.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    value_eager = step_bytes / (wall_eager / a.steps) / 1e9
    value_wall = step_bytes / (wall_graph / a.steps) / 1e9

    detail = {
        "gate_up_us": round(gu_avg * 1e3, 2), "down_us": round(dn_avg * 1e3, 2),
        "gate_up_us_back_to_back": round(gu_b2b, 2), "down_us_back_to_back": round(dn_b2b, 2),
        "ffn_us_back_to_back": round(ffn_b2b, 2),
        "gate_up_GBs_back_to_back": round(gu_bytes / gu_b2b / 1e3, 1),
        "down_GBs_back_to_back": round(tens[2].weight_bytes / dn_b2b / 1e3, 1),
        "gate_up_GBs": round(achieved, 1),
        "down_GBs": round(tens[2].weight_bytes / (dn_avg * 1e-3) / 1e9, 1),
        "ffn_device_us": round((gu_avg + dn_avg) * 1e3, 2),
        "ffn_device_GBs": round(step_bytes / ((gu_avg + dn_avg) * 1e-3) / 1e9, 1),
        "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
        "value_wall_clock": round(value_wall, 1),
        "ms_per_step_wall_clock": round(wall_graph * 1e3 / a.steps, 5),
        "value_eager_launches": round(value_eager, 1),
        "value_graph_uploaded": bool(uploaded),
        "ms_per_step_eager_launches": round(wall_eager * 1e3 / a.steps, 5),
        "rotating_copies": ncopy,
    }
    if a.no_extras:
        for k in ("gate_up_us_back_to_back", "down_us_back_to_back", "gate_up_GBs_back_to_back",
                  "down_GBs_back_to_back", "ffn_us_back_to_back"):
            detail[k] = None
    if a.warm:
        g, u, dn = copies[0]
        for _ in range(10):
            qg.swiglu_gate_up("q4_0", g, u, xd, d_model, ffn, h=h, stream=sptr)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(100):
            qg.swiglu_gate_up("q4_0", g, u, xd, d_model, ffn, h=h, stream=sptr)
        e1.record(stream)
        torch.cuda.synchronize()
        detail["gate_up_warm_GBs_cache_resident"] = round(gu_bytes / (e0.elapsed_time(e1) / 100 * 1e-3) / 1e9, 1)

    # the roofline rate: the gate/up kernel back to back (a HIP graph of 32
    # launches timed with events on its stream), as the step runs it; the
    # pass with events on every launch (idle between kernels) is reported
    # beside it
    achieved_isolated = achieved
    if math.isfinite(gu_b2b):
        achieved = gu_bytes / gu_b2b / 1e3
    rec = {
        "metric": "weight-stream GB/s and % of HBM peak, batch-1 quant GEMV + SwiGLU FFN",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Q4_0 blocks: f16 d~U(0.005,0.05), codes U{0..15}; x~N(0,1))",
        "config": {"workload": "27B-class dense SwiGLU FFN, Q4_0, d_model 5120, ffn 17408, n_tok 1",
                   "format": "q4_0", "d_model": d_model, "ffn": ffn, "n_tok": 1,
                   "weight_bytes_per_step": step_bytes, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "fused gate/up row-streaming GEMV (gemv_xs_kernel<Q4_0, NMAT=2>)",
                     "bytes_per_launch": gu_bytes,
                     "timing": "back to back (HIP graph of 32 launches, events)" if math.isfinite(gu_b2b)
                     else "isolated launches (events on each)",
                     "achieved_isolated_launches": round(achieved_isolated, 1)},
        "detail": detail,
    }
    del copies
    torch.cuda.empty_cache()
    if ceil is not None:
        rec["read_ceiling"] = dict(ceil, unit="GB/s", kernel="qgemv_read_probe (plain 16-byte grid-stride read)")
        cg = ceil[f"GBs_{gu_bytes}_per_launch"]
        rec["roofline"]["read_ceiling_per_launch"] = cg
        rec["roofline"]["frac_of_read_ceiling"] = round(achieved / cg, 4)
        detail["gate_up_frac_of_read_ceiling_back_to_back"] = round(gu_bytes / gu_b2b / 1e3 / cg, 4)
        detail["down_frac_of_read_ceiling_back_to_back"] = round(
            tens[2].weight_bytes / dn_b2b / 1e3 / ceil[f"GBs_{tens[2].weight_bytes}_per_launch"], 4)
        detail["step_frac_of_read_ceiling"] = round(value / ceil["GBs_1GiB"], 4)
    if a.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not a.no_workloads:
        rec["workloads"] = workload_report(qg, synth, torch, np, dev,
                                           only=tuple(k for k in a.workloads.split(",") if k))
    if not a.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(tens, x, w, a.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
