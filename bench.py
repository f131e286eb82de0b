"""Benchmark: weight-stream GB/s of the batch-1 quantized SwiGLU FFN on one MI355X.

Workload (one step): the 27B-class dense FFN, Q4_0, d_model 5120, ffn 17408,
one token: h = silu(Wg x) * (Wu x) (the fused gate/up GEMV kernel), then
out = Wd h (the GEMV kernel) -- exactly the two launches swiglu_ffn makes.
Synthetic seeded weights and activations (synth.CFG5), repacked once at load.
Enough packed copies of the three matrices rotate through the steps that the
working set is >= 1 GiB (over 4x the 256 MB Infinity Cache), so each step
streams its weights from HBM.

value = algorithmic weight bytes per step (150,405,120 B: 18 B per 32 weights)
        / wall time per step (K steps between two device synchronizations).
roofline: the dominant kernel (fused gate/up, 100,270,080 B per launch) timed
with HIP events on the stream it runs on, against 8 TB/s HBM.
cpu_baseline: the CPU oracle (scalar C, binary64) on the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--warm", action="store_true", help="also report a cache-resident (single copy) rate")
    return ap.parse_args()


def cpu_baseline(tens, x, w, min_seconds):
    import oracle
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.swiglu("q4_0", tens[0].raw, tens[1].raw, tens[2].raw, x, w.d_model, w.ffn)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per = el / reps
    wb = sum(t.weight_bytes for t in tens)
    return {"value": round(wb / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full FFN (gate, up, down) x {reps} runs, {el:.1f} s, {per * 1e3:.0f} ms per FFN, "
                      f"1 thread, binary64 scalar C"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported "
              "(the path shards by rows across GPUs, but this build runs and reports one GPU only)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import dequant_matrix_vector_amd as qg
    import synth

    dev = torch.device("cuda:0")
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
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(i, ev=None):
        g, u, dn = copies[i % ncopy]
        if ev is not None:
            ev[0].record(stream)
        qg.swiglu_gate_up("q4_0", g, u, xd, d_model, ffn, h=h, stream=sptr)
        if ev is not None:
            ev[1].record(stream)
        qg.qgemv("q4_0", dn, h, d_model, ffn, y=out, stream=sptr)
        if ev is not None:
            ev[2].record(stream)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gu_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = wall * 1e3 / a.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    gu_avg = float(np.mean(gu_ms))
    dn_avg = float(np.mean(dn_ms))
    achieved = gu_bytes / (gu_avg * 1e-3) / 1e9

    detail = {
        "gate_up_us": round(gu_avg * 1e3, 2), "down_us": round(dn_avg * 1e3, 2),
        "gate_up_GBs": round(achieved, 1),
        "down_GBs": round(tens[2].weight_bytes / (dn_avg * 1e-3) / 1e9, 1),
        "ffn_device_us": round((gu_avg + dn_avg) * 1e3, 2),
        "ffn_device_GBs": round(step_bytes / ((gu_avg + dn_avg) * 1e-3) / 1e9, 1),
        "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
        "rotating_copies": ncopy,
    }
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
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "fused gate/up GEMV (gemv_kernel<Q4_0, NMAT=2>)",
                     "bytes_per_launch": gu_bytes},
        "detail": detail,
    }
    if not a.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(tens, x, w, a.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
