"""Benchmark: fused decode-GEMV over one Llama-style 8B decoder layer at batch 1.

One step = one grouped lbf_gemv launch over the layer's seven coded weight
tensors (q, k, v, o, gate, up, down; 218,103,808 BF16 weights), batch 1, fp32
output.  Inputs are synthetic and seeded (decode_byte_split_amd.synth), coded
on the GPU and resident in HBM before timing.  Steps rotate over several
copies of the coded layer so the working set (> 1 GB) cannot sit in the
256 MB Infinity Cache.

Printed: one JSON line with the metric (BF16-equivalent weight GB/s), the
roofline of the GEMV kernel (algorithmic bytes per launch / mean launch time
from HIP events on the launch stream, against 8 TB/s HBM), the HBM traffic
read from the committed rocprofv3 counter summary (null if the kernel source
changed since), and the CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "fused decode-GEMV BF16-equiv weight GB/s + % HBM roofline, 8B-shaped layer"
COUNTERS = os.path.join(ROOT, "profiles", "gemv_layer_b1_counters.json")
KERNEL_SOURCES = ("decode_byte_split_amd/csrc/lbf_gemv.hip", "decode_byte_split_amd/csrc/lbf_device.h")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def algorithmic_bytes(blob, batch: int, y_bytes: int) -> int:
    """Bytes one fused product must move: the coded planes it reads (raw,
    nibbles, tile index, escapes), x, and y."""
    n = blob.rows * blob.cols
    n_tiles = (n + 1023) // 1024
    return n + (n + 1) // 2 + 4 * (n_tiles + 1) + blob.n_esc + 2 * batch * blob.cols + y_bytes * batch * blob.rows


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def time_launches(torch, fn, steps: int, warmup: int):
    """Run fn(i) warmup + steps times; returns (ms per step over the timed
    region, mean ms per launch from per-launch events)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        ev[i][0].record()
        fn(warmup + i)
        ev[i][1].record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    per = [a.elapsed_time(b) for a, b in ev]
    return total / steps, float(np.mean(per)), float(np.median(per))


def cpu_baseline(Ws, xs, min_seconds: float):
    """The oracle (plain scalar C, one thread) on this host: decode the
    layer's blobs and run the float64 matvec, repeated until min_seconds."""
    from oracle import oracle as O

    blobs = [O.encode(W) for W in Ws]  # untimed: the baseline is decode + product
    n = sum(W.size for W in Ws)
    passes = 0
    t = 0.0
    while passes == 0 or t < min_seconds:
        t0 = time.perf_counter()
        for blob, x in zip(blobs, xs):
            W = O.decode(blob)
            O.matvec(W, x)
        t += time.perf_counter() - t0
        passes += 1
    gbs = 2.0 * n * passes / t / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "full 8B-shaped layer (7 tensors, %d weights) x %d pass(es): oracle decode of each "
                      "oracle-coded blob + float64 matvec at batch 1, %.1f s" % (n, passes, t)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--extras", action="store_true", help="also time decode, the batch sweep and raw BF16")
    ap.add_argument("--rotate-gb", type=float, default=1.1)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused decode-GEMV has no cross-GPU step in this build "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_byte_split_amd import lbf, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lbf.lib()
    t0 = time.time()
    Ws = [synth.layer_tensor(m) for m in range(len(synth.LAYER))]
    xs = [synth.layer_x(m) for m in range(len(synth.LAYER))]
    log("layer generated in %.1f s" % (time.time() - t0))
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    torch.cuda.synchronize()
    n_weights = sum(W.size for W in Ws)
    layer_blob_bytes = sum(b.nbytes for b in blobs)
    copies = max(1, int(np.ceil(args.rotate_gb * 1e9 / layer_blob_bytes)))
    rot = [blobs] + [[lbf.Blob(b.desc, b.data.clone()) for b in blobs] for _ in range(copies - 1)]
    xd = [dev(torch, x) for x in xs]
    ys = [torch.empty((1, b.rows), dtype=torch.float32, device="cuda") for b in blobs]
    torch.cuda.synchronize()
    log("coded layer: %d bytes (%.4f bits/weight, %d escapes), %d rotation copies"
        % (layer_blob_bytes, 8.0 * layer_blob_bytes / n_weights, sum(b.n_esc for b in blobs), copies))

    step = lambda i: lbf.gemv(rot[i % copies], xd, lbf.LBF_F32, outs=ys)
    ms_step, ms_launch, ms_launch_med = time_launches(torch, step, args.steps, args.warmup)
    alg = sum(algorithmic_bytes(b, 1, 4) for b in blobs)
    achieved = alg / (ms_launch * 1e-3) / 1e9
    value = 2.0 * n_weights / (ms_step * 1e-3) / 1e9
    log("step %.2f us, launch mean %.2f us (median %.2f): %.1f GB/s BF16-equiv, %.1f GB/s algorithmic (%.1f %% of 8 TB/s)"
        % (ms_step * 1e3, ms_launch * 1e3, ms_launch_med * 1e3, value, achieved, 100 * achieved / HBM_PEAK_GBS))

    traffic = None
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            c = json.load(f)
        if c.get("kernel_hash") == kernel_hash():
            traffic = c.get("hbm_bytes_per_launch")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama8b_layer_fused_decode_gemv_b1", "tensors": [m[0] for m in synth.LAYER],
                   "weights": n_weights, "batch": 1, "y_dtype": "f32", "coded_bytes": layer_blob_bytes,
                   "bits_per_weight": round(8.0 * layer_blob_bytes / n_weights, 4), "rotation_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_gemv<1,8>", "algorithmic_bytes_per_launch": alg,
                     "launch_ms_mean": round(ms_launch, 5), "launch_ms_median": round(ms_launch_med, 5)},
    }

    if args.extras:
        out["extra"] = extras(torch, lbf, synth, Ws, blobs, rot, copies, args)

    if not args.no_cpu:
        log("timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(Ws, xs, args.cpu_seconds)
    print(json.dumps(out))


def extras(torch, lbf, synth, Ws, blobs, rot, copies, args):
    res = {}
    # standalone decode of the layer: reads the planes, writes 2 bytes per weight
    outs = [torch.empty((b.rows, b.cols), dtype=torch.bfloat16, device="cuda") for b in blobs]

    def dec(i):
        for b, o in zip(rot[i % copies], outs):
            lbf.decode(b, out=o)

    ms, _, _ = time_launches(torch, dec, 20, 3)
    n = sum(W.size for W in Ws)
    alg = sum(algorithmic_bytes(b, 0, 0) for b in blobs) + 2 * n
    res["decode_layer"] = {"us": round(ms * 1e3, 2), "bf16_equiv_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1),
                           "hbm_GBs": round(alg / (ms * 1e-3) / 1e9, 1)}
    # raw BF16 lane: torch F.linear over the same layer, uncompressed weights
    wd = [dev(torch, W) for W in Ws]
    xd = [dev(torch, synth.layer_x(m)) for m in range(len(Ws))]
    wrot = [wd] + [[w.clone() for w in wd] for _ in range(1)]

    def raw(i):
        for w, x in zip(wrot[i % 2], xd):
            torch.nn.functional.linear(x, w)

    ms, _, _ = time_launches(torch, raw, 20, 3)
    res["raw_bf16_linear_layer"] = {"us": round(ms * 1e3, 2), "GBs": round(2 * n / (ms * 1e-3) / 1e9, 1)}
    # gate_proj batch sweep
    g = synth.GATE
    sweep = {}
    for batch in (1, 2, 4, 8):
        x = dev(torch, synth.gate_batch_x(batch))
        y = torch.empty((batch, blobs[g].rows), dtype=torch.bfloat16, device="cuda")
        f = lambda i: lbf.gemv(rot[i % copies][g], x, lbf.LBF_BF16, outs=y)
        ms_s, ms_l, _ = time_launches(torch, f, 30, 5)
        alg = algorithmic_bytes(blobs[g], batch, 2)
        sweep[str(batch)] = {"us": round(ms_l * 1e3, 2), "bf16_equiv_GBs": round(2 * Ws[g].size / (ms_l * 1e-3) / 1e9, 1),
                             "hbm_frac": round(alg / (ms_l * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    res["gate_proj_sweep"] = sweep
    return res


if __name__ == "__main__":
    main()
