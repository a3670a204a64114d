"""Benchmark: fused decode-GEMV over one Llama-style 8B decoder layer at batch 1.

One step = one grouped lbf_gemv launch over the layer's seven coded weight
tensors (q, k, v, o, gate, up, down; 218,103,808 BF16 weights), batch 1, fp32
output.  Inputs are synthetic and seeded (decode_byte_split_amd.synth), coded
on the GPU and resident in HBM before timing.  Steps rotate over several
copies of the coded layer (4 GB) so the working set cannot sit in the
256 MB Infinity Cache and the timing averages over many placements in memory.

Printed: one JSON line with the metric (BF16-equivalent weight GB/s), the
roofline of the GEMV kernel (algorithmic bytes per launch / mean launch time
from HIP events on the launch stream, against 8 TB/s HBM; also the median of
10-launch batch means), the HBM traffic read from the committed rocprofv3
counter summary (null if the kernel source changed since), the other
workloads' own roofline fractions under "configs" (gate_proj alone at batch
1, 8, 16, 64 and the 64 experts at batch 4), and the CPU oracle timed on
this host as a baseline, on the headline layer and per workload, on one core
and on all cores.
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
COUNTERS = os.path.join(ROOT, "profiles", "gemv_ring_layer_b1_counters.json")
KERNEL = "lbf::k_gemv_ring<1, 16, false, 4, 3, false>"
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


def product_path(blob, batch: int) -> str:
    """Which kernel lbf_gemv / lbf_gemm run for one tensor: the fused GEMV up
    to batch 8, the MFMA GEMM above, and at batch 8 when escapes are at most
    1 % of the weights."""
    mfma = batch > 8 or (batch == 8 and 100 * blob.n_esc <= blob.rows * blob.cols)
    return "gemm_mfma_16x16x32_bf16" if mfma else "gemv"


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def warm_gpu(torch, fn, min_ms: float, start: int = 0) -> int:
    """Run fn back to back, in batches of 10 calls between HIP events, until
    the GPU has spent at least min_ms on them; returns the number of calls.
    The GPU needs tens of milliseconds of sustained load before its clocks
    settle: a launch timed after a short warm-up reads several per cent
    slow."""
    n, spent = 0, 0.0
    while spent < min_ms:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            fn(start + n)
            n += 1
        b.record()
        b.synchronize()
        spent += a.elapsed_time(b)
    return n


def time_torch_linear(torch, pairs_per_copy, steps: int = 30) -> float:
    """torch's F.linear on uncompressed BF16 weights, the comparison lane:
    the calls of rotation copy i % copies per step, back to back (ms per
    step).  Replaying the same calls from HIP graphs measured slower, not
    faster, so the host's dispatch is not what bounds them."""
    F = torch.nn.functional
    return time_region(torch, lambda i: [F.linear(x, w) for x, w in pairs_per_copy[i % len(pairs_per_copy)]], steps, 3)


def time_region(torch, fn, steps: int, warmup: int, warm_ms: float = 30.0) -> float:
    """Run fn(i) warmup times untimed (then on until the GPU has been busy
    warm_ms with them), then steps times back to back between two HIP events
    on the launch stream; returns ms per call.  One call is one kernel launch
    here, so this is the mean launch duration (the gaps between back-to-back
    launches are included, host marshalling is not: each call is a single
    prepared ctypes call)."""
    for i in range(warmup):
        fn(i)
    warmup += warm_gpu(torch, fn, warm_ms, warmup) if warm_ms > 0 else 0
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        fn(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_batches(torch, fn, batches: int, per_batch: int, warmup: int):
    """Back-to-back launches timed in batches: each batch is per_batch calls
    between two HIP events; returns the per-call mean of every batch (ms).
    Same quantity as time_region, so its median and min describe the spread
    of the back-to-back figure across the run."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
    ev[0].record()
    k = warmup
    for j in range(batches):
        for _ in range(per_batch):
            fn(k)
            k += 1
        ev[j + 1].record()
    torch.cuda.synchronize()
    return [ev[j].elapsed_time(ev[j + 1]) / per_batch for j in range(batches)]


def time_each(torch, fn, steps: int, warmup: int):
    """Per-launch durations (ms): each call between its own pair of HIP
    events on the launch stream (the event pair adds its own overhead to
    every launch); returns (median, min)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(warmup + i)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2], t[0]


READ_BYTES = 1 << 30  # the read-stream ceiling runs over 1 GiB


def read_ceiling(torch, reps: int = 10, nbytes: int = READ_BYTES) -> float:
    """GB/s of a plain read stream (liblbf_measure.so: 128-bit non-temporal
    loads, XOR-reduced, one stored word per workgroup) over nbytes (default 1 GiB: the practical ceiling for
    a kernel that only reads HBM).  Smaller reads rotate over enough buffers
    to keep the working set at 1 GiB or more, past the 256 MB cache."""
    import ctypes

    L = ctypes.CDLL(os.path.join(ROOT, "decode_byte_split_amd", "liblbf_measure.so"))
    L.lbfm_read_stream.restype = ctypes.c_int
    L.lbfm_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    nbytes = max(16, nbytes // 16 * 16)
    nbuf = -(-READ_BYTES // nbytes)
    bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda") for _ in range(nbuf)]
    blocks = torch.cuda.get_device_properties(0).multi_processor_count  # one workgroup per CU
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")  # one word per workgroup
    s = torch.cuda.current_stream().cuda_stream

    def run(i):
        rc = L.lbfm_read_stream(bufs[i % nbuf].data_ptr(), nbytes, out.data_ptr(), blocks, s)
        assert rc == 0, "read-stream kernel failed (%d)" % rc

    ms = time_region(torch, run, max(reps, 3 * nbuf), 3)
    del bufs, out
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


COPY_ELEMS = 1 << 28  # float32 elements of the calibration copy: 1 GiB read, 1 GiB written


def copy_calibration(torch, reps: int = 3):
    """A plain elementwise kernel with known traffic (out = -in over 1 GiB of
    float32) so a counter run can scale FETCH_SIZE / WRITE_SIZE to bytes."""
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_counters(fetch_csv: str, write_csv: str, kernel_key: str, alg_bytes: int):
    """Scale the mean FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the
    kernel whose name contains kernel_key by what the same counters read for
    the calibration copy (4 * COPY_ELEMS bytes each way)."""
    out = {"kernel_hash": kernel_hash(), "copy_bytes_each_way": 4 * COPY_ELEMS}
    for label, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == label]
        cal = [float(r["Counter_Value"]) for r in rows if "neg_kernel" in r["Kernel_Name"]]
        ker = [float(r["Counter_Value"]) for r in rows if kernel_key in r["Kernel_Name"]]
        if not cal or not ker:
            raise SystemExit("%s: no calibration (%d) or kernel (%d) dispatches" % (path, len(cal), len(ker)))
        factor = float(np.mean(cal)) * 1024.0 / (4 * COPY_ELEMS)
        out[label] = {"kernel_kib_mean": float(np.mean(ker)), "kernel_dispatches": len(ker),
                      "copy_kib_mean": float(np.mean(cal)), "copy_dispatches": len(cal),
                      "factor": factor, "bytes_per_launch": float(np.mean(ker)) * 1024.0 / factor}
    out["kernel"] = kernel_key
    out["hbm_bytes_per_launch"] = int(round(out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]))
    out["algorithmic_bytes_per_launch"] = alg_bytes
    out["traffic_over_algorithmic"] = out["hbm_bytes_per_launch"] / alg_bytes
    return out


def _oracle_worker_init():
    from oracle import oracle as O

    O.lib()  # load the oracle library before any job is timed


def _oracle_job(item):
    """One oracle job (in this process or a worker): ("dm", blob file, x
    file) decodes an oracle-coded blob and runs the float64 matvec of its
    batch; ("enc", weights file) encodes a tensor.  Returns the weights
    processed."""
    from oracle import oracle as O

    if item[0] == "enc":
        W = np.load(item[1], mmap_mode="r")
        O.encode(np.ascontiguousarray(W))
        return W.size
    _, blob_path, x_path = item
    W = O.decode(np.load(blob_path, mmap_mode="r"))
    O.matvec(W, np.load(x_path))
    return W.size


def _write_jobs(d, name, jobs, coded):
    """Arrays of a leg's jobs -> file-based job tuples (memory-mapped by the
    workers).  ("dm", W, x): W is coded by the oracle first (untimed; one blob
    file per distinct W, kept in `coded`); ("enc", W): W itself."""
    from oracle import oracle as O

    out = []
    for i, j in enumerate(jobs):
        if j[0] == "enc":
            wp = os.path.join(d, "%s_w%d.npy" % (name, i))
            np.save(wp, j[1])
            out.append(("enc", wp))
            continue
        key = id(j[1])
        if key not in coded:
            bp = os.path.join(d, "blob%d.npy" % len(coded))
            np.save(bp, O.encode(j[1]))
            coded[key] = (bp, j[1])  # keeps W alive so its id stays unique
        xp = os.path.join(d, "%s_x%d.npy" % (name, i))
        np.save(xp, j[2])
        out.append(("dm", coded[key][0], xp))
    return out


def _one_core(jobs, min_seconds):
    weights, t, passes = 0, 0.0, 0
    while passes == 0 or t < min_seconds:
        t0 = time.perf_counter()
        for j in jobs:
            weights += _oracle_job(j)
        t += time.perf_counter() - t0
        passes += 1
    return weights, t, passes


def _all_cores(pool, jobs, min_seconds, workers):
    def run(js):
        return sum(f.result(timeout=120.0) for f in [pool.submit(_oracle_job, j) for j in js])

    per_round = max(1, -(-workers // len(jobs)))  # at least one job per worker a round
    weights, t, rounds = 0, 0.0, 0
    while rounds == 0 or t < min_seconds:
        t0 = time.perf_counter()
        weights += run(jobs * per_round)
        t += time.perf_counter() - t0
        rounds += 1
    return weights, t


def cpu_baseline(Ws, xs, min_seconds: float, workers: int = 0, legs=None, leg_seconds: float = 1.0):
    """The oracle (plain scalar C, one thread) on this host.  Headline: decode
    the layer's oracle-coded blobs and run the float64 matvec at batch 1,
    repeated until min_seconds.  legs: more workloads, {name: (description,
    [("dm", W, x) | ("enc", W), ...])}, each timed for leg_seconds (at
    least one pass).  With workers > 1, every leg is also run in that many
    processes at once (jobs shared out, files memory-mapped): the host's
    all-cores figure.  BF16-equivalent GB/s = 2 bytes per weight processed."""
    import shutil
    import tempfile

    d = tempfile.mkdtemp(prefix="lbf_oracle_")
    try:
        coded = {}
        head = _write_jobs(d, "layer", [("dm", W, x) for W, x in zip(Ws, xs)], coded)
        legs = legs or {}
        leg_jobs = {name: (desc, _write_jobs(d, name, jobs, coded)) for name, (desc, jobs) in legs.items()}
        n = sum(W.size for W in Ws)
        w, t, passes = _one_core(head, min_seconds)
        out = {"value": 2.0 * w / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "full 8B-shaped layer (7 tensors, %d weights) x %d pass(es): oracle decode of each "
                         "oracle-coded blob + float64 matvec at batch 1, %.1f s" % (n, passes, t),
               "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
        configs = {}
        for name, (desc, jobs) in leg_jobs.items():
            w, t, passes = _one_core(jobs, leg_seconds)
            configs[name] = {"one_core_GBs": round(2.0 * w / t / 1e9, 4), "sample": "%s; %d pass(es), %.1f s on 1 core"
                             % (desc, passes, t)}
        if workers > 1:
            out["all_cores"] = _all_cores_legs(head, leg_jobs, configs, min_seconds, leg_seconds, workers)
        if configs:
            out["configs"] = configs
        return out
    finally:
        shutil.rmtree(d, ignore_errors=True)


def _all_cores_legs(head, leg_jobs, configs, min_seconds, leg_seconds, workers):
    """The same jobs in `workers` processes at once.  A worker that dies or a
    job slower than two minutes ends this part with an error entry, never the
    benchmark."""
    import concurrent.futures as cf
    import multiprocessing as mp

    try:
        # fresh interpreters (spawn): nothing of this process's GPU state
        with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"),
                                    initializer=_oracle_worker_init) as pool:
            list(pool.map(_oracle_job, [head[-1]] * workers))  # every worker up and warm
            w, t = _all_cores(pool, head, min_seconds, workers)
            res = {"value": 2.0 * w / t / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
                   "sample": "the same layer passes in %d processes at once: %d weights in %.1f s" % (workers, w, t)}
            for name, (_, jobs) in leg_jobs.items():
                w, t = _all_cores(pool, jobs, leg_seconds, workers)
                configs[name]["all_cores_GBs"] = round(2.0 * w / t / 1e9, 4)
                configs[name]["all_cores"] = workers
            return res
    except Exception as e:  # noqa: BLE001 - reported in the JSON line instead
        return {"error": "%s: %s" % (type(e).__name__, e), "cores": workers}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--cpu-seconds", type=float, default=6.0)
    ap.add_argument("--no-configs", action="store_true", help="only the headline layer line (no gate_proj / expert "
                    "keys and no per-config CPU oracle legs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--extras", action="store_true", help="also time decode, the batch sweep, the experts, "
                    "raw BF16 and a copy ceiling")
    ap.add_argument("--gate-batch", type=int, default=0, metavar="B",
                    help="time only the gate_proj product (14336 x 4096) at batch B (GEMV for B <= 8, MFMA GEMM "
                         "above) and print its own line; for profiling")
    ap.add_argument("--model-sweep", action="store_true",
                    help="also code the full 32-layer weight set and time GEMV and decode sweeps over it (minutes)")
    ap.add_argument("--layer-step", action="store_true",
                    help="time only one decode step of the whole layer at batch 1 (QKV grouped, o_proj, gate/up "
                         "with the SiLU-mul epilogue fused, down_proj on its output) against raw BF16; own line")
    ap.add_argument("--k15h", action="store_true",
                    help="time only the entropy-coded (K15H) variant on the layer: sizes against the order-0 bound, "
                         "re-coding and decode; prints its own line")
    ap.add_argument("--rotate-gb", type=float, default=4.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB elementwise copy first (scale for FETCH_SIZE / WRITE_SIZE counter runs)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "BENCH_JSON"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (and the JSON line bench.py "
                         "printed in one of those runs) into the traffic summary, print it and exit")
    args = ap.parse_args()

    if args.summarize_counters:
        fetch_csv, write_csv, bench_json = args.summarize_counters
        with open(bench_json) as f:
            line = [l for l in f if l.startswith("{")][-1]
        alg = json.loads(line)["roofline"]["algorithmic_bytes_per_launch"]
        print(json.dumps(summarize_counters(fetch_csv, write_csv, KERNEL.split("::")[1].split("<")[0], alg), indent=1))
        return

    if args.gate_batch:
        return gate_batch(args)
    if args.k15h:
        return k15h_only(args)
    if args.layer_step:
        return layer_step_only(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused decode-GEMV runs on one GPU and has no cross-GPU step "
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

    if args.copy_calibration:
        copy_calibration(torch)
    calls = [lbf.prepare(r, xd, lbf.LBF_F32, outs=ys) for r in rot]
    step = lambda i: calls[i % copies]()
    # exactly the requested warm-up here (500 launches by default: about
    # 28 ms, enough for the clocks to settle)
    ms_step = time_region(torch, step, args.steps, args.warmup, warm_ms=0)
    batch_ms = time_batches(torch, step, max(args.steps // 10, 5), 10, 3)
    ms_single, _ = time_each(torch, step, max(args.steps // 2, 10), 3)
    alg = sum(algorithmic_bytes(b, 1, 4) for b in blobs)
    achieved = alg / (ms_step * 1e-3) / 1e9
    value = 2.0 * n_weights / (ms_step * 1e-3) / 1e9
    log("launch mean %.2f us: %.1f GB/s BF16-equiv, %.1f GB/s algorithmic (%.1f %% of 8 TB/s)"
        % (ms_step * 1e3, value, achieved, 100 * achieved / HBM_PEAK_GBS))

    # side lanes, same run: the read-stream ceiling, and the uncompressed
    # layer through torch's F.linear (four rotating BF16 copies)
    ceiling = read_ceiling(torch)
    # the same read over exactly the launch's algorithmic bytes: a kernel that
    # only streams them, with its own launch, ramp-up and tail
    same_us = alg / (read_ceiling(torch, 40, alg) * 1e9) * 1e6
    wrot = [[dev(torch, W) for W in Ws] for _ in range(4)]
    raw_ms = time_torch_linear(torch, [list(zip(xd, wr)) for wr in wrot], 20)
    del wrot
    torch.cuda.empty_cache()
    log("read-stream ceiling %.1f GB/s; the same read over the launch's %d bytes %.2f us; raw BF16 F.linear layer "
        "%.2f us" % (ceiling, alg, same_us, raw_ms * 1e3))

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
                     "kernel": KERNEL, "algorithmic_bytes_per_launch": alg,
                     "launch_us_mean": round(ms_step * 1e3, 2),
                     "batch_mean_us_median": round(float(np.median(batch_ms)) * 1e3, 2),
                     "batch_mean_us_min": round(float(np.min(batch_ms)) * 1e3, 2),
                     "frac_batch_median": round(alg / (float(np.median(batch_ms)) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "batches": "%d batches of 10 back-to-back launches" % len(batch_ms),
                     "single_launch_event_us_median": round(ms_single * 1e3, 2),
                     "read_stream_ceiling": round(ceiling, 1),
                     "frac_of_read_stream_ceiling": round(achieved / ceiling, 4),
                     "read_stream_same_bytes_us": round(same_us, 2),
                     "speed_vs_same_bytes_read": round(same_us / (ms_step * 1e3), 4)},
        "side_lanes": {"raw_bf16_linear_layer_us": round(raw_ms * 1e3, 2),
                       "speedup_vs_raw_bf16": round(raw_ms / ms_step, 3),
                       "read_stream_ceiling_GBs": round(ceiling, 1)},
    }

    if not args.no_configs:
        out["configs"] = config_keys(torch, lbf, synth, Ws, blobs, rot, copies)
    if args.extras:
        out["extra"] = extras(torch, lbf, synth, Ws, blobs, rot, copies, args)
        out["extra"]["k15h_layer"] = k15h(torch, lbf, Ws, blobs)
        out["extra"]["layer_step_b1"] = layer_step(torch, lbf, synth, Ws, blobs)
    if args.model_sweep:
        del rot, calls
        torch.cuda.empty_cache()
        out.setdefault("extra", {})["model_sweep"] = model_sweep(torch, lbf, synth)

    if not args.no_cpu:
        log("timing the CPU oracle (~%.0f s)" % (3 * args.cpu_seconds))
        out["cpu_baseline"] = cpu_baseline(Ws, xs, args.cpu_seconds, min(16, os.cpu_count() or 1),
                                           legs=None if args.no_configs else cpu_legs(synth, Ws),
                                           leg_seconds=0.5)
    print(json.dumps(out))


def _timed(torch, calls, alg, steps=50):
    """Back-to-back mean and the median of 10-launch batch means (us), and the
    fractions of 8 TB/s they give for alg bytes a launch."""
    n = len(calls)
    ms = time_region(torch, lambda i: calls[i % n](), steps, 5)
    bm = float(np.median(time_batches(torch, lambda i: calls[i % n](), 5, 10, 2)))
    return {"us": round(ms * 1e3, 2), "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "batch_median_us": round(bm * 1e3, 2), "frac_batch_median": round(alg / (bm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": alg}


def config_keys(torch, lbf, synth, Ws, blobs, rot, copies):
    """The other workloads beside the headline, each with its own roofline
    fraction (algorithmic bytes / time against 8 TB/s): gate_proj (14336 x
    4096) alone at batch 1 (fused GEMV), 8, 16 and 64 (fused GEMM on MFMA),
    bf16 output, with torch's F.linear on the uncompressed tensor beside it;
    and the 64 expert tensors (1536 x 4096, escape-rate stress) in one grouped
    call at batch 4, fp32 output.  Rotation copies keep the working set past
    the 256 MB cache."""
    g = synth.GATE
    res = {}
    wraw = [dev(torch, Ws[g]) for _ in range(4)]
    for batch in (1, 8, 16, 64):
        x = dev(torch, synth.gate_batch_x(batch))
        y = torch.empty((batch, blobs[g].rows), dtype=torch.bfloat16, device="cuda")
        calls = [lbf.prepare(r[g], x, lbf.LBF_BF16, outs=y) for r in rot]
        r = _timed(torch, calls, algorithmic_bytes(blobs[g], batch, 2))
        r["path"] = product_path(blobs[g], batch)
        r["raw_bf16_linear_us"] = round(time_torch_linear(torch, [[(x, w)] for w in wraw]) * 1e3, 2)
        res["gate_proj_b%d" % batch] = r
        log("gate_proj batch %d: %.2f us (%.3f of 8 TB/s), raw BF16 F.linear %.2f us"
            % (batch, r["us"], r["frac"], r["raw_bf16_linear_us"]))
    del wraw
    Wx = [synth.expert_tensor(e) for e in range(64)]
    ex = [lbf.encode(dev(torch, W)) for W in Wx]
    exr = [ex] + [[lbf.Blob(b.desc, b.data.clone()) for b in ex] for _ in range(3)]
    xe = [dev(torch, synth.expert_x(e)) for e in range(64)]
    ye = [torch.empty((4, b.rows), dtype=torch.float32, device="cuda") for b in ex]
    calls = [lbf.prepare(r, xe, lbf.LBF_F32, outs=ye) for r in exr]
    r = _timed(torch, calls, sum(algorithmic_bytes(b, 4, 4) for b in ex), 20)
    r.update({"groups": 64, "launches": 1, "coded_bytes": sum(b.nbytes for b in ex), "escapes": sum(b.n_esc for b in ex)})
    res["experts64_b4"] = r
    log("64 experts at batch 4: %.2f us (%.3f of 8 TB/s)" % (r["us"], r["frac"]))
    del ex, exr, calls, Wx
    torch.cuda.empty_cache()
    return res


def cpu_legs(synth, Ws):
    """The CPU oracle's workloads beside the headline: the single 1024 x 1024
    tensor, gate_proj at every batch of the sweep, a sample of the 64 experts
    at batch 4 (every fourth Gaussian expert plus the Laplace and all-patterns
    ones), and encoding the layer."""
    W0, x0 = synth.single_tensor()
    g = Ws[synth.GATE]
    legs = {"single_1024x1024_b1": ("single 1024x1024 tensor: oracle decode + float64 matvec at batch 1",
                                    [("dm", W0, x0)])}
    for b in (1, 2, 4, 8, 16, 32, 64):
        legs["gate_proj_b%d" % b] = ("gate_proj 14336x4096: oracle decode + float64 matvec at batch %d" % b,
                                     [("dm", g, synth.gate_batch_x(b))])
    es = list(range(0, 62, 4)) + [62, 63]
    legs["experts64_b4_sample"] = ("%d of the 64 experts (1536x4096): oracle decode + float64 matvec at batch 4"
                                   % len(es), [("dm", synth.expert_tensor(e), synth.expert_x(e)) for e in es])
    legs["encode_layer"] = ("oracle encode of the 7 layer tensors", [("enc", W) for W in Ws])
    return legs


def extras(torch, lbf, synth, Ws, blobs, rot, copies, args):
    """Context lines beside the headline: standalone decode of the layer, the
    uncompressed BF16 layer through torch's F.linear, and a batch sweep of the
    fused product on gate_proj alone."""
    res = {}
    outs = [torch.empty((b.rows, b.cols), dtype=torch.bfloat16, device="cuda") for b in blobs]

    def dec(i):
        for b, o in zip(rot[i % copies], outs):
            lbf.decode(b, out=o)

    ms = time_region(torch, dec, 20, 3)
    n = sum(W.size for W in Ws)
    alg = sum(algorithmic_bytes(b, 0, 0) for b in blobs) + 2 * n
    res["decode_layer"] = {"us": round(ms * 1e3, 2), "bf16_equiv_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1),
                           "hbm_GBs": round(alg / (ms * 1e-3) / 1e9, 1)}
    del outs
    # integrity checks of the resident layer: structural verification of every
    # blob (reads the nibble plane, index, escapes, header and padding) and
    # CRC-32 of every whole blob
    flags = torch.empty((len(blobs), 1), dtype=torch.int32, device="cuda")

    def ver(i):
        for j, b in enumerate(rot[i % copies]):
            lbf.verify_into(b, flags[j])

    ms = time_region(torch, ver, 20, 3)
    assert int(flags.abs().sum()) == 0, "a resident blob failed verification"
    vb = sum(b.nbytes - b.rows * b.cols for b in blobs)  # everything but the raw plane
    res["verify_layer"] = {"us": round(ms * 1e3, 2), "GBs": round(vb / (ms * 1e-3) / 1e9, 1),
                           "bytes_read": vb}

    def crc(i):
        for j, b in enumerate(rot[i % copies]):
            lbf.crc32_into(b.data, flags[j])

    ms = time_region(torch, crc, 20, 3)
    cb = sum(b.nbytes for b in blobs)
    res["crc32_layer"] = {"us": round(ms * 1e3, 2), "GBs": round(cb / (ms * 1e-3) / 1e9, 1), "bytes_read": cb}
    wd = [dev(torch, W) for W in Ws]
    xd = [dev(torch, synth.layer_x(m)) for m in range(len(Ws))]
    wrot = [wd] + [[w.clone() for w in wd] for _ in range(3)]

    ms = time_torch_linear(torch, [list(zip(xd, wr)) for wr in wrot], 20)
    res["raw_bf16_linear_layer"] = {"us": round(ms * 1e3, 2), "GBs": round(2 * n / (ms * 1e-3) / 1e9, 1),
                                    "hbm_frac": round(2 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del wd, wrot
    torch.cuda.empty_cache()
    g = synth.GATE
    sweep = {}
    wg = [dev(torch, Ws[g])] + [dev(torch, Ws[g]) for _ in range(3)]
    for batch in (1, 2, 4, 8, 16, 32, 64):
        x = dev(torch, synth.gate_batch_x(batch))
        y = torch.empty((batch, blobs[g].rows), dtype=torch.bfloat16, device="cuda")
        calls = [lbf.prepare(r[g], x, lbf.LBF_BF16, outs=y) for r in rot]
        ms = time_region(torch, lambda i: calls[i % copies](), 30, 5)
        alg = algorithmic_bytes(blobs[g], batch, 2)
        flops = 2.0 * batch * Ws[g].size
        ms_raw = time_torch_linear(torch, [[(x, w)] for w in wg])
        path = product_path(blobs[g], batch)
        mfma = path != "gemv"
        sweep[str(batch)] = {"path": path, "us": round(ms * 1e3, 2),
                             "bf16_equiv_GBs": round(2 * Ws[g].size / (ms * 1e-3) / 1e9, 1),
                             "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "mfma_frac_of_2.5PF": round(flops / (ms * 1e-3) / 2.5e15, 4) if mfma else None,
                             "raw_bf16_linear_us": round(ms_raw * 1e3, 2)}
    del wg
    res["gate_proj_sweep"] = sweep
    # the 64-expert set (1536 x 4096 each, escape-rate stress) grouped at batch 4
    Wx = [synth.expert_tensor(e) for e in range(64)]
    ex = [lbf.encode(dev(torch, W)) for W in Wx]
    exr = [ex] + [[lbf.Blob(b.desc, b.data.clone()) for b in ex] for _ in range(3)]
    n_e = sum(W.size for W in Wx)
    for eb in (4, 1):
        xe = [dev(torch, synth.expert_x(e, eb)) for e in range(64)]
        ye = [torch.empty((eb, b.rows), dtype=torch.float32, device="cuda") for b in ex]
        ecalls = [lbf.prepare(r, xe, lbf.LBF_F32, outs=ye) for r in exr]
        ms = time_region(torch, lambda i: ecalls[i % 4](), 20, 3)
        alg = sum(algorithmic_bytes(b, eb, 4) for b in ex)
        res[f"experts64_b{eb}"] = {"us": round(ms * 1e3, 2), "bf16_equiv_GBs": round(2 * n_e / (ms * 1e-3) / 1e9, 1),
                                   "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "coded_bytes": sum(b.nbytes for b in ex), "escapes": sum(b.n_esc for b in ex)}
    del ex, exr, ecalls, Wx
    torch.cuda.empty_cache()
    # the layer at batch 2 / 4 / 8 with its own x for every tensor (x of all
    # seven does not fit in LDS at once: CUs split into teams)
    one_x = {}
    for lb in (2, 4, 8):
        xl = [dev(torch, synth.layer_x(m, lb)) for m in range(len(Ws))]
        yl = [torch.empty((lb, b.rows), dtype=torch.float32, device="cuda") for b in blobs]
        lcalls = [lbf.prepare(r, xl, lbf.LBF_F32, outs=yl) for r in rot]
        ms = time_region(torch, lambda i: lcalls[i % copies](), 20, 3)
        alg = sum(algorithmic_bytes(b, lb, 4) for b in blobs)
        one_x[str(lb)] = {"us": round(ms * 1e3, 2), "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    res["layer_one_x_per_tensor"] = one_x
    # mixed read + write ceiling: an elementwise copy of 1 GiB (read and written)
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = time_region(torch, lambda i: torch.neg(src, out=dst), 10, 2)
    res["copy_1GiB_ceiling"] = {"us": round(ms * 1e3, 2), "GBs_read_plus_write": round(8 * COPY_ELEMS / (ms * 1e-3) / 1e9, 1)}
    del src, dst
    torch.cuda.empty_cache()
    return res


def order0_bits(Ws) -> float:
    """Order-0 entropy of the 16-bit values, bits per weight, pooled per tensor
    (the lower bound for any code that stores each weight on its own)."""
    total, n = 0.0, 0
    for W in Ws:
        c = np.bincount(W.reshape(-1), minlength=65536).astype(np.float64)
        p = c[c > 0] / W.size
        total += -float((p * np.log2(p)).sum()) * W.size
        n += W.size
    return total / n


def k15h(torch, lbf, Ws, blobs, reps: int = 20):
    """The entropy-coded variant on the layer: re-code every v1 blob on the
    GPU, then time the standalone decode of all seven tensors (outputs in HBM)."""
    t0 = time.time()
    hb = [lbf.hencode(b) for b in blobs]
    torch.cuda.synchronize()
    t_code = time.time() - t0
    n = sum(W.size for W in Ws)
    hbytes = sum(h.nbytes for h in hb)
    vbytes = sum(b.nbytes for b in blobs)
    hrot = [hb] + [[lbf.HBlob(h.desc, h.data.clone()) for h in hb] for _ in range(3)]
    outs = [torch.empty((h.rows, h.cols), dtype=torch.bfloat16, device="cuda") for h in hb]

    def dec(i):
        for h, o in zip(hrot[i % 4], outs):
            lbf.hdecode(h, out=o)

    ms = time_region(torch, dec, reps, 3)
    del hrot, outs
    torch.cuda.empty_cache()
    h0 = order0_bits(Ws)
    bits = 8.0 * hbytes / n
    return {"bytes": hbytes, "bits_per_weight": round(bits, 4), "reduction_vs_bf16": round(1 - bits / 16, 5),
            "order0_bound_bits": round(h0, 4), "above_bound_bits": round(bits - h0, 4),
            "v1_bits_per_weight": round(8.0 * vbytes / n, 4),
            "max_code_len": max(int(h.desc.max_len) for h in hb),
            "recode_s": round(t_code, 3), "decode_us": round(ms * 1e3, 2),
            "decode_bf16_equiv_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "decode_read_plus_write_GBs": round((hbytes + 2 * n) / (ms * 1e-3) / 1e9, 1)}


def layer_step(torch, lbf, synth, Ws, blobs, reps: int = 50):
    """One batch-1 decode step of the 8B-shaped layer, weights only (attention
    itself is not part of the coded path): q/k/v in one grouped launch on one
    x, o_proj on its own x, gate/up in one launch with the SiLU-mul epilogue,
    down_proj on that output (bf16).  Compared with the same step unfused
    (gate/up as a grouped GEMV, then silu * up in torch) and with raw BF16
    torch (concatenated QKV and gate/up weights, F.linear)."""
    F = torch.nn.functional
    Q, K, V, O_, G, U, D = range(7)
    copies = 4
    brot = [blobs] + [[lbf.Blob(b.desc, b.data.clone()) for b in blobs] for _ in range(copies - 1)]
    x_attn = dev(torch, synth.layer_x(Q))
    x_o = dev(torch, synth.layer_x(O_))
    x_mlp = dev(torch, synth.layer_x(G))
    f32, bf = lbf.LBF_F32, lbf.LBF_BF16
    qkv_out = [torch.empty((1, blobs[m].rows), dtype=torch.float32, device="cuda") for m in (Q, K, V)]
    o_out = torch.empty((1, blobs[O_].rows), dtype=torch.float32, device="cuda")
    h = torch.empty((1, blobs[G].rows), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((1, blobs[D].rows), dtype=torch.float32, device="cuda")
    gu = [torch.empty((1, blobs[m].rows), dtype=torch.float32, device="cuda") for m in (G, U)]
    qkv_calls = [lbf.prepare([r[Q], r[K], r[V]], [x_attn] * 3, f32, outs=qkv_out) for r in brot]
    o_calls = [lbf.prepare([r[O_]], [x_o], f32, outs=[o_out]) for r in brot]
    d_calls = [lbf.prepare([r[D]], [h], f32, outs=[y]) for r in brot]
    gu_calls = [lbf.prepare([r[G], r[U]], [x_mlp] * 2, f32, outs=gu) for r in brot]

    def fused(i):
        r = brot[i % copies]
        qkv_calls[i % copies]()
        o_calls[i % copies]()
        lbf.swiglu(r[G], r[U], x_mlp, bf, out=h)
        d_calls[i % copies]()

    def unfused(i):
        qkv_calls[i % copies]()
        o_calls[i % copies]()
        gu_calls[i % copies]()
        torch.mul(F.silu(gu[0]), gu[1], out=gu[0])
        h.copy_(gu[0])
        d_calls[i % copies]()

    ms_fused = time_region(torch, fused, reps, 5)
    ms_unfused = time_region(torch, unfused, reps, 5)
    ms_swiglu = time_region(torch, lambda i: lbf.swiglu(brot[i % copies][G], brot[i % copies][U], x_mlp, bf, out=h),
                            reps, 5)
    del brot, qkv_calls, o_calls, d_calls, gu_calls
    torch.cuda.empty_cache()
    # raw BF16: best case for torch, concatenated weights
    raw = []
    for _ in range(copies):
        w = [dev(torch, W) for W in Ws]
        raw.append((torch.cat([w[Q], w[K], w[V]]), w[O_], torch.cat([w[G], w[U]]), w[D]))
        del w
    rows_g = Ws[G].shape[0]

    def torch_step(i):
        wqkv, wo, wgu, wd = raw[i % copies]
        F.linear(x_attn, wqkv)
        F.linear(x_o, wo)
        t = F.linear(x_mlp, wgu)
        hh = F.silu(t[:, :rows_g]) * t[:, rows_g:]
        F.linear(hh, wd)

    ms_torch = time_region(torch, torch_step, reps, 5)
    del raw
    torch.cuda.empty_cache()
    n = sum(W.size for W in Ws)
    coded = sum(b.nbytes for b in blobs)
    return {"weights": n, "coded_bytes": coded, "bf16_bytes": 2 * n, "launches_fused": 4,
            "fused_step_us": round(ms_fused * 1e3, 2), "unfused_step_us": round(ms_unfused * 1e3, 2),
            "torch_bf16_step_us": round(ms_torch * 1e3, 2),
            "speedup_vs_bf16": round(ms_torch / ms_fused, 3),
            "gate_up_swiglu_us": round(ms_swiglu * 1e3, 2),
            "fused_step_hbm_frac": round(coded / (ms_fused * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "torch_step_hbm_frac": round(2 * n / (ms_torch * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def layer_step_only(args):
    import torch

    from decode_byte_split_amd import lbf, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    Ws = [synth.layer_tensor(m) for m in range(len(synth.LAYER))]
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    torch.cuda.synchronize()
    r = layer_step(torch, lbf, synth, Ws, blobs, reps=args.steps)
    print(json.dumps({"workload": "llama8b_layer_decode_step_b1", **r}))


def k15h_only(args):
    import torch

    from decode_byte_split_amd import lbf, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    Ws = [synth.layer_tensor(m) for m in range(len(synth.LAYER))]
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    torch.cuda.synchronize()
    r = k15h(torch, lbf, Ws, blobs, reps=args.steps)
    print(json.dumps({"workload": "llama8b_layer_k15h", "tensors": [m[0] for m in synth.LAYER], **r}))


def gate_batch(args):
    """gate_proj (14336 x 4096) at one batch size, bf16 output: the fused
    product alone, rotated over 4 GB of coded copies, HIP-event timed."""
    import torch

    from decode_byte_split_amd import lbf, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B = args.gate_batch
    W = synth.layer_tensor(synth.GATE)
    blob = lbf.encode(dev(torch, W))
    copies = max(1, int(np.ceil(args.rotate_gb * 1e9 / blob.nbytes)))
    rot = [blob] + [lbf.Blob(blob.desc, blob.data.clone()) for _ in range(copies - 1)]
    x = dev(torch, synth.gate_batch_x(B))
    y = torch.empty((B, blob.rows), dtype=torch.bfloat16, device="cuda")
    calls = [lbf.prepare(r, x, lbf.LBF_BF16, outs=y) for r in rot]
    ms = time_region(torch, lambda i: calls[i % copies](), args.steps, args.warmup)
    alg = algorithmic_bytes(blob, B, 2)
    flops = 2.0 * B * W.size
    out = {"metric": "fused decode product BF16-equiv weight GB/s, gate_proj", "value": round(2 * W.size / (ms * 1e-3) / 1e9, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "gate_proj_14336x4096", "batch": B, "y_dtype": "bf16",
                      "path": product_path(blob, B), "rotation_copies": copies},
           "roofline": {"bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes_per_launch": alg},
           "mfma": {"tflops": round(flops / (ms * 1e-3) / 1e12, 2), "frac_of_2.5PF_bf16": round(flops / (ms * 1e-3) / 2.5e15, 4)}
           if B > 8 else None}
    print(json.dumps(out))


def model_sweep(torch, lbf, synth):
    """The full 32-layer 8B-shaped weight set (224 tensors, 6.98e9 weights):
    coded tensor by tensor on the GPU, then a fused batch-1 GEMV sweep (one
    grouped launch per layer, each tensor with its own x) and a standalone
    decode sweep over every tensor."""
    t0 = time.time()
    layers, xs = [], []
    for L in range(32):
        blobs = []
        for m in range(len(synth.LAYER)):
            W = synth.model_tensor(L, m)
            blobs.append(lbf.encode(dev(torch, W)))
            del W
        layers.append(blobs)
        xs.append([dev(torch, synth.model_x(L, m)) for m in range(len(synth.LAYER))])
        if L % 8 == 7:
            torch.cuda.synchronize()
            log("model sweep: %d layers coded (%.0f s)" % (L + 1, time.time() - t0))
    n = sum(r * c for _, r, c in synth.LAYER) * 32
    coded = sum(b.nbytes for bl in layers for b in bl)
    ys = [[torch.empty((1, b.rows), dtype=torch.float32, device="cuda") for b in bl] for bl in layers]
    calls = [lbf.prepare(bl, x, lbf.LBF_F32, outs=y) for bl, x, y in zip(layers, xs, ys)]

    def sweep(i):
        for c in calls:
            c()

    ms = time_region(torch, sweep, 5, 2)
    alg = sum(algorithmic_bytes(b, 1, 4) for bl in layers for b in bl)
    outs = {}
    for bl in layers[:1]:
        for b in bl:
            outs[(b.rows, b.cols)] = torch.empty((b.rows, b.cols), dtype=torch.bfloat16, device="cuda")

    def dec(i):
        for bl in layers:
            for b in bl:
                lbf.decode(b, out=outs[(b.rows, b.cols)])

    ms_d = time_region(torch, dec, 3, 1)
    return {"workload": "llama8b_32_layers", "tensors": 32 * len(synth.LAYER), "weights": n, "coded_bytes": coded,
            "bits_per_weight": round(8.0 * coded / n, 4), "reduction_vs_bf16": round(1 - coded / (2.0 * n), 5),
            "gemv_sweep_us": round(ms * 1e3, 1), "gemv_bf16_equiv_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "gemv_hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_sweep_us": round(ms_d * 1e3, 1),
            "decode_hbm_GBs": round((sum(algorithmic_bytes(b, 0, 0) for bl in layers for b in bl) + 2 * n)
                                    / (ms_d * 1e-3) / 1e9, 1)}


if __name__ == "__main__":
    main()
