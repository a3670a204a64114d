"""Concurrent calls from several host threads, each on a stream of its own,
with the first launch of every kernel instance made concurrently (this module
runs before the other product tests): every result matches the float64
oracle and is bitwise equal to the same call made again alone afterwards.
The library's per-device launch facts (CU count, resident workgroups, each
kernel's dynamic LDS limit) are looked up under a lock; this checks that
racing first calls still launch every kernel with a valid configuration."""
import threading

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth
from gpu_util import check_product, dev, make_env, say
from test_gpu_swiglu import check_h

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    return make_env()


def test_threads_first_calls(env):
    torch, lbf = env
    rng = np.random.default_rng(2024)
    # (rows, cols, batch, op): ring GEMV at batch 1/3, the static GEMV (x of
    # 8 x 14336 columns does not fit the ring's LDS x area), GEMM at 16 / 40
    # columns, and the fused gate/up product
    cases = [(64, 2048, 1, "gemv"), (48, 3072, 3, "gemv"), (32, 14336, 8, "gemv"),
             (64, 4096, 16, "gemm"), (80, 2048, 40, "gemm"), (64, 2048, 2, "swiglu")]
    jobs = []
    for rows, cols, batch, op in cases:
        W = synth.gaussian(rng, rows, cols, 0.02, 0.001, 100.0)
        x = synth.activations(rng, batch, cols)
        if op == "swiglu":
            U = synth.gaussian(rng, rows, cols, 0.02, 0.001, 100.0)
            ref = O.swiglu(W, U, x)
            blobs = (lbf.from_host_blob(O.encode(W)), lbf.from_host_blob(O.encode(U)))
        else:
            ref = O.matvec(W, x)
            blobs = (lbf.from_host_blob(O.encode(W)),)
        jobs.append((op, blobs, dev(torch, x), ref))
    torch.cuda.synchronize()

    def call(op, blobs, x, stream):
        if op == "gemv":
            return lbf.gemv(blobs[0], x, lbf.LBF_F32, stream=stream)
        if op == "gemm":
            return lbf.gemm(blobs[0], x, lbf.LBF_F32, stream=stream)
        return lbf.swiglu(blobs[0], blobs[1], x, lbf.LBF_F32, stream=stream)

    streams = [torch.cuda.Stream() for _ in jobs]
    start = threading.Barrier(len(jobs))
    out = [None] * len(jobs)
    err = []

    def worker(i):
        op, blobs, x, _ = jobs[i]
        try:
            with torch.cuda.stream(streams[i]):
                start.wait(timeout=60)
                for _ in range(3):  # later calls take the cached facts
                    out[i] = call(op, blobs, x, streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported below, in the main thread
            err.append((i, repr(e)))

    say("concurrent first calls: %d threads" % len(jobs))
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not err, err
    torch.cuda.synchronize()
    for i, (op, blobs, x, ref) in enumerate(jobs):
        say("concurrent case %d: %s %s" % (i, op, tuple(x.shape)))
        if op == "swiglu":
            check_h(out[i], ref, False)
        else:
            check_product(out[i], ref[0], ref[1], False)
        again = call(op, blobs, x, None)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int32), out[i].view(torch.int32))
