"""The fused products under HIP graph capture: a captured grouped GEMV (the
8B-shaped layer, batch 1) and a captured GEMM (gate_proj, batch 16) replay to
exactly the eager results, replay after replay, with new x copied in between
and eager work on the stream between the replays."""
import numpy as np
import pytest

from decode_byte_split_amd import synth
from gpu_util import dev, make_env, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    return make_env()


def _replays(torch, lbf, blobs, x_bufs, x_sets, y_dtype):
    """Eager outputs and graph-replay outputs for each x set."""
    lbf.matmul(blobs, x_bufs, y_dtype)  # first use sets kernel attributes outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ys = lbf.matmul(blobs, x_bufs, y_dtype)
    eager, replayed = [], []
    for xs in x_sets:
        for buf, x in zip(x_bufs, xs):
            buf.copy_(x)
        e = [y.clone() for y in lbf.matmul(blobs, x_bufs, y_dtype)]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager.append(e)
        replayed.append([y.clone() for y in ys])
        _ = torch.ones(1 << 20, device="cuda").sum()  # unrelated eager work between replays
    return eager, replayed


def test_graph_layer_gemv(env):
    torch, lbf = env
    blobs = [lbf.encode(dev(torch, synth.layer_tensor(m))) for m in range(len(synth.LAYER))]
    x_bufs = [torch.empty((1, b.cols), dtype=torch.bfloat16, device="cuda") for b in blobs]
    rng = np.random.default_rng(41)
    x_sets = [[dev(torch, synth.activations(rng, 1, b.cols)) for b in blobs] for _ in range(4)]
    eager, replayed = _replays(torch, lbf, blobs, x_bufs, x_sets, lbf.LBF_F32)
    for i, (e, r) in enumerate(zip(eager, replayed)):
        for a, b in zip(e, r):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), i
    say("layer GEMV: %d graph replays equal the eager results" % len(eager))


def test_graph_gate_gemm(env):
    torch, lbf = env
    blob = lbf.encode(dev(torch, synth.layer_tensor(synth.GATE)))
    x_buf = torch.empty((16, blob.cols), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(42)
    x_sets = [[dev(torch, synth.activations(rng, 16, blob.cols))] for _ in range(4)]
    eager, replayed = _replays(torch, lbf, [blob], [x_buf], x_sets, lbf.LBF_BF16)
    for i, (e, r) in enumerate(zip(eager, replayed)):
        assert torch.equal(e[0].view(torch.int16), r[0].view(torch.int16)), i
