"""The full 32-layer 8B-shaped weight set (224 tensors, 6.98e9 weights), every
tensor on the GPU.

Per tensor: GPU encode, GPU decode compared bit for bit with the source on the
device (decoding must give back the source bits: "Lossless LLM Weight
Compression vs 8-bit GGUF", section "What does 'lossless' mean for LLM
weights?"), and lbf_verify clean.  Per layer: the k_proj blob equals the
oracle's byte for byte; the grouped batch-1 GEMV matches the float64 oracle on
row ranges at the start, middle and end of every tensor; and the layer goes
through a hashed artifact file, is loaded back with host and GPU checks and
decoded tensor by tensor against its source, the shipped-container check of
the same page's section "A 14-day production-readiness pilot", step 2.
Layers are generated one ahead in a worker thread.  Tensor seeds are those of
``synth.model_tensor`` (layer, matrix index).
"""
import concurrent.futures as cf
import os
import time

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth
from gpu_util import check_product, dev, make_env, say

pytestmark = pytest.mark.gpu

N_LAYERS = 32
PER_TEST = 4  # layers per test, so each test stays well inside its time limit


@pytest.fixture(scope="module")
def env():
    return make_env()


def _gen_layer(layer):
    Ws = [synth.model_tensor(layer, m) for m in range(len(synth.LAYER))]
    xs = [synth.model_x(layer, m) for m in range(len(synth.LAYER))]
    return Ws, xs


@pytest.mark.parametrize("first", range(0, N_LAYERS, PER_TEST))
def test_model_layers_every_tensor(env, tmp_path, first):
    torch, lbf = env
    from decode_byte_split_amd import artifact as A

    names = [m[0] for m in synth.LAYER]
    K = names.index("k_proj")
    pool = cf.ThreadPoolExecutor(1)
    nxt = pool.submit(_gen_layer, first)
    totals = {"weights": 0, "file_bytes": 0}
    try:
        for layer in range(first, first + PER_TEST):
            t0 = time.time()
            Ws, xs = nxt.result()
            if layer + 1 < first + PER_TEST:
                nxt = pool.submit(_gen_layer, layer + 1)
            say("model layer %d: generated (%.1f s wait)" % (layer, time.time() - t0))
            blobs = []
            flags = torch.zeros(len(Ws), dtype=torch.int32, device="cuda")
            for m, W in enumerate(Ws):
                wd = dev(torch, W)
                b = lbf.encode(wd)
                out = lbf.decode(b)
                assert torch.equal(out.view(torch.int16), wd.view(torch.int16)), (layer, names[m])
                lbf.verify_into(b, flags[m])
                blobs.append(b)
                del wd, out
            assert int(flags.abs().sum()) == 0, (layer, flags.cpu().numpy())
            assert np.array_equal(blobs[K].data.cpu().numpy(), O.encode(Ws[K])), layer
            ys = lbf.gemv(blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
            torch.cuda.synchronize()
            for W, x, y in zip(Ws, xs, ys):
                R = W.shape[0]
                for r0 in (0, R // 2 - 64, R - 128):
                    y_ref, a_ref = O.matvec(W, x, rows=(r0, r0 + 128))
                    check_product(y[:, r0:r0 + 128], y_ref, a_ref, False)
            # the shipped container: save, load with every check, decode each tensor
            path = str(tmp_path / ("layer%d.lbfa" % layer))
            A.save(path, dict(zip(names, blobs)))
            del blobs, ys
            ok = A.check_against(path, lambda name: Ws[names.index(name)])
            assert len(ok) == len(names) and all(ok.values()), (layer, ok)
            rep = A.size_report(path)
            assert rep["reduction_vs_bf16"] >= 0.24, rep
            totals["weights"] += rep["weights"]
            totals["file_bytes"] += rep["file_bytes"]
            os.remove(path)
            say("model layer %d: 7/7 tensors bit-exact (GPU decode and artifact), verify clean, GEMV rows ok, "
                "artifact %.4f bits/weight (%.1f s)" % (layer, rep["bits_per_weight"], time.time() - t0))
    finally:
        pool.shutdown(wait=True)
    red = 1.0 - totals["file_bytes"] / (2.0 * totals["weights"])
    say("layers %d-%d: %d weights, artifact files %d bytes, %.3f %% smaller than BF16"
        % (first, first + PER_TEST - 1, totals["weights"], totals["file_bytes"], 100 * red))
    assert red >= 0.24
