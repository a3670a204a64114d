"""GPU parity of the fused decode-GEMM (bf16 MFMA, batch 9..256) against the
float64 oracle, through the C ABI.

Bar as for the GEMV: |y - y_ref| <= 1e-3 * sum_k |W[r,k]| |x[b,k]| per
output (plus half a bf16 ulp of y_ref for bf16 output); non-finite outputs
match in class; rows of the identity as x extract columns of W exactly.
"""
import time

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth
from gpu_util import check_product, dev, host, make_env, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    return make_env()


@pytest.mark.parametrize("batch", [9, 16, 17, 31, 48, 64, 65, 100, 256])
def test_gemm_single_tensor(env, batch):
    torch, lbf = env
    W, _ = synth.single_tensor()
    x = synth.activations(np.random.default_rng([0, 2, batch]), batch, 1024)
    say("gemm single_tensor B=%d" % batch)
    blob = lbf.from_host_blob(O.encode(W))
    y_ref, a_ref = O.matvec(W, x)
    y = lbf.gemm(blob, dev(torch, x), lbf.LBF_F32)
    torch.cuda.synchronize()
    check_product(y, y_ref, a_ref, False)
    yb = lbf.gemm(blob, dev(torch, x), lbf.LBF_BF16)
    torch.cuda.synchronize()
    check_product(yb, y_ref, a_ref, True)


@pytest.mark.parametrize("name", ["laplace", "rate20pct"])
def test_gemm_identity_extracts_columns_exactly(env, name):
    """x = rows of the identity: every product but one is an exact zero, so
    y[b] is column k_b of W, bit for bit (as values: -0 compares equal to 0)."""
    torch, lbf = env
    rng = np.random.default_rng(11)
    W = synth.laplace(rng, 200, 3072, 0.02) if name == "laplace" else synth.gaussian(rng, 200, 3072, 0.02, 0.2, 100.0)
    blob = lbf.from_host_blob(O.encode(W))
    ks = [0, 1, 7, 8, 15, 16, 31, 32, 255, 256, 1023, 1024, 2047, 2048, 3000, 3071, 5, 1500]
    x = np.zeros((len(ks), 3072), dtype=np.uint16)
    for b, k in enumerate(ks):
        x[b, k] = 0x3F80
    y = lbf.gemm(blob, dev(torch, x), lbf.LBF_F32)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for b, k in enumerate(ks):
        assert np.array_equal(y[b], synth.bf16_to_f32(W[:, k])), k


def test_gemm_gate_batch_sweep(env):
    """gate_proj (14336 x 4096) at batch 16, 32, 64: bf16 and fp32 output,
    checked on row ranges at the start, middle and end of the tensor."""
    torch, lbf = env
    W = synth.layer_tensor(synth.GATE)
    blob = lbf.encode(dev(torch, W))
    ranges = [(0, 320), (7040, 7296), (14016, 14336)]
    for batch in (16, 32, 64):
        x = synth.gate_batch_x(batch)
        xd = dev(torch, x)
        yb = lbf.gemm(blob, xd, lbf.LBF_BF16)
        yf = lbf.gemm(blob, xd, lbf.LBF_F32)
        torch.cuda.synchronize()
        for r0, r1 in ranges:
            y_ref, a_ref = O.matvec(W, x, rows=(r0, r1))
            check_product(yb[:, r0:r1], y_ref, a_ref, True)
            check_product(yf[:, r0:r1], y_ref, a_ref, False)
        say("gemm gate sweep B=%d ok" % batch)


def test_gemm_layer_grouped(env):
    """The 8B-shaped layer's 7 tensors in one grouped call at batch 16."""
    torch, lbf = env
    Ws = [synth.layer_tensor(m) for m in range(len(synth.LAYER))]
    xs = [synth.layer_x(m, 16) for m in range(len(synth.LAYER))]
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    ys = lbf.gemm(blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for m, (W, x, y) in enumerate(zip(Ws, xs, ys)):
        R = W.shape[0]
        for r0 in (0, R // 2 - 64, R - 128):
            y_ref, a_ref = O.matvec(W, x, rows=(r0, r0 + 128))
            check_product(y[:, r0:r0 + 128], y_ref, a_ref, False)
        say("gemm layer %s ok" % synth.LAYER[m][0])


def test_gemm_experts_grouped(env):
    """64 expert tensors (escape-rate stress, all patterns) at batch 16."""
    torch, lbf = env
    t0 = time.time()
    Ws = [synth.expert_tensor(e) for e in range(64)]
    xs = [synth.expert_x(e, 16) for e in range(64)]
    say("experts generated in %.1fs" % (time.time() - t0))
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    ys = lbf.gemm(blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for e in range(64):
        rows = None if e in (3, 4, 62, 63) else (0, 96)
        y_ref, a_ref = O.matvec(Ws[e], xs[e], rows=rows)
        y = ys[e] if rows is None else ys[e][:, :96]
        check_product(y, y_ref, a_ref, False)
    say("gemm experts ok")


@pytest.mark.parametrize("rows,cols,batch", [(1, 1024, 9), (7, 14336, 16), (33, 5120, 40), (130, 2048, 64),
                                             (3, 30720, 17), (70, 3072, 100), (16, 65536, 12)])
def test_gemm_odd_shapes(env, rows, cols, batch):
    torch, lbf = env
    rng = np.random.default_rng([6, rows, cols])
    W = synth.gaussian(rng, rows, cols, 0.03, 0.003, 80.0)
    x = synth.activations(rng, batch, cols)
    say("gemm odd shape %dx%d B=%d" % (rows, cols, batch))
    blob = lbf.from_host_blob(O.encode(W))
    y_ref, a_ref = O.matvec(W, x)
    guard = 256
    buf = torch.full((batch * rows + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    y = buf[guard:guard + batch * rows].view(batch, rows)
    lbf.gemm(blob, dev(torch, x), lbf.LBF_F32, outs=y)
    torch.cuda.synchronize()
    check_product(y, y_ref, a_ref, False)
    h = buf.cpu().numpy()
    assert (h[:guard] == 7.0).all() and (h[guard + batch * rows:] == 7.0).all()


def test_gemm_bf16_output_guard_bands(env):
    torch, lbf = env
    rng = np.random.default_rng(12)
    rows, cols, batch = 45, 2048, 19
    W = synth.gaussian(rng, rows, cols, 0.02, 0.01, 100.0)
    x = synth.activations(rng, batch, cols)
    blob = lbf.from_host_blob(O.encode(W))
    y_ref, a_ref = O.matvec(W, x)
    guard = 512
    buf = torch.full((batch * rows + 2 * guard,), -12345, dtype=torch.int16, device="cuda")
    y = buf[guard:guard + batch * rows].view(torch.bfloat16).view(batch, rows)
    lbf.gemm(blob, dev(torch, x), lbf.LBF_BF16, outs=y)
    torch.cuda.synchronize()
    check_product(y, y_ref, a_ref, True)
    h = buf.cpu().numpy()
    assert (h[:guard] == -12345).all() and (h[guard + batch * rows:] == -12345).all()


def test_gemm_deterministic(env):
    torch, lbf = env
    W = synth.layer_tensor(1)
    x = synth.layer_x(1, 32)
    blob = lbf.encode(dev(torch, W))
    xs = dev(torch, x)
    y1 = lbf.gemm(blob, xs, lbf.LBF_F32).cpu().numpy()
    y2 = lbf.gemm(blob, xs, lbf.LBF_F32).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_gemm_many_groups_mixed_shapes(env):
    """More groups than one launch takes, mixed shapes and table kinds, batch 20."""
    torch, lbf = env
    rng = np.random.default_rng(78)
    Ws, xs = [], []
    for g in range(37):
        rows = int(rng.integers(1, 200))
        cols = 1024 * int(rng.integers(1, 6))
        if g % 3 == 0:
            W = synth.gaussian(rng, rows, cols, 0.02, 0.002, 100.0)
        elif g % 3 == 1:
            W = synth.laplace(rng, rows, cols, 0.05)
        else:
            W = synth.all_patterns(rows, cols)
        Ws.append(W)
        xs.append(synth.activations(rng, 20, cols))
    blobs = [lbf.from_host_blob(O.encode(W)) for W in Ws]
    ys = lbf.gemm(blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for W, x, y in zip(Ws, xs, ys):
        y_ref, a_ref = O.matvec(W, x)
        check_product(y, y_ref, a_ref, False)


def test_matmul_dispatch_matches(env):
    """lbf.matmul sends batch <= 8 to the GEMV and larger batches to the GEMM;
    both agree with the oracle on the same tensor."""
    torch, lbf = env
    W, _ = synth.single_tensor()
    blob = lbf.from_host_blob(O.encode(W))
    for batch in (8, 9):
        x = synth.activations(np.random.default_rng([0, 3, batch]), batch, 1024)
        y_ref, a_ref = O.matvec(W, x)
        y = lbf.matmul(blob, dev(torch, x), lbf.LBF_F32)
        torch.cuda.synchronize()
        check_product(y, y_ref, a_ref, False)
