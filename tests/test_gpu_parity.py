"""GPU parity: liblbf.so (HIP, gfx950) against the CPU oracle, through the C ABI.

Bar: decode and encode are bit-exact (byte-equal blobs, byte-equal tensors);
the fused products stay within |y - y_ref| <= 1e-3 * sum_k |W[r,k]| |x[b,k]|
of the float64 oracle (plus half a bf16 ulp of y_ref when y is rounded to
bf16); non-finite outputs must match in class (NaN <-> NaN, same-signed Inf).
"""
import os
import sys
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


def tensors():
    g = {}
    g["single_1024x1024"] = synth.single_tensor()[0]
    g["patterns_256x256"] = synth.all_patterns(256, 256)
    rng = np.random.default_rng(7)
    g["ragged_7x333"] = synth.gaussian(rng, 7, 333, 0.02, 0.01, 100.0)
    g["ragged_1x1"] = synth.gaussian(rng, 1, 1, 0.02, 0.0, 1.0)
    g["ragged_5x4097"] = synth.gaussian(rng, 5, 4097, 0.02, 0.002, 100.0)
    g["uniform_bits_3x1500"] = rng.integers(0, 65536, (3, 1500), dtype=np.uint32).astype(np.uint16)
    g["expert_rate20pct_256x1024"] = synth.gaussian(rng, 256, 1024, 0.02, 0.2, 100.0)
    g["laplace_128x2048"] = synth.laplace(rng, 128, 2048, 0.02)
    # an escape in every tile at the first and last element, and a tile of escapes
    W = synth.gaussian(rng, 4, 4096, 0.02, 0.0, 1.0)
    flat = W.reshape(-1)
    flat[::1024] = 0x7F80  # +Inf, exponent 255: never coded here
    flat[1023::1024] = 0x0001  # smallest denormal, exponent 0
    flat[4096:5120] = (np.arange(1024) % 65536).astype(np.uint16) | 0x7000
    g["edge_escapes_4x4096"] = W
    # escapes of different exponents around each tile's half boundary (the
    # decoder gives lane l the weights 8l..8l+7 of each half) and in the
    # partial second half of the last tile (3000 weights: 952 in tile 2)
    W = synth.gaussian(rng, 3, 1000, 0.02, 0.0, 1.0)
    flat = W.reshape(-1)
    for t0 in (0, 1024, 2048):
        flat[t0 + np.array([7, 8, 504, 511, 512, 513, 519, 520, 900])] = [
            0x7F80, 0x0001, 0xFF81, 0x0001, 0x7F80, 0x0002, 0xFF80, 0x0001, 0x7F80]
    flat[-1] = 0x0003
    g["half_edges_3x1000"] = W
    return g


TENSORS = tensors()


@pytest.mark.parametrize("name", sorted(TENSORS))
def test_decode_oracle_blob_bit_exact(env, name):
    torch, lbf = env
    W = TENSORS[name]
    say("decode %s %s" % (name, W.shape))
    blob = lbf.from_host_blob(O.encode(W))
    out = lbf.decode(blob)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), W)


@pytest.mark.parametrize("name", sorted(TENSORS))
def test_encode_blob_equals_oracle(env, name):
    torch, lbf = env
    W = TENSORS[name]
    say("encode %s %s" % (name, W.shape))
    b = lbf.encode(dev(torch, W))
    torch.cuda.synchronize()
    ref = O.encode(W)
    got = b.data.cpu().numpy()
    assert got.size == ref.size
    assert np.array_equal(got, ref)
    assert np.array_equal(O.decode(got), W)  # the oracle decodes the GPU's blob


def test_encode_decode_empty(env):
    torch, lbf = env
    W = np.zeros((0, 1024), dtype=np.uint16)
    b = lbf.encode(torch.zeros((0, 1024), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(b.data.cpu().numpy(), O.encode(W))
    assert lbf.decode(b).shape == (0, 1024)


@pytest.mark.parametrize("name", ["ragged_7x333", "half_edges_3x1000"])
def test_decode_leaves_neighbours_untouched(env, name):
    torch, lbf = env
    W = TENSORS[name]
    blob = lbf.from_host_blob(O.encode(W))
    n = W.size
    guard = 4096
    buf = torch.full((guard + n + guard,), -12345, dtype=torch.int16, device="cuda")
    out = buf[guard:guard + n].view(torch.bfloat16).view(*W.shape)
    lbf.decode(blob, out=out)
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert (h[:guard] == -12345).all() and (h[guard + n:] == -12345).all()
    assert np.array_equal(h[guard:guard + n].view(np.uint16).reshape(W.shape), W)


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 8])
def test_gemv_single_tensor(env, batch):
    torch, lbf = env
    W, x1 = synth.single_tensor()
    x = x1 if batch == 1 else synth.activations(np.random.default_rng([0, 1, batch]), batch, 1024)
    say("gemv single_tensor B=%d" % batch)
    blob = lbf.from_host_blob(O.encode(W))
    y_ref, a_ref = O.matvec(W, x)
    y = lbf.gemv(blob, dev(torch, x), lbf.LBF_F32)
    torch.cuda.synchronize()
    check_product(y, y_ref, a_ref, False)
    yb = lbf.gemv(blob, dev(torch, x), lbf.LBF_BF16)
    torch.cuda.synchronize()
    check_product(yb, y_ref, a_ref, True)


def test_gemv_one_hot_extracts_column_exactly(env):
    torch, lbf = env
    W = TENSORS["laplace_128x2048"]
    blob = lbf.from_host_blob(O.encode(W))
    x = np.zeros((8, 2048), dtype=np.uint16)
    ks = [0, 1, 15, 16, 1023, 1024, 2000, 2047]
    for b, k in enumerate(ks):
        x[b, k] = 0x3F80
    y = lbf.gemv(blob, dev(torch, x), lbf.LBF_F32)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for b, k in enumerate(ks):
        assert np.array_equal(y[b], synth.bf16_to_f32(W[:, k])), k


def test_gemv_deterministic(env):
    torch, lbf = env
    W = synth.layer_tensor(1)
    x = synth.layer_x(1, 4)
    blob = lbf.encode(dev(torch, W))
    xs = dev(torch, x)
    y1 = lbf.gemv(blob, xs).cpu().numpy()
    y2 = lbf.gemv(blob, xs).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_gemv_nonfinite_all_patterns(env):
    torch, lbf = env
    W = synth.all_patterns(1536, 4096)
    x = synth.expert_x(63)
    say("gemv all-patterns expert B=4")
    blob = lbf.encode(dev(torch, W))
    y_ref, a_ref = O.matvec(W, x)
    y = lbf.gemv(blob, dev(torch, x))
    torch.cuda.synchronize()
    check_product(y, y_ref, a_ref, False)


def test_gemv_layer_grouped_full(env):
    """One 8B-shaped layer (7 tensors) in one grouped launch, every output checked."""
    torch, lbf = env
    t0 = time.time()
    Ws = [synth.layer_tensor(m) for m in range(len(synth.LAYER))]
    xs = [synth.layer_x(m) for m in range(len(synth.LAYER))]
    say("layer generated in %.1fs" % (time.time() - t0))
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    # the GPU blob of the largest tensor equals the oracle's, byte for byte
    ref = O.encode(Ws[synth.GATE])
    assert np.array_equal(blobs[synth.GATE].data.cpu().numpy(), ref)
    ys = lbf.gemv(blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for m, (W, x, y) in enumerate(zip(Ws, xs, ys)):
        y_ref, a_ref = O.matvec(W, x)
        check_product(y, y_ref, a_ref, False)
        say("layer %s ok" % synth.LAYER[m][0])
    # standalone decode of every tensor is bit-exact
    for W, b in zip(Ws, blobs):
        assert np.array_equal(host(lbf.decode(b)), W)


@pytest.mark.parametrize("layer", [0, 31])
def test_gemv_model_layer_sampled(env, layer):
    """A layer of the full 32-layer weight set (per-tensor sigma ~ U(0.01, 0.05)):
    GPU blobs equal the oracle's for k and v, the grouped batch-1 GEMV matches
    the oracle on row ranges at the start, middle and end of every tensor."""
    torch, lbf = env
    t0 = time.time()
    Ws = [synth.model_tensor(layer, m) for m in range(len(synth.LAYER))]
    xs = [synth.model_x(layer, m) for m in range(len(synth.LAYER))]
    say("model layer %d generated in %.1fs" % (layer, time.time() - t0))
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    for m in (1, 2):
        assert np.array_equal(blobs[m].data.cpu().numpy(), O.encode(Ws[m])), m
    ys = lbf.gemv(blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for W, x, y in zip(Ws, xs, ys):
        R = W.shape[0]
        for r0 in (0, R // 2 - 64, R - 128):
            y_ref, a_ref = O.matvec(W, x, rows=(r0, r0 + 128))
            check_product(y[:, r0:r0 + 128], y_ref, a_ref, False)


def test_gemv_gate_batch_sweep(env):
    torch, lbf = env
    W = synth.layer_tensor(synth.GATE)
    blob = lbf.encode(dev(torch, W))
    for batch in (1, 2, 4, 8):
        x = synth.gate_batch_x(batch)
        y_ref, a_ref = O.matvec(W, x, rows=(0, 14336))
        yb = lbf.gemv(blob, dev(torch, x), lbf.LBF_BF16)
        yf = lbf.gemv(blob, dev(torch, x), lbf.LBF_F32)
        torch.cuda.synchronize()
        check_product(yb, y_ref, a_ref, True)
        check_product(yf, y_ref, a_ref, False)
        say("gate sweep B=%d ok" % batch)


def test_gemv_experts_grouped(env):
    """64 expert tensors (escape-rate stress) at batch 4, grouped launches."""
    torch, lbf = env
    t0 = time.time()
    Ws = [synth.expert_tensor(e) for e in range(64)]
    xs = [synth.expert_x(e) for e in range(64)]
    say("experts generated in %.1fs" % (time.time() - t0))
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    for e in (0, 3, 4, 62, 63):
        assert np.array_equal(blobs[e].data.cpu().numpy(), O.encode(Ws[e])), e
    ys = lbf.gemv(blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for e in range(64):
        y_ref, a_ref = O.matvec(Ws[e], xs[e])
        check_product(ys[e], y_ref, a_ref, False)
    for e in (4, 62, 63):
        assert np.array_equal(host(lbf.decode(blobs[e])), Ws[e]), e


@pytest.mark.parametrize("rows,cols,batch", [(1, 1024, 1), (5, 3072, 2), (7, 14336, 8), (33, 5120, 3),
                                             (130, 2048, 4), (3, 30720, 1)])
def test_gemv_odd_shapes(env, rows, cols, batch):
    torch, lbf = env
    rng = np.random.default_rng([5, rows, cols])
    W = synth.gaussian(rng, rows, cols, 0.03, 0.003, 80.0)
    x = synth.activations(rng, batch, cols)
    say("gemv odd shape %dx%d B=%d" % (rows, cols, batch))
    blob = lbf.from_host_blob(O.encode(W))
    y_ref, a_ref = O.matvec(W, x)
    guard = 256
    buf = torch.full((batch * rows + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    y = buf[guard:guard + batch * rows].view(batch, rows)
    lbf.gemv(blob, dev(torch, x), lbf.LBF_F32, outs=y)
    torch.cuda.synchronize()
    check_product(y, y_ref, a_ref, False)
    h = buf.cpu().numpy()
    assert (h[:guard] == 7.0).all() and (h[guard + batch * rows:] == 7.0).all()


def test_gemv_many_groups_mixed_shapes(env):
    """More groups than one launch takes, with mixed shapes and both table kinds."""
    torch, lbf = env
    rng = np.random.default_rng(77)
    Ws, xs = [], []
    for g in range(40):
        rows = int(rng.integers(1, 300))
        cols = 1024 * int(rng.integers(1, 9))
        if g % 3 == 0:
            W = synth.gaussian(rng, rows, cols, 0.02, 0.002, 100.0)
        elif g % 3 == 1:
            W = synth.laplace(rng, rows, cols, 0.05)
        else:
            W = synth.all_patterns(rows, cols)
        Ws.append(W)
        xs.append(synth.activations(rng, 2, cols))
    blobs = [lbf.from_host_blob(O.encode(W)) for W in Ws]
    ys = lbf.gemv(blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for W, x, y in zip(Ws, xs, ys):
        y_ref, a_ref = O.matvec(W, x)
        check_product(y, y_ref, a_ref, False)


@pytest.mark.parametrize("batch", [1, 2])
def test_gemv_tiny_groups_share_x(env, batch):
    """31 one-row tensors sharing one x tensor, then a 300 x 30720 tensor, in
    one grouped call: outputs of tensors that share an x and of a tensor with
    a 60 KB (batch 1) or 120 KB (batch 2) x all match the oracle."""
    torch, lbf = env
    rng = np.random.default_rng([9, batch])
    Ws = [synth.gaussian(rng, 1, 1024, 0.02, 0.01, 100.0) for _ in range(31)]
    Ws.append(synth.gaussian(rng, 300, 30720, 0.02, 0.002, 100.0))
    xs_small = dev(torch, synth.activations(rng, batch, 1024))
    x_big = synth.activations(rng, batch, 30720)
    blobs = [lbf.from_host_blob(O.encode(W)) for W in Ws]
    ys = lbf.gemv(blobs, [xs_small] * 31 + [dev(torch, x_big)], lbf.LBF_F32)
    torch.cuda.synchronize()
    x_small = host(xs_small)
    for W, y in zip(Ws[:31], ys[:31]):
        y_ref, a_ref = O.matvec(W, x_small)
        check_product(y, y_ref, a_ref, False)
    y_ref, a_ref = O.matvec(Ws[31], x_big)
    check_product(ys[31], y_ref, a_ref, False)


@pytest.mark.parametrize("batch", [3, 8])
def test_gemv_teams_x_over_lds(env, batch):
    """Tensors whose x arrays together pass the 128 KiB LDS x area, so the
    call is split into teams of CUs that each stage only their tensors' x:
    mixed widths and row counts (one-row tensors: teams with fewer rows than
    CUs), one x array shared by tensors that land in different teams, an
    escape-dense all-patterns tensor.  Every output matches the oracle."""
    torch, lbf = env
    rng = np.random.default_rng([31, batch])
    shapes = [(200, 8192), (1, 8192), (150, 4096), (37, 8192), (1, 1024), (90, 6144), (64, 8192), (3, 2048),
              (120, 8192), (45, 5120)]
    Ws, xs = [], []
    shared = synth.activations(rng, batch, 8192)
    for i, (rows, cols) in enumerate(shapes):
        Ws.append(synth.all_patterns(rows, cols) if i == 6 else synth.gaussian(rng, rows, cols, 0.02, 0.003, 100.0))
        xs.append(shared if cols == 8192 and i % 3 == 0 else synth.activations(rng, batch, cols))
    say("gemv teams, B=%d, %d KiB of x" % (batch, sum(x.nbytes for x in xs) // 1024))
    blobs = [lbf.from_host_blob(O.encode(W)) for W in Ws]
    xd = {}
    ys = lbf.gemv(blobs, [xd.setdefault(id(x), dev(torch, x)) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for W, x, y in zip(Ws, xs, ys):
        y_ref, a_ref = O.matvec(W, x)
        check_product(y, y_ref, a_ref, False)


@pytest.mark.parametrize("batch", [1, 3, 8])
def test_gemv_same_x_pointer_different_widths(env, batch):
    """Two groups given the same x pointer with different column counts read
    different [batch, cols] views of that memory (row stride = cols), so the
    launcher must not stage them as one x; a third group shares the first
    group's x exactly.  Every output matches the oracle on its own view."""
    torch, lbf = env
    rng = np.random.default_rng([98, batch])
    Wa = synth.gaussian(rng, 37, 1024, 0.02, 0.002, 100.0)
    Wb = synth.gaussian(rng, 29, 2048, 0.02, 0.002, 100.0)
    Wc = synth.gaussian(rng, 18, 1024, 0.02, 0.002, 100.0)
    flat = synth.activations(rng, 1, batch * 2048).reshape(-1)
    xt = dev(torch, flat.reshape(batch, 2048))
    xa = xt.view(-1)[: batch * 1024].view(batch, 1024)  # same pointer, 1024-column view
    say("gemv same x pointer, widths 1024/2048, B=%d" % batch)
    blobs = [lbf.from_host_blob(O.encode(W)) for W in (Wa, Wb, Wc)]
    ys = lbf.gemv(blobs, [xa, xt, xa], lbf.LBF_F32)
    torch.cuda.synchronize()
    for W, y, x in ((Wa, ys[0], flat[: batch * 1024].reshape(batch, 1024)), (Wb, ys[1], flat.reshape(batch, 2048)),
                    (Wc, ys[2], flat[: batch * 1024].reshape(batch, 1024))):
        y_ref, a_ref = O.matvec(W, x)
        check_product(y, y_ref, a_ref, False)


@pytest.mark.parametrize("batch,cols", [(2, 32768), (4, 16384), (8, 8192)])
def test_gemv_x_at_the_lds_limit(env, batch, cols):
    """One tensor whose x is exactly 128 KiB, the most the ring kernel
    stages in LDS, and the same tensor grouped with a second one of 1024
    columns (x no longer fits: the static kernel): both match the oracle."""
    torch, lbf = env
    rng = np.random.default_rng([97, batch])
    W = synth.gaussian(rng, 24, cols, 0.02, 0.002, 100.0)
    W2 = synth.gaussian(rng, 16, 1024, 0.02, 0.002, 100.0)
    x = synth.activations(rng, batch, cols)
    x2 = synth.activations(rng, batch, 1024)
    say("gemv x at the LDS limit B=%d cols=%d" % (batch, cols))
    b, b2 = lbf.from_host_blob(O.encode(W)), lbf.from_host_blob(O.encode(W2))
    y_ref, a_ref = O.matvec(W, x)
    y = lbf.gemv(b, dev(torch, x), lbf.LBF_F32)
    torch.cuda.synchronize()
    check_product(y, y_ref, a_ref, False)
    ys = lbf.gemv([b, b2], [dev(torch, x), dev(torch, x2)], lbf.LBF_F32)
    torch.cuda.synchronize()
    check_product(ys[0], y_ref, a_ref, False)
    y2_ref, a2_ref = O.matvec(W2, x2)
    check_product(ys[1], y2_ref, a2_ref, False)


@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_layer_twice_static_kernel(env, batch):
    """The layer's seven tensors twice in one call, each time with its own x
    (14 distinct x arrays: 152 KB at batch 1, too much for LDS, so the static
    kernel runs, with 4- and 14-tile rows mixed): row ranges at the start,
    middle and end of every output match the oracle."""
    torch, lbf = env
    Ws = [synth.layer_tensor(m) for m in range(len(synth.LAYER))]
    blobs = [lbf.encode(dev(torch, W)) for W in Ws]
    rng = np.random.default_rng([11, batch])
    xs = [synth.activations(rng, batch, W.shape[1]) for W in Ws + Ws]
    ys = lbf.gemv(blobs + blobs, [dev(torch, x) for x in xs], lbf.LBF_F32)
    torch.cuda.synchronize()
    for i, (W, x, y) in enumerate(zip(Ws + Ws, xs, ys)):
        R = W.shape[0]
        for r0 in (0, R // 2 - 64, R - 128):
            y_ref, a_ref = O.matvec(W, x, rows=(r0, r0 + 128))
            check_product(y[:, r0:r0 + 128], y_ref, a_ref, False)
        say("layer twice, batch %d, tensor %d ok" % (batch, i))
