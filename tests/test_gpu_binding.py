"""The Python binding refuses buffers that would let a kernel read or write
past them: wrong-size outputs, truncated blob buffers, one-word outputs too
small, x of the wrong width.  Each case raises before any launch."""
import numpy as np
import pytest

from decode_byte_split_amd import synth
from gpu_util import dev, make_env

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    return make_env()


def test_binding_guards(env):
    torch, lbf = env
    W = synth.gaussian(np.random.default_rng(7), 16, 2048, 0.02, 0.001, 100.0)
    b = lbf.encode(dev(torch, W))
    bf = torch.bfloat16
    with pytest.raises(ValueError):
        lbf.decode(b, out=torch.empty((16, 2047), dtype=bf, device="cuda"))
    with pytest.raises(ValueError):
        lbf.decode(b, out=torch.empty((16, 2048), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        lbf.decode(b, out=torch.empty((2048, 16), dtype=bf, device="cuda").t())  # not contiguous
    short = lbf.Blob(b.desc, b.data[:-256].clone())
    for call in (lambda: lbf.decode(short), lambda: lbf.verify(short), lambda: lbf.hencode(short),
                 lambda: lbf.gemv(short, dev(torch, synth.activations(np.random.default_rng(1), 1, 2048)))):
        with pytest.raises(ValueError):
            call()
    with pytest.raises(ValueError):
        lbf.crc32_into(b.data, torch.empty(0, dtype=torch.int32, device="cuda"))
    x = dev(torch, synth.activations(np.random.default_rng(2), 2, 2048))
    with pytest.raises(ValueError):
        lbf.swiglu(b, b, x[:, :1024].contiguous())
    with pytest.raises(ValueError):
        lbf.swiglu(b, b, x, out=torch.empty((2, 15), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        lbf.gemv([b, b], [x])
    with pytest.raises(ValueError):
        lbf.gemv(b, x, outs=torch.empty((2, 17), dtype=torch.float32, device="cuda"))
    hb = lbf.hencode(b)
    with pytest.raises(ValueError):
        lbf.hdecode(lbf.HBlob(hb.desc, hb.data[:128].clone()))
    # the well-formed calls still work
    assert torch.equal(lbf.decode(b).view(torch.int16).cpu(), torch.from_numpy(W.view(np.int16)))
    assert torch.equal(lbf.hdecode(hb).view(torch.int16).cpu(), torch.from_numpy(W.view(np.int16)))


def test_encode_phase2_with_changed_weights_stays_in_the_blob(env):
    """Phase 1 on weights with few escapes, phase 2 on weights with many more
    (the descriptor and the weights disagree): phase 2 writes nothing outside
    the blob, and lbf_verify flags the blob's index.  Through the C ABI, with
    guard bands on both sides of the blob."""
    import ctypes

    torch, lbf = env
    L = lbf.lib()
    rng = np.random.default_rng(31)
    W1 = synth.gaussian(rng, 64, 2048, 0.02, 0.001, 100.0)  # a few escapes under its own table
    W2 = synth.gaussian(rng, 64, 2048, 0.02, 0.2, 1e4)  # under W1's table: far more escapes
    w1, w2 = dev(torch, W1), dev(torch, W2)
    rows, cols = W1.shape
    wb = int(L.lbf_encode_work_bytes(rows, cols))
    work = torch.empty(wb, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    d = lbf.Desc()
    assert L.lbf_encode(w1.data_ptr(), rows, cols, work.data_ptr(), wb, None, 0, ctypes.byref(d), s) == 0
    assert 0 < d.n_esc < 0.01 * W1.size
    guard = 1 << 16
    n = int(d.blob_bytes)
    buf = torch.full((guard + n + guard,), 0x5A, dtype=torch.uint8, device="cuda")
    blob = buf[guard:guard + n]
    assert L.lbf_encode(w2.data_ptr(), rows, cols, work.data_ptr(), wb, blob.data_ptr(), n, ctypes.byref(d), s) == 0
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert (h[:guard] == 0x5A).all() and (h[guard + n:] == 0x5A).all()
    assert lbf.verify(lbf.Blob(d, blob)) & lbf.VERIFY_INDEX
    # the same call on the unchanged weights gives a clean blob
    assert L.lbf_encode(w1.data_ptr(), rows, cols, work.data_ptr(), wb, blob.data_ptr(), n, ctypes.byref(d), s) == 0
    assert lbf.verify(lbf.Blob(d, blob)) == 0


def test_explicit_stream_orders_after_the_current_stream(env):
    """A non-contiguous x copied on the current stream and used by a product
    on another stream: the product waits for the copy (results equal to the
    same call on the current stream)."""
    torch, lbf = env
    rng = np.random.default_rng(32)
    W = synth.gaussian(rng, 256, 4096, 0.02, 0.001, 100.0)
    b = lbf.encode(dev(torch, W))
    xt = dev(torch, synth.activations(rng, 4096, 3))  # [4096, 3]; its transpose is not contiguous
    ref = lbf.gemv(b, xt.t().contiguous())
    side = torch.cuda.Stream()
    for _ in range(3):
        torch.cuda._sleep(2_000_000)  # keep the current stream busy so a missing wait would show
        y = lbf.gemv(b, xt.t(), stream=side)
        side.synchronize()
        assert torch.equal(y, ref)
