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
