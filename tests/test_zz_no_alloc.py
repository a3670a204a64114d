"""lbf_encode_noalloc, the encoder entry point that allocates nothing (its
workspace is a device array inside the library), against lbf_encode with a
workspace from the caller, through the C ABI: the same descriptor and the same
blob bytes on calls in a row, each later one on a smaller tensor (the array
keeps the previous call's contents), and the blobs equal the oracle's.  A
tensor too large for the library's array is refused before anything runs."""
import ctypes

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth
from gpu_util import dev, make_env, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    return make_env()


def _encode(torch, lbf, W, noalloc):
    """Both phases through the C ABI; returns (descriptor bytes, blob bytes)."""
    L = lbf.lib()
    rows, cols = W.shape
    w = dev(torch, W)
    s = torch.cuda.current_stream().cuda_stream
    d = lbf.Desc()
    if noalloc:
        rc = L.lbf_encode_noalloc(w.data_ptr(), rows, cols, None, 0, ctypes.byref(d), s)
    else:
        wb = int(L.lbf_encode_work_bytes(rows, cols))
        work = torch.empty(max(wb, 256), dtype=torch.uint8, device="cuda")
        rc = L.lbf_encode(w.data_ptr(), rows, cols, work.data_ptr(), work.numel(), None, 0, ctypes.byref(d), s)
    assert rc == 0, lbf.strerror(rc)
    blob = torch.empty(int(d.blob_bytes), dtype=torch.uint8, device="cuda")
    if noalloc:
        rc = L.lbf_encode_noalloc(w.data_ptr(), rows, cols, blob.data_ptr(), blob.numel(), ctypes.byref(d), s)
    else:
        rc = L.lbf_encode(w.data_ptr(), rows, cols, work.data_ptr(), work.numel(), blob.data_ptr(), blob.numel(),
                          ctypes.byref(d), s)
    assert rc == 0, lbf.strerror(rc)
    torch.cuda.synchronize()
    return d.to_bytes(), blob.cpu().numpy()


def test_noalloc_encode_equals_encode_on_calls_in_a_row(env):
    torch, lbf = env
    rng = np.random.default_rng(41)
    cases = [
        ("gaussian_2048x4096_outliers", synth.gaussian(rng, 2048, 4096, 0.02, 0.001, 100.0)),
        ("patterns_256x256", synth.all_patterns(256, 256)),  # 94 % escapes
        ("ragged_7x333", synth.gaussian(rng, 7, 333, 0.02, 0.01, 100.0)),
        ("one_weight", synth.gaussian(rng, 1, 1, 0.02, 0.0, 1.0)),
    ]
    for name, W in cases:  # each tensor smaller than the one before
        say("noalloc encode %s %s" % (name, W.shape))
        d_ref, b_ref = _encode(torch, lbf, W, noalloc=False)
        d_new, b_new = _encode(torch, lbf, W, noalloc=True)
        assert d_new == d_ref, name
        assert np.array_equal(b_new, b_ref), name
        assert np.array_equal(b_new, O.encode(W)), name


def test_noalloc_encode_refuses_tensors_past_its_array(env):
    torch, lbf = env
    L = lbf.lib()
    d = lbf.Desc()
    w = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    cap = lbf.NOALLOC_SCRATCH_BYTES
    fit = (cap - 1024) // 4  # tiles the array holds besides the histogram
    assert int(L.lbf_encode_work_bytes(fit, 1024)) <= cap < int(L.lbf_encode_work_bytes(fit + 1, 1024))
    # one 1024-weight tile more than that: refused before anything runs
    assert L.lbf_encode_noalloc(w.data_ptr(), fit + 1, 1024, None, 0, ctypes.byref(d), s) == lbf.LBF_E_CAPACITY
    assert L.lbf_encode_noalloc(w.data_ptr(), 1, (fit + 1) * 1024, None, 0, ctypes.byref(d), s) == lbf.LBF_E_CAPACITY
    torch.cuda.synchronize()
    # the entry point still works after the refusals
    W = synth.gaussian(np.random.default_rng(42), 64, 1024, 0.02, 0.001, 100.0)
    assert np.array_equal(_encode(torch, lbf, W, noalloc=True)[1], O.encode(W))
