"""GPU parity of the fused gate/up product with its SiLU·mul epilogue
(lbf_gemv_swiglu) against the oracle's float64 SwiGLU.

Bound: the GPU's g and u each meet the GEMV bar |e| <= 1e-3 * sum|w||x|
(eps_g, eps_u); silu is Lipschitz with constant < 1.1 (its slope peaks at
1.0998 near z = 2.4), so
    |h_gpu - h| <= 1.1 eps_g (|u| + eps_u) + |silu(g)| eps_u + 1e-5 |silu(g)| (|u| + eps_u),
the last term covering the float32 exponential, division and product.  A
bf16 output adds half a bf16 ulp (2^-8 relative) of the result."""
import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth
from gpu_util import dev, make_env, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    return make_env()


def check_h(h_gpu, ref, bf16_out):
    h, g, u, ag, au = ref
    got = h_gpu.float().cpu().numpy().astype(np.float64)
    eg, eu = 1e-3 * ag, 1e-3 * au
    sg = np.abs(g / (1.0 + np.exp(-g)))
    tol = 1.1 * eg * (np.abs(u) + eu) + sg * eu + 1e-5 * sg * (np.abs(u) + eu) + 1e-30
    if bf16_out:
        tol = tol + 2.0 ** -8 * (np.abs(h) + tol)
    err = np.abs(got - h)
    assert np.all(err <= tol), "max excess %g" % np.max(err - tol)


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_swiglu_small(env, batch, bf16_out):
    torch, lbf = env
    rng = np.random.default_rng([95, batch])
    rows, cols = 67, 3072
    G = synth.gaussian(rng, rows, cols, 1 / 55, 0.001, 50.0)
    U = synth.gaussian(rng, rows, cols, 1 / 55, 0.001, 50.0)
    x = synth.activations(rng, batch, cols)
    gb, ub = lbf.encode(dev(torch, G)), lbf.encode(dev(torch, U))
    h = lbf.swiglu(gb, ub, dev(torch, x), lbf.LBF_BF16 if bf16_out else lbf.LBF_F32)
    check_h(h, O.swiglu(G, U, x), bf16_out)


def test_swiglu_x_at_the_lds_limit(env):
    """x of exactly 128 KiB (batch 8 x 8192 columns), the largest the fused
    launch stages in LDS, and one column more is refused."""
    torch, lbf = env
    rng = np.random.default_rng(96)
    rows, cols = 40, 8192
    G = synth.gaussian(rng, rows, cols, 1 / 90, 0.002, 50.0)
    U = synth.gaussian(rng, rows, cols, 1 / 90, 0.002, 50.0)
    x = synth.activations(rng, 8, cols)
    gb, ub = lbf.encode(dev(torch, G)), lbf.encode(dev(torch, U))
    h = lbf.swiglu(gb, ub, dev(torch, x), lbf.LBF_F32)
    check_h(h, O.swiglu(G, U, x), False)
    W2 = synth.gaussian(rng, 8, cols + 1024, 1 / 90, 0.002, 50.0)
    b2 = lbf.encode(dev(torch, W2))
    with pytest.raises(lbf.LbfError) as refused:
        lbf.swiglu(b2, b2, dev(torch, synth.activations(rng, 8, cols + 1024)), lbf.LBF_F32)
    assert refused.value.status == lbf.LBF_E_UNSUPPORTED


def test_swiglu_one_hot_columns(env):
    torch, lbf = env
    rng = np.random.default_rng(96)
    G = synth.gaussian(rng, 40, 2048, 0.5, 0.0, 1.0)
    U = synth.gaussian(rng, 40, 2048, 0.5, 0.0, 1.0)
    x = np.zeros((2, 2048), dtype=np.uint16)
    x[0, 5] = 0x3F80
    x[1, 2047] = 0x3F80
    h = lbf.swiglu(lbf.encode(dev(torch, G)), lbf.encode(dev(torch, U)), dev(torch, x)).cpu().numpy()
    for b, k in ((0, 5), (1, 2047)):
        gk = synth.bf16_to_f32(G[:, k]).astype(np.float64)
        uk = synth.bf16_to_f32(U[:, k]).astype(np.float64)
        ref = gk / (1 + np.exp(-gk)) * uk
        assert np.allclose(h[b], ref, rtol=2e-6, atol=1e-30)


def test_swiglu_outlier_and_escape_heavy(env):
    torch, lbf = env
    rng = np.random.default_rng(97)
    G = synth.gaussian(rng, 33, 4096, 0.02, 0.2, 100.0)  # 20 % outliers: many escapes
    U = synth.laplace(rng, 33, 4096, 0.02)
    x = synth.activations(rng, 4, 4096)
    h = lbf.swiglu(lbf.encode(dev(torch, G)), lbf.encode(dev(torch, U)), dev(torch, x))
    check_h(h, O.swiglu(G, U, x), False)


def test_swiglu_full_size_gate_up_sampled(env):
    # the 8B-shaped layer's gate_proj / up_proj (14336 x 4096) at batch 1, the
    # launch the layer step uses; 256 sampled rows checked against the oracle
    torch, lbf = env
    G = synth.layer_tensor(synth.GATE)
    U = synth.layer_tensor(synth.GATE + 1)
    x = synth.layer_x(synth.GATE)
    h = lbf.swiglu(lbf.encode(dev(torch, G)), lbf.encode(dev(torch, U)), dev(torch, x), lbf.LBF_BF16)
    rows = np.sort(np.random.default_rng(98).choice(G.shape[0], 256, replace=False))
    rows[0], rows[-1] = 0, G.shape[0] - 1
    ref = O.swiglu(np.ascontiguousarray(G[rows]), np.ascontiguousarray(U[rows]), x)
    check_h(h[:, rows], ref, True)
    say("swiglu gate/up 14336x4096 batch 1: 256 sampled rows within the bound")


def test_swiglu_matches_unfused_components(env):
    # the same wave-level sums as the plain grouped GEMV: recombining the
    # unfused g and u on the host lands within float32 rounding of the fused h
    torch, lbf = env
    rng = np.random.default_rng(99)
    G = synth.gaussian(rng, 300, 4096, 1 / 64, 0.0003, 50.0)
    U = synth.gaussian(rng, 300, 4096, 1 / 64, 0.0003, 50.0)
    x = dev(torch, synth.activations(rng, 2, 4096))
    gb, ub = lbf.encode(dev(torch, G)), lbf.encode(dev(torch, U))
    h = lbf.swiglu(gb, ub, x).cpu().numpy().astype(np.float64)
    g, u = [y.cpu().numpy().astype(np.float64) for y in lbf.matmul([gb, ub], [x, x], lbf.LBF_F32)]
    ref = g / (1 + np.exp(-g)) * u
    assert np.allclose(h, ref, rtol=1e-5, atol=1e-12)
