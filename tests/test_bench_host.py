"""Host-side pieces of bench.py that run without a GPU: the CPU oracle
baseline on one core and in several processes at once."""
import numpy as np

import bench
from decode_byte_split_amd import synth


def test_cpu_baseline_one_core_and_all_cores():
    rng = np.random.default_rng(3)
    Ws = [synth.gaussian(rng, 64, 1024, 0.02, 0.001, 50.0) for _ in range(2)]
    xs = [synth.activations(rng, 1, 1024) for _ in range(2)]
    r = bench.cpu_baseline(Ws, xs, 0.2, 2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    a = r["all_cores"]
    assert "error" not in a, a
    assert a["cores"] == 2 and a["kind"] == "oracle" and a["value"] > 0


def test_cpu_baseline_legs_one_core_and_all_cores():
    """Extra workloads (decode + matvec at a batch, and encode) timed on one
    core and in two processes."""
    rng = np.random.default_rng(4)
    Ws = [synth.gaussian(rng, 32, 1024, 0.02, 0.001, 50.0)]
    xs = [synth.activations(rng, 1, 1024)]
    W2 = synth.gaussian(rng, 48, 2048, 0.02, 0.01, 100.0)
    legs = {"b4": ("decode + matvec, batch 4", [("dm", W2, synth.activations(rng, 4, 2048))]),
            "enc": ("encode", [("enc", W2), ("enc", Ws[0])])}
    r = bench.cpu_baseline(Ws, xs, 0.1, 2, legs=legs, leg_seconds=0.1)
    assert r["cores"] == 1 and r["value"] > 0
    for name in legs:
        c = r["configs"][name]
        assert c["one_core_GBs"] > 0 and c["all_cores_GBs"] > 0 and c["all_cores"] == 2, c
