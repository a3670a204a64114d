"""Helpers shared by the GPU test modules (host <-> device bf16, the product
tolerance check)."""
import sys

import numpy as np
import pytest


def say(msg):
    sys.stdout.write("[gpu-parity] %s\n" % msg)
    sys.stdout.flush()


def make_env():
    import torch
    from decode_byte_split_amd import lbf

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lbf.lib()
    return torch, lbf


def dev(torch, a: np.ndarray):
    """uint16 bf16 patterns (numpy) -> torch.bfloat16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def host(t) -> np.ndarray:
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def check_product(y_gpu, y_ref, a_ref, bf16_out):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    fin = np.isfinite(y_ref)
    # non-finite reference entries: same class on the GPU
    assert np.array_equal(np.isnan(y[~fin]), np.isnan(y_ref[~fin]))
    inf = np.isinf(y_ref)
    assert np.array_equal(y[inf], y_ref[inf])
    tol = 1e-3 * a_ref[fin]
    if bf16_out:
        tol = tol + 2.0 ** -8 * np.abs(y_ref[fin])
    err = np.abs(y[fin] - y_ref[fin])
    worst = np.max(err - tol) if err.size else -1
    assert np.all(err <= tol), "max excess %g" % worst
