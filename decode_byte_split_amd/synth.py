"""Seeded synthetic inputs: BF16 weight tensors and activations.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It holds none of the codec's arithmetic: it only draws numbers
(numpy ``default_rng``, PCG64) and rounds float32 draws to BF16 once, with
round-to-nearest-even.

The shapes are those of one Llama-style 8B decoder layer.  The value
distributions stand in for real checkpoints, which are not available here: a
Gaussian with standard deviation ``sigma`` (or a Laplace law) plus a small
fraction of outliers scaled up by a constant.  Their exponent entropy, about
2.55 bits, sits next to the 2.59-2.64 bits that the meowlab page ("你的 bf16
模型,有 5 個 bit 是廢的", section 一, second table) measured on Qwen3-8B layer
18, and the outlier rates span the 0.03-0.23 % escape rates the setupai page
("GPU 友善 12 位無損 BF16 壓縮格式", key points) reports for large models.

Draw order inside one generator: the normal (or Laplace) matrix, then the
outlier positions (``choice`` without replacement), in that order.
"""
from __future__ import annotations

import math

import numpy as np

# One Llama-style 8B decoder layer: (name, out_features = rows, in_features = cols)
LAYER = (
    ("q_proj", 4096, 4096),
    ("k_proj", 1024, 4096),
    ("v_proj", 1024, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 14336, 4096),
    ("up_proj", 14336, 4096),
    ("down_proj", 4096, 14336),
)
GATE = 4  # index of gate_proj in LAYER
EXPERT_OUTLIER_RATES = (0.0, 0.0003, 0.0023, 0.02, 0.20)


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round finite float32 values to BF16 (nearest, ties to even); uint16 bits."""
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    u = f32.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian(rng: np.random.Generator, rows: int, cols: int, sigma: float, outlier_rate: float,
             outlier_mult: float) -> np.ndarray:
    """bf16(N(0, sigma^2)) with round(rate * n) entries, chosen without
    replacement, multiplied by ``outlier_mult`` in float32 before rounding."""
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(sigma)
    n = rows * cols
    k = int(round(outlier_rate * n))
    if k:
        pos = rng.choice(n, size=k, replace=False)
        flat = w.reshape(-1)
        flat[pos] *= np.float32(outlier_mult)
    return bf16_bits(w)


def laplace(rng: np.random.Generator, rows: int, cols: int, scale: float) -> np.ndarray:
    """bf16(Laplace(0, scale)) drawn in float64, narrowed to float32, then rounded."""
    w = rng.laplace(0.0, scale, size=(rows, cols)).astype(np.float32)
    return bf16_bits(w)


def all_patterns(rows: int, cols: int) -> np.ndarray:
    """Element i (flat, row-major) holds bit pattern i mod 65536: every BF16
    value, NaN payloads, both infinities, both zeros and denormals included."""
    return (np.arange(rows * cols, dtype=np.int64) % 65536).astype(np.uint16).reshape(rows, cols)


def activations(rng: np.random.Generator, batch: int, cols: int) -> np.ndarray:
    """bf16(N(0, 1)) activations, [batch, cols]."""
    return bf16_bits(rng.standard_normal((batch, cols), dtype=np.float32))


# ---- the workloads ------------------------------------------------------------

def single_tensor():
    """1024x1024 weights, N(0, 0.02^2), 0.1 % outliers x100 (seed 0); x [1, 1024]."""
    W = gaussian(np.random.default_rng(0), 1024, 1024, 0.02, 0.001, 100.0)
    x = activations(np.random.default_rng([0, 1]), 1, 1024)
    return W, x


def layer_tensor(m: int) -> np.ndarray:
    """Matrix m of one 8B-shaped layer: N(0, 1/fan_in), 0.03 % outliers x50."""
    _, rows, cols = LAYER[m]
    return gaussian(np.random.default_rng([1, 0, m]), rows, cols, 1.0 / math.sqrt(cols), 0.0003, 50.0)


def layer_x(m: int, batch: int = 1) -> np.ndarray:
    _, _, cols = LAYER[m]
    return activations(np.random.default_rng([1, 0, m, 1]), batch, cols)


def gate_batch_x(batch: int) -> np.ndarray:
    """Activations for the gate_proj batch sweep, [batch, 4096]."""
    return activations(np.random.default_rng([2, batch, 1]), batch, 4096)


def model_tensor(layer: int, m: int) -> np.ndarray:
    """Matrix m of layer ``layer`` of the 32-layer weight set: sigma ~ U(0.01, 0.05)
    drawn first from the same generator, then as ``layer_tensor``."""
    _, rows, cols = LAYER[m]
    rng = np.random.default_rng([3, layer, m])
    sigma = float(rng.uniform(0.01, 0.05))
    return gaussian(rng, rows, cols, sigma, 0.0003, 50.0)


def model_x(layer: int, m: int) -> np.ndarray:
    _, _, cols = LAYER[m]
    return activations(np.random.default_rng([3, layer, m, 1]), 1, cols)


def expert_tensor(e: int, rows: int = 1536, cols: int = 4096) -> np.ndarray:
    """Expert e of 64: Gaussian sigma 0.02 with outlier rate
    EXPERT_OUTLIER_RATES[e % 5] x100 for e < 62; Laplace(0, 0.02) for e = 62;
    every BF16 pattern tiled for e = 63."""
    if e == 63:
        return all_patterns(rows, cols)
    rng = np.random.default_rng([4, e])
    if e == 62:
        return laplace(rng, rows, cols, 0.02)
    return gaussian(rng, rows, cols, 0.02, EXPERT_OUTLIER_RATES[e % 5], 100.0)


def expert_x(e: int, batch: int = 4, cols: int = 4096) -> np.ndarray:
    return activations(np.random.default_rng([4, e, 1]), batch, cols)
