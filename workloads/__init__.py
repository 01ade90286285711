"""Seeded synthetic inputs for the FP4 quantized linear layer.

This module only draws random matrices. It holds none of the method's
arithmetic (no quantile, no clamp, no quantizer, no product), so both the CPU
oracle and the HIP path can take their inputs from it.

The inputs stand in for LLaMA training activations and weights: the FP4
training paper (arXiv 2501.17116, news write-up "微软首创FP4训练框架") says
hidden activations are long-tailed with a few channels far larger than the
rest. No dataset or trained checkpoint is used; every value comes from
``numpy.random.default_rng(seed)``, drawn in the order written below.

Recipe per workload:
  * A: N(0,1) or Student-t(3), drawn as float32 (t(3) drawn in float64 and
    rounded to float32), then ``n_out = max(1, round(0.001*K))`` columns
    (chosen without replacement) multiplied by the outlier factor; the tiny
    workload uses 4 columns x30 instead.
  * W: N(0, 0.02^2) drawn as float32.
  * dY (dgrad workload): N(0, 1e-3^2) drawn as float32.
  * bf16 workloads round the float32 draws to bfloat16, round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite; NaN handling is not needed for generated data.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Matrix:
    """A host matrix as the library receives it.

    ``bits`` holds the raw storage (float32 array, or uint16 bfloat16 bits);
    ``f32`` is the exact float32 widening of it (identical for float32).
    """
    dtype: str
    bits: np.ndarray

    @property
    def f32(self) -> np.ndarray:
        if self.dtype == F32:
            return self.bits
        return bf16_bits_to_f32(self.bits)

    @property
    def shape(self):
        return self.bits.shape


def _as_dtype(x32: np.ndarray, dtype: str) -> Matrix:
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == F32:
        return Matrix(F32, x32)
    return Matrix(BF16, f32_to_bf16_bits(x32))


def outlier_channel_count(K: int) -> int:
    """0.1% of the input channels, at least one."""
    return max(1, int(round(0.001 * K)))


def draw_activation(rng: np.random.Generator, M: int, K: int, dist: str,
                    n_out: int, factor: float) -> np.ndarray:
    """Float32 activation matrix with ``n_out`` outlier channels scaled by ``factor``."""
    if dist == "normal":
        a = rng.standard_normal((M, K), dtype=np.float32)
    elif dist == "t3":
        a = rng.standard_t(3.0, size=(M, K)).astype(np.float32)
    else:
        raise ValueError(dist)
    cols = rng.choice(K, size=n_out, replace=False)
    a[:, cols] *= np.float32(factor)
    return a


def draw_weight(rng: np.random.Generator, K: int, N: int, std: float = 0.02) -> np.ndarray:
    w = rng.standard_normal((K, N), dtype=np.float32)
    w *= np.float32(std)
    return w


@dataclasses.dataclass
class Layer:
    """One linear layer problem: Y = f(A, W) with clamp quantile q."""
    name: str
    A: Matrix
    W: Matrix
    q: float

    @property
    def M(self):
        return self.A.shape[0]

    @property
    def K(self):
        return self.A.shape[1]

    @property
    def N(self):
        return self.W.shape[1]


# Workload table: (name, M, K, N, A distribution, outlier factor, tiny-style
# outlier count or None for 0.1% of K, quantile, dtype)
_SPECS = {
    "tiny": dict(M=256, K=512, N=512, dist="normal", factor=30.0, n_out=4, q=0.99, dtype=F32),
    "llama1.3b_ffn_up": dict(M=4096, K=2048, N=5632, dist="normal", factor=50.0, n_out=None, q=0.99, dtype=BF16),
    "llama7b_ffn_up": dict(M=8192, K=4096, N=11008, dist="t3", factor=50.0, n_out=None, q=0.99, dtype=BF16),
    "llama13b_ffn_up": dict(M=8192, K=5120, N=13824, dist="t3", factor=50.0, n_out=None, q=0.999, dtype=BF16),
    "llama13b_ffn_down": dict(M=8192, K=13824, N=5120, dist="t3", factor=50.0, n_out=None, q=0.999, dtype=BF16),
    "llama13b_qkv": dict(M=16384, K=5120, N=15360, dist="t3", factor=50.0, n_out=None, q=0.99, dtype=BF16),
}

WORKLOADS = tuple(_SPECS)


def spec(name: str) -> dict:
    return dict(_SPECS[name])


def make_layer(name: str, seed: int = 0, M: Optional[int] = None) -> Layer:
    """Draw workload ``name``. ``M`` optionally overrides the token count
    (a row sample of the same distribution, used for bounded CPU timing)."""
    s = spec(name)
    rng = np.random.default_rng(seed)
    m = s["M"] if M is None else int(M)
    K, N = s["K"], s["N"]
    n_out = s["n_out"] if s["n_out"] is not None else outlier_channel_count(K)
    a = draw_activation(rng, m, K, s["dist"], n_out, s["factor"])
    w = draw_weight(rng, K, N)
    return Layer(name, _as_dtype(a, s["dtype"]), _as_dtype(w, s["dtype"]), s["q"])


def make_13b_pair(seed: int = 0):
    """The 13B FFN up/down pair: both layers from one generator, up first."""
    up = make_layer("llama13b_ffn_up", seed)
    down = make_layer("llama13b_ffn_down", seed + 1)
    return up, down


def make_grad_output(M: int, N: int, seed: int = 0, std: float = 1e-3,
                     dtype: str = BF16) -> Matrix:
    """dY for the dgrad workload: N(0, std^2)."""
    rng = np.random.default_rng(seed + 1000)
    g = rng.standard_normal((M, N), dtype=np.float32)
    g *= np.float32(std)
    return _as_dtype(g, dtype)


def random_matrix(rng: np.random.Generator, M: int, K: int, dtype: str,
                  dist: str = "normal", scale: float = 1.0) -> Matrix:
    """Small generic test matrix."""
    if dist == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(scale)
    elif dist == "t3":
        x = (rng.standard_t(3.0, size=(M, K)) * scale).astype(np.float32)
    else:
        raise ValueError(dist)
    return _as_dtype(x, dtype)


def from_f32(x32: np.ndarray, dtype: str) -> Matrix:
    """Wrap explicit float32 values (rounded to bf16 for ``dtype='bf16'``)."""
    return _as_dtype(x32, dtype)


def all_bf16_values_matrix(rows: int = 256) -> Matrix:
    """Every finite bfloat16 bit pattern exactly once (row-major), padded with
    zeros to fill ``rows`` rows. Used to exercise every input the encoder can see."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    b = b[exp != 0xFF]  # drop Inf/NaN: inputs are finite by contract
    K = int(math.ceil(b.size / rows))
    out = np.zeros(rows * K, dtype=np.uint16)
    out[: b.size] = b
    return Matrix(BF16, out.reshape(rows, K))
