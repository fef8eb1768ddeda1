"""Seeded synthetic workloads for the W8A8 linear layer.

This module only draws random numbers and rounds them to the storage dtype
of each workload; it holds none of the quantization arithmetic.  Both the
CPU oracle (through the tests) and the HIP path (through the binding) are
fed from here, so that they see the identical input bits.

Value distributions follow the pages:
  * activations ~ N(0,1) with a handful of fixed "outlier" hidden channels
    at least 100x larger (LLM.int8() blog, "Emergent Features": about six
    dimensions out of thousands, >=100x magnitude, same dimensions across
    inputs) -- so the recipes scale 6 fixed channels by 100;
  * weights ~ N(0, 0.02) (random init; no trained checkpoint exists here);
  * decode activations carry a +0.1 offset so that the static per-tensor
    range is asymmetric (PDMIX terms entry, section 2.3: decode uses an
    asymmetric per-tensor scale and zero point);
  * 50 calibration batches (PDMIX usage guide, section 2 "Inputs": 50
    calibration samples recommended).

Every array is returned as float32 whose values are exactly representable
in the workload's storage dtype ("f32", "bf16" or "f16"); rounding to the
16-bit dtypes is round-to-nearest-even, done by torch's CPU cast.
"""
from __future__ import annotations

import dataclasses

import numpy as np

DTYPES = ("f32", "bf16", "f16")


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to `dtype` (RNE) and widen back to float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    import torch

    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16).to(torch.float32).numpy()
    if dtype == "f16":
        return t.to(torch.float16).to(torch.float32).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def swiglu_inputs(seed: int, m: int, k: int, dtype: str = "bf16", gate_std: float = 2.0,
                  up_std: float = 1.0):
    """Gate and up projections of a SwiGLU MLP (the two halves of a gate/up GEMM
    output), [m, k] each: independent normals rounded to dtype."""
    return (round_to(normal(seed, (m, k), gate_std), dtype),
            round_to(normal(seed + 1, (m, k), up_std), dtype))


def choose_channels(seed: int, k: int, count: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(k, size=count, replace=False)).astype(np.int64)


def activations(seed: int, m: int, k: int, channels, factor: float = 100.0,
                offset: float = 0.0, dtype: str = "bf16") -> np.ndarray:
    """N(0,1) [+offset], then the listed hidden channels multiplied by `factor`."""
    x = normal(seed, (m, k))
    if offset:
        x += np.float32(offset)
    if len(channels):
        x[:, np.asarray(channels)] *= np.float32(factor)
    return round_to(x, dtype)


def weights(seed: int, n: int, k: int, dtype: str = "bf16", std: float = 0.02) -> np.ndarray:
    return round_to(normal(seed, (n, k), std), dtype)


def bias(seed: int, n: int, std: float = 0.1) -> np.ndarray:
    return normal(seed, (n,), std)


def random_int8(seed: int, shape, lo: int = -128, hi: int = 127) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int8)


# --------------------------------------------------------------------------
# The named workloads.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Tiny:
    """16x256 activations, 512x256 weights, fp32; channels 3 and 77 x50."""
    M: int = 16
    K: int = 256
    N: int = 512
    channels: tuple = (3, 77)
    factor: float = 50.0
    dtype: str = "f32"
    n_calib: int = 8

    def x(self):
        return activations(101, self.M, self.K, self.channels, self.factor, dtype=self.dtype)

    def w(self):
        return weights(102, self.N, self.K, self.dtype)

    def bias(self):
        return bias(103, self.N)

    def calib(self, b: int):
        return activations(110 + b, self.M, self.K, self.channels, self.factor, dtype=self.dtype)


@dataclasses.dataclass(frozen=True)
class Prefill7B:
    """Prefill linear 4096 tokens x (4096 -> 11008), bf16, 6 fixed channels x100."""
    M: int = 4096
    K: int = 4096
    N: int = 11008
    dtype: str = "bf16"

    def channels(self):
        return choose_channels(200, self.K, 6)

    def x(self, rows: int | None = None):
        return activations(201, rows or self.M, self.K, self.channels(), 100.0, dtype=self.dtype)

    def w(self):
        return weights(202, self.N, self.K, self.dtype)


@dataclasses.dataclass(frozen=True)
class Decode:
    """Decode linear 4096 -> 4096, bf16, static per-tensor asym activations.

    Calibration: 50 batches of 512 tokens, N(0,1)+0.1 with 6 channels x100.
    """
    K: int = 4096
    N: int = 4096
    batches: tuple = (1, 8, 32, 64)
    n_calib: int = 50
    calib_tokens: int = 512
    dtype: str = "bf16"

    def channels(self):
        return choose_channels(300, self.K, 6)

    def calib(self, b: int):
        return activations(310 + b, self.calib_tokens, self.K, self.channels(), 100.0,
                           offset=0.1, dtype=self.dtype)

    def x(self, m: int, seed: int | None = None):
        return activations(3000 + m if seed is None else seed, m, self.K, self.channels(), 100.0,
                           offset=0.1, dtype=self.dtype)

    def w(self, copy: int = 0):
        return weights(302 + 1000 * copy, self.N, self.K, self.dtype)


@dataclasses.dataclass(frozen=True)
class LlmInt8:
    """LLM.int8() decomposition: 2048 x (8192 -> 28672), fp16, 8 columns ~N(0,60)."""
    M: int = 2048
    K: int = 8192
    N: int = 28672
    n_outlier_cols: int = 8
    outlier_std: float = 60.0
    threshold: float = 6.0
    dtype: str = "f16"

    def columns(self):
        return choose_channels(400, self.K, self.n_outlier_cols)

    def x(self, rows: int | None = None):
        m = rows or self.M
        x = normal(401, (self.M, self.K))[:m]
        cols = self.columns()
        x[:, cols] = normal(403, (self.M, len(cols)), self.outlier_std)[:m]
        return round_to(x, self.dtype)

    def w(self, rows: int | None = None):
        n = rows or self.N
        return round_to(normal(402, (self.N, self.K), 0.02)[:n], self.dtype)


@dataclasses.dataclass(frozen=True)
class DecoderBlock:
    """One decoder block's linear set at hidden 4096 (32 heads).

    QKV 4096->12288, O 4096->4096, gate+up 4096->28672, down 14336->4096;
    prefill 8192 tokens, then decode steps at batch 32 sharing one INT8 copy.
    """
    hidden: int = 4096
    prefill_tokens: int = 8192
    decode_batch: int = 32
    decode_steps: int = 256
    linears: tuple = (("qkv", 12288, 4096), ("o", 4096, 4096),
                      ("gate_up", 28672, 4096), ("down", 4096, 14336))
    dtype: str = "bf16"

    def channels(self, l: int, k: int):
        return choose_channels(520 + l, k, 6)

    def w(self, l: int):
        _, n, k = self.linears[l]
        return weights(500 + l, n, k, self.dtype)

    def prefill_x(self, l: int, rows: int | None = None):
        _, _, k = self.linears[l]
        return activations(510 + l, rows or self.prefill_tokens, k, self.channels(l, k), 100.0,
                           dtype=self.dtype)

    def calib(self, l: int, b: int):
        _, _, k = self.linears[l]
        return activations(6000 + 100 * l + b, 512, k, self.channels(l, k), 100.0, offset=0.1,
                           dtype=self.dtype)

    def down_gate_up(self, rows: int | None = None):
        """Input of the down projection before the activation: gate and up
        [rows, intermediate] (intermediate = the down projection's K)."""
        _, _, k = self.linears[3]
        return swiglu_inputs(530, rows or self.prefill_tokens, k, self.dtype)

    def decode_x(self, l: int, t: int):
        _, _, k = self.linears[l]
        return activations(700000 + 4 * t + l, self.decode_batch, k, self.channels(l, k), 100.0,
                           offset=0.1, dtype=self.dtype)
