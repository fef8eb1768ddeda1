"""Seeded sweep of random shapes through every linear-layer call, against the oracle.

Each case draws its call (per-token prefill, per-token asymmetric prefill,
static asymmetric decode, static symmetric, static zero-point, LLM.int8),
input dtype, M, N and K (log-uniform; every other group of six cases over
1..3000 rows, 1..5000 channels and K a multiple of 16 up to 6400, the others
over 1024..4096 rows, 2048..6000 channels and K up to 1600, so that both GEMM
kernels run; M * N * K capped so that the oracle's product stays well under a
second), the number of large hidden channels, and whether a bias
is added, from its own seed.  The bar is the one of the other parity tests:
codes, scales, zero points, saturation counts, outlier indices and INT32
accumulators bit for bit, 16-bit outputs within the stated tolerance (and bit
for bit where both sides run the same binary32 sequence), every output
surrounded by sentinel margins.
"""
import math

import numpy as np
import pytest

import oracle.pdq_oracle as O
from w8a8_int8_quantized_absmax_amd import synth
from test_gpu_parity import (decode_case, outlier_case, prefill_asym_case, prefill_case, static_sym_case,
                             zeropoint_case)

pytestmark = pytest.mark.gpu

PATHS = ("prefill", "prefill_asym", "decode", "static_sym", "zeropoint", "int8_outlier")
CASES = 96
MAX_MNK = 2e9


def draw(i: int):
    rng = np.random.default_rng(90000 + i)
    path = PATHS[i % len(PATHS)]
    dtypes = ("f16", "bf16") if path == "int8_outlier" else ("bf16", "f16", "f32")
    dtype = dtypes[int(rng.integers(len(dtypes)))]

    def logu(lo, hi):
        return max(1, int(math.exp(rng.uniform(math.log(lo), math.log(hi)))))

    if (i // len(PATHS)) % 2 == 0:  # any shape: mostly the skinny kernel
        m, n, k = logu(1, 3000), logu(1, 5000), 16 * logu(1, 400)
    else:  # many rows and channels: mostly the tiled GEMM
        m, n, k = logu(1024, 4096), logu(2048, 6000), 16 * logu(1, 100)
    while m * n * k > MAX_MNK:  # shrink the largest dimension
        if m >= n and m * 16 >= k:
            m = max(1, m // 2)
        elif n * 16 >= k:
            n = max(1, n // 2)
        else:
            k = max(16, k // 32 * 16)
    nch = int(rng.integers(0, 7))
    bias = bool(rng.integers(2))
    return path, dtype, m, n, k, nch, bias


def _channels(seed, k, count):
    return synth.choose_channels(seed, k, min(count, k)) if count else np.zeros(0, np.int64)


def test_draws_cover_every_path_and_kernel():
    from w8a8_int8_quantized_absmax_amd import pdq

    draws = [draw(i) for i in range(CASES)]
    assert {d[0] for d in draws} == set(PATHS)
    kernels = {pdq.gemm_kernel(m, n) for _, _, m, n, _, _, _ in draws}
    assert kernels == {"skinny", "tiled"}, kernels


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape(i):
    path, dtype, m, n, k, nch, with_bias = draw(i)
    seed = 91000 + 10 * i
    print(f"case {i}: {path} {dtype} M={m} N={n} K={k} channels={nch} bias={with_bias}", flush=True)
    ch = _channels(seed, k, nch)
    w = synth.weights(seed + 1, n, k, dtype)
    b = synth.bias(seed + 2, n) if with_bias else None
    if path == "prefill":
        x = synth.activations(seed + 3, m, k, ch, 100.0, dtype=dtype)
        prefill_case(x, w, dtype, bias=b)
    elif path == "prefill_asym":
        x = synth.activations(seed + 3, m, k, ch, 100.0, offset=0.3, dtype=dtype)
        prefill_asym_case(x, w, dtype, bias=b)
    elif path == "decode":
        cal = [synth.activations(seed + 4 + j, 32, k, ch, 100.0, offset=0.1, dtype=dtype) for j in range(3)]
        _, s, z = O.calibrate(cal)
        x = synth.activations(seed + 3, m, k, ch, 100.0, offset=0.1, dtype=dtype)
        decode_case(x, w, dtype, s, z, bias=b)
    elif path == "static_sym":
        cal = [synth.activations(seed + 4 + j, 32, k, ch, 8.0, dtype=dtype) for j in range(3)]
        _, s = O.calibrate_absmax(cal)
        x = synth.activations(seed + 3, m, k, ch, 20.0, dtype=dtype)
        static_sym_case(x, w, dtype, s, bias=b)
    elif path == "zeropoint":
        cal = [synth.activations(seed + 4 + j, 32, k, ch, 8.0, offset=0.5, dtype=dtype) for j in range(3)]
        _, s, z = O.calibrate_zeropoint(cal)
        x = synth.activations(seed + 3, m, k, ch, 20.0, offset=0.5, dtype=dtype)
        zeropoint_case(x, w, dtype, s, z, bias=b)
    else:
        x = synth.normal(seed + 3, (m, k))
        cols = _channels(seed + 5, k, min(8, max(1, k // 4)))
        x[:, cols] = synth.normal(seed + 6, (m, len(cols)), 60.0)
        x = synth.round_to(x, dtype)
        outlier_case(x, w, dtype, 6.0, bias=b)
