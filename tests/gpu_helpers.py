"""Shared plumbing of the GPU parity tests: host <-> device copies and the output bar."""
from __future__ import annotations

import numpy as np
import torch

import oracle.pdq_oracle as O

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# The bar for 16-bit outputs, checked against the oracle's binary32 dequant
# y32 (prefill, decode) or binary64 sum y64 (LLM.int8): max relative error
# <= 1e-2 with the denominator floored at 1e-3 * max|y| (near-zero outputs
# carry only absolute error), and mean absolute error <= 1e-3 against that
# reference rounded to the output dtype.
MAX_REL = 1e-2
MAE = 1e-3


def dev(a: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    """A float32 host array (values representable in `dtype`) as a device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(TORCH_DT[dtype]).cuda()


def host(t) -> np.ndarray:
    """A device tensor as a host array (16-bit floats as their bit patterns);
    packed activation codes as their [rows, K] matrix."""
    from w8a8_int8_quantized_absmax_amd import pdq

    if isinstance(t, pdq.Codes):
        return t.unpack()
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def codes_equal(xq, ref: np.ndarray) -> bool:
    """Packed device codes (pdq.Codes) hold exactly the packed image of the
    oracle's [M, K] codes: layout, values and the zero padding."""
    from packing import pack

    assert xq.shape == ref.shape, (xq.shape, ref.shape)
    img = pack(np.asarray(ref, np.int8))
    return bool(np.array_equal(xq.data.detach().cpu().numpy()[:img.size], img))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return O.bf16_bits_to_f32(bits).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def check_16bit(y_bits: np.ndarray, y_ref: np.ndarray, out: str, exact: bool):
    """y_bits: the GPU's 16-bit output bits; y_ref: oracle y32 / y64."""
    y_ref = np.asarray(y_ref, np.float64)
    if out == "bf16":
        got = bf16_to_f64(y_bits)
        ref_rounded_bits = O.to_bf16_bits(y_ref.astype(np.float32))
        ref_rounded = bf16_to_f64(ref_rounded_bits)
    else:
        got = f16_to_f64(y_bits)
        ref_rounded_bits = O.to_f16(y_ref).view(np.uint16)
        ref_rounded = f16_to_f64(ref_rounded_bits)
    assert np.all(np.isfinite(got))
    floor = 1e-3 * max(float(np.abs(y_ref).max()), 1e-30)
    rel = np.abs(got - y_ref) / np.maximum(np.abs(y_ref), floor)
    assert rel.max() <= MAX_REL, f"max rel err {rel.max():.3e}"
    mae = float(np.mean(np.abs(got - ref_rounded)))
    assert mae <= MAE, f"MAE {mae:.3e}"
    if exact:
        # same binary32 operation sequence on both sides: the bits agree
        mism = int(np.count_nonzero(np.asarray(y_bits, np.uint16) != ref_rounded_bits))
        assert mism == 0, f"{mism} of {y_bits.size} outputs differ from the oracle's rounding"


def sample_rows(m: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, size=min(count, m), replace=False).tolist())
    rows.update({0, m - 1})
    return np.array(sorted(rows), np.int64)
