"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check is a value the
pages print (tests/golden/), a closed form, an invariant of the method, a
special case that reduces to a library routine, or brute force in plain
Python integers/floats on tiny inputs.  The last block plants plausible
mistakes into a copy of the oracle and shows that a pin catches each one.
"""
import json
import math
import os
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.pdq_oracle as O
from w8a8_int8_quantized_absmax_amd import synth

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Worked examples printed on the LLM.int8() page
# ---------------------------------------------------------------------------

def check_worked_row(oracle=O):
    g = golden("llm_int8_worked_example.json")
    row = np.array([g["row_regular_values"]], F32)
    q, s = oracle.quantize_rows_absmax(row)
    # C_x = 2 (printed); S = C_x / 127
    assert s[0] == F32(g["row_absmax_C_x"]) / F32(127)
    # absmax formula: round(127 * x / C_x) = round(127, -63.5, 63.5)
    expect = [round(127 * v / g["row_absmax_C_x"]) for v in g["row_regular_values"]]
    assert expect == [127, -64, 64]
    assert q.tolist() == [expect]


def test_worked_example_row_scale():
    check_worked_row()


def test_worked_example_weight_column():
    g = golden("llm_int8_worked_example.json")
    col = np.array([g["weight_column_values"]], F32)  # one output channel of W
    wq, sw, colsum = O.quantize_weight(col)
    assert sw[0] == F32(g["weight_column_absmax"]) / F32(127)
    assert wq.tolist() == [[-64, 0, -127, -64]]
    assert colsum.tolist() == [-255]


def outlier_fixture():
    """The figure's 3-row X: 1st and 3rd columns are the printed outliers.

    Row 1's regular values are the printed [2, -1, 1]; the regular values
    of rows 2 and 3 are not printed and are filled with small numbers here.
    """
    g = golden("llm_int8_worked_example.json")
    c1, c3 = g["outlier_column_magnitudes"]
    r1 = g["row_regular_values"]
    x = np.array([[c1[0], r1[0], c3[0], r1[1], r1[2]],
                  [c1[1], 0.0, c3[1], 3.0, -1.0],
                  [c1[2], -1.0, c3[2], 2.0, 0.0]], F32)
    return x, g


def check_outlier_example(oracle=O):
    x, g = outlier_fixture()
    cols = oracle.outlier_columns(x, g["threshold"])
    assert (cols + 1).tolist() == g["outlier_column_positions_1based"]
    q, s = oracle.quantize_rows_regular(x, cols)
    assert s[0] == F32(g["row_absmax_C_x"]) / F32(127)
    assert q[0].tolist() == [0, 127, 0, -64, 64]
    assert q[:, cols].tolist() == [[0, 0]] * 3


def test_worked_example_outlier_columns():
    check_outlier_example()


def check_threshold_strict(oracle=O):
    x = np.array([[6.0, -6.0, 6.0000005, 1.0]], F32)
    assert oracle.outlier_columns(x, 6.0).tolist() == [2]
    x = np.array([[1.0, -7.0], [-6.5, 0.0]], F32)
    assert oracle.outlier_columns(x, 6.0).tolist() == [0, 1]


def test_outlier_threshold_is_strict():
    check_threshold_strict()


# ---------------------------------------------------------------------------
# Library routines the oracle's primitives must agree with
# ---------------------------------------------------------------------------

def test_rint_is_round_half_even():
    v = np.array([-3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 126.5, -127.5, 2.4999998], F32)
    assert np.rint(v).tolist() == [float(round(float(a))) for a in v]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    y = rng.standard_normal(200000).astype(F32) * F32(37)
    # ties and near-ties: low halves 0x8000, 0x7fff, 0x8001 with both parities
    base = rng.integers(0x3f000000, 0x42000000, 5000, dtype=np.uint32) & np.uint32(0xFFFF0000)
    ties = np.concatenate([base | 0x8000, (base | 0x18000), base | 0x7FFF, base | 0x8001]).view(F32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-40, -1e-40], F32)
    y = np.concatenate([y, ties, special])
    ours = O.to_bf16_bits(y)
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_rounding_matches_torch():
    rng = np.random.default_rng(8)
    y = rng.standard_normal(100000) * 300.0
    ours = O.to_f16(y.astype(F32)).view(np.uint16)
    ref = torch.from_numpy(y.astype(F32)).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# Exact integer contraction and the zero-point (four-term) expansion
# ---------------------------------------------------------------------------

def brute_int_matmul(a, b):
    a = a.astype(int).tolist()
    b = b.astype(int).tolist()
    return [[sum(x * y for x, y in zip(ra, rb)) for rb in b] for ra in a]


def test_int_matmul_brute_force():
    a = synth.random_int8(11, (5, 48))
    b = synth.random_int8(12, (7, 48))
    assert O.int_matmul(a, b).tolist() == brute_int_matmul(a, b)


def test_int_matmul_extremes_exact():
    k = 16384
    a = np.full((2, k), -128, np.int8)
    b = np.full((3, k), -128, np.int8)
    b[1] = 127
    acc = O.int_matmul(a, b)
    assert acc[0, 0] == 128 * 128 * k and acc[1, 1] == -128 * 127 * k
    # a single odd term must survive next to a large sum
    a2 = np.full((1, k), 127, np.int8)
    b2 = np.full((1, k), 127, np.int8)
    b2[0, 5] = 126
    assert O.int_matmul(a2, b2)[0, 0] == 127 * 127 * k - 127


def check_four_term(oracle=O):
    """[LLM.int8] part 1 section 2: sum (a - za)(b - zb) expanded in four terms."""
    k = 40
    a = synth.random_int8(21, (4, k))
    b = synth.random_int8(22, (6, k), -127, 127)
    # general four-term form with za, zb != 0, checked in plain Python ints
    for za, zb in [(3, -5), (-128, 7), (0, 0), (127, -1)]:
        for i in range(4):
            for j in range(6):
                lhs = sum((int(a[i, t]) - za) * (int(b[j, t]) - zb) for t in range(k))
                ab = sum(int(a[i, t]) * int(b[j, t]) for t in range(k))
                rhs = ab - zb * sum(int(v) for v in a[i]) - za * sum(int(v) for v in b[j]) + k * za * zb
                assert lhs == rhs
    # the oracle's specialisation to a symmetric weight (zb = 0)
    colsum = b.astype(np.int64).sum(axis=1)
    for z in (-3, 0, 11, -128, 127):
        got = oracle.zero_point_correct(oracle.int_matmul(a, b), colsum, z)
        want = [[sum((int(a[i, t]) - z) * int(b[j, t]) for t in range(k)) for j in range(6)]
                for i in range(4)]
        assert got.tolist() == want


def test_four_term_zero_point_expansion():
    check_four_term()


def test_weight_colsum_is_code_sum():
    w = synth.weights(31, 9, 64, "f32")
    wq, sw, colsum = O.quantize_weight(w)
    assert colsum.tolist() == [sum(int(v) for v in r) for r in wq]


# ---------------------------------------------------------------------------
# Quantizer bounds and extremes
# ---------------------------------------------------------------------------

def test_symmetric_dequant_error_bound():
    x = synth.activations(41, 64, 512, [3, 100], 100.0, dtype="f32")
    q, s = O.quantize_rows_absmax(x)
    err = np.abs(x.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 2.0**-20))
    # the absmax element of every row reaches +-127 with the sign of x
    idx = np.argmax(np.abs(x), axis=1)
    r = np.arange(x.shape[0])
    assert np.all(q[r, idx] == np.where(x[r, idx] > 0, 127, -127))
    assert q.min() >= -127


def test_asymmetric_calibration_extremes():
    batches = [synth.activations(50 + b, 32, 256, [5], 100.0, offset=0.1, dtype="f32") for b in range(4)]
    (lo, hi), s, z = O.calibrate(batches)
    assert lo < 0 < hi
    assert s == F32(F32(hi - lo) / F32(255))
    xall = np.concatenate(batches)
    q, sat = O.quantize_static(xall, s, z)
    # the range minimum lands exactly on -128; the maximum on 127
    assert q.flat[np.argmin(xall)] == -128
    assert q.flat[np.argmax(xall)] == 127
    # unclamped code of the maximum is 127 or 128 (rounding of both ends)
    r_max = int(np.rint(F32(F32(hi) / s))) + z
    assert r_max in (127, 128)
    assert sat == int(r_max == 128) * int(np.count_nonzero(xall == hi))
    # dequant error bound for every unclamped value
    r = np.rint(xall / s).astype(np.int64) + z
    ok = (r >= -128) & (r <= 127)
    err = np.abs(xall.astype(np.float64) - float(s) * (q.astype(np.float64) - z))
    assert np.all(err[ok] <= float(s) / 2 * (1 + 2.0**-20))


def test_calibration_range_contains_zero():
    pos = [np.full((2, 16), 3.0, F32), np.full((2, 16), 5.0, F32)]
    (lo, hi), s, z = O.calibrate(pos)
    assert (lo, hi) == (3.0, 5.0)
    assert s == F32(F32(5.0) / F32(255)) and z == -128
    q, _ = O.quantize_static(np.zeros((1, 16), F32), s, z)
    assert np.all(q == z)  # 0 is exactly representable
    assert O.minmax_finalize((F32(0), F32(0))) == (1.0, 0)


def test_static_saturation_counting():
    s, z = F32(0.5), -3
    x = np.array([[0.0, 63.0, 64.0, 65.25, -62.0, -63.0, 1e30, -np.inf]], F32)
    q, sat = O.quantize_static(x, s, z)
    # codes: rne(x/S) + Z = -3, 123, 125, 127(130.5->130+(-3)=127), -127, -129, huge, -inf
    assert q.tolist() == [[-3, 123, 125, 127, -127, -128, 127, -128]]
    assert sat == 3


def test_static_round_then_add_zero_point():
    # x/S = 2.5 exactly: rne(2.5) = 2, then + Z (odd) = 3 ; rne(2.5 + 1) would be 4
    q, _ = O.quantize_static(np.array([[1.25]], F32), F32(0.5), 1)
    assert q[0, 0] == 3


def test_identity_quantization_special_case():
    xi = synth.random_int8(61, (3, 32), -127, 127).astype(F32)
    q, sat = O.quantize_static(xi, F32(1), 0)
    assert sat == 0 and np.array_equal(q.astype(F32), xi)
    w = synth.random_int8(62, (5, 32), -127, 127)
    res = O.linear_decode(xi, F32(1), 0, w, np.ones(5, F32), w.astype(np.int64).sum(1))
    assert np.array_equal(res["y32"].astype(np.float64), xi.astype(np.float64) @ w.astype(np.float64).T)


# ---------------------------------------------------------------------------
# Invariances
# ---------------------------------------------------------------------------

def test_sign_and_power_of_two_invariance():
    x = synth.activations(71, 8, 128, [1], 100.0, dtype="f32")
    q, s = O.quantize_rows_absmax(x)
    qn, sn = O.quantize_rows_absmax(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for e in (-3, 5):
        q2, s2 = O.quantize_rows_absmax(x * F32(2.0**e))
        assert np.array_equal(q2, q) and np.array_equal(s2, s * F32(2.0**e))


def test_joint_k_permutation_invariance():
    x = synth.activations(72, 6, 96, [4], 100.0, dtype="f32")
    w = synth.weights(73, 10, 96, "f32")
    wq, sw, _ = O.quantize_weight(w)
    perm = np.random.default_rng(5).permutation(96)
    a = O.linear_prefill(x, wq, sw)
    b = O.linear_prefill(x[:, perm], wq[:, perm], sw)
    assert np.array_equal(a["acc"], b["acc"]) and np.array_equal(a["y32"], b["y32"])


def test_single_token_per_token_equals_per_tensor():
    x = synth.activations(74, 1, 64, [2], 100.0, dtype="f32")
    q, s = O.quantize_rows_absmax(x)
    s_t = O.absmax_scale(np.max(np.abs(x)))
    assert s[0] == s_t and np.array_equal(q, O.quantize_symmetric(x, np.array([s_t], F32)))


def test_calibration_resume_is_exact():
    batches = [synth.activations(80 + b, 16, 64, [7], 100.0, offset=0.1, dtype="f32") for b in range(10)]
    state_all, s_all, z_all = O.calibrate(batches)
    st = None
    for b in batches[:5]:
        st = O.minmax_update(st, b)
    saved = (F32(st[0]), F32(st[1]))
    for b in batches[5:]:
        saved = O.minmax_update(saved, b)
    assert saved == state_all and O.minmax_finalize(saved) == (s_all, z_all)


# ---------------------------------------------------------------------------
# Static tensor-wise symmetric quantization (absmax over calibration batches)
# ---------------------------------------------------------------------------

def check_tensor_absmax(oracle=O):
    """The worked example's values as one tensor: C = 2 over both rows, and the
    page's absmax formula round(127 x / C) (round half to even) gives the codes;
    a value beyond the calibrated magnitude saturates at +-127 and is counted."""
    g = golden("llm_int8_worked_example.json")
    row = g["row_regular_values"]                # [2, -1, 1]
    second = [1, 0.5, -2]                        # filled in by this test, |v| <= C
    x = np.array([row, second], F32)
    _, s = oracle.calibrate_absmax([x[:1], x[1:]])
    assert s == F32(g["row_absmax_C_x"]) / F32(127)
    q, sat = oracle.quantize_static_sym(x, s)
    want = [[round(127 * v / g["row_absmax_C_x"]) for v in r] for r in (row, second)]
    assert want == [[127, -64, 64], [64, 32, -127]] and q.tolist() == want and sat == 0
    q2, sat2 = oracle.quantize_static_sym(np.array([[3.0, -3.0, 2.0, -2.0]], F32), s)
    assert q2.tolist() == [[127, -127, 127, -127]] and sat2 == 2


def test_tensor_absmax_worked_example_and_saturation():
    check_tensor_absmax()


def test_finalize_of_a_state_that_saw_nothing():
    """Reading R8 (an empty range gets S = 1, Z = 0) on all three grids, for a
    fresh observer state {+inf, -inf} (no batch seen) and for a state that saw
    only zeros; the codes on that grid are then all 0.  A planted mistake --
    finalising the fresh state without its empty-state branch -- gives an
    infinite scale."""
    fresh = (F32(np.inf), F32(-np.inf))
    assert O.absmax_finalize(fresh) == F32(1)
    assert O.minmax_finalize(fresh) == (F32(1), 0)
    assert O.zeropoint_finalize(fresh) == (F32(1), 0)
    zeros = O.minmax_update(None, np.zeros((3, 16), F32))
    assert O.absmax_finalize(zeros) == F32(1)
    assert O.minmax_finalize(zeros) == (F32(1), 0) and O.zeropoint_finalize(zeros) == (F32(1), 0)
    q, sat = O.quantize_static_sym(np.zeros((2, 16), F32), O.absmax_finalize(fresh))
    assert not q.any() and sat == 0

    def no_empty_branch(state):
        c = max(abs(F32(state[0])), abs(F32(state[1])))
        return F32(O.absmax_scale(np.array([c], F32))[0])

    assert not np.isfinite(no_empty_branch(fresh))


def test_tensor_absmax_calibration_is_the_largest_magnitude():
    batches = [synth.activations(60 + b, 16, 128, [4], 30.0, offset=0.2, dtype="f32") for b in range(5)]
    batches[3][7, 9] = -500.0  # the largest magnitude, negative, in one batch
    state, s = O.calibrate_absmax(batches)
    assert s == F32(500) / F32(127)
    # a saved state resumes bit-exactly, in any batch order
    st2, s2 = O.calibrate_absmax(batches[::-1])
    assert (st2, s2) == (state, s)
    q, sat = O.quantize_static_sym(batches[3], s)
    assert sat == 0 and q[7, 9] == -127


def test_tensor_absmax_equals_per_token_when_rows_share_the_absmax():
    x = synth.activations(66, 9, 64, [], dtype="f32")
    x[:, 5] = 4.0  # every row's absmax, so the tensor's too
    q_row, s_row = O.quantize_rows_absmax(x)
    _, s = O.calibrate_absmax([x])
    q, sat = O.quantize_static_sym(x, s)
    assert np.all(s_row == s) and np.array_equal(q, q_row) and sat == 0
    err = np.abs(np.float64(s) * q - x.astype(np.float64))
    assert np.all(err <= np.float64(s) / 2 * (1 + 2.0**-20))


# ---------------------------------------------------------------------------
# Static tensor-wise zero-point quantization (254 levels)
# ---------------------------------------------------------------------------

def check_zeropoint(oracle=O):
    """Closed forms of the 254-step grid, derived by hand: the calibrated range
    (widened to contain 0) spans 2 * 127 steps with its low end on -127."""
    cases = [([-1, 0, 1, 2], 3, -42, [-1, 0, 1, 2, 3, -2], [-127, -42, 43, 127, 127, -127], 2),
             ([0, 0.5, 1], 1, -127, [0, 0.5, 1], [-127, 0, 127], 0),
             ([-2, -1], 2, 127, [-2, -1, 0], [-127, 0, 127], 0),
             ([0, 0], None, 0, [0, 0], [0, 0], 0)]
    for cal, width, z_want, x, q_want, sat_want in cases:
        _, s, z = oracle.calibrate_zeropoint([np.array([cal], F32)])
        assert z == z_want
        if width is None:
            assert s == 1
        else:
            assert abs(float(s) * 254 - width) <= width * 2.0**-23
        q, sat = oracle.quantize_zeropoint(np.array([x], F32), s, z)
        assert q.tolist() == [q_want] and sat == sat_want


def test_zeropoint_closed_forms():
    check_zeropoint()


def test_zeropoint_symmetric_range_is_the_absmax_grid():
    """Over a range symmetric about 0 the zero-point grid is the tensor-wise
    absmax grid: S = 2c / 254 = c / 127 (both correctly rounded), Z = 0."""
    x = synth.activations(70, 12, 96, [4], 10.0, dtype="f32")
    c = float(np.abs(x).max())
    x[0, 0], x[1, 1] = c, -c
    _, s, z = O.calibrate_zeropoint([x])
    _, s_abs = O.calibrate_absmax([x])
    assert (s, z) == (s_abs, 0)
    q, sat = O.quantize_zeropoint(x, s, z)
    q_abs, sat_abs = O.quantize_static_sym(x, s_abs)
    assert np.array_equal(q, q_abs) and sat == sat_abs == 0


def test_zeropoint_error_bound_and_ends():
    cal = [synth.activations(71 + b, 16, 128, [5], 30.0, offset=0.7, dtype="f32") for b in range(4)]
    state, s, z = O.calibrate_zeropoint(cal)
    xa = np.concatenate(cal)
    q, sat = O.quantize_zeropoint(xa, s, z)
    assert sat == 0
    err = np.abs(np.float64(s) * (q.astype(np.int64) - z) - xa.astype(np.float64))
    assert np.all(err <= np.float64(s) / 2 * (1 + 2.0**-18))
    assert q.min() == -127 and q.max() == 127


# ---------------------------------------------------------------------------
# Per-token dynamic asymmetric quantization (the prefill formula with Z_token)
# ---------------------------------------------------------------------------

def check_asym_rows(oracle=O):
    """Closed forms of the per-token asymmetric grid, derived by hand: 255 steps
    over the row's range widened to contain 0, the range's low end on -128."""
    x = np.array([[-1, 0, 1, 2],            # width 3: S = 3/255; -1 -> -128 => Z = -128 + 85
                  [0, 0.25, 1, 1],          # low end 0 => Z = -128; 0.25 * 255 = 63.75 -> 64
                  [0, 0, 0, 0],             # empty range: S = 1, Z = 0
                  [3, 3, 3, 3],             # widened to [0, 3]: Z = -128, all at the top
                  [-2, -0.8, -1.2, -0.1]],  # widened to [-2, 0]: Z = -128 + 255
                 F32)
    q, s, z = oracle.quantize_rows_asym(x)
    assert z.tolist() == [-43, -128, 0, -128, 127]
    assert q.tolist() == [[-128, -43, 42, 127], [-128, -64, 127, 127], [0, 0, 0, 0],
                          [127, 127, 127, 127], [-128, 25, -26, 114]]
    for width, sr in zip([3, 1, None, 3, 2], s):
        if width is None:
            assert sr == 1
        else:
            assert abs(float(sr) * 255 - width) <= width * 2.0**-23


def test_per_token_asym_closed_forms():
    check_asym_rows()


def test_per_token_asym_error_bound_and_range():
    """Every value of a token lies inside its grid: |S (q - Z) - x| <= S / 2, and the
    token's minimum lands on -128 (its maximum on 127 when positive)."""
    x = synth.activations(45, 48, 320, [3, 100], 100.0, offset=0.3, dtype="f32")
    x[5] = np.abs(x[5])   # all non-negative
    x[6] = -np.abs(x[6])  # all non-positive
    q, s, z = O.quantize_rows_asym(x)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(s64 * (q.astype(np.int64) - z[:, None]) - x.astype(np.float64))
    assert np.all(err <= s64 / 2 * (1 + 2.0**-18))
    r = np.arange(x.shape[0])
    assert np.all(q[r, np.argmin(x, axis=1)] == -128)
    pos = np.max(x, axis=1) > 0
    assert np.all(q[r, np.argmax(x, axis=1)][pos] == 127)


def test_per_token_asym_one_token_is_the_per_tensor_grid():
    """One token's per-token parameters are the per-tensor ones of a calibration on
    that token alone, and its codes the decode formula's (itself pinned above)."""
    x = synth.activations(46, 7, 256, [9], 50.0, offset=0.1, dtype="f32")
    q, s, z = O.quantize_rows_asym(x)
    for r in range(x.shape[0]):
        _, s1, z1 = O.calibrate([x[r:r + 1]])
        q1, sat = O.quantize_static(x[r:r + 1], s1, z1)
        assert (s[r], z[r], sat) == (s1, z1, 0)
        assert np.array_equal(q[r], q1[0])


def check_prefill_asym(oracle=O):
    """The zero-point epilogue equals the binary64 product of the dequantized
    operands S_x (q - Z) and S_w q_w ([PDMIX-term] 2.3 dequantization per
    operand; [LLM.int8] part 1 section 2 expansion), up to the epilogue's own
    binary32 roundings."""
    x = synth.activations(47, 24, 192, [5, 77], 100.0, offset=0.2, dtype="f32")
    w = synth.weights(48, 40, 192, "f32")
    b = synth.bias(49, 40)
    wq, sw, colsum = oracle.quantize_weight(w)
    q, sx, zx = oracle.quantize_rows_asym(x)
    acc = oracle.zero_point_correct(oracle.int_matmul(q, wq), colsum, zx)
    y32 = oracle.dequantize(acc, sx, sw, b)
    xd = sx.astype(np.float64)[:, None] * (q.astype(np.float64) - zx[:, None])
    wd = sw.astype(np.float64)[:, None] * wq.astype(np.float64)
    y64 = xd @ wd.T + b
    scale = np.abs(xd) @ np.abs(wd).T + np.abs(b)
    assert np.all(np.abs(y32 - y64) <= 4 * 2.0**-24 * scale)


def test_prefill_asym_epilogue_is_the_dequantized_product():
    check_prefill_asym()
    res = O.linear_prefill_asym(*[synth.activations(50, 3, 64, [], dtype="f32")] +
                                list(O.quantize_weight(synth.weights(51, 5, 64, "f32"))))
    assert set(res) == {"xq", "x_scale", "x_zp", "acc", "y32"}


# ---------------------------------------------------------------------------
# Brute force of whole layers on tiny shapes
# ---------------------------------------------------------------------------

def test_prefill_brute_force_error_bound():
    x = synth.activations(91, 3, 16, [2], 50.0, dtype="f32")
    w = synth.weights(92, 4, 16, "f32")
    wq, sw, _ = O.quantize_weight(w)
    res = O.linear_prefill(x, wq, sw)
    sx = res["x_scale"]
    for m in range(3):
        for n in range(4):
            exact = sum(float(x[m, k]) * float(w[n, k]) for k in range(16))
            bound = sum(abs(float(x[m, k])) * float(sw[n]) / 2 + abs(float(w[n, k])) * float(sx[m]) / 2
                        + float(sx[m]) * float(sw[n]) / 4 for k in range(16))
            assert abs(float(res["y32"][m, n]) - exact) <= bound * (1 + 1e-5) + 1e-6 * abs(exact)


def test_decode_brute_force_error_bound():
    cal = [synth.activations(93 + b, 8, 32, [1], 20.0, offset=0.1, dtype="f32") for b in range(3)]
    _, s, z = O.calibrate(cal)
    x = synth.activations(96, 2, 32, [1], 20.0, offset=0.1, dtype="f32")
    w = synth.weights(97, 5, 32, "f32")
    wq, sw, colsum = O.quantize_weight(w)
    res = O.linear_decode(x, s, z, wq, sw, colsum)
    assert res["sat"] == 0
    for m in range(2):
        for n in range(5):
            exact = sum(float(x[m, k]) * float(w[n, k]) for k in range(32))
            bound = sum(abs(float(x[m, k])) * float(sw[n]) / 2 + abs(float(w[n, k])) * float(s) / 2
                        + float(s) * float(sw[n]) / 4 for k in range(32))
            assert abs(float(res["y32"][m, n]) - exact) <= bound * (1 + 1e-5) + 1e-6 * abs(exact)


def _layer_bound(x, w, sa, sw, ha=None):
    """|x w^T - y| bound of a quantized layer: each activation within sa[m]/2 of
    its grid point (plus ha[m, k] of its own rounding), each weight within
    sw[n]/2, and the cross term."""
    m_, k_ = x.shape
    n_ = w.shape[0]
    b = np.zeros((m_, n_))
    for m in range(m_):
        for n in range(n_):
            b[m, n] = sum((abs(float(w[n, k])) * (float(sa[m]) / 2 + (0.0 if ha is None else ha[m, k]))
                           + abs(float(x[m, k])) * float(sw[n]) / 2 + float(sa[m]) * float(sw[n]) / 4)
                          for k in range(k_))
    return b


def check_static_sym_layer(oracle=O):
    """[LLM.int8] part 1 section 1 absmax, tensor-wise with a calibrated static
    scale: the layer approximates X W^T within the quantization bound when no
    value saturates."""
    cal = [synth.activations(110 + b, 8, 32, [3], 20.0, dtype="f32") for b in range(3)]
    _, s = oracle.calibrate_absmax(cal)
    x = np.clip(synth.activations(114, 3, 32, [3], 20.0, dtype="f32"), -127 * s, 127 * s).astype(F32)
    w = synth.weights(115, 5, 32, "f32")
    wq, sw, _ = oracle.quantize_weight(w)
    res = oracle.linear_static_sym(x, s, wq, sw)
    assert res["sat"] == 0
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    bound = _layer_bound(x, w, np.full(3, s), sw)
    assert np.all(np.abs(res["y32"] - exact) <= bound * (1 + 1e-5) + 1e-6 * np.abs(exact))


def test_static_sym_brute_force_error_bound():
    check_static_sym_layer()


def test_static_sym_of_one_row_is_per_token_prefill():
    """With one activation row and S its own absmax / 127, the tensor-wise
    static code is the per-token code: the whole layer equals the prefill
    linear, bit for bit."""
    x = synth.activations(116, 1, 64, [5], 30.0, dtype="f32")
    w = synth.weights(117, 6, 64, "f32")
    wq, sw, _ = O.quantize_weight(w)
    s = O.absmax_scale(np.max(np.abs(x)))
    a = O.linear_static_sym(x, s, wq, sw)
    b = O.linear_prefill(x, wq, sw)
    assert np.array_equal(a["xq"], b["xq"]) and np.array_equal(a["acc"], b["acc"])
    assert np.array_equal(np.asarray(a["y32"], F32).view(np.uint32), np.asarray(b["y32"], F32).view(np.uint32))


def check_zeropoint_layer(oracle=O):
    """The 254-level zero-point grid ([LLM.int8] part 1 section 2) over a range
    not centred on 0: the layer, with the zero point removed through the code
    sums, approximates X W^T within the quantization bound."""
    cal = [synth.activations(120 + b, 8, 32, [1], 10.0, offset=2.0, dtype="f32") for b in range(3)]
    _, s, z = oracle.calibrate_zeropoint(cal)
    assert z != 0
    lo, hi = (-127 - z) * float(s), (127 - z) * float(s)
    x = np.clip(synth.activations(124, 3, 32, [1], 10.0, offset=2.0, dtype="f32"), lo, hi).astype(F32)
    w = synth.weights(125, 5, 32, "f32")
    wq, sw, colsum = oracle.quantize_weight(w)
    res = oracle.linear_zeropoint(x, s, z, wq, sw, colsum)
    assert res["sat"] == 0
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    bound = _layer_bound(x, w, np.full(3, s), sw)
    assert np.all(np.abs(res["y32"] - exact) <= bound * (1 + 1e-5) + 1e-6 * np.abs(exact))


def test_zeropoint_brute_force_error_bound():
    check_zeropoint_layer()


def test_zeropoint_over_a_symmetric_range_is_static_sym():
    """A calibrated range symmetric about 0 puts the 254-level grid's zero point
    at 0 and its step at C / 127: the zero-point layer equals the static
    symmetric one, bit for bit."""
    x = synth.activations(126, 4, 48, [2], 25.0, dtype="f32")
    c = float(np.max(np.abs(x)))
    state = (F32(-c), F32(c))
    s, z = O.zeropoint_finalize(state)
    assert z == 0 and s == O.absmax_finalize(state)
    w = synth.weights(127, 7, 48, "f32")
    wq, sw, colsum = O.quantize_weight(w)
    a = O.linear_zeropoint(x, s, z, wq, sw, colsum)
    b = O.linear_static_sym(x, s, wq, sw)
    assert np.array_equal(a["xq"], b["xq"]) and np.array_equal(a["acc"], b["acc"])
    assert np.array_equal(np.asarray(a["y32"], F32).view(np.uint32), np.asarray(b["y32"], F32).view(np.uint32))


def check_silu_mul_layer(oracle=O):
    """The down projection fed by SiLU(gate) * up: against the exact product of
    the unrounded SiLU(g) u (math.exp, binary64) with W, within the bound of
    the bf16 rounding of h (2^-9 relative), its per-token quantization and
    the weight's."""
    rng = np.random.default_rng(128)
    g = _bf16_values(rng, 3 * 32, -3, 2).reshape(3, 32)
    u = _bf16_values(rng, 3 * 32, -3, 2).reshape(3, 32)
    w = synth.weights(129, 5, 32, "f32")
    wq, sw, _ = oracle.quantize_weight(w)
    res = oracle.linear_prefill_silu_mul(g, u, wq, sw)
    hx = np.array([[float(g[m, k]) / (1.0 + math.exp(-float(g[m, k]))) * float(u[m, k]) for k in range(32)]
                   for m in range(3)])
    exact = hx @ w.astype(np.float64).T
    bound = _layer_bound(hx, w, res["x_scale"], sw, ha=np.abs(hx) * 2.0 ** -9 * (1 + 1e-9))
    assert np.all(np.abs(res["y32"] - exact) <= bound * (1 + 1e-5) + 1e-6 * np.abs(exact))


def test_prefill_silu_mul_brute_force_error_bound():
    check_silu_mul_layer()


def test_epilogue_matches_binary64_evaluation():
    x = synth.activations(98, 32, 256, [9], 100.0, dtype="f32")
    w = synth.weights(99, 48, 256, "f32")
    b = synth.bias(100, 48)
    wq, sw, _ = O.quantize_weight(w)
    res = O.linear_prefill(x, wq, sw, b)
    y64 = (res["x_scale"].astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]) * res["acc"] + b
    scale = np.abs(res["x_scale"][:, None].astype(np.float64) * sw[None, :] * res["acc"]) + np.abs(b)
    assert np.all(np.abs(res["y32"] - y64) <= 4 * 2.0**-24 * scale + 1e-30)


def test_outlier_infinite_threshold_is_vector_wise():
    x = synth.activations(111, 12, 64, [3, 40], 100.0, dtype="f16")
    w = synth.weights(112, 20, 64, "f16")
    wq, sw, _ = O.quantize_weight(w)
    a = O.linear_int8_outlier(x, w, wq, sw, np.inf)
    b = O.linear_prefill(x, wq, sw)
    assert a["cols"].size == 0
    assert np.array_equal(a["xq"], b["xq"]) and np.array_equal(a["acc"], b["acc"])
    assert np.array_equal(a["y64"], b["y32"].astype(np.float64))


def test_outlier_all_columns_is_plain_16bit_matmul():
    x = synth.activations(113, 5, 32, [], dtype="f16")
    w = synth.weights(114, 7, 32, "f16")
    wq, sw, _ = O.quantize_weight(w)
    a = O.linear_int8_outlier(x, w, wq, sw, -1.0)
    assert a["cols"].tolist() == list(range(32))
    assert not a["xq"].any() and not a["acc"].any()
    ref = [[sum(float(x[m, k]) * float(w[n, k]) for k in range(32)) for n in range(7)] for m in range(5)]
    assert np.allclose(a["y64"], np.array(ref), rtol=1e-12, atol=1e-12)


def test_outlier_decomposition_reconstructs_matmul():
    """INT8 part + 16-bit part approximates X W^T within the INT8 error bound."""
    x = synth.activations(115, 6, 48, [7, 30], 100.0, dtype="f16")
    w = synth.weights(116, 9, 48, "f16")
    wq, sw, _ = O.quantize_weight(w)
    a = O.linear_int8_outlier(x, w, wq, sw, 6.0)
    assert a["cols"].tolist() == [7, 30]
    xr = x.astype(np.float64).copy()
    xr[:, a["cols"]] = 0
    sx = a["x_scale"].astype(np.float64)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    bound = (np.abs(xr) @ np.abs(w.astype(np.float64)).T) * 0  # filled below
    for m in range(6):
        for n in range(9):
            bound[m, n] = sum(abs(xr[m, k]) * float(sw[n]) / 2 + abs(float(w[n, k])) * sx[m] / 2
                              + sx[m] * float(sw[n]) / 4 for k in range(48) if k not in (7, 30))
    assert np.all(np.abs(a["y64"] - exact) <= bound * (1 + 1e-5) + 1e-6)


# ---------------------------------------------------------------------------
# Fused SiLU * up producer: pinned to an exact evaluation of the definition
# (decimal exponential, correctly rounded at 60 digits, then an exact
# rational rounding to the 16-bit type) -- no numpy in the reference path
# ---------------------------------------------------------------------------

def _exact_round(v: Fraction, sig: int, emin: int, emax: int, near=None) -> float:
    """Round an exact rational to a binary format with `sig` significant bits,
    smallest normal 2^emin and largest finite value below 2^emax, ties to even.
    near: a list that receives whether v lies within 2^-50 |v| of a tie (where
    a binary64 evaluation may round either way)."""
    if v == 0:
        if near is not None:
            near.append(False)
        return 0.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^(e-1) <= a < 2^(e+1)
    if Fraction(2) ** e <= a:
        e += 1                                                 # now 2^(e-1) <= a < 2^e
    e = max(e, emin + 1)                                       # subnormals keep the smallest spacing
    step = Fraction(2) ** (e - sig)
    q = a / step
    n = q.numerator // q.denominator
    rem = q - n
    if near is not None:
        near.append(abs(rem - Fraction(1, 2)) * step <= a / 2 ** 50)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * step
    out = math.inf if r >= Fraction(2) ** emax else float(r)
    return out if v > 0 else -out


def _exact_bf16(v: Fraction, near=None) -> float:
    return _exact_round(v, 8, -126, 128, near)


def _exact_f16(v: Fraction, near=None) -> float:
    return _exact_round(v, 11, -14, 16, near)


def _silu_mul_exact(g: float, u: float, rnd=_exact_bf16, near=None) -> float:
    """SiLU(g) * u rounded once to the 16-bit type.  SiLU(g) is transcendental
    for g != 0, so the exact product is never a tie, but it can lie closer to
    one than binary64 resolves (SiLU(g) = g to binary64 precision for g > 37),
    which `near` reports."""
    with localcontext() as ctx:
        ctx.prec = 60
        G, U = Decimal(float(g)), Decimal(float(u))
        if G < -10000:  # |SiLU(g) * u| < 10^-4000: zero with the product's sign
            if near is not None:
                near.append(False)
            return math.copysign(0.0, -float(u))
        return rnd(Fraction(G / (1 + (-G).exp()) * U), near)


def _agree_off_ties(got, g, u, rnd):
    """got equals the exactly rounded SiLU(g) * u, except within binary64's
    resolution of a tie, where it must be one of the two neighbours."""
    for a, b, x in zip(g, u, got):
        near = []
        want = _silu_mul_exact(a, b, rnd, near)
        if near[0]:
            lo = _silu_mul_exact(a, float(b) * (1 - 2.0 ** -40), rnd)
            hi = _silu_mul_exact(a, float(b) * (1 + 2.0 ** -40), rnd)
            assert x in (lo, hi), (a, b, x, lo, hi)
        else:
            assert x == want, (a, b, x, want)


def _bf16_values(rng, n, lo_exp, hi_exp):
    """Random bfloat16 values (as float32) with magnitudes 2^[lo_exp, hi_exp), both signs."""
    mag = 2.0 ** rng.uniform(lo_exp, hi_exp, n) * rng.choice([-1.0, 1.0], n)
    return O.bf16_bits_to_f32(O.to_bf16_bits(mag.astype(np.float32)))


def _double_rounding_cases(n=2_000_000, seed=11):
    """(g, u) pairs whose binary64 product SiLU(g) * u lies within half a
    binary32 unit of a bfloat16 tie: rounding to binary32 first lands on the
    tie, so only a single rounding gets them right."""
    rng = np.random.default_rng(seed)
    g = _bf16_values(rng, n, -4, 4).astype(np.float64)
    u = _bf16_values(rng, n, -4, 4).astype(np.float64)
    v = g / (1.0 + np.exp(-g)) * u
    m, e = np.frexp(v)
    t = np.ldexp(v, 8 - e)                  # bfloat16 units
    dist = np.abs(t - np.floor(t) - 0.5)    # distance to a tie, in bfloat16 units
    pick = np.nonzero(dist < 2.0 ** -17)[0]
    return g[pick], u[pick]


def check_silu_mul(oracle=O):
    rng = np.random.default_rng(5)
    g = np.concatenate([_bf16_values(rng, 150, -6, 7), [0.0, -0.0, 1.0, -1.0, 88.0, -88.0, 100.0, -100.0,
                                                         1000.0, -1000.0, 3.0e38, -3.0e38]])
    u = np.concatenate([_bf16_values(rng, 150, -6, 7), [2.5, 1.0, 1.0, 1.0, -1.5, 1.0, 1.0, 3.0,
                                                         1.0, 7.0, 1.0, 0.5]])
    dg, du = _double_rounding_cases()
    assert len(dg) >= 3
    g = np.concatenate([g, dg[:40]]).astype(np.float32)
    u = np.concatenate([u, du[:40]]).astype(np.float32)
    _agree_off_ties(oracle.silu_mul(g[None, :], u[None, :])[0], g, u, _exact_bf16)
    _agree_off_ties(oracle.silu_mul(g[None, :150], u[None, :150], "f16")[0], g[:150], u[:150], _exact_f16)


def test_silu_mul_is_the_exactly_rounded_definition():
    check_silu_mul()


def test_silu_textbook_values():
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 0.7310585786300049) < 1e-16      # sigmoid(1)
    assert abs(O.silu(-1.0) + 0.2689414213699951) < 1e-16     # -sigmoid(-1)
    x = np.linspace(-30, 30, 601)
    assert np.allclose(O.silu(x) - O.silu(-x), x, rtol=1e-15, atol=1e-14)   # sigmoid(x) + sigmoid(-x) = 1
    assert O.silu(1000.0) == 1000.0 and O.silu(-1000.0) == 0.0 and math.copysign(1, O.silu(-1000.0)) < 0


def test_round_to_bf16_ties_ranges_and_double_rounding():
    r = O.round_to_bf16
    assert r(1.0) == 1.0 and r(1.0 + 2 ** -7) == 1.0 + 2 ** -7
    assert r(1.0 + 2 ** -8) == 1.0                        # tie -> even
    assert r(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6          # tie -> even (upwards)
    assert r(1.0 + 2 ** -8 + 2 ** -40) == 1.0 + 2 ** -7   # just past the tie: a binary32 detour would say 1.0
    assert r(2.0 ** -133) == 2.0 ** -133 and r(2.0 ** -134) == 0.0 and r(3 * 2.0 ** -134) == 2.0 ** -132
    big = (2 - 2 ** -7) * 2.0 ** 127
    assert r(big) == np.float32(big) and r(2.0 ** 128) == np.inf and r(-(2.0 ** 128)) == -np.inf
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(20000) * 2.0 ** rng.integers(-60, 60, 20000)).astype(np.float32)
    assert np.array_equal(r(v.astype(np.float64)).view(np.uint32) >> 16, O.to_bf16_bits(v).astype(np.uint32))


def test_silu_mul_quantize_error_bound():
    rng = np.random.default_rng(8)
    g = _bf16_values(rng, 4 * 96, -3, 3).reshape(4, 96)
    u = _bf16_values(rng, 4 * 96, -3, 3).reshape(4, 96)
    h, q, s = O.silu_mul_quantize_per_token(g, u)
    for hr, gr, ur in zip(h, g, u):
        _agree_off_ties(hr, gr, ur, _exact_bf16)
    want = h
    c = np.max(np.abs(want.astype(np.float64)), axis=1)
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
    assert np.all(np.abs(want - q * s[:, None].astype(np.float64)) <= s[:, None] / 2 * (1 + 1e-6))
    assert np.allclose(s, c / 127, rtol=2 ** -23)


# ---------------------------------------------------------------------------
# Planted mistakes: a copy of the oracle with one plausible error each
# ---------------------------------------------------------------------------

class _Mutant:
    def __init__(self, **over):
        self.__dict__.update({k: getattr(O, k) for k in dir(O) if not k.startswith("__")})
        self.__dict__.update(over)


def _half_up_rows(x):
    x = np.asarray(x, F32)
    s = O.absmax_scale(np.max(np.abs(x), axis=1))
    return np.clip(np.floor(x / s[:, None] + F32(0.5)), -127, 127).astype(np.int8), s


def _truncating_rows(x):
    x = np.asarray(x, F32)
    c = np.max(np.abs(x), axis=1)
    s = O.absmax_scale(c)
    return np.clip(np.trunc(x * (F32(127) / c)[:, None]), -127, 127).astype(np.int8), s


def _plus_zero_point(acc, colsum, z):
    return np.asarray(acc, np.int64) + np.int64(z) * np.asarray(colsum, np.int64)[None, :]


def _static_sym_asym_clamp(x, s):
    """Clamped to the asymmetric range [-128, 127]."""
    r = np.rint(np.asarray(x, F32) / F32(s))
    return np.clip(r, -128, 127).astype(np.int8), int(np.count_nonzero((r < -128) | (r > 127)))


def _zeropoint_255_levels(state):
    """255 steps instead of 254."""
    lo, hi = min(F32(state[0]), F32(0)), max(F32(state[1]), F32(0))
    if hi == lo:
        return F32(1), 0
    s = F32(F32(hi - lo) / F32(255))
    return s, int(min(max(-127 - int(np.rint(F32(lo / s))), -127), 127))


def _zeropoint_wide_clamp(x, s, z):
    """Clamped to [-128, 127]."""
    return O.quantize_static(x, s, z)


def _plus_zero_point_rows(acc, colsum, z):
    z = np.asarray(z, np.int64)
    if z.ndim == 0:
        return O.zero_point_correct(acc, colsum, z)
    return np.asarray(acc, np.int64) + z[:, None] * np.asarray(colsum, np.int64)[None, :]


def _asym_rows_unwidened(x):
    """Range not widened to contain 0."""
    x = np.asarray(x, F32)
    q = np.zeros(x.shape, np.int8)
    s = np.ones(x.shape[0], F32)
    z = np.zeros(x.shape[0], np.int32)
    for r in range(x.shape[0]):
        lo, hi = F32(x[r].min()), F32(x[r].max())
        if hi > lo:
            s[r] = F32(F32(hi - lo) / F32(255))
            z[r] = min(max(-128 - int(np.rint(F32(lo / s[r]))), -128), 127)
        q[r], _ = O.quantize_static(x[r:r + 1], s[r], z[r])
    return q, s, z


def _asym_rows_zero_point_sign(x):
    """Z = -128 + rne(lo / S) instead of -128 - rne(lo / S)."""
    q, s, z = O.quantize_rows_asym(x)
    x = np.asarray(x, F32)
    for r in range(x.shape[0]):
        lo = min(F32(x[r].min()), F32(0))
        z[r] = min(max(-128 + int(np.rint(F32(lo / s[r]))), -128), 127)
        q[r], _ = O.quantize_static(x[r:r + 1], s[r], z[r])
    return q, s, z


def _nonstrict_outliers(x, thr):
    return np.nonzero(np.max(np.abs(np.asarray(x, F32)), axis=0) >= F32(thr))[0]


def _rowwise_over_all_columns(x, cols):
    q, s = O.quantize_rows_absmax(x)
    q = q.copy()
    q[:, cols] = 0
    return q, s


def _silu_mul_flipped_sigmoid(g, u, dtype="bf16"):
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return O.round_to_bf16(g / (1.0 + np.exp(g)) * np.asarray(u, np.float64))


def _silu_mul_without_up(g, u, dtype="bf16"):
    return O.round_to_bf16(O.silu(g))


def _silu_mul_via_binary32(g, u, dtype="bf16"):
    v = (O.silu(g) * np.asarray(u, np.float64)).astype(np.float32)
    return O.bf16_bits_to_f32(O.to_bf16_bits(v))


def _static_sym_layer_without_activation_scale(x, s, wq, sw, bias=None):
    xq, sat = O.quantize_static_sym(x, s)
    acc = O.int_matmul(xq, wq)
    return dict(xq=xq, sat=sat, acc=acc, y32=O.dequantize(acc, F32(1), sw, bias))


def _zeropoint_layer_adding_zero_point(x, s, z, wq, sw, colsum, bias=None):
    xq, sat = O.quantize_zeropoint(x, s, z)
    acc = O.int_matmul(xq, wq)
    return dict(xq=xq, sat=sat, acc=acc, y32=O.dequantize(acc + z * colsum.astype(np.int64)[None, :], F32(s), sw,
                                                           bias))


def _silu_mul_layer_quantizing_gate(gate, up, wq, sw, bias=None, dtype="bf16"):
    xq, sx = O.quantize_rows_absmax(np.asarray(gate, F32))
    acc = O.int_matmul(xq, wq)
    return dict(h=None, xq=xq, x_scale=sx, acc=acc, y32=O.dequantize(acc, sx, sw, bias))


@pytest.mark.parametrize("mutant,check", [
    (_Mutant(silu_mul=_silu_mul_flipped_sigmoid), check_silu_mul),
    (_Mutant(silu_mul=_silu_mul_without_up), check_silu_mul),
    (_Mutant(silu_mul=_silu_mul_via_binary32), check_silu_mul),
    (_Mutant(quantize_rows_absmax=_half_up_rows), check_worked_row),
    (_Mutant(quantize_rows_absmax=_truncating_rows), check_worked_row),
    (_Mutant(zero_point_correct=_plus_zero_point), check_four_term),
    (_Mutant(quantize_rows_regular=_rowwise_over_all_columns), check_outlier_example),
    (_Mutant(outlier_columns=_nonstrict_outliers), check_threshold_strict),
    (_Mutant(zero_point_correct=_plus_zero_point_rows), check_prefill_asym),
    (_Mutant(quantize_static_sym=_static_sym_asym_clamp), check_tensor_absmax),
    (_Mutant(zeropoint_finalize=_zeropoint_255_levels,
             calibrate_zeropoint=lambda b: (None, *_zeropoint_255_levels(O.calibrate(b)[0]))), check_zeropoint),
    (_Mutant(quantize_zeropoint=_zeropoint_wide_clamp), check_zeropoint),
    (_Mutant(quantize_rows_asym=_asym_rows_unwidened), check_asym_rows),
    (_Mutant(quantize_rows_asym=_asym_rows_zero_point_sign), check_asym_rows),
    (_Mutant(linear_static_sym=_static_sym_layer_without_activation_scale), check_static_sym_layer),
    (_Mutant(linear_zeropoint=_zeropoint_layer_adding_zero_point), check_zeropoint_layer),
    (_Mutant(linear_prefill_silu_mul=_silu_mul_layer_quantizing_gate), check_silu_mul_layer),
])
def test_planted_mistake_is_caught(mutant, check):
    with pytest.raises(AssertionError):
        check(mutant)

