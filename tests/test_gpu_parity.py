"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

INT8 codes, scales, zero point, outlier indices, saturation counts and INT32
accumulators must match bit for bit; 16-bit outputs must meet the bar in
gpu_helpers.check_16bit (and, where both sides run the same binary32
sequence, match bit for bit as well).
"""
import numpy as np
import pytest
import torch

import oracle.pdq_oracle as O
from w8a8_int8_quantized_absmax_amd import pdq, synth
from gpu_helpers import check_16bit, codes_equal, dev, host, sample_rows
from guards import gapped, guarded
from packing import pack, pack_weight

pytestmark = pytest.mark.gpu
F32 = np.float32


def weight_case(w, dtype):
    wq, ws, cs = pdq.quantize_weight(dev(w, dtype))
    rq, rs, rc = O.quantize_weight(w)
    # the whole packed image, padding included, and the binding's unpacking
    assert np.array_equal(host(wq), pack_weight(rq))
    assert np.array_equal(pdq.unpack_weight(wq, *w.shape), rq)
    assert np.array_equal(host(ws).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(cs), rc)
    return wq, ws, cs, (rq, rs, rc)


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,n,k", [("f32", 512, 256), ("bf16", 700, 1040), ("f16", 33, 16),
                                       ("bf16", 5, 14336 + 64), ("f32", 3, 20480)])
def test_weight_quant(dtype, n, k):
    w = synth.weights(1000 + n, n, k, dtype)
    w[1, :] = 0.0  # an all-zero channel gets scale 1 and zero codes
    weight_case(w, dtype)


def test_weight_quant_prefill_7b_full():
    c = synth.Prefill7B()
    weight_case(c.w(), c.dtype)


# ---------------------------------------------------------------------------
# prefill: per-token dynamic symmetric
# ---------------------------------------------------------------------------

def prefill_case(x, w, dtype, bias=None, rows=None, exact=True):
    """Every output of the call surrounded by sentinel margins, y with a row
    pitch past N; codes, scales, accumulators and outputs against the oracle
    (all rows unless `rows` is given)."""
    wq, ws, _, (rq, rs, _) = weight_case(w, dtype)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    y, y_check = gapped(x.shape[0], w.shape[0])
    with guarded():
        res = pdq.linear_prefill(dev(x, dtype), wq, ws, b, want_acc=True, out=y)
    y_check()
    xq_ref, sx_ref = O.quantize_rows_absmax(x)
    assert codes_equal(res["xq"], xq_ref)
    assert np.array_equal(host(res["x_scale"]).view(np.uint32), sx_ref.view(np.uint32))
    r = np.arange(x.shape[0]) if rows is None else rows
    acc_ref = O.int_matmul(xq_ref[r], rq)
    assert np.array_equal(host(res["acc"])[r], acc_ref)
    y_ref = O.dequantize(acc_ref, sx_ref[r], rs, bias)
    check_16bit(host(res["y"])[r], y_ref, "bf16", exact)
    return res


def test_prefill_tiny_f32():
    c = synth.Tiny()
    prefill_case(c.x(), c.w(), "f32")
    prefill_case(c.x(), c.w(), "f32", bias=c.bias())


# (2048, 2600, 1040) runs on the tiled GEMM, the others on the skinny kernel
# ((200, 4100) with 48 channels per workgroup, the last one's second group
# partly and its third wholly past N).
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(300, 700, 1040), (1, 257, 128), (257, 1, 16), (513, 256, 2048),
                                   (200, 4100, 1040), (2048, 2600, 1040)])
def test_prefill_ragged(dtype, m, n, k):
    assert pdq.gemm_kernel(m, n) == ("tiled" if m == 2048 else "skinny")
    assert (m, n) != (200, 4100) or pdq.skinny_channels(m, n) == 48
    x = synth.activations(2000 + m, m, k, [0, k - 1, k // 3], 100.0, dtype=dtype)
    if m > 2:
        x[2, :] = 0.0  # all-zero token: scale 1, codes 0
    w = synth.weights(2100 + n, n, k, dtype)
    prefill_case(x, w, dtype, bias=synth.bias(2200 + n, n))


# K tiles of 64: every count modulo the depth of the tiled GEMM's LDS ring
# (four) and of the skinny kernel's batches (two in flight of up to eight
# tiles per wavefront, four wavefronts), whole and ragged, with and without
# bias; M x N = 2048 x 2600 runs on the tiled GEMM, 300 x 520 (16 channels per
# workgroup) and 256 x 4112 (32) on the skinny kernel.
@pytest.mark.parametrize("m,n", [(2048, 2600), (300, 520), (256, 4112)])
@pytest.mark.parametrize("k", [64, 128, 192, 256, 320, 336, 640, 656, 1216, 1280, 2112, 4160])
def test_prefill_k_depths(m, n, k):
    assert pdq.gemm_kernel(m, n) == ("tiled" if m == 2048 else "skinny")
    x = synth.activations(2300 + k, m, k, [1, k - 2], 100.0, dtype="bf16")
    w = synth.weights(2400 + k, n, k, "bf16")
    bias = synth.bias(2500 + k, n) if k % 128 == 0 else None
    res = prefill_case(x, w, "bf16", bias=bias)
    # the same output without the INT32 accumulator copy
    wq, ws, _ = pdq.quantize_weight(dev(w, "bf16"))
    b = None if bias is None else torch.from_numpy(bias).cuda()
    y2 = pdq.linear_prefill(dev(x, "bf16"), wq, ws, b)["y"]
    assert torch.equal(res["y"], y2)


# Per-token codes at decode sizes: the weight-streaming kernel runs with
# per-row scales in its epilogue.
@pytest.mark.parametrize("m,n,k", [(1, 300, 1040), (17, 4096, 4096), (64, 520, 2048), (65, 520, 2048),
                                   (130, 700, 1040), (600, 1000, 1040), (256, 4096, 4096), (200, 4100, 1040),
                                   (32, 12300, 512)])
def test_per_token_skinny(m, n, k):
    assert pdq.gemm_kernel(m, n) == "skinny"
    x = synth.activations(2600 + m, m, k, [0, k - 1], 100.0, dtype="bf16")
    prefill_case(x, synth.weights(2700 + n, n, k, "bf16"), "bf16", bias=synth.bias(2800 + n, n))


# ---------------------------------------------------------------------------
# prefill, per-token dynamic asymmetric (the prefill formula with Z_token)
# ---------------------------------------------------------------------------

def prefill_asym_case(x, w, dtype, bias=None, rows=None):
    wq, ws, cs, (rq, rs, rc) = weight_case(w, dtype)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    y, y_check = gapped(x.shape[0], w.shape[0])
    with guarded():
        res = pdq.linear_prefill_asym(dev(x, dtype), wq, ws, cs, b, want_acc=True, out=y)
    y_check()
    q_ref, s_ref, z_ref = O.quantize_rows_asym(x)
    assert codes_equal(res["xq"], q_ref)
    assert np.array_equal(host(res["x_scale"]).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(res["x_zp"]), z_ref)
    r = np.arange(x.shape[0]) if rows is None else rows
    acc_ref = O.int_matmul(q_ref[r], rq)
    assert np.array_equal(host(res["acc"])[r], acc_ref)
    y_ref = O.dequantize(O.zero_point_correct(acc_ref, rc, z_ref[r]), s_ref[r], rs, bias)
    check_16bit(host(res["y"])[r], y_ref, "bf16", exact=True)
    return res


# Both GEMM kernels: (2048, 2600) runs on the tiled one, the others on the
# skinny one ((200, 4100) with 48 channels per workgroup).
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(1, 300, 1040), (37, 520, 2048), (300, 700, 1040), (257, 1, 16),
                                   (200, 4100, 1040), (2048, 2600, 1040)])
def test_prefill_asym_ragged(dtype, m, n, k):
    assert pdq.gemm_kernel(m, n) == ("tiled" if m == 2048 else "skinny")
    x = synth.activations(7000 + m, m, k, [0, k - 1, k // 3], 100.0, offset=0.3, dtype=dtype)
    if m > 5:
        x[2, :] = 0.0                # empty range: S = 1, Z = 0
        x[3, :] = np.abs(x[3, :])    # non-negative token: Z = -128
        x[4, :] = -np.abs(x[4, :])   # non-positive token: Z = 127
        x[5, :] = 1.5                # one value: range [0, 1.5]
    prefill_asym_case(x, synth.weights(7100 + n, n, k, dtype), dtype, bias=synth.bias(7200 + n, n))


def test_prefill_asym_7b_full():
    c = synth.Prefill7B()
    prefill_asym_case(c.x(), c.w(), c.dtype)


@pytest.mark.parametrize("m,n,k", [(20, 300, 512), (800, 3000, 512)])
def test_prefill_asym_building_blocks(m, n, k):
    """Quantizer + GEMM entry points give the composite call's bits."""
    x = synth.activations(7300 + m, m, k, [5], 100.0, offset=-0.2, dtype="bf16")
    w = synth.weights(7301, n, k, "bf16")
    wq, ws, cs = pdq.quantize_weight(dev(w, "bf16"))
    xd = dev(x, "bf16")
    one = pdq.linear_prefill_asym(xd, wq, ws, cs, want_acc=True)
    xq, xs, xz = pdq.quantize_per_token_asym(xd)
    two = pdq.gemm_per_token_asym(xq, xs, xz, wq, ws, cs, want_acc=True)
    assert torch.equal(one["xq"].data, xq.data) and torch.equal(one["x_zp"], xz)
    assert torch.equal(one["y"], two["y"]) and torch.equal(one["acc"], two["acc"])


# Rows with a pitch past K (a view of the first K columns of a wider buffer):
# both per-token quantizers -- a wavefront per row up to K = 2048, a workgroup
# per row beyond -- and both GEMM kernels read the right rows.
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(37, 520, 1040), (300, 700, 4096), (2048, 2600, 2112)])
def test_prefill_strided_rows(dtype, m, n, k):
    pad = 40
    wide = synth.activations(5200 + k, m, k + pad, [3, k - 1], 100.0, dtype=dtype)
    x = np.ascontiguousarray(wide[:, :k])
    wq, ws, cs, (rq, rs, rc) = weight_case(synth.weights(5201, n, k, dtype), dtype)
    xt = dev(wide, dtype)[:, :k]
    assert xt.stride(0) == k + pad
    res = pdq.linear_prefill(xt, wq, ws, want_acc=True)
    xq_ref, sx_ref = O.quantize_rows_absmax(x)
    assert codes_equal(res["xq"], xq_ref)
    assert np.array_equal(host(res["x_scale"]).view(np.uint32), sx_ref.view(np.uint32))
    acc_ref = O.int_matmul(xq_ref, rq)
    assert np.array_equal(host(res["acc"]), acc_ref)
    check_16bit(host(res["y"]), O.dequantize(acc_ref, sx_ref, rs, None), "bf16", True)
    res = pdq.linear_prefill_asym(xt, wq, ws, cs, want_acc=True)
    q_ref, s_ref, z_ref = O.quantize_rows_asym(x)
    assert codes_equal(res["xq"], q_ref)
    assert np.array_equal(host(res["x_scale"]).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(res["x_zp"]), z_ref)
    acc_ref = O.int_matmul(q_ref, rq)
    assert np.array_equal(host(res["acc"]), acc_ref)
    check_16bit(host(res["y"]), O.dequantize(O.zero_point_correct(acc_ref, rc, z_ref), s_ref, rs, None), "bf16",
                True)


def test_prefill_empty_batch():
    w = synth.weights(7, 64, 64, "bf16")
    wq, ws, _ = pdq.quantize_weight(dev(w, "bf16"))
    res = pdq.linear_prefill(dev(np.zeros((0, 64), F32), "bf16"), wq, ws)
    assert res["y"].shape == (0, 64)


def test_prefill_7b_full():
    c = synth.Prefill7B()
    prefill_case(c.x(), c.w(), c.dtype)


def test_prefill_deterministic():
    x = synth.activations(3001, 512, 2048, [5], 100.0, dtype="bf16")
    w = synth.weights(3002, 1024, 2048, "bf16")
    wq, ws, _ = pdq.quantize_weight(dev(w, "bf16"))
    xd = dev(x, "bf16")
    a = pdq.linear_prefill(xd, wq, ws, want_acc=True)
    for _ in range(3):
        b = pdq.linear_prefill(xd, wq, ws, want_acc=True)
        assert torch.equal(a["acc"], b["acc"]) and torch.equal(a["y"].view(torch.int16),
                                                               b["y"].view(torch.int16))


# ---------------------------------------------------------------------------
# static calibration
# ---------------------------------------------------------------------------

def gpu_calibrate(batches, dtype):
    mm = pdq.minmax_state("cuda")
    s = z = None
    for i, b in enumerate(batches):
        out = pdq.calibrate_static(dev(b, dtype), mm, finalize=(i == len(batches) - 1))
        if out:
            s, z = out
    return mm, s, z


def test_calibration_tiny():
    c = synth.Tiny()
    batches = [c.calib(b) for b in range(c.n_calib)]
    mm, s, z = gpu_calibrate(batches, c.dtype)
    state, rs, rz = O.calibrate(batches)
    assert host(mm).tolist() == [float(state[0]), float(state[1])]
    assert host(s).view(np.uint32)[0] == np.float32(rs).view(np.uint32) and int(host(z)[0]) == rz


def test_calibration_decode_50_batches_and_resume():
    c = synth.Decode()
    batches = [c.calib(b) for b in range(c.n_calib)]
    mm, s, z = gpu_calibrate(batches, c.dtype)
    state, rs, rz = O.calibrate(batches)
    assert host(mm).tolist() == [float(state[0]), float(state[1])]
    assert host(s).view(np.uint32)[0] == np.float32(rs).view(np.uint32) and int(host(z)[0]) == rz
    # resume: 25 batches, state copied to the host and back, 25 more
    mm1, _, _ = gpu_calibrate(batches[:25], c.dtype)
    saved = host(mm1).copy()
    mm2 = torch.from_numpy(saved).cuda()
    for i, b in enumerate(batches[25:]):
        out = pdq.calibrate_static(dev(b, c.dtype), mm2, finalize=(i == 24))
    s2, z2 = out
    assert torch.equal(mm2, mm) and torch.equal(s2, s) and torch.equal(z2, z)


def test_calibration_finalize_only_and_positive_range():
    mm = torch.tensor([3.0, 5.0], device="cuda")
    s, z = pdq.calibrate_static(torch.zeros((0, 16), device="cuda"), mm, finalize=True)
    rs, rz = O.minmax_finalize((F32(3.0), F32(5.0)))
    assert host(s)[0] == rs and int(host(z)[0]) == rz == -128


# ---------------------------------------------------------------------------
# decode: per-tensor static asymmetric
# ---------------------------------------------------------------------------

def decode_case(x, w, dtype, s, z, bias=None, exact=True):
    wq, ws, cs, (rq, rs, rc) = weight_case(w, dtype)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    b = None if bias is None else torch.from_numpy(bias).cuda()
    y, y_check = gapped(x.shape[0], w.shape[0])
    with guarded():
        res = pdq.linear_decode(dev(x, dtype), s, z, wq, ws, cs, b, sat_count=sat, want_acc=True, out=y)
    y_check()
    ref = O.linear_decode(x, F32(s), z, rq, rs, rc, bias)
    assert codes_equal(res["xq"], ref["xq"])
    assert int(host(sat)[0]) == ref["sat"]
    assert np.array_equal(host(res["acc"]), ref["acc"])
    check_16bit(host(res["y"]), ref["y32"], "bf16", exact)
    return ref


# ---------------------------------------------------------------------------
# static tensor-wise symmetric (absmax over calibration batches)
# ---------------------------------------------------------------------------

def static_sym_case(x, w, dtype, s, bias=None):
    wq, ws, _, (rq, rs, _) = weight_case(w, dtype)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    b = None if bias is None else torch.from_numpy(bias).cuda()
    y, y_check = gapped(x.shape[0], w.shape[0])
    with guarded():
        res = pdq.linear_static_sym(dev(x, dtype), s, wq, ws, b, sat_count=sat, want_acc=True, out=y)
    y_check()
    ref = O.linear_static_sym(x, F32(s), rq, rs, bias)
    assert codes_equal(res["xq"], ref["xq"])
    assert int(host(sat)[0]) == ref["sat"]
    assert np.array_equal(host(res["acc"]), ref["acc"])
    check_16bit(host(res["y"]), ref["y32"], "bf16", exact=True)
    return ref


def test_static_sym_calibration():
    batches = [synth.activations(7400 + b, 64, 1024, [3, 700], 100.0, offset=0.1, dtype="bf16") for b in range(6)]
    mm = pdq.minmax_state("cuda")
    for i, xb in enumerate(batches):
        s = pdq.calibrate_static_sym(dev(xb, "bf16"), mm, finalize=i == len(batches) - 1)
    _, s_ref = O.calibrate_absmax(batches)
    assert host(s).view(np.uint32)[0] == np.array([s_ref], F32).view(np.uint32)[0]
    # a fresh state finalised before any batch gives S = 1
    empty = pdq.minmax_state("cuda")
    s0 = pdq.calibrate_static_sym(dev(np.zeros((0, 64), F32), "bf16"), empty, finalize=True)
    assert float(host(s0)[0]) == 1.0 == O.absmax_finalize((np.inf, -np.inf))


# One launch (M * K <= 8192), the skinny kernel, and the tiled GEMM (2048 x 2600);
# the scale comes from calibration rows that do not cover the decode values'
# largest magnitudes, so some saturate.
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(1, 300, 1024), (4, 100, 2048), (37, 1000, 1040), (2048, 2600, 1040)])
def test_static_sym_linear(dtype, m, n, k):
    cal = [synth.activations(7500 + b, 32, k, [2], 8.0, dtype=dtype) for b in range(3)]
    _, s = O.calibrate_absmax(cal)
    x = synth.activations(7600 + m, m, k, [2, k - 5], 20.0, dtype=dtype)
    big = 3.0 * max(float(np.abs(c).max()) for c in cal)
    x[0, 7], x[m - 1, 9] = big, -big
    x = synth.round_to(x, dtype)
    ref = static_sym_case(x, synth.weights(7700 + n, n, k, dtype), dtype, s, bias=synth.bias(7800, n))
    assert ref["sat"] > 0
    if m * k > 8192:
        assert pdq.gemm_kernel(m, n) == ("tiled" if m == 2048 else "skinny")


# ---------------------------------------------------------------------------
# static tensor-wise zero-point grid (254 levels)
# ---------------------------------------------------------------------------

def test_zeropoint_calibration():
    batches = [synth.activations(8100 + b, 64, 1024, [3, 700], 100.0, offset=0.4, dtype="bf16") for b in range(6)]
    mm = pdq.minmax_state("cuda")
    for i, xb in enumerate(batches):
        out = pdq.calibrate_zeropoint(dev(xb, "bf16"), mm, finalize=i == len(batches) - 1)
    _, s, z = O.calibrate_zeropoint(batches)
    assert host(out[0]).view(np.uint32)[0] == np.array([s], F32).view(np.uint32)[0] and int(host(out[1])[0]) == z


def zeropoint_case(x, w, dtype, s, z, bias=None):
    wq, ws, cs, (rq, rs, rc) = weight_case(w, dtype)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    b = None if bias is None else torch.from_numpy(bias).cuda()
    y, y_check = gapped(x.shape[0], w.shape[0])
    with guarded():
        res = pdq.linear_zeropoint(dev(x, dtype), s, z, wq, ws, cs, b, sat_count=sat, want_acc=True, out=y)
    y_check()
    ref = O.linear_zeropoint(x, F32(s), z, rq, rs, rc, bias)
    assert codes_equal(res["xq"], ref["xq"])
    assert int(host(sat)[0]) == ref["sat"]
    assert np.array_equal(host(res["acc"]), ref["acc"])
    check_16bit(host(res["y"]), ref["y32"], "bf16", exact=True)
    return ref


# One launch (M * K <= 8192), the skinny kernel (16 and 48 channels per
# workgroup) and the tiled GEMM; decode values beyond the calibrated range
# saturate at both ends.
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(1, 300, 1024), (4, 100, 2048), (37, 1000, 1040), (300, 4100, 1040),
                                   (2048, 2600, 1040)])
def test_zeropoint_linear(dtype, m, n, k):
    cal = [synth.activations(8200 + b, 32, k, [2], 8.0, offset=0.5, dtype=dtype) for b in range(3)]
    _, s, z = O.calibrate_zeropoint(cal)
    x = synth.activations(8300 + m, m, k, [2, k - 5], 20.0, offset=0.5, dtype=dtype)
    big = 3.0 * max(float(np.abs(c).max()) for c in cal)
    x[0, 7], x[m - 1, 9] = big, -big
    x = synth.round_to(x, dtype)
    ref = zeropoint_case(x, synth.weights(8400 + n, n, k, dtype), dtype, s, z, bias=synth.bias(8500, n))
    assert ref["sat"] > 0
    if m * k > 8192:
        assert pdq.gemm_kernel(m, n) == ("tiled" if m == 2048 else "skinny")


@pytest.mark.parametrize("m,n,k", [(9, 300, 1040), (2048, 2600, 512)])
def test_gemm_static_zero_point_zero_needs_no_colsum(m, n, k):
    """With Z = 0 the static GEMM takes no code sums, on either kernel."""
    xq = synth.random_int8(7900 + m, (m, k), -127, 127)
    w = synth.weights(7901, n, k, "bf16")
    wq, ws, cs, (rq, rs, rc) = weight_case(w, "bf16")
    codes = pdq.Codes(torch.from_numpy(pack(xq)).cuda(), m, k)
    a = pdq.gemm_static(codes, F32(0.11), 0, wq, ws, None, want_acc=True)
    b = pdq.gemm_static(codes, F32(0.11), 0, wq, ws, cs, want_acc=True)
    acc = O.int_matmul(xq, rq)
    assert np.array_equal(host(a["acc"]), acc) and torch.equal(a["y"], b["y"])
    check_16bit(host(a["y"]), O.dequantize(acc, F32(0.11), rs), "bf16", exact=True)


@pytest.fixture(scope="module")
def decode_params():
    c = synth.Decode()
    _, s, z = O.calibrate([c.calib(b) for b in range(c.n_calib)])
    return c, s, z


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_decode_batches(decode_params, m):
    c, s, z = decode_params
    ref = decode_case(c.x(m), c.w(), c.dtype, s, z)
    print(f"decode M={m}: S={s} Z={z} saturated={ref['sat']}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(37, 1000, 1040), (100, 33, 512), (3, 16, 16), (64, 4096, 14336)])
def test_decode_ragged(dtype, m, n, k):
    cal = [synth.activations(4000 + b, 64, k, [1, k - 2], 100.0, offset=0.1, dtype=dtype) for b in range(3)]
    _, s, z = O.calibrate(cal)
    x = synth.activations(4100 + m, m, k, [1, k - 2], 100.0, offset=0.1, dtype=dtype)
    decode_case(x, synth.weights(4200 + n, n, k, dtype), dtype, s, z, bias=synth.bias(4300, n))


# One-launch path (static quantization inside the GEMM): M <= 16 and M * K <=
# 8192 (the one-row shapes up to K = 8192 and (5, 17, 80)); the other shapes
# take the two-kernel path, (17, 50, 64) just past the row limit.
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (1, 300, 1024), (1, 33, 1040), (1, 4096, 4096),
                                   (1, 20, 4160), (1, 7, 8192), (5, 17, 80), (16, 1000, 1040),
                                   (16, 300, 2048), (2, 64, 14336), (8, 4096, 4096), (9, 100, 4096),
                                   (17, 50, 64)])
def test_decode_fused_shapes(dtype, m, n, k):
    cal = [synth.activations(4500 + b, 64, k, [1, k - 2], 100.0, offset=0.1, dtype=dtype) for b in range(3)]
    _, s, z = O.calibrate(cal)
    x = synth.activations(4600 + m, m, k, [1, k - 2], 100.0, offset=0.1, dtype=dtype)
    decode_case(x, synth.weights(4700 + n, n, k, dtype), dtype, s, z, bias=synth.bias(4800, n))


# Static codes past 64 rows: the zero-point correction in the epilogue of
# the skinny kernel (the first four; 300 x 4100 with 48 channels per
# workgroup) and of the tiled GEMM (the others).
@pytest.mark.parametrize("m,n,k", [(65, 700, 1040), (300, 256, 2048), (513, 1000, 4096), (300, 4100, 1040),
                                   (2048, 2600, 1040), (1600, 4096, 2048), (3000, 1500, 2048)])
def test_static_large_m(m, n, k):
    assert pdq.gemm_kernel(m, n) == ("tiled" if m in (2048, 1600, 3000) else "skinny")
    if (m, n) == (300, 4100):
        assert pdq.skinny_channels(m, n) == 48
    cal = [synth.activations(4900 + b, 64, k, [2, k - 3], 100.0, offset=0.1, dtype="bf16") for b in range(3)]
    _, s, z = O.calibrate(cal)
    x = synth.activations(4950 + m, m, k, [2, k - 3], 100.0, offset=0.1, dtype="bf16")
    decode_case(x, synth.weights(4960 + n, n, k, "bf16"), "bf16", s, z, bias=synth.bias(4970, n))


# K tile counts that differ between the four wavefronts of a skinny-kernel
# workgroup (K not a multiple of 4 x 64; at K = 64 three wavefronts get no
# tile at all): a tile a wavefront does not have must add nothing (MFMA
# instructions ignore the lane mask, so the kernel must branch around them).
# 16, 32, 48 and 64 channels per workgroup, one to three row blocks of 16.
@pytest.mark.parametrize("m,n,k,ch", [(20, 300, 4288, 16), (10, 12300, 4288, 16), (20, 9000, 320, 48),
                                      (3, 12300, 576, 16), (32, 8200, 64, 48), (17, 5000, 1088, 32),
                                      (40, 12328, 64, 64)])
def test_skinny_uneven_tiles_per_wavefront(m, n, k, ch):
    assert pdq.gemm_kernel(m, n) == "skinny" and pdq.skinny_channels(m, n) == ch
    x = synth.activations(4980 + m, m, k, [1, k - 2], 100.0, offset=0.1, dtype="bf16")
    w = synth.weights(4990 + n, n, k, "bf16")
    prefill_case(x, w, "bf16", bias=synth.bias(4991, n))
    decode_case(x, w, "bf16", F32(0.9), -3, bias=synth.bias(4992, n))


# Each width of the skinny kernel (32, 48, 64 weight channels per workgroup)
# with a ragged last workgroup (N not a multiple of the width: its last
# channel group partly past N, or wholly, then clamped onto the last one and
# not stored), ragged rows and K, and, past 64 rows, two to four row blocks
# with a short last one; static (zero-point) and per-token epilogues.
@pytest.mark.parametrize("m,n,k,ch", [(24, 8200, 4096, 48), (40, 12328, 1040, 64), (33, 6000, 2048, 32),
                                      (100, 6144, 2048, 48), (200, 4096, 1040, 64), (64, 12280, 1088, 48)])
def test_skinny_channel_widths(m, n, k, ch):
    assert pdq.gemm_kernel(m, n) == "skinny" and pdq.skinny_channels(m, n) == ch
    x = synth.activations(5050 + m, m, k, [1, k - 2], 100.0, offset=0.1, dtype="bf16")
    w = synth.weights(5060 + n, n, k, "bf16")
    prefill_case(x, w, "bf16", bias=synth.bias(5070, n))
    decode_case(x, w, "bf16", F32(0.9), -3, bias=synth.bias(5071, n))


# Layout conversion: plain int8 [rows, K] <-> the packed tile image.  The
# packed image equals the numpy packer's (written from the header's
# definition) byte for byte, padding included, at ragged row counts, K and row
# pitches; unpacking gives the matrix back and leaves a wider destination's
# gap bytes alone; a weight packed this way (codes and scales from the
# oracle) runs the GEMMs to the oracle's results.
@pytest.mark.parametrize("rows,k,ld", [(1, 16, 16), (5, 48, 64), (16, 64, 64), (37, 1040, 1072),
                                       (300, 4096, 4096), (4100, 208, 224)])
def test_pack_unpack_int8(rows, k, ld):
    codes = synth.random_int8(9300 + rows, (rows, k))
    src = torch.full((rows, ld), 77, dtype=torch.int8)
    src[:, :k] = torch.from_numpy(codes)
    src = src.cuda()[:, :k]
    packed = pdq.pack_int8(src)
    assert packed.numel() == pdq.weight_bytes(rows, k)
    assert np.array_equal(host(packed), pack(codes))
    dst = torch.full((rows, ld + 16), -5, dtype=torch.int8, device="cuda")
    pdq.unpack_int8(packed, rows, k, out=dst[:, :k])
    back = host(dst)
    assert np.array_equal(back[:, :k], codes)
    assert (back[:, k:] == -5).all()


@pytest.mark.parametrize("m,n,k", [(40, 300, 1040), (300, 520, 2048)])
def test_gemm_on_a_weight_packed_from_plain_codes(m, n, k):
    w = synth.weights(9400 + n, n, k, "bf16")
    rq, rs, rc = O.quantize_weight(w)
    wq = pdq.pack_int8(torch.from_numpy(rq).cuda())
    x = synth.activations(9410 + m, m, k, [2, k - 3], 100.0, dtype="bf16")
    res = pdq.linear_prefill(dev(x, "bf16"), wq, torch.from_numpy(rs).cuda(), want_acc=True)
    xq_ref, sx_ref = O.quantize_rows_absmax(x)
    acc = O.int_matmul(xq_ref, rq)
    assert np.array_equal(host(res["acc"]), acc)
    check_16bit(host(res["y"]), O.dequantize(acc, sx_ref, rs), "bf16", exact=True)
    # the codes read back as a plain matrix on the device
    assert np.array_equal(host(pdq.unpack_int8(res["xq"].data, m, k)), xq_ref)


def test_decode_fused_strided_rows():
    m, n, k = 6, 300, 1024
    wide = synth.activations(4900, m, k + 48, [5], 100.0, offset=0.1, dtype="bf16")
    x = wide[:, :k]
    s, z = F32(0.9), 4
    wq, ws, cs, (rq, rs, rc) = weight_case(synth.weights(4901, n, k, "bf16"), "bf16")
    xt = dev(wide, "bf16")[:, :k]
    assert xt.stride(0) == k + 48
    res = pdq.linear_decode(xt, s, z, wq, ws, cs, want_acc=True)
    ref = O.linear_decode(np.ascontiguousarray(x), s, z, rq, rs, rc)
    assert codes_equal(res["xq"], ref["xq"])
    assert np.array_equal(host(res["acc"]), ref["acc"])
    check_16bit(host(res["y"]), ref["y32"], "bf16", True)


def test_decode_saturation_counted():
    x = synth.activations(4400, 8, 256, [3, 9], 100.0, offset=0.1, dtype="bf16")
    ref = decode_case(x, synth.weights(4401, 64, 256, "bf16"), "bf16", 0.05, 17)
    assert ref["sat"] > 0


# ---------------------------------------------------------------------------
# LLM.int8(): vector-wise INT8 + 16-bit outlier decomposition
# ---------------------------------------------------------------------------

def outlier_case(x, w, dtype, thr, bias=None, max_out=64, rows=None):
    wq, ws, _, (rq, rs, _) = weight_case(w, dtype)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    y, y_check = gapped(x.shape[0], w.shape[0], torch.float16 if dtype == "f16" else torch.bfloat16)
    with guarded():
        res = pdq.linear_int8_outlier(dev(x, dtype), thr, wq, ws, dev(w, dtype), b, max_outliers=max_out,
                                      want_acc=True, out=y)
    y_check()
    cols = O.outlier_columns(x, thr)
    cnt = int(host(res["count"])[0])
    assert cnt == len(cols)
    assert host(res["idx"])[:min(cnt, max_out)].tolist() == cols[:max_out].tolist()
    xq_ref, sx_ref = O.quantize_rows_regular(x, cols)
    assert codes_equal(res["xq"], xq_ref)
    assert np.array_equal(host(res["x_scale"]).view(np.uint32), sx_ref.view(np.uint32))
    r = np.arange(x.shape[0]) if rows is None else rows
    ref = O.linear_int8_outlier(x[r], w, rq, rs, thr, bias) if rows is None else None
    if rows is not None:
        # the sampled rows see the full-batch outlier set
        acc = O.int_matmul(xq_ref[r], rq)
        y64 = O.dequantize(acc, sx_ref[r], rs).astype(np.float64)
        y64 += x[r][:, cols].astype(np.float64) @ w[:, cols].astype(np.float64).T
        if bias is not None:
            y64 += bias.astype(np.float64)[None, :]
        ref = dict(acc=acc, y64=y64)
    assert np.array_equal(host(res["acc"])[r], ref["acc"])
    if cnt <= max_out:
        check_16bit(host(res["y"])[r], ref["y64"], dtype, exact=False)
    return res, cnt


def test_outlier_worked_example_on_gpu():
    """The LLM.int8 page's figure matrix, padded with zero columns to K = 16."""
    from test_oracle_pins import outlier_fixture
    x5, g = outlier_fixture()
    x = np.zeros((3, 16), F32)
    x[:, :5] = x5
    w = synth.weights(5000, 4, 16, "f16")
    res, cnt = outlier_case(x, w, "f16", g["threshold"])
    assert cnt == 2 and host(res["idx"])[:2].tolist() == [0, 2]
    assert host(res["xq"])[0, :5].tolist() == [0, 127, 0, -64, 64]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("m,n,k", [(300, 700, 1040), (64, 256, 8192), (5, 3, 32)])
def test_outlier_ragged(dtype, m, n, k):
    x = synth.normal(5100 + m, (m, k))
    cols = synth.choose_channels(5200 + k, k, min(8, k // 4))
    x[:, cols] = synth.normal(5300, (m, len(cols)), 60.0)
    x = synth.round_to(x, dtype)
    outlier_case(x, synth.weights(5400 + n, n, k, dtype), dtype, 6.0, bias=synth.bias(5500, n))


def test_outlier_threshold_infinite_equals_vector_wise():
    x = synth.activations(5600, 70, 256, [4, 100], 100.0, dtype="f16")
    w = synth.weights(5601, 90, 256, "f16")
    res, cnt = outlier_case(x, w, "f16", float("inf"))
    assert cnt == 0
    wq, ws, _ = pdq.quantize_weight(dev(w, "f16"))
    pre = pdq.linear_prefill(dev(x, "f16"), wq, ws, want_acc=True)
    assert torch.equal(pre["xq"].data, res["xq"].data) and torch.equal(pre["acc"], res["acc"])


def test_outlier_all_columns_is_16bit_matmul():
    x = synth.activations(5700, 20, 64, [], dtype="f16")
    w = synth.weights(5701, 48, 64, "f16")
    res, cnt = outlier_case(x, w, "f16", -1.0, max_out=64)
    assert cnt == 64 and not res["xq"].data.any() and not res["acc"].any()


def test_outlier_capacity_exceeded_poisons_output():
    x = synth.activations(5800, 16, 64, [], dtype="f16")
    w = synth.weights(5801, 32, 64, "f16")
    res, cnt = outlier_case(x, w, "f16", -1.0, max_out=16)
    assert cnt == 64
    assert torch.isnan(res["y"].float()).all()


def test_outlier_capacity_beyond_fused_gather():
    """A capacity of 5000 columns with 3 outliers spread over K = 8192, one of
    them the last column: the capacity sets only the pitch of X_out and W_out."""
    k = 8192
    x = synth.normal(5900, (33, k))
    cols = [3, 4100, k - 1]
    x[:, cols] = synth.normal(5901, (33, len(cols)), 60.0)
    x = synth.round_to(x, "f16")
    res, cnt = outlier_case(x, synth.weights(5902, 40, k, "f16"), "f16", 6.0, max_out=5000)
    assert cnt == 3


@pytest.mark.parametrize("k", [1024, 4096])
def test_outlier_more_columns_than_a_workgroup_has_threads(k):
    """300 outlier columns (304 with the zero padding), more than the 256
    threads of a gather workgroup: X_out and W_out are gathered by loops over
    the columns, on the wavefront-per-row quantizer (K = 1024) and on the
    workgroup-per-row one (K = 4096); 203 weight rows end in a short gather
    slab."""
    m, n = 40, 203
    x = synth.normal(6100 + k, (m, k))
    cols = synth.choose_channels(6200 + k, k, 300)
    x[:, cols] = synth.normal(6300 + k, (m, len(cols)), 60.0)
    x = synth.round_to(x, "f16")
    res, cnt = outlier_case(x, synth.weights(6400 + k, n, k, "f16"), "f16", 6.0,
                            bias=synth.bias(6500, n), max_out=512)
    assert cnt == 300


def test_outlier_single_hits_in_far_row_blocks():
    """One outlier element in the first and one in the last row of a tall batch
    (32 row blocks, the last one short), the rest regular; x with a row pitch
    wider than K gives the same result as a dense copy."""
    m, k, n = 3001, 256, 72
    x = synth.normal(6000, (m, k))
    x[0, k - 1] = 40.0
    x[m - 1, 5] = -9.5
    x = synth.round_to(x, "bf16")
    res, cnt = outlier_case(x, synth.weights(6001, n, k, "bf16"), "bf16", 6.0)
    assert cnt == 2 and host(res["idx"])[:2].tolist() == [5, k - 1]
    wide = torch.zeros((m, k + 40), dtype=torch.bfloat16, device="cuda")
    wide[:, :k] = dev(x, "bf16")
    w = dev(synth.weights(6001, n, k, "bf16"), "bf16")
    wq, ws, _ = pdq.quantize_weight(w)
    a = pdq.linear_int8_outlier(wide[:, :k], 6.0, wq, ws, w)
    b = pdq.linear_int8_outlier(wide[:, :k].contiguous(), 6.0, wq, ws, w)
    for key in ("y", "x_scale", "count"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["xq"].data, b["xq"].data)
    assert torch.equal(a["idx"][:2], b["idx"][:2])


def test_outlier_llm_int8_full():
    c = synth.LlmInt8()
    x, w = c.x(), c.w()
    res, cnt = outlier_case(x, w, c.dtype, c.threshold)
    print(f"LLM.int8 full: {cnt} outlier columns: {host(res['idx'])[:cnt].tolist()}")
    assert cnt >= c.n_outlier_cols


# ---------------------------------------------------------------------------
# building blocks: quantize once, GEMM against several weights
# ---------------------------------------------------------------------------

def test_decoder_block_linear_set():
    """The decoder-block workload at full size: QKV 4096->12288, O 4096->4096,
    gate+up 4096->28672, down 14336->4096, one INT8 weight copy per linear
    serving both phases.  Prefill: 8192 tokens per-token dynamic (codes,
    scales, accumulators and outputs of every token).  Calibration: 50
    batches of 512 tokens.  Decode: all 256 steps at batch 32 through the same
    weight buffers (codes, saturation counts, accumulators and outputs of
    every step; the oracle's rows are independent, so it evaluates the 256
    steps as one 8192-row product)."""
    c = synth.DecoderBlock()
    B, T = c.decode_batch, c.decode_steps
    for l, (name, n, k) in enumerate(c.linears):
        print(f"[block] {name}: {n} x {k}", flush=True)
        wq, ws, cs, (rq, rs, rc) = weight_case(c.w(l), c.dtype)
        x = c.prefill_x(l)
        res = pdq.linear_prefill(dev(x, c.dtype), wq, ws, want_acc=True)
        xq_ref, sx_ref = O.quantize_rows_absmax(x)
        assert codes_equal(res["xq"], xq_ref)
        assert np.array_equal(host(res["x_scale"]).view(np.uint32), sx_ref.view(np.uint32))
        del x
        acc = O.int_matmul(xq_ref, rq)
        assert np.array_equal(host(res["acc"]), acc)
        del res["acc"]
        check_16bit(host(res["y"]), O.dequantize(acc, sx_ref, rs), "bf16", exact=True)
        del res, acc, xq_ref
        cal = [c.calib(l, b) for b in range(50)]
        mm = pdq.minmax_state("cuda")
        for b, xb in enumerate(cal):
            out = pdq.calibrate_static(dev(xb, c.dtype), mm, finalize=b == len(cal) - 1)
        _, s, z = O.calibrate(cal)
        del cal
        assert host(out[0]).view(np.uint32)[0] == np.array([s], F32).view(np.uint32)[0] and int(host(out[1])[0]) == z
        sat = torch.zeros(1, dtype=torch.int32, device="cuda")
        xs = np.stack([c.decode_x(l, t) for t in range(T)])          # [T, B, k]
        acc_all = torch.empty((T, B, n), dtype=torch.int32, device="cuda")
        y_all = torch.empty((T, B, n), dtype=torch.bfloat16, device="cuda")
        codes = []
        for t in range(T):
            res = pdq.linear_decode(dev(xs[t], c.dtype), s, z, wq, ws, cs, sat_count=sat, want_acc=True,
                                    out=y_all[t])
            acc_all[t] = res["acc"]
            codes.append(res["xq"])
        ref = O.linear_decode(xs.reshape(T * B, k), s, z, rq, rs, rc)
        for t in range(T):
            assert codes_equal(codes[t], ref["xq"][t * B:(t + 1) * B]), t
        assert int(host(sat)[0]) == ref["sat"]
        assert np.array_equal(host(acc_all).reshape(T * B, n), ref["acc"])
        check_16bit(host(y_all).reshape(T * B, n), ref["y32"], "bf16", exact=True)
        print(f"[block] {name}: S={s} Z={z}, {ref['sat']} saturated decode values", flush=True)
        del xs, ref, codes, acc_all, y_all


def test_per_token_blocks_shared_activation():
    x = synth.activations(6000, 200, 1024, [7, 900], 100.0, dtype="bf16")
    xq, xs = pdq.quantize_per_token(dev(x, "bf16"))
    xq_ref, sx_ref = O.quantize_rows_absmax(x)
    assert codes_equal(xq, xq_ref) and np.array_equal(host(xs), sx_ref)
    for n in (96, 300):  # e.g. two projections of one hidden state
        w = synth.weights(6001 + n, n, 1024, "bf16")
        wq, ws, _ = pdq.quantize_weight(dev(w, "bf16"))
        rq, rs, _ = O.quantize_weight(w)
        res = pdq.gemm_per_token(xq, xs, wq, ws, want_acc=True)
        acc = O.int_matmul(xq_ref, rq)
        assert np.array_equal(host(res["acc"]), acc)
        check_16bit(host(res["y"]), O.dequantize(acc, sx_ref, rs), "bf16", exact=True)


def test_static_blocks():
    x = synth.activations(6100, 24, 512, [3], 100.0, offset=0.1, dtype="f16")
    s, z = F32(1.7), -5
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    xq = pdq.quantize_static(dev(x, "f16"), s, z, sat_count=sat)
    ref_q, ref_sat = O.quantize_static(x, s, z)
    assert codes_equal(xq, ref_q) and int(host(sat)[0]) == ref_sat
    w = synth.weights(6101, 130, 512, "f16")
    wq, ws, cs = pdq.quantize_weight(dev(w, "f16"))
    rq, rs, rc = O.quantize_weight(w)
    res = pdq.gemm_static(xq, s, z, wq, ws, cs, want_acc=True)
    acc = O.int_matmul(ref_q, rq)
    assert np.array_equal(host(res["acc"]), acc)
    check_16bit(host(res["y"]), O.dequantize(O.zero_point_correct(acc, rc, z), s, rs), "bf16", exact=True)


@pytest.mark.parametrize("m,n,k", [(1, 4096, 4096), (1, 33, 1040), (1, 7, 16), (2, 300, 4096),
                                   (16, 100, 3072), (17, 64, 512), (1, 50, 4112)])
def test_static_gemm_skinny(m, n, k):
    # the GEMM alone on already-quantized activations (packed on the host
    # from the layout's definition), on the skinny kernel
    xq = synth.random_int8(6200 + m, (m, k))
    s, z = F32(0.37), -11
    w = synth.weights(6201 + n, n, k, "bf16")
    wq, ws, cs, (rq, rs, rc) = weight_case(w, "bf16")
    bias = synth.bias(6202, n)
    res = pdq.gemm_static(pdq.Codes(torch.from_numpy(pack(xq)).cuda(), m, k), s, z, wq, ws, cs,
                          torch.from_numpy(bias).cuda(), want_acc=True)
    acc = O.int_matmul(xq, rq)
    assert np.array_equal(host(res["acc"]), acc)
    check_16bit(host(res["y"]), O.dequantize(O.zero_point_correct(acc, rc, z), s, rs, bias), "bf16", exact=True)


# ---------------------------------------------------------------------------
# rounding at and around the ties: inputs at (k + 1/2) S and a few ulps away
# ---------------------------------------------------------------------------

def _near_ties(s, kmax, ulps=3):
    k = np.arange(-kmax, kmax, dtype=np.float64)
    base = ((k + 0.5) * np.float64(s)).astype(F32)
    vals = [base]
    up, down = base.copy(), base.copy()
    for _ in range(ulps):
        up = np.nextafter(up, F32(np.inf))
        down = np.nextafter(down, F32(-np.inf))
        vals += [up, down]
    return np.concatenate(vals).astype(F32)


@pytest.mark.parametrize("m,n", [(1, 200), (5, 200), (37, 200), (70, 200), (300, 200), (300, 4100),
                                 (2050, 2600)])
def test_gemm_ignores_code_padding(m, n):
    """Only the codes reach the results: the GEMMs (skinny with 16 and 32
    channels per workgroup, tiled for 2050 x 2600) give the same bits when the
    padding of the packed activations (rows past M, K values past K) holds
    arbitrary bytes instead of zeros."""
    k = 1040
    xq = synth.random_int8(6300 + m, (m, k))
    img = pack(xq)
    pad = pack(np.ones((m, k), np.int8)) == 0
    dirty = np.where(pad, synth.random_int8(6301 + m, img.shape), img)
    assert (dirty != img).any() or not pad.any()
    w = synth.weights(6302, n, k, "bf16")
    wq, ws, cs = pdq.quantize_weight(dev(w, "bf16"))
    xs = torch.from_numpy(np.linspace(0.01, 0.2, m, dtype=F32)).cuda()
    outs = []
    for image in (img, dirty):
        codes = pdq.Codes(torch.from_numpy(image).cuda(), m, k)
        a = pdq.gemm_static(codes, F32(0.37), -11, wq, ws, cs, want_acc=True)
        b = pdq.gemm_per_token(codes, xs, wq, ws, want_acc=True)
        outs.append([host(t) for t in (a["y"], a["acc"], b["y"], b["acc"])])
    for clean, junk in zip(*outs):
        assert np.array_equal(clean, junk)


# The largest K the library accepts with the most extreme codes: |acc - Z colsum|
# reaches 255 * 127 * 65536 = 2122383360, just inside INT32, on the skinny
# kernel (3 x 20) and the tiled GEMM (4096 x 1408), for the static zero point
# at both ends of its range, for per-token zero points, and symmetric.
@pytest.mark.parametrize("m,n", [(3, 20), (4096, 1408)])
def test_max_k_extreme_codes(m, n):
    k = 65536
    assert pdq.gemm_kernel(m, n) == ("skinny" if m == 3 else "tiled")
    xq = synth.random_int8(8000 + m, (m, k))
    xq[0, :], xq[m - 1, :] = -128, 127
    wq = synth.random_int8(8001 + m, (n, k), -127, 127)
    wq[0, :], wq[1, :] = 127, -127
    ws = np.linspace(1e-3, 2e-3, n, dtype=F32)
    cs = wq.astype(np.int64).sum(axis=1).astype(np.int32)
    codes = pdq.Codes(torch.from_numpy(pack(xq)).cuda(), m, k)
    wd = torch.from_numpy(pack_weight(wq)).cuda()
    wsd, csd = torch.from_numpy(ws).cuda(), torch.from_numpy(cs).cuda()
    rows = sample_rows(m, 6, 8002)
    acc = O.int_matmul(xq[rows], wq)
    assert acc.min() == -128 * 127 * k
    for z in (127, -128, 0):
        s = F32(0.05)
        res = pdq.gemm_static(codes, s, z, wd, wsd, csd, want_acc=True)
        assert np.array_equal(host(res["acc"])[rows], acc)
        corr = O.zero_point_correct(acc, cs, z)
        if z == 127:
            assert corr.min() == -255 * 127 * k
        check_16bit(host(res["y"])[rows], O.dequantize(corr, s, ws), "bf16", exact=True)
    za = np.where(np.arange(m) % 2 == 0, 127, -128).astype(np.int32)
    sx = np.linspace(0.01, 0.02, m, dtype=F32)
    res = pdq.gemm_per_token_asym(codes, torch.from_numpy(sx).cuda(), torch.from_numpy(za).cuda(), wd, wsd, csd,
                                  want_acc=True)
    assert np.array_equal(host(res["acc"])[rows], acc)
    corr = O.zero_point_correct(acc, cs, za[rows])
    check_16bit(host(res["y"])[rows], O.dequantize(corr, sx[rows], ws), "bf16", exact=True)


def test_per_token_rounding_near_ties():
    rows = []
    for c in (127.0, 1.0, 3.3, 0.021, 5e4, 2.0):
        s = F32(F32(c) / F32(127))
        v = _near_ties(s, 127)
        v = v[np.abs(v) < F32(c)]
        row = np.zeros(4096, F32)
        row[: v.size] = v
        row[-1] = F32(c)  # the row absmax is exactly c
        rows.append(row)
    x = np.stack(rows)
    xq, xs = pdq.quantize_per_token(dev(x, "f32"))
    q_ref, s_ref = O.quantize_rows_absmax(x)
    assert np.array_equal(host(xs), s_ref)
    assert codes_equal(xq, q_ref)


def test_per_token_asym_rounding_near_ties():
    """Per-token asymmetric codes for values a few ulps around every half-step
    of each token's own grid (the range ends placed in the row)."""
    rows = []
    for lo, hi in ((-1.0, 2.0), (0.0, 3.3), (-0.021, 0.0), (-5e4, 7e3), (-2.0, 2.0), (-0.7, 1e-3)):
        lo, hi = F32(lo), F32(hi)
        s = F32(F32(hi - lo) / F32(255))
        v = _near_ties(s, 255)
        v = v[(v > lo) & (v < hi)]
        row = np.zeros(4096, F32)
        row[: v.size] = v[:4094]
        row[-2], row[-1] = lo, hi
        rows.append(row)
    x = np.stack(rows)
    xq, xs, xz = pdq.quantize_per_token_asym(dev(x, "f32"))
    q_ref, s_ref, z_ref = O.quantize_rows_asym(x)
    assert np.array_equal(host(xs), s_ref) and np.array_equal(host(xz), z_ref)
    assert codes_equal(xq, q_ref)


@pytest.mark.parametrize("s", [0.5, 3.3963, 17.25, 1e-3])
def test_decode_fused_rounding_near_ties(s):
    # the same tie-straddling inputs through the one-launch decode path (16 rows
    # at a time), codes and saturation count against the oracle
    s = F32(s)
    v = _near_ties(s, 700)
    v = v[: (v.size // 256) * 256].reshape(-1, 256)
    w = synth.weights(5100, 40, 256, "f32")
    wq, ws, cs, (rq, rs, rc) = weight_case(w, "f32")
    for z in (0, -3, 100):
        for r0 in range(0, v.shape[0], 16):
            x = np.ascontiguousarray(v[r0:r0 + 16])
            sat = torch.zeros(1, dtype=torch.int32, device="cuda")
            res = pdq.linear_decode(dev(x, "f32"), s, z, wq, ws, cs, sat_count=sat, want_acc=True)
            ref = O.linear_decode(x, s, z, rq, rs, rc)
            assert codes_equal(res["xq"], ref["xq"])
            assert int(host(sat)[0]) == ref["sat"]
            assert np.array_equal(host(res["acc"]), ref["acc"])


@pytest.mark.parametrize("s", [0.5, 3.3963, 0.0078125, 17.25, 1e-3])
def test_static_rounding_near_ties(s):
    s = F32(s)
    v = _near_ties(s, 700)  # reaches well past the clamp on both sides
    v = v[: (v.size // 16) * 16].reshape(-1, 16)
    for z in (0, -3, 100, -128):
        sat = torch.zeros(1, dtype=torch.int32, device="cuda")
        xq = pdq.quantize_static(dev(v, "f32"), s, z, sat_count=sat)
        q_ref, sat_ref = O.quantize_static(v, s, z)
        assert codes_equal(xq, q_ref)
        assert int(host(sat)[0]) == sat_ref


# ---------------------------------------------------------------------------
# Fused SiLU(gate) * up producer + per-token quantizer
# ---------------------------------------------------------------------------

def silu_binary64_undecided(g, u, dtype):
    """Elements whose binary64 SiLU(g) * u lies within 2^-50 of its magnitude
    from a tie of the 16-bit grid: binary64 (the oracle's, or the device
    library's exponential) cannot tell which neighbour the exact value rounds
    to, so either is the oracle's answer within its own precision."""
    v = O.silu(g) * np.asarray(u, np.float64)
    sig, emin = (8, -126) if dtype == "bf16" else (11, -14)
    _, e = np.frexp(v)
    step = np.ldexp(1.0, np.maximum(e, emin + 1) - sig)
    t = v / step
    return np.abs(t - np.floor(t) - 0.5) * step <= np.abs(v) * 2.0 ** -50


def check_silu_mul_h(hv, g, u, dtype):
    """The GPU's h equals the oracle's binary64 SiLU(g) * u rounded once, bit
    for bit, except where binary64 itself cannot decide the rounding; returns
    the mask of elements that differ (allowed only there)."""
    ref = O.silu_mul(g, u, dtype)
    bad = hv.view(np.uint32) != ref.view(np.uint32)
    if bad.any():
        und = silu_binary64_undecided(g[bad], u[bad], dtype)
        assert und.all(), f"{int((~und).sum())} of {hv.size} h values differ from the oracle's"
    return bad


def _h_values(h, dtype):
    b = host(h)
    return O.bf16_bits_to_f32(b) if dtype == "bf16" else b.view(np.float16).astype(np.float32)


def silu_reference(g, u, dtype, hv):
    """The oracle's codes and scales of SiLU(g) * u; rows where the GPU's h took
    the other neighbour of a binary64-undecidable tie (see above) are taken
    from the oracle's quantizer applied to the GPU's h."""
    _, q_ref, s_ref = O.silu_mul_quantize_per_token(g, u, dtype)
    bad = check_silu_mul_h(hv, g, u, dtype)
    rows = np.nonzero(bad.any(axis=1))[0]
    if rows.size:
        q_alt, s_alt = O.quantize_rows_absmax(hv[rows])
        q_ref[rows], s_ref[rows] = q_alt, s_alt
    return q_ref, s_ref, rows.size


def silu_mul_case(g, u, dtype, halves=False):
    m, k = g.shape
    if halves:  # the two halves of one [M, 2K] gate/up buffer
        gu = dev(np.concatenate([g, u], axis=1), dtype)
        gd, ud = gu[:, :k], gu[:, k:]
    else:
        gd, ud = dev(g, dtype), dev(u, dtype)
    h, h_check = gapped(m, k, gd.dtype)
    with guarded():
        xq, xs = pdq.silu_mul_quantize_per_token(gd, ud, h=h)
    h_check()
    hv = _h_values(h, dtype)
    q_ref, s_ref, nalt = silu_reference(g, u, dtype, hv)
    # a row whose h overflowed to infinity has no finite scale: its codes are
    # outside the contract (finite inputs only) and are not compared
    inf_rows = ~np.isfinite(hv).all(axis=1)
    if inf_rows.any():
        q_ref[inf_rows] = xq.unpack()[inf_rows]
        s_ref[inf_rows] = host(xs)[inf_rows]
    assert codes_equal(xq, q_ref)
    assert np.array_equal(host(xs).view(np.uint32), s_ref.view(np.uint32))
    with guarded():
        xq2, xs2 = pdq.silu_mul_quantize_per_token(gd, ud)  # h not stored: same codes
    nb = pdq.act_bytes(m, k)
    assert torch.equal(xq2.data[:nb], xq.data[:nb]) and torch.equal(xs2, xs)
    return hv, q_ref, s_ref


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,m,k", [
    ("bf16", 1, 16), ("bf16", 37, 1040), ("bf16", 64, 4096), ("bf16", 19, 11008), ("bf16", 5, 16384),
    ("bf16", 3, 20480), ("f16", 33, 2048), ("f16", 17, 14336), ("bf16", 2, 40960), ("f16", 1, 65536),
])
def test_silu_mul_quant_shapes(dtype, m, k):
    g, u = synth.swiglu_inputs(9000 + m, m, k, dtype)
    silu_mul_case(g, u, dtype)


@pytest.mark.gpu
def test_silu_mul_quant_gate_up_halves_and_empty():
    g, u = synth.swiglu_inputs(9100, 20, 2048, "bf16")
    silu_mul_case(g, u, "bf16", halves=True)
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    xq, xs = pdq.silu_mul_quantize_per_token(e, e)
    assert xs.numel() == 0


@pytest.mark.gpu
def test_silu_mul_quant_extremes():
    k = 256
    g, u = synth.swiglu_inputs(9200, 4, k, "bf16")
    g[0, :8] = [0.0, -0.0, 100.0, -100.0, 1000.0, -1000.0, 3.0e38, -3.0e38]
    u[0, :8] = [5.0, -5.0, 1.0, 1.0, -2.0, 1.0, 0.5, 1.0]
    g[1] = 0.0                      # all-zero row: scale 1, codes 0
    g[2, :] = 40.0                  # SiLU(g) = g to binary64: exact products, ties possible
    u[2, :] = synth.round_to(np.linspace(-3, 3, k, dtype=np.float32), "bf16")
    g[3, :] = np.linspace(-95.0, 95.0, k)  # past the fast path's range, and e^-g beyond binary32
    g, u = synth.round_to(g, "bf16"), synth.round_to(u, "bf16")
    hv, q, s = silu_mul_case(g, u, "bf16")
    assert s[1] == 1.0 and not q[1].any()


@pytest.mark.gpu
def test_silu_mul_quant_extremes_f16():
    """binary16 producer: gates past the fast path's range, products in the
    binary16 subnormal range, and products around the overflow threshold
    65520 (the tie between 65504 and infinity)."""
    k = 256
    g, u = synth.swiglu_inputs(9250, 3, k, "f16")
    g[0, :64] = np.linspace(-20.0, 20.0, 64)
    u[0, :64] = np.linspace(-3.0, 3.0, 64)
    g[1, :64] = np.linspace(-4.0, 4.0, 64)
    u[1, :64] = 1e-6 * (np.arange(64) - 32)
    g[2, :64] = 8.0
    u[2, :64] = (65520.0 / 7.997317) * np.linspace(0.998, 1.002, 64)
    g, u = synth.round_to(g, "f16"), synth.round_to(u, "f16")
    hv, q, s = silu_mul_case(g, u, "f16")
    assert np.isinf(hv[2]).any() and np.isfinite(hv[2]).any()


@pytest.mark.gpu
def test_silu_mul_quant_down_projection_full():
    c = synth.DecoderBlock()
    g, u = c.down_gate_up()
    silu_mul_case(g, u, c.dtype, halves=True)


@pytest.mark.gpu
@pytest.mark.parametrize("m,n,k", [(40, 96, 1040), (300, 520, 2048), (2, 4096, 14336)])
def test_linear_prefill_silu_mul(m, n, k):
    g, u = synth.swiglu_inputs(9300 + m, m, k, "bf16")
    w = synth.weights(9400 + m, n, k, "bf16")
    wq, ws, _, (rq, rs, _) = weight_case(w, "bf16")
    gd, ud = dev(g, "bf16"), dev(u, "bf16")
    h = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    pdq.silu_mul_quantize_per_token(gd, ud, h=h)
    q_ref, s_ref, _ = silu_reference(g, u, "bf16", _h_values(h, "bf16"))
    y, y_check = gapped(m, n)
    with guarded():
        res = pdq.linear_prefill_silu_mul(gd, ud, wq, ws, want_acc=True, out=y)
    y_check()
    assert codes_equal(res["xq"], q_ref)
    assert np.array_equal(host(res["x_scale"]).view(np.uint32), s_ref.view(np.uint32))
    acc_ref = O.int_matmul(q_ref, rq)
    assert np.array_equal(host(res["acc"]), acc_ref)
    check_16bit(host(res["y"]), O.dequantize(acc_ref, s_ref, rs), "bf16", True)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,m,k", [
    ("bf16", 21, 4112), ("f16", 17, 8192), ("bf16", 33, 14336), ("f32", 5, 20480), ("bf16", 3, 32768),
    ("bf16", 2, 40960),
])
def test_quantize_per_token_long_rows(dtype, m, k):
    """Rows beyond 4096 values: a workgroup per row up to 32768, then a
    wavefront streaming the row twice; codes and scales exactly the oracle's."""
    x = synth.activations(9500 + m, m, k, synth.choose_channels(9600 + m, k, 6), 100.0, dtype=dtype)
    xq, xs = pdq.quantize_per_token(dev(x, dtype))
    q_ref, s_ref = O.quantize_rows_absmax(x)
    assert codes_equal(xq, q_ref)
    assert np.array_equal(host(xs).view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,m,k", [
    ("bf16", 21, 4112), ("f16", 9, 8192), ("bf16", 33, 14336), ("f32", 5, 20480), ("bf16", 2, 40960),
])
def test_quantize_per_token_asym_long_rows(dtype, m, k):
    """The per-token asymmetric quantizer on rows beyond 2048 values (a
    workgroup per row, min and max reduced across its waves): codes, scales
    and zero points exactly the oracle's; one row all positive, one all zero."""
    x = synth.activations(9700 + m, m, k, synth.choose_channels(9800 + m, k, 6), 100.0, offset=0.1, dtype=dtype)
    x[0] = np.abs(x[0])
    x[m - 1] = 0.0
    xq, xs, xz = pdq.quantize_per_token_asym(dev(x, dtype))
    q_ref, s_ref, z_ref = O.quantize_rows_asym(x)
    assert codes_equal(xq, q_ref)
    assert np.array_equal(host(xs).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(xz), z_ref)


@pytest.mark.gpu
@pytest.mark.parametrize("m,n,k", [(2048, 10240, 64), (2000, 10000, 128)])
def test_gemm_half_tile_last_round(m, n, k):
    """Shapes whose last round of 256x256 tiles holds at most 128 tiles in whole
    tile columns (320 tiles: 64 left over, 8 columns): those columns run as
    half tiles in a second launch.  Every epilogue, exact against the oracle."""
    assert pdq.gemm_kernel(m, n) == "tiled"
    x = synth.activations(9900 + m, m, k, synth.choose_channels(9901, k, 3), 20.0, dtype="bf16")
    w = synth.weights(9902 + m, n, k, "bf16")
    b = synth.bias(9903, n)
    prefill_case(x, w, "bf16", bias=b)
    prefill_asym_case(x, w, "bf16", bias=b)
    s, z = 0.0625, -5
    decode_case(x, w, "bf16", s, z, bias=b)


@pytest.mark.gpu
def test_outlier_half_tile_last_round():
    # 4 x 80 = 320 tiles: the last 16 tile columns as half tiles
    x = synth.activations(9910, 1000, 256, synth.choose_channels(9911, 256, 4), 50.0, dtype="f16")
    w = synth.weights(9912, 20400, 256, "f16")
    outlier_case(x, w, "f16", 6.0, bias=synth.bias(9913, 20400))
