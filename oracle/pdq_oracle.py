"""CPU oracle for the W8A8 INT8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding)
never calls it, and it shares no code with the HIP path.

Plain, slow, obviously-correct numpy, one function per step of the method,
in the order the pages give them.  Sources (cited by title and section):

  [PDMIX-term]  "PDMIX inter-phase mixed quantization" terminology entry
                (msModelSlim knowledge base), section 2.1 core idea,
                section 2.3 mathematical description, section 2.4 key
                properties.
  [PDMIX-guide] "PDMIX Parameter Configuration Workflow Guide", section 3
                process overview, section 4 step 2 (recommended qconfig) and
                step 3 (configuration item table).
  [LLM.int8]    "LLM.int8(): 8-bit Matrix Multiplication for Transformers at
                Scale" reading notes (blog.rainlin.top): part 1 section 1
                "Absmax quantization", section 2 "Zeropoint quantization"
                (four-term expansion), section 3 granularity; part 2
                "vector-wise quantization", the four-step flow (1)-(4), the
                "16-bit decomposition" and "mixed-precision decomposition".
  [HW-accel]    "Hardware acceleration of quantized operations" (apxml
                course, chapter 2): the role of compilers and runtime
                libraries (kernel fusion).

Precision.  The quantization decisions (scales, integer codes, zero point)
are taken in IEEE binary32 exactly as written: S = fl(C / 127) with a
correctly rounded division, q = rne(fl(x / S)), because the GPU takes the
same decision in the same precision and both must agree bit for bit.  The
integer contraction is exact (see int_matmul).  The dequantizing epilogue
is written out in binary32 with one rounding per operation and no fused
multiply-add: t = fl(S_x * S_w), y = fl(t * fl(float(acc'))), then
fl(y + bias).  The 16-bit side product of the outlier decomposition is
evaluated in binary64.

Readings where the pages are silent or garbled:
  * round() is round-half-to-even (np.rint);
  * symmetric codes are clamped to [-127, 127] ([LLM.int8] part 1 section 1
    gives that range); asymmetric codes to [-128, 127] ([PDMIX-term] 2.3);
  * the decode quantizer rounds first, then adds the integer zero point
    (the order of [PDMIX-term] 2.3);
  * the asymmetric MinMax scale is (max - min) / 255 over a range widened to
    contain 0, zero point Z = -128 - rne(min / S) clamped to [-128, 127];
  * an all-zero row/column (or an empty range) gets scale 1.0;
  * the outlier test is strict |x| > threshold on the column max over all
    rows of the call; the row scale of the INT8 part covers the regular
    columns only, while the weight keeps its one full-K INT8 copy.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
QMIN_SYM, QMAX_SYM = -127, 127
QMIN_ASYM, QMAX_ASYM = -128, 127


def _f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# Scales
# ---------------------------------------------------------------------------

def absmax_scale(c) -> np.ndarray:
    """S = C / 127 in binary32 for an absmax C; S = 1 where C == 0.

    [LLM.int8] part 1 section 1: the absmax maps max|X| onto 127, i.e. the
    scale factor is 127 / ||X||_inf; written as a step size S = C / 127 as in
    [PDMIX-term] 2.3 (q = round(x / S)).
    """
    c = _f32(c)
    s = (c / F32(127)).astype(F32)
    return np.where(c == 0, F32(1), s).astype(F32)


# ---------------------------------------------------------------------------
# Symmetric quantization (weights per output channel; prefill per token)
# ---------------------------------------------------------------------------

def quantize_symmetric(x, s) -> np.ndarray:
    """q = clamp(rne(fl(x / S)), -127, 127) with S broadcast along rows."""
    x = _f32(x)
    s = _f32(s)
    r = np.rint(x / s[:, None])
    return np.clip(r, QMIN_SYM, QMAX_SYM).astype(np.int8)


def quantize_rows_absmax(x):
    """Per-row absmax symmetric INT8: returns (q int8 [R,K], S float32 [R]).

    One scale per row: per-token for activations ([PDMIX-term] 2.1 and 2.3,
    prefill per-token dynamic; [PDMIX-guide] step 3, prefill is per-token
    symmetric), per output channel for weights ([PDMIX-guide] step 2,
    weight scope per_channel, symmetric, minmax).  Row-wise granularity:
    [LLM.int8] part 1 section 3.
    """
    x = _f32(x)
    c = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], F32)
    s = absmax_scale(c)
    return quantize_symmetric(x, s), s


def quantize_weight(w):
    """Offline weight quantization, one copy shared by both phases.

    Returns (wq int8 [N,K], S_w float32 [N], colsum int32 [N]) where colsum[n]
    = sum_k wq[n,k] is the per-output-channel code sum that the zero-point
    correction needs ([LLM.int8] part 1 section 2, term B*zp_a of the
    four-term expansion).  [PDMIX-term] 2.1 / 2.4: the weight quantization is
    identical in both phases, so a single quantized copy is stored.
    """
    wq, sw = quantize_rows_absmax(w)
    colsum = wq.astype(np.int64).sum(axis=1)
    assert np.all(np.abs(colsum) < 2**31)
    return wq, sw, colsum.astype(np.int32)


# ---------------------------------------------------------------------------
# Static per-tensor asymmetric calibration and quantization (decode)
# ---------------------------------------------------------------------------

def minmax_update(state, x):
    """MinMax observer: running (min, max) over every value seen so far.

    [PDMIX-term] section 3 and [PDMIX-guide] step 3: the statistics come
    from the MinMax observer.  `state` is (min, max) or None.
    """
    x = _f32(x)
    lo, hi = F32(np.min(x)), F32(np.max(x))
    if state is None:
        return lo, hi
    return min(F32(state[0]), lo), max(F32(state[1]), hi)


def minmax_finalize(state):
    """(S, Z) of the asymmetric INT8 grid [-128, 127] from a (min, max) range.

    [PDMIX-term] 2.3: decode uses an offline per-tensor scale S_tensor and
    zero point Z_tensor on the INT8 range [-128, 127]; [PDMIX-guide] section 3
    and step 3: decode measures and exports per-tensor asymmetric parameters.
    The range is widened to contain 0 so that 0 is exactly representable.
    """
    lo = min(F32(state[0]), F32(0))
    hi = max(F32(state[1]), F32(0))
    if hi == lo:
        return F32(1), 0
    s = F32(F32(hi - lo) / F32(QMAX_ASYM - QMIN_ASYM))
    z = QMIN_ASYM - int(np.rint(F32(lo / s)))
    return s, int(min(max(z, QMIN_ASYM), QMAX_ASYM))


def calibrate(batches):
    state = None
    for b in batches:
        state = minmax_update(state, b)
    s, z = minmax_finalize(state)
    return state, s, z


def quantize_static(x, s, z, qmin=QMIN_ASYM):
    """q = clamp(rne(fl(x / S)) + Z, -128, 127); also counts saturations.

    [PDMIX-term] 2.3, decode formula; 2.4: static decode scales can saturate
    on out-of-distribution inputs, so the count of values whose unclamped
    code r' = rne(x/S) + Z falls outside [-128, 127] is returned.  The float
    quotient is limited to +-512 before conversion to an integer; this
    changes neither the clamped code nor the saturation flag.  qmin =
    -127 gives the narrow range [-127, 127] of the zero-point grid below.
    """
    x = _f32(x)
    r = np.rint(x / F32(s))
    r = np.clip(r, -512, 512).astype(np.int64) + int(z)
    sat = int(np.count_nonzero((r < qmin) | (r > QMAX_ASYM)))
    return np.clip(r, qmin, QMAX_ASYM).astype(np.int8), sat


# ---------------------------------------------------------------------------
# Static per-tensor symmetric quantization (tensor-wise absmax)
# ---------------------------------------------------------------------------

def absmax_finalize(state):
    """S of the tensor-wise absmax grid from a (min, max) range: S = C / 127
    with C = max(|min|, |max|), the largest magnitude seen; S = 1 if C == 0.

    [LLM.int8] part 1 section 1: absmax quantization maps the tensor's
    largest magnitude onto 127, one scale for the whole tensor by default
    (section 3, tensor-wise); taken here with static activation parameters,
    measured offline over calibration batches: the conventional static W8A8
    scheme, with static activation scales, that [PDMIX-term] section 2
    compares PDMIX with.
    """
    if F32(state[0]) > F32(state[1]):  # no value seen yet
        return F32(1)
    c = max(abs(F32(state[0])), abs(F32(state[1])))
    return F32(absmax_scale(np.array([c], F32))[0])


def calibrate_absmax(batches):
    state = None
    for b in batches:
        state = minmax_update(state, b)
    return state, absmax_finalize(state)


def quantize_static_sym(x, s):
    """q = clamp(rne(fl(x / S)), -127, 127) with one static S; also counts the
    values whose rne(x / S) leaves [-127, 127] (inputs beyond the calibrated
    magnitude, the static-scale saturation risk of [PDMIX-term] 2.4)."""
    x = _f32(x)
    r = np.rint(x / F32(s))
    sat = int(np.count_nonzero(np.abs(r) > QMAX_SYM))
    return np.clip(r, QMIN_SYM, QMAX_SYM).astype(np.int8), sat


def linear_static_sym(x, s, wq, sw, bias=None):
    """Static tensor-wise symmetric W8A8 linear: y = (S * S_w[n]) * acc (+ bias).

    Returns dict(xq, sat, acc, y32).
    """
    xq, sat = quantize_static_sym(x, s)
    acc = int_matmul(xq, wq)
    assert np.all(np.abs(acc) < 2**31)
    return dict(xq=xq, sat=sat, acc=acc, y32=dequantize(acc, F32(s), sw, bias))


# ---------------------------------------------------------------------------
# Static tensor-wise zero-point quantization (254 levels)
# ---------------------------------------------------------------------------

def zeropoint_finalize(state):
    """(S, Z) of the zero-point grid of [LLM.int8] part 1 section 2: the range
    is spread over 2 * 127 steps, nd_x = 254 / (max - min), i.e. a step
    S = (max - min) / 254, and the minimum lands on -127, so that codes fill
    [-127, 127].  The page's own formulas for the zero point and the code are
    garbled; taken here in the same form as the decode phase's grid (range
    widened to contain 0, codes rne(x / S) + Z): Z = clamp(-127 - rne(lo /
    S), -127, 127); S = 1 and Z = 0 for an empty range.
    """
    lo = min(F32(state[0]), F32(0))
    hi = max(F32(state[1]), F32(0))
    if hi == lo:
        return F32(1), 0
    s = F32(F32(hi - lo) / F32(2 * QMAX_SYM))
    z = QMIN_SYM - int(np.rint(F32(lo / s)))
    return s, int(min(max(z, QMIN_SYM), QMAX_SYM))


def calibrate_zeropoint(batches):
    state = None
    for b in batches:
        state = minmax_update(state, b)
    s, z = zeropoint_finalize(state)
    return state, s, z


def quantize_zeropoint(x, s, z):
    """q = clamp(rne(fl(x / S)) + Z, -127, 127) and the saturation count."""
    return quantize_static(x, s, z, qmin=QMIN_SYM)


def linear_zeropoint(x, s, z, wq, sw, colsum, bias=None):
    """Static tensor-wise zero-point W8A8 linear: y = (S * S_w[n]) * (acc - Z * colsum[n]).

    The GEMM removes the zero point through the weight code sums, the
    four-term expansion of [LLM.int8] part 1 section 2 with a symmetric
    weight.  Returns dict(xq, sat, acc (raw), y32).
    """
    xq, sat = quantize_zeropoint(x, s, z)
    acc = int_matmul(xq, wq)
    acc_c = zero_point_correct(acc, colsum, z)
    return dict(xq=xq, sat=sat, acc=acc, y32=dequantize(acc_c, F32(s), sw, bias))


# ---------------------------------------------------------------------------
# Per-token dynamic asymmetric quantization (prefill with Z_token)
# ---------------------------------------------------------------------------

def quantize_rows_asym(x):
    """Per-token dynamic asymmetric INT8: (q int8 [R,K], S float32 [R], Z int32 [R]).

    [PDMIX-term] 2.3, the prefill formula with its per-token zero point:
    Q = clamp(round(X / S_token) + Z_token, -128, 127), where S_token and
    Z_token are computed online from each token's own values.  A token's
    (S, Z) are those of the MinMax asymmetric grid of its range -- the
    decode phase's per-tensor parameters (minmax_finalize), one token at a
    time -- and its codes follow the decode formula with them
    (quantize_static).  The range of a token always covers its values, so
    nothing saturates.
    """
    x = _f32(x)
    rows = x.shape[0]
    q = np.zeros(x.shape, np.int8)
    s = np.ones(rows, F32)
    z = np.zeros(rows, np.int32)
    for r in range(rows):
        if x.shape[1] == 0:
            continue
        s[r], z[r] = minmax_finalize(minmax_update(None, x[r]))
        q[r], _ = quantize_static(x[r:r + 1], s[r], z[r])
    return q, s, z


# ---------------------------------------------------------------------------
# INT8 x INT8 -> INT32 contraction and the dequantizing epilogue
# ---------------------------------------------------------------------------

def int_matmul(a, b) -> np.ndarray:
    """acc[m, n] = sum_k a[m, k] * b[n, k] exactly, returned as int64.

    [LLM.int8] part 2 step (3): INT8 x INT8 products overflow 8 bits, so they
    are accumulated in INT32.  Evaluated with a binary64 matrix product:
    every product is an integer of magnitude <= 2^14 and every partial sum
    has magnitude < 2^53, so each addition in any order is exact.
    """
    a = np.asarray(a)
    b = np.asarray(b)
    k = a.shape[1]
    assert b.shape[1] == k
    assert 128 * 128 * k < 2**53
    acc = a.astype(np.float64) @ b.astype(np.float64).T
    return np.rint(acc).astype(np.int64)


def zero_point_correct(acc, colsum, z):
    """acc' = acc - Z * colsum[n]: the activation zero point removed.

    [LLM.int8] part 1 section 2 expands a zero-point product into four terms.
    With a symmetric weight (zp_b = 0) the expansion reduces to
    sum_k (q_a - Z) q_b = sum_k q_a q_b - Z * sum_k q_b.  Z is one per-tensor
    value, or one value per row of acc (per-token zero points).
    """
    acc = np.asarray(acc, dtype=np.int64)
    colsum = np.asarray(colsum, dtype=np.int64)[None, :]
    z = np.asarray(z, dtype=np.int64)
    if z.ndim == 0:
        if z:
            acc = acc - z * colsum
    else:
        acc = acc - z.reshape(-1)[:, None] * colsum
    assert np.all(np.abs(acc) < 2**31), "accumulator leaves int32"
    return acc


def dequantize(acc, sx, sw, bias=None) -> np.ndarray:
    """y = fl(fl(S_x[m] * S_w[n]) * fl(acc[m, n])) (+ bias[n]) in binary32.

    [LLM.int8] part 2, vector-wise quantization and step (4): each output
    element is rescaled by the outer product of the row (token) scale and
    the column (output channel) scale; [PDMIX-term] 2.3 gives the same
    dequantization as S * (q - Z) per operand.
    """
    sx = _f32(sx).reshape(-1)
    sw = _f32(sw).reshape(-1)
    if sx.size == 1:
        sx = np.full(np.asarray(acc).shape[0], sx[0], F32)
    t = (sx[:, None] * sw[None, :]).astype(F32)
    y = (t * np.asarray(acc).astype(F32)).astype(F32)
    if bias is not None:
        y = (y + _f32(bias)[None, :]).astype(F32)
    return y


# ---------------------------------------------------------------------------
# The two PDMIX phases
# ---------------------------------------------------------------------------

def linear_prefill(x, wq, sw, bias=None):
    """Prefill: per-token dynamic symmetric activations ([PDMIX-term] 2.3).

    Returns dict(xq, x_scale, acc, y32).
    """
    xq, sx = quantize_rows_absmax(x)
    acc = int_matmul(xq, wq)
    assert np.all(np.abs(acc) < 2**31)
    return dict(xq=xq, x_scale=sx, acc=acc, y32=dequantize(acc, sx, sw, bias))


def linear_prefill_asym(x, wq, sw, colsum, bias=None):
    """Prefill with per-token dynamic asymmetric activations ([PDMIX-term] 2.3,
    the prefill formula with Z_token): y = S_x[m] S_w[n] (acc - Z_x[m] colsum[n]).

    Returns dict(xq, x_scale, x_zp, acc (raw, before the zero-point term), y32).
    """
    xq, sx, zx = quantize_rows_asym(x)
    acc = int_matmul(xq, wq)
    acc_c = zero_point_correct(acc, colsum, zx)
    return dict(xq=xq, x_scale=sx, x_zp=zx, acc=acc, y32=dequantize(acc_c, sx, sw, bias))


def linear_decode(x, s, z, wq, sw, colsum, bias=None):
    """Decode: per-tensor static asymmetric activations ([PDMIX-term] 2.3).

    Returns dict(xq, sat, acc (raw, before the zero-point term), y32).
    """
    xq, sat = quantize_static(x, s, z)
    acc = int_matmul(xq, wq)
    acc_c = zero_point_correct(acc, colsum, z)
    return dict(xq=xq, sat=sat, acc=acc, y32=dequantize(acc_c, F32(s), sw, bias))


# ---------------------------------------------------------------------------
# LLM.int8() vector-wise quantization with the 16-bit outlier decomposition
# ---------------------------------------------------------------------------

def outlier_columns(x, threshold) -> np.ndarray:
    """Ascending indices k with max_m |x[m, k]| > threshold.

    [LLM.int8] part 2, 16-bit decomposition step (1) and mixed-precision
    decomposition step 1: the hidden dimensions (columns of X) whose
    magnitude exceeds the threshold (6.0 in the text) are outliers.
    """
    x = _f32(x)
    if x.shape[0] == 0:
        return np.zeros(0, np.int64)
    colmax = np.max(np.abs(x), axis=0)
    return np.nonzero(colmax > F32(threshold))[0].astype(np.int64)


def quantize_rows_regular(x, cols):
    """Row absmax over the regular columns only; outlier columns coded 0.

    [LLM.int8] part 2 step (1): C_x is the row absmax; the mixed-precision
    formula quantizes X_normal only, so the outlier columns take no part in
    C_x and contribute nothing to the INT8 product.
    """
    x = _f32(x)
    keep = np.ones(x.shape[1], bool)
    keep[np.asarray(cols, dtype=np.int64)] = False
    xr = np.where(keep[None, :], x, F32(0))
    c = np.max(np.abs(xr), axis=1) if x.shape[1] else np.zeros(x.shape[0], F32)
    s = absmax_scale(c)
    q = quantize_symmetric(xr, s)
    return q, s


def linear_int8_outlier(x, w16, wq, sw, threshold, bias=None):
    """Y = dequant(Q(X_normal) Q(W)) + X_outlier W_outlier (16-bit path).

    [LLM.int8] part 2: the INT8 path (steps (1)-(4)) and the 16-bit path on
    the outlier columns are computed separately and summed into a 16-bit
    output.  The weight's INT8 copy is the shared per-output-channel one.
    Returns dict(cols, xq, x_scale, acc, y64) -- y64 in binary64 before the
    final rounding to the 16-bit output dtype.
    """
    x = _f32(x)
    w16 = _f32(w16)
    cols = outlier_columns(x, threshold)
    xq, sx = quantize_rows_regular(x, cols)
    acc = int_matmul(xq, wq)
    assert np.all(np.abs(acc) < 2**31)
    y8 = dequantize(acc, sx, sw).astype(np.float64)
    side = x[:, cols].astype(np.float64) @ w16[:, cols].astype(np.float64).T
    y = y8 + side
    if bias is not None:
        y = y + _f32(bias).astype(np.float64)[None, :]
    return dict(cols=cols, xq=xq, x_scale=sx, acc=acc, y64=y)


# ---------------------------------------------------------------------------
# Fused producer: SiLU(gate) * up, then per-token INT8
# ---------------------------------------------------------------------------

def silu(g) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + e^-g) in binary64, no rounding to a
    narrower type.

    The pages define no activation function; this is the textbook SiLU (the
    gate of a SwiGLU MLP, whose product with the up projection is the input
    of the down projection).  The pages ask for the quantizer to be fused
    into the kernel that produces its input ([HW-accel], the role of
    compilers and runtime libraries: kernel fusion to cut memory traffic and
    launches).  For g -> -inf, e^-g overflows to inf and the quotient is -0,
    the limit of g * sigmoid(g).
    """
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def round_to_bf16(v) -> np.ndarray:
    """Round binary64 values straight to bfloat16 (nearest, ties to even),
    returned as binary32 (every bfloat16 value is one).

    bfloat16 has 8 significant bits and binary32's exponent range: a value
    m * 2^e (0.5 <= |m| < 1) is rounded to a multiple of 2^(e - 8); below the
    smallest normal 2^-126 the spacing stays 2^-133.  One rounding from the
    binary64 value: rounding to binary32 first and then to bfloat16 would
    round twice and can land on the wrong side of a tie.  Values that round
    beyond the largest bfloat16 become infinite.
    """
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    ex = np.maximum(e, -125)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.rint(np.ldexp(v, 8 - ex)), ex - 8)
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
    return r.astype(F32)


def silu_mul(gate, up, dtype="bf16") -> np.ndarray:
    """h = SiLU(gate) * up, evaluated in binary64 and rounded once to the
    producer's 16-bit type ("bf16" or "f16"); returned as binary32.

    Reading: the fused kernel hands the quantizer the same h that an unfused
    SiLU-and-multiply kernel would have written to memory in the model's
    16-bit type, so that fusing changes where h lives (registers instead of
    HBM), not the codes.
    """
    v = silu(gate) * np.asarray(up, np.float64)
    if dtype == "f16":
        return v.astype(np.float16).astype(F32)
    return round_to_bf16(v)


def silu_mul_quantize_per_token(gate, up, dtype="bf16"):
    """SiLU(gate) * up quantized per token: returns (h, q, S).

    The per-token dynamic symmetric quantizer of prefill ([PDMIX-term] 2.3)
    applied to the fused producer's output h (see silu_mul).
    """
    h = silu_mul(gate, up, dtype)
    q, s = quantize_rows_absmax(h)
    return h, q, s


def linear_prefill_silu_mul(gate, up, wq, sw, bias=None, dtype="bf16"):
    """Prefill linear whose input is SiLU(gate) * up (a down projection):
    returns dict(h, xq, x_scale, acc, y32)."""
    h, xq, sx = silu_mul_quantize_per_token(gate, up, dtype)
    acc = int_matmul(xq, wq)
    assert np.all(np.abs(acc) < 2**31)
    return dict(h=h, xq=xq, x_scale=sx, acc=acc, y32=dequantize(acc, sx, sw, bias))


# ---------------------------------------------------------------------------
# Output rounding
# ---------------------------------------------------------------------------

def to_bf16_bits(y) -> np.ndarray:
    """Round binary32 values to bfloat16 (nearest, ties to even); uint16 bits.

    bfloat16 keeps the upper 16 bits of a binary32 word.  The discarded low
    half is compared with one half unit of the kept part: more rounds up,
    less rounds down, exactly half rounds to the even kept value.  NaN is
    kept quiet.
    """
    u = _f32(y).view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    r = hi + up.astype(np.uint64)
    nan = np.isnan(_f32(y))
    r = np.where(nan, hi | np.uint64(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def to_f16(y) -> np.ndarray:
    """Round to IEEE binary16 (nearest, ties to even)."""
    return np.asarray(y).astype(np.float16)
