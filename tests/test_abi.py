"""The C ABI of libpdq on the host: symbols and argument validation.

Every call here is rejected by the host-side checks before anything is
enqueued (the pointers are never dereferenced), so these run without a GPU.
"""
import ctypes
import os

import numpy as np
import pytest

from w8a8_int8_quantized_absmax_amd import pdq

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5, 6
P = 0x10000  # 64 KiB-aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pdq.LIB_PATH):
        pytest.skip("libpdq.so not built")
    return pdq.lib()


def test_header_functions_all_exported(L):
    names = pdq.header_functions()
    assert set(names) == set(pdq.SIGNATURES), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in (OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, 8):
        assert L.pdq_status_string(s)
    assert L.pdq_status_string(SHAPE).startswith(b"invalid shape")


def qw(L, w=P, dt=1, N=4, K=32, ldw=32, wq=P, ws=P, cs=P):
    return L.pdq_quantize_weight(w, dt, N, K, ldw, wq, ws, cs, None)


def test_quantize_weight_validation(L):
    assert qw(L, dt=7) == DTYPE
    assert qw(L, K=17, ldw=17) == SHAPE
    assert qw(L, K=32, ldw=16) == SHAPE
    assert qw(L, N=-1) == SHAPE
    assert qw(L, K=65536 + 16, ldw=65536 + 16) == SHAPE
    assert qw(L, w=None) == NULL
    assert qw(L, wq=None) == NULL
    assert qw(L, ws=None) == NULL
    assert qw(L, w=P + 8) == ALIGN
    assert qw(L, dt=1, ldw=36) == ALIGN     # bf16 pitch 72 bytes
    assert qw(L, wq=P + 4) == ALIGN
    assert qw(L, N=0) == OK                # nothing to do, nothing launched


def pre(L, x=P, dt=1, M=8, K=64, ldx=64, wq=P, ws=P, bias=None, N=16, xq=P, xs=P, y=P, ldy=16, acc=None):
    return L.pdq_linear_prefill(x, dt, M, K, ldx, wq, ws, bias, N, xq, xs, y, ldy, acc, None)


def test_prefill_validation(L):
    assert pre(L, dt=3) == DTYPE
    assert pre(L, K=40, ldx=40) == SHAPE
    assert pre(L, ldy=15) == SHAPE
    assert pre(L, N=-2) == SHAPE
    assert pre(L, x=None) == NULL
    assert pre(L, xq=None) == NULL
    assert pre(L, xs=None) == NULL
    assert pre(L, y=None) == NULL
    assert pre(L, ws=None) == NULL
    assert pre(L, wq=P + 1) == ALIGN
    assert pre(L, y=P + 1) == ALIGN
    assert pre(L, bias=P + 2) == ALIGN
    assert pre(L, M=0) == OK


def dec(L, x=P, dt=1, M=4, K=64, ldx=64, s=0.5, z=-3, wq=P, ws=P, cs=P, bias=None, N=16, xq=P, y=P,
        ldy=16, acc=None, sat=None):
    return L.pdq_linear_decode(x, dt, M, K, ldx, s, z, wq, ws, cs, bias, N, xq, y, ldy, acc, sat, None)


def test_pack_validation(L):
    pk, up = L.pdq_pack_int8, L.pdq_unpack_int8
    assert pk(P, 4, 40, 48, P, None) == SHAPE          # K not a multiple of 16
    assert pk(P, 4, 64, 32, P, None) == SHAPE          # pitch below K
    assert pk(None, 4, 64, 64, P, None) == NULL
    assert pk(P, 4, 64, 64, None, None) == NULL
    assert pk(P + 8, 4, 64, 64, P, None) == ALIGN
    assert pk(P, 4, 64, 72, P, None) == ALIGN          # row pitch not 16-byte aligned
    assert pk(P, 4, 64, 64, P + 4, None) == ALIGN
    assert pk(P, 0, 64, 64, None, None) == OK
    assert up(P, 4, 40, P, 48, None) == SHAPE
    assert up(None, 4, 64, P, 64, None) == NULL
    assert up(P, 4, 64, None, 64, None) == NULL
    assert up(P + 4, 4, 64, P, 64, None) == ALIGN
    assert up(P, 4, 64, P, 80 + 8, None) == ALIGN
    assert up(P, 0, 64, None, 64, None) == OK


def test_decode_validation(L):
    assert dec(L, dt=-1) == DTYPE
    assert dec(L, K=8, ldx=8) == SHAPE
    assert dec(L, s=0.0) == UNSUP
    assert dec(L, s=-1.0) == UNSUP
    assert dec(L, s=float("inf")) == UNSUP
    assert dec(L, s=float("nan")) == UNSUP
    assert dec(L, z=128) == UNSUP
    assert dec(L, z=-129) == UNSUP
    assert dec(L, cs=None) == NULL
    assert dec(L, xq=None) == NULL
    assert dec(L, sat=P + 2) == ALIGN
    assert dec(L, M=0) == OK


def test_calibrate_validation(L):
    f = L.pdq_calibrate_static
    assert f(P, 1, 4, 64, 64, None, None, None, None) == NULL     # no state
    assert f(P, 1, 4, 64, 64, P, P, None, None) == NULL          # scale without zero point
    assert f(P, 5, 4, 64, 64, P, None, None, None) == DTYPE
    assert f(P, 1, 4, 60, 64, P, None, None, None) == SHAPE
    assert f(P, 1, 4, 64, 64, P + 2, None, None, None) == ALIGN


def test_outlier_workspace_size(L):
    ws = L.pdq_linear_int8_outlier_workspace
    # predicate bytes (row blocks x pitch, pitch = ceil16(K / 8); at most 32 row
    # blocks of ceil32(ceil(M / 32)) rows) + mask (pitch) + X_out (M x P f16)
    # + W_out (N x P f16), each 256-aligned, P = ceil16(max)
    assert ws(2048, 28672, 8192, 64) == 32 * 1024 + 1024 + 2048 * 64 * 2 + 28672 * 64 * 2
    assert ws(3, 5, 16, 1) == 4 * 256
    assert ws(3, 5, 16, 0) == 2 * 256
    assert ws(0, 5, 16, 1) == 2 * 256  # no predicate rows, no X_out
    assert ws(-1, 5, 16, 1) == 0


def out8(L, x=P, dt=2, M=8, K=64, ldx=64, thr=6.0, wq=P, ws=P, w16=P, ldw=64, bias=None, N=16, y=P,
         ldy=16, xq=P, xs=P, idx=P, cnt=P, maxo=8, work=P, work_bytes=1 << 20, acc=None):
    return L.pdq_linear_int8_outlier(x, dt, M, K, ldx, thr, wq, ws, w16, ldw, bias, N, y, ldy, xq, xs,
                                     idx, cnt, maxo, work, work_bytes, acc, None)


def test_outlier_validation(L):
    assert out8(L, dt=0) == DTYPE      # the 16-bit path takes F16 or BF16 only
    assert out8(L, thr=float("nan")) == UNSUP
    assert out8(L, maxo=65) == SHAPE
    assert out8(L, maxo=-1) == SHAPE
    assert out8(L, cnt=None) == NULL
    assert out8(L, idx=None) == NULL
    assert out8(L, w16=None) == NULL
    assert out8(L, work=None) == WS
    need = L.pdq_linear_int8_outlier_workspace(8, 16, 64, 8)
    assert out8(L, work_bytes=need - 1) == WS
    assert out8(L, work=P + 16) == ALIGN
    assert out8(L, w16=P + 1) == ALIGN


def test_k_zero_is_refused_before_any_launch(L):
    """K == 0 with rows present is a shape error on every entry point (the
    pointers here are fake and never dereferenced: a launch would fault)."""
    assert qw(L, K=0, ldw=0) == SHAPE
    assert qw(L, N=0, K=0, ldw=0) == SHAPE
    assert pre(L, K=0, ldx=0) == SHAPE
    assert dec(L, K=0, ldx=0) == SHAPE
    assert out8(L, K=0, ldx=0, ldw=0, maxo=0) == SHAPE
    assert L.pdq_calibrate_static(P, 1, 4, 0, 0, P, None, None, None) == SHAPE
    assert L.pdq_quantize_per_token(P, 1, 4, 0, 0, P, P, None) == SHAPE
    assert L.pdq_quantize_per_token_asym(P, 1, 4, 0, 0, P, P, P, None) == SHAPE
    assert L.pdq_gemm_per_token(P, P, 4, 0, P, P, None, 16, P, 16, None, None) == SHAPE
    assert L.pdq_gemm_static(P, 4, 0, 0.5, 0, P, P, P, None, 16, P, 16, None, None) == SHAPE
    assert L.pdq_quantize_static(P, 1, 4, 0, 0, 0.5, 0, P, None, None) == SHAPE
    assert L.pdq_silu_mul_quantize_per_token(P, P, 1, 4, 0, 0, 0, P, P, None, 0, None) == SHAPE


def out8na(L, x=P, dt=2, M=8, K=64, ldx=64, thr=6.0, wq=P, ws=P, w16=P, ldw=64, bias=None, N=16, y=P,
           ldy=16, xq=P, xs=P, idx=P, cnt=P, maxo=8, acc=None):
    return L.pdq_linear_int8_outlier_noalloc(x, dt, M, K, ldx, thr, wq, ws, w16, ldw, bias, N, y, ldy, xq, xs,
                                             idx, cnt, maxo, acc, None)


def test_outlier_noalloc_validation(L):
    """The no-allocation variant runs the same host checks as the workspace
    call, and refuses a problem whose workspace exceeds its fixed scratch
    before any HIP call (these pointers are fake)."""
    assert L.pdq_noalloc_scratch_bytes() == 8 << 20
    assert out8na(L, dt=0) == DTYPE
    assert out8na(L, thr=float("nan")) == UNSUP
    assert out8na(L, maxo=65) == SHAPE
    assert out8na(L, K=0, ldx=0, ldw=0, maxo=0) == SHAPE
    assert out8na(L, cnt=None) == NULL
    assert out8na(L, w16=P + 1) == ALIGN
    ws = L.pdq_linear_int8_outlier_workspace
    assert ws(2048, 28672, 8192, 64) <= 8 << 20            # the LLM.int8 layer fits
    big_n = 70000
    assert ws(2048, big_n, 8192, 64) > 8 << 20
    assert out8na(L, M=2048, K=8192, ldx=8192, N=big_n, ldw=8192, ldy=big_n, maxo=64) == WS


def test_weight_bytes(L):
    # ceil(N / 16) x ceil(K / 64) blocks of 1024 bytes
    assert L.pdq_weight_bytes(11008, 4096) == 688 * 64 * 1024 == 11008 * 4096
    assert L.pdq_weight_bytes(1, 16) == 1024
    assert L.pdq_weight_bytes(257, 80) == 17 * 2 * 1024
    assert L.pdq_weight_bytes(0, 64) == 0
    assert L.pdq_weight_bytes(-1, 64) == 0


def test_act_bytes(L):
    # activation codes: the same layout, M rows in place of N channels
    for m, k in [(1, 16), (1, 4096), (17, 4096), (4096, 4096), (0, 64), (300, 1040)]:
        assert L.pdq_act_bytes(m, k) == L.pdq_weight_bytes(m, k)
    assert L.pdq_act_bytes(1, 4096) == 16 * 4096
    assert L.pdq_act_bytes(-3, 64) == 0


def test_unpack_weight_inverts_the_layout():
    """pdq.unpack_weight against the test-side packer written from the header."""
    import torch
    from packing import pack_weight
    from w8a8_int8_quantized_absmax_amd import pdq

    rng = np.random.default_rng(7)
    for n, k in [(1, 16), (300, 80), (256, 64), (513, 1040)]:
        codes = rng.integers(-127, 128, (n, k)).astype(np.int8)
        image = pack_weight(codes)
        assert image.size == -(-n // 16) * -(-k // 64) * 1024
        assert np.array_equal(pdq.unpack_weight(torch.from_numpy(image), n, k), codes)
        assert np.count_nonzero(image) == np.count_nonzero(codes)  # padding is zero
    # one chunk placed by hand: channel 21 = group 1, r = 5 (r >> 2 = 1), chunk 2
    # of K tile 1 -> position 3 of block (1, 1)
    codes = np.zeros((22, 128), np.int8)
    codes[21, 64 + 32:64 + 48] = np.arange(1, 17)
    image = pack_weight(codes)
    base = (1 * 2 + 1) * 1024 + 5 * 64 + 3 * 16
    assert image[base:base + 16].tolist() == list(range(1, 17))


def pre_asym(L, x=P, dt=1, M=8, K=64, ldx=64, wq=P, ws=P, cs=P, bias=None, N=16, xq=P, xs=P, xz=P, y=P,
             ldy=16, acc=None):
    return L.pdq_linear_prefill_asym(x, dt, M, K, ldx, wq, ws, cs, bias, N, xq, xs, xz, y, ldy, acc, None)


def test_prefill_asym_validation(L):
    assert pre_asym(L, dt=9) == DTYPE
    assert pre_asym(L, K=24, ldx=24) == SHAPE
    assert pre_asym(L, ldy=8) == SHAPE
    assert pre_asym(L, cs=None) == NULL        # the zero point needs the code sums
    assert pre_asym(L, xz=None) == NULL
    assert pre_asym(L, xs=None) == NULL
    assert pre_asym(L, xq=None) == NULL
    assert pre_asym(L, xz=P + 2) == ALIGN
    assert pre_asym(L, M=0) == OK
    q = L.pdq_quantize_per_token_asym
    assert q(P, 1, 4, 64, 64, P, P, None, None) == NULL
    assert q(P, 1, 4, 64, 64, P + 8, P, P, None) == ALIGN
    g = L.pdq_gemm_per_token_asym
    assert g(P, P, None, 4, 64, P, P, P, None, 16, P, 16, None, None) == NULL
    assert g(P, P, P, 4, 64, P, P, None, None, 16, P, 16, None, None) == NULL
    assert g(P, P, P, 0, 64, P, P, P, None, 16, P, 16, None, None) == OK


def test_static_sym_validation(L):
    lin = L.pdq_linear_static_sym

    def call(x=P, dt=1, M=4, K=64, s=0.5, ws=P, xq=P, y=P, ldy=16, sat=None):
        return lin(x, dt, M, K, K, s, P, ws, None, 16, xq, y, ldy, None, sat, None)

    assert call(dt=4) == DTYPE
    assert call(K=20) == SHAPE
    assert call(ldy=3) == SHAPE
    for s in (0.0, -2.0, float("inf"), float("nan")):
        assert call(s=s) == UNSUP
    assert call(ws=None) == NULL
    assert call(xq=None) == NULL
    assert call(sat=P + 1) == ALIGN
    assert call(M=0) == OK
    cal = L.pdq_calibrate_static_sym
    assert cal(P, 1, 4, 64, 64, None, None, None) == NULL
    assert cal(P, 1, 4, 64, 64, P, P + 2, None) == ALIGN
    qs = L.pdq_quantize_static_sym
    assert qs(P, 1, 4, 64, 64, 0.0, P, None, None) == UNSUP
    assert qs(P, 1, 4, 64, 64, 1.0, None, None, None) == NULL
    # the static GEMM needs code sums only for a nonzero zero point
    gs = L.pdq_gemm_static
    assert gs(P, 4, 64, 0.5, 3, P, P, None, None, 16, P, 16, None, None) == NULL
    assert gs(P, 0, 64, 0.5, 0, P, P, None, None, 16, P, 16, None, None) == OK


def test_gemm_kernel_choice(L):
    k = L.pdq_gemm_kernel
    assert k(0, 16) == -1 and k(16, 0) == -1
    for m in (1, 17, 64):                       # decode batches: always the skinny kernel
        assert k(m, 4096) == 0 and k(m, 28672) == 0
    assert k(4096, 11008) == 1                  # the 7B prefill linear: tiled
    assert k(8192, 4096) == 1
    assert k(256, 4096) == 0                    # a few hundred rows of a 4096-wide weight


def test_skinny_channels_choice(L):
    """Channels per workgroup of the skinny kernel: 16 up to 16 rows; beyond,
    the width that moves the fewest bytes through the busiest of 256 CUs."""
    c = L.pdq_skinny_channels
    assert c(0, 16) == -1 and c(16, 0) == -1
    for n in (4096, 12288, 28672):              # up to 16 rows: the most workgroups
        assert c(1, n) == c(8, n) == c(16, n) == 16
    assert c(32, 4096) == 16 and c(64, 4096) == 16     # O projection: 256 workgroups of 16
    # QKV: 16 channels give 3 workgroups per CU x (16 + 32) bytes per K value,
    # 48 channels exactly 256 workgroups x (48 + 32)
    assert c(32, 12288) == 48 and c(64, 12288) == 48
    assert c(32, 28672) == 64 and c(64, 28672) == 64   # gate+up: 448 workgroups of 64
    assert c(17, 5000) == 32
    assert c(96, 4096) == 32 and c(256, 4096) == 64    # beyond 64 rows: one workgroup row per 64


def test_zeropoint_validation(L):
    lin = L.pdq_linear_zeropoint

    def call(dt=1, M=4, K=64, s=0.5, z=-3, cs=P, xq=P, y=P, sat=None):
        return lin(P, dt, M, K, K, s, z, P, P, cs, None, 16, xq, y, 16, None, sat, None)

    assert call(dt=7) == DTYPE
    assert call(K=40) == SHAPE
    assert call(z=-128) == UNSUP            # the zero-point grid's codes stop at -127
    assert call(z=128) == UNSUP
    assert call(s=0.0) == UNSUP
    assert call(cs=None) == NULL
    assert call(xq=None) == NULL
    assert call(sat=P + 1) == ALIGN
    assert call(M=0) == OK
    cal = L.pdq_calibrate_zeropoint
    assert cal(P, 1, 4, 64, 64, P, P, None, None) == NULL    # scale without zero point
    assert cal(P, 1, 4, 64, 64, None, None, None, None) == NULL
    q = L.pdq_quantize_zeropoint
    assert q(P, 1, 4, 64, 64, 1.0, 127, None, None, None) == NULL
    assert q(P, 1, 4, 64, 64, 1.0, -128, P, None, None) == UNSUP


def test_silu_mul_validation(L):
    q = L.pdq_silu_mul_quantize_per_token

    def call(dt=1, M=4, K=64, ldg=128, ldu=128, xq=P, xs=P, h=None, ldh=0):
        return q(P, P + 128, dt, M, K, ldg, ldu, xq, xs, h, ldh, None)

    assert call(dt=0) == DTYPE                # binary32 producers are not accepted
    assert call(dt=5) == DTYPE
    assert call(K=40, ldg=40, ldu=40) == SHAPE
    assert call(ldu=32) == SHAPE
    assert call(xq=None) == NULL
    assert call(xs=None) == NULL
    assert call(ldg=68) == ALIGN              # row pitch of 136 bytes
    assert call(h=P, ldh=32) == SHAPE
    assert call(h=P + 2, ldh=64) == ALIGN
    assert call(M=0) == OK
    lin = L.pdq_linear_prefill_silu_mul

    def lcall(dt=2, M=4, K=64, ws=P, xq=P, y=P, ldy=16):
        return lin(P, P, dt, M, K, K, K, P, ws, None, 16, xq, P, y, ldy, None, None)

    assert lcall(dt=0) == DTYPE
    assert lcall(K=24) == SHAPE
    assert lcall(ldy=8) == SHAPE
    assert lcall(ws=None) == NULL
    assert lcall(y=None) == NULL
    assert lcall(xq=None) == NULL
    assert lcall(M=0) == OK


def test_shapes_beyond_the_launch_limits_are_refused(L):
    """Rows beyond 2^21, more than 2^34 values in one operand or 2^39 outputs
    in one product are shape errors (fake pointers: a launch would fault)."""
    big = 1 << 21
    assert qw(L, N=big + 1, K=16, ldw=16) == SHAPE
    assert pre(L, M=big + 1, K=16, ldx=16) == SHAPE
    assert pre(L, M=big, K=16384, ldx=16384) == SHAPE            # 2^35 values
    assert pre(L, M=big, N=big, K=16, ldx=16, ldy=big) == SHAPE  # 2^42 outputs
    assert dec(L, M=big + 1) == SHAPE
    assert dec(L, N=big + 1, ldy=big + 1) == SHAPE
    assert L.pdq_quantize_static(P, 1, big, 16384, 16384, 0.5, 0, P, None, None) == SHAPE
    assert L.pdq_gemm_per_token(P, P, 4, 64, P, P, None, big + 1, P, big + 1, None, None) == SHAPE
    assert L.pdq_skinny_channels(big + 1, 16) == -1
