// Device-side helpers shared by the HIP kernels of libpdq (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdq {

enum DType : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int DT>
struct Elem;
template <>
struct Elem<kF32> {
    static constexpr int bytes = 4;
};
template <>
struct Elem<kBF16> {
    static constexpr int bytes = 2;
};
template <>
struct Elem<kF16> {
    static constexpr int bytes = 2;
};

// Packed INT8 operand, the layout of every INT8 matrix of the library (the
// weight codes and the activation codes alike): groups of 16 rows x 64 K
// values, group g's K tile s a contiguous 1 KB block at
// (g * ceil(K / 64) + s) * 1024; row r of the group at r * 64 within it, its
// 16-byte chunk c (K values 16 c .. 16 c + 15 of the tile) at position
// c ^ ((r >> 2) & 3).  One block is then exactly what one global_load_lds
// instruction of the GEMM moves into its swizzled LDS tile (every request a
// whole cache line), and also one 16 x 64 fragment of the skinny kernel's
// v_mfma_i32_16x16x64_i8, loaded by one contiguous instruction.  Rows past
// the matrix (up to the next multiple of 16) and K values >= K are stored
// as 0.
constexpr int kWGroup = 16, kWTileK = 64, kWBlock = kWGroup * kWTileK;
__device__ __forceinline__ int wpack_pos(int r, int c) { return r * kWTileK + ((c ^ ((r >> 2) & 3)) << 4); }
__device__ __forceinline__ int64_t wpack_block(int64_t g, int64_t s, int64_t ktiles) {
    return (g * ktiles + s) * kWBlock;
}

// One 8-element chunk of a K-contiguous row in its storage format: 16 bytes
// for the 16-bit types, 32 bytes for binary32.
template <int DT>
struct Raw8 {
    uint4 w[DT == kF32 ? 2 : 1];
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// binary32 -> bfloat16, round to nearest, ties to even (NaN stays NaN): the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// binary32 -> binary16, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two values converted by one instruction (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32, same rounding as above), `lo` in the low half.
typedef float v2f __attribute__((ext_vector_type(2)));
template <int OUT>
__device__ __forceinline__ uint32_t f32x2_to_16(float lo, float hi) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    typedef _Float16 v2h __attribute__((ext_vector_type(2)));
    if constexpr (OUT == kF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2h));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf));
}

template <int DT>
__device__ __forceinline__ Raw8<DT> load_raw8(const void* row, int chunk) {
    Raw8<DT> r;
    const uint4* p = reinterpret_cast<const uint4*>(row) + chunk * (DT == kF32 ? 2 : 1);
    r.w[0] = p[0];
    if constexpr (DT == kF32) r.w[1] = p[1];
    return r;
}

template <int DT>
__device__ __forceinline__ Raw8<DT> zero_raw8() {
    Raw8<DT> r;
    r.w[0] = make_uint4(0, 0, 0, 0);
    if constexpr (DT == kF32) r.w[1] = make_uint4(0, 0, 0, 0);
    return r;
}

template <int DT>
__device__ __forceinline__ void widen8(const Raw8<DT>& r, float (&v)[8]) {
    if constexpr (DT == kF32) {
        v[0] = __uint_as_float(r.w[0].x);
        v[1] = __uint_as_float(r.w[0].y);
        v[2] = __uint_as_float(r.w[0].z);
        v[3] = __uint_as_float(r.w[0].w);
        v[4] = __uint_as_float(r.w[1].x);
        v[5] = __uint_as_float(r.w[1].y);
        v[6] = __uint_as_float(r.w[1].z);
        v[7] = __uint_as_float(r.w[1].w);
    } else {
        const uint32_t u[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == kBF16) {
                v[2 * i] = bf16_to_f32(u[i] & 0xffffu);
                v[2 * i + 1] = bf16_to_f32(u[i] >> 16);
            } else {
                v[2 * i] = f16_to_f32(u[i] & 0xffffu);
                v[2 * i + 1] = f16_to_f32(u[i] >> 16);
            }
        }
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

// Maximum over all 64 lanes through DPP row permutations (quad swaps, then
// the half-row and row mirrors leave every lane of a 16-lane row holding the
// row maximum) and four lane reads, instead of a chain of LDS-routed
// shuffles.  Every lane of the wavefront must be active.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_max_full(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1, 0, 3, 2]
    v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2, 3, 0, 1]
    v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Symmetric step size from an absmax: S = C / 127 (correctly rounded), 1 if C == 0.
__device__ __forceinline__ float absmax_step(float c) { return c == 0.0f ? 1.0f : c / 127.0f; }

// rne(fl(x[j] / s)) for 8 values, bit-identical to rounding the correctly
// rounded quotients, given inv = fl(1 / s) (itself correctly rounded).
// a = fl(x * inv) differs from x / s by at most (2^-23 + 2^-48) |x / s|
// (reciprocal error plus one rounding) and fl(x / s) from x / s by at most
// 2^-24 |x / s|, so |a - fl(x / s)| <= 3 * 2^-24 * |x / s|, which is below the
// window w = 2^-15 when |x / s| <= 128 (kSmall: every absmax-scaled value) and
// below w = 2^-12 when |x / s| <= 1365.  Unless a lies within w of a
// half-integer -- i.e. unless |a - rint(a)| >= 1/2 - w, a subtraction that is
// exact -- a and fl(x / s) round to the same integer (and neither is a tie).
// When any value of any lane of the wavefront is that close, the whole chunk
// takes the exact division instead (a wavefront-uniform branch, rarely
// taken).  Without kSmall, beyond |x / s| = 1365 every caller clamps the code,
// and a and fl(x / s) have the same sign and both exceed 512 in magnitude.  A
// multiply, a subtraction and half a max per value replace the ~10-instruction
// division sequence.
template <bool kSmall>
__device__ __forceinline__ void rne_quotient8(const float (&x)[8], float s, float inv, float (&r)[8]) {
    constexpr float kEdge = 0.5f - (kSmall ? 0x1p-15f : 0x1p-12f);
    float dmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float a = x[j] * inv;
        r[j] = __builtin_rintf(a);
        dmax = fmaxf(dmax, fabsf(a - r[j]));
    }
    if (__builtin_expect(__any(dmax >= kEdge), 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = __builtin_rintf(x[j] / s);
    }
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// Static codes of 8 values (decode phase): r = rne(fl(x / s)), pre-clamped to
// +-512 so that the integer conversion stays in range (the clamped value
// saturates exactly when the unclamped one does), r' = r + z, code =
// clamp(r', qmin, 127) with qmin = -128 (asymmetric grid) or -127 (symmetric,
// z = 0).  Adds the number of r' outside [qmin, 127] to nsat.  inv = fl(1 / s).
__device__ __forceinline__ uint2 static_codes8(const float (&v)[8], float s, float inv, int z, int& nsat,
                                               int qmin = -128) {
    float rq[8];
    rne_quotient8<false>(v, s, inv, rq);
    int code[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float r = fminf(fmaxf(rq[j], -512.0f), 512.0f);
        const int ri = (int)r + z;
        nsat += (ri < qmin) | (ri > 127);
        code[j] = min(max(ri, qmin), 127);
    }
    return make_uint2(pack4_i8(code[0], code[1], code[2], code[3]),
                      pack4_i8(code[4], code[5], code[6], code[7]));
}

// Float max / min through integer atomics (valid for every non-NaN value,
// including +-INF and the {+INF, -INF} starting state).  -0 is taken as +0 so
// that the sign test below routes it through the signed-integer branch.
__device__ __forceinline__ void atomic_max_f32(float* addr, float v) {
    if (v == 0.0f) v = 0.0f;
    if (v >= 0.0f)
        atomicMax(reinterpret_cast<int*>(addr), __float_as_int(v));
    else
        atomicMin(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

__device__ __forceinline__ void atomic_min_f32(float* addr, float v) {
    if (v == 0.0f) v = 0.0f;
    if (v >= 0.0f)
        atomicMin(reinterpret_cast<int*>(addr), __float_as_int(v));
    else
        atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

}  // namespace pdq
