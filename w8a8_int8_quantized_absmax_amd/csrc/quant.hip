// Activation and weight quantizers of libpdq (gfx950).
//
//  * k_quant_rows   per-row absmax symmetric INT8 -- per output channel for
//                   weights, per token for prefill activations (PDMIX
//                   terminology entry, section 2.3 prefill formula with a zero
//                   zero point; LLM.int8() notes, part 1 "Absmax
//                   quantization"), optionally skipping the outlier columns of
//                   the LLM.int8() decomposition (part 2, vector-wise step (1)
//                   on X_normal).  One wavefront per row: the row is read from
//                   HBM once with 16-byte loads, kept in registers in its
//                   storage format, reduced with cross-lane shuffles, then
//                   quantized and written as INT8 codes.
//                   ASYM: per-token dynamic asymmetric instead (the same
//                   entry's prefill formula with its per-token zero point):
//                   a row's range widened to contain 0, S = (hi - lo) / 255,
//                   Z = -128 - rne(lo / S), codes by the decode formula.
//  * k_quant_static per-tensor static asymmetric INT8 of the decode phase
//                   (PDMIX terminology entry, section 2.3 decode formula),
//                   with the saturation count of section 2.4.
//
//  * k_silu_mul_quant  the per-token quantizer fused into the producer of its
//                   input: h = SiLU(gate) * up of a SwiGLU MLP, rounded to the
//                   16-bit type, quantized like k_quant_rows without h ever
//                   leaving registers ("Hardware acceleration of quantized
//                   operations", role of compilers and runtime libraries:
//                   kernel fusion).
//
// Every code matrix is written in the packed tile layout of pdq_device.h,
// the layout the GEMMs read, padding rows and K values as zeros.
//  * k_minmax       the MinMax observer of the static calibration, and
//    k_minmax_finalize its (S, Z) (PDMIX usage guide, section 3), or the
//                   tensor-wise absmax scale S = max(|min|, |max|) / 127 of
//                   the static symmetric variant (LLM.int8() notes, part 1
//                   section 1, with a static scale), or the (S, Z) of the
//                   254-step zero-point grid (same notes, section 2).
//
// Every division is the correctly rounded binary32 division and every
// rounding to an integer is round-half-to-even (v_rndne_f32), so the codes
// and scales match a host evaluation of the same formulas bit for bit.

#include "pdq_device.h"
#include "pdq_kernels.h"

namespace pdq {

namespace {

constexpr int kRowsPerBlock = 4;  // one wavefront per row, four per workgroup

template <bool SKIP>
__device__ __forceinline__ uint32_t skip_mask(const OutlierSkip& sk, int chunk) {
    if constexpr (!SKIP)
        return 0u;
    else
        return sk.mask[chunk];
}

// W_out rows [b * wrows, ...) of the LLM.int8() decomposition: wo[n, j] =
// w16[n, idx[j]] for j < count, zeros up to the next multiple of 16, nothing
// when the count exceeds max_out.  Up to 256 columns one per thread, 256 /
// used rows at a time, eight rows' loads issued (clamped) before any of them
// is stored (the reads are scattered: a 64-byte sector per 2-byte value);
// beyond, a loop over the columns.  The index list and the count are
// published by the index kernel earlier on the stream.
__device__ __forceinline__ void gather_w_block(const OutlierSkip& sk, int64_t b) {
    const int tid = threadIdx.x;
    const int total = *sk.count;
    if (total > sk.max_out) return;
    const int used = (total + 15) / 16 * 16;
    const int64_t row0 = b * sk.wrows;
    const int nrows = (int)min((int64_t)sk.wrows, sk.N - row0);
    if (used == 0 || nrows <= 0) return;
    if (used <= 256) {
        constexpr int kG = 8;
        const int rpi = 256 / used, rl = tid / used, j = tid - rl * used;
        const int col = sk.idx[min(j, total - 1)];
        if (rl < rpi) {
            for (int rb = rl; rb < nrows; rb += rpi * kG) {
                uint16_t v[kG];
#pragma unroll
                for (int u = 0; u < kG; ++u) v[u] = sk.w16[(row0 + min(rb + u * rpi, nrows - 1)) * sk.ldw + col];
#pragma unroll
                for (int u = 0; u < kG; ++u) {
                    const int r = rb + u * rpi;
                    if (r < nrows) sk.wo[(row0 + r) * sk.P + j] = j < total ? v[u] : (uint16_t)0;
                }
            }
        }
    } else {
        for (int r = 0; r < nrows; ++r)
            for (int j = tid; j < used; j += 256)
                sk.wo[(row0 + r) * sk.P + j] = j < total ? sk.w16[(row0 + r) * sk.ldw + sk.idx[j]] : (uint16_t)0;
    }
}

// The chunk with its skipped elements (bit j of m) replaced by +0: they then
// neither raise the absmax nor get a nonzero code.  Plain bit operations, so
// no per-element lane masks stay live between the absmax and the codes.
template <int DT>
__device__ __forceinline__ Raw8<DT> zero_skipped(Raw8<DT> r, uint32_t m) {
    if constexpr (DT == kF32) {
        uint32_t* w = reinterpret_cast<uint32_t*>(r.w);
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] &= ((m >> j) & 1u) - 1u;
    } else {
        uint32_t* w = reinterpret_cast<uint32_t*>(r.w);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = ((m >> (2 * k)) & 1u) - 1u, hi = ((m >> (2 * k + 1)) & 1u) - 1u;
            w[k] &= (lo & 0xffffu) | (hi & 0xffff0000u);
        }
    }
    return r;
}

template <int DT>
__device__ __forceinline__ float chunk_absmax(const Raw8<DT>& r, uint32_t skipm, float amax) {
    float v[8];
    widen8<DT>(r, v);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (!((skipm >> j) & 1u)) amax = fmaxf(amax, fabsf(v[j]));
    return amax;
}

template <int DT>
__device__ __forceinline__ uint2 chunk_codes(const Raw8<DT>& r, uint32_t skipm, float s, float inv,
                                             int& csum) {
    float v[8], q[8];
    widen8<DT>(r, v);
    rne_quotient8<true>(v, s, inv, q);  // |x / s| <= 127 (1 + 2^-22): absmax scale
    int c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        c[j] = ((skipm >> j) & 1u) ? 0 : (int)fminf(fmaxf(q[j], -127.0f), 127.0f);
        csum += c[j];
    }
    return make_uint2(pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7]));
}

// Codes of one chunk of an absmax-scaled row (|x / s| <= 127 (1 + 2^-22)),
// skipped elements 0.  b = fma(x, inv, 1.5 * 2^23) rounds the exact product
// x * inv to the nearest integer, ties to even, and leaves that integer (two's
// complement) in the low byte of b's encoding, so one FMA does the scaling,
// the rounding and the conversion.  x * inv is within 2^-24 |x / s| of x / s,
// and fl(x / s) within 2^-24 |x / s| as well, so both lie within 2^-16 of each
// other: unless x * inv is within 2^-15 of a half-integer, rounding it gives
// the same integer as rounding the correctly rounded quotient (and neither is
// a tie).  The residual d = fma(x, inv, -(b - 1.5 * 2^23)) = x * inv - rint(x *
// inv), rounded once, tells: when any |d| of the wavefront reaches 1/2 - 2^-15
// the whole chunk is recomputed with the correctly rounded division.
template <int DT, bool SKIP>
__device__ __forceinline__ uint2 chunk_codes_absmax(const Raw8<DT>& r, uint32_t skipm, float s, float inv) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    float v[8], b[8];
    widen8<DT>(r, v);
    float dmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        b[j] = __builtin_fmaf(v[j], inv, kMagic);
        const float d = fabsf(__builtin_fmaf(v[j], inv, -(b[j] - kMagic)));
        if (!SKIP || !((skipm >> j) & 1u)) dmax = fmaxf(dmax, d);
    }
    if (__builtin_expect(__any(dmax >= 0.5f - 0x1p-15f), 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = v[j] / s + kMagic;  // exact: |v / s| < 2^22 for kept elements
    }
    uint32_t u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = (SKIP && ((skipm >> j) & 1u)) ? 0u : __float_as_uint(b[j]);
    // low bytes of u[0..7] -> two words of packed codes
    const uint32_t t0 = __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u);
    const uint32_t t1 = __builtin_amdgcn_perm(u[3], u[2], 0x0c0c0400u);
    const uint32_t t2 = __builtin_amdgcn_perm(u[5], u[4], 0x0c0c0400u);
    const uint32_t t3 = __builtin_amdgcn_perm(u[7], u[6], 0x0c0c0400u);
    return make_uint2(__builtin_amdgcn_perm(t1, t0, 0x05040100u), __builtin_amdgcn_perm(t3, t2, 0x05040100u));
}

// Codes of one chunk on a row's own asymmetric grid: clamp(rne(fl(x / s)) +
// z, -128, 127), where every value of the row lies in the grid's range, so
// |x / s| <= 255.  Same single-FMA rounding as chunk_codes_absmax: x * inv is
// within 2^-23 |x / s| <= 2^-15 of x / s and fl(x / s) within 2^-16, so
// rounding x * inv gives rne(fl(x / s)) unless x * inv lies within 2^-14 of a
// half-integer; when any value of the wavefront is within 2^-13, the chunk
// takes the correctly rounded division.  The integer is read from b's
// encoding (b - 1.5 * 2^23 in two's complement), then z added and clamped.
template <int DT>
__device__ __forceinline__ uint2 chunk_codes_asym(const Raw8<DT>& r, float s, float inv, int z) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    float v[8], b[8];
    widen8<DT>(r, v);
    float dmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        b[j] = __builtin_fmaf(v[j], inv, kMagic);
        dmax = fmaxf(dmax, fabsf(__builtin_fmaf(v[j], inv, -(b[j] - kMagic))));
    }
    if (__builtin_expect(__any(dmax >= 0.5f - 0x1p-13f), 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = v[j] / s + kMagic;  // exact: |v / s| <= 256
    }
    int c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        c[j] = min(max((int)(__float_as_uint(b[j]) - __float_as_uint(kMagic)) + z, -128), 127);
    return make_uint2(pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7]));
}

// One wavefront per row.  CPL > 0: each lane keeps CPL chunks of 8 elements
// in registers (one HBM read), issued together and unconditionally (FULL: the
// row is exactly CPL wavefront-wide chunks; otherwise lanes past the row
// re-read its last chunk and zero it), so the compiler's waits count them
// exactly.  CPL == 0: rows too long for registers are streamed twice (the
// second pass hits the L2).  `rowint` receives the code sum of each row
// (COLSUM) or its zero point (ASYM).
template <int DT, int CPL, bool FULL, bool SKIP, bool COLSUM, bool ASYM = false>
__global__ __launch_bounds__(256) void k_quant_rows(const void* __restrict__ x, int64_t ld_bytes,
                                                    int64_t rows, int nch, int8_t* __restrict__ q,
                                                    float* __restrict__ scale,
                                                    int32_t* __restrict__ rowint,
                                                    OutlierSkip skip) {
    int64_t blk = blockIdx.x;
    if constexpr (SKIP) {
        if (blk < skip.gblocks) {  // a W_out gather workgroup
            gather_w_block(skip, blk);
            return;
        }
        blk -= skip.gblocks;
    }
    const int lane = threadIdx.x & 63;
    const int64_t row = blk * kRowsPerBlock + (threadIdx.x >> 6);
    // whole wavefronts leave together; the rows of the last 16-row group past
    // `rows` are padding, written as zeros
    if (row >= (rows + kWGroup - 1) / kWGroup * kWGroup) return;
    const char* xr = static_cast<const char*>(x) + row * ld_bytes;
    // codes of chunk c (8 values) into the packed blocks: K tile c / 8,
    // 16-byte chunk (c % 8) / 2, half c % 2
    const int ktiles = (nch + 7) / 8;
    int8_t* const qg = q + wpack_block(row / kWGroup, 0, ktiles);
    const int rg = (int)(row % kWGroup);
    auto store_code = [&](int c, uint2 code) {
        *reinterpret_cast<uint2*>(qg + (int64_t)(c >> 3) * kWBlock + wpack_pos(rg, (c & 7) >> 1) + ((c & 1) << 3)) =
            code;
    };
    if (row >= rows) {
        for (int c = lane; c < ktiles * 8; c += 64) store_code(c, make_uint2(0u, 0u));
        return;
    }
    int csum = 0, zq = 0;
    float s;
    // The asymmetric grid of a row's range [lo, hi] (both already widened to
    // contain 0): S = fl(fl(hi - lo) / 255), 1 for an empty range;
    // Z = clamp(-128 - rne(fl(lo / S)), -128, 127).
    auto asym_grid = [&](float lo, float hi) {
        hi = wave_max_full(hi);
        lo = -wave_max_full(-lo);
        s = hi == lo ? 1.0f : (hi - lo) / 255.0f;
        zq = hi == lo ? 0 : min(max(-128 - (int)__builtin_rintf(lo / s), -128), 127);
    };
    auto asym_codes = [&](const Raw8<DT>& r, float inv) { return chunk_codes_asym<DT>(r, s, inv, zq); };
    auto range8 = [&](const Raw8<DT>& r, float& lo, float& hi) {
        float v[8];
        widen8<DT>(r, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            lo = fminf(lo, v[j]);
            hi = fmaxf(hi, v[j]);
        }
    };
    // Outlier gather into X_out: lane j fetches x[row, idx[j]] (j < 64; the
    // index is clamped into the row, entries past the count are unset) while
    // the row is being quantized, and stores it, or the zero padding, once
    // the count is known to fit.  The index and the count are loaded before
    // the row, so that the dependent load of the value waits for them alone.
    const bool gather = SKIP && DT != kF32 && skip.xo != nullptr && skip.max_out > 0;
    const uint16_t* xr16 = reinterpret_cast<const uint16_t*>(xr);
    int gidx = 0, gcnt = 0;
    uint16_t gval = 0;
    if (gather) {
        gidx = skip.idx[min(lane, skip.max_out - 1)];
        gcnt = *skip.count;
    }
    auto gather_store = [&]() {
        const int cnt = gcnt;
        if (cnt > skip.max_out) return;
        uint16_t* xo_row = skip.xo + row * skip.P;
        const int used = (cnt + 15) / 16 * 16;
        if (lane < used) xo_row[lane] = lane < cnt ? gval : (uint16_t)0;
        for (int j = lane + 64; j < used; j += 64) {
            const uint16_t v = xr16[skip.idx[min(j, cnt - 1)]];
            xo_row[j] = j < cnt ? v : (uint16_t)0;
        }
    };

    if constexpr (CPL > 0) {
        Raw8<DT> raw[CPL];
        uint32_t sk[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            if constexpr (FULL) {
                raw[i] = load_raw8<DT>(xr, c);
            } else {
                raw[i] = load_raw8<DT>(xr, min(c, nch - 1));
                if (c >= nch) raw[i] = zero_raw8<DT>();
            }
            sk[i] = (FULL || c < nch) ? skip_mask<SKIP>(skip, min(c, nch - 1)) : 0u;
        }
        if (gather) gval = xr16[min(max(gidx, 0), nch * 8 - 1)];
        float amax = 0.0f, lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            if constexpr (SKIP) {
                raw[i] = zero_skipped<DT>(raw[i], sk[i]);
                sk[i] = 0;
            }
            if constexpr (ASYM)
                range8(raw[i], lo, hi);  // zeros past the row leave the widened range as it is
            else
                amax = chunk_absmax<DT>(raw[i], sk[i], amax);
        }
        if constexpr (ASYM) {
            asym_grid(lo, hi);
        } else {
            amax = wave_max_full(amax);
            s = absmax_step(amax);
        }
        const float inv = 1.0f / s;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            uint2 code;
            if constexpr (ASYM)
                code = asym_codes(raw[i], inv);
            else if constexpr (COLSUM)
                code = chunk_codes<DT>(raw[i], sk[i], s, inv, csum);
            else
                code = chunk_codes_absmax<DT, false>(raw[i], 0u, s, inv);
            if (FULL || c < nch) store_code(c, code);
        }
    } else {
        float amax = 0.0f, lo = 0.0f, hi = 0.0f;
        for (int c = lane; c < nch; c += 64) {
            if constexpr (ASYM)
                range8(load_raw8<DT>(xr, c), lo, hi);
            else
                amax = chunk_absmax<DT>(load_raw8<DT>(xr, c), skip_mask<SKIP>(skip, c), amax);
        }
        if constexpr (ASYM) {
            asym_grid(lo, hi);
        } else {
            amax = wave_max_full(amax);
            s = absmax_step(amax);
        }
        const float inv = 1.0f / s;
        if (gather) gval = xr16[min(max(gidx, 0), nch * 8 - 1)];
        for (int c = lane; c < nch; c += 64) {
            const Raw8<DT> r = load_raw8<DT>(xr, c);
            const uint32_t m = skip_mask<SKIP>(skip, c);
            if constexpr (ASYM)
                store_code(c, asym_codes(r, inv));
            else if constexpr (COLSUM)
                store_code(c, chunk_codes<DT>(r, m, s, inv, csum));
            else
                store_code(c, chunk_codes_absmax<DT, SKIP>(r, m, s, inv));
        }
    }
    if (gather) gather_store();
    for (int c = nch + lane; c < ktiles * 8; c += 64) store_code(c, make_uint2(0u, 0u));  // K padding
    if (lane == 0) scale[row] = s;
    if constexpr (COLSUM) {
        csum = wave_sum(csum);
        if (lane == 0) rowint[row] = csum;
    }
    if constexpr (ASYM)
        if (lane == 0) rowint[row] = zq;
}

// h = SiLU(g) * u, evaluated in binary64 and rounded once to DT's grid
// (bf16: 8 significant bits, binary32's exponent range, spacing 2^-133 below
// 2^-126; f16: 11 significant bits, spacing 2^-24 below 2^-14, values from
// 65520 up round to infinity), returned as DT's bit pattern.  The rare path of
// silu_mul8: the library's binary64 exponential and a correctly rounded
// binary64 division, then one rounding by scaling the value's last kept place
// to 1, rounding to the nearest integer (ties to even) and scaling back --
// every step exact but the rounding.
template <int DT>
__device__ uint32_t silu_mul_exact16(float g, float u) {
    constexpr int kSig = DT == kF16 ? 11 : 8;
    constexpr int kEmin = DT == kF16 ? -13 : -125;  // frexp exponent of the smallest normal
    const double gd = g;
    const double v = gd / (1.0 + exp(-gd)) * (double)u;
    int e;
    (void)__builtin_frexp(v, &e);
    e = max(e, kEmin);
    const double r = __builtin_ldexp(__builtin_rint(__builtin_ldexp(v, kSig - e)), e - kSig);
    if constexpr (DT == kF16) {
        const float rf = fabs(r) > 65504.0 ? __builtin_copysignf(__builtin_inff(), (float)r) : (float)r;
        return f32_to_f16(rf);  // exact: rf is on the binary16 grid (or infinite)
    } else {
        const float rf = fabs(r) >= 0x1p128 ? __builtin_copysignf(__builtin_inff(), (float)v) : (float)r;
        return __float_as_uint(rf) >> 16;  // exact: rf has at most 8 significant bits
    }
}

// Bound of the fast path (below): for |g| <= kSiluGMax its binary32 h is
// within kSiluTol units in the last place of binary32 of SiLU(g) * u.  The
// exponent argument x log2(e) is rounded twice (the binary32 log2(e) is within
// 0.23 2^-24 of it, the product within 2^-24), which moves e by a relative
// 1.224 |x| 2^-24; v_exp_f32 and v_rcp_f32 add one unit each, the sum 1 + e
// and the two products half a unit each: within (1.224 |g| + 7) units,
// 19.3 at |g| = 10, taken as 24.
constexpr float kSiluGMax = 10.0f;
constexpr uint32_t kSiluTol = 24;

// Tie test on a binary32 bit pattern b: the low `drop` bits are what rounding
// to DT discards (16 for bf16 at every magnitude; 13 for f16 in its normal
// range), and a tie sits at half of that.  t = (b << (32 - drop)) + bias is
// (discarded + kSiluTol - half) mod 2^drop in the top bits, at most `lim`
// exactly when the discarded bits are within kSiluTol of the tie.
template <int DT>
struct SiluTie {
    static constexpr int kDrop = DT == kF16 ? 13 : 16;
    static constexpr uint32_t kBias = (kSiluTol - (1u << (kDrop - 1))) << (32 - kDrop);
    static constexpr uint32_t kLim = (2u * kSiluTol) << (32 - kDrop);
    static __device__ __forceinline__ uint32_t t(float p) {
        return (__float_as_uint(p) << (32 - kDrop)) + kBias;
    }
};

// h = SiLU(g) * u for one chunk, rounded to DT (nearest even), bit-identical to
// silu_mul_exact16 of every element.  Fast path in binary32: e = 2^(-g
// log2(e)) on the hardware exponential (v_exp_f32; e overflows to +inf for
// very negative g and the product to -0, the limit), SiLU(g) = g * (1 / (1 +
// e)) on the hardware reciprocal (v_rcp_f32), rounded to DT by the conversion
// instruction: two transcendental instructions per element.  That rounding
// is the correct one unless the binary32 value lies within the bound above of
// a tie of DT's grid, or |g| exceeds the bound's range, or (f16) the value is
// a nonzero binary16 subnormal, whose grid is coarser: such elements -- a few
// in ten thousand -- are recomputed by silu_mul_exact16 in a branch that the
// wavefront takes only when one of its lanes has one in this chunk.
template <int DT>
__device__ __forceinline__ Raw8<DT> silu_mul8(const Raw8<DT>& g, const Raw8<DT>& u) {
    constexpr float kLog2e = 1.44269504088896340736f;
    float gv[8], uv[8], p[8];
    widen8<DT>(g, gv);
    widen8<DT>(u, uv);
    uint32_t w[4];
    uint32_t tmin = 0xffffffffu, sub = 0xffffffffu;
    float gmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float x = gv[j + k];
            const float e = __builtin_amdgcn_exp2f(-x * kLog2e);
            p[j + k] = (x * __builtin_amdgcn_rcpf(1.0f + e)) * uv[j + k];
        }
        w[j / 2] = f32x2_to_16<DT>(p[j], p[j + 1]);
        tmin = min(tmin, min(SiluTie<DT>::t(p[j]), SiluTie<DT>::t(p[j + 1])));
        gmax = fmaxf(gmax, fmaxf(fabsf(gv[j]), fabsf(gv[j + 1])));
        if constexpr (DT == kF16)  // |p| - 1 ulp as an integer: below 2^-14 - 1 ulp for nonzero subnormals
            sub = min(sub, min((__float_as_uint(p[j]) & 0x7fffffffu) - 1u,
                               (__float_as_uint(p[j + 1]) & 0x7fffffffu) - 1u));
    }
    const bool unsure = tmin <= SiluTie<DT>::kLim || !(gmax <= kSiluGMax) ||
                        (DT == kF16 && sub < 0x387fffffu);
    if (__builtin_expect(__any(unsure), 0)) {
        // element by element, each branch taken only when a lane of the
        // wavefront needs that element recomputed
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t pb = __float_as_uint(p[j]) & 0x7fffffffu;
            const bool near = unsure && (SiluTie<DT>::t(p[j]) <= SiluTie<DT>::kLim || !(fabsf(gv[j]) <= kSiluGMax) ||
                                         (DT == kF16 && pb - 1u < 0x387fffffu));
            if (__builtin_expect(__any(near), 0)) {
                if (near) {
                    const uint32_t h16 = silu_mul_exact16<DT>(gv[j], uv[j]);
                    const int sh = (j & 1) * 16;
                    w[j >> 1] = (w[j >> 1] & ~(0xffffu << sh)) | (h16 << sh);
                }
            }
        }
    }
    Raw8<DT> h;
    h.w[0] = make_uint4(w[0], w[1], w[2], w[3]);
    return h;
}

// One wavefront per row, as k_quant_rows, for rows up to 64 * 8 * 8 values:
// CPL > 0 keeps the row's h in registers (gate and up read from HBM once);
// CPL == 0 (rows longer than 256 * 8 * 16 values) forms h twice, for the
// absmax and for the codes -- the same operations, so the same bits.  h_out
// (nullable) receives h.
template <int DT, int CPL, bool FULL>
__global__ __launch_bounds__(256, 2) void k_silu_mul_quant(const void* __restrict__ gate, int64_t ldg_bytes,
                                                        const void* __restrict__ up, int64_t ldu_bytes,
                                                        int64_t rows, int nch, int8_t* __restrict__ q,
                                                        float* __restrict__ scale, void* __restrict__ h_out,
                                                        int64_t ldh_bytes) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= (rows + kWGroup - 1) / kWGroup * kWGroup) return;
    const int ktiles = (nch + 7) / 8;
    int8_t* const qg = q + wpack_block(row / kWGroup, 0, ktiles);
    const int rg = (int)(row % kWGroup);
    auto store_code = [&](int c, uint2 code) {
        *reinterpret_cast<uint2*>(qg + (int64_t)(c >> 3) * kWBlock + wpack_pos(rg, (c & 7) >> 1) + ((c & 1) << 3)) =
            code;
    };
    if (row >= rows) {
        for (int c = lane; c < ktiles * 8; c += 64) store_code(c, make_uint2(0u, 0u));
        return;
    }
    const char* gr = static_cast<const char*>(gate) + row * ldg_bytes;
    const char* ur = static_cast<const char*>(up) + row * ldu_bytes;
    uint4* hr = h_out ? reinterpret_cast<uint4*>(static_cast<char*>(h_out) + row * ldh_bytes) : nullptr;
    float amax = 0.0f, s, inv;
    if constexpr (CPL > 0) {
        Raw8<DT> hv[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            const int cc = FULL ? c : min(c, nch - 1);
            hv[i] = silu_mul8<DT>(load_raw8<DT>(gr, cc), load_raw8<DT>(ur, cc));
            if (!FULL && c >= nch) hv[i] = zero_raw8<DT>();
            amax = chunk_absmax<DT>(hv[i], 0u, amax);
        }
        amax = wave_max_full(amax);
        s = absmax_step(amax);
        inv = 1.0f / s;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            const uint2 code = chunk_codes_absmax<DT, false>(hv[i], 0u, s, inv);
            if (FULL || c < nch) {
                store_code(c, code);
                if (hr) hr[c] = hv[i].w[0];
            }
        }
    } else {
        for (int c = lane; c < nch; c += 64)
            amax = chunk_absmax<DT>(silu_mul8<DT>(load_raw8<DT>(gr, c), load_raw8<DT>(ur, c)), 0u, amax);
        amax = wave_max_full(amax);
        s = absmax_step(amax);
        inv = 1.0f / s;
        for (int c = lane; c < nch; c += 64) {
            const Raw8<DT> hc = silu_mul8<DT>(load_raw8<DT>(gr, c), load_raw8<DT>(ur, c));
            store_code(c, chunk_codes_absmax<DT, false>(hc, 0u, s, inv));
            if (hr) hr[c] = hc.w[0];
        }
    }
    for (int c = nch + lane; c < ktiles * 8; c += 64) store_code(c, make_uint2(0u, 0u));  // K padding
    if (lane == 0) scale[row] = s;
}

// Rows longer than 64 * 8 * 8 values: one workgroup per row, CPT chunks per
// thread, the row's absmax reduced across the four wavefronts through LDS.
// Fewer registers per thread than a wavefront per row, so that several rows
// are in flight per CU while others compute.  The absmax, the scale and the
// codes are the same as with a wavefront per row (max is exact in any order).
// MODE kRowSilu: the row is h = SiLU(gate) * up (gate = x); kRowPlain: the
// row of x itself, the plain per-token quantizer of k_quant_rows (DT may be
// binary32); kRowAsym: the row of x on its own asymmetric grid, as
// k_quant_rows<..., ASYM> (min and max reduced instead of the absmax, the
// zero point into rowint).  SKIP (kRowPlain, 16-bit types): the outlier
// columns of the LLM.int8() decomposition take no part in the absmax and are
// coded 0, and their values are gathered into X_out, as k_quant_rows<...,
// SKIP> does with a wavefront per row.
constexpr int kRowPlain = 0, kRowSilu = 1, kRowAsym = 2;
template <int DT, int CPT, int MODE, bool SKIP = false>
__global__ __launch_bounds__(256) void k_silu_mul_quant_wg(const void* __restrict__ gate, int64_t ldg_bytes,
                                                           const void* __restrict__ up, int64_t ldu_bytes,
                                                           int64_t rows, int nch, int8_t* __restrict__ q,
                                                           float* __restrict__ scale, int32_t* __restrict__ rowint,
                                                           void* __restrict__ h_out, int64_t ldh_bytes,
                                                           OutlierSkip skip) {
    static_assert(!SKIP || (MODE == kRowPlain && DT != kF32), "outlier columns: plain 16-bit rows only");
    int64_t row = blockIdx.x;
    if constexpr (SKIP) {
        if (row < skip.gblocks) {  // a W_out gather workgroup
            gather_w_block(skip, row);
            return;
        }
        row -= skip.gblocks;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ktiles = (nch + 7) / 8;
    int8_t* const qg = q + wpack_block(row / kWGroup, 0, ktiles);
    const int rg = (int)(row % kWGroup);
    auto store_code = [&](int c, uint2 code) {
        *reinterpret_cast<uint2*>(qg + (int64_t)(c >> 3) * kWBlock + wpack_pos(rg, (c & 7) >> 1) + ((c & 1) << 3)) =
            code;
    };
    if (row >= rows) {  // padding row of the last 16-row group (whole workgroup)
        for (int c = tid; c < ktiles * 8; c += 256) store_code(c, make_uint2(0u, 0u));
        return;
    }
    const char* gr = static_cast<const char*>(gate) + row * ldg_bytes;
    const char* ur = static_cast<const char*>(up) + row * ldu_bytes;
    uint4* hr = h_out ? reinterpret_cast<uint4*>(static_cast<char*>(h_out) + row * ldh_bytes) : nullptr;
    // Outlier gather into X_out (SKIP): thread j fetches x[row, idx[j]] (j <
    // 256; the index is clamped into the row, entries past the count are
    // unset) while the row is being quantized, and stores it, or the zero
    // padding, once the count is known to fit.
    const bool gather = SKIP && skip.xo != nullptr && skip.max_out > 0;
    const uint16_t* gr16 = reinterpret_cast<const uint16_t*>(gr);
    int gidx = 0, gcnt = 0;
    uint16_t gval = 0;
    if (gather) {
        gidx = skip.idx[min(tid, skip.max_out - 1)];
        gcnt = *skip.count;
    }
    Raw8<DT> hv[CPT];
    uint32_t sk[CPT];
    float amax = 0.0f, lo = 0.0f, hi = 0.0f;  // the asymmetric range starts widened to contain 0
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tid + 256 * i;
        const int cc = min(c, nch - 1);
        if constexpr (MODE == kRowSilu)
            hv[i] = silu_mul8<DT>(load_raw8<DT>(gr, cc), load_raw8<DT>(ur, cc));
        else
            hv[i] = load_raw8<DT>(gr, cc);
        sk[i] = SKIP ? skip.mask[cc] : 0u;
        if (c >= nch) hv[i] = zero_raw8<DT>();
    }
    if (gather) gval = gr16[min(max(gidx, 0), nch * 8 - 1)];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        if constexpr (SKIP) hv[i] = zero_skipped<DT>(hv[i], sk[i]);  // +0: no part in the absmax, code 0
        if constexpr (MODE == kRowAsym) {
            float v[8];
            widen8<DT>(hv[i], v);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                lo = fminf(lo, v[j]);
                hi = fmaxf(hi, v[j]);
            }
        } else {
            amax = chunk_absmax<DT>(hv[i], 0u, amax);
        }
    }
    __shared__ float s_red[2][4];
    float s;
    int zq = 0;
    if constexpr (MODE == kRowAsym) {
        hi = wave_max_full(hi);
        lo = -wave_max_full(-lo);
        if (lane == 0) {
            s_red[0][wave] = hi;
            s_red[1][wave] = lo;
        }
        __syncthreads();
        hi = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
        lo = fminf(fminf(s_red[1][0], s_red[1][1]), fminf(s_red[1][2], s_red[1][3]));
        // S = fl(fl(hi - lo) / 255), 1 for an empty range; Z = clamp(-128 - rne(fl(lo / S)), -128, 127)
        s = hi == lo ? 1.0f : (hi - lo) / 255.0f;
        zq = hi == lo ? 0 : min(max(-128 - (int)__builtin_rintf(lo / s), -128), 127);
    } else {
        amax = wave_max_full(amax);
        if (lane == 0) s_red[0][wave] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
        s = absmax_step(amax);
    }
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tid + 256 * i;
        uint2 code;
        if constexpr (MODE == kRowAsym)
            code = chunk_codes_asym<DT>(hv[i], s, inv, zq);
        else
            code = chunk_codes_absmax<DT, false>(hv[i], 0u, s, inv);
        if (c < nch) {
            store_code(c, code);
            if constexpr (MODE == kRowSilu)
                if (hr) hr[c] = hv[i].w[0];
        }
    }
    for (int c = nch + tid; c < ktiles * 8; c += 256) store_code(c, make_uint2(0u, 0u));  // K padding
    if (gather && gcnt <= skip.max_out) {
        uint16_t* xo_row = skip.xo + row * skip.P;
        const int used = (gcnt + 15) / 16 * 16;
        if (tid < used) xo_row[tid] = tid < gcnt ? gval : (uint16_t)0;
        for (int j = tid + 256; j < used; j += 256) {
            const uint16_t v = gr16[skip.idx[min(j, gcnt - 1)]];
            xo_row[j] = j < gcnt ? v : (uint16_t)0;
        }
    }
    if (tid == 0) {
        scale[row] = s;
        if constexpr (MODE == kRowAsym) rowint[row] = zq;
    }
}

template <int DT, int CPT, int MODE = kRowSilu, bool SKIP = false>
void silu_mul_quant_wg(const void* gate, int64_t ldg, const void* up, int64_t ldu, int64_t rows, int nch,
                       int8_t* q, float* scale, void* h, int64_t ldh, hipStream_t st, int32_t* rowint = nullptr,
                       const OutlierSkip* skip = nullptr) {
    const int64_t rows_pad = (rows + kWGroup - 1) / kWGroup * kWGroup;
    constexpr int eb = Elem<DT>::bytes;
    OutlierSkip sk = skip ? *skip : OutlierSkip{};
    sk.gblocks = sk.w16 && sk.N > 0 ? (int)((sk.N + sk.wrows - 1) / sk.wrows) : 0;
    hipLaunchKernelGGL((k_silu_mul_quant_wg<DT, CPT, MODE, SKIP>), dim3((unsigned)(rows_pad + sk.gblocks)), dim3(256),
                       0, st, gate, ldg * eb, up, ldu * eb, rows, nch, q, scale, rowint, h, ldh * eb, sk);
}

template <int DT, int CPL>
void silu_mul_quant_cpl(const void* gate, int64_t ldg, const void* up, int64_t ldu, int64_t rows, int nch,
                        int8_t* q, float* scale, void* h, int64_t ldh, hipStream_t st) {
    const int64_t rows_pad = (rows + kWGroup - 1) / kWGroup * kWGroup;
    const dim3 grid((unsigned)((rows_pad + kRowsPerBlock - 1) / kRowsPerBlock));
    if (CPL > 0 && nch == 64 * CPL)
        hipLaunchKernelGGL((k_silu_mul_quant<DT, CPL, true>), grid, dim3(256), 0, st, gate, ldg * 2, up,
                           ldu * 2, rows, nch, q, scale, h, ldh * 2);
    else
        hipLaunchKernelGGL((k_silu_mul_quant<DT, CPL, false>), grid, dim3(256), 0, st, gate, ldg * 2, up,
                           ldu * 2, rows, nch, q, scale, h, ldh * 2);
}

template <int DT>
void silu_mul_quant_dt(const void* gate, int64_t ldg, const void* up, int64_t ldu, int64_t rows, int64_t K,
                       int8_t* q, float* scale, void* h, int64_t ldh, hipStream_t st) {
    const int nch = (int)(K / 8);
    const int64_t per_lane = (nch + 63) / 64;
    if (per_lane <= 1)
        silu_mul_quant_cpl<DT, 1>(gate, ldg, up, ldu, rows, nch, q, scale, h, ldh, st);
    else if (per_lane <= 2)
        silu_mul_quant_cpl<DT, 2>(gate, ldg, up, ldu, rows, nch, q, scale, h, ldh, st);
    else if (per_lane <= 4)
        silu_mul_quant_cpl<DT, 4>(gate, ldg, up, ldu, rows, nch, q, scale, h, ldh, st);
    else if (per_lane <= 8)
        silu_mul_quant_cpl<DT, 8>(gate, ldg, up, ldu, rows, nch, q, scale, h, ldh, st);
    else if (per_lane <= 16)
        silu_mul_quant_wg<DT, 4>(gate, ldg, up, ldu, rows, nch, q, scale, h, ldh, st);
    else if (per_lane <= 32)
        silu_mul_quant_wg<DT, 8>(gate, ldg, up, ldu, rows, nch, q, scale, h, ldh, st);
    else if (per_lane <= 64)
        silu_mul_quant_wg<DT, 16>(gate, ldg, up, ldu, rows, nch, q, scale, h, ldh, st);
    else
        silu_mul_quant_cpl<DT, 0>(gate, ldg, up, ldu, rows, nch, q, scale, h, ldh, st);
}

template <int DT, int CPL, bool FULL>
void launch_rows(int64_t rows, const void* x, int64_t ldb, int nch, int8_t* q, float* scale,
                 int32_t* colsum, const OutlierSkip* skip, bool asym, hipStream_t st) {
    const OutlierSkip none{};
    const int64_t rows_pad = (rows + kWGroup - 1) / kWGroup * kWGroup;
    const int64_t qblocks = (rows_pad + kRowsPerBlock - 1) / kRowsPerBlock;
    const dim3 grid((unsigned)qblocks);
    if (asym) {
        hipLaunchKernelGGL((k_quant_rows<DT, CPL, FULL, false, false, true>), grid, dim3(256), 0, st, x,
                           ldb, rows, nch, q, scale, colsum, none);
    } else if (skip) {
        OutlierSkip sk = *skip;
        sk.gblocks = sk.w16 && sk.N > 0 ? (int)((sk.N + sk.wrows - 1) / sk.wrows) : 0;
        hipLaunchKernelGGL((k_quant_rows<DT, CPL, FULL, true, false>), dim3((unsigned)(qblocks + sk.gblocks)),
                           dim3(256), 0, st, x, ldb, rows, nch, q, scale, colsum, sk);
    } else if (colsum) {
        hipLaunchKernelGGL((k_quant_rows<DT, CPL, FULL, false, true>), grid, dim3(256), 0, st, x, ldb,
                           rows, nch, q, scale, colsum, none);
    } else {
        hipLaunchKernelGGL((k_quant_rows<DT, CPL, FULL, false, false>), grid, dim3(256), 0, st, x, ldb,
                           rows, nch, q, scale, colsum, none);
    }
}

template <int DT, int CPL>
void quant_rows_cpl(const void* x, int64_t rows, int64_t K, int64_t ldx, int8_t* q, float* scale,
                    int32_t* colsum, const OutlierSkip* skip, bool asym, hipStream_t st) {
    const int64_t ldb = ldx * Elem<DT>::bytes;
    const int nch = (int)(K / 8);
    if (CPL > 0 && nch == 64 * CPL)
        launch_rows<DT, CPL, true>(rows, x, ldb, nch, q, scale, colsum, skip, asym, st);
    else
        launch_rows<DT, CPL, false>(rows, x, ldb, nch, q, scale, colsum, skip, asym, st);
}

template <int DT>
void quant_rows_dt(const void* x, int64_t rows, int64_t K, int64_t ldx, int8_t* q, float* scale,
                   int32_t* colsum, const OutlierSkip* skip, bool asym, hipStream_t st) {
    const int64_t per_lane = (K / 8 + 63) / 64;  // chunks of 8 per lane
    if constexpr (DT != kF32) {
        // the regular columns of the LLM.int8() decomposition, rows longer than
        // 2048 values: a workgroup per row as well (outlier columns skipped,
        // their values gathered into X_out)
        if (skip && !asym && !colsum && per_lane > 4 && per_lane <= 64) {
            const int nch = (int)(K / 8);
            if (per_lane <= 8)
                silu_mul_quant_wg<DT, 2, kRowPlain, true>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st,
                                                          nullptr, skip);
            else if (per_lane <= 16)
                silu_mul_quant_wg<DT, 4, kRowPlain, true>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st,
                                                          nullptr, skip);
            else if (per_lane <= 32)
                silu_mul_quant_wg<DT, 8, kRowPlain, true>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st,
                                                          nullptr, skip);
            else
                silu_mul_quant_wg<DT, 16, kRowPlain, true>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st,
                                                           nullptr, skip);
            return;
        }
    }
    if (!skip && (asym || !colsum) && per_lane > 4 && per_lane <= 64) {
        // the per-token quantizers (symmetric, or asymmetric with the zero
        // points in `colsum`) of rows longer than 2048 values: a workgroup per
        // row (more rows in flight per CU than a wavefront per row)
        const int nch = (int)(K / 8);
        if (asym) {
            if (per_lane <= 8)
                silu_mul_quant_wg<DT, 2, kRowAsym>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st, colsum);
            else if (per_lane <= 16)
                silu_mul_quant_wg<DT, 4, kRowAsym>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st, colsum);
            else if (per_lane <= 32)
                silu_mul_quant_wg<DT, 8, kRowAsym>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st, colsum);
            else
                silu_mul_quant_wg<DT, 16, kRowAsym>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st, colsum);
        } else {
            if (per_lane <= 8)
                silu_mul_quant_wg<DT, 2, kRowPlain>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st);
            else if (per_lane <= 16)
                silu_mul_quant_wg<DT, 4, kRowPlain>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st);
            else if (per_lane <= 32)
                silu_mul_quant_wg<DT, 8, kRowPlain>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st);
            else
                silu_mul_quant_wg<DT, 16, kRowPlain>(x, ldx, nullptr, 0, rows, nch, q, scale, nullptr, 0, st);
        }
        return;
    }
    constexpr int kMaxCpl = DT == kF32 ? 16 : 32;
    if (per_lane <= 1)
        quant_rows_cpl<DT, 1>(x, rows, K, ldx, q, scale, colsum, skip, asym, st);
    else if (per_lane <= 2)
        quant_rows_cpl<DT, 2>(x, rows, K, ldx, q, scale, colsum, skip, asym, st);
    else if (per_lane <= 4)
        quant_rows_cpl<DT, 4>(x, rows, K, ldx, q, scale, colsum, skip, asym, st);
    else if (per_lane <= 8)
        quant_rows_cpl<DT, 8>(x, rows, K, ldx, q, scale, colsum, skip, asym, st);
    else if (per_lane <= 16)
        quant_rows_cpl<DT, 16>(x, rows, K, ldx, q, scale, colsum, skip, asym, st);
    else if (per_lane <= kMaxCpl)
        quant_rows_cpl<DT, kMaxCpl>(x, rows, K, ldx, q, scale, colsum, skip, asym, st);
    else
        quant_rows_cpl<DT, 0>(x, rows, K, ldx, q, scale, colsum, skip, asym, st);
}

// ---------------------------------------------------------------------------

// One thread per 8-value chunk of the padded code matrix (rows rounded up to
// 16, K to 64): chunk (row, col) of the activations, or a zero of the padding.
// WIDE: the chunk index needs 64 bits.
// qmin: -128 (asymmetric grid) or -127 (symmetric, z = 0).
template <int DT, bool WIDE>
__global__ __launch_bounds__(256) void k_quant_static(const void* __restrict__ x, int64_t ld_bytes,
                                                      int64_t rows, int nch, int cpr, int64_t total,
                                                      int8_t* __restrict__ q, float s, int z, int qmin,
                                                      uint32_t* __restrict__ sat) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const float inv = 1.0f / s;
    int nsat = 0;
    if (c < total) {
        int64_t row;
        int col;
        if constexpr (WIDE) {
            row = c / cpr;
            col = (int)(c - row * cpr);
        } else {
            const uint32_t r32 = (uint32_t)c / (uint32_t)cpr;
            row = r32;
            col = (int)((uint32_t)c - r32 * (uint32_t)cpr);
        }
        uint2 code = make_uint2(0u, 0u);
        if (row < rows && col < nch) {
            float v[8];
            widen8<DT>(load_raw8<DT>(static_cast<const char*>(x) + row * ld_bytes, col), v);
            code = static_codes8(v, s, inv, z, nsat, qmin);
        }
        const int ktiles = cpr / 8;
        *reinterpret_cast<uint2*>(q + wpack_block(row / kWGroup, col >> 3, ktiles) +
                                  wpack_pos((int)(row % kWGroup), (col & 7) >> 1) + ((col & 1) << 3)) = code;
    }
    if (sat) {
        nsat = wave_sum(nsat);
        if ((threadIdx.x & 63) == 0 && nsat) atomicAdd(sat, (uint32_t)nsat);
    }
}

template <int DT>
__global__ __launch_bounds__(256) void k_minmax(const void* __restrict__ x, int64_t ld_bytes,
                                                int64_t total, int nch, float* __restrict__ mm) {
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * 256) {
        const int64_t row = c / nch;
        const int col = (int)(c - row * nch);
        float v[8];
        widen8<DT>(load_raw8<DT>(static_cast<const char*>(x) + row * ld_bytes, col), v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            lo = fminf(lo, v[j]);
            hi = fmaxf(hi, v[j]);
        }
    }
    // one atomic pair per workgroup: the running state lives at two addresses,
    // and same-address atomics are serialized in the L2
    __shared__ float s_lo[4], s_hi[4];
    lo = wave_min(lo);
    hi = wave_max(hi);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_lo[wave] = lo;
        s_hi[wave] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        lo = fminf(fminf(s_lo[0], s_lo[1]), fminf(s_lo[2], s_lo[3]));
        hi = fmaxf(fmaxf(s_hi[0], s_hi[1]), fmaxf(s_hi[2], s_hi[3]));
        if (lo <= hi) {
            atomic_min_f32(mm, lo);
            atomic_max_f32(mm + 1, hi);
        }
    }
}

// grid 0: the decode phase's asymmetric grid, 255 steps on [-128, 127];
// 1: tensor-wise absmax, S = max(|min|, |max|) / 127 (1 before any value);
// 2: the zero-point grid of 254 steps on [-127, 127].
__global__ void k_minmax_finalize(const float* __restrict__ mm, float* __restrict__ s_out,
                                  int32_t* __restrict__ z_out, int grid) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    if (grid == 1) {
        const float c = mm[0] > mm[1] ? 0.0f : fmaxf(fabsf(mm[0]), fabsf(mm[1]));
        *s_out = absmax_step(c);
        return;
    }
    const int qmin = grid == 2 ? -127 : -128;
    const float steps = grid == 2 ? 254.0f : 255.0f;
    const float lo = fminf(mm[0], 0.0f);
    const float hi = fmaxf(mm[1], 0.0f);
    float s = 1.0f;
    int z = 0;
    if (hi != lo) {
        s = (hi - lo) / steps;
        z = qmin - (int)__builtin_rintf(lo / s);
        z = min(max(z, qmin), 127);
    }
    *s_out = s;
    *z_out = z;
}

}  // namespace

void launch_quant_rows(const void* x, int dt, int64_t rows, int64_t K, int64_t ldx, int8_t* q,
                       float* scale, int32_t* colsum, const OutlierSkip* skip, hipStream_t st) {
    if (rows <= 0) return;
    switch (dt) {
        case kF32: quant_rows_dt<kF32>(x, rows, K, ldx, q, scale, colsum, skip, false, st); break;
        case kBF16: quant_rows_dt<kBF16>(x, rows, K, ldx, q, scale, colsum, skip, false, st); break;
        default: quant_rows_dt<kF16>(x, rows, K, ldx, q, scale, colsum, skip, false, st); break;
    }
}

void launch_quant_rows_asym(const void* x, int dt, int64_t rows, int64_t K, int64_t ldx, int8_t* q,
                            float* scale, int32_t* zp, hipStream_t st) {
    if (rows <= 0) return;
    switch (dt) {
        case kF32: quant_rows_dt<kF32>(x, rows, K, ldx, q, scale, zp, nullptr, true, st); break;
        case kBF16: quant_rows_dt<kBF16>(x, rows, K, ldx, q, scale, zp, nullptr, true, st); break;
        default: quant_rows_dt<kF16>(x, rows, K, ldx, q, scale, zp, nullptr, true, st); break;
    }
}

void launch_silu_mul_quant(const void* gate, int64_t ldg, const void* up, int64_t ldu, int dt, int64_t rows,
                           int64_t K, int8_t* q, float* scale, void* h, int64_t ldh, hipStream_t st) {
    if (rows <= 0) return;
    if (dt == kF16)
        silu_mul_quant_dt<kF16>(gate, ldg, up, ldu, rows, K, q, scale, h, ldh, st);
    else
        silu_mul_quant_dt<kBF16>(gate, ldg, up, ldu, rows, K, q, scale, h, ldh, st);
}

template <int DT>
void quant_static_dt(const void* x, int64_t M, int64_t ldb, int nch, int cpr, int64_t total, int8_t* q,
                     float s, int z, int qmin, uint32_t* sat, hipStream_t st) {
    const dim3 grid((unsigned)((total + 255) / 256));
    if (total <= 0xffffffffll)
        hipLaunchKernelGGL((k_quant_static<DT, false>), grid, dim3(256), 0, st, x, ldb, M, nch, cpr, total,
                           q, s, z, qmin, sat);
    else
        hipLaunchKernelGGL((k_quant_static<DT, true>), grid, dim3(256), 0, st, x, ldb, M, nch, cpr, total,
                           q, s, z, qmin, sat);
}

void launch_quant_static(const void* x, int dt, int64_t M, int64_t K, int64_t ldx, float s, int z,
                         int8_t* q, uint32_t* sat, hipStream_t st, bool narrow) {
    if (M <= 0 || K <= 0) return;
    const int qmin = narrow ? -127 : -128;
    const int nch = (int)(K / 8);
    const int cpr = (int)((K + kWTileK - 1) / kWTileK * 8);  // chunks per padded row
    const int64_t total = (M + kWGroup - 1) / kWGroup * kWGroup * cpr;
    switch (dt) {
        case kF32: quant_static_dt<kF32>(x, M, ldx * 4, nch, cpr, total, q, s, z, qmin, sat, st); break;
        case kBF16: quant_static_dt<kBF16>(x, M, ldx * 2, nch, cpr, total, q, s, z, qmin, sat, st); break;
        default: quant_static_dt<kF16>(x, M, ldx * 2, nch, cpr, total, q, s, z, qmin, sat, st); break;
    }
}

void launch_minmax(const void* x, int dt, int64_t M, int64_t K, int64_t ldx, float* mm,
                   hipStream_t st) {
    const int64_t total = M * (K / 8);
    if (total <= 0) return;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 256) blocks = 256;  // one per CU, each striding over the tensor
    const int nch = (int)(K / 8);
    switch (dt) {
        case kF32:
            hipLaunchKernelGGL(k_minmax<kF32>, dim3((unsigned)blocks), dim3(256), 0, st, x, ldx * 4,
                               total, nch, mm);
            break;
        case kBF16:
            hipLaunchKernelGGL(k_minmax<kBF16>, dim3((unsigned)blocks), dim3(256), 0, st, x,
                               ldx * 2, total, nch, mm);
            break;
        default:
            hipLaunchKernelGGL(k_minmax<kF16>, dim3((unsigned)blocks), dim3(256), 0, st, x, ldx * 2,
                               total, nch, mm);
            break;
    }
}

void launch_minmax_finalize(const float* mm, float* a_scale, int32_t* a_zp, hipStream_t st) {
    hipLaunchKernelGGL(k_minmax_finalize, dim3(1), dim3(64), 0, st, mm, a_scale, a_zp, 0);
}

void launch_absmax_finalize(const float* mm, float* a_scale, hipStream_t st) {
    hipLaunchKernelGGL(k_minmax_finalize, dim3(1), dim3(64), 0, st, mm, a_scale, nullptr, 1);
}

void launch_zeropoint_finalize(const float* mm, float* a_scale, int32_t* a_zp, hipStream_t st) {
    hipLaunchKernelGGL(k_minmax_finalize, dim3(1), dim3(64), 0, st, mm, a_scale, a_zp, 2);
}

}  // namespace pdq
