// Host-side launchers of the libpdq kernels.  Shapes and pointers are
// validated by the entry points (pdq_api.hip) before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pdq {

// quant.hip ---------------------------------------------------------------
// Per-row absmax symmetric INT8: q[r,:] (dense, pitch K), scale[r]; optional
// code sums.  `skip_cols` (nullable, K flags) marks outlier columns by a
// nonzero flag: they take no part in the absmax and are coded 0.
void launch_quant_rows(const void* x, int dt, int64_t rows, int64_t K, int64_t ldx, int8_t* q,
                       float* scale, int32_t* colsum, const uint32_t* skip_cols, hipStream_t st);

// Static asymmetric code: q = clamp(rne(x / s) + z, -128, 127); saturation
// count added to *sat (nullable).
void launch_quant_static(const void* x, int dt, int64_t M, int64_t K, int64_t ldx, float s, int z,
                         int8_t* q, uint32_t* sat, hipStream_t st);

// MinMax observer update of minmax[2]; optional finalisation to (S, Z).
void launch_minmax(const void* x, int dt, int64_t M, int64_t K, int64_t ldx, float* minmax,
                   hipStream_t st);
void launch_minmax_finalize(const float* minmax, float* a_scale, int32_t* a_zp, hipStream_t st);

// gemm_i8.hip -------------------------------------------------------------
struct GemmArgs {
    const int8_t* A;  // [M, K] dense
    const int8_t* B;  // [N, K] dense
    int M, N, K;
    const float* sa;  // [M] row scales
    const float* sb;  // [N] column scales
    const float* bias;  // [N] or null
    void* y;
    int64_t ldy;
    int32_t* acc_out;  // [M, N] dense or null
    // 16-bit side product (outlier decomposition), used when xo != null
    const uint16_t* xo;  // [M, P]
    const uint16_t* wo;  // [N, P]
    int P;
    const int32_t* count;
    int max_count;
};
// out_dt: kBF16 output without side product, or kF16 / kBF16 with the side
// product when args.xo is set.
void launch_gemm_i8(const GemmArgs& a, int out_dt, bool side, hipStream_t st);

// decode.hip --------------------------------------------------------------
struct DecodeArgs {
    const int8_t* xq;  // [M, K] dense (launch_decode_gemv input)
    const int8_t* wq;  // [N, K] dense
    int M, N, K;
    float s;
    int z;
    const float* sw;
    const int32_t* colsum;
    const float* bias;
    uint16_t* y;
    int64_t ldy;
    int32_t* acc_out;
    // launch_decode_fused only: 16-bit or f32 activations, quantized in-kernel
    const void* x;
    int x_dt;
    int64_t ldx;
    int8_t* xq_out;  // [M, K] dense, written by workgroup 0
    uint32_t* sat;   // nullable saturation counter
};
// Activations already quantized (xq).
void launch_decode_gemv(const DecodeArgs& a, hipStream_t st);
// Static quantization fused into the GEMM; only when decode_fusable(M, K).
bool decode_fusable(int64_t M, int64_t K);
void launch_decode_fused(const DecodeArgs& a, hipStream_t st);

// outlier.hip -------------------------------------------------------------
void launch_fill_zero_u32(uint32_t* p, int64_t n, hipStream_t st);
// flags[k] |= (|x[m,k]| > threshold) for some m; flags must start at zero.
void launch_outlier_flags(const void* x, int dt, int64_t M, int64_t K, int64_t ldx,
                          float threshold, uint32_t* flags, hipStream_t st);
// Ascending indices of the nonzero flags (first max_out of them) and their count.
void launch_outlier_compact(const uint32_t* flags, int64_t K, int32_t* idx, int32_t* count,
                            int64_t max_out, hipStream_t st);
// dst[r, j] = src[r, idx[j]] for j < count, 0 for count <= j < round_up(count, 16);
// nothing when count > max_out.  16-bit elements.
void launch_gather_cols(const void* src, int64_t rows, int64_t ld, const int32_t* idx,
                        const int32_t* count, int max_out, uint16_t* dst, int P, hipStream_t st);

}  // namespace pdq
