// Host-side launchers of the libpdq kernels.  Shapes and pointers are
// validated by the entry points (pdq_api.hip) before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pdq {

// quant.hip ---------------------------------------------------------------
// Outlier columns of the LLM.int8() decomposition, for the row quantizer:
// they take no part in the absmax and are coded 0, and with xo set their
// 16-bit values are also packed into xo[r, :] (pitch P, zero-padded to a
// multiple of 16) when *count <= max_out.  With w16 set, the same launch also
// gathers wo[n, :] = w16[n, idx[:]] (pitch P, zero-padded likewise) in extra
// workgroups of wrows weight rows each, placed first in the grid.
struct OutlierSkip {
    const uint8_t* mask;   // [K/8] bit j of byte c: column 8c + j is an outlier
    const int32_t* idx;    // [max_out] ascending outlier columns (the first max_out)
    const int32_t* count;  // total number of outlier columns
    int max_out;
    uint16_t* xo;          // [rows, P] or null
    int P;
    const uint16_t* w16;   // [N, ldw] 16-bit weight, or null: no W gather
    int64_t ldw;
    int64_t N;
    uint16_t* wo;          // [N, P]
    int wrows;             // weight rows per gather workgroup
    int gblocks;           // the launch's first gblocks workgroups gather W (set by the launcher)
};
// Per-row absmax symmetric INT8: q (packed tiles of pdq_device.h, padding
// zeroed), scale[r]; optional code sums; optional outlier columns to skip
// (16-bit inputs only).
void launch_quant_rows(const void* x, int dt, int64_t rows, int64_t K, int64_t ldx, int8_t* q,
                       float* scale, int32_t* colsum, const OutlierSkip* skip, hipStream_t st);

// Per-row (per-token) dynamic asymmetric INT8: range [min(min, 0), max(max,
// 0)] of each row, scale[r] = (hi - lo) / 255 (1 if empty), zp[r] =
// clamp(-128 - rne(lo / scale), -128, 127), q = clamp(rne(x / scale) + zp,
// -128, 127), packed, padding zeroed.
void launch_quant_rows_asym(const void* x, int dt, int64_t rows, int64_t K, int64_t ldx, int8_t* q,
                            float* scale, int32_t* zp, hipStream_t st);

// Fused SwiGLU producer + per-token quantizer (16-bit dt only): h = SiLU(gate)
// * up rounded to dt, then exactly launch_quant_rows' codes and scales of h;
// h also stored when h != nullptr (row pitch ldh).  ld* in elements.
void launch_silu_mul_quant(const void* gate, int64_t ldg, const void* up, int64_t ldu, int dt, int64_t rows,
                           int64_t K, int8_t* q, float* scale, void* h, int64_t ldh, hipStream_t st);

// Static code: q = clamp(rne(x / s) + z, -128, 127) (narrow: the range
// [-127, 127]), packed, padding zeroed; saturation count added to *sat
// (nullable).
void launch_quant_static(const void* x, int dt, int64_t M, int64_t K, int64_t ldx, float s, int z,
                         int8_t* q, uint32_t* sat, hipStream_t st, bool narrow = false);

// MinMax observer update of minmax[2]; optional finalisation to (S, Z).
void launch_minmax(const void* x, int dt, int64_t M, int64_t K, int64_t ldx, float* minmax,
                   hipStream_t st);
void launch_minmax_finalize(const float* minmax, float* a_scale, int32_t* a_zp, hipStream_t st);
// Tensor-wise absmax scale of the state: max(|min|, |max|) / 127 (1 if 0 or no value seen).
void launch_absmax_finalize(const float* minmax, float* a_scale, hipStream_t st);
// (S, Z) of the 254-step zero-point grid on [-127, 127] of the state's range.
void launch_zeropoint_finalize(const float* minmax, float* a_scale, int32_t* a_zp, hipStream_t st);

// gemm_i8.hip -------------------------------------------------------------
struct GemmArgs {
    const int8_t* A;  // packed activation codes (pdq_device.h)
    const int8_t* B;  // packed weight
    int M, N, K;
    const float* sa;  // [M] row scales, or null: the per-tensor scale s
    float s;
    int z;                  // zero point of A (static path), with colsum
    const int32_t* za;      // [M] per-row zero points of A (zp_mode 2), with colsum
    const int32_t* colsum;  // [N] code sums of B; used when zp_mode != 0
    const float* sb;  // [N] column scales
    const float* bias;  // [N] or null
    void* y;
    int64_t ldy;
    int32_t* acc_out;  // [M, N] or null, row pitch ldacc
    int64_t ldacc;     // 0: N (set by launch_gemm_i8)
    // 16-bit side product (outlier decomposition), used when xo != null
    const uint16_t* xo;  // [M, P]
    const uint16_t* wo;  // [N, P]
    int P;
    const int32_t* count;
    int max_count;
};
// out_dt: kBF16 output without side product, or kF16 / kBF16 with the side
// product when args.xo is set.  zp_mode (no side product): 1, y uses
// (float)(acc - z * colsum[n]) -- the static decode formula at any M; 2,
// (float)(acc - za[m] * colsum[n]) with the per-row scales sa.
void launch_gemm_i8(const GemmArgs& a, int out_dt, bool side, hipStream_t st, int zp_mode = 0);

// decode.hip --------------------------------------------------------------
struct DecodeArgs {
    const int8_t* xq;  // packed activation codes (pdq_device.h; launch_decode_gemv input)
    const int8_t* wq;  // packed weight
    int M, N, K;
    const float* sa;  // [M] per-token scales (launch_decode_gemv), or null: s, z
    const int32_t* za;  // [M] per-token zero points (with sa), or null
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
    int8_t* xq_out;  // packed activation codes, written by workgroup 0 (padding rows by others)
    uint32_t* sat;   // nullable saturation counter
    int narrow;      // codes clamped to [-127, 127] (symmetric or zero-point grid)
};
// Activations already quantized (xq); 16 x decode_groups(M, N) weight
// channels per workgroup (1 to 4 groups of 16).
void launch_decode_gemv(const DecodeArgs& a, hipStream_t st);
int decode_groups(int64_t M, int64_t N);
// Static quantization fused into the GEMM; only when decode_fusable(M, K).
bool decode_fusable(int64_t M, int64_t K);
void launch_decode_fused(const DecodeArgs& a, hipStream_t st);

// layout.hip --------------------------------------------------------------
// Plain row-major INT8 [rows, K] (row pitch ld bytes, 16-byte aligned rows)
// to the packed tile layout of pdq_device.h and back; the packed image has
// pdq_weight_bytes(rows, K) bytes, its padding written as zeros.
void launch_pack_int8(const int8_t* src, int64_t rows, int64_t K, int64_t ld, int8_t* packed, hipStream_t st);
void launch_unpack_int8(const int8_t* packed, int64_t rows, int64_t K, int8_t* dst, int64_t ld, hipStream_t st);

// outlier.hip -------------------------------------------------------------
// Row blocks of the partial predicate pass (at most 32), rows per block, and
// the byte pitch of one block's predicate row (K/8 chunks, padded to 16).
int outlier_row_blocks(int64_t M);
int64_t outlier_rows_per_block(int64_t M);
int outlier_partial_pitch(int64_t K);
// partial[b, c]: bit j set when some |x[m, 8c + j]| > threshold, m in row block b.
void launch_outlier_partial(const void* x, int dt, int64_t M, int64_t K, int64_t ldx,
                            float threshold, uint8_t* partial, hipStream_t st);
// From the partial predicates: mask[c] (K/8 bytes, padded to a multiple of
// 4), idx (first max_out ascending outlier columns), *count.
void launch_outlier_index(const uint8_t* partial, int64_t M, int64_t K, uint8_t* mask, int32_t* idx,
                          int32_t* count, int64_t max_out, hipStream_t st);

}  // namespace pdq
