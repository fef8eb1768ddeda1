/*
 * pdq.h -- W8A8 INT8 quantized linear layer for AMD MI355X (gfx950).
 *
 * C ABI of libpdq.so.  The operations are those of two sources:
 *
 *   [PDMIX-term]  "PDMIX inter-phase mixed quantization" terminology entry
 *                 (msModelSlim knowledge base): section 2.1 core idea,
 *                 section 2.3 mathematical description, section 2.4 key
 *                 properties.
 *   [PDMIX-guide] "PDMIX Parameter Configuration Workflow Guide": section 3
 *                 process overview; section 4 step 2 (recommended qconfig:
 *                 act scope pd_mix / int8 / symmetric false / minmax; weight
 *                 per_channel / int8 / symmetric true / minmax) and step 3
 *                 (configuration item table).
 *   [LLM.int8]    "LLM.int8(): 8-bit Matrix Multiplication for Transformers at
 *                 Scale" reading notes (blog.rainlin.top): part 1 section 1
 *                 absmax quantization, section 2 zero-point quantization and
 *                 its four-term expansion, section 3 granularity; part 2
 *                 vector-wise quantization, the four-step INT8 flow, the 16-bit
 *                 decomposition and the mixed-precision decomposition.
 *   [HW-accel]    "Hardware acceleration of quantized operations" (apxml course,
 *                 chapter 2): the role of compilers and runtime libraries
 *                 (kernel fusion: fewer memory round trips and launches).
 *
 * Arithmetic (identical on every entry point):
 *   rne(v)            round to nearest integer, ties to even
 *   symmetric scale   S = C / 127 (binary32, correctly rounded division) for
 *                     an absmax C; S = 1 when C == 0
 *   symmetric code    q = clamp(rne(x / S), -127, 127)       (x / S correctly rounded)
 *   asymmetric code   q = clamp(rne(x / S) + Z, -128, 127)
 *   dequant epilogue  y = (S_x * S_w) * (float)acc' [+ bias], every operation
 *                     rounded to binary32, no fused multiply-add; 16-bit
 *                     outputs are rounded to nearest even.
 *
 * Conventions:
 *   - Every pointer argument is DEVICE memory owned by the caller.  The
 *     library never allocates, frees or keeps a pointer after returning, and
 *     never synchronises: all work is enqueued on `stream` (a hipStream_t;
 *     NULL means the null stream), and buffers must stay valid until that
 *     work has completed.
 *   - Floating-point matrices are row-major; leading dimensions (ld*) are in
 *     elements.  INT8 matrices (weights wq, activation codes xq) are in the
 *     packed tile layout described at pdq_quantize_weight.  Inner dimension K
 *     must be a positive multiple of 16 (at most 65536; K == 0 is
 *     PDQ_ERR_SHAPE, since every kernel reads at least one 16-value chunk of
 *     each row it touches); every base pointer and every row pitch (ld *
 *     element size) of a K-wide operand must be a multiple of 16 bytes.  M and
 *     N may be 0 (nothing is written then); each is at most 2^21 (2097152),
 *     one operand holds at most 2^34 values (M * K, N * K) and one product at
 *     most 2^39 outputs (M * N), so that every launch grid stays inside the
 *     dispatch limits; larger shapes are PDQ_ERR_SHAPE.
 *   - Every argument check runs on the host before anything is enqueued; on
 *     error nothing is launched and no output is touched.  After the
 *     launches, a HIP launch error is reported as PDQ_ERR_HIP.
 *   - The library holds no mutable global state; calls are reentrant.
 *     Outputs of one call must not alias its inputs.
 */
#ifndef PDQ_H_
#define PDQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PDQ_OK = 0,
    PDQ_ERR_NULL = 1,        /* a required pointer is NULL                      */
    PDQ_ERR_SHAPE = 2,       /* negative or too large size, K not in 16, 32, .., 65536, ld too small */
    PDQ_ERR_DTYPE = 3,       /* dtype not accepted by this entry point          */
    PDQ_ERR_ALIGN = 4,       /* pointer or row pitch not 16-byte aligned        */
    PDQ_ERR_UNSUPPORTED = 5, /* value out of range (scale, zero point, ...)     */
    PDQ_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required         */
    PDQ_ERR_HIP = 8,         /* the HIP runtime reported a launch error         */
    /* range sentinels, never returned: every 32-bit value is a valid value of
       the type, so an unknown code passed to pdq_status_string is defined */
    PDQ_STATUS_MIN_ENUM_ = -0x7fffffff - 1,
    PDQ_STATUS_MAX_ENUM_ = 0x7fffffff
} pdq_status;

typedef enum {
    PDQ_F32 = 0,  /* IEEE binary32                */
    PDQ_BF16 = 1, /* bfloat16 (upper half of f32) */
    PDQ_F16 = 2,  /* IEEE binary16                */
    /* range sentinels, not dtypes: any 32-bit value a caller passes is a
       valid value of the type, and anything but the three above is refused
       with PDQ_ERR_DTYPE */
    PDQ_DTYPE_MIN_ENUM_ = -0x7fffffff - 1,
    PDQ_DTYPE_MAX_ENUM_ = 0x7fffffff
} pdq_dtype;

/* Human-readable name of a status code (static string; never NULL). */
const char* pdq_status_string(pdq_status s);

/*
 * Offline weight quantization, per output channel, symmetric, MinMax
 * (= absmax for a symmetric grid).  [PDMIX-guide] step 2 weight qconfig;
 * [PDMIX-term] 2.1/2.4: one INT8 copy serves both phases; [LLM.int8] part 1
 * section 1 absmax formula.
 *
 *   w        [N, K] of w_dt (F32, BF16 or F16), row pitch ldw >= K
 *   wq       packed INT8 weight out, pdq_weight_bytes(N, K) bytes: the codes
 *            wq[n, k] in blocks of 16 output channels x 64 K values; block
 *            (g, s) -- channels 16 g .., K values 64 s .. -- is the 1024 bytes
 *            at (g * ceil(K / 64) + s) * 1024, channel r of the group its 64
 *            bytes at r * 64, and within them the 16-byte chunk c (K values
 *            64 s + 16 c ..) sits at position c ^ ((r >> 2) & 3).  Channels
 *            >= N and K values >= K are written as 0.  Every GEMM entry point
 *            takes its weight in this layout.
 *   w_scale  [N] float out: S_w[n] = max_k |w[n,k]| / 127
 *   w_colsum [N] int32 out, or NULL: sum_k wq[n,k] (needed by decode's
 *            zero-point correction, [LLM.int8] part 1 section 2)
 */
size_t pdq_weight_bytes(int64_t N, int64_t K);

/*
 * Layout conversion for callers that hold INT8 matrices in plain row-major
 * form (weights quantized by another tool, codes to be read back on the
 * device): no quantization, only the byte order.
 *
 * pdq_pack_int8: src [rows, K] int8, row pitch ld bytes (ld >= K, src and ld
 *   16-byte aligned, K a multiple of 16) -> packed, pdq_weight_bytes(rows, K)
 *   bytes in the layout described above (rows >= rows and K values >= K
 *   written as 0).  A weight packed this way, with its own per-channel scales
 *   and code sums, is a valid wq for every GEMM entry point.
 * pdq_unpack_int8: the inverse, packed -> dst [rows, K] int8 with row pitch
 *   ld bytes (the padding is not copied; the bytes of dst between K and ld are
 *   left untouched).
 * Errors as elsewhere: PDQ_ERR_SHAPE, PDQ_ERR_NULL, PDQ_ERR_ALIGN, checked
 * before anything is enqueued.
 */
pdq_status pdq_pack_int8(const int8_t* src, int64_t rows, int64_t K, int64_t ld, int8_t* packed, void* stream);
pdq_status pdq_unpack_int8(const int8_t* packed, int64_t rows, int64_t K, int8_t* dst, int64_t ld, void* stream);

/*
 * Activation codes (the xq of every entry point below) use the same packed
 * layout with M rows in place of the N channels: pdq_act_bytes(M, K) bytes
 * (= pdq_weight_bytes(M, K)), rows >= M and K values >= K written as 0.  The
 * quantizers write xq in it and the GEMMs read it: as the 16-row x 64 tiles
 * of the MFMA operands, every load a whole cache line.
 */
size_t pdq_act_bytes(int64_t M, int64_t K);

/*
 * The INT8 GEMM kernel that pdq_gemm_per_token, pdq_gemm_per_token_asym,
 * pdq_gemm_static and the linear entry points run for M activation rows and N
 * weight channels (pdq_linear_decode runs neither when it fuses the
 * quantizer into the skinny kernel; pdq_linear_int8_outlier always runs the
 * tiled one).  Both give the same bits.  -1 when M < 1 or N < 1.
 *   PDQ_GEMM_SKINNY  one pass over the weight per 64 activation rows,
 *                    16 to 64 channels per workgroup (all M <= 64, and
 *                    larger M while that is estimated to be faster)
 *   PDQ_GEMM_TILED   256 x 256 output tiles staged through LDS
 */
enum { PDQ_GEMM_SKINNY = 0, PDQ_GEMM_TILED = 1 };
int pdq_gemm_kernel(int64_t M, int64_t N);

/*
 * Weight channels per workgroup of the skinny kernel for M activation rows
 * and N weight channels: 16, 32, 48 or 64 (16 up to 16 rows; beyond, the
 * width that moves the fewest bytes through the busiest compute unit).  A
 * performance choice only: every width gives the same bits.  -1 when M < 1
 * or N < 1.
 */
int pdq_skinny_channels(int64_t M, int64_t N);

pdq_status pdq_quantize_weight(const void* w, pdq_dtype w_dt, int64_t N, int64_t K, int64_t ldw,
                               int8_t* wq, float* w_scale, int32_t* w_colsum, void* stream);

/*
 * Static calibration for the decode phase: MinMax observer over calibration
 * batches, then the per-tensor asymmetric scale and zero point.
 * [PDMIX-term] 2.3 decode formula and section 3 (MinMax); [PDMIX-guide]
 * section 3: decode measures and exports per-tensor asymmetric parameters.
 *
 *   x        [M, K] batch of x_dt, row pitch ldx; may be NULL when M == 0
 *   minmax   float[2] in/out running {min, max}; initialise to {+INF, -INF}
 *            before the first batch.  min/max are exact and order-free, so
 *            a saved state resumes calibration bit-exactly.
 *   a_scale  float[1] out or NULL; a_zp int32[1] out or NULL.  When both are
 *            non-NULL the updated state is finalised (after this batch):
 *            range [lo, hi] = [min(min, 0), max(max, 0)];
 *            S = (hi - lo) / 255 (S = 1 if hi == lo);
 *            Z = clamp(-128 - rne(lo / S), -128, 127).
 *            Passing only one of them is PDQ_ERR_NULL.
 */
pdq_status pdq_calibrate_static(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                float* minmax, float* a_scale, int32_t* a_zp, void* stream);

/*
 * Prefill linear: per-token dynamic symmetric activation quantization, INT8
 * GEMM with INT32 accumulation, fused dequantizing epilogue, bf16 output.
 * [PDMIX-term] 2.3 prefill formula with Z_token = 0 ([PDMIX-guide] step 3:
 * prefill is per-token symmetric); [LLM.int8] part 2 steps (2)-(4) and the
 * vector-wise outer product of scales.
 *
 *   x        [M, K] of x_dt (F32, BF16, F16), row pitch ldx
 *   wq       packed INT8 weight from pdq_quantize_weight; w_scale [N] float
 *   bias     [N] float or NULL
 *   xq       packed int8 codes out (pdq_act_bytes(M, K) bytes), x_scale [M]
 *            float out: the quantized activations and their per-token
 *            scales (also the GEMM operand)
 *   y        [M, N] bfloat16 out (uint16 bit patterns), row pitch ldy >= N
 *            y = bf16((S_x[m] * S_w[n]) * (float)acc[m,n] [+ bias[n]])
 *   acc_out  [M, N] int32 out (dense) or NULL: acc = sum_k xq[m,k] wq[n,k]
 */
pdq_status pdq_linear_prefill(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                              const int8_t* wq, const float* w_scale, const float* bias, int64_t N,
                              int8_t* xq, float* x_scale, uint16_t* y, int64_t ldy,
                              int32_t* acc_out, void* stream);

/*
 * Decode linear: per-tensor static asymmetric activation quantization with
 * the offline (S, Z), INT8 GEMM, zero-point correction through the weight
 * code sums, fused epilogue, bf16 output.  [PDMIX-term] 2.3 decode formula
 * (round, then add Z); 2.4: static scales may saturate on inputs the
 * calibration did not cover; [LLM.int8] part 1 section 2 four-term expansion
 * reduced to a symmetric weight: acc' = acc - Z * colsum[n].
 *
 *   x          [M, K] of x_dt, row pitch ldx (any M; decode batches are small)
 *   a_scale    S > 0 and finite; a_zp Z in [-128, 127] (host values, from
 *              pdq_calibrate_static)
 *   wq, w_scale, w_colsum  from pdq_quantize_weight (w_colsum required)
 *   bias       [N] float or NULL
 *   xq         packed int8 codes out (pdq_act_bytes(M, K) bytes):
 *              q = clamp(rne(x / S) + Z, -128, 127)
 *   y          [M, N] bfloat16 out, row pitch ldy:
 *              y = bf16((S * S_w[n]) * (float)(acc - Z * colsum[n]) [+ bias[n]])
 *   acc_out    [M, N] int32 out or NULL: raw acc = sum_k xq wq (before the
 *              zero-point term)
 *   sat_count  uint32[1] or NULL: INCREMENTED by the number of values whose
 *              unclamped code rne(x / S) + Z lies outside [-128, 127]; the
 *              caller resets it when it wants a fresh count.
 */
pdq_status pdq_linear_decode(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                             float a_scale, int32_t a_zp, const int8_t* wq, const float* w_scale,
                             const int32_t* w_colsum, const float* bias, int64_t N, int8_t* xq,
                             uint16_t* y, int64_t ldy, int32_t* acc_out, uint32_t* sat_count,
                             void* stream);

/*
 * Static tensor-wise SYMMETRIC W8A8: [LLM.int8] part 1 section 1 absmax
 * quantization, one scale for the whole activation tensor (section 3,
 * tensor-wise), measured offline over calibration batches: the conventional
 * static W8A8 scheme, with static activation scales, that [PDMIX-term]
 * section 2 compares PDMIX with.  Same kernels as the decode linear with
 * Z = 0 and the symmetric code range.
 *
 * pdq_calibrate_static_sym: updates the same MinMax state as
 *   pdq_calibrate_static (minmax[2] in/out, initialise to {+INF, -INF});
 *   when a_scale is non-NULL it is finalised to S = C / 127 with
 *   C = max(|min|, |max|) (S = 1 if C == 0 or no value was seen).
 * pdq_quantize_static_sym: xq = clamp(rne(x / S), -127, 127) (packed,
 *   pdq_act_bytes(M, K) bytes); sat_count (nullable) INCREMENTED by the
 *   number of values with |rne(x / S)| > 127.
 * pdq_linear_static_sym: the quantizer then the GEMM, y = bf16((S * S_w[n]) *
 *   (float)acc [+ bias[n]]) (one launch for M * K <= 8192); acc_out [M, N]
 *   int32 or NULL.  a_scale > 0 and finite, else PDQ_ERR_UNSUPPORTED.
 */
pdq_status pdq_calibrate_static_sym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                    float* minmax, float* a_scale, void* stream);

pdq_status pdq_quantize_static_sym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                   float a_scale, int8_t* xq, uint32_t* sat_count, void* stream);

pdq_status pdq_linear_static_sym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                 float a_scale, const int8_t* wq, const float* w_scale, const float* bias,
                                 int64_t N, int8_t* xq, uint16_t* y, int64_t ldy, int32_t* acc_out,
                                 uint32_t* sat_count, void* stream);

/*
 * Static tensor-wise ZERO-POINT W8A8 with 254 levels: [LLM.int8] part 1
 * section 2 zero-point quantization, nd_x = 2 * 127 / (max - min), taken
 * tensor-wise with a static scale like the symmetric variant above.  The
 * page's formulas for the zero point and the code are garbled; read in the
 * decode grid's form: over the calibrated range [lo, hi] = [min(min, 0),
 * max(max, 0)], S = (hi - lo) / 254 (1 if hi == lo), Z = clamp(-127 - rne(lo
 * / S), -127, 127), codes clamp(rne(x / S) + Z, -127, 127); the GEMM removes
 * Z through the weight code sums (the four-term expansion with a symmetric
 * weight): y = bf16((S * S_w[n]) * (float)(acc - Z * colsum[n]) [+ bias[n]]).
 *
 * pdq_calibrate_zeropoint: the MinMax state as pdq_calibrate_static; a_scale
 *   and a_zp (both or neither) receive the finalised (S, Z).
 * pdq_quantize_zeropoint: xq packed (pdq_act_bytes(M, K) bytes); sat_count
 *   (nullable) INCREMENTED by the number of rne(x / S) + Z outside [-127, 127].
 * pdq_linear_zeropoint: quantizer + GEMM (one launch for M * K <= 8192);
 *   w_colsum required; acc_out [M, N] int32 (raw acc) or NULL.
 *   a_scale > 0 and finite and a_zp in [-127, 127], else PDQ_ERR_UNSUPPORTED.
 */
pdq_status pdq_calibrate_zeropoint(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                   float* minmax, float* a_scale, int32_t* a_zp, void* stream);

pdq_status pdq_quantize_zeropoint(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                  float a_scale, int32_t a_zp, int8_t* xq, uint32_t* sat_count, void* stream);

pdq_status pdq_linear_zeropoint(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                float a_scale, int32_t a_zp, const int8_t* wq, const float* w_scale,
                                const int32_t* w_colsum, const float* bias, int64_t N, int8_t* xq,
                                uint16_t* y, int64_t ldy, int32_t* acc_out, uint32_t* sat_count,
                                void* stream);

/*
 * Prefill linear with per-token dynamic ASYMMETRIC activations: the
 * [PDMIX-term] 2.3 prefill formula taken with its per-token zero point
 * Z_token, Q = clamp(round(X / S_token) + Z_token, -128, 127), both computed
 * online per token.  A token's (S, Z) are the MinMax asymmetric grid of its
 * own range (as pdq_calibrate_static finalises a per-tensor range, one token
 * at a time): lo = min(min_k x[m,k], 0), hi = max(max_k x[m,k], 0);
 * S_x[m] = (hi - lo) / 255 (1 if hi == lo); Z_x[m] = clamp(-128 - rne(lo /
 * S_x[m]), -128, 127); xq = clamp(rne(x / S_x[m]) + Z_x[m], -128, 127).  The
 * GEMM removes the zero point through the weight code sums ([LLM.int8] part 1
 * section 2 with a symmetric weight):
 *   y = bf16((S_x[m] * S_w[n]) * (float)(acc - Z_x[m] * colsum[n]) [+ bias[n]]).
 * (The default PDMIX prefill, pdq_linear_prefill, is per-token symmetric.)
 *
 *   x, wq, w_scale, bias, y, ldy   as in pdq_linear_prefill
 *   w_colsum  [N] int32 from pdq_quantize_weight (required)
 *   xq        packed int8 codes out (pdq_act_bytes(M, K) bytes)
 *   x_scale   [M] float out; x_zp [M] int32 out
 *   acc_out   [M, N] int32 out or NULL: raw acc = sum_k xq wq (before the
 *             zero-point term)
 */
pdq_status pdq_linear_prefill_asym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                   const int8_t* wq, const float* w_scale, const int32_t* w_colsum,
                                   const float* bias, int64_t N, int8_t* xq, float* x_scale, int32_t* x_zp,
                                   uint16_t* y, int64_t ldy, int32_t* acc_out, void* stream);

/*
 * Building blocks of the two PDMIX phases.  pdq_linear_prefill is
 * pdq_quantize_per_token followed by pdq_gemm_per_token; pdq_linear_decode is
 * pdq_quantize_static followed by pdq_gemm_static.  They are exposed for
 * callers that quantize an activation once and feed several weight matrices
 * with it (e.g. separate Q, K and V projections of one hidden state), or that
 * produce the INT8 activations themselves.  Arguments as in the composite
 * calls above; xq is the packed [M, K] codes (pdq_act_bytes(M, K) bytes).
 */
/* Per-token quantizer: S_x[m] = max_k |x[m,k]| / 127, xq = clamp(rne(x / S_x), -127, 127). */
pdq_status pdq_quantize_per_token(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                  int8_t* xq, float* x_scale, void* stream);

/* INT8 GEMM + per-token epilogue: y = bf16((S_x[m] * S_w[n]) * (float)(sum_k xq wq) [+ bias[n]]). */
pdq_status pdq_gemm_per_token(const int8_t* xq, const float* x_scale, int64_t M, int64_t K,
                              const int8_t* wq, const float* w_scale, const float* bias, int64_t N,
                              uint16_t* y, int64_t ldy, int32_t* acc_out, void* stream);

/* The two halves of pdq_linear_prefill_asym: the per-token asymmetric quantizer (x_scale,
 * x_zp [M] out) and the GEMM with the per-token zero-point epilogue. */
pdq_status pdq_quantize_per_token_asym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                       int8_t* xq, float* x_scale, int32_t* x_zp, void* stream);

pdq_status pdq_gemm_per_token_asym(const int8_t* xq, const float* x_scale, const int32_t* x_zp, int64_t M,
                                   int64_t K, const int8_t* wq, const float* w_scale,
                                   const int32_t* w_colsum, const float* bias, int64_t N, uint16_t* y,
                                   int64_t ldy, int32_t* acc_out, void* stream);

/* Static quantizer: xq = clamp(rne(x / S) + Z, -128, 127); sat_count (nullable) incremented. */
pdq_status pdq_quantize_static(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                               float a_scale, int32_t a_zp, int8_t* xq, uint32_t* sat_count,
                               void* stream);

/* INT8 GEMM + zero-point epilogue:
 * y = bf16((S * S_w[n]) * (float)(sum_k xq wq - Z * colsum[n]) [+ bias[n]]);
 * w_colsum is required unless a_zp == 0 (then also the static symmetric GEMM). */
pdq_status pdq_gemm_static(const int8_t* xq, int64_t M, int64_t K, float a_scale, int32_t a_zp,
                           const int8_t* wq, const float* w_scale, const int32_t* w_colsum,
                           const float* bias, int64_t N, uint16_t* y, int64_t ldy, int32_t* acc_out,
                           void* stream);

/*
 * Fused producer + per-token quantizer for the input of an MLP down
 * projection: h = SiLU(gate) * up is formed in registers and quantized per
 * token, instead of being written to memory by one kernel and read back by
 * the quantizer ([HW-accel], kernel fusion).  SiLU(g) = g * sigmoid(g), the
 * gate of a SwiGLU MLP (the pages define no activation function; this is the
 * textbook one).  Each element is computed in binary32 -- e = 2^(-|g| log2 e)
 * and r = 1 / (1 + e) on the hardware exp2 and reciprocal (1 ulp each),
 * sigmoid = (g >= 0 ? r : e * r), h = (g * sigmoid) * up; relative error
 * below (1.5 |g| + 8) 2^-24 for |g| < 87 -- and then rounded to dt, so that h
 * is the value an unfused kernel of that dtype would store (up to that error
 * next to a tie of dt).  The codes are exactly those of
 * pdq_quantize_per_token applied to h.
 *
 *   gate, up     [M, K] of dt (BF16 or F16; F32 is rejected), row pitches
 *                ldg, ldu (e.g. the two halves of a fused gate/up GEMM
 *                output [M, 2K]: up = gate + K, ldg = ldu = 2K)
 *   xq           packed int8 codes out (pdq_act_bytes(M, K) bytes)
 *   x_scale      [M] float out: max_k |h[m,k]| / 127 (1 for an all-zero row)
 *   h            [M, K] of dt out, row pitch ldh, or NULL: also store h
 *                (must not overlap gate or up)
 */
pdq_status pdq_silu_mul_quantize_per_token(const void* gate, const void* up, pdq_dtype dt, int64_t M,
                                           int64_t K, int64_t ldg, int64_t ldu, int8_t* xq,
                                           float* x_scale, uint16_t* h, int64_t ldh, void* stream);

/* pdq_silu_mul_quantize_per_token (h not stored) followed by pdq_gemm_per_token: the
 * down projection y = bf16((S_x[m] * S_w[n]) * (float)(sum_k xq wq) [+ bias[n]]) of
 * h = SiLU(gate) * up, with K the intermediate size.  Other arguments as in
 * pdq_linear_prefill. */
pdq_status pdq_linear_prefill_silu_mul(const void* gate, const void* up, pdq_dtype dt, int64_t M, int64_t K,
                                       int64_t ldg, int64_t ldu, const int8_t* wq, const float* w_scale,
                                       const float* bias, int64_t N, int8_t* xq, float* x_scale,
                                       uint16_t* y, int64_t ldy, int32_t* acc_out, void* stream);

/*
 * LLM.int8() vector-wise quantization with the 16-bit outlier decomposition.
 * [LLM.int8] part 2: outlier columns are the hidden dimensions whose
 * magnitude exceeds the threshold (6.0 in the text); the regular part is
 * quantized per row (absmax over the regular columns) against the
 * per-output-channel INT8 weight and multiplied in INT8; the outlier columns
 * of x and of the 16-bit weight are multiplied in 16-bit floating point
 * (binary32 accumulation); the two results are summed into a 16-bit output.
 *
 *   x            [M, K] of dt (F16 or BF16), row pitch ldx
 *   threshold    column k is an outlier iff max_m |x[m,k]| > threshold
 *                (strict; +INF gives no outliers; NaN is rejected)
 *   wq, w_scale  the shared INT8 weight (pdq_quantize_weight over full K)
 *   w16          [N, K] of dt: the original 16-bit weight, row pitch ldw
 *   bias         [N] float or NULL
 *   y            [M, N] of dt out, row pitch ldy
 *   xq           packed int8 codes out (pdq_act_bytes(M, K) bytes): regular
 *                columns quantized, outliers 0
 *   x_scale      [M] float out: absmax over regular columns / 127
 *   outlier_idx  int32[max_outliers] out: ascending outlier columns (the
 *                first max_outliers of them)
 *   n_outlier    int32[1] out: the number of outlier columns found
 *   max_outliers capacity for the 16-bit part, >= 0.  If more columns than
 *                this exceed the threshold, every element of y is set to
 *                NaN (n_outlier still reports the true count).
 *   workspace    device scratch of at least
 *                pdq_linear_int8_outlier_workspace(M, N, K, max_outliers)
 *                bytes, 256-byte aligned; its contents on entry do not matter
 *   acc_out      [M, N] int32 out or NULL: the INT8 part's accumulator
 */
size_t pdq_linear_int8_outlier_workspace(int64_t M, int64_t N, int64_t K, int64_t max_outliers);

pdq_status pdq_linear_int8_outlier(const void* x, pdq_dtype dt, int64_t M, int64_t K, int64_t ldx,
                                   float threshold, const int8_t* wq, const float* w_scale,
                                   const void* w16, int64_t ldw, const float* bias, int64_t N,
                                   void* y, int64_t ldy, int8_t* xq, float* x_scale,
                                   int32_t* outlier_idx, int32_t* n_outlier, int64_t max_outliers,
                                   void* workspace, size_t workspace_bytes, int32_t* acc_out,
                                   void* stream);

/*
 * pdq_linear_int8_outlier without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Arguments, checks, results and
 * kernels are those of pdq_linear_int8_outlier; the workspace is instead a
 * scratch array compiled into the library, one copy per GPU (allocated when
 * the library's code is loaded on that GPU, held until the process ends) of
 * pdq_noalloc_scratch_bytes() = 8 MiB.  Calls whose
 * pdq_linear_int8_outlier_workspace(M, N, K, max_outliers) exceeds that are
 * refused with PDQ_ERR_WORKSPACE before anything is enqueued (the 2048 x 8192
 * -> 28672 layer with 64 outlier columns needs 3.9 MB).  The stream must belong
 * to the current device (else PDQ_ERR_UNSUPPORTED).  The first call on a
 * device looks up that device's scratch address (a HIP symbol query, no
 * allocation); no call allocates or frees memory.
 *
 * Every call on a GPU shares that GPU's scratch, and nothing in it carries
 * over between calls (every byte a call reads, it first writes): calls that
 * overlap in time on one GPU -- on different streams, or from different host
 * threads without ordering -- race and give undefined results.  Calls on one
 * stream are ordered and safe.
 */
size_t pdq_noalloc_scratch_bytes(void);

pdq_status pdq_linear_int8_outlier_noalloc(const void* x, pdq_dtype dt, int64_t M, int64_t K, int64_t ldx,
                                           float threshold, const int8_t* wq, const float* w_scale,
                                           const void* w16, int64_t ldw, const float* bias, int64_t N,
                                           void* y, int64_t ldy, int8_t* xq, float* x_scale,
                                           int32_t* outlier_idx, int32_t* n_outlier, int64_t max_outliers,
                                           int32_t* acc_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PDQ_H_ */
