// The C entry points of libpdq: host-side argument checks, then the kernel
// launches of each operation on the caller's stream.  Declared and
// documented in include/pdq.h.

#include <math.h>

#include <algorithm>
#include <mutex>

#include "pdq.h"
#include "pdq_device.h"
#include "pdq_kernels.h"

using namespace pdq;

#define PDQ_TRY(expr)                         \
    do {                                      \
        const pdq_status s_ = (expr);         \
        if (s_ != PDQ_OK) return s_;          \
    } while (0)


namespace {

constexpr int64_t kMaxK = 65536;        // |sum_k (q_x - Z) q_w| < 255 * 127 * K stays in int32
// Rows of any operand (M activation rows, N weight rows = output channels).
// Together with the two products below this keeps every launch grid inside
// the dispatch limits with room to spare: the skinny GEMM's second grid
// dimension is rows / 64, the per-token quantizers run 256 threads per row,
// the static quantizer one thread per 8 values, the tiled GEMM 256 threads
// per 256 x 256 output tile.
constexpr int64_t kMaxRows = int64_t(1) << 21;
constexpr int64_t kMaxValues = int64_t(1) << 34;   // M x K of one operand
constexpr int64_t kMaxOutputs = int64_t(1) << 39;  // M x N of one product
// Which kernel runs an M x N INT8 GEMM, whichever quantization scheme
// produced the codes: the skinny (weight-streaming) kernel of decode.hip or
// the 256 x 256-tile GEMM.  The skinny kernel's work is ceil(N / 16) x
// ceil(M / 64) units, each one pass over the K tiles of 16 weight channels
// for up to 64 activation rows, and costs about 4 us plus 4.7 us per 256 of
// them with 16 channels per workgroup, 3.6 us with more; the tiled GEMM costs
// about 52 us per round of 256 tiles, however few tiles the round holds (all
// measured on MI355X at K = 4096; K scales both alike).  Up to 64 rows the
// skinny kernel always runs.
bool skinny_gemm(int64_t M, int64_t N) {
    if (M <= 64) return true;
    const double units = (double)((N + 15) / 16) * (double)((M + 63) / 64);
    const double tiles = (double)((M + 255) / 256) * (double)((N + 255) / 256);
    const double per256 = decode_groups(M, N) > 1 ? 3.6 : 4.7;
    return 4.0 + per256 * units / 256.0 < 52.0 * ceil(tiles / 256.0);
}

int elem_bytes(int dt) { return dt == PDQ_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == PDQ_F32 || dt == PDQ_BF16 || dt == PDQ_F16; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape rules shared by every K-wide operand.  K == 0 is refused: the kernels
// read at least one 16-value chunk of every row they touch.
pdq_status check_mk(int64_t M, int64_t K, int64_t ld) {
    if (M < 0 || K <= 0 || M > kMaxRows || K > kMaxK || K % 16 != 0) return PDQ_ERR_SHAPE;
    if (M * K > kMaxValues) return PDQ_ERR_SHAPE;
    if (ld < K || ld < 0) return PDQ_ERR_SHAPE;
    return PDQ_OK;
}

// A [rows, K] operand with `ebytes`-byte elements and row pitch `ld`.
pdq_status check_operand(const void* p, int ebytes, int64_t rows, int64_t K, int64_t ld) {
    pdq_status s = check_mk(rows, K, ld);
    if (s != PDQ_OK) return s;
    if (rows > 0 && K > 0 && !p) return PDQ_ERR_NULL;
    if (!aligned(p, 16) || (ld * ebytes) % 16 != 0) return PDQ_ERR_ALIGN;
    return PDQ_OK;
}

pdq_status launched() { return hipGetLastError() == hipSuccess ? PDQ_OK : PDQ_ERR_HIP; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int64_t side_pitch(int64_t max_out) { return (max_out + 15) / 16 * 16; }

}  // namespace

// Scratch of pdq_linear_int8_outlier_noalloc: one copy per device, held until
// the process ends.  Host code never passes `scratch` itself to a kernel (on
// the host it names a stand-in, not device memory): the device address comes
// from hipGetSymbolAddress, looked up once per device with that device current
// and kept in scratch_ptr[device].
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
char* scratch_ptr[kMaxDevices] = {};

// The scratch address on the device of `st` (the current device: a stream of
// another device is refused).
pdq_status scratch_for_stream(hipStream_t st, char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PDQ_ERR_HIP;
    if (st) {
        int sdev = -1;
        if (hipStreamGetDevice(st, &sdev) != hipSuccess) return PDQ_ERR_HIP;
        if (sdev != dev) return PDQ_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PDQ_ERR_HIP;
        scratch_ptr[dev] = static_cast<char*>(p);
    }
    *out = scratch_ptr[dev];
    return PDQ_OK;
}

// Host-side checks of the LLM.int8 call, shared by both of its entry points
// (no HIP call).
pdq_status check_int8_outlier(const void* x, pdq_dtype dt, int64_t M, int64_t K, int64_t ldx, float threshold,
                              const int8_t* wq, const float* w_scale, const void* w16, int64_t ldw,
                              const float* bias, int64_t N, void* y, int64_t ldy, int8_t* xq, float* x_scale,
                              int32_t* outlier_idx, int32_t* n_outlier, int64_t max_outliers, int32_t* acc_out) {
    if (dt != PDQ_F16 && dt != PDQ_BF16) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(dt), M, K, ldx));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N || ldw < K) return PDQ_ERR_SHAPE;
    if (max_outliers < 0 || max_outliers > K) return PDQ_ERR_SHAPE;
    if (isnan(threshold)) return PDQ_ERR_UNSUPPORTED;
    if (!n_outlier || (max_outliers > 0 && !outlier_idx)) return PDQ_ERR_NULL;
    if (N > 0 && (!w_scale || (K > 0 && !w16))) return PDQ_ERR_NULL;
    if (M > 0 && ((K > 0 && !xq) || !x_scale)) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(bias, 4) ||
        !aligned(y, 2) || !aligned(w16, 2) || !aligned(acc_out, 4) || !aligned(outlier_idx, 4) ||
        !aligned(n_outlier, 4))
        return PDQ_ERR_ALIGN;
    return PDQ_OK;
}

// The launches of the LLM.int8 call on a workspace of at least
// pdq_linear_int8_outlier_workspace(M, N, K, max_outliers) bytes, 256-byte
// aligned: predicates per row block -> mask, index list, count and the W
// gather -> INT8 codes of the regular columns with the X gather -> INT8 GEMM
// with the 16-bit side product in its epilogue.  Every byte of the workspace
// that is read is first written by the same call.
void run_int8_outlier(const void* x, pdq_dtype dt, int64_t M, int64_t K, int64_t ldx, float threshold,
                      const int8_t* wq, const float* w_scale, const void* w16, int64_t ldw, const float* bias,
                      int64_t N, void* y, int64_t ldy, int8_t* xq, float* x_scale, int32_t* outlier_idx,
                      int32_t* n_outlier, int64_t max_outliers, char* ws, int32_t* acc_out, hipStream_t st) {
    const int64_t P = side_pitch(max_outliers);
    const size_t pitch = (size_t)outlier_partial_pitch(K);
    uint8_t* partial = reinterpret_cast<uint8_t*>(ws);
    ws += align256((size_t)outlier_row_blocks(M) * pitch);
    uint8_t* mask = reinterpret_cast<uint8_t*>(ws);
    ws += align256(pitch);
    uint16_t* xo = reinterpret_cast<uint16_t*>(ws);
    ws += align256((size_t)(M * P * 2));
    uint16_t* wo = reinterpret_cast<uint16_t*>(ws);

    launch_outlier_partial(x, dt, M, K, ldx, threshold, partial, st);
    launch_outlier_index(partial, M, K, mask, outlier_idx, n_outlier, max_outliers, st);
    if (M > 0) {
        // the regular-column quantizer; extra workgroups of its launch gather
        // W_out (at most 256 of them)
        OutlierSkip skip{};
        skip.mask = mask;
        skip.idx = outlier_idx;
        skip.count = n_outlier;
        skip.max_out = (int)max_outliers;
        skip.xo = xo;
        skip.P = (int)P;
        skip.w16 = static_cast<const uint16_t*>(w16);
        skip.ldw = ldw;
        skip.N = N;
        skip.wo = wo;
        skip.wrows = (int)std::max<int64_t>(64, (N + 255) / 256);
        launch_quant_rows(x, dt, M, K, ldx, xq, x_scale, nullptr, &skip, st);
    }
    GemmArgs g{};
    g.A = xq;
    g.B = wq;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.sa = x_scale;
    g.sb = w_scale;
    g.bias = bias;
    g.y = y;
    g.ldy = ldy;
    g.acc_out = acc_out;
    g.xo = xo;
    g.wo = wo;
    g.P = (int)P;
    g.count = n_outlier;
    g.max_count = (int)max_outliers;
    launch_gemm_i8(g, dt, true, st);
}

}  // namespace

extern "C" {

const char* pdq_status_string(pdq_status s) {
    switch (s) {
        case PDQ_OK: return "ok";
        case PDQ_ERR_NULL: return "required pointer is NULL";
        case PDQ_ERR_SHAPE:
            return "invalid shape (negative or too large size, K not a positive multiple of 16 up to 65536, or ld "
                   "too small)";
        case PDQ_ERR_DTYPE: return "dtype not accepted by this entry point";
        case PDQ_ERR_ALIGN: return "pointer or row pitch not 16-byte aligned";
        case PDQ_ERR_UNSUPPORTED: return "argument value out of range";
        case PDQ_ERR_WORKSPACE: return "workspace missing or too small";
        case PDQ_ERR_HIP: return "HIP launch error";
        default: return "unknown status";  // any other value, the range sentinels included
    }
}

size_t pdq_weight_bytes(int64_t N, int64_t K) {
    if (N < 0 || K < 0) return 0;
    return (size_t)((N + kWGroup - 1) / kWGroup) * (size_t)((K + kWTileK - 1) / kWTileK) * kWBlock;
}

size_t pdq_act_bytes(int64_t M, int64_t K) { return pdq_weight_bytes(M, K); }

int pdq_gemm_kernel(int64_t M, int64_t N) {
    if (M < 1 || N < 1) return -1;
    return skinny_gemm(M, N) ? PDQ_GEMM_SKINNY : PDQ_GEMM_TILED;
}

int pdq_skinny_channels(int64_t M, int64_t N) {
    if (M < 1 || N < 1 || M > kMaxRows || N > kMaxRows) return -1;
    return 16 * decode_groups(M, N);
}

pdq_status pdq_pack_int8(const int8_t* src, int64_t rows, int64_t K, int64_t ld, int8_t* packed, void* stream) {
    PDQ_TRY(check_operand(src, 1, rows, K, ld));
    if (rows > 0 && !packed) return PDQ_ERR_NULL;
    if (!aligned(packed, 16)) return PDQ_ERR_ALIGN;
    if (rows == 0) return PDQ_OK;
    launch_pack_int8(src, rows, K, ld, packed, static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_unpack_int8(const int8_t* packed, int64_t rows, int64_t K, int8_t* dst, int64_t ld, void* stream) {
    PDQ_TRY(check_operand(dst, 1, rows, K, ld));
    if (rows > 0 && !packed) return PDQ_ERR_NULL;
    if (!aligned(packed, 16)) return PDQ_ERR_ALIGN;
    if (rows == 0) return PDQ_OK;
    launch_unpack_int8(packed, rows, K, dst, ld, static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_quantize_weight(const void* w, pdq_dtype w_dt, int64_t N, int64_t K, int64_t ldw,
                               int8_t* wq, float* w_scale, int32_t* w_colsum, void* stream) {
    if (!dtype_ok(w_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(w, elem_bytes(w_dt), N, K, ldw));
    if (N > 0 && ((K > 0 && !wq) || !w_scale)) return PDQ_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(w_scale, 4) || !aligned(w_colsum, 4)) return PDQ_ERR_ALIGN;
    if (N == 0) return PDQ_OK;
    launch_quant_rows(w, w_dt, N, K, ldw, wq, w_scale, w_colsum, nullptr, static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_calibrate_static(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                float* minmax, float* a_scale, int32_t* a_zp, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    if (!minmax) return PDQ_ERR_NULL;
    if ((a_scale == nullptr) != (a_zp == nullptr)) return PDQ_ERR_NULL;
    if (!aligned(minmax, 4) || !aligned(a_scale, 4) || !aligned(a_zp, 4)) return PDQ_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    launch_minmax(x, x_dt, M, K, ldx, minmax, st);
    if (a_scale) launch_minmax_finalize(minmax, a_scale, a_zp, st);
    return launched();
}

pdq_status pdq_quantize_per_token(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                  int8_t* xq, float* x_scale, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    if (M > 0 && ((K > 0 && !xq) || !x_scale)) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(x_scale, 4)) return PDQ_ERR_ALIGN;
    if (M == 0) return PDQ_OK;
    launch_quant_rows(x, x_dt, M, K, ldx, xq, x_scale, nullptr, nullptr, static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_gemm_per_token(const int8_t* xq, const float* x_scale, int64_t M, int64_t K,
                              const int8_t* wq, const float* w_scale, const float* bias, int64_t N,
                              uint16_t* y, int64_t ldy, int32_t* acc_out, void* stream) {
    PDQ_TRY(check_operand(xq, 1, M, K, K));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (N > 0 && !w_scale) return PDQ_ERR_NULL;
    if (M > 0 && !x_scale) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(bias, 4) || !aligned(y, 2) ||
        !aligned(acc_out, 4))
        return PDQ_ERR_ALIGN;
    if (M == 0 || N == 0) return PDQ_OK;
    if (skinny_gemm(M, N)) {
        DecodeArgs d{};
        d.xq = xq;
        d.wq = wq;
        d.M = (int)M;
        d.N = (int)N;
        d.K = (int)K;
        d.sa = x_scale;
        d.sw = w_scale;
        d.bias = bias;
        d.y = y;
        d.ldy = ldy;
        d.acc_out = acc_out;
        launch_decode_gemv(d, static_cast<hipStream_t>(stream));
        return launched();
    }
    GemmArgs g{};
    g.A = xq;
    g.B = wq;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.sa = x_scale;
    g.sb = w_scale;
    g.bias = bias;
    g.y = y;
    g.ldy = ldy;
    g.acc_out = acc_out;
    launch_gemm_i8(g, PDQ_BF16, false, static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_linear_prefill(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                              const int8_t* wq, const float* w_scale, const float* bias, int64_t N,
                              int8_t* xq, float* x_scale, uint16_t* y, int64_t ldy,
                              int32_t* acc_out, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (N > 0 && !w_scale) return PDQ_ERR_NULL;
    if (M > 0 && ((K > 0 && !xq) || !x_scale)) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(bias, 4) ||
        !aligned(y, 2) || !aligned(acc_out, 4))
        return PDQ_ERR_ALIGN;
    PDQ_TRY(pdq_quantize_per_token(x, x_dt, M, K, ldx, xq, x_scale, stream));
    return pdq_gemm_per_token(xq, x_scale, M, K, wq, w_scale, bias, N, y, ldy, acc_out, stream);
}

pdq_status pdq_silu_mul_quantize_per_token(const void* gate, const void* up, pdq_dtype dt, int64_t M,
                                           int64_t K, int64_t ldg, int64_t ldu, int8_t* xq,
                                           float* x_scale, uint16_t* h, int64_t ldh, void* stream) {
    if (dt != PDQ_BF16 && dt != PDQ_F16) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(gate, 2, M, K, ldg));
    PDQ_TRY(check_operand(up, 2, M, K, ldu));
    if (h) PDQ_TRY(check_operand(h, 2, M, K, ldh));
    if (M > 0 && ((K > 0 && !xq) || !x_scale)) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(x_scale, 4)) return PDQ_ERR_ALIGN;
    if (M == 0) return PDQ_OK;
    launch_silu_mul_quant(gate, ldg, up, ldu, dt, M, K, xq, x_scale, h, ldh, static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_linear_prefill_silu_mul(const void* gate, const void* up, pdq_dtype dt, int64_t M, int64_t K,
                                       int64_t ldg, int64_t ldu, const int8_t* wq, const float* w_scale,
                                       const float* bias, int64_t N, int8_t* xq, float* x_scale,
                                       uint16_t* y, int64_t ldy, int32_t* acc_out, void* stream) {
    if (dt != PDQ_BF16 && dt != PDQ_F16) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(gate, 2, M, K, ldg));
    PDQ_TRY(check_operand(up, 2, M, K, ldu));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (N > 0 && !w_scale) return PDQ_ERR_NULL;
    if (M > 0 && ((K > 0 && !xq) || !x_scale)) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(bias, 4) ||
        !aligned(y, 2) || !aligned(acc_out, 4))
        return PDQ_ERR_ALIGN;
    PDQ_TRY(pdq_silu_mul_quantize_per_token(gate, up, dt, M, K, ldg, ldu, xq, x_scale, nullptr, 0, stream));
    return pdq_gemm_per_token(xq, x_scale, M, K, wq, w_scale, bias, N, y, ldy, acc_out, stream);
}

pdq_status pdq_quantize_per_token_asym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                       int8_t* xq, float* x_scale, int32_t* x_zp, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    if (M > 0 && ((K > 0 && !xq) || !x_scale || !x_zp)) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(x_zp, 4)) return PDQ_ERR_ALIGN;
    if (M == 0) return PDQ_OK;
    launch_quant_rows_asym(x, x_dt, M, K, ldx, xq, x_scale, x_zp, static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_gemm_per_token_asym(const int8_t* xq, const float* x_scale, const int32_t* x_zp, int64_t M,
                                   int64_t K, const int8_t* wq, const float* w_scale,
                                   const int32_t* w_colsum, const float* bias, int64_t N, uint16_t* y,
                                   int64_t ldy, int32_t* acc_out, void* stream) {
    PDQ_TRY(check_operand(xq, 1, M, K, K));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (N > 0 && (!w_scale || !w_colsum)) return PDQ_ERR_NULL;
    if (M > 0 && (!x_scale || !x_zp)) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(x_scale, 4) || !aligned(x_zp, 4) || !aligned(w_scale, 4) || !aligned(w_colsum, 4) ||
        !aligned(bias, 4) || !aligned(y, 2) || !aligned(acc_out, 4))
        return PDQ_ERR_ALIGN;
    if (M == 0 || N == 0) return PDQ_OK;
    if (skinny_gemm(M, N)) {
        DecodeArgs d{};
        d.xq = xq;
        d.wq = wq;
        d.M = (int)M;
        d.N = (int)N;
        d.K = (int)K;
        d.sa = x_scale;
        d.za = x_zp;
        d.sw = w_scale;
        d.colsum = w_colsum;
        d.bias = bias;
        d.y = y;
        d.ldy = ldy;
        d.acc_out = acc_out;
        launch_decode_gemv(d, static_cast<hipStream_t>(stream));
        return launched();
    }
    GemmArgs g{};
    g.A = xq;
    g.B = wq;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.sa = x_scale;
    g.za = x_zp;
    g.colsum = w_colsum;
    g.sb = w_scale;
    g.bias = bias;
    g.y = y;
    g.ldy = ldy;
    g.acc_out = acc_out;
    launch_gemm_i8(g, PDQ_BF16, false, static_cast<hipStream_t>(stream), 2);
    return launched();
}

pdq_status pdq_linear_prefill_asym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                   const int8_t* wq, const float* w_scale, const int32_t* w_colsum,
                                   const float* bias, int64_t N, int8_t* xq, float* x_scale, int32_t* x_zp,
                                   uint16_t* y, int64_t ldy, int32_t* acc_out, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (N > 0 && (!w_scale || !w_colsum)) return PDQ_ERR_NULL;
    if (M > 0 && ((K > 0 && !xq) || !x_scale || !x_zp)) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(x_zp, 4) || !aligned(w_scale, 4) ||
        !aligned(w_colsum, 4) || !aligned(bias, 4) || !aligned(y, 2) || !aligned(acc_out, 4))
        return PDQ_ERR_ALIGN;
    PDQ_TRY(pdq_quantize_per_token_asym(x, x_dt, M, K, ldx, xq, x_scale, x_zp, stream));
    return pdq_gemm_per_token_asym(xq, x_scale, x_zp, M, K, wq, w_scale, w_colsum, bias, N, y, ldy, acc_out,
                                   stream);
}

pdq_status pdq_quantize_static(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                               float a_scale, int32_t a_zp, int8_t* xq, uint32_t* sat_count,
                               void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    if (!(a_scale > 0.0f) || !isfinite(a_scale) || a_zp < -128 || a_zp > 127)
        return PDQ_ERR_UNSUPPORTED;
    if (M > 0 && K > 0 && !xq) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(sat_count, 4)) return PDQ_ERR_ALIGN;
    if (M == 0) return PDQ_OK;
    launch_quant_static(x, x_dt, M, K, ldx, a_scale, a_zp, xq, sat_count,
                        static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_gemm_static(const int8_t* xq, int64_t M, int64_t K, float a_scale, int32_t a_zp,
                           const int8_t* wq, const float* w_scale, const int32_t* w_colsum,
                           const float* bias, int64_t N, uint16_t* y, int64_t ldy, int32_t* acc_out,
                           void* stream) {
    PDQ_TRY(check_operand(xq, 1, M, K, K));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (!(a_scale > 0.0f) || !isfinite(a_scale) || a_zp < -128 || a_zp > 127)
        return PDQ_ERR_UNSUPPORTED;
    if (N > 0 && (!w_scale || (a_zp != 0 && !w_colsum))) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(w_scale, 4) || !aligned(w_colsum, 4) || !aligned(bias, 4) || !aligned(y, 2) ||
        !aligned(acc_out, 4))
        return PDQ_ERR_ALIGN;
    if (M == 0 || N == 0) return PDQ_OK;
    if (!skinny_gemm(M, N)) {
        GemmArgs g{};
        g.A = xq;
        g.B = wq;
        g.M = (int)M;
        g.N = (int)N;
        g.K = (int)K;
        g.s = a_scale;
        g.z = a_zp;
        g.colsum = w_colsum;
        g.sb = w_scale;
        g.bias = bias;
        g.y = y;
        g.ldy = ldy;
        g.acc_out = acc_out;
        launch_gemm_i8(g, PDQ_BF16, false, static_cast<hipStream_t>(stream), a_zp != 0 ? 1 : 0);
        return launched();
    }
    DecodeArgs d{};
    d.xq = xq;
    d.wq = wq;
    d.M = (int)M;
    d.N = (int)N;
    d.K = (int)K;
    d.s = a_scale;
    d.z = a_zp;
    d.sw = w_scale;
    d.colsum = a_zp != 0 ? w_colsum : nullptr;
    d.bias = bias;
    d.y = y;
    d.ldy = ldy;
    d.acc_out = acc_out;
    launch_decode_gemv(d, static_cast<hipStream_t>(stream));
    return launched();
}

pdq_status pdq_calibrate_static_sym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                    float* minmax, float* a_scale, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    if (!minmax) return PDQ_ERR_NULL;
    if (!aligned(minmax, 4) || !aligned(a_scale, 4)) return PDQ_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    launch_minmax(x, x_dt, M, K, ldx, minmax, st);
    if (a_scale) launch_absmax_finalize(minmax, a_scale, st);
    return launched();
}

pdq_status pdq_quantize_static_sym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                   float a_scale, int8_t* xq, uint32_t* sat_count, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    if (!(a_scale > 0.0f) || !isfinite(a_scale)) return PDQ_ERR_UNSUPPORTED;
    if (M > 0 && K > 0 && !xq) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(sat_count, 4)) return PDQ_ERR_ALIGN;
    if (M == 0) return PDQ_OK;
    launch_quant_static(x, x_dt, M, K, ldx, a_scale, 0, xq, sat_count, static_cast<hipStream_t>(stream),
                        true);
    return launched();
}

pdq_status pdq_linear_static_sym(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                 float a_scale, const int8_t* wq, const float* w_scale, const float* bias,
                                 int64_t N, int8_t* xq, uint16_t* y, int64_t ldy, int32_t* acc_out,
                                 uint32_t* sat_count, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (!(a_scale > 0.0f) || !isfinite(a_scale)) return PDQ_ERR_UNSUPPORTED;
    if (N > 0 && !w_scale) return PDQ_ERR_NULL;
    if (M > 0 && K > 0 && !xq) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(w_scale, 4) || !aligned(bias, 4) || !aligned(y, 2) ||
        !aligned(acc_out, 4) || !aligned(sat_count, 4))
        return PDQ_ERR_ALIGN;
    if (N > 0 && decode_fusable(M, K)) {
        DecodeArgs d{};
        d.wq = wq;
        d.M = (int)M;
        d.N = (int)N;
        d.K = (int)K;
        d.s = a_scale;
        d.z = 0;
        d.narrow = 1;
        d.sw = w_scale;
        d.bias = bias;
        d.y = y;
        d.ldy = ldy;
        d.acc_out = acc_out;
        d.x = x;
        d.x_dt = x_dt;
        d.ldx = ldx;
        d.xq_out = xq;
        d.sat = sat_count;
        launch_decode_fused(d, static_cast<hipStream_t>(stream));
        return launched();
    }
    PDQ_TRY(pdq_quantize_static_sym(x, x_dt, M, K, ldx, a_scale, xq, sat_count, stream));
    return pdq_gemm_static(xq, M, K, a_scale, 0, wq, w_scale, nullptr, bias, N, y, ldy, acc_out, stream);
}

pdq_status pdq_calibrate_zeropoint(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                   float* minmax, float* a_scale, int32_t* a_zp, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    if (!minmax) return PDQ_ERR_NULL;
    if ((a_scale == nullptr) != (a_zp == nullptr)) return PDQ_ERR_NULL;
    if (!aligned(minmax, 4) || !aligned(a_scale, 4) || !aligned(a_zp, 4)) return PDQ_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    launch_minmax(x, x_dt, M, K, ldx, minmax, st);
    if (a_scale) launch_zeropoint_finalize(minmax, a_scale, a_zp, st);
    return launched();
}

pdq_status pdq_quantize_zeropoint(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                  float a_scale, int32_t a_zp, int8_t* xq, uint32_t* sat_count, void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    if (!(a_scale > 0.0f) || !isfinite(a_scale) || a_zp < -127 || a_zp > 127) return PDQ_ERR_UNSUPPORTED;
    if (M > 0 && K > 0 && !xq) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(sat_count, 4)) return PDQ_ERR_ALIGN;
    if (M == 0) return PDQ_OK;
    launch_quant_static(x, x_dt, M, K, ldx, a_scale, a_zp, xq, sat_count, static_cast<hipStream_t>(stream),
                        true);
    return launched();
}

pdq_status pdq_linear_zeropoint(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                                float a_scale, int32_t a_zp, const int8_t* wq, const float* w_scale,
                                const int32_t* w_colsum, const float* bias, int64_t N, int8_t* xq,
                                uint16_t* y, int64_t ldy, int32_t* acc_out, uint32_t* sat_count,
                                void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (!(a_scale > 0.0f) || !isfinite(a_scale) || a_zp < -127 || a_zp > 127) return PDQ_ERR_UNSUPPORTED;
    if (N > 0 && (!w_scale || !w_colsum)) return PDQ_ERR_NULL;
    if (M > 0 && K > 0 && !xq) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(w_scale, 4) || !aligned(w_colsum, 4) || !aligned(bias, 4) ||
        !aligned(y, 2) || !aligned(acc_out, 4) || !aligned(sat_count, 4))
        return PDQ_ERR_ALIGN;
    if (N > 0 && decode_fusable(M, K)) {
        DecodeArgs d{};
        d.wq = wq;
        d.M = (int)M;
        d.N = (int)N;
        d.K = (int)K;
        d.s = a_scale;
        d.z = a_zp;
        d.narrow = 1;
        d.sw = w_scale;
        d.colsum = w_colsum;
        d.bias = bias;
        d.y = y;
        d.ldy = ldy;
        d.acc_out = acc_out;
        d.x = x;
        d.x_dt = x_dt;
        d.ldx = ldx;
        d.xq_out = xq;
        d.sat = sat_count;
        launch_decode_fused(d, static_cast<hipStream_t>(stream));
        return launched();
    }
    PDQ_TRY(pdq_quantize_zeropoint(x, x_dt, M, K, ldx, a_scale, a_zp, xq, sat_count, stream));
    return pdq_gemm_static(xq, M, K, a_scale, a_zp, wq, w_scale, w_colsum, bias, N, y, ldy, acc_out, stream);
}

pdq_status pdq_linear_decode(const void* x, pdq_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                             float a_scale, int32_t a_zp, const int8_t* wq, const float* w_scale,
                             const int32_t* w_colsum, const float* bias, int64_t N, int8_t* xq,
                             uint16_t* y, int64_t ldy, int32_t* acc_out, uint32_t* sat_count,
                             void* stream) {
    if (!dtype_ok(x_dt)) return PDQ_ERR_DTYPE;
    PDQ_TRY(check_operand(x, elem_bytes(x_dt), M, K, ldx));
    PDQ_TRY(check_operand(wq, 1, N, K, K));
    if (N < 0 || N > kMaxRows || M * N > kMaxOutputs || ldy < N) return PDQ_ERR_SHAPE;
    if (!(a_scale > 0.0f) || !isfinite(a_scale) || a_zp < -128 || a_zp > 127)
        return PDQ_ERR_UNSUPPORTED;
    if (N > 0 && (!w_scale || !w_colsum)) return PDQ_ERR_NULL;
    if (M > 0 && K > 0 && !xq) return PDQ_ERR_NULL;
    if (M > 0 && N > 0 && !y) return PDQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(w_scale, 4) || !aligned(w_colsum, 4) || !aligned(bias, 4) ||
        !aligned(y, 2) || !aligned(acc_out, 4) || !aligned(sat_count, 4))
        return PDQ_ERR_ALIGN;
    if (N > 0 && decode_fusable(M, K)) {
        // one launch: the GEMM quantizes the activations itself (and writes xq)
        if (!y) return PDQ_ERR_NULL;
        DecodeArgs d{};
        d.wq = wq;
        d.M = (int)M;
        d.N = (int)N;
        d.K = (int)K;
        d.s = a_scale;
        d.z = a_zp;
        d.sw = w_scale;
        d.colsum = w_colsum;
        d.bias = bias;
        d.y = y;
        d.ldy = ldy;
        d.acc_out = acc_out;
        d.x = x;
        d.x_dt = x_dt;
        d.ldx = ldx;
        d.xq_out = xq;
        d.sat = sat_count;
        launch_decode_fused(d, static_cast<hipStream_t>(stream));
        return launched();
    }
    PDQ_TRY(pdq_quantize_static(x, x_dt, M, K, ldx, a_scale, a_zp, xq, sat_count, stream));
    return pdq_gemm_static(xq, M, K, a_scale, a_zp, wq, w_scale, w_colsum, bias, N, y, ldy, acc_out,
                           stream);
}

size_t pdq_linear_int8_outlier_workspace(int64_t M, int64_t N, int64_t K, int64_t max_outliers) {
    if (M < 0 || N < 0 || K < 0 || max_outliers < 0) return 0;
    const int64_t P = side_pitch(max_outliers);
    const size_t pitch = (size_t)outlier_partial_pitch(K);
    return align256((size_t)outlier_row_blocks(M) * pitch) + align256(pitch) +
           align256((size_t)(M * P * 2)) + align256((size_t)(N * P * 2));
}

pdq_status pdq_linear_int8_outlier(const void* x, pdq_dtype dt, int64_t M, int64_t K, int64_t ldx,
                                   float threshold, const int8_t* wq, const float* w_scale,
                                   const void* w16, int64_t ldw, const float* bias, int64_t N,
                                   void* y, int64_t ldy, int8_t* xq, float* x_scale,
                                   int32_t* outlier_idx, int32_t* n_outlier, int64_t max_outliers,
                                   void* workspace, size_t workspace_bytes, int32_t* acc_out,
                                   void* stream) {
    PDQ_TRY(check_int8_outlier(x, dt, M, K, ldx, threshold, wq, w_scale, w16, ldw, bias, N, y, ldy, xq,
                               x_scale, outlier_idx, n_outlier, max_outliers, acc_out));
    const size_t need = pdq_linear_int8_outlier_workspace(M, N, K, max_outliers);
    if (!workspace || workspace_bytes < need) return PDQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PDQ_ERR_ALIGN;
    run_int8_outlier(x, dt, M, K, ldx, threshold, wq, w_scale, w16, ldw, bias, N, y, ldy, xq, x_scale,
                     outlier_idx, n_outlier, max_outliers, static_cast<char*>(workspace), acc_out,
                     static_cast<hipStream_t>(stream));
    return launched();
}

size_t pdq_noalloc_scratch_bytes(void) { return kScratchBytes; }

pdq_status pdq_linear_int8_outlier_noalloc(const void* x, pdq_dtype dt, int64_t M, int64_t K, int64_t ldx,
                                           float threshold, const int8_t* wq, const float* w_scale,
                                           const void* w16, int64_t ldw, const float* bias, int64_t N,
                                           void* y, int64_t ldy, int8_t* xq, float* x_scale,
                                           int32_t* outlier_idx, int32_t* n_outlier, int64_t max_outliers,
                                           int32_t* acc_out, void* stream) {
    PDQ_TRY(check_int8_outlier(x, dt, M, K, ldx, threshold, wq, w_scale, w16, ldw, bias, N, y, ldy, xq,
                               x_scale, outlier_idx, n_outlier, max_outliers, acc_out));
    if (pdq_linear_int8_outlier_workspace(M, N, K, max_outliers) > kScratchBytes) return PDQ_ERR_WORKSPACE;
    // the argument checks above make no HIP call; from here on the device's
    // own copy of the scratch array is looked up (once per device)
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = nullptr;
    PDQ_TRY(scratch_for_stream(st, &ws));
    run_int8_outlier(x, dt, M, K, ldx, threshold, wq, w_scale, w16, ldw, bias, N, y, ldy, xq, x_scale,
                     outlier_idx, n_outlier, max_outliers, ws, acc_out, st);
    return launched();
}

}  // extern "C"
