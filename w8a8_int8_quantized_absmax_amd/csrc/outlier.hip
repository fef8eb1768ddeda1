// Outlier-column detection and gathers of the LLM.int8() decomposition (gfx950).
//
// LLM.int8() notes, part 2 "16-bit decomposition" step (1) and
// "mixed-precision decomposition" step 1: the hidden dimensions (columns of
// X) with a magnitude above the threshold are outliers; they and the matching
// weight columns go to a 16-bit GEMM, the rest to the INT8 path.
//
//  * k_outlier_flags  flags[k] = 1 if some |x[m,k]| > threshold.  Only the
//                     predicate matters (not the column maximum), so each
//                     thread ORs it over its rows and touches memory with an
//                     atomic only where an outlier actually is.
//  * k_outlier_compact one workgroup: ascending index list + count by a
//                     block-wide prefix sum of the flags.
//  * k_gather_cols    X_out / W_out: the outlier columns of a 16-bit matrix,
//                     packed and zero-padded to a multiple of 16 for the 16-bit
//                     MFMA in the GEMM epilogue.

#include "pdq_device.h"
#include "pdq_kernels.h"

namespace pdq {

namespace {

__global__ __launch_bounds__(256) void k_fill_zero_u32(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int kFlagRows = 64;     // rows per workgroup
constexpr int kFlagChunks = 64;   // 8-column chunks per workgroup (512 columns)

// Block (256 threads) = 64 column chunks x 4 row groups; each thread ORs the
// predicate over 16 rows of its 8 columns.
template <int DT>
__global__ __launch_bounds__(256) void k_outlier_flags(const void* __restrict__ x, int64_t ld_bytes,
                                                       int64_t M, int nch, float thr,
                                                       uint32_t* __restrict__ flags) {
    const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
    const int c = blockIdx.x * kFlagChunks + cl;
    if (c >= nch) return;
    const int64_t r0 = (int64_t)blockIdx.y * kFlagRows + rg;
    uint32_t hit = 0;
    for (int i = 0; i < kFlagRows / 4; ++i) {
        const int64_t r = r0 + 4 * i;
        if (r >= M) break;
        float v[8];
        widen8<DT>(load_raw8<DT>(static_cast<const char*>(x) + r * ld_bytes, c), v);
#pragma unroll
        for (int j = 0; j < 8; ++j) hit |= (uint32_t)(fabsf(v[j]) > thr) << j;
    }
    if (hit) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if ((hit >> j) & 1u) atomicOr(flags + c * 8 + j, 1u);
    }
}

constexpr int kCompactThreads = 1024;

__global__ __launch_bounds__(1024) void k_outlier_compact(const uint32_t* __restrict__ flags, int K,
                                                          int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ count,
                                                          int max_out) {
    __shared__ int wave_tot[kCompactThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (K + kCompactThreads - 1) / kCompactThreads;
    const int k0 = tid * per;
    int local = 0;
    for (int k = k0; k < k0 + per && k < K; ++k) local += flags[k] != 0;
    // inclusive scan inside the wavefront
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kCompactThreads / 64; ++w) {
        if (w < wave) before += wave_tot[w];
        total += wave_tot[w];
    }
    int pos = before + incl - local;
    for (int k = k0; k < k0 + per && k < K; ++k) {
        if (flags[k] != 0) {
            if (pos < max_out) idx[pos] = k;
            ++pos;
        }
    }
    if (tid == 0) *count = total;
}

__global__ __launch_bounds__(256) void k_gather_cols(const uint16_t* __restrict__ src, int64_t rows,
                                                     int64_t ld, const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ count, int max_out,
                                                     uint16_t* __restrict__ dst, int P) {
    const int cnt = *count;
    if (cnt > max_out) return;
    const int used = (cnt + 15) / 16 * 16;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = t / P;
    const int j = (int)(t - r * P);
    if (r >= rows || j >= used) return;
    dst[r * P + j] = j < cnt ? src[r * ld + idx[j]] : (uint16_t)0;
}

}  // namespace

void launch_fill_zero_u32(uint32_t* p, int64_t n, hipStream_t st) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_fill_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
}

void launch_outlier_flags(const void* x, int dt, int64_t M, int64_t K, int64_t ldx, float thr,
                          uint32_t* flags, hipStream_t st) {
    const int nch = (int)(K / 8);
    if (M <= 0 || nch <= 0) return;
    const dim3 grid((nch + kFlagChunks - 1) / kFlagChunks, (unsigned)((M + kFlagRows - 1) / kFlagRows));
    if (dt == kF16)
        hipLaunchKernelGGL(k_outlier_flags<kF16>, grid, dim3(256), 0, st, x, ldx * 2, M, nch, thr,
                           flags);
    else
        hipLaunchKernelGGL(k_outlier_flags<kBF16>, grid, dim3(256), 0, st, x, ldx * 2, M, nch, thr,
                           flags);
}

void launch_outlier_compact(const uint32_t* flags, int64_t K, int32_t* idx, int32_t* count,
                            int64_t max_out, hipStream_t st) {
    hipLaunchKernelGGL(k_outlier_compact, dim3(1), dim3(kCompactThreads), 0, st, flags, (int)K, idx,
                       count, (int)max_out);
}

void launch_gather_cols(const void* src, int64_t rows, int64_t ld, const int32_t* idx,
                        const int32_t* count, int max_out, uint16_t* dst, int P, hipStream_t st) {
    if (rows <= 0 || P <= 0) return;
    const int64_t total = rows * P;
    hipLaunchKernelGGL(k_gather_cols, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(src), rows, ld, idx, count, max_out, dst, P);
}

}  // namespace pdq
