// Outlier-column detection and gathers of the LLM.int8() decomposition (gfx950).
//
// LLM.int8() notes, part 2 "16-bit decomposition" step (1) and
// "mixed-precision decomposition" step 1: the hidden dimensions (columns of
// X) with a magnitude above the threshold are outliers; they and the matching
// weight columns go to a 16-bit GEMM, the rest to the INT8 path.
//
//  * k_outlier_partial one predicate byte per (row block, chunk of 8 columns):
//                     bit j set when some |x[m, 8c + j]| > threshold in the
//                     block.  Every byte is written, so nothing needs clearing
//                     first and no atomics are involved.
//  * k_outlier_index  ORs the row blocks into the final per-chunk mask, counts
//                     and lists the outlier columns in ascending order: one
//                     workgroup writes the mask, the index list and the count.
//
// Both gathers are fused into the regular-column quantizer (quant.hip): its
// row workgroups gather X_out from the rows they read anyway, and extra
// workgroups of the same launch gather W_out, so that the scattered reads of
// the W gather overlap the quantization.  X_out and W_out are packed and
// zero-padded to a multiple of 16 columns for the 16-bit MFMA in the GEMM
// epilogue.

#include "pdq_device.h"
#include "pdq_kernels.h"

namespace pdq {

namespace {

constexpr int kPartialGroups = 4;  // row groups per workgroup (64 chunks each)
constexpr int kPartialUnroll = 8;  // rows in flight per thread

// Block (256 threads) = 64 column chunks x 4 row groups.  Row block
// blockIdx.y covers rows [R y, min(M, R y + R)); each thread ORs the
// predicate of its 8 columns over every fourth row of it, eight loads in
// flight (rows past the block re-read its last row: the OR is unchanged),
// then the four row groups combine through LDS.
template <int DT>
__global__ __launch_bounds__(256) void k_outlier_partial(const void* __restrict__ x, int64_t ld_bytes,
                                                         int64_t M, int nch, int R, float thr,
                                                         uint8_t* __restrict__ partial,
                                                         int pitch) {
    __shared__ uint32_t s_hit[kPartialGroups][64];
    const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
    const int craw = blockIdx.x * 64 + cl;
    const int c = min(craw, nch - 1);
    const int64_t r0 = (int64_t)blockIdx.y * R;
    const int64_t rlast = min(M, r0 + R) - 1;
    const char* xb = static_cast<const char*>(x);
    uint32_t hit = 0;
    for (int64_t r = r0 + rg; r <= rlast; r += kPartialGroups * kPartialUnroll) {
        Raw8<DT> raw[kPartialUnroll];
#pragma unroll
        for (int u = 0; u < kPartialUnroll; ++u)
            raw[u] = load_raw8<DT>(xb + min(r + kPartialGroups * u, rlast) * ld_bytes, c);
#pragma unroll
        for (int u = 0; u < kPartialUnroll; ++u) {
            float v[8];
            widen8<DT>(raw[u], v);
#pragma unroll
            for (int j = 0; j < 8; ++j) hit |= (uint32_t)(fabsf(v[j]) > thr) << j;
        }
    }
    s_hit[rg][cl] = hit;
    __syncthreads();
    if (rg == 0 && craw < nch)
        partial[(int64_t)blockIdx.y * pitch + craw] =
            (uint8_t)(s_hit[0][cl] | s_hit[1][cl] | s_hit[2][cl] | s_hit[3][cl]);
}

constexpr int kIndexThreads = 256;
constexpr int kMaxRowBlocks = 32;
constexpr int kMaxMaskWords = (65536 / 8 + 3) / 4;  // K <= 65536

__device__ __forceinline__ int block_exclusive_scan(int v, int& total, int* s_wave) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d);
        if (lane >= d) incl += t;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kIndexThreads / 64; ++w) {
        before += w < wave ? s_wave[w] : 0;
        total += s_wave[w];
    }
    return before + incl - v;
}

// Thread t owns the mask words (4 chunks each) [t * wpt, t * wpt + wpt).
__global__ __launch_bounds__(kIndexThreads) void k_outlier_index(const uint8_t* __restrict__ partial, int nrb,
                                                                 int pitch, int nch, uint8_t* __restrict__ mask,
                                                                 int32_t* __restrict__ idx,
                                                                 int32_t* __restrict__ count, int max_out) {
    __shared__ uint32_t s_words[kMaxMaskWords];
    __shared__ int s_wave[kIndexThreads / 64];
    const int tid = threadIdx.x;
    const int nwords = (nch + 3) / 4;
    const int wpt = (nwords + kIndexThreads - 1) / kIndexThreads;
    const int w0 = tid * wpt;
    const int nw = max(0, min(wpt, nwords - w0));

    // pass 1: OR of the row blocks (32 loads in flight per word), count
    int mine = 0;
    for (int k = 0; k < nw; ++k) {
        const int w = w0 + k;
        uint32_t m = 0;
        if (nrb > 0) {
#pragma unroll
            for (int b = 0; b < kMaxRowBlocks; ++b)  // clamped: repeats OR the same bytes
                m |= reinterpret_cast<const uint32_t*>(partial + (int64_t)min(b, nrb - 1) * pitch)[w];
        }
        const int valid = min(4, nch - 4 * w);  // chunks of the last word past nch
        if (valid < 4) m &= (1u << (8 * valid)) - 1u;
        mine += __popc(m);
        s_words[w] = m;
        reinterpret_cast<uint32_t*>(mask)[w] = m;
    }
    int total;
    int run = block_exclusive_scan(mine, total, s_wave);

    // pass 2: ascending index list (the first max_out columns)
    for (int k = 0; k < nw; ++k) {
        const int w = w0 + k;
        const uint32_t m = s_words[w];
        const int valid = min(4, nch - 4 * w);
        for (int e = 0; e < valid; ++e) {
            const int c = 4 * w + e;
            uint32_t byte = (m >> (8 * e)) & 0xffu;
            while (byte) {
                const int j = __ffs(byte) - 1;
                byte &= byte - 1;
                if (run < max_out) idx[run] = 8 * c + j;
                ++run;
            }
        }
    }
    if (tid == 0) *count = total;
}

}  // namespace

int outlier_row_blocks(int64_t M) {
    if (M <= 0) return 0;
    const int64_t R = outlier_rows_per_block(M);
    return (int)((M + R - 1) / R);
}

int64_t outlier_rows_per_block(int64_t M) {
    const int64_t per = (M + kMaxRowBlocks - 1) / kMaxRowBlocks;
    const int64_t step = kPartialGroups * kPartialUnroll;
    return (per + step - 1) / step * step;
}

int outlier_partial_pitch(int64_t K) { return (int)((K / 8 + 15) / 16 * 16); }

void launch_outlier_partial(const void* x, int dt, int64_t M, int64_t K, int64_t ldx, float thr,
                            uint8_t* partial, hipStream_t st) {
    const int nch = (int)(K / 8);
    if (M <= 0 || nch <= 0) return;
    const int64_t R = outlier_rows_per_block(M);
    const dim3 grid((nch + 63) / 64, (unsigned)outlier_row_blocks(M));
    const int pitch = outlier_partial_pitch(K);
    if (dt == kF16)
        hipLaunchKernelGGL(k_outlier_partial<kF16>, grid, dim3(256), 0, st, x, ldx * 2, M, nch, (int)R,
                           thr, partial, pitch);
    else
        hipLaunchKernelGGL(k_outlier_partial<kBF16>, grid, dim3(256), 0, st, x, ldx * 2, M, nch, (int)R,
                           thr, partial, pitch);
}

void launch_outlier_index(const uint8_t* partial, int64_t M, int64_t K, uint8_t* mask, int32_t* idx,
                          int32_t* count, int64_t max_out, hipStream_t st) {
    hipLaunchKernelGGL(k_outlier_index, dim3(1), dim3(kIndexThreads), 0, st, partial, outlier_row_blocks(M),
                       outlier_partial_pitch(K), (int)(K / 8), mask, idx, count, (int)max_out);
}

}  // namespace pdq
