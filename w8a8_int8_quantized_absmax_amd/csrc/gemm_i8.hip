// INT8 x INT8 -> INT32 GEMM with the fused dequantizing epilogue (gfx950).
//
// acc[m, n] = sum_k A[m, k] * B[n, k]   (LLM.int8() notes, part 2 step (3):
// INT8 products accumulated in INT32), then per element
//   y = (S_a[m] * S_b[n]) * (float)acc  [+ side[m, n]] [+ bias[n]]
// (part 2 step (4) and the vector-wise outer product of row and column
// scales; PDMIX terminology entry section 2.3 for S * q), each operation
// rounded to binary32, written as bf16 or f16.  With the side product, side
// is the 16-bit GEMM over the outlier columns (part 2, "16-bit
// decomposition" and "mixed-precision decomposition"), run on the 16-bit
// MFMA into a separate binary32 accumulator per 32x32 sub-tile.
//
// Tiling: 256x256 output tile per 256-thread workgroup (4 wavefronts in a
// 2x2 arrangement, 128x128 each = 4x4 v_mfma_i32_32x32x32_i8 tiles with
// their INT32 accumulators in registers), K staged through LDS 128 bytes at
// a time.  A and B are both K-contiguous, so a K tile of 256 rows is 256
// lines of 128 bytes; the 16-byte chunk c of row r sits at chunk c ^ (r & 7)
// so that the 128-bit fragment reads of 8 consecutive rows hit 8 distinct
// chunk positions.  Tiles move global -> LDS directly (global_load_lds, no
// register staging) into two LDS buffers: tile k+1 is in flight while tile k
// feeds the MFMAs.

#include "pdq_device.h"
#include "pdq_kernels.h"

#include <type_traits>

namespace pdq {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;

__device__ __forceinline__ int swz(int r, int kc) { return r * BK + ((kc ^ (r & 7)) << 4); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int OUT, bool SIDE>
__global__ __launch_bounds__(256) void k_gemm_i8(GemmArgs a) {
    // Two K-tile buffers, each A[256][128] followed by B[256][128].
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2][(BM + BN) * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = a.M, N = a.N, K = a.K;
    const int tiles_n = (N + BN - 1) / BN;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nkt = (K + BK - 1) / BK;

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};

    // Global -> LDS without registers: one global_load_lds_dwordx4 moves 64
    // lanes x 16 bytes into 1 KB of LDS (8 rows of the tile), lane l landing in
    // row l/8, chunk position l%8.  The lane therefore fetches logical chunk
    // (l%8) ^ (row & 7) so that the LDS image is the swizzled layout.  Wave w
    // fills rows [64w, 64w + 64) of both the A and the B tile.  Rows past M
    // (N) are clamped onto the last row: they only feed outputs that are never
    // stored.  Chunks past K are clamped onto the last chunk and zeroed in the
    // A fragments of the last K tile, which zeroes their products.
    const int lr = lane >> 3;
    const int kc_ld = (lane & 7) ^ lr;
    const int rbase = wave * 64 + lr;
    auto issue = [&](int kt, int buf) {
        const int gk = min(kt * BK + kc_ld * 16, K - 16);
        uint8_t* la = &smem[buf][wave * 64 * BK];
        uint8_t* lb = &smem[buf][BM * BK + wave * 64 * BK];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int gm = min(m0 + rbase + 8 * i, M - 1);
            __builtin_amdgcn_global_load_lds(a.A + (size_t)gm * K + gk, (lds_ptr_t)(la + i * 8 * BK),
                                             16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int gn = min(n0 + rbase + 8 * i, N - 1);
            __builtin_amdgcn_global_load_lds(a.B + (size_t)gn * K + gk, (lds_ptr_t)(lb + i * 8 * BK),
                                             16, 0, 0);
        }
    };
    // Fragments of one 32-wide K step: lane l reads row (l%32) of each 32-row
    // block, chunk 2*s + l/32 (16 bytes = 16 K values).
    auto read_frags = [&](const uint8_t* sbase, int s, v4i (&fa)[4], v4i (&fb)[4]) {
        const int kc = 2 * s + (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fa[i] = *reinterpret_cast<const v4i*>(sbase + swz(wm * 128 + i * 32 + (lane & 31), kc));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fb[j] = *reinterpret_cast<const v4i*>(sbase + BM * BK +
                                                  swz(wn * 128 + j * 32 + (lane & 31), kc));
    };

    // One K tile from LDS buffer `sb`: 4 steps of 32, each 16 MFMAs, with the
    // next step's fragments read while the current step's MFMAs run.  MASK
    // (last tile only, when K % 128 != 0) zeroes A past K.
    auto compute = [&](const uint8_t* sb, int kvalid, auto mask) {
        v4i fa[2][4], fb[2][4];
        read_frags(sb, 0, fa[0], fb[0]);
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            const int cur = s & 1;
            if (s + 1 < BK / 32) read_frags(sb, s + 1, fa[cur ^ 1], fb[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this step's MFMAs
            if constexpr (decltype(mask)::value) {
                const bool dead = (2 * s + (lane >> 5)) * 16 >= kvalid;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (dead) fa[cur][i] = v4i{};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[cur][i], fb[cur][j],
                                                                      acc[i][j], 0, 0, 0);
        }
    };

    if (nkt > 0) issue(0, 0);
    for (int kt = 0; kt + 1 < nkt; ++kt) {
        const int buf = kt & 1;
        issue(kt + 1, buf ^ 1);
        // this wave's 16 loads of tile kt have landed; then all waves'.
        // (__syncthreads() would also wait for tile kt+1's loads.)
        asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
        compute(smem[buf], BK, std::false_type{});
        // every wave is done reading `buf` before the next iteration refills it
        asm volatile("s_barrier" ::: "memory");
    }
    if (nkt > 0) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        const int kvalid = K - (nkt - 1) * BK;
        if (kvalid >= BK)
            compute(smem[(nkt - 1) & 1], kvalid, std::false_type{});
        else
            compute(smem[(nkt - 1) & 1], kvalid, std::true_type{});
    }

    // Epilogue.  32x32 accumulator layout: lane l, register r holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the sub-tile.  The 16-bit
    // results go to LDS (the 256x256 tile is exactly the 128 KB of the two
    // K buffers) and leave in 16-byte row chunks.
    bool poison = false;
    int side_steps = 0;
    if constexpr (SIDE) {
        const int cnt = *a.count;
        poison = cnt > a.max_count;
        side_steps = poison ? 0 : (cnt + 15) / 16;
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    uint16_t* sY = reinterpret_cast<uint16_t*>(&smem[0][0]);
    const int ml0 = wm * 128 + 4 * (lane >> 5), nl0 = wn * 128 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sam[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = m0 + ml0 + i * 32 + 8 * (r >> 2) + (r & 3);
            sam[r] = m < M ? a.sa[m] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int nl = nl0 + j * 32;
            const int n = n0 + nl;
            const bool nvalid = n < N;
            const float sbn = nvalid ? a.sb[n] : 0.0f;
            const float bn = (a.bias && nvalid) ? a.bias[n] : 0.0f;
            v16f side = v16f{};
            if constexpr (SIDE) {
                const int xm = m0 + wm * 128 + i * 32 + (lane & 31);
                for (int ks = 0; ks < side_steps; ++ks) {
                    const int koff = ks * 16 + 8 * (lane >> 5);
                    uint4 xv = make_uint4(0, 0, 0, 0), wv = make_uint4(0, 0, 0, 0);
                    if (xm < M) xv = *reinterpret_cast<const uint4*>(a.xo + (size_t)xm * a.P + koff);
                    if (nvalid) wv = *reinterpret_cast<const uint4*>(a.wo + (size_t)n * a.P + koff);
                    if constexpr (OUT == kF16)
                        side = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, xv),
                                                                      __builtin_bit_cast(v8h, wv),
                                                                      side, 0, 0, 0);
                    else
                        side = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xv),
                                                                       __builtin_bit_cast(v8bf, wv),
                                                                       side, 0, 0, 0);
                }
            }
            if (a.acc_out && nvalid) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + ml0 + i * 32 + 8 * (r >> 2) + (r & 3);
                    if (m < M) a.acc_out[(size_t)m * N + n] = acc[i][j][r];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = ml0 + i * 32 + 8 * (r >> 2) + (r & 3);
                const float t = __fmul_rn(sam[r], sbn);
                float y = __fmul_rn(t, (float)acc[i][j][r]);
                if constexpr (SIDE) y = __fadd_rn(y, side[r]);
                if (a.bias) y = __fadd_rn(y, bn);
                if (poison) y = __builtin_nanf("");
                sY[ml * BN + nl] = OUT == kF16 ? f32_to_f16(y) : f32_to_bf16(y);
            }
        }
    }
    __syncthreads();
    // 256 rows x 32 chunks of 8 outputs; consecutive threads take consecutive
    // chunks of a row.
    uint16_t* y = static_cast<uint16_t*>(a.y);
    const bool vec = ((reinterpret_cast<uintptr_t>(y) & 15) == 0) && (a.ldy % 8 == 0);
    for (int c = tid; c < BM * (BN / 8); c += 256) {
        const int ml = c >> 5, nl = (c & 31) * 8;
        const int m = m0 + ml, n = n0 + nl;
        if (m >= M || n >= N) continue;
        uint16_t* dst = y + (size_t)m * a.ldy + n;
        const uint16_t* src = sY + ml * BN + nl;
        if (vec && n + 8 <= N) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
            for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = src[e];
        }
    }
}

}  // namespace

void launch_gemm_i8(const GemmArgs& a, int out_dt, bool side, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return;
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const dim3 grid(tiles), block(256);
    if (!side)
        hipLaunchKernelGGL((k_gemm_i8<kBF16, false>), grid, block, 0, st, a);
    else if (out_dt == kF16)
        hipLaunchKernelGGL((k_gemm_i8<kF16, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((k_gemm_i8<kBF16, true>), grid, block, 0, st, a);
}

}  // namespace pdq
