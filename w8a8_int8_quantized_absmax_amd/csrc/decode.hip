// Decode-phase skinny INT8 GEMM (M small) with the zero-point epilogue (gfx950).
//
// acc[m, n] = sum_k xq[m, k] * wq[n, k], then
//   y = (S * S_w[n]) * (float)(acc - Z * colsum[n]) [+ bias[n]]
// i.e. the PDMIX terminology entry's decode formula (section 2.3, static
// per-tensor S and Z) pushed through the zero-point expansion of the LLM.int8()
// notes (part 1 section 2) with a symmetric weight.
//
// The weight matrix is read exactly once and is the whole cost (the
// hardware-acceleration page's "data movement and memory bandwidth": decode is
// bandwidth-bound).  Each 256-thread workgroup owns 16 weight rows; its four
// wavefronts interleave over the K dimension in 64-byte steps (wavefront w
// takes steps w, w + 4, ...) and multiply with v_mfma_i32_16x16x64_i8, weight
// rows as the row operand, activation rows as the column operand.  The
// epilogue's per-column operands are loaded first, so their latency hides
// under the weight stream; the four partial accumulators are summed through
// LDS.
//
//  * k_decode_lds (M <= 16, while the rows fit in LDS): the 16 weight rows are
//    copied global -> LDS in contiguous 1 KB pieces, all issued up front, and
//    the MFMA fragments are read from LDS.  The activations arrive the same
//    way from xq, or -- the one-launch path, for M * K up to 8192 -- are
//    quantized by the workgroup itself (static quantization, the PDMIX
//    terminology entry's section 2.3 decode formula and section 2.4
//    saturation count): every workgroup quantizes the M rows into LDS while
//    its copies are in flight, and workgroup 0 writes xq and counts the
//    saturated values.
//  * k_decode_gemv (otherwise; up to 64 activation rows per workgroup row):
//    fragments loaded straight into registers, in batches of steps with two
//    batches in flight.  Every load is unconditional (rows and steps past the
//    end are clamped onto valid addresses; the fragments are masked where
//    they are used), so the compiler waits for exactly the batch it is about
//    to use.

#include "pdq_device.h"
#include "pdq_kernels.h"

#include <algorithm>

namespace pdq {

namespace {

constexpr int kRows = 16;   // weight rows per workgroup
constexpr int kMRows = 64;  // activation rows per workgroup of k_decode_gemv

// Epilogue operands of this lane's four outputs n = n0 + 4 (lane / 16) + r
// (16x16 accumulator layout: register r is row 4 (lane / 16) + r, the weight
// row n).  Loaded unconditionally: columns past N are clamped, a missing bias
// reads the scales and is ignored.
struct EpiOps {
    float sw[4], bias[4];
    int32_t cs[4];
};

__device__ __forceinline__ EpiOps load_epi(const DecodeArgs& a, int n0, int lane) {
    EpiOps e;
    const float* bp = a.bias ? a.bias : a.sw;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = min(n0 + 4 * (lane >> 4) + r, a.N - 1);
        e.sw[r] = a.sw[n];
        e.cs[r] = a.colsum[n];
        e.bias[r] = bp[n];
    }
    return e;
}

// Sum of the four wavefronts' partial accumulators and the epilogue for the
// 16 activation rows [mb, mb + 16) handled by register block `blk`.
template <int NMB>
__device__ __forceinline__ void reduce_and_store(const DecodeArgs& a, const v4i (&acc)[NMB],
                                                 const EpiOps& e, int n0, int mbase,
                                                 v4i (&red)[4][NMB][64]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) red[wave][mb][lane] = acc[mb];
    __syncthreads();
    if (wave >= NMB) return;
    const v4i tot = red[0][wave][lane] + red[1][wave][lane] + red[2][wave][lane] + red[3][wave][lane];
    const int m = mbase + wave * 16 + (lane & 15);
    if (m >= a.M) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = n0 + 4 * (lane >> 4) + r;
        if (n < a.N) {
            const int raw = tot[r];
            if (a.acc_out) a.acc_out[(size_t)m * a.N + n] = raw;
            const int corr = raw - a.z * e.cs[r];
            const float t = __fmul_rn(a.s, e.sw[r]);
            float y = __fmul_rn(t, (float)corr);
            if (a.bias) y = __fadd_rn(y, e.bias[r]);
            a.y[(size_t)m * a.ldy + n] = f32_to_bf16(y);
        }
    }
}

constexpr int kPiece = 1024;              // bytes of K per wavefront (K <= 4 kPiece)
constexpr int kPitch = kPiece + 16;       // LDS row pitch: rows 65 chunks apart, so the 16
                                          // lanes of a fragment read (16 rows, one chunk)
                                          // hit 16 distinct groups of four banks

// M <= 16, K <= 4096: wavefront w owns bytes [1024 w, 1024 w + 1024) of K.  It
// loads that piece of the 16 weight rows with one contiguous 1 KB load per row
// (a fragment-shaped load -- 16 rows x 64 bytes per instruction -- streams HBM
// markedly slower), turns it into MFMA fragments through its own LDS region
// (no barrier: one wavefront writes and reads it) and runs its 16 steps; the
// wavefronts meet only in the final reduction.  The activations are either
// fragment-shaped loads of xq (a few KB, from the cache), or -- FUSED, the
// one-launch path -- quantized by the wavefront from the 16-bit input into
// LDS (static quantization, the PDMIX terminology entry's section 2.3 decode
// formula and section 2.4 saturation count; workgroup 0 writes xq and counts
// the saturated values).
template <bool FUSED, int DT, int CPT>
__global__ __launch_bounds__(256) void k_decode_lds(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t wst[4][kRows][kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t xst[FUSED ? 4 : 1][FUSED ? 16 : 1][kPitch];
    __shared__ v4i red[4][1][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = a.M, K = a.K;
    const int n0 = blockIdx.x * kRows;
    const int kl = 16 * (lane >> 4);
    const int k0 = wave * kPiece;                        // this wavefront's piece
    const int kend = min(K, k0 + kPiece);                // <= k0 when the piece is empty

    // (1) epilogue operands, (2) activations, (3) the 16 weight rows
    const EpiOps e = load_epi(a, n0, lane);
    __builtin_amdgcn_sched_barrier(0);
    const int kc0 = min(k0, K - 16);  // a clamped, in-row start for an empty piece
    Raw8<DT> xr[FUSED ? CPT : 1];
    v4i xf[FUSED ? 1 : 16];
    // FUSED: chunk c = m * pch + j of this piece: row m, elements k0 + 8 j .. + 8
    const int pch = max((kend - k0) / 8, 1);
    if constexpr (FUSED) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = lane + 64 * i;
            const int m = min(c / pch, M - 1);
            const int kk = min(k0 + 8 * (c % pch), K - 8);
            xr[i] = load_raw8<DT>(static_cast<const char*>(a.x) + ((size_t)m * a.ldx + kk) * Elem<DT>::bytes, 0);
        }
    } else {
        const int8_t* xp = a.xq + (size_t)min(lane & 15, M - 1) * K;
#pragma unroll
        for (int t = 0; t < 16; ++t) xf[t] = *reinterpret_cast<const v4i*>(xp + min(kc0 + 64 * t + kl, K - 16));
    }
    __builtin_amdgcn_sched_barrier(0);
    v4i wr[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
        wr[r] = *reinterpret_cast<const v4i*>(a.wq + (size_t)min(n0 + r, a.N - 1) * K +
                                              min(kc0 + lane * 16, K - 16));
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (FUSED) {
        const float inv = 1.0f / a.s;
        int nsat = 0;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = lane + 64 * i;
            const int m = c / pch, j = c % pch;
            if (k0 < kend && m < M) {
                float v[8];
                widen8<DT>(xr[i], v);
                const uint2 code = static_codes8(v, a.s, inv, a.z, nsat);
                *reinterpret_cast<uint2*>(&xst[wave][m][8 * j]) = code;
                if (blockIdx.x == 0) *reinterpret_cast<uint2*>(a.xq_out + (size_t)m * K + k0 + 8 * j) = code;
            }
        }
        if (blockIdx.x == 0 && a.sat) {
            nsat = wave_sum(nsat);
            if (lane == 0 && nsat) atomicAdd(a.sat, (uint32_t)nsat);
        }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) *reinterpret_cast<v4i*>(&wst[wave][r][lane * 16]) = wr[r];

    // Lane l: weight row l % 16 (rows past N repeat row N - 1 and feed outputs
    // never stored), activation row l % 16 (zero past M), the same 16 bytes of
    // K; chunks past K zeroed.
    const int rl = lane & 15;
    const bool xvalid = rl < M;
    // All 16 fragment reads first, then the 16 MFMAs; steps past the piece (a
    // partial last piece, or no piece at all) are zeroed by the K test.
    v4i wv[16], xv[FUSED ? 16 : 1];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        wv[t] = *reinterpret_cast<const v4i*>(&wst[wave][rl][64 * t + kl]);
        if constexpr (FUSED) xv[t] = *reinterpret_cast<const v4i*>(&xst[wave][min(rl, M - 1)][64 * t + kl]);
    }
    v4i part[4] = {v4i{}, v4i{}, v4i{}, v4i{}};  // four independent accumulation chains
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const bool kin = k0 + 64 * t + kl < K;
        const v4i x = FUSED ? xv[FUSED ? t : 0] : xf[FUSED ? 0 : t];
        part[t & 3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kin ? wv[t] : v4i{}, xvalid ? x : v4i{},
                                                             part[t & 3], 0, 0, 0);
    }
    v4i acc[1] = {(part[0] + part[1]) + (part[2] + part[3])};
    reduce_and_store<1>(a, acc, e, n0, 0, red);
}

// Sum over the 16 lanes of a DPP row (quad swaps, then the half-row and row
// mirrors); every lane of the row receives the total.
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v) { return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false); }

__device__ __forceinline__ int row16_sum(int v) {
    v += dpp_i32<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_i32<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_i32<0x141>(v);  // row_half_mirror
    v += dpp_i32<0x140>(v);  // row_mirror
    return v;
}

// M == 1, K <= 4096 (one activation row: the MFMA fragments would be 15/16
// padding, and their LDS transposition dominates the kernel's tail).
// Wavefront w owns bytes [1024 w, 1024 w + 1024) of K and lane l the 16 bytes
// at 1024 w + 16 l: one contiguous 1 KB load per weight row, one 16-byte
// activation chunk (FUSED: quantized by the lane from the 16-bit input --
// section 2.3 decode formula, section 2.4 saturation count -- workgroup 0
// writing xq), and four v_dot4_i32_i8 per row.  The 64 x 4 partial sums of a
// row are added through LDS and a 16-lane DPP reduction; lane 0 of each row
// group runs the epilogue.
template <bool FUSED, int DT>
__global__ __launch_bounds__(256) void k_decode_dot(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) int red[4][kRows][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    const int n0 = blockIdx.x * kRows;
    const int kk = wave * kPiece + 16 * lane;  // this lane's 16 bytes of K
    const bool kin = kk < K;                   // K % 16 == 0: the chunk is wholly in or out
    const int kc = min(kk, K - 16);

    // (1) epilogue operands of row n0 + tid / 16, (2) the activation chunk,
    // (3) the 16 weight rows
    const int er = tid >> 4;
    const int en = min(n0 + er, a.N - 1);
    const float e_sw = a.sw[en];
    const int e_cs = a.colsum[en];
    const float e_b = (a.bias ? a.bias : a.sw)[en];
    __builtin_amdgcn_sched_barrier(0);
    Raw8<DT> xr[2];
    v4i xv;
    if constexpr (FUSED) {
        xr[0] = load_raw8<DT>(a.x, kc / 8);
        xr[1] = load_raw8<DT>(a.x, kc / 8 + 1);
    } else {
        xv = *reinterpret_cast<const v4i*>(a.xq + kc);
    }
    __builtin_amdgcn_sched_barrier(0);
    v4i wr[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
        wr[r] = *reinterpret_cast<const v4i*>(a.wq + (size_t)min(n0 + r, a.N - 1) * K + kc);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (FUSED) {
        const float inv = 1.0f / a.s;
        int nsat = 0;
        float v[8];
        widen8<DT>(xr[0], v);
        const uint2 c0 = static_codes8(v, a.s, inv, a.z, nsat);
        widen8<DT>(xr[1], v);
        const uint2 c1 = static_codes8(v, a.s, inv, a.z, nsat);
        xv = v4i{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
        if (blockIdx.x == 0) {
            if (kin) *reinterpret_cast<v4i*>(a.xq_out + kk) = xv;
            if (a.sat) {
                nsat = wave_sum(kin ? nsat : 0);
                if (lane == 0 && nsat) atomicAdd(a.sat, (uint32_t)nsat);
            }
        }
    }
    const v4i x = kin ? xv : v4i{};
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        int p = __builtin_amdgcn_sdot4(wr[r].x, x.x, 0, false);
        p = __builtin_amdgcn_sdot4(wr[r].y, x.y, p, false);
        p = __builtin_amdgcn_sdot4(wr[r].z, x.z, p, false);
        red[wave][r][lane] = __builtin_amdgcn_sdot4(wr[r].w, x.w, p, false);
    }
    __syncthreads();
    // thread t: row er = t / 16 of the group, lanes 4 j .. 4 j + 3 of every wavefront
    const int j = tid & 15;
    int sum = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const v4i q = *reinterpret_cast<const v4i*>(&red[w][er][4 * j]);
        sum += (q.x + q.y) + (q.z + q.w);
    }
    sum = row16_sum(sum);
    const int n = n0 + er;
    if (j == 0 && n < a.N) {
        if (a.acc_out) a.acc_out[n] = sum;
        const int corr = sum - a.z * e_cs;
        const float t = __fmul_rn(a.s, e_sw);
        float y = __fmul_rn(t, (float)corr);
        if (a.bias) y = __fadd_rn(y, e_b);
        a.y[n] = f32_to_bf16(y);
    }
}

template <int NMB, bool FULLK>
__global__ __launch_bounds__(256) void k_decode_gemv(DecodeArgs a) {
    constexpr int KB = NMB == 1 ? 8 : (NMB == 2 ? 6 : 4);  // steps per batch, two batches in flight
    __shared__ v4i red[4][NMB][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = a.M, K = a.K;
    const int n0 = blockIdx.x * kRows;
    const int mbase = blockIdx.y * kMRows;
    const int nsteps = (K + 63) / 64;
    const int kl = 16 * (lane >> 4);
    const EpiOps e = load_epi(a, n0, lane);
    __builtin_amdgcn_sched_barrier(0);
    const int8_t* wp = a.wq + (size_t)min(n0 + (lane & 15), a.N - 1) * K;
    const int8_t* xp[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) xp[mb] = a.xq + (size_t)min(mbase + mb * 16 + (lane & 15), M - 1) * K;
    const int tsteps = (nsteps - wave + 3) / 4;
    const int nbatch = (tsteps + KB - 1) / KB;

    struct Frags {
        v4i w[KB];
        v4i x[NMB][KB];
    };
    // Unconditional loads with clamped steps and chunks; steps past the
    // wave's last are skipped and chunks past K zeroed where the fragments
    // are used (activation rows past M only feed outputs never stored).
    auto load = [&](int b, Frags& f) {
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int k = min(min(wave + 4 * (b * KB + i), nsteps - 1) * 64 + kl, K - 16);
            f.w[i] = *reinterpret_cast<const v4i*>(wp + k);
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) f.x[mb][i] = *reinterpret_cast<const v4i*>(xp[mb] + k);
        }
    };
    v4i acc[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[mb] = v4i{};
    auto compute = [&](int b, const Frags& f) {
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            if (b * KB + i < tsteps) {  // wavefront-uniform
                const int s = wave + 4 * (b * KB + i);
                const v4i wv = (FULLK || s * 64 + kl < K) ? f.w[i] : v4i{};
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, f.x[mb][i], acc[mb], 0, 0, 0);
            }
        }
    };
    Frags f0, f1;
    load(0, f0);
    load(1, f1);
    __builtin_amdgcn_sched_barrier(0);
    // steady state with both refills, then the last one to three batches
    int b = 0;
    for (; b + 3 < nbatch; b += 2) {
        compute(b, f0);
        __builtin_amdgcn_sched_barrier(0);
        load(b + 2, f0);
        __builtin_amdgcn_sched_barrier(0);
        compute(b + 1, f1);
        __builtin_amdgcn_sched_barrier(0);
        load(b + 3, f1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (b + 2 < nbatch) {
        compute(b, f0);
        __builtin_amdgcn_sched_barrier(0);
        load(b + 2, f0);
        __builtin_amdgcn_sched_barrier(0);
        compute(b + 1, f1);
        compute(b + 2, f0);
    } else {
        compute(b, f0);
        if (b + 1 < nbatch) compute(b + 1, f1);
    }
    reduce_and_store<NMB>(a, acc, e, n0, mbase, red);
}

bool lds_path(int64_t M, int64_t K) { return M >= 1 && M <= 16 && K <= 4 * kPiece; }

template <bool FUSED, int DT, int CPT>
void launch_lds(const DecodeArgs& a, hipStream_t st) {
    const dim3 grid((a.N + kRows - 1) / kRows), block(256);
    hipLaunchKernelGGL((k_decode_lds<FUSED, DT, CPT>), grid, block, 0, st, a);
}

template <bool FUSED, int DT>
void launch_dot(const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_decode_dot<FUSED, DT>), dim3((a.N + kRows - 1) / kRows), dim3(256), 0, st, a);
}

template <int DT>
void launch_fused(const DecodeArgs& a, hipStream_t st) {
    if (a.M == 1) {
        launch_dot<true, DT>(a, st);
        return;
    }
    // 8-element chunks per lane: M rows of one wavefront's piece
    const int per_lane = (int)((a.M * (std::min<int64_t>(a.K, kPiece) / 8) + 63) / 64);
    if (per_lane <= 1) launch_lds<true, DT, 1>(a, st);
    else if (per_lane <= 2) launch_lds<true, DT, 2>(a, st);
    else if (per_lane <= 4) launch_lds<true, DT, 4>(a, st);
    else if (per_lane <= 8) launch_lds<true, DT, 8>(a, st);
    else launch_lds<true, DT, 16>(a, st);
}

template <int NMB>
void launch_gemv_nmb(const DecodeArgs& a, dim3 grid, hipStream_t st) {
    if (a.K % 64 == 0)
        hipLaunchKernelGGL((k_decode_gemv<NMB, true>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_decode_gemv<NMB, false>), grid, dim3(256), 0, st, a);
}

}  // namespace

// The one-launch path quantizes the activations in every workgroup: worth it
// while that is a few chunks per thread.
bool decode_fusable(int64_t M, int64_t K) { return lds_path(M, K) && M * K <= 4 * 256 * 8; }

void launch_decode_fused(const DecodeArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return;
    switch (a.x_dt) {
        case kF32: launch_fused<kF32>(a, st); break;
        case kF16: launch_fused<kF16>(a, st); break;
        default: launch_fused<kBF16>(a, st); break;
    }
}

void launch_decode_gemv(const DecodeArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return;
    if (lds_path(a.M, a.K)) {
        if (a.M == 1)
            launch_dot<false, kBF16>(a, st);
        else
            launch_lds<false, kBF16, 1>(a, st);
        return;
    }
    const dim3 grid((a.N + kRows - 1) / kRows, (a.M + kMRows - 1) / kMRows);
    const int mrows = a.M < kMRows ? a.M : kMRows;
    switch ((mrows + 15) / 16) {
        case 1: launch_gemv_nmb<1>(a, grid, st); break;
        case 2: launch_gemv_nmb<2>(a, grid, st); break;
        case 3: launch_gemv_nmb<3>(a, grid, st); break;
        default: launch_gemv_nmb<4>(a, grid, st); break;
    }
}

}  // namespace pdq
