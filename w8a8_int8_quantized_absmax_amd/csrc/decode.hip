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
// bandwidth-bound).  Each 256-thread workgroup owns 16 weight rows and up to 64
// activation rows; its four wavefronts interleave over the K dimension in
// 64-byte steps.  Weight and activation fragments (the activations are already
// quantized, a few hundred KB at most, and come from the L2) are loaded a
// batch at a time, all before the batch's first v_mfma_i32_16x16x64_i8, with
// the next batch in flight during the current one's MFMAs.  The four partial
// accumulators are summed through LDS.

#include "pdq_device.h"
#include "pdq_kernels.h"

namespace pdq {

namespace {

constexpr int kRows = 16;   // weight rows per workgroup
constexpr int kMRows = 64;  // activation rows per workgroup

// 64-byte K steps per batch: a batch's weight and activation fragments are all
// loaded before its first MFMA, and the next batch's loads are in flight while
// this batch computes (two register sets).  (1 + NMB) * KB fragments of 16
// bytes per lane per set.
template <int NMB>
struct DecodeBatch {
    static constexpr int KB = NMB == 1 ? 8 : (NMB == 2 ? 6 : 4);
};

template <int NMB>
__global__ __launch_bounds__(256) void k_decode_gemv(DecodeArgs a) {
    constexpr int KB = DecodeBatch<NMB>::KB;
    __shared__ v4i red[4][NMB][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = a.M, N = a.N, K = a.K;
    const int n0 = blockIdx.x * kRows;
    const int mbase = blockIdx.y * kMRows;
    const int nsteps = (K + 63) / 64;
    const int kl = 16 * (lane >> 4);
    const int wrow = n0 + (lane & 15);
    const bool wvalid = wrow < N;
    const int8_t* wp = a.wq + (size_t)(wvalid ? wrow : 0) * K + kl;
    const int8_t* xp[NMB];
    bool xvalid[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        const int xm = mbase + mb * 16 + (lane & 15);
        xvalid[mb] = xm < M;
        xp[mb] = a.xq + (size_t)(xvalid[mb] ? xm : 0) * K + kl;
    }
    // wave w takes the steps s = w + 4 t, t = 0, 1, ...; batch b holds t in
    // [b KB, b KB + KB)
    const int tsteps = (nsteps - wave + 3) / 4;
    const int nbatch = (tsteps + KB - 1) / KB;

    struct Frags {
        uint4 w[KB];
        uint4 x[NMB][KB];
    };
    auto load = [&](int b, Frags& f) {
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int s = wave + 4 * (b * KB + i);
            const bool kin = s < nsteps && s * 64 + kl < K;
            f.w[i] = (wvalid && kin) ? *reinterpret_cast<const uint4*>(wp + (size_t)s * 64)
                                     : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
                f.x[mb][i] = (xvalid[mb] && kin) ? *reinterpret_cast<const uint4*>(xp[mb] + (size_t)s * 64)
                                                 : make_uint4(0, 0, 0, 0);
        }
    };
    v4i acc[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[mb] = v4i{};
    auto compute = [&](const Frags& f) {
#pragma unroll
        for (int i = 0; i < KB; ++i)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, f.w[i]),
                                                                __builtin_bit_cast(v4i, f.x[mb][i]),
                                                                acc[mb], 0, 0, 0);
    };
    Frags f0, f1;
    if (nbatch > 0) load(0, f0);
    for (int b = 0; b < nbatch; b += 2) {
        if (b + 1 < nbatch) load(b + 1, f1);
        compute(f0);
        if (b + 1 < nbatch) {
            if (b + 2 < nbatch) load(b + 2, f0);
            compute(f1);
        }
    }

#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) red[wave][mb][lane] = acc[mb];
    __syncthreads();
    if (wave >= NMB) return;
    const v4i tot = red[0][wave][lane] + red[1][wave][lane] + red[2][wave][lane] + red[3][wave][lane];

    // 16x16 accumulator layout: lane l, register r holds row 4*(l/16) + r
    // (the weight row n) and column l%16 (the activation row m).
    const int m = mbase + wave * 16 + (lane & 15);
    if (m >= M) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = n0 + 4 * (lane >> 4) + r;
        if (n < N) {
            const int raw = tot[r];
            if (a.acc_out) a.acc_out[(size_t)m * N + n] = raw;
            const int corr = raw - a.z * a.colsum[n];
            const float t = __fmul_rn(a.s, a.sw[n]);
            float y = __fmul_rn(t, (float)corr);
            if (a.bias) y = __fadd_rn(y, a.bias[n]);
            a.y[(size_t)m * a.ldy + n] = f32_to_bf16(y);
        }
    }
}

}  // namespace

void launch_decode_gemv(const DecodeArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return;
    const dim3 grid((a.N + kRows - 1) / kRows, (a.M + kMRows - 1) / kMRows), block(256);
    const int mrows = a.M < kMRows ? a.M : kMRows;
    const int nmb = (mrows + 15) / 16;
    switch (nmb) {
        case 1: hipLaunchKernelGGL(k_decode_gemv<1>, grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_decode_gemv<2>, grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL(k_decode_gemv<3>, grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL(k_decode_gemv<4>, grid, block, 0, st, a); break;
    }
}

}  // namespace pdq
