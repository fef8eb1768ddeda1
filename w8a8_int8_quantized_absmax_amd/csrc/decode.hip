// Decode-phase skinny INT8 GEMM (M small) with the zero-point epilogue (gfx950).
//
// acc[m, n] = sum_k xq[m, k] * wq[n, k], then
//   y = (S * S_w[n]) * (float)(acc - Z * colsum[n]) [+ bias[n]]
// i.e. the PDMIX terminology entry's decode formula (section 2.3, static
// per-tensor S and Z) pushed through the zero-point expansion of the LLM.int8()
// notes (part 1 section 2) with a symmetric weight; or, with per-token scales
// (the same entry's prefill formula, for the per-token GEMM entry points),
// y = (S_x[m] * S_w[n]) * (float)(acc [- Z_x[m] * colsum[n]]) [+ bias[n]].
// The static symmetric grid (tensor-wise absmax with a static scale, LLM.int8()
// notes part 1 section 1) is the static one with Z = 0 and codes clamped to
// [-127, 127].
//
// The weight matrix is read exactly once and is the whole cost (the
// hardware-acceleration page's "data movement and memory bandwidth": decode is
// bandwidth-bound).  Each 256-thread workgroup owns 16, 32, 48 or 64 weight
// channels (decode_groups); its four wavefronts interleave
// over the K tiles of the packed weight (wavefront w takes tiles w, w + 4,
// ...) and multiply with v_mfma_i32_16x16x64_i8,
// weight channels as the row operand, activation rows as the column operand.
// In the packed layout the 16 channels' K tile is one contiguous 1 KB block
// (and all of them one contiguous run), so lane l loads its fragment (channel
// l % 16, K bytes 16 (l / 16) ..) directly: one whole-line, fully coalesced
// instruction per tile, no LDS transposition.  The epilogue's per-channel
// operands are loaded first, so their latency hides under the weight stream;
// the four partial accumulators are summed through LDS.
//
// Activations: fragment loads of the packed xq (from the cache), up to 64
// rows per workgroup row (four register blocks of 16), one 16-row block per
// K tile and register block -- again one contiguous 1 KB load (the rows of a
// partial block past M are clamped onto its last row, so that they cost no
// extra lines); or -- FUSED, the one-launch path, for M * K up to 8192 --
// quantized inside the kernel while the first weight tiles are in flight
// (static quantization, the PDMIX terminology entry's section 2.3 decode
// formula and section 2.4 saturation count; workgroup 0 writes the codes of
// xq and counts the saturated values, the first few others write its zero
// padding rows): each wavefront quantizes exactly the activations of its own
// K tiles, into its own LDS region, or for one activation row into
// registers.  Loads are issued in batches of K tiles, two batches in flight,
// all unconditional (tiles past the wavefront's last are clamped and skipped
// at use; K values past K are zeros in the packed operands, and in the
// quantized LDS copy).

#include "pdq_device.h"
#include "pdq_kernels.h"

#include <algorithm>
#include <type_traits>

namespace pdq {

namespace {

constexpr int kRows = 16;   // weight rows per channel group
constexpr int kMRows = 64;  // activation rows per workgroup (four register blocks of 16)
constexpr int kCUs = 256;   // compute units of an MI355X

// Epilogue operands of this lane's four outputs n = n0 + 4 (lane / 16) + r
// (16x16 accumulator layout: register r is row 4 (lane / 16) + r, the weight
// row n).  Loaded unconditionally: one 16-byte load per array where the four
// channels are inside N and the arrays 16-byte aligned, else element by
// element with columns past N clamped; a missing bias or code sum (per-token
// scales, no zero point) reads the scales and is ignored.
struct EpiOps {
    float sw[4], bias[4];
    int32_t cs[4];
};

__device__ __forceinline__ EpiOps load_epi(const DecodeArgs& a, int n0, int lane) {
    EpiOps e;
    const float* bp = a.bias ? a.bias : a.sw;
    const int32_t* cp = a.colsum ? a.colsum : reinterpret_cast<const int32_t*>(a.sw);
    const int nb = n0 + 4 * (lane >> 4);
    const uintptr_t al = reinterpret_cast<uintptr_t>(a.sw) | reinterpret_cast<uintptr_t>(bp) |
                         reinterpret_cast<uintptr_t>(cp);
    if (nb + 3 < a.N && (al & 15) == 0) {
        const v4i s4 = *reinterpret_cast<const v4i*>(a.sw + nb);
        const v4i c4 = *reinterpret_cast<const v4i*>(cp + nb);
        const v4i b4 = *reinterpret_cast<const v4i*>(bp + nb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            e.sw[r] = __int_as_float(s4[r]);
            e.cs[r] = c4[r];
            e.bias[r] = __int_as_float(b4[r]);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = min(nb + r, a.N - 1);
            e.sw[r] = a.sw[n];
            e.cs[r] = cp[n];
            e.bias[r] = bp[n];
        }
    }
    return e;
}

// Sum of the four wavefronts' partial accumulators and the epilogue: block
// (g, mb) holds weight channels n0 + 16 g .. + 16 and activation rows
// mbase + 16 mb .. + 16, and wavefront (g NMB + mb) % 4 finishes it.
template <int NG, int NMB>
__device__ __forceinline__ void reduce_and_store(const DecodeArgs& a, const v4i (&acc)[NG][NMB],
                                                 const EpiOps (&e)[NG], int n0, int mbase,
                                                 v4i (&red)[4][NG * NMB][64]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // vector stores need 8-byte aligned y row pieces (16-byte for acc)
    const bool y_vec = (reinterpret_cast<uintptr_t>(a.y) & 7) == 0 && a.ldy % 4 == 0;
    const bool acc_vec = (reinterpret_cast<uintptr_t>(a.acc_out) & 15) == 0 && a.N % 4 == 0;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) red[wave][g * NMB + mb][lane] = acc[g][mb];
    __syncthreads();
#pragma unroll
    for (int blk = 0; blk < NG * NMB; ++blk) {
        if (blk % 4 != wave) continue;  // wavefront-uniform
        constexpr int kNMB = NMB;
        const int g = blk / kNMB, mb = blk % kNMB;
        const v4i tot = red[0][blk][lane] + red[1][blk][lane] + red[2][blk][lane] + red[3][blk][lane];
        const int m = mbase + mb * 16 + (lane & 15);
        if (m >= a.M) continue;
        // this lane's outputs: row m, the 4 consecutive channels nb .. nb + 3
        const int nb = n0 + 16 * g + 4 * (lane >> 4);
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int raw = tot[r];
            // per-token: (S_x[m] * S_w[n]) * (acc [- Z_x[m] colsum[n]]);
            // static: (S * S_w[n]) * (acc - Z colsum[n])
            const int corr = a.za ? raw - a.za[m] * e[g].cs[r] : (a.sa ? raw : raw - a.z * e[g].cs[r]);
            const float t = __fmul_rn(a.sa ? a.sa[m] : a.s, e[g].sw[r]);
            y[r] = __fmul_rn(t, (float)corr);
            if (a.bias) y[r] = __fadd_rn(y[r], e[g].bias[r]);
        }
        // One store per lane and output (8 bytes of y, 16 of acc) where the row
        // piece is aligned and inside N: four 2-byte stores per lane made the
        // stores the longest part of the kernel's tail.
        const bool whole = nb + 3 < a.N;
        if (a.acc_out) {
            int32_t* ap = a.acc_out + (size_t)m * a.N + nb;
            if (whole && acc_vec)
                *reinterpret_cast<v4i*>(ap) = tot;
            else
                for (int r = 0; r < 4 && nb + r < a.N; ++r) ap[r] = tot[r];
        }
        uint16_t* yp = a.y + (size_t)m * a.ldy + nb;
        if (whole && y_vec)
            *reinterpret_cast<uint2*>(yp) = make_uint2(f32x2_to_16<kBF16>(y[0], y[1]), f32x2_to_16<kBF16>(y[2], y[3]));
        else
            for (int r = 0; r < 4 && nb + r < a.N; ++r) yp[r] = f32_to_bf16(y[r]);
    }
}

template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v) { return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false); }

// Lane 16 r + t receives lane 16 r + t + J of its DPP row (row_shl J).
template <int J>
__device__ __forceinline__ v4i row_shl(v4i v) {
    if constexpr (J == 0)
        return v;
    else
        return v4i{dpp_i32<0x100 + J>(v.x), dpp_i32<0x100 + J>(v.y), dpp_i32<0x100 + J>(v.z),
                   dpp_i32<0x100 + J>(v.w)};
}

constexpr int kFusedBytes = 8192;  // M * K limit of the one-launch path
// LDS codes per wavefront on that path: M rows x ceil(ceil(K / 64) / 4) K tiles x 64
constexpr int kFusedWave = kFusedBytes / 4 + 16 * 64;

// ONEROW (FUSED, M == 1, K <= 4096): lane l quantizes chunk (tile l % 16 of
// its wavefront, quarter l / 16) into registers, and for tile j the lanes
// 16 r -- the only ones whose MFMA column is the activation row -- take
// quarter r from lane 16 r + j of their DPP row: no LDS round trip.
//
// NG: 16-channel groups per workgroup (1 to 4, chosen by decode_groups):
// each activation fragment then serves 16 NG channels per load.
template <int NMB, bool FUSED, int DT, int kQ = 1, bool ONEROW = false, int NG = 1>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
    static_assert(!FUSED || NG == 1, "the one-launch path has one channel group");
    // K tiles per batch, two batches in flight.  Measured per shape (graph
    // replays, weights rotated beyond the MALL): 16 channels and 17..32 rows
    // run 5% faster with 4 tiles (three workgroups per CU) than with 6 (two);
    // 33..64 rows are best at 4, and 32 channels with 17..32 rows at 4 (2 or
    // 3 were slower or no faster).  48 channels with 17..32 rows take 4 (one
    // workgroup per CU, as where that width is chosen: 12288 channels x 32
    // rows 12.6 us against 13.0 with 3), otherwise 2; 64 channels take 2
    // (3 was 4-12% slower at 24..512 rows).
    constexpr int KB = NG == 1   ? (NMB == 1 ? 8 : 4)
                       : NG == 2 ? (NMB == 1 ? 6 : (NMB == 2 ? 4 : 3))
                       : NG == 3 ? (NMB == 1 ? 4 : (NMB == 2 ? 4 : 2))
                                 : (NMB == 1 ? 4 : 2);
    __shared__ v4i red[4][NG * NMB][64];
    __shared__ __attribute__((aligned(16))) int8_t xs[FUSED ? 4 : 1][FUSED ? kFusedWave : 16];
    // The wavefront index read through readfirstlane is known to be uniform,
    // so that branches on it (tiles a wavefront skips) are scalar branches:
    // MFMA instructions ignore EXEC, and an MFMA under a lane mask that the
    // compiler does not skip with a branch would still accumulate.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = a.M, K = a.K;
    const int n0 = blockIdx.x * kRows * NG;
    const int mbase = blockIdx.y * kMRows;
    const int nsteps = (K + 63) / 64;  // K tiles
    const int kl = 16 * (lane >> 4);
    EpiOps e[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) e[g] = load_epi(a, n0 + kRows * g, lane);
    __builtin_amdgcn_sched_barrier(0);

    // FUSED: each wavefront quantizes exactly the activations of its own K
    // tiles (tiles wave + 4 j), 16 values per lane and chunk: chunk c = (row m,
    // local tile j, quarter q) of the M x twmax x 4; at most kQ per lane.  The
    // codes go to the wavefront's own LDS region (no barrier), their loads go
    // out before the weight's.
    const int twmax = (nsteps + 3) / 4;
    const int nq = M * twmax * 4;
    Raw8<DT> xa[FUSED ? kQ : 1], xb[FUSED ? kQ : 1];
    auto qchunk = [&](int c, int& m, int& s, int& kk) {
        if constexpr (ONEROW) {  // c = lane: tile c % 16, quarter c / 16
            m = 0;
            s = wave + 4 * (c & 15);
            kk = s * 64 + 16 * (c >> 4);
        } else {
            m = c / (twmax * 4);
            const int r = c - m * twmax * 4;
            s = wave + 4 * (r >> 2);
            kk = s * 64 + 16 * (r & 3);
        }
    };
    if constexpr (FUSED) {
#pragma unroll
        for (int i = 0; i < kQ; ++i) {
            int m, s, kk;
            qchunk(ONEROW ? lane : min(lane + 64 * i, nq - 1), m, s, kk);
            const char* row = static_cast<const char*>(a.x) + (size_t)m * a.ldx * Elem<DT>::bytes;
            const int ck = min(kk, K - 16) / 8;
            xa[i] = load_raw8<DT>(row, ck);
            xb[i] = load_raw8<DT>(row, ck + 1);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // this lane's weight fragment of group g in K tile s: wp[g] + s * kWBlock
    // (a group past the last is clamped onto it: its outputs are not stored)
    const int8_t* wp[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)
        wp[g] = a.wq + wpack_block(min(n0 / kWGroup + g, (a.N - 1) / kWGroup), 0, nsteps) +
                wpack_pos(lane & 15, lane >> 4);
    // this lane's activation fragment of register block mb in K tile s:
    // xp[mb] + s * kWBlock (row lane % 16 of the block, clamped into M)
    const int8_t* xp[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        const int g = min(mbase / 16 + mb, (M - 1) / 16);
        xp[mb] = a.xq + wpack_block(g, 0, nsteps) + wpack_pos(min(lane & 15, M - 1 - 16 * g), lane >> 4);
    }
    const int xrow = min(lane & 15, M - 1);  // FUSED (M <= 16)
    const int8_t* xw = xs[FUSED ? wave : 0];
    const int tsteps = (nsteps - wave + 3) / 4;
    const int nbatch = (tsteps + KB - 1) / KB;

    struct Frags {
        v4i w[NG][KB];
        v4i x[FUSED ? 1 : NMB][KB];
    };
    auto load = [&](int b, Frags& f) {
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int s = min(wave + 4 * (b * KB + i), nsteps - 1);
#pragma unroll
            for (int g = 0; g < NG; ++g) f.w[g][i] = *reinterpret_cast<const v4i*>(wp[g] + (size_t)s * kWBlock);
            if constexpr (!FUSED) {
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) f.x[mb][i] = *reinterpret_cast<const v4i*>(xp[mb] + (size_t)s * kWBlock);
            }
        }
    };
    v4i acc[NG][NMB];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[g][mb] = v4i{};
    auto compute = [&](int b, const Frags& f) {
        // FUSED: the batch's activation fragments from LDS first, then the MFMAs
        v4i xv[FUSED ? KB : 1];
        if constexpr (FUSED) {
#pragma unroll
            for (int i = 0; i < KB; ++i)
                xv[i] = *reinterpret_cast<const v4i*>(&xw[(xrow * twmax + min(b * KB + i, twmax - 1)) * 64 + kl]);
        }
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            if (b * KB + i < tsteps) {  // wavefront-uniform
                if constexpr (FUSED) {
                    acc[0][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.w[0][i], xv[i], acc[0][0], 0, 0, 0);
                } else {
#pragma unroll
                    for (int g = 0; g < NG; ++g)
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb)
                            acc[g][mb] =
                                __builtin_amdgcn_mfma_i32_16x16x64_i8(f.w[g][i], f.x[mb][i], acc[g][mb], 0, 0, 0);
                }
            }
        }
    };
    Frags f0, f1;
    load(0, f0);
    load(1, f1);
    __builtin_amdgcn_sched_barrier(0);

    v4i xcode = v4i{};  // ONEROW: this lane's codes
    if constexpr (FUSED) {
        const float inv = 1.0f / a.s;
        const int qmin = a.narrow ? -127 : -128;
        int nsat = 0;
#pragma unroll
        for (int i = 0; i < kQ; ++i) {
            const int c = lane + 64 * i;
            if (ONEROW || c < nq) {
                int m, s, kk;
                qchunk(c, m, s, kk);
                v4i code = v4i{};  // zeros past K (the weight is zero there too)
                if (s < nsteps) {
                    if (kk < K) {
                        float v[8];
                        widen8<DT>(xa[i], v);
                        const uint2 lo = static_codes8(v, a.s, inv, a.z, nsat, qmin);
                        widen8<DT>(xb[i], v);
                        const uint2 hi = static_codes8(v, a.s, inv, a.z, nsat, qmin);
                        code = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
                    }
                    if (blockIdx.x == 0)
                        *reinterpret_cast<v4i*>(a.xq_out + wpack_block(0, s, nsteps) + wpack_pos(m, (kk >> 4) & 3)) =
                            code;
                }
                if constexpr (ONEROW)
                    xcode = code;
                else
                    *reinterpret_cast<v4i*>(&xs[wave][c * 16]) = code;
            }
        }
        if (blockIdx.x == 0 && a.sat) {
            nsat = wave_sum(nsat);
            if (lane == 0 && nsat) atomicAdd(a.sat, (uint32_t)nsat);
        }
        // the zero rows M .. 15 of the codes' one 16-row group: 16-byte chunk
        // p = (row - M, tile, chunk) of them per thread, by the workgroups
        // after the first (or by the only one)
        const int first = gridDim.x > 1 ? 1 : 0, nwg = gridDim.x - first;
        const int npad = (kWGroup - M) * nsteps * 4;
        if ((int)blockIdx.x >= first) {
            for (int p = (blockIdx.x - first) * 256 + tid; p < npad; p += nwg * 256) {
                const int r = M + p / (nsteps * 4), t = (p / 4) % nsteps;
                *reinterpret_cast<v4i*>(a.xq_out + wpack_block(0, t, nsteps) + wpack_pos(r, p & 3)) = v4i{};
            }
        }
    }

    if constexpr (ONEROW) {  // at most 16 tiles per wavefront: batches 0 and 1
        auto run = [&](auto bb, const Frags& f) {
            constexpr int B = decltype(bb)::value;
            const v4i xv[KB] = {row_shl<B * KB + 0>(xcode), row_shl<B * KB + 1>(xcode),
                                row_shl<B * KB + 2>(xcode), row_shl<B * KB + 3>(xcode),
                                row_shl<B * KB + 4>(xcode), row_shl<B * KB + 5>(xcode),
                                row_shl<B * KB + 6>(xcode), row_shl<B * KB + 7>(xcode)};
#pragma unroll
            for (int i = 0; i < KB; ++i)
                if (B * KB + i < tsteps)
                    acc[0][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.w[0][i], xv[i], acc[0][0], 0, 0, 0);
        };
        run(std::integral_constant<int, 0>{}, f0);
        run(std::integral_constant<int, 1>{}, f1);
    } else {
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
    }
    reduce_and_store<NG, NMB>(a, acc, e, n0, mbase, red);
}

template <int NMB, bool FUSED, int DT, int kQ = 1, bool ONEROW = false, int NG = 1>
void launch_k(const DecodeArgs& a, hipStream_t st) {
    const dim3 grid((a.N + kRows * NG - 1) / (kRows * NG), FUSED ? 1 : (a.M + kMRows - 1) / kMRows);
    hipLaunchKernelGGL((k_decode<NMB, FUSED, DT, kQ, ONEROW, NG>), grid, dim3(256), 0, st, a);
}

// One-launch path: kQ = 16-value chunks per lane = ceil(M x ceil(tiles / 4) x 4 / 64).
template <int DT>
void launch_fused(const DecodeArgs& a, hipStream_t st) {
    const int nq = a.M * (((a.K + 63) / 64 + 3) / 4) * 4;
    if (a.M == 1 && a.K <= 64 * 64) launch_k<1, true, DT, 1, true>(a, st);
    else if (nq <= 64) launch_k<1, true, DT, 1>(a, st);
    else if (nq <= 128) launch_k<1, true, DT, 2>(a, st);
    else launch_k<1, true, DT, 4>(a, st);
}

}  // namespace

// The one-launch path quantizes the activations in every workgroup: worth it
// while that is a few chunks per thread.
bool decode_fusable(int64_t M, int64_t K) { return M >= 1 && M <= 16 && M * K <= kFusedBytes; }

void launch_decode_fused(const DecodeArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return;
    switch (a.x_dt) {
        case kF32: launch_fused<kF32>(a, st); break;
        case kF16: launch_fused<kF16>(a, st); break;
        default: launch_fused<kBF16>(a, st); break;
    }
}

// Channel groups per workgroup.  Each workgroup reads the activation
// fragments of all its rows once, whatever its channel count, so wider
// workgroups cut those bytes per weight byte but leave fewer workgroups.  Up
// to 16 rows the fragments cost no more than the weight and 16 channels (the
// most workgroups, the most weight bytes in flight) run.  Beyond, the time
// follows the bytes that the busiest CU pulls from the L2: ceil(workgroups /
// 256) x (16 g + rows) x K for g groups; the g in 1..4 with the fewest runs
// (ties to the smaller).  Measured with the weights streamed from HBM: at
// 8, 32 and 64 rows (12288, 4096 and 28672 channels at K = 4096, 4096 at K =
// 14336) the choice is the fastest of the four widths; from 8 to 512 rows
// (also 11008 channels) it is never more than 2% slower than the earlier
// rule (32 channels once that gave 512 workgroups, else 16), except at 16
// rows x 28672 channels (4%), and up to 35% faster: 12288 channels at 32 /
// 64 rows 15.5 / 21.7 -> 13.0 / 15.3 us (48 channels), 28672 at 64 rows
// 42.2 -> 32.2 us (64), 4096 x 4096 at 256 rows 19.9 -> 14.7 us (64).
int decode_groups(int64_t M, int64_t N) {
    const int64_t rows = M < kMRows ? M : kMRows;
    if (rows <= 16) return 1;
    const int64_t rowblocks = (M + kMRows - 1) / kMRows;
    int best = 1;
    int64_t best_bytes = 0;
    for (int g = 1; g <= 4; ++g) {
        const int64_t wgs = (N + kRows * g - 1) / (kRows * g) * rowblocks;
        const int64_t bytes = (wgs + kCUs - 1) / kCUs * (kRows * g + rows);
        if (g == 1 || bytes < best_bytes) {
            best = g;
            best_bytes = bytes;
        }
    }
    return best;
}

template <int NG>
void launch_gemv_ng(const DecodeArgs& a, hipStream_t st) {
    const int mrows = a.M < kMRows ? a.M : kMRows;
    switch ((mrows + 15) / 16) {
        case 1: launch_k<1, false, kBF16, 1, false, NG>(a, st); break;
        case 2: launch_k<2, false, kBF16, 1, false, NG>(a, st); break;
        case 3: launch_k<3, false, kBF16, 1, false, NG>(a, st); break;
        default: launch_k<4, false, kBF16, 1, false, NG>(a, st); break;
    }
}

void launch_decode_gemv(const DecodeArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return;
    switch (decode_groups(a.M, a.N)) {
        case 1: launch_gemv_ng<1>(a, st); break;
        case 2: launch_gemv_ng<2>(a, st); break;
        case 3: launch_gemv_ng<3>(a, st); break;
        default: launch_gemv_ng<4>(a, st); break;
    }
}

}  // namespace pdq
