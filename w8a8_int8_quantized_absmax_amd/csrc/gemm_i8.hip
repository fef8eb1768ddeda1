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
// MFMA into a separate binary32 accumulator per 32x32 sub-tile.  With a zero
// point acc becomes acc - Z * colsum[n] before the conversion (PDMIX
// terminology entry section 2.3 through the zero-point expansion of the
// LLM.int8() notes, part 1 section 2): ZP == 1, the static path's per-tensor
// S and Z; ZP == 2, per-token scales S_a[m] with per-token zero points Z[m].
//
// Tiling: 256x256 output tile per 256-thread workgroup (4 wavefronts in a
// 2x2 arrangement, 128x128 each = 4x4 v_mfma_i32_32x32x32_i8 tiles with
// their INT32 accumulators in registers, W rows as the MFMA row operand so
// that each lane ends up with runs of 4 consecutive outputs), K staged through
// LDS 64 bytes at a time.  A K tile of 256 rows is 256 lines of 64 bytes,
// XOR-swizzled in 16-byte chunks so that the 128-bit fragment reads are free
// of bank conflicts (see swz).  Tiles move global -> LDS directly
// (global_load_lds, no register staging) through a ring of four LDS buffers:
// three K tiles are in flight while one feeds the MFMAs.  A and B are both
// packed (pdq_device.h): their 1 KB blocks already are the LDS images of 16
// rows, so every load instruction is one block, every request a whole cache
// line (a row-major panel costs a half-line request per row), and the zeros
// of the K padding make a partial last K tile need no masking.  The weight
// is the MFMA's row operand and the activation codes the column operand: the
// other way round the same products draw more power and the kernel runs
// about 6% slower under the board's power limit.  The epilogue goes
// wavefront by wavefront and 32 rows at a time through the LDS output tile
// (see below), with no workgroup barrier.

#include "pdq_device.h"
#include "pdq_kernels.h"

#include <type_traits>

namespace pdq {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;  // BK in bytes = K values per LDS stage
constexpr int kStages = 4;                   // LDS ring: 4 x 32 KB, three K tiles in flight
static_assert((kStages & (kStages - 1)) == 0, "ring index uses a mask");
constexpr int kStageBytes = (BM + BN) * BK;
// Output tile in LDS after the K loop: 256 rows of 256 16-bit values, padded
// to 520 bytes so that the 8-byte writes of 32 lanes (32 rows, 4 values each)
// hit 32 distinct bank pairs; rows [64 s, 64 s + 64) live in stage buffer s.
constexpr int kYPitch = BN * 2 + 8;
constexpr int kStageAlloc = kStageBytes > 64 * kYPitch ? kStageBytes : 64 * kYPitch;

// LDS image of a K tile: row r (64 bytes) holds its 16-byte chunk kc at
// position kc ^ ((r >> 2) & 3).  A 128-bit read instruction is served 16
// lanes at a time over 64 four-byte banks (256 bytes = 4 rows): the 16 lanes
// read rows r..r+15 at one logical chunk; rows r, r+1, r+2, r+3 fall in the
// four bank quarters and, within a quarter, the 4 rows land on 4 distinct
// chunk positions.
__device__ __forceinline__ int swz_pos(int r, int kc) { return kc ^ ((r >> 2) & 3); }
__device__ __forceinline__ int swz(int r, int kc) { return r * BK + (swz_pos(r, kc) << 4); }

constexpr int kXcds = 8;     // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kGroupM = 4;   // tile rows per group of the grouped order

// Tile of workgroup `bid`.  Consecutive workgroup ids land on different XCDs,
// each with its own L2; renumber so that every XCD works through a contiguous
// run of tiles, and walk tiles in groups of kGroupM tile rows (column by
// column inside a group) so that the tiles resident on one XCD at a time share
// a few A and B panels.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int num = tiles_m * tiles_n;
    const int q = num / kXcds, r = num % kXcds;
    const int xcd = bid % kXcds, local = bid / kXcds;
    const int id = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
    const int per_group = kGroupM * tiles_n;
    const int g = id / per_group;
    const int first_m = g * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int in = id - g * per_group;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate (gfx9 layout): at most `vm` vector-memory loads and
// `lgkm` LDS operations of this wave still outstanding, export count untouched.
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// Wait until at most VM of this wave's K-tile loads are in flight and all its
// LDS reads have returned, then join the workgroup barrier.  Written with the
// builtins rather than assembly so that the compiler sees the wait: its own
// waits before the LDS reads that follow then only cover loads that are really
// still outstanding (with an opaque wait it assumes every earlier
// global -> LDS load may still be writing and drains them all).  The empty
// asm statements keep the compiler from moving memory accesses across.
template <int VM>
__device__ __forceinline__ void wait_loads_and_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// MI: 32-row MFMA blocks per wave.  4: the 256x256 tile.  2: half of it,
// rows [128 h, 128 h + 128) of the 256-row tile at m0 (h from the tile
// index), computed by the 4 waves as 2x2 blocks of 64x128; only those 128 A
// rows of each K tile are loaded (6 loads per wave and K tile instead of 8),
// and the MFMAs and the A fragment reads halve.  Used for a last round of at most 128 tiles, so that
// it fills the 256 CUs with half the work each instead of leaving half of
// them idle.
template <int OUT, bool SIDE, int ZP, int MI>
__global__ __launch_bounds__(256) void k_gemm_i8(GemmArgs a) {
    // The four K-tile buffers (each A[256][64] followed by B[256][64]) are
    // four separate LDS objects, and every access below names its buffer
    // statically (the K loop is unrolled by four).  The compiler then knows
    // that fragment reads of one buffer do not alias the global->LDS loads in
    // flight into the others and waits only for the loads of the buffer it
    // reads; with one array it has to drain every load in flight first.
    __shared__ __attribute__((aligned(1024))) uint8_t st0[kStageAlloc];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[kStageAlloc];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[kStageAlloc];
    __shared__ __attribute__((aligned(1024))) uint8_t st3[kStageAlloc];
    // the tile's row scales, column scales and bias, staged once at the start
    __shared__ __attribute__((aligned(16))) float s_sa[BM], s_sb[BN], s_bias[BN];
    // ZP == 1: z * colsum[n]; ZP == 2: colsum[n], with the row zero points in s_za
    __shared__ __attribute__((aligned(16))) int32_t s_zc[ZP ? BN : 1];
    __shared__ __attribute__((aligned(16))) int32_t s_za[ZP == 2 ? BM : 1];
    auto stage = [&](auto idx) -> uint8_t* {
        constexpr int i = decltype(idx)::value & (kStages - 1);
        if constexpr (i == 0) return st0;
        else if constexpr (i == 1) return st1;
        else if constexpr (i == 2) return st2;
        else return st3;
    };

    // The wavefront index through readfirstlane: wave-uniform, so it and what
    // derives from it (the tile quadrant, the LDS rows this wave fills) live
    // in scalar registers; the K loop uses every vector register.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int M = a.M, N = a.N, K = a.K;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn, mh = 0;
    if constexpr (MI == 4) {
        tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    } else {
        int th;
        tile_of(blockIdx.x, 2 * tiles_m, tiles_n, th, tn);
        tm = th >> 1;
        mh = (th & 1) * 128;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int nkt = (K + BK - 1) / BK;

    v16i acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};

    {
        const int m = m0 + tid, n = n0 + tid;  // 256 threads = BM = BN
        s_sa[tid] = m < M ? (a.sa ? a.sa[m] : a.s) : 0.0f;
        s_sb[tid] = n < N ? a.sb[n] : 0.0f;
        s_bias[tid] = (a.bias && n < N) ? a.bias[n] : 0.0f;
        if constexpr (ZP == 1) s_zc[tid] = n < N ? a.z * a.colsum[n] : 0;
        if constexpr (ZP == 2) {
            s_zc[tid] = n < N ? a.colsum[n] : 0;
            s_za[tid] = m < M ? a.za[m] : 0;
        }
    }
    __syncthreads();


    // Global -> LDS without registers: one global_load_lds_dwordx4 moves 64
    // lanes x 16 bytes into 1 KB of LDS, lane l's 16 bytes at 16 l: one packed
    // block, which already is the swizzled image of its 16 rows.  Wave w fills
    // rows [64w, 64w + 64) of the B tile, four 16-row groups, and of the A tile
    // the rows the workgroup multiplies: [64w, 64w + 64) of a whole tile (four
    // groups), [mh + 32w, mh + 32w + 32) of a half tile (two), each at its row
    // of the 256-row LDS image: 4 + 4 or 2 + 4 instructions per K tile.  Groups
    // past the last (of A or B) are clamped onto it: they only feed outputs
    // that are never stored.
    constexpr int kLA = MI == 4 ? 4 : 2;  // A loads per wave and K tile
    constexpr int kLoads = kLA + 4;       // loads per wave and K tile
    const int8_t* pa[4];  // the first kLA used (an array of kLA elements drops the host stubs)
    const int8_t* pb[4];
    const int lastga = (M - 1) / kWGroup, lastgb = (N - 1) / kWGroup;
    [[maybe_unused]] const int arow0 = mh + wave * 32;  // half tile: this wave's first A row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (MI == 4)
            pa[i] = a.A + wpack_block(min(m0 / kWGroup + wave * 4 + i, lastga), 0, nkt) + lane * 16;
        else if (i < kLA)
            pa[i] = a.A + wpack_block(min((m0 + arow0) / kWGroup + i, lastga), 0, nkt) + lane * 16;
        pb[i] = a.B + wpack_block(min(n0 / kWGroup + wave * 4 + i, lastgb), 0, nkt) + lane * 16;
    }
    // Load number `i` (0 .. kLoads - 1: A groups, then B groups) of K tile kt into `buf`.
    auto issue_one = [&](uint8_t* buf, int kt, int i) {
        uint8_t* la = buf + wave * 64 * BK;
        if constexpr (MI == 4) {
            if (i < 4)
                __builtin_amdgcn_global_load_lds(pa[i] + (size_t)kt * kWBlock, (lds_ptr_t)(la + i * 16 * BK), 16, 0,
                                                 0);
            else
                __builtin_amdgcn_global_load_lds(pb[i - 4] + (size_t)kt * kWBlock,
                                                 (lds_ptr_t)(la + BM * BK + (i - 4) * 16 * BK), 16, 0, 0);
        } else {
            if (i < kLA)
                __builtin_amdgcn_global_load_lds(pa[i] + (size_t)kt * kWBlock,
                                                 (lds_ptr_t)(buf + (arow0 + i * 16) * BK), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds(pb[i - kLA] + (size_t)kt * kWBlock,
                                                 (lds_ptr_t)(la + BM * BK + (i - kLA) * 16 * BK), 16, 0, 0);
        }
    };
    // Fragments of one 32-wide K step: lane l reads row (l%32) of each 32-row
    // block, chunk 2*s + l/32 (16 bytes = 16 K values).
    auto read_frags = [&](const uint8_t* sbase, int s, v4i (&fa)[4], v4i (&fb)[4]) {
        const int kc = 2 * s + (lane >> 5);
#pragma unroll
        for (int i = 0; i < MI; ++i)
            fa[i] = *reinterpret_cast<const v4i*>(
                sbase + swz((MI == 4 ? wm * 128 : mh + wm * 64) + i * 32 + (lane & 31), kc));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fb[j] = *reinterpret_cast<const v4i*>(sbase + BM * BK +
                                                  swz(wn * 128 + j * 32 + (lane & 31), kc));
    };
    auto mfma = [&](const v4i (&fa)[4], const v4i (&fb)[4], int i, int j) {
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
    };
    // K loop.  Each 64-byte K tile is two steps of 16 MFMAs on register set
    // f0 (step 0) and f1 (step 1).  Step 0 reads step 1's fragments and spreads
    // the 8 loads of tile kt+3 (into the buffer tile kt-1 used) over its MFMAs.
    // Step 1 runs one MFMA, then this wave waits for its loads of tile kt+1 and
    // joins the barrier: past it every wave holds tile kt's step-1 fragments in
    // registers (so buffer kt may be refilled) and every wave's loads of tile
    // kt+1 have landed, so step 0 of tile kt+1 is read during the remaining 15
    // MFMAs.  One barrier per tile, and no LDS latency exposed between tiles.
    //
    // Every tile issues exactly kLoads loads per wave, also past the last tile
    // (those re-load the last tile into a buffer nobody reads again), so the
    // number of loads in flight is the same on every path and each wait below
    // -- and each wait the compiler derives for the LDS reads -- is exact.
    v4i f0a[4], f0b[4], f1a[4], f1b[4];
    auto issue_tile = [&](uint8_t* buf, int t, int i) { issue_one(buf, min(t, nkt - 1), i); };
    if (nkt > 0) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) issue_tile(st0, 0, i);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) issue_tile(st1, 1, i);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) issue_tile(st2, 2, i);
        wait_loads_and_sync<2 * kLoads>();
        read_frags(st0, 0, f0a, f0b);
        auto body = [&](auto S, int kt) {
            constexpr int s0 = decltype(S)::value;
            const uint8_t* sb = stage(std::integral_constant<int, s0>{});
            const uint8_t* sn = stage(std::integral_constant<int, s0 + 1>{});
            uint8_t* sd = stage(std::integral_constant<int, s0 + kStages - 1>{});
            const int next = kt + kStages - 1;
            read_frags(sb, 1, f1a, f1b);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mfma(f0a, f0b, i, j);
                    if constexpr (MI == 4) {
                        if (j & 1) issue_tile(sd, next, 2 * i + (j >> 1));
                    } else {
                        if (4 * i + j < kLoads) issue_tile(sd, next, 4 * i + j);  // 8 MFMAs, 6 loads
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            mfma(f1a, f1b, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            // Loads issued after tile kt+1's: tiles kt+2 and kt+3.  Also after
            // the last tile (tile kt+1 then re-loads the last one), so that the
            // wait is on every path and the compiler's count stays exact.
            wait_loads_and_sync<2 * kLoads>();
            read_frags(sn, 0, f0a, f0b);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (i | j) mfma(f1a, f1b, i, j);
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        int kt = 0;
        for (; kt + 4 <= nkt; kt += 4) {
            body(I0{}, kt);
            body(I1{}, kt + 1);
            body(I2{}, kt + 2);
            body(I3{}, kt + 3);
        }
        const int rem = nkt - kt;  // tile kt sits in buffer 0
        if (rem > 0) body(I0{}, kt);
        if (rem > 1) body(I1{}, kt + 1);
        if (rem > 2) body(I2{}, kt + 2);
    }  // nkt > 0

    // Epilogue.  acc[i][j] is the 32x32 block (W rows n, X rows m) of the
    // wave's 128x128 tile: lane l, register r holds n = 8*(r/4) + 4*(l/32) +
    // r%4 and m = l%32, i.e. 4 consecutive outputs of one row of y per
    // register quad.  They are rounded, packed and written to the LDS output
    // tile with one 8-byte write, and leave in 16-byte row chunks.
    // The lane index again, from the lane masks (v_mbcnt) rather than kept in
    // a register across the K loop.
    const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    int side_steps = 0;
    bool poison = false;
    const int ml0 = (MI == 4 ? wm * 128 : mh + wm * 64) + (elane & 31);
    const int nl0 = wn * 128 + 4 * (elane >> 5);
    [[maybe_unused]] uint4 xs0[4], ws0[4];
    if constexpr (SIDE) {
        const int cnt = *a.count;
        poison = cnt > a.max_count;
        side_steps = poison ? 0 : (cnt + 15) / 16;
        // The first 16 outlier columns of this wave's X_out and W_out rows,
        // fetched while the last K tiles land.  Rows past M or N are clamped:
        // they only feed outputs that are never stored.
        if (side_steps > 0) {
            const int koff = 8 * (elane >> 5);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int m = min(m0 + ml0 + 32 * i, M - 1);
                xs0[i] = *reinterpret_cast<const uint4*>(a.xo + (size_t)m * a.P + koff);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int wr = min(n0 + wn * 128 + 32 * j + (elane & 31), N - 1);
                ws0[j] = *reinterpret_cast<const uint4*>(a.wo + (size_t)wr * a.P + koff);
            }
        }
    }
    wait_loads_and_sync<0>();  // the ring is no longer read or written
    auto yrow = [&](int ml) -> uint8_t* {
        uint8_t* b = ml < 128 ? (ml < 64 ? st0 : st1) : (ml < 192 ? st2 : st3);
        return b + (ml & 63) * kYPitch;
    };
    float sam[4];
    [[maybe_unused]] int zam[4];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        sam[i] = s_sa[ml0 + 32 * i];
        if constexpr (ZP == 2) zam[i] = -s_za[ml0 + 32 * i];  // negated: one multiply-add below
    }
    auto side_mfma = [&](uint4 wv, uint4 xv, v16f c) -> v16f {
        if constexpr (OUT == kF16)
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, wv),
                                                          __builtin_bit_cast(v8h, xv), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, wv),
                                                           __builtin_bit_cast(v8bf, xv), c, 0, 0, 0);
    };
    if (a.acc_out) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int m = m0 + ml0 + 32 * i, n = n0 + nl0 + 32 * j + 8 * g;
                    if (m < M) {
                        int32_t* ap = a.acc_out + (size_t)m * a.ldacc + n;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N) ap[e] = acc[i][j][4 * g + e];
                    }
                }
    }
    // One 32-row block of the wave's outputs at a time: the wave converts its
    // 32 rows x 128 columns of block i into its own part of the LDS output
    // tile, reads them back as 16-byte row chunks and stores them, then
    // converts block i + 1 while those stores drain.  No workgroup barrier:
    // a wave only reads back what it wrote itself (LDS operations of one wave
    // complete in order), and the four waves' parts of the tile are disjoint.
    // The bias test is taken once for the whole tile, not per element.
    uint16_t* y = static_cast<uint16_t*>(a.y);
    const bool vec = ((reinterpret_cast<uintptr_t>(y) & 15) == 0) && (a.ldy % 8 == 0);
    const int rbase = MI == 4 ? wm * 128 : mh + wm * 64;  // the wave's first tile row
    auto convert = [&](auto bias_tag) {
        constexpr bool kBias = decltype(bias_tag)::value;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int ml = ml0 + 32 * i;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float sbv[4][4], bv[4][4];
                int32_t zcv[4][4];
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sbv[g][e] = s_sb[nl0 + 32 * j + 8 * g + e];
                        if constexpr (kBias) bv[g][e] = s_bias[nl0 + 32 * j + 8 * g + e];
                        if constexpr (ZP) zcv[g][e] = s_zc[nl0 + 32 * j + 8 * g + e];
                    }
                v16f side = v16f{};
                if constexpr (SIDE) {
                    // 16-bit product of the outlier columns for this 32x32
                    // block, in the same (n, m) orientation: W_out rows x
                    // X_out rows.
                    if (side_steps > 0) {
                        side = side_mfma(ws0[j], xs0[i], side);
                        const int m = min(m0 + ml, M - 1);
                        const int wr = min(n0 + wn * 128 + 32 * j + (elane & 31), N - 1);
                        for (int ks = 1; ks < side_steps; ++ks) {
                            const int koff = ks * 16 + 8 * (elane >> 5);
                            const uint4 xv = *reinterpret_cast<const uint4*>(a.xo + (size_t)m * a.P + koff);
                            const uint4 wv = *reinterpret_cast<const uint4*>(a.wo + (size_t)wr * a.P + koff);
                            side = side_mfma(wv, xv, side);
                        }
                    }
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float t = __fmul_rn(sam[i], sbv[g][e]);
                        // |Z| <= 128 and |colsum| < 127 * 65536 < 2^23: a 24-bit
                        // multiply-add (v_mad_i32_i24)
                        const int32_t q = ZP == 1   ? acc[i][j][4 * g + e] - zcv[g][e]
                                          : ZP == 2 ? __mul24(zam[i], zcv[g][e]) + acc[i][j][4 * g + e]
                                                    : acc[i][j][4 * g + e];
                        v[e] = __fmul_rn(t, (float)q);
                        if constexpr (SIDE) v[e] = __fadd_rn(v[e], side[4 * g + e]);
                        if constexpr (kBias) v[e] = __fadd_rn(v[e], bv[g][e]);
                        if constexpr (SIDE)
                            if (poison) v[e] = __builtin_nanf("");
                    }
                    const int nl = nl0 + 32 * j + 8 * g;
                    *reinterpret_cast<uint2*>(yrow(ml) + nl * 2) =
                        make_uint2(f32x2_to_16<OUT>(v[0], v[1]), f32x2_to_16<OUT>(v[2], v[3]));
                }
            }
            // Rows rbase + 32 i .. + 32, columns wn * 128 .. + 128 of the tile:
            // 8 passes of 4 rows x 16 chunks of 8 outputs.  A chunk is read as
            // two 8-byte halves (rows are 8-byte aligned at the 520-byte
            // pitch), as two separate ds_read_b64: in each, lanes 0..15 read
            // every other 8 bytes of 256 consecutive bytes of one row and lanes
            // 16..31 those of the next row, 130 words further, so the 32 lanes
            // of a pass hit 64 distinct banks.  (Merged into one ds_read2_b64
            // the same reads counted 1024 bank-conflict cycles per workgroup.)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int r = rbase + 32 * i + 4 * q + (elane >> 4);
                const int nl = wn * 128 + 8 * (elane & 15);
                const int m = m0 + r, n = n0 + nl;
                const uint2* src = reinterpret_cast<const uint2*>(yrow(r) + nl * 2);
                const uint2 lo = src[0];
                asm volatile("" ::: "memory");  // keeps the two reads apart
                const uint2 hi = src[1];
                if (m >= M || n >= N) continue;
                uint16_t* dst = y + (size_t)m * a.ldy + n;
                if (vec && n + 8 <= N) {
                    *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
                } else {
                    const uint16_t v[8] = {(uint16_t)lo.x, (uint16_t)(lo.x >> 16), (uint16_t)lo.y,
                                           (uint16_t)(lo.y >> 16), (uint16_t)hi.x, (uint16_t)(hi.x >> 16),
                                           (uint16_t)hi.y, (uint16_t)(hi.y >> 16)};
                    for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = v[e];
                }
            }
        }
    };
    if (a.bias)
        convert(std::true_type{});
    else
        convert(std::false_type{});
}

}  // namespace

template <int MI>
void launch_tiles(const GemmArgs& a, int out_dt, bool side, hipStream_t st, int zp_mode) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * (4 / MI);
    const dim3 grid(tiles), block(256);
    if (!side && zp_mode == 1)
        hipLaunchKernelGGL((k_gemm_i8<kBF16, false, 1, MI>), grid, block, 0, st, a);
    else if (!side && zp_mode == 2)
        hipLaunchKernelGGL((k_gemm_i8<kBF16, false, 2, MI>), grid, block, 0, st, a);
    else if (!side)
        hipLaunchKernelGGL((k_gemm_i8<kBF16, false, 0, MI>), grid, block, 0, st, a);
    else if (out_dt == kF16)
        hipLaunchKernelGGL((k_gemm_i8<kF16, true, 0, MI>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((k_gemm_i8<kBF16, true, 0, MI>), grid, block, 0, st, a);
}

// One tile per CU and round (one 160 KB workgroup fills a CU).  When the last
// round would hold at most 128 tiles and they make up whole tile columns, those
// columns run as a second launch of half tiles: twice the workgroups, half
// the work each, so that the last round occupies all 256 CUs.
void launch_gemm_i8(const GemmArgs& args, int out_dt, bool side, hipStream_t st, int zp_mode) {
    if (args.M <= 0 || args.N <= 0) return;
    GemmArgs a = args;
    if (a.ldacc == 0) a.ldacc = a.N;  // the launches below may cover column ranges of it
    constexpr int kCUs = 256;
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n, last = tiles % kCUs;
    const int cols = (tiles > kCUs && last > 0 && last <= kCUs / 2 && last % tiles_m == 0) ? last / tiles_m : 0;
    if (cols == 0 || cols >= tiles_n) {
        launch_tiles<4>(a, out_dt, side, st, zp_mode);
        return;
    }
    const int n1 = (tiles_n - cols) * BN;  // whole tiles: columns [0, n1)
    GemmArgs a1 = a;
    a1.N = n1;
    launch_tiles<4>(a1, out_dt, side, st, zp_mode);
    // half tiles: columns [n1, N), every pointer indexed by n moved to column n1
    GemmArgs a2 = a;
    a2.N = a.N - n1;
    a2.B = a.B + (size_t)(n1 / kWGroup) * ((a.K + BK - 1) / BK) * kWBlock;  // packed 16-row groups
    a2.sb = a.sb + n1;
    if (a.bias) a2.bias = a.bias + n1;
    if (a.colsum) a2.colsum = a.colsum + n1;
    a2.y = static_cast<uint16_t*>(a.y) + n1;
    if (a.acc_out) a2.acc_out = a.acc_out + n1;
    if (a.wo) a2.wo = a.wo + (size_t)n1 * a.P;
    launch_tiles<2>(a2, out_dt, side, st, zp_mode);
}

}  // namespace pdq
