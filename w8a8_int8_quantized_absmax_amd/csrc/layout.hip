// Conversion between plain row-major INT8 matrices and the packed tile layout
// that the GEMMs read (pdq_device.h: blocks of 16 rows x 64 K values, the
// 16-byte chunk c of row r at position c ^ ((r >> 2) & 3)), for callers that
// hold INT8 weights quantized elsewhere or want the activation codes in plain
// form.  One thread per 16-byte chunk of the packed image, so both directions
// are whole-line copies on the packed side; rows past the last and K values
// past K are zeros in the packed image.

#include "pdq_device.h"
#include "pdq_kernels.h"

namespace pdq {

namespace {

// Chunk t of the packed image: block (g, s) = t / 64, row r = (t / 4) % 16,
// stored position p = t % 4 of that row, which holds the chunk c = p ^ ((r >>
// 2) & 3) of K values 64 s + 16 c ...
__device__ __forceinline__ void chunk_coords(int64_t t, int64_t ktiles, int64_t& row, int64_t& k0, int64_t& off) {
    const int64_t blk = t >> 6;
    const int r = (int)((t >> 2) & 15), p = (int)(t & 3);
    const int c = p ^ ((r >> 2) & 3);
    const int64_t g = blk / ktiles, s = blk - g * ktiles;
    row = g * kWGroup + r;
    k0 = s * kWTileK + 16 * c;
    off = wpack_block(g, s, ktiles) + wpack_pos(r, c);
}

__global__ __launch_bounds__(256) void k_pack_int8(const int8_t* __restrict__ src, int64_t rows, int64_t K,
                                                   int64_t ld, int8_t* __restrict__ packed, int64_t nchunks,
                                                   int64_t ktiles) {
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < nchunks; t += (int64_t)gridDim.x * 256) {
        int64_t row, k0, off;
        chunk_coords(t, ktiles, row, k0, off);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (row < rows && k0 < K) v = *reinterpret_cast<const uint4*>(src + row * ld + k0);
        *reinterpret_cast<uint4*>(packed + off) = v;
    }
}

__global__ __launch_bounds__(256) void k_unpack_int8(const int8_t* __restrict__ packed, int64_t rows, int64_t K,
                                                     int8_t* __restrict__ dst, int64_t ld, int64_t nchunks,
                                                     int64_t ktiles) {
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < nchunks; t += (int64_t)gridDim.x * 256) {
        int64_t row, k0, off;
        chunk_coords(t, ktiles, row, k0, off);
        if (row < rows && k0 < K)
            *reinterpret_cast<uint4*>(dst + row * ld + k0) = *reinterpret_cast<const uint4*>(packed + off);
    }
}

// Chunks of the packed image of a rows x K matrix, and a grid for them (up
// to 8 workgroups of 256 per CU, each thread looping beyond).
int64_t packed_chunks(int64_t rows, int64_t K) {
    return (rows + kWGroup - 1) / kWGroup * ((K + kWTileK - 1) / kWTileK) * (kWBlock / 16);
}

unsigned layout_grid(int64_t nchunks) {
    const int64_t wgs = (nchunks + 255) / 256;
    return (unsigned)(wgs < 2048 ? wgs : 2048);
}

}  // namespace

void launch_pack_int8(const int8_t* src, int64_t rows, int64_t K, int64_t ld, int8_t* packed, hipStream_t st) {
    const int64_t n = packed_chunks(rows, K);
    if (n <= 0) return;
    hipLaunchKernelGGL(k_pack_int8, dim3(layout_grid(n)), dim3(256), 0, st, src, rows, K, ld, packed, n,
                       (K + kWTileK - 1) / kWTileK);
}

void launch_unpack_int8(const int8_t* packed, int64_t rows, int64_t K, int8_t* dst, int64_t ld, hipStream_t st) {
    const int64_t n = packed_chunks(rows, K);
    if (n <= 0) return;
    hipLaunchKernelGGL(k_unpack_int8, dim3(layout_grid(n)), dim3(256), 0, st, packed, rows, K, dst, ld, n,
                       (K + kWTileK - 1) / kWTileK);
}

}  // namespace pdq
