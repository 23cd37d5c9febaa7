// Expert weight packing: reorders each expert matrix [R rows, KB bytes per
// row] into the tiled layout the expert GEMM streams from.
//
// A tile is 16 rows x 256 bytes = 4 KiB, stored as [piece s: 4][lane L: 64]
// [16 bytes], where lane L = r + 16 g holds bytes [64 s + 16 g, +16) of row
// r of the tile.  Tiles of one 16-row block follow each other along K, so a
// row block stays contiguous.  A wave that loads piece s of a tile issues
// one 1 KiB contiguous load (whole 128-byte lines), and lane L receives
// exactly its MFMA A-operand fragment (row r, k-group g).
#include "common.h"
#include "kernels.h"

namespace beam {

// one thread per 16-byte piece of the destination
__global__ __launch_bounds__(256) void beam_pack_rows(const uint8_t* __restrict__ src,
                                                      uint8_t* __restrict__ dst, size_t n_pieces,
                                                      int kb) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_pieces) return;
    const int lane = (int)(i & 63);
    const int s = (int)((i >> 6) & 3);
    const size_t tile = i >> 8;                 // 256 pieces per tile
    const size_t tiles_per_block = kb / 256;
    const size_t rb = tile / tiles_per_block;
    const size_t c = tile - rb * tiles_per_block;
    const int r = lane & 15, g = lane >> 4;
    const size_t src_off = (rb * 16 + r) * (size_t)kb + c * 256 + 64 * s + 16 * g;
    *reinterpret_cast<uint4*>(dst + i * 16) = *reinterpret_cast<const uint4*>(src + src_off);
}

hipError_t launch_pack(const void* src, void* dst, size_t rows, int kb, hipStream_t st) {
    const size_t n_pieces = rows * (size_t)kb / 16;
    const size_t blocks = (n_pieces + 255) / 256;
    hipLaunchKernelGGL(beam_pack_rows, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), n_pieces, kb);
    return hipGetLastError();
}

}  // namespace beam
