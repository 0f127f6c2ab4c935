// Packing 4-bit codes into the weight order the kernels stream.
//
// Eight codes per 32-bit word along K, lowest nibble first: code k = 8j + i
// of a row sits in bits 4i..4i+3 of that row's word j.  The words are not
// stored row after row: the rows are padded to a multiple of 16 and taken in
// blocks of 16 rows, and inside a block piece P (words 4P .. 4P + 3, codes
// 32P .. 32P + 31) of rows 0..15 comes first, then piece P + 1 of the same 16
// rows.  One 128-code tile of a row block is therefore 1 KB of consecutive
// memory in exactly the order a 64-lane wave loads it, lane 16 h + r taking
// piece h of the tile for row r, which is the operand order of a 16x16x32
// MFMA; a weight stream is then a run of whole 1 KB reads.
//
// Two producers of that order: from unpacked codes (spear_pack_int4) and
// from words already packed row after row (spear_tile_int4).  Each thread
// writes one 16-byte piece; consecutive threads write consecutive pieces.
#include "device_common.h"
#include "internal.h"

namespace spear {

__device__ __forceinline__ uint32_t pack_8(uint32_t lo, uint32_t hi) {
  // bytes b0..b3 of lo are codes 0..3, of hi codes 4..7
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w |= ((lo >> (8 * i)) & 0xFu) << (4 * i);
    w |= ((hi >> (8 * i)) & 0xFu) << (4 * (i + 4));
  }
  return w;
}

// Piece c of the tiled order -> (row n, first code k0).  A row block holds
// K / 2 pieces: K / 32 pieces along K, each for 16 rows.
__device__ __forceinline__ void piece_origin(int64_t c, int64_t K, int64_t &n, int64_t &k0) {
  const int64_t per_block = K / 2;
  const int64_t rb = c / per_block, w = c - rb * per_block;
  n = rb * 16 + (w & 15);
  k0 = (w >> 4) * 32;
}

template <bool VEC>
__global__ __launch_bounds__(256) void pack_tiled_kernel(const uint8_t *__restrict__ q,
                                                         u32x4_t *__restrict__ out, int64_t N,
                                                         int64_t K, int64_t n_pieces) {
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_pieces;
       c += (int64_t)gridDim.x * blockDim.x) {
    int64_t n, k0;
    piece_origin(c, K, n, k0);
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (n < N) {
      const uint8_t *p = q + n * K + k0;
      if constexpr (VEC) {
        const u32x4_t a = *(const u32x4_t *)p;
        const u32x4_t b = *(const u32x4_t *)(p + 16);
        w[0] = pack_8(a[0], a[1]);
        w[1] = pack_8(a[2], a[3]);
        w[2] = pack_8(b[0], b[1]);
        w[3] = pack_8(b[2], b[3]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t v = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) v |= ((uint32_t)p[8 * t + i] & 0xFu) << (4 * i);
          w[t] = v;
        }
      }
    }
    out[c] = w;
  }
}

__global__ __launch_bounds__(256) void tile_words_kernel(const u32x4_t *__restrict__ words,
                                                         u32x4_t *__restrict__ out, int64_t N,
                                                         int64_t K, int64_t n_pieces) {
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_pieces;
       c += (int64_t)gridDim.x * blockDim.x) {
    int64_t n, k0;
    piece_origin(c, K, n, k0);
    out[c] = n < N ? words[(n * K + k0) / 32] : u32x4_t{0u, 0u, 0u, 0u};
  }
}

static int grid_for(int64_t n) {
  const int64_t blocks = (n + 255) / 256;
  return (int)(blocks < 65536 ? blocks : 65536);
}

hipError_t launch_pack_int4(const uint8_t *q, int32_t *out, int64_t N, int64_t K,
                            hipStream_t s) {
  const int64_t n_pieces = (N + 15) / 16 * (K / 2);
  if (n_pieces == 0) return hipSuccess;
  if ((uintptr_t)q % 16 == 0)
    hipLaunchKernelGGL(pack_tiled_kernel<true>, dim3(grid_for(n_pieces)), dim3(256), 0, s, q,
                       (u32x4_t *)out, N, K, n_pieces);
  else
    hipLaunchKernelGGL(pack_tiled_kernel<false>, dim3(grid_for(n_pieces)), dim3(256), 0, s, q,
                       (u32x4_t *)out, N, K, n_pieces);
  return hipGetLastError();
}

hipError_t launch_tile_int4(const int32_t *words, int32_t *out, int64_t N, int64_t K,
                            hipStream_t s) {
  const int64_t n_pieces = (N + 15) / 16 * (K / 2);
  if (n_pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_words_kernel, dim3(grid_for(n_pieces)), dim3(256), 0, s,
                     (const u32x4_t *)words, (u32x4_t *)out, N, K, n_pieces);
  return hipGetLastError();
}

}  // namespace spear
