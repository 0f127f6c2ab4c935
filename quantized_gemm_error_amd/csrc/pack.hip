// Packing 4-bit codes: uint8 q[N][K] -> int32 words [N][K/8], code k = 8j+i
// of a row in bits 4i..4i+3 of word j (lowest nibble first).
//
// Memory-bound: each thread turns 32 input bytes (two 16-byte loads) into 4
// words (one 16-byte store) when the row allows it, else one word at a time.
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

__global__ __launch_bounds__(256) void pack_int4_vec_kernel(const u32x4_t *__restrict__ q,
                                                            u32x4_t *__restrict__ out,
                                                            int64_t n_quads) {
  // one "quad" = 4 output words = 32 input bytes
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_quads;
       i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4_t a = q[2 * i];
    const u32x4_t b = q[2 * i + 1];
    u32x4_t w;
    w[0] = pack_8(a[0], a[1]);
    w[1] = pack_8(a[2], a[3]);
    w[2] = pack_8(b[0], b[1]);
    w[3] = pack_8(b[2], b[3]);
    out[i] = w;
  }
}

__global__ __launch_bounds__(256) void pack_int4_word_kernel(const uint8_t *__restrict__ q,
                                                             uint32_t *__restrict__ out,
                                                             int64_t n_words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint8_t *p = q + 8 * i;
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) w |= ((uint32_t)p[k] & 0xFu) << (4 * k);
    out[i] = w;
  }
}

hipError_t launch_pack_int4(const uint8_t *q, int32_t *out, int64_t N, int64_t K,
                            hipStream_t s) {
  const int64_t n_words = N * (K / 8);
  if (n_words == 0) return hipSuccess;
  const bool vec = ((uintptr_t)q % 16 == 0) && ((uintptr_t)out % 16 == 0) && (n_words % 4 == 0);
  if (vec) {
    const int64_t n_quads = n_words / 4;
    const int64_t blocks = (n_quads + 255) / 256;
    const int grid = (int)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(pack_int4_vec_kernel, dim3(grid), dim3(256), 0, s,
                       (const u32x4_t *)q, (u32x4_t *)out, n_quads);
  } else {
    const int64_t blocks = (n_words + 255) / 256;
    const int grid = (int)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(pack_int4_word_kernel, dim3(grid), dim3(256), 0, s, q, (uint32_t *)out,
                       n_words);
  }
  return hipGetLastError();
}

}  // namespace spear
