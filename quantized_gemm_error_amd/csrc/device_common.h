// Device helpers for the gfx950 kernels of libspear: vector types, the
// 4-bit dequantization into MFMA operands, MFMA wrappers, the sigmoid gate
// and the packed-operand permutation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spear {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

enum { DT_F16 = 0, DT_BF16 = 1 };

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From &v) {
  static_assert(sizeof(To) == sizeof(From), "bitcast size");
  return __builtin_bit_cast(To, v);
}

// D = A * B + C for one 16x16x32 block.  Lane l supplies row (l % 16) of A
// and column (l % 16) of B, eight K-values each from K-slot group l / 16.
// D lands as rows 4 * (l / 16) + v, column l % 16, v = 0..3.
template <int DT>
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c,
                                                  0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b),
                                                   c, 0, 0, 0);
  }
}

// fp32 16x16x4 block: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16].
__device__ __forceinline__ f32x4_t mfma_16x16x4_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The packed weight's tiled order: rows in blocks of 16 (row count padded to
// a multiple of 16), each block 2 K words long, made of 1 KB tiles of 128
// codes in which lane 16 h + r of a wave finds, at word 4 (16 h + r), the
// four words of row r that hold the tile's codes 32 h .. 32 h + 31.
// tiled_block gives that lane's piece in tile 0 of the block holding row
// n_block (a multiple of 16; past the last row the last block, so that every
// address stays inside the array); tile kb is 256 kb words further on.  A
// piece that would start past K (a partial last tile, or K < 128) must be
// read from 4 lane words back, the block's first piece, which is always
// inside the array.
__device__ __forceinline__ const uint32_t *tiled_block(const uint32_t *qw, int n_block, int N,
                                                       int K, int lane) {
  const int rb = min(n_block, N - 1) >> 4;
  return qw + (size_t)rb * 2 * K + 4 * lane;
}

// The same block as a buffer resource of its 2 K words (n_block uniform
// across the wave): tile kb of it is 1 KB at byte kb * 1024, a lane's piece
// at 16 lane bytes into the tile (tile_piece).  A piece past K lies past the
// block's end and reads as zeros through the range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tiled_block_rsrc(const uint32_t *qw, int n_block,
                                                                   int N, int K) {
  const int rb = min(n_block, N - 1) >> 4;
  return __builtin_amdgcn_make_buffer_rsrc((void *)(qw + (size_t)rb * 2 * K), (short)0, K * 8,
                                           0x00020000);
}

// A lane's 16-byte piece of tile kb, read once per call (non-temporal).
__device__ __forceinline__ u32x4_t tile_piece(__amdgpu_buffer_rsrc_t blk, int kb, int lane) {
  return __builtin_amdgcn_raw_buffer_load_b128(blk, 16 * lane, kb * 1024, 2);
}

// Workgroup barrier for LDS only: this wave's LDS operations complete
// (lgkmcnt(0)), then s_barrier.  __syncthreads() also carries a release fence
// that waits for every outstanding global load (vmcnt(0)), which would drain
// the weight and activation prefetches at every staged chunk.  The signal
// fences keep the compiler from moving memory operations across.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Four consecutive fp32 values published by another workgroup, read
// coherently across the XCDs' L2 caches (cache policy sc1, as a relaxed
// agent-scope atomic load has).
__device__ __forceinline__ f32x4_t load_partials4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return bitcast<f32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16));
}

// The same four values stored for other workgroups (sc1: written through to
// the level every XCD reads with sc1 loads).
__device__ __forceinline__ void store_partials4(f32x4_t v, __amdgpu_buffer_rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(bitcast<u32x4_t>(v), r, byte_off, 0, 16);
}

// Completion of this wave's agent-scope stores before the count that
// publishes them.  Those stores (sc1) are written through to the level that
// every XCD reads with sc1 loads, so they need no write-back of the L2, only
// an s_waitcnt vmcnt(0) (gfx9 counts stores in vmcnt; this encoding leaves
// expcnt and lgkmcnt at their maxima).  The signal fences keep the compiler
// from moving memory operations across the wait.
__device__ __forceinline__ void publish_wait() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Round to bf16 and the bf16 of the remainder: hi + lo equals v to a relative
// 2^-16 (exactly when v has at most 16 significant bits, as fp16 values do).
__device__ __forceinline__ void split_bf16(float v, uint16_t &hi, uint16_t &lo) {
  const __bf16 h = (__bf16)v;
  hi = bitcast<uint16_t>(h);
  lo = bitcast<uint16_t>((__bf16)(v - (float)h));
}

// Per-row zero-point constant for dequant_word.
//   fp16: packed pair of -(1024 + z) (exact: 1024 + z is an integer < 2048).
//   bf16: 2^23 + z as an fp32 bit pattern.
template <int DT>
__device__ __forceinline__ uint32_t zero_constant(uint16_t z_f16_bits) {
  const float z = (float)bitcast<_Float16>(z_f16_bits);
  if constexpr (DT == DT_F16) {
    const _Float16 nz = (_Float16)(-(1024.0f + z));
    const uint32_t b = bitcast<uint16_t>(nz);
    return b | (b << 16);
  } else {
    return bitcast<uint32_t>(8388608.0f + z);
  }
}

// v_and_or_b32: (x & m) | c in one instruction (VOP3; m and c in registers).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(c));
  return r;
}

// One packed word (codes q0..q7, lowest nibble first) to the exact values
// q_i - z in the activation type, as four dwords holding the pairs
// (q0,q4) (q1,q5) (q2,q6) (q3,q7).  The activation operand that meets these
// in an MFMA is permuted the same way (permute_8).
//
// fp16: a low nibble OR 0x6400 read as binary16 is 1024 + q exactly, and a
//       high nibble (bits 4..7) OR 0x6400 is 1024 + 16 q exactly.  One packed
//       add of -(1024 + z), or one packed fma by 1/16 with -(64 + z), leaves
//       q - z exactly (an integer of magnitude <= 15).  zc is the packed pair
//       -(1024 + z); -(64 + z) is zc + 960.
// bf16: (nibble | 0x4B000000) read as binary32 is 2^23 + q exactly; after
//       subtracting 2^23 + z (zc holds that fp32 bit pattern) the integer
//       q - z converts to bf16 exactly.
template <int DT>
__device__ __forceinline__ u32x4_t dequant_word(uint32_t w, uint32_t zc) {
  u32x4_t r;
  if constexpr (DT == DT_F16) {
    const uint32_t lo_mask = 0x000F000Fu, hi_mask = 0x00F000F0u, magic = 0x64006400u;
    const f16x2_t nz = bitcast<f16x2_t>(zc);
    const f16x2_t nz64 = nz + f16x2_t{(_Float16)960.0f, (_Float16)960.0f};
    const f16x2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t w8 = w >> 8;
    r[0] = bitcast<uint32_t>(bitcast<f16x2_t>(and_or(w, lo_mask, magic)) + nz);
    r[1] = bitcast<uint32_t>(bitcast<f16x2_t>(and_or(w, hi_mask, magic)) * sixteenth + nz64);
    r[2] = bitcast<uint32_t>(bitcast<f16x2_t>(and_or(w8, lo_mask, magic)) + nz);
    r[3] = bitcast<uint32_t>(bitcast<f16x2_t>(and_or(w8, hi_mask, magic)) * sixteenth + nz64);
  } else {
    const float zf = bitcast<float>(zc);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float lo = bitcast<float>(((w >> (4 * t)) & 0xFu) | 0x4B000000u) - zf;
      const float hi = bitcast<float>(((w >> (4 * t + 16)) & 0xFu) | 0x4B000000u) - zf;
      const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
      r[t] = bitcast<uint32_t>(p);
    }
  }
  return r;
}

// The four bytes of x as fp32 (exact), one v_cvt_f32_ubyteN each.
__device__ __forceinline__ void cvt_f32_ubytes(uint32_t x, float (&f)[4]) {
  asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f[0]) : "v"(x));
  asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f[1]) : "v"(x));
  asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f[2]) : "v"(x));
  asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f[3]) : "v"(x));
}

// bf16 only: one packed word to the exact values q_i - z in natural order,
// four dwords holding (q0,q1) (q2,q3) (q4,q5) (q6,q7).  Each nibble is
// extracted on its own (as in dequant_word's bf16 form), so the order costs
// nothing here, and the activation operand it meets needs no permutation.
// The even nibbles and the odd ones go to the bytes of two words, and each
// byte converts to fp32 exactly (v_cvt_f32_ubyteN); q - z is then one exact
// fp32 subtraction (z = zc's 2^23 + z less 2^23, exact) and one rounding-free
// conversion of the integer pair to bf16.
__device__ __forceinline__ u32x4_t dequant_word_bf16_natural(uint32_t w, uint32_t zc) {
  const float z = bitcast<float>(zc) - 8388608.0f;
  const uint32_t ev = w & 0x0F0F0F0Fu;         // nibbles 0, 2, 4, 6
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;  // nibbles 1, 3, 5, 7
  float fe[4], fo[4];
  cvt_f32_ubytes(ev, fe);
  cvt_f32_ubytes(od, fo);
  u32x4_t r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bf16x2_t p = {(__bf16)(fe[t] - z), (__bf16)(fo[t] - z)};
    r[t] = bitcast<uint32_t>(p);
  }
  return r;
}

// Eight consecutive activation values (natural order) to the order
// (x0,x4,x1,x5,x2,x6,x3,x7) that matches dequant_word's pairs.
__device__ __forceinline__ u32x4_t permute_8(u32x4_t v) {
  const u16x8_t h = bitcast<u16x8_t>(v);
  const u16x8_t p = __builtin_shufflevector(h, h, 0, 4, 1, 5, 2, 6, 3, 7);
  return bitcast<u32x4_t>(p);
}

template <int DT>
__device__ __forceinline__ float to_f32(uint16_t bits) {
  if constexpr (DT == DT_F16) {
    return (float)bitcast<_Float16>(bits);
  } else {
    return bitcast<float>((uint32_t)bits << 16);
  }
}

// Round to nearest even into the activation type.
template <int DT>
__device__ __forceinline__ uint16_t from_f32(float v) {
  if constexpr (DT == DT_F16) {
    return bitcast<uint16_t>((_Float16)v);
  } else {
    return bitcast<uint16_t>((__bf16)v);
  }
}

// Logistic gate.  exp(-z) overflows to +inf for very negative z, which
// gives exactly 0; z = +inf gives exactly 1; z = 0 gives exactly 1/2.
__device__ __forceinline__ float gate_sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace spear
