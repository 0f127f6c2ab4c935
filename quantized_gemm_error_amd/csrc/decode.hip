// Decode path: y = dequant(W_q) x + sigmoid(w_g . x + b_g) * B (A x) for
// 1 <= M <= 32 tokens in ONE kernel launch.
//
// The pages' decode design fuses the compensator into the epilogue of the
// low-bit product so that no second kernel sits on the critical path (SPEAR
// explanation page, Technical Summary 2.2 A, decode phase).  On gfx950 the
// launch holds two kinds of workgroup:
//
//  * producers (workgroups 0 .. producers-1, which the dispatcher starts
//    first) compute 16-row blocks of [A; w_g] x over one K-split each with
//    MFMA and publish the partial sums to the workspace.  A producer never
//    waits on anything; a consumer's wait is bounded (kSpinLimit) and sets
//    a flag in the workspace if it ever expires;
//  * consumers each own 16 output rows.  Eight waves take interleaved
//    128-wide K blocks; each keeps kDepth 16-byte pieces of its rows' packed
//    nibbles in flight, dequantizes them exactly in registers (dequant_word)
//    and feeds 16x16x32 MFMAs whose other operand is the activation, staged
//    in LDS in the matching order: all of x at once when it fits, else in
//    chunks.  After its last block a wave waits for the producers, forms
//    u = g * (A x) for its tokens and adds u B^T with fp32 16x16x4 MFMAs; the
//    eight waves' sums are reduced in a fixed order and y is rounded once.
//
// Partial sums travel through agent-scope atomic stores and, on the consumer
// side, 16-byte buffer loads with the sc1 cache policy (the same access that
// a relaxed agent-scope atomic load makes), which are coherent across the
// XCDs' separate L2 caches on their own, so no wave needs a cache-wide
// invalidate or write-back: a producer only waits for its stores to complete
// before it counts itself in.  The K-splits of one element sit next to each
// other, so a consumer gathers them with ks / 4 loads, all in flight at once.
// Those uncached loads cost far more per CU than cached ones, so no gather
// issues a load it does not need.
//
// With more tokens and a long K, every consumer staging all of x dominates
// (workgroups x M K 2 bytes from L2).  From a token threshold on, the launch
// instead splits K across the workgroups of each 128-row output tile
// (consume_split): x is staged once per tile and K-split, and the split that
// completes a tile sums the tile's partials and adds the compensator.
//
// Every loop that touches memory has a compile-time shape, so its loads
// issue back to back and the waits count them exactly.  The last workgroup
// to finish (counted over eight slots, then across the slots) resets the
// workspace counters for the next call.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "internal.h"


namespace spear {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kDepth = 4;                  // K blocks in flight per wave (one straight-line group)
constexpr uint32_t kSpinLimit = 1u << 20;  // bounded wait for the producers
constexpr int kWholeLdsBytes = 132 * 1024; // whole-x staging budget
constexpr int kChunkLdsBytes = 68 * 1024;  // chunked staging budget
constexpr int kMaxLds = 160 * 1024;  // dynamic LDS cap (x, scale table, reduction)

enum { XWHOLE = 0, XCHUNK = 1 };

struct DecodeArgs {
  const uint32_t *qw;
  const uint16_t *scales, *zeros;
  const uint16_t *x;
  uint16_t *y;
  const uint16_t *A, *B, *wg;
  float b_gate;
  int N, K, G, ngroups, M, rank;
  int n_tiles, producers;
  int nb, nbw;     // 128-wide K blocks; block iterations per wave
  int ci, xc;      // chunked staging: iterations and K elements per chunk
  int xstr;        // LDS row stride of the staged activation (halves)
  int xzero;       // column of the 128-wide zero strip in each staged row
  int nbw_pad;     // block iterations rounded up to a multiple of kDepth
  int sz_off;      // byte offset of the scale/zero table in dynamic LDS
  int gmul;        // ceil(2^20 / (G / 128)): kb * gmul >> 20 == kb / (G / 128)
  int ks;          // producer K-splits per 16-row block of [A; w_g] (a multiple of 4)
  int rows;        // rows of [A; w_g]: rank + 1, or rank with the per-rank gate
  // per-rank gate (rg_hidden > 0): u = alpha gamma(t) * t, t = A x
  int rg_hidden;
  const float *rg_W1, *rg_b1, *rg_W2, *rg_b2;
  float rg_alpha;
  int rg_off;      // byte offset of its scratch in dynamic LDS
  int part_bytes;  // bytes of the partial-sum array
  int red_off;     // byte offset of the wave-reduction buffer in dynamic LDS
  WsHeader *hdr;
  float *part;     // [rb_a][16 rows of A'][16 * MB tokens][ks]: a split's sums are contiguous
  // split-K consumers
  int ksp, nbs;    // K-splits per 128-row tile; 128-wide blocks per split
  int ngs;         // scale/zero table groups per row
  int party_bytes;
  float *party;    // partial output tiles (split_piece_off)
};

// Sum of the waves' partial tiles in a fixed order (wave 0's own, then 1..7).
template <int MB>
__device__ __forceinline__ f32x4_t reduce_waves(f32x4_t own, f32x4_t (*red)[MB][64], int mb,
                                                int lane) {
  f32x4_t v = own;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) v = v + red[w][mb][lane];
  return v;
}

// Four consecutive partial sums, read coherently across the XCDs' L2 caches
// (cache policy sc1, as a relaxed agent-scope atomic load has).
__device__ __forceinline__ f32x4_t load_partials4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return bitcast<f32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16));
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

// ---------------------------------------------------------------------------
// Producers: partial [A; w_g] x over one K-split for one 16-row block.
// ---------------------------------------------------------------------------
template <int DT, int MB>
__device__ void produce(const DecodeArgs &a, int p, f32x4_t (*red)[MB][64], int wave, int lane) {
  const int col = lane & 15, h = lane >> 4;
  const int rb = p / a.ks, ksi = p % a.ks;
  const int j = rb * 16 + col;  // row of [A; w_g]
  const bool jin = j < a.rows;
  // j >= rank: w_g, or (per-rank gate, no w_g) any valid row, masked by jin
  const uint16_t *arow = (j < a.rank) ? a.A + (size_t)j * a.K : (a.wg ? a.wg : a.A);
  const int nsteps = a.K / 32;
  const int per = (nsteps + a.ks - 1) / a.ks;
  const int s0 = ksi * per;
  const int s1 = min(nsteps, s0 + per);

  f32x4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  for (int base = s0 + wave; base < s1; base += kWaves * 8) {
    u32x4_t bo[8], ao[MB][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = min(base + kWaves * i, s1 - 1);
      const int k = s * 32 + 8 * h;
      bo[i] = *(const u32x4_t *)(arow + k);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = min(col + 16 * mb, a.M - 1);
        ao[mb][i] = *(const u32x4_t *)(a.x + (size_t)m * a.K + k);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (base + kWaves * i < s1) {
        const u32x4_t b = jin ? bo[i] : zero;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4_t av = (col + 16 * mb < a.M) ? ao[mb][i] : zero;
          acc[mb] = mfma_16x16x32<DT>(av, b, acc[mb]);
        }
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t *dst = (uint32_t *)a.part + ((size_t)(rb * 16 + col) * (16 * MB)) * a.ks + ksi;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4_t v = reduce_waves(acc[mb], red, mb, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __hip_atomic_store(&dst[(size_t)(16 * mb + 4 * h + e) * a.ks], bitcast<uint32_t>(v[e]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    publish_wait();
    if (lane == 0)
      __hip_atomic_fetch_add(&a.hdr->arrive.v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Bounded wait until every producer has counted itself in.  The partial
// sums are then read with agent-scope atomic loads (load_partial), issued
// after this wait has observed the count.
__device__ void wait_producers(const DecodeArgs &a, int tid) {
  if (tid == 0) {
    uint32_t it = 0;
    while (__hip_atomic_load(&a.hdr->arrive.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           (uint32_t)a.producers) {
      __builtin_amdgcn_s_sleep(1);
      if (++it > kSpinLimit) {
        __hip_atomic_fetch_or(&a.hdr->flags.v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Activation staging into LDS, 8-blocks permuted to match dequant_word.
// Rows m < M only; row stride xstr; zeros past K.
// ---------------------------------------------------------------------------

// All of x (M rows x nb*128 columns), in batches of 8 pieces per thread.
// whole_load issues one batch; whole_store writes it to LDS.
struct XBatch {
  u32x4_t v[8];
};

__device__ __forceinline__ void whole_load(const DecodeArgs &a, XBatch &xb, int p0, int tid) {
  const int per_row = a.nb * 16;  // 8-element pieces per row
  const int total = a.M * per_row;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (p0 + kThreads * i < total) {  // uniform across the workgroup
      const int p = min(p0 + tid + kThreads * i, total - 1);
      const int m = p / per_row, j = p - m * per_row;
      const int k = min(8 * j, a.K - 8);
      xb.v[i] = *(const u32x4_t *)(a.x + (size_t)m * a.K + k);
    }
  }
}

// Zeros in columns [xzero, xzero + 128) of every staged row: blocks past the
// end of K read them, so they add exact zeros.
__device__ __forceinline__ void zero_strip(const DecodeArgs &a, uint16_t *xs, int tid) {
  for (int p = tid; p < a.M * 16; p += kThreads) {
    const int m = p / 16, j = p % 16;
    *(u32x4_t *)(xs + m * a.xstr + a.xzero + 8 * j) = u32x4_t{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void whole_store(const DecodeArgs &a, const XBatch &xb, uint16_t *xs,
                                            int p0, int tid) {
  const int per_row = a.nb * 16;
  const int total = a.M * per_row;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = p0 + tid + kThreads * i;
    if (p0 + kThreads * i < total && p < total) {
      const int m = p / per_row, j = p - m * per_row;
      const u32x4_t val = (8 * j < a.K) ? xb.v[i] : u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t *)(xs + m * a.xstr + 8 * j) = permute_8(val);
    }
  }
}

// The tile's scales and zero-points as two LDS words per (row, group): the
// dequant_word zero constant and the scale as fp32.  The tile's rows are
// consecutive, so their groups form one contiguous range of rows * ngroups
// elements in each array.  Entries [8 p, 8 p + 8) of the range go to thread
// p mod kThreads; sz_load fetches one batch (8 entries per thread) into
// registers and sz_store converts it into LDS, so the first batch can be in
// flight together with the weight loads.
struct SzBatch {
  u16x8_t s, z;
};

__device__ __forceinline__ void sz_load(const DecodeArgs &a, SzBatch &sb, int n0, int rows, int p) {
  const int ng = a.ngroups;
  const size_t base = (size_t)n0 * ng;
  const size_t end = (size_t)a.N * ng;
  const int cnt = rows * ng;
  sb.s = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  sb.z = sb.s;
  if (8 * p >= cnt) return;
  const size_t e0 = base + 8 * (size_t)p;
  if (e0 + 8 <= end && ((uintptr_t)(a.scales + e0) % 16) == 0 &&
      ((uintptr_t)(a.zeros + e0) % 16) == 0) {
    sb.s = *(const u16x8_t *)(a.scales + e0);
    sb.z = *(const u16x8_t *)(a.zeros + e0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (e0 + i < end) {
        sb.s[i] = a.scales[e0 + i];
        sb.z[i] = a.zeros[e0 + i];
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void sz_store(const DecodeArgs &a, const SzBatch &sb, int rows, int p,
                                         uint32_t *szs) {
  const int cnt = rows * a.ngroups;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (8 * p + i < cnt) {
      szs[2 * (8 * p + i)] = zero_constant<DT>(sb.z[i]);
      szs[2 * (8 * p + i) + 1] = bitcast<uint32_t>((float)bitcast<_Float16>(sb.s[i]));
    }
  }
}

constexpr int kChunkPieces = 4;  // staged 16-byte pieces per thread per chunk

struct XChunk {
  u32x4_t v[kChunkPieces];
};

// One chunk (xc columns) of x into registers: at most kChunkPieces per thread.
__device__ __forceinline__ void chunk_load(const DecodeArgs &a, XChunk &c, int chunk, int tid) {
  const int per_row = a.xc / 8;
  const int k0 = chunk * a.xc;
#pragma unroll
  for (int i = 0; i < kChunkPieces; ++i) {
    const int p = tid + kThreads * i;
    const int m = min(p / per_row, a.M - 1);
    const int j = p % per_row;
    const int k = min(k0 + 8 * j, a.K - 8);
    c.v[i] = *(const u32x4_t *)(a.x + (size_t)m * a.K + k);
  }
}

__device__ __forceinline__ void chunk_store(const DecodeArgs &a, const XChunk &c, uint16_t *xs,
                                            int chunk, int tid) {
  const int per_row = a.xc / 8;
  const int k0 = chunk * a.xc;
#pragma unroll
  for (int i = 0; i < kChunkPieces; ++i) {
    const int p = tid + kThreads * i;
    const int m = p / per_row, j = p % per_row;
    if (m < a.M) {
      const u32x4_t val = (k0 + 8 * j < a.K) ? c.v[i] : u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t *)(xs + m * a.xstr + 8 * j) = permute_8(val);
    }
  }
}

// ---------------------------------------------------------------------------
// The pages' per-rank gate in a consumer's epilogue, after the producers are
// in: the workgroup gathers t = A x for every token (the sum of each
// element's K-split partials, in split order), computes
// hidden = relu(W1 t + b1), gamma = sigmoid(W2 hidden + b2) and
// u = alpha gamma * t in LDS, and each wave adds u B^T for its rank steps.
// ---------------------------------------------------------------------------
template <int DT, int MB, int KG>
__device__ void rank_gate_epilogue(const DecodeArgs &a, uint16_t *xs, f32x4_t (&acc)[MB], int row,
                                   int wk, int tid) {
  const int lane = tid & 63, col = lane & 15, h = lane >> 4;
  const int PS = 16 * MB;
  const int rs = a.rank + 1, hs = a.rg_hidden + 1;
  float *tl = (float *)((char *)xs + a.rg_off);  // [16 MB][rs]
  float *hl = tl + PS * rs;                       // [16 MB][hs]
  // each element's ks <= 16 partials are contiguous: up to four 16-byte
  // loads, all issued before the sum, which runs in split order
  const __amdgpu_buffer_rsrc_t pr =
      __builtin_amdgcn_make_buffer_rsrc(a.part, (short)0, a.part_bytes, 0x00020000);
  const int kq = a.ks / 4;
  for (int i = tid; i < a.M * a.rank; i += kThreads) {
    const int m = i / a.rank, j = i - m * a.rank;
    f32x4_t v[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      v[qq] = load_partials4(pr, ((j * PS + m) * a.ks + 4 * min(qq, kq - 1)) * 4);
    float t = 0.f;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      if (qq < kq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) t += v[qq][e];
      }
    tl[m * rs + j] = t;
  }
  __syncthreads();
  for (int i = tid; i < a.M * a.rg_hidden; i += kThreads) {
    const int m = i / a.rg_hidden, c = i - m * a.rg_hidden;
    float v = a.rg_b1[c];
    for (int k = 0; k < a.rank; ++k) v += a.rg_W1[(size_t)c * a.rank + k] * tl[m * rs + k];
    hl[m * hs + c] = v > 0.f ? v : 0.f;
  }
  __syncthreads();
  for (int i = tid; i < a.M * a.rank; i += kThreads) {
    const int m = i / a.rank, j = i - m * a.rank;
    float v = a.rg_b2[j];
    for (int c = 0; c < a.rg_hidden; ++c) v += a.rg_W2[(size_t)j * a.rg_hidden + c] * hl[m * hs + c];
    tl[m * rs + j] *= a.rg_alpha * gate_sigmoid(v);
  }
  __syncthreads();
  const int nst = (a.rank + 3) / 4;
  for (int st = wk; st < nst; st += KG) {
    const int j = 4 * st + h;
    const bool jin = j < a.rank;
    const float bval = jin ? to_f32<DT>(a.B[(size_t)row * a.rank + j]) : 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = col + 16 * mb;
      acc[mb] = mfma_16x16x4_f32((jin && m < a.M) ? tl[m * rs + j] : 0.f, bval, acc[mb]);
    }
  }
}

// The compensator in a consumer's epilogue, after its main loop: wait for
// the producers, then add u B^T for the wave's rows, u = g * (A x) with the
// scalar gate (or the per-rank gate's u).  Each of a row-block's KG waves
// takes every KG-th rank step, starting at wk.
template <int DT, int MB, int KG>
__device__ void ec_epilogue(const DecodeArgs &a, uint16_t *xs, f32x4_t (&acc)[MB], int row, int wk,
                            int tid) {
  const int lane = tid & 63, col = lane & 15, h = lane >> 4;
  // element (j, m) of [A; w_g] x is the sum of its ks partials at
  // ((j * 16 MB + m) * ks + [0, ks)) in the partial array
  const int PS = 16 * MB;
  const int nst = (a.rank + 3) / 4;  // rank steps of four; this wave takes st = wk + KG i
  // B for the wave's first rank step does not depend on the producers
  float b_first = 0.f;
  if (wk < nst) b_first = to_f32<DT>(a.B[(size_t)row * a.rank + min(4 * wk + h, a.rank - 1)]);
  wait_producers(a, tid);
  if (a.rg_hidden > 0) {
    rank_gate_epilogue<DT, MB, KG>(a, xs, acc, row, wk, tid);
  } else {
  const __amdgpu_buffer_rsrc_t pr =
      __builtin_amdgcn_make_buffer_rsrc(a.part, (short)0, a.part_bytes, 0x00020000);
  const int kq = a.ks / 4;
  float g[MB];
  // one rank step; the first also gathers the gate row j = rank, with its
  // loads in flight together with the step's own
  auto step = [&](int st, float bval, auto gate_tag) {
    constexpr bool kGate = decltype(gate_tag)::value;
    const int j = min(4 * st + h, a.rank - 1);
    float t[MB], z[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) t[mb] = z[mb] = 0.f;
    for (int q0 = 0; q0 < kq; q0 += 2) {
      f32x4_t tv[MB][2], zv[MB][2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          // uncached loads are costly per CU: none past the element's ks partials, and
          // the gate row only in the h == 0 lanes (shared with the others below)
          const int q = q0 + qq;
          tv[mb][qq] = zv[mb][qq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (q < kq) {
            tv[mb][qq] = load_partials4(pr, (((j * PS + col + 16 * mb) * a.ks) + 4 * q) * 4);
            if (kGate && h == 0)
              zv[mb][qq] = load_partials4(pr, (((a.rank * PS + col + 16 * mb) * a.ks) + 4 * q) * 4);
          }
        }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          if (q0 + qq < kq) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              t[mb] += tv[mb][qq][e];
              if constexpr (kGate) z[mb] += zv[mb][qq][e];
            }
          }
        }
    }
    if constexpr (kGate) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) g[mb] = gate_sigmoid(__shfl(z[mb], col) + a.b_gate);
    }
    const bool jin = 4 * st + h < a.rank;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const float u = (jin && col + 16 * mb < a.M) ? g[mb] * t[mb] : 0.f;
      acc[mb] = mfma_16x16x4_f32(u, jin ? bval : 0.f, acc[mb]);
    }
  };
  if (wk < nst) {
    step(wk, b_first, std::true_type{});
    for (int st = wk + KG; st < nst; st += KG)
      step(st, to_f32<DT>(a.B[(size_t)row * a.rank + min(4 * st + h, a.rank - 1)]),
           std::false_type{});
  }
  }  // scalar gate
}

// ---------------------------------------------------------------------------
// Consumers: 16 * WR output rows, full K.  The eight waves form WR row-blocks
// of KG = 8 / WR waves; the KG waves of a row-block take interleaved K blocks
// and all waves share the staged activation.
// ---------------------------------------------------------------------------
template <int DT, int MB, bool EC, bool PERCH, int XMODE, int WR>
__device__ void consume(const DecodeArgs &a, int tile, uint16_t *xs, f32x4_t (*red)[MB][64],
                        int tid) {
  constexpr int KG = kWaves / WR;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar indices
  const int lane = tid & 63, col = lane & 15, h = lane >> 4;
  const int wr = wave / KG, wk = wave % KG;
  const int n0 = tile * 16 * WR;
  const int n = n0 + 16 * wr + col;
  const int row = min(n, a.N - 1);
  const uint32_t *wrow = a.qw + (size_t)row * (a.K / 8);
  const int nb = a.nb, nbw = a.nbw;

  uint32_t zc_row = 0;
  float s_row = 0.f;
  if constexpr (PERCH) {
    zc_row = zero_constant<DT>(a.zeros[row]);
    s_row = (float)bitcast<_Float16>(a.scales[row]);
  }

  // piece of block iteration b: block kb = KG b + wk (clamped), words [4h, 4h + 4)
  u32x4_t wr_ring[kDepth];
  auto wload = [&](int b, u32x4_t &w) {
    const int kb = min(b * KG + wk, nb - 1);
    const int off = (kb * 128 + 32 * h < a.K) ? kb * 16 + 4 * h : 0;
    // read once per call: non-temporal, so the stream does not displace the
    // layer's small operands from the caches
    w = __builtin_nontemporal_load((const u32x4_t *)(wrow + off));
  };

  // activation loads first, then the weight ring, so that storing the
  // activation to LDS waits only for its own loads
  uint32_t *szs = (uint32_t *)((char *)xs + a.sz_off);
  XChunk xc;
  XBatch xb;
  SzBatch sb;
  if constexpr (XMODE == XWHOLE) {
    whole_load(a, xb, 0, tid);
  } else {
    chunk_load(a, xc, 0, tid);
  }
  if constexpr (!PERCH) sz_load(a, sb, n0, 16 * WR, tid);
  // the weight ring is issued last: the LDS stores below wait only for the
  // loads issued before it, and each block of the first group waits only
  // for its own piece
#pragma unroll
  for (int i = 0; i < kDepth; ++i) wload(i, wr_ring[i]);
  if constexpr (!PERCH) {
    sz_store<DT>(a, sb, 16 * WR, tid, szs);
    for (int p = tid + kThreads; 8 * p < 16 * WR * a.ngroups; p += kThreads) {
      sz_load(a, sb, n0, 16 * WR, p);
      sz_store<DT>(a, sb, 16 * WR, p, szs);
    }
  }
  zero_strip(a, xs, tid);
  if constexpr (XMODE == XWHOLE) {
    whole_store(a, xb, xs, 0, tid);
    const int total = a.M * a.nb * 16;
    for (int p0 = kThreads * 8; p0 < total; p0 += kThreads * 8) {
      whole_load(a, xb, p0, tid);
      whole_store(a, xb, xs, p0, tid);
    }
  }
  __syncthreads();

  f32x4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int szrow = 2 * (16 * wr + col) * a.ngroups;
  // A-operand rows past M read row M - 1: MFMA output rows depend only on
  // their own A rows, and rows >= M are never stored
  int xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xrow[mb] = min(col + 16 * mb, a.M - 1) * a.xstr;

  // groups of kDepth blocks per wave, straight-line: blocks past the end of K
  // read the zero strip and clamped weights.  Every group but the last refills
  // the ring; the two kinds are separate compile-time copies, so a group has
  // no branch and its loads, LDS reads and MFMAs can interleave.
  auto group = [&](int b0, auto refill_tag) {
    constexpr bool kRefill = decltype(refill_tag)::value;
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int b = b0 + i;
      int kbase = 0;  // first K column of the staged activation
      if constexpr (XMODE == XCHUNK) {
        const int chunk = b / a.ci;
        kbase = chunk * a.xc;
        if (b % a.ci == 0) {
          __syncthreads();
          chunk_store(a, xc, xs, chunk, tid);
          __syncthreads();
          if ((chunk + 1) * a.xc < a.K) chunk_load(a, xc, chunk + 1, tid);
        }
      }
      const u32x4_t w = wr_ring[i];
      if constexpr (kRefill) wload(b + kDepth, wr_ring[i]);
      const int kb = b * KG + wk;
      const bool live = kb < nb;
      uint32_t zc = zc_row;
      float sc = 1.f;
      if constexpr (!PERCH) {
        // group of block kb: kb / (G / 128) as an exact multiply-shift
        const int g = (int)(((uint32_t)min(kb, nb - 1) * a.gmul) >> 20);
        zc = szs[szrow + 2 * g];
        sc = bitcast<float>(szs[szrow + 2 * g + 1]);
      }
      const int kloc = (live ? kb * 128 - kbase : a.xzero) + 32 * h;
      u32x4_t bop[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) bop[t] = dequant_word<DT>(w[t], zc);
      f32x4_t accg[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        u32x4_t aop[4];
        const uint16_t *xp = xs + xrow[mb] + kloc;
#pragma unroll
        for (int t = 0; t < 4; ++t) aop[t] = *(const u32x4_t *)(xp + 8 * t);
        if constexpr (PERCH) {
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[mb] = mfma_16x16x32<DT>(aop[t], bop[t], acc[mb]);
        } else {
          // two independent chains of two, then one add
          const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
          f32x4_t c0 = mfma_16x16x32<DT>(aop[0], bop[0], z4);
          f32x4_t c1 = mfma_16x16x32<DT>(aop[2], bop[2], z4);
          c0 = mfma_16x16x32<DT>(aop[1], bop[1], c0);
          c1 = mfma_16x16x32<DT>(aop[3], bop[3], c1);
          accg[mb] = c0 + c1;
        }
      }
      if constexpr (!PERCH) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] += sc * accg[mb];
      }
    }
  };
  const int last = a.nbw_pad - kDepth;
  for (int b0 = 0; b0 < last; b0 += kDepth) group(b0, std::true_type{});
  group(last, std::false_type{});

  if constexpr (PERCH) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] *= s_row;
  }

  if constexpr (EC) ec_epilogue<DT, MB, KG>(a, xs, acc, row, wk, tid);

  // fixed-order sum over the row-block's KG waves
  if (wk > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  }
  __syncthreads();
  if (wk == 0 && n < a.N) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t v = acc[mb];
#pragma unroll
      for (int w = 1; w < KG; ++w) v = v + red[wave + w][mb][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mb + 4 * h + e;
        if (m < a.M) a.y[(size_t)m * a.N + n] = from_f32<DT>(v[e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K consumers (ksp > 1).  Consumer c takes output tile c / ksp (128
// rows: one 16-row block per wave) and K-split c % ksp (nbs consecutive
// 128-wide blocks).  x is staged once per workgroup for its split only, so a
// call stages M K 2 bytes per tile instead of per 16 rows.  Each wave runs its
// rows over the split and stores its fp32 partial tile; the workgroup that
// completes a tile (its arrival counter reaches ksp) sums the tile's ksp
// partials in split order, adds the compensator and rounds y once.
// ---------------------------------------------------------------------------

// Byte offset of wave w's partial for 16-token block mb, split q, tile t:
// [ksp][tiles][8 waves][MB][64 lanes] 16-byte pieces.
template <int MB>
__device__ __forceinline__ int split_piece_off(const DecodeArgs &a, int q, int t, int w, int mb,
                                               int lane) {
  return ((((q * a.n_tiles + t) * kWaves + w) * MB + mb) * 64 + lane) * 16;
}

// The compensator of a completed tile: the workgroup gathers [A; w_g] x for
// every token into LDS (each element the sum of its ks producer partials in
// split order), forms u (the scalar gate's g t, or the per-rank gate's
// alpha gamma(t) t) and each wave adds u B^T for its 16 rows.
template <int DT, int MB>
__device__ void split_ec_epilogue(const DecodeArgs &a, uint16_t *xs, f32x4_t (&acc)[MB], int row,
                                  int tid) {
  const int lane = tid & 63, col = lane & 15, h = lane >> 4;
  const int PS = 16 * MB;
  const int rows = a.rows;             // rank (+ the gate row with the scalar gate)
  const int rs = a.rank + 1, hs = a.rg_hidden + 1;
  float *tl = (float *)((char *)xs + a.rg_off);  // [16 MB][rs]
  float *hl = tl + PS * rs;                       // [16 MB][hs] (per-rank gate)
  const int nst = (a.rank + 3) / 4;
  // B for the first eight rank steps does not depend on the producers
  float bv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = min(4 * min(i, nst - 1) + h, a.rank - 1);
    bv[i] = to_f32<DT>(a.B[(size_t)row * a.rank + j]);
  }
  wait_producers(a, tid);
  const __amdgpu_buffer_rsrc_t pr =
      __builtin_amdgcn_make_buffer_rsrc(a.part, (short)0, a.part_bytes, 0x00020000);
  const int kq = a.ks / 4;
  const int E = a.M * rows;
  // four elements per thread per round, their (up to 4 x 4) loads in flight together
  for (int e0 = 0; e0 < E; e0 += 4 * kThreads) {
    f32x4_t v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + tid + kThreads * u;
      const int m = e / rows, j = e - m * rows;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        v[u][qq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (e < E && qq < kq) v[u][qq] = load_partials4(pr, ((j * PS + m) * a.ks + 4 * qq) * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + tid + kThreads * u;
      if (e < E) {
        const int m = e / rows, j = e - m * rows;
        float t = 0.f;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (qq < kq) {
#pragma unroll
            for (int i = 0; i < 4; ++i) t += v[u][qq][i];
          }
        tl[m * rs + j] = t;
      }
    }
  }
  __syncthreads();
  if (a.rg_hidden > 0) {
    for (int i = tid; i < a.M * a.rg_hidden; i += kThreads) {
      const int m = i / a.rg_hidden, c = i - m * a.rg_hidden;
      float v = a.rg_b1[c];
      for (int k = 0; k < a.rank; ++k) v += a.rg_W1[(size_t)c * a.rank + k] * tl[m * rs + k];
      hl[m * hs + c] = v > 0.f ? v : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < a.M * a.rank; i += kThreads) {
      const int m = i / a.rank, j = i - m * a.rank;
      float v = a.rg_b2[j];
      for (int c = 0; c < a.rg_hidden; ++c) v += a.rg_W2[(size_t)j * a.rg_hidden + c] * hl[m * hs + c];
      tl[m * rs + j] *= a.rg_alpha * gate_sigmoid(v);
    }
  } else {
    // g from the gate row (column rank), which this pass does not overwrite
    for (int i = tid; i < a.M * a.rank; i += kThreads) {
      const int m = i / a.rank, j = i - m * a.rank;
      tl[m * rs + j] *= gate_sigmoid(tl[m * rs + a.rank] + a.b_gate);
    }
  }
  __syncthreads();
  for (int st0 = 0; st0 < nst; st0 += 8) {
    if (st0 > 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = min(4 * min(st0 + i, nst - 1) + h, a.rank - 1);
        bv[i] = to_f32<DT>(a.B[(size_t)row * a.rank + j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 4 * (st0 + i) + h;
      if (st0 + i < nst) {
        const bool jin = j < a.rank;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = col + 16 * mb;
          acc[mb] = mfma_16x16x4_f32((jin && m < a.M) ? tl[m * rs + j] : 0.f, jin ? bv[i] : 0.f,
                                     acc[mb]);
        }
      }
    }
  }
}

template <int DT, int MB, bool EC, bool PERCH>
__device__ void consume_split(const DecodeArgs &a, int c, uint16_t *xs, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 15, h = lane >> 4;
  const int q = c % a.ksp, tile = c / a.ksp;
  const int n0 = tile * 16 * kWaves;
  const int n = n0 + 16 * wave + col;
  const int row = min(n, a.N - 1);
  const uint32_t *wrow = a.qw + (size_t)row * (a.K / 8);
  const int kb0 = q * a.nbs;                // the plan leaves no split empty
  const int kb1 = min(a.nb, kb0 + a.nbs);
  const int kx0 = kb0 * 128;                // first staged K column

  uint32_t zc_row = 0;
  float s_row = 0.f;
  if constexpr (PERCH) {
    zc_row = zero_constant<DT>(a.zeros[row]);
    s_row = (float)bitcast<_Float16>(a.scales[row]);
  }

  u32x4_t wr_ring[kDepth];
  auto wload = [&](int b, u32x4_t &w) {
    const int kb = min(kb0 + b, kb1 - 1);
    const int off = (kb * 128 + 32 * h < a.K) ? kb * 16 + 4 * h : 0;
    w = __builtin_nontemporal_load((const u32x4_t *)(wrow + off));
  };

  // x columns [kx0, kx0 + nbs 128) of every token, in batches of 8 pieces per
  // thread; columns past K are staged as zeros
  const int per_row = a.nbs * 16;
  const int total = a.M * per_row;
  XBatch xb;
  auto xload = [&](int p0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = min(p0 + tid + kThreads * i, total - 1);
      const int m = p / per_row, j = p - m * per_row;
      const int k = min(kx0 + 8 * j, a.K - 8);
      xb.v[i] = *(const u32x4_t *)(a.x + (size_t)m * a.K + k);
    }
  };
  auto xstore = [&](int p0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = p0 + tid + kThreads * i;
      if (p < total) {
        const int m = p / per_row, j = p - m * per_row;
        const u32x4_t val = (kx0 + 8 * j < a.K) ? xb.v[i] : u32x4_t{0u, 0u, 0u, 0u};
        *(u32x4_t *)(xs + m * a.xstr + 8 * j) = permute_8(val);
      }
    }
  };

  // scale/zero table of the split's groups g0 .. g0 + ngs - 1 for the tile's
  // 128 rows: entry (r, gi) at 2 (r ngs + gi); at most 4 entries per thread
  // (the plan checks 128 ngs <= 4 kThreads)
  uint32_t *szs = (uint32_t *)((char *)xs + a.sz_off);
  const int gpb = a.G / 128;  // 128-wide blocks per group (G a multiple of 128 here)
  const int g0 = kb0 / gpb;
  uint16_t sv[4], zv[4];
  if constexpr (!PERCH) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + kThreads * u;
      const int r = e / a.ngs, gi = e - r * a.ngs;
      const int nr = min(n0 + r, a.N - 1), g = min(g0 + gi, a.ngroups - 1);
      sv[u] = a.scales[(size_t)nr * a.ngroups + g];
      zv[u] = a.zeros[(size_t)nr * a.ngroups + g];
    }
  }
  xload(0);
#pragma unroll
  for (int i = 0; i < kDepth; ++i) wload(i, wr_ring[i]);
  if constexpr (!PERCH) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + kThreads * u;
      if (e < 16 * kWaves * a.ngs) {
        szs[2 * e] = zero_constant<DT>(zv[u]);
        szs[2 * e + 1] = bitcast<uint32_t>((float)bitcast<_Float16>(sv[u]));
      }
    }
  }
  zero_strip(a, xs, tid);
  xstore(0);
  for (int p0 = kThreads * 8; p0 < total; p0 += kThreads * 8) {
    xload(p0);
    xstore(p0);
  }
  __syncthreads();

  f32x4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int szrow = 2 * (16 * wave + col) * a.ngs;
  int xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xrow[mb] = min(col + 16 * mb, a.M - 1) * a.xstr;

  auto group = [&](int b0, auto refill_tag) {
    constexpr bool kRefill = decltype(refill_tag)::value;
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int b = b0 + i;
      const u32x4_t w = wr_ring[i];
      if constexpr (kRefill) wload(b + kDepth, wr_ring[i]);
      const int kb = kb0 + b;
      const bool live = kb < kb1;
      uint32_t zc = zc_row;
      float sc = 1.f;
      if constexpr (!PERCH) {
        const int g = (int)(((uint32_t)min(kb, kb1 - 1) * a.gmul) >> 20) - g0;
        zc = szs[szrow + 2 * g];
        sc = bitcast<float>(szs[szrow + 2 * g + 1]);
      }
      const int kloc = (live ? b * 128 : a.xzero) + 32 * h;
      u32x4_t bop[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) bop[t] = dequant_word<DT>(w[t], zc);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        u32x4_t aop[4];
        const uint16_t *xp = xs + xrow[mb] + kloc;
#pragma unroll
        for (int t = 0; t < 4; ++t) aop[t] = *(const u32x4_t *)(xp + 8 * t);
        if constexpr (PERCH) {
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[mb] = mfma_16x16x32<DT>(aop[t], bop[t], acc[mb]);
        } else {
          const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
          f32x4_t c0 = mfma_16x16x32<DT>(aop[0], bop[0], z4);
          f32x4_t c1 = mfma_16x16x32<DT>(aop[2], bop[2], z4);
          c0 = mfma_16x16x32<DT>(aop[1], bop[1], c0);
          c1 = mfma_16x16x32<DT>(aop[3], bop[3], c1);
          acc[mb] += sc * (c0 + c1);
        }
      }
    }
  };
  const int last = a.nbw_pad - kDepth;
  for (int b0 = 0; b0 < last; b0 += kDepth) group(b0, std::true_type{});
  group(last, std::false_type{});

  if constexpr (PERCH) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] *= s_row;
  }

  // publish this split's partial tile, then count it in
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc(a.party, (short)0, a.party_bytes, 0x00020000);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    __builtin_amdgcn_raw_buffer_store_b128(bitcast<u32x4_t>(acc[mb]), yr,
                                           split_piece_off<MB>(a, q, tile, wave, mb, lane), 0, 16);
  publish_wait();
  int *last_flag = (int *)((char *)xs + a.red_off);
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.hdr->tile[tile].v, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *last_flag = (old + 1 == (uint32_t)a.ksp) ? 1 : 0;
  }
  __syncthreads();
  if (*last_flag == 0) return;  // uniform: another split completes this tile

  // the tile's sum over its splits, in split order (this split's own from registers)
  f32x4_t v[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) v[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < a.ksp; q0 += 8) {
    f32x4_t pv[MB][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        pv[mb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // the tile's other splits only, no duplicates: uncached loads are costly per CU
        if (q0 + i < a.ksp && q0 + i != q)
          pv[mb][i] = load_partials4(yr, split_piece_off<MB>(a, q0 + i, tile, wave, mb, lane));
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (q0 + i < a.ksp) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) v[mb] += (q0 + i == q) ? acc[mb] : pv[mb][i];
      }
  }
  if constexpr (EC) split_ec_epilogue<DT, MB>(a, xs, v, row, tid);
  if (n < a.N) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mb + 4 * h + e;
        if (m < a.M) a.y[(size_t)m * a.N + n] = from_f32<DT>(v[mb][e]);
      }
  }
  if (tid == 0)
    __hip_atomic_store(&a.hdr->tile[tile].v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count this workgroup out; the last one resets the counters.  Workgroup b
// counts into slot b % 8; the workgroup that completes a slot counts the
// slot into the top counter, and the one that completes the top counter is
// last overall.
__device__ void finish(const DecodeArgs &a) {
  const uint32_t g = gridDim.x, b = blockIdx.x, slot = b % 8;
  const uint32_t in_slot = (g - 1 - slot) / 8 + 1;  // workgroups counted in this slot
  const uint32_t old = __hip_atomic_fetch_add(&a.hdr->done[slot].v, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1 != in_slot) return;
  const uint32_t slots = g < 8 ? g : 8;
  const uint32_t top = __hip_atomic_fetch_add(&a.hdr->done_top.v, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  if (top + 1 != slots) return;
  __hip_atomic_store(&a.hdr->arrive.v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&a.hdr->done_top.v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = 0; i < 8; ++i)
    __hip_atomic_store(&a.hdr->done[i].v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int MB, bool EC, bool PERCH, int XMODE, int WR>
__global__ __launch_bounds__(kThreads, XMODE == XWHOLE ? 4 : 2) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint16_t xs[];
  f32x4_t(*red)[MB][64] = (f32x4_t(*)[MB][64])((char *)xs + a.red_off);

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if constexpr (EC) {
    if (b < a.producers) {
      produce<DT, MB>(a, b, red, tid >> 6, tid & 63);
    } else {
      consume<DT, MB, EC, PERCH, XMODE, WR>(a, b - a.producers, xs, red, tid);
    }
    if (tid == 0) finish(a);
  } else {
    consume<DT, MB, EC, PERCH, XMODE, WR>(a, b, xs, red, tid);
  }
}

template <int DT, int MB, bool EC, bool PERCH>
__global__ __launch_bounds__(kThreads, 4) void decode_split_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint16_t xs[];
  f32x4_t(*red)[MB][64] = (f32x4_t(*)[MB][64])((char *)xs + a.red_off);
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if constexpr (EC) {
    if (b < a.producers) {
      produce<DT, MB>(a, b, red, tid >> 6, tid & 63);
    } else {
      consume_split<DT, MB, EC, PERCH>(a, b - a.producers, xs, tid);
    }
    if (tid == 0) finish(a);
  } else {
    consume_split<DT, MB, EC, PERCH>(a, b, xs, tid);
  }
}

template <int DT, int MB, bool EC, bool PERCH>
hipError_t launch_split_t(const DecodeArgs &a, int grid, size_t lds, hipStream_t s) {
  auto kern = decode_split_kernel<DT, MB, EC, PERCH>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   kMaxLds);
  });
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_split(const DecodeArgs &a, const DecodePlan &p, bool ec, bool perch,
                        hipStream_t s) {
  const int grid = p.n_tiles * p.ksp + p.producers;
  if (p.mb == 1) {
    if (ec) return perch ? launch_split_t<DT, 1, true, true>(a, grid, p.lds, s)
                         : launch_split_t<DT, 1, true, false>(a, grid, p.lds, s);
    return perch ? launch_split_t<DT, 1, false, true>(a, grid, p.lds, s)
                 : launch_split_t<DT, 1, false, false>(a, grid, p.lds, s);
  }
  if (ec) return perch ? launch_split_t<DT, 2, true, true>(a, grid, p.lds, s)
                       : launch_split_t<DT, 2, true, false>(a, grid, p.lds, s);
  return perch ? launch_split_t<DT, 2, false, true>(a, grid, p.lds, s)
               : launch_split_t<DT, 2, false, false>(a, grid, p.lds, s);
}

template <int DT, int MB, bool EC, bool PERCH, int XMODE, int WR>
hipError_t launch_t(const DecodeArgs &a, int grid, size_t lds, hipStream_t s) {
  auto kern = decode_kernel<DT, MB, EC, PERCH, XMODE, WR>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   kMaxLds);
  });
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int DT, int MB, bool EC, bool PERCH, int XMODE>
hipError_t launch_wr(const DecodeArgs &a, int wr, int grid, size_t lds, hipStream_t s) {
  switch (wr) {
    case 1: return launch_t<DT, MB, EC, PERCH, XMODE, 1>(a, grid, lds, s);
    case 2: return launch_t<DT, MB, EC, PERCH, XMODE, 2>(a, grid, lds, s);
    case 4: return launch_t<DT, MB, EC, PERCH, XMODE, 4>(a, grid, lds, s);
    default: return launch_t<DT, MB, EC, PERCH, XMODE, 8>(a, grid, lds, s);
  }
}

template <int DT, int MB, bool EC, bool PERCH>
hipError_t launch_x(const DecodeArgs &a, const DecodePlan &p, hipStream_t s) {
  const int grid = p.n_tiles + p.producers;
  return p.xmode == XWHOLE ? launch_wr<DT, MB, EC, PERCH, XWHOLE>(a, p.wr, grid, p.lds, s)
                           : launch_wr<DT, MB, EC, PERCH, XCHUNK>(a, p.wr, grid, p.lds, s);
}

template <int DT, int MB, bool EC>
hipError_t launch_pc(const DecodeArgs &a, const DecodePlan &p, bool perch, hipStream_t s) {
  return perch ? launch_x<DT, MB, EC, true>(a, p, s) : launch_x<DT, MB, EC, false>(a, p, s);
}

template <int DT, int MB>
hipError_t launch_ec(const DecodeArgs &a, const DecodePlan &p, bool ec, bool perch,
                     hipStream_t s) {
  return ec ? launch_pc<DT, MB, true>(a, p, perch, s) : launch_pc<DT, MB, false>(a, p, perch, s);
}

template <int DT>
hipError_t launch_mb(const DecodeArgs &a, const DecodePlan &p, bool ec, bool perch,
                     hipStream_t s) {
  return p.mb == 1 ? launch_ec<DT, 1>(a, p, ec, perch, s) : launch_ec<DT, 2>(a, p, ec, perch, s);
}

}  // namespace

// K-splits of the compensator producers: enough that every producer wave
// covers its split in one pass of eight 32-wide steps (8 waves x 8 steps =
// 2048 columns per split), rounded up to a multiple of 4 so that the
// consumers read whole 16-byte groups of partials; at least 4, at most 16.
static int decode_ksplit(int K) {
  const int need = (K / 32 + 63) / 64;
  const int ks = (need + 3) / 4 * 4;
  return ks < 4 ? 4 : (ks > 16 ? 16 : ks);
}

// Residency estimate: workgroups of 8 waves per CU that the LDS and the
// register budget of each staging mode allow.
static int resident_per_cu(const DecodePlan &p) {
  const int by_lds = (int)((160 * 1024) / p.lds);
  const int by_vgpr = p.xmode == XWHOLE ? 2 : 1;  // 8-wave workgroups at 4 (whole) or 2 waves per SIMD
  const int r = by_lds < by_vgpr ? by_lds : by_vgpr;
  return r < 1 ? 1 : r;
}

// One candidate launch shape with wr row-blocks per workgroup; ok == false
// when it cannot fit the LDS or the staging limits.
static DecodePlan plan_for(const LayerDesc &L, int M, int wr) {
  DecodePlan p{};
  p.mb = M <= 16 ? 1 : 2;
  p.rb_a = L.rank > 0 ? (L.rank + L.gate_rows() + 15) / 16 : 0;
  p.ks = L.rank > 0 ? decode_ksplit(L.K) : 0;
  p.producers = p.rb_a * p.ks;
  p.nb = (L.K + 127) / 128;
  p.wr = wr;
  const int kg = kWaves / wr;
  p.nbw = (p.nb + kg - 1) / kg;
  const int kr = p.nb * 128;
  const size_t whole = (size_t)M * (kr + 136) * 2;
  const size_t sz_bytes = L.per_channel ? 0 : (size_t)16 * wr * L.ngroups * 8 + 16;
  const size_t red_bytes = (size_t)kWaves * p.mb * 64 * 16 + 16;
  if (whole <= (size_t)kWholeLdsBytes && whole + sz_bytes + red_bytes <= (size_t)kMaxLds) {
    p.xmode = XWHOLE;
    p.ci = 1 << 30;
    p.xc = kr;
  } else {
    // chunk of ci block iterations = 128 * kg * ci columns; each thread stages
    // at most kChunkPieces 16-byte pieces: M * 128 * kg * ci / 8 <= kChunkPieces * kThreads
    auto fits = [&](int ci) {
      return (size_t)M * 16 * kg * ci <= (size_t)kChunkPieces * kThreads &&
             (size_t)M * (128 * kg * ci + 136) * 2 <= (size_t)kChunkLdsBytes;
    };
    if (!fits(1)) {
      p.ok = false;
      return p;
    }
    int ci = 1;
    while (ci * 2 <= p.nbw && fits(ci * 2)) ci *= 2;
    p.xmode = XCHUNK;
    p.ci = ci;
    p.xc = 128 * kg * ci;
  }
  p.xzero = p.xc;
  p.xstr = p.xc + 128 + 8;
  p.nbw_pad = (p.nbw + kDepth - 1) / kDepth * kDepth;
  p.lds = (size_t)M * p.xstr * 2;
  p.sz_off = (int)((p.lds + 15) / 16 * 16);
  if (!L.per_channel) p.lds = p.sz_off + (size_t)16 * wr * L.ngroups * 8;
  p.red_off = (int)((p.lds + 15) / 16 * 16);
  p.lds = p.red_off + (size_t)kWaves * p.mb * 64 * 16;
  if (L.rank > 0 && L.rg_hidden > 0) {  // per-rank gate scratch: t and hidden for 16 mb tokens
    p.rg_off = (int)((p.lds + 15) / 16 * 16);
    p.lds = p.rg_off + (size_t)16 * p.mb * (L.rank + 1 + L.rg_hidden + 1) * sizeof(float);
  }
  p.n_tiles = (L.N + 16 * wr - 1) / (16 * wr);
  p.ok = p.lds <= (size_t)kMaxLds;
  return p;
}

// Row-blocks per workgroup: the fewest that fit and let the whole grid be
// resident at once (16 * wr rows share one staged activation); else the
// largest that fits.
DecodePlan plan_decode(const LayerDesc &L, int M) {
  DecodePlan best{};
  best.ok = false;
  for (int wr = 1; wr <= 8; wr *= 2) {
    const DecodePlan p = plan_for(L, M, wr);
    if (!p.ok) continue;
    best = p;
    if (p.n_tiles + p.producers <= 256 * resident_per_cu(p)) break;
  }
  return best;
}

bool decode_supported(const LayerDesc &L, int M) { return plan_decode(L, M).ok; }

size_t decode_workspace_bytes(const LayerDesc &L, int M) {
  if (L.rank == 0) return 0;
  const DecodePlan p = plan_decode(L, M);
  if (!p.ok) return 0;
  return kWsDataOff + (size_t)p.producers * 16 * (16 * p.mb) * sizeof(float);
}

// Split-K consumers are considered from this many tokens on and for K of at
// least this many columns (process-wide).  Below K = 8192 a split's tail (its
// partial tile stored, the tile's arrival counted, the partials gathered:
// three memory round trips, about 3.5 us on MI355X) is not paid back by the
// shorter K loop (measured at M = 16 and 32 on the 4096-wide projections).
static std::atomic<int> g_split_min_m{16};
static std::atomic<int> g_split_min_k{8192};
void set_decode_split_min_m(int m) { g_split_min_m.store(m); }
int get_decode_split_min_m() { return g_split_min_m.load(); }
void set_decode_split_min_k(int k) { g_split_min_k.store(k); }
int get_decode_split_min_k() { return g_split_min_k.load(); }


// The split-K launch: 128-row tiles (one 16-row block per wave) and the most
// K-splits, at most 8, with which every workgroup (producers included) is
// resident at once.  ok == false when no split of at least 2 fits: too many
// tiles, too little K, or the LDS.
DecodePlan plan_decode_split(const LayerDesc &L, int M) {
  DecodePlan p{};
  p.ok = false;
  p.mb = M <= 16 ? 1 : 2;
  p.rb_a = L.rank > 0 ? (L.rank + L.gate_rows() + 15) / 16 : 0;
  p.ks = L.rank > 0 ? decode_ksplit(L.K) : 0;
  p.producers = p.rb_a * p.ks;
  p.nb = (L.K + 127) / 128;
  p.wr = kWaves;
  p.n_tiles = (L.N + 16 * kWaves - 1) / (16 * kWaves);
  if (p.n_tiles > kMaxSplitTiles || p.nb < 2 || L.K < g_split_min_k.load()) return p;
  const int gpb = L.per_channel ? 1 : L.G / 128;
  for (int want = 8; want >= 2; --want) {
    DecodePlan c = p;
    c.nbs = (c.nb + want - 1) / want;
    c.ksp = (c.nb + c.nbs - 1) / c.nbs;  // every split non-empty
    if (c.ksp < 2) continue;
    c.ngs = L.per_channel ? 0 : (c.nbs - 1) / gpb + 2;
    if (!L.per_channel && 16 * kWaves * c.ngs > 4 * kThreads) continue;
    c.xmode = XWHOLE;
    c.xzero = c.nbs * 128;
    c.xstr = c.xzero + 128 + 8;
    c.nbw = c.nbs;
    c.nbw_pad = (c.nbs + kDepth - 1) / kDepth * kDepth;
    c.lds = (size_t)M * c.xstr * 2;
    c.sz_off = (int)((c.lds + 15) / 16 * 16);
    c.lds = c.sz_off + (size_t)16 * kWaves * c.ngs * 8;
    c.red_off = (int)((c.lds + 15) / 16 * 16);
    c.lds = c.red_off + (size_t)kWaves * c.mb * 64 * 16;
    c.rg_off = (int)((c.lds + 15) / 16 * 16);
    if (L.rank > 0) c.lds = c.rg_off + (size_t)16 * c.mb * (L.rank + 1 + L.rg_hidden + 1) * sizeof(float);
    if (c.lds > (size_t)kMaxLds) continue;
    const int by_lds = (int)((size_t)kMaxLds / c.lds);
    const int resident = by_lds < 2 ? by_lds : 2;  // 8-wave workgroups at 4 waves per SIMD
    if (c.n_tiles * c.ksp + c.producers > 256 * resident) continue;
    const size_t ec_bytes = (size_t)c.producers * 16 * (16 * c.mb) * sizeof(float);
    c.split_off = kWsDataOff + (ec_bytes + 255) / 256 * 256;
    c.split_bytes = (size_t)c.ksp * c.n_tiles * kWaves * c.mb * 64 * 16;
    c.ok = true;
    return c;
  }
  return p;
}

// The split-K launch is taken for M >= the threshold when its plan fits and
// the workspace holds its partial tiles.
static bool use_split(const DecodePlan &sp, int M, size_t ws_bytes) {
  return sp.ok && M >= g_split_min_m.load() && ws_bytes >= sp.split_off + sp.split_bytes;
}

size_t decode_fast_workspace_bytes(const LayerDesc &L, int M) {
  size_t need = decode_workspace_bytes(L, M);
  if (M >= g_split_min_m.load()) {
    const DecodePlan sp = plan_decode_split(L, M);
    if (sp.ok && sp.split_off + sp.split_bytes > need) need = sp.split_off + sp.split_bytes;
  }
  return need;
}

hipError_t launch_decode(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                         void *ws, size_t ws_bytes, hipStream_t s) {
  const DecodePlan sp = plan_decode_split(L, M);
  const bool split = ws && use_split(sp, M, ws_bytes);
  const DecodePlan p = split ? sp : plan_decode(L, M);
  if (!p.ok) return hipErrorInvalidConfiguration;
  DecodeArgs a{};
  a.qw = L.qw;
  a.scales = L.scales;
  a.zeros = L.zeros;
  a.x = x;
  a.y = y;
  a.A = L.A;
  a.B = L.B;
  a.wg = L.wg;
  a.b_gate = L.b_gate;
  a.N = L.N;
  a.K = L.K;
  a.G = L.G;
  a.ngroups = L.ngroups;
  a.M = M;
  a.rank = L.rank;
  a.n_tiles = p.n_tiles;
  a.producers = p.producers;
  a.nb = p.nb;
  a.nbw = p.nbw;
  a.ci = p.ci;
  a.xc = p.xc;
  a.xstr = p.xstr;
  a.xzero = p.xzero;
  a.nbw_pad = p.nbw_pad;
  a.sz_off = p.sz_off;
  // exact for kb * (G / 128) < 2^20, which K <= 131072 guarantees
  a.gmul = L.per_channel ? 0 : (int)(((1u << 20) + (uint32_t)(L.G / 128) - 1) / (uint32_t)(L.G / 128));
  a.red_off = p.red_off;
  a.ks = p.ks;
  a.rows = L.rank + L.gate_rows();
  a.rg_hidden = L.rg_hidden;
  a.rg_W1 = L.rg_W1;
  a.rg_b1 = L.rg_b1;
  a.rg_W2 = L.rg_W2;
  a.rg_b2 = L.rg_b2;
  a.rg_alpha = L.rg_alpha;
  a.rg_off = p.rg_off;
  a.part_bytes = (int)((size_t)p.producers * 16 * (16 * p.mb) * sizeof(float));
  a.hdr = (WsHeader *)ws;
  a.part = ws ? (float *)((char *)ws + kWsDataOff) : nullptr;
  const bool ec = L.rank > 0;
  if (split) {
    a.ksp = p.ksp;
    a.nbs = p.nbs;
    a.ngs = p.ngs;
    a.party_bytes = (int)p.split_bytes;
    a.party = (float *)((char *)ws + p.split_off);
    return dtype == DT_F16 ? launch_split<DT_F16>(a, p, ec, L.per_channel, s)
                           : launch_split<DT_BF16>(a, p, ec, L.per_channel, s);
  }
  return dtype == DT_F16 ? launch_mb<DT_F16>(a, p, ec, L.per_channel, s)
                         : launch_mb<DT_BF16>(a, p, ec, L.per_channel, s);
}

}  // namespace spear
