// Decode for 33..128 tokens ("wide" launch): y = dequant(W_q) x + g(x) B (A x),
// still bound by the weight stream.
//
// The pages fuse the compensator into the memory-bound low-bit product and
// keep a separate compensator kernel for the compute-bound phase (SPEAR
// explanation page, Technical Summary 2.2 A).  Past 32 tokens a layer can
// still be bound by its weight stream: Llama-70B's 8192 x 8192 at 64 tokens
// needs 4.2 us of streaming at 8 TB/s for 3.4 us of dense fp16 MFMA work.
// But with that many tokens the activation x (M K 2 bytes, 1 MiB at 64
// tokens and K = 8192) must be reused across many output rows, which the
// small-M decode kernels (16 to 64 rows per workgroup, each staging all of
// x) do not do, and the K-splits that fill the chip need their partial sums
// reduced.
//
//  * wide_kernel: consumer workgroups of 8 waves own a tile of 128 R output
//    rows (R 16-row blocks per wave) and one of ksp K-splits.  x for the
//    split is streamed through LDS 512 columns at a time while each wave
//    keeps the next four 128-wide blocks of its rows' packed nibbles in
//    flight; each staged x fragment feeds R row blocks of 16x16x32 MFMAs and
//    each dequantized weight word (exact, in registers) feeds every token
//    block.  Producer workgroups in the same launch compute the K-split sums
//    of [A; w_g] x for every token.
//  * One launch (FUSED, the scalar gate): the producer that completes the
//    producers' count forms U = g (A x); the K-split that completes a tile's
//    count sums the tile's partials in split order, waits (bounded) for U,
//    adds U B^T and rounds y once (finish_tile).  At rank 0 with one split
//    every workgroup rounds its own y.
//  * Three launches (the per-rank gate, or K-splits over more tiles than the
//    workspace header has counters): the consumers store fp32 partial
//    outputs [ksp][M][N], then the compensator's U is formed once, then the
//    finish kernel (both shared with the prefill path) sums the partials in
//    split order, adds U B^T and rounds y once.
//
// Every loop that touches memory has a compile-time shape, so its waits
// count its loads exactly.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCb = 4;               // 128-wide blocks per staged x chunk (= ring depth)
constexpr int kChunkCols = 128 * kCb;
constexpr int kXStr = kChunkCols + 8;  // LDS row stride of a staged chunk (halves)

// Place of 16-byte piece p (of 64) within a staged row: bits 2 and 4 of p
// swapped.  Piece p = 16 i + 4 h + t is what lane (token m, quarter h) reads
// for block i, step t.  With the row stride of 65 pieces, that read falls in
// bank group (m + place(p)) mod 32 of the 32 groups of 16 bytes; one pass of
// a 16-byte LDS read serves 32 lanes, quarters h and h + 1 of all 16 tokens,
// and the swap puts those two quarters 16 groups apart, so the pass touches
// 32 distinct groups (in natural order quarter h + 1 landed 4 groups on, and
// 12 of its 16 lanes met a lane of quarter h).  The place is additive over
// the fields of p, so every read keeps a compile-time offset.
__host__ __device__ constexpr int xplace(int p) {
  return (p & 0x2B) | ((p >> 2) & 1) << 4 | ((p >> 4) & 1) << 2;
}
constexpr int kMaxLds = 160 * 1024;
constexpr int kMaxProducerSplits = 8;  // wide_producer_ksplit's largest count
// Launch-shape constants of plan_wide (measured on MI355X).
#ifndef SPEAR_WIDE_R2_MIN_TILES
// Two 16-row blocks per wave (256-row tiles: half the LDS fragment reads per
// MFMA and half the x staging per weight byte) at up to 64 tokens for
// per-channel layers with at least this many such tiles; measured at 64
// tokens: 8192 -> 28672 (112 tiles) 44.6 against 48.0 us, 8192^2 (32 tiles,
// which then needs twice the K-splits) 27.9 against 22.8 us.  The group-wise
// kernel spills at two blocks.
#define SPEAR_WIDE_R2_MIN_TILES 96
#endif
#ifndef SPEAR_WIDE_WG_RATE
#define SPEAR_WIDE_WG_RATE 25e9  // bytes/s of weights one workgroup streams
#endif
#ifndef SPEAR_WIDE_MAX_KSP
#define SPEAR_WIDE_MAX_KSP 16
#endif
#ifndef SPEAR_WIDE_LOOKAHEAD
#define SPEAR_WIDE_LOOKAHEAD 2  // steps by which the x-fragment reads run ahead of their MFMAs
#endif
// The same at 128 tokens, where 0 leaves the order of each step's reads and
// MFMAs to the compiler.  Measured: one step ahead is faster with one scale
// per row (per-channel), while with group-wise scales, whose per-block scale
// and zero-point registers already hold the kernel at its register limit,
// the compiler's order is.
#ifndef SPEAR_WIDE_LOOKAHEAD128_PC
#define SPEAR_WIDE_LOOKAHEAD128_PC 1
#endif
#ifndef SPEAR_WIDE_LOOKAHEAD128
#define SPEAR_WIDE_LOOKAHEAD128 0
#endif
#ifndef SPEAR_WIDE_PROD_STEPS
#define SPEAR_WIDE_PROD_STEPS 32  // 32-wide steps of K per producer split (before the 4..8 clamp)
#endif
#ifndef SPEAR_WIDE_FORCE_KSP
#define SPEAR_WIDE_FORCE_KSP 0  // > 0: that many K-splits (or the nearest count with no empty split)
#endif

struct WideArgs {
  const uint32_t *qw;
  const uint16_t *scales, *zeros;
  const uint16_t *x;
  uint16_t *y;
  const uint16_t *A, *wg;
  int N, K, G, ngroups, M, rank, rows;  // rows of [A; w_g]
  int producers, ks, rp1;                // producers: row blocks of [A; w_g] x ks
  int n_tiles, ksp, nbs, nb;             // tiles; K-splits; blocks per split; blocks of K
  float *tp;        // [A; w_g] x sums [ks][M][rp1]
  float *part;      // partial outputs [ksp][M][N] (null: y directly)
  int buf_halves;   // halves of the staged x chunk (16 MB rows x kXStr)
  int red_off;      // byte offset of the producers' wave sums in dynamic LDS
  // one launch for the whole call (fused): the kernel finishes its tiles
  int fused;
  WsHeader *hdr;          // counters: producers (arrive), K-splits per tile, counting out
  float *U;               // [M][rp1]: U = g (A x), formed by the last producer
  const uint16_t *B;      // [N][rank]
  float b_gate;
  uint32_t spin_limit;    // polls of the producers' count before computing U itself
  int part_bytes;         // bytes of the partial-tile pieces (fused, ksp > 1)
};

// Fused launch: workgroup b counts itself out in slot b % 8 once it reads the
// producers' count no more; the one that completes every slot resets the
// counters (the scheme of the decode launch), so the workspace is left at
// zero for the next call.  tile_piece_off is the byte offset of the 16-byte
// piece (lane) of a partial tile: split q, tile t, wave w, row block r,
// token block mb.
constexpr uint32_t kNotCounted = 0xFFFFFFFFu;
__device__ __forceinline__ uint32_t count_out(const WideArgs &a) {
  return __hip_atomic_fetch_add(&a.hdr->done[blockIdx.x % 8].v, 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
__device__ void finish_after(const WideArgs &a, uint32_t old) {
  const uint32_t g = gridDim.x, slot = blockIdx.x % 8;
  const uint32_t in_slot = (g - 1 - slot) / 8 + 1;
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
template <int R, int MB>
__device__ __forceinline__ int tile_piece_off(const WideArgs &a, int q, int t, int w, int r, int mb,
                                              int lane) {
  return (((((q * a.n_tiles + t) * kWaves + w) * R + r) * MB + mb) * 64 + lane) * 16;
}

// U = g (A x) from the producers' K-split sums, by the last producer of a
// fused launch: for token m, t_j = sum_q tp[q][m][j] (j < rank) and z = the
// same sum of row rank, each in split order; g = sigmoid(z + b_g); U[m][j] =
// g t_j, zeros in columns rank .. rp1 - 1 (as prefill_u_kernel forms it).
// The sums are read and U is stored with sc1 (every producer published its
// sums before counting itself in).
__device__ void form_u(const WideArgs &a, int tid) {
  const size_t stride = (size_t)a.M * a.rp1;
  const int q4 = a.rp1 / 4;
  const int items = a.M * q4;
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      a.tp, (short)0, (int)(a.ks * stride * sizeof(float)), 0x00020000);
  const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
      a.U, (short)0, (int)(stride * sizeof(float)), 0x00020000);
  // kUItems items per thread and round, all their loads in flight together
  // (one round at up to 64 tokens and rank 64)
  constexpr int kUItems = 3;
  for (int i0 = tid; i0 < items; i0 += kUItems * kThreads) {
    f32x4_t v[kUItems][kMaxProducerSplits];
    float w[kUItems][kMaxProducerSplits];
#pragma unroll
    for (int u = 0; u < kUItems; ++u) {
      const int i = min(i0 + u * kThreads, items - 1);
      const int m = i / q4, j = 4 * (i - m * q4);
#pragma unroll
      for (int q = 0; q < kMaxProducerSplits; ++q) {
        const int base = (int)((min(q, a.ks - 1) * stride + (size_t)m * a.rp1) * sizeof(float));
        v[u][q] = load_partials4(tr, base + j * 4);
        w[u][q] = bitcast<float>(__builtin_amdgcn_raw_buffer_load_b32(tr, base + a.rank * 4, 0, 16));
      }
    }
#pragma unroll
    for (int u = 0; u < kUItems; ++u) {
      const int i = i0 + u * kThreads;
      if (i < items) {
        const int m = i / q4, j = 4 * (i - m * q4);
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
        float z = 0.f;
#pragma unroll
        for (int q = 0; q < kMaxProducerSplits; ++q)
          if (q < a.ks) {
            t += v[u][q];
            z += w[u][q];
          }
        const float g = gate_sigmoid(z + a.b_gate);
        f32x4_t uo;
#pragma unroll
        for (int c = 0; c < 4; ++c) uo[c] = (j + c < a.rank) ? g * t[c] : 0.f;
        store_partials4(uo, ur, (m * a.rp1 + j) * 4);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Producers: one 16-row block of [A; w_g] over one K-split, for every token;
// the sums go to tp[ksi][m][j].
// ---------------------------------------------------------------------------
template <int DT, int MB>
__device__ void produce(const WideArgs &a, int p, f32x4_t *red, int tid) {
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, h = lane >> 4;
  const int rb = p / a.ks, ksi = p % a.ks;
  const int j = rb * 16 + col;
  const bool jin = j < a.rows;
  const uint16_t *arow = (j < a.rank) ? a.A + (size_t)j * a.K : (a.wg ? a.wg : a.A);
  const int nsteps = a.K / 32;
  const int per = (nsteps + a.ks - 1) / a.ks;
  const int s0 = ksi * per, s1 = min(nsteps, s0 + per);
  f32x4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int base = s0 + wave; base < s1; base += kWaves * 4) {
    u32x4_t bo[4], ao[MB][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
    for (int i = 0; i < 4; ++i) {
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
  // fixed-order sum over the waves (wave 0's own, then 1..7), one token block at a time
  float *dst = a.tp + (size_t)ksi * a.M * a.rp1 + j;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (wave > 0) red[wave * 64 + lane] = acc[mb];
    __syncthreads();
    if (wave == 0) {
      f32x4_t v = acc[mb];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v = v + red[w * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mb + 4 * h + e;
        if (jin && m < a.M) {
          if (a.fused)  // read by the last producer of this launch: written through (sc1)
            __hip_atomic_store((uint32_t *)&dst[(size_t)m * a.rp1], bitcast<uint32_t>(v[e]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            dst[(size_t)m * a.rp1] = v[e];
        }
      }
    }
    __syncthreads();
  }
  if (!a.fused) return;
  // Fused launch: count in.  The producer that completes the count forms U
  // and counts in once more, so the consumers' wait is for producers + 1.
  // The stores complete before each count (publish_wait), and each count is
  // performed before this workgroup counts itself out.
  volatile int *last = (volatile int *)red;
  if (wave == 0) publish_wait();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.hdr->arrive.v, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *last = (old + 1 == (uint32_t)a.producers) ? 1 : 0;
  }
  __syncthreads();
  if (*last) {
    form_u(a, tid);
    publish_wait();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_fetch_add(&a.hdr->arrive.v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid == 0) {
    publish_wait();
    finish_after(a, count_out(a));
  }
}

// U without the producers (their count was not seen within the wait): the
// sums t = [A; w_g] x of every token straight from global memory in fp32
// (column rank holds the gate's z), then U = g t in place.  Ends with a
// barrier.
template <int DT>
__device__ void self_u(const WideArgs &a, float *ul, int tid) {
  for (int e = tid; e < a.M * a.rows; e += kThreads) {
    const int m = e / a.rows, j = e - m * a.rows;
    const uint16_t *arow = j < a.rank ? a.A + (size_t)j * a.K : a.wg;
    const uint16_t *xrow = a.x + (size_t)m * a.K;
    float t = 0.f;
    for (int k = 0; k < a.K; k += 8) {
      const u16x8_t av = *(const u16x8_t *)(arow + k);
      const u16x8_t xv = *(const u16x8_t *)(xrow + k);
#pragma unroll
      for (int c = 0; c < 8; ++c) t += to_f32<DT>(av[c]) * to_f32<DT>(xv[c]);
    }
    ul[m * a.rp1 + j] = t;
  }
  __syncthreads();
  for (int e = tid; e < a.M * a.rank; e += kThreads) {
    const int m = e / a.rank, j = e - m * a.rank;
    ul[m * a.rp1 + j] *= gate_sigmoid(ul[m * a.rp1 + a.rank] + a.b_gate);
  }
  __syncthreads();
}

// The end of a fused launch's consumer: this split's fp32 tile (acc, scale
// applied) becomes y.
//  * K-splits (ksp > 1): each split publishes its tile (sc1 stores, then
//    their completion) and counts itself in on the tile's counter; the split
//    that completes the count sums the ksp tiles in split order, its own from
//    registers, and resets the counter.  The others are done.
//  * Compensator: after a bounded wait for the producers' count plus the
//    last producer's U (on expiry the workgroup computes U itself and sets
//    bit 0 of the workspace flags), U goes to LDS and each wave adds U B^T
//    with fp32 16x16x4 MFMAs, rank steps in order.
// y is rounded once.  This is the arithmetic, in the same order, of the
// finish kernel that completes the three-launch form.
template <int DT, int MB, int R, bool EC>
__device__ void finish_tile(const WideArgs &a, const f32x4_t (&acc)[R][MB], int q, int tile,
                            const int (&row)[R], uint16_t *lds, int tid) {
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, h = lane >> 4;
  const int n0 = tile * 16 * R * kWaves;
  volatile int *vote = (volatile int *)((char *)lds + a.red_off);
  uint32_t counted = kNotCounted;
  f32x4_t v[R][MB];
  // the first read of the producers' count, issued before the split sums
  // are gathered so that the two round trips overlap (used by thread 0)
  uint32_t seen = 0;
  auto poll = [&]() {
    return __hip_atomic_load(&a.hdr->arrive.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (a.ksp > 1) {
    const __amdgpu_buffer_rsrc_t pr =
        __builtin_amdgcn_make_buffer_rsrc(a.part, (short)0, a.part_bytes, 0x00020000);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        store_partials4(acc[r][mb], pr, tile_piece_off<R, MB>(a, q, tile, wave, r, mb, lane));
    publish_wait();
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&a.hdr->tile[tile].v, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      vote[0] = (old + 1 == (uint32_t)a.ksp) ? 1 : 0;
    }
    __syncthreads();
    if (vote[0] == 0) {  // uniform: another split completes this tile
      if (EC && tid == 0) finish_after(a, count_out(a));
      return;
    }
    // the first read of the producers' count goes out before the split
    // sums' loads (a wait for it then covers no later load)
    if (EC && tid == 0) seen = poll();
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) v[r][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int kQB = MB <= 4 ? 4 : 2;  // splits whose pieces are in flight together
    for (int q0 = 0; q0 < a.ksp; q0 += kQB) {
      f32x4_t pv[kQB][R][MB];
#pragma unroll
      for (int i = 0; i < kQB; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            pv[i][r][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // the other splits only: uncached loads are costly per CU
            if (q0 + i < a.ksp && q0 + i != q)
              pv[i][r][mb] =
                  load_partials4(pr, tile_piece_off<R, MB>(a, q0 + i, tile, wave, r, mb, lane));
          }
#pragma unroll
      for (int i = 0; i < kQB; ++i)
        if (q0 + i < a.ksp) {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) v[r][mb] += (q0 + i == q) ? acc[r][mb] : pv[i][r][mb];
        }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) v[r][mb] = acc[r][mb];
  }

  if constexpr (EC) {
    // U B^T in 32-rank chunks of bf16 16x16x32 MFMAs on hi/lo halves: u =
    // u_hi + u_lo and b = b_hi + b_lo (exact for fp16 and bf16 B), the
    // products u_hi b_hi + u_lo b_hi + u_hi b_lo accumulated in fp32, which
    // leaves a relative error near 2^-17 in the compensator term.  A lane
    // holds ranks 32 c + 8 h .. + 7 of its token (A operand) and of its
    // output row (B operand); ranks past rank are zeros.
    const int nch = (a.rank + 31) / 32;
    if (a.ksp == 1 && tid == 0) seen = poll();  // before the B loads, as above
    // all of this lane's B (it does not depend on the producers), loaded
    // before the wait: 16-byte pieces when every row's piece is aligned
    // (rank % 8 == 0 and B 16-byte aligned; a piece past rank then reads
    // the row's first and is masked), else value by value
    constexpr int kMaxChunks = (SPEAR_MAX_RANK + 31) / 32;
    u16x8_t bq[kMaxChunks][R];
    const bool bvec = (a.rank % 8) == 0 && ((uintptr_t)a.B % 16) == 0;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      if (c < nch) {
        const int j0 = 32 * c + 8 * h;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint16_t *brow = a.B + (size_t)row[r] * a.rank;
          if (bvec) {
            bq[c][r] = *(const u16x8_t *)(brow + (j0 < a.rank ? j0 : 0));
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) bq[c][r][i] = brow[min(j0 + i, a.rank - 1)];
          }
        }
      }
    auto split8 = [](const float (&f)[8], u32x4_t &hi, u32x4_t &lo) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t h0, l0, h1, l1;
        split_bf16(f[2 * i], h0, l0);
        split_bf16(f[2 * i + 1], h1, l1);
        hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
    };
    // every wave is done with the staged x (the LDS takes U next); an
    // LDS-only barrier, so the B loads stay in flight
    lds_barrier();
    if (tid == 0) {
      int expired = 0;
      for (uint32_t it = 0;; ++it) {
        if (it >= a.spin_limit) {
          expired = 1;
          __hip_atomic_fetch_or(&a.hdr->flags.v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        if (seen >= (uint32_t)a.producers + 1u) break;
        __builtin_amdgcn_s_sleep(1);
        seen = poll();
      }
      vote[1] = expired;
    }
    lds_barrier();
    if (tid == 0) counted = count_out(a);  // the count is read no more
    float *ul = (float *)lds;  // U [M][rp1]
    if (vote[1] == 0) {
      const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
          a.U, (short)0, a.M * a.rp1 * (int)sizeof(float), 0x00020000);
      for (int i = tid; i < a.M * (a.rp1 / 4); i += kThreads)
        *(f32x4_t *)(ul + 4 * i) = load_partials4(ur, 16 * i);
      __syncthreads();
    } else {
      self_u<DT>(a, ul, tid);
    }
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c >= nch) break;
      u32x4_t bh[R], bl[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          f[i] = (32 * c + 8 * h + i < a.rank) ? to_f32<DT>(bq[c][r][i]) : 0.f;
        split8(f, bh[r], bl[r]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = col + 16 * mb;
        // two unconditional 16-byte reads (past the row's rank they read
        // the next row or the LDS beyond U, still inside the allocation),
        // then zeros selected where j >= rank or m >= M: a read under the
        // mask's condition would wait for each value on its own
        const float *up = ul + min(m, a.M - 1) * a.rp1 + 32 * c + 8 * h;
        const f32x4_t u0 = *(const f32x4_t *)up, u1 = *(const f32x4_t *)(up + 4);
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = 32 * c + 8 * h + i;
          f[i] = (j < a.rank && m < a.M) ? (i < 4 ? u0[i] : u1[i - 4]) : 0.f;
        }
        u32x4_t ah, al;
        split8(f, ah, al);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          v[r][mb] = mfma_16x16x32<DT_BF16>(ah, bh[r], v[r][mb]);
          v[r][mb] = mfma_16x16x32<DT_BF16>(al, bh[r], v[r][mb]);
          v[r][mb] = mfma_16x16x32<DT_BF16>(ah, bl[r], v[r][mb]);
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = n0 + 16 * (wave * R + r) + col;
    if (n < a.N) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * mb + 4 * h + e;
          if (m < a.M) a.y[(size_t)m * a.N + n] = from_f32<DT>(v[r][mb][e]);
        }
    }
  }
  if (tid == 0) {
    if (a.ksp > 1)
      __hip_atomic_store(&a.hdr->tile[tile].v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (EC) finish_after(a, counted);
  }
}

// ---------------------------------------------------------------------------
// Consumers.
// ---------------------------------------------------------------------------
template <int DT, int MB, int R, int D, bool EC, bool PERCH, bool FUSED>
__device__ void consume(const WideArgs &a, int c, uint16_t *lds, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 15, h = lane >> 4;
  const int q = c % a.ksp, tile = c / a.ksp;
  const int n0 = tile * 16 * R * kWaves;
  // each wave's 16-row blocks of packed weights as buffer resources (a
  // lane's piece of a tile past K reads as zeros; the staged x is zero there
  // too).  Rows past N repeat the last block.
  int row[R];
  __amdgpu_buffer_rsrc_t wrs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row[r] = min(n0 + 16 * (wave * R + r) + col, a.N - 1);
    wrs[r] = tiled_block_rsrc(a.qw, n0 + 16 * (wave * R + r), a.N, a.K);
  }
  const int kb0 = q * a.nbs;                 // the plan leaves no split empty
  const int nbl = min(a.nb, kb0 + a.nbs) - kb0;
  const int kx0 = kb0 * 128;
  const int kend = min(a.K, kx0 + nbl * 128);  // staged columns past this are zeros

  // per-channel: one zero-point constant and scale per row
  uint32_t zc_row[R];
  float s_row[R];
  if constexpr (PERCH) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      zc_row[r] = zero_constant<DT>(a.zeros[row[r]]);
      s_row[r] = (float)bitcast<_Float16>(a.scales[row[r]]);
    }
  }

  // Groups of D blocks.  Group g's activation columns (kx0 + g D 128 ..) for
  // every token are one staged chunk, loaded into registers (2 MB pieces of
  // 16 bytes per thread) a group ahead.  Every address is clamped into its
  // array and every load is issued unconditionally, so a group is
  // straight-line code whose waits count its loads exactly; columns past the
  // split's end or past K are staged as zeros, which makes the padding blocks
  // of the last group add exact zeros.
  //  * Up to 64 tokens (kDB) the chunks alternate between two LDS buffers:
  //    chunk g + 1 is stored at the end of group g, then one barrier, after
  //    which every wave has finished reading chunk g's buffer (which chunk
  //    g + 2 overwrites) and chunk g + 1 is complete.
  //  * At 128 tokens one buffer: stored at the start of group g, between two
  //    barriers.
  constexpr int kPieces = 2 * MB;  // (16 MB tokens x D 128 / 8 pieces) / 512 threads, D = 4
  static_assert(D == 4, "one staged chunk per group of four blocks");
  constexpr bool kDB = MB <= 4;
  u32x4_t xr[kPieces];
  auto xload = [&](int g) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int p = tid + kThreads * i;  // (token m, piece j): 64 pieces per token row
      const int m = min(p >> 6, a.M - 1), j = p & 63;
      const int k = min(kx0 + g * kChunkCols + 8 * j, a.K - 8);
      xr[i] = *(const u32x4_t *)(a.x + (size_t)m * a.K + k);
    }
  };
  auto xbuf = [&](int g) { return kDB ? lds + (g & 1) * a.buf_halves : lds; };
  // Only the split's last group reaches past its end (or past K): its
  // columns there are staged as zeros, through a bit mask.  Rows past M hold
  // copies of row M - 1 (xload clamps), which no kept output reads.
  auto xstore = [&](int g, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    uint16_t *dst = xbuf(g);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int p = tid + kThreads * i;
      const int m = p >> 6, j = p & 63;
      u32x4_t v = xr[i];
      if constexpr (kMask) {
        const uint32_t keep = (kx0 + g * kChunkCols + 8 * j < kend) ? ~0u : 0u;
        v = u32x4_t{v[0] & keep, v[1] & keep, v[2] & keep, v[3] & keep};
      }
      *(u32x4_t *)(dst + m * kXStr + 8 * xplace(j)) = permute_8(v);
    }
  };

  // the weight ring: block b of the split for row block r (clamped to the
  // split's last block), with its group's scale and zero-point (group-wise)
  // (scale and zero-point bits widened to 32-bit registers: two 16-bit values
  // packed into one register would be loaded into its halves, each load then
  // waiting for the other)
  u32x4_t ring[D][R];
  uint32_t sr[D][R], zr[D][R];
  auto wload = [&](int b, int r, u32x4_t &w, uint32_t &sv, uint32_t &zv) {
    const int kb = kb0 + min(b, nbl - 1);
    w = tile_piece(wrs[r], kb, lane);
    if constexpr (!PERCH) {
      const int g = (kb * 128) / a.G;
      const size_t e = (size_t)row[r] * a.ngroups + g;
      sv = (uint32_t)a.scales[e];
      zv = (uint32_t)a.zeros[e];
    }
  };

  // the same order of loads as each group issues them (activation chunk,
  // then the ring), so that the waits in the loop count the same loads
  // whether the loop is entered or repeated
  xload(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < D; ++i) {
#pragma unroll
    for (int r = 0; r < R; ++r) wload(i, r, ring[i][r], sr[i][r], zr[i][r]);
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4_t acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // A-operand rows past M read row M - 1 (their outputs are never stored)
  int xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xrow[mb] = min(col + 16 * mb, a.M - 1) * kXStr;

  // One group's blocks.  Each ring slot is dequantized before its refill is
  // issued, so the refill can load into the slot's own registers: a slot
  // still live when its refill issues would take a register copy at the
  // loop's back edge, and that copy waits for the load, draining the ring
  // every group.  The x fragments of the group's 4 D steps (block i, step t)
  // are read kLookahead steps ahead of their MFMAs, the order pinned by
  // scheduling barriers, so that the LDS latency overlaps the MFMAs of the
  // steps before (with kLookahead 0, each step reads its own, in an order
  // the compiler chooses).
  constexpr int kSteps = 4 * D;
  constexpr int kLookahead = MB <= 4 ? SPEAR_WIDE_LOOKAHEAD
                                     : (PERCH ? SPEAR_WIDE_LOOKAHEAD128_PC : SPEAR_WIDE_LOOKAHEAD128);
  auto blocks = [&](int g) {
    const uint16_t *xg = xbuf(g) + 8 * xplace(4 * h);
    u32x4_t xq[kSteps][MB];
    auto xread = [&](int st) {
      const uint16_t *xb = xg + 8 * xplace(16 * (st >> 2)) + 8 * (st & 3);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xq[st][mb] = *(const u32x4_t *)(xb + xrow[mb]);
    };
#pragma unroll
    for (int st = 0; st < kLookahead; ++st) xread(st);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int b = g * D + i;
      u32x4_t bop[R][4];
      float sc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t zc;
        if constexpr (PERCH) {
          zc = zc_row[r];
        } else {
          zc = zero_constant<DT>((uint16_t)zr[i][r]);
          sc[r] = (float)bitcast<_Float16>((uint16_t)sr[i][r]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) bop[r][t] = dequant_word<DT>(ring[i][r][t], zc);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) wload(b + D, r, ring[i][r], sr[i][r], zr[i][r]);
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t gacc[R][MB];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int st = 4 * i + t;
        if constexpr (kLookahead == 0) {
          xread(st);
        } else {
          if (st + kLookahead < kSteps) xread(st + kLookahead);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            if constexpr (PERCH) {
              acc[r][mb] = mfma_16x16x32<DT>(xq[st][mb], bop[r][t], acc[r][mb]);
            } else {
              gacc[r][mb] = mfma_16x16x32<DT>(xq[st][mb], bop[r][t],
                                              t == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : gacc[r][mb]);
            }
          }
        }
        if constexpr (kLookahead > 0) __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!PERCH) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[r][mb] += sc[r] * gacc[r][mb];
      }
    }
  };

  const int ngr = (nbl + D - 1) / D;
  if constexpr (kDB) {
    if (ngr == 1)
      xstore(0, std::true_type{});
    else
      xstore(0, std::false_type{});
    xload(1);  // clamped: past the split it reloads valid columns, never stored
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    // every group but the last two, then the one that stores the last
    // (masked) chunk, then the last
    for (int g = 0; g + 2 < ngr; ++g) {
      blocks(g);
      xstore(g + 1, std::false_type{});
      xload(g + 2);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
    }
    if (ngr >= 2) {
      blocks(ngr - 2);
      xstore(ngr - 1, std::true_type{});
      lds_barrier();
    }
    blocks(ngr - 1);
  } else {
    auto run_group = [&](int g, auto mask_tag) {
      lds_barrier();  // every wave is done with group g - 1's chunk
      xstore(g, mask_tag);
      lds_barrier();
      xload(g + 1);  // clamped: past the split it reloads valid columns, staged as zeros
      // keep the prefetches here: the scheduler would otherwise move loads
      // whose results are only used by the next group down to just before
      // that use
      __builtin_amdgcn_sched_barrier(0);
      blocks(g);
    };
    // every group but the last as one loop of straight-line code, then the last
    for (int g = 0; g + 1 < ngr; ++g) run_group(g, std::false_type{});
    run_group(ngr - 1, std::true_type{});
  }
  if constexpr (PERCH) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[r][mb] *= s_row[r];
  }

  if constexpr (!FUSED) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = n0 + 16 * (wave * R + r) + col;
      if (n < a.N) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 16 * mb + 4 * h + e;
            if (m < a.M) {
              if (a.part)
                a.part[((size_t)q * a.M + m) * a.N + n] = acc[r][mb][e];
              else
                a.y[(size_t)m * a.N + n] = from_f32<DT>(acc[r][mb][e]);
            }
          }
      }
    }
  } else {
    finish_tile<DT, MB, R, EC>(a, acc, q, tile, row, lds, tid);
  }
}

// One workgroup per CU: its 8 waves are 2 per SIMD (the launch bound's
// second figure, waves per SIMD, lets each use up to 256 registers), and the
// staged x takes most of the LDS.  FUSED: the one-launch form (the tile
// finishing is compiled only into it, so the other form keeps its
// registers for the main loop).
template <int DT, int MB, int R, int D, bool EC, bool PERCH, bool FUSED>
__global__ __launch_bounds__(kThreads, 2) void wide_kernel(WideArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, b = blockIdx.x;
  if constexpr (EC) {
    if (b < a.producers) {
      produce<DT, MB>(a, b, (f32x4_t *)((char *)lds + a.red_off), tid);
      return;
    }
    consume<DT, MB, R, D, true, PERCH, FUSED>(a, b - a.producers, lds, tid);
  } else {
    consume<DT, MB, R, D, false, PERCH, FUSED>(a, b, lds, tid);
  }
}

template <int DT, int MB, int R, bool EC, bool PERCH, bool FUSED>
hipError_t launch_t(const WideArgs &a, int grid, size_t lds, hipStream_t s) {
  auto kern = wide_kernel<DT, MB, R, kCb, EC, PERCH, FUSED>;
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

template <int DT, int MB, int R, bool FUSED>
hipError_t launch_ec(const WideArgs &a, int grid, size_t lds, bool ec, bool perch, hipStream_t s) {
  if (ec) return perch ? launch_t<DT, MB, R, true, true, FUSED>(a, grid, lds, s)
                       : launch_t<DT, MB, R, true, false, FUSED>(a, grid, lds, s);
  return perch ? launch_t<DT, MB, R, false, true, FUSED>(a, grid, lds, s)
               : launch_t<DT, MB, R, false, false, FUSED>(a, grid, lds, s);
}

template <int DT, int MB, int R>
hipError_t launch_fused(const WideArgs &a, int grid, size_t lds, bool ec, bool perch, bool fused,
                        hipStream_t s) {
  return fused ? launch_ec<DT, MB, R, true>(a, grid, lds, ec, perch, s)
               : launch_ec<DT, MB, R, false>(a, grid, lds, ec, perch, s);
}

template <int DT>
hipError_t launch_mb(const WideArgs &a, const WidePlan &p, bool ec, bool perch, hipStream_t s) {
  const int grid = p.n_tiles * p.ksp + p.producers;
  if (p.mb == 4) {
    return p.r == 1 ? launch_fused<DT, 4, 1>(a, grid, p.lds, ec, perch, p.fused, s)
                    : launch_fused<DT, 4, 2>(a, grid, p.lds, ec, perch, p.fused, s);
  }
  // 128 tokens: one row block per wave
  return launch_fused<DT, 8, 1>(a, grid, p.lds, ec, perch, p.fused, s);
}

// K-splits of the producers: enough that each wave covers its split in one
// round of loads (32 steps of 32 columns per workgroup), a multiple of 4 from
// 4 to 8: under the consumers' weight stream every round trip of a producer
// is long.
int wide_producer_ksplit(int K) {
  const int need = (K / 32 + SPEAR_WIDE_PROD_STEPS - 1) / SPEAR_WIDE_PROD_STEPS;
  const int ks = (need + 3) / 4 * 4;
  return ks < 4 ? 4 : (ks > 8 ? 8 : ks);
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// Launch shape for M tokens (33..128): 16-token blocks MB (4 or 8), rows per
// wave 16 R, and the K-split count ksp of the tiles of 128 R rows.  ksp is
// the count whose estimated time is least, where too few workgroups leave
// the weight stream short of loads in flight, and each split adds its fp32
// partial outputs (M N 4 bytes) to write and for the finish kernel to read:
//   time ~ max(weights / (resident workgroups x per-workgroup rate),
//              (weights + partials) / HBM rate) + partials / re-read rate.
WidePlan plan_wide(const LayerDesc &L, int M) {
  WidePlan p{};
  p.ok = false;
  if (M < 1 || M > 128) return p;
  p.mb = M <= 64 ? 4 : 8;
  p.r = (p.mb == 4 && L.per_channel && (L.N + 255) / 256 >= SPEAR_WIDE_R2_MIN_TILES) ? 2 : 1;
  p.rb_a = L.rank > 0 ? (L.rank + L.gate_rows() + 15) / 16 : 0;
  p.ks = L.rank > 0 ? wide_producer_ksplit(L.K) : 0;
  p.producers = p.rb_a * p.ks;
  p.rp1 = (L.rank + 1 + 3) / 4 * 4;
  p.nb = (L.K + 127) / 128;
  const int tile_rows = 16 * p.r * kWaves;
  p.n_tiles = (L.N + tile_rows - 1) / tile_rows;
  const int resident = 256;  // one workgroup per CU
  const double wbytes = (double)L.N * L.K / 2;
  double best = 1e30;
  for (int ks = 1; ks <= std::min(SPEAR_WIDE_MAX_KSP, p.nb); ++ks) {
    const int nbs = (p.nb + ks - 1) / ks;
    const int ksp = (p.nb + nbs - 1) / nbs;  // no empty split
    if (ksp != ks) continue;
    const int wgs = p.n_tiles * ksp;
    const double live = std::min(wgs, resident);
    // fp32 partial outputs: with K-splits, or for the per-rank gate's finish kernel
    const bool parts = ksp > 1 || L.rg_hidden > 0;
    const double part = parts ? (double)ksp * L.N * M * 4 : 0.0;
    double t = std::max(wbytes / (live * SPEAR_WIDE_WG_RATE), (wbytes + part) / 5e12) +
               part / 8e12;
    if (SPEAR_WIDE_FORCE_KSP > 0) t = std::abs(ksp - SPEAR_WIDE_FORCE_KSP);
    if (t < best * 0.999) {
      best = t;
      p.ksp = ksp;
      p.nbs = nbs;
    }
  }
  // fewer producer splits where consumers and producers would not all be
  // resident at once (the last consumers would wait for a second round)
  while (p.ks > 4 && p.n_tiles * p.ksp + p.rb_a * p.ks > 256) p.ks -= 4;
  // If even the fewest producer splits leave no room (the tiles' splits alone
  // take every slot), the tiles get the largest K-split count that does,
  // and the producers their splits again.  At 28672 -> 8192, 17 and 24
  // tokens, rank 64: 4 splits and 20 producers (276 workgroups) ran 66.7 /
  // 70.4 us, 3 splits and 40 producers (232) 56.1 / 56.2 us.
  if (SPEAR_WIDE_FORCE_KSP == 0 && p.rb_a > 0 && p.n_tiles * p.ksp + p.rb_a * p.ks > 256) {
    for (int ks = p.ksp - 1; ks >= 1; --ks) {
      const int nbs = (p.nb + ks - 1) / ks;
      if ((p.nb + nbs - 1) / nbs != ks) continue;  // no empty split
      if (p.n_tiles * ks + p.rb_a * 4 > 256) continue;
      p.ksp = ks;
      p.nbs = nbs;
      p.ks = wide_producer_ksplit(L.K);
      while (p.ks > 4 && p.n_tiles * p.ksp + p.rb_a * p.ks > 256) p.ks -= 4;
      break;
    }
  }
  p.producers = p.rb_a * p.ks;
  p.direct = L.rank == 0 && p.ksp == 1;
  // One launch finishes the tiles (the K-splits' sums through the tile
  // counters, the scalar gate's U from the last producer); the per-rank gate
  // keeps its U kernel and the finish kernel, as do K-split calls with more
  // tiles than the header has counters.
  p.fused = !p.direct && L.rg_hidden == 0 && (p.ksp == 1 || p.n_tiles <= kMaxSplitTiles);
  p.buf_halves = 16 * p.mb * kXStr;
  // up to 64 tokens the staged chunks alternate between two buffers
  p.red_off = (int)round256((size_t)p.buf_halves * 2 * (p.mb <= 4 ? 2 : 1));
  p.lds = p.red_off + (size_t)kWaves * 64 * 16;  // the producers' wave sums
  p.tp_off = kWsDataOff;
  p.u_off = p.tp_off + (L.rank > 0 ? round256((size_t)p.ks * M * p.rp1 * sizeof(float)) : 0);
  p.part_off = p.u_off + (L.rank > 0 ? round256((size_t)M * p.rp1 * sizeof(float)) : 0);
  // partial outputs: fused, the K-splits' tiles as 16-byte pieces of each
  // wave's fragments (tile_piece_off); else [ksp][M][N] for the finish kernel
  const size_t part_bytes =
      p.fused ? (p.ksp > 1 ? (size_t)p.ksp * p.n_tiles * tile_rows * 16 * p.mb * sizeof(float) : 0)
              : (size_t)p.ksp * M * L.N * sizeof(float);
  p.end = p.direct ? 0 : p.part_off + round256(part_bytes);
  p.ok = p.lds <= (size_t)kMaxLds;
  return p;
}

size_t wide_workspace_bytes(const LayerDesc &L, int M) {
  const WidePlan p = plan_wide(L, M);
  return p.ok ? p.end : 0;
}

void describe_wide(const LayerDesc &L, int M, spear_plan_t *out) {
  const WidePlan p = plan_wide(L, M);
  out->path = SPEAR_PATH_DECODE_WIDE;
  out->workgroups = p.n_tiles * p.ksp + p.producers;
  out->waves_per_workgroup = kWaves;
  out->producers = p.producers;
  out->k_splits = p.ksp;
  out->workspace_bytes = p.end;
}

hipError_t launch_wide(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                       void *ws, hipStream_t s) {
  const WidePlan p = plan_wide(L, M);
  if (!p.ok || (!p.direct && !ws)) return hipErrorInvalidConfiguration;
  char *base = (char *)ws;
  WideArgs a{};
  a.qw = L.qw;
  a.scales = L.scales;
  a.zeros = L.zeros;
  a.x = x;
  a.y = y;
  a.A = L.A;
  a.wg = L.wg;
  a.N = L.N;
  a.K = L.K;
  a.G = L.G;
  a.ngroups = L.ngroups;
  a.M = M;
  a.rank = L.rank;
  a.rows = L.rank + L.gate_rows();
  a.producers = p.producers;
  a.ks = p.ks;
  a.rp1 = p.rp1;
  a.n_tiles = p.n_tiles;
  a.ksp = p.ksp;
  a.nbs = p.nbs;
  a.nb = p.nb;
  a.tp = L.rank > 0 ? (float *)(base + p.tp_off) : nullptr;
  a.part = p.direct ? nullptr : (float *)(base + p.part_off);
  a.buf_halves = p.buf_halves;
  a.red_off = p.red_off;
  a.fused = p.fused ? 1 : 0;
  a.hdr = (WsHeader *)ws;
  a.U = L.rank > 0 ? (float *)(base + p.u_off) : nullptr;
  a.B = L.B;
  a.b_gate = L.b_gate;
  a.spin_limit = get_decode_spin_limit();
  a.part_bytes = (int)(p.end - p.part_off);
  const bool ec = L.rank > 0;
  hipError_t e = dtype == DT_F16 ? launch_mb<DT_F16>(a, p, ec, L.per_channel, s)
                                 : launch_mb<DT_BF16>(a, p, ec, L.per_channel, s);
  if (e != hipSuccess || p.direct || p.fused) return e;
  float *U = nullptr;
  if (ec) {
    U = (float *)(base + p.u_off);
    if ((e = launch_form_u(L, a.tp, p.ks, M, U, s)) != hipSuccess) return e;
  }
  // the scale is already applied to the partials (per-channel: at the end of the main loop)
  return launch_finish_parts(L, dtype, y, M, a.part, p.ksp, U, false, s);
}

}  // namespace spear
