// Prefill path: y = dequant(W_q) x + sigmoid(w_g . x + b_g) * B (A x) for
// many tokens (M in the hundreds to thousands).
//
// The pages run the compensator of the compute-bound prefill as a separate
// kernel that overlaps the low-bit GEMM instead of fusing it (SPEAR
// explanation page, Technical Summary 2.2 A, prefill phase).  Here:
//
//  * prefill_ec_kernel computes the sums [A; w_g] x per token (rows 0..rank,
//    the last being the gate's pre-activation z) into the workspace, with K
//    split over several workgroups per 32 tokens; each split stores its own
//    partial sums;
//  * prefill_u_kernel (or, with the per-rank gate, prefill_rgate_kernel)
//    forms U = diag(g) (X A^T) once from those partials: g = sigmoid(z + b_g),
//    each sum taken in split order;
//  * prefill_gemm_kernel, a 128x128x128-tiled MFMA GEMM.  Each k-block stages
//    the activation tile and the exactly dequantized weight tile (q - z in
//    the activation type) in LDS; four waves each own a 64x64 quarter of the
//    output tile and run 16x16x32 MFMAs, applying each row's fp32 scale once
//    per 128-wide block (or once at the end when one scale covers the row).
//    When the output has too few tiles to fill the chip, K is split over
//    several workgroups that store fp32 partial tiles;
//  * prefill_finish_kernel completes 64x64 output tiles: the sum of the GEMM's
//    split partials (with the per-channel scale) or the rounded y of the
//    two-stream concurrent schedule, plus U B^T, rounded once into y.
//
// Schedules:
//  * serial (no aux stream): compensator, then the GEMM, whose epilogue adds
//    U B^T before y is rounded once (or, with K split, the finish kernel
//    does).  Every reduction across workgroups happens across a kernel
//    boundary;
//  * concurrent (aux stream given, the pages' overlap of the compensator with
//    the GEMM).  A kernel on a second stream gets no CU while the GEMM's
//    workgroups fill every CU, so on MI355X the overlap happens inside one
//    launch: its first workgroups are compensator producers (ec_block, four
//    waves each), dispatched ahead of the GEMM tiles; they publish their
//    K-split sums with agent-scope stores and count themselves in, and each
//    tile's epilogue, after a bounded wait for that count, forms its U rows
//    from the sums exactly as prefill_u_kernel does (or, if the wait
//    expires, computes its tokens' sums itself) and adds U B^T before y is
//    rounded once.  The last workgroup to finish resets the counters.  With
//    the per-rank gate or a K-split GEMM past K = 16384 the compensator
//    kernels run on the aux stream beside the GEMM, and after the join the
//    finish kernel adds U B^T;
//  * either schedule, a K-split GEMM with the scalar gate up to K = 16384
//    (SPROD): the producers run in the split GEMM launch ahead of its tiles,
//    the producer that completes each 32-token block forms that block's U
//    rows, and the finish kernel (the next launch) adds U B^T.
#include <algorithm>
#include <mutex>
#include <unordered_map>

#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
// LDS row strides (halves) of the activation and weight tiles.  A 16x16x32
// fragment read puts 16 rows x 2 column groups in flight; a 288-byte stride
// spreads them over distinct banks.  Measured at M = 2048 (bf16, rank 0):
// padding by 16 halves runs the GEMM 6-7% faster than by 8 or 24, and by 40
// or 48 costs the second workgroup per CU.  (An unpadded layout with an XOR
// swizzle that also frees the tile stores of conflicts ran 10% slower, most
// likely because its per-lane addresses replace the LDS instructions'
// immediate offsets in a kernel already near its register budget.)
constexpr int LSTR = BK + 16;
constexpr int WSTR = BK + 16;

// U = diag(g) (X A^T) as the consumers read it: U[m][j] for j < rank and
// zeros in columns rank .. rp1-1 (rp1 a multiple of 4), so that every 16-byte
// piece of a row can be read whole.
struct UView {
  const float *U;  // [M][rp1]
  int M, rank, rp1;
};

// Sums over split partials.  kSplitBatch loads (clamped to the last split, so
// always valid) are issued before any of them is added, so a sum over ks
// splits waits for ceil(ks / kSplitBatch) rounds of loads instead of ks; the
// additions still run in split order.
constexpr int kSplitBatch = 8;

// sum_q p[q * stride] over q < ks, in order
template <int NB = kSplitBatch>
__device__ __forceinline__ float split_sum(const float *p, size_t stride, int ks) {
  float t = 0.f;
  for (int q0 = 0; q0 < ks; q0 += NB) {
    float v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) v[i] = p[(size_t)min(q0 + i, ks - 1) * stride];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (q0 + i < ks) t += v[i];
  }
  return t;
}

// the same over 16-byte pieces (p and stride 16-byte aligned)
template <int NB = kSplitBatch>
__device__ __forceinline__ f32x4_t split_sum4(const float *p, size_t stride, int ks) {
  f32x4_t t = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < ks; q0 += NB) {
    f32x4_t v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) v[i] = *(const f32x4_t *)(p + (size_t)min(q0 + i, ks - 1) * stride);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (q0 + i < ks) t += v[i];
  }
  return t;
}



constexpr int kEpiRc = 32;           // ranks per epilogue chunk: the K of one 16x16x32 MFMA
// LDS row stride of a chunk's bf16 operands (halves): 24 dwords, so a
// fragment read's 16 rows x 2 column groups fall on distinct banks
constexpr int kEpiStr = kEpiRc + 16;
static_assert(2 * BM * kEpiStr <= BM * LSTR, "epilogue U hi/lo fit the activation tile");
static_assert(2 * BN * kEpiStr <= BN * WSTR, "epilogue B hi/lo fit the weight tile");

// ---------------------------------------------------------------------------
// Compensator sums: Tp[ksi][m][j] = sum over split ksi's K range of
// [A; w_g][j][k] x[m][k], j = 0..rank.
//
// Workgroup (blk, ksi) takes kEcTok = 32 tokens (two MFMA row blocks) and K
// split ksi of ks; its eight waves take interleaved 32-wide K steps.  Up to
// kEcRb 16-row blocks of [A; w_g] are accumulated together, so each weight
// piece feeds both token blocks and each activation piece feeds kEcRb MFMAs;
// each wave keeps kEcU steps of loads in flight before it multiplies.
// ---------------------------------------------------------------------------
struct EcArgs {
  const uint16_t *x, *A, *wg;
  int K, M, rank, rows, rp1, ks;  // rows of [A; w_g]: rank + 1, or rank (per-rank gate)
  float *Tp;  // [ks][M][rp1]
  // ks == 1 with the scalar gate: U = diag(g) (X A^T) written here directly
  // (zeros in columns rank .. rp1-1), and no partials
  float *U;
  float b_gate;
};

constexpr int kEcWaves = 8, kEcRb = 3, kEcU = 4, kEcTok = 32, kEcMb = kEcTok / 16;
// rows of [A; w_g] round up to 16: up to 16 * ceil((SPEAR_MAX_RANK + 1) / 16) = 144
constexpr int kTzStride = 145;
static_assert(kTzStride > 16 * ((SPEAR_MAX_RANK + 1 + 15) / 16), "tz stride");

// One compensator block: tokens blk * kEcTok .. + kEcTok, K split ksi of a.ks,
// by WAVES waves (the stand-alone kernel's eight, or the four of a producer
// workgroup in the GEMM launch, whose sums other workgroups of that launch
// read: AGENT stores them with agent-scope stores).  red and tz are LDS.
template <int DT, int WAVES, bool AGENT>
__device__ void ec_block(const EcArgs &a, int blk, int ksi, f32x4_t (*red)[kEcRb][kEcMb][64],
                         float (*tz)[kTzStride], int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, h = lane >> 4;
  const int m0 = blk * kEcTok;
  // A-operand rows of this lane: tokens m0 + col + 16 mb; rows past M repeat
  // M - 1 (MFMA output rows depend only on their own A rows, and those are
  // never stored)
  const uint16_t *xrow[kEcMb];
#pragma unroll
  for (int mb = 0; mb < kEcMb; ++mb) xrow[mb] = a.x + (size_t)min(m0 + col + 16 * mb, a.M - 1) * a.K;
  const int rb_a = (a.rows + 15) / 16;
  const int nsteps = a.K / 32;
  const int per = (nsteps + a.ks - 1) / a.ks;
  const int s_lo = ksi * per, s_hi = min(nsteps, s_lo + per);
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  for (int rb0 = 0; rb0 < rb_a; rb0 += kEcRb) {
    const uint16_t *arow[kEcRb];
    bool jin[kEcRb];
#pragma unroll
    for (int r = 0; r < kEcRb; ++r) {
      const int j = (rb0 + r) * 16 + col;
      jin[r] = rb0 + r < rb_a && j < a.rows;
      // j >= rank: w_g, or (per-rank gate, no w_g) any valid row; masked past the rows
      arow[r] = (j < a.rank) ? a.A + (size_t)j * a.K : (a.wg ? a.wg : a.A);
    }
    f32x4_t acc[kEcRb][kEcMb];
#pragma unroll
    for (int r = 0; r < kEcRb; ++r)
#pragma unroll
      for (int mb = 0; mb < kEcMb; ++mb) acc[r][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int s0 = s_lo + wave; s0 < s_hi; s0 += WAVES * kEcU) {
      u32x4_t xo[kEcU][kEcMb], ao[kEcU][kEcRb];
#pragma unroll
      for (int u = 0; u < kEcU; ++u) {
        const int k = min(s0 + WAVES * u, s_hi - 1) * 32 + 8 * h;
#pragma unroll
        for (int mb = 0; mb < kEcMb; ++mb) xo[u][mb] = *(const u32x4_t *)(xrow[mb] + k);
#pragma unroll
        for (int r = 0; r < kEcRb; ++r) ao[u][r] = *(const u32x4_t *)(arow[r] + k);
      }
#pragma unroll
      for (int u = 0; u < kEcU; ++u) {
        if (s0 + WAVES * u < s_hi) {
#pragma unroll
          for (int r = 0; r < kEcRb; ++r) {
            const u32x4_t b = jin[r] ? ao[u][r] : zero;
#pragma unroll
            for (int mb = 0; mb < kEcMb; ++mb) acc[r][mb] = mfma_16x16x32<DT>(xo[u][mb], b, acc[r][mb]);
          }
        }
      }
    }
    // fixed-order sum over the waves: wave 0's own, then 1..7
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < kEcRb; ++r)
#pragma unroll
        for (int mb = 0; mb < kEcMb; ++mb) red[wave][r][mb][lane] = acc[r][mb];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int r = 0; r < kEcRb; ++r) {
        if (rb0 + r < rb_a) {
#pragma unroll
          for (int mb = 0; mb < kEcMb; ++mb) {
            f32x4_t v = acc[r][mb];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) v = v + red[w][r][mb][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) tz[16 * mb + 4 * h + e][(rb0 + r) * 16 + col] = v[e];
          }
        }
      }
    }
    __syncthreads();
  }


  if (a.U) {
    // the whole of K in this workgroup: U = g t for its tokens, g from row rank
    const int nval = kEcTok * a.rp1;
    for (int i = tid; i < nval; i += 64 * WAVES) {
      const int mm = i / a.rp1, j = i - mm * a.rp1;
      if (m0 + mm < a.M)
        a.U[(size_t)(m0 + mm) * a.rp1 + j] =
            j < a.rank ? gate_sigmoid(tz[mm][a.rank] + a.b_gate) * tz[mm][j] : 0.f;
    }
    return;
  }
  // this split's sums, rows 0..rows-1 of its tokens
  const int nval = kEcTok * a.rows;
  float *tp = a.Tp + ((size_t)ksi * a.M + m0) * a.rp1;
  for (int i = tid; i < nval; i += 64 * WAVES) {
    const int mm = i / a.rows, j = i - mm * a.rows;
    if (m0 + mm < a.M) {
      if constexpr (AGENT)  // read by other workgroups of the same launch
        __hip_atomic_store((uint32_t *)&tp[(size_t)mm * a.rp1 + j], bitcast<uint32_t>(tz[mm][j]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        tp[(size_t)mm * a.rp1 + j] = tz[mm][j];
    }
  }
}

template <int DT>
__global__ __launch_bounds__(64 * kEcWaves) void prefill_ec_kernel(EcArgs a) {
  __shared__ f32x4_t red[kEcWaves][kEcRb][kEcMb][64];
  __shared__ float tz[kEcTok][kTzStride];
  ec_block<DT, kEcWaves, false>(a, blockIdx.x / a.ks, blockIdx.x % a.ks, red, tz, threadIdx.x);
}

struct GemmArgs {
  const uint32_t *qw;
  const uint16_t *scales, *zeros;
  const uint16_t *x;
  uint16_t *y;
  int N, K, G, ngroups, M;
  UView u;            // EPI: U, complete before the launch; SPROD: where the producers form U
  const uint16_t *B;  // EPI: [N][rank]
  int ks;             // SPLIT: K splits (blockIdx.z), each a contiguous range of k-blocks
  float *part;        // SPLIT: [ks][M][N] fp32 partial outputs
  // PROD (the concurrent schedule): the first nprod workgroups of a 1-D grid
  // (nprod a multiple of 8; those past nprod_real only count themselves in)
  // compute the compensator's K-split sums ec.Tp, and the ntn x ntm GEMM tiles
  // after them read those sums in their epilogue once every producer is in
  int nprod, nprod_real, ntn, ntm;
  EcArgs ec;
  WsHeader *hdr;
  uint32_t spin_limit;  // polls of the producers' count before a tile computes the sums itself
  float *Tfb;           // [M][rp1]: the sums of a tile whose wait expired
};

// Output tile of this workgroup.  Workgroups go to the eight XCDs in turn
// (linear id mod 8) and each XCD has its own L2, so the tiles are renumbered:
// each XCD's workgroups take one run of consecutive numbers, and numbers walk
// the output in bands of kGroupM tile rows, column by column.  The
// workgroups that one XCD holds at a time then cover a compact block of the
// output and share its activation rows and weight columns in that L2.
constexpr int kGroupM = 8;
__device__ __forceinline__ void gemm_tile(int L, int ntn, int ntm, int &tm, int &tn) {
  const int T = ntn * ntm;
  const int c = L & 7;
  int p = L >> 3;  // after the tiles of XCDs 0 .. c-1; XCD c' holds ceil((T - c') / 8)
  for (int cc = 0; cc < c; ++cc) p += (T - cc + 7) >> 3;
  const int per_group = kGroupM * ntn;
  const int grp = p / per_group;
  const int first = grp * kGroupM;
  const int gsz = min(ntm - first, kGroupM);
  const int r = p - grp * per_group;
  tm = first + r % gsz;
  tn = r / gsz;
}

// Weight piece p (0 .. 511) of a BN-row tile's k-block: lane p & 63 of the
// tile's 16-row block p >> 6, i.e. tile row 16 (p >> 6) + (p & 15) and
// codes 32 q .. 32 q + 31 of the block for q = (p & 63) >> 4.
__device__ __forceinline__ int wpiece_row(int p) { return 16 * (p >> 6) + (p & 15); }
__device__ __forceinline__ int wpiece_quarter(int p) { return (p & 63) >> 4; }

// Count this workgroup out of a PROD launch; the last one resets the
// producers' count and these counters.  Workgroup b counts into slot b % 8;
// the one that completes a slot counts the slot into the top counter, and
// the one that completes the top counter is last overall.
__device__ void prod_finish(WsHeader *hdr) {
  const uint32_t g = gridDim.x, b = blockIdx.x, slot = b % 8;
  const uint32_t in_slot = (g - 1 - slot) / 8 + 1;
  const uint32_t old = __hip_atomic_fetch_add(&hdr->done[slot].v, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1 != in_slot) return;
  const uint32_t slots = g < 8 ? g : 8;
  const uint32_t top = __hip_atomic_fetch_add(&hdr->done_top.v, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  if (top + 1 != slots) return;
  __hip_atomic_store(&hdr->arrive.v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&hdr->done_top.v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = 0; i < 8; ++i)
    __hip_atomic_store(&hdr->done[i].v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Completion of this wave's agent-scope stores (s_waitcnt vmcnt(0); expcnt
// and lgkmcnt left at their maxima), fenced against compiler motion.
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// SPROD: U's rows for one 32-token block, formed by the producer that
// completed the block's count from the block's K-split sums (read with sc1:
// every producer published its sums before counting in), each element's sum
// in split order, then U = g t as prefill_u_kernel forms it.  U goes to
// a.u.U with plain stores: the finish kernel that reads it is the next launch.
constexpr int kMaxFusedSplits = 8;  // fused_ksplit's largest count
__device__ void block_u(const GemmArgs &a, int blk, int tid) {
  const EcArgs &e = a.ec;
  const int m0 = blk * kEcTok, nt = min(kEcTok, e.M - m0);
  const int q4 = e.rp1 / 4, items = nt * q4;
  const size_t stride = (size_t)e.M * e.rp1;
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      e.Tp, (short)0, (int)(e.ks * stride * sizeof(float)), 0x00020000);
  float *U = (float *)a.u.U;
  constexpr int kItems = 3;  // items per thread and round, all their loads in flight together
  for (int i0 = tid; i0 < items; i0 += kItems * 256) {
    f32x4_t v[kItems][kMaxFusedSplits];
    float w[kItems][kMaxFusedSplits];
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
      const int i = min(i0 + u * 256, items - 1);
      const int m = m0 + i / q4, j = 4 * (i % q4);
#pragma unroll
      for (int q = 0; q < kMaxFusedSplits; ++q) {
        const int base = (int)((min(q, e.ks - 1) * stride + (size_t)m * e.rp1) * sizeof(float));
        v[u][q] = bitcast<f32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(tr, base + 4 * j, 0, 16));
        w[u][q] = bitcast<float>(__builtin_amdgcn_raw_buffer_load_b32(tr, base + 4 * e.rank, 0, 16));
      }
    }
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
      const int i = i0 + u * 256;
      if (i < items) {
        const int m = m0 + i / q4, j = 4 * (i % q4);
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
        float z = 0.f;
#pragma unroll
        for (int q = 0; q < kMaxFusedSplits; ++q)
          if (q < e.ks) {
            t += v[u][q];
            z += w[u][q];
          }
        const float g = gate_sigmoid(z + e.b_gate);
        f32x4_t uo;
#pragma unroll
        for (int c = 0; c < 4; ++c) uo[c] = (j + c < e.rank) ? g * t[c] : 0.f;
        *(f32x4_t *)(U + (size_t)m * e.rp1 + j) = uo;
      }
    }
  }
}

// SPROD (the serial schedule with a K-split GEMM and the scalar gate): the
// first nprod workgroups of a 1-D grid (nprod a multiple of 8, so that the
// tiles after them keep their XCD mapping; those past nprod_real do nothing)
// compute the compensator's K-split sums; the producer that completes a
// token block's count (the header's tile counters, one per 32-token block)
// forms that block's U rows and resets the counter.  The split tiles after
// them never wait: the finish kernel, the next launch, reads U.
template <int DT, bool PERCH, bool EPI, bool SPLIT, bool PROD = false, bool SPROD = false>
__global__ __launch_bounds__(256, 2) void prefill_gemm_kernel(GemmArgs a) {
  static_assert(!(EPI && SPLIT), "split tiles are finished by prefill_finish_kernel");
  static_assert(!PROD || (EPI && !SPLIT), "producers serve the epilogue of unsplit tiles");
  static_assert(!SPROD || (SPLIT && !PROD), "SPROD: producers ahead of split tiles");
  __shared__ __align__(16) uint16_t xs[BM * LSTR];
  __shared__ __align__(16) uint16_t wsm[BN * WSTR];
  __shared__ float ss[BN];
  __shared__ int vote;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, h = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  int split = blockIdx.z;  // SPLIT: this workgroup's K split
  if constexpr (PROD) {
    if ((int)blockIdx.x < a.nprod) {
      // a compensator producer: one (32-token block, K split) of the sums
      static_assert(sizeof(f32x4_t) * 4 * kEcRb * kEcMb * 64 <= sizeof(xs), "producer red in xs");
      static_assert(sizeof(float) * kEcTok * kTzStride <= sizeof(wsm), "producer tz in wsm");
      if ((int)blockIdx.x < a.nprod_real)
        ec_block<DT, 4, true>(a.ec, blockIdx.x / a.ec.ks, blockIdx.x % a.ec.ks,
                              (f32x4_t(*)[kEcRb][kEcMb][64])xs, (float(*)[kTzStride])wsm, tid);
      stores_done();
      __syncthreads();
      if (tid == 0) {
        __hip_atomic_fetch_add(&a.hdr->arrive.v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prod_finish(a.hdr);
      }
      return;
    }
    gemm_tile(blockIdx.x - a.nprod, a.ntn, a.ntm, tm, tn);
  } else if constexpr (SPROD) {
    if ((int)blockIdx.x < a.nprod) {
      static_assert(sizeof(f32x4_t) * 4 * kEcRb * kEcMb * 64 <= sizeof(xs), "producer red in xs");
      static_assert(sizeof(float) * kEcTok * kTzStride <= sizeof(wsm), "producer tz in wsm");
      if ((int)blockIdx.x >= a.nprod_real) return;
      const int blk = blockIdx.x / a.ec.ks;
      ec_block<DT, 4, true>(a.ec, blk, blockIdx.x % a.ec.ks, (f32x4_t(*)[kEcRb][kEcMb][64])xs,
                            (float(*)[kTzStride])wsm, tid);
      stores_done();
      __syncthreads();
      if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&a.hdr->tile[blk].v, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        vote = (old + 1 == (uint32_t)a.ec.ks) ? 1 : 0;
      }
      __syncthreads();
      if (vote) {
        block_u(a, blk, tid);
        if (tid == 0)
          __hip_atomic_store(&a.hdr->tile[blk].v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    const int L = blockIdx.x - a.nprod, T = a.ntn * a.ntm;
    split = L / T;
    gemm_tile(L - split * T, a.ntn, a.ntm, tm, tn);
  } else {
    gemm_tile(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, gridDim.y, tm, tn);
  }
  const int n0 = tn * BN, m0 = tm * BM;
  const int nkb = (a.K + BK - 1) / BK;
  const int kw = a.K / 8;

  u32x4_t xr[8];
  u32x4_t wr[2];
  uint16_t zr[2];
  uint16_t sv = 0;

  // Loads of k-block kb.  Over the tile's rows, buffer resources return zeros
  // past M (x) and past N (weights, zero-points, scales), every per-lane
  // offset is loop-invariant, and the k-block's advance goes into the
  // scalar offset.  The scalar offset is not range-checked, so a k-block
  // that runs past K (K % 128 != 0) takes the guarded loads instead.
  // (the packed weight's rows are padded to a multiple of 16 in memory; the
  // padding is part of the tiled order, so the weight resource covers it)
  const int mrows = min(BM, a.M - m0), nrows = min(BN, a.N - n0);
  const int nrows_p = min(BN, ((a.N + 15) & ~15) - n0);
  const __amdgpu_buffer_rsrc_t x_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.x + (size_t)m0 * a.K), (short)0, mrows * a.K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.qw + (size_t)n0 * kw), (short)0, nrows_p * kw * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t z_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.zeros + (size_t)n0 * a.ngroups), (short)0, nrows * a.ngroups * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.scales + (size_t)n0 * a.ngroups), (short)0, nrows * a.ngroups * 2, 0x00020000);
  int x_off[8], w_off[2], z_off[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = tid + 256 * i;
    x_off[i] = ((p >> 4) * a.K + 8 * (p & 15)) * 2;
  }
  // weight piece i of this thread: lane p & 63 of 16-row block p >> 6 in the
  // tiled order (row 16 (p >> 6) + (p & 15), codes 32 ((p & 63) >> 4) .. of
  // each 128-code tile); the k-block's advance is 1 KB per tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i;
    w_off[i] = ((p >> 6) * 2 * a.K + 4 * (p & 63)) * 4;
    z_off[i] = wpiece_row(p) * a.ngroups * 2;
  }
  const int s_off = tid * a.ngroups * 2;

  auto gload_guarded = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + 256 * i;
      const int r = p >> 4, j8 = p & 15;
      const int m = m0 + r, k = kb * BK + 8 * j8;
      xr[i] = (m < a.M && k < a.K) ? *(const u32x4_t *)(a.x + (size_t)m * a.K + k)
                                   : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int g = PERCH ? 0 : min((kb * BK) / a.G, a.ngroups - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int r = wpiece_row(p), q4 = wpiece_quarter(p);
      const int n = min(n0 + r, a.N - 1);
      const int k = kb * BK + 32 * q4;
      wr[i] = (k < a.K) ? *(const u32x4_t *)(tiled_block(a.qw, n0 + 16 * (p >> 6), a.N, a.K,
                                                         p & 63) + kb * 256)
                        : u32x4_t{0u, 0u, 0u, 0u};
      zr[i] = a.zeros[(size_t)n * a.ngroups + g];
    }
    if (!PERCH && tid < BN) sv = a.scales[(size_t)min(n0 + tid, a.N - 1) * a.ngroups + g];
  };
  auto gload = [&](int kb) {
    if (kb * BK + BK > a.K) {  // uniform
      gload_guarded(kb);
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xr[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rs, x_off[i], kb * BK * 2, 0);
    const int g = PERCH ? 0 : min((kb * BK) / a.G, a.ngroups - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      wr[i] = __builtin_amdgcn_raw_buffer_load_b128(w_rs, w_off[i], kb * 1024, 0);
      zr[i] = __builtin_amdgcn_raw_buffer_load_b16(z_rs, z_off[i], g * 2, 0);
    }
    if (!PERCH && tid < BN) sv = __builtin_amdgcn_raw_buffer_load_b16(s_rs, s_off, g * 2, 0);
  };


  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + 256 * i;
      const int r = p >> 4, j8 = p & 15;
      // fp16 weights come in dequant_word's pair order, bf16 in natural order
      *(u32x4_t *)(xs + r * LSTR + 8 * j8) = DT == DT_F16 ? permute_8(xr[i]) : xr[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int r = wpiece_row(p), q4 = wpiece_quarter(p);
      const uint32_t zc = zero_constant<DT>(zr[i]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *(u32x4_t *)(wsm + r * WSTR + 32 * q4 + 8 * t) =
            DT == DT_F16 ? dequant_word<DT>(wr[i][t], zc) : dequant_word_bf16_natural(wr[i][t], zc);
    }
    if (!PERCH && tid < BN) ss[tid] = (float)bitcast<_Float16>(sv);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one k-block from the staged tiles
  auto compute = [&]() {
    u32x4_t af[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        af[mi][t] = *(const u32x4_t *)(xs + (64 * wm + 16 * mi + col) * LSTR + 32 * t + 8 * h);

#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      u32x4_t bf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        bf[t] = *(const u32x4_t *)(wsm + (64 * wn + 16 * ni + col) * WSTR + 32 * t + 8 * h);
      if constexpr (PERCH) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[mi][ni] = mfma_16x16x32<DT>(af[mi][t], bf[t], acc[mi][ni]);
      } else {
        const float s = ss[64 * wn + 16 * ni + col];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          f32x4_t g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) g = mfma_16x16x32<DT>(af[mi][t], bf[t], g);
          acc[mi][ni] += s * g;
        }
      }
    }
  };

  // EPI operands of one rank chunk: this thread's 4 pieces of U (4 ranks of
  // a row each) and, when r % 8 == 0 and B is 16-byte aligned, its 2 pieces of
  // B (8 ranks of a row each; otherwise B is read value by value when the
  // chunk is staged).  epi_load reads them raw from clamped, valid addresses;
  // the staging selects zeros for rows past M or N and ranks past r.  The
  // first chunk is loaded during the last k-block, and as nothing reads the
  // registers before the staging, the loads stay in flight behind that
  // block's MFMAs.
  f32x4_t u_pre[4];
  u16x8_t b_pre[2];
  const bool bvec = (a.u.rank % 8) == 0 && ((uintptr_t)a.B % 16) == 0;
  // PROD: U is formed here from the producers' K-split sums (or, when the
  // wait for them expired, from this tile's own full sums in Tfb), exactly as
  // prefill_u_kernel forms it: each sum in split order, g = sigmoid(z + b_g)
  // from the gate row, u = g t.  The sums are read with the sc1 policy, which
  // reads across the XCDs' L2 caches.
  bool expired = false;
  float gv[4] = {0.f, 0.f, 0.f, 0.f};
  auto epi_load = [&](int j0) {
    const UView &u = a.u;
    if constexpr (PROD) {
      const float *T = expired ? a.Tfb : a.ec.Tp;
      const int ks = expired ? 1 : a.ec.ks;
      const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
          (void *)T, (short)0, ks * a.M * u.rp1 * 4, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i;  // BM rows x 8 pieces
        const int r = p >> 3, j = min(j0 + 4 * (p & 7), u.rp1 - 4);
        const int m = min(m0 + r, a.M - 1);
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
        float z = 0.f;
        for (int q0 = 0; q0 < ks; q0 += 4) {  // four splits' loads in flight at a time
          f32x4_t tv[4];
          float zv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = (min(q0 + q, ks - 1) * a.M + m) * u.rp1;
            tv[q] = bitcast<f32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(tr, (row + j) * 4, 0, 16));
            zv[q] = j0 == 0 ? bitcast<float>(__builtin_amdgcn_raw_buffer_load_b32(
                                  tr, (row + u.rank) * 4, 0, 16))
                            : 0.f;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q0 + q < ks) {
              t += tv[q];
              z += zv[q];
            }
        }
        if (j0 == 0) gv[i] = gate_sigmoid(z + a.ec.b_gate);
#pragma unroll
        for (int c = 0; c < 4; ++c) u_pre[i][c] = (j + c < u.rank) ? gv[i] * t[c] : 0.f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i;  // BM rows x 8 pieces
        const int r = p >> 3, j = j0 + 4 * (p & 7);
        u_pre[i] = *(const f32x4_t *)(u.U + (size_t)min(m0 + r, a.M - 1) * u.rp1 + min(j, u.rp1 - 4));
      }
    }
    if (bvec) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int p = tid + 256 * i;  // BN rows x 4 pieces of 8 ranks
        const int r = p >> 2, j = j0 + 8 * (p & 3);
        b_pre[i] = *(const u16x8_t *)(a.B + (size_t)min(n0 + r, a.N - 1) * u.rank + min(j, u.rank - 8));
      }
    }
  };

  // this workgroup's k-blocks: all of them, or split `split` of ks; the
  // last one is peeled off, as it loads the epilogue's operands instead of a
  // next block
  int kb_lo = 0, kb_hi = nkb;
  if constexpr (SPLIT) {
    const int per = (nkb + a.ks - 1) / a.ks;
    kb_lo = min(nkb, split * per);
    kb_hi = min(nkb, kb_lo + per);
  }
  // PROD: wave 0 reads the producers' count two blocks before the last one,
  // so that the value is in by the last block
  uint32_t arrived = 0;
  if (kb_lo < kb_hi) gload(kb_lo);
  for (int kb = kb_lo; kb + 1 < kb_hi; ++kb) {
    if constexpr (PROD) {
      if (wave == 0 && kb == max(kb_lo, kb_hi - 3))
        arrived = __hip_atomic_load(&a.hdr->arrive.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    lstore();
    __syncthreads();
    gload(kb + 1);
    compute();
  }
  if constexpr (PROD) {
    // If every producer was in when wave 0 read the count (a single block:
    // read now), the epilogue's sums are loaded before the last block's MFMAs,
    // behind which they stay in flight.  Otherwise the count is polled after
    // them: a bounded wait (spin_limit polls), and on expiry this tile
    // computes the sums of its tokens itself.
    if (wave == 0 && kb_hi - kb_lo < 2)
      arrived = __hip_atomic_load(&a.hdr->arrive.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool early = false;
    if (kb_lo < kb_hi) {
      __syncthreads();
      lstore();
      if (tid == 0) vote = (a.spin_limit > 0 && arrived >= (uint32_t)a.nprod) ? 2 : 0;
      __syncthreads();
      early = vote == 2;
      if (early && a.u.rank > 0) epi_load(0);
      compute();
    }
    if (!early && tid == 0) {
      // (a limit of 0 polls: no wait at all, every tile computes its own sums)
      int ex = a.spin_limit == 0 ? 1 : 0;
      for (uint32_t it = 0; !ex && arrived < (uint32_t)a.nprod; ++it) {
        if (it >= a.spin_limit) {
          ex = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        arrived = __hip_atomic_load(&a.hdr->arrive.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (ex)
        __hip_atomic_fetch_or(&a.hdr->flags.v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      vote = ex;
    }
    __syncthreads();
    expired = !early && vote == 1;
    if (expired) {
      // [A; w_g] x over all of K for this tile's tokens, into Tfb (tiles of
      // one token band write the same values there, computed the same way)
      const EcArgs &e = a.ec;
      const int nval = min(BM, a.M - m0) * e.rows;
      for (int i = tid; i < nval; i += 256) {
        const int mm = i / e.rows, j = i - mm * e.rows;
        const uint16_t *arow = j < e.rank ? e.A + (size_t)j * a.K : e.wg;
        const uint16_t *xrow = a.x + (size_t)(m0 + mm) * a.K;
        float t = 0.f;
        for (int k = 0; k < a.K; k += 8) {
          const u16x8_t av = *(const u16x8_t *)(arow + k);
          const u16x8_t xv = *(const u16x8_t *)(xrow + k);
#pragma unroll
          for (int c = 0; c < 8; ++c) t += to_f32<DT>(av[c]) * to_f32<DT>(xv[c]);
        }
        a.Tfb[(size_t)(m0 + mm) * e.rp1 + j] = t;
      }
      stores_done();
      __syncthreads();
    }
    if (!early && a.u.rank > 0) epi_load(0);
  } else if (kb_lo < kb_hi) {
    __syncthreads();
    lstore();
    __syncthreads();
    if constexpr (EPI) {
      if (a.u.rank > 0) epi_load(0);
    }
    compute();
  } else if constexpr (EPI) {
    if (a.u.rank > 0) epi_load(0);
  }

  if constexpr (SPLIT) {
    // this split's fp32 partial tile; the finish kernel sums the splits
    float *P = a.part + (size_t)split * a.M * a.N;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int n = n0 + 64 * wn + 16 * ni + col;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + 64 * wm + 16 * mi + 4 * h + e;
          if (m < a.M && n < a.N) P[(size_t)m * a.N + n] = acc[mi][ni][e];
        }
    }
    return;
  }

  if constexpr (PERCH) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int n = min(n0 + 64 * wn + 16 * ni + col, a.N - 1);
      const float s = (float)bitcast<_Float16>(a.scales[n]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) acc[mi][ni] *= s;
    }
  }

  if constexpr (EPI) {
    // y tile += U[m0.., :] B[n0.., :]^T, kEpiRc ranks at a time staged in the
    // (now free) LDS tiles as bf16 pairs: hi = the value rounded to bf16, lo =
    // the remainder rounded to bf16.  U hi and lo times B (hi and lo when B is
    // fp16, which the pair holds exactly) in 16x16x32 bf16 MFMAs with fp32
    // accumulation give U B^T to a relative 2^-16.  Rows past M or N and
    // ranks past r stage zeros.
    const UView &u = a.u;
    uint16_t *uh = xs, *ul = xs + BM * kEpiStr;
    uint16_t *bh = wsm, *bl = wsm + BN * kEpiStr;
    for (int j0 = 0; j0 < u.rank; j0 += kEpiRc) {
      if (j0 > 0) epi_load(j0);
      __syncthreads();  // the tiles' (or the previous chunk's) last readers are done
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i;
        const int r = p >> 3, q = p & 7;
        const bool in = m0 + r < a.M && j0 + 4 * q < u.rp1;
        uint16_t hv[4], lv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) split_bf16(in ? u_pre[i][c] : 0.f, hv[c], lv[c]);
        *(uint2 *)(uh + r * kEpiStr + 4 * q) =
            uint2{hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16)};
        *(uint2 *)(ul + r * kEpiStr + 4 * q) =
            uint2{lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16)};
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // value i of this thread: rank jj of row r (two 8-rank pieces when
        // prefetched, else one value per row-rank slot, loaded now)
        int r, jj;
        uint16_t v;
        if (bvec) {
          const int p = tid + 256 * (i >> 3);
          r = p >> 2;
          jj = 8 * (p & 3) + (i & 7);
          v = b_pre[i >> 3][i & 7];
        } else {
          const int p = tid + 256 * i;
          r = p / kEpiRc;
          jj = p - r * kEpiRc;
          v = a.B[(size_t)min(n0 + r, a.N - 1) * u.rank + min(j0 + jj, u.rank - 1)];
        }
        if (n0 + r >= a.N || j0 + jj >= u.rank) v = 0;
        if constexpr (DT == DT_BF16) {
          bh[r * kEpiStr + jj] = v;
        } else {
          uint16_t hv, lv;
          split_bf16(to_f32<DT>(v), hv, lv);
          bh[r * kEpiStr + jj] = hv;
          bl[r * kEpiStr + jj] = lv;
        }
      }
      __syncthreads();
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int ro = (64 * wm + 16 * mi + col) * kEpiStr + 8 * h;
        const u32x4_t ah = *(const u32x4_t *)(uh + ro);
        const u32x4_t al = *(const u32x4_t *)(ul + ro);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int co = (64 * wn + 16 * ni + col) * kEpiStr + 8 * h;
          const u32x4_t b0 = *(const u32x4_t *)(bh + co);
          acc[mi][ni] = mfma_16x16x32<DT_BF16>(ah, b0, acc[mi][ni]);
          acc[mi][ni] = mfma_16x16x32<DT_BF16>(al, b0, acc[mi][ni]);
          if constexpr (DT == DT_F16) {
            const u32x4_t b1 = *(const u32x4_t *)(bl + co);
            acc[mi][ni] = mfma_16x16x32<DT_BF16>(ah, b1, acc[mi][ni]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int n = n0 + 64 * wn + 16 * ni + col;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 64 * wm + 16 * mi + 4 * h + e;
        if (m < a.M && n < a.N) a.y[(size_t)m * a.N + n] = from_f32<DT>(acc[mi][ni][e]);
      }
    }
  }
  if constexpr (PROD) {
    if (tid == 0) prod_finish(a.hdr);  // every workgroup of the launch counts itself out
  }
}


// The pages' per-rank gate: for each token, t = the sum of its split
// partials (rows 0..rank-1, split order), hidden = relu(W1 t + b1),
// gamma = sigmoid(W2 hidden + b2), and U[m][j] = alpha gamma_j t_j, with
// zeros in columns rank .. rp1-1.
struct RgArgs {
  const float *Tp;
  float *Ts;  // U: [M][rp1]
  int ks, M, rank, rp1, hidden;
  const float *W1, *b1, *W2, *b2;
  float alpha;
};
constexpr int kRgTok = 8;  // tokens per workgroup

__global__ __launch_bounds__(256) void prefill_rgate_kernel(RgArgs a) {
  __shared__ float tl[kRgTok][SPEAR_MAX_RANK + 1];
  __shared__ float hl[kRgTok][SPEAR_MAX_GATE_HIDDEN + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kRgTok;
  for (int i = tid; i < kRgTok * a.rank; i += 256) {
    const int mm = i / a.rank, j = i - mm * a.rank;
    float t = 0.f;
    if (m0 + mm < a.M) t = split_sum(a.Tp + (size_t)(m0 + mm) * a.rp1 + j, (size_t)a.M * a.rp1, a.ks);
    tl[mm][j] = t;
  }
  __syncthreads();
  for (int i = tid; i < kRgTok * a.hidden; i += 256) {
    const int mm = i / a.hidden, c = i - mm * a.hidden;
    float v = a.b1[c];
    for (int k = 0; k < a.rank; ++k) v += a.W1[(size_t)c * a.rank + k] * tl[mm][k];
    hl[mm][c] = v > 0.f ? v : 0.f;
  }
  __syncthreads();
  for (int i = tid; i < kRgTok * a.rank; i += 256) {
    const int mm = i / a.rank, j = i - mm * a.rank;
    const int m = m0 + mm;
    if (m >= a.M) continue;
    float v = a.b2[j];
    for (int c = 0; c < a.hidden; ++c) v += a.W2[(size_t)j * a.hidden + c] * hl[mm][c];
    a.Ts[(size_t)m * a.rp1 + j] = a.alpha * gate_sigmoid(v) * tl[mm][j];
  }
  for (int i = tid; i < kRgTok * (a.rp1 - a.rank); i += 256) {
    const int mm = i / (a.rp1 - a.rank), j = a.rank + i - mm * (a.rp1 - a.rank);
    if (m0 + mm < a.M) a.Ts[(size_t)(m0 + mm) * a.rp1 + j] = 0.f;
  }
}

// U = diag(g) (X A^T) from the compensator's split partials: for token m,
// t_j = sum_q Tp[q][m][j] (j < rank) and z = the same sum of row rank, each
// in split order; g = sigmoid(z + b_g); U[m][j] = g t_j, and zeros in
// columns rank .. rp1-1.  One thread per 4-column piece.
struct UArgs {
  const float *Tp;
  float *U;  // [M][rp1]
  int ks, M, rank, rp1;
  float b_gate;
};

__global__ __launch_bounds__(256) void prefill_u_kernel(UArgs a) {
  const int q4 = a.rp1 / 4;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.M * q4) return;
  const int m = i / q4, j = 4 * (i - m * q4);
  const float *row = a.Tp + (size_t)m * a.rp1;
  const size_t stride = (size_t)a.M * a.rp1;
  // up to 64 splits: 16 loads of each kind in flight per round
  const f32x4_t t = split_sum4<16>(row + j, stride, a.ks);
  const float z = split_sum<16>(row + a.rank, stride, a.ks);
  const float g = gate_sigmoid(z + a.b_gate);
  f32x4_t u;
#pragma unroll
  for (int c = 0; c < 4; ++c) u[c] = (j + c < a.rank) ? g * t[c] : 0.f;
  *(f32x4_t *)(a.U + (size_t)m * a.rp1 + j) = u;
}

// ---------------------------------------------------------------------------
// Finish a 64-token x 64-output tile:
//   y[m][n] = round( base[m][n] + sum_j U[m][j] B[n][j] )
// where base is the sum of the GEMM's split partials in split order (times
// the row's scale when one scale covers the row) or, in the concurrent
// schedule, the GEMM's rounded y; the U B^T term is present when the layer
// has a compensator.  The base tile, the U rows and the B rows are staged in
// LDS; four waves each
// take 16 tokens with fp32 16x16x4 MFMAs; y goes back in 16-byte stores when
// its rows are 16-byte aligned.
// ---------------------------------------------------------------------------
struct FinishArgs {
  uint16_t *y;
  const float *part;  // PARTS: [ks][M][N]
  int ks;
  const uint16_t *scales;  // PARTS && PERCH: [N]
  UView u;                 // EC
  const uint16_t *B;       // EC: [N][rank]
  int N, M;
};

constexpr int kFT = 64;              // tokens and outputs per tile
constexpr int kFStr = kFT + 4;       // fp32 base tile row stride
constexpr int kFRc = 32;             // ranks per chunk
constexpr int kFRStr = kFRc + 4;

template <int DT, bool PARTS, bool PERCH, bool EC>
__global__ __launch_bounds__(256) void prefill_finish_kernel(FinishArgs a) {
  __shared__ __align__(16) float ts[kFT][kFStr];
  __shared__ __align__(16) float us[kFT][kFRStr];
  __shared__ __align__(16) float bs[kFT][kFRStr];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * kFT, m0 = blockIdx.y * kFT;

  // EC: this thread's share of a rank chunk, 2 pieces of U (4 ranks of a
  // row) and 8 values of B, read raw from clamped, valid addresses and masked
  // when staged.  Chunk 0 is loaded first, so that its loads are in flight
  // with the base tile's.
  f32x4_t u_pre[2];
  uint16_t b_pre[8];
  auto ec_load = [&](int j0) {
    const UView &e = a.u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;  // 64 rows x 8 pieces
      const int r = p >> 3, j = j0 + 4 * (p & 7);
      u_pre[i] = *(const f32x4_t *)(e.U + (size_t)min(m0 + r, a.M - 1) * e.rp1 + min(j, e.rp1 - 4));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + 256 * i;  // 64 rows x 32 ranks
      const int r = p >> 5, j = j0 + (p & 31);
      b_pre[i] = a.B[(size_t)min(n0 + r, a.N - 1) * e.rank + min(j, e.rank - 1)];
    }
  };
  if constexpr (EC) {
    if (a.u.rank > 0) ec_load(0);
  }

  // --- base tile: 64 rows x 16 pieces of 4
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    const int r = p >> 4, c4 = (p & 15) * 4;
    const int m = m0 + r, n = n0 + c4;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (m < a.M) {
      if constexpr (PARTS) {
        const bool vec = (a.N % 4) == 0 && n + 4 <= a.N;
        const float *src = a.part + (size_t)m * a.N + n;
        const size_t stride = (size_t)a.M * a.N;
        if (vec) {
          v = split_sum4(src, stride, a.ks);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (n + c < a.N) v[c] = split_sum(src + c, stride, a.ks);
        }
        if constexpr (PERCH) {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            v[c] *= (n + c < a.N) ? (float)bitcast<_Float16>(a.scales[n + c]) : 0.f;
        }
      } else if ((a.N % 4) == 0 && n + 4 <= a.N && ((uintptr_t)a.y % 8) == 0) {
        const uint2 w = *(const uint2 *)(a.y + (size_t)m * a.N + n);  // 4 values in one load
        v = f32x4_t{to_f32<DT>((uint16_t)w.x), to_f32<DT>((uint16_t)(w.x >> 16)),
                    to_f32<DT>((uint16_t)w.y), to_f32<DT>((uint16_t)(w.y >> 16))};
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          v[c] = (n + c < a.N) ? to_f32<DT>(a.y[(size_t)m * a.N + n + c]) : 0.f;
      }
    }
    *(f32x4_t *)&ts[r][c4] = v;
  }

  if constexpr (EC) {
    const UView &e = a.u;
    for (int j0 = 0; j0 < e.rank; j0 += kFRc) {
      if (j0 > 0) ec_load(j0);
      __syncthreads();  // base tile written; the previous chunk's readers are done
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int p = tid + 256 * i;  // 64 rows x 8 pieces
        const int r = p >> 3, q = p & 7;
        const bool in = m0 + r < a.M && j0 + 4 * q < e.rp1;
        *(f32x4_t *)&us[r][4 * q] = in ? u_pre[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = tid + 256 * i;  // 64 rows x 32 ranks
        const int r = p >> 5, jj = p & 31;
        bs[r][jj] = (n0 + r < a.N && j0 + jj < e.rank) ? to_f32<DT>(b_pre[i]) : 0.f;
      }
      __syncthreads();
      const int tk = 16 * wave + col;  // A-operand row (token) of this lane
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        f32x4_t acc;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = ts[16 * wave + 4 * h + c][16 * nb + col];
#pragma unroll
        for (int st = 0; st < kFRc / 4; ++st) {
          const int j = 4 * st + h;
          acc = mfma_16x16x4_f32(us[tk][j], bs[16 * nb + col][j], acc);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) ts[16 * wave + 4 * h + c][16 * nb + col] = acc[c];
      }
    }
  }
  __syncthreads();

  // --- round and store: 64 rows x 8 pieces of 8
  const bool yvec = (a.N % 8) == 0 && ((uintptr_t)a.y % 16) == 0;  // y itself need only be 2-byte aligned
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i;
    const int r = p >> 3, c8 = (p & 7) * 8;
    const int m = m0 + r, n = n0 + c8;
    if (m < a.M) {
      u16x8_t t;
#pragma unroll
      for (int c = 0; c < 8; ++c) t[c] = from_f32<DT>(ts[r][c8 + c]);
      if (yvec && n + 8 <= a.N) {
        *(u16x8_t *)(a.y + (size_t)m * a.N + n) = t;
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (n + c < a.N) a.y[(size_t)m * a.N + n + c] = t[c];
      }
    }
  }
}

struct StreamEvents {
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_event_mu;
std::unordered_map<int, StreamEvents> g_events;

hipError_t get_events(StreamEvents **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  StreamEvents &ev = g_events[dev];
  if (!ev.fork) {
    e = hipEventCreateWithFlags(&ev.fork, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    e = hipEventCreateWithFlags(&ev.join, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  *out = &ev;
  return hipSuccess;
}

}  // namespace

static int rank_pad(int rank) { return (rank + 3) / 4 * 4; }
static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Compensator K splits: about 256 workgroups of 32 tokens, at least one
// 32-wide step per wave, at most 64.  ks * ceil(M / 32) <= 256 + ceil(M / 32)
// bounds the partials.
static int ec_ksplit(int M, int K) {
  const int nblk = (M + kEcTok - 1) / kEcTok;
  int ks = (256 + nblk - 1) / nblk;
  if (ks > 64) ks = 64;
  const int cap = (K / 32) / kEcWaves;
  if (ks > cap) ks = cap;
  return ks < 1 ? 1 : ks;
}

// K splits of the compensator producers inside the GEMM launch (four waves
// each): enough producer workgroups to keep about 256 busy, at most 8 splits
// (a tile's epilogue reads every split of its sums) and at least 4 waves x 32
// columns of K per split.
static int fused_ksplit(int M, int K) {
  const int nblk = (M + kEcTok - 1) / kEcTok;
  int ks = (256 + nblk - 1) / nblk;
  if (ks > 8) ks = 8;
  const int cap = (K / 32) / 4;
  if (ks > cap) ks = cap;
  return ks < 1 ? 1 : ks;
}

// The K-split GEMM with the compensator's producers in its launch (SPROD):
// the scalar gate, at most kMaxSplitTiles token blocks (one header counter
// each), and K up to 16384: past it the producers' K-splits (at most 8) run
// long and hold CU slots the tiles wait for (measured at 28672 -> 8192,
// M = 256: 175.9 against 163.3 us in four launches; 8192^2: 68.3 against
// 71.9, and the 7B shapes 7-21% faster).  Its producers' K-splits.
constexpr int kSprodMaxK = 16384;
static bool sprod_form(const LayerDesc &L, int M, int gks) {
  return L.rank > 0 && L.rg_hidden == 0 && gks > 1 && (M + kEcTok - 1) / kEcTok <= kMaxSplitTiles &&
         L.K <= kSprodMaxK;
}
static int sprod_ksplit(int M, int K) { return std::min(fused_ksplit(M, K), kMaxFusedSplits); }

// GEMM K splits: when the output has too few 128x128 tiles to fill the chip,
// split K so that about kGemmSplitWgs workgroups run, each with at least 4
// k-blocks and none empty.  ks * tiles <= kGemmSplitWgs bounds the partials.
constexpr int kGemmSplitWgs = 512;
static int gemm_ksplit(int M, int N, int K) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int nkb = (K + BK - 1) / BK;
  if (tiles >= kGemmSplitWgs * 3 / 4) return 1;
  int ks = kGemmSplitWgs / tiles;
  if (ks > nkb / 4) ks = nkb / 4;
  if (ks > 16) ks = 16;
  if (ks < 2) return 1;
  const int per = (nkb + ks - 1) / ks;
  return (nkb + per - 1) / per;  // no empty split
}

// The GEMM's K splits in the SPROD form: one fewer (not below 2) when the
// split tiles alone take all kGemmSplitWgs resident workgroups, where the
// producers ahead of them would push tiles to a second round.  Measured at
// M = 256: 8192^2 61.5 against 67.0 us, 4096^2 29.9 against 34.7; at M = 288,
// whose 480 split tiles leave room, the same cut lost 4-11%.
static int sprod_gemm_ksplit(int M, int N, int K, int gks) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int nkb = (K + BK - 1) / BK;
  int ks = gks;
  if (ks > 2 && tiles * ks >= kGemmSplitWgs) --ks;
  const int per = (nkb + ks - 1) / ks;
  return (nkb + per - 1) / per;
}

// Rows of a ragged tail.  An unsplit GEMM whose tiles are a few more than a
// whole number of workgroups per CU (256 CUs) leaves the CUs that get one
// more tile working while the rest wait: with 288 tiles, 32 CUs hold two
// workgroups and take up to twice as long.  Its last tile rows then go to a
// K-split GEMM of their own, whose workgroups are short, and to the finish
// kernel.  Returns how many rows that is (0: none): the rows past the whole
// tile rows that fit the whole number of workgroups per CU, when their tiles
// are at most a quarter of the CUs and can be split.
constexpr int kGemmCus = 256;
static int prefill_tail_rows(int M, int N, int K) {
  const int ntn = (N + BN - 1) / BN, ntm = (M + BM - 1) / BM;
  const int T = ntn * ntm;
  if (T <= kGemmCus || gemm_ksplit(M, N, K) > 1) return 0;
  const int main_tile_rows = (T / kGemmCus) * kGemmCus / ntn;
  const int tail_tiles = T - main_tile_rows * ntn;
  if (main_tile_rows == 0 || tail_tiles == 0 || tail_tiles * 4 > kGemmCus) return 0;
  const int tail = M - main_tile_rows * BM;
  return gemm_ksplit(tail, N, K) > 1 ? tail : 0;
}

// Bytes of the GEMM's split partials [ks][m][N] fp32 that any call with 1..M
// tokens stores: a K-split GEMM over all m rows, or over the ragged tail's
// rows.  ks depends on m only through its tile rows, so ks m peaks at the
// last m of each band of 128 rows; both loops stop where no split happens
// (the output fills the chip, or the tail exceeds a quarter of the CUs).
static size_t gemm_partial_bytes(int M, int N, int K) {
  const int ntn = (N + BN - 1) / BN;
  size_t most = 0;
  for (int tr = 1; (tr - 1) * BM < M && tr * ntn < kGemmSplitWgs * 3 / 4; ++tr) {
    const int m = std::min(M, tr * BM);
    const int ks = gemm_ksplit(m, N, K);
    if (ks > 1) most = std::max(most, (size_t)ks * m * N * sizeof(float));
  }
  for (int tr = 1; (tr - 1) * BM < M && tr * ntn * 4 <= kGemmCus; ++tr) {
    const int t = std::min(M, tr * BM);  // tail rows of at most tr tile rows
    const int ks = gemm_ksplit(t, N, K);
    if (ks > 1) most = std::max(most, (size_t)ks * t * N * sizeof(float));
  }
  return most;
}

// Workspace layout after the header: the compensator's split partials
// [ks][M][rp1], U [M][rp1] formed from them, and the GEMM's split partials
// (at most kGemmSplitWgs tiles of 128 x 128 fp32, and only as many as a call
// with at most M tokens can split into).  All are rewritten in full by every
// call before they are read and are sized by bounds that grow with M, so a
// workspace for M serves every call with fewer tokens, and any other layer
// whose size it covers.
struct PrefillWs {
  size_t tp, ts, gpart, end;
};
static PrefillWs prefill_ws_layout(const LayerDesc &L, int M) {
  PrefillWs w;
  w.tp = kWsDataOff;
  const size_t rp1 = rank_pad(L.rank + 1);
  const size_t nblk = (M + kEcTok - 1) / kEcTok;
  const size_t tb = L.rank > 0 ? round256((256 + nblk) * kEcTok * rp1 * sizeof(float)) : 0;
  const size_t sb = L.rank > 0 ? round256((size_t)M * rp1 * sizeof(float)) : 0;
  w.ts = w.tp + tb;
  w.gpart = w.ts + sb;
  w.end = w.gpart + round256(gemm_partial_bytes(M, L.N, L.K));
  return w;
}

size_t prefill_workspace_bytes(const LayerDesc &L, int M) { return prefill_ws_layout(L, M).end; }

bool prefill_needs_workspace(const LayerDesc &L) { return L.rank > 0; }

// Tokens at the end of an M-token call that the phase-aware dispatch hands
// to the decode path: the r = M mod BM tokens of a last, partly filled tile
// row, when r <= kDecodeTailMax and at least kDecodeTailRows full tile rows
// come before them.  That tile row costs the GEMM a whole row of 128-token
// tiles (a ninth, at eight full rows) for r tokens, while the fused decode
// handles r <= 32 tokens in about the time of streaming the weights once;
// measured on the serving stack's merged batches (a 1024-token chunk plus 32
// decode tokens: 13.3 ms a step in one GEMM, 11.6 ms in two calls), while at
// 256 and 512 tokens the single GEMM stays ahead.  0: no split.
constexpr int kDecodeTailMax = 32;
constexpr int kDecodeTailRows = 8;
int prefill_decode_tail(int M) {
  const int r = M % BM;
  return (r >= 1 && r <= kDecodeTailMax && M - r >= kDecodeTailRows * BM) ? r : 0;
}

void describe_prefill(const LayerDesc &L, int M, size_t ws_bytes, spear_plan_t *out) {
  int gks = ws_bytes > 0 ? gemm_ksplit(M, L.N, L.K) : 1;
  if (sprod_form(L, M, gks))
    gks = sprod_gemm_ksplit(M, L.N, L.K, gks);
  const int tail = (ws_bytes > 0 && gks == 1) ? prefill_tail_rows(M, L.N, L.K) : 0;
  const int ntn = (L.N + BN - 1) / BN;
  out->path = SPEAR_PATH_PREFILL;
  out->workgroups = ntn * ((M - tail + BM - 1) / BM) * gks;
  out->waves_per_workgroup = 4;
  out->producers = 0;
  if (sprod_form(L, M, gks)) {  // producers ahead of the split tiles, in multiples of 8
    out->producers = (M + kEcTok - 1) / kEcTok * sprod_ksplit(M, L.K);
    out->workgroups += (out->producers + 7) / 8 * 8;
  }
  out->k_splits = gks;
  out->workspace_bytes = prefill_needs_workspace(L) ? prefill_workspace_bytes(L, M) : 0;
}

template <int DT, bool PERCH>
static void launch_gemm(const GemmArgs &g, dim3 grid, bool epi, hipStream_t s) {
  if (grid.z > 1)
    hipLaunchKernelGGL((prefill_gemm_kernel<DT, PERCH, false, true>), grid, dim3(256), 0, s, g);
  else if (epi)
    hipLaunchKernelGGL((prefill_gemm_kernel<DT, PERCH, true, false>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<DT, PERCH, false, false>), grid, dim3(256), 0, s, g);
}

template <int DT, bool PARTS>
static void launch_finish(const FinishArgs &f, dim3 grid, bool perch, bool ec, hipStream_t s) {
  if (perch && ec)
    hipLaunchKernelGGL((prefill_finish_kernel<DT, PARTS, true, true>), grid, dim3(256), 0, s, f);
  else if (perch)
    hipLaunchKernelGGL((prefill_finish_kernel<DT, PARTS, true, false>), grid, dim3(256), 0, s, f);
  else if (ec)
    hipLaunchKernelGGL((prefill_finish_kernel<DT, PARTS, false, true>), grid, dim3(256), 0, s, f);
  else
    hipLaunchKernelGGL((prefill_finish_kernel<DT, PARTS, false, false>), grid, dim3(256), 0, s, f);
}

// U = diag(g) (X A^T) (or the per-rank gate's U) [M][rp1] from K-split sums
// [ks][M][rp1] of [A; w_g] x, each summed in split order.
hipError_t launch_form_u(const LayerDesc &L, const float *Tp, int ks, int M, float *U,
                         hipStream_t s) {
  const int rp1 = rank_pad(L.rank + 1);
  if (L.rg_hidden > 0) {
    const RgArgs ra{Tp, U, ks, M, L.rank, rp1, L.rg_hidden, L.rg_W1, L.rg_b1, L.rg_W2, L.rg_b2,
                    L.rg_alpha};
    hipLaunchKernelGGL(prefill_rgate_kernel, dim3((M + kRgTok - 1) / kRgTok), dim3(256), 0, s, ra);
    return hipGetLastError();
  }
  const UArgs ua{Tp, U, ks, M, L.rank, rp1, L.b_gate};
  const int n = M * (rp1 / 4);
  hipLaunchKernelGGL(prefill_u_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ua);
  return hipGetLastError();
}

// y = round(sum over ks splits of part [ks][M][N] (times the row's scale when
// scale_rows) + U B^T when U is given), in 64 x 64 tiles.
hipError_t launch_finish_parts(const LayerDesc &L, int dtype, uint16_t *y, int M, const float *part,
                               int ks, const float *U, bool scale_rows, hipStream_t s) {
  const UView uv = U ? UView{U, M, L.rank, rank_pad(L.rank + 1)} : UView{};
  const FinishArgs fa{y, part, ks, L.scales, uv, L.B, L.N, M};
  const dim3 fgrid((L.N + kFT - 1) / kFT, (M + kFT - 1) / kFT);
  if (dtype == DT_F16)
    launch_finish<DT_F16, true>(fa, fgrid, scale_rows, U != nullptr, s);
  else
    launch_finish<DT_BF16, true>(fa, fgrid, scale_rows, U != nullptr, s);
  return hipGetLastError();
}

hipError_t launch_prefill(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                          void *ws, hipStream_t main_s, hipStream_t aux_s) {
  const bool ec = L.rank > 0;
  const bool concurrent = ec && aux_s != nullptr && aux_s != main_s;
  const PrefillWs w = prefill_ws_layout(L, M);
  char *base = (char *)ws;
  UView uv{};
  EcArgs ea{};
  int eks = 1;
  const bool rgate = ec && L.rg_hidden > 0;
  if (ec) {
    const int rp1 = rank_pad(L.rank + 1);
    eks = ec_ksplit(M, L.K);
    ea = EcArgs{x, L.A, L.wg, L.K, M, L.rank, L.rank + L.gate_rows(), rp1, eks, (float *)(base + w.tp),
                (eks == 1 && !rgate) ? (float *)(base + w.ts) : nullptr, L.b_gate};
    // consumers read U, formed once from the split partials
    uv = UView{(const float *)(base + w.ts), M, L.rank, rp1};
  }
  // split K only with a workspace (a rank-0 call may come without one)
  int gks = ws ? gemm_ksplit(M, L.N, L.K) : 1;
  if (sprod_form(L, M, gks))
    gks = sprod_gemm_ksplit(M, L.N, L.K, gks);
  const bool split = gks > 1;
  GemmArgs g{L.qw, L.scales, L.zeros, x, y, L.N, L.K, L.G, L.ngroups, M, uv, L.B, gks,
             split ? (float *)(base + w.gpart) : nullptr};
  const dim3 ggrid((L.N + BN - 1) / BN, (M + BM - 1) / BM, gks);
  const dim3 egrid(((M + kEcTok - 1) / kEcTok) * eks);
  const dim3 fgrid((L.N + kFT - 1) / kFT, (M + kFT - 1) / kFT);
  FinishArgs fa{y, g.part, gks, L.scales, uv, L.B, L.N, M};
  hipError_t e = hipSuccess;

  auto launch_ec = [&](hipStream_t s) {
    if (dtype == DT_F16)
      hipLaunchKernelGGL(prefill_ec_kernel<DT_F16>, egrid, dim3(64 * kEcWaves), 0, s, ea);
    else
      hipLaunchKernelGGL(prefill_ec_kernel<DT_BF16>, egrid, dim3(64 * kEcWaves), 0, s, ea);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess) return r;
    if (rgate) {
      const RgArgs ra{ea.Tp, (float *)(base + w.ts), eks, M, L.rank, ea.rp1, L.rg_hidden,
                      L.rg_W1, L.rg_b1, L.rg_W2, L.rg_b2, L.rg_alpha};
      hipLaunchKernelGGL(prefill_rgate_kernel, dim3((M + kRgTok - 1) / kRgTok), dim3(256), 0, s, ra);
      return hipGetLastError();
    }
    if (ea.U) return hipSuccess;  // U written by the compensator kernel
    const UArgs ua{ea.Tp, (float *)(base + w.ts), eks, M, L.rank, ea.rp1, L.b_gate};
    const int n = M * (ea.rp1 / 4);
    hipLaunchKernelGGL(prefill_u_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ua);
    return hipGetLastError();
  };
  // the GEMM, then (split) the finish kernel over the partials; `epi` adds
  // U B^T in the GEMM's own epilogue when it is not split
  auto launch_main = [&](bool with_ec) {
    const bool epi = with_ec && !split;
    if (dtype == DT_F16)
      L.per_channel ? launch_gemm<DT_F16, true>(g, ggrid, epi, main_s)
                    : launch_gemm<DT_F16, false>(g, ggrid, epi, main_s);
    else
      L.per_channel ? launch_gemm<DT_BF16, true>(g, ggrid, epi, main_s)
                    : launch_gemm<DT_BF16, false>(g, ggrid, epi, main_s);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess || !split) return r;
    if (dtype == DT_F16)
      launch_finish<DT_F16, true>(fa, fgrid, L.per_channel, with_ec, main_s);
    else
      launch_finish<DT_BF16, true>(fa, fgrid, L.per_channel, with_ec, main_s);
    return hipGetLastError();
  };

  // A K-split GEMM with the scalar gate (sprod_form): the compensator's
  // producers run in the GEMM launch ahead of its tiles (the producer that
  // completes a token block forms the block's U rows), and the finish kernel
  // adds U B^T: two launches on main_stream, in either schedule (the
  // producers overlap the GEMM inside its launch).
  if (sprod_form(L, M, gks)) {
    const int nblk = (M + kEcTok - 1) / kEcTok;
    GemmArgs gs = g;
    const int pks = sprod_ksplit(M, L.K);
    gs.ec = EcArgs{x, L.A, L.wg, L.K, M, L.rank, L.rank + 1, ea.rp1, pks, (float *)(base + w.tp),
                   nullptr, L.b_gate};
    gs.nprod_real = nblk * pks;
    gs.nprod = (gs.nprod_real + 7) / 8 * 8;
    gs.ntn = ggrid.x;
    gs.ntm = ggrid.y;
    gs.hdr = (WsHeader *)ws;
    const dim3 sg(gs.nprod + gs.ntn * gs.ntm * gks);
    if (dtype == DT_F16) {
      if (L.per_channel)
        hipLaunchKernelGGL((prefill_gemm_kernel<DT_F16, true, false, true, false, true>), sg,
                           dim3(256), 0, main_s, gs);
      else
        hipLaunchKernelGGL((prefill_gemm_kernel<DT_F16, false, false, true, false, true>), sg,
                           dim3(256), 0, main_s, gs);
    } else {
      if (L.per_channel)
        hipLaunchKernelGGL((prefill_gemm_kernel<DT_BF16, true, false, true, false, true>), sg,
                           dim3(256), 0, main_s, gs);
      else
        hipLaunchKernelGGL((prefill_gemm_kernel<DT_BF16, false, false, true, false, true>), sg,
                           dim3(256), 0, main_s, gs);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (dtype == DT_F16)
      launch_finish<DT_F16, true>(fa, fgrid, L.per_channel, true, main_s);
    else
      launch_finish<DT_BF16, true>(fa, fgrid, L.per_channel, true, main_s);
    return hipGetLastError();
  }

  if (!concurrent) {
    if (ec && (e = launch_ec(main_s)) != hipSuccess) return e;
    const int tail = ws ? prefill_tail_rows(M, L.N, L.K) : 0;
    if (tail == 0) return launch_main(ec);
    // rows [0, Mm): the unsplit GEMM (with U B^T in its epilogue when
    // compensated); rows [Mm, M): a K-split GEMM and the finish kernel
    const int Mm = M - tail;
    GemmArgs gm = g;
    gm.M = Mm;
    if (dtype == DT_F16)
      L.per_channel ? launch_gemm<DT_F16, true>(gm, dim3(ggrid.x, Mm / BM, 1), ec, main_s)
                    : launch_gemm<DT_F16, false>(gm, dim3(ggrid.x, Mm / BM, 1), ec, main_s);
    else
      L.per_channel ? launch_gemm<DT_BF16, true>(gm, dim3(ggrid.x, Mm / BM, 1), ec, main_s)
                    : launch_gemm<DT_BF16, false>(gm, dim3(ggrid.x, Mm / BM, 1), ec, main_s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int tks = gemm_ksplit(tail, L.N, L.K);
    const UView ut = ec ? UView{uv.U + (size_t)Mm * uv.rp1, tail, uv.rank, uv.rp1} : UView{};
    GemmArgs gt = g;
    gt.x = x + (size_t)Mm * L.K;
    gt.y = y + (size_t)Mm * L.N;
    gt.M = tail;
    gt.u = ut;
    gt.ks = tks;
    gt.part = (float *)(base + w.gpart);
    const dim3 tgrid(ggrid.x, (tail + BM - 1) / BM, tks);
    if (dtype == DT_F16)
      L.per_channel ? launch_gemm<DT_F16, true>(gt, tgrid, false, main_s)
                    : launch_gemm<DT_F16, false>(gt, tgrid, false, main_s);
    else
      L.per_channel ? launch_gemm<DT_BF16, true>(gt, tgrid, false, main_s)
                    : launch_gemm<DT_BF16, false>(gt, tgrid, false, main_s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const FinishArgs ft{gt.y, gt.part, tks, L.scales, ut, L.B, L.N, tail};
    const dim3 tfgrid((L.N + kFT - 1) / kFT, (tail + kFT - 1) / kFT);
    if (dtype == DT_F16)
      launch_finish<DT_F16, true>(ft, tfgrid, L.per_channel, ec, main_s);
    else
      launch_finish<DT_BF16, true>(ft, tfgrid, L.per_channel, ec, main_s);
    return hipGetLastError();
  }

  if (!rgate && !split) {
    // concurrent, scalar gate: the compensator's workgroups run inside the
    // GEMM launch, ahead of its tiles (the aux stream is not needed)
    const int nblk = (M + kEcTok - 1) / kEcTok;
    const EcArgs ep{x, L.A, L.wg, L.K, M, L.rank, L.rank + 1, ea.rp1, fused_ksplit(M, L.K),
                    (float *)(base + w.tp), nullptr, L.b_gate};
    GemmArgs gf = g;
    gf.nprod_real = nblk * ep.ks;
    gf.nprod = (gf.nprod_real + 7) / 8 * 8;
    gf.ntn = ggrid.x;
    gf.ntm = ggrid.y;
    gf.ec = ep;
    gf.hdr = (WsHeader *)ws;
    gf.spin_limit = get_decode_spin_limit();
    gf.Tfb = (float *)(base + w.ts);
    const dim3 fg(gf.nprod + gf.ntn * gf.ntm);
    if (dtype == DT_F16) {
      if (L.per_channel)
        hipLaunchKernelGGL((prefill_gemm_kernel<DT_F16, true, true, false, true>), fg, dim3(256), 0,
                           main_s, gf);
      else
        hipLaunchKernelGGL((prefill_gemm_kernel<DT_F16, false, true, false, true>), fg, dim3(256), 0,
                           main_s, gf);
    } else {
      if (L.per_channel)
        hipLaunchKernelGGL((prefill_gemm_kernel<DT_BF16, true, true, false, true>), fg, dim3(256), 0,
                           main_s, gf);
      else
        hipLaunchKernelGGL((prefill_gemm_kernel<DT_BF16, false, true, false, true>), fg, dim3(256),
                           0, main_s, gf);
    }
    return hipGetLastError();
  }

  // concurrent with the per-rank gate or a K-split GEMM: the compensator on
  // the aux stream alongside the GEMM; U B^T after the join
  std::lock_guard<std::mutex> lock(g_event_mu);
  StreamEvents *evs = nullptr;
  if ((e = get_events(&evs)) != hipSuccess) return e;
  if ((e = hipEventRecord(evs->fork, main_s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(aux_s, evs->fork, 0)) != hipSuccess) return e;
  if ((e = launch_ec(aux_s)) != hipSuccess) return e;
  if ((e = hipEventRecord(evs->join, aux_s)) != hipSuccess) return e;
  if (split) {
    // the finish kernel both sums the partials and adds U B^T: join first
    if (dtype == DT_F16)
      L.per_channel ? launch_gemm<DT_F16, true>(g, ggrid, false, main_s)
                    : launch_gemm<DT_F16, false>(g, ggrid, false, main_s);
    else
      L.per_channel ? launch_gemm<DT_BF16, true>(g, ggrid, false, main_s)
                    : launch_gemm<DT_BF16, false>(g, ggrid, false, main_s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(main_s, evs->join, 0)) != hipSuccess) return e;
    if (dtype == DT_F16)
      launch_finish<DT_F16, true>(fa, fgrid, L.per_channel, true, main_s);
    else
      launch_finish<DT_BF16, true>(fa, fgrid, L.per_channel, true, main_s);
    return hipGetLastError();
  }
  if ((e = launch_main(false)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(main_s, evs->join, 0)) != hipSuccess) return e;
  if (dtype == DT_F16)
    launch_finish<DT_F16, false>(fa, fgrid, false, true, main_s);
  else
    launch_finish<DT_BF16, false>(fa, fgrid, false, true, main_s);
  return hipGetLastError();
}

}  // namespace spear
