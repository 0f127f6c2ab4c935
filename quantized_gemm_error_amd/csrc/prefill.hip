// Prefill path: y = dequant(W_q) x + sigmoid(w_g . x + b_g) * B (A x) for
// many tokens (M in the hundreds to thousands).
//
// The pages run the compensator of the compute-bound prefill as a separate
// kernel that overlaps the low-bit GEMM instead of fusing it (SPEAR
// explanation page, Technical Summary 2.2 A, prefill phase).  Here:
//
//  * prefill_ec_kernel computes U = diag(g) (X A^T), g = sigmoid(X w_g + b_g),
//    into the workspace (fp32).  K is split over several workgroups per 16
//    tokens; the last split to finish sums the partials in a fixed order;
//  * prefill_gemm_kernel, a 128x128x128-tiled MFMA GEMM.  Each k-block stages
//    the activation tile and the exactly dequantized weight tile (q - z in
//    the activation type) in LDS; four waves each own a 64x64 quarter of the
//    output tile and run 16x16x32 MFMAs, applying each row's fp32 scale once
//    per 128-wide block (or once at the end when one scale covers the row).
//
// Two schedules:
//  * serial (no aux stream): the EC kernel, then the GEMM, whose epilogue adds
//    U B^T with fp32 16x16x4 MFMAs before y is rounded once.  On MI355X this
//    is the faster order: the GEMM's workgroups fill every CU, so a kernel on
//    another stream only runs as they retire;
//  * concurrent (aux stream given, the pages' schedule): the EC kernel on the
//    aux stream alongside the GEMM on the main stream, then, after joining,
//    prefill_merge_kernel adds U B^T to the rounded y.
#include <mutex>
#include <unordered_map>

#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LSTR = BK + 8;  // LDS row stride (halves), padded against bank conflicts

struct GemmArgs {
  const uint32_t *qw;
  const uint16_t *scales, *zeros;
  const uint16_t *x;
  uint16_t *y;
  int N, K, G, ngroups, M;
  const float *U;     // EPI: [M][rp] gated compensator input, ready before the launch
  const uint16_t *B;  // EPI: [N][rank]
  int rank, rp;
};

constexpr int kEpiRc = 32;           // ranks per epilogue chunk
constexpr int kEpiStr = kEpiRc + 4;  // LDS row stride of the chunk (floats)
static_assert(BM * kEpiStr * 4 <= BM * LSTR * 2, "epilogue U chunk fits the activation tile");
static_assert(BN * kEpiStr * 4 <= BN * LSTR * 2, "epilogue B chunk fits the weight tile");

template <int DT, bool PERCH, bool EPI>
__global__ __launch_bounds__(256, 2) void prefill_gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) uint16_t xs[BM * LSTR];
  __shared__ __align__(16) uint16_t wsm[BN * LSTR];
  __shared__ float ss[BN];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, h = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int nkb = (a.K + BK - 1) / BK;
  const int kw = a.K / 8;

  u32x4_t xr[8];
  u32x4_t wr[2];
  uint16_t zr[2];
  uint16_t sv = 0;

  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + 256 * i;
      const int r = p >> 4, j8 = p & 15;
      const int m = m0 + r, k = kb * BK + 8 * j8;
      xr[i] = (m < a.M && k < a.K) ? *(const u32x4_t *)(a.x + (size_t)m * a.K + k)
                                   : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int g = PERCH ? 0 : (kb * BK) / a.G;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int r = p >> 2, q4 = p & 3;
      const int n = min(n0 + r, a.N - 1);
      const int k = kb * BK + 32 * q4;
      wr[i] = (k < a.K) ? *(const u32x4_t *)(a.qw + (size_t)n * kw + kb * 16 + 4 * q4)
                        : u32x4_t{0u, 0u, 0u, 0u};
      zr[i] = a.zeros[(size_t)n * a.ngroups + g];
    }
    if (!PERCH && tid < BN) sv = a.scales[(size_t)min(n0 + tid, a.N - 1) * a.ngroups + g];
  };

  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + 256 * i;
      const int r = p >> 4, j8 = p & 15;
      *(u32x4_t *)(xs + r * LSTR + 8 * j8) = permute_8(xr[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int r = p >> 2, q4 = p & 3;
      const uint32_t zc = zero_constant<DT>(zr[i]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *(u32x4_t *)(wsm + r * LSTR + 32 * q4 + 8 * t) = dequant_word<DT>(wr[i][t], zc);
    }
    if (!PERCH && tid < BN) ss[tid] = (float)bitcast<_Float16>(sv);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  gload(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (kb + 1 < nkb) gload(kb + 1);

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
        bf[t] = *(const u32x4_t *)(wsm + (64 * wn + 16 * ni + col) * LSTR + 32 * t + 8 * h);
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
    // (now free) LDS tiles; rows past M or N and ranks past r stage zeros
    float *us = (float *)xs;
    float *bs = (float *)wsm;
    const int uq = kEpiRc / 4;
    for (int j0 = 0; j0 < a.rank; j0 += kEpiRc) {
      f32x4_t uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i;  // BM rows x uq pieces
        const int r = p / uq, q = p - r * uq;
        const int j = j0 + 4 * q;
        uv[i] = (m0 + r < a.M && j < a.rp) ? *(const f32x4_t *)(a.U + (size_t)(m0 + r) * a.rp + j)
                                           : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e >= a.rank) uv[i][e] = 0.f;
      }
      uint16_t bv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int p = tid + 256 * i;  // BN rows x kEpiRc ranks
        const int r = p / kEpiRc, jj = p - r * kEpiRc;
        bv[i] = (n0 + r < a.N && j0 + jj < a.rank) ? a.B[(size_t)(n0 + r) * a.rank + j0 + jj]
                                                  : (uint16_t)0;
      }
      __syncthreads();  // the tiles' last readers are done
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i;
        const int r = p / uq, q = p - r * uq;
        *(f32x4_t *)(us + r * kEpiStr + 4 * q) = uv[i];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int p = tid + 256 * i;
        const int r = p / kEpiRc, jj = p - r * kEpiRc;
        bs[r * kEpiStr + jj] = to_f32<DT>(bv[i]);
      }
      __syncthreads();
#pragma unroll
      for (int st = 0; st < kEpiRc / 4; ++st) {
        const int j = 4 * st + h;
        float ua[4], ba[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) ua[mi] = us[(64 * wm + 16 * mi + col) * kEpiStr + j];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) ba[ni] = bs[(64 * wn + 16 * ni + col) * kEpiStr + j];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_16x16x4_f32(ua[mi], ba[ni], acc[mi][ni]);
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
}

// ---------------------------------------------------------------------------
// Compensator: U[m][j] = g[m] * sum_k A[j][k] x[m][k], g[m] = sigmoid(z[m] + b_g),
// z[m] = sum_k w_g[k] x[m][k].
//
// Workgroup (blk, ksi) takes kEcTok = 32 tokens (two MFMA row blocks) and K
// split ksi of ks; its eight waves take interleaved 32-wide K steps.  Up to
// kEcRb 16-row blocks of [A; w_g] are accumulated together, so each weight
// piece feeds both token blocks and each activation piece feeds kEcRb MFMAs;
// each wave keeps kEcU steps of loads in flight before it multiplies.  Wave 0
// publishes the split's sums (rows 0..rank, the last being z) with
// agent-scope atomic stores, a release and a per-block counter; the split
// that completes the count sums the ks partials in split order, applies the
// gate, writes U and resets the counter for the next call.
// ---------------------------------------------------------------------------
struct EcArgs {
  const uint16_t *x, *A, *wg;
  float b_gate;
  int K, M, rank, rp, rp1, ks;
  float *U;        // [M][rp]
  float *Tp;       // [ks][M][rp1]: partial sums of [A; w_g] x per split
  uint32_t *cnt;   // [ceil(M / kEcTok)] splits finished per token block
};

constexpr int kEcWaves = 8, kEcRb = 3, kEcU = 4, kEcTok = 32, kEcMb = kEcTok / 16;
// rows of [A; w_g] round up to 16: up to 16 * ceil((SPEAR_MAX_RANK + 1) / 16) = 144
constexpr int kTzStride = 145;
static_assert(kTzStride > 16 * ((SPEAR_MAX_RANK + 1 + 15) / 16), "tz stride");

template <int DT>
__global__ __launch_bounds__(64 * kEcWaves) void prefill_ec_kernel(EcArgs a) {
  __shared__ f32x4_t red[kEcWaves][kEcRb][kEcMb][64];
  __shared__ float tz[kEcTok][kTzStride];
  __shared__ uint32_t last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, h = lane >> 4;
  const int blk = blockIdx.x / a.ks, ksi = blockIdx.x % a.ks;
  const int m0 = blk * kEcTok;
  // A-operand rows of this lane: tokens m0 + col + 16 mb; rows past M repeat
  // M - 1 (MFMA output rows depend only on their own A rows, and those are
  // never stored)
  const uint16_t *xrow[kEcMb];
#pragma unroll
  for (int mb = 0; mb < kEcMb; ++mb) xrow[mb] = a.x + (size_t)min(m0 + col + 16 * mb, a.M - 1) * a.K;
  const int rb_a = (a.rank + 16) / 16;
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
      jin[r] = rb0 + r < rb_a && j <= a.rank;
      arow[r] = (j < a.rank) ? a.A + (size_t)j * a.K : a.wg;  // j >= rank: w_g (masked if past it)
    }
    f32x4_t acc[kEcRb][kEcMb];
#pragma unroll
    for (int r = 0; r < kEcRb; ++r)
#pragma unroll
      for (int mb = 0; mb < kEcMb; ++mb) acc[r][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int s0 = s_lo + wave; s0 < s_hi; s0 += kEcWaves * kEcU) {
      u32x4_t xo[kEcU][kEcMb], ao[kEcU][kEcRb];
#pragma unroll
      for (int u = 0; u < kEcU; ++u) {
        const int k = min(s0 + kEcWaves * u, s_hi - 1) * 32 + 8 * h;
#pragma unroll
        for (int mb = 0; mb < kEcMb; ++mb) xo[u][mb] = *(const u32x4_t *)(xrow[mb] + k);
#pragma unroll
        for (int r = 0; r < kEcRb; ++r) ao[u][r] = *(const u32x4_t *)(arow[r] + k);
      }
#pragma unroll
      for (int u = 0; u < kEcU; ++u) {
        if (s0 + kEcWaves * u < s_hi) {
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
            for (int w = 1; w < kEcWaves; ++w) v = v + red[w][r][mb][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) tz[16 * mb + 4 * h + e][(rb0 + r) * 16 + col] = v[e];
          }
        }
      }
    }
    __syncthreads();
  }

  const int nval = kEcTok * (a.rank + 1);  // this block's values: its tokens x rows 0..rank
  if (wave == 0) {
    uint32_t *tp = (uint32_t *)a.Tp + ((size_t)ksi * a.M + m0) * a.rp1;
    for (int i = lane; i < nval; i += 64) {
      const int mm = i / (a.rank + 1), j = i - mm * (a.rank + 1);
      if (m0 + mm < a.M)
        __hip_atomic_store(&tp[(size_t)mm * a.rp1 + j], bitcast<uint32_t>(tz[mm][j]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0)
      last = __hip_atomic_fetch_add(&a.cnt[blk], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(a.ks - 1);
  }
  __syncthreads();
  if (!last) return;
  // the last split: every partial of this block has been published
  for (int i = tid; i < nval; i += 64 * kEcWaves) {
    const int mm = i / (a.rank + 1), j = i - mm * (a.rank + 1);
    float t = 0.f;
    if (m0 + mm < a.M) {
      for (int q = 0; q < a.ks; ++q)
        t += bitcast<float>(__hip_atomic_load(
            (const uint32_t *)a.Tp + ((size_t)q * a.M + m0 + mm) * a.rp1 + j, __ATOMIC_RELAXED,
            __HIP_MEMORY_SCOPE_AGENT));
    }
    tz[mm][j] = t;
  }
  __syncthreads();
  for (int i = tid; i < kEcTok * a.rank; i += 64 * kEcWaves) {
    const int mm = i / a.rank, j = i - mm * a.rank;
    const int m = m0 + mm;
    if (m < a.M) {
      const float g = gate_sigmoid(tz[mm][a.rank] + a.b_gate);
      a.U[(size_t)m * a.rp + j] = g * tz[mm][j];
    }
  }
  if (tid == 0) __hip_atomic_store(&a.cnt[blk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Merge on the main stream after the join: y[m][n] += sum_j U[m][j] B[n][j]
// for a 64-token x 64-output tile.  The y tile, the 64 U rows and the 64 B
// rows are staged in LDS (loads issued together, 16 bytes where the layout
// allows), four waves each take 16 tokens with fp32 16x16x4 MFMAs, and y
// goes back in 16-byte stores when its rows are 16-byte aligned.
// ---------------------------------------------------------------------------
struct MergeArgs {
  uint16_t *y;
  const uint16_t *B;
  const float *U;  // [M][rp]
  int N, M, rank, rp;
};

constexpr int kMgT = 64;              // tokens and outputs per tile
constexpr int kMgYStr = kMgT + 8;     // LDS row stride of the y tile (halves)

__host__ __device__ constexpr int merge_rstr(int rp) { return rp + 4; }  // floats; 16-byte rows
__host__ __device__ constexpr size_t merge_lds_bytes(int rp) {
  return (size_t)2 * kMgT * merge_rstr(rp) * 4 + (size_t)kMgT * kMgYStr * 2;
}

template <int DT>
__global__ __launch_bounds__(256) void prefill_merge_kernel(MergeArgs a) {
  extern __shared__ __align__(16) float mlds[];
  const int rstr = merge_rstr(a.rp);
  float *us = mlds;                                    // [64][rstr]
  float *bs = us + kMgT * rstr;                        // [64][rstr]
  uint16_t *ys = (uint16_t *)(bs + kMgT * rstr);       // [64][kMgYStr]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * kMgT, m0 = blockIdx.y * kMgT;
  const bool yvec = (a.N % 8) == 0;

  // --- stage: y tile (8 halves per piece), U rows (4 floats), B rows (scalars)
  u32x4_t yv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i;  // 512 pieces of 8 halves
    const int r = p >> 3, c8 = (p & 7) * 8;
    const int m = m0 + r, n = n0 + c8;
    yv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (m < a.M) {
      if (yvec && n + 8 <= a.N) {
        yv[i] = *(const u32x4_t *)(a.y + (size_t)m * a.N + n);
      } else {
        uint16_t t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (n + e < a.N) ? a.y[(size_t)m * a.N + n + e] : 0;
        yv[i] = bitcast<u32x4_t>(t);
      }
    }
  }
  const int uq = a.rp / 4;  // 16-byte pieces per U row
  for (int p0 = 0; p0 < kMgT * uq; p0 += 256 * 4) {
    f32x4_t uv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + tid + 256 * i;
      const int r = p / uq, q = p - r * uq;
      uv[i] = (p < kMgT * uq && m0 + r < a.M)
                  ? *(const f32x4_t *)(a.U + (size_t)(m0 + r) * a.rp + 4 * q)
                  : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + tid + 256 * i;
      const int r = p / uq, q = p - r * uq;
      // columns rank .. rp-1 of U are never written: zero them, whatever the
      // workspace held there
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e >= a.rank) uv[i][e] = 0.f;
      if (p < kMgT * uq) *(f32x4_t *)(us + r * rstr + 4 * q) = uv[i];
    }
  }
  for (int p0 = 0; p0 < kMgT * a.rp; p0 += 256 * 8) {
    uint16_t bv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = p0 + tid + 256 * i;
      const int r = p / a.rp, j = p - r * a.rp;
      bv[i] = (p < kMgT * a.rp && n0 + r < a.N && j < a.rank)
                  ? a.B[(size_t)(n0 + r) * a.rank + j] : (uint16_t)0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = p0 + tid + 256 * i;
      const int r = p / a.rp, j = p - r * a.rp;
      if (p < kMgT * a.rp) bs[r * rstr + j] = to_f32<DT>(bv[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i;
    const int r = p >> 3, c8 = (p & 7) * 8;
    *(u32x4_t *)(ys + r * kMgYStr + c8) = yv[i];
  }
  __syncthreads();

  // --- multiply: wave takes tokens 16 wave .. +16, all 64 outputs
  const int nst = a.rp / 4;
  const int tk = 16 * wave + col;  // A-operand row (token) of this lane
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    f32x4_t acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = to_f32<DT>(ys[(16 * wave + 4 * h + e) * kMgYStr + 16 * nb + col]);
    for (int st = 0; st < nst; ++st) {
      const int j = 4 * st + h;
      acc = mfma_16x16x4_f32(us[tk * rstr + j], bs[(16 * nb + col) * rstr + j], acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ys[(16 * wave + 4 * h + e) * kMgYStr + 16 * nb + col] = from_f32<DT>(acc[e]);
  }
  __syncthreads();

  // --- store the tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i;
    const int r = p >> 3, c8 = (p & 7) * 8;
    const int m = m0 + r, n = n0 + c8;
    if (m < a.M) {
      const u32x4_t v = *(const u32x4_t *)(ys + r * kMgYStr + c8);
      if (yvec && n + 8 <= a.N) {
        *(u32x4_t *)(a.y + (size_t)m * a.N + n) = v;
      } else {
        const u16x8_t t = bitcast<u16x8_t>(v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < a.N) a.y[(size_t)m * a.N + n + e] = t[e];
      }
    }
  }
}

// Merge launch; the dynamic LDS can exceed the 64 KB default (rank 128: 78 KB).
template <int DT>
hipError_t launch_merge(const MergeArgs &ma, dim3 grid, size_t lds, hipStream_t s) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute((const void *)prefill_merge_kernel<DT>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)merge_lds_bytes((SPEAR_MAX_RANK + 3) / 4 * 4));
  });
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(prefill_merge_kernel<DT>, grid, dim3(256), lds, s, ma);
  return hipGetLastError();
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

// Compensator K-splits: enough workgroups (about 512) to keep the activation
// stream busy, at most 16, and at least one 32-wide step per wave per split.
constexpr int kEcMaxKs = 16;
static int ec_ksplit(int M, int K) {
  const int nblk = (M + kEcTok - 1) / kEcTok;
  int ks = (256 + nblk - 1) / nblk;
  if (ks > 4) ks = 4;  // each extra split adds a publish and a gather
  const int cap = (K / 32) / kEcWaves;
  if (ks > cap) ks = cap;
  if (ks > kEcMaxKs) ks = kEcMaxKs;
  return ks < 1 ? 1 : ks;
}

// Workspace after the 2048-byte header: split counters [ceil(M/32)], U
// [M][rp] and the split partials [ks][M][rp1], each 256-byte aligned.  The
// counters must start at zero, so they sit past the largest region a decode
// call writes (its partial sums follow the header); U and the partials are
// rewritten in full by every call and may share bytes with decode's.
struct PrefillWs {
  size_t cnt_off, u_off, tp_off, end;
};
static PrefillWs prefill_ws_layout(const LayerDesc &L, int M) {
  PrefillWs w;
  const int nblk = (M + kEcTok - 1) / kEcTok;
  size_t dec = 0;  // decode's bytes for one (M <= 16) and two (M <= 32) token blocks
  for (int dm : {16, SPEAR_MAX_DECODE_M}) {
    const size_t b = decode_workspace_bytes(L, dm);
    if (b > dec) dec = b;
  }
  w.cnt_off = dec > sizeof(WsHeader) ? round256(dec) : sizeof(WsHeader);
  w.u_off = w.cnt_off + round256((size_t)nblk * sizeof(uint32_t));
  w.tp_off = w.u_off + round256((size_t)M * rank_pad(L.rank) * sizeof(float));
  // sized for the most splits, so that a workspace for M serves every call
  // with fewer tokens too (the split count is not monotone in M)
  w.end = w.tp_off + round256((size_t)kEcMaxKs * M * rank_pad(L.rank + 1) * sizeof(float));
  return w;
}

size_t prefill_workspace_bytes(const LayerDesc &L, int M) {
  if (L.rank == 0) return 0;
  return prefill_ws_layout(L, M).end;
}

template <int DT, bool PERCH, bool EPI>
static void launch_gemm(const GemmArgs &g, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((prefill_gemm_kernel<DT, PERCH, EPI>), grid, dim3(256), 0, s, g);
}

template <int DT>
static void launch_gemm_dt(const GemmArgs &g, dim3 grid, bool perch, bool epi, hipStream_t s) {
  if (perch)
    epi ? launch_gemm<DT, true, true>(g, grid, s) : launch_gemm<DT, true, false>(g, grid, s);
  else
    epi ? launch_gemm<DT, false, true>(g, grid, s) : launch_gemm<DT, false, false>(g, grid, s);
}

hipError_t launch_prefill(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                          void *ws, hipStream_t main_s, hipStream_t aux_s) {
  const bool ec = L.rank > 0;
  const bool concurrent = ec && aux_s != nullptr && aux_s != main_s;
  const int rp = rank_pad(L.rank);
  float *U = nullptr;
  EcArgs ea{};
  if (ec) {
    const PrefillWs w = prefill_ws_layout(L, M);
    char *base = (char *)ws;
    U = (float *)(base + w.u_off);
    ea = EcArgs{x, L.A, L.wg, L.b_gate, L.K, M, L.rank, rp, rank_pad(L.rank + 1), ec_ksplit(M, L.K),
                U, (float *)(base + w.tp_off), (uint32_t *)(base + w.cnt_off)};
  }
  GemmArgs g{L.qw, L.scales, L.zeros, x, y, L.N, L.K, L.G, L.ngroups, M, U, L.B, L.rank, rp};
  const dim3 ggrid((L.N + BN - 1) / BN, (M + BM - 1) / BM);
  const dim3 egrid(((M + kEcTok - 1) / kEcTok) * (ec ? ea.ks : 1));
  hipError_t e = hipSuccess;

  auto launch_ec = [&](hipStream_t s) {
    if (dtype == DT_F16)
      hipLaunchKernelGGL(prefill_ec_kernel<DT_F16>, egrid, dim3(64 * kEcWaves), 0, s, ea);
    else
      hipLaunchKernelGGL(prefill_ec_kernel<DT_BF16>, egrid, dim3(64 * kEcWaves), 0, s, ea);
    return hipGetLastError();
  };

  if (!concurrent) {
    // serial: U first, then the GEMM adds U B^T in its epilogue
    if (ec && (e = launch_ec(main_s)) != hipSuccess) return e;
    if (dtype == DT_F16)
      launch_gemm_dt<DT_F16>(g, ggrid, L.per_channel, ec, main_s);
    else
      launch_gemm_dt<DT_BF16>(g, ggrid, L.per_channel, ec, main_s);
    return hipGetLastError();
  }

  // concurrent: EC on aux alongside the GEMM, merge after the join
  std::lock_guard<std::mutex> lock(g_event_mu);
  StreamEvents *ev = nullptr;
  if ((e = get_events(&ev)) != hipSuccess) return e;
  if ((e = hipEventRecord(ev->fork, main_s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(aux_s, ev->fork, 0)) != hipSuccess) return e;
  if ((e = launch_ec(aux_s)) != hipSuccess) return e;
  if ((e = hipEventRecord(ev->join, aux_s)) != hipSuccess) return e;
  if (dtype == DT_F16)
    launch_gemm_dt<DT_F16>(g, ggrid, L.per_channel, false, main_s);
  else
    launch_gemm_dt<DT_BF16>(g, ggrid, L.per_channel, false, main_s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(main_s, ev->join, 0)) != hipSuccess) return e;
  MergeArgs ma{y, L.B, U, L.N, M, L.rank, rp};
  const dim3 mgrid((L.N + kMgT - 1) / kMgT, (M + kMgT - 1) / kMgT);
  const size_t mlds = merge_lds_bytes(rp);
  return dtype == DT_F16 ? launch_merge<DT_F16>(ma, mgrid, mlds, main_s)
                         : launch_merge<DT_BF16>(ma, mgrid, mlds, main_s);
}

}  // namespace spear
