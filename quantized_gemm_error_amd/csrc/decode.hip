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
// Partial sums travel through agent-scope atomic stores and loads, which are
// coherent across the XCDs' separate L2 caches on their own, so no wave
// needs a cache-wide invalidate; only the producers' release (before they
// count themselves in) writes back their L2.
//
// Every loop that touches memory has a compile-time shape, so its loads
// issue back to back and the waits count them exactly.  The last workgroup
// to finish (counted over eight slots, then across the slots) resets the
// workspace counters for the next call.
#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kDepth = 8;                  // K blocks in flight per wave
constexpr int kKS = kDecodeKSplit;         // producer K-splits
constexpr int kMaxStepsPerWave = (SPEAR_MAX_RANK / 4 + kWaves - 1) / kWaves;  // rank steps of 4
constexpr uint32_t kSpinLimit = 1u << 20;  // bounded wait for the producers
constexpr int kWholeLdsBytes = 100 * 1024; // whole-x staging budget
constexpr int kChunkLdsBytes = 68 * 1024;  // chunked staging budget

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
  WsHeader *hdr;
  float *part;     // [producers][16 rows of A'][16 * MB tokens]
};

// Sum of the waves' partial tiles in a fixed order (wave 0's own, then 1..7).
template <int MB>
__device__ __forceinline__ f32x4_t reduce_waves(f32x4_t own, f32x4_t (*red)[MB][64], int mb,
                                                int lane) {
  f32x4_t v = own;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) v = v + red[w][mb][lane];
  return v;
}

__device__ __forceinline__ float load_partial(const float *p) {
  return bitcast<float>(__hip_atomic_load((const uint32_t *)p, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT));
}

// ---------------------------------------------------------------------------
// Producers: partial [A; w_g] x over one K-split for one 16-row block.
// ---------------------------------------------------------------------------
template <int DT, int MB>
__device__ void produce(const DecodeArgs &a, int p, f32x4_t (*red)[MB][64], int wave, int lane) {
  const int col = lane & 15, h = lane >> 4;
  const int rb = p / kKS, ksi = p % kKS;
  const int j = rb * 16 + col;  // row of [A; w_g]
  const bool jin = j <= a.rank;
  const uint16_t *arow = (j < a.rank) ? a.A + (size_t)j * a.K : a.wg;
  const int nsteps = a.K / 32;
  const int per = (nsteps + kKS - 1) / kKS;
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
    for (int mb = 0; mb < MB; ++mb) red[wave - 1][mb][lane] = acc[mb];
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t *dst = (uint32_t *)a.part + (size_t)p * 16 * (16 * MB);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4_t v = reduce_waves(acc[mb], red, mb, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __hip_atomic_store(&dst[col * (16 * MB) + 16 * mb + 4 * h + e], bitcast<uint32_t>(v[e]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
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
    const int p = min(p0 + tid + kThreads * i, total - 1);
    const int m = p / per_row, j = p - m * per_row;
    const int k = min(8 * j, a.K - 8);
    xb.v[i] = *(const u32x4_t *)(a.x + (size_t)m * a.K + k);
  }
}

__device__ __forceinline__ void whole_store(const DecodeArgs &a, const XBatch &xb, uint16_t *xs,
                                            int p0, int tid) {
  const int per_row = a.nb * 16;
  const int total = a.M * per_row;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = p0 + tid + kThreads * i;
    if (p < total) {
      const int m = p / per_row, j = p - m * per_row;
      const u32x4_t val = (8 * j < a.K) ? xb.v[i] : u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t *)(xs + m * a.xstr + 8 * j) = permute_8(val);
    }
  }
}

struct XChunk {
  u32x4_t v[8];
};

// One chunk (xc columns) of x into registers: at most 8 pieces per thread.
__device__ __forceinline__ void chunk_load(const DecodeArgs &a, XChunk &c, int chunk, int tid) {
  const int per_row = a.xc / 8;
  const int k0 = chunk * a.xc;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
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
  for (int i = 0; i < 8; ++i) {
    const int p = tid + kThreads * i;
    const int m = p / per_row, j = p % per_row;
    if (m < a.M) {
      const u32x4_t val = (k0 + 8 * j < a.K) ? c.v[i] : u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t *)(xs + m * a.xstr + 8 * j) = permute_8(val);
    }
  }
}

// ---------------------------------------------------------------------------
// Consumers: 16 output rows, full K, four waves.
// ---------------------------------------------------------------------------
template <int DT, int MB, bool EC, bool PERCH, int XMODE>
__device__ void consume(const DecodeArgs &a, int tile, uint16_t *xs, f32x4_t (*red)[MB][64],
                        int tid) {
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, h = lane >> 4;
  const int n = tile * 16 + col;
  const int row = min(n, a.N - 1);
  const uint32_t *wrow = a.qw + (size_t)row * (a.K / 8);
  const uint16_t *srow = a.scales + (size_t)row * a.ngroups;
  const uint16_t *zrow = a.zeros + (size_t)row * a.ngroups;
  const int nb = a.nb, nbw = a.nbw;

  uint32_t zc_row = 0;
  float s_row = 0.f;
  if constexpr (PERCH) {
    zc_row = zero_constant<DT>(zrow[0]);
    s_row = (float)bitcast<_Float16>(srow[0]);
  }

  // piece of block iteration b: block kb = kWaves b + wave (clamped), words [4h, 4h + 4)
  u32x4_t wr[kDepth];
  uint16_t sr[kDepth], zr[kDepth];
  auto wload = [&](int b, u32x4_t &w, uint16_t &sv, uint16_t &zv) {
    const int kb = min(b * kWaves + wave, nb - 1);
    const int off = (kb * 128 + 32 * h < a.K) ? kb * 16 + 4 * h : 0;
    w = *(const u32x4_t *)(wrow + off);
    if constexpr (!PERCH) {
      const int g = (kb * 128) / a.G;
      sv = srow[g];
      zv = zrow[g];
    } else {
      sv = 0;
      zv = 0;
    }
  };
  // activation loads first, then the weight ring, so that storing the
  // activation to LDS waits only for its own loads
  XChunk xc;
  XBatch xb;
  if constexpr (XMODE == XWHOLE) {
    whole_load(a, xb, 0, tid);
  } else {
    chunk_load(a, xc, 0, tid);
  }
#pragma unroll
  for (int i = 0; i < kDepth; ++i) wload(i, wr[i], sr[i], zr[i]);
  if constexpr (XMODE == XWHOLE) {
    whole_store(a, xb, xs, 0, tid);
    const int total = a.M * a.nb * 16;
    for (int p0 = kThreads * 8; p0 < total; p0 += kThreads * 8) {
      whole_load(a, xb, p0, tid);
      whole_store(a, xb, xs, p0, tid);
    }
    __syncthreads();
  }

  f32x4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int b0 = 0; b0 < nbw; b0 += kDepth) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int b = b0 + i;
      int kbase = 0;  // first K column of the staged activation
      if constexpr (XMODE == XCHUNK) {
        const int chunk = b / a.ci;
        kbase = chunk * a.xc;
        if (b < nbw && b % a.ci == 0) {
          __syncthreads();
          chunk_store(a, xc, xs, chunk, tid);
          __syncthreads();
          if ((chunk + 1) * a.xc < a.K) chunk_load(a, xc, chunk + 1, tid);
        }
      }
      const u32x4_t w = wr[i];
      const uint16_t sv = sr[i], zv = zr[i];
      if (b + kDepth < nbw) wload(b + kDepth, wr[i], sr[i], zr[i]);
      const int kb = b * kWaves + wave;
      if (b < nbw && kb < nb) {
        const uint32_t zc = PERCH ? zc_row : zero_constant<DT>(zv);
        const int kloc = kb * 128 - kbase + 32 * h;
        u32x4_t bop[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) bop[t] = dequant_word<DT>(w[t], zc);
        f32x4_t accg[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = col + 16 * mb;
          u32x4_t aop[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) aop[t] = u32x4_t{0u, 0u, 0u, 0u};
          if (m < a.M) {
            const uint16_t *xp = xs + m * a.xstr + kloc;
#pragma unroll
            for (int t = 0; t < 4; ++t) aop[t] = *(const u32x4_t *)(xp + 8 * t);
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if constexpr (PERCH) {
              acc[mb] = mfma_16x16x32<DT>(aop[t], bop[t], acc[mb]);
            } else {
              accg[mb] = mfma_16x16x32<DT>(aop[t], bop[t],
                                           t == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : accg[mb]);
            }
          }
        }
        if constexpr (!PERCH) {
          const float s = (float)bitcast<_Float16>(sv);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb] += s * accg[mb];
        }
      }
    }
  }

  if constexpr (PERCH) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] *= s_row;
  }

  if constexpr (EC) {
    wait_producers(a, tid);
    const int PS = 16 * MB;  // token stride of a partial row
    // gate of this lane's A-operand token (m = col + 16 mb)
    const int rbz = a.rank / 16, jz = a.rank % 16;
    float zp[MB][kKS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        zp[mb][ks] = load_partial(a.part + ((size_t)(rbz * kKS + ks) * 16 + jz) * PS + col + 16 * mb);
    // this wave's rank steps st = wave + 4 i: all loads first
    const int nst = (a.rank + 3) / 4;
    float tp[kMaxStepsPerWave][MB][kKS];
    float bv[kMaxStepsPerWave];
#pragma unroll
    for (int i = 0; i < kMaxStepsPerWave; ++i) {
      const int st = wave + kWaves * i;
      if (st < nst) {
        const int j = min(4 * st + h, a.rank - 1);
        const int rbj = j / 16, jj = j % 16;
        bv[i] = to_f32<DT>(a.B[(size_t)row * a.rank + j]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
            tp[i][mb][ks] = load_partial(a.part + ((size_t)(rbj * kKS + ks) * 16 + jj) * PS + col + 16 * mb);
      }
    }
    float g[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float z = 0.f;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) z += zp[mb][ks];
      g[mb] = gate_sigmoid(z + a.b_gate);
    }
#pragma unroll
    for (int i = 0; i < kMaxStepsPerWave; ++i) {
      const int st = wave + kWaves * i;
      if (st < nst) {
        const bool jin = 4 * st + h < a.rank;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          float t = 0.f;
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) t += tp[i][mb][ks];
          const float u = (jin && col + 16 * mb < a.M) ? g[mb] * t : 0.f;
          acc[mb] = mfma_16x16x4_f32(u, jin ? bv[i] : 0.f, acc[mb]);
        }
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave - 1][mb][lane] = acc[mb];
  }
  __syncthreads();
  if (wave == 0 && n < a.N) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4_t v = reduce_waves(acc[mb], red, mb, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mb + 4 * h + e;
        if (m < a.M) a.y[(size_t)m * a.N + n] = from_f32<DT>(v[e]);
      }
    }
  }
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

template <int DT, int MB, bool EC, bool PERCH, int XMODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint16_t xs[];
  __shared__ f32x4_t red[kWaves - 1][MB][64];

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if constexpr (EC) {
    if (b < a.producers) {
      produce<DT, MB>(a, b, red, tid >> 6, tid & 63);
    } else {
      consume<DT, MB, EC, PERCH, XMODE>(a, b - a.producers, xs, red, tid);
    }
    if (tid == 0) finish(a);
  } else {
    consume<DT, MB, EC, PERCH, XMODE>(a, b, xs, red, tid);
  }
}

template <int DT, int MB, bool EC, bool PERCH, int XMODE>
hipError_t launch_t(const DecodeArgs &a, int grid, size_t lds, hipStream_t s) {
  auto kern = decode_kernel<DT, MB, EC, PERCH, XMODE>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   kWholeLdsBytes);
  });
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int DT, int MB, bool EC, bool PERCH>
hipError_t launch_x(const DecodeArgs &a, int xmode, int grid, size_t lds, hipStream_t s) {
  return xmode == XWHOLE ? launch_t<DT, MB, EC, PERCH, XWHOLE>(a, grid, lds, s)
                         : launch_t<DT, MB, EC, PERCH, XCHUNK>(a, grid, lds, s);
}

template <int DT, int MB, bool EC>
hipError_t launch_pc(const DecodeArgs &a, bool perch, int xmode, int grid, size_t lds,
                     hipStream_t s) {
  return perch ? launch_x<DT, MB, EC, true>(a, xmode, grid, lds, s)
               : launch_x<DT, MB, EC, false>(a, xmode, grid, lds, s);
}

template <int DT, int MB>
hipError_t launch_ec(const DecodeArgs &a, bool ec, bool perch, int xmode, int grid, size_t lds,
                     hipStream_t s) {
  return ec ? launch_pc<DT, MB, true>(a, perch, xmode, grid, lds, s)
            : launch_pc<DT, MB, false>(a, perch, xmode, grid, lds, s);
}

template <int DT>
hipError_t launch_mb(const DecodeArgs &a, int mb, bool ec, bool perch, int xmode, int grid,
                     size_t lds, hipStream_t s) {
  return mb == 1 ? launch_ec<DT, 1>(a, ec, perch, xmode, grid, lds, s)
                 : launch_ec<DT, 2>(a, ec, perch, xmode, grid, lds, s);
}

}  // namespace

DecodePlan plan_decode(const LayerDesc &L, int M) {
  DecodePlan p{};
  p.mb = M <= 16 ? 1 : 2;
  p.n_tiles = (L.N + 15) / 16;
  p.rb_a = L.rank > 0 ? (L.rank + 1 + 15) / 16 : 0;
  p.ks = L.rank > 0 ? kKS : 0;
  p.producers = p.rb_a * p.ks;
  p.nb = (L.K + 127) / 128;
  p.nbw = (p.nb + kWaves - 1) / kWaves;
  const int kr = p.nb * 128;
  const size_t whole = (size_t)M * (kr + 8) * 2;
  if (whole <= (size_t)kWholeLdsBytes) {
    p.xmode = XWHOLE;
    p.ci = 1 << 30;
    p.xc = kr;
    p.xstr = kr + 8;
    p.lds = whole;
  } else {
    // largest chunk of ci iterations (512 * ci columns) within the LDS budget
    // and at most 8 staged pieces per thread (M * ci <= 32)
    // pieces per thread: M * 128 * kWaves * ci / 8 / kThreads = M * ci / 4 <= 8
    int ci = 1;
    while (ci * 2 <= p.nbw && M * ci * 2 <= 32 &&
           (size_t)M * (128 * kWaves * ci * 2 + 8) * 2 <= (size_t)kChunkLdsBytes)
      ci *= 2;
    p.xmode = XCHUNK;
    p.ci = ci;
    p.xc = 128 * kWaves * ci;
    p.xstr = p.xc + 8;
    p.lds = (size_t)M * p.xstr * 2;
  }
  return p;
}

size_t decode_workspace_bytes(const LayerDesc &L, int M) {
  if (L.rank == 0) return 0;
  const DecodePlan p = plan_decode(L, M);
  return sizeof(WsHeader) + (size_t)p.producers * 16 * (16 * p.mb) * sizeof(float);
}

hipError_t launch_decode(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                         void *ws, hipStream_t s) {
  const DecodePlan p = plan_decode(L, M);
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
  a.hdr = (WsHeader *)ws;
  a.part = ws ? (float *)((char *)ws + sizeof(WsHeader)) : nullptr;
  const bool ec = L.rank > 0;
  const int grid = p.n_tiles + p.producers;
  return dtype == DT_F16 ? launch_mb<DT_F16>(a, p.mb, ec, L.per_channel, p.xmode, grid, p.lds, s)
                         : launch_mb<DT_BF16>(a, p.mb, ec, L.per_channel, p.xmode, grid, p.lds, s);
}

}  // namespace spear
