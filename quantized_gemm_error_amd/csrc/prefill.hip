// Prefill path: y = dequant(W_q) x + sigmoid(w_g . x + b_g) * B (A x) for
// many tokens (M in the hundreds to thousands).
//
// The pages run the compensator of the compute-bound prefill as a separate
// kernel that overlaps the low-bit GEMM instead of fusing it (SPEAR
// explanation page, Technical Summary 2.2 A, prefill phase).  Here:
//
//  * main stream: prefill_gemm_kernel, a 128x128x128-tiled MFMA GEMM.  Each
//    k-block stages the activation tile and the exactly dequantized weight
//    tile (q - z in the activation type) in LDS; four waves each own a 64x64
//    quarter of the output tile and run 16x16x32 MFMAs, applying each row's
//    fp32 scale once per 128-wide block (or once at the end when one scale
//    covers the row);
//  * aux stream, concurrently: prefill_ec_kernel computes U = diag(g) (X A^T)
//    with g = sigmoid(X w_g + b_g) into the workspace (fp32);
//  * main stream after joining aux: prefill_merge_kernel adds U B^T to y.
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
};

template <int DT, bool PERCH>
__global__ __launch_bounds__(256) void prefill_gemm_kernel(GemmArgs a) {
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

#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int n = n0 + 64 * wn + 16 * ni + col;
    float s = 1.f;
    if constexpr (PERCH) s = (float)bitcast<_Float16>(a.scales[(size_t)min(n, a.N - 1)]);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 64 * wm + 16 * mi + 4 * h + e;
        if (m < a.M && n < a.N) {
          const float v = PERCH ? acc[mi][ni][e] * s : acc[mi][ni][e];
          a.y[(size_t)m * a.N + n] = from_f32<DT>(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Compensator on the aux stream: U[m][j] = g[m] * sum_k A[j][k] x[m][k].
// One workgroup per 32 tokens; four waves split K; all rows of [A; w_g].
// ---------------------------------------------------------------------------
struct EcArgs {
  const uint16_t *x, *A, *wg;
  float b_gate;
  int K, M, rank;
  float *U;  // [M][rank]
};

// rows of [A; w_g] round up to 16: up to 16 * ceil((SPEAR_MAX_RANK + 1) / 16) = 144
constexpr int kTzStride = 145;
static_assert(kTzStride > 16 * ((SPEAR_MAX_RANK + 1 + 15) / 16), "tz stride");

template <int DT>
__global__ __launch_bounds__(256) void prefill_ec_kernel(EcArgs a) {
  __shared__ f32x4_t red[3][2][64];
  __shared__ float tz[32][kTzStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, h = lane >> 4;
  const int m0 = blockIdx.x * 32;
  const int rb_a = (a.rank + 16) / 16;
  const int nsteps = a.K / 32;

  for (int rb = 0; rb < rb_a; ++rb) {
    const int j = rb * 16 + col;
    const uint16_t *arow = nullptr;
    if (j < a.rank) arow = a.A + (size_t)j * a.K;
    else if (j == a.rank) arow = a.wg;
    f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
    for (int s = wave; s < nsteps; s += 4) {
      const int k = s * 32 + 8 * h;
      u32x4_t bop = {0u, 0u, 0u, 0u};
      if (arow) bop = *(const u32x4_t *)(arow + k);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + col + 16 * mb;
        u32x4_t aop = {0u, 0u, 0u, 0u};
        if (m < a.M) aop = *(const u32x4_t *)(a.x + (size_t)m * a.K + k);
        acc[mb] = mfma_16x16x32<DT>(aop, bop, acc[mb]);
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) red[wave - 1][mb][lane] = acc[mb];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const f32x4_t v = ((acc[mb] + red[0][mb][lane]) + red[1][mb][lane]) + red[2][mb][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) tz[16 * mb + 4 * h + e][rb * 16 + col] = v[e];
      }
    }
    __syncthreads();
  }
  for (int idx = tid; idx < 32 * a.rank; idx += 256) {
    const int mm = idx / a.rank, j = idx - mm * a.rank;
    const int m = m0 + mm;
    if (m < a.M) {
      const float g = gate_sigmoid(tz[mm][a.rank] + a.b_gate);
      a.U[(size_t)m * a.rank + j] = g * tz[mm][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Merge on the main stream after the join: y[m][n] += sum_j U[m][j] B[n][j].
// Workgroup tile 64 tokens x 64 outputs; fp32 16x16x4 MFMAs.
// ---------------------------------------------------------------------------
struct MergeArgs {
  uint16_t *y;
  const uint16_t *B;
  const float *U;
  int N, M, rank;
};

template <int DT>
__global__ __launch_bounds__(256) void prefill_merge_kernel(MergeArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, h = lane >> 4;
  const int m0 = blockIdx.y * 64 + 16 * wave;
  const int nst = (a.rank + 3) / 4;
  const int mu = m0 + col;  // token of this lane's A-operand row
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = blockIdx.x * 64 + 16 * nb + col;
    const int nrow = min(n, a.N - 1);
    f32x4_t acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 4 * h + e;
      acc[e] = (m < a.M && n < a.N) ? to_f32<DT>(a.y[(size_t)m * a.N + n]) : 0.f;
    }
    for (int st = 0; st < nst; ++st) {
      const int j = 4 * st + h;
      const float u = (mu < a.M && j < a.rank) ? a.U[(size_t)mu * a.rank + j] : 0.f;
      const float bv = (j < a.rank) ? to_f32<DT>(a.B[(size_t)nrow * a.rank + j]) : 0.f;
      acc = mfma_16x16x4_f32(u, bv, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 4 * h + e;
      if (m < a.M && n < a.N) a.y[(size_t)m * a.N + n] = from_f32<DT>(acc[e]);
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

size_t prefill_workspace_bytes(const LayerDesc &L, int M) {
  if (L.rank == 0) return 0;
  return sizeof(WsHeader) + (((size_t)M * L.rank * sizeof(float) + 255) / 256) * 256;
}

hipError_t launch_prefill(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                          void *ws, hipStream_t main_s, hipStream_t aux_s) {
  GemmArgs g{L.qw, L.scales, L.zeros, x, y, L.N, L.K, L.G, L.ngroups, M};
  const dim3 ggrid((L.N + BN - 1) / BN, (M + BM - 1) / BM);
  const bool ec = L.rank > 0;
  const bool concurrent = ec && aux_s != nullptr && aux_s != main_s;
  float *U = ec ? (float *)((char *)ws + sizeof(WsHeader)) : nullptr;
  EcArgs ea{x, L.A, L.wg, L.b_gate, L.K, M, L.rank, U};
  const dim3 egrid((M + 31) / 32);
  hipError_t e = hipSuccess;

  std::unique_lock<std::mutex> lock(g_event_mu, std::defer_lock);
  StreamEvents *ev = nullptr;
  if (concurrent) {
    lock.lock();
    if ((e = get_events(&ev)) != hipSuccess) return e;
    if ((e = hipEventRecord(ev->fork, main_s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(aux_s, ev->fork, 0)) != hipSuccess) return e;
  }
  if (ec) {
    hipStream_t es = concurrent ? aux_s : main_s;
    if (dtype == DT_F16)
      hipLaunchKernelGGL(prefill_ec_kernel<DT_F16>, egrid, dim3(256), 0, es, ea);
    else
      hipLaunchKernelGGL(prefill_ec_kernel<DT_BF16>, egrid, dim3(256), 0, es, ea);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (concurrent && (e = hipEventRecord(ev->join, aux_s)) != hipSuccess) return e;
  }
  if (dtype == DT_F16) {
    if (L.per_channel)
      hipLaunchKernelGGL((prefill_gemm_kernel<DT_F16, true>), ggrid, dim3(256), 0, main_s, g);
    else
      hipLaunchKernelGGL((prefill_gemm_kernel<DT_F16, false>), ggrid, dim3(256), 0, main_s, g);
  } else {
    if (L.per_channel)
      hipLaunchKernelGGL((prefill_gemm_kernel<DT_BF16, true>), ggrid, dim3(256), 0, main_s, g);
    else
      hipLaunchKernelGGL((prefill_gemm_kernel<DT_BF16, false>), ggrid, dim3(256), 0, main_s, g);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ec) {
    if (concurrent && (e = hipStreamWaitEvent(main_s, ev->join, 0)) != hipSuccess) return e;
    MergeArgs ma{y, L.B, U, L.N, M, L.rank};
    const dim3 mgrid((L.N + 63) / 64, (M + 63) / 64);
    if (dtype == DT_F16)
      hipLaunchKernelGGL(prefill_merge_kernel<DT_F16>, mgrid, dim3(256), 0, main_s, ma);
    else
      hipLaunchKernelGGL(prefill_merge_kernel<DT_BF16>, mgrid, dim3(256), 0, main_s, ma);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace spear
