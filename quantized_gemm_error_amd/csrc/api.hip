// C ABI of libspear: host-side validation, workspace sizing, phase-aware
// dispatch and the chunk selector.  Every check happens before any launch;
// on error nothing is enqueued and the outputs are untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "internal.h"

using namespace spear;

namespace {

thread_local char g_last_error[512] = "";
constexpr int32_t kSmallDecodeM = 32;  // the per-row-group decode kernels; past it, the wide one
// Layers of at most this many 128-row tiles take the wide launch at 17..32
// tokens where the split-K decode launch is wanted but does not fit
// (small_decode).
constexpr int kWideLongKMaxTiles = 64;
// spear_linear's dispatch threshold.  Measured on MI355X (compensated calls):
// at 64 tokens the wide decode launch beats the prefill path on every Llama-7B
// and Llama-70B projection (e.g. 8192 x 8192: 36.7 vs 49.8 us; 8192 -> 28672:
// 67.9 vs 99.9 us); at 128 tokens the prefill path wins on most of them.
constexpr int32_t kDefaultDecodeMaxM = 64;
std::atomic<int32_t> g_decode_max_m{kDefaultDecodeMaxM};

spear_status_t fail(spear_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

spear_status_t ok() {
  g_last_error[0] = '\0';
  return SPEAR_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Validate a layer; fill the descriptor.
spear_status_t check_layer(const spear_layer_t *layer, LayerDesc *d) {
  if (!layer) return fail(SPEAR_ERR_INVALID_ARGUMENT, "layer is NULL");
  const spear_layer_t &l = *layer;
  if (l.N < 1 || l.K < 1) return fail(SPEAR_ERR_INVALID_ARGUMENT, "N=%d K=%d must be >= 1", l.N, l.K);
  if (l.K % 8 != 0) return fail(SPEAR_ERR_INVALID_ARGUMENT, "K=%d is not a multiple of 8", l.K);
  if (l.K % 32 != 0)
    return fail(SPEAR_ERR_UNSUPPORTED, "K=%d: the kernels need K %% 32 == 0", l.K);
  if (l.K > SPEAR_MAX_K) return fail(SPEAR_ERR_UNSUPPORTED, "K=%d above %d", l.K, SPEAR_MAX_K);
  if (l.group_size < 1 || l.K % l.group_size != 0)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "group_size=%d must divide K=%d", l.group_size, l.K);
  if (l.group_size != l.K && l.group_size % 128 != 0)
    return fail(SPEAR_ERR_UNSUPPORTED, "group_size=%d: need a multiple of 128 or G == K",
                l.group_size);
  if (!l.qweight || !l.scales || !l.zeros)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "qweight/scales/zeros must not be NULL");
  if (!aligned(l.qweight, 16)) return fail(SPEAR_ERR_INVALID_ARGUMENT, "qweight not 16-byte aligned");
  if (!aligned(l.scales, 2) || !aligned(l.zeros, 2))
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "scales/zeros not 2-byte aligned");
  if (l.rank < 0 || l.rank > SPEAR_MAX_RANK)
    return fail(l.rank < 0 ? SPEAR_ERR_INVALID_ARGUMENT : SPEAR_ERR_UNSUPPORTED,
                "rank=%d outside 0..%d", l.rank, SPEAR_MAX_RANK);
  const spear_rank_gate_t *rg = l.rank > 0 ? l.rank_gate : nullptr;
  if (l.rank > 0) {
    if (!l.A || !l.B) return fail(SPEAR_ERR_INVALID_ARGUMENT, "rank>0 needs A and B");
    if (!aligned(l.A, 16)) return fail(SPEAR_ERR_INVALID_ARGUMENT, "A must be 16-byte aligned");
    if (!aligned(l.B, 2)) return fail(SPEAR_ERR_INVALID_ARGUMENT, "B not 2-byte aligned");
    if (!rg) {
      if (!l.w_gate) return fail(SPEAR_ERR_INVALID_ARGUMENT, "the scalar gate needs w_gate");
      if (!aligned(l.w_gate, 16))
        return fail(SPEAR_ERR_INVALID_ARGUMENT, "w_gate must be 16-byte aligned");
      if (isnan(l.b_gate)) return fail(SPEAR_ERR_INVALID_ARGUMENT, "b_gate is NaN");
    } else {
      if (rg->hidden < 1 || rg->hidden > SPEAR_MAX_GATE_HIDDEN)
        return fail(rg->hidden < 1 ? SPEAR_ERR_INVALID_ARGUMENT : SPEAR_ERR_UNSUPPORTED,
                    "rank_gate hidden=%d outside 1..%d", rg->hidden, SPEAR_MAX_GATE_HIDDEN);
      if (!rg->W1 || !rg->b1 || !rg->W2 || !rg->b2)
        return fail(SPEAR_ERR_INVALID_ARGUMENT, "rank_gate needs W1, b1, W2 and b2");
      if (!aligned(rg->W1, 4) || !aligned(rg->b1, 4) || !aligned(rg->W2, 4) || !aligned(rg->b2, 4))
        return fail(SPEAR_ERR_INVALID_ARGUMENT, "rank_gate arrays not 4-byte aligned");
      if (!isfinite(rg->alpha)) return fail(SPEAR_ERR_INVALID_ARGUMENT, "rank_gate alpha not finite");
    }
  }
  d->N = l.N;
  d->K = l.K;
  d->G = l.group_size;
  d->ngroups = l.K / l.group_size;
  d->rank = l.rank;
  d->per_channel = (l.group_size == l.K);
  d->qw = (const uint32_t *)l.qweight;
  d->scales = l.scales;
  d->zeros = l.zeros;
  d->A = (const uint16_t *)l.A;
  d->B = (const uint16_t *)l.B;
  d->wg = (const uint16_t *)l.w_gate;
  d->b_gate = l.b_gate;
  d->rg_hidden = rg ? rg->hidden : 0;
  d->rg_W1 = rg ? rg->W1 : nullptr;
  d->rg_b1 = rg ? rg->b1 : nullptr;
  d->rg_W2 = rg ? rg->W2 : nullptr;
  d->rg_b2 = rg ? rg->b2 : nullptr;
  d->rg_alpha = rg ? rg->alpha : 1.f;
  if (rg) {
    d->wg = nullptr;
    d->b_gate = 0.f;
  }
  return SPEAR_OK;
}

spear_status_t check_io(spear_dtype_t dtype, const void *x, void *y) {
  if (dtype != SPEAR_F16 && dtype != SPEAR_BF16)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "dtype=%d is not SPEAR_F16 or SPEAR_BF16", (int)dtype);
  if (!x || !y) return fail(SPEAR_ERR_INVALID_ARGUMENT, "x and y must not be NULL");
  if (!aligned(x, 16)) return fail(SPEAR_ERR_INVALID_ARGUMENT, "x not 16-byte aligned");
  if (!aligned(y, 2)) return fail(SPEAR_ERR_INVALID_ARGUMENT, "y not 2-byte aligned");
  if (x == y) return fail(SPEAR_ERR_INVALID_ARGUMENT, "y must not alias x");
  return SPEAR_OK;
}

spear_status_t check_ws(void *ws, size_t have, size_t need) {
  if (need == 0) return SPEAR_OK;
  if (!ws) return fail(SPEAR_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned(ws, 256)) return fail(SPEAR_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (have < need)
    return fail(SPEAR_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, have);
  return SPEAR_OK;
}

spear_status_t hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(SPEAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Whether decode for M tokens takes the per-row-group kernels (else the
// wide launch).  Up to 32 tokens it does, except past 16 tokens (two token
// blocks) where the column threshold wants the split-K launch but no split
// fits (two token blocks of a long split's x with its scale table, or with a
// rank-64 compensator's sums, overflow the LDS) and the layer has at most 64 tiles of 128
// rows.  There the unsplit launch has few workgroups, each streaming all of
// x through its LDS along the whole of K, while the wide launch splits K
// over 128-row tiles.  Measured at 17..32 tokens (fp16, graph-replayed,
// against the unsplit launch): 16384->4096 at 32 tokens 26% and 28672->4096
// 35-38% faster, 28672->8192 15-17% rank 0 and 1-30% compensated (where a
// split fits, it beats both: 16384->4096 at 17 tokens); with more tiles the unsplit launch fills
// the chip and stays ahead (16384->16384: wide 15-22% slower, 8192->28672
// rank 0 13% slower).  The rule reads the layer's shape, rank and M only.
bool small_decode(const LayerDesc &d, int M) {
  if (M > kSmallDecodeM) return false;
  if (M <= 16 || !decode_split_wanted(M, d.K) || decode_split_fits(d, M)) return true;
  if ((d.N + 127) / 128 > kWideLongKMaxTiles) return true;
  return !plan_wide(d, M).ok;
}

// Decode for M tokens (1..SPEAR_MAX_DECODE_M): whether a launch shape fits,
// the least workspace, and the launch.
bool decode_fits(const LayerDesc &d, int M) {
  return small_decode(d, M) ? decode_supported(d, M) : plan_wide(d, M).ok;
}
size_t decode_need(const LayerDesc &d, int M) {
  return small_decode(d, M) ? decode_workspace_bytes(d, M) : wide_workspace_bytes(d, M);
}

// The decode tail of a prefill-sized call (prefill_decode_tail), when the
// decode path takes those tokens with this workspace; 0 otherwise.
int dispatch_decode_tail(const LayerDesc &d, int M, void *workspace, size_t workspace_bytes) {
  const int r = prefill_decode_tail(M);
  if (r == 0 || r > g_decode_max_m.load() || !decode_fits(d, r)) return 0;
  const size_t need = decode_need(d, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return 0;
  return r;
}
hipError_t decode_launch(const LayerDesc &d, int dtype, const void *x, void *y, int M, void *ws,
                         size_t ws_bytes, hipStream_t s) {
  if (small_decode(d, M))
    return launch_decode(d, dtype, (const uint16_t *)x, (uint16_t *)y, M, ws, ws_bytes, s);
  return launch_wide(d, dtype, (const uint16_t *)x, (uint16_t *)y, M, ws, s);
}

// The no-allocation decode entry point's workspace: one array per GPU, in
// this file's device code object, zero when loaded.  In host code `scratch`
// names a host-side stand-in, never the device array: host code only ever
// uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SPEAR_NOALLOC_SCRATCH_BYTES];

static_assert(SPEAR_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Zeroes n 32-bit words (the workspace header's counters).
__global__ void clear_words(uint32_t *p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's scratch address.  Set-up, once per device with that
// device current: look the array up (no allocation) and clear its header
// with a kernel on `stream`, ordered before the call's own launch.
spear_status_t noalloc_scratch(hipStream_t stream, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPEAR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SPEAR_ERR_UNSUPPORTED, "device %d: the no-allocation path serves devices 0..%d",
                dev, kMaxDevices - 1);
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(SPEAR_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      const int words = (int)(kWsDataOff / sizeof(uint32_t));
      hipLaunchKernelGGL(clear_words, dim3(4), dim3(256), 0, stream, (uint32_t *)p, words);
      if ((e = hipGetLastError()) != hipSuccess)
        return fail(SPEAR_ERR_HIP, "scratch set-up on device %d: %s", dev, hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SPEAR_OK;
}

}  // namespace

extern "C" {

size_t spear_workspace_bytes(const spear_layer_t *layer, int32_t M) {
  LayerDesc d;
  if (check_layer(layer, &d) != SPEAR_OK || M < 0) return 0;
  // enough for every call with 1..M tokens: both needs grow with M
  size_t need = prefill_workspace_bytes(d, M < 1 ? 1 : M);
  const int dm = M < 1 ? 1 : (M < SPEAR_MAX_DECODE_M ? M : SPEAR_MAX_DECODE_M);
  for (int m = 1; m <= dm; ++m) {  // the split launches' needs vary with M's tile plan
    const size_t dec = small_decode(d, m) ? decode_fast_workspace_bytes(d, m)
                                          : wide_workspace_bytes(d, m);
    if (dec > need) need = dec;
  }
  return need < 256 ? 256 : need;
}

spear_status_t spear_pack_int4(const uint8_t *q, int32_t *qweight, int64_t N, int64_t K,
                               spear_stream_t stream) {
  if (N < 0 || K < 0) return fail(SPEAR_ERR_INVALID_ARGUMENT, "N and K must be >= 0");
  if (K % 32 != 0)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "K=%lld is not a multiple of 32", (long long)K);
  if (N == 0 || K == 0) return ok();
  if (!q || !qweight) return fail(SPEAR_ERR_INVALID_ARGUMENT, "q and qweight must not be NULL");
  if (!aligned(qweight, 16)) return fail(SPEAR_ERR_INVALID_ARGUMENT, "qweight not 16-byte aligned");
  return hip_status(launch_pack_int4(q, qweight, N, K, (hipStream_t)stream), "pack launch");
}

spear_status_t spear_tile_int4(const int32_t *words, int32_t *qweight, int64_t N, int64_t K,
                               spear_stream_t stream) {
  if (N < 0 || K < 0) return fail(SPEAR_ERR_INVALID_ARGUMENT, "N and K must be >= 0");
  if (K % 32 != 0)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "K=%lld is not a multiple of 32", (long long)K);
  if (N == 0 || K == 0) return ok();
  if (!words || !qweight) return fail(SPEAR_ERR_INVALID_ARGUMENT, "words and qweight must not be NULL");
  if (!aligned(words, 16) || !aligned(qweight, 16))
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "words and qweight must be 16-byte aligned");
  const uintptr_t w0 = (uintptr_t)words, w1 = w0 + (uintptr_t)(N * (K / 2));
  const uintptr_t q0 = (uintptr_t)qweight, q1 = q0 + (uintptr_t)((N + 15) / 16 * 8 * K);
  if (w0 < q1 && q0 < w1)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "words and qweight overlap (not an in-place call)");
  return hip_status(launch_tile_int4(words, qweight, N, K, (hipStream_t)stream), "tile launch");
}

spear_status_t spear_linear_decode(const spear_layer_t *layer, spear_dtype_t dtype, const void *x,
                                   void *y, int32_t M, void *workspace, size_t workspace_bytes,
                                   spear_stream_t stream) {
  LayerDesc d;
  spear_status_t st = check_layer(layer, &d);
  if (st != SPEAR_OK) return st;
  if (M < 0 || M > SPEAR_MAX_DECODE_M)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "decode M=%d outside 0..%d", M, SPEAR_MAX_DECODE_M);
  if (M == 0) return ok();
  if ((st = check_io(dtype, x, y)) != SPEAR_OK) return st;
  if (!decode_fits(d, M))
    return fail(SPEAR_ERR_UNSUPPORTED, "no decode launch shape fits K=%d G=%d M=%d", d.K, d.G, M);
  if ((st = check_ws(workspace, workspace_bytes, decode_need(d, M))) != SPEAR_OK) return st;
  return hip_status(decode_launch(d, (int)dtype, x, y, M, workspace,
                                  aligned(workspace, 256) ? workspace_bytes : 0,
                                  (hipStream_t)stream),
                    "decode launch");
}

spear_status_t spear_linear_decode_noalloc(const spear_layer_t *layer, spear_dtype_t dtype,
                                           const void *x, void *y, int32_t M,
                                           spear_stream_t stream) {
  LayerDesc d;
  spear_status_t st = check_layer(layer, &d);
  if (st != SPEAR_OK) return st;
  if (M < 0 || M > SPEAR_MAX_DECODE_M)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "decode M=%d outside 0..%d", M, SPEAR_MAX_DECODE_M);
  if (M == 0) return ok();
  if ((st = check_io(dtype, x, y)) != SPEAR_OK) return st;
  if (!decode_fits(d, M))
    return fail(SPEAR_ERR_UNSUPPORTED, "no decode launch shape fits K=%d G=%d M=%d", d.K, d.G, M);
  const size_t need = decode_need(d, M);
  if (need > (size_t)SPEAR_NOALLOC_SCRATCH_BYTES)
    return fail(SPEAR_ERR_WORKSPACE,
                "decode needs %zu bytes of workspace; the no-allocation scratch holds %zu", need,
                (size_t)SPEAR_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if ((st = noalloc_scratch((hipStream_t)stream, &ws)) != SPEAR_OK) return st;
  return hip_status(decode_launch(d, (int)dtype, x, y, M, ws, SPEAR_NOALLOC_SCRATCH_BYTES,
                                  (hipStream_t)stream),
                    "decode launch");
}

spear_status_t spear_linear_prefill(const spear_layer_t *layer, spear_dtype_t dtype, const void *x,
                                    void *y, int32_t M, void *workspace, size_t workspace_bytes,
                                    spear_stream_t main_stream, spear_stream_t aux_stream) {
  LayerDesc d;
  spear_status_t st = check_layer(layer, &d);
  if (st != SPEAR_OK) return st;
  if (M < 0) return fail(SPEAR_ERR_INVALID_ARGUMENT, "prefill M=%d must be >= 0", M);
  if (M == 0) return ok();
  if (M > (1 << 24)) return fail(SPEAR_ERR_UNSUPPORTED, "prefill M=%d too large", M);
  if ((st = check_io(dtype, x, y)) != SPEAR_OK) return st;
  // a rank-0 layer may come without a workspace (then K is never split)
  if ((workspace || prefill_needs_workspace(d)) &&
      (st = check_ws(workspace, workspace_bytes, prefill_workspace_bytes(d, M))) != SPEAR_OK)
    return st;
  return hip_status(launch_prefill(d, (int)dtype, (const uint16_t *)x, (uint16_t *)y, M, workspace,
                                   (hipStream_t)main_stream, (hipStream_t)aux_stream),
                    "prefill launch");
}

spear_status_t spear_linear(const spear_layer_t *layer, spear_dtype_t dtype, const void *x, void *y,
                            int32_t M, void *workspace, size_t workspace_bytes,
                            spear_stream_t main_stream, spear_stream_t aux_stream) {
  if (M >= 0 && M <= g_decode_max_m.load())
    return spear_linear_decode(layer, dtype, x, y, M, workspace, workspace_bytes, main_stream);
  // a call whose last tile row holds few tokens: the prefill path for the
  // tokens before it, then the decode path for those few, both on
  // main_stream (rows are independent); everything is validated first
  LayerDesc d;
  int r = 0;
  if (M > 0 && check_layer(layer, &d) == SPEAR_OK && check_io(dtype, x, y) == SPEAR_OK)
    r = dispatch_decode_tail(d, M, workspace, workspace_bytes);
  if (r == 0)
    return spear_linear_prefill(layer, dtype, x, y, M, workspace, workspace_bytes, main_stream,
                                aux_stream);
  const int m0 = M - r;
  spear_status_t st = spear_linear_prefill(layer, dtype, x, y, m0, workspace, workspace_bytes,
                                           main_stream, aux_stream);
  if (st != SPEAR_OK) return st;
  return spear_linear_decode(layer, dtype, (const char *)x + (size_t)m0 * d.K * 2,
                             (char *)y + (size_t)m0 * d.N * 2, r, workspace, workspace_bytes,
                             main_stream);
}

spear_status_t spear_linear_plan(const spear_layer_t *layer, int32_t M, size_t workspace_bytes,
                                 int32_t phase, spear_plan_t *plan) {
  if (!plan) return fail(SPEAR_ERR_INVALID_ARGUMENT, "plan must not be NULL");
  if (phase < 0 || phase > 2)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "phase=%d: 0 (dispatch), 1 (decode) or 2 (prefill)", phase);
  *plan = spear_plan_t{};
  LayerDesc d;
  spear_status_t st = check_layer(layer, &d);
  if (st != SPEAR_OK) return st;
  const bool decode = phase == 1 || (phase == 0 && M >= 0 && M <= g_decode_max_m.load());
  if (decode && (M < 0 || M > SPEAR_MAX_DECODE_M))
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "decode M=%d outside 0..%d", M, SPEAR_MAX_DECODE_M);
  if (!decode && M < 0) return fail(SPEAR_ERR_INVALID_ARGUMENT, "prefill M=%d must be >= 0", M);
  if (!decode && M > (1 << 24)) return fail(SPEAR_ERR_UNSUPPORTED, "prefill M=%d too large", M);
  if (M == 0) return ok();
  // the workspace checks of the calls, with any non-null 256-byte aligned pointer
  void *const ws = workspace_bytes > 0 ? (void *)(uintptr_t)256 : nullptr;
  if (decode) {
    if (!decode_fits(d, M))
      return fail(SPEAR_ERR_UNSUPPORTED, "no decode launch shape fits K=%d G=%d M=%d", d.K, d.G, M);
    if ((st = check_ws(ws, workspace_bytes, decode_need(d, M))) != SPEAR_OK) return st;
    if (small_decode(d, M))
      describe_decode(d, M, workspace_bytes, plan);
    else
      describe_wide(d, M, plan);
  } else {
    if ((ws || prefill_needs_workspace(d)) &&
        (st = check_ws(ws, workspace_bytes, prefill_workspace_bytes(d, M))) != SPEAR_OK)
      return st;
    const int r = phase == 0 ? dispatch_decode_tail(d, M, ws, workspace_bytes) : 0;
    describe_prefill(d, M - r, workspace_bytes, plan);
    if (r > 0) plan->path = SPEAR_PATH_PREFILL_DECODE_TAIL;
  }
  return ok();
}

}  // extern "C"

// A graph under construction (capturing on its own stream) or instantiated.
struct spear_graph {
  hipStream_t main = nullptr, aux = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  bool capturing = false;
  int calls = 0;
};

namespace {

void graph_release(spear_graph *g) {
  if (g->capturing) {  // abandon the capture
    hipGraph_t tmp = nullptr;
    if (hipStreamEndCapture(g->main, &tmp) == hipSuccess && tmp) (void)hipGraphDestroy(tmp);
    (void)hipGetLastError();
  }
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->aux) (void)hipStreamDestroy(g->aux);
  if (g->main) (void)hipStreamDestroy(g->main);
}

}  // namespace

extern "C" {

spear_status_t spear_graph_begin(spear_graph_t *graph) {
  if (!graph) return fail(SPEAR_ERR_INVALID_ARGUMENT, "graph must not be NULL");
  *graph = nullptr;
  spear_graph *g = new spear_graph();
  hipError_t e = hipStreamCreateWithFlags(&g->main, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&g->aux, hipStreamNonBlocking);
  // relaxed: the calling thread may make other HIP calls while the graph is built
  if (e == hipSuccess) e = hipStreamBeginCapture(g->main, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    graph_release(g);
    delete g;
    return hip_status(e, "graph begin");
  }
  g->capturing = true;
  *graph = g;
  return ok();
}

spear_status_t spear_graph_add(spear_graph_t graph, const spear_layer_t *layer,
                               spear_dtype_t dtype, const void *x, void *y, int32_t M,
                               void *workspace, size_t workspace_bytes) {
  if (!graph) return fail(SPEAR_ERR_INVALID_ARGUMENT, "graph must not be NULL");
  if (!graph->capturing) return fail(SPEAR_ERR_INVALID_ARGUMENT, "graph already ended");
  const spear_status_t st = spear_linear(layer, dtype, x, y, M, workspace, workspace_bytes,
                                         graph->main, graph->aux);
  if (st == SPEAR_OK) ++graph->calls;
  return st;
}

spear_status_t spear_graph_end(spear_graph_t graph) {
  if (!graph) return fail(SPEAR_ERR_INVALID_ARGUMENT, "graph must not be NULL");
  if (!graph->capturing) return fail(SPEAR_ERR_INVALID_ARGUMENT, "graph already ended");
  graph->capturing = false;
  hipError_t e = hipStreamEndCapture(graph->main, &graph->graph);
  if (e != hipSuccess) return hip_status(e, "graph capture");
  e = hipGraphInstantiate(&graph->exec, graph->graph, nullptr, nullptr, 0);
  return hip_status(e, "graph instantiate");
}

spear_status_t spear_graph_launch(spear_graph_t graph, spear_stream_t stream) {
  if (!graph) return fail(SPEAR_ERR_INVALID_ARGUMENT, "graph must not be NULL");
  if (!graph->exec) return fail(SPEAR_ERR_INVALID_ARGUMENT, "graph not ended");
  return hip_status(hipGraphLaunch(graph->exec, (hipStream_t)stream), "graph launch");
}

spear_status_t spear_graph_destroy(spear_graph_t graph) {
  if (!graph) return ok();
  graph_release(graph);
  delete graph;
  return ok();
}

spear_status_t spear_set_decode_max_m(int32_t m) {
  if (m < 1 || m > SPEAR_MAX_DECODE_M)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "decode_max_m=%d outside 1..%d", m, SPEAR_MAX_DECODE_M);
  g_decode_max_m.store(m);
  return ok();
}

int32_t spear_get_decode_max_m(void) { return g_decode_max_m.load(); }

spear_status_t spear_set_decode_split_min_m(int32_t m) {
  if (m < 1 || m > kSmallDecodeM + 1)
    return fail(SPEAR_ERR_INVALID_ARGUMENT, "decode_split_min_m=%d outside 1..%d", m,
                kSmallDecodeM + 1);
  set_decode_split_min_m(m);
  return ok();
}

int32_t spear_get_decode_split_min_m(void) { return get_decode_split_min_m(); }

spear_status_t spear_set_decode_split_min_k(int32_t k) {
  if (k < 1) return fail(SPEAR_ERR_INVALID_ARGUMENT, "decode_split_min_k=%d must be >= 1", k);
  set_decode_split_min_k(k);
  return ok();
}

int32_t spear_get_decode_split_min_k(void) { return get_decode_split_min_k(); }

spear_status_t spear_set_decode_spin_limit(uint32_t polls) {
  set_decode_spin_limit(polls);
  return ok();
}

uint32_t spear_get_decode_spin_limit(void) { return get_decode_spin_limit(); }

int32_t spear_select_chunk(const int32_t *chunks, const float *pred_ms, int32_t n, float budget_ms,
                           int32_t *violated) {
  if (!chunks || !pred_ms || n < 1) {
    fail(SPEAR_ERR_INVALID_ARGUMENT, "select_chunk needs n >= 1 candidates");
    return -1;
  }
  int32_t best = -1, smallest = -1;
  for (int32_t i = 0; i < n; ++i) {
    if (chunks[i] < 1) {
      fail(SPEAR_ERR_INVALID_ARGUMENT, "chunk %d is %d (< 1)", i, chunks[i]);
      return -1;
    }
    if (smallest < 0 || chunks[i] < smallest) smallest = chunks[i];
    if (pred_ms[i] <= budget_ms && chunks[i] > best) best = chunks[i];
  }
  if (violated) *violated = best < 0 ? 1 : 0;
  ok();
  return best < 0 ? smallest : best;
}

const char *spear_status_string(spear_status_t status) {
  switch (status) {
    case SPEAR_OK: return "ok";
    case SPEAR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SPEAR_ERR_UNSUPPORTED: return "unsupported";
    case SPEAR_ERR_WORKSPACE: return "workspace missing or too small";
    case SPEAR_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *spear_last_error(void) { return g_last_error; }

spear_status_t spear_workspace_flags(const void *workspace, uint32_t *flags, spear_stream_t stream) {
  if (!workspace || !flags) return fail(SPEAR_ERR_INVALID_ARGUMENT, "workspace and flags required");
  hipError_t e = hipMemcpyAsync(flags, (const char *)workspace + offsetof(WsHeader, flags) + offsetof(WsCounter, v),
                                sizeof(uint32_t), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  return hip_status(e, "workspace flags read");
}

int32_t spear_version(void) { return 100; }

}  // extern "C"
