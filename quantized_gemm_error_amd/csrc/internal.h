// Host-side declarations shared by the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spear.h"

namespace spear {

// One counter per 128-byte line, so that atomics on different counters do
// not queue on the same line.
struct alignas(128) WsCounter {
  uint32_t v;
  uint32_t pad[31];
};

// Output tiles (128 rows each) of the split-K decode launch: one arrival
// counter each in the header.
constexpr int kMaxSplitTiles = 128;

// Workspace header: the first 18432 bytes of every workspace.  Zeroed once by
// the caller; each decode launch that uses it leaves the counters at zero.
struct WsHeader {
  WsCounter arrive;    // compensator producers that published their partials
  WsCounter flags;     // sticky diagnostics (bit 0: bounded wait expired)
  WsCounter done_top;  // slots of finished workgroups that are complete
  WsCounter done[8];   // finished workgroups, by blockIdx % 8
  WsCounter pad[5];
  WsCounter tile[kMaxSplitTiles];  // split-K decode: K-splits of each output tile that are in
};
static_assert(sizeof(WsHeader) == 2048 + 128 * kMaxSplitTiles, "workspace header size");

// The header holds every counter a call relies on finding at zero; from
// kWsDataOff on, every byte a call reads it has written itself first, so one
// workspace may serve several layers.
constexpr size_t kWsDataOff = sizeof(WsHeader);
static_assert(kWsDataOff % 256 == 0, "data region 256-byte aligned");


// Everything a launcher needs, already validated.
struct LayerDesc {
  int N, K, G, ngroups, rank;
  bool per_channel;
  const uint32_t *qw;
  const uint16_t *scales, *zeros;
  const uint16_t *A, *B, *wg;
  float b_gate;
  // per-rank gate (rg_hidden > 0): y += rg_alpha B (gamma(t) * t), t = A x
  int rg_hidden;
  const float *rg_W1, *rg_b1, *rg_W2, *rg_b2;
  float rg_alpha;
  int gate_rows() const { return rg_hidden > 0 ? 0 : 1; }  // rows of [A; w_g] past A
};

// Derived decode launch geometry.
struct DecodePlan {
  bool ok;         // the shape fits the LDS and staging limits
  int mb;          // 16-token blocks (1 or 2)
  int wr;          // 16-row blocks per consumer workgroup
  int n_tiles;     // consumer workgroups
  int rb_a;        // 16-row blocks of [A; w_g]
  int ks;          // K-splits of the producers
  int producers;   // rb_a * ks (0 when rank == 0)
  int nb, nbw;     // 128-wide K blocks; block iterations per wave
  int xmode;       // 0: all of x staged once; 1: staged in chunks
  int ci, xc;      // chunk: block iterations and K columns
  int xstr;        // LDS row stride of the staged activation (halves)
  int xzero;       // column of the zero strip in each staged row
  int nbw_pad;     // block iterations rounded up to a multiple of the ring depth
  int sz_off;      // byte offset of the scale/zero table in dynamic LDS
  int red_off;     // byte offset of the wave-reduction buffer in dynamic LDS
  int rg_off;      // per-rank gate scratch (0 when the layer has none)
  size_t lds;      // dynamic LDS bytes
  // split-K consumers (ksp > 1): ksp K-splits of nbs blocks for each 128-row
  // tile; their fp32 partial tiles start at split_off in the workspace
  int ksp, nbs, ngs;
  size_t split_off, split_bytes;
};

// Launch geometry of the wide decode kernel (33..128 tokens, wide.hip).
struct WidePlan {
  bool ok;
  int mb, r;             // 16-token blocks (4 or 8); 16-row blocks per wave
  int rb_a, ks, producers, rp1;
  int nb, n_tiles, ksp, nbs;
  int buf_halves, red_off;
  bool direct;           // rank 0, one split: the main kernel writes y itself
  bool fused;            // one launch: the kernel finishes its tiles (split sums, U B^T)
  size_t lds;
  size_t tp_off, u_off, part_off, end;  // workspace: [A; w_g] x sums, U, partial outputs
};
WidePlan plan_wide(const LayerDesc &L, int M);
size_t wide_workspace_bytes(const LayerDesc &L, int M);
void describe_wide(const LayerDesc &L, int M, spear_plan_t *out);
hipError_t launch_wide(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                       void *ws, hipStream_t s);

// Decode, dispatched per call to one of two compilations of the same kernels
// (8 or 4 waves per workgroup; decode.hip picks).
bool decode_supported(const LayerDesc &L, int M);
size_t decode_workspace_bytes(const LayerDesc &L, int M);       // required
size_t decode_fast_workspace_bytes(const LayerDesc &L, int M);  // enough for the split-K launch
bool decode_split_wanted(int M, int K);  // the token and column thresholds (decode.hip)
bool decode_split_fits(const LayerDesc &L, int M);  // a split-K launch shape exists
void set_decode_split_min_m(int m);
int get_decode_split_min_m();
void set_decode_split_min_k(int k);
int get_decode_split_min_k();
void set_decode_spin_limit(uint32_t polls);
uint32_t get_decode_spin_limit();

#define SPEAR_DECODE_VARIANT_API                                                          \
  DecodePlan plan_decode(const LayerDesc &L, int M);                                      \
  DecodePlan plan_decode_split(const LayerDesc &L, int M); /* ok == false: no split */    \
  bool decode_supported(const LayerDesc &L, int M);                                       \
  size_t decode_workspace_bytes(const LayerDesc &L, int M);                               \
  size_t decode_fast_workspace_bytes(const LayerDesc &L, int M);                          \
  hipError_t launch_decode(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, \
                           int M, void *ws, size_t ws_bytes, hipStream_t s);               \
  void describe_decode(const LayerDesc &L, int M, size_t ws_bytes, spear_plan_t *out);
namespace w8 { SPEAR_DECODE_VARIANT_API }
namespace w4 { SPEAR_DECODE_VARIANT_API }
#undef SPEAR_DECODE_VARIANT_API
void describe_decode(const LayerDesc &L, int M, size_t ws_bytes, spear_plan_t *out);
void describe_prefill(const LayerDesc &L, int M, size_t ws_bytes, spear_plan_t *out);
size_t prefill_workspace_bytes(const LayerDesc &L, int M);
bool prefill_needs_workspace(const LayerDesc &L);  // false: optional (splits K when given)
int prefill_decode_tail(int M);  // tokens of an M-token call the dispatch gives to decode (0: none)

// prefill.hip kernels shared with the wide decode launch
hipError_t launch_form_u(const LayerDesc &L, const float *Tp, int ks, int M, float *U,
                         hipStream_t s);
hipError_t launch_finish_parts(const LayerDesc &L, int dtype, uint16_t *y, int M, const float *part,
                               int ks, const float *U, bool scale_rows, hipStream_t s);

hipError_t launch_pack_int4(const uint8_t *q, int32_t *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_tile_int4(const int32_t *words, int32_t *out, int64_t N, int64_t K,
                            hipStream_t s);
hipError_t launch_decode(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                         void *ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_prefill(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                          void *ws, hipStream_t main_s, hipStream_t aux_s);

}  // namespace spear
