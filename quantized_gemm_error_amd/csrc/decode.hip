// Decode dispatch: which compilation of the decode kernels (8 or 4 waves per
// workgroup) serves a call, and the process-wide split-K thresholds.
//
// Fewer waves in flight shorten the compensator's exchange between the
// producer and consumer workgroups (see decode_impl.inc), but leave each wave
// more K to cover.  Measured on MI355X at the Llama-7B projections: for at
// most 4 tokens and K <= 4096, 4-wave workgroups run the call faster
// (4096x4096, M = 1, compensated: 8.7 vs 10.3 us; rank 0 5.7 vs 5.9 us); with
// more tokens or a longer K, 8-wave workgroups do (11008->4096 at M = 32:
// 24.0 vs 44.8 us).  The choice depends on the shape and M only, never on
// the rank, so a layer and its rank-0 twin take the same launch shape.
#include <atomic>

#include "internal.h"

namespace spear {

namespace {

bool four_waves(const LayerDesc &L, int M) { return M <= 4 && L.K <= 4096; }

// Split-K consumers are considered from this many tokens on and for K of at
// least this many columns.  Below K = 8192 a split's tail (its partial tile
// stored, the tile's arrival counted, the partials gathered: three memory
// round trips, about 3.5 us on MI355X) is not paid back by the shorter K loop
// (measured at M = 16 and 32 on the 4096-wide projections).
std::atomic<int> g_split_min_m{16};
std::atomic<int> g_split_min_k{8192};

// Polls of the producers' count before a consumer computes the compensator's
// projections itself (a poll with a short sleep takes about a microsecond
// under load, so the default allows about a second).
std::atomic<uint32_t> g_spin_limit{1u << 20};

}  // namespace

// Split-K wanted for M tokens at K columns (its plan must still fit and the
// workspace hold its partial tiles): from the token threshold on, and, where
// K is at least twice the column threshold, from an eighth of it on, but
// never below 2 tokens (at 28672 -> 8192 the split call takes 43.9 / 44.0 /
// 44.4 us at M = 2 / 3 / 4 against 49.0 / 54.2 / 54.7 unsplit; at M = 1 it
// loses, 43.4 against 34.2).  A token threshold past 32 turns the split off.
bool decode_split_wanted(int M, int K) {
  const int mm = g_split_min_m.load(), mk = g_split_min_k.load();
  if (mm > 32 || K < mk) return false;
  const int long_k_min = (mm + 7) / 8 < 2 ? 2 : (mm + 7) / 8;
  return M >= mm || ((long long)K >= 2LL * mk && M >= long_k_min);
}

void set_decode_spin_limit(uint32_t polls) { g_spin_limit.store(polls); }
uint32_t get_decode_spin_limit() { return g_spin_limit.load(); }

void set_decode_split_min_m(int m) { g_split_min_m.store(m); }
int get_decode_split_min_m() { return g_split_min_m.load(); }
void set_decode_split_min_k(int k) { g_split_min_k.store(k); }
int get_decode_split_min_k() { return g_split_min_k.load(); }

bool decode_split_fits(const LayerDesc &L, int M) {
  return (four_waves(L, M) ? w4::plan_decode_split(L, M) : w8::plan_decode_split(L, M)).ok;
}

bool decode_supported(const LayerDesc &L, int M) {
  return four_waves(L, M) ? w4::decode_supported(L, M) : w8::decode_supported(L, M);
}

size_t decode_workspace_bytes(const LayerDesc &L, int M) {
  return four_waves(L, M) ? w4::decode_workspace_bytes(L, M) : w8::decode_workspace_bytes(L, M);
}

size_t decode_fast_workspace_bytes(const LayerDesc &L, int M) {
  return four_waves(L, M) ? w4::decode_fast_workspace_bytes(L, M)
                          : w8::decode_fast_workspace_bytes(L, M);
}

void describe_decode(const LayerDesc &L, int M, size_t ws_bytes, spear_plan_t *out) {
  four_waves(L, M) ? w4::describe_decode(L, M, ws_bytes, out)
                   : w8::describe_decode(L, M, ws_bytes, out);
}

hipError_t launch_decode(const LayerDesc &L, int dtype, const uint16_t *x, uint16_t *y, int M,
                         void *ws, size_t ws_bytes, hipStream_t s) {
  return four_waves(L, M) ? w4::launch_decode(L, dtype, x, y, M, ws, ws_bytes, s)
                          : w8::launch_decode(L, dtype, x, y, M, ws, ws_bytes, s);
}

}  // namespace spear
