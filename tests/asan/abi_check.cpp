// Host-side exercise of the libspear C ABI, built with AddressSanitizer on
// the host code of the library and of this program (the library's device code
// is built as usual and never runs here).  Every call made here is one that returns on
// the host: size and plan queries, the chunk selector, settings, status
// strings, and compute calls whose arguments are invalid, which the library
// must reject before it launches anything.  No call reaches a kernel launch,
// so the program runs without a GPU.  Layer pointers are fake device
// addresses that the host code never dereferences.
//
// Exit status 0 when every expectation holds; AddressSanitizer aborts the
// program on the first invalid host memory access.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "spear.h"

namespace {

int failures = 0;

#define EXPECT(cond)                                                                   \
  do {                                                                                 \
    if (!(cond)) {                                                                     \
      std::fprintf(stderr, "abi_check: expectation failed at line %d: %s\n", __LINE__, \
                   #cond);                                                             \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

// A distinct, 256-byte aligned fake device address per index.
template <typename T>
const T *fake(uintptr_t i) {
  return reinterpret_cast<const T *>(static_cast<uintptr_t>(0x100000000ull + i * 0x1000000ull));
}

struct LayerSpec {
  int N, K, G, rank, hidden;
};

spear_rank_gate_t rank_gate(int hidden) {
  spear_rank_gate_t g{};
  g.hidden = hidden;
  g.W1 = fake<float>(20);
  g.b1 = fake<float>(21);
  g.W2 = fake<float>(22);
  g.b2 = fake<float>(23);
  g.alpha = 1.0f;
  return g;
}

spear_layer_t layer(const LayerSpec &s, const spear_rank_gate_t *rg) {
  spear_layer_t L{};
  L.N = s.N;
  L.K = s.K;
  L.group_size = s.G;
  L.qweight = fake<int32_t>(1);
  L.scales = fake<uint16_t>(2);
  L.zeros = fake<uint16_t>(3);
  L.rank = s.rank;
  L.A = s.rank ? fake<void>(4) : nullptr;
  L.B = s.rank ? fake<void>(5) : nullptr;
  L.w_gate = s.rank ? fake<void>(6) : nullptr;
  L.b_gate = 0.25f;
  L.rank_gate = rg;
  return L;
}

bool valid_status(spear_status_t st) { return st >= SPEAR_OK && st <= SPEAR_ERR_HIP; }

void check_strings() {
  for (int s = -3; s <= 10; ++s) {
    const char *t = spear_status_string(static_cast<spear_status_t>(s));
    EXPECT(t != nullptr && std::strlen(t) > 0);
  }
  EXPECT(spear_last_error() != nullptr);
  EXPECT(spear_version() > 0);
}

void check_settings() {
  const int32_t max_m = spear_get_decode_max_m();
  const int32_t smin_m = spear_get_decode_split_min_m();
  const int32_t smin_k = spear_get_decode_split_min_k();
  const uint32_t spin = spear_get_decode_spin_limit();
  for (int32_t v : {-5, 0, 1, 16, 64, 128, 129, 1 << 30}) {
    const spear_status_t st = spear_set_decode_max_m(v);
    EXPECT((st == SPEAR_OK) == (v >= 1 && v <= 128));
    const int32_t now = spear_get_decode_max_m();
    EXPECT(now >= 1 && now <= 128);
    EXPECT(std::strlen(spear_last_error()) < 4096);
    spear_set_decode_split_min_m(v);
    spear_set_decode_split_min_k(v);
  }
  spear_set_decode_spin_limit(0);
  EXPECT(spear_get_decode_spin_limit() == 0);
  EXPECT(spear_set_decode_max_m(max_m) == SPEAR_OK);
  EXPECT(spear_set_decode_split_min_m(smin_m) == SPEAR_OK);
  EXPECT(spear_set_decode_split_min_k(smin_k) == SPEAR_OK);
  EXPECT(spear_set_decode_spin_limit(spin) == SPEAR_OK);
}

// Size and plan queries over many shapes, valid and not.
void check_plans() {
  const std::vector<int> Ns = {0, 1, 15, 16, 17, 200, 4096, 11008, 28672};
  const std::vector<int> Ks = {0, 16, 32, 96, 128, 160, 4096, 11008, 28672};
  const std::vector<int> ranks = {0, 1, 32, 64, 128, 129};
  const std::vector<int> Ms = {-1, 0, 1, 2, 4, 16, 32, 33, 64, 65, 128, 129, 256, 1025, 1056, 2048};
  for (int N : Ns)
    for (int K : Ks)
      for (int G : {0, 32, 128, K, 100})
        for (int rank : ranks)
          for (int hidden : {0, 64, 65}) {
            if (hidden && !rank) continue;
            const spear_rank_gate_t rg = rank_gate(hidden);
            const spear_layer_t L = layer({N, K, G, rank, hidden}, hidden ? &rg : nullptr);
            for (int M : Ms) {
              const size_t ws = spear_workspace_bytes(&L, M);
              for (int phase = -1; phase <= 3; ++phase)
                for (size_t have : {size_t(0), ws > 0 ? ws - 1 : size_t(0), ws, 2 * ws}) {
                  spear_plan_t p;
                  std::memset(&p, 0xAB, sizeof p);
                  const spear_status_t st = spear_linear_plan(&L, M, have, phase, &p);
                  EXPECT(valid_status(st));
                  if (st == SPEAR_OK) {
                    EXPECT(p.path >= SPEAR_PATH_NONE && p.path <= SPEAR_PATH_PREFILL_DECODE_TAIL);
                    EXPECT(p.workgroups >= 0 && p.producers >= 0 && p.k_splits >= 0);
                    EXPECT(p.workspace_bytes <= have || p.workspace_bytes == 0);
                  }
                }
            }
            spear_plan_t p;
            EXPECT(spear_linear_plan(&L, 1, 0, 0, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
            EXPECT(spear_linear_plan(nullptr, 1, 0, 0, &p) == SPEAR_ERR_INVALID_ARGUMENT);
          }
  EXPECT(spear_workspace_bytes(nullptr, 1) == 0);
}

// Compute entry points with one invalid argument each: rejected, nothing launched.
void check_rejections() {
  const spear_rank_gate_t rg = rank_gate(64);
  for (const LayerSpec &s : {LayerSpec{4096, 4096, 128, 32, 0}, LayerSpec{200, 512, 512, 16, 0},
                             LayerSpec{11008, 4096, 128, 64, 64}, LayerSpec{4096, 11008, 11008, 0, 0}}) {
    const spear_layer_t L = layer(s, s.hidden ? &rg : nullptr);
    const void *x = fake<void>(10);
    void *y = const_cast<void *>(fake<void>(11));
    void *ws = const_cast<void *>(fake<void>(12));
    const size_t wsb = spear_workspace_bytes(&L, 2048);
    for (int M : {1, 16, 64, 1056}) {
      // bad dtype
      EXPECT(spear_linear(&L, static_cast<spear_dtype_t>(7), x, y, M, ws, wsb, nullptr, nullptr) ==
             SPEAR_ERR_INVALID_ARGUMENT);
      // null and misaligned activations, aliasing output
      EXPECT(spear_linear(&L, SPEAR_F16, nullptr, y, M, ws, wsb, nullptr, nullptr) ==
             SPEAR_ERR_INVALID_ARGUMENT);
      EXPECT(spear_linear(&L, SPEAR_F16, static_cast<const char *>(x) + 2, y, M, ws, wsb, nullptr,
                          nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
      EXPECT(spear_linear(&L, SPEAR_F16, x, const_cast<void *>(x), M, ws, wsb, nullptr, nullptr) ==
             SPEAR_ERR_INVALID_ARGUMENT);
      EXPECT(spear_linear_prefill(&L, SPEAR_F16, x, nullptr, M, ws, wsb, nullptr, nullptr) ==
             SPEAR_ERR_INVALID_ARGUMENT);
      if (M <= 128)
        EXPECT(spear_linear_decode(&L, SPEAR_BF16, nullptr, y, M, ws, wsb, nullptr) ==
               SPEAR_ERR_INVALID_ARGUMENT);
      if (s.rank > 0) {
        // a compensated layer needs a workspace, 256-byte aligned and large enough
        EXPECT(spear_linear(&L, SPEAR_F16, x, y, M, nullptr, 0, nullptr, nullptr) ==
               SPEAR_ERR_WORKSPACE);
        EXPECT(spear_linear(&L, SPEAR_F16, x, y, M, static_cast<char *>(ws) + 16, wsb, nullptr,
                            nullptr) == SPEAR_ERR_WORKSPACE);
        EXPECT(spear_linear(&L, SPEAR_F16, x, y, M, ws, 64, nullptr, nullptr) ==
               SPEAR_ERR_WORKSPACE);
      }
    }
    EXPECT(spear_linear_decode(&L, SPEAR_F16, x, y, 129, ws, wsb, nullptr) ==
           SPEAR_ERR_INVALID_ARGUMENT);
    EXPECT(spear_linear_decode(&L, SPEAR_F16, x, y, -1, ws, wsb, nullptr) ==
           SPEAR_ERR_INVALID_ARGUMENT);
    EXPECT(spear_linear_prefill(&L, SPEAR_F16, x, y, -1, ws, wsb, nullptr, nullptr) ==
           SPEAR_ERR_INVALID_ARGUMENT);
    EXPECT(spear_linear_prefill(&L, SPEAR_F16, x, y, 1 << 25, ws, wsb, nullptr, nullptr) ==
           SPEAR_ERR_UNSUPPORTED);
    EXPECT(spear_linear_decode_noalloc(&L, static_cast<spear_dtype_t>(3), x, y, 1, nullptr) ==
           SPEAR_ERR_INVALID_ARGUMENT);
    EXPECT(spear_linear_decode_noalloc(&L, SPEAR_F16, nullptr, y, 1, nullptr) ==
           SPEAR_ERR_INVALID_ARGUMENT);
    // M = 0 is a no-op that launches nothing
    EXPECT(spear_linear(&L, SPEAR_F16, x, y, 0, ws, wsb, nullptr, nullptr) == SPEAR_OK);
  }
  // invalid layers
  const spear_layer_t bad_k = layer({64, 48, 48, 0, 0}, nullptr);
  EXPECT(spear_linear(&bad_k, SPEAR_F16, fake<void>(10), const_cast<void *>(fake<void>(11)), 1,
                      nullptr, 0, nullptr, nullptr) != SPEAR_OK);
  spear_layer_t no_a = layer({64, 64, 64, 8, 0}, nullptr);
  no_a.A = nullptr;
  EXPECT(spear_linear(&no_a, SPEAR_F16, fake<void>(10), const_cast<void *>(fake<void>(11)), 1,
                      const_cast<void *>(fake<void>(12)), 1 << 24, nullptr, nullptr) ==
         SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_linear(nullptr, SPEAR_F16, fake<void>(10), const_cast<void *>(fake<void>(11)), 1,
                      nullptr, 0, nullptr, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
}

void check_pack_and_graph() {
  int32_t *qw = const_cast<int32_t *>(fake<int32_t>(30));
  EXPECT(spear_pack_int4(nullptr, qw, 16, 32, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_pack_int4(fake<uint8_t>(31), qw, 16, 48, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_pack_int4(fake<uint8_t>(31), qw, -1, 32, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_pack_int4(fake<uint8_t>(31), qw, 0, 32, nullptr) == SPEAR_OK);
  EXPECT(spear_tile_int4(nullptr, qw, 16, 32, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_tile_int4(fake<int32_t>(32), qw + 1, 16, 32, nullptr) ==
         SPEAR_ERR_INVALID_ARGUMENT);
  const spear_layer_t L = layer({64, 64, 64, 0, 0}, nullptr);
  EXPECT(spear_graph_add(nullptr, &L, SPEAR_F16, fake<void>(10), const_cast<void *>(fake<void>(11)),
                         1, nullptr, 0) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_graph_begin(nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_graph_end(nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_graph_launch(nullptr, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_graph_destroy(nullptr) == SPEAR_OK);
  uint32_t flags = 0;
  EXPECT(spear_workspace_flags(nullptr, &flags, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
  EXPECT(spear_workspace_flags(fake<void>(12), nullptr, nullptr) == SPEAR_ERR_INVALID_ARGUMENT);
}

// The chunk selector against its definition, on random inputs.
void check_selector() {
  std::mt19937 rng(7);
  std::uniform_int_distribution<int> nd(1, 24), cd(1, 4096);
  std::uniform_real_distribution<float> pd(0.f, 40.f);
  for (int trial = 0; trial < 20000; ++trial) {
    const int n = nd(rng);
    std::vector<int32_t> c(n);
    std::vector<float> p(n);
    for (int i = 0; i < n; ++i) {
      c[i] = cd(rng);
      p[i] = pd(rng);
    }
    const float budget = pd(rng);
    int32_t violated = -1;
    const int32_t got = spear_select_chunk(c.data(), p.data(), n, budget, &violated);
    int32_t best = -1, smallest = c[0];
    for (int i = 0; i < n; ++i) {
      if (p[i] <= budget && c[i] > best) best = c[i];
      if (c[i] < smallest) smallest = c[i];
    }
    if (best >= 0) {
      EXPECT(got == best && violated == 0);
    } else {
      EXPECT(got == smallest && violated == 1);
    }
    EXPECT(spear_select_chunk(c.data(), p.data(), n, budget, nullptr) == got);
  }
  const int32_t c1[1] = {0};
  const float p1[1] = {1.f};
  EXPECT(spear_select_chunk(c1, p1, 1, 2.f, nullptr) == -1);
  EXPECT(spear_select_chunk(nullptr, p1, 1, 2.f, nullptr) == -1);
  EXPECT(spear_select_chunk(c1, nullptr, 1, 2.f, nullptr) == -1);
  EXPECT(spear_select_chunk(c1, p1, 0, 2.f, nullptr) == -1);
}

}  // namespace

int main() {
  check_strings();
  check_settings();
  check_plans();
  check_rejections();
  check_pack_and_graph();
  check_selector();
  std::printf("abi_check: %d failed expectations\n", failures);
  return failures == 0 ? 0 : 1;
}
