// Host-layer check under AddressSanitizer and UndefinedBehaviorSanitizer:
// pisa_host.cpp compiled for the CPU with g++ and linked against stub kernel
// launchers that only count their calls.  Every rejected call must return
// its status, launch nothing and leave sentinel-filled outputs untouched;
// valid calls must reach exactly one launcher; random problem statements
// through the host-only calls must run without undefined behaviour.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "pisa.h"
#include "pisa_internal.h"

static int g_launches = 0;

hipError_t launch_block_stats(const PisaDims &, const void *, const void *, const void *, void *, void *,
                              float *, float *, void *, float *, void *, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_indexer(const PisaDims &, const void *, const void *, const void *, const float *, int32_t *,
                          int32_t *, int32_t *, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode(const PisaDims &, int, int, const void *, const void *, const void *, const float *,
                         const float *, const void *, const int32_t *, void *, float *, void *, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_topk(const PisaDims &, int, const void *, const void *, const float *, int32_t *,
                              int32_t *, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attn(const PisaDims &, const void *, const void *, const void *, const float *, const float *,
                       const void *, const int32_t *, void *, float *, void *, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
alignas(256) static unsigned char g_scratch[256];
hipError_t decode_scratch(void **ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}
extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }

static int g_fail = 0;
#define CHECK(cond)                                                    \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAIL line %d: %s (%s)\n", __LINE__, #cond, pisa_last_error()); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

// sentinel-filled, 16-byte aligned host buffers standing in for device memory
struct Buf {
  std::vector<unsigned char> v;
  explicit Buf(size_t n) : v(n + 16, 0xA5) {}
  void *p() { return reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(v.data()) + 15) & ~uintptr_t(15)); }
  bool untouched() const {
    for (unsigned char c : v)
      if (c != 0xA5) return false;
    return true;
  }
};

static pisa_params base() {
  pisa_params p{};
  p.B = 1; p.Hq = 4; p.Hkv = 2; p.L = 1000; p.d = 128; p.dtype = PISA_BF16; p.block = 64; p.topk = 4;
  p.window = 0; p.group = 0; p.n_cand = 0; p.causal = 0; p.taylor = PISA_TAYLOR_ORDER1; p.scale = 0.f;
  p.sink = 0; p.route_lambda = 0.f;
  return p;
}

int main() {
  Buf Q(1 << 12), K(1 << 12), V(1 << 12), O(1 << 12), lse(1 << 10), idx(1 << 10), cand(1 << 10);
  Buf qsel(1 << 10), ksel(1 << 10), kbar(1 << 10), vsum(1 << 10), HT(1 << 10), mcov(1 << 10), ws(1 << 20);
  std::vector<Buf *> outs = {&O, &lse, &idx, &cand, &qsel, &ksel, &kbar, &vsum, &HT, &mcov, &ws};
  pisa_stats st{qsel.p(), ksel.p(), static_cast<float *>(kbar.p()), static_cast<float *>(vsum.p()), HT.p(),
                static_cast<float *>(mcov.p())};
  auto clean = [&]() {
    bool ok = g_launches == 0;
    for (Buf *b : outs) ok &= b->untouched();
    return ok;
  };
  const char *mis = static_cast<const char *>(K.p()) + 4;

  // ---- rejected calls: status, nothing launched, nothing written
  pisa_params p = base();
  CHECK(pisa_validate(nullptr) == PISA_E_ARG);
  CHECK(pisa_block_stats(&p, nullptr, K.p(), V.p(), &st, nullptr, 0, nullptr) == PISA_E_ARG);
  CHECK(pisa_block_stats(&p, Q.p(), mis, V.p(), &st, nullptr, 0, nullptr) == PISA_E_ARG);
  CHECK(pisa_block_stats(&p, Q.p(), K.p(), V.p(), nullptr, nullptr, 0, nullptr) == PISA_E_ARG);
  {
    pisa_stats s2 = st;
    s2.kbar = nullptr;
    CHECK(pisa_block_stats(&p, Q.p(), K.p(), V.p(), &s2, nullptr, 0, nullptr) == PISA_E_ARG);
  }
  pisa_params hy = base();
  hy.taylor = PISA_TAYLOR_HYBRID;
  CHECK(pisa_block_stats(&hy, Q.p(), K.p(), V.p(), &st, nullptr, 0, nullptr) == PISA_E_WORKSPACE);
  size_t need = 0;
  CHECK(pisa_workspace_size(&hy, 0, &need) == PISA_OK && need > 16);
  CHECK(pisa_block_stats(&hy, Q.p(), K.p(), V.p(), &st, ws.p(), need - 16, nullptr) == PISA_E_WORKSPACE);
  pisa_params rc = base();
  rc.causal = 1;
  rc.route_lambda = 0.5f;
  CHECK(pisa_block_stats(&rc, Q.p(), K.p(), V.p(), &st, ws.p(), 1 << 12, nullptr) == PISA_E_UNSUPPORTED);
  CHECK(pisa_indexer_topk(&p, Q.p(), &st, nullptr, nullptr, nullptr, 0, nullptr) == PISA_E_ARG);
  CHECK(pisa_sparse_attn_fwd(&p, Q.p(), K.p(), V.p(), &st, static_cast<int32_t *>(idx.p()), nullptr, nullptr,
                             nullptr, 0, nullptr) == PISA_E_ARG);
  CHECK(pisa_sparse_attn_fwd(&p, Q.p(), K.p(), V.p(), nullptr, static_cast<int32_t *>(idx.p()), O.p(), nullptr,
                             nullptr, 0, nullptr) == PISA_E_ARG);
  pisa_params dc = base();
  dc.causal = 1;
  dc.window = 128;
  CHECK(pisa_decode_topk(&p, 5, Q.p(), &st, static_cast<int32_t *>(idx.p()), nullptr) == PISA_E_ARG);
  CHECK(pisa_decode_fwd(&dc, 1000, 0, Q.p(), K.p(), V.p(), &st, static_cast<int32_t *>(idx.p()), O.p(), nullptr,
                        ws.p(), 1 << 12, nullptr) == PISA_E_ARG);
  CHECK(pisa_decode_fwd(&dc, 5, 128, Q.p(), K.p(), V.p(), &st, static_cast<int32_t *>(idx.p()), O.p(), nullptr,
                        ws.p(), 1 << 12, nullptr) == PISA_E_ARG);
  CHECK(pisa_decode_fwd(&dc, 5, 0, Q.p(), K.p(), V.p(), &st, static_cast<int32_t *>(idx.p()), O.p(), nullptr,
                        ws.p(), 16, nullptr) == PISA_E_WORKSPACE);
  pisa_params big = base();
  big.B = 64; big.Hq = 128; big.Hkv = 128; big.L = 64; big.causal = 1; big.topk = 0; big.taylor = PISA_TAYLOR_NONE;
  CHECK(pisa_decode_fwd_noalloc(&big, 5, 0, Q.p(), K.p(), V.p(), &st, nullptr, O.p(), nullptr, nullptr) ==
        PISA_E_WORKSPACE);
  size_t six[6];
  CHECK(pisa_stats_layout(&p, nullptr) == PISA_E_ARG);
  CHECK(pisa_index_layout(&p, nullptr) == PISA_E_ARG);
  CHECK(pisa_workspace_size(&p, 7, &need) == PISA_E_ARG);
  CHECK(clean());

  // ---- valid calls reach exactly one launcher each (the stubs write nothing)
  CHECK(pisa_stats_layout(&p, six) == PISA_OK);
  CHECK(pisa_block_stats(&p, Q.p(), K.p(), V.p(), &st, nullptr, 0, nullptr) == PISA_OK && g_launches == 1);
  CHECK(pisa_indexer_topk(&p, Q.p(), &st, static_cast<int32_t *>(idx.p()), nullptr, nullptr, 0, nullptr) ==
            PISA_OK && g_launches == 2);
  CHECK(pisa_sparse_attn_fwd(&p, Q.p(), K.p(), V.p(), &st, static_cast<int32_t *>(idx.p()), O.p(), nullptr,
                             nullptr, 0, nullptr) == PISA_OK && g_launches == 3);
  size_t dneed = 0;
  CHECK(pisa_workspace_size(&dc, 3, &dneed) == PISA_OK && dneed <= (1u << 20));
  CHECK(pisa_decode_fwd(&dc, 5, 0, Q.p(), K.p(), V.p(), &st, static_cast<int32_t *>(idx.p()), O.p(), nullptr,
                        ws.p(), dneed, nullptr) == PISA_OK && g_launches == 4);
  CHECK(pisa_decode_fwd_noalloc(&dc, 5, 0, Q.p(), K.p(), V.p(), &st, static_cast<int32_t *>(idx.p()), O.p(),
                                nullptr, nullptr) == PISA_OK && g_launches == 5);
  CHECK(pisa_decode_topk(&dc, 5, Q.p(), &st, static_cast<int32_t *>(idx.p()), nullptr) == PISA_OK &&
        g_launches == 6);
  g_launches = 0;
  CHECK(clean());

  // ---- random problem statements through the host-only calls (UBSan)
  std::mt19937_64 rng(7);
  const int32_t edge[] = {0, 1, -1, 2, 3, 7, 8, 63, 64, 65, 128, 1000, 4096, 65536, 1 << 20, INT32_MAX,
                          INT32_MIN, INT32_MAX - 1, -64};
  auto pick = [&]() -> int32_t {
    const uint64_t r = rng();
    return (r & 3) ? edge[(r >> 8) % (sizeof(edge) / sizeof(edge[0]))] : (int32_t)(r >> 16);
  };
  int accepted = 0;
  for (int it = 0; it < 200000; ++it) {
    pisa_params f{};
    f.B = pick(); f.Hq = pick(); f.Hkv = pick(); f.L = pick(); f.d = pick(); f.dtype = pick() & 3;
    f.block = pick(); f.topk = pick(); f.window = pick(); f.group = pick(); f.n_cand = pick();
    f.causal = pick() & 1; f.taylor = pick() & 3; f.sink = pick();
    f.scale = (rng() & 1) ? 0.f : 0.125f;
    f.route_lambda = (rng() & 3) ? 0.f : 0.5f;
    if (rng() & 1) {   // mostly valid shapes, knobs near their limits or wild
      f.B = 1 + (rng() % 4); f.Hkv = 1 + (rng() % 8); f.Hq = f.Hkv * (1 << (rng() % 4));
      f.d = (rng() & 1) ? 64 : 128; f.block = (rng() & 1) ? 64 : 128; f.dtype = rng() & 1;
      f.L = 1 + (int32_t)(rng() % 70000);
      if (rng() & 1) {
        f.topk = (int32_t)(rng() % 70); f.sink = (int32_t)(rng() % 4);
        f.group = (int32_t)((rng() & 1) ? 0 : 1 << (rng() % 4)); f.n_cand = (int32_t)(rng() % 300);
        f.window = (int32_t)(rng() % 5000); f.route_lambda = 0.f;
      }
    }
    size_t b6[6], b2[2], w;
    const pisa_status s = pisa_validate(&f);
    if (s == PISA_OK) ++accepted;
    CHECK(pisa_stats_layout(&f, b6) == s);
    CHECK(pisa_index_layout(&f, b2) == s);
    for (int op = 0; op < 4; ++op) CHECK(pisa_workspace_size(&f, op, &w) == s);
  }
  CHECK(accepted > 100);
  CHECK(g_launches == 0);
  std::printf("%s: %d failures, %d accepted random problems\n", g_fail ? "FAIL" : "OK", g_fail, accepted);
  return g_fail ? 1 : 0;
}
