// Host layer of libpisa: argument validation, buffer sizing, error reporting
// and dispatch to the gfx950 kernels.  Every check runs before anything is
// enqueued; a failing call launches nothing and writes nothing.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/pisa.h"
#include "pisa_internal.h"

namespace {

thread_local char g_err[512] = "";

pisa_status fail(pisa_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  if (getenv("PISA_LOG")) fprintf(stderr, "[pisa] %s: %s\n", pisa_status_string(s), g_err);
  return s;
}

constexpr int kMaxBlocks = 1024;   // candidates per selection row (indexer registers)
constexpr int kMaxTopk = 256;
constexpr int kMaxCand = 256;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int dtype) { return dtype == PISA_BF16 ? 2 : 4; }

pisa_status make_dims(const pisa_params *p, PisaDims *dm) {
  if (!p) return fail(PISA_E_ARG, "params is NULL");
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->L < 1 || p->d < 1)
    return fail(PISA_E_ARG, "B, Hq, Hkv, L, d must be >= 1 (got %d, %d, %d, %d, %d)", p->B, p->Hq,
                p->Hkv, p->L, p->d);
  if (p->Hq % p->Hkv != 0) return fail(PISA_E_ARG, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  const int ratio = p->Hq / p->Hkv;
  if (ratio != 1 && ratio != 2 && ratio != 4 && ratio != 8)
    return fail(PISA_E_UNSUPPORTED, "Hq/Hkv = %d not supported (1, 2, 4 or 8)", ratio);
  if (p->dtype != PISA_BF16 && p->dtype != PISA_F32) return fail(PISA_E_ARG, "unknown dtype %d", p->dtype);
  if (p->d != 64 && p->d != 128) return fail(PISA_E_UNSUPPORTED, "head dim d = %d not supported (64 or 128)", p->d);
  if (p->block != 64 && p->block != 128)
    return fail(PISA_E_UNSUPPORTED, "block size %d not supported (64 or 128)", p->block);
  if (p->causal != 0 && p->causal != 1) return fail(PISA_E_ARG, "causal must be 0 or 1");
  if (p->taylor < PISA_TAYLOR_NONE || p->taylor > PISA_TAYLOR_HYBRID)
    return fail(PISA_E_ARG, "unknown taylor mode %d", p->taylor);
  if (p->topk < 0) return fail(PISA_E_ARG, "topk must be >= 0");
  if (p->sink < 0) return fail(PISA_E_ARG, "sink must be >= 0");
  if (p->topk > kMaxTopk) return fail(PISA_E_UNSUPPORTED, "topk %d > %d", p->topk, kMaxTopk);
  if ((long long)p->topk + p->sink > kMaxTopk)
    return fail(PISA_E_UNSUPPORTED, "topk + sink = %lld > %d", (long long)p->topk + p->sink, kMaxTopk);
  if (p->window < 0) return fail(PISA_E_ARG, "window must be >= 0");
  if (p->window > 0 && !p->causal)
    return fail(PISA_E_UNSUPPORTED, "a sliding window needs causal attention");
  if (p->group < 0) return fail(PISA_E_ARG, "group must be >= 0");
  if (p->group >= 1) {
    if (p->block % p->group != 0)
      return fail(PISA_E_ARG, "block (%d) must be a multiple of group (%d)", p->block, p->group);
    if (p->n_cand < 1 || p->n_cand < p->topk)
      return fail(PISA_E_ARG, "n_cand (%d) must be >= max(1, topk)", p->n_cand);
    if (p->n_cand > kMaxCand) return fail(PISA_E_UNSUPPORTED, "n_cand %d > %d", p->n_cand, kMaxCand);
  }
  if (!std::isfinite(p->scale)) return fail(PISA_E_ARG, "scale is not finite");
  if (!std::isfinite(p->route_lambda) || p->route_lambda < 0.f)
    return fail(PISA_E_ARG, "route_lambda must be finite and >= 0");
  if (p->route_lambda > 0.f && p->taylor == PISA_TAYLOR_NONE)
    return fail(PISA_E_ARG, "covariance routing decides which blocks go to the Taylor term: taylor is NONE");
  if (p->route_lambda > 0.f && p->causal)
    return fail(PISA_E_UNSUPPORTED,
                "covariance routing is defined for non-causal rows only (its mean first-order matrix "
                "would carry later tokens into a causal row)");
  if (!p->causal && p->topk == 0 && p->sink == 0 && p->taylor == PISA_TAYLOR_NONE)
    return fail(PISA_E_ARG, "non-causal with topk = 0, no sinks and no Taylor term attends to nothing");
  const long long n_blk = (p->L + (long long)p->block - 1) / p->block;
  if (n_blk > kMaxBlocks) return fail(PISA_E_UNSUPPORTED, "%lld blocks > %d", n_blk, kMaxBlocks);
  const double elems = (double)p->B * p->Hq * p->L * p->d;
  if (elems > 4.0e12) return fail(PISA_E_ARG, "problem too large");
  dm->B = p->B; dm->Hq = p->Hq; dm->Hkv = p->Hkv; dm->L = p->L; dm->d = p->d;
  dm->dtype = p->dtype; dm->bs = p->block; dm->n_blk = (int)n_blk; dm->topk = p->topk;
  dm->window = p->window; dm->group = p->group; dm->n_cand = p->group >= 1 ? p->n_cand : 0;
  dm->causal = p->causal; dm->taylor = p->taylor; dm->ratio = ratio;
  dm->n_sel = p->group >= 1 ? (p->L + p->group - 1) / p->group : (int)n_blk;
  dm->n_rows = p->group >= 1 ? p->L : (int)n_blk;
  dm->scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->d);
  dm->sink = p->sink;
  dm->klist = p->topk + p->sink;
  dm->route_lambda = p->route_lambda;
  return PISA_OK;
}

pisa_status check_ptr(const void *ptr, const char *name, bool required) {
  if (!ptr) return required ? fail(PISA_E_ARG, "%s is NULL", name) : PISA_OK;
  if (!aligned16(ptr)) return fail(PISA_E_ARG, "%s is not 16-byte aligned", name);
  return PISA_OK;
}

pisa_status check_ws(const void *ws, size_t ws_bytes, size_t need) {
  if (ws_bytes > 0 && !ws) return fail(PISA_E_ARG, "workspace is NULL but ws_bytes = %zu", ws_bytes);
  if (ws_bytes < need) return fail(PISA_E_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  return PISA_OK;
}

pisa_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(PISA_E_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return PISA_OK;
}

#define PISA_TRY(x)                 \
  do {                              \
    pisa_status _s = (x);           \
    if (_s != PISA_OK) return _s;   \
  } while (0)

}  // namespace

extern "C" {

const char *pisa_status_string(pisa_status s) {
  switch (s) {
    case PISA_OK: return "PISA_OK";
    case PISA_E_ARG: return "PISA_E_ARG";
    case PISA_E_UNSUPPORTED: return "PISA_E_UNSUPPORTED";
    case PISA_E_WORKSPACE: return "PISA_E_WORKSPACE";
    case PISA_E_HIP: return "PISA_E_HIP";
  }
  return "PISA_E_UNKNOWN";
}

const char *pisa_last_error(void) { return g_err; }

int pisa_abi_version(void) { return PISA_ABI_VERSION; }

pisa_status pisa_validate(const pisa_params *p) {
  PisaDims dm;
  return make_dims(p, &dm);
}

pisa_status pisa_stats_layout(const pisa_params *p, size_t bytes[6]) {
  PisaDims dm;
  PISA_TRY(make_dims(p, &dm));
  if (!bytes) return fail(PISA_E_ARG, "bytes is NULL");
  const size_t es = esize(dm.dtype);
  const size_t kv = (size_t)dm.B * dm.Hkv * dm.n_blk;
  bytes[0] = (size_t)dm.B * dm.Hq * dm.n_sel * dm.d * es;
  bytes[1] = kv * dm.d * es;
  bytes[2] = kv * dm.d * sizeof(float);
  bytes[3] = kv * dm.d * sizeof(float);
  bytes[4] = dm.taylor == PISA_TAYLOR_ORDER1 ? kv * dm.d * dm.d * es
             : dm.taylor == PISA_TAYLOR_HYBRID
                 ? (dm.causal ? kv : (size_t)dm.B * dm.Hkv) * dm.d * dm.d * es   // causal: one per lo
                 : 0;
  bytes[5] = dm.route_lambda > 0.f ? kv * sizeof(float) : 0;
  return PISA_OK;
}

pisa_status pisa_index_layout(const pisa_params *p, size_t bytes[2]) {
  PisaDims dm;
  PISA_TRY(make_dims(p, &dm));
  if (!bytes) return fail(PISA_E_ARG, "bytes is NULL");
  bytes[0] = (size_t)dm.B * dm.Hq * dm.n_rows * dm.klist * sizeof(int32_t);
  bytes[1] = dm.group >= 1 ? (size_t)dm.B * dm.Hq * dm.n_sel * dm.n_cand * sizeof(int32_t) : 0;
  return PISA_OK;
}

pisa_status pisa_workspace_size(const pisa_params *p, int op, size_t *bytes) {
  PisaDims dm;
  PISA_TRY(make_dims(p, &dm));
  if (!bytes) return fail(PISA_E_ARG, "bytes is NULL");
  if (op < 0 || op > 3) return fail(PISA_E_ARG, "unknown op %d", op);
  *bytes = op == 0   ? stats_workspace_bytes(dm)
           : op == 2 ? pivot_kg_workspace_bytes(dm)
           : op == 3 ? decode_workspace_bytes(dm)
                     : 0;
  return PISA_OK;
}

pisa_status pisa_block_stats(const pisa_params *p, const void *Q, const void *K, const void *V,
                             const pisa_stats *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  PisaDims dm;
  PISA_TRY(make_dims(p, &dm));
  PISA_TRY(check_ptr(Q, "Q", true));
  PISA_TRY(check_ptr(K, "K", true));
  PISA_TRY(check_ptr(V, "V", true));
  if (!out) return fail(PISA_E_ARG, "stats is NULL");
  const bool ty = dm.taylor != PISA_TAYLOR_NONE;
  PISA_TRY(check_ptr(out->qsel, "stats.qsel", true));
  PISA_TRY(check_ptr(out->ksel, "stats.ksel", true));
  PISA_TRY(check_ptr(out->kbar, "stats.kbar", ty));
  PISA_TRY(check_ptr(out->vsum, "stats.vsum", ty));
  PISA_TRY(check_ptr(out->HT, "stats.HT", dm.taylor == PISA_TAYLOR_ORDER1 || dm.taylor == PISA_TAYLOR_HYBRID));
  PISA_TRY(check_ptr(out->mcov, "stats.mcov", dm.route_lambda > 0.f));
  const size_t need = stats_workspace_bytes(dm);
  PISA_TRY(check_ws(ws, ws_bytes, need));
  if (need && !aligned16(ws)) return fail(PISA_E_ARG, "workspace is not 16-byte aligned");
  return launched(launch_block_stats(dm, Q, K, V, out->qsel, out->ksel, out->kbar, out->vsum,
                                     out->HT, dm.route_lambda > 0.f ? out->mcov : nullptr, need ? ws : nullptr,
                                     stream),
                  "block_stats");
}

pisa_status pisa_indexer_topk(const pisa_params *p, const void *Q, const pisa_stats *stats,
                              int32_t *idx, int32_t *cand, void *ws, size_t ws_bytes,
                              hipStream_t stream) {
  PisaDims dm;
  PISA_TRY(make_dims(p, &dm));
  PISA_TRY(check_ptr(Q, "Q", dm.group >= 1));
  if (!stats) return fail(PISA_E_ARG, "stats is NULL");
  PISA_TRY(check_ptr(stats->qsel, "stats.qsel", true));
  PISA_TRY(check_ptr(stats->ksel, "stats.ksel", true));
  PISA_TRY(check_ptr(stats->mcov, "stats.mcov", dm.route_lambda > 0.f));
  PISA_TRY(check_ptr(idx, "idx", dm.klist > 0));
  PISA_TRY(check_ptr(cand, "cand", false));
  PISA_TRY(check_ws(ws, ws_bytes, 0));
  int32_t *diag = nullptr;
  if (ws && ws_bytes >= PISA_DIAG_BYTES) {
    if (!aligned16(ws)) return fail(PISA_E_ARG, "workspace is not 16-byte aligned");
    diag = static_cast<int32_t *>(ws);
  }
  if (dm.klist == 0 && !(dm.group >= 1 && cand)) return PISA_OK;  // nothing to select or write
  return launched(launch_indexer(dm, Q, stats->qsel, stats->ksel, dm.route_lambda > 0.f ? stats->mcov : nullptr,
                                 idx, cand, diag, stream),
                  "indexer_topk");
}

pisa_status pisa_sparse_attn_fwd(const pisa_params *p, const void *Q, const void *K, const void *V,
                                 const pisa_stats *stats, const int32_t *idx, void *O, float *lse,
                                 void *ws, size_t ws_bytes, hipStream_t stream) {
  PisaDims dm;
  PISA_TRY(make_dims(p, &dm));
  PISA_TRY(check_ptr(Q, "Q", true));
  PISA_TRY(check_ptr(K, "K", true));
  PISA_TRY(check_ptr(V, "V", true));
  PISA_TRY(check_ptr(O, "O", true));
  PISA_TRY(check_ptr(lse, "lse", false));
  PISA_TRY(check_ptr(idx, "idx", dm.klist > 0));
  const bool ty = dm.taylor != PISA_TAYLOR_NONE;
  if (ty) {
    if (!stats) return fail(PISA_E_ARG, "stats is NULL but taylor != NONE");
    PISA_TRY(check_ptr(stats->kbar, "stats.kbar", true));
    PISA_TRY(check_ptr(stats->vsum, "stats.vsum", true));
    PISA_TRY(check_ptr(stats->HT, "stats.HT", dm.taylor == PISA_TAYLOR_ORDER1 || dm.taylor == PISA_TAYLOR_HYBRID));
  }
  const size_t need = pivot_kg_workspace_bytes(dm);
  PISA_TRY(check_ws(ws, ws_bytes, need));
  if (need && !aligned16(ws)) return fail(PISA_E_ARG, "workspace is not 16-byte aligned");
  dm.topk = dm.klist;   // the attention kernels take topk as the width of a kept list
  return launched(launch_attn(dm, Q, K, V, ty ? stats->kbar : nullptr, ty ? stats->vsum : nullptr,
                              ty ? stats->HT : nullptr, idx, O, lse, need ? ws : nullptr, stream),
                  "sparse_attn_fwd");
}

pisa_status pisa_decode_topk(const pisa_params *p, int32_t pos, const void *q, const pisa_stats *stats,
                             int32_t *idx, hipStream_t stream) {
  PisaDims dm;
  PISA_TRY(make_dims(p, &dm));
  if (!dm.causal) return fail(PISA_E_ARG, "decode needs causal attention");
  if (pos < 0 || pos >= dm.L) return fail(PISA_E_ARG, "pos %d outside the cache [0, %d)", pos, dm.L);
  PISA_TRY(check_ptr(q, "q", true));
  if (!stats) return fail(PISA_E_ARG, "stats is NULL");
  PISA_TRY(check_ptr(stats->ksel, "stats.ksel", true));
  PISA_TRY(check_ptr(stats->mcov, "stats.mcov", dm.route_lambda > 0.f));
  PISA_TRY(check_ptr(idx, "idx", dm.klist > 0));
  if (dm.klist == 0) return PISA_OK;
  return launched(launch_decode_topk(dm, pos, q, stats->ksel, dm.route_lambda > 0.f ? stats->mcov : nullptr, idx,
                                     nullptr, stream),
                  "decode_topk");
}

}  // extern "C"

namespace {

// Checks shared by the two decode_fwd entry points (everything but the
// workspace); on success dm holds the geometry with topk = the list width.
pisa_status decode_fwd_check(const pisa_params *p, int32_t pos, int32_t ring, const void *q, const void *K,
                             const void *V, const pisa_stats *stats, const int32_t *idx, void *O, float *lse,
                             PisaDims *dm_out) {
  PisaDims dm;
  PISA_TRY(make_dims(p, &dm));
  if (!dm.causal) return fail(PISA_E_ARG, "decode needs causal attention");
  if (pos < 0 || pos >= dm.L) return fail(PISA_E_ARG, "pos %d outside the cache [0, %d)", pos, dm.L);
  if (ring < 0) return fail(PISA_E_ARG, "ring must be >= 0");
  if (ring > 0 && (dm.topk != 0 || dm.sink != 0 || dm.taylor != PISA_TAYLOR_NONE || dm.window != ring))
    return fail(PISA_E_ARG, "a ring buffer holds a pure sliding window: topk = sink = 0, taylor NONE, window = ring");
  PISA_TRY(check_ptr(q, "q", true));
  PISA_TRY(check_ptr(K, "K", true));
  PISA_TRY(check_ptr(V, "V", true));
  PISA_TRY(check_ptr(O, "O", true));
  PISA_TRY(check_ptr(lse, "lse", false));
  PISA_TRY(check_ptr(idx, "idx", ring == 0 && dm.klist > 0));
  const bool ty = dm.taylor != PISA_TAYLOR_NONE;
  if (ty) {
    if (!stats) return fail(PISA_E_ARG, "stats is NULL but taylor != NONE");
    PISA_TRY(check_ptr(stats->kbar, "stats.kbar", true));
    PISA_TRY(check_ptr(stats->vsum, "stats.vsum", true));
    PISA_TRY(check_ptr(stats->HT, "stats.HT", dm.taylor == PISA_TAYLOR_ORDER1 || dm.taylor == PISA_TAYLOR_HYBRID));
  }
  *dm_out = dm;
  return PISA_OK;
}

pisa_status decode_fwd_launch(PisaDims dm, int32_t pos, int32_t ring, const void *q, const void *K, const void *V,
                              const pisa_stats *stats, const int32_t *idx, void *O, float *lse, void *ws,
                              hipStream_t stream, const char *what) {
  const bool ty = dm.taylor != PISA_TAYLOR_NONE;
  dm.topk = dm.klist;   // the kernels take topk as the width of a kept list
  return launched(launch_decode(dm, pos, ring, q, K, V, ty ? stats->kbar : nullptr, ty ? stats->vsum : nullptr,
                                ty ? stats->HT : nullptr, ring == 0 ? idx : nullptr, O, lse, ws, stream),
                  what);
}

}  // namespace

extern "C" {

pisa_status pisa_decode_fwd(const pisa_params *p, int32_t pos, int32_t ring, const void *q, const void *K,
                            const void *V, const pisa_stats *stats, const int32_t *idx, void *O, float *lse,
                            void *ws, size_t ws_bytes, hipStream_t stream) {
  PisaDims dm;
  PISA_TRY(decode_fwd_check(p, pos, ring, q, K, V, stats, idx, O, lse, &dm));
  const size_t need = decode_workspace_bytes(dm);
  PISA_TRY(check_ws(ws, ws_bytes, need));
  if (!aligned16(ws)) return fail(PISA_E_ARG, "workspace is not 16-byte aligned");
  return decode_fwd_launch(dm, pos, ring, q, K, V, stats, idx, O, lse, ws, stream, "decode_fwd");
}

pisa_status pisa_decode_fwd_noalloc(const pisa_params *p, int32_t pos, int32_t ring, const void *q, const void *K,
                                    const void *V, const pisa_stats *stats, const int32_t *idx, void *O,
                                    float *lse, hipStream_t stream) {
  PisaDims dm;
  PISA_TRY(decode_fwd_check(p, pos, ring, q, K, V, stats, idx, O, lse, &dm));
  const size_t need = decode_workspace_bytes(dm);
  if (need > kDecodeScratchBytes)
    return fail(PISA_E_WORKSPACE, "decode needs %zu bytes of scratch, the library's fixed scratch holds %zu",
                need, kDecodeScratchBytes);
  void *ws = nullptr;
  const hipError_t e = decode_scratch(&ws);
  if (e != hipSuccess) return fail(PISA_E_HIP, "decode scratch address: %s", hipGetErrorString(e));
  return decode_fwd_launch(dm, pos, ring, q, K, V, stats, idx, O, lse, ws, stream, "decode_fwd_noalloc");
}

}  // extern "C"
