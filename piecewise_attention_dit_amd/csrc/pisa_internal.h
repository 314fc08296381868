// Internal interface between the host layer (pisa_host.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

// Problem geometry derived from pisa_params on the host, passed by value to
// every kernel.
struct PisaDims {
  int B, Hq, Hkv, L, d;
  int dtype;       // 0 bf16, 1 fp32
  int bs;          // block size
  int n_blk;       // ceil(L / bs)
  int topk;
  int window;
  int group;       // 0: block rows; >= 1 PIVOT
  int n_cand;
  int causal;
  int taylor;      // 0 none, 1 order0, 2 order1, 3 hybrid
  int ratio;       // Hq / Hkv
  int n_sel;       // rows of qsel
  int n_rows;      // rows of idx
  float scale;     // softmax scale (resolved)
  int sink;        // leading candidate blocks always kept
  int klist;       // entries of an idx row: topk + sink
  float route_lambda;  // covariance-aware routing weight (0: off)
};

// Selection-row geometry shared by the indexer and the attention kernels.
// Returns the number of candidate blocks; *own and *lo receive the row's own
// block and the first block of its exact window range (lo == own without a
// window; non-causal rows have no range and lo = n_blk).
#if defined(__HIPCC__)
__host__ __device__
#endif
inline int pisa_row_geometry(const PisaDims &dm, int start_token, int *own, int *lo) {
  const int o = start_token / dm.bs;
  *own = o;
  if (!dm.causal) {
    *lo = dm.n_blk;
    return dm.n_blk;
  }
  int l = o;
  if (dm.window > 0) {
    int s = start_token - dm.window + 1;
    l = (s > 0 ? s : 0) / dm.bs;
  }
  *lo = l;
  return l;
}

// The mean first-order matrix Hbar (hybrid order, covariance routing).  bf16:
// summed over runs of kHbarRun consecutive blocks into an fp32 workspace
// [B, Hkv, runs, d, d], then the runs are added in order.  Routing also keeps
// an fp32 copy of Hbar^T [B, Hkv, d, d] after the run sums.
constexpr int kHbarRun = 16;
inline bool needs_hbar(const PisaDims &dm) { return dm.taylor == 3 || dm.route_lambda > 0.f; }
inline size_t hbar_runs_bytes(const PisaDims &dm) {
  if (!needs_hbar(dm) || dm.dtype != 0) return 0;
  const size_t runs = (size_t)(dm.n_blk + kHbarRun - 1) / kHbarRun;
  return (size_t)dm.B * dm.Hkv * runs * dm.d * dm.d * sizeof(float);
}
inline size_t stats_workspace_bytes(const PisaDims &dm) {
  const size_t hb32 = dm.route_lambda > 0.f ? (size_t)dm.B * dm.Hkv * dm.d * dm.d * sizeof(float) : 0;
  return hbar_runs_bytes(dm) + hb32;
}

// launchers (return the hipError_t of the launch)
hipError_t launch_block_stats(const PisaDims &dm, const void *Q, const void *K, const void *V,
                              void *qsel, void *ksel, float *kbar, float *vsum, void *HT, float *mcov,
                              void *ws, hipStream_t st);
hipError_t launch_indexer(const PisaDims &dm, const void *Q, const void *qsel, const void *ksel,
                          const float *mcov, int32_t *idx, int32_t *cand, int32_t *diag, hipStream_t st);
// decode (one new token per row): split-K partials in a workspace, then a merge
size_t decode_workspace_bytes(const PisaDims &dm);
hipError_t launch_decode(const PisaDims &dm, int pos, int ring, const void *q, const void *K, const void *V,
                         const float *kbar, const float *vsum, const void *HT, const int32_t *idx, void *O,
                         float *lse, void *ws, hipStream_t st);
hipError_t launch_decode_topk(const PisaDims &dm, int pos, const void *q, const void *ksel, const float *mcov,
                              int32_t *idx, int32_t *diag, hipStream_t st);
hipError_t launch_attn(const PisaDims &dm, const void *Q, const void *K, const void *V,
                       const float *kbar, const float *vsum, const void *HT, const int32_t *idx,
                       void *O, float *lse, hipStream_t st);
