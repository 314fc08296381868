// Internal interface between the host layer (pisa_host.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pisa.h"

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

// Whether entry j of a kept list counts for a selection row with nc
// candidate blocks (pisa_row_geometry's return value): only candidates of the
// row, 0 <= j < nc.  The -1 padding, blocks of the row's exact window range
// [lo, own] or later ones, and any other value a caller's list (reused from
// another layer) may hold are dropped, so no kernel indexes with them.
#if defined(__HIPCC__)
__host__ __device__
#endif
inline bool pisa_list_entry_kept(int j, int nc) { return j >= 0 && j < nc; }

// The mean first-order matrix Hbar (hybrid order, covariance routing).  bf16:
// summed over runs of kHbarRun consecutive blocks into an fp32 workspace
// [B, Hkv, runs, d, d], then the runs are added in order.  Causal rows use
// the prefix means Hbar(lo) over blocks [0, lo) instead, one per lo: the run
// sums are turned into exclusive prefix sums in place, and a second pass over
// the runs writes the mean before each of its blocks.  Routing also keeps an
// fp32 copy of Hbar^T [B, Hkv, d, d] after the run sums.
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
// Element offset of the Hbar^T matrix a selection row with window start lo
// uses: the one matrix of the (b, kv head) for non-causal rows, the prefix
// mean over [0, lo) for causal rows.
#if defined(__HIPCC__)
__host__ __device__
#endif
inline size_t hbar_offset(const PisaDims &dm, int bk, int lo) {
  const size_t dd = (size_t)dm.d * dm.d;
  return dm.causal ? ((size_t)bk * dm.n_blk + (size_t)lo) * dd : (size_t)bk * dd;
}

// launchers (return the hipError_t of the launch)
hipError_t launch_block_stats(const PisaDims &dm, const void *Q, const void *K, const void *V,
                              void *qsel, void *ksel, float *kbar, float *vsum, void *HT, float *mcov,
                              void *ws, hipStream_t st);
hipError_t launch_indexer(const PisaDims &dm, const void *Q, const void *qsel, const void *ksel,
                          const float *mcov, int32_t *idx, int32_t *cand, int32_t *diag, hipStream_t st);
// decode (one new token per row): split-K partials in a workspace, then a
// merge.  One group of `splits` workgroups of kDecodeWaves waves per (batch,
// kv head), about kDecodeWorkgroups workgroups over the chip in all; every
// wave writes (m, l, A, pad, o[d]) fp32 partials for each query head of its
// kv head.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeWorkgroups = 512;
inline int decode_splits(const PisaDims &dm) {
  const int groups = dm.B * dm.Hkv;
  const int s = (kDecodeWorkgroups + groups - 1) / groups;
  return s < 1 ? 1 : (s > 32 ? 32 : s);
}
inline size_t decode_workspace_bytes(const PisaDims &dm) {
  return (size_t)dm.B * dm.Hq * decode_splits(dm) * kDecodeWaves * (4 + dm.d) * sizeof(float);
}
// the library's own fixed decode scratch (pisa_decode_fwd_noalloc): capacity
// in bytes, and its device address on the current device
constexpr size_t kDecodeScratchBytes = PISA_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch(void **ptr);
hipError_t launch_decode(const PisaDims &dm, int pos, int ring, const void *q, const void *K, const void *V,
                         const float *kbar, const float *vsum, const void *HT, const int32_t *idx, void *O,
                         float *lse, void *ws, hipStream_t st);
hipError_t launch_decode_topk(const PisaDims &dm, int pos, const void *q, const void *ksel, const float *mcov,
                              int32_t *idx, int32_t *diag, hipStream_t st);
hipError_t launch_attn(const PisaDims &dm, const void *Q, const void *K, const void *V,
                       const float *kbar, const float *vsum, const void *HT, const int32_t *idx,
                       void *O, float *lse, void *ws, hipStream_t st);
// PIVOT rows in bf16 with no Taylor tail run key-gathered: a workgroup
// takes kPivotRows rows (tokens x the query heads of one KV head), inverts
// their kept sets into per-block row lists and accumulates every row's
// output in LDS; the workspace holds K and V^T of every 64-key unit in MFMA
// fragment order, 4 B Hkv n_blk block d bytes.  The LDS layout depends on the problem:
//   acc    fp32 [kPivotRows + 1][d] output accumulators, the last row a
//          dummy target (the set-up's bitmaps [32 words][kPivotRows] and four
//          int[1024] block arrays overlay it)
//   ml     fp32 running maxima, one copy per wave [4][kPivotRows + 1], and
//          the running sums [kPivotRows + 1]
//   px     four tile slots of kPivotSlotBytes: P^T fragments (64 lanes x 32
//          bytes), the 16 row maxima and the 16 row sums
//   bkt    u8 row ids of the per-block lists, ent_cap entries
//   til    u32 tiles, tile_cap entries
//   small  int[4]: list entries, tiles
constexpr int kPivotRows = 256;
constexpr int kPivotLdsMax = 160 * 1024;
constexpr int kPivotSlotBytes = 64 * 32 + 32 * 4;
struct PivotLds {
  int acc, ml, px, bkt, til, small, total;
  int ent_cap, tile_cap;
};
#if defined(__HIPCC__)
__host__ __device__
#endif
inline PivotLds pivot_lds(const PisaDims &dm) {
  PivotLds y;
  // a row keeps its list entries and, causal, the window range [lo, own]
  const int win = dm.causal ? (dm.window > 0 ? (dm.window - 1) / dm.bs + 2 : 1) : 0;
  const long long ent = (long long)kPivotRows * (dm.klist + win);
  y.ent_cap = ent > (1 << 20) ? (1 << 20) : (int)ent;
  const int nh = dm.bs / 64;
  const int used = dm.n_blk < y.ent_cap ? dm.n_blk : y.ent_cap;   // blocks with a non-empty list
  y.tile_cap = nh * (y.ent_cap / 16 + used);
  y.acc = 0;
  y.ml = (kPivotRows + 1) * dm.d * 4;                 // one dummy row
  y.px = y.ml + ((5 * (kPivotRows + 1) * 4 + 15) & ~15);
  y.bkt = y.px + 4 * kPivotSlotBytes;
  y.til = y.bkt + ((y.ent_cap + 15) & ~15);
  y.small = y.til + y.tile_cap * 4;
  y.total = y.small + 16;
  return y;
}
inline bool pivot_kg_supported(const PisaDims &dm) {
  if (dm.dtype != 0 || dm.group < 1 || dm.taylor != 0) return false;
  if ((dm.d != 64 && dm.d != 128) || (dm.bs != 64 && dm.bs != 128)) return false;
  // bitmaps of 32 words per row; row ids in a byte; tiles pack the block in
  // 10 bits and the list offset in 15
  if (dm.n_blk > 1024 || dm.ratio < 1 || dm.ratio > kPivotRows) return false;
  const PivotLds y = pivot_lds(dm);
  return y.ent_cap <= 32768 && y.total <= kPivotLdsMax;
}
inline size_t pivot_kg_workspace_bytes(const PisaDims &dm) {
  return pivot_kg_supported(dm) ? (size_t)dm.B * dm.Hkv * dm.n_blk * dm.d * dm.bs * 4 : 0;
}
