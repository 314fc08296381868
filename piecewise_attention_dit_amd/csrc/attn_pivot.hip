// Stage C, bf16, PIVOT rows (one kept list per token) with no Taylor tail:
// exact online-softmax attention over each token's own kept blocks, computed
// key-gathered on gfx950 MFMA.
//
// PIVOT page, steps 1-4: every member of a group re-ranks its proxy's list,
// so the tokens of a tile keep different blocks (a row needs 33 of the ~600
// blocks its neighbours keep between them).  PISA page, section 2: exact
// terms e^{q k} v over the selected blocks, o = N / D.  Sliding Window
// Attention page: the causal window range is kept exactly; blocks outside
// the kept set are never read.
//
// Walking the union of a tile's lists would multiply every query row by
// every block any of its neighbours keeps.  Instead a workgroup takes a pool
// of 256 rows (tokens x the query heads of one KV head), inverts their kept
// sets into per-block row lists and cuts each list into tiles of up to 16
// rows that all keep the block (a 64-key half of it for 128-key blocks).
// Four waves, one per SIMD, take a round of four tiles at a time:
//   phase 1  wave p computes tile p of the round on MFMA 16x16x32, transposed
//            so a lane owns a query row: S^T = K Q^T (the gathered Q rows
//            from memory), its own row maxima, and P^T in bf16 as the MFMA B
//            operand, into an LDS slot;
//   phase 2  wave p takes the quarter p of the features for all four tiles:
//            O^T = V^T P^T.  During the next round's phase 1 each tile row
//            folds into the row's fp32 accumulator in LDS (rescale by the
//            running maximum); the softmax of that round's tile runs in
//            four steps while the folds wait on LDS.  The row sums of the
//            bf16 weights come from phase 1; wave 0 folds them.
// With one wave per SIMD every wait is exposed, and a kilobyte load ties up
// the CU's load path for about 16 cycles, so no round issues its loads in
// one burst: this round's V^T quarters, then the next own tile's Q and K, go
// out between the folds of phase 1 (phase 2 issues no loads), and the list
// lookups behind those addresses come one phase earlier still.
// K and V^T come from a copy of every 64-key unit in MFMA fragment order
// (V^T keys in the order the MFMA takes P^T from the S^T registers): an
// operand load reads one contiguous kilobyte, where loading a fragment from
// the row-major tensors makes every lane touch its own 16 bytes.
// Each wave keeps its own copy of the running maxima, so the four quarters
// of a row never race; tiles are folded in list order and each row meets a
// block at most once, so every row merges its partials in ascending block
// order, whatever the order of rows inside a block's list: results are
// bitwise reproducible.
#include "attn_tiles.h"

using namespace pisa_attn;

namespace {

constexpr int kPvRows = kPivotRows;   // rows per workgroup
constexpr int kPvRowsA = kPvRows + 1; // accumulator rows: the last is a dummy
constexpr int kPvWaves = 4;
constexpr int kPvThreads = kPvWaves * 64;
constexpr int kPvTile = 16;           // rows per tile
static_assert(kPvThreads == kPvRows, "set-up takes one thread per row");

// position q (0..31) of a 32-key group of the V^T fragments holds key
// perm32(q): the MFMA 16x16x32 B operand that a lane builds from the S^T
// accumulators of two 16-key tiles takes key 16 (i / 4) + 4 g + i % 4 as its
// k index 8 g + i
PISA_DEV int perm32(int q) { return 16 * ((q & 7) >> 2) + 4 * (q >> 3) + (q & 3); }

// K and V^T of every 64-key unit (half hh of block j) in MFMA fragment order,
// so that each operand load of the attention kernel reads one contiguous
// kilobyte (lane l at bytes 16 l .. 16 l + 15).  Unit u = (bk, j, hh) holds
// 16 D sixteen-byte chunks:
//   KF chunk (m KQ + ks) 64 + l: K[key 16 m + l % 16][32 ks + 8 (l / 16) ..+7]
//      (the A operand of S^T = K Q^T, 16-key tile m, K-step ks);
//   VF chunk 8 D + (ft 2 + s2) 64 + l: V[key(32 s2 + 8 (l / 16) + i)][16 ft + l % 16],
//      i = 0..7, key(p) = 32 (p / 32) + perm32(p % 32) (the A operand of
//      O^T = V^T P^T, feature tile ft, K-step s2);
// keys past the sequence end are zero.
template <int D, int BS>
__global__ __launch_bounds__(256) void kv_prep(PisaDims dm, const uint16_t *__restrict__ K,
                                               const uint16_t *__restrict__ V, u32x4_t *__restrict__ KVF) {
  constexpr int NH = BS / 64, KQ = D / 32;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long units = (long long)dm.B * dm.Hkv * dm.n_blk * NH;
  if (gid >= units * 16 * D) return;
  const long long u = gid / (16 * D);
  const int r = (int)(gid % (16 * D));
  const int hh = (int)(u % NH);
  const long long bj = u / NH;
  const int j = (int)(bj % dm.n_blk);
  const long long bk = bj / dm.n_blk;
  const int key0 = j * BS + 64 * hh;
  u32x4_t out = {0u, 0u, 0u, 0u};
  if (r < 8 * D) {
    const int l = r % 64, q = r / 64, m = q / KQ, ks = q % KQ;
    const int key = key0 + 16 * m + l % 16;
    if (key < dm.L)
      out = *reinterpret_cast<const u32x4_t *>(K + ((size_t)bk * dm.L + key) * D + 32 * ks + 8 * (l / 16));
  } else {
    const int r2 = r - 8 * D;
    const int l = r2 % 64, q = r2 / 64, ft = q / 2, s2 = q % 2;
    const int e = 16 * ft + l % 16, g = l / 16;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const int k0 = key0 + 32 * s2 + perm32(8 * g + i), k1 = key0 + 32 * s2 + perm32(8 * g + i + 1);
      const uint32_t lo = k0 < dm.L ? V[((size_t)bk * dm.L + k0) * D + e] : 0u;
      const uint32_t hi = k1 < dm.L ? V[((size_t)bk * dm.L + k1) * D + e] : 0u;
      out[i / 2] = lo | (hi << 16);
    }
  }
  KVF[gid] = out;
}

// max and sum of x over lanes l and l ^ 16 (v_permlane16_swap_b32, as
// pair_max_f)
PISA_DEV float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
PISA_DEV float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// accumulator float index of (row, 16-byte chunk): chunks of a row permuted
// by the row's low bits, so the 16 rows of a tile fall on different banks
template <int D>
PISA_DEV int acc_at(int row, int chunk) {
  return row * D + 4 * (chunk ^ (row & (D / 4 - 1)));
}

struct Tile {
  int j, hh, start, n;   // block, 64-key half, first list entry, rows
};
PISA_DEV Tile tile_of(uint32_t v) {
  return Tile{(int)(v & 1023u), (int)((v >> 29) & 1u), (int)((v >> 10) & 0x7FFFu), (int)((v >> 25) & 15u) + 1};
}

template <int D, int BS>
__global__ __launch_bounds__(kPvThreads, 1) void attn_pivot_kg(AttnArgs a, const u32x4_t *__restrict__ KVF,
                                                                PivotLds ly) {
  constexpr int NH = BS / 64;   // 64-key halves of a block (a tile takes one)
  constexpr int KQ = D / 32;    // K-steps of S^T = K Q^T
  constexpr int QF = D / 4;     // features of a wave's quarter
  constexpr int MQ = QF / 16;   // 16-feature tiles of a quarter
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const PisaDims &dm = a.dm;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = l & 15, g = l >> 4;

  // ---- workgroup -> (b, kv head, token tile); row r < NR -> (head r / TT, token T0 + r % TT)
  const int R = dm.ratio;
  const int TT = kPvRows / R, NR = R * TT;
  const int ntile = (dm.L + TT - 1) / TT;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  // causal pools see more blocks the later their tokens: the longest first,
  // so the grid does not end on them
  const int tile = dm.causal ? ntile - 1 - logical % ntile : logical % ntile;
  const int bk = logical / ntile;
  const int b = bk / dm.Hkv, hk = bk % dm.Hkv;
  const int T0 = tile * TT;
  const bool causal = dm.causal != 0;

  float *acc = reinterpret_cast<float *>(lds + ly.acc);
  float *mrun = reinterpret_cast<float *>(lds + ly.ml);   // [4][257]
  float *lrun = mrun + kPvWaves * kPvRowsA;                // [257]
  uint8_t *px = lds + ly.px;
  uint8_t *bkt = lds + ly.bkt;
  uint32_t *til = reinterpret_cast<uint32_t *>(lds + ly.til);
  int *small = reinterpret_cast<int *>(lds + ly.small);
  // set-up arrays, on top of the accumulators
  uint32_t *bm = reinterpret_cast<uint32_t *>(lds + ly.acc);   // [32 words][256 rows]
  int *cnt = reinterpret_cast<int *>(bm + 32 * kPvRows);       // rows per block
  int *cnt2 = cnt + 1024;                                      // slots handed out
  int *off = cnt2 + 1024;                                      // list offsets
  int *tof = off + 1024;                                       // tile offsets

  // ---- 1. kept sets as bitmaps [word][row], one thread per row: list
  // entries that are candidates of the row, and the causal window range
  for (int i = tid; i < 32 * kPvRows + 2 * 1024; i += kPvThreads) bm[i] = 0u;
  __syncthreads();
  const int klist = dm.topk;
  const int r_me = tid;
  const int t_me = T0 + r_me % TT;
  const bool row_ok = r_me < NR && t_me < dm.L;
  if (row_ok) {
    const int h = hk * R + r_me / TT;
    int own, lo;
    const int nc = pisa_row_geometry(dm, t_me, &own, &lo);
    if (a.idx && klist > 0) {
      const int32_t *lst = a.idx + ((size_t)(b * dm.Hq + h) * dm.n_rows + t_me) * klist;
      for (int k0 = 0; k0 < klist; k0 += 16) {
        int jj[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) jj[i] = k0 + i < klist ? lst[k0 + i] : -1;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (pisa_list_entry_kept(jj[i], nc)) atomicOr(&bm[(jj[i] >> 5) * kPvRows + r_me], 1u << (jj[i] & 31));
      }
    }
    if (causal)
      for (int j = lo; j <= own; ++j) atomicOr(&bm[(j >> 5) * kPvRows + r_me], 1u << (j & 31));
  }
  __syncthreads();
  // ---- 2. rows per block: each row walks its bits.  Causal rows reach no
  // block past the last row's own block.
  const int jmax = causal ? min(dm.n_blk - 1, (min(T0 + TT, dm.L) - 1) / BS) : dm.n_blk - 1;
  const int nwd = jmax / 32 + 1;
  if (row_ok)
    for (int wd = 0; wd < nwd; ++wd) {
      uint32_t bits = bm[wd * kPvRows + r_me];
      while (bits) {
        const int bb = __builtin_ctz(bits);
        bits &= bits - 1u;
        atomicAdd(&cnt[wd * 32 + bb], 1);
      }
    }
  __syncthreads();
  // ---- 3. list and tile offsets (wave 0, 16 blocks per lane)
  if (w == 0) {
    int se = 0, stl = 0;
    int ce[16], ct[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = l * 16 + i;
      ce[i] = j <= jmax ? cnt[j] : 0;
      ct[i] = NH * ((ce[i] + kPvTile - 1) / kPvTile);
      se += ce[i];
      stl += ct[i];
    }
    const int ie = wave_incl_scan(se), it = wave_incl_scan(stl);
    int pe = ie - se, pt = it - stl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = l * 16 + i;
      if (j <= jmax) {
        off[j] = pe;
        tof[j] = pt;
      }
      pe += ce[i];
      pt += ct[i];
    }
    if (l == 63) {
      small[0] = ie;
      small[1] = it;
    }
  }
  __syncthreads();
  // ---- 4. the per-block row lists (a row's slot from a second count) and
  // the tiles, half by half
  if (row_ok)
    for (int wd = 0; wd < nwd; ++wd) {
      uint32_t bits = bm[wd * kPvRows + r_me];
      while (bits) {
        const int j = wd * 32 + __builtin_ctz(bits);
        bits &= bits - 1u;
        const int s = atomicAdd(&cnt2[j], 1);
        bkt[off[j] + s] = (uint8_t)r_me;
      }
    }
  for (int j = tid; j <= jmax; j += kPvThreads) {
    const int n = cnt[j];
    const int nt = (n + kPvTile - 1) / kPvTile;
    for (int i = 0; i < NH * nt; ++i) {
      const int hh = i / nt, it = i % nt;
      til[tof[j] + i] = (uint32_t)j | ((uint32_t)(off[j] + kPvTile * it) << 10) |
                        ((uint32_t)(min(kPvTile, n - kPvTile * it) - 1) << 25) | ((uint32_t)hh << 29);
    }
  }
  __syncthreads();
  const int n_tiles = small[1];
  __syncthreads();   // the set-up arrays are dead: the accumulators take their place
  // ---- 5. accumulators 0, running maxima -inf, sums 0
  for (int i = tid; i < kPvRowsA * D / 4; i += kPvThreads) reinterpret_cast<f32x4_t *>(acc)[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int i = tid; i < kPvWaves * kPvRowsA; i += kPvThreads) mrun[i] = kNegInf;
  for (int i = tid; i < kPvRowsA; i += kPvThreads) lrun[i] = 0.f;
  __syncthreads();

  const int p = w;
  const float sl2 = a.sl2;
  const uint16_t *Qb = static_cast<const uint16_t *>(a.Q);
  // this kv head's units: 16 D chunks each, KF then VF
  const u32x4_t *KVh = KVF + (size_t)bk * dm.n_blk * NH * 16 * D;
  float *mown = mrun + p * kPvRowsA;

  // A tile as its own-tile wave sees it: block, half, rows, the lane's token
  // (row c), and where the lane's Q and K loads read.  Q rows are read four
  // lanes to a row (lane l: row l / 4, bytes 16 (l % 4) of each 64-byte
  // chunk) and moved to the MFMA layout (lane c + 16 g: row c, chunk g) at use.
  struct Own {
    Tile ot;
    int ott;
    const uint16_t *qp;
    const u32x4_t *kp;
  };
  auto own_of = [&](const Tile &ot, int orow, int qrow) {
    Own o;
    o.ot = ot;
    o.ott = T0 + orow % TT;
    const int tq = T0 + qrow % TT, hq = hk * R + qrow / TT;
    o.qp = Qb + ((size_t)(b * dm.Hq + hq) * dm.L + tq) * D + 8 * (l & 3);
    o.kp = KVh + (size_t)(ot.j * NH + ot.hh) * 16 * D + l;
    return o;
  };
  auto own_read = [&](int ti) {
    const Tile ot = tile_of(til[ti]);
    return own_of(ot, bkt[ot.start + min(c, ot.n - 1)], bkt[ot.start + min(l >> 2, ot.n - 1)]);
  };
  // operands of the current round: the own tile's Q and K (phase 1), the
  // lane's row of each tile (-1 for none) and V^T quarter p (phase 2)
  constexpr int NOWN = 5 * KQ;   // loads of an own tile: KQ of Q, 4 KQ of K
  u32x4_t qf[KQ], kf[4][KQ], vq[4][MQ][2];
  int rrow[4];
  auto own_load = [&](const Own &o, int i) {
    if (i < KQ)
      qf[i] = *reinterpret_cast<const u32x4_t *>(o.qp + 32 * i);
    else
      kf[(i - KQ) / KQ][(i - KQ) % KQ] = o.kp[(i - KQ) * 64];
  };
  // rows and V^T quarter of tile t0 + s (tiles past the end of the list
  // repeat the last one and are not used: every round issues the same loads
  // in the same order, so the compiler's wait counts see later loads as
  // younger on every path)
  auto round_rows = [&](int t0, const uint32_t (&tw)[4], int (&rr)[4], const u32x4_t *(&vp)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const Tile tt = tile_of(tw[s]);
      const int r = bkt[tt.start + min(c, tt.n - 1)];
      rr[s] = c < tt.n ? r : -1;   // tiles past the end: phase 2 drops them
      vp[s] = KVh + (size_t)(tt.j * NH + tt.hh) * 16 * D + 8 * D + MQ * p * 2 * 64 + l;
    }
  };
  // A round's O^T quarters wait in registers and fold into the accumulators
  // during the next round's phase 1, in tile order.  Entries that fold
  // nothing (no row, or no visible key) go to a dummy row, so the folds have
  // no branches and their LDS traffic can overlap the softmax.
  f32x4_t po[4][MQ];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int mq = 0; mq < MQ; ++mq) po[s][mq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int prow[4] = {kPvRows, kPvRows, kPvRows, kPvRows};
  float pmt[4] = {0.f, 0.f, 0.f, 0.f}, plt[4] = {0.f, 0.f, 0.f, 0.f};
  // between(s) runs while the reads of tile s's rows are in flight
  auto fold = [&](auto &&between) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int row = prow[s];
      // every read of the row before any write: one LDS round trip per tile
      f32x4_t *ap[MQ];
      f32x4_t av[MQ];
#pragma unroll
      for (int mq = 0; mq < MQ; ++mq) {
        ap[mq] = reinterpret_cast<f32x4_t *>(acc + acc_at<D>(row, (QF * p + 16 * mq + 4 * g) / 4));
        av[mq] = *ap[mq];
      }
      const float mo = mown[row];
      const float lo = p == 0 ? lrun[row] : 0.f;
      __builtin_amdgcn_sched_barrier(0);
      between(s);
      __builtin_amdgcn_sched_barrier(0);
      const float mn = fmaxf(mo, pmt[s]);
      const float ca = fast_exp2(mo - mn), cb = fast_exp2(pmt[s] - mn);
#pragma unroll
      for (int mq = 0; mq < MQ; ++mq) {
        f32x4_t nv;
#pragma unroll
        for (int r = 0; r < 4; ++r) nv[r] = av[mq][r] * ca + po[s][mq][r] * cb;
        *ap[mq] = nv;
      }
      // the four lanes of a row store the same values
      mown[row] = mn;
      if (p == 0) lrun[row] = lo * ca + plt[s] * cb;
    }
  };
  // own tiles of this round (m0) and the next (m1, loaded during this round)
  Own m0, m1;
  const u32x4_t *vpc[4];   // this round's V^T quarters
  auto round = [&](int rd) {
    const int t0 = kPvWaves * rd, ti = t0 + p;
    const bool act = ti < n_tiles;
    uint8_t *slot = px + p * kPivotSlotBytes;
    // ================= phase 1: tile t0 + p, and the folds of the last round
    u32x4_t qm[KQ];
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) qm[ks][i] = __builtin_amdgcn_ds_bpermute((4 * c + g) << 2, (int)qf[ks][i]);
    const int j = m0.ot.j, hh = m0.ot.hh, t = m0.ott;
    const bool rv = act && c < m0.ot.n;
    // S^T = K Q^T per 16-key tile: lane holds keys 16 m + 4 g + r of row c
    f32x4_t sacc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f32x4_t sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) sa = mfma16(kf[m][ks], qm[ks], sa);
      sacc[m] = sa;
    }
    __builtin_amdgcn_sched_barrier(0);
    // masks: the last visible key of the unit is the sequence end or, in the
    // token's own block (causal), the token itself
    const int kbase = j * BS + 64 * hh;
    const bool diag = causal && j == t / BS;
    const int lim = (diag ? t : dm.L - 1) - kbase;
    float mx = kNegInf, mref = 0.f, ls = 0.f;
    bool any = false;
    u32x4_t pb[2];
    // P^T as the B operand of O^T = V^T P^T: K-step h takes the 16-key tiles
    // 2 h and 2 h + 1; the row sum from the same bf16 weights
    auto weights = [&](int h) {
      float e[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[r] = fast_exp2(sacc[2 * h][r] - mref);
        e[4 + r] = fast_exp2(sacc[2 * h + 1][r] - mref);
      }
      pb[h] = u32x4_t{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                      pack_bf16x2(e[6], e[7])};
      ls = sum_bf16x8_f(pb[h], ls);
    };
    // the softmax in four steps, each while a fold waits on LDS
    auto softmax_step = [&](int s) {
      if (s == 0) {
        if (ballot64(lim < 63) == 0) {
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              sacc[m][r] *= sl2;
              mx = fmaxf(mx, sacc[m][r]);
            }
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float x = 16 * m + 4 * g + r <= lim ? sacc[m][r] * sl2 : kNegInf;
              sacc[m][r] = x;
              mx = fmaxf(mx, x);
            }
        }
      } else if (s == 1) {
        mx = pair_max_f(max_xor16(mx));
        // a row with no visible key in this unit (the future half of its
        // own 128-key block) folds nothing
        any = rv && mx != kNegInf;
        mref = mx != kNegInf ? mx : 0.f;
        weights(0);
      } else if (s == 2) {
        weights(1);
      } else {
        ls = pair_sum_f(sum_xor16(ls));
      }
    };
    // the next round's tiles: list words now, rows during the folds; the
    // next own tile's loads and this tile's softmax go between the folds,
    // while the folds wait on LDS
    uint32_t tw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) tw[s] = til[min(t0 + kPvWaves + s, n_tiles - 1)];
    int rrow_n[4];
    const u32x4_t *vp_n[4];
    const Own nx = m1;
    // this round's V^T quarters first (phase 2 takes them), two tiles per
    // fold; the next own tile's Q and K after them
    fold([&](int s) {
      if (s < 2) {
#pragma unroll
        for (int s2 = 2 * s; s2 < 2 * s + 2; ++s2)
#pragma unroll
          for (int mq = 0; mq < MQ; ++mq) {
            vq[s2][mq][0] = vpc[s2][(2 * mq) * 64];
            vq[s2][mq][1] = vpc[s2][(2 * mq + 1) * 64];
          }
      } else {
#pragma unroll
        for (int i = ((s - 2) * NOWN) / 2; i < ((s - 1) * NOWN) / 2; ++i) own_load(nx, i);
      }
      if (s == 1) round_rows(t0 + kPvWaves, tw, rrow_n, vp_n);
      softmax_step(s);
    });
    if (act) {
      *reinterpret_cast<u32x4_t *>(slot + l * 32) = pb[0];
      *reinterpret_cast<u32x4_t *>(slot + l * 32 + 16) = pb[1];
      if (g == 0) {
        reinterpret_cast<float *>(slot + 64 * 32)[c] = any ? mx : kNegInf;
        reinterpret_cast<float *>(slot + 64 * 32)[16 + c] = ls;
      }
    }
    lds_barrier();
    // ================= phase 2: quarter p of the round's tiles; the
    // products wait in registers for the next round's phase 1
    // every LDS read of the phase first: the slots, and the list word of the
    // own tile two rounds ahead
    u32x4_t pbs[4][2];
    float mt[4], lt[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint8_t *sl = px + s * kPivotSlotBytes;
      pbs[s][0] = *reinterpret_cast<const u32x4_t *>(sl + l * 32);
      pbs[s][1] = *reinterpret_cast<const u32x4_t *>(sl + l * 32 + 16);
      mt[s] = reinterpret_cast<const float *>(sl + 64 * 32)[c];
      lt[s] = reinterpret_cast<const float *>(sl + 64 * 32)[16 + c];
    }
    const uint32_t tw2 = til[min(ti + 2 * kPvWaves, n_tiles - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool ok = t0 + s < n_tiles && rrow[s] >= 0 && mt[s] != kNegInf;
      prow[s] = ok ? rrow[s] : kPvRows;
      pmt[s] = ok ? mt[s] : 0.f;
      plt[s] = p == 0 && ok ? lt[s] : 0.f;
    }
    // its rows now, its addresses after the products
    const Tile t2 = tile_of(tw2);
    const int orow2 = bkt[t2.start + min(c, t2.n - 1)], qrow2 = bkt[t2.start + min(l >> 2, t2.n - 1)];
    __builtin_amdgcn_sched_barrier(0);
    // O^T quarter p of each tile (no loads in this phase)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mq = 0; mq < MQ; ++mq) {
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
        o = mfma16(vq[s][mq][0], pbs[s][0], o);
        o = mfma16(vq[s][mq][1], pbs[s][1], o);
        po[s][mq] = o;
      }
    __builtin_amdgcn_sched_barrier(0);
    const Own m2 = own_of(t2, orow2, qrow2);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      rrow[s] = rrow_n[s];
      vpc[s] = vp_n[s];
    }
    m0 = m1;
    m1 = m2;
    lds_barrier();
  };

  const int rounds = (n_tiles + kPvWaves - 1) / kPvWaves;
  if (n_tiles > 0) {
    m0 = own_read(min(p, n_tiles - 1));
    m1 = own_read(min(p + kPvWaves, n_tiles - 1));
    uint32_t tw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) tw[s] = til[min(s, n_tiles - 1)];
    round_rows(0, tw, rrow, vpc);
    // the loads in the order the rounds issue them, so the wait counts at
    // the top of the loop hold for every round
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
      own_load(m0, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (int rd = 0; rd < rounds; ++rd) round(rd);
  fold([](int) {});
  __syncthreads();
  // ---- epilogue: O = N / D in bf16 (16 lanes per row), lse
  for (int i = tid; i < NR * (D / 8); i += kPvThreads) {
    const int row = i / (D / 8), ch8 = i % (D / 8);
    const int t = T0 + row % TT;
    if (t >= dm.L) continue;
    const int h = hk * R + row / TT;
    const float inv = 1.f / lrun[row];
    const f32x4_t x0 = *reinterpret_cast<const f32x4_t *>(acc + acc_at<D>(row, 2 * ch8));
    const f32x4_t x1 = *reinterpret_cast<const f32x4_t *>(acc + acc_at<D>(row, 2 * ch8 + 1));
    const u32x4_t ov = {pack_bf16x2(x0[0] * inv, x0[1] * inv), pack_bf16x2(x0[2] * inv, x0[3] * inv),
                        pack_bf16x2(x1[0] * inv, x1[1] * inv), pack_bf16x2(x1[2] * inv, x1[3] * inv)};
    *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(a.O) + ((size_t)(b * dm.Hq + h) * dm.L + t) * D + 8 * ch8) = ov;
  }
  if (a.lse && row_ok) {
    const int h = hk * R + r_me / TT;
    a.lse[(size_t)(b * dm.Hq + h) * dm.L + t_me] = (mrun[r_me] + log2f(lrun[r_me])) * kLn2;
  }
}

template <int D, int BS>
hipError_t launch(const AttnArgs &a, void *ws, hipStream_t st) {
  const PisaDims &dm = a.dm;
  const PivotLds ly = pivot_lds(dm);
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_pivot_kg<D, BS>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kPivotLdsMax);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  u32x4_t *KVF = static_cast<u32x4_t *>(ws);
  const long long nch = (long long)dm.B * dm.Hkv * dm.n_blk * (BS / 64) * 16 * D;
  kv_prep<D, BS><<<(unsigned)((nch + 255) / 256), 256, 0, st>>>(dm, static_cast<const uint16_t *>(a.K),
                                                                 static_cast<const uint16_t *>(a.V), KVF);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int TT = kPvRows / dm.ratio;
  const unsigned grid = (unsigned)dm.B * dm.Hkv * ((dm.L + TT - 1) / TT);
  attn_pivot_kg<D, BS><<<grid, kPvThreads, ly.total, st>>>(a, KVF, ly);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_pivot(const AttnArgs &a, void *ws, hipStream_t st) {
  if (a.dm.d == 64) return a.dm.bs == 64 ? launch<64, 64>(a, ws, st) : launch<64, 128>(a, ws, st);
  return a.dm.bs == 64 ? launch<128, 64>(a, ws, st) : launch<128, 128>(a, ws, st);
}
