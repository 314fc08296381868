// Stage B: block scores and top-k selection.
//
// PISA page, section 2 (routing by attention score): a selection row r scores
// every candidate key block j by the dot product of its pooled query with the
// pooled key, s_rj = qsel_r . ksel_j, and keeps the top k (ties to the lower
// block index).  PIVOT page, steps 1-4: a proxy (mean of g consecutive
// queries) scores the candidates once and keeps C of them; each member of the
// group re-ranks only that list with its own query.
//
// bf16 (indexer_pivot_mfma): a workgroup takes 32 selection rows of one KV
// head (block rows, or PIVOT proxies followed by their members), scores them
// on MFMA and selects each row on one wave in three tiers (fast fp32 with a
// certified bound, float64 re-score of the straddling candidates, exact);
// see the comment above that kernel.  fp32 (indexer_blockrows,
// indexer_pivot): one wavefront per selection unit, select_row below.
// Selection is bit-exact with respect to the exact real scores; select_row:
//   1. float64 scores (the bf16 / fp32 products are exact in float64) with a
//      rigorous rounding bound  |s - S| <= gamma_D ||p|| ||k||;
//   2. radix select (8-bit digits, LDS histograms) of the n-th largest unique
//      64-bit key  (fp32(score), ~index)  -> provisional set;
//   3. the set is certified when every kept lower bound exceeds every dropped
//      upper bound; otherwise the few undecided candidates are ranked by
//      exact comparisons (float64 bounds, then an exact fixed-point
//      accumulator of the 2*D products when the bounds overlap).
#include "device_common.h"

namespace {

constexpr int kMaxSlots = 16;     // 64 lanes x 16 = 1024 candidates per row
constexpr int kLimbs = 20;        // exact accumulator: 20 x 32-bit digits
constexpr int kExpOffset = 352;   // shifts product exponents (>= -344) to >= 0

PISA_DEV uint32_t ord32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
PISA_DEV float load_elem(const T *p, int c) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(p[c]);
  else return p[c];
}

// (integer significand, exponent) of a finite nonzero float: x = m * 2^e.
PISA_DEV void decompose(float x, uint32_t &m, int &e) {
  int ex;
  const float f = frexpf(fabsf(x), &ex);
  m = (uint32_t)(f * 16777216.0f);  // exact: f has at most 24 significant bits
  e = ex - 24;
}

// Exact sign of  (p . kb + lam mb) - (p . ka + lam ma)  (p, kb, ka are fp32 /
// bf16 values, lam, mb, ma fp32; lam = 0 without routing) using a per-lane
// fixed-point accumulator of kLimbs 32-bit digits held in LDS
// (acc[limb * 64 + lane]).
template <typename T, int D>
PISA_DEV int exact_cmp(const float *p, const T *kb, const T *ka, float lam, float mb, float ma, int64_t *acc) {
  const int l = lane_id();
  bool same = lam == 0.f || mb == ma;
  for (int c = 0; c < D && same; ++c) same = kb[c] == ka[c];
  if (same) return 0;  // identical pooled keys (and routing terms) tie exactly
  for (int i = 0; i < kLimbs; ++i) acc[i * 64 + l] = 0;
  // add (or subtract) the exact product x * y
  auto add_product = [&](float x, float y, bool sub) {
    if (x == 0.f || y == 0.f) return;
    uint32_t mx, my;
    int ex, ey;
    decompose(x, mx, ex);
    decompose(y, my, ey);
    const bool neg = ((x < 0.f) != (y < 0.f)) != sub;
    const uint64_t m = (uint64_t)mx * my;     // < 2^48
    const int b = ex + ey + kExpOffset;       // >= 0
    const int L = b >> 5, sh = b & 31;
    const uint64_t lo = m << sh;
    const uint64_t hi = sh ? (m >> (64 - sh)) : 0;
    const int64_t p0 = (int64_t)(lo & 0xFFFFFFFFull), p1 = (int64_t)(lo >> 32), p2 = (int64_t)hi;
    if (neg) {
      acc[L * 64 + l] -= p0;
      acc[(L + 1) * 64 + l] -= p1;
      acc[(L + 2) * 64 + l] -= p2;
    } else {
      acc[L * 64 + l] += p0;
      acc[(L + 1) * 64 + l] += p1;
      acc[(L + 2) * 64 + l] += p2;
    }
  };
  for (int side = 0; side < 2; ++side) {
    const T *kr = side == 0 ? kb : ka;
    for (int c = 0; c < D; ++c) add_product(p[c], load_elem(kr, c), side == 1);
  }
  if (lam != 0.f) {
    add_product(lam, mb, false);
    add_product(lam, ma, true);
  }
  int64_t carry = 0;
  bool nz = false;
  for (int i = 0; i < kLimbs; ++i) {
    const int64_t v = acc[i * 64 + l] + carry;
    nz |= (v & 0xFFFFFFFFll) != 0;
    carry = v >> 32;
  }
  if (carry < 0) return -1;
  if (carry > 0) return 1;
  return nz ? 1 : 0;
}

struct Shared {
  double p[128];          // selection vector (float64)
  float pf[128];          // same values as float (exact)
  uint32_t hist[256];
  int32_t clist[256];     // PIVOT proxy list (ascending block ids)
  int64_t kul[kLimbs * 64];
};

// float64 score p . k and |k|^2 (fp32) of one candidate row per lane: the
// row's 16-byte chunks loaded eight at a time (one memory latency per group,
// not per chunk), summed in feature order.  A lane with ok false scores 0.
template <typename T, int D>
PISA_DEV void score_slot(const Shared &sh, const T *row, bool ok, double &sc, float &k2) {
  constexpr int EPC = 16 / sizeof(T), CPR = D / EPC, CPG = CPR < 8 ? CPR : 8;
  sc = 0.0;
  k2 = 0.f;
#pragma unroll
  for (int c0 = 0; c0 < CPR; c0 += CPG) {
    __builtin_amdgcn_sched_barrier(0);   // one group of loads in registers at a time
    u32x4_t w[CPG];
#pragma unroll
    for (int c = 0; c < CPG; ++c)
      w[c] = ok ? *reinterpret_cast<const u32x4_t *>(row + (c0 + c) * EPC) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < CPG; ++c)
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        float kv;
        if constexpr (sizeof(T) == 2) kv = (i & 1) ? bf16hi(w[c][i >> 1]) : bf16lo(w[c][i >> 1]);
        else kv = __uint_as_float(w[c][i]);
        sc = fma(sh.p[(c0 + c) * EPC + i], (double)kv, sc);
        k2 = fmaf(kv, kv, k2);
      }
  }
}

// Rank the candidates cand(c) = (list ? list[c] : base + c), c < nc, of one
// row and mark the n_take best in sel[].  NS slots per lane (candidate
// c = s*64+lane).  Routing (mb non-null): a candidate's score gains
// lam * mb[cand].
// ROWWISE: score slot by slot (score_slot: few memory latencies, more
// registers); otherwise chunk by chunk over all slots.  PRE: the scores and
// squared norms were computed by score_slot beforehand and stand in LDS
// (psc, pk2: [NS][64], slot-major).  All three sum every score in feature
// order (identical results).
template <typename T, int D, int NS, bool ROWWISE = true, bool PRE = false>
PISA_DEV void select_row(Shared &sh, const T *kbase, const int32_t *list, int base, int nc, int n_take,
                         const float *mb, float lam, bool (&sel)[NS], int (&cj)[NS], int32_t *diag,
                         const double *psc = nullptr, const float *pk2 = nullptr) {
  const int l = lane_id();
  bool valid[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = s * 64 + l;
    valid[s] = c < nc;
    cj[s] = valid[s] ? (list ? list[c] : base + c) : 0;
    sel[s] = false;
  }
  if (n_take <= 0) return;
  if (n_take >= nc) {
#pragma unroll
    for (int s = 0; s < NS; ++s) sel[s] = valid[s];
    return;
  }
  // ---- 1. float64 scores and bounds
  double sc[NS];
  float k2[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    sc[s] = 0.0;
    k2[s] = 0.f;
  }
  if constexpr (PRE) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s * 64 >= nc) break;
      sc[s] = psc[s * 64 + l];
      k2[s] = pk2[s * 64 + l];
    }
  } else if constexpr (ROWWISE) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s * 64 >= nc) break;
      score_slot<T, D>(sh, kbase + (size_t)cj[s] * D, valid[s], sc[s], k2[s]);
    }
  } else {
    // chunk by chunk over every slot (fewer registers; one memory latency
    // per chunk)
    constexpr int EPC = 16 / sizeof(T);
    for (int c0 = 0; c0 < D; c0 += EPC) {
      double pc[EPC];
#pragma unroll
      for (int i = 0; i < EPC; ++i) pc[i] = sh.p[c0 + i];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (!valid[s]) continue;
        const u32x4_t w = *reinterpret_cast<const u32x4_t *>(kbase + (size_t)cj[s] * D + c0);
#pragma unroll
        for (int i = 0; i < EPC; ++i) {
          float kv;
          if constexpr (sizeof(T) == 2) kv = (i & 1) ? bf16hi(w[i >> 1]) : bf16lo(w[i >> 1]);
          else kv = __uint_as_float(w[i]);
          sc[s] = fma(pc[i], (double)kv, sc[s]);
          k2[s] = fmaf(kv, kv, k2[s]);
        }
      }
    }
  }
  double p2 = 0.0;
  for (int c = 0; c < D; ++c) p2 = fma(sh.p[c], sh.p[c], p2);
  constexpr double u = 0x1p-53;
  const double gamma = (D * u) / (1.0 - D * u) * (1.0 + 0x1p-10);
  double dl[NS];
  uint64_t key[NS];
  uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    dl[s] = gamma * sqrt(p2 * (double)k2[s]) + 0x1p-1000;
    if (mb && valid[s]) {   // routing term: the product is exact, the sum rounds once
      sc[s] += (double)lam * (double)mb[cj[s]];
      dl[s] += 0x1p-52 * fabs(sc[s]);
    }
    key[s] = valid[s] ? (((uint64_t)ord32((float)sc[s]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)cj[s])) : 0ull;
    if (valid[s]) {
      kmax = key[s] > kmax ? key[s] : kmax;
      kmin = key[s] < kmin ? key[s] : kmin;
    }
  }
  // ---- 2. radix select of the n_take-th largest (unique) key
  kmax = wave_max_u64(kmax);
  kmin = wave_min_u64(kmin);
  const uint64_t diff = kmax ^ kmin;
  int shift = diff ? ((63 - __clzll(diff)) & ~7) : 0;
  uint64_t prefix = (shift + 8 >= 64) ? 0ull : (kmax >> (shift + 8)) << (shift + 8);
  int need = n_take;
  uint64_t tau = 0;
  for (;;) {
    for (int b = l; b < 256; b += 64) sh.hist[b] = 0;
    wave_lds_sync();
    const uint64_t hi_mask = (shift + 8 >= 64) ? 0ull : ~((1ull << (shift + 8)) - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (valid[s] && (key[s] & hi_mask) == prefix) atomicAdd(&sh.hist[(key[s] >> shift) & 255u], 1u);
    wave_lds_sync();
    int h[4];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = (int)sh.hist[255 - 4 * l - q];
      cnt += h[q];
    }
    const int incl = wave_incl_scan(cnt);
    const int excl = incl - cnt;
    const bool mine = excl < need && need <= incl;
    const uint64_t bal = ballot64(mine);
    if (!bal) {  // unreachable for consistent counts; keeps the loop finite
      tau = prefix;
      break;
    }
    const int owner = __ffsll((unsigned long long)bal) - 1;
    int bin = 0, above = 0, hb = 0;
    if (mine) {
      int run = excl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run + h[q] >= need) {
          bin = 255 - 4 * l - q;
          above = run;
          hb = h[q];
          break;
        }
        run += h[q];
      }
    }
    bin = __shfl(bin, owner);
    above = __shfl(above, owner);
    hb = __shfl(hb, owner);
    wave_lds_sync();
    need -= above;
    prefix |= (uint64_t)bin << shift;
    if (hb == need || shift == 0) {
      tau = prefix;
      break;
    }
    shift -= 8;
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) sel[s] = valid[s] && key[s] >= tau;
  // ---- 3. certify with the float64 bounds
  double t_in = __builtin_huge_val(), t_out = -__builtin_huge_val();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (!valid[s]) continue;
    if (sel[s]) t_in = fmin(t_in, sc[s] - dl[s]);
    else t_out = fmax(t_out, sc[s] + dl[s]);
  }
  t_in = wave_min_f64(t_in);
  t_out = wave_max_f64(t_out);
  if (diag && l == 0) atomicAdd(&diag[0], 1);
  if (t_in > t_out) return;

  // ---- cold path: rank the undecided candidates exactly.  Every lane ranks
  // its own undecided candidates against all undecided ones, visiting them
  // through wave shuffles (no per-candidate LDS storage).
  bool amb[NS];
  int n_sure = 0, n_amb = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    amb[s] = valid[s] && (sel[s] ? (sc[s] - dl[s] <= t_out) : (sc[s] + dl[s] >= t_in));
    n_sure += __popcll(ballot64(sel[s] && !amb[s]));
    n_amb += __popcll(ballot64(amb[s]));
  }
  const int want = n_take - n_sure;
  int rank[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) rank[s] = 0;
#pragma unroll
  for (int sb = 0; sb < NS; ++sb) {
    uint64_t m = ballot64(amb[sb]);
    while (m) {
      const int lb = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int jb = __shfl(cj[sb], lb);
      const double sbv = __shfl(sc[sb], lb), dbv = __shfl(dl[sb], lb);
#pragma unroll
      for (int sa = 0; sa < NS; ++sa) {
        if (!amb[sa] || (sa == sb && lb == l)) continue;
        bool beats;
        if (sbv - dbv > sc[sa] + dl[sa]) beats = true;
        else if (sbv + dbv < sc[sa] - dl[sa]) beats = false;
        else {
          const int c = exact_cmp<T, D>(sh.pf, kbase + (size_t)jb * D, kbase + (size_t)cj[sa] * D, mb ? lam : 0.f,
                                        mb ? mb[jb] : 0.f, mb ? mb[cj[sa]] : 0.f, sh.kul);
          beats = c > 0 || (c == 0 && jb < cj[sa]);
        }
        rank[sa] += beats;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (amb[s]) sel[s] = rank[s] < want;
  if (diag && l == 0) {
    atomicAdd(&diag[1], 1);
    atomicAdd(&diag[2], n_amb);
  }
}

// Write the kept ids ascending (slot-major candidate order is ascending),
// padded with -1 up to len entries.
template <int NS>
PISA_DEV int write_sorted(const bool (&sel)[NS], const int (&cj)[NS], int32_t *out, int len) {
  const int l = lane_id();
  int base = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint64_t m = ballot64(sel[s]);
    if (sel[s]) out[base + __popcll(m & ((1ull << l) - 1))] = cj[s];
    base += __popcll(m);
  }
  for (int pos = base + l; pos < len; pos += 64) out[pos] = -1;
  return base;
}

template <typename T, int D>
PISA_DEV void load_p(Shared &sh, const T *src) {
  const int l = lane_id();
  for (int c = l; c < D; c += 64) {
    const float v = load_elem(src, c);
    sh.pf[c] = v;
    sh.p[c] = (double)v;
  }
  __syncthreads();
}

template <typename T, int D>
__global__ __launch_bounds__(64) void indexer_blockrows(PisaDims dm, const T *__restrict__ qsel,
                                                        const T *__restrict__ ksel, const float *__restrict__ mcov,
                                                        int32_t *__restrict__ idx, int32_t *diag) {
  __shared__ Shared sh;
  const int unit = blockIdx.x;
  // causal rows have more candidates the later their block: the longest first
  const int i = dm.causal ? dm.n_blk - 1 - unit % dm.n_blk : unit % dm.n_blk;
  const int bh = unit / dm.n_blk;  // b * Hq + h
  const int b = bh / dm.Hq, h = bh % dm.Hq;
  const int hk = h * dm.Hkv / dm.Hq;
  const T *kbase = ksel + ((size_t)b * dm.Hkv + hk) * dm.n_blk * D;
  int own, lo;
  const int nc = pisa_row_geometry(dm, i * dm.bs, &own, &lo);
  const int c0 = min(dm.sink, nc);            // sink blocks, kept and listed first
  const int n_take = min(dm.topk, nc - c0);
  load_p<T, D>(sh, qsel + ((size_t)bh * dm.n_sel + i) * D);
  bool sel[kMaxSlots];
  int cj[kMaxSlots];
  const float *mb = mcov ? mcov + ((size_t)b * dm.Hkv + hk) * dm.n_blk : nullptr;
  select_row<T, D, kMaxSlots>(sh, kbase, nullptr, c0, nc - c0, n_take, mb, dm.route_lambda, sel, cj, diag);
  int32_t *out = idx + ((size_t)bh * dm.n_rows + i) * dm.klist;
  for (int c = lane_id(); c < c0; c += 64) out[c] = c;
  write_sorted<kMaxSlots>(sel, cj, out + c0, dm.klist - c0);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void indexer_pivot(PisaDims dm, const T *__restrict__ Q,
                                                    const T *__restrict__ qsel, const T *__restrict__ ksel,
                                                    const float *__restrict__ mcov, int32_t *__restrict__ idx,
                                                    int32_t *__restrict__ cand, int32_t *diag) {
  __shared__ Shared sh;
  const int unit = blockIdx.x;
  // causal rows have more candidates the later their group: the longest first
  const int gm = dm.causal ? dm.n_sel - 1 - unit % dm.n_sel : unit % dm.n_sel;
  const int bh = unit / dm.n_sel;
  const int b = bh / dm.Hq, h = bh % dm.Hq;
  const int hk = h * dm.Hkv / dm.Hq;
  const T *kbase = ksel + ((size_t)b * dm.Hkv + hk) * dm.n_blk * D;
  const int g = dm.group;
  int own, lo;
  const int nc = pisa_row_geometry(dm, gm * g, &own, &lo);
  const int c0 = min(dm.sink, nc);
  const int C = min(dm.n_cand, nc - c0);
  const float *mb = mcov ? mcov + ((size_t)b * dm.Hkv + hk) * dm.n_blk : nullptr;
  // proxy pass over every candidate block past the sinks
  load_p<T, D>(sh, qsel + ((size_t)bh * dm.n_sel + gm) * D);
  {
    bool sel[kMaxSlots];
    int cj[kMaxSlots];
    select_row<T, D, kMaxSlots, false>(sh, kbase, nullptr, c0, nc - c0, C, mb, dm.route_lambda, sel, cj, diag);
    write_sorted<kMaxSlots>(sel, cj, sh.clist, C);
    if (cand) {
      __syncthreads();
      int32_t *cout = cand + ((size_t)bh * dm.n_sel + gm) * dm.n_cand;
      for (int c = lane_id(); c < dm.n_cand; c += 64) cout[c] = c < C ? sh.clist[c] : -1;
    }
  }
  __syncthreads();
  if (dm.klist == 0) return;
  // member pass over the proxy's list, after each member's own sinks
  const int n_take = min(dm.topk, C);
  const int t1 = min(dm.L, (gm + 1) * g);
  for (int t = gm * g; t < t1; ++t) {
    load_p<T, D>(sh, Q + ((size_t)bh * dm.L + t) * D);
    bool sel[4];
    int cj[4];
    select_row<T, D, 4, false>(sh, kbase, sh.clist, 0, C, n_take, mb, dm.route_lambda, sel, cj, diag);
    const int ct = min(dm.sink, pisa_row_geometry(dm, t, &own, &lo));
    int32_t *out = idx + ((size_t)bh * dm.n_rows + t) * dm.klist;
    for (int c = lane_id(); c < ct; c += 64) out[c] = c;
    write_sorted<4>(sel, cj, out + ct, dm.klist - ct);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// PIVOT rows on the matrix cores (bf16, d 64 or 128).
//
// A workgroup of kPW waves takes up to 32 proxies that share a KV head and a
// query block (the query heads of the KV head times the groups of the
// block), so they share the candidate blocks up to their causal limit:
//   1. proxy scores S[p][j] = qsel_p . ksel_j for all candidates at once on
//      MFMA 32x32x16 (ksel rows as A straight from memory, the 32 proxies
//      as B), with |ksel_j| from the same loads;
//   2. each proxy's top-C from its row of S;
//   3. each member's top-k of its proxy's list: MFMA of the gathered list
//      rows against up to 8 member queries, then the same selection.
// Selection of one row by one wave, in three tiers:
//   fast    keys ord(fp32 score); the n-th largest key found by bisection
//           over the key bits with ballot counts (bisect32);
//           the set is accepted when it is certified: every kept
//           lower bound s - e exceeds every dropped upper bound s + e, with
//           e = (d / 4 + 3) 2^-22 |p| |k| + 2^-110 (see pivot_bound below);
//   re-score  (rare, a function of its own) candidates whose intervals
//           straddle the threshold get float64 scores with a float64 bound,
//           the row is selected again on float64 keys and certified;
//   exact   rows still undecided (exact ties of different vectors) are left to
//           wave 0, which re-runs them with select_row's exact path once the
//           other waves are done.

constexpr int kPX = 32;        // proxies per workgroup
constexpr int kPCap = 128;     // proxy list capacity of this path
constexpr int kPNc = 1024;     // candidate capacity
constexpr int kPW = 16;        // waves
constexpr int kPG = 16;        // group size capacity (members per proxy)
constexpr int kPM = 8;         // members scored per MFMA pass

// Rounding bound of an fp32 score computed by MFMA from bf16 operands.  The
// products are exact in fp32.  A score is taken as NP = 4 partial sums, each
// an MFMA 32x32x16 chain over KS / 4 K-steps of 16 products (n = d / 4
// products), added in fp32 one after the other (mfma32_split).  A
// sum of n exact products in fp32 (any order, round to nearest or toward
// zero) is off by at most 2 n 2^-24 sum|p_i k_i|, so each partial errs by at
// most n 2^-23 of its own sum|p_i k_i|, and each of the NP - 1 additions by
// at most 2^-23 of the sum of all |p_i k_i|: in all (n + NP - 1) 2^-23
// sum|p_i k_i| <= (n + NP - 1) 2^-23 |p| |k|.  The factor used,
// (n + NP - 1) 2^-22, is twice that, which also covers the rounding of the
// norms (fp32 sums of squares, square roots), of the bound's own products
// and of the subtraction s - e / addition s + e in the certification (each
// a few units of 2^-24 |p| |k|).  The norms are taken of |x|^2 + 2^-118, so
// squares that underflow cannot make them too small, and the absolute term
// 2^-110 covers products and partial sums flushed to zero (at most
// 2 d 2^-126).  One chain over all d products would need d 2^-22: at d = 128,
// 35 against 128 units, and that many times more rows left to the float64
// tier.  Eight one-step partials (23 units) ran out of registers.
constexpr float kAbsBound = 0x1p-110f;
constexpr float kSqFloor = 0x1p-118f;
constexpr int kNP = 4;   // partial sums of a score
template <int KS>
constexpr float pivot_bound() { return (float)(16 * KS / kNP + kNP - 1) * 0x1p-22f; }

// A . B over KS K-steps as kNP partial sums (MFMA chains of KS / kNP K-steps
// of 16 products each), added in fp32 in K-step order
template <int KS>
PISA_DEV f32x16_t mfma32_split(const u32x4_t (&a)[KS], const u32x4_t (&b)[KS]) {
  static_assert(KS % kNP == 0, "whole K-steps per partial sum");
  constexpr int PK = KS / kNP;
  f32x16_t part[kNP];
#pragma unroll
  for (int q = 0; q < kNP; ++q) {
    part[q] = f32x16_t{};
#pragma unroll
    for (int k = 0; k < PK; ++k) part[q] = mfma32(a[q * PK + k], b[q * PK + k], part[q]);
  }
  f32x16_t acc = part[0];
#pragma unroll
  for (int q = 1; q < kNP; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += part[q][r];
  return acc;
}

struct PivotLayout {
  static constexpr int SLD = kPNc + 4;                 // floats per proxy row of S (padded)
  static constexpr int MLD = kPCap + 4;                // floats per member row of the member scores
  static constexpr int S = 0;                          // fp32 [kPX][SLD]; then member scores
                                                       // [kPW][kPM][MLD]; then select_row's Shared
  static constexpr int SKN = S + kPX * SLD * 4;        // fp32 [kPNc] |ksel_j|
  static constexpr int SPN = SKN + kPNc * 4;           // fp32 [kPX] |qsel_p|
  static constexpr int MC = SPN + kPX * 4;             // fp32 [kPNc] covariance norms (routing)
  static constexpr int PV = MC + kPNc * 4;             // fp32 [kPW][128] row vector under re-score
  static constexpr int LIST = PV + kPW * 128 * 4;      // uint16 [kPX][kPCap] proxy lists, ascending
  static constexpr int DEFN = LIST + kPX * kPCap * 2;  // int [4]: deferred proxies, deferred members,
                                                       // next proxy of passes 2 and 3
  static constexpr int DEFP = DEFN + 16;               // int [kPX]
  static constexpr int DEFM = DEFP + kPX * 4;          // int [kPX * kPG] (token * 64 + proxy)
  static constexpr int TOTAL = DEFM + kPX * kPG * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  static_assert(kPW * kPM * MLD * 4 <= kPX * SLD * 4, "member scores fit in S");
  static_assert((int)sizeof(Shared) <= kPX * SLD * 4, "select_row's Shared fits in S");
};

// wave max / min of unsigned 32-bit values on the cross-lane data path
// (DPP row operations and the permlane swaps); every lane gets the result
template <bool MAX>
PISA_DEV uint32_t wave_ureduce_xl(uint32_t v) {
  auto op = [](uint32_t x, uint32_t y) { return MAX ? (x > y ? x : y) : (x < y ? x : y); };
  auto dpp = [](uint32_t x, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, decltype(ctrl)::value, 0xF, 0xF, false);
  };
  v = op(v, dpp(v, std::integral_constant<int, 0xB1>{}));    // quad_perm [1,0,3,2]
  v = op(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
  v = op(v, dpp(v, std::integral_constant<int, 0x141>{}));   // row_half_mirror
  v = op(v, dpp(v, std::integral_constant<int, 0x140>{}));   // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);
}

// Largest threshold t with at least `need` keys >= t, by bisection over the
// 32 key bits: each step counts the keys at or above a trial threshold with
// one ballot per slot (no LDS, no cross-lane scan), and stops as soon as the
// count is exactly `need`.  Keys of 0 (invalid slots) are no candidates;
// slots s >= nsl (uniform) hold none.  Returns true with t such that exactly
// `need` keys are >= t (the top set is unique at 32 bits), false when keys tie
// across the boundary at 32 bits or fewer than `need` candidates exist.
template <int NS>
PISA_DEV bool bisect32(const uint32_t (&key)[NS], int nsl, int need, uint32_t &t) {
  t = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < nsl) cnt += __builtin_popcountll(ballot64(key[s] >= c));
    if (cnt >= need) {
      t = c;
      if (cnt == need) return true;
    }
  }
  // t is the largest threshold with at least need keys >= t: more than need
  // (keys equal to t straddle the boundary), or t = 0 with too few keys
  return false;
}

// Fast tier: select the `need` best of fp32 scores sc (bounds dl) and certify.
template <int NS>
PISA_DEV bool fast_select(const float (&sc)[NS], const float (&dl)[NS], const bool (&valid)[NS], int nsl,
                          int need, bool (&sel)[NS]) {
  uint32_t key[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) key[s] = valid[s] ? ord32(sc[s]) : 0u;
  uint32_t t;
  if (!bisect32<NS>(key, nsl, need, t)) return false;
  float t_out = -__builtin_huge_valf();
  bool bad = false;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s >= nsl) {
      sel[s] = false;
      continue;
    }
    sel[s] = key[s] >= t;
    const float hi = sc[s] + dl[s], lo = sc[s] - dl[s];
    if (valid[s]) {
      if (!sel[s]) t_out = fmaxf(t_out, hi);
      bad |= !(__builtin_isfinite(hi) && __builtin_isfinite(lo));
    }
  }
  t_out = wave_max_xl(t_out);
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nsl) bad |= sel[s] && !(sc[s] - dl[s] > t_out);
  return ballot64(bad) == 0;
}

PISA_DEV uint64_t ord64(double d) {
  const uint64_t u = __builtin_bit_cast(uint64_t, d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Provisional top `need` of float64 scores: bisection over the 64 key bits,
// keys equal at the threshold taken in slot order (= ascending block id).
template <int NS>
PISA_DEV void provisional64(const double (&sc)[NS], const bool (&valid)[NS], int need, bool (&sel)[NS]) {
  const int l = lane_id();
  uint64_t t = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t c = t | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) cnt += __builtin_popcountll(ballot64(valid[s] && ord64(sc[s]) >= c));
    if (cnt >= need) {
      t = c;
      if (cnt == need) break;
    }
  }
  int above = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) above += __builtin_popcountll(ballot64(valid[s] && ord64(sc[s]) > t));
  const int rem = need - above;
  const uint64_t lt = (1ull << l) - 1;
  int base = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint64_t k = valid[s] ? ord64(sc[s]) : 0ull;
    const uint64_t tie = ballot64(valid[s] && k == t);
    sel[s] = valid[s] && (k > t || (k == t && base + __builtin_popcountll(tie & lt) < rem));
    base += __builtin_popcountll(tie);
  }
}

// Provisional top `need` of the same scores on 32-bit keys (the float
// rounding of the float64 score): bisection over the key bits, keys equal at
// the threshold taken in slot order.  Any set of `need` works as a provisional
// set: the float64 bounds decide which candidates stay undecided.
template <int NS>
PISA_DEV void provisional32(const double (&sc)[NS], const bool (&valid)[NS], int need, bool (&sel)[NS]) {
  const int l = lane_id();
  uint32_t key[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) key[s] = valid[s] ? ord32((float)sc[s]) : 0u;
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) cnt += __builtin_popcountll(ballot64(valid[s] && key[s] >= c));
    if (cnt >= need) {
      t = c;
      if (cnt == need) break;
    }
  }
  int above = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) above += __builtin_popcountll(ballot64(valid[s] && key[s] > t));
  const int rem = need - above;
  const uint64_t lt = (1ull << l) - 1;
  int base = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint64_t tie = ballot64(valid[s] && key[s] == t);
    sel[s] = valid[s] && (key[s] > t || (key[s] == t && base + __builtin_popcountll(tie & lt) < rem));
    base += __builtin_popcountll(tie);
  }
}

// Lowest kept lower bound and highest dropped upper bound (float64); false
// if any bound is not finite.
template <int NS>
PISA_DEV bool bounds64(const double (&sc)[NS], const double (&dl)[NS], const bool (&valid)[NS],
                       const bool (&sel)[NS], double &t_in, double &t_out) {
  double a = __builtin_huge_val(), b = -__builtin_huge_val();
  bool bad = false;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (!valid[s]) continue;
    const double lo = sc[s] - dl[s], hi = sc[s] + dl[s];
    bad |= !(__builtin_isfinite(lo) && __builtin_isfinite(hi));
    if (sel[s]) a = fmin(a, lo);
    else b = fmax(b, hi);
  }
  t_in = wave_min_f64(a);
  t_out = wave_max_f64(b);
  return ballot64(bad) == 0;
}

// float64 score p . k of one candidate row by one lane (features in order,
// p from LDS, the row's 16-byte chunks loaded together) and a bound on its
// rounding: the products are exact in float64, so the error is that of D - 1
// sequential additions, at most (D - 1) 2^-53 sum |x| (first order; D + 2
// covers the rest and the rounding of the sum of |x| itself).
template <int D>
PISA_DEV double rescore64_lane(const float *p, const uint16_t *kr, double *bound) {
  u32x4_t kk[D / 8];
#pragma unroll
  for (int c = 0; c < D / 8; ++c) kk[c] = *reinterpret_cast<const u32x4_t *>(kr + 8 * c);
  double s = 0.0, a = 0.0;
#pragma unroll
  for (int c = 0; c < D / 8; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double x0 = (double)p[8 * c + 2 * i] * (double)bf16lo(kk[c][i]);
      const double x1 = (double)p[8 * c + 2 * i + 1] * (double)bf16hi(kk[c][i]);
      s += x0;
      a += fabs(x0);
      s += x1;
      a += fabs(x1);
    }
  *bound = (double)(D + 2) * 0x1p-53 * a + 0x1p-1000;
  return s;
}

PISA_DEV double readlane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// ids of the selected slots, ascending, to LDS (uint16) and optionally to
// global memory (int32, -1 padded to len)
template <int NS>
PISA_DEV void write_sorted_lds(const bool (&sel)[NS], const int (&cj)[NS], uint16_t *lout, int32_t *gout,
                               int len) {
  const int l = lane_id();
  int base = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint64_t m = ballot64(sel[s]);
    if (sel[s]) {
      const int pos = base + __popcll(m & ((1ull << l) - 1));
      if (lout) lout[pos] = (uint16_t)cj[s];
      if (gout) gout[pos] = cj[s];
    }
    base += __popcll(m);
  }
  if (gout)
    for (int pos = base + l; pos < len; pos += 64) gout[pos] = -1;
}

template <int D>
PISA_DEV void load_vec_f32(float *dst, const uint16_t *src) {
  for (int c = lane_id(); c < D; c += 64) dst[c] = bf16_to_f32(src[c]);
  wave_lds_sync();
}

// Re-score tier for one row whose fast selection was not certified.  srow:
// fp32 scores by list position; list: block ids by position (nullptr: the
// position is the id); positions lo .. nc-1 are candidates; bounds
// cb |k_j| + 2^-110 as in the fast tier; vec: the row's own vector (bf16,
// global), staged to pv.  On success writes the row like write_sorted_lds
// and returns true.
template <int D, int NS>
__device__ __attribute__((noinline)) bool rescore_select(const float *srow, const uint16_t *list, int lo,
                                                         int nc, int n_take, float cb, const float *skn,
                                                         const float *mc, float lam,
                                                         const uint16_t *vec, float *pv, const uint16_t *kbase,
                                                         uint16_t *lout, int32_t *gout, int len, int32_t *diag) {
  const int l = lane_id();
  if (diag && l == 0) atomicAdd(&diag[1], 1);
  double sc[NS], dl[NS];
  int cj[NS];
  bool valid[NS], sel[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int pos = s * 64 + l;
    valid[s] = pos >= lo && pos < nc;
    cj[s] = valid[s] ? (list ? (int)list[pos] : pos) : 0;
    sc[s] = valid[s] ? (double)srow[pos] : 0.0;
    dl[s] = valid[s] ? (double)fmaf(cb, skn[cj[s]], kAbsBound) : 0.0;
  }
  // routing term lam * mc[j]: the product is exact in float64, the sum rounds once
  auto add_route = [&](int s) {
    if (mc && valid[s]) {
      sc[s] += (double)lam * (double)mc[cj[s]];
      dl[s] += 0x1p-52 * fabs(sc[s]);
    }
  };
#pragma unroll
  for (int s = 0; s < NS; ++s) add_route(s);
  load_vec_f32<D>(pv, vec);
  provisional32<NS>(sc, valid, n_take, sel);
  double t_in, t_out;
  bounds64<NS>(sc, dl, valid, sel, t_in, t_out);
  // undecided: kept ones not above every dropped bound and vice versa (a
  // non-finite bound counts as undecided).  A kept candidate that is not
  // undecided is above every dropped one, so it is in the top set; a dropped
  // one that is not undecided is below every kept one, so it is out.  Only
  // the undecided are ranked again, among themselves, on float64 scores
  // computed side by side: undecided candidate k (in slot, lane order) on
  // lane k % 64.
  bool amb[NS];
  uint64_t ambm[NS];
  int namb = 0, n_in = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const double lo = sc[s] - dl[s], hi = sc[s] + dl[s];
    amb[s] = valid[s] && (sel[s] ? !(lo > t_out) : !(hi < t_in));
    ambm[s] = ballot64(amb[s]);
    namb += __popcll(ambm[s]);
    n_in += __popcll(ballot64(valid[s] && sel[s] && !amb[s]));
  }
  auto score_undecided = [&](int k0, double &v, double &bnd) -> int {
    int myj = -1, k = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      for (uint64_t m = ambm[s]; m; m &= m - 1, ++k) {
        const int lb = __ffsll((unsigned long long)m) - 1;
        if (k >= k0 && k < k0 + 64) {
          const int j = __builtin_amdgcn_readlane(cj[s], lb);
          if (l == k - k0) myj = j;
        }
      }
    v = 0.0;
    bnd = 0.0;
    if (myj >= 0) {
      v = rescore64_lane<D>(pv, kbase + (size_t)myj * D, &bnd);
      if (mc) {   // as add_route
        v += (double)lam * (double)mc[myj];
        bnd += 0x1p-52 * fabs(v);
      }
    }
    return myj;
  };
  if (namb <= 64) {
    double v, bnd;
    const bool act = score_undecided(0, v, bnd) >= 0;
    // the need2 best of the undecided by float64 score, certified among them
    const int need2 = n_take - n_in;
    const uint64_t key = act ? ord64(v) : 0ull;
    uint64_t t = 0;
    bool found = need2 <= 0;
    if (!found)
      for (int bit = 63; bit >= 0; --bit) {
        const uint64_t c = t | (1ull << bit);
        const int cnt = __popcll(ballot64(act && key >= c));
        if (cnt >= need2) {
          t = c;
          if (cnt == need2) {
            found = true;
            break;
          }
        }
      }
    if (!found) return false;   // equal float64 scores across the boundary
    const bool ch = act && need2 > 0 && key >= t;
    const double lo = v - bnd, hi = v + bnd;
    const bool bad = act && !(__builtin_isfinite(lo) && __builtin_isfinite(hi));
    const double lo_in = wave_min_f64(ch ? lo : __builtin_huge_val());
    const double hi_out = wave_max_f64(act && !ch ? hi : -__builtin_huge_val());
    if (ballot64(bad) != 0 || !(lo_in > hi_out)) return false;
    int k = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      for (uint64_t m = ambm[s]; m; m &= m - 1, ++k) {
        const int lb = __ffsll((unsigned long long)m) - 1;
        const int c = __builtin_amdgcn_readlane(ch ? 1 : 0, k);
        if (l == lb) sel[s] = c != 0;
      }
    write_sorted_lds<NS>(sel, cj, lout, gout, len);
    return true;
  }
  // many undecided: rescore them all, select the row again on float64 keys
  for (int k0 = 0; k0 < namb; k0 += 64) {
    double v, bnd;
    score_undecided(k0, v, bnd);
    int k = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      for (uint64_t m = ambm[s]; m; m &= m - 1, ++k) {
        const int lb = __ffsll((unsigned long long)m) - 1;
        if (k >= k0 && k < k0 + 64) {
          const double vv = readlane_f64(v, k - k0), bb = readlane_f64(bnd, k - k0);
          if (l == lb) {
            sc[s] = vv;
            dl[s] = bb;
          }
        }
      }
  }
  provisional64<NS>(sc, valid, n_take, sel);
  if (!bounds64<NS>(sc, dl, valid, sel, t_in, t_out) || !(t_in > t_out)) return false;
  write_sorted_lds<NS>(sel, cj, lout, gout, len);
  return true;
}

// Exact tier for one row: select_row over the candidates (list: nc block
// ids in LDS, or nullptr for base .. base+nc-1), written like
// write_sorted_lds.
template <int D, int NS>
__device__ __attribute__((noinline)) void exact_select(Shared &sh, const uint16_t *kbase, const uint16_t *list,
                                                       int base, int nc, int n_take, const float *mb, float lam,
                                                       const uint16_t *vec, uint16_t *lout, int32_t *gout, int len,
                                                       int32_t *diag) {
  const int l = lane_id();
  if (list)
    for (int c = l; c < nc; c += 64) sh.clist[c] = list[c];
  for (int c = l; c < D; c += 64) {
    const float v = bf16_to_f32(vec[c]);
    sh.pf[c] = v;
    sh.p[c] = (double)v;
  }
  wave_lds_sync();
  bool sel[NS];
  int cj[NS];
  select_row<uint16_t, D, NS, false>(sh, kbase, list ? sh.clist : nullptr, base, nc, n_take, mb, lam, sel, cj, diag);
  write_sorted_lds<NS>(sel, cj, lout, gout, len);
  if (diag && l == 0) atomicAdd(&diag[2], 1);
  wave_lds_sync();
}

// ROWS: the same kernel for block rows (no groups): a workgroup takes 32
// block rows of one KV head, in (query block, head) order, and writes each
// row's kept list (sinks, then the top-k ascending) instead of a proxy list;
// there is no member pass.  NSX: 64-candidate slots per lane (n_blk <= 64 NSX),
// which sizes the selection's per-lane arrays.
template <int D, bool ROWS, int NSX>
__global__ __launch_bounds__(kPW * 64, 1) void indexer_pivot_mfma(PisaDims dm, const uint16_t *__restrict__ Q,
                                                                 const uint16_t *__restrict__ qsel,
                                                                 const uint16_t *__restrict__ ksel,
                                                                 const float *__restrict__ mcov,
                                                                 int32_t *__restrict__ idx,
                                                                 int32_t *__restrict__ cand, int32_t *diag,
                                                                 int blo, int nbr) {
  using LY = PivotLayout;
  constexpr int KS = D / 16;
  constexpr float kG = pivot_bound<KS>();
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, l = tid & 63, lq = l & 31, hl = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = ROWS ? dm.bs : dm.group;
  const int gpb = dm.bs / g;                  // groups per block
  // proxies per (KV head, block); block rows: rows per KV head
  const int npb = ROWS ? dm.ratio * dm.n_blk : dm.ratio * gpb;
  const int nchunk = (npb + kPX - 1) / kPX;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  // causal rows have more candidates the later their block: the longest first
  const int cq = (ROWS && dm.causal) ? nchunk - 1 - logical % nchunk : logical % nchunk;
  const int rest = logical / nchunk;
  // PIVOT: query blocks [blo, blo + nbr) of the launch
  const int iblk = ROWS ? 0 : blo + (dm.causal ? nbr - 1 - rest % nbr : rest % nbr);
  const int bk = ROWS ? rest : rest / nbr;
  const int b = bk / dm.Hkv, hk = bk % dm.Hkv;
  const uint16_t *kbase = ksel + ((size_t)b * dm.Hkv + hk) * dm.n_blk * D;
  float *S = reinterpret_cast<float *>(lds + LY::S);
  float *SKN = reinterpret_cast<float *>(lds + LY::SKN);
  float *SPN = reinterpret_cast<float *>(lds + LY::SPN);
  float *MC = reinterpret_cast<float *>(lds + LY::MC);
  const bool route = mcov != nullptr;
  const float lam = dm.route_lambda;
  float *PVw = reinterpret_cast<float *>(lds + LY::PV) + w * 128;
  uint16_t *LIST = reinterpret_cast<uint16_t *>(lds + LY::LIST);
  int *defn = reinterpret_cast<int *>(lds + LY::DEFN);
  int *defp = reinterpret_cast<int *>(lds + LY::DEFP);
  int *defm = reinterpret_cast<int *>(lds + LY::DEFM);
  Shared &sh = *reinterpret_cast<Shared *>(lds + LY::S);

  // proxy pp of this workgroup -> (query head, group), candidate count
  auto proxy = [&](int pl, int &h, int &gm, int &nc) -> bool {
    const int pp = cq * kPX + pl;
    if constexpr (ROWS) {   // row pp: query block pp / ratio of head pp % ratio
      const int ppc = pp < npb ? pp : npb - 1;
      h = hk * dm.ratio + ppc % dm.ratio;
      gm = ppc / dm.ratio;
    } else {
      h = hk * dm.ratio + pp / gpb;
      gm = iblk * gpb + pp % gpb;
    }
    int own, lo;
    nc = pisa_row_geometry(dm, gm * g, &own, &lo);
    return pp < npb && gm * g < dm.L;
  };
  int ph, pgm, pnc;
  const bool pval = proxy(lq, ph, pgm, pnc);
  const int ncmax = __builtin_amdgcn_readfirstlane(wave_max_f32(pval ? (float)pnc : 0.f));
  if (tid < 4) defn[tid] = 0;
  // passes 2 and 3 hand proxies to the waves one at a time from a counter, so
  // a wave held up by a re-score does not hold up the workgroup's last proxy
  auto next_proxy = [&](int *ctr) -> int {
    int v = 0;
    if (l == 0) v = atomicAdd(ctr, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  if (route)   // this kv head's covariance norms (routing term lam * MC[j])
    for (int j = tid; j < dm.n_blk; j += kPW * 64) MC[j] = mcov[((size_t)b * dm.Hkv + hk) * dm.n_blk + j];

  // ---- 1. proxy scores, |k| and |p|
  u32x4_t pf[KS];
  float p2 = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    pf[ks] = pval ? *reinterpret_cast<const u32x4_t *>(qsel + ((size_t)(b * dm.Hq + ph) * dm.n_sel + pgm) * D +
                                                       16 * ks + 8 * hl)
                  : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) p2 += bf16lo(pf[ks][i]) * bf16lo(pf[ks][i]) + bf16hi(pf[ks][i]) * bf16hi(pf[ks][i]);
  }
  p2 = pair_sum_f(p2);
  if (w == 0 && hl == 0) SPN[lq] = sqrtf(p2 + kSqFloor);
  const int ntile = (ncmax + 31) / 32;
  for (int t = w; t < ntile; t += kPW) {
    const int j = t * 32 + lq;
    const int jr = j < dm.n_blk ? j : dm.n_blk - 1;
    u32x4_t ka[KS];
    float k2 = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ka[ks] = *reinterpret_cast<const u32x4_t *>(kbase + (size_t)jr * D + 16 * ks + 8 * hl);
#pragma unroll
      for (int i = 0; i < 4; ++i) k2 += bf16lo(ka[ks][i]) * bf16lo(ka[ks][i]) + bf16hi(ka[ks][i]) * bf16hi(ka[ks][i]);
    }
    k2 = pair_sum_f(k2);
    if (hl == 0 && j < kPNc) SKN[j] = sqrtf(k2 + kSqFloor);
    const f32x16_t acc = mfma32_split<KS>(ka, pf);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int j0 = t * 32 + 8 * g4 + 4 * hl;
      if (j0 < kPNc)
        *reinterpret_cast<f32x4_t *>(S + lq * LY::SLD + j0) =
            f32x4_t{acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]};
    }
  }
  __syncthreads();

  // ---- 2. proxy top-C
  {
    constexpr int NS = NSX;
    float skr[NS];   // |ksel_c| of this lane's slots, shared by every proxy
    int cid[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      cid[s] = s * 64 + l;
      skr[s] = cid[s] < ncmax ? SKN[cid[s]] : 0.f;
    }
    for (int pl = next_proxy(&defn[2]); pl < kPX; pl = next_proxy(&defn[2])) {
      int h, gm, nc;
      if (!proxy(pl, h, gm, nc)) continue;
      const int c0 = min(dm.sink, nc);   // sink blocks are no candidates of the list
      const int C = min(ROWS ? dm.topk : dm.n_cand, nc - c0);
      int32_t *gout;
      int glen;
      uint16_t *lout;
      if constexpr (ROWS) {   // the row's kept list: sinks, then the selection
        int32_t *row = idx + ((size_t)(b * dm.Hq + h) * dm.n_rows + gm) * dm.klist;
        for (int c = l; c < c0; c += 64) row[c] = c;
        gout = row + c0;
        glen = dm.klist - c0;
        lout = nullptr;
      } else {
        gout = cand ? cand + ((size_t)(b * dm.Hq + h) * dm.n_sel + gm) * dm.n_cand : nullptr;
        glen = dm.n_cand;
        lout = LIST + pl * kPCap;
      }
      if (diag && l == 0) atomicAdd(&diag[0], 1);
      if (C == 0 || C >= nc - c0) {   // no candidate to take, or every one
        if (lout)
          for (int c = l; c < C; c += 64) lout[c] = (uint16_t)(c0 + c);
        if (gout)
          for (int c = l; c < glen; c += 64) gout[c] = c < C ? c0 + c : -1;
        continue;
      }
      const float cb = kG * SPN[pl];
      const int nsl = (nc + 63) / 64;
      float sc[NS], dl[NS];
      bool valid[NS], sel[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        valid[s] = cid[s] < nc && cid[s] >= c0;
        sc[s] = (s < nsl && valid[s]) ? S[pl * LY::SLD + cid[s]] : 0.f;
        dl[s] = fmaf(cb, skr[s], kAbsBound);
        if (route && s < nsl && valid[s]) {   // + lam M_j: exact product, one rounding (covered below)
          sc[s] = fmaf(lam, MC[cid[s]], sc[s]);
          dl[s] = fmaf(0x1p-22f, fabsf(sc[s]), dl[s]);
        }
      }
      if (fast_select<NS>(sc, dl, valid, nsl, C, sel)) {
        write_sorted_lds<NS>(sel, cid, lout, gout, glen);
      } else {
        const uint16_t *vec = qsel + ((size_t)(b * dm.Hq + h) * dm.n_sel + gm) * D;
        if (!rescore_select<D, NS>(S + pl * LY::SLD, nullptr, c0, nc, C, cb, SKN, route ? MC : nullptr, lam,
                                   vec, PVw, kbase, lout, gout, glen, diag) &&
            l == 0)
          defp[atomicAdd(&defn[0], 1)] = pl;
      }
    }
  }
  __syncthreads();
  if (w == 0) {   // undecided proxies: the exact tier
    const int nd = defn[0];
    for (int q = 0; q < nd; ++q) {
      const int pl = defp[q];
      int h, gm, nc;
      proxy(pl, h, gm, nc);
      const int c0 = min(dm.sink, nc);
      const int C = min(ROWS ? dm.topk : dm.n_cand, nc - c0);
      const uint16_t *vec = qsel + ((size_t)(b * dm.Hq + h) * dm.n_sel + gm) * D;
      if constexpr (ROWS) {   // the sinks are written already
        int32_t *row = idx + ((size_t)(b * dm.Hq + h) * dm.n_rows + gm) * dm.klist;
        exact_select<D, NSX>(sh, kbase, nullptr, c0, nc - c0, C, route ? MC : nullptr, lam, vec, nullptr,
                                   row + c0, dm.klist - c0, diag);
      } else {
        int32_t *gout = cand ? cand + ((size_t)(b * dm.Hq + h) * dm.n_sel + gm) * dm.n_cand : nullptr;
        exact_select<D, NSX>(sh, kbase, nullptr, c0, nc - c0, C, route ? MC : nullptr, lam, vec,
                             LIST + pl * kPCap, gout, dm.n_cand, diag);
      }
    }
  }
  if (ROWS) return;
  __syncthreads();
  if (dm.klist == 0) return;

  // ---- 3. members: their sinks, then the top-k of the proxy's list
  // member t's row: sink blocks 0 .. ct-1, then ascending selected ids
  auto member_row = [&](size_t qrow0, int t, int &ct) -> int32_t * {
    int own, lo;
    ct = min(dm.sink, pisa_row_geometry(dm, t, &own, &lo));
    int32_t *out = idx + (qrow0 + t) * dm.klist;
    for (int c = l; c < ct; c += 64) out[c] = c;
    return out + ct;
  };
  float *Mw = S + w * kPM * LY::MLD;
  for (int pl = next_proxy(&defn[3]); pl < kPX; pl = next_proxy(&defn[3])) {
    int h, gm, nc;
    if (!proxy(pl, h, gm, nc)) continue;
    const int C = min(dm.n_cand, nc - min(dm.sink, nc));
    const int n_take = min(dm.topk, C);
    const uint16_t *list = LIST + pl * kPCap;
    const int t0 = gm * g, t1 = min(dm.L, t0 + g);
    const size_t qrow0 = (size_t)(b * dm.Hq + h) * dm.L;
    if (n_take == 0 || n_take >= C) {   // nothing to choose: none, or the whole list
      const int m = n_take == 0 ? 0 : C;
      for (int t = t0; t < t1; ++t) {
        int ct;
        int32_t *out = member_row(qrow0, t, ct);
        for (int c = l; c < dm.klist - ct; c += 64) out[c] = c < m ? (int32_t)list[c] : -1;
        if (diag && l == 0) atomicAdd(&diag[0], 1);
      }
      continue;
    }
    constexpr int NS = kPCap / 64;
    int cj[NS];
    float skm[NS];
    bool valid[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int pos = s * 64 + l;
      valid[s] = pos < C;
      cj[s] = valid[s] ? (int)list[pos] : 0;
      skm[s] = SKN[cj[s]];
    }
    const int nsl = (C + 63) / 64;
    const int nct = (C + 31) / 32;
    for (int m0 = t0; m0 < t1; m0 += kPM) {
      const int nm = min(kPM, t1 - m0);
      // member queries as B (lane lq = member), the gathered list rows as A
      const bool mval = lq < nm;
      u32x4_t mq[KS];
      float q2 = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        mq[ks] = mval ? *reinterpret_cast<const u32x4_t *>(Q + (qrow0 + m0 + lq) * D + 16 * ks + 8 * hl)
                      : u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q2 += bf16lo(mq[ks][i]) * bf16lo(mq[ks][i]) + bf16hi(mq[ks][i]) * bf16hi(mq[ks][i]);
      }
      q2 = pair_sum_f(q2);
      const float qn = sqrtf(q2 + kSqFloor);
      for (int ct = 0; ct < nct; ++ct) {
        const int pos = ct * 32 + lq;
        const int j = list[pos < C ? pos : 0];
        u32x4_t ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[ks] = *reinterpret_cast<const u32x4_t *>(kbase + (size_t)j * D + 16 * ks + 8 * hl);
        // keep the gathered row's loads together (otherwise they are issued
        // one at a time, each waited for before its MFMA)
        __builtin_amdgcn_sched_barrier(0);
        const f32x16_t acc = mfma32_split<KS>(ka, mq);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int p0 = ct * 32 + 8 * g4 + 4 * hl;
          if (mval)
            *reinterpret_cast<f32x4_t *>(Mw + lq * LY::MLD + p0) =
                f32x4_t{acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]};
        }
      }
      wave_lds_sync();
      for (int m = 0; m < nm; ++m) {
        const int t = m0 + m;
        if (diag && l == 0) atomicAdd(&diag[0], 1);
        const float cb = kG * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qn), m));
        float sc[NS], dl[NS];
        bool sel[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          sc[s] = valid[s] ? Mw[m * LY::MLD + s * 64 + l] : 0.f;
          dl[s] = fmaf(cb, skm[s], kAbsBound);
          if (route && valid[s]) {
            sc[s] = fmaf(lam, MC[cj[s]], sc[s]);
            dl[s] = fmaf(0x1p-22f, fabsf(sc[s]), dl[s]);
          }
        }
        int ct;
        int32_t *out = member_row(qrow0, t, ct);
        if (fast_select<NS>(sc, dl, valid, nsl, n_take, sel)) {
          write_sorted_lds<NS>(sel, cj, nullptr, out, dm.klist - ct);
        } else if (!rescore_select<D, NS>(Mw + m * LY::MLD, list, 0, C, n_take, cb, SKN, route ? MC : nullptr, lam,
                                          Q + (qrow0 + t) * D, PVw, kbase, nullptr, out, dm.klist - ct, diag) &&
                   l == 0) {
          defm[atomicAdd(&defn[1], 1)] = t * 64 + pl;
        }
      }
      wave_lds_sync();
    }
  }
  __syncthreads();
  if (w == 0) {   // undecided members: the exact tier over the proxy's list
    const int nd = defn[1];
    for (int q = 0; q < nd; ++q) {
      const int t = defm[q] >> 6, pl = defm[q] & 63;
      int h, gm, nc;
      proxy(pl, h, gm, nc);
      const int C = min(dm.n_cand, nc - min(dm.sink, nc));
      const int n_take = min(dm.topk, C);
      const size_t row = (size_t)(b * dm.Hq + h) * dm.L + t;
      int own, lo;
      const int ct = min(dm.sink, pisa_row_geometry(dm, t, &own, &lo));
      exact_select<D, kPCap / 64>(sh, kbase, LIST + pl * kPCap, 0, C, n_take, route ? MC : nullptr, lam,
                                  Q + row * D, nullptr, idx + row * dm.klist + ct, dm.klist - ct, diag);
    }
  }
}

// Decode: the kept list of one new token (q [B, Hq, d]) at position pos, a
// causal token row: sinks, then the top-k of candidates [c0, lo) by q . ksel_j
// (+ lam mcov_j), as select_row decides it.
// Decode: one workgroup of kDecIdxWaves waves per (b, head).  The waves
// score the candidate slots s = w, w + kDecIdxWaves, ... (score_slot, into
// LDS), then wave 0 selects over all of them (select_row with the scores
// given).  A decode row has a single wave's worth of selection work but up
// to 16 slots of candidate rows to load; sharing the loads cuts the chain of
// memory latencies the row waits for.
constexpr int kDecIdxWaves = 4;

template <typename T, int D>
__global__ __launch_bounds__(kDecIdxWaves * 64) void indexer_decode(PisaDims dm, int pos, const T *__restrict__ q,
                                                                    const T *__restrict__ ksel,
                                                                    const float *__restrict__ mcov,
                                                                    int32_t *__restrict__ idx, int32_t *diag) {
  __shared__ Shared sh;
  __shared__ double psc[kMaxSlots * 64];
  __shared__ float pk2[kMaxSlots * 64];
  const int row = blockIdx.x;   // b * Hq + h
  const int b = row / dm.Hq, h = row % dm.Hq;
  const int hk = h * dm.Hkv / dm.Hq;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const T *kbase = ksel + ((size_t)b * dm.Hkv + hk) * dm.n_blk * D;
  int own, lo;
  const int nc = pisa_row_geometry(dm, pos, &own, &lo);
  const int c0 = min(dm.sink, nc);
  const int n_take = min(dm.topk, nc - c0);
  const int ncand = nc - c0;
  for (int c = threadIdx.x; c < D; c += kDecIdxWaves * 64) {
    const float v = load_elem(q + (size_t)row * D, c);
    sh.pf[c] = v;
    sh.p[c] = (double)v;
  }
  __syncthreads();
  if (n_take > 0 && n_take < ncand) {
    for (int sl = w; sl * 64 < ncand; sl += kDecIdxWaves) {
      const int c = sl * 64 + l;
      const bool ok = c < ncand;
      double scv;
      float k2v;
      score_slot<T, D>(sh, kbase + (size_t)(ok ? c0 + c : 0) * D, ok, scv, k2v);
      psc[sl * 64 + l] = scv;
      pk2[sl * 64 + l] = k2v;
    }
  }
  __syncthreads();
  if (w != 0) return;
  bool sel[kMaxSlots];
  int cj[kMaxSlots];
  const float *mb = mcov ? mcov + ((size_t)b * dm.Hkv + hk) * dm.n_blk : nullptr;
  select_row<T, D, kMaxSlots, true, true>(sh, kbase, nullptr, c0, ncand, n_take, mb, dm.route_lambda, sel, cj,
                                          diag, psc, pk2);
  int32_t *out = idx + (size_t)row * dm.klist;
  for (int c = lane_id(); c < c0; c += 64) out[c] = c;
  write_sorted<kMaxSlots>(sel, cj, out + c0, dm.klist - c0);
}

__global__ void zero_diag(int32_t *d) {
  if (threadIdx.x < 16) d[threadIdx.x] = 0;
}

// PIVOT proxies and members, or block rows (ROWS), on the matrix cores: 32
// proxies (rows) per workgroup
template <int D, bool ROWS, int NSX>
hipError_t launch_pivot_mfma(const PisaDims &dm, const void *Q, const void *qsel, const void *ksel,
                             const float *mcov, int32_t *idx, int32_t *cand, int32_t *diag, hipStream_t st,
                             int blo = 0, int nbr = -1) {
  if (nbr < 0) nbr = dm.n_blk;
  using LY = PivotLayout;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&indexer_pivot_mfma<D, ROWS, NSX>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::TOTAL);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int npb = ROWS ? dm.ratio * dm.n_blk : dm.ratio * (dm.bs / dm.group);
  const unsigned chunks = (unsigned)((npb + kPX - 1) / kPX);
  const unsigned grid = ROWS ? (unsigned)dm.B * dm.Hkv * chunks : (unsigned)dm.B * dm.Hkv * nbr * chunks;
  indexer_pivot_mfma<D, ROWS, NSX><<<grid, kPW * 64, LY::TOTAL, st>>>(
      dm, static_cast<const uint16_t *>(Q), static_cast<const uint16_t *>(qsel),
      static_cast<const uint16_t *>(ksel), mcov, idx, cand, diag, blo, nbr);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(const PisaDims &dm, const void *Q, const void *qsel, const void *ksel, const float *mcov,
                    int32_t *idx, int32_t *cand, int32_t *diag, hipStream_t st) {
  if (diag) zero_diag<<<1, 64, 0, st>>>(diag);
  if constexpr (sizeof(T) == 2) {
    if ((dm.group >= 1 && dm.n_cand <= kPCap && dm.group <= kPG) || (dm.group == 0 && dm.n_blk <= kPNc)) {
      const bool rows = dm.group == 0;
      if (!rows && dm.causal && dm.n_blk > 256) {
        // causal proxies of query block i have at most i candidates: blocks
        // [0, 256) take the 4-slot build, [256, 512) the 8-slot one,
        // [512, 768) 12 slots, the rest 16 (fewer registers held, fewer
        // spilled)
        hipError_t e = hipSuccess;
        if (dm.n_blk > 768)
          e = launch_pivot_mfma<D, false, 16>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st, 768, dm.n_blk - 768);
        if (e != hipSuccess) return e;
        if (dm.n_blk > 512)
          e = launch_pivot_mfma<D, false, 12>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st, 512,
                                              (dm.n_blk < 768 ? dm.n_blk : 768) - 512);
        if (e != hipSuccess) return e;
        e = launch_pivot_mfma<D, false, 8>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st, 256,
                                           (dm.n_blk < 512 ? dm.n_blk : 512) - 256);
        if (e != hipSuccess) return e;
        return launch_pivot_mfma<D, false, 4>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st, 0, 256);
      }
      if (dm.n_blk <= 256) return rows ? launch_pivot_mfma<D, true, 4>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st)
                                       : launch_pivot_mfma<D, false, 4>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st);
      if (dm.n_blk <= 512) return rows ? launch_pivot_mfma<D, true, 8>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st)
                                       : launch_pivot_mfma<D, false, 8>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st);
      return rows ? launch_pivot_mfma<D, true, 16>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st)
                  : launch_pivot_mfma<D, false, 16>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st);
    }
  }
  if (dm.group >= 1) {
    const unsigned grid = (unsigned)dm.B * dm.Hq * dm.n_sel;
    indexer_pivot<T, D><<<grid, 64, 0, st>>>(dm, static_cast<const T *>(Q), static_cast<const T *>(qsel),
                                             static_cast<const T *>(ksel), mcov, idx, cand, diag);
  } else {
    const unsigned grid = (unsigned)dm.B * dm.Hq * dm.n_blk;
    indexer_blockrows<T, D><<<grid, 64, 0, st>>>(dm, static_cast<const T *>(qsel), static_cast<const T *>(ksel),
                                                 mcov, idx, diag);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_topk(const PisaDims &dm, int pos, const void *q, const void *ksel, const float *mcov,
                              int32_t *idx, int32_t *diag, hipStream_t st) {
  if (diag) zero_diag<<<1, 64, 0, st>>>(diag);
  const unsigned grid = (unsigned)dm.B * dm.Hq;
  if (dm.dtype == 0) {
    if (dm.d == 64)
      indexer_decode<uint16_t, 64><<<grid, kDecIdxWaves * 64, 0, st>>>(dm, pos, static_cast<const uint16_t *>(q),
                                                        static_cast<const uint16_t *>(ksel), mcov, idx, diag);
    else
      indexer_decode<uint16_t, 128><<<grid, kDecIdxWaves * 64, 0, st>>>(dm, pos, static_cast<const uint16_t *>(q),
                                                         static_cast<const uint16_t *>(ksel), mcov, idx, diag);
  } else {
    if (dm.d == 64)
      indexer_decode<float, 64><<<grid, kDecIdxWaves * 64, 0, st>>>(dm, pos, static_cast<const float *>(q),
                                                     static_cast<const float *>(ksel), mcov, idx, diag);
    else
      indexer_decode<float, 128><<<grid, kDecIdxWaves * 64, 0, st>>>(dm, pos, static_cast<const float *>(q),
                                                      static_cast<const float *>(ksel), mcov, idx, diag);
  }
  return hipGetLastError();
}

hipError_t launch_indexer(const PisaDims &dm, const void *Q, const void *qsel, const void *ksel, const float *mcov,
                          int32_t *idx, int32_t *cand, int32_t *diag, hipStream_t st) {
  if (dm.dtype == 0)
    return dm.d == 64 ? launch_t<uint16_t, 64>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st)
                      : launch_t<uint16_t, 128>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st);
  return dm.d == 64 ? launch_t<float, 64>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st)
                    : launch_t<float, 128>(dm, Q, qsel, ksel, mcov, idx, cand, diag, st);
}
