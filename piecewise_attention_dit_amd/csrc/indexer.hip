// Stage B: block scores and top-k selection.
//
// PISA page, section 2 (routing by attention score): a selection row r scores
// every candidate key block j by the dot product of its pooled query with the
// pooled key, s_rj = qsel_r . ksel_j, and keeps the top k (ties to the lower
// block index).  PIVOT page, steps 1-4: a proxy (mean of g consecutive
// queries) scores the candidates once and keeps C of them; each member of the
// group re-ranks only that list with its own query.
//
// One wavefront per selection unit (a block row, or a PIVOT group with its
// members).  Selection is bit-exact with respect to the exact real scores:
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

// Exact sign of  p . kb - p . ka  (p, kb, ka are fp32 / bf16 values) using a
// per-lane fixed-point accumulator of kLimbs 32-bit digits held in LDS
// (acc[limb * 64 + lane]).
template <typename T, int D>
PISA_DEV int exact_cmp(const float *p, const T *kb, const T *ka, int64_t *acc) {
  const int l = lane_id();
  bool same = true;
  for (int c = 0; c < D && same; ++c) same = kb[c] == ka[c];
  if (same) return 0;  // identical pooled keys tie exactly
  for (int i = 0; i < kLimbs; ++i) acc[i * 64 + l] = 0;
  for (int side = 0; side < 2; ++side) {
    const T *kr = side == 0 ? kb : ka;
    for (int c = 0; c < D; ++c) {
      const float x = p[c], y = load_elem(kr, c);
      if (x == 0.f || y == 0.f) continue;
      uint32_t mx, my;
      int ex, ey;
      decompose(x, mx, ex);
      decompose(y, my, ey);
      const bool neg = ((x < 0.f) != (y < 0.f)) != (side == 1);
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
    }
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

// Rank the candidates cand(c) = (list ? list[c] : c), c < nc, of one row and
// mark the n_take best in sel[].  NS slots per lane (candidate c = s*64+lane).
template <typename T, int D, int NS>
PISA_DEV void select_row(Shared &sh, const T *kbase, const int32_t *list, int nc, int n_take,
                         bool (&sel)[NS], int (&cj)[NS], int32_t *diag) {
  const int l = lane_id();
  bool valid[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = s * 64 + l;
    valid[s] = c < nc;
    cj[s] = valid[s] ? (list ? list[c] : c) : 0;
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
    __syncthreads();
    const uint64_t hi_mask = (shift + 8 >= 64) ? 0ull : ~((1ull << (shift + 8)) - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (valid[s] && (key[s] & hi_mask) == prefix) atomicAdd(&sh.hist[(key[s] >> shift) & 255u], 1u);
    __syncthreads();
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
    __syncthreads();
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
          const int c = exact_cmp<T, D>(sh.pf, kbase + (size_t)jb * D, kbase + (size_t)cj[sa] * D, sh.kul);
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
                                                        const T *__restrict__ ksel, int32_t *__restrict__ idx,
                                                        int32_t *diag) {
  __shared__ Shared sh;
  const int unit = blockIdx.x;
  const int i = unit % dm.n_blk;
  const int bh = unit / dm.n_blk;  // b * Hq + h
  const int b = bh / dm.Hq, h = bh % dm.Hq;
  const int hk = h * dm.Hkv / dm.Hq;
  const T *kbase = ksel + ((size_t)b * dm.Hkv + hk) * dm.n_blk * D;
  int own, lo;
  const int nc = pisa_row_geometry(dm, i * dm.bs, &own, &lo);
  const int n_take = min(dm.topk, nc);
  load_p<T, D>(sh, qsel + ((size_t)bh * dm.n_sel + i) * D);
  bool sel[kMaxSlots];
  int cj[kMaxSlots];
  select_row<T, D, kMaxSlots>(sh, kbase, nullptr, nc, n_take, sel, cj, diag);
  write_sorted<kMaxSlots>(sel, cj, idx + ((size_t)bh * dm.n_rows + i) * dm.topk, dm.topk);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void indexer_pivot(PisaDims dm, const T *__restrict__ Q,
                                                    const T *__restrict__ qsel, const T *__restrict__ ksel,
                                                    int32_t *__restrict__ idx, int32_t *__restrict__ cand,
                                                    int32_t *diag) {
  __shared__ Shared sh;
  const int unit = blockIdx.x;
  const int gm = unit % dm.n_sel;
  const int bh = unit / dm.n_sel;
  const int b = bh / dm.Hq, h = bh % dm.Hq;
  const int hk = h * dm.Hkv / dm.Hq;
  const T *kbase = ksel + ((size_t)b * dm.Hkv + hk) * dm.n_blk * D;
  const int g = dm.group;
  int own, lo;
  const int nc = pisa_row_geometry(dm, gm * g, &own, &lo);
  const int C = min(dm.n_cand, nc);
  // proxy pass over every candidate block
  load_p<T, D>(sh, qsel + ((size_t)bh * dm.n_sel + gm) * D);
  {
    bool sel[kMaxSlots];
    int cj[kMaxSlots];
    select_row<T, D, kMaxSlots>(sh, kbase, nullptr, nc, C, sel, cj, diag);
    write_sorted<kMaxSlots>(sel, cj, sh.clist, C);
    if (cand) {
      __syncthreads();
      int32_t *cout = cand + ((size_t)bh * dm.n_sel + gm) * dm.n_cand;
      for (int c = lane_id(); c < dm.n_cand; c += 64) cout[c] = c < C ? sh.clist[c] : -1;
    }
  }
  __syncthreads();
  if (dm.topk == 0) return;
  // member pass over the proxy's list
  const int n_take = min(dm.topk, C);
  const int t1 = min(dm.L, (gm + 1) * g);
  for (int t = gm * g; t < t1; ++t) {
    load_p<T, D>(sh, Q + ((size_t)bh * dm.L + t) * D);
    bool sel[4];
    int cj[4];
    select_row<T, D, 4>(sh, kbase, sh.clist, C, n_take, sel, cj, diag);
    write_sorted<4>(sel, cj, idx + ((size_t)bh * dm.n_rows + t) * dm.topk, dm.topk);
    __syncthreads();
  }
}

__global__ void zero_diag(int32_t *d) {
  if (threadIdx.x < 16) d[threadIdx.x] = 0;
}

template <typename T, int D>
hipError_t launch_t(const PisaDims &dm, const void *Q, const void *qsel, const void *ksel, int32_t *idx,
                    int32_t *cand, int32_t *diag, hipStream_t st) {
  if (diag) zero_diag<<<1, 64, 0, st>>>(diag);
  if (dm.group >= 1) {
    const unsigned grid = (unsigned)dm.B * dm.Hq * dm.n_sel;
    indexer_pivot<T, D><<<grid, 64, 0, st>>>(dm, static_cast<const T *>(Q), static_cast<const T *>(qsel),
                                             static_cast<const T *>(ksel), idx, cand, diag);
  } else {
    const unsigned grid = (unsigned)dm.B * dm.Hq * dm.n_blk;
    indexer_blockrows<T, D><<<grid, 64, 0, st>>>(dm, static_cast<const T *>(qsel), static_cast<const T *>(ksel),
                                                 idx, diag);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const PisaDims &dm, const void *Q, const void *qsel, const void *ksel, int32_t *idx,
                          int32_t *cand, int32_t *diag, hipStream_t st) {
  if (dm.dtype == 0)
    return dm.d == 64 ? launch_t<uint16_t, 64>(dm, Q, qsel, ksel, idx, cand, diag, st)
                      : launch_t<uint16_t, 128>(dm, Q, qsel, ksel, idx, cand, diag, st);
  return dm.d == 64 ? launch_t<float, 64>(dm, Q, qsel, ksel, idx, cand, diag, st)
                    : launch_t<float, 128>(dm, Q, qsel, ksel, idx, cand, diag, st);
}
