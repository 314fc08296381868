// Stage A: mean-pooled block statistics (PISA page, section 2: precompute of
// block centroids, value sums and per-block first-order matrices; PIVOT page,
// step 2: the proxy query is the mean of its group).
//
//   kv_stats_*   one workgroup per (b, kv head, key block j):
//                ksel_j = RNE_dtype(mean key), kbar_j = fp32(mean key),
//                vsum_j = sum of value rows, HT_j[e][c] = sum_n v_{n,e} (k_{n,c} - kbar_c)
//   q_pool       one thread per (selection row, 16-byte column chunk):
//                qsel = RNE_dtype(mean of the row's queries)
//   hbar_*       hybrid order: HbarT = transposed mean of H_j over all blocks
//                of a (b, kv head) (the global first-order statistic); for
//                causal rows one mean per lo, over the blocks [0, lo)
//
// The means are float64 cascaded sums divided once (IEEE division) and rounded
// once into the dtype.  HBM-bound: Q, K and V are read exactly once.
#include "attn_tiles.h"

using namespace pisa_attn;

namespace {

constexpr int kStatsThreads = 256;

// ---------------------------------------------------------------------------
// Exact float64 sums of bf16 values, cheap path.  A bf16 value is an integer
// of at most 8 bits times 2^(max(E, 1) - 134), E its exponent field, so n
// values are integer multiples of the smallest nonzero one's quantum and every
// running sum of them stays below n * 2^(span + 8) of those quanta, span being
// the spread of max(E, 1) over the nonzero values.  Below 2^53 quanta a plain
// float64 sum is exact.  The packed u16 max of |bits| and min of |bits| - 1
// (zeros wrap to 0xFFFF and drop out) give the spread of each half of a word.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

struct SpanCert {
  u16x2_t amax = {0, 0}, amin = {0xFFFF, 0xFFFF};
  PISA_DEV void add(uint32_t w) {
    const u16x2_t a = __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
    amax = __builtin_elementwise_max(amax, a);
    amin = __builtin_elementwise_min(amin, a - u16x2_t{1, 1});
  }
  // every partial sum of the half h (0: low bf16) is exact for n <= 2^lg addends
  PISA_DEV bool exact(int h, int lg) const {
    const int mx = h ? amax[1] : amax[0], mn = h ? amin[1] : amin[0];
    if (mn == 0xFFFF) return true;   // all zero
    const int emax = mx >> 7, emin = max((mn + 1) >> 7, 1);
    return emax - emin <= 45 - lg;
  }
};

// ---------------------------------------------------------------------------
// bf16 K/V statistics, one workgroup of eight waves per key block (two
// workgroups fit a CU, so one block's loads overlap another's arithmetic):
//   * K and V tiles move global -> LDS by DMA, row-major, 16-byte chunks
//     permuted by vswz (tokens past the sequence end read as zeros);
//   * lane (feature pair, token class p) sums the tokens t = p (mod PARTS) of
//     its two features; key sums exactly (certified float64, double-double
//     when the certificate fails) and merged across the PARTS lanes of the
//     pair with exact double-double additions; value sums in float64;
//   * first order: the K tile is centred in place, 16 bytes at a time (bf16
//     of k - kbar, so keys that all equal their mean give exactly zero), then
//     HT = V^T Kc on MFMA 32x32x16 as T = Kc^T V with both operands read
//     transposed from the tiles (ds_read_b64_tr_b16), rounded once to bf16,
//     staged in LDS and written with 16-byte stores.
constexpr int kKvWaves = 8, kKvThreads = 64 * kKvWaves;

template <int D, int BS>
struct KvCfg {
  static constexpr int TILE = BS * D * 2;                 // bytes of one K (or V) tile
  static constexpr int CPW = TILE / 1024 / kKvWaves;      // DMA kilobytes per wave and tile
  static constexpr int NPAIR = D / 2;                     // feature pairs
  static constexpr int PARTS = kKvThreads / NPAIR;        // token classes per pair (8 or 16)
  static constexpr int SEG = BS / PARTS;                  // tokens per lane
  static constexpr int LG = SEG <= 4 ? 2 : SEG <= 8 ? 3 : 4;
  static constexpr int NT = D / 32;                       // 32x32 output tiles per dimension
  static constexpr int MW = NT * NT < kKvWaves ? NT * NT : kKvWaves;   // waves with MFMA tiles
  static constexpr int TPW = NT * NT / MW;                // tiles per such wave (same e tile)
  static constexpr int OP = D + 4;                        // staging pitch (bf16)
  static constexpr int STG = D * OP * 2;
  static constexpr int TILES = 2 * TILE > STG ? 2 * TILE : STG;
  static constexpr int MEAN = TILES;                      // float [D]: kbar
  static constexpr int TOTAL = MEAN + D * 4;
  static_assert(SEG >= 4 && SEG <= 16 && TILE % (1024 * kKvWaves) == 0, "token split and DMA split");
  static_assert(NT % TPW == 0, "a wave's tiles share one e tile");
  static_assert(TOTAL <= 80 * 1024, "two workgroups per CU");
};

template <int D, int BS>
__global__ __launch_bounds__(kKvThreads) void kv_stats_bf16(PisaDims dm, const uint16_t *__restrict__ K,
                                                           const uint16_t *__restrict__ V,
                                                           uint16_t *__restrict__ ksel,
                                                           float *__restrict__ kbar,
                                                           float *__restrict__ vsum,
                                                           uint16_t *__restrict__ HT) {
  using C = KvCfg<D, BS>;
  constexpr int PARTS = C::PARTS, SEG = C::SEG, TPW = C::TPW, NT = C::NT, OP = C::OP;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t *kt = lds, *vt = lds + C::TILE;
  float *kmean = reinterpret_cast<float *>(lds + C::MEAN);

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, lq = l & 31, hl = l >> 5;
  const int j = blockIdx.x % dm.n_blk;
  const int bh = blockIdx.x / dm.n_blk;  // b * Hkv + hk
  const int n = min(BS, dm.L - j * BS);
  const size_t base = ((size_t)bh * dm.L + (size_t)j * BS) * D;
  const bool has_v = dm.taylor != 0, order1 = dm.taylor == 2;

  // ---- tiles: kilobyte c of a tile holds 16-byte chunks 64 c .. 64 c + 63
#pragma unroll
  for (int u = 0; u < C::CPW; ++u) {
    const int c = wave + kKvWaves * u, pos = c * 64 + l;
    const int row = pos / (D / 8), phys = pos % (D / 8);
    const int voff = (row * D + ((phys ^ vswz<D>(row)) << 3)) * 2;
    dma16_buf(K + base, n * D * 2, voff, kt + c * 1024);
    if (has_v) dma16_buf(V + base, n * D * 2, voff, vt + c * 1024);
  }
  wait_vmcnt<0>();
  __syncthreads();

  // ---- column sums: lane (pair pr, class p), tokens p, p + PARTS, ...
  {
    const int pr = wave * (64 / PARTS) + l / PARTS, p = l % PARTS;
    // the swizzle of row t depends on t & 3 = p & 3 only
    const int off0 = p * (2 * D) + (((pr >> 2) ^ vswz<D>(p)) << 4) + (pr & 3) * 4;
    double sk[2] = {0.0, 0.0}, sv[2] = {0.0, 0.0};
    SpanCert ck;
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int off = off0 + i * PARTS * (2 * D);
      const uint32_t kw = *reinterpret_cast<const uint32_t *>(kt + off);
      sk[0] += (double)bf16lo(kw);
      sk[1] += (double)bf16hi(kw);
      ck.add(kw);
      if (has_v) {
        const uint32_t vw = *reinterpret_cast<const uint32_t *>(vt + off);
        sv[0] += (double)bf16lo(vw);
        sv[1] += (double)bf16hi(vw);
      }
    }
    DD dk[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      dk[h] = {sk[h], 0.0};
      // a certificate that fails (exponent spread near 45 bits): redo exactly
      if (!ck.exact(h, C::LG)) {
        dk[h] = {0.0, 0.0};
        for (int i = 0; i < SEG; ++i) {
          const uint32_t kw = *reinterpret_cast<const uint32_t *>(kt + off0 + i * PARTS * (2 * D));
          dd_add(dk[h], (double)(h ? bf16hi(kw) : bf16lo(kw)));
        }
      }
    }
    // merge the PARTS classes of a pair (lanes l ^ m)
#pragma unroll
    for (int m = 1; m < PARTS; m <<= 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const DD ok = {__shfl_xor(dk[h].hi, m), __shfl_xor(dk[h].lo, m)};
        dd_merge(dk[h], ok);
        if (has_v) sv[h] += __shfl_xor(sv[h], m);
      }
    }
    if (p == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int f = 2 * pr + h;
        const double mean = dd_value(dk[h]) / (double)n;
        const size_t so = ((size_t)bh * dm.n_blk + j) * D + f;
        ksel[so] = (uint16_t)f64_to_bf16_bits(mean);
        const float m32 = (float)mean;
        kmean[f] = m32;
        if (has_v) {
          kbar[so] = m32;
          vsum[so] = (float)sv[h];
        }
      }
    }
  }
  if (!order1) return;
  __syncthreads();   // the column sums have read the tiles; kbar is in LDS

  // ---- centre the keys in place, one 16-byte chunk (8 features of a token)
  // at a time: bf16(k - kbar), tokens past n stay zero
  for (int ci = tid; ci < C::TILE / 16; ci += kKvThreads) {
    const int row = ci / (D / 8), phys = ci % (D / 8);
    const int f0 = (phys ^ vswz<D>(row)) << 3;
    u32x4_t *cp = reinterpret_cast<u32x4_t *>(kt + ci * 16);
    u32x4_t w = *cp;
    if (row < n) {
      const f32x4_t m0 = *reinterpret_cast<const f32x4_t *>(kmean + f0);
      const f32x4_t m1 = *reinterpret_cast<const f32x4_t *>(kmean + f0 + 4);
      w[0] = pack_bf16x2(bf16lo(w[0]) - m0[0], bf16hi(w[0]) - m0[1]);
      w[1] = pack_bf16x2(bf16lo(w[1]) - m0[2], bf16hi(w[1]) - m0[3]);
      w[2] = pack_bf16x2(bf16lo(w[2]) - m1[0], bf16hi(w[2]) - m1[1]);
      w[3] = pack_bf16x2(bf16lo(w[3]) - m1[2], bf16hi(w[3]) - m1[3]);
    } else {
      w = u32x4_t{0, 0, 0, 0};
    }
    *cp = w;
  }
  __syncthreads();

  // ---- T = Kc^T V (rows c, columns e) on MFMA: wave w < MW takes e tile te
  // and c tiles tc0 .. tc0 + TPW - 1
  f32x16_t acc[TPW];
  const int te = wave / (NT / TPW), tc0 = (wave % (NT / TPW)) * TPW;
  if (wave < C::MW) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = f32x16_t{};
    const int srow = (l & 15) >> 2, ecol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
#pragma unroll
    for (int ks = 0; ks < BS / 16; ++ks) {
      const int rr = ks * 16 + 4 * hl + srow;
      const u32x4_t b = frag_vt<D>(vt, rr, te * 32 + ecol);
#pragma unroll
      for (int i = 0; i < TPW; ++i) acc[i] = mfma32(frag_vt<D>(kt, rr, (tc0 + i) * 32 + ecol), b, acc[i]);
    }
  }
  __syncthreads();   // the MFMA reads of the tiles are done: reuse them for staging

  // ---- HT[e][c] = T[c][e] -> bf16, staged [e][c], then 16-byte stores
  uint16_t *ot = reinterpret_cast<uint16_t *>(lds);
  if (wave < C::MW) {
    const int e = te * 32 + lq;
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c0 = (tc0 + i) * 32 + 8 * q + 4 * hl;
        u32x2_t o;
        o[0] = pack_bf16x2(acc[i][4 * q], acc[i][4 * q + 1]);
        o[1] = pack_bf16x2(acc[i][4 * q + 2], acc[i][4 * q + 3]);
        *reinterpret_cast<u32x2_t *>(ot + e * OP + c0) = o;
      }
  }
  __syncthreads();
  uint16_t *Hb = HT + ((size_t)bh * dm.n_blk + j) * D * D;
  for (int u = tid; u < D * D / 8; u += kKvThreads) {
    const int e = u / (D / 8), c8 = (u % (D / 8)) * 8;
    const u32x2_t lo2 = *reinterpret_cast<const u32x2_t *>(ot + e * OP + c8);
    const u32x2_t hi2 = *reinterpret_cast<const u32x2_t *>(ot + e * OP + c8 + 4);
    *reinterpret_cast<u32x4_t *>(Hb + (size_t)e * D + c8) = u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  }
}

// ---------------------------------------------------------------------------
// fp32 K/V statistics (VALU; the fp32 path has no MFMA moment GEMM).
template <int D, int BS>
__global__ __launch_bounds__(kStatsThreads) void kv_stats_f32(PisaDims dm, const float *__restrict__ K,
                                                             const float *__restrict__ V,
                                                             float *__restrict__ ksel,
                                                             float *__restrict__ kbar,
                                                             float *__restrict__ vsum,
                                                             float *__restrict__ HT) {
  constexpr int PARTS = kStatsThreads / D;
  __shared__ double red[2][PARTS][D][2];
  __shared__ float kmean[D];
  const int tid = threadIdx.x;
  const int bid = blockIdx.x;
  const int j = bid % dm.n_blk;
  const int bh = bid / dm.n_blk;
  const int n = min(BS, dm.L - j * BS);
  const size_t base = ((size_t)bh * dm.L + (size_t)j * BS) * D;
  const float *Kb = K + base;
  const float *Vb = V + base;
  const bool taylor = dm.taylor != 0;
  {
    const int f = tid % D, part = tid / D;
    DD sk = {0.0, 0.0}, sv = {0.0, 0.0};
    for (int t = part; t < n; t += PARTS) {
      dd_add(sk, (double)Kb[(size_t)t * D + f]);
      if (taylor) dd_add(sv, (double)Vb[(size_t)t * D + f]);
    }
    red[0][part][f][0] = sk.hi;
    red[0][part][f][1] = sk.lo;
    red[1][part][f][0] = sv.hi;
    red[1][part][f][1] = sv.lo;
  }
  __syncthreads();
  if (tid < D) {
    const int f = tid;
    DD sk = {red[0][0][f][0], red[0][0][f][1]}, sv = {red[1][0][f][0], red[1][0][f][1]};
    for (int part = 1; part < PARTS; ++part) {
      DD o = {red[0][part][f][0], red[0][part][f][1]};
      dd_merge(sk, o);
      DD ov = {red[1][part][f][0], red[1][part][f][1]};
      dd_merge(sv, ov);
    }
    const double mean = dd_value(sk) / (double)n;
    const size_t so = ((size_t)bh * dm.n_blk + j) * D + f;
    ksel[so] = (float)round_to_format(mean, 24);
    kmean[f] = (float)mean;
    if (taylor) {
      kbar[so] = (float)mean;
      vsum[so] = (float)dd_value(sv);
    }
  }
  if (dm.taylor != 2) return;
  __syncthreads();
  // HT[e][c] = sum_n v[n][e] (k[n][c] - kbar_c), summed over n in order.
  // The block's rows pass through LDS kTC tokens at a time (keys centred
  // there); thread (te, tc) of a 16 x 16 grid owns the RT x RT outputs
  // e in [RT te, RT te + RT), c in [RT tc, RT tc + RT).
  constexpr int kTC = 32, RT = D / 16;
  static_assert(kStatsThreads == 256, "a 16 x 16 thread grid");
  __shared__ __attribute__((aligned(16))) float kc[kTC * D];
  __shared__ __attribute__((aligned(16))) float vr[kTC * D];
  const int e0 = RT * (tid / 16), c0 = RT * (tid % 16);
  float s[RT][RT];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b2 = 0; b2 < RT; ++b2) s[a][b2] = 0.f;
  for (int t0 = 0; t0 < n; t0 += kTC) {
    const int nt = min(kTC, n - t0);
    __syncthreads();   // the previous tokens are consumed
    for (int i = tid; i < nt * D; i += kStatsThreads) {
      const size_t g = (size_t)(t0 + i / D) * D + i % D;
      kc[i] = Kb[g] - kmean[i % D];
      vr[i] = Vb[g];
    }
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      float ve[RT], kk[RT];
#pragma unroll
      for (int a = 0; a < RT; a += 4) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t *>(vr + t * D + e0 + a);
        const f32x4_t y = *reinterpret_cast<const f32x4_t *>(kc + t * D + c0 + a);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ve[a + i] = x[i];
          kk[a + i] = y[i];
        }
      }
#pragma unroll
      for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b2 = 0; b2 < RT; ++b2) s[a][b2] = fmaf(ve[a], kk[b2], s[a][b2]);
    }
  }
  float *Hb = HT + ((size_t)bh * dm.n_blk + j) * D * D;
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b2 = 0; b2 < RT; b2 += 4)
      *reinterpret_cast<f32x4_t *>(Hb + (size_t)(e0 + a) * D + c0 + b2) =
          f32x4_t{s[a][b2], s[a][b2 + 1], s[a][b2 + 2], s[a][b2 + 3]};
}

// ---------------------------------------------------------------------------
// Hybrid order: HbarT[e][c] = (1 / n_blk) sum_j H_j[c][e] (PISA page, section
// 2: the global first-order statistic, the mean of the per-block matrices).
//
// bf16, two kernels:
//   hbar_run    one workgroup of four waves per (b, kv head, run of kHbarRun
//               consecutive blocks).  Each block of the run is staged in LDS
//               by DMA (K and V tiles in the transposed-read layout, two
//               slots); the waves form its raw moment R_j^T[e][c] =
//               sum_n v_{n,e} k_{n,c} on MFMA (exact bf16 products, fp32 sums
//               of at most 128 terms) and add H_j^T = R_j^T - sigma_j kbar_j^T
//               to the run's fp32 sum in the workspace;
//   hbar_final  one thread per (b, kv head, e, c): the runs in order, / n_blk.
// Causal rows (the mean over a row's Taylor candidates [0, lo), one matrix
// per lo):
//   hbar_run    as above, the run sums;
//   hbar_scan   one thread per (b, kv head, e, c): the run sums become
//               exclusive prefix sums over the runs, in place;
//   hbar_run    PREFIX: each run starts from its prefix sum and writes
//               sum / j as HbarT(lo = j) before it adds block j (HbarT(0) = 0).
// The centring follows the exact products, so no rounded centred key enters,
// and every sum has a fixed order, so the result is deterministic.
template <int D, int BS>
struct HbarCfg {
  static constexpr int NE = D / 32;              // 32 x 32 tiles per dimension
  static constexpr int TPW = NE * NE / 4;        // tiles per wave: one e tile, TPW c tiles
  static constexpr int TILE = BS * D * 2;        // bytes of one K (or V) tile
  static constexpr int CPW = TILE / 1024 / 4;    // DMA kilobytes per wave and tile
  static constexpr int TOTAL = 4 * TILE;         // two slots of (K, V)
  static_assert(CPW >= 1 && (TILE / 1024) % 4 == 0, "tile must split over four waves");
};

template <int D, int BS, bool PREFIX>
__global__ __launch_bounds__(256) void hbar_run(PisaDims dm, const uint16_t *__restrict__ K,
                                                const uint16_t *__restrict__ V,
                                                const float *__restrict__ kbar,
                                                const float *__restrict__ vsum, float *__restrict__ ws,
                                                uint16_t *__restrict__ HbT) {
  using C = HbarCfg<D, BS>;
  constexpr int NE = C::NE, TPW = C::TPW, TILE = C::TILE, CPW = C::CPW;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, l = tid & 63, lq = l & 31, hl = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrun = (dm.n_blk + kHbarRun - 1) / kHbarRun;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);   // a head's runs share an XCD
  const int run = logical % nrun, bh = logical / nrun;
  const int j0 = run * kHbarRun, j1 = min(dm.n_blk, j0 + kHbarRun);
  const int et = (w * TPW) / NE;                           // this wave's e tile
  const int ct0 = (w * TPW) % NE;                          // and its first c tile
  const size_t base = (size_t)bh * dm.L * D;
  const uint16_t *Kb = K + base, *Vb = V + base;
  const float *kb = kbar + (size_t)bh * dm.n_blk * D;
  const float *vs = vsum + (size_t)bh * dm.n_blk * D;
  int off[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int pos = (w + 4 * u) * 64 + l;
    const int row = pos / (D / 8), phys = pos % (D / 8);
    off[u] = (row * D + ((phys ^ vswz<D>(row)) << 3)) * 2;
  }
  auto dma = [&](int j) {
    const int k0 = j * BS, bytes = max(dm.L - k0, 0) * D * 2;   // past the last key: zeros
    uint8_t *dk = lds + ((j - j0) & 1) * 2 * TILE, *dv = dk + TILE;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      dma16_buf(Kb + (size_t)k0 * D, bytes, off[u], dk + (w + 4 * u) * 1024);
      dma16_buf(Vb + (size_t)k0 * D, bytes, off[u], dv + (w + 4 * u) * 1024);
    }
  };
  // accumulator entries of this lane: column c = 32 ct + lq, rows
  // e = 32 et + 8 g + 4 hl + q at register 4 g + q
  auto ldstat = [&](int j, float (&k1)[TPW], f32x4_t (&v4)[4]) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) k1[i] = kb[(size_t)j * D + (ct0 + i) * 32 + lq];
#pragma unroll
    for (int g = 0; g < 4; ++g) v4[g] = *reinterpret_cast<const f32x4_t *>(vs + (size_t)j * D + et * 32 + 8 * g + 4 * hl);
  };
  const int srow = (l & 15) >> 2, ecol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  f32x16_t tot[TPW];
  float *runp = ws + ((size_t)bh * nrun + run) * D * D;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (PREFIX) {   // the exclusive prefix sum of the earlier runs
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          tot[i][4 * g + q] = runp[(size_t)(et * 32 + 8 * g + 4 * hl + q) * D + (ct0 + i) * 32 + lq];
    } else {
      tot[i] = f32x16_t{};
    }
  }
  float ck[TPW];
  f32x4_t cv[4];
  ldstat(j0, ck, cv);
  dma(j0);
  for (int j = j0; j < j1; ++j) {
    wait_vmcnt<0>();
    __syncthreads();   // block j landed for every wave; the other slot is free
    float nk[TPW] = {};
    f32x4_t nv[4] = {};
    if (j + 1 < j1) {
      ldstat(j + 1, nk, nv);
      dma(j + 1);
    }
    if (PREFIX) {   // HbarT(lo = j): the mean over blocks [0, j)
      uint16_t *dst = HbT + ((size_t)bh * dm.n_blk + j) * D * D;
      const float inv = j > 0 ? 1.f / (float)j : 0.f;
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[(size_t)(et * 32 + 8 * g + 4 * hl + q) * D + (ct0 + i) * 32 + lq] =
                (uint16_t)f32_to_bf16(j > 0 ? tot[i][4 * g + q] * inv : 0.f);
      if (j + 1 == dm.n_blk) break;   // no row has lo = n_blk
    }
    const uint8_t *kt = lds + ((j - j0) & 1) * 2 * TILE, *vt = kt + TILE;
    f32x16_t r[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) r[i] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < BS / 16; ++s) {
      const int r1 = 16 * s + 4 * hl + srow;
      const u32x4_t av = frag_vt<D>(vt, r1, et * 32 + ecol);
#pragma unroll
      for (int i = 0; i < TPW; ++i) r[i] = mfma32(av, frag_vt<D>(kt, r1, (ct0 + i) * 32 + ecol), r[i]);
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[i][4 * g + q] += r[i][4 * g + q] - cv[g][q] * ck[i];
#pragma unroll
    for (int i = 0; i < TPW; ++i) ck[i] = nk[i];
#pragma unroll
    for (int g = 0; g < 4; ++g) cv[g] = nv[g];
  }
  if (PREFIX) return;
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        runp[(size_t)(et * 32 + 8 * g + 4 * hl + q) * D + (ct0 + i) * 32 + lq] = tot[i][4 * g + q];
}

// causal rows: the run sums of a (b, kv head) become exclusive prefix sums
__global__ __launch_bounds__(256) void hbar_scan(PisaDims dm, float *__restrict__ ws) {
  const int DD = dm.d * dm.d;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)dm.B * dm.Hkv * DD) return;
  const int nrun = (dm.n_blk + kHbarRun - 1) / kHbarRun;
  float *p = ws + (size_t)(gid / DD) * nrun * DD + (int)(gid % DD);
  float s = 0.f;
  for (int r = 0; r < nrun; ++r) {
    const float x = p[(size_t)r * DD];
    p[(size_t)r * DD] = s;
    s += x;
  }
}

// HbT (bf16, hybrid order) and hb32 (fp32 copy, routing): either may be null
__global__ __launch_bounds__(256) void hbar_final(PisaDims dm, const float *__restrict__ ws,
                                                  uint16_t *__restrict__ HbT, float *__restrict__ hb32) {
  const int DD = dm.d * dm.d;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)dm.B * dm.Hkv * DD) return;
  const int nrun = (dm.n_blk + kHbarRun - 1) / kHbarRun;
  const long long bh = gid / DD;
  const int o = (int)(gid % DD);
  const float *src = ws + (size_t)bh * nrun * DD + o;
  float s = 0.f;
  for (int r = 0; r < nrun; ++r) s += src[(size_t)r * DD];
  const float m = s / (float)dm.n_blk;
  if (HbT) HbT[gid] = (uint16_t)f32_to_bf16(m);
  if (hb32) hb32[gid] = m;
}

// ---------------------------------------------------------------------------
// Covariance-aware routing (PISA page, section 2): mcov_j = ||H_j - Hbar||_F.
// bf16: one workgroup of four waves per (b, kv head, run of kMcovRun blocks);
// H_j^T is formed as in hbar_run (raw MFMA moment minus sigma_j kbar_j^T, in
// fp32), Hbar^T (fp32) held in registers for the run, and the squared
// differences summed per lane, over the wave (fixed tree) and over the four
// waves in order.
constexpr int kMcovRun = 4;

template <int D, int BS>
__global__ __launch_bounds__(256) void mcov_bf16(PisaDims dm, const uint16_t *__restrict__ K,
                                                 const uint16_t *__restrict__ V,
                                                 const float *__restrict__ kbar,
                                                 const float *__restrict__ vsum,
                                                 const float *__restrict__ hb32, float *__restrict__ mcov) {
  using C = HbarCfg<D, BS>;
  constexpr int NE = C::NE, TPW = C::TPW, TILE = C::TILE, CPW = C::CPW;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *red = reinterpret_cast<float *>(lds + C::TOTAL);   // [4] per-wave sums
  const int tid = threadIdx.x, l = tid & 63, lq = l & 31, hl = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrun = (dm.n_blk + kMcovRun - 1) / kMcovRun;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int run = logical % nrun, bh = logical / nrun;
  const int j0 = run * kMcovRun, j1 = min(dm.n_blk, j0 + kMcovRun);
  const int et = (w * TPW) / NE, ct0 = (w * TPW) % NE;
  const size_t base = (size_t)bh * dm.L * D;
  const uint16_t *Kb = K + base, *Vb = V + base;
  const float *kb = kbar + (size_t)bh * dm.n_blk * D;
  const float *vs = vsum + (size_t)bh * dm.n_blk * D;
  float hb[TPW][16];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        hb[i][4 * g + q] = hb32[(size_t)bh * D * D + (size_t)(et * 32 + 8 * g + 4 * hl + q) * D + (ct0 + i) * 32 + lq];
  int off[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int pos = (w + 4 * u) * 64 + l;
    const int row = pos / (D / 8), phys = pos % (D / 8);
    off[u] = (row * D + ((phys ^ vswz<D>(row)) << 3)) * 2;
  }
  auto dma = [&](int j) {
    const int k0 = j * BS, bytes = max(dm.L - k0, 0) * D * 2;
    uint8_t *dk = lds + ((j - j0) & 1) * 2 * TILE, *dv = dk + TILE;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      dma16_buf(Kb + (size_t)k0 * D, bytes, off[u], dk + (w + 4 * u) * 1024);
      dma16_buf(Vb + (size_t)k0 * D, bytes, off[u], dv + (w + 4 * u) * 1024);
    }
  };
  const int srow = (l & 15) >> 2, ecol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  dma(j0);
  for (int j = j0; j < j1; ++j) {
    wait_vmcnt<0>();
    __syncthreads();   // block j landed; the other slot and red are free
    if (j + 1 < j1) dma(j + 1);
    float ck[TPW];
    f32x4_t cv[4];
#pragma unroll
    for (int i = 0; i < TPW; ++i) ck[i] = kb[(size_t)j * D + (ct0 + i) * 32 + lq];
#pragma unroll
    for (int g = 0; g < 4; ++g) cv[g] = *reinterpret_cast<const f32x4_t *>(vs + (size_t)j * D + et * 32 + 8 * g + 4 * hl);
    const uint8_t *kt = lds + ((j - j0) & 1) * 2 * TILE, *vt = kt + TILE;
    f32x16_t r[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) r[i] = f32x16_t{};
#pragma unroll
    for (int st = 0; st < BS / 16; ++st) {
      const int r1 = 16 * st + 4 * hl + srow;
      const u32x4_t av = frag_vt<D>(vt, r1, et * 32 + ecol);
#pragma unroll
      for (int i = 0; i < TPW; ++i) r[i] = mfma32(av, frag_vt<D>(kt, r1, (ct0 + i) * 32 + ecol), r[i]);
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float h = r[i][4 * g + q] - cv[g][q] * ck[i] - hb[i][4 * g + q];
          ss = fmaf(h, h, ss);
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    if (l == 0) red[w] = ss;
    __syncthreads();
    if (tid == 0) mcov[(size_t)bh * dm.n_blk + j] = sqrtf(((red[0] + red[1]) + red[2]) + red[3]);
  }
}

// fp32: one workgroup per (b, kv head, block), each thread D * D / 256 entries
template <int D, int BS>
__global__ __launch_bounds__(kStatsThreads) void mcov_f32(PisaDims dm, const float *__restrict__ K,
                                                          const float *__restrict__ V,
                                                          const float *__restrict__ kbar,
                                                          const float *__restrict__ vsum,
                                                          const float *__restrict__ hb32, float *__restrict__ mcov) {
  __shared__ float red[kStatsThreads];
  const int j = blockIdx.x % dm.n_blk, bh = blockIdx.x / dm.n_blk;
  const int t0 = j * BS, t1 = min(dm.L, t0 + BS);
  const float *Kb = K + (size_t)bh * dm.L * D, *Vb = V + (size_t)bh * dm.L * D;
  const float *kb = kbar + ((size_t)bh * dm.n_blk + j) * D, *vs = vsum + ((size_t)bh * dm.n_blk + j) * D;
  const float *hb = hb32 + (size_t)bh * D * D;
  float ss = 0.f;
  for (int o = threadIdx.x; o < D * D; o += kStatsThreads) {
    const int e = o / D, c = o % D;
    float r = 0.f;
    for (int t = t0; t < t1; ++t) r = fmaf(Vb[(size_t)t * D + e], Kb[(size_t)t * D + c], r);
    const float h = r - vs[e] * kb[c] - hb[o];
    ss = fmaf(h, h, ss);
  }
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int n = kStatsThreads / 2; n > 0; n >>= 1) {
    if ((int)threadIdx.x < n) red[threadIdx.x] += red[threadIdx.x + n];
    __syncthreads();
  }
  if (threadIdx.x == 0) mcov[(size_t)bh * dm.n_blk + j] = sqrtf(red[0]);
}

// fp32: one thread per (e, c), the same order of operations on the VALU.
template <int D, int BS>
__global__ __launch_bounds__(kStatsThreads) void hbar_f32(PisaDims dm, const float *__restrict__ K,
                                                          const float *__restrict__ V,
                                                          const float *__restrict__ kbar,
                                                          const float *__restrict__ vsum,
                                                          float *__restrict__ HbT, float *__restrict__ hb32) {
  constexpr int PER = D * D / kStatsThreads;
  const int bh = blockIdx.x / PER;
  const int o = (blockIdx.x % PER) * kStatsThreads + threadIdx.x;
  const int e = o / D, c = o % D;
  const float *Kb = K + (size_t)bh * dm.L * D, *Vb = V + (size_t)bh * dm.L * D;
  const float *kb = kbar + (size_t)bh * dm.n_blk * D, *vs = vsum + (size_t)bh * dm.n_blk * D;
  float tot = 0.f;
  const bool prefix = dm.causal != 0;   // one mean per lo, over blocks [0, lo)
  for (int j = 0; j < dm.n_blk; ++j) {
    if (prefix && HbT) {
      HbT[((size_t)bh * dm.n_blk + j) * D * D + o] = j > 0 ? tot / (float)j : 0.f;
      if (j + 1 == dm.n_blk) return;
    }
    const int t1 = min(dm.L, (j + 1) * BS);
    float r = 0.f;
    for (int t = j * BS; t < t1; ++t) r = fmaf(Vb[(size_t)t * D + e], Kb[(size_t)t * D + c], r);
    tot += r - vs[(size_t)j * D + e] * kb[(size_t)j * D + c];
  }
  if (prefix) return;
  const float m = tot / (float)dm.n_blk;
  if (HbT) HbT[(size_t)bh * D * D + o] = m;
  if (hb32) hb32[(size_t)bh * D * D + o] = m;
}

// Hbar (hybrid order and/or routing), then the covariance norms (routing)
template <int D, int BS>
hipError_t launch_hbar(const PisaDims &dm, const void *K, const void *V, const float *kbar, const float *vsum,
                       void *HT, float *mcov, void *ws, hipStream_t st) {
  const bool hybrid = dm.taylor == 3, route = dm.route_lambda > 0.f;
  float *hb32 = route ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + hbar_runs_bytes(dm)) : nullptr;
  const long long n = (long long)dm.B * dm.Hkv * D * D;
  if (dm.dtype == 0) {
    using C = HbarCfg<D, BS>;
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&hbar_run<D, BS, false>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::TOTAL);
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&hbar_run<D, BS, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::TOTAL);
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mcov_bf16<D, BS>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::TOTAL + 16);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    const int nrun = (dm.n_blk + kHbarRun - 1) / kHbarRun;
    const unsigned rgrid = (unsigned)dm.B * dm.Hkv * nrun;
    hbar_run<D, BS, false><<<rgrid, 256, C::TOTAL, st>>>(dm, static_cast<const uint16_t *>(K),
                                                         static_cast<const uint16_t *>(V), kbar, vsum,
                                                         static_cast<float *>(ws), nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dm.causal) {   // hybrid order only (routing is non-causal): one mean per lo
      hbar_scan<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(dm, static_cast<float *>(ws));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      hbar_run<D, BS, true><<<rgrid, 256, C::TOTAL, st>>>(dm, static_cast<const uint16_t *>(K),
                                                          static_cast<const uint16_t *>(V), kbar, vsum,
                                                          static_cast<float *>(ws), static_cast<uint16_t *>(HT));
      return hipGetLastError();
    }
    hbar_final<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(dm, static_cast<const float *>(ws),
                                                             hybrid ? static_cast<uint16_t *>(HT) : nullptr, hb32);
    if (route) {
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int nmr = (dm.n_blk + kMcovRun - 1) / kMcovRun;
      mcov_bf16<D, BS><<<(unsigned)dm.B * dm.Hkv * nmr, 256, C::TOTAL + 16, st>>>(
          dm, static_cast<const uint16_t *>(K), static_cast<const uint16_t *>(V), kbar, vsum, hb32, mcov);
    }
  } else {
    const unsigned grid = (unsigned)dm.B * dm.Hkv * (D * D / kStatsThreads);
    hbar_f32<D, BS><<<grid, kStatsThreads, 0, st>>>(dm, static_cast<const float *>(K),
                                                    static_cast<const float *>(V), kbar, vsum,
                                                    hybrid ? static_cast<float *>(HT) : nullptr, hb32);
    if (route) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      mcov_f32<D, BS><<<(unsigned)dm.B * dm.Hkv * dm.n_blk, kStatsThreads, 0, st>>>(
          dm, static_cast<const float *>(K), static_cast<const float *>(V), kbar, vsum, hb32, mcov);
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// query pooling: one thread per (selection row, 16-byte chunk of the row)
template <typename T, int D>
__global__ __launch_bounds__(kStatsThreads) void q_pool(PisaDims dm, const T *__restrict__ Q, T *__restrict__ qsel) {
  constexpr int EPC = 16 / sizeof(T);  // elements per chunk
  constexpr int CPR = D / EPC;         // chunks per row
  const long long gid = (long long)blockIdx.x * kStatsThreads + threadIdx.x;
  const long long total = (long long)dm.B * dm.Hq * dm.n_sel * CPR;
  if (gid >= total) return;
  const int ch = (int)(gid % CPR);
  const long long sr = gid / CPR;          // (b*Hq + h) * n_sel + r
  const int r = (int)(sr % dm.n_sel);
  const long long bh = sr / dm.n_sel;
  const int span = dm.group >= 1 ? dm.group : dm.bs;
  const int t0 = r * span, t1 = min(dm.L, t0 + span);
  const T *src = Q + ((size_t)bh * dm.L) * D + ch * EPC;
  DD acc[EPC];
#pragma unroll
  for (int i = 0; i < EPC; ++i) acc[i] = DD{0.0, 0.0};
  for (int t = t0; t < t1; ++t) {
    u32x4_t w = *reinterpret_cast<const u32x4_t *>(src + (size_t)t * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (sizeof(T) == 2) {
        dd_add(acc[2 * i], (double)bf16lo(w[i]));
        dd_add(acc[2 * i + 1], (double)bf16hi(w[i]));
      } else {
        dd_add(acc[i], (double)__uint_as_float(w[i]));
      }
    }
  }
  const double cnt = (double)(t1 - t0);
  u32x4_t out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 2) {
      uint32_t lo = f64_to_bf16_bits(dd_value(acc[2 * i]) / cnt);
      uint32_t hi = f64_to_bf16_bits(dd_value(acc[2 * i + 1]) / cnt);
      out[i] = lo | (hi << 16);
    } else {
      out[i] = __float_as_uint((float)round_to_format(dd_value(acc[i]) / cnt, 24));
    }
  }
  *reinterpret_cast<u32x4_t *>(qsel + (size_t)sr * D + ch * EPC) = out;
}

// One wave per query block, four blocks per workgroup: lane (chunk ch, slice
// ts) loads rows ts, ts + SPW, ... of its block up front and sums them
// (certified float64 for bf16, double-double where the certificate fails or
// for fp32); the SPW slices of a chunk then merge by lane shuffles with
// exact double-double additions, and the first slice writes the means.
template <typename T, int D, int BS>
__global__ __launch_bounds__(kStatsThreads) void q_pool_wave(PisaDims dm, const T *__restrict__ Q,
                                                            T *__restrict__ qsel) {
  constexpr int EPC = 16 / sizeof(T);          // elements per chunk
  constexpr int CPR = D / EPC;                 // chunks per row
  constexpr int SPW = 64 / CPR;                // row slices per wave
  constexpr int RPS = BS / SPW;                // rows per slice
  static_assert(SPW * CPR == 64 && RPS * SPW == BS, "one block per wave");
  const int l = threadIdx.x & 63, ch = l % CPR, ts = l / CPR;
  const long long blk = (long long)blockIdx.x * (kStatsThreads / 64) + (threadIdx.x >> 6);
  if (blk >= (long long)dm.B * dm.Hq * dm.n_sel) return;   // whole waves
  const int r = (int)(blk % dm.n_sel);
  const long long bh = blk / dm.n_sel;
  const int t0 = r * dm.bs, t1 = min(dm.L, t0 + dm.bs);
  const T *src = Q + ((size_t)bh * dm.L) * D + ch * EPC;
  // rows in batches of RB per lane, each batch loaded up front
  constexpr int RB = RPS < 16 / (int)sizeof(T) * 2 ? RPS : 16 / (int)sizeof(T) * 2;   // 16 bf16, 8 fp32
  DD acc[EPC];
#pragma unroll
  for (int i = 0; i < EPC; ++i) acc[i] = DD{0.0, 0.0};
  for (int k0 = 0; k0 < RPS; k0 += RB) {
    u32x4_t w[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int t = t0 + ts + (k0 + k) * SPW;
      w[k] = t < t1 ? *reinterpret_cast<const u32x4_t *>(src + (size_t)t * D) : u32x4_t{0, 0, 0, 0};
    }
    if constexpr (sizeof(T) == 2) {
      // the batch's sums in float64, exact when certified; double-double
      // additions otherwise
      constexpr int LG = RB <= 4 ? 2 : RB <= 8 ? 3 : 4;
      double sm[EPC];
      SpanCert cert[4];
#pragma unroll
      for (int i = 0; i < EPC; ++i) sm[i] = 0.0;
#pragma unroll
      for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm[2 * i] += (double)bf16lo(w[k][i]);
          sm[2 * i + 1] += (double)bf16hi(w[k][i]);
          cert[i].add(w[k][i]);
        }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (cert[i].exact(h, LG)) {
            dd_add(acc[2 * i + h], sm[2 * i + h]);
          } else {
#pragma unroll
            for (int k = 0; k < RB; ++k) dd_add(acc[2 * i + h], (double)(h ? bf16hi(w[k][i]) : bf16lo(w[k][i])));
          }
        }
    } else {
#pragma unroll
      for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) dd_add(acc[i], (double)__uint_as_float(w[k][i]));
    }
  }
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
    for (int i = 0; i < EPC; ++i) {
      const DD x = {__shfl_xor(acc[i].hi, o), __shfl_xor(acc[i].lo, o)};
      dd_merge(acc[i], x);
    }
  if (ts == 0) {
    const double inv_n = (double)(t1 - t0);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (sizeof(T) == 2) {
        const uint32_t lo = f64_to_bf16_bits(dd_value(acc[2 * i]) / inv_n);
        const uint32_t hi = f64_to_bf16_bits(dd_value(acc[2 * i + 1]) / inv_n);
        o[i] = lo | (hi << 16);
      } else {
        o[i] = __float_as_uint((float)round_to_format(dd_value(acc[i]) / inv_n, 24));
      }
    }
    *reinterpret_cast<u32x4_t *>(qsel + ((size_t)bh * dm.n_sel + r) * D + ch * EPC) = o;
  }
}

template <typename T, int D>
hipError_t launch_q_pool(const PisaDims &dm, const void *Q, void *qsel, hipStream_t st) {
  if (dm.group == 0) {   // query blocks of 64 or 128 rows, one per wave
    const long long nblk = (long long)dm.B * dm.Hq * dm.n_sel;
    const unsigned grid = (unsigned)((nblk + kStatsThreads / 64 - 1) / (kStatsThreads / 64));
    if (dm.bs == 64) q_pool_wave<T, D, 64><<<grid, kStatsThreads, 0, st>>>(dm, static_cast<const T *>(Q),
                                                                          static_cast<T *>(qsel));
    else q_pool_wave<T, D, 128><<<grid, kStatsThreads, 0, st>>>(dm, static_cast<const T *>(Q),
                                                                static_cast<T *>(qsel));
    return hipGetLastError();
  }
  constexpr int CPR = D / (16 / sizeof(T));
  const long long total = (long long)dm.B * dm.Hq * dm.n_sel * CPR;
  const unsigned grid = (unsigned)((total + kStatsThreads - 1) / kStatsThreads);
  q_pool<T, D><<<grid, kStatsThreads, 0, st>>>(dm, static_cast<const T *>(Q), static_cast<T *>(qsel));
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_kv_bf16(const PisaDims &dm, const void *K, const void *V, void *ksel, float *kbar,
                          float *vsum, void *HT, hipStream_t st) {
  using C = KvCfg<D, BS>;
  const unsigned grid = (unsigned)dm.B * dm.Hkv * dm.n_blk;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kv_stats_bf16<D, BS>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::TOTAL);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kv_stats_bf16<D, BS><<<grid, kKvThreads, C::TOTAL, st>>>(
      dm, static_cast<const uint16_t *>(K), static_cast<const uint16_t *>(V), static_cast<uint16_t *>(ksel),
      kbar, vsum, static_cast<uint16_t *>(HT));
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_kv_f32(const PisaDims &dm, const void *K, const void *V, void *ksel, float *kbar,
                         float *vsum, void *HT, hipStream_t st) {
  const unsigned grid = (unsigned)dm.B * dm.Hkv * dm.n_blk;
  kv_stats_f32<D, BS><<<grid, kStatsThreads, 0, st>>>(dm, static_cast<const float *>(K),
                                                      static_cast<const float *>(V), static_cast<float *>(ksel),
                                                      kbar, vsum, static_cast<float *>(HT));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_stats(const PisaDims &dm, const void *Q, const void *K, const void *V, void *qsel,
                              void *ksel, float *kbar, float *vsum, void *HT, float *mcov, void *ws,
                              hipStream_t st) {
  hipError_t e;
  const bool bf = dm.dtype == 0;
  if (bf) {
    if (dm.d == 64) e = dm.bs == 64 ? launch_kv_bf16<64, 64>(dm, K, V, ksel, kbar, vsum, HT, st)
                                    : launch_kv_bf16<64, 128>(dm, K, V, ksel, kbar, vsum, HT, st);
    else e = dm.bs == 64 ? launch_kv_bf16<128, 64>(dm, K, V, ksel, kbar, vsum, HT, st)
                         : launch_kv_bf16<128, 128>(dm, K, V, ksel, kbar, vsum, HT, st);
  } else {
    if (dm.d == 64) e = dm.bs == 64 ? launch_kv_f32<64, 64>(dm, K, V, ksel, kbar, vsum, HT, st)
                                    : launch_kv_f32<64, 128>(dm, K, V, ksel, kbar, vsum, HT, st);
    else e = dm.bs == 64 ? launch_kv_f32<128, 64>(dm, K, V, ksel, kbar, vsum, HT, st)
                         : launch_kv_f32<128, 128>(dm, K, V, ksel, kbar, vsum, HT, st);
  }
  if (e != hipSuccess) return e;
  if (needs_hbar(dm)) {   // the mean first-order matrix (and covariance norms), after kbar and vsum
    if (dm.d == 64) e = dm.bs == 64 ? launch_hbar<64, 64>(dm, K, V, kbar, vsum, HT, mcov, ws, st)
                                    : launch_hbar<64, 128>(dm, K, V, kbar, vsum, HT, mcov, ws, st);
    else e = dm.bs == 64 ? launch_hbar<128, 64>(dm, K, V, kbar, vsum, HT, mcov, ws, st)
                         : launch_hbar<128, 128>(dm, K, V, kbar, vsum, HT, mcov, ws, st);
    if (e != hipSuccess) return e;
  }
  if (bf) return dm.d == 64 ? launch_q_pool<uint16_t, 64>(dm, Q, qsel, st) : launch_q_pool<uint16_t, 128>(dm, Q, qsel, st);
  return dm.d == 64 ? launch_q_pool<float, 64>(dm, Q, qsel, st) : launch_q_pool<float, 128>(dm, Q, qsel, st);
}
