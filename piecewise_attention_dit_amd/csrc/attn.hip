// Stage C: exact online-softmax attention over the kept blocks, fused with the
// per-block first-order Taylor tail for every other candidate block.
//
// PISA page, section 2: o_t = N_t / D_t; exact terms e^{q k} v over the
// selected blocks; for a non-selected block j, alpha = e^{q . kbar_j} times
// (sum of its values + q H_j) in N_t and alpha * n_j in D_t, so that the
// approximation sits inside both numerator and denominator.  Hardware
// implementation section: one fused online-softmax kernel, selected blocks
// staged on chip, pooled statistics scanned for the rest.  Sliding Window
// Attention page, related term "FlashAttention": blocks outside the kept set
// are never touched.
//
// bf16 kernel (MFMA 32x32x16, gfx950):
//   workgroup = NW waves; a wave owns NQ tiles of 32 consecutive query rows of
//   one head (NQ = 2 lets every LDS operand fragment feed two MFMAs); the
//   workgroup's heads share one KV head (GQA), so each staged K / V / H tile
//   serves all of them.  Everything is computed transposed so that a lane
//   always owns one query (lane % 32) per tile:
//     S^T  = K   Q^T         A = K tile (LDS),    B = Q (registers)
//     O^T += V^T P^T         A = V^T tile (LDS),  B = P (registers, bf16)
//     a^T  = Kbar Q^T        (Taylor logits, kbar split into bf16 hi + lo)
//     O^T += Sig^T alpha^T   (zero order, hi/lo splits)
//     T    = H_j^T Q^T, O^T += alpha_j * scale * T   (first order, per block)
//   The workgroup walks the union of its rows' kept blocks (exact phase) and
//   then the union of their Taylor blocks, 32 per batch; a wave (or a query
//   tile) skips a block none of its rows uses; per-row masks handle rows that
//   differ within a tile (PIVOT per-token lists).
#include "device_common.h"

namespace {

struct AttnArgs {
  PisaDims dm;
  const void *Q, *K, *V;
  const float *kbar, *vsum;
  const void *HT;
  const int32_t *idx;
  void *O;
  float *lse;
  float sl2;  // scale * log2(e)
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTyBatch = 32;
constexpr float kNegInf = -__builtin_huge_valf();
// The running max of a row moves only when a new logit exceeds it by more
// than kRescale (log2 units): probabilities then stay below 2^kRescale, far
// inside the fp32 / bf16 range, and the output accumulators are rescaled
// rarely (they live in accumulation registers that only MFMAs touch).
constexpr float kRescale = 8.f;

// Position of key x inside its 16-key group of a transposed V (and Sigma)
// tile: keys 4-7 and 8-11 trade places (bits 2 and 3 swap), so that the S^T
// accumulator layout (lane half hl holds keys {0-3, 8-11} or {4-7, 12-15} of
// each 16) is directly the B operand of the PV product.
PISA_DEV int perm16(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

constexpr int kStage = 64;   // keys per pipeline stage (a block is 1 or 2 stages)

// Row-major tiles (K stages, H_j^T, kbar hi/lo) use a padded pitch of
// D * 2 + 16 bytes: eight consecutive rows start 16 bytes apart modulo the
// bank width, so the 8-lane groups of a ds_read_b128 never collide, and every
// fragment address is one per-lane base plus an immediate offset.
template <int D>
constexpr int row_pitch() { return D * 2 + 16; }

template <int D, int BS, int NW, int NQ>
struct Lds {
  static constexpr int PR = row_pitch<D>();
  static constexpr int K_BYTES = kStage * PR;
  static constexpr int VT_BYTES = D * kStage * 2;
  static constexpr int EX_K0 = 0;
  static constexpr int EX_V0 = 2 * K_BYTES;
  static constexpr int EX_END = 2 * K_BYTES + 2 * VT_BYTES;
  // Taylor phase (overlays the exact phase)
  static constexpr int KB_BYTES = kTyBatch * PR;
  static constexpr int ST_BYTES = D * kTyBatch * 2;
  static constexpr int TY_KBH = 0;
  static constexpr int TY_KBL = TY_KBH + KB_BYTES;
  static constexpr int TY_STH = TY_KBL + KB_BYTES;
  static constexpr int TY_STL = TY_STH + ST_BYTES;
  static constexpr int TY_ALPHA = TY_STL + ST_BYTES;
  static constexpr int ALPHA_PER_WAVE = kTyBatch * NQ * 32;   // floats
  static constexpr int TY_H0 = TY_ALPHA + NW * ALPHA_PER_WAVE * 4;
  static constexpr int H_BYTES = D * PR;
  static constexpr int TY_NJ = TY_H0 + 2 * H_BYTES;
  static constexpr int TY_END = TY_NJ + kTyBatch * 4;
  static constexpr int MAIN = EX_END > TY_END ? EX_END : TY_END;
  static constexpr int EXL = MAIN;              // union lists (uint16) and bitmaps
  static constexpr int TYL = EXL + 1024 * 2;
  static constexpr int EXB = TYL + 1024 * 2;
  static constexpr int TYB = EXB + 32 * 4;
  static constexpr int CNT = TYB + 32 * 4;
  static constexpr int TOTAL = CNT + 16;
};

// ---------------------------------------------------------------------------
// per-row helpers

struct RowInfo {
  int t;                 // token
  bool valid;            // t < L
  int own, lo, nc;       // own block, window start block, candidate count
  const int32_t *list;   // kept list (ascending, -1 padded), topk entries
};

PISA_DEV bool list_has(const RowInfo &r, int topk, int &ptr, int j) {
  while (ptr < topk) {
    const int v = r.list[ptr];
    if (v < 0 || v > j) return false;
    if (v == j) return true;
    ++ptr;
  }
  return false;
}

// ---------------------------------------------------------------------------
// staging helpers (global -> registers -> LDS with XOR swizzles)

template <int D, int BS, int NT>
struct KVRegs {
  static constexpr int KCH = BS * D / 8;                    // 16-byte chunks of a K tile
  static constexpr int KPT = (KCH + NT - 1) / NT;
  static constexpr int VU = (BS / 4) * (D / 8);             // V units: 4 keys x 8 features
  static constexpr int VPT = (VU + NT - 1) / NT;
  u32x4_t k[KPT];
  u32x4_t v[VPT][4];
};

template <int D, int BS, int NT>
PISA_DEV void k_load(KVRegs<D, BS, NT> &r, const uint16_t *Kb, int nkeys, int tid) {
  using R = KVRegs<D, BS, NT>;
#pragma unroll
  for (int i = 0; i < R::KPT; ++i) {
    const int u = tid + i * NT;
    const int key = u / (D / 8), ch = u % (D / 8);
    const int kc = min(key, nkeys - 1);    // clamped address, zero-filled below
    const u32x4_t x = *reinterpret_cast<const u32x4_t *>(Kb + (size_t)kc * D + ch * 8);
    const bool ok = (R::KCH % NT == 0 || u < R::KCH) && key < nkeys;
    r.k[i] = ok ? x : u32x4_t{0, 0, 0, 0};
  }
}

template <int D, int BS, int NT>
PISA_DEV void k_store(const KVRegs<D, BS, NT> &r, uint8_t *kl, int tid) {
  using R = KVRegs<D, BS, NT>;
#pragma unroll
  for (int i = 0; i < R::KPT; ++i) {
    const int u = tid + i * NT;
    if (u < R::KCH) {
      const int key = u / (D / 8), ch = u % (D / 8);
      *reinterpret_cast<u32x4_t *>(kl + key * row_pitch<D>() + (ch << 4)) = r.k[i];
    }
  }
}

// V is stored transposed: row e (feature), key positions permuted by perm16,
// 16-byte chunks XOR-swizzled with ((e & 7) ^ (e >> 3)).
template <int D, int BS, int NT>
PISA_DEV void v_load(KVRegs<D, BS, NT> &r, const uint16_t *Vb, int nkeys, int tid) {
  using R = KVRegs<D, BS, NT>;
#pragma unroll
  for (int i = 0; i < R::VPT; ++i) {
    const int u = tid + i * NT;
    const int ec = u % (D / 8), q4 = u / (D / 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int key = 4 * q4 + k;
      const int kc = min(min(key, nkeys - 1), BS - 1);
      const u32x4_t x = *reinterpret_cast<const u32x4_t *>(Vb + (size_t)kc * D + ec * 8);
      const bool ok = (R::VU % NT == 0 || u < R::VU) && key < nkeys;
      r.v[i][k] = ok ? x : u32x4_t{0, 0, 0, 0};
    }
  }
}

template <int D, int BS, int NT>
PISA_DEV void v_store(const KVRegs<D, BS, NT> &r, uint8_t *vl, int tid) {
  using R = KVRegs<D, BS, NT>;
#pragma unroll
  for (int i = 0; i < R::VPT; ++i) {
    const int u = tid + i * NT;
    if (u >= R::VU) continue;
    const int ec = u % (D / 8), q4 = u / (D / 8);
    const int k0 = 4 * q4;
    const int pos = (k0 & ~15) + perm16(k0 & 15);
    const int chunk = pos >> 3, half = (pos >> 2) & 1;
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int e = ec * 8 + f;
      const int sh = (f & 1) * 16;
      const uint32_t a0 = (r.v[i][0][f >> 1] >> sh) & 0xFFFFu, a1 = (r.v[i][1][f >> 1] >> sh) & 0xFFFFu;
      const uint32_t a2 = (r.v[i][2][f >> 1] >> sh) & 0xFFFFu, a3 = (r.v[i][3][f >> 1] >> sh) & 0xFFFFu;
      const int phys = chunk ^ (((e & 7) ^ (e >> 3)) & (BS / 8 - 1));
      *reinterpret_cast<u32x2_t *>(vl + e * (BS * 2) + (phys << 4) + (half << 3)) =
          u32x2_t{a0 | (a1 << 16), a2 | (a3 << 16)};
    }
  }
}

template <int D, int NT>
struct HRegs {
  static constexpr int PT = D * D / 8 / NT;
  u32x4_t h[PT];
};

template <int D, int NT>
PISA_DEV void h_load(HRegs<D, NT> &r, const uint16_t *Hb, int tid) {
#pragma unroll
  for (int i = 0; i < HRegs<D, NT>::PT; ++i) r.h[i] = *reinterpret_cast<const u32x4_t *>(Hb + (size_t)(tid + i * NT) * 8);
}

template <int D, int NT>
PISA_DEV void h_store(const HRegs<D, NT> &r, uint8_t *hl, int tid) {
#pragma unroll
  for (int i = 0; i < HRegs<D, NT>::PT; ++i) {
    const int u = tid + i * NT;
    const int e = u / (D / 8), ch = u % (D / 8);
    *reinterpret_cast<u32x4_t *>(hl + e * row_pitch<D>() + (ch << 4)) = r.h[i];
  }
}

// A-operand fragments: lane reads 8 bf16 of row `row`, 16-byte chunk `ch`
template <int D>
PISA_DEV u32x4_t frag_rowmajor(const uint8_t *base, int row, int ch) {
  return *reinterpret_cast<const u32x4_t *>(base + row * row_pitch<D>() + (ch << 4));
}
template <int BS>
PISA_DEV u32x4_t frag_vt(const uint8_t *base, int e, int ch) {
  const int phys = ch ^ (((e & 7) ^ (e >> 3)) & (BS / 8 - 1));
  return *reinterpret_cast<const u32x4_t *>(base + e * (BS * 2) + (phys << 4));
}
PISA_DEV u32x4_t frag_st(const uint8_t *base, int e, int ch) {
  const int phys = ch ^ ((e >> 1) & 3);
  return *reinterpret_cast<const u32x4_t *>(base + e * 64 + (phys << 4));
}

PISA_DEV u32x4_t pack8(const f32x16_t &v, int off) {
  u32x4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[off + 2 * i], v[off + 2 * i + 1]);
  return w;
}

// ---------------------------------------------------------------------------

template <int D, int BS, int NW, int NQ>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16(AttnArgs a) {
  using LY = Lds<D, BS, NW, NQ>;
  constexpr int NT = NW * 64;
  constexpr int ROWS = NW * NQ * 32;
  constexpr int NE = D / 32;        // 32-feature output tiles
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const PisaDims &dm = a.dm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 31, hl = l >> 5;

  // ---- workgroup -> (b, kv head, head group, token tile); waves -> (head, tokens)
  const int hpw = dm.ratio < NW ? dm.ratio : NW;     // query heads per workgroup
  const int ngrp = dm.ratio / hpw;                   // head groups per KV head
  const int tpw = ROWS / hpw;                        // tokens per workgroup
  const int ntile = (dm.L + tpw - 1) / tpw;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = logical % ntile;
  const int rest = logical / ntile;
  const int grp = rest % ngrp;
  const int bk = rest / ngrp;                        // b * Hkv + hk
  const int b = bk / dm.Hkv, hk = bk % dm.Hkv;
  const int wph = NW / hpw;                          // waves per head
  const int h = hk * dm.ratio + grp * hpw + w / wph;
  const int tw = tile * tpw + (w % wph) * (NQ * 32);  // first token of the wave
  const bool pivot = dm.group >= 1;
  const int topk = dm.topk;
  const bool causal = dm.causal != 0;
  const int taylor = dm.taylor;

  RowInfo row[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    row[n].t = tw + n * 32 + lq;
    row[n].valid = row[n].t < dm.L;
    const int r = pivot ? row[n].t : row[n].t / dm.bs;
    const int start = pivot ? row[n].t : r * dm.bs;
    row[n].nc = pisa_row_geometry(dm, start, &row[n].own, &row[n].lo);
    row[n].list = a.idx ? a.idx + ((size_t)(b * dm.Hq + h) * dm.n_rows + r) * topk : nullptr;
  }

  uint32_t *exb = reinterpret_cast<uint32_t *>(lds + LY::EXB);
  uint32_t *tyb = reinterpret_cast<uint32_t *>(lds + LY::TYB);
  uint16_t *exl = reinterpret_cast<uint16_t *>(lds + LY::EXL);
  uint16_t *tyl = reinterpret_cast<uint16_t *>(lds + LY::TYL);
  int *cnt = reinterpret_cast<int *>(lds + LY::CNT);
  const int nwords = (dm.n_blk + 31) >> 5;

  // ---- 1. unions of the kept and Taylor block sets of the workgroup's rows
  for (int i = tid; i < 32; i += NT) {
    exb[i] = 0;
    tyb[i] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const RowInfo &rw = row[n];
    // block rows: one lane per wave speaks for all its rows (same list)
    const bool leader = rw.valid && (pivot ? hl == 0 : (l == 0 && n == 0));
    if (!leader) continue;
    for (int i = 0; i < topk; ++i) {
      const int j = rw.list[i];
      if (j < 0) break;
      atomicOr(&exb[j >> 5], 1u << (j & 31));
    }
    for (int j = rw.lo; j <= rw.own && j < dm.n_blk; ++j) atomicOr(&exb[j >> 5], 1u << (j & 31));
    if (taylor) {
      int ptr = 0;
      for (int wd = 0; wd * 32 < rw.nc; ++wd) {
        uint32_t bits = (rw.nc - wd * 32 >= 32) ? 0xFFFFFFFFu : ((1u << (rw.nc - wd * 32)) - 1u);
        while (ptr < topk) {
          const int j = rw.list[ptr];
          if (j < 0 || j >= (wd + 1) * 32) break;
          bits &= ~(1u << (j & 31));
          ++ptr;
        }
        if (bits) atomicOr(&tyb[wd], bits);
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    const uint32_t eb = l < nwords ? exb[l] : 0u, tb = l < nwords ? tyb[l] : 0u;
    const int ce = __popc(eb), ct = __popc(tb);
    const int ie = wave_incl_scan(ce), it = wave_incl_scan(ct);
    int pe = ie - ce, pt = it - ct;
    for (uint32_t m = eb; m; m &= m - 1) exl[pe++] = (uint16_t)(l * 32 + __ffs(m) - 1);
    for (uint32_t m = tb; m; m &= m - 1) tyl[pt++] = (uint16_t)(l * 32 + __ffs(m) - 1);
    if (l == 63) {
      cnt[0] = ie;
      cnt[1] = it;
    }
  }

  // ---- 2. Q fragments (B operand: query lq of tile n, features 16 ks + 8 hl .. + 7)
  const uint16_t *Qh = static_cast<const uint16_t *>(a.Q) + ((size_t)(b * dm.Hq + h) * dm.L) * D;
  u32x4_t qf[NQ][D / 16];
#pragma unroll
  for (int n = 0; n < NQ; ++n)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[n][ks] = row[n].valid ? *reinterpret_cast<const u32x4_t *>(Qh + (size_t)row[n].t * D + ks * 16 + hl * 8)
                               : u32x4_t{0, 0, 0, 0};
  __syncthreads();
  const int n_ex = cnt[0], n_ty = cnt[1];

  f32x16_t oacc[NQ][NE];
  float m_run[NQ], d_run[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    m_run[n] = kNegInf;
    d_run[n] = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i) oacc[n][i] = f32x16_t{};
  }
  const float sl2 = a.sl2;

  const size_t kvoff = ((size_t)(b * dm.Hkv + hk) * dm.L) * D;
  const uint16_t *Kh = static_cast<const uint16_t *>(a.K) + kvoff;
  const uint16_t *Vh = static_cast<const uint16_t *>(a.V) + kvoff;

  // ---- 3. exact phase over the union of kept blocks.  Blocks are walked as
  // 64-key stages, double-buffered in LDS; each stage is split into the
  // S^T / softmax part and the PV part, with the next stage's K fetched across
  // the first and its V across the second (16 prefetch registers live).
  constexpr int SPB = BS / kStage;   // stages per block
  using KV = KVRegs<D, kStage, NT>;
  if (n_ex > 0) {
    KV pre;
    {
      const int j = exl[0];
      const int nk = min(kStage, dm.L - j * BS);
      k_load<D, kStage, NT>(pre, Kh + (size_t)j * BS * D, nk, tid);
      k_store<D, kStage, NT>(pre, lds + LY::EX_K0, tid);
      v_load<D, kStage, NT>(pre, Vh + (size_t)j * BS * D, nk, tid);
      v_store<D, kStage, NT>(pre, lds + LY::EX_V0, tid);
    }
    __syncthreads();
    int ptr[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) ptr[n] = 0;
    bool mem[NQ];
    bool active = false;
    const int n_st = n_ex * SPB;
    for (int it = 0; it < n_st; ++it) {
      const int cur = it & 1;
      const int j = exl[it / SPB], kh = it % SPB;
      const bool has_next = it + 1 < n_st;
      const int jn = has_next ? exl[(it + 1) / SPB] : 0, khn = (it + 1) % SPB;
      const int key0n = jn * BS + khn * kStage;
      const int nkn = min(kStage, dm.L - key0n);
      if (has_next) k_load<D, kStage, NT>(pre, Kh + (size_t)key0n * D, nkn, tid);
      if (kh == 0) {
        bool any_mem = false;
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          const RowInfo &rw = row[n];
          mem[n] = rw.valid && ((j >= rw.lo && j <= rw.own) || (topk > 0 && list_has(rw, topk, ptr[n], j)));
          any_mem |= mem[n];
        }
        active = ballot64(any_mem) != 0;   // wave-uniform
      }
      const uint8_t *kl = lds + LY::EX_K0 + cur * LY::K_BYTES;
      const uint8_t *vl = lds + LY::EX_V0 + cur * LY::VT_BYTES;
      f32x16_t s[NQ][2];
      if (active) {
        // S^T for two 32-key tiles of the stage
#pragma unroll
        for (int n = 0; n < NQ; ++n)
#pragma unroll
          for (int q = 0; q < 2; ++q) s[n][q] = f32x16_t{};
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const u32x4_t af = frag_rowmajor<D>(kl, q * 32 + lq, 2 * ks + hl);
#pragma unroll
            for (int n = 0; n < NQ; ++n) s[n][q] = mfma32(af, qf[n][ks], s[n][q]);
            if ((ks & 1) == 1) __builtin_amdgcn_sched_barrier(0);
          }
        const int kbase = j * BS + kh * kStage;
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          float mloc = kNegInf;
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbase + q * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
              const bool ok = mem[n] && key < dm.L && (!causal || key <= row[n].t);
              const float x = ok ? s[n][q][r] * sl2 : kNegInf;
              s[n][q][r] = x;
              mloc = fmaxf(mloc, x);
            }
          mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
          const bool grow = mloc > m_run[n] + kRescale;   // includes the first visible block
          if (ballot64(grow)) {
            const float corr = grow ? exp2f(m_run[n] - mloc) : 1.f;
            d_run[n] *= corr;
#pragma unroll
            for (int et = 0; et < NE; ++et) oacc[n][et] *= corr;
            m_run[n] = grow ? mloc : m_run[n];
          }
          const float mref = m_run[n];
          float psum = 0.f;
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = mref == kNegInf ? 0.f : exp2f(s[n][q][r] - mref);
              s[n][q][r] = p;
              psum += p;
            }
          psum += __shfl_xor(psum, 32);
          d_run[n] += psum;
        }
      }
      if (has_next) {
        k_store<D, kStage, NT>(pre, lds + LY::EX_K0 + (cur ^ 1) * LY::K_BYTES, tid);
        v_load<D, kStage, NT>(pre, Vh + (size_t)key0n * D, nkn, tid);
      }
      if (active) {
        // O^T += V^T P^T
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            u32x4_t pb[NQ];
#pragma unroll
            for (int n = 0; n < NQ; ++n) pb[n] = pack8(s[n][q], 8 * hf);
#pragma unroll
            for (int et = 0; et < NE; ++et) {
              const u32x4_t vf = frag_vt<kStage>(vl, et * 32 + lq, q * 4 + hf * 2 + hl);
#pragma unroll
              for (int n = 0; n < NQ; ++n) oacc[n][et] = mfma32(vf, pb[n], oacc[n][et]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      if (has_next) v_store<D, kStage, NT>(pre, lds + LY::EX_V0 + (cur ^ 1) * LY::VT_BYTES, tid);
      __syncthreads();
    }
  }

  // ---- 4. Taylor phase over the union of Taylor blocks, kTyBatch at a time
  if (taylor && n_ty > 0) {
    const size_t soff = (size_t)(b * dm.Hkv + hk) * dm.n_blk;
    const float *kbar = a.kbar + soff * D;
    const float *vsum = a.vsum + soff * D;
    const uint16_t *HTh = static_cast<const uint16_t *>(a.HT) + soff * D * D;
    uint8_t *kbh = lds + LY::TY_KBH, *kbl = lds + LY::TY_KBL;
    uint8_t *sth = lds + LY::TY_STH, *stl = lds + LY::TY_STL;
    float *alpha = reinterpret_cast<float *>(lds + LY::TY_ALPHA) + w * LY::ALPHA_PER_WAVE;
    float *nj = reinterpret_cast<float *>(lds + LY::TY_NJ);
    const bool order1 = taylor == 2;
    int ptr[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) ptr[n] = 0;
    HRegs<D, NT> hpre;
    for (int b0 = 0; b0 < n_ty; b0 += kTyBatch) {
      const int nb = min(kTyBatch, n_ty - b0);
      // stage kbar (bf16 hi/lo rows), Sigma^T (bf16 hi/lo, permuted), n_j, first H
      for (int u = tid; u < kTyBatch * (D / 8); u += NT) {
        const int e = u / (D / 8), ch = u % (D / 8);
        u32x4_t hi = {0, 0, 0, 0}, lo = {0, 0, 0, 0};
        float sv[8];
        if (e < nb) {
          const int j = tyl[b0 + e];
          const f32x4_t x0 = *reinterpret_cast<const f32x4_t *>(kbar + (size_t)j * D + ch * 8);
          const f32x4_t x1 = *reinterpret_cast<const f32x4_t *>(kbar + (size_t)j * D + ch * 8 + 4);
          const f32x4_t v0 = *reinterpret_cast<const f32x4_t *>(vsum + (size_t)j * D + ch * 8);
          const f32x4_t v1 = *reinterpret_cast<const f32x4_t *>(vsum + (size_t)j * D + ch * 8 + 4);
          const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t p = pack_bf16x2(x[2 * i], x[2 * i + 1]);
            hi[i] = p;
            lo[i] = pack_bf16x2(x[2 * i] - bf16lo(p), x[2 * i + 1] - bf16hi(p));
          }
          sv[0] = v0[0]; sv[1] = v0[1]; sv[2] = v0[2]; sv[3] = v0[3];
          sv[4] = v1[0]; sv[5] = v1[1]; sv[6] = v1[2]; sv[7] = v1[3];
          if (ch == 0) nj[e] = (float)min(dm.bs, dm.L - j * dm.bs);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) sv[i] = 0.f;
          if (ch == 0) nj[e] = 0.f;
        }
        *reinterpret_cast<u32x4_t *>(kbh + e * row_pitch<D>() + (ch << 4)) = hi;
        *reinterpret_cast<u32x4_t *>(kbl + e * row_pitch<D>() + (ch << 4)) = lo;
        const int pos = (e & ~15) + perm16(e & 15);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int f = ch * 8 + i;
          const uint32_t shi = f32_to_bf16(sv[i]);
          const uint32_t slo = f32_to_bf16(sv[i] - bf16_to_f32(shi));
          const int off = f * 64 + (((pos >> 3) ^ ((f >> 1) & 3)) << 4) + ((pos & 7) << 1);
          *reinterpret_cast<uint16_t *>(sth + off) = (uint16_t)shi;
          *reinterpret_cast<uint16_t *>(stl + off) = (uint16_t)slo;
        }
      }
      if (order1) {
        h_load<D, NT>(hpre, HTh + (size_t)tyl[b0] * D * D, tid);
        h_store<D, NT>(hpre, lds + LY::TY_H0, tid);
      }
      __syncthreads();

      // per-row Taylor membership of the batch entries
      uint32_t tmask[NQ];
      bool wave_on = false;
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        tmask[n] = 0;
        if (row[n].valid) {
          for (int e = 0; e < nb; ++e) {
            const int j = tyl[b0 + e];
            if (j < row[n].nc && !(topk > 0 && list_has(row[n], topk, ptr[n], j))) tmask[n] |= 1u << e;
          }
        }
        wave_on |= ballot64(tmask[n] != 0) != 0;
      }
      if (wave_on) {
        f32x16_t at[NQ];
#pragma unroll
        for (int n = 0; n < NQ; ++n) at[n] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4_t fh = frag_rowmajor<D>(kbh, lq, 2 * ks + hl);
          const u32x4_t fl = frag_rowmajor<D>(kbl, lq, 2 * ks + hl);
#pragma unroll
          for (int n = 0; n < NQ; ++n) {
            at[n] = mfma32(fh, qf[n][ks], at[n]);
            at[n] = mfma32(fl, qf[n][ks], at[n]);
          }
        }
        u32x4_t bh[NQ][2], blo[NQ][2];
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          float mloc = kNegInf;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = 8 * (r >> 2) + 4 * hl + (r & 3);
            const float x = ((tmask[n] >> e) & 1u) ? at[n][r] * sl2 : kNegInf;
            at[n][r] = x;
            mloc = fmaxf(mloc, x);
          }
          mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
          const bool grow = mloc > m_run[n] + kRescale;
          if (ballot64(grow)) {
            const float corr = grow ? exp2f(m_run[n] - mloc) : 1.f;
            d_run[n] *= corr;
#pragma unroll
            for (int et = 0; et < NE; ++et) oacc[n][et] *= corr;
            m_run[n] = grow ? mloc : m_run[n];
          }
          const float mref = m_run[n];
          float dpart = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = 8 * (r >> 2) + 4 * hl + (r & 3);
            const float al = mref == kNegInf ? 0.f : exp2f(at[n][r] - mref);
            at[n][r] = al;
            dpart += al * nj[e];
          }
          dpart += __shfl_xor(dpart, 32);
          d_run[n] += dpart;
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            u32x4_t ph, pl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x0 = at[n][8 * hf + 2 * i], x1 = at[n][8 * hf + 2 * i + 1];
              const uint32_t p = pack_bf16x2(x0, x1);
              ph[i] = p;
              pl[i] = pack_bf16x2(x0 - bf16lo(p), x1 - bf16hi(p));
            }
            bh[n][hf] = ph;
            blo[n][hf] = pl;
          }
          if (order1) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int e = 8 * (r >> 2) + 4 * hl + (r & 3);
              alpha[(e * NQ + n) * 32 + lq] = at[n][r] * dm.scale;
            }
          }
        }
        // zero order: O^T += Sig^T alpha^T (hi*hi + lo*hi + hi*lo)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int et = 0; et < NE; ++et) {
            const int e = et * 32 + lq, ch = hf * 2 + hl;
            const u32x4_t sh = frag_st(sth, e, ch), sl = frag_st(stl, e, ch);
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
              oacc[n][et] = mfma32(sh, bh[n][hf], oacc[n][et]);
              oacc[n][et] = mfma32(sl, bh[n][hf], oacc[n][et]);
              oacc[n][et] = mfma32(sh, blo[n][hf], oacc[n][et]);
            }
          }
      }
      // first order, one block at a time (H_j^T double-buffered in LDS)
      if (order1) {
        for (int e = 0; e < nb; ++e) {
          const int cur = e & 1;
          if (e + 1 < nb) h_load<D, NT>(hpre, HTh + (size_t)tyl[b0 + e + 1] * D * D, tid);
          uint32_t bit = 0;
#pragma unroll
          for (int n = 0; n < NQ; ++n) bit |= (tmask[n] >> e) & 1u;
          if (ballot64(bit != 0)) {
            const uint8_t *hlp = lds + LY::TY_H0 + cur * LY::H_BYTES;
            float al[NQ];
#pragma unroll
            for (int n = 0; n < NQ; ++n) al[n] = alpha[(e * NQ + n) * 32 + lq];
            // O^T += H_j^T (alpha_j scale Q)^T: the per-query weight goes into
            // the B operand so the accumulators stay MFMA-only
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
              u32x4_t bq[NQ];
#pragma unroll
              for (int n = 0; n < NQ; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  bq[n][i] = pack_bf16x2(bf16lo(qf[n][ks][i]) * al[n], bf16hi(qf[n][ks][i]) * al[n]);
#pragma unroll
              for (int et = 0; et < NE; ++et) {
                const u32x4_t hf = frag_rowmajor<D>(hlp, et * 32 + lq, 2 * ks + hl);
#pragma unroll
                for (int n = 0; n < NQ; ++n) oacc[n][et] = mfma32(hf, bq[n], oacc[n][et]);
              }
              __builtin_amdgcn_sched_barrier(0);   // keep the live set to one k-step
            }
          }
          if (e + 1 < nb) h_store<D, NT>(hpre, lds + LY::TY_H0 + (cur ^ 1) * LY::H_BYTES, tid);
          __syncthreads();
        }
      } else {
        __syncthreads();
      }
    }
  }

  // ---- 5. epilogue: O = N / D in bf16, lse
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    if (!row[n].valid) continue;
    const float inv = 1.f / d_run[n];
    uint16_t *Oh = static_cast<uint16_t *>(a.O) + ((size_t)(b * dm.Hq + h) * dm.L + row[n].t) * D;
#pragma unroll
    for (int et = 0; et < NE; ++et)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = et * 32 + 8 * g + 4 * hl;
        u32x2_t o;
        o[0] = pack_bf16x2(oacc[n][et][4 * g] * inv, oacc[n][et][4 * g + 1] * inv);
        o[1] = pack_bf16x2(oacc[n][et][4 * g + 2] * inv, oacc[n][et][4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t *>(Oh + e) = o;
      }
    if (a.lse && hl == 0) a.lse[(size_t)(b * dm.Hq + h) * dm.L + row[n].t] = (m_run[n] + log2f(d_run[n])) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: plain VALU kernel, one wave per query row at a time.

PISA_DEV void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D>
__global__ __launch_bounds__(256) void attn_f32(AttnArgs a) {
  constexpr int NE = D / 64;  // output features per lane
  __shared__ float qs[4][D];
  __shared__ float ps[4][64];
  const PisaDims &dm = a.dm;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nchunk = (dm.L + 15) / 16;
  const int chunk = blockIdx.x % nchunk;
  const int bh = blockIdx.x / nchunk;
  const int b = bh / dm.Hq, h = bh % dm.Hq, hk = h * dm.Hkv / dm.Hq;
  const bool pivot = dm.group >= 1, causal = dm.causal != 0;
  const float *Q = static_cast<const float *>(a.Q) + (size_t)bh * dm.L * D;
  const size_t kvoff = (size_t)(b * dm.Hkv + hk) * dm.L * D;
  const float *K = static_cast<const float *>(a.K) + kvoff;
  const float *V = static_cast<const float *>(a.V) + kvoff;
  const size_t soff = (size_t)(b * dm.Hkv + hk) * dm.n_blk * D;
  const float sl2 = a.sl2;
  for (int rr = w; rr < 16; rr += 4) {
    const int t = chunk * 16 + rr;
    if (t >= dm.L) break;
    for (int c = l; c < D; c += 64) qs[w][c] = Q[(size_t)t * D + c];
    wave_sync();
    const int r = pivot ? t : t / dm.bs;
    int own, lo;
    const int nc = pisa_row_geometry(dm, pivot ? t : r * dm.bs, &own, &lo);
    const int32_t *list = a.idx ? a.idx + ((size_t)bh * dm.n_rows + r) * dm.topk : nullptr;
    float m = kNegInf, dsum = 0.f, o[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) o[i] = 0.f;
    // exact blocks: the kept list, then the window range [lo, own] (causal)
    int li = 0;
    bool range_done = !causal;
    for (;;) {
      int jlo, jhi;
      if (li < dm.topk && list[li] >= 0) {
        jlo = jhi = list[li++];
      } else if (!range_done) {
        jlo = lo;
        jhi = min(own, dm.n_blk - 1);
        range_done = true;
        li = dm.topk;
      } else {
        break;
      }
      for (int jj = jlo; jj <= jhi; ++jj) {
        const int kend = min(dm.L, (jj + 1) * dm.bs);
        for (int k0 = jj * dm.bs; k0 < kend; k0 += 64) {
          const int s = k0 + l;
          const bool ok = s < kend && (!causal || s <= t);
          float x = kNegInf;
          if (ok) {
            float acc = 0.f;
            for (int c = 0; c < D; ++c) acc = fmaf(qs[w][c], K[(size_t)s * D + c], acc);
            x = acc * sl2;
          }
          const float mn = fmaxf(m, wave_max_f32(x));
          if (mn == kNegInf) continue;
          const float corr = exp2f(m - mn);
          const float p = ok ? exp2f(x - mn) : 0.f;
          ps[w][l] = p;
          float psum = p;
#pragma unroll
          for (int o2 = 32; o2 >= 1; o2 >>= 1) psum += __shfl_xor(psum, o2);
          dsum = dsum * corr + psum;
          m = mn;
          wave_sync();
          const int nk = min(64, kend - k0);
#pragma unroll
          for (int i = 0; i < NE; ++i) {
            float acc = o[i] * corr;
            for (int kk = 0; kk < nk; ++kk) acc = fmaf(ps[w][kk], V[(size_t)(k0 + kk) * D + l + 64 * i], acc);
            o[i] = acc;
          }
          wave_sync();
        }
      }
    }
    // Taylor blocks: candidates [0, nc) not in the kept list
    if (dm.taylor) {
      int ptr = 0;
      for (int j = 0; j < nc; ++j) {
        while (ptr < dm.topk && list[ptr] >= 0 && list[ptr] < j) ++ptr;
        if (ptr < dm.topk && list[ptr] == j) continue;
        const float *kb = a.kbar + soff + (size_t)j * D;
        float part = 0.f;
        for (int c = l; c < D; c += 64) part = fmaf(qs[w][c], kb[c], part);
#pragma unroll
        for (int o2 = 32; o2 >= 1; o2 >>= 1) part += __shfl_xor(part, o2);
        const float x = part * sl2;
        const float mn = fmaxf(m, x);
        const float corr = exp2f(m - mn);
        const float al = exp2f(x - mn);
        const float njf = (float)min(dm.bs, dm.L - j * dm.bs);
        dsum = dsum * corr + al * njf;
        m = mn;
        const float *vs = a.vsum + soff + (size_t)j * D;
        const float *Hj = static_cast<const float *>(a.HT) + (soff + (size_t)j * D) * D;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
          const int e = l + 64 * i;
          float num = vs[e];
          if (dm.taylor == 2) {
            float qh = 0.f;
            for (int c = 0; c < D; ++c) qh = fmaf(qs[w][c], Hj[(size_t)e * D + c], qh);
            num = fmaf(dm.scale, qh, num);
          }
          o[i] = fmaf(al, num, o[i] * corr);
        }
      }
    }
    float *O = static_cast<float *>(a.O) + ((size_t)bh * dm.L + t) * D;
#pragma unroll
    for (int i = 0; i < NE; ++i) O[l + 64 * i] = o[i] / dsum;
    if (a.lse && l == 0) a.lse[(size_t)bh * dm.L + t] = (m + log2f(dsum)) * kLn2;
    wave_sync();
  }
}

template <int D, int BS, int NW, int NQ>
hipError_t launch_bf16(const AttnArgs &a, hipStream_t st) {
  using LY = Lds<D, BS, NW, NQ>;
  const PisaDims &dm = a.dm;
  const int hpw = dm.ratio < NW ? dm.ratio : NW;
  const int tpw = NW * NQ * 32 / hpw;
  const unsigned grid = (unsigned)dm.B * dm.Hkv * (dm.ratio / hpw) * ((dm.L + tpw - 1) / tpw);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_bf16<D, BS, NW, NQ>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::TOTAL);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  attn_bf16<D, BS, NW, NQ><<<grid, NW * 64, LY::TOTAL, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const PisaDims &dm, const void *Q, const void *K, const void *V, const float *kbar,
                       const float *vsum, const void *HT, const int32_t *idx, void *O, float *lse,
                       hipStream_t st) {
  AttnArgs a;
  a.dm = dm;
  a.Q = Q; a.K = K; a.V = V; a.kbar = kbar; a.vsum = vsum; a.HT = HT; a.idx = idx; a.O = O; a.lse = lse;
  a.sl2 = dm.scale * kLog2e;
  if (dm.dtype == 1) {
    const unsigned grid = (unsigned)dm.B * dm.Hq * ((dm.L + 15) / 16);
    if (dm.d == 64) attn_f32<64><<<grid, 256, 0, st>>>(a);
    else attn_f32<128><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  if (dm.d == 64) return dm.bs == 64 ? launch_bf16<64, 64, 8, 1>(a, st) : launch_bf16<64, 128, 4, 2>(a, st);
  return dm.bs == 64 ? launch_bf16<128, 64, 8, 1>(a, st) : launch_bf16<128, 128, 8, 1>(a, st);
}
