// Stage C, bf16 path: exact online-softmax attention over the kept blocks,
// fused with the per-block first-order Taylor tail for every other candidate
// block, on gfx950 MFMA.
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
// Structure (MI355X):
//   * workgroup = 8 waves x 32 query rows = 256 rows of the query heads that
//     share one KV head (GQA packing), two waves per SIMD;
//   * everything is computed transposed so a lane owns one query (lane % 32):
//       S^T  = K Q^T           A = K tile (LDS),  B = Q (registers)
//       O^T += V^T P^T         A = V tile read transposed (ds_read_b64_tr_b16)
//       a^T  = Kbar Q^T        Taylor logits, kbar as bf16 hi + lo
//       O^T += Sig^T alpha^T   zero order, hi/lo splits
//       O^T += H_j^T (alpha_j scale Q)^T   first order, alpha on the B operand
//   * K / V tiles of 64 keys and H_j^T tiles are fetched global -> LDS by the
//     DMA path (global_load_lds_dwordx4, no registers): K/V in a 4-deep ring
//     two stages ahead, H in a 3-deep ring one block ahead, one barrier per
//     step; waits are explicit vmcnt counts;
//   * the workgroup walks the union of its rows' kept blocks, then the union
//     of their Taylor blocks 32 per batch; a wave skips blocks none of its rows
//     uses; per-row masks handle PIVOT rows whose lists differ within a wave;
//   * row maxima move only when a logit exceeds them by more than 2^8, so the
//     output accumulators (MFMA-only registers) are rarely rescaled.
#include "attn_tiles.h"

using namespace pisa_attn;

namespace {

constexpr int kStage = 64;       // keys per pipeline stage
constexpr int kTyBatch = 32;     // Taylor blocks per logits batch
constexpr float kRescale = 8.f;  // lazy max threshold (log2 units)
constexpr int kRingKV = 4, kRingH = 3;

// A tile of R rows x D bf16 into LDS, row-major, 16-byte chunks XOR-swizzled:
// SWZ 0: chunk ^ (row & 7)  (rows read with ds_read_b128 by 8-row lane groups)
// SWZ 1: chunk ^ 2 (row & 3) (rows read 4 at a time by ds_read_b64_tr_b16)
// The NW waves issue R * D / (512 NW) one-kilobyte DMA transfers each; rows past nvalid
// repeat the last valid row (finite data, masked or weighted by zero).
template <int D, int R, int SWZ, int NW>
PISA_DEV void dma_tile(const uint16_t *g, int nvalid, uint8_t *tile, int w, int l) {
  constexpr int CPR = D / 8;
  constexpr int NCH = R * CPR / 64;
  static_assert(NCH % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < NCH / NW; ++i) {
    const int c = w + i * NW;
    const int p = c * 64 + l;
    const int row = p / CPR, phys = p % CPR;
    const int logical = phys ^ (SWZ ? 2 * (row & 3) : (row & 7));
    const int rr = row < nvalid ? row : nvalid - 1;
    dma16(g + (size_t)rr * D + logical * 8, tile + c * 1024);
  }
}

template <int D, int NW, int NQ>
struct Lay {
  static constexpr int TILE = kStage * D * 2;        // one K or V stage
  static constexpr int STAGE = 2 * TILE;
  static constexpr int EX_END = kRingKV * STAGE;
  static constexpr int HT = D * D * 2;
  static constexpr int TY_H = 0;
  static constexpr int TY_KBH = TY_H + kRingH * HT;
  static constexpr int TY_KBL = TY_KBH + kTyBatch * D * 2;
  static constexpr int TY_STH = TY_KBL + kTyBatch * D * 2;
  static constexpr int TY_STL = TY_STH + D * kTyBatch * 2;
  static constexpr int TY_ALPHA = TY_STL + D * kTyBatch * 2;   // bf16 [wave][entry][tile][row]
  static constexpr int TY_NJ = TY_ALPHA + NW * kTyBatch * NQ * 32 * 2;
  static constexpr int TY_END = TY_NJ + kTyBatch * 4;
  static constexpr int MAIN = EX_END > TY_END ? EX_END : TY_END;
  static constexpr int EXL = MAIN;                 // union lists (uint16)
  static constexpr int TYL = EXL + 1024 * 2;
  static constexpr int EXB = TYL + 1024 * 2;       // union bitmaps
  static constexpr int TYB = EXB + 32 * 4;
  static constexpr int TBITS = TYB + 32 * 4;       // per-wave kept bitmaps (block rows)
  static constexpr int CNT = TBITS + NW * 32 * 4;
  static constexpr int TOTAL = CNT + 16;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Sigma^T tile [D][32 entries]: entry e sits at position perm16 within its
// group of 16 so the alpha accumulator layout is the MFMA B operand as is.
PISA_DEV u32x4_t frag_st(const uint8_t *base, int e, int ch) {
  const int phys = ch ^ ((e >> 1) & 3);
  return *reinterpret_cast<const u32x4_t *>(base + e * 64 + (phys << 4));
}

// Kept-list cursor of one PIVOT row, for walks that visit blocks in
// ascending order: the head is the next list entry that is a candidate of
// the row (0 <= j < nc; other entries are skipped), entries below the block
// asked for are passed over, and past the end the head is INT_MAX.
struct Cursor {
  const int32_t *p;
  int left;
  int nc;
  int head;
};
PISA_DEV void cursor_next(Cursor &c) {
  c.head = 0x7FFFFFFF;
  while (c.left > 0) {
    const int v = *c.p;
    ++c.p;
    --c.left;
    if (pisa_list_entry_kept(v, c.nc)) {
      c.head = v;
      break;
    }
  }
}
PISA_DEV void cursor_init(Cursor &c, const int32_t *list, int n, int nc) {
  c.p = list;
  c.left = n;
  c.nc = nc;
  cursor_next(c);
}
PISA_DEV bool cursor_match(Cursor &c, int j) {
  while (c.head < j) cursor_next(c);
  if (c.head != j) return false;
  cursor_next(c);
  return true;
}

// ---------------------------------------------------------------------------

template <int D, int BS, int NW, int NQ>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16(AttnArgs a) {
  using LY = Lay<D, NW, NQ>;
  constexpr int NT = NW * 64;
  constexpr int ROWS = NW * NQ * 32;
  constexpr int NE = D / 32;          // 32-feature output tiles
  constexpr int SPB = BS / kStage;    // stages per block
  constexpr int PER_STAGE = 2 * (kStage * D / 8 / 64) / NW;   // DMA ops per wave per stage
  constexpr int PER_H = (D * D / 8 / 64) / NW;                // DMA ops per wave per H tile
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const PisaDims &dm = a.dm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 31, hl = l >> 5;

  // ---- workgroup -> (b, kv head, head group, token tile); wave -> (head, NQ x 32 tokens)
  const int hpw = dm.ratio < NW ? dm.ratio : NW;
  const int ngrp = dm.ratio / hpw;
  const int tpw = ROWS / hpw;
  const int ntile = (dm.L + tpw - 1) / tpw;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  // causal rows: the longest tiles (latest tokens) first
  const int tile = dm.causal ? ntile - 1 - logical % ntile : logical % ntile;
  const int rest = logical / ntile;
  const int grp = rest % ngrp;
  const int bk = rest / ngrp;
  const int b = bk / dm.Hkv, hk = bk % dm.Hkv;
  const int wph = NW / hpw;
  const int h = hk * dm.ratio + grp * hpw + w / wph;
  const bool pivot = dm.group >= 1;
  const int topk = dm.topk;
  const bool causal = dm.causal != 0;
  const int taylor = dm.taylor;
  const int tw = tile * tpw + (w % wph) * (NQ * 32);   // first token of the wave

  // per query tile n: this lane's token and its selection row
  int t[NQ], own[NQ], lo[NQ], nc[NQ];
  bool valid[NQ];
  const int32_t *list[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    t[n] = tw + n * 32 + lq;
    valid[n] = t[n] < dm.L;
    const int rsel = pivot ? t[n] : t[n] / dm.bs;
    nc[n] = pisa_row_geometry(dm, pivot ? t[n] : rsel * dm.bs, &own[n], &lo[n]);
    list[n] = a.idx ? a.idx + ((size_t)(b * dm.Hq + h) * dm.n_rows + rsel) * topk : nullptr;
  }

  uint32_t *exb = reinterpret_cast<uint32_t *>(lds + LY::EXB);
  uint32_t *tyb = reinterpret_cast<uint32_t *>(lds + LY::TYB);
  uint32_t *tbits = reinterpret_cast<uint32_t *>(lds + LY::TBITS) + w * 32;
  uint16_t *exl = reinterpret_cast<uint16_t *>(lds + LY::EXL);
  uint16_t *tyl = reinterpret_cast<uint16_t *>(lds + LY::TYL);
  int *cnt = reinterpret_cast<int *>(lds + LY::CNT);
  const int nwords = (dm.n_blk + 31) >> 5;

  // ---- 1. unions of the kept and Taylor block sets; per-wave kept bitmaps
  // (block rows: all NQ x 32 rows of a wave lie in one query block, one list)
  for (int i = tid; i < 32; i += NT) {
    exb[i] = 0;
    tyb[i] = 0;
  }
  if (l < 32) tbits[l] = 0;
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const bool leader = valid[n] && (pivot ? hl == 0 : (l == 0 && n == 0));
    if (!leader) continue;
    // list entries that are not candidates of the row are dropped
    for (int i = 0; i < topk; ++i) {
      const int j = list[n][i];
      if (!pisa_list_entry_kept(j, nc[n])) continue;
      atomicOr(&exb[j >> 5], 1u << (j & 31));
      if (!pivot) tbits[j >> 5] |= 1u << (j & 31);
    }
    for (int j = lo[n]; j <= own[n] && j < dm.n_blk; ++j) atomicOr(&exb[j >> 5], 1u << (j & 31));
    if (taylor) {
      int ptr = 0;
      for (int wd = 0; wd * 32 < nc[n]; ++wd) {
        uint32_t bits = (nc[n] - wd * 32 >= 32) ? 0xFFFFFFFFu : ((1u << (nc[n] - wd * 32)) - 1u);
        for (ptr = 0; ptr < topk; ++ptr) {   // the row's kept candidates in this word
          const int j = list[n][ptr];
          if (j >= wd * 32 && j < (wd + 1) * 32 && j < nc[n]) bits &= ~(1u << (j & 31));
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
      qf[n][ks] = valid[n] ? *reinterpret_cast<const u32x4_t *>(Qh + (size_t)t[n] * D + ks * 16 + hl * 8)
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

  // per-lane constants of the fragment addresses
  const int xk = lq & 7;                        // K / H / kbar row swizzle
  const int srow = (l & 15) >> 2;               // transposed-read source row in its 4-row group
  const int ecol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  // ---- 3. exact phase: union of kept blocks, 64-key stages
  if (n_ex > 0) {
    const int n_st = n_ex * SPB;
    auto issue = [&](int s) {
      const int j = exl[s / SPB];
      const int key0 = j * BS + (s % SPB) * kStage;
      const int nk = min(kStage, dm.L - key0);
      uint8_t *buf = lds + (s % kRingKV) * LY::STAGE;
      dma_tile<D, kStage, 0, NW>(Kh + (size_t)key0 * D, nk, buf, w, l);
      dma_tile<D, kStage, 1, NW>(Vh + (size_t)key0 * D, nk, buf + LY::TILE, w, l);
    };
    issue(0);
    if (n_st > 1) issue(1);
    Cursor cur[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) cursor_init(cur[n], list[n], valid[n] && pivot ? topk : 0, nc[n]);
    bool mem[NQ];
    bool active = false;
#pragma unroll
    for (int n = 0; n < NQ; ++n) mem[n] = false;
    // One barrier per pair of stages.  At stage it (even): this wave's DMA of
    // stages it, it + 1 (issued after the previous barrier) has landed; after
    // the barrier so has every wave's, and every wave has finished stages
    // it - 2, it - 1, whose ring slots then take the DMA of stages it + 2 and
    // it + 3.  Waves drift by up to two stages between barriers.
    for (int it = 0; it < n_st; ++it) {
      const int j = exl[it / SPB], kh = it % SPB;
      if ((it & 1) == 0) {
        wait_vmcnt<0>();
        __syncthreads();
        if (it + 2 < n_st) issue(it + 2);
        if (it + 3 < n_st) issue(it + 3);
      }
      if (kh == 0) {
        bool any = false;
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          bool inlist;
          if (pivot) inlist = cursor_match(cur[n], j);
          else inlist = (tbits[j >> 5] >> (j & 31)) & 1u;
          mem[n] = valid[n] && ((j >= lo[n] && j <= own[n]) || inlist);
          any |= mem[n];
        }
        active = ballot64(any) != 0;
      }
      if (!active) continue;
      const uint8_t *kl = lds + (it % kRingKV) * LY::STAGE;
      const uint8_t *vl = kl + LY::TILE;
      f32x16_t s[NQ][2];
#pragma unroll
      for (int n = 0; n < NQ; ++n) s[n][0] = s[n][1] = f32x16_t{};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = q * 32 + lq;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int ch = (2 * ks + hl) ^ xk;
          const u32x4_t af = *reinterpret_cast<const u32x4_t *>(kl + row * (2 * D) + (ch << 4));
#pragma unroll
          for (int n = 0; n < NQ; ++n) s[n][q] = mfma32(af, qf[n][ks], s[n][q]);
        }
      }
      const int kbase = j * BS + kh * kStage;
      // keys past the last token or (causal) past a row's own token: only the
      // stages that reach them need an element mask
      const bool edge = kbase + kStage > dm.L || (causal && kbase + kStage - 1 > tw);
      u32x4_t pb[NQ][2][2];
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        if (edge && mem[n]) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbase + q * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
              if (key >= dm.L || (causal && key > t[n])) s[n][q][r] = kNegInf;
            }
        }
        // the row's maximum of the raw scores (rows that do not keep the
        // block take no weight from it: their exponent offset is -inf)
        float mloc = kNegInf;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int r = 0; r < 16; r += 2) mloc = fmaxf(fmaxf(mloc, s[n][q][r]), s[n][q][r + 1]);
        mloc = mem[n] ? mloc * sl2 : kNegInf;
        mloc = pair_max_f(mloc);
        const bool grow = mloc > m_run[n] + kRescale;   // includes the first visible block
        if (ballot64(grow)) {
          const float corr = grow ? fast_exp2(m_run[n] - mloc) : 1.f;
          d_run[n] *= corr;
#pragma unroll
          for (int et = 0; et < NE; ++et) oacc[n][et] *= corr;
          m_run[n] = grow ? mloc : m_run[n];
        }
        const float mneg = mem[n] ? -(m_run[n] == kNegInf ? 0.f : m_run[n]) : kNegInf;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[n][q][r] = fast_exp2(fmaf(s[n][q][r], sl2, mneg));
        // the row sum of the bf16 weights that P V uses (N and D agree)
        float psum = 0.f;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            pb[n][q][hf] = pack8(s[n][q], 8 * hf);
            psum = sum_bf16x8_f(pb[n][q][hf], psum);
          }
        d_run[n] += pair_sum_f(psum);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r1 = q * 32 + 16 * hf + 4 * hl + srow;
#pragma unroll
          for (int et = 0; et < NE; ++et) {
            const int e = et * 32 + ecol;
            const int off = (((e >> 3) ^ (2 * srow)) << 4) + (((e >> 2) & 1) << 3);
            const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t *)(vl + r1 * (2 * D) + off));
            const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t *)(vl + (r1 + 8) * (2 * D) + off));
            const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
            const u32x4_t af = {w0[0], w0[1], w1[0], w1[1]};
#pragma unroll
            for (int n = 0; n < NQ; ++n) oacc[n][et] = mfma32(af, pb[n][q][hf], oacc[n][et]);
          }
        }
    }
    __syncthreads();   // the Taylor phase reuses the stage ring's LDS
  }

  // ---- 4. Taylor phase: union of Taylor blocks, logits 32 at a time,
  // first-order term block by block
  if (taylor && n_ty > 0) {
    const size_t soff = (size_t)(b * dm.Hkv + hk) * dm.n_blk;
    const float *kbar = a.kbar + soff * D;
    const float *vsum = a.vsum + soff * D;
    const uint16_t *HTh = static_cast<const uint16_t *>(a.HT) + soff * D * D;
    uint8_t *kbh = lds + LY::TY_KBH, *kbl = lds + LY::TY_KBL;
    uint8_t *sth = lds + LY::TY_STH, *stl = lds + LY::TY_STL;
    uint16_t *alpha = reinterpret_cast<uint16_t *>(lds + LY::TY_ALPHA) + w * kTyBatch * NQ * 32;
    float *nj = reinterpret_cast<float *>(lds + LY::TY_NJ);
    const bool order1 = taylor == 2, hybrid = taylor == 3;
    float a_run[NQ];   // hybrid: sum of the rows' Taylor weights, on the scale of d_run
#pragma unroll
    for (int n = 0; n < NQ; ++n) a_run[n] = 0.f;
    Cursor cur[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) cursor_init(cur[n], list[n], valid[n] && pivot ? topk : 0, nc[n]);
    uint32_t tmask[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) tmask[n] = 0;
    if (order1) dma_tile<D, D, 0, NW>(HTh + (size_t)tyl[0] * D * D, D, lds + LY::TY_H, w, l);
    else if (hybrid && !causal)   // the mean matrix Hbar^T of this kv head
      dma_tile<D, D, 0, NW>(static_cast<const uint16_t *>(a.HT) + hbar_offset(dm, b * dm.Hkv + hk, 0), D,
                            lds + LY::TY_H, w, l);
    for (int eg = 0; eg < n_ty; ++eg) {
      const int e = eg & (kTyBatch - 1);
      if (e == 0) {
        const int b0 = eg;
        const int nb = min(kTyBatch, n_ty - b0);
        __syncthreads();   // the previous batch's tables are consumed
        for (int u = tid; u < kTyBatch * (D / 8); u += NT) {
          const int en = u / (D / 8), ch = u % (D / 8);
          u32x4_t hi = {0, 0, 0, 0}, lo4 = {0, 0, 0, 0};
          float sv[8];
          if (en < nb) {
            const int j = tyl[b0 + en];
            const f32x4_t x0 = *reinterpret_cast<const f32x4_t *>(kbar + (size_t)j * D + ch * 8);
            const f32x4_t x1 = *reinterpret_cast<const f32x4_t *>(kbar + (size_t)j * D + ch * 8 + 4);
            const f32x4_t v0 = *reinterpret_cast<const f32x4_t *>(vsum + (size_t)j * D + ch * 8);
            const f32x4_t v1 = *reinterpret_cast<const f32x4_t *>(vsum + (size_t)j * D + ch * 8 + 4);
            const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t pk = pack_bf16x2(x[2 * i], x[2 * i + 1]);
              hi[i] = pk;
              lo4[i] = pack_bf16x2(x[2 * i] - bf16lo(pk), x[2 * i + 1] - bf16hi(pk));
            }
            sv[0] = v0[0]; sv[1] = v0[1]; sv[2] = v0[2]; sv[3] = v0[3];
            sv[4] = v1[0]; sv[5] = v1[1]; sv[6] = v1[2]; sv[7] = v1[3];
            if (ch == 0) nj[en] = (float)min(dm.bs, dm.L - j * dm.bs);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) sv[i] = 0.f;
            if (ch == 0) nj[en] = 0.f;
          }
          const int sw = (ch ^ (en & 7)) << 4;
          *reinterpret_cast<u32x4_t *>(kbh + en * (2 * D) + sw) = hi;
          *reinterpret_cast<u32x4_t *>(kbl + en * (2 * D) + sw) = lo4;
          const int pos = (en & ~15) + perm16(en & 15);
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
        __syncthreads();
        // membership of the batch entries for each of this lane's rows
        bool any = false;
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          tmask[n] = 0;
          if (valid[n]) {
            for (int en = 0; en < nb; ++en) {
              const int j = tyl[b0 + en];
              bool inlist;
              if (pivot) inlist = cursor_match(cur[n], j);
              else inlist = (tbits[j >> 5] >> (j & 31)) & 1u;
              if (j < nc[n] && !inlist) tmask[n] |= 1u << en;
            }
          }
          any |= tmask[n] != 0;
        }
        if (ballot64(any)) {
          f32x16_t at[NQ];
#pragma unroll
          for (int n = 0; n < NQ; ++n) at[n] = f32x16_t{};
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const int ch = (2 * ks + hl) ^ xk;
            const u32x4_t fh = *reinterpret_cast<const u32x4_t *>(kbh + lq * (2 * D) + (ch << 4));
            const u32x4_t fl = *reinterpret_cast<const u32x4_t *>(kbl + lq * (2 * D) + (ch << 4));
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
              at[n] = mfma32(fh, qf[n][ks], at[n]);
              at[n] = mfma32(fl, qf[n][ks], at[n]);
            }
          }
          u32x4_t ph[NQ][2], pl[NQ][2];
#pragma unroll
          for (int n = 0; n < NQ; ++n) {
            float mloc = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int en = 8 * (r >> 2) + 4 * hl + (r & 3);
              const float x = ((tmask[n] >> en) & 1u) ? at[n][r] * sl2 : kNegInf;
              at[n][r] = x;
              mloc = fmaxf(mloc, x);
            }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
            const bool grow = mloc > m_run[n] + kRescale;
            if (ballot64(grow)) {
              const float corr = grow ? fast_exp2(m_run[n] - mloc) : 1.f;
              d_run[n] *= corr;
              a_run[n] *= corr;
#pragma unroll
              for (int et = 0; et < NE; ++et) oacc[n][et] *= corr;
              m_run[n] = grow ? mloc : m_run[n];
            }
            const float mref = m_run[n] == kNegInf ? 0.f : m_run[n];
            float dpart = 0.f, apart = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int en = 8 * (r >> 2) + 4 * hl + (r & 3);
              const float al = fast_exp2(at[n][r] - mref);
              at[n][r] = al;
              dpart += al * nj[en];
              apart += al;
            }
            dpart += __shfl_xor(dpart, 32);
            d_run[n] += dpart;
            if (hybrid) a_run[n] += apart + __shfl_xor(apart, 32);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float x0 = at[n][8 * hf + 2 * i], x1 = at[n][8 * hf + 2 * i + 1];
                const uint32_t pk = pack_bf16x2(x0, x1);
                ph[n][hf][i] = pk;
                pl[n][hf][i] = pack_bf16x2(x0 - bf16lo(pk), x1 - bf16hi(pk));
              }
            }
            if (order1) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int en = 8 * (r >> 2) + 4 * hl + (r & 3);
                alpha[(en * NQ + n) * 32 + lq] = (uint16_t)f32_to_bf16(at[n][r] * dm.scale);
              }
            }
          }
          // zero order: O^T += Sig^T alpha^T (hi*hi + lo*hi + hi*lo)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int et = 0; et < NE; ++et) {
              const int ee = et * 32 + lq, ch = hf * 2 + hl;
              const u32x4_t sh = frag_st(sth, ee, ch), sl = frag_st(stl, ee, ch);
#pragma unroll
              for (int n = 0; n < NQ; ++n) {
                oacc[n][et] = mfma32(sh, ph[n][hf], oacc[n][et]);
                oacc[n][et] = mfma32(sl, ph[n][hf], oacc[n][et]);
                oacc[n][et] = mfma32(sh, pl[n][hf], oacc[n][et]);
              }
            }
        }
      }
      if (!order1) continue;
      // first order for entry eg: H ring (3 deep, one block ahead)
      if (eg + 1 < n_ty) {
        dma_tile<D, D, 0, NW>(HTh + (size_t)tyl[eg + 1] * D * D, D,
                              lds + LY::TY_H + ((eg + 1) % kRingH) * LY::HT, w, l);
        wait_vmcnt<PER_H>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();   // H_eg landed for all waves; H_{eg+1} stays in flight
      uint32_t bit = 0;
#pragma unroll
      for (int n = 0; n < NQ; ++n) bit |= (tmask[n] >> e) & 1u;
      if (ballot64(bit != 0)) {
        const uint8_t *hlp = lds + LY::TY_H + (eg % kRingH) * LY::HT;
        float al[NQ];
#pragma unroll
        for (int n = 0; n < NQ; ++n) al[n] = bf16_to_f32(alpha[(e * NQ + n) * 32 + lq]);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          u32x4_t bq[NQ];
#pragma unroll
          for (int n = 0; n < NQ; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              bq[n][i] = pack_bf16x2(bf16lo(qf[n][ks][i]) * al[n], bf16hi(qf[n][ks][i]) * al[n]);
          const int ch = (2 * ks + hl) ^ xk;
#pragma unroll
          for (int et = 0; et < NE; ++et) {
            const u32x4_t hf = *reinterpret_cast<const u32x4_t *>(hlp + (et * 32 + lq) * (2 * D) + (ch << 4));
#pragma unroll
            for (int n = 0; n < NQ; ++n) oacc[n][et] = mfma32(hf, bq[n], oacc[n][et]);
          }
        }
      }
    }
    if (hybrid && causal) {
      // O^T += Hbar(lo)^T (scale * sum alpha) q^T, once per row, Hbar(lo) the
      // mean over the row's candidates [0, lo): one pass per distinct lo
      // among the wave's rows (rows of other lo take a zero weight), the
      // A fragments read straight from memory
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const float al = a_run[n] * dm.scale;
        uint64_t pend = ballot64(valid[n] && al != 0.f);
        while (pend) {
          const int l0 = __builtin_amdgcn_readlane(lo[n], (int)__builtin_ctzll(pend));
          const float aln = (valid[n] && lo[n] == l0) ? al : 0.f;
          const uint16_t *hg = static_cast<const uint16_t *>(a.HT) + hbar_offset(dm, b * dm.Hkv + hk, l0);
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            u32x4_t bq;
#pragma unroll
            for (int i = 0; i < 4; ++i) bq[i] = pack_bf16x2(bf16lo(qf[n][ks][i]) * aln, bf16hi(qf[n][ks][i]) * aln);
            u32x4_t hf[NE];
#pragma unroll
            for (int et = 0; et < NE; ++et)
              hf[et] = *reinterpret_cast<const u32x4_t *>(hg + (size_t)(et * 32 + lq) * D + (2 * ks + hl) * 8);
#pragma unroll
            for (int et = 0; et < NE; ++et) oacc[n][et] = mfma32(hf[et], bq, oacc[n][et]);
          }
          pend &= ~ballot64(lo[n] == l0);
        }
      }
    } else if (hybrid) {   // O^T += Hbar^T (scale * sum alpha) q^T, once per row
      wait_vmcnt<0>();
      __syncthreads();
      const uint8_t *hlp = lds + LY::TY_H;
      float al[NQ];
#pragma unroll
      for (int n = 0; n < NQ; ++n) al[n] = a_run[n] * dm.scale;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        u32x4_t bq[NQ];
#pragma unroll
        for (int n = 0; n < NQ; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            bq[n][i] = pack_bf16x2(bf16lo(qf[n][ks][i]) * al[n], bf16hi(qf[n][ks][i]) * al[n]);
        const int ch = (2 * ks + hl) ^ xk;
#pragma unroll
        for (int et = 0; et < NE; ++et) {
          const u32x4_t hf = *reinterpret_cast<const u32x4_t *>(hlp + (et * 32 + lq) * (2 * D) + (ch << 4));
#pragma unroll
          for (int n = 0; n < NQ; ++n) oacc[n][et] = mfma32(hf, bq[n], oacc[n][et]);
        }
      }
    }
  }

  // ---- 5. epilogue: O = N / D in bf16, lse
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    if (!valid[n]) continue;
    const float inv = 1.f / d_run[n];
    uint16_t *Oh = static_cast<uint16_t *>(a.O) + ((size_t)(b * dm.Hq + h) * dm.L + t[n]) * D;
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
    if (a.lse && hl == 0) a.lse[(size_t)(b * dm.Hq + h) * dm.L + t[n]] = (m_run[n] + log2f(d_run[n])) * kLn2;
  }
}

template <int D, int BS, int NW, int NQ>
hipError_t launch(const AttnArgs &a, hipStream_t st) {
  using LY = Lay<D, NW, NQ>;
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

hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t st) {
  // block rows: one kept list per query block, walked part by part
  if (a.dm.group == 0) return launch_attn_blocks(a, st);
  // PIVOT rows (one list per token): the union walk with per-row masks,
  // eight waves of 32 rows (two waves per SIMD)
  if (a.dm.d == 64) return a.dm.bs == 64 ? launch<64, 64, 8, 1>(a, st) : launch<64, 128, 8, 1>(a, st);
  return a.dm.bs == 64 ? launch<128, 64, 8, 1>(a, st) : launch<128, 128, 8, 1>(a, st);
}

hipError_t launch_attn(const PisaDims &dm, const void *Q, const void *K, const void *V, const float *kbar,
                       const float *vsum, const void *HT, const int32_t *idx, void *O, float *lse, void *ws,
                       hipStream_t st) {
  AttnArgs a;
  a.dm = dm;
  a.Q = Q; a.K = K; a.V = V; a.kbar = kbar; a.vsum = vsum; a.HT = HT; a.idx = idx; a.O = O; a.lse = lse;
  a.sl2 = dm.scale * kLog2e;
  if (dm.dtype == 1) return launch_attn_f32(a, st);
  if (ws && pivot_kg_supported(dm)) return launch_attn_pivot(a, ws, st);
  return launch_attn_bf16(a, st);
}
