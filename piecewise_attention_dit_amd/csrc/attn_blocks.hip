// Stage C, bf16, block-row selection: exact online-softmax attention over
// each query block's kept key blocks, fused with the per-block Taylor tail
// for every other candidate block, on gfx950 MFMA.
//
// PISA page, section 2: o_t = N_t / D_t; exact terms e^{q k} v over the
// selected blocks; for a non-selected block j, alpha = e^{q . kbar_j} times
// (sum of its values + q H_j) in N_t and alpha * n_j in D_t.  Hardware
// implementation section: one fused online-softmax kernel, selected blocks
// staged on chip, pooled statistics scanned for the rest.  Sliding Window
// Attention page (causal window, widened here to whole blocks).
//
// Work split (MI355X):
//   * workgroup = 8 waves x 32 query rows = 256 rows, two waves per SIMD;
//     the rows form P = 256 / block "parts", each one selection row (one
//     query block of one head; GQA heads that share a KV head are packed);
//   * the exact phase runs in steps.  In a step every part takes SK keys of
//     its own kept list (its own LDS region), so no wave ever waits on a
//     block it does not use; the causal window range, identical for heads
//     and overlapping for neighbouring block rows, is walked first with one
//     shared region;
//   * a wave computes everything transposed, lane = query (lane % 32):
//       S^T  = K Q^T           A = K tile (LDS),  B = Q (registers)
//       O^T += V^T P^T         A = V tile through ds_read_b64_tr_b16
//     and software-pipelines its steps: in step i it issues the MFMAs of
//     S_{i+1} and of P_{i-1} V_{i-1} around the exponentials of step i, so
//     the matrix cores and the VALU work at the same time;
//   * K and V move global -> LDS by the DMA path (no registers) in two
//     2-deep rings, one step ahead, one barrier per step;
//   * the Taylor phase walks the union of the parts' Taylor blocks, 16 per
//     logits batch (a^T = Kbar Q^T, zero order Sigma^T alpha^T with bf16
//     hi/lo splits), and per block the first order u = H_j^T Q^T, added as
//     O^T += (alpha scale) u in fp32; H tiles stream through an LDS ring in
//     groups of blocks (two for d = 128, one group ahead; four for d = 64,
//     two groups ahead), one barrier per group
//     (hybrid order: the zero order only, plus one u = Hbar^T Q^T per row
//     scaled by the row's summed Taylor weights);
//   * row maxima move only when a logit exceeds them by more than 2^8.
#include "attn_tiles.h"

using namespace pisa_attn;

namespace {

constexpr int NW = 8;              // waves per workgroup
constexpr int NT = NW * 64;
constexpr int ROWS = NW * 32;      // query rows per workgroup
constexpr int kNB = 16;            // Taylor entries per logits batch
constexpr float kRescale = 8.f;    // lazy max threshold (log2 units)
constexpr int kMaxK = 256;         // kept-list capacity per part

template <int D, int BS>
struct Cfg {
  static constexpr int P = ROWS / BS;                         // parts per workgroup
  static constexpr int WPP = NW / P;                          // waves per part
  static constexpr int SK = (BS == 64 && D == 128) ? 32 : 64; // keys per part per step
  static constexpr int SPB = BS / SK;                         // steps per block
  static constexpr int NQT = SK / 32;                         // 32-key tiles per step
  static constexpr int NE = D / 32;                           // 32-feature output tiles
  static constexpr int SUB = SK * D * 2;                      // one part's K (or V) bytes per step
  static constexpr int SLOT = P * SUB;
  static constexpr int CPS = SUB / 1024;                      // DMA kilobytes per sub-tile
  static constexpr int EX_K = 0, EX_V = 2 * SLOT, EX_END = 4 * SLOT;
  static constexpr int HT = D * D * 2;
  static constexpr int HCH = HT / 1024;
  // first-order entries per barrier (a group) and the H ring.  d = 64: an
  // entry is 8 MFMAs per wave, so four share a barrier, in a ring of three
  // groups (the one in use and two ahead).  d = 128: two entries per barrier
  // in a ring of two groups (the one in use and the next), which is what
  // fits in LDS beside the batch tables.
  static constexpr int GE = D == 64 ? 4 : 2;
  static constexpr int RINGH = D == 64 ? 12 : 4;
  static constexpr int AHEAD = RINGH / GE - 1;                // groups in flight ahead
  static_assert(RINGH >= P, "causal hybrid rows stage one mean matrix per block row");
  // the next batch's rows are staged at group SG, its tables built in group
  // SG + 1 and published by the barrier of group SG + 2, inside the batch
  static constexpr int SG = (kNB / 2) / GE < kNB / GE - 3 ? (kNB / 2) / GE : kNB / GE - 3;
  static_assert(kNB % GE == 0 && SG >= 1 && SG + 2 < kNB / GE, "batch too short for the table pipeline");
  static constexpr int TY_H = 0;
  static constexpr int TY_KBH = TY_H + RINGH * HT;
  static constexpr int TY_KBL = TY_KBH + kNB * D * 2;
  static constexpr int TY_STH = TY_KBL + kNB * D * 2;
  static constexpr int TY_STL = TY_STH + D * kNB * 2;
  static constexpr int TY_AL = TY_STL + D * kNB * 2;          // bf16 [wave][entry][32 rows]
  static constexpr int TY_NJ = TY_AL + NW * kNB * 32 * 2;
  static constexpr int TY_END = TY_NJ + kNB * 4;
  // staging of the next batch's kbar, vsum rows (fp32 [2][kNB][D]): at first
  // order over the batch tables (dead between a batch's start and the next
  // build), otherwise in ring slot 1 (unused without first order)
  static constexpr int STG_BYTES = 2 * kNB * D * 4;
  static_assert(STG_BYTES == TY_AL - TY_KBH, "the staging area overlays the four batch tables");
  static_assert(STG_BYTES <= HT, "the staging area fits a ring slot");
  static constexpr int MAIN = EX_END > TY_END ? EX_END : TY_END;
  static constexpr int PRV = MAIN;                            // uint16 [P][kMaxK] private parts
  static constexpr int SHL = PRV + P * kMaxK * 2;             // uint16 [kMaxK] shared by all parts
  static constexpr int KBM = SHL + kMaxK * 2;                 // u32 [P][32] kept bitmaps
  static constexpr int ITB = KBM + P * 32 * 4;                // u32 [32] intersection bitmap
  static constexpr int TYL = ITB + 32 * 4;                    // uint16 [1024] Taylor union
  static constexpr int CNT = TYL + 1024 * 2;                  // int [16]
  static constexpr int TOTAL = CNT + 64;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  static constexpr int STGCH = STG_BYTES / 1024;               // staging kilobytes per batch
  static_assert(CPS % (NW / 2) == 0 && HCH % (NW / 2) == 0 && STGCH % (NW / 2) == 0,
                "DMA must split evenly over the issuing waves");
  static_assert(kNB * (D / 8) <= NT / 2 && 2 * D <= NT / 2, "a table unit per thread, in either half");
};

// Instruction order of a pipelined step, for the scheduler: a few LDS reads
// up front, then every MFMA followed by one LDS read, TPM exponentials and
// VPM other VALU instructions of the current step's softmax, so the matrix
// core and the VALU of a wave stay busy together.
template <int NM, int ND, int TPM, int VPM>
PISA_DEV void interleave_step() {
  __builtin_amdgcn_sched_group_barrier(0x100, ND - NM, 0);   // DS reads
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // DS read
    __builtin_amdgcn_sched_group_barrier(0x400, TPM, 0);     // transcendental
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);     // other VALU
  }
}

struct Item {
  int key0;    // first key of the step's sub-tile
  int reg;     // LDS region (part) holding it
  bool mem;    // this wave's rows use it
  bool full;   // no causal or ragged-tail mask needed
};

// LONG: kept lists of more than 64 blocks (entries past 64 read from LDS);
// shorter lists take the variant without that path.
template <int D, int BS, bool LONG>
__global__ __launch_bounds__(NT, 1) void attn_blocks(AttnArgs a) {
  using C = Cfg<D, BS>;
  constexpr int P = C::P, WPP = C::WPP, SK = C::SK, SPB = C::SPB, NQT = C::NQT, NE = C::NE;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const PisaDims &dm = a.dm;
  const int tid = threadIdx.x, l = tid & 63, lq = l & 31, hl = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- workgroup -> (b, kv head, head group, tile of TB block rows)
  const int G = dm.ratio < P ? dm.ratio : P;   // query heads per workgroup
  const int TB = P / G;                        // block rows per workgroup
  const int ngrp = dm.ratio / G;
  const int ntile = (dm.n_blk + TB - 1) / TB;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  // causal rows take longer the later their tokens (more Taylor blocks):
  // the longest tiles first, so the grid does not end on them
  const int tile = dm.causal ? ntile - 1 - logical % ntile : logical % ntile;
  const int rest = logical / ntile;
  const int grp = rest % ngrp;
  const int bk = rest / ngrp;
  const int b = bk / dm.Hkv, hk = bk % dm.Hkv;
  // ---- wave -> part (head, block row) and 32 of its rows
  const int part = w / WPP, rg = w % WPP;
  const int h = hk * dm.ratio + grp * G + part / TB;
  const int iblk = tile * TB + part % TB;
  const bool pvalid = iblk < dm.n_blk;
  const int t = iblk * BS + rg * 32 + lq;
  const bool valid = t < dm.L;
  const bool causal = dm.causal != 0;
  const int taylor = dm.taylor;
  int own, lo;
  const int nc = pisa_row_geometry(dm, iblk * BS, &own, &lo);

  uint16_t *prv = reinterpret_cast<uint16_t *>(lds + C::PRV);
  uint16_t *shl = reinterpret_cast<uint16_t *>(lds + C::SHL);
  uint32_t *kbm = reinterpret_cast<uint32_t *>(lds + C::KBM);
  uint32_t *itb = reinterpret_cast<uint32_t *>(lds + C::ITB);
  uint16_t *tyl = reinterpret_cast<uint16_t *>(lds + C::TYL);
  int *cnt = reinterpret_cast<int *>(lds + C::CNT);   // [p] private counts, [4] shared, [7] Taylor

  // ---- 1. kept lists per part; blocks kept by every part (walked once, in
  // one shared LDS region) and each part's private rest; union of the
  // parts' Taylor sets.  The kept set is the set of list entries that are
  // candidates of the row, 0 <= j < nc: other entries (padding, blocks of the
  // window range or past it, garbage in a caller's list) are dropped, and the
  // lists are rebuilt ascending from bitmaps, so order and repeats do not
  // matter.  The part's first wave reads the list, one entry per lane.
  for (int i = tid; i < P * 32; i += NT) kbm[i] = 0;
  const bool lister = rg == 0 && pvalid && a.idx && dm.topk > 0;
  const int32_t *lrow = lister ? a.idx + ((size_t)(b * dm.Hq + h) * dm.n_rows + iblk) * dm.topk : nullptr;
  const int j0 = lister && l < dm.topk ? lrow[l] : -1;

  // ---- 2. Q fragments (B operand: query lq, features 16 ks + 8 hl .. + 7),
  // issued here so that they land during the list work (the barriers below
  // wait for LDS operations only)
  const uint16_t *Qh = static_cast<const uint16_t *>(a.Q) + ((size_t)(b * dm.Hq + h) * dm.L) * D;
  u32x4_t qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = valid ? *reinterpret_cast<const u32x4_t *>(Qh + (size_t)t * D + ks * 16 + hl * 8)
                   : u32x4_t{0, 0, 0, 0};
  lds_barrier();   // the bitmaps are cleared
  if (lister) {
    if (pisa_list_entry_kept(j0, nc)) atomicOr(&kbm[part * 32 + (j0 >> 5)], 1u << (j0 & 31));
    if (LONG)
      for (int k = 64 + l; k < dm.topk; k += 64) {
        const int j = lrow[k];
        if (pisa_list_entry_kept(j, nc)) atomicOr(&kbm[part * 32 + (j >> 5)], 1u << (j & 31));
      }
  }
  lds_barrier();
  if (w == 0) {
    const int nwords = (dm.n_blk + 31) >> 5;
    uint32_t ib = l < nwords ? 0xFFFFFFFFu : 0u, tb = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int ip = tile * TB + p % TB;
      if (ip >= dm.n_blk) continue;
      const uint32_t kw = l < nwords ? kbm[p * 32 + l] : 0u;
      ib &= kw;
      if (taylor) {
        int o2, l2;
        const int nc2 = pisa_row_geometry(dm, ip * BS, &o2, &l2) - l * 32;
        const uint32_t rm = nc2 >= 32 ? 0xFFFFFFFFu : (nc2 > 0 ? (1u << nc2) - 1u : 0u);
        tb |= rm & ~kw;
      }
    }
    if (l < 32) itb[l] = ib;
    const int ci = __popc(ib), ct = __popc(tb);
    const int ii = wave_incl_scan(ci), it = wave_incl_scan(ct);
    int pi = ii - ci, pt = it - ct;
    for (uint32_t m = ib; m; m &= m - 1) shl[pi++] = (uint16_t)(l * 32 + __ffs(m) - 1);
    for (uint32_t m = tb; m; m &= m - 1) tyl[pt++] = (uint16_t)(l * 32 + __ffs(m) - 1);
    if (l == 63) {
      cnt[4] = ii;
      cnt[7] = it;
    }
  }
  lds_barrier();
  if (rg == 0) {   // the part's private blocks: kept, not by every part; word l on lane l
    const uint32_t pw = l < 32 ? kbm[part * 32 + l] & ~itb[l] : 0u;
    const int cp = __popc(pw), ip = wave_incl_scan(cp);
    int pos = ip - cp;
    for (uint32_t m = pw; m; m &= m - 1) prv[part * kMaxK + pos++] = (uint16_t)(l * 32 + __ffs(m) - 1);
    if (l == 63) cnt[part] = ip;
  }
  lds_barrier();
  const int cnt_me = __builtin_amdgcn_readfirstlane(cnt[part]);   // private blocks of this part
  const int n_ty = __builtin_amdgcn_readfirstlane(cnt[7]);
  const int n_s = __builtin_amdgcn_readfirstlane(cnt[4]) * SPB;      // shared steps
  int n_t = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) n_t = max(n_t, __builtin_amdgcn_readfirstlane(cnt[p]));
  n_t *= SPB;                                                         // private steps
  // causal window range of the workgroup's block rows (contiguous)
  int wlo = 0, n_w = 0;
  if (causal) {
    const int i0 = tile * TB, i1 = min(tile * TB + TB, dm.n_blk) - 1;
    int o0, l0;
    pisa_row_geometry(dm, i0 * BS, &o0, &l0);
    wlo = l0;
    n_w = (i1 - l0 + 1) * SPB;
  }
  const int n = n_w + n_s + n_t;
  const int n_one = n_w + n_s;   // steps with one region shared by all parts

  f32x16_t oacc[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) oacc[i] = f32x16_t{};
  float m_run = kNegInf, d_run = 0.f;
  const float sl2 = a.sl2;

  const size_t kvoff = ((size_t)(b * dm.Hkv + hk) * dm.L) * D;
  const uint16_t *Kh = static_cast<const uint16_t *>(a.K) + kvoff;
  const uint16_t *Vh = static_cast<const uint16_t *>(a.V) + kvoff;
  const int srow = (l & 15) >> 2;
  const int ecol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  // ---- 3. exact phase
  if (n > 0) {
    // The DMA of a step is issued by waves 0..NW/2-1 only (kilobyte
    // w + NDW uu of each part's sub-tile, uu < UPP): while they drain it
    // through the CU's load path, the other wave on each SIMD already runs
    // its MFMA block, and the two swap roles within the step.  The per-lane
    // source offsets (bytes from the sub-tile's first key) never change.
    constexpr int NDW = NW / 2;           // DMA-issuing waves
    constexpr int UPP = C::CPS / NDW;     // kilobytes of one sub-tile per issuing wave
    const bool dma_wave = w < NDW;
    int offk[UPP], offv[UPP];
#pragma unroll
    for (int u = 0; u < UPP; ++u) {
      const int pos = ((w % NDW) + NDW * u) * 64 + l;
      const int row = pos / (D / 8), phys = pos % (D / 8);
      offk[u] = (row * D + ((phys ^ kswz<D>(row)) << 3)) * 2;
      offv[u] = (row * D + ((phys ^ vswz<D>(row)) << 3)) * 2;
    }
    // the block lists' first 64 entries live in VGPRs, entry e in lane e; a
    // step reads its entry with v_readlane (entries past 64, for lists of
    // more than 64 blocks, from LDS)
    int cnt_s[P], vprv[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      cnt_s[p] = __builtin_amdgcn_readfirstlane(cnt[p]);
      vprv[p] = l < cnt_s[p] ? (int)prv[p * kMaxK + l] : 0;
    }
    const int vshl = l < n_s / SPB ? (int)shl[l] : 0;
    int vme = vprv[0];   // this wave's own private list
#pragma unroll
    for (int p = 1; p < P; ++p)
      if (part == p) vme = vprv[p];
    // first key of the sub-tile of a step with one region: window steps,
    // then the shared blocks
    auto key0_one = [&](int s) -> int {
      const int s1 = s - n_w;
      const int e = s1 / SPB;
      const int jw = wlo + s / SPB;
      const int js = (!LONG || e < 64) ? __builtin_amdgcn_readlane(vshl, e & 63) : (int)shl[e];
      return (s < n_w ? jw * BS + (s % SPB) * SK : js * BS + (s1 % SPB) * SK);
    };
    // ... of part p's sub-tile in a private step (idle parts load block 0,
    // finite data that their zero weights ignore)
    auto key0_prv = [&](int s, int vlist, int count, int p) -> int {
      const int s2 = s - n_one, bi = s2 / SPB;
      const int j = (!LONG || bi < 64) ? __builtin_amdgcn_readlane(vlist, bi & 63)
                                       : bi < count ? (int)prv[p * kMaxK + bi] : 0;
      return (bi < count ? j : 0) * BS + (s2 % SPB) * SK;
    };
    // K (isv false) or V sub-tiles of step s into the ring slot at byte offset base
    auto dma_step = [&](int s, bool isv, int base) {
      if (!dma_wave) return;
      const uint16_t *g = isv ? Vh : Kh;
      if (s < n_one) {
        const int k0 = key0_one(s);
#pragma unroll
        for (int u = 0; u < UPP; ++u)
          dma16_buf(g + (size_t)k0 * D, max(dm.L - k0, 0) * D * 2, isv ? offv[u] : offk[u],
                    lds + base + (w + NDW * u) * 1024);
      } else {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const int k0 = key0_prv(s, vprv[p], cnt_s[p], p);
#pragma unroll
          for (int u = 0; u < UPP; ++u)
            dma16_buf(g + (size_t)k0 * D, max(dm.L - k0, 0) * D * 2, isv ? offv[u] : offk[u],
                      lds + base + p * C::SUB + (w + NDW * u) * 1024);
        }
      }
    };
    auto info = [&](int s) -> Item {
      Item it;
      const bool win = s < n_w, one = s < n_one;
      const int jw = wlo + s / SPB;
      it.key0 = one ? key0_one(s) : key0_prv(s, vme, cnt_me, part);
      it.reg = one ? 0 : part;
      it.mem = win ? (pvalid && jw >= lo && jw <= own) : (one ? pvalid : (s - n_one) / SPB < cnt_me);
      it.full = it.key0 + SK <= dm.L && !(win && causal && jw == own);
      return it;
    };
    auto scores = [&](const uint8_t *kt, f32x16_t (&s)[NQT]) {
#pragma unroll
      for (int q = 0; q < NQT; ++q) {
        s[q] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) s[q] = mfma32(frag_a<D>(kt, q * 32 + lq, 2 * ks + hl), qf[ks], s[q]);
      }
    };

    // V slot 1 starts as zeros: step 0 multiplies it by an all-zero P
    for (int i = tid; i < C::SLOT / 16; i += NT)
      reinterpret_cast<u32x4_t *>(lds + C::EX_V + C::SLOT)[i] = u32x4_t{0, 0, 0, 0};
    dma_step(0, false, C::EX_K);
    if (n > 1) dma_step(1, false, C::EX_K + C::SLOT);
    wait_vmcnt<0>();
    __syncthreads();

    f32x16_t sa[NQT], sb[NQT];
    u32x4_t pprev[NQT][2];
#pragma unroll
    for (int q = 0; q < NQT; ++q) pprev[q][0] = pprev[q][1] = u32x4_t{0, 0, 0, 0};
    {
      const Item c0 = info(0);
      scores(lds + C::EX_K + c0.reg * C::SUB, sa);
    }

    // softmax weights of the current step against the running max reference
    auto weights = [&](const f32x16_t (&sc)[NQT], float mneg, u32x4_t (&pc)[NQT][2]) -> float {
      float psum = 0.f;
#pragma unroll
      for (int q = 0; q < NQT; ++q) {
        f32x16_t e;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(sc[q][r], sl2, mneg));
        pc[q][0] = pack8(e, 0);
        pc[q][1] = pack8(e, 8);
        psum = sum_bf16x8_f(pc[q][0], psum);
        psum = sum_bf16x8_f(pc[q][1], psum);
      }
      return psum;
    };

    auto step = [&](int i, f32x16_t (&sc)[NQT], f32x16_t (&sn)[NQT]) {
      wait_vmcnt<0>();   // K_{i+1} and V_{i-1} have landed (this wave's share)
      __syncthreads();   // ... for every wave; K slot i%2 and V slot i%2 are free
      if (i + 2 < n) dma_step(i + 2, false, C::EX_K + (i & 1) * C::SLOT);
      dma_step(i, true, C::EX_V + (i & 1) * C::SLOT);
      const Item cur = info(i);
      const Item nxt = info(i + 1 < n ? i + 1 : i);
      const Item prv = info(i > 0 ? i - 1 : 0);
      // causal diagonal / ragged tail: mask in place
      if (cur.mem && !cur.full) {
        const int lim = min(causal ? t : dm.L - 1, dm.L - 1) - cur.key0 - 4 * hl;
#pragma unroll
        for (int q = 0; q < NQT; ++q)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (q * 32 + 8 * (r >> 2) + (r & 3) > lim) sc[q][r] = kNegInf;
      }
      const float mold = m_run;
      const float mneg = cur.mem ? -(mold == kNegInf ? 0.f : mold) : kNegInf;
      // One block, scheduled by hand: MFMA k of S_{i+1} = K_{i+1} Q^T and of
      // P_{i-1} V_{i-1}, the LDS reads of the fragment three MFMAs ahead, and
      // E softmax elements of step i (max, exponential, bf16 pair, row sum),
      // so the matrix core and the VALU of the wave work side by side.
      const uint8_t *kt = lds + C::EX_K + ((i + 1) & 1) * C::SLOT + nxt.reg * C::SUB;
      const uint8_t *vt = lds + C::EX_V + ((i + 1) & 1) * C::SLOT + prv.reg * C::SUB;
      constexpr int KS = D / 16, NS = NQT * KS, NM = NS + NQT * 2 * NE, E = NQT * 16 / NM;
      static_assert(E * NM == NQT * 16, "softmax elements must split evenly over the MFMAs");
      auto frag = [&](int k) -> u32x4_t {
        if (k < NS) return frag_a<D>(kt, (k / KS) * 32 + lq, 2 * (k % KS) + hl);
        const int k2 = k - NS, q = k2 / (2 * NE), hf = (k2 / NE) % 2, et = k2 % NE;
        return frag_vt<D>(vt, q * 32 + 16 * hf + 4 * hl + srow, et * 32 + ecol);
      };
      u32x4_t fr[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) fr[k] = frag(k);
      const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
      float mx = kNegInf, psum = 0.f, ehold = 0.f;
      u32x4_t pc[NQT][2];
#pragma unroll
      for (int k = 0; k < NM; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        if (k < NS) {
          const int q = k / KS, ks = k % KS;
          sn[q] = mfma32(fr[k % 3], qf[ks], ks == 0 ? f32x16_t{} : sn[q]);
        } else {
          const int k2 = k - NS, q = k2 / (2 * NE), hf = (k2 / NE) % 2, et = k2 % NE;
          oacc[et] = mfma32(fr[k % 3], pprev[q][hf], oacc[et]);
        }
        if (k + 3 < NM) fr[k % 3] = frag(k + 3);
#pragma unroll
        for (int u = 0; u < E; ++u) {
          const int el = k * E + u, q = el / 16, r = el % 16;
          const float x = sc[q][r];
          const float e = fast_exp2(fmaf(x, sl2, mneg));
          if (el & 1) {
            mx = fmaxf(fmaxf(mx, sc[q][r - 1]), x);
            const f32x2_t v2 = {ehold, e};
            const bf16x2_t b2 = __builtin_convertvector(v2, bf16x2_t);
            pc[q][r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, b2);
            psum = __builtin_amdgcn_fdot2_f32_bf16(b2, one2, psum, false);
          } else {
            ehold = e;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // keep this computation here (it must not be merged into the rare
      // recomputation below)
      asm volatile("" : "+v"(psum), "+v"(mx));
      // the max moved by more than 2^8 (or the row's first visible step):
      // rescale and recompute this step's weights
      mx = pair_max_f(mx);
      const float ms = cur.mem ? mx * sl2 : kNegInf;
      const bool grow = ms > mold + kRescale;
      if (ballot64(grow)) {
        const float corr = grow ? fast_exp2(mold - ms) : 1.f;
        m_run = grow ? ms : mold;
        d_run *= corr;
#pragma unroll
        for (int et = 0; et < NE; ++et) oacc[et] *= corr;
        psum = weights(sc, cur.mem ? -(m_run == kNegInf ? 0.f : m_run) : kNegInf, pc);
      }
      d_run += pair_sum_f(psum);
#pragma unroll
      for (int q = 0; q < NQT; ++q) {
        pprev[q][0] = pc[q][0];
        pprev[q][1] = pc[q][1];
      }
    };

    for (int i = 0; i < n; i += 2) {
      step(i, sa, sb);
      if (i + 1 >= n) break;
      step(i + 1, sb, sa);
    }
    // drain: P_{n-1} V_{n-1}
    wait_vmcnt<0>();
    __syncthreads();
    {
      const Item last = info(n - 1);
      const uint8_t *vt = lds + C::EX_V + ((n - 1) & 1) * C::SLOT + last.reg * C::SUB;
#pragma unroll
      for (int q = 0; q < NQT; ++q)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r1 = q * 32 + 16 * hf + 4 * hl + srow;
#pragma unroll
          for (int et = 0; et < NE; ++et)
            oacc[et] = mfma32(frag_vt<D>(vt, r1, et * 32 + ecol), pprev[q][hf], oacc[et]);
        }
    }
    __syncthreads();   // the Taylor phase reuses the rings' LDS
  }

  // ---- 4. Taylor phase: union of the parts' Taylor blocks
  if (taylor && n_ty > 0) {
    const size_t soff = (size_t)(b * dm.Hkv + hk) * dm.n_blk;
    const float *kbar = a.kbar + soff * D;
    const float *vsum = a.vsum + soff * D;
    const uint16_t *HTh = static_cast<const uint16_t *>(a.HT) + soff * D * D;
    uint8_t *kbh = lds + C::TY_KBH, *kbl = lds + C::TY_KBL;
    uint8_t *sth = lds + C::TY_STH, *stl = lds + C::TY_STL;
    uint16_t *alp = reinterpret_cast<uint16_t *>(lds + C::TY_AL) + w * kNB * 32;
    float *nj = reinterpret_cast<float *>(lds + C::TY_NJ);
    const uint32_t *kb_me = kbm + part * 32;
    const bool order1 = taylor == 2, hybrid = taylor == 3;
    float a_run = 0.f;   // hybrid: sum of this row's Taylor weights, on the scale of d_run
    // Loads of the Taylor phase are issued by waves 0..NDW-1 (as in the exact
    // phase): H_j tiles (PH kilobytes per issuing wave) and, half a batch
    // ahead, the next batch's kbar and vsum rows into an LDS staging area.
    constexpr int NDW = NW / 2, PH = C::HCH / NDW, PS = C::STGCH / NDW;
    const bool issuer = w < NDW;
    int offh[PH];
#pragma unroll
    for (int u = 0; u < PH; ++u) {
      const int pos = (w % NDW + NDW * u) * 64 + l;
      const int row = pos / (D / 8), phys = pos % (D / 8);
      offh[u] = (row * D + ((phys ^ kswz<D>(row)) << 3)) * 2;
    }
    auto dma_h = [&](int eg) {
      if (!issuer) return;
      const uint16_t *src = HTh + (size_t)__builtin_amdgcn_readfirstlane(tyl[eg]) * D * D;
      uint8_t *dst = lds + C::TY_H + (eg % C::RINGH) * C::HT;
#pragma unroll
      for (int u = 0; u < PH; ++u) dma16_buf(src, D * D * 2, offh[u], dst + (w + NDW * u) * 1024);
    };
    // staging kilobyte c holds rows c * RPC .. of [kbar entries | vsum entries]
    constexpr int RPC = 1024 / (D * 4), LPR = 64 / RPC;   // rows per kilobyte, lanes per row
    const int tbl_bytes = dm.n_blk * D * 4;
    uint8_t *stgb = lds + (order1 ? C::TY_KBH : C::TY_H + C::HT);
    auto stage = [&](int b0) {
      if (!issuer) return;
      const int nb = min(kNB, n_ty - b0);
#pragma unroll
      for (int u = 0; u < PS; ++u) {
        const int c = w + NDW * u;
        const int row = c * RPC + l / LPR;             // 0 .. 2 kNB - 1
        const int en = row % kNB;
        const int j = tyl[b0 + min(en, nb - 1)];
        const int voff = en < nb ? j * D * 4 + (l % LPR) * 16 : tbl_bytes;   // past the end: zeros
        dma16_buf(row < kNB ? (const void *)kbar : (const void *)vsum, tbl_bytes, voff,
                  stgb + c * 1024);
      }
    };
    stage(0);
    if (order1) {
      for (int i = 0; i < C::AHEAD * C::GE && i < n_ty; ++i) dma_h(i);
    } else if (hybrid && !causal && issuer) {   // the mean matrix Hbar^T of this kv head, into ring slot 0
      const uint16_t *src = static_cast<const uint16_t *>(a.HT) + hbar_offset(dm, b * dm.Hkv + hk, 0);
#pragma unroll
      for (int u = 0; u < PH; ++u) dma16_buf(src, D * D * 2, offh[u], lds + C::TY_H + (w + NDW * u) * 1024);
    }
    const float *stg = reinterpret_cast<const float *>(stgb);
    // Taylor tables of the batch that starts at entry b0, from its staged
    // kbar / vsum rows: kbar as bf16 hi + lo rows (swizzled like K tiles),
    // Sigma^T as bf16 hi and lo in the perm16 layout, and n_j.  At first
    // order the waves that issue no DMA build both tables (thread
    // (tid + NT / 2) % NT), between the group barriers; otherwise the two
    // tables are split between the two halves of the workgroup.  Every
    // thread calls it: at first order the staged rows overlay the tables, so
    // all of them are read before the workgroup meets and any is written.
    auto build = [&](int b0) {
      const int nb = min(kNB, n_ty - b0);
      const int bt = (tid + NT / 2) % NT;
      // without first order every wave builds: the kbar rows on waves 0 ..
      // NW / 2 - 1, Sigma^T on the others
      const int bk2 = order1 ? bt : tid, bs2 = order1 ? bt : tid - NT / 2;
      // kbar rows: thread (entry en, 16-byte chunk ch)
      const bool act = bk2 >= 0 && bk2 < kNB * (D / 8) && (order1 || tid < NT / 2);
      const int en = bk2 / (D / 8), ch = bk2 % (D / 8);
      u32x4_t hi = {0, 0, 0, 0}, lo4 = {0, 0, 0, 0};
      float njv = 0.f;
      if (act && en < nb) {
        const int j = tyl[b0 + en];
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t *>(stg + en * D + ch * 8);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t *>(stg + en * D + ch * 8 + 4);
        const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t pk = pack_bf16x2(x[2 * i], x[2 * i + 1]);
          hi[i] = pk;
          lo4[i] = pack_bf16x2(x[2 * i] - bf16lo(pk), x[2 * i + 1] - bf16hi(pk));
        }
        njv = (float)min(dm.bs, dm.L - j * dm.bs);
      }
      // Sigma^T [feature][16 entries]: entry en at K position perm16(en),
      // the two 16-byte halves of a row swapped on odd groups of 8 rows.
      // Thread (feature f, physical half ph) gathers the eight entries of
      // that half from the staged vsum rows and writes them in one piece.
      const bool acts = bs2 >= 0 && bs2 < 2 * D && (order1 || tid >= NT / 2);
      const int f = bs2 >> 1, ph = bs2 & 1;
      const int lh = ph ^ ((f >> 3) & 1);   // logical half: K positions 8 lh .. 8 lh + 7
      u32x4_t shi = {0, 0, 0, 0}, slo = {0, 0, 0, 0};
      if (acts) {
        float sv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int e2 = perm16(8 * lh + k);
          sv[k] = e2 < nb ? stg[(kNB + e2) * D + f] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t pk = pack_bf16x2(sv[2 * i], sv[2 * i + 1]);
          shi[i] = pk;
          slo[i] = pack_bf16x2(sv[2 * i] - bf16lo(pk), sv[2 * i + 1] - bf16hi(pk));
        }
      }
      if (order1) lds_barrier();
      if (act) {
        if (ch == 0) nj[en] = njv;
        const int sw = (ch ^ kswz<D>(en)) << 4;
        *reinterpret_cast<u32x4_t *>(kbh + en * (2 * D) + sw) = hi;
        *reinterpret_cast<u32x4_t *>(kbl + en * (2 * D) + sw) = lo4;
      }
      if (acts) {
        *reinterpret_cast<u32x4_t *>(sth + f * (2 * kNB) + (ph << 4)) = shi;
        *reinterpret_cast<u32x4_t *>(stl + f * (2 * kNB) + (ph << 4)) = slo;
      }
    };
    uint32_t tmask = 0;
    // one Taylor entry (first order), or one batch start (the other orders)
    auto entry = [&](int eg) {
      const int e = eg % kNB;
      if (e == 0) {
        const int nb = min(kNB, n_ty - eg);
        // first order: the tables of every batch after the first were built
        // about half a batch earlier, between per-group barriers; the first
        // batch, and the orders without those barriers, build them here once
        // the staged rows have landed
        if (!order1 || eg == 0) {
          // the staged rows were issued before the first two groups' H tiles
          if (order1 && n_ty >= C::AHEAD * C::GE) wait_vmcnt<C::AHEAD * C::GE * PH>();
          else wait_vmcnt<0>();
          lds_barrier();   // the previous batch's tables are consumed; staging landed
          build(eg);
          lds_barrier();
          // without first order the next batch's rows go to the staging
          // area now (build read this batch's), to land during this batch
          if (!order1 && eg + kNB < n_ty) stage(eg + kNB);
        }
        {   // lane en < nb decides entry en for this wave's part
          bool mine = false;
          if (pvalid && l < nb) {
            const int j = tyl[eg + l];
            mine = j < nc && !((kb_me[j >> 5] >> (j & 31)) & 1u);
          }
          tmask = (uint32_t)ballot64(mine);
        }
        if (tmask) {
          // A rows 0..15 are the entries' kbar hi parts, rows 16..31 their lo
          // parts: entry en's logit is the sum of result rows en and en + 16
          f32x16_t at = f32x16_t{};
          const uint8_t *kbs = lq < 16 ? kbh : kbl;
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) at = mfma32(frag_a<D>(kbs, lq & 15, 2 * ks + hl), qf[ks], at);
#pragma unroll
          for (int r = 0; r < 8; ++r) at[r] += at[r + 8];
          // entries 0..15 sit in registers 0..7: entry 8 (r / 4) + 4 hl + r % 4
          float mx = kNegInf;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int en = 8 * (r >> 2) + 4 * hl + (r & 3);
            const float x = ((tmask >> en) & 1u) ? at[r] * sl2 : kNegInf;
            at[r] = x;
            mx = fmaxf(mx, x);
          }
          mx = pair_max_f(mx);
          const bool grow = mx > m_run + kRescale;
          if (ballot64(grow)) {
            const float corr = grow ? fast_exp2(m_run - mx) : 1.f;
            d_run *= corr;
            a_run *= corr;
#pragma unroll
            for (int et = 0; et < NE; ++et) oacc[et] *= corr;
            m_run = grow ? mx : m_run;
          }
          const float mref = m_run == kNegInf ? 0.f : m_run;
          float dpart = 0.f, apart = 0.f;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int en = 8 * (r >> 2) + 4 * hl + (r & 3);
            const float al = fast_exp2(at[r] - mref);
            at[r] = al;
            dpart += al * nj[en];
            apart += al;
            if (order1) alp[en * 32 + lq] = (uint16_t)f32_to_bf16(al * dm.scale);
          }
          dpart = pair_sum_f(dpart);
          d_run += dpart;
          if (hybrid) a_run += pair_sum_f(apart);
          u32x4_t ph, pl;
          pack8_split(at, 0, ph, pl);
          // zero order: O^T += Sigma^T alpha^T  (hi*hi + lo*hi + hi*lo)
#pragma unroll
          for (int et = 0; et < NE; ++et) {
            const int f = et * 32 + lq;
            const int off = f * (2 * kNB) + ((hl ^ ((f >> 3) & 1)) << 4);
            const u32x4_t sh = *reinterpret_cast<const u32x4_t *>(sth + off);
            const u32x4_t sl = *reinterpret_cast<const u32x4_t *>(stl + off);
            oacc[et] = mfma32(sh, ph, oacc[et]);
            oacc[et] = mfma32(sl, ph, oacc[et]);
            oacc[et] = mfma32(sh, pl, oacc[et]);
          }
        }
      }
      // the next batch's kbar / vsum rows, about half a batch ahead (this
      // batch's tables were built before the batch-start barrier)
      const bool staging = order1 && e == C::SG * C::GE && eg - e + kNB < n_ty;
      if (staging) stage(eg - e + kNB);
      if (!order1) return;
      // first order for entry eg: H ring of groups of GE entries, the group
      // in use and AHEAD groups in flight; one barrier per group
      if (e % C::GE == 0) {
        // wait for this group's tiles: later groups' tiles (issued after them)
        // and the rows just staged may stay in flight; a short next group
        // (the phase's end) is waited for too
        if (eg + C::AHEAD * C::GE <= n_ty) {
          if (staging) wait_vmcnt<(C::AHEAD - 1) * C::GE * PH + PS>();
          else wait_vmcnt<(C::AHEAD - 1) * C::GE * PH>();
        } else {
          wait_vmcnt<0>();
        }
        // the group's H tiles landed for all waves; the previous group's slots
        // are free (the next group's tiles stay in flight)
        lds_barrier();
        for (int i = 0; i < C::GE && eg + C::AHEAD * C::GE + i < n_ty; ++i) dma_h(eg + C::AHEAD * C::GE + i);
      }
      if ((tmask >> e) & 1u) {
        // u = H_j^T Q^T tile by tile (MFMA k: output tile k / KS, K-step
        // k % KS), scheduled by hand: the LDS read of the fragment four MFMAs
        // ahead, and chunk c of O += (alpha scale) u, 16 / KS values of tile
        // c / KS, two MFMAs after that tile's last MFMA.
        const uint8_t *hp = lds + C::TY_H + (eg % C::RINGH) * C::HT;
        const float al = bf16_to_f32(alp[e * 32 + lq]);
        constexpr int KS = D / 16, NMT = NE * KS, FPC = 16 / KS;
        auto hfrag = [&](int k) { return frag_a<D>(hp, (k / KS) * 32 + lq, 2 * (k % KS) + hl); };
        auto fchunk = [&](const f32x16_t (&uu)[NE], int c) {
#pragma unroll
          for (int i = 0; i < FPC; ++i) {
            const int et = c / KS, r = (c % KS) * FPC + i;
            oacc[et][r] = fmaf(al, uu[et][r], oacc[et][r]);
          }
        };
        u32x4_t fr[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) fr[k] = hfrag(k);
        f32x16_t u[NE];
#pragma unroll
        for (int k = 0; k < NMT; ++k) {
          __builtin_amdgcn_sched_barrier(0);
          const int et = k / KS, ks = k % KS;
          u[et] = mfma32(fr[k % 4], qf[ks], ks == 0 ? f32x16_t{} : u[et]);
          if (k + 4 < NMT) fr[k % 4] = hfrag(k + 4);
          if (k >= KS + 1) fchunk(u, k - KS - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = NMT - KS - 1; c < NMT; ++c) fchunk(u, c);
      }
      // the next batch's tables, at the end of group SG + 1: its staged rows
      // landed before this group's barrier (they were issued ahead of the
      // following group's H tiles), this batch's tables were read before the
      // batch's first barrier, and the barrier of group SG + 2 publishes them
      if (e == (C::SG + 1) * C::GE + C::GE - 1 && eg - e + kNB < n_ty) build(eg - e + kNB);
    };
    // first order walks the entries one by one; the other orders only have
    // batch starts, so they step a batch at a time
    if (order1) {
      for (int eg = 0; eg < n_ty; ++eg) entry(eg);
    } else {
      for (int eg = 0; eg < n_ty; eg += kNB) entry(eg);
    }
    if (hybrid) {   // O^T += (scale sum alpha) Hbar^T Q^T, once per row
      wait_vmcnt<0>();
      __syncthreads();
      if (causal) {
        // causal rows: the mean over each block row's candidates [0, lo),
        // the TB block rows' matrices into ring slots 0 .. TB - 1
        if (issuer) {
          for (int p = 0; p < TB; ++p) {
            const int ip = tile * TB + p;
            int o2, l2 = 0;
            if (ip < dm.n_blk) pisa_row_geometry(dm, ip * BS, &o2, &l2);
            const uint16_t *src = static_cast<const uint16_t *>(a.HT) + hbar_offset(dm, b * dm.Hkv + hk, l2);
#pragma unroll
            for (int u = 0; u < PH; ++u)
              dma16_buf(src, D * D * 2, offh[u], lds + C::TY_H + p * C::HT + (w + NDW * u) * 1024);
          }
        }
        wait_vmcnt<0>();
        __syncthreads();
      }
      const uint8_t *hp = lds + C::TY_H + (causal ? (part % TB) * C::HT : 0);
      const float al = a_run * dm.scale;
#pragma unroll
      for (int et = 0; et < NE; ++et) {
        f32x16_t u = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) u = mfma32(frag_a<D>(hp, et * 32 + lq, 2 * ks + hl), qf[ks], u);
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[et][r] = fmaf(al, u[r], oacc[et][r]);
      }
    }
  }

  // ---- 5. epilogue: O = N / D in bf16, lse
  if (valid) {
    const float inv = 1.f / d_run;
    uint16_t *Oh = static_cast<uint16_t *>(a.O) + ((size_t)(b * dm.Hq + h) * dm.L + t) * D;
#pragma unroll
    for (int et = 0; et < NE; ++et)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = et * 32 + 8 * g + 4 * hl;
        u32x2_t o;
        o[0] = pack_bf16x2(oacc[et][4 * g] * inv, oacc[et][4 * g + 1] * inv);
        o[1] = pack_bf16x2(oacc[et][4 * g + 2] * inv, oacc[et][4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t *>(Oh + e) = o;
      }
    if (a.lse && hl == 0) a.lse[(size_t)(b * dm.Hq + h) * dm.L + t] = (m_run + log2f(d_run)) * kLn2;
  }
}

template <int D, int BS, bool LONG>
hipError_t launch_v(const AttnArgs &a, hipStream_t st) {
  using C = Cfg<D, BS>;
  const PisaDims &dm = a.dm;
  const int G = dm.ratio < C::P ? dm.ratio : C::P;
  const int TB = C::P / G;
  const unsigned grid = (unsigned)dm.B * dm.Hkv * (dm.ratio / G) * ((dm.n_blk + TB - 1) / TB);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_blocks<D, BS, LONG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::TOTAL);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  attn_blocks<D, BS, LONG><<<grid, NT, C::TOTAL, st>>>(a);
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch(const AttnArgs &a, hipStream_t st) {
  // the kernels take topk as the width of a kept list (topk + sink)
  return a.dm.topk > 64 ? launch_v<D, BS, true>(a, st) : launch_v<D, BS, false>(a, st);
}

}  // namespace

hipError_t launch_attn_blocks(const AttnArgs &a, hipStream_t st) {
  if (a.dm.d == 64) return a.dm.bs == 64 ? launch<64, 64>(a, st) : launch<64, 128>(a, st);
  return a.dm.bs == 64 ? launch<128, 64>(a, st) : launch<128, 128>(a, st);
}
