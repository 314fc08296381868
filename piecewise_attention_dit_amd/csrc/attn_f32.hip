// Stage C, fp32 path: a plain VALU kernel (one wave per query row at a
// time) computing the same definition as the bf16 MFMA kernel -- PISA page,
// section 2: o_t = N_t / D_t with exact terms over the kept blocks and the
// per-block first-order Taylor term for the other candidates (or, in the
// hybrid order, zero order per block plus q Hbar times the blocks' weights).  Used for fp32
// problems, where bf16 MFMA operands would not meet fp32 accuracy.
#include "attn_common.h"

namespace {
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
    float m = kNegInf, dsum = 0.f, asum = 0.f, o[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) o[i] = 0.f;
    // a list entry counts once, and only if it is a candidate of the row
    // (0 <= j < nc): padding, blocks of the window range or past it and
    // repeats are skipped
    auto kept_entry = [&](int i) -> bool {
      const int j = list[i];
      if (!pisa_list_entry_kept(j, nc)) return false;
      for (int i2 = 0; i2 < i; ++i2)
        if (list[i2] == j) return false;
      return true;
    };
    // exact blocks: the kept list, then the window range [lo, own] (causal)
    int li = 0;
    bool range_done = !causal;
    for (;;) {
      int jlo, jhi;
      while (li < dm.topk && !kept_entry(li)) ++li;
      if (li < dm.topk) {
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
      for (int j = 0; j < nc; ++j) {
        bool kept = false;
        for (int i = 0; i < dm.topk; ++i) kept |= list[i] == j;
        if (kept) continue;
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
        asum = asum * corr + al;
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
      if (dm.taylor == 3 && asum > 0.f) {   // hybrid: + (scale sum alpha) q Hbar
        // non-causal: the mean over all blocks; causal: over the row's candidates [0, lo)
        const float *Hb = static_cast<const float *>(a.HT) + hbar_offset(dm, b * dm.Hkv + hk, lo);
#pragma unroll
        for (int i = 0; i < NE; ++i) {
          const int e = l + 64 * i;
          float qh = 0.f;
          for (int c = 0; c < D; ++c) qh = fmaf(qs[w][c], Hb[(size_t)e * D + c], qh);
          o[i] = fmaf(dm.scale * asum, qh, o[i]);
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


// ---------------------------------------------------------------------------
// fp32 path, block rows (group == 0).  A workgroup takes kFR consecutive rows
// of one (batch, head), all inside one query block, so they share the kept
// list, the window range and the Taylor set.  Every K / V chunk of 64 keys,
// every batch of up to 64 Taylor blocks' kbar / vsum rows and every H^T tile
// is staged in LDS once for the kFR rows (K, kbar and H^T rows padded to
// D + 1 floats, so the 64 lanes reading 64 rows at one feature hit 64
// banks), and a wave computes kFW rows together, so each LDS read of a tile
// feeds kFW rows.  Scores: lane = key (or Taylor block); P V and the Taylor
// terms: lane = output feature.
constexpr int kFR = 16;   // rows per workgroup
constexpr int kFW = 4;    // rows per wave

template <int D>
struct F32Lds {
  static constexpr int KP = D + 1;                 // padded pitch (floats)
  static constexpr int KT = 0;                     // float [64][KP]: K chunk / the batch's kbar rows
  static constexpr int VT = KT + 64 * KP * 4;      // float [64][D]: V chunk / the batch's vsum rows
  static constexpr int HTT = VT + 64 * D * 4;      // float [D][KP]: H^T of a Taylor block, or Hbar^T
  static constexpr int QS = HTT + D * KP * 4;      // float [kFR][D]: the rows' queries
  static constexpr int PS = QS + kFR * D * 4;      // float [4 waves][kFW][64]: weights of a chunk / batch
  static constexpr int BM = PS + 4 * kFW * 64 * 4; // u32 [32]: kept bitmap
  static constexpr int XL = BM + 32 * 4;           // int [1024 + 1024]: exact blocks (kept, then the window range)
  static constexpr int TL = XL + 2048 * 4;         // int [1024]: Taylor blocks
  static constexpr int CNT = TL + 1024 * 4;        // int [2]
  static constexpr int TOTAL = CNT + 16;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <int D>
__global__ __launch_bounds__(256) void attn_f32_rows(AttnArgs a) {
  using LY = F32Lds<D>;
  constexpr int NE = D / 64, KP = LY::KP, D4 = D / 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *kt = reinterpret_cast<float *>(lds + LY::KT);
  float *vt = reinterpret_cast<float *>(lds + LY::VT);
  float *ht = reinterpret_cast<float *>(lds + LY::HTT);
  float *qs = reinterpret_cast<float *>(lds + LY::QS);
  uint32_t *bm = reinterpret_cast<uint32_t *>(lds + LY::BM);
  int *xl = reinterpret_cast<int *>(lds + LY::XL);
  int *tl = reinterpret_cast<int *>(lds + LY::TL);
  int *cnt = reinterpret_cast<int *>(lds + LY::CNT);
  const PisaDims &dm = a.dm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  float *ps = reinterpret_cast<float *>(lds + LY::PS) + w * kFW * 64;
  const int nchunk = (dm.L + kFR - 1) / kFR;
  const int chunk = blockIdx.x % nchunk;
  const int bh = blockIdx.x / nchunk;
  const int b = bh / dm.Hq, h = bh % dm.Hq, hk = h * dm.Hkv / dm.Hq;
  const int t0 = chunk * kFR;
  const int r = t0 / dm.bs;   // the query block of all kFR rows (kFR divides the block)
  const bool causal = dm.causal != 0;
  const int taylor = dm.taylor;
  const float sl2 = a.sl2;
  int own, lo;
  const int nc = pisa_row_geometry(dm, r * dm.bs, &own, &lo);
  const float *Q = static_cast<const float *>(a.Q) + (size_t)bh * dm.L * D;
  const size_t kvoff = (size_t)(b * dm.Hkv + hk) * dm.L * D;
  const float *K = static_cast<const float *>(a.K) + kvoff;
  const float *V = static_cast<const float *>(a.V) + kvoff;
  const size_t soff = (size_t)(b * dm.Hkv + hk) * dm.n_blk;

  // ---- kept bitmap (entries that are candidates of the row, once), the rows' queries
  if (tid < 32) bm[tid] = 0u;
  for (int i = tid; i < kFR * D; i += 256) {
    const int t = t0 + i / D;
    qs[i] = t < dm.L ? Q[(size_t)t * D + i % D] : 0.f;
  }
  __syncthreads();
  if (a.idx)
    for (int i = tid; i < dm.topk; i += 256) {
      const int j = a.idx[((size_t)bh * dm.n_rows + r) * dm.topk + i];
      if (pisa_list_entry_kept(j, nc)) atomicOr(&bm[j >> 5], 1u << (j & 31));
    }
  __syncthreads();
  // ---- exact blocks (kept ascending, then the causal window range) and Taylor blocks
  if (w == 0) {
    const uint32_t kw = l < 32 ? bm[l] : 0u;
    const int nbits = nc - 32 * l;
    const uint32_t cm = l < 32 ? (nbits >= 32 ? 0xFFFFFFFFu : (nbits > 0 ? (1u << nbits) - 1u : 0u)) : 0u;
    const uint32_t tw = taylor ? (cm & ~kw) : 0u;
    const int ck = __popc(kw), ct = __popc(tw);
    const int ik = wave_incl_scan(ck), it = wave_incl_scan(ct);
    int pk = ik - ck, pt = it - ct;
    for (uint32_t m = kw; m; m &= m - 1) xl[pk++] = 32 * l + __ffs(m) - 1;
    for (uint32_t m = tw; m; m &= m - 1) tl[pt++] = 32 * l + __ffs(m) - 1;
    if (l == 63) {
      int n = ik;
      if (causal)
        for (int j = lo; j <= min(own, dm.n_blk - 1); ++j) xl[n++] = j;
      cnt[0] = n;
      cnt[1] = it;
    }
  }
  __syncthreads();
  const int nx = cnt[0], nt = cnt[1];

  float m[kFW], dsum[kFW], asum[kFW], o[kFW][NE];
  int trow[kFW];
#pragma unroll
  for (int q = 0; q < kFW; ++q) {
    m[q] = kNegInf;
    dsum[q] = asum[q] = 0.f;
    trow[q] = t0 + w * kFW + q;
#pragma unroll
    for (int i = 0; i < NE; ++i) o[q][i] = 0.f;
  }
  const float *qw = qs + w * kFW * D;
  // x[q] = q_q . (row l of kt)
  auto scores = [&](float (&x)[kFW]) {
#pragma unroll
    for (int q = 0; q < kFW; ++q) x[q] = 0.f;
    const float *krow = kt + l * KP;
#pragma unroll 2
    for (int c = 0; c < D; c += 4) {
      const float k0 = krow[c], k1 = krow[c + 1], k2 = krow[c + 2], k3 = krow[c + 3];
#pragma unroll
      for (int q = 0; q < kFW; ++q) {
        const f32x4_t qv = *reinterpret_cast<const f32x4_t *>(qw + q * D + c);
        x[q] = fmaf(qv[0], k0, x[q]);
        x[q] = fmaf(qv[1], k1, x[q]);
        x[q] = fmaf(qv[2], k2, x[q]);
        x[q] = fmaf(qv[3], k3, x[q]);
      }
    }
  };
  // online softmax of one chunk / batch: weights into ps, rescale factors cr;
  // wt: the lane's weight in the denominator (1 per key, n_j per Taylor block)
  auto update = [&](const float (&x)[kFW], const bool (&ok)[kFW], float wt, bool tay, float (&cr)[kFW]) {
#pragma unroll
    for (int q = 0; q < kFW; ++q) {
      const float xs = ok[q] ? x[q] * sl2 : kNegInf;
      const float mn = fmaxf(m[q], wave_max_xl(xs));
      float p = 0.f;
      cr[q] = 1.f;
      if (mn != kNegInf) {   // uniform: the wave's maximum
        cr[q] = exp2f(m[q] - mn);
        p = ok[q] ? exp2f(xs - mn) : 0.f;
        dsum[q] = dsum[q] * cr[q] + wave_sum_xl(p * wt);
        if (tay) asum[q] = asum[q] * cr[q] + wave_sum_xl(p);
        else asum[q] *= cr[q];
        m[q] = mn;
      }
      ps[q * 64 + l] = p;
    }
    wave_sync();
  };
  // o = o cr + sum_k ps[k] (row k of vt), k < nk
  auto pv = [&](const float (&cr)[kFW], int nk) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int f = l + 64 * i;
      float acc[kFW];
#pragma unroll
      for (int q = 0; q < kFW; ++q) acc[q] = o[q][i] * cr[q];
#pragma unroll 4
      for (int k = 0; k < nk; ++k) {
        const float v = vt[k * D + f];
#pragma unroll
        for (int q = 0; q < kFW; ++q) acc[q] = fmaf(ps[q * 64 + k], v, acc[q]);
      }
#pragma unroll
      for (int q = 0; q < kFW; ++q) o[q][i] = acc[q];
    }
    wave_sync();   // ps is read before the next update writes it
  };
  // u[q][i] = q_q . (row l + 64 i of ht)
  auto qht = [&](float (&u)[kFW][NE]) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const float *hrow = ht + (l + 64 * i) * KP;
#pragma unroll
      for (int q = 0; q < kFW; ++q) u[q][i] = 0.f;
#pragma unroll 2
      for (int c = 0; c < D; c += 4) {
        const float h0 = hrow[c], h1 = hrow[c + 1], h2 = hrow[c + 2], h3 = hrow[c + 3];
#pragma unroll
        for (int q = 0; q < kFW; ++q) {
          const f32x4_t qv = *reinterpret_cast<const f32x4_t *>(qw + q * D + c);
          u[q][i] = fmaf(qv[0], h0, u[q][i]);
          u[q][i] = fmaf(qv[1], h1, u[q][i]);
          u[q][i] = fmaf(qv[2], h2, u[q][i]);
          u[q][i] = fmaf(qv[3], h3, u[q][i]);
        }
      }
    }
  };
  // a D x D matrix (row-major) into ht, rows padded: fetch_h loads this
  // thread's share into registers (the loads stay in flight), put_h waits
  // for the tile in use to be consumed and writes the share
  constexpr int HS = D * D4 / 256;   // 16-byte pieces per thread
  f32x4_t hreg[HS];
  auto fetch_h = [&](const float *src) {
#pragma unroll
    for (int u = 0; u < HS; ++u) {
      const int i = tid + 256 * u, e = i / D4, c4 = i % D4;
      hreg[u] = *reinterpret_cast<const f32x4_t *>(src + (size_t)e * D + 4 * c4);
    }
  };
  auto put_h = [&]() {
    __syncthreads();   // the previous tile is consumed
#pragma unroll
    for (int u = 0; u < HS; ++u) {
      const int i = tid + 256 * u, e = i / D4, c4 = i % D4;
      float *d = ht + e * KP + 4 * c4;
      d[0] = hreg[u][0];
      d[1] = hreg[u][1];
      d[2] = hreg[u][2];
      d[3] = hreg[u][3];
    }
    __syncthreads();
  };

  // ---- exact blocks, 64 keys at a time
  for (int e = 0; e < nx; ++e) {
    const int jj = xl[e];
    const int kend = min(dm.L, (jj + 1) * dm.bs);
    for (int k0 = jj * dm.bs; k0 < kend; k0 += 64) {
      const int nk = min(64, kend - k0);
      __syncthreads();   // the previous chunk is consumed
      for (int i = tid; i < 64 * D4; i += 256) {
        const int key = i / D4, c4 = i % D4;
        f32x4_t kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (key < nk) {
          kv = *reinterpret_cast<const f32x4_t *>(K + (size_t)(k0 + key) * D + 4 * c4);
          vv = *reinterpret_cast<const f32x4_t *>(V + (size_t)(k0 + key) * D + 4 * c4);
        }
        float *d = kt + key * KP + 4 * c4;
        d[0] = kv[0];
        d[1] = kv[1];
        d[2] = kv[2];
        d[3] = kv[3];
        *reinterpret_cast<f32x4_t *>(vt + key * D + 4 * c4) = vv;
      }
      __syncthreads();
      float x[kFW], cr[kFW];
      bool ok[kFW];
      scores(x);
      const int s = k0 + l;
#pragma unroll
      for (int q = 0; q < kFW; ++q) ok[q] = l < nk && (!causal || s <= trow[q]);
      update(x, ok, 1.f, false, cr);
      pv(cr, nk);
    }
  }
  // ---- Taylor blocks, 64 per batch: kbar rows into kt, vsum rows into vt
  for (int tb0 = 0; tb0 < nt; tb0 += 64) {
    const int nb = min(64, nt - tb0);
    __syncthreads();
    for (int i = tid; i < 64 * D4; i += 256) {
      const int en = i / D4, c4 = i % D4;
      f32x4_t kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (en < nb) {
        const size_t row = (soff + tl[tb0 + en]) * D + 4 * c4;
        kv = *reinterpret_cast<const f32x4_t *>(a.kbar + row);
        vv = *reinterpret_cast<const f32x4_t *>(a.vsum + row);
      }
      float *d = kt + en * KP + 4 * c4;
      d[0] = kv[0];
      d[1] = kv[1];
      d[2] = kv[2];
      d[3] = kv[3];
      *reinterpret_cast<f32x4_t *>(vt + en * D + 4 * c4) = vv;
    }
    __syncthreads();
    float x[kFW], cr[kFW];
    bool ok[kFW];
    scores(x);
    const int jl = l < nb ? tl[tb0 + l] : 0;
    const float njf = (float)min(dm.bs, dm.L - jl * dm.bs);
#pragma unroll
    for (int q = 0; q < kFW; ++q) ok[q] = l < nb;
    update(x, ok, njf, true, cr);
    pv(cr, nb);   // zero order: alpha sigma_j
    if (taylor == 2) {   // first order: alpha scale q H_j, one H^T tile at a time, the next in flight
      const float *HTf = static_cast<const float *>(a.HT);
      fetch_h(HTf + (soff + tl[tb0]) * D * D);
      for (int en = 0; en < nb; ++en) {
        put_h();
        if (en + 1 < nb) fetch_h(HTf + (soff + tl[tb0 + en + 1]) * D * D);
        float u[kFW][NE];
        qht(u);
#pragma unroll
        for (int q = 0; q < kFW; ++q) {
          const float al = ps[q * 64 + en] * dm.scale;
#pragma unroll
          for (int i = 0; i < NE; ++i) o[q][i] = fmaf(al, u[q][i], o[q][i]);
        }
      }
    }
  }
  if (taylor == 3 && nt > 0) {   // hybrid: + (scale sum alpha) q Hbar (causal: the mean over [0, lo))
    fetch_h(static_cast<const float *>(a.HT) + hbar_offset(dm, b * dm.Hkv + hk, lo));
    put_h();
    float u[kFW][NE];
    qht(u);
#pragma unroll
    for (int q = 0; q < kFW; ++q)
#pragma unroll
      for (int i = 0; i < NE; ++i) o[q][i] = fmaf(dm.scale * asum[q], u[q][i], o[q][i]);
  }
  // ---- O = N / D, lse
#pragma unroll
  for (int q = 0; q < kFW; ++q) {
    const int t = trow[q];
    if (t >= dm.L) continue;
    float *O = static_cast<float *>(a.O) + ((size_t)bh * dm.L + t) * D;
#pragma unroll
    for (int i = 0; i < NE; ++i) O[l + 64 * i] = o[q][i] / dsum[q];
    if (a.lse && l == 0) a.lse[(size_t)bh * dm.L + t] = (m[q] + log2f(dsum[q])) * kLn2;
  }
}

template <int D>
hipError_t launch_rows(const AttnArgs &a, hipStream_t st) {
  using LY = F32Lds<D>;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_f32_rows<D>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::TOTAL);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = (unsigned)a.dm.B * a.dm.Hq * ((a.dm.L + kFR - 1) / kFR);
  attn_f32_rows<D><<<grid, 256, LY::TOTAL, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st) {
  const PisaDims &dm = a.dm;
  // block rows (blocks of 64 or 128 rows hold whole kFR-row chunks)
  if (dm.group == 0 && dm.bs % kFR == 0) return dm.d == 64 ? launch_rows<64>(a, st) : launch_rows<128>(a, st);
  const unsigned grid = (unsigned)dm.B * dm.Hq * ((dm.L + 15) / 16);
  if (dm.d == 64) attn_f32<64><<<grid, 256, 0, st>>>(a);
  else attn_f32<128><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}
