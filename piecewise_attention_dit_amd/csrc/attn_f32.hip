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

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st) {
  const PisaDims &dm = a.dm;
  const unsigned grid = (unsigned)dm.B * dm.Hq * ((dm.L + 15) / 16);
  if (dm.d == 64) attn_f32<64><<<grid, 256, 0, st>>>(a);
  else attn_f32<128><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}
