// Decode: one new token per (batch, query head) against a key/value cache.
//
// HyLRA page, section 2.3 (hybrid inference strategy): sensitive layers
// select the critical blocks, tolerant layers reuse the lists of an earlier
// layer and attend only to that part of the cache; section 2.4: block-level
// sparsity over fixed-size token blocks.  PISA page, section 2: the blocks
// that are not kept still enter through the block Taylor terms.  Sliding
// Window Attention page: the w-slot ring buffer (token i in slot i mod w).
//
// The token at position pos is the causal token row of the prefill path:
// exact terms over its kept list and the window range [lo, own] (keys
// s <= pos), Taylor terms over the other candidates [0, lo).
//
// One query row offers no matrix shape: the work is HBM-bound streaming of
// key/value rows (and Taylor statistics), done on the VALU.  The query heads
// of a kv head are served together, so each key and value row is read once
// for all of them.  Split-K: the kv head's blocks are dealt to NW = 4 S
// workers (S workgroups of four waves); a worker keeps each head's
// online-softmax state and writes its partials (m, l, A, o[d]) to the
// workspace, and decode_combine merges the partials of a row in worker order
// (deterministic), adding the hybrid order's (scale sum alpha) q Hbar(lo)
// once per row, Hbar(lo) the mean over the candidates [0, lo).
#include <mutex>

#include "device_common.h"
#include "pisa_internal.h"

namespace {

constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.6931471805599453f;
constexpr float kNegInfD = -__builtin_huge_valf();

template <typename T>
PISA_DEV float ld(const T *p) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(*p);
  else return *p;
}

PISA_DEV float wsum(float v) { return wave_sum_xl(v); }
PISA_DEV float wmax(float v) { return wave_max_xl(v); }

// dot of the fp32 row vector q (LDS) with a length-D row of T
template <typename T, int D>
PISA_DEV float dot_row(const float *q, const T *row) {
  float acc = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < D; c += 8) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t *>(row + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(q[c + 2 * i], bf16lo(w[i]), acc);
        acc = fmaf(q[c + 2 * i + 1], bf16hi(w[i]), acc);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const f32x4_t w = *reinterpret_cast<const f32x4_t *>(row + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(q[c + i], w[i], acc);
    }
  }
  return acc;
}

constexpr int kDecWaves = kDecodeWaves;
constexpr int kRM = 8;   // query heads per kv head, at most

// eight consecutive elements of a row as fp32
template <typename T>
PISA_DEV void load8(const T *p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16lo(w[i]);
      v[2 * i + 1] = bf16hi(w[i]);
    }
  } else {
    const f32x4_t x = *reinterpret_cast<const f32x4_t *>(p), y = *reinterpret_cast<const f32x4_t *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = x[i];
      v[4 + i] = y[i];
    }
  }
}

// EPL consecutive elements of a row as fp32
template <typename T, int EPL>
PISA_DEV void load_e(const T *p, float (&v)[EPL]) {
  if constexpr (sizeof(T) == 2 && EPL == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
    v[0] = bf16lo(w);
    v[1] = bf16hi(w);
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = ld(p + i);
  }
}

struct DecArgs {
  PisaDims dm;
  int pos, ring, splits;
  const void *q, *K, *V;
  const float *kbar, *vsum;
  const void *HT;
  const int32_t *idx;
  float *part;   // [rows][workers][4 + d]: m, l, A, pad, o
};

PISA_DEV float readl(float v, int k) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), k));
}

// A worker (one wave) of the kv head's group: the online-softmax state of
// each query head r < R of the kv head, lane l holding features
// EPL l .. EPL l + EPL - 1.  Key and value rows, Taylor statistics and H_j
// are read once for all R heads; a head only takes the terms of its own
// kept set (hmask / tmask).
template <typename T, int D, int BS>
__global__ __launch_bounds__(kDecWaves * 64) void decode_partial(DecArgs a) {
  constexpr int EPL = D / 64;
  __shared__ float qs[kRM][D];
  __shared__ uint32_t kbits[kRM][32];   // per head: its kept blocks before the window range
  __shared__ uint32_t ubits[32];
  __shared__ int elist[1024];            // exact blocks of any head (n_blk <= 1024)
  __shared__ int n_exact;
  __shared__ float fbuf[sizeof(T) == 2 ? kDecWaves : 1][kRM * D];   // first-order relayout, per wave
  const PisaDims &dm = a.dm;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int R = dm.ratio;
  const int grp = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
  const int b = grp / dm.Hkv, hk = grp % dm.Hkv;
  const int row0 = b * dm.Hq + hk * R;   // rows row0 .. row0 + R - 1
  const int NWK = a.splits * kDecWaves, wk = split * kDecWaves + w;
  const int pos = a.pos;
  const float sl2 = dm.scale * kLog2eD;
  const T *Q = static_cast<const T *>(a.q) + (size_t)row0 * D;
  for (int i = tid; i < R * D; i += kDecWaves * 64) qs[i / D][i % D] = ld(Q + i);
  const bool ring = a.ring > 0;
  int own, lo;
  const int nc = ring ? 0 : pisa_row_geometry(dm, pos, &own, &lo);
  for (int i = tid; i < kRM * 32; i += kDecWaves * 64) kbits[i / 32][i % 32] = 0u;
  if (tid < 32) ubits[tid] = 0u;
  __syncthreads();
  // the heads' kept blocks before the window range, as bitmaps (every thread
  // one list entry; the range itself is kept anyway, entries past it are not
  // attended)
  if (!ring && a.idx)
    for (int i = tid; i < R * dm.topk; i += kDecWaves * 64) {
      const int r = i / dm.topk;
      const int j = a.idx[(size_t)(row0 + r) * dm.topk + i % dm.topk];
      if (pisa_list_entry_kept(j, lo)) {   // candidates [0, lo) only
        atomicOr(&kbits[r][j >> 5], 1u << (j & 31));
        atomicOr(&ubits[j >> 5], 1u << (j & 31));
      }
    }
  __syncthreads();
  if (tid == 0) {   // exact blocks of any head: the union, then the window range
    int n = 0;
    if (!ring) {
      for (int wd = 0; wd < 32; ++wd)
        for (uint32_t u = ubits[wd]; u; u &= u - 1) elist[n++] = wd * 32 + __builtin_ctz(u);
      for (int j = lo; j <= own; ++j) elist[n++] = j;
    }
    n_exact = n;
  }
  __syncthreads();
  float m[kRM], L[kRM], A[kRM], o[kRM][EPL];
#pragma unroll
  for (int r = 0; r < kRM; ++r) {
    m[r] = kNegInfD;
    L[r] = A[r] = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[r][i] = 0.f;
  }
  auto rescale = [&](int r, float mn) {
    const float c = m[r] == kNegInfD ? 0.f : exp2f(m[r] - mn);
    L[r] *= c;
    A[r] *= c;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[r][i] *= c;
    m[r] = mn;
  };
  // bf16 first order on MFMA 16x16x32: A = q (row m = query head m of the kv
  // head, zero past R), loaded once
  u32x4_t qa[D / 32];
  if constexpr (sizeof(T) == 2) {
    const int mq = l & 15, kg = l >> 4;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qa[ks] = mq < R ? *reinterpret_cast<const u32x4_t *>(Q + (size_t)mq * D + ks * 32 + 8 * kg)
                      : u32x4_t{0, 0, 0, 0};
  }
  const size_t kvrows = ring ? (size_t)a.ring : (size_t)dm.L;
  const T *Kh = static_cast<const T *>(a.K) + (size_t)(b * dm.Hkv + hk) * kvrows * D;
  const T *Vh = static_cast<const T *>(a.V) + (size_t)(b * dm.Hkv + hk) * kvrows * D;

  // exact keys [k0, kend) (at most 64, all <= pos) for the heads of hmask
  auto chunk = [&](int k0, int kend, uint32_t hmask) {
    const int n = k0 + l;
    const bool ok = n < kend;
    const int nk = kend - k0;
    // every value entry of this lane for the chunk, issued before the scores
    // (rows past the chunk repeat its last row: their weights are zero)
    float vv[64][EPL];
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int kk = k0 + min(i, nk - 1);
      load_e<T, EPL>(Vh + (size_t)(ring ? kk % a.ring : kk) * D + EPL * l, vv[i]);
    }
    float x[kRM];
#pragma unroll
    for (int r = 0; r < kRM; ++r) x[r] = 0.f;
    if (ok) {
      const T *kr = Kh + (size_t)(ring ? n % a.ring : n) * D;
      for (int c = 0; c < D; c += 8) {
        float kv[8];
        load8(kr + c, kv);
#pragma unroll
        for (int r = 0; r < kRM; ++r) {
          if (r >= R) break;
#pragma unroll
          for (int i = 0; i < 8; ++i) x[r] = fmaf(qs[r][c + i], kv[i], x[r]);
        }
      }
    }
    float p[kRM];
#pragma unroll
    for (int r = 0; r < kRM; ++r) {
      p[r] = 0.f;
      if (r >= R || !((hmask >> r) & 1u)) continue;
      const float xs = ok ? x[r] * sl2 : kNegInfD;
      const float mx = wmax(xs);
      if (mx > m[r]) rescale(r, mx);
      p[r] = ok ? exp2f(xs - m[r]) : 0.f;
      L[r] += wsum(p[r]);
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) {
#pragma unroll
      for (int r = 0; r < kRM; ++r) {
        if (r >= R || !((hmask >> r) & 1u)) continue;
        const float pk = readl(p[r], i);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(pk, vv[i][e], o[r][e]);
      }
    }
  };

  if (ring) {
    // the last ring tokens: max(0, pos - ring + 1) .. pos, 64-key chunks dealt to workers
    const int t0 = max(0, pos - a.ring + 1);
    for (int k0 = t0 + wk * 64; k0 <= pos; k0 += NWK * 64) chunk(k0, min(k0 + 64, pos + 1), 0xFFu);
  } else {
    // exact blocks of the kv head's rows, dealt to the workers block by block
    for (int e = wk; e < n_exact; e += NWK) {
      const int j = elist[e];
      uint32_t hm = 0;
      for (int r = 0; r < R; ++r)
        if (j >= lo || ((kbits[r][j >> 5] >> (j & 31)) & 1u)) hm |= 1u << r;
      const int kend = min(min(dm.L, (j + 1) * BS), pos + 1);
      for (int k0 = j * BS; k0 < kend; k0 += 64) chunk(k0, min(k0 + 64, kend), hm);
    }
    // Taylor blocks: candidates [0, lo); lane = block, 64 per batch
    if (dm.taylor != 0 && nc > 0) {
      const size_t soff = (size_t)(b * dm.Hkv + hk) * dm.n_blk;
      const float *kb = a.kbar + soff * D, *vs = a.vsum + soff * D;
      const bool order1 = dm.taylor == 2;
      for (int base = 0; base * NWK < nc; base += 64) {
        const int j = wk + (base + l) * NWK;
        const bool in = j < nc;
        float x[kRM];
#pragma unroll
        for (int r = 0; r < kRM; ++r) x[r] = 0.f;
        if (in) {
          for (int c = 0; c < D; c += 8) {
            float kv[8];
            load8(kb + (size_t)j * D + c, kv);
#pragma unroll
            for (int r = 0; r < kRM; ++r) {
              if (r >= R) break;
#pragma unroll
              for (int i = 0; i < 8; ++i) x[r] = fmaf(qs[r][c + i], kv[i], x[r]);
            }
          }
        }
        float al[kRM];
        bool any = false;
#pragma unroll
        for (int r = 0; r < kRM; ++r) {
          al[r] = 0.f;
          if (r >= R) continue;
          const bool t = in && !((kbits[r][j >> 5] >> (j & 31)) & 1u);
          const float xs = t ? x[r] * sl2 : kNegInfD;
          const float mx = wmax(xs);
          if (mx == kNegInfD) continue;
          if (mx > m[r]) rescale(r, mx);
          al[r] = t ? exp2f(xs - m[r]) : 0.f;
          const float s = wsum(al[r]);
          L[r] = fmaf(s, (float)BS, L[r]);   // candidate blocks lie before the window: complete
          A[r] += s;
          any = true;
        }
        if (!any) continue;
        const int nb = min(64, (nc - wk + NWK - 1) / NWK - base);   // blocks of this batch
        // bf16 first order of the batch: F[m][e] += alpha_m scale (q_m H_j)[e]
        // in the MFMA layout (rows m = 4 (l / 16) + t, columns e = 16 nt + l % 16)
        f32x4_t F[D / 16];
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) F[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        bool fo = false;
        for (int k1 = 0; k1 < nb; k1 += 16) {
          float vv[16][EPL];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int jk = __builtin_amdgcn_readlane(j, min(k1 + i, 63));
            if (k1 + i < nb) load_e<float, EPL>(vs + (size_t)jk * D + EPL * l, vv[i]);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (k1 + i >= nb) break;
            float ak[kRM];
            bool use = false;
#pragma unroll
            for (int r = 0; r < kRM; ++r) {
              ak[r] = r < R ? readl(al[r], k1 + i) : 0.f;
              use |= ak[r] != 0.f;
#pragma unroll
              for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(ak[r], vv[i][e], o[r][e]);
            }
            if (!order1 || !use) continue;
            const int jk = __builtin_amdgcn_readlane(j, k1 + i);
            if constexpr (sizeof(T) == 2) {
              // u = Q H_j^T^T on MFMA, B = rows e of H_j^T straight from memory
              const uint16_t *Hj = static_cast<const uint16_t *>(a.HT) + (soff + jk) * D * D;
              float am[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int mrow = 4 * (l >> 4) + t;
                float v = 0.f;
#pragma unroll
                for (int r = 0; r < kRM; ++r)
                  if (r == mrow) v = ak[r];
                am[t] = v * dm.scale;
              }
              // the fragments of NG output tiles are loaded together (one
              // memory latency per group, not one per fragment)
              constexpr int NG = 4;
#pragma unroll
              for (int n0 = 0; n0 < D / 16; n0 += NG) {
                u32x4_t hb[NG][D / 32];
#pragma unroll
                for (int g = 0; g < NG; ++g)
#pragma unroll
                  for (int ks = 0; ks < D / 32; ++ks)
                    hb[g][ks] = *reinterpret_cast<const u32x4_t *>(Hj + (size_t)((n0 + g) * 16 + (l & 15)) * D +
                                                                   ks * 32 + 8 * (l >> 4));
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                  f32x4_t u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                  for (int ks = 0; ks < D / 32; ++ks) u = mfma16(qa[ks], hb[g][ks], u);
#pragma unroll
                  for (int t = 0; t < 4; ++t) F[n0 + g][t] = fmaf(am[t], u[t], F[n0 + g][t]);
                }
              }
              fo = true;
              continue;
            }
            // + alpha scale q H_j for every head: rows EPL l .. of H_j^T read once
            const T *Hj = static_cast<const T *>(a.HT) + (soff + jk) * D * D + (size_t)EPL * l * D;
            float u[kRM][EPL];
#pragma unroll
            for (int r = 0; r < kRM; ++r)
#pragma unroll
              for (int e = 0; e < EPL; ++e) u[r][e] = 0.f;
            for (int c = 0; c < D; c += 8) {
#pragma unroll
              for (int e = 0; e < EPL; ++e) {
                float hv[8];
                load8(Hj + (size_t)e * D + c, hv);
#pragma unroll
                for (int r = 0; r < kRM; ++r) {
                  if (r >= R) break;
#pragma unroll
                  for (int t = 0; t < 8; ++t) u[r][e] = fmaf(qs[r][c + t], hv[t], u[r][e]);
                }
              }
            }
#pragma unroll
            for (int r = 0; r < kRM; ++r)
#pragma unroll
              for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(ak[r] * dm.scale, u[r][e], o[r][e]);
          }
        }
        if constexpr (sizeof(T) == 2) {
          if (fo) {   // F into the heads' accumulators (lane l: features EPL l ..), through LDS
            float *buf = fbuf[w];
#pragma unroll
            for (int nt = 0; nt < D / 16; ++nt)
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int mrow = 4 * (l >> 4) + t;
                if (mrow < kRM) buf[mrow * D + nt * 16 + (l & 15)] = F[nt][t];
              }
            wave_lds_sync();
#pragma unroll
            for (int r = 0; r < kRM; ++r) {
              if (r >= R) break;
#pragma unroll
              for (int e = 0; e < EPL; ++e) o[r][e] += buf[r * D + EPL * l + e];
            }
            wave_lds_sync();   // read before the next batch writes
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRM; ++r) {
    if (r >= R) break;
    float *out = a.part + ((size_t)(row0 + r) * NWK + wk) * (4 + D);
    if (l == 0) {
      out[0] = m[r];
      out[1] = L[r];
      out[2] = A[r];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[4 + EPL * l + e] = o[r][e];
  }
}

// one wave per row: merge the workers' partials in worker order (lane i
// takes partial i for the scalars), add the hybrid term, O = N / D in the
// dtype, lse
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine(DecArgs a, void *O, float *lse) {
  constexpr int EPL = D / 64;
  constexpr int PW = 4 + D;
  __shared__ float qs[D];
  __shared__ float cw[128];   // weight of each partial
  const PisaDims &dm = a.dm;
  const int row = blockIdx.x, l = threadIdx.x;
  const int NWK = a.splits * kDecWaves;   // <= 128
  const float *pr = a.part + (size_t)row * NWK * PW;
  float mi[2], li[2], ai[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {   // both loads issued before either is used
    const int i = l + 64 * u, ic = i < NWK ? i : NWK - 1;
    mi[u] = pr[(size_t)ic * PW];
    li[u] = pr[(size_t)ic * PW + 1];
    ai[u] = pr[(size_t)ic * PW + 2];
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (l + 64 * u >= NWK) {
      mi[u] = kNegInfD;
      li[u] = 0.f;
      ai[u] = 0.f;
    }
  const float m = wmax(fmaxf(mi[0], mi[1]));
  float Ls = 0.f, As = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = l + 64 * u;
    const float c = mi[u] == kNegInfD ? 0.f : exp2f(mi[u] - m);
    if (i < NWK) cw[i] = c;
    Ls = fmaf(c, li[u], Ls);
    As = fmaf(c, ai[u], As);
  }
  // fixed-order tree sums (the same for every run)
  const float L = wsum(Ls), A = wsum(As);
  __syncthreads();
  float o[EPL] = {};
  // partials in groups of 32, each group's loads issued together (four
  // memory latencies for 128 partials), summed in worker order; rows past
  // the last partial are a valid row weighted by zero (adds exactly nothing)
  constexpr int PG = 32;
  for (int i0 = 0; i0 < NWK; i0 += PG) {
    float v[PG][EPL];
#pragma unroll
    for (int t = 0; t < PG; ++t) {
      const int i = i0 + t < NWK ? i0 + t : NWK - 1;
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[t][e] = pr[(size_t)i * PW + 4 + EPL * l + e];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < PG; ++t) {
      const float c = i0 + t < NWK ? cw[i0 + t] : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(c, v[t][e], o[e]);
    }
  }
  if (dm.taylor == 3 && A > 0.f) {   // hybrid: + (scale sum alpha) q Hbar
    const int b = row / dm.Hq, h = row % dm.Hq, hk = h * dm.Hkv / dm.Hq;
    const T *Q = static_cast<const T *>(a.q) + (size_t)row * D;
    for (int c = l; c < D; c += 64) qs[c] = ld(Q + c);
    __syncthreads();
    // the mean over the token's candidates [0, lo): statistics of complete
    // blocks before the window range only
    int own, lo;
    pisa_row_geometry(dm, a.pos, &own, &lo);
    const T *Hb = static_cast<const T *>(a.HT) + hbar_offset(dm, b * dm.Hkv + hk, lo);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      o[e] = fmaf(dm.scale * A, dot_row<T, D>(qs, Hb + (size_t)(EPL * l + e) * D), o[e]);
  }
  const float inv = 1.f / L;
  if constexpr (sizeof(T) == 2) {
    uint16_t *Oh = static_cast<uint16_t *>(O) + (size_t)row * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) Oh[EPL * l + e] = (uint16_t)f32_to_bf16(o[e] * inv);
  } else {
    float *Of = static_cast<float *>(O) + (size_t)row * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) Of[EPL * l + e] = o[e] * inv;
  }
  if (lse && l == 0) lse[row] = (m + log2f(L)) * kLn2D;
}

template <typename T, int D, int BS>
hipError_t launch_t(const DecArgs &a, void *O, float *lse, hipStream_t st) {
  const int rows = a.dm.B * a.dm.Hq;
  decode_partial<T, D, BS><<<(unsigned)a.dm.B * a.dm.Hkv * a.splits, kDecWaves * 64, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine<T, D><<<(unsigned)rows, 64, 0, st>>>(a, O, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const PisaDims &dm, int pos, int ring, const void *q, const void *K, const void *V,
                         const float *kbar, const float *vsum, const void *HT, const int32_t *idx, void *O,
                         float *lse, void *ws, hipStream_t st) {
  DecArgs a;
  a.dm = dm;
  a.pos = pos;
  a.ring = ring;
  a.splits = decode_splits(dm);
  a.q = q; a.K = K; a.V = V; a.kbar = kbar; a.vsum = vsum; a.HT = HT; a.idx = idx;
  a.part = static_cast<float *>(ws);
  const bool bf = dm.dtype == 0;
  if (dm.d == 64) {
    if (bf) return dm.bs == 64 ? launch_t<uint16_t, 64, 64>(a, O, lse, st) : launch_t<uint16_t, 64, 128>(a, O, lse, st);
    return dm.bs == 64 ? launch_t<float, 64, 64>(a, O, lse, st) : launch_t<float, 64, 128>(a, O, lse, st);
  }
  if (bf) return dm.bs == 64 ? launch_t<uint16_t, 128, 64>(a, O, lse, st) : launch_t<uint16_t, 128, 128>(a, O, lse, st);
  return dm.bs == 64 ? launch_t<float, 128, 64>(a, O, lse, st) : launch_t<float, 128, 128>(a, O, lse, st);
}

// ---------------------------------------------------------------------------
// Fixed scratch for pisa_decode_fwd_noalloc: the split-K partials live in a
// device array of the library instead of a caller workspace, for callers
// that cannot allocate.  Each device holds its own copy of the array for the
// life of the process.  Its device address comes from hipGetSymbolAddress,
// taken once per device with that device current; host code never passes
// the array's own name (a host-side stand-in, not a device address).
// decode_partial writes every partial before decode_combine reads it, so no
// part of the array needs clearing between calls.  Calls that overlap on one
// device share the array and race.
namespace {
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}
