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
// key/value rows (and Taylor statistics), done on the VALU.  Split-K: the
// row's blocks are dealt to NW = 4 S workers (S workgroups of four waves);
// a worker keeps its own online-softmax state and writes a partial
// (m, l, A, o[d]) to the workspace, and decode_combine merges the partials
// of a row in worker order (deterministic), adding the hybrid order's
// (scale sum alpha) q Hbar once per row.
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

PISA_DEV float wsum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
PISA_DEV float wmax(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

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

constexpr int kDecWaves = 4;
constexpr int kMaxList = 64;

struct DecArgs {
  PisaDims dm;
  int pos, ring, splits;
  const void *q, *K, *V;
  const float *kbar, *vsum;
  const void *HT;
  const int32_t *idx;
  float *part;   // [rows][workers][4 + d]: m, l, A, pad, o
};

// Worker state: o holds features EPL * l .. EPL * l + EPL - 1.
template <int D>
struct Acc {
  static constexpr int EPL = D / 64;
  float m = kNegInfD, l = 0.f, A = 0.f, o[EPL] = {};
  PISA_DEV void rescale(float m_new) {
    const float c = m == kNegInfD ? 0.f : exp2f(m - m_new);
    l *= c;
    A *= c;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] *= c;
    m = m_new;
  }
};

template <typename T, int D, int BS>
__global__ __launch_bounds__(kDecWaves * 64) void decode_partial(DecArgs a) {
  constexpr int EPL = D / 64;
  __shared__ float qs[D];
  __shared__ uint32_t kept_bits[32];   // blocks of the kept list (n_blk <= 1024)
  __shared__ int elist[kMaxList + 1024];   // exact blocks of the row
  __shared__ int n_exact;
  const PisaDims &dm = a.dm;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int row = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
  const int b = row / dm.Hq, h = row % dm.Hq, hk = h * dm.Hkv / dm.Hq;
  const int NWK = a.splits * kDecWaves, wk = split * kDecWaves + w;
  const int pos = a.pos;
  const float sl2 = dm.scale * kLog2eD;
  const T *Q = static_cast<const T *>(a.q) + (size_t)row * D;
  for (int c = tid; c < D; c += kDecWaves * 64) qs[c] = ld(Q + c);
  const bool ring = a.ring > 0;
  int own, lo;
  const int nc = ring ? 0 : pisa_row_geometry(dm, pos, &own, &lo);
  if (tid < 32) kept_bits[tid] = 0u;
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    if (!ring) {
      const int32_t *list = a.idx ? a.idx + (size_t)row * dm.topk : nullptr;
      for (int i = 0; i < dm.topk && list && list[i] >= 0; ++i) {
        const int j = list[i];
        // kept blocks before the window range, each once (the range itself is
        // kept anyway; entries past it are not attended)
        if (j < lo && !((kept_bits[j >> 5] >> (j & 31)) & 1u)) {
          kept_bits[j >> 5] |= 1u << (j & 31);
          elist[n++] = j;
        }
      }
      for (int j = lo; j <= own; ++j) elist[n++] = j;
    }
    n_exact = n;
  }
  __syncthreads();
  Acc<D> acc;
  const size_t kvrows = ring ? (size_t)a.ring : (size_t)dm.L;
  const T *Kh = static_cast<const T *>(a.K) + (size_t)(b * dm.Hkv + hk) * kvrows * D;
  const T *Vh = static_cast<const T *>(a.V) + (size_t)(b * dm.Hkv + hk) * kvrows * D;

  // exact keys [k0, k0 + 64) (all <= pos), rows at slot(key)
  auto exact64 = [&](int k0, int kend) {
    const int n = k0 + l;
    const bool ok = n < kend;
    const int slot = ring ? n % a.ring : n;
    const float x = ok ? dot_row<T, D>(qs, Kh + (size_t)slot * D) * sl2 : kNegInfD;
    const float mx = wmax(x);
    if (mx > acc.m) acc.rescale(mx);
    const float p = ok ? exp2f(x - acc.m) : 0.f;
    acc.l += wsum(p);
    const int nk = min(64, kend - k0);
    for (int kk = 0; kk < nk; ++kk) {
      const float pk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), kk));
      const int sl = ring ? (k0 + kk) % a.ring : k0 + kk;
      const T *vr = Vh + (size_t)sl * D + EPL * l;
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc.o[i] = fmaf(pk, ld(vr + i), acc.o[i]);
    }
  };

  if (ring) {
    // the last ring tokens: max(0, pos - ring + 1) .. pos, 64-key chunks dealt to workers
    const int t0 = max(0, pos - a.ring + 1);
    for (int k0 = t0 + wk * 64; k0 <= pos; k0 += NWK * 64) exact64(k0, pos + 1);
  } else {
    // exact blocks of the row, dealt to the workers block by block
    for (int e = wk; e < n_exact; e += NWK) {
      const int j = elist[e];
      const int kend = min(min(dm.L, (j + 1) * BS), pos + 1);
      for (int k0 = j * BS; k0 < kend; k0 += 64) exact64(k0, kend);
    }
    // Taylor blocks: candidates [0, lo) not kept, lane = block, 64 per batch
    if (dm.taylor != 0 && nc > 0) {
      const size_t soff = (size_t)(b * dm.Hkv + hk) * dm.n_blk;
      const float *kb = a.kbar + soff * D, *vs = a.vsum + soff * D;
      const bool order1 = dm.taylor == 2;
      for (int base = 0; base * NWK < nc; base += 64) {
        const int j = wk + (base + l) * NWK;
        const bool ok = j < nc && !((kept_bits[j >> 5] >> (j & 31)) & 1u);
        const float x = ok ? dot_row<float, D>(qs, kb + (size_t)j * D) * sl2 : kNegInfD;
        const float mx = wmax(x);
        if (mx == kNegInfD) continue;
        if (mx > acc.m) acc.rescale(mx);
        const float al = ok ? exp2f(x - acc.m) : 0.f;
        const float asum = wsum(al);
        acc.l = fmaf(asum, (float)BS, acc.l);   // candidate blocks lie before the window: complete
        acc.A += asum;
        for (int kk = 0; kk < 64; ++kk) {
          const float ak = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, al), kk));
          if (ak == 0.f) continue;
          const int jk = __builtin_amdgcn_readlane(j, kk);
          const float *vr = vs + (size_t)jk * D + EPL * l;
#pragma unroll
          for (int i = 0; i < EPL; ++i) acc.o[i] = fmaf(ak, vr[i], acc.o[i]);
          if (order1) {   // + alpha scale q H_j: features of this lane, rows of H_j^T
            const T *Hj = static_cast<const T *>(a.HT) + (soff + jk) * D * D;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
              const float u = dot_row<T, D>(qs, Hj + (size_t)(EPL * l + i) * D);
              acc.o[i] = fmaf(ak * dm.scale, u, acc.o[i]);
            }
          }
        }
      }
    }
  }
  float *out = a.part + ((size_t)row * NWK + wk) * (4 + D);
  if (l == 0) {
    out[0] = acc.m;
    out[1] = acc.l;
    out[2] = acc.A;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) out[4 + EPL * l + i] = acc.o[i];
}

// one wave per row: merge the workers' partials in order, add the hybrid
// term, O = N / D in the dtype, lse
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine(DecArgs a, void *O, float *lse) {
  constexpr int EPL = D / 64;
  __shared__ float qs[D];
  const PisaDims &dm = a.dm;
  const int row = blockIdx.x, l = threadIdx.x;
  const int NWK = a.splits * kDecWaves;
  const float *pr = a.part + (size_t)row * NWK * (4 + D);
  float m = kNegInfD;
  for (int i = 0; i < NWK; ++i) m = fmaxf(m, pr[(size_t)i * (4 + D)]);
  float L = 0.f, A = 0.f, o[EPL] = {};
  for (int i = 0; i < NWK; ++i) {
    const float *p = pr + (size_t)i * (4 + D);
    if (p[0] == kNegInfD) continue;
    const float c = exp2f(p[0] - m);
    L = fmaf(c, p[1], L);
    A = fmaf(c, p[2], A);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = fmaf(c, p[4 + EPL * l + e], o[e]);
  }
  if (dm.taylor == 3 && A > 0.f) {   // hybrid: + (scale sum alpha) q Hbar
    const int b = row / dm.Hq, h = row % dm.Hq, hk = h * dm.Hkv / dm.Hq;
    const T *Q = static_cast<const T *>(a.q) + (size_t)row * D;
    for (int c = l; c < D; c += 64) qs[c] = ld(Q + c);
    __syncthreads();
    const T *Hb = static_cast<const T *>(a.HT) + (size_t)(b * dm.Hkv + hk) * D * D;
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
  decode_partial<T, D, BS><<<(unsigned)rows * a.splits, kDecWaves * 64, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine<T, D><<<(unsigned)rows, 64, 0, st>>>(a, O, lse);
  return hipGetLastError();
}

}  // namespace

int decode_splits(const PisaDims &dm) {
  const int rows = dm.B * dm.Hq;
  int s = (512 + rows - 1) / rows;
  return s < 1 ? 1 : (s > 16 ? 16 : s);
}

size_t decode_workspace_bytes(const PisaDims &dm) {
  return (size_t)dm.B * dm.Hq * decode_splits(dm) * kDecWaves * (4 + dm.d) * sizeof(float);
}

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
