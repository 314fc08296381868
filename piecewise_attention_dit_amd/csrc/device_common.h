// Device helpers shared by the gfx950 kernels of libpisa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pisa_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define PISA_DEV __device__ __forceinline__

// ---------------------------------------------------------------- bf16 / f32

PISA_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
PISA_DEV uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
PISA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// bf16 pair (packed in a u32) -> the two floats
PISA_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
PISA_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round a float64 to the nearest value with p significand bits in a format
// with an 8-bit exponent (bf16: p = 8, fp32: p = 24), ties to even, once.
// The quantum of x is 2^(max(e, -126) - (p - 1)) with 2^e <= |x| < 2^(e+1).
PISA_DEV double round_to_format(double x, int p) {
  if (x == 0.0) return x;
  int e = ilogb(x);
  int qe = (e > -126 ? e : -126) - (p - 1);
  double y = ldexp(rint(ldexp(x, -qe)), qe);
  double maxf = (2.0 - ldexp(1.0, 1 - p)) * 0x1p127;
  if (fabs(y) > maxf) y = copysign(__builtin_huge_val(), x);
  return y;
}

// float64 -> bf16 bits (single rounding) and -> fp32 (single rounding).
PISA_DEV uint32_t f64_to_bf16_bits(double x) {
  return __float_as_uint((float)round_to_format(x, 8)) >> 16;
}
PISA_DEV float f64_to_f32_rne(double x) { return (float)x; }

// ---------------------------------------------------------------- exact sums

// Cascaded (double-double) summation: hi carries the running float64 sum,
// lo the exact rounding errors of every addition (TwoSum).  For addends that
// are bf16/fp32 values the lo accumulation is itself exact as long as the
// exponent span from the sum's top bit to the smallest addend quantum stays
// below 98 bits, and fl(hi + lo) is then the correctly rounded sum.
struct DD {
  double hi, lo;
};
PISA_DEV void dd_add(DD &a, double x) {
  double s = a.hi + x;
  double bp = s - a.hi;
  double err = (a.hi - (s - bp)) + (x - bp);
  a.hi = s;
  a.lo += err;
}
PISA_DEV void dd_merge(DD &a, const DD &b) {
  dd_add(a, b.hi);
  a.lo += b.lo;
}
PISA_DEV double dd_value(const DD &a) { return a.hi + a.lo; }

// ---------------------------------------------------------------- wave utils

PISA_DEV int lane_id() { return __lane_id(); }

PISA_DEV float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
PISA_DEV double wave_min_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmin(v, __shfl_xor(v, o));
  return v;
}
PISA_DEV double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
PISA_DEV int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
PISA_DEV uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}
PISA_DEV uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = __shfl_xor(v, o);
    v = w < v ? w : v;
  }
  return v;
}
// inclusive prefix sum over lanes 0..63
PISA_DEV int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int w = __shfl_up(v, o);
    if (l >= o) v += w;
  }
  return v;
}
PISA_DEV uint64_t ballot64(bool p) { return __ballot(p); }

// x plus the value of lane l ^ 32 (v_permlane32_swap_b32 swaps the upper
// half of one register with the lower half of another: with both operands x
// the two results hold x and its partner on every lane)
PISA_DEV float pair_sum_f(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- wave reductions on the cross-lane data path (DPP row operations and
// the permlane swaps, no LDS); every lane ends with the same value
template <int Ctrl>
PISA_DEV float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Ctrl, 0xF, 0xF, false));
}
template <bool MAX>
PISA_DEV float wave_reduce_xl(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  v = op(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_f<0x141>(v));   // row_half_mirror
  v = op(v, dpp_f<0x140>(v));   // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
PISA_DEV float wave_max_xl(float v) { return wave_reduce_xl<true>(v); }
PISA_DEV float wave_sum_xl(float v) { return wave_reduce_xl<false>(v); }

// max of x and the value of lane l ^ 32 (permlane32 swap, as pair_sum_f)
PISA_DEV float pair_max_f(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum of eight packed bf16 (a u32x4), accumulated in fp32 (v_dot2c_f32_bf16
// with (1, 1)).  The pairs are taken from a bf16x8 view of the whole vector:
// a bit_cast of one u32 element inside an unrolled loop was compiled to read
// element 0 every time.
PISA_DEV float sum_bf16x8_f(const u32x4_t &p, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t x = {b[2 * i], b[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
  }
  return acc;
}

// Make this wave's LDS writes (and LDS atomics) visible to its own later LDS
// reads, without a workgroup barrier: a memory fence plus a code-motion
// barrier for the wave.
PISA_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------- MFMA

// Operands travel as packed u32x4 (8 bf16 in 4 registers) and are
// reinterpreted only at the MFMA, so no bf16 vector is ever split into
// one value per register.
PISA_DEV f32x16_t mfma32(const u32x4_t &a, const u32x4_t &b, const f32x16_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}
PISA_DEV bf16x8_t as_bf16x8(const u32x4_t &v) { return __builtin_bit_cast(bf16x8_t, v); }
// 16x16x32: lane l holds A row l % 16 and B column l % 16, k = 8 (l / 16) .. + 7;
// the result column l % 16, rows 4 (l / 16) .. + 3
PISA_DEV f32x4_t mfma16(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}

// Logical block id -> id such that consecutive logical ids run on the same XCD
// (workgroups are dispatched round-robin over the 8 XCDs of an MI355X).
PISA_DEV int xcd_remap(int bid, int n) {
  const int x = bid & 7, local = bid >> 3;
  const int q = n >> 3, r = n & 7;
  return (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}
