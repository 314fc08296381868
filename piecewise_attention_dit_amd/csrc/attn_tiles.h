// LDS tile formats, DMA and MFMA fragment loaders shared by the bf16
// attention kernels (gfx950).
//
// gfx950 LDS has 64 banks of 4 bytes: a ds_read_b128 is served 16 lanes
// (256 bytes) at a time and a ds_read_b64_tr_b16 32 lanes at a time, so a
// phase is conflict-free when its lanes cover every bank once.  Row-major
// bf16 tiles [rows][D] keep each row's 16-byte chunks in a permuted order:
//   kswz  rows read as MFMA A fragments (16 consecutive rows per phase, one
//         chunk column): the 16 rows must land on 16 distinct chunk slots;
//   vswz  rows read with the transposing load (4 consecutive rows x 4
//         chunks per phase).
// Tiles are written by the LDS-DMA path (global_load_lds_dwordx4): a wave
// moves one kilobyte per instruction into LDS contiguously, lane l to bytes
// 16 l .. 16 l + 15, so the permutation is applied on the global side.
#pragma once

#include "attn_common.h"

namespace pisa_attn {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

// wait until at most N vector-memory loads of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, other counters max)
template <int N>
PISA_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

PISA_DEV void dma16(const void *src, uint8_t *lds_chunk) {
  __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)lds_chunk, 16, 0, 0);
}

// Sixteen bytes per lane global -> LDS through a raw buffer descriptor that
// starts at `base` and holds `bytes` bytes: lanes whose byte offset voff is
// at or past the end read zeros (the descriptor's range check), so a tile
// that runs past the last key needs no clamping.  LDS destination as dma16.
PISA_DEV void dma16_buf(const void *base, int bytes, int voff, uint8_t *lds_chunk) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes,
                                                                     0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_chunk, 16, voff, 0, 0, 0);
}

template <int D>
PISA_DEV int kswz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
PISA_DEV int vswz(int row) {
  return (row & 3) * (D / 32);
}

// One kilobyte (chunk c) of a [rows][D] tile whose row r holds global row
// src_row(r) of g; V selects the transposed-read permutation.
template <int D, bool V, typename RowFn>
PISA_DEV void dma_chunk(const uint16_t *g, uint8_t *tile, int c, int l, RowFn src_row) {
  const int p = c * 64 + l;
  const int row = p / (D / 8), phys = p % (D / 8);
  const int logical = phys ^ (V ? vswz<D>(row) : kswz<D>(row));
  dma16(g + (size_t)src_row(row) * D + logical * 8, tile + c * 1024);
}

// MFMA A fragment of a kswz tile: row `row`, 16-byte chunk `ch` (features 8 ch .. 8 ch + 7)
template <int D>
PISA_DEV u32x4_t frag_a(const uint8_t *tile, int row, int ch) {
  return *reinterpret_cast<const u32x4_t *>(tile + row * (2 * D) + ((ch ^ kswz<D>(row)) << 4));
}

// MFMA A fragment of V^T from a vswz tile with two transposing reads:
// rows r1 and r1 + 8 (keys), features e .. e + 3 of this lane's 16-lane group.
template <int D>
PISA_DEV u32x4_t frag_vt(const uint8_t *tile, int r1, int e) {
  const int off = (((e >> 3) ^ vswz<D>(r1)) << 4) + (((e >> 2) & 1) << 3);
  const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t *)(tile + r1 * (2 * D) + off));
  const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t *)(tile + (r1 + 8) * (2 * D) + off));
  const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
  return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
}

// eight consecutive accumulator values -> one bf16 B fragment
PISA_DEV u32x4_t pack8(const f32x16_t &v, int off) {
  u32x4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[off + 2 * i], v[off + 2 * i + 1]);
  return w;
}

// hi + lo bf16 split of eight accumulator values (hi = RNE(x), lo = RNE(x - hi))
PISA_DEV void pack8_split(const f32x16_t &v, int off, u32x4_t &hi, u32x4_t &lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = v[off + 2 * i], x1 = v[off + 2 * i + 1];
    const uint32_t pk = pack_bf16x2(x0, x1);
    hi[i] = pk;
    lo[i] = pack_bf16x2(x0 - bf16lo(pk), x1 - bf16hi(pk));
  }
}

PISA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row k of an MFMA B operand held by lane (l % 32, l / 32) at register r is
// k = 8 (l / 32) + r, while row k of a 32x32 accumulator sits at lane half
// (k / 4) % 2, register 4 (k / 8) + k % 4.  A K-step over accumulator rows
// 16 s .. 16 s + 15 taken straight from registers 8 s .. 8 s + 7 therefore
// visits them in the order perm16 (an involution on 0..15).
PISA_DEV int perm16(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

}  // namespace pisa_attn
