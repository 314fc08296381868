// Definitions shared by the two attention kernels (bf16 MFMA and fp32 VALU).
#pragma once

#include "device_common.h"

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
constexpr float kNegInf = -__builtin_huge_valf();

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st);
hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t st);
hipError_t launch_attn_blocks(const AttnArgs &a, hipStream_t st);
