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

// Workgroup barrier for LDS that is filled by DMA and waited for explicitly
// (wait_vmcnt on the fills a wave issued): this wave's LDS instructions
// complete, then the waves meet.  __syncthreads' release fence also waits for
// every DMA fill still in flight, since they count as writes to LDS, so a
// tile prefetched ahead would have to land at the barrier.  The empty asm
// statements keep the compiler from moving memory accesses across it.
PISA_DEV void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st);
hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t st);
hipError_t launch_attn_blocks(const AttnArgs &a, hipStream_t st);
// PIVOT rows without a Taylor tail, key-gathered (workspace: V^T per block)
hipError_t launch_attn_pivot(const AttnArgs &a, void *ws, hipStream_t st);
