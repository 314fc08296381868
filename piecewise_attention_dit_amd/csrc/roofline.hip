// Roofline probes: the bf16 MFMA rate and the HBM copy / read bandwidth this
// MI355X actually sustains, the denominators beside the datasheet peaks.
#include "../../include/pisa_roofline.h"
#include "device_common.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kReadBlocks = 65536;

// four independent chains per wave on register operands: the dependent-issue
// latency of one chain is covered by the other three and by the other waves
// of the SIMD
__global__ __launch_bounds__(kProbeThreads) void mfma_peak(int iters, float *sink) {
  const int l = threadIdx.x & 63;
  const uint32_t v = 0x3F803F80u ^ (uint32_t)(l & 7);   // bf16 values near 1
  const u32x4_t a = {v, v ^ 1u, v ^ 2u, v ^ 3u}, b = {v ^ 4u, v, v ^ 5u, v ^ 6u};
  f32x16_t acc[4] = {f32x16_t{}, f32x16_t{}, f32x16_t{}, f32x16_t{}};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// four independent 16-byte loads in flight per thread and iteration
__global__ __launch_bounds__(kProbeThreads) void hbm_copy(u32x4_t *__restrict__ dst,
                                                          const u32x4_t *__restrict__ src, size_t n) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kProbeThreads) void hbm_read(const u32x4_t *__restrict__ src, size_t n,
                                                          float *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  uint32_t x = 0;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    x ^= (a[0] ^ b[0] ^ c[0] ^ d[0]) + (a[1] ^ b[1] ^ c[1] ^ d[1]) + (a[2] ^ b[2] ^ c[2] ^ d[2]) +
         (a[3] ^ b[3] ^ c[3] ^ d[3]);
  }
  for (; i < n; i += stride) {
    const u32x4_t w = src[i];
    x ^= w[0] ^ w[1] ^ w[2] ^ w[3];
  }
  x = (uint32_t)wave_sum_i32((int)x);
  if ((threadIdx.x & 63) == 0 && x == 0x9E3779B9u) sink[blockIdx.x] = 1.f;   // keeps the loads
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

unsigned stream_grid(size_t n16) {
  size_t g = (n16 + kProbeThreads * 16 - 1) / (kProbeThreads * 16);   // ~16 chunks per thread
  if (g < 1) g = 1;
  if (g > (size_t)kReadBlocks) g = kReadBlocks;
  return (unsigned)g;
}

}  // namespace

extern "C" {

pisa_status pisa_probe_mfma_bf16(int32_t workgroups, int32_t iters, float *sink, hipStream_t stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || !sink || !aligned16(sink)) return PISA_E_ARG;
  mfma_peak<<<(unsigned)workgroups, kProbeThreads, 0, stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_E_HIP;
}

pisa_status pisa_probe_hbm_copy(void *dst, const void *src, size_t bytes, hipStream_t stream) {
  if (!dst || !src || bytes == 0 || bytes % 16 || !aligned16(dst) || !aligned16(src)) return PISA_E_ARG;
  const size_t n = bytes / 16;
  hbm_copy<<<stream_grid(n), kProbeThreads, 0, stream>>>(static_cast<u32x4_t *>(dst),
                                                        static_cast<const u32x4_t *>(src), n);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_E_HIP;
}

pisa_status pisa_probe_hbm_read(const void *src, size_t bytes, float *sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || !aligned16(src) || !aligned16(sink)) return PISA_E_ARG;
  const size_t n = bytes / 16;
  hbm_read<<<stream_grid(n), kProbeThreads, 0, stream>>>(static_cast<const u32x4_t *>(src), n, sink);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_E_HIP;
}

}  // extern "C"
