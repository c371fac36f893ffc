// Peak probes: what the MI355X's matrix pipes and HBM sustain in isolation,
// so that each stage of the path can be reported against a measured ceiling
// next to the published one.  Not part of the method.
//
//  * k_probe_mfma: v_mfma_f32_32x32x16_bf16 on register operands, four
//    independent accumulator chains per wave, no memory traffic in the loop.
//  * k_probe_read: streams a buffer once with 16-byte loads (grid-stride),
//    folding the words with xor so the loads cannot be dropped.
//  * k_probe_copy: 16-byte loads and stores, grid-stride.
#include "common.h"

namespace adas {

namespace {
typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t pu32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeChains = 4;
constexpr int kProbeUnroll = 4;  // MFMAs per chain per loop trip
}  // namespace

__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  pbf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.001f * (lane + i));
    b[i] = (__bf16)(0.5f - 0.001f * (lane - i));
  }
  pf32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // never true for these operands; keeps the loop
}

__global__ __launch_bounds__(256) void k_probe_read(const pu32x4* __restrict__ src, long n16,
                                                    uint32_t* sink) {
  uint32_t x = 0;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256) {
    const pu32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

__global__ __launch_bounds__(256) void k_probe_copy(const pu32x4* __restrict__ src, pu32x4* __restrict__ dst,
                                                    long n16) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

double probe_mfma_flops_per_wg(int iters) {
  // 4 waves, each kProbeChains x kProbeUnroll MFMAs of 32x32x16 per trip
  return 4.0 * iters * kProbeChains * kProbeUnroll * (2.0 * 32 * 32 * 16);
}

hipError_t launch_probe_mfma(int wgs, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_mfma, dim3((unsigned)wgs), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, long bytes, uint32_t* sink, int wgs, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_read, dim3((unsigned)wgs), dim3(256), 0, s, (const pu32x4*)src, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, long bytes, int wgs, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)wgs), dim3(256), 0, s, (const pu32x4*)src, (pu32x4*)dst,
                     bytes / 16);
  return hipGetLastError();
}

}  // namespace adas
