// Cube partition (AdaSpark, papernotes.org, key design 1: h x w x t cubes as
// the atomic unit) and cube mean keys (key design 2: kbar_j).
//
// Both kernels are HBM-bound streaming passes.
//   partition : reads and writes every element once (2 * bytes of the tensor)
//   mean keys : reads K once, writes Nc*d floats
#include "common.h"

namespace adas {

// One workgroup copies one cube of one head: S rows of `vpr` 16-byte vectors.
// Rows are contiguous on both sides, so every 16-byte access is part of a
// fully used row segment; the destination is written sequentially.
// Frames [f_lo, f_hi) are copied (a whole tensor: 0, T); src holds those
// frames only, in raster order, and blockIdx.x counts cubes from c_lo.
__global__ __launch_bounds__(256) void k_partition(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst,
                                                   int32_t* __restrict__ perm, KGeom g, int nh,
                                                   int vpr, int f_lo, int f_hi, int c_lo) {
  const int c = c_lo + blockIdx.x;
  const int h = blockIdx.y;
  // cube -> block coordinates (uniform per workgroup)
  const int bx = c % g.nW;
  const int by = (c / g.nW) % g.nH;
  const int bt = c / (g.nW * g.nH);
  const int hw = g.ch * g.cw;
  const size_t dst_row0 = ((size_t)h * g.NS + (size_t)c * g.S);
  const int total = g.S * vpr;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int r = e / vpr;
    const int v = e - r * vpr;
    const int dt = r / hw;
    const int rem = r - dt * hw;
    const int dy = rem / g.cw;
    const int dx = rem - dy * g.cw;
    const int f = bt * g.ct + dt;
    if (f < f_lo || f >= f_hi) continue;
    const int n = ((f - f_lo) * g.H + by * g.ch + dy) * g.W + bx * g.cw + dx;
    dst[(dst_row0 + r) * vpr + v] = src[((size_t)n * nh + h) * vpr + v];
    if (perm != nullptr && h == 0 && v == 0) perm[c * g.S + r] = n;
  }
}

// ADAS_LAYOUT_VT: one workgroup per (cube, head) stages up to 64 offsets x d
// in LDS, then writes each d-row of the transposed cube: position p of row e
// takes offset vt_column(p).  Both sides move 16 bytes per thread: a load is
// one token's 16-byte piece of d (written to LDS as 4-byte words, rows padded
// to an odd word count, so the gathers below do not collide on banks); a
// store is EPV consecutive positions of one d-row, gathered from LDS.  A
// store whose positions straddle the frame window is done element by element.
template <typename T>
__global__ __launch_bounds__(256) void k_partition_vt(const T* __restrict__ src, T* __restrict__ dst,
                                                      int32_t* __restrict__ perm, KGeom g, int nh,
                                                      int f_lo, int f_hi, int c_lo) {
  constexpr int EPV = 16 / (int)sizeof(T);   // elements per 16-byte vector
  constexpr int WPT = (int)sizeof(T) == 2 ? 2 : 1;  // elements per 4-byte LDS word
  constexpr int TS = 128 / WPT + 1;          // LDS row stride in words (d <= 128)
  __shared__ uint32_t tile[64 * TS];
  const int c = c_lo + blockIdx.x;
  const int h = blockIdx.y;
  const int bx = c % g.nW;
  const int by = (c / g.nW) % g.nH;
  const int bt = c / (g.nW * g.nH);
  const int hw = g.ch * g.cw;
  const int D = g.D;
  const int VPR = D / EPV;  // 16-byte vectors per token row
  T* out = dst + ((size_t)h * (g.NS / g.S) + c) * (size_t)D * g.S;
  auto in_window = [&](int r) { const int f = bt * g.ct + r / hw; return f >= f_lo && f < f_hi; };
  for (int r0 = 0; r0 < g.S; r0 += 64) {
    const int nk = min(64, g.S - r0);
    __syncthreads();  // the previous chunk's reads of `tile` are done
    for (int e = threadIdx.x; e < nk * VPR; e += blockDim.x) {
      const int rr = e / VPR, v = e - rr * VPR;
      const int r = r0 + rr;
      if (!in_window(r)) continue;
      const int dt = r / hw;
      const int rem = r - dt * hw;
      const int dy = rem / g.cw;
      const int dx = rem - dy * g.cw;
      const int f = bt * g.ct + dt;
      const int n = ((f - f_lo) * g.H + by * g.ch + dy) * g.W + bx * g.cw + dx;
      const uint4 x = *reinterpret_cast<const uint4*>(src + ((size_t)n * nh + h) * D + v * EPV);
      uint32_t* t = &tile[rr * TS + v * (EPV / WPT)];
      t[0] = x.x;
      t[1] = x.y;
      t[2] = x.z;
      t[3] = x.w;
      if (perm != nullptr && h == 0 && v == 0) perm[c * g.S + r] = n;
    }
    __syncthreads();
    if (g.S % EPV != 0) {
      // rows not 16-byte aligned: one element per thread
      for (int e = threadIdx.x; e < nk * D; e += blockDim.x) {
        const int d = e / nk, pl = e - d * nk;
        const int r = vt_column(r0 + pl, g.S);
        if (!in_window(r)) continue;
        const uint32_t w = tile[(r - r0) * TS + d / WPT];
        out[(size_t)d * g.S + r0 + pl] = (T)(WPT == 2 ? ((d & 1) ? (w >> 16) : (w & 0xFFFFu)) : w);
      }
      continue;
    }
    const int GPR = nk / EPV;  // 16-byte groups per d-row of the chunk
    for (int e = threadIdx.x; e < D * GPR; e += blockDim.x) {
      const int d = e / GPR, q = e - d * GPR;
      T val[EPV];
      bool all = true, any = false;
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        const int r = vt_column(r0 + EPV * q + i, g.S);  // groups of 16 never straddle r0
        const bool ok = in_window(r);
        all = all && ok;
        any = any || ok;
        const uint32_t w = tile[(r - r0) * TS + d / WPT];
        val[i] = (T)(WPT == 2 ? ((d & 1) ? (w >> 16) : (w & 0xFFFFu)) : w);
      }
      T* o = out + (size_t)d * g.S + r0 + EPV * q;
      if (all) {
        uint4 v;
        __builtin_memcpy(&v, val, 16);
        *reinterpret_cast<uint4*>(o) = v;
      } else if (any) {
#pragma unroll
        for (int i = 0; i < EPV; ++i)
          if (in_window(vt_column(r0 + EPV * q + i, g.S))) o[i] = val[i];
      }
    }
  }
}

// Keys: partition and mean keys in one pass, so K is read once.  One
// workgroup per (cube, KV head) copies the cube's S rows as k_partition does;
// with 256 threads and VPR 16-byte vectors per row (VPR divides 256), thread
// t always copies vector t % VPR of rows t / VPR, t / VPR + 256 / VPR, ...,
// and sums those EPV columns in float64.  The 256 / VPR threads of one vector
// fold their sums with xor shuffles inside each wave, then across the four
// waves through LDS.  The order of the additions differs from k_mean_keys';
// the results agree bit for bit whenever the float64 sums are exact.
template <typename T, int VPR>
__global__ __launch_bounds__(256) void k_partition_keys(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        int32_t* __restrict__ perm, float* __restrict__ kbar,
                                                        KGeom g) {
  constexpr int EPV = 16 / (int)sizeof(T);
  constexpr int TPV = 256 / VPR;  // threads per vector column
  static_assert(256 % VPR == 0 && VPR <= 64, "vectors per row");
  __shared__ double part[4][VPR][EPV];
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int bx = c % g.nW;
  const int by = (c / g.nW) % g.nH;
  const int bt = c / (g.nW * g.nH);
  const int hw = g.ch * g.cw;
  const size_t dst_row0 = ((size_t)h * g.NS + (size_t)c * g.S);
  const int v = threadIdx.x % VPR;
  double acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
  for (int r = threadIdx.x / VPR; r < g.S; r += TPV) {
    const int dt = r / hw;
    const int rem = r - dt * hw;
    const int dy = rem / g.cw;
    const int dx = rem - dy * g.cw;
    const int n = ((bt * g.ct + dt) * g.H + by * g.ch + dy) * g.W + bx * g.cw + dx;
    const uint4 x = src[((size_t)n * g.Hkv + h) * VPR + v];
    dst[(dst_row0 + r) * VPR + v] = x;
    if (perm != nullptr && h == 0 && v == 0) perm[c * g.S + r] = n;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)__uint_as_float(w[e] << 16);
        acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += (double)__uint_as_float(w[e]);
    }
  }
  // lanes v, v + VPR, ... of a wave hold the same column
#pragma unroll
  for (int o = VPR; o < kWave; o <<= 1)
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (lane < VPR) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) part[wave][lane][e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < VPR) {
    float res[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const double sum = part[0][v][e] + part[1][v][e] + part[2][v][e] + part[3][v][e];
      res[e] = (float)(sum / (double)g.S);
    }
    float* out = kbar + ((size_t)h * (g.NS / g.S) + c) * g.D + v * EPV;
#pragma unroll
    for (int e = 0; e < EPV; e += 4)
      *reinterpret_cast<float4*>(out + e) = make_float4(res[e], res[e + 1], res[e + 2], res[e + 3]);
  }
}

hipError_t launch_partition_keys(const KGeom& g, adas_dtype dt, const void* src, void* dst, int32_t* perm,
                                 float* kbar, hipStream_t s) {
  const dim3 grid(g.Nc, g.Hkv);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, kbar, g);
  };
  if (dt == ADAS_BF16) {
    if (g.D == 128) go(k_partition_keys<uint16_t, 16>);
    else go(k_partition_keys<uint16_t, 8>);
  } else {
    if (g.D == 128) go(k_partition_keys<float, 32>);
    else go(k_partition_keys<float, 16>);
  }
  return hipGetLastError();
}

hipError_t launch_partition_frames(const KGeom& g, int elem_bytes, int nh, bool vt, const void* src,
                                   void* dst, int32_t* perm, int f_lo, int f_hi, hipStream_t s) {
  const int per_block = g.nH * g.nW;
  const int c_lo = f_lo / g.ct * per_block;
  const int c_hi = ((f_hi - 1) / g.ct + 1) * per_block;
  dim3 grid(c_hi - c_lo, nh);
  if (vt) {
    if (elem_bytes == 2)
      hipLaunchKernelGGL((k_partition_vt<uint16_t>), grid, dim3(256), 0, s, (const uint16_t*)src,
                         (uint16_t*)dst, perm, g, nh, f_lo, f_hi, c_lo);
    else
      hipLaunchKernelGGL((k_partition_vt<uint32_t>), grid, dim3(256), 0, s, (const uint32_t*)src,
                         (uint32_t*)dst, perm, g, nh, f_lo, f_hi, c_lo);
    return hipGetLastError();
  }
  const int vpr = g.D * elem_bytes / 16;
  hipLaunchKernelGGL(k_partition, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, g,
                     nh, vpr, f_lo, f_hi, c_lo);
  return hipGetLastError();
}

hipError_t launch_partition(const KGeom& g, int elem_bytes, int nh, bool vt, const void* src,
                            void* dst, int32_t* perm, hipStream_t s) {
  return launch_partition_frames(g, elem_bytes, nh, vt, src, dst, perm, 0, g.T, s);
}

// One wave per (kv head, cube).  Lanes are laid out LPR per row (16 bytes
// each) and RPI = 64 / LPR rows per step; each lane accumulates its EPV
// columns in float64, then the RPI row groups are folded with xor shuffles.
// Every cube size S is a power of two in the configurations this serves, so
// the float64 sum of bf16 values is exact and the final division by S is
// exact; the single float32 rounding then matches any exact evaluation.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_mean_keys(const T* __restrict__ k, float* __restrict__ kbar,
                                                   KGeom g) {
  constexpr int EPV = 16 / sizeof(T);     // elements per 16-byte vector
  constexpr int LPR = D / EPV;            // lanes per row
  constexpr int RPI = kWave / LPR;        // rows per step
  const int lane = threadIdx.x & (kWave - 1);
  const int cube = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (cube >= g.Hkv * g.Nc) return;
  const int col = (lane % LPR) * EPV;
  const int r0 = lane / LPR;
  const int kv = cube / g.Nc, j = cube - kv * g.Nc;
  const T* base = k + ((size_t)kv * g.NS + (size_t)j * g.S) * D;  // the S rows of cube (kv, j)
  double acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
  for (int r = r0; r < g.S; r += RPI) {
    const uint4 raw = *reinterpret_cast<const uint4*>(base + (size_t)r * D + col);
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)__uint_as_float(w[e] << 16);
        acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
      acc[0] += (double)__uint_as_float(raw.x);
      acc[1] += (double)__uint_as_float(raw.y);
      acc[2] += (double)__uint_as_float(raw.z);
      acc[3] += (double)__uint_as_float(raw.w);
    }
  }
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
  if (lane < LPR) {
    float res[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) res[e] = (float)(acc[e] / (double)g.S);
    float* dst = kbar + ((size_t)kv * (g.NS / g.S) + j) * D + col;
#pragma unroll
    for (int e = 0; e < EPV; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(res[e], res[e + 1], res[e + 2], res[e + 3]);
  }
}

hipError_t launch_mean_keys(const KGeom& g, adas_dtype dt, const void* k, float* kbar,
                            hipStream_t s) {
  const int cubes = g.Hkv * g.Nc;
  dim3 grid((cubes + 3) / 4);
  if (dt == ADAS_BF16) {
    if (g.D == 128)
      hipLaunchKernelGGL((k_mean_keys<uint16_t, 128>), grid, dim3(256), 0, s, (const uint16_t*)k,
                         kbar, g);
    else
      hipLaunchKernelGGL((k_mean_keys<uint16_t, 64>), grid, dim3(256), 0, s, (const uint16_t*)k,
                         kbar, g);
  } else {
    if (g.D == 128)
      hipLaunchKernelGGL((k_mean_keys<float, 128>), grid, dim3(256), 0, s, (const float*)k, kbar,
                         g);
    else
      hipLaunchKernelGGL((k_mean_keys<float, 64>), grid, dim3(256), 0, s, (const float*)k, kbar,
                         g);
  }
  return hipGetLastError();
}

// Streaming mean keys.  One wave per (kv head, cube of the temporal blocks
// frames [f_lo, f_hi) touch); lane l owns columns l and l + 64 (D = 128) or
// l (D = 64).  The rows of the new frames are summed in float64 from the
// cache; a block that began before f_lo continues the running sums kept in
// `ksum` (one slot per cube of a temporal block), and a block that ends by
// f_hi gets its float32 mean key.  Sums of a cube's bf16 values are exact in
// float64 (as for the one-pass mean keys), so the order of the partial sums
// does not change the result.
template <int D>
__global__ __launch_bounds__(256) void k_stream_kbar(const uint16_t* __restrict__ k, float* __restrict__ kbar,
                                                     double* __restrict__ ksum, KGeom g, int f_lo, int f_hi,
                                                     int c_lo, int n_cubes) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= g.Hkv * n_cubes) return;
  const int kv = item / n_cubes;
  const int c = c_lo + (item - kv * n_cubes);
  const int per_block = g.nH * g.nW;
  const int bt = c / per_block, slot = c - bt * per_block;
  const int hw = g.ch * g.cw;
  const int b0 = bt * g.ct, b1 = b0 + g.ct;  // frames of this cube
  const int dt_lo = max(f_lo, b0) - b0, dt_hi = min(f_hi, b1) - b0;
  double* run = ksum + ((size_t)kv * per_block + slot) * D;
  double acc[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) acc[u] = (f_lo > b0) ? run[lane + 64 * u] : 0.0;
  const uint16_t* base = k + ((size_t)kv * g.NS + (size_t)c * g.S) * D;
  for (int r = dt_lo * hw; r < dt_hi * hw; ++r)
#pragma unroll
    for (int u = 0; u < CPL; ++u) acc[u] += (double)bf16_bits_to_f32(base[(size_t)r * D + lane + 64 * u]);
  if (f_hi >= b1) {
#pragma unroll
    for (int u = 0; u < CPL; ++u)
      kbar[((size_t)kv * (g.NS / g.S) + c) * D + lane + 64 * u] = (float)(acc[u] / (double)g.S);
  } else {
#pragma unroll
    for (int u = 0; u < CPL; ++u) run[lane + 64 * u] = acc[u];
  }
}

hipError_t launch_cache_append(const KGeom& g, int f_lo, int f_hi, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, float* kbar, double* ksum, hipStream_t s) {
  hipError_t e = launch_partition_frames(g, 2, g.Hkv, false, k_new, k_cache, nullptr, f_lo, f_hi, s);
  if (e != hipSuccess) return e;
  e = launch_partition_frames(g, 2, g.Hkv, true, v_new, v_cache, nullptr, f_lo, f_hi, s);
  if (e != hipSuccess) return e;
  const int per_block = g.nH * g.nW;
  const int c_lo = f_lo / g.ct * per_block;
  const int n_cubes = ((f_hi - 1) / g.ct + 1) * per_block - c_lo;
  dim3 grid((g.Hkv * n_cubes + 3) / 4);
  if (g.D == 128)
    hipLaunchKernelGGL((k_stream_kbar<128>), grid, dim3(256), 0, s, (const uint16_t*)k_cache, kbar, ksum, g,
                       f_lo, f_hi, c_lo, n_cubes);
  else
    hipLaunchKernelGGL((k_stream_kbar<64>), grid, dim3(256), 0, s, (const uint16_t*)k_cache, kbar, ksum, g,
                       f_lo, f_hi, c_lo, n_cubes);
  return hipGetLastError();
}

}  // namespace adas
