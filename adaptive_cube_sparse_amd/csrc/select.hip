// Selection softmax and Top-p cube sets (AdaSpark, papernotes.org, key design
// 2: P_i = softmax_j(q . kbar_j / sqrt(d_k)) over the preceding cubes,
// S_i = Top-p(P_i, p); key design 4: one threshold p).
//
// bf16 path.  A workgroup (8 waves) owns a tile of RT rows that share a KV
// head and a candidate count n (video rows of one query cube, or extra rows).
//   phase A  scores: z = Q_tile x kbar^T on MFMA (v_mfma_f32_16x16x32_bf16).
//            Each float32 kbar chunk is split in registers into hi + mid + lo
//            bf16 parts, so that three bf16 products reproduce float32
//            accuracy (rounding kbar to bf16 alone would move logits by
//            ~1e-3).  Waves stride over 16-candidate blocks, every kbar load
//            serves all RT rows; logits land in LDS.
//   phase B  per row (one wave): max, exp, sum, then the Top-p threshold
//            search and ascending compaction of topp_select_row().
// f32 path: one wave per row, float32 dot products on the vector ALUs.
#include <algorithm>
#include <utility>

#include "common.h"

namespace adas {

namespace {

struct TileSched {
  int video_tiles_per_group;  // tiles per (kv head, query cube)
  int extra_tiles_per_group;
  int n_extra_tiles;          // Hkv * extra_tiles_per_group (0 in launches without extra rows)
  int c_lo, c_hi;             // video query cubes [c_lo, c_hi) served by this launch
};

// Row rho of a KV-head group -> (query head, position).  Video rows enumerate
// (head slot, offset in cube); extra rows (head slot, token).
struct RowRef {
  int hq;      // -1 = padding row
  int pos;     // cube-layout position (video) or extra token index
  bool video;
};

__device__ __forceinline__ RowRef video_row(const HeadGroups& hg, int grp, int c, int S, int rho) {
  RowRef rr;
  const int slot = rho / S;
  const int gsz = hg.start[grp + 1] - hg.start[grp];
  rr.video = true;
  rr.hq = slot < gsz ? hg.heads[hg.start[grp] + slot] : -1;
  rr.pos = c * S + (rho - slot * S);
  return rr;
}
__device__ __forceinline__ RowRef extra_row(const HeadGroups& hg, int grp, int n_extra, int rho) {
  RowRef rr;
  const int slot = rho / n_extra;
  const int gsz = hg.start[grp + 1] - hg.start[grp];
  rr.video = false;
  rr.hq = slot < gsz ? hg.heads[hg.start[grp] + slot] : -1;
  rr.pos = rho - slot * n_extra;
  return rr;
}

// Decode a workgroup index into (group, candidate count, first row, kind).
// Extra tiles (every cube a candidate) come first, then video tiles in
// descending query-cube order, so the heaviest tiles start first.
__device__ __forceinline__ void decode_tile(int b, const TileSched& ts, int Hkv, int Nc, int RT,
                                            int& grp, int& c, int& rho0, bool& video) {
  if (b < ts.n_extra_tiles) {
    video = false;
    grp = b / ts.extra_tiles_per_group;
    rho0 = (b - grp * ts.extra_tiles_per_group) * RT;
    c = Nc;
  } else {
    video = true;
    b -= ts.n_extra_tiles;
    const int per_c = Hkv * ts.video_tiles_per_group;
    c = ts.c_hi - 1 - b / per_c;
    const int rem = b % per_c;
    grp = rem / ts.video_tiles_per_group;
    rho0 = (rem - grp * ts.video_tiles_per_group) * RT;
  }
}

}  // namespace

// hi + mid + lo bf16 parts of 8 float32 values, so that three bf16 products
// reproduce a float32 product: hi = bf16(x), mid = bf16(x - hi),
// lo = bf16(x - hi - mid) (each subtraction is exact in float32).
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)x[i];
    const float r1 = x[i] - (float)h;
    const __bf16 m = (__bf16)r1;
    hi[i] = h;
    mid[i] = m;
    lo[i] = (__bf16)(r1 - (float)m);
  }
}

constexpr int kSelWaves = 8;

// RT rows per tile (a multiple of 16, or 8), NPL candidate slots per lane
// (capacity 64 * NPL).  Eight waves share every kbar load across RT rows.
template <int D, int RT, int NPL>
__global__ __launch_bounds__(64 * kSelWaves) void k_select_bf16(SelectArgs a, TileSched ts) {
  constexpr int NCAP = kWave * NPL;
  constexpr int RB = (RT + 15) / 16;  // 16-row MFMA blocks
  __shared__ float sZ[RT * NCAP];
  const KGeom& g = a.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  int grp, n, rho0;
  bool video;
  decode_tile(blockIdx.x, ts, g.Hkv, g.Nc, RT, grp, n, rho0, video);
  // n == candidate count: c for a video row in cube c, Nc for extra rows.
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  const int group_rows = video ? gsz * g.S : gsz * a.n_extra;

  // ---- phase A: scores --------------------------------------------------
  // A operand of row block rb: tile row 16*rb + lane%16 (rows beyond the tile
  // are zero), k = 32*s + 8*(lane/16) + [0..7].
  bf16x8 qa[RB][D / 32];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = 16 * rb + lane % 16;
    RowRef rr = {-1, 0, false};
    if (i < RT && rho0 + i < group_rows)
      rr = video ? video_row(a.hg, grp, n, g.S, rho0 + i) : extra_row(a.hg, grp, a.n_extra, rho0 + i);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (rr.hq >= 0 && n > 0) {
        const uint16_t* q = video
            ? (const uint16_t*)a.q_cube + ((size_t)rr.hq * g.N + rr.pos) * D
            : (const uint16_t*)a.q_extra + ((size_t)rr.pos * g.Hq + rr.hq) * D;
        raw = *reinterpret_cast<const uint4*>(q + 32 * s + 8 * (lane / 16));
      }
      qa[rb][s] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const float scale = 1.0f / sqrtf((float)D);
  const float* kb = a.kbar + (size_t)grp * g.Nc * D;
  const int nblk = (n + 15) / 16;
  for (int blk = wave; blk < nblk; blk += kSelWaves) {
    const int j = blk * 16 + lane % 16;
    const int jj = j < n ? j : n - 1;
    f32x4 acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const float4* src = reinterpret_cast<const float4*>(kb + (size_t)jj * D + 32 * s + 8 * (lane / 16));
      const float4 x0 = src[0], x1 = src[1];
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      bf16x8 hi, mid, lo;
      split3(x, hi, mid, lo);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rb][s], lo, acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rb][s], mid, acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rb][s], hi, acc[rb], 0, 0, 0);
      }
    }
    // acc[rb][i] = z for tile row 16*rb + 4*(lane/16) + i, candidate j
    if (j < n) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * rb + 4 * (lane / 16) + i;
          if (row < RT) sZ[row * NCAP + j] = acc[rb][i] * scale;
        }
    }
  }
  __syncthreads();

  // ---- phase B: softmax + Top-p, one row at a time per wave ------------------
  // The row's LDS logits are dead once loaded, so they serve as the wave's
  // 64-float scratch for the Top-p gather.
  for (int row = wave; row < RT; row += kSelWaves) {
    const int rho = rho0 + row;
    if (rho >= group_rows) break;
    const RowRef rr = video ? video_row(a.hg, grp, n, g.S, rho) : extra_row(a.hg, grp, a.n_extra, rho);
    int64_t off;
    int row_index;
    if (video) {
      const int c = rr.pos / g.S;
      off = video_list_offset(a.capv, rr.hq, g.S, c, rr.pos - c * g.S);
      row_index = rr.pos;
    } else {
      off = extra_list_offset(a.capv, g.Hq, a.n_extra, g.Nc, rr.hq, rr.pos);
      row_index = (a.has_video ? g.N : 0) + rr.pos;
    }
    float E[NPL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int j = lane + kWave * i;
      E[i] = j < n ? sZ[row * NCAP + j] : -INFINITY;
      m = fmaxf(m, E[i]);
    }
    m = wave_max(m);
    float zs = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int j = lane + kWave * i;
      E[i] = j < n ? fast_exp(E[i] - m) : -1.0f;
      zs += j < n ? E[i] : 0.0f;
    }
    zs = wave_sum(zs);
    __builtin_amdgcn_wave_barrier();  // all lanes have read the row before it is reused
    const int cnt = topp_select_row<NPL>(E, n, zs, a.p, a.sel_idx + off, &sZ[row * NCAP]);
    if (lane == 0) a.sel_count[(size_t)rr.hq * a.rows_per_head + row_index] = cnt;
  }
}

// f32 path: one wave per row.  Candidates are strided over lanes; each lane
// computes its dot products serially in float32.
template <int D, int NPL>
__global__ __launch_bounds__(256) void k_select_f32(SelectArgs a, int total_video_rows) {
  __shared__ float scratch[4][kWave];
  const KGeom& g = a.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int row_id = blockIdx.x * 4 + threadIdx.x / kWave;
  const int total = total_video_rows + g.Hq * a.n_extra;
  if (row_id >= total) return;
  int hq, n, row_index;
  const float* q;
  int64_t off;
  if (row_id < total_video_rows) {
    hq = row_id / g.N;
    const int pos = row_id - hq * g.N;
    const int c = pos / g.S;
    n = c;
    q = (const float*)a.q_cube + ((size_t)hq * g.N + pos) * D;
    off = video_list_offset(a.capv, hq, g.S, c, pos - c * g.S);
    row_index = pos;
  } else {
    const int e = row_id - total_video_rows;
    hq = e / a.n_extra;
    const int m = e - hq * a.n_extra;
    n = g.Nc;
    q = (const float*)a.q_extra + ((size_t)m * g.Hq + hq) * D;
    off = extra_list_offset(a.capv, g.Hq, a.n_extra, g.Nc, hq, m);
    row_index = (a.has_video ? g.N : 0) + m;
  }
  int grp = 0;
  for (int gg = 0; gg < g.Hkv; ++gg)
    for (int t = a.hg.start[gg]; t < a.hg.start[gg + 1]; ++t)
      if (a.hg.heads[t] == hq) grp = gg;
  const float* kb = a.kbar + (size_t)grp * g.Nc * D;
  const float scale = 1.0f / sqrtf((float)D);
  float E[NPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = lane + kWave * i;
    float z = -INFINITY;
    if (j < n) {
      float s = 0.f;
      for (int k = 0; k < D; ++k) s = fmaf(q[k], kb[(size_t)j * D + k], s);
      z = s * scale;
    }
    E[i] = z;
    m = fmaxf(m, z);
  }
  m = wave_max(m);
  float zs = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = lane + kWave * i;
    E[i] = j < n ? fast_exp(E[i] - m) : -1.0f;
    zs += j < n ? E[i] : 0.0f;
  }
  zs = wave_sum(zs);
  const int cnt = topp_select_row<NPL>(E, n, zs, a.p, a.sel_idx + off, scratch[threadIdx.x / kWave]);
  if (lane == 0) a.sel_count[(size_t)hq * a.rows_per_head + row_index] = cnt;
}

// One launch serves video query cubes [c_lo, c_hi) and, if with_extra, the
// extra rows (which have Nc candidates).
template <int D, int RT, int NPL>
static void launch_bf16(const SelectArgs& a, hipStream_t s, int c_lo, int c_hi, bool with_extra) {
  TileSched ts;
  const int gmax = a.hg.gmax;
  ts.video_tiles_per_group = a.has_video ? (gmax * a.g.S + RT - 1) / RT : 0;
  ts.extra_tiles_per_group = (with_extra && a.n_extra) ? (gmax * a.n_extra + RT - 1) / RT : 0;
  ts.n_extra_tiles = a.g.Hkv * ts.extra_tiles_per_group;
  ts.c_lo = c_lo;
  ts.c_hi = c_hi;
  const int nc = a.has_video && c_hi > c_lo ? c_hi - c_lo : 0;
  const int blocks = ts.n_extra_tiles + nc * a.g.Hkv * ts.video_tiles_per_group;
  if (blocks > 0)
    hipLaunchKernelGGL((k_select_bf16<D, RT, NPL>), dim3(blocks), dim3(64 * kSelWaves), 0, s, a, ts);
}

// Video rows of query cube c have c candidates; split them by capacity so
// that every launch runs loops sized for its candidates (heaviest first).
template <int D>
static void launch_bf16_all(const SelectArgs& a, hipStream_t s) {
  const int Nc = a.g.Nc;
  const int cap_extra = Nc;  // extra rows' candidate count
  auto range = [&](int lo, int hi) { return std::make_pair(std::min(lo, Nc), std::min(hi, Nc)); };
  // [lo, hi) of query cubes handled at each capacity; extra rows go with the
  // capacity that holds Nc.
  {
    auto r = range(1024, 4096);
    if (r.second > r.first || cap_extra > 1024) launch_bf16<D, 8, 64>(a, s, r.first, r.second, cap_extra > 1024);
  }
  {
    auto r = range(512, 1024);
    const bool ex = cap_extra > 512 && cap_extra <= 1024;
    if (r.second > r.first || ex) launch_bf16<D, 32, 16>(a, s, r.first, r.second, ex);
  }
  {
    auto r = range(256, 512);
    const bool ex = cap_extra > 256 && cap_extra <= 512;
    if (r.second > r.first || ex) launch_bf16<D, 32, 8>(a, s, r.first, r.second, ex);
  }
  {
    auto r = range(0, 256);
    const bool ex = cap_extra <= 256;
    if (r.second > r.first || ex) launch_bf16<D, 32, 4>(a, s, r.first, r.second, ex);
  }
}

template <int D, int NPL>
static void launch_f32(const SelectArgs& a, hipStream_t s) {
  const int video_rows = a.has_video ? a.g.Hq * a.g.N : 0;
  const int total = video_rows + a.g.Hq * a.n_extra;
  hipLaunchKernelGGL((k_select_f32<D, NPL>), dim3((total + 3) / 4), dim3(256), 0, s, a, video_rows);
}

hipError_t launch_select(const SelectArgs& a, adas_dtype dt, hipStream_t s) {
  const int Nc = a.g.Nc;
  if (dt == ADAS_BF16) {
    if (a.g.D == 128) launch_bf16_all<128>(a, s);
    else launch_bf16_all<64>(a, s);
  } else {
    if (a.g.D == 128) {
      if (Nc <= 1024) launch_f32<128, 16>(a, s);
      else launch_f32<128, 64>(a, s);
    } else {
      if (Nc <= 1024) launch_f32<64, 16>(a, s);
      else launch_f32<64, 64>(a, s);
    }
  }
  return hipGetLastError();
}

size_t select_workspace_bytes(const KGeom&, adas_dtype) { return 0; }

}  // namespace adas
