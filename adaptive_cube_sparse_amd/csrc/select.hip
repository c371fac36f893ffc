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
// Extra rows with more than 1024 candidates (decode over a long cache) are few
// and each needs every kbar row, so they take a split path instead: a grid of
// (KV head, 64-cube chunk) workgroups writes their float32 logits to the
// workspace, then one wave per row runs the same softmax and Top-p search.
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


// The split path serves extra rows with more than 1024 candidates when a KV
// head has few of them (at most 64, e.g. decode steps); many extra rows fill
// the GPU through the fused kernel's row tiles instead.
bool use_split_select(const KGeom& g, int n_extra, int gmax) {
  return n_extra > 0 && g.Nc > 1024 && gmax * n_extra <= 64;
}

// RT rows per tile (a multiple of 16, or 8), NPL candidate slots per lane
// (capacity 64 * NPL), NW waves that share every kbar load across RT rows.
// Bands whose logits fill most of the LDS (one workgroup per CU) take 16
// waves, so that each SIMD still holds four of them.
// Tile b of a band (sZ: RT * 64 * NPL floats of LDS).
template <int D, int RT, int NPL, int NW>
__device__ __forceinline__ void select_tile(const SelectArgs& a, const TileSched& ts, int b, float* sZ) {
  constexpr int NCAP = kWave * NPL;
  constexpr int RB = (RT + 15) / 16;  // 16-row MFMA blocks
  const KGeom& g = a.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  int grp, n, rho0;
  bool video;
  decode_tile(b, ts, g.Hkv, g.Nc, RT, grp, n, rho0, video);
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
            ? (const uint16_t*)a.q_cube + ((size_t)rr.hq * g.NS + rr.pos) * D
            : (const uint16_t*)a.q_extra + ((size_t)rr.pos * g.Hq + rr.hq) * D;
        raw = *reinterpret_cast<const uint4*>(q + 32 * s + 8 * (lane / 16));
      }
      qa[rb][s] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const float scale = 1.0f / sqrtf((float)D);
  const float* kb = a.kbar + (size_t)grp * (g.NS / g.S) * D;
  const int nblk = (n + 15) / 16;
  for (int blk = wave; blk < nblk; blk += NW) {
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
  for (int row = wave; row < RT; row += NW) {
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
    int cnt;
    if (a.topk > 0) {
      cnt = topk_select_row<NPL>(E, n, a.topk, a.sel_idx + off);
    } else {
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
      cnt = topp_select_row<NPL>(E, n, zs, a.p, a.sel_idx + off, &sZ[row * NCAP]);
    }
    if (lane == 0) a.sel_count[(size_t)rr.hq * a.rows_per_head + row_index] = cnt;
  }
}

// One band per launch.
template <int D, int RT, int NPL, int NW>
__global__ __launch_bounds__(64 * NW) void k_select_bf16(SelectArgs a, TileSched ts) {
  __shared__ float sZ[RT * kWave * NPL];
  select_tile<D, RT, NPL, NW>(a, ts, blockIdx.x, sZ);
}

// Several bands of 32-row tiles with one workgroup size in one launch, so the
// partly filled last round of each band's workgroups overlaps the next band
// instead of leaving CUs idle; the LDS holds the largest band's logits.
// NW = 16: the 768 and 1024-candidate bands; NW = 8: bands of at most 384.
constexpr int kMaxBands = 4;
struct BandSet {
  TileSched ts[kMaxBands];
  int npl[kMaxBands];
  int first[kMaxBands + 1];  // first workgroup of each band; first[n] = total
  int n;
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_select_bands(SelectArgs a, BandSet bs) {
  constexpr int MAXNPL = NW == 16 ? 16 : 6;
  __shared__ float sZ[32 * kWave * MAXNPL];
  const int b = blockIdx.x;
  int i = 0;
  while (i + 1 < bs.n && b >= bs.first[i + 1]) ++i;
  const int lb = b - bs.first[i];
  if constexpr (NW == 16) {
    if (bs.npl[i] == 16) select_tile<D, 32, 16, 16>(a, bs.ts[i], lb, sZ);
    else select_tile<D, 32, 12, 16>(a, bs.ts[i], lb, sZ);
  } else {
    switch (bs.npl[i]) {
      case 6: select_tile<D, 32, 6, 8>(a, bs.ts[i], lb, sZ); break;
      case 4: select_tile<D, 32, 4, 8>(a, bs.ts[i], lb, sZ); break;
      case 2: select_tile<D, 32, 2, 8>(a, bs.ts[i], lb, sZ); break;
      default: select_tile<D, 32, 1, 8>(a, bs.ts[i], lb, sZ); break;
    }
  }
}

// Split selection, step 1: logits of the extra rows of KV head blockIdx.y for
// candidates 64*blockIdx.x .. +64.  The kbar chunk and the group's (at most
// 64) query rows sit in LDS as float32 (kbar rows padded by one float);
// thread pairs (row, candidate) take float32 dot products.
template <int D>
__global__ __launch_bounds__(256) void k_select_scores(SelectArgs a) {
  __shared__ float kb[64 * (D + 1)];
  __shared__ float qs[64 * D];
  const KGeom& g = a.g;
  const int grp = blockIdx.y;
  const int j0 = 64 * blockIdx.x;
  const int nj = min(64, g.Nc - j0);
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  const int rows = gsz * a.n_extra;  // <= 64 on this path
  // 16-byte loads, all issued before any LDS store (the chunk is 64*D floats)
  const float4* src = reinterpret_cast<const float4*>(a.kbar + ((size_t)grp * (g.NS / g.S) + j0) * D);
  constexpr int NV = 64 * D / 4 / 256;
  float4 v[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = threadIdx.x + 256 * u;
    v[u] = e < nj * D / 4 ? src[e] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int e = threadIdx.x; e < rows * D / 8; e += blockDim.x) {
    const int rho = e / (D / 8), c8 = e % (D / 8);
    const RowRef rr = extra_row(a.hg, grp, a.n_extra, rho);
    const uint4 raw = *reinterpret_cast<const uint4*>((const uint16_t*)a.q_extra +
                                                      ((size_t)rr.pos * g.Hq + rr.hq) * D + 8 * c8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qs[rho * D + 8 * c8 + 2 * t] = __uint_as_float(w[t] << 16);
      qs[rho * D + 8 * c8 + 2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = 4 * (threadIdx.x + 256 * u);
    float* dst = &kb[(e / D) * (D + 1) + e % D];
    dst[0] = v[u].x;
    dst[1] = v[u].y;
    dst[2] = v[u].z;
    dst[3] = v[u].w;
  }
  __syncthreads();
  const float scale = 1.0f / sqrtf((float)D);
  for (int e = threadIdx.x; e < rows * 64; e += blockDim.x) {
    const int rho = e >> 6, jl = e & 63;
    if (jl >= nj) continue;
    const float* q = &qs[rho * D];
    const float* k = &kb[jl * (D + 1)];
    float s = 0.f;
#pragma unroll 16
    for (int d = 0; d < D; ++d) s = fmaf(q[d], k[d], s);
    const RowRef rr = extra_row(a.hg, grp, a.n_extra, rho);
    a.zbuf[((size_t)rr.hq * a.n_extra + rr.pos) * g.Nc + j0 + jl] = s * scale;
  }
}

// Split selection, step 2: one workgroup (SW waves) per extra row (hq, m).
// The same Top-p search as topp_select_row(), spread over the workgroup: wave
// w holds candidates w*C .. w*C + C - 1 (C = 64*NPL, stripe i of lane L is
// candidate w*C + 64*i + L), mass and count sums go through LDS (two slots
// used alternately, so one barrier per bisection step), the <= 64 elements
// left between the bounds are gathered for wave 0 to finish on single
// registers, and the ascending compaction gives each wave its output offset
// from the per-wave counts.
constexpr int SW = 8;  // waves per row in the split path

template <int NPL>
__global__ __launch_bounds__(64 * SW) void k_select_rows(SelectArgs a) {
  constexpr int C = kWave * NPL;
  __shared__ float red_f[2][SW];
  __shared__ int red_i[2][SW];
  __shared__ float gath[kWave];
  __shared__ int n_gath;
  __shared__ float tau_s;
  __shared__ int cgt_s[SW], ceq_s[SW];
  const KGeom& g = a.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int row = blockIdx.x;  // hq * n_extra + m
  const int hq = row / a.n_extra, m = row - hq * a.n_extra;
  const int n = g.Nc;
  const float* z = a.zbuf + (size_t)row * n;
  int slot = 0;
  // workgroup-wide sum of (x, c); every thread gets the totals
  auto block_sum = [&](float x, int c, float& xs, int& cs) __attribute__((always_inline)) {
    x = wave_sum(x);
    if (lane == 0) {
      red_f[slot][wave] = x;
      red_i[slot][wave] = c;
    }
    __syncthreads();
    xs = 0.f;
    cs = 0;
#pragma unroll
    for (int w = 0; w < SW; ++w) {
      xs += red_f[slot][w];
      cs += red_i[slot][w];
    }
    slot ^= 1;
  };
  float E[NPL];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = wave * C + kWave * i + lane;
    E[i] = j < n ? z[j] : -INFINITY;
    mx = fmaxf(mx, E[i]);
  }
  const int64_t off0 = extra_list_offset(a.capv, g.Hq, a.n_extra, g.Nc, hq, m);
  if (a.topk > 0) {
    // Top-K: the k-th largest ordered key, built bit by bit with block-wide
    // counts, then the keys above it and the lowest-index ties, ascending
    const int K = a.topk;
    int32_t* outk = a.sel_idx + off0;
    if (K >= n) {
      for (int j = threadIdx.x; j < n; j += blockDim.x) outk[j] = j;
      if (threadIdx.x == 0) a.sel_count[(size_t)hq * a.rows_per_head + (a.has_video ? g.N : 0) + m] = n;
      return;
    }
    uint32_t u[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) u[i] = wave * C + kWave * i + lane < n ? ordered_key(E[i]) : 0u;
    uint32_t t = 0u;
    float unused;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) c += popc64(__ballot(u[i] >= cand));
      int call;
      block_sum(0.f, c, unused, call);
      if (call >= K) t = cand;
    }
    int cgt = 0, ceq = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      cgt += popc64(__ballot(u[i] > t));
      ceq += popc64(__ballot(u[i] == t));
    }
    if (lane == 0) {
      cgt_s[wave] = cgt;
      ceq_s[wave] = ceq;
    }
    int cgt_all;
    block_sum(0.f, cgt, unused, cgt_all);
    const int keq = K - cgt_all;
    int eqb = 0, basek = 0;
    for (int w = 0; w < wave; ++w) {
      basek += cgt_s[w] + max(0, min(ceq_s[w], keq - eqb));
      eqb += ceq_s[w];
    }
    int eq_seen = eqb;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const bool eq = u[i] == t;
      const uint64_t beq = __ballot(eq);
      const bool sel = u[i] > t || (eq && eq_seen + lanes_below(beq) < keq);
      const uint64_t bs = __ballot(sel);
      if (sel) outk[basek + lanes_below(bs)] = wave * C + kWave * i + lane;
      basek += popc64(bs);
      eq_seen += popc64(beq);
    }
    if (threadIdx.x == 0) a.sel_count[(size_t)hq * a.rows_per_head + (a.has_video ? g.N : 0) + m] = K;
    return;
  }
  mx = wave_max(mx);
  if (lane == 0) red_f[slot][wave] = mx;
  __syncthreads();
  mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < SW; ++w) mx = fmaxf(mx, red_f[slot][w]);
  slot ^= 1;
  float zs = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = wave * C + kWave * i + lane;
    E[i] = j < n ? fast_exp(E[i] - mx) : -1.0f;
    zs += j < n ? E[i] : 0.0f;
  }
  float Z;
  int dummy;
  block_sum(zs, 0, Z, dummy);
  const int64_t off = extra_list_offset(a.capv, g.Hq, a.n_extra, g.Nc, hq, m);
  int32_t* out = a.sel_idx + off;
  uint32_t* const bits = a.extra_bits != nullptr ? a.extra_bits + (size_t)row * a.bits_words : nullptr;
  if (a.p >= 1.0f) {
    for (int j = threadIdx.x; j < n; j += blockDim.x) out[j] = j;
    if (bits != nullptr)
      for (int w = threadIdx.x; w < a.bits_words; w += blockDim.x) {
        const int left = n - 32 * w;  // >= 1: bits_words = ceil(n / 32)
        bits[w] = left >= 32 ? 0xFFFFFFFFu : (1u << left) - 1u;
      }
    if (threadIdx.x == 0) a.sel_count[(size_t)hq * a.rows_per_head + (a.has_video ? g.N : 0) + m] = n;
    return;
  }
  const float target = a.p * Z;
  // 1. bisection on float bits over all candidates, from the bracket
  //    [x0, 1] with x0 = (1 - p) Z / (2n) (see topp_select_row)
  uint32_t lo = __float_as_uint(0.5f * (1.0f - a.p) * Z / (float)n), hi = 0x3F800001u;
  int cnt_lo = 0, cnt_hi = 0;
  {
    const float f0 = __uint_as_float(lo);
    int c0 = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) c0 += popc64(__ballot(E[i] >= f0));
    float unused;
    block_sum(0.f, c0, unused, cnt_lo);
  }
  float tau = 0.0f;
  bool found = false;
  while (cnt_lo - cnt_hi > kWave && hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const float fm = __uint_as_float(mid);
    float ms = 0.0f;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const bool ge = E[i] >= fm;
      ms += ge ? E[i] : 0.0f;
      cnt += popc64(__ballot(ge));
    }
    block_sum(ms, cnt, ms, cnt);
    if (ms >= target) {
      lo = mid;
      cnt_lo = cnt;
    } else {
      hi = mid;
      cnt_hi = cnt;
    }
  }
  if (hi - lo <= 1u) {
    tau = __uint_as_float(lo);
    found = true;
  }
  if (!found) {
    // 2. fixed mass at or above hi; gather the (<= 64) elements in [lo, hi)
    const float flo = __uint_as_float(lo), fhi = __uint_as_float(hi);
    if (threadIdx.x == 0) n_gath = 0;
    __syncthreads();
    float mhi = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      mhi += E[i] >= fhi ? E[i] : 0.0f;
      const bool in = E[i] >= flo && E[i] < fhi;
      const uint64_t bl = __ballot(in);
      int base = 0;
      if (bl != 0ull && lane == 0) base = atomicAdd(&n_gath, popc64(bl));
      base = __shfl(base, 0, kWave);
      if (in) gath[base + lanes_below(bl)] = E[i];
    }
    block_sum(mhi, 0, mhi, dummy);  // its barrier also publishes gath / n_gath
    if (wave == 0) {
      const int ng = n_gath;
      const float v = lane < ng ? gath[lane] : -1.0f;
      // 3. bisection on one value per lane below the gather-time bound
      const int cnt_hi0 = cnt_hi;
      for (;;) {
        if (cnt_lo - cnt_hi == 1) {
          tau = wave_max(v >= __uint_as_float(lo) && v < __uint_as_float(hi) ? v : -1.0f);
          break;
        }
        if (hi - lo <= 1u) {
          tau = __uint_as_float(lo);
          break;
        }
        const uint32_t mid = lo + ((hi - lo) >> 1);
        const float fm = __uint_as_float(mid);
        const bool ge = v >= fm;
        const int cnt = cnt_hi0 + popc64(__ballot(ge));
        const float ms = mhi + wave_sum(ge ? v : 0.0f);
        if (ms >= target) {
          lo = mid;
          cnt_lo = cnt;
        } else {
          hi = mid;
          cnt_hi = cnt;
        }
      }
      if (lane == 0) tau_s = tau;
    }
    __syncthreads();
    tau = tau_s;
  }
  // mass strictly above tau, ties at tau, per-wave counts for the compaction
  float mgt = 0.0f;
  int cgt = 0, ceq = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    mgt += E[i] > tau ? E[i] : 0.0f;
    cgt += popc64(__ballot(E[i] > tau));
    ceq += popc64(__ballot(E[i] == tau));
  }
  if (lane == 0) {
    cgt_s[wave] = cgt;
    ceq_s[wave] = ceq;
  }
  int ceq_all;
  block_sum(mgt, ceq, mgt, ceq_all);
  int keq = ceq_all;
  if (tau > 0.0f) {
    int k = (int)ceilf((target - mgt) / tau);
    if (k < 1) k = 1;
    if (k < keq) keq = k;
  }
  // ties are taken in ascending candidate order: waves below this one first
  int eq_before = 0, base = 0, total = 0;
  {
    int eqb = 0;
    for (int w = 0; w < SW; ++w) {
      const int take = max(0, min(ceq_s[w], keq - eqb));
      const int sel_w = cgt_s[w] + take;
      if (w < wave) base += sel_w;
      if (w == wave) eq_before = eqb;
      total += sel_w;
      eqb += ceq_s[w];
    }
  }
  int eq_seen = eq_before;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool eq = E[i] == tau;
    const uint64_t beq = __ballot(eq);
    const int eq_rank = eq_seen + lanes_below(beq);
    const bool sel = (E[i] > tau) || (eq && eq_rank < keq);
    const uint64_t bs = __ballot(sel);
    if (sel) out[base + lanes_below(bs)] = wave * C + kWave * i + lane;
    base += popc64(bs);
    eq_seen += popc64(beq);
    // candidates wave*C + 64*i + lane are bits of words w0 (lanes 0..31) and
    // w0 + 1 (lanes 32..63); every word below bits_words has one writer
    if (bits != nullptr) {
      const int w0 = (wave * C + kWave * i) >> 5;
      if (lane < 2 && w0 + lane < a.bits_words) bits[w0 + lane] = (uint32_t)(bs >> (32 * lane));
    }
  }
  if (threadIdx.x == 0) a.sel_count[(size_t)hq * a.rows_per_head + (a.has_video ? g.N : 0) + m] = total;
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
    q = (const float*)a.q_cube + ((size_t)hq * g.NS + pos) * D;
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
  const float* kb = a.kbar + (size_t)grp * (g.NS / g.S) * D;
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
  if (a.topk > 0) {
    const int cnt = topk_select_row<NPL>(E, n, a.topk, a.sel_idx + off);
    if (lane == 0) a.sel_count[(size_t)hq * a.rows_per_head + row_index] = cnt;
    return;
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
// Tiles of RT rows for video query cubes [c_lo, c_hi) and, if with_extra, the
// extra rows; returns the workgroup count.
static int band_sched(const SelectArgs& a, int RT, int c_lo, int c_hi, bool with_extra, TileSched& ts) {
  const int gmax = a.hg.gmax;
  ts.video_tiles_per_group = a.has_video ? (gmax * a.g.S + RT - 1) / RT : 0;
  ts.extra_tiles_per_group = (with_extra && a.n_extra) ? (gmax * a.n_extra + RT - 1) / RT : 0;
  ts.n_extra_tiles = a.g.Hkv * ts.extra_tiles_per_group;
  ts.c_lo = c_lo;
  ts.c_hi = c_hi;
  const int nc = a.has_video && c_hi > c_lo ? c_hi - c_lo : 0;
  return ts.n_extra_tiles + nc * a.g.Hkv * ts.video_tiles_per_group;
}

template <int D, int RT, int NPL, int NW>
static void launch_bf16(const SelectArgs& a, hipStream_t s, int c_lo, int c_hi, bool with_extra) {
  TileSched ts;
  const int blocks = band_sched(a, RT, c_lo, c_hi, with_extra, ts);
  if (blocks > 0)
    hipLaunchKernelGGL((k_select_bf16<D, RT, NPL, NW>), dim3(blocks), dim3(64 * NW), 0, s, a, ts);
}

// Adds band (npl, c_lo, c_hi, with_extra) of 32-row tiles to a band set.
static void add_band(const SelectArgs& a, BandSet& bs, int npl, int c_lo, int c_hi, bool with_extra) {
  TileSched ts;
  const int blocks = band_sched(a, 32, c_lo, c_hi, with_extra, ts);
  if (blocks <= 0) return;
  if (bs.n == 0) bs.first[0] = 0;
  bs.ts[bs.n] = ts;
  bs.npl[bs.n] = npl;
  bs.first[bs.n + 1] = bs.first[bs.n] + blocks;
  ++bs.n;
}

template <int D, int NW>
static void launch_bands(const SelectArgs& a, hipStream_t s, const BandSet& bs) {
  if (bs.n > 0)
    hipLaunchKernelGGL((k_select_bands<D, NW>), dim3(bs.first[bs.n]), dim3(64 * NW), 0, s, a, bs);
}

// Video rows of query cube c have c candidates; split them by capacity so
// that every launch runs loops sized for its candidates (heaviest first).
// Each band [lo, hi) gets NPL = hi / 64 slots per lane; extra rows (Nc
// candidates) go with the band that holds Nc, unless the split path takes them.
template <int D>
static void launch_bf16_all(const SelectArgs& a, hipStream_t s) {
  const int Nc = a.g.Nc;
  const bool split = use_split_select(a.g, a.n_extra, a.hg.gmax);
  const bool extra = a.n_extra > 0 && !split;
  auto band = [&](auto launch, int lo, int hi) {
    const int l = std::min(lo, Nc), h = std::min(hi, Nc);
    const bool ex = extra && Nc > lo && Nc <= hi;
    if (h > l || ex) launch(l, h, ex);
  };
  BandSet big{}, small{};
  band([&](int l, int h, bool ex) { launch_bf16<D, 8, 64, 16>(a, s, l, h, ex); }, 2048, 4096);
  band([&](int l, int h, bool ex) { launch_bf16<D, 16, 32, 16>(a, s, l, h, ex); }, 1024, 2048);
  band([&](int l, int h, bool ex) { add_band(a, big, 16, l, h, ex); }, 768, 1024);
  band([&](int l, int h, bool ex) { add_band(a, big, 12, l, h, ex); }, 512, 768);
  launch_bands<D, 16>(a, s, big);
  // 512 candidates (64 KB of logits, two workgroups per CU) alone: with the
  // smaller bands it would lower their occupancy
  band([&](int l, int h, bool ex) { launch_bf16<D, 32, 8, 8>(a, s, l, h, ex); }, 384, 512);
  band([&](int l, int h, bool ex) { add_band(a, small, 6, l, h, ex); }, 256, 384);
  band([&](int l, int h, bool ex) { add_band(a, small, 4, l, h, ex); }, 128, 256);
  band([&](int l, int h, bool ex) { add_band(a, small, 2, l, h, ex); }, 64, 128);
  band([&](int l, int h, bool ex) { add_band(a, small, 1, l, h, ex); }, 0, 64);
  launch_bands<D, 8>(a, s, small);
  if (split) {
    // split path for the extra rows (workspace holds their logits)
    hipLaunchKernelGGL((k_select_scores<D>), dim3((Nc + 63) / 64, a.g.Hkv), dim3(256), 0, s, a);
    const int rows = a.g.Hq * a.n_extra;
    static_assert(ADAS_MAX_CUBES <= kWave * 8 * SW, "split-path capacity");
    hipLaunchKernelGGL((k_select_rows<8>), dim3(rows), dim3(64 * SW), 0, s, a);
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

// Only the split path keeps logits in the workspace.
size_t select_workspace_bytes(const KGeom& g, adas_dtype dt, int n_extra, int gmax) {
  if (dt != ADAS_BF16 || !use_split_select(g, n_extra, gmax)) return 0;
  return (size_t)g.Hq * n_extra * g.Nc * sizeof(float);
}

}  // namespace adas
