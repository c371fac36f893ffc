// Attention over the selected cubes plus the own cube (AdaSpark,
// papernotes.org, key design 2: attend to the Top-p cube set, always keep full
// attention to the own cube; one exact softmax with scale 1/sqrt(d_k)).
//
// This file holds the float32 path (one wave per row on the vector ALUs, for
// small problems), the merge of split extra-row partials, and the host-side
// planning and dispatch.  The bfloat16 MFMA kernel is in attn_union.hip.
#include "common.h"

namespace adas {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace

// Merge split partial results of extra rows: one wave per row.
// Partials of tile t, chunk q, row r sit at ((t * chunks + q) * TR + r) * (D + 2):
// the row's log2-domain max, its sum, then D unnormalised outputs.
template <int D, int TR>
__global__ __launch_bounds__(256) void k_merge_bf16(AttnArgs a, int n_tiles) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = blockIdx.x * 4 + threadIdx.x / kWave;
  const int tile = wid / TR, r = wid % TR;
  if (tile >= n_tiles) return;
  const int grp = tile / a.extra_tiles_per_group;
  const int rho = (tile - grp * a.extra_tiles_per_group) * TR + r;
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  if (rho >= gsz * a.n_extra) return;
  const int slot = rho / a.n_extra;
  const int hq = a.hg.heads[a.hg.start[grp] + slot];
  const int m = rho - slot * a.n_extra;
  const float* base = a.partials + (size_t)tile * a.extra_chunks * TR * (D + 2);
  float M = -INFINITY;
  for (int q = 0; q < a.extra_chunks; ++q) M = fmaxf(M, base[((size_t)q * TR + r) * (D + 2)]);
  constexpr int PER = D / kWave;
  float o[PER] = {};
  float L = 0.f;
  for (int q = 0; q < a.extra_chunks; ++q) {
    const float* p = base + ((size_t)q * TR + r) * (D + 2);
    const float mq = p[0];
    if (mq == -INFINITY) continue;
    const float w = exp2_fast(mq - M);
    L = fmaf(w, p[1], L);
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = fmaf(w, p[2 + lane * PER + i], o[i]);
  }
  uint16_t* dst = (uint16_t*)a.out_extra + ((size_t)m * a.g.Hq + hq) * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[i] = f32_to_bf16_bits(o[i] / L);
}

// ---------------------------------------------------------------------------
// f32 path: one wave per row.  Keys are processed 64 at a time (one per lane);
// each lane owns D/64 output dims.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a, int total_video_rows) {
  const KGeom& g = a.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int row_id = blockIdx.x * 4 + threadIdx.x / kWave;
  const int total = total_video_rows + g.Hq * a.n_extra;
  if (row_id >= total) return;
  constexpr int PER = D / kWave;
  const float scale = kLog2e / sqrtf((float)D);
  int hq, pos = 0, m = 0, own = -1, row_index;
  bool video = row_id < total_video_rows;
  const float* q;
  int64_t off;
  if (video) {
    hq = row_id / g.N;
    pos = row_id - hq * g.N;
    own = pos / g.S;
    q = (const float*)a.q_cube + ((size_t)hq * g.N + pos) * D;
    off = video_list_offset(a.capv, hq, g.S, own, pos - own * g.S);
    row_index = pos;
  } else {
    const int e = row_id - total_video_rows;
    hq = e / a.n_extra;
    m = e - hq * a.n_extra;
    q = (const float*)a.q_extra + ((size_t)m * g.Hq + hq) * D;
    off = extra_list_offset(a.capv, g.Hq, a.n_extra, g.Nc, hq, m);
    row_index = (a.has_video ? g.N : 0) + m;
  }
  int grp = 0;
  for (int gg = 0; gg < g.Hkv; ++gg)
    for (int t = a.hg.start[gg]; t < a.hg.start[gg + 1]; ++t)
      if (a.hg.heads[t] == hq) grp = gg;
  const int cnt = a.sel_count[(size_t)hq * a.rows_per_head + row_index];
  const int32_t* list = a.sel_idx + off;
  const float* kc = (const float*)a.k_cube + (size_t)grp * g.N * D;
  const float* vc = (const float*)a.v_cube + (size_t)grp * g.N * D;  // [Nc][D][S] per group
  float M = -INFINITY, L = 0.f, o[PER] = {};
  // key sources: own cube (video), selected cubes, then causal text.
  // vat(key, e) reads value dim e of key `key` of the current source.
  auto run_keys = [&](const float* kbase, size_t stride, int nkeys, auto vat) {
    for (int k0 = 0; k0 < nkeys; k0 += kWave) {
      const int key = k0 + lane;
      float s = -INFINITY;
      if (key < nkeys) {
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(q[d], kbase[key * stride + d], acc);
        s = acc * scale;
      }
      const float mb = wave_max(s);
      const float Mn = fmaxf(M, mb);
      const float alpha = exp2_fast(M - Mn);
      const float pv = key < nkeys ? exp2_fast(s - Mn) : 0.f;
      L = L * alpha + wave_sum(pv);
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] *= alpha;
      const int kn = min(kWave, nkeys - k0);
      for (int kk = 0; kk < kn; ++kk) {
        const float pk = __shfl(pv, kk, kWave);
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] = fmaf(pk, vat(k0 + kk, lane * PER + i), o[i]);
      }
      M = Mn;
    }
  };
  auto cube_keys = [&](int j) {
    const float* vcube = vc + (size_t)j * g.S * D;
    run_keys(kc + (size_t)j * g.S * D, D, g.S,
             [&](int key, int e) { return vcube[(size_t)e * g.S + vt_column(key, g.S)]; });
  };
  if (video) cube_keys(own);
  for (int t = 0; t < cnt; ++t) cube_keys(list[t]);
  if (!video && a.n_text_kv > 0) {
    const float* vtext = (const float*)a.v_text + (size_t)grp * D;
    run_keys((const float*)a.k_text + (size_t)grp * D, (size_t)g.Hkv * D, m + 1,
             [&](int key, int e) { return vtext[(size_t)key * g.Hkv * D + e]; });
  }
  float* dst;
  if (video) {
    const int n = raster_of(g, own, pos - own * g.S);
    dst = (float*)a.out_raster + ((size_t)n * g.Hq + hq) * D;
  } else {
    dst = (float*)a.out_extra + ((size_t)m * g.Hq + hq) * D;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[lane * PER + i] = o[i] / L;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
void plan_attention(AttnArgs& a, adas_dtype dt) {
  a.extra_tiles_per_group = 0;
  a.extra_chunks = 1;
  a.extra_chunk_cubes = a.g.Nc;
  if (dt != ADAS_BF16 || a.n_extra == 0) return;
  const int TR = union_tile_rows();
  a.extra_tiles_per_group = (a.hg.gmax * a.n_extra + TR - 1) / TR;
  const int extra_tiles = a.g.Hkv * a.extra_tiles_per_group;
  const long video_wgs = a.has_video
      ? (long)a.g.Nc * a.g.Hkv * ((a.hg.gmax * a.g.S + TR - 1) / TR) : 0;
  int chunks = 1;
  if (video_wgs < 1024) {
    const int want = (2048 + extra_tiles - 1) / extra_tiles;
    const int max_chunks = (a.g.Nc + 7) / 8;  // at least 8 cubes per chunk
    chunks = want < max_chunks ? want : max_chunks;
    if (chunks < 1) chunks = 1;
  }
  a.extra_chunk_cubes = (a.g.Nc + chunks - 1) / chunks;
  a.extra_chunks = (a.g.Nc + a.extra_chunk_cubes - 1) / a.extra_chunk_cubes;
}

size_t attention_workspace_bytes(const AttnArgs& a, adas_dtype dt) {
  if (dt != ADAS_BF16 || a.n_extra == 0 || a.extra_chunks <= 1) return 0;
  const int TR = union_tile_rows();
  return (size_t)a.g.Hkv * a.extra_tiles_per_group * a.extra_chunks * TR * (a.g.D + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, adas_dtype dt, hipStream_t s) {
  if (dt == ADAS_BF16) {
    hipError_t e = a.g.D == 128 ? launch_union<128>(a, s) : launch_union<64>(a, s);
    if (e != hipSuccess) return e;
    if (a.n_extra > 0 && a.extra_chunks > 1) {
      const int n_tiles = a.g.Hkv * a.extra_tiles_per_group;
      constexpr int TRU = 256;
      static_assert(TRU % 4 == 0, "four rows per merge workgroup");
      if (union_tile_rows() != TRU) return hipErrorInvalidValue;
      const int waves = n_tiles * TRU;
      if (a.g.D == 128)
        hipLaunchKernelGGL((k_merge_bf16<128, TRU>), dim3((waves + 3) / 4), dim3(256), 0, s, a, n_tiles);
      else
        hipLaunchKernelGGL((k_merge_bf16<64, TRU>), dim3((waves + 3) / 4), dim3(256), 0, s, a, n_tiles);
      e = hipGetLastError();
    }
    return e;
  }
  const int video_rows = a.has_video ? a.g.Hq * a.g.N : 0;
  const int total = video_rows + a.g.Hq * a.n_extra;
  if (a.g.D == 128)
    hipLaunchKernelGGL((k_attn_f32<128>), dim3((total + 3) / 4), dim3(256), 0, s, a, video_rows);
  else
    hipLaunchKernelGGL((k_attn_f32<64>), dim3((total + 3) / 4), dim3(256), 0, s, a, video_rows);
  return hipGetLastError();
}

}  // namespace adas
