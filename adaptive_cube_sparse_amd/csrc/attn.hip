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
// the row's log2-domain max, its sum, then D unnormalised outputs.  One
// workgroup (4 waves) per row: the chunk maxima are reduced first, then each
// wave folds every fourth chunk (lanes own D/64 output dims, loads unrolled so
// several chunks are in flight), and the four waves are summed through LDS.
template <int D, int TR>
__global__ __launch_bounds__(256) void k_merge_bf16(AttnArgs a, int n_tiles) {
  constexpr int PER = D / kWave;
  __shared__ float red_m[4];
  __shared__ float red_o[4][D + 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tile = blockIdx.x / TR, r = blockIdx.x % TR;
  if (tile >= n_tiles) return;
  const int grp = tile / a.extra_tiles_per_group;
  const int rho = (tile - grp * a.extra_tiles_per_group) * TR + r;
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  if (rho >= gsz * a.n_extra) return;  // uniform over the workgroup
  const int slot = rho / a.n_extra;
  const int hq = a.hg.heads[a.hg.start[grp] + slot];
  const int m = rho - slot * a.n_extra;
  const int chunks = a.extra_chunks;
  const size_t stride = (size_t)TR * (D + 2);
  const float* base = a.partials + ((size_t)tile * chunks * TR + r) * (D + 2);
  float M = -INFINITY;
  for (int q = threadIdx.x; q < chunks; q += blockDim.x) M = fmaxf(M, base[q * stride]);
  M = wave_max(M);
  if (lane == 0) red_m[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  float o[PER] = {};
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int q = wave; q < chunks; q += 4) {
      const float* p = base + q * stride;
      const float mq = p[0];
      const float w = mq == -INFINITY ? 0.f : exp2_fast(mq - M);
      L = fmaf(w, p[1], L);
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] = fmaf(w, p[2 + lane * PER + i], o[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) red_o[wave][lane * PER + i] = o[i];
  if (lane == 0) red_o[wave][D] = L;
  __syncthreads();
  if (wave != 0) return;
  const float Lt = red_o[0][D] + red_o[1][D] + red_o[2][D] + red_o[3][D];
  if (a.lse != nullptr && lane == 0)
    a.lse[(size_t)hq * a.rows_per_head + (a.has_video ? a.g.N : 0) + m] = (M + __log2f(Lt)) * 0.69314718055994531f;
  uint16_t* dst = (uint16_t*)a.out_extra + ((size_t)m * a.g.Hq + hq) * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = lane * PER + i;
    const float v = red_o[0][d] + red_o[1][d] + red_o[2][d] + red_o[3][d];
    dst[i] = f32_to_bf16_bits(v / Lt);
  }
}

// Selection bitmap of the extra rows: one workgroup per row (hq, m) turns the
// row's ascending cube list into Nc bits (bit j%32 of word j/32), built with
// LDS atomics and written out once.  The union kernel reads one word per 32
// cubes instead of searching the list.
__global__ __launch_bounds__(256) void k_extra_bitmap(AttnArgs a) {
  __shared__ uint32_t words[ADAS_MAX_CUBES / 32];
  const int row = blockIdx.x;  // hq * n_extra + m
  const int hq = row / a.n_extra, m = row - hq * a.n_extra;
  const int W = a.bits_words;
  for (int w = threadIdx.x; w < W; w += blockDim.x) words[w] = 0u;
  __syncthreads();
  const int cnt = a.sel_count[(size_t)hq * a.rows_per_head + (a.has_video ? a.g.N : 0) + m];
  const int32_t* list = a.sel_idx + extra_list_offset(a.capv, a.g.Hq, a.n_extra, a.g.Nc, hq, m);
  // four list entries per thread in flight before the first LDS update
  for (int i0 = threadIdx.x; i0 < cnt; i0 += 4 * blockDim.x) {
    int j[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * blockDim.x;
      j[u] = i < cnt ? list[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j[u] >= 0) atomicOr(&words[j[u] >> 5], 1u << (j[u] & 31));
  }
  __syncthreads();
  uint32_t* dst = a.extra_bits + (size_t)row * W;
  for (int w = threadIdx.x; w < W; w += blockDim.x) dst[w] = words[w];
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
    q = (const float*)a.q_cube + ((size_t)hq * g.NS + pos) * D;
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
  const float* kc = (const float*)a.k_cube + (size_t)grp * g.NS * D;
  const float* vc = (const float*)a.v_cube + (size_t)grp * g.NS * D;  // [Nc][D][S] per group
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
  if (a.lse != nullptr && lane == 0)
    a.lse[(size_t)hq * a.rows_per_head + row_index] = (M + __log2f(L)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Extra rows (text, decode) are few, so when video tiles do not fill the GPU
// the cube range of each extra tile is split into chunks of a multiple of 32
// cubes, aiming at about two workgroups per CU; each chunk writes partial
// (max, sum, output) rows that k_merge_bf16 combines.
void plan_attention(AttnArgs& a, adas_dtype dt) {
  a.extra_tiles_per_group = 0;
  a.extra_chunks = 1;
  a.extra_chunk_cubes = a.g.Nc;
  a.decode_chunks = 0;
  a.bits_words = (a.g.Nc + 31) / 32;
  if (dt != ADAS_BF16 || a.n_extra == 0) return;
  if (!a.has_video && a.n_text_kv == 0 && a.hg.gmax * a.n_extra <= 32 && a.g.S % 64 == 0) {
    // decode mode: k_attn_decode, one workgroup per (KV head, chunk), about one
    // per CU; each chunk leaves one partial row per extra row.  The decode
    // kernel reads no text keys, so a text prefill (causal text keys) always
    // takes the union tiles, which attend the text keys in chunk 0.
    const int want = (256 + a.g.Hkv - 1) / a.g.Hkv;
    int cubes = (a.g.Nc + want - 1) / want;
    cubes = ((cubes + decode_waves() - 1) / decode_waves()) * decode_waves();
    if (cubes > decode_max_chunk_cubes()) cubes = decode_max_chunk_cubes();
    a.extra_chunk_cubes = cubes;
    a.decode_chunks = (a.g.Nc + cubes - 1) / cubes;
    a.extra_tiles_per_group = 1;
    a.extra_chunks = a.decode_chunks;
    return;
  }
  const int TR = union_tile_rows();
  a.extra_tiles_per_group = (a.hg.gmax * a.n_extra + TR - 1) / TR;
  const int extra_tiles = a.g.Hkv * a.extra_tiles_per_group;
  const long video_wgs = a.has_video
      ? (long)a.g.Nc * a.g.Hkv * ((a.hg.gmax * a.g.S + TR - 1) / TR) : 0;
  if (video_wgs < 1024) {
    const int want = (512 + extra_tiles - 1) / extra_tiles;
    int cubes = (a.g.Nc + want - 1) / want;
    cubes = ((cubes + 31) / 32) * 32;
    if (cubes < 32) cubes = 32;
    a.extra_chunk_cubes = cubes < a.g.Nc ? cubes : a.g.Nc;
  }
  a.extra_chunks = (a.g.Nc + a.extra_chunk_cubes - 1) / a.extra_chunk_cubes;
}

// Workspace of the bf16 attention: [extra-row bitmap][partials], each part
// 256-byte aligned.
static size_t bitmap_bytes(const AttnArgs& a) {
  return ((size_t)a.g.Hq * a.n_extra * a.bits_words * sizeof(uint32_t) + 255) & ~(size_t)255;
}

size_t attention_workspace_bytes(const AttnArgs& a, adas_dtype dt) {
  if (dt != ADAS_BF16 || a.n_extra == 0) return 0;
  size_t bytes = bitmap_bytes(a);
  // the decode kernel always leaves partial rows for k_merge_bf16, even with one chunk
  if (a.extra_chunks > 1 || a.decode_chunks > 0) {
    const int TR = a.decode_chunks > 0 ? 32 : union_tile_rows();
    bytes += (size_t)a.g.Hkv * a.extra_tiles_per_group * a.extra_chunks * TR * (a.g.D + 2) * sizeof(float);
  }
  return bytes;
}

void bind_attention_workspace(AttnArgs& a, adas_dtype dt, void* ws) {
  a.extra_bits = nullptr;
  a.partials = nullptr;
  if (dt != ADAS_BF16 || a.n_extra == 0) return;
  a.extra_bits = (uint32_t*)ws;
  if (a.extra_chunks > 1 || a.decode_chunks > 0) a.partials = (float*)((char*)ws + bitmap_bytes(a));
}

hipError_t launch_attention(const AttnArgs& a, adas_dtype dt, hipStream_t s) {
  if (dt == ADAS_BF16) {
    if (a.n_extra > 0 && !a.bits_ready) {
      hipLaunchKernelGGL(k_extra_bitmap, dim3((unsigned)(a.g.Hq * a.n_extra)), dim3(256), 0, s, a);
      const hipError_t eb = hipGetLastError();
      if (eb != hipSuccess) return eb;
    }
    if (a.decode_chunks > 0) {
      hipError_t e = launch_decode(a, s);
      if (e != hipSuccess) return e;
      const int rows = a.g.Hkv * 32;
      if (a.g.D == 128)
        hipLaunchKernelGGL((k_merge_bf16<128, 32>), dim3(rows), dim3(256), 0, s, a, a.g.Hkv);
      else
        hipLaunchKernelGGL((k_merge_bf16<64, 32>), dim3(rows), dim3(256), 0, s, a, a.g.Hkv);
      return hipGetLastError();
    }
    hipError_t e = a.g.D == 128 ? launch_union<128>(a, s) : launch_union<64>(a, s);
    if (e != hipSuccess) return e;
    if (a.n_extra > 0 && a.extra_chunks > 1) {
      const int n_tiles = a.g.Hkv * a.extra_tiles_per_group;
      constexpr int TRU = 256;
      if (union_tile_rows() != TRU) return hipErrorInvalidValue;
      const int rows = n_tiles * TRU;
      if (a.g.D == 128)
        hipLaunchKernelGGL((k_merge_bf16<128, TRU>), dim3(rows), dim3(256), 0, s, a, n_tiles);
      else
        hipLaunchKernelGGL((k_merge_bf16<64, TRU>), dim3(rows), dim3(256), 0, s, a, n_tiles);
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
