// Attention over the selected cubes plus the own cube (AdaSpark,
// papernotes.org, key design 2: attend to the Top-p cube set, always keep full
// attention to the own cube; one exact softmax with scale 1/sqrt(d_k)).
//
// bf16 path, MFMA (v_mfma_f32_16x16x32_bf16), one workgroup = 4 waves per
// tile of TR rows that read the same KV head.
//
// Rows of a tile choose *different* cube sets, so a dense tile would spend
// most MFMA work on masked keys.  Instead, for every key block (64 keys of a
// cube) the rows that selected that cube are gathered into 16-row MFMA
// blocks; each block computes S^T = K Q^T, a per-row online-softmax update,
// and O^T += V^T P^T, then folds O into the row's float32 accumulator in LDS.
// Key blocks are processed one at a time by the whole workgroup, so every row
// appears at most once per block and the LDS updates never race.  The next
// key block's K and V are fetched into registers while the current one is
// computed.
//
// LDS (D = 128, TR = 128): Q tile 34 KB, accumulators 66 KB, K 17 KB,
// V^T 18 KB, masks/lists ~2 KB.
//
// f32 path: one wave per row on the vector ALUs (small problems).
#include <cstdlib>

#include "common.h"

namespace adas {

namespace {

constexpr int KB = 64;        // keys per key block
constexpr int PASS = 64;      // cubes per mask-building pass
constexpr float kLog2e = 1.4426950408889634f;

struct AttnSched {
  int video_tiles_per_group;
  int extra_tiles_per_group;
  int extra_chunks;
  int extra_chunk_cubes;
  int n_extra_wgs;  // Hkv * extra_tiles_per_group * extra_chunks
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace

template <int D, int TR>
struct AttnSmem {
  static constexpr int QS = D + 8;     // bf16 stride of a Q row
  static constexpr int AS = D + 4;     // float stride of an accumulator row
  static constexpr int KS = D + 8;     // bf16 stride of a K row
  static constexpr int VS = KB + 8;    // bf16 stride of a V^T row
  static constexpr int MW = TR / 32;   // mask words per cube
  uint16_t q[TR * QS];
  float acc[TR * AS];
  float m[TR];
  float l[TR];
  uint16_t k[KB * KS];
  uint16_t vt[D * VS];
  uint32_t mask[PASS * MW];
  int16_t rows[TR];
  int32_t row_hq[TR];
  int32_t row_pos[TR];
  int32_t cubes[PASS];
  int32_t n_cubes;
};

template <int D, int TR>
__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a, AttnSched sc) {
  using Sm = AttnSmem<D, TR>;
  __shared__ Sm sm;
  const KGeom& g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int lg = lane / 16;   // lane group 0..3
  const int li = lane % 16;   // lane index in group

  // ---- decode the tile ------------------------------------------------------
  bool video;
  int grp, rho0, c = 0, chunk = 0;
  int b = blockIdx.x;
  if (b < sc.n_extra_wgs) {
    video = false;
    const int tile = b / sc.extra_chunks;
    chunk = b - tile * sc.extra_chunks;
    grp = tile / sc.extra_tiles_per_group;
    rho0 = (tile - grp * sc.extra_tiles_per_group) * TR;
  } else {
    video = true;
    b -= sc.n_extra_wgs;
    const int per_c = g.Hkv * sc.video_tiles_per_group;
    c = g.Nc - 1 - b / per_c;
    const int rem = b % per_c;
    grp = rem / sc.video_tiles_per_group;
    rho0 = (rem - grp * sc.video_tiles_per_group) * TR;
  }
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  const int group_rows = video ? gsz * g.S : gsz * a.n_extra;
  const int n_rows = min(TR, group_rows - rho0);
  if (n_rows <= 0) return;
  const int hstart = a.hg.start[grp];

  // ---- row metadata, Q tile, state init -------------------------------------
  for (int t = tid; t < TR; t += 256) {
    int hq = -1, pos = 0;
    if (t < n_rows) {
      const int rho = rho0 + t;
      if (video) {
        const int slot = rho / g.S;
        hq = a.hg.heads[hstart + slot];
        pos = c * g.S + (rho - slot * g.S);
      } else {
        const int slot = rho / a.n_extra;
        hq = a.hg.heads[hstart + slot];
        pos = rho - slot * a.n_extra;
      }
    }
    sm.row_hq[t] = hq;
    sm.row_pos[t] = pos;
    sm.m[t] = -INFINITY;
    sm.l[t] = 0.f;
  }
  for (int e = tid; e < TR * D / 4; e += 256) {
    const int r = e / (D / 4), cc = e % (D / 4);
    *reinterpret_cast<float4*>(&sm.acc[r * Sm::AS + cc * 4]) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  constexpr int VPR = D / 8;  // 16-byte vectors per bf16 row
  for (int e = tid; e < TR * VPR; e += 256) {
    const int r = e / VPR, v = e % VPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < n_rows) {
      const int hq = sm.row_hq[r], pos = sm.row_pos[r];
      const uint16_t* src = video ? (const uint16_t*)a.q_cube + ((size_t)hq * g.N + pos) * D
                                  : (const uint16_t*)a.q_extra + ((size_t)pos * g.Hq + hq) * D;
      val = *reinterpret_cast<const uint4*>(src + v * 8);
    }
    *reinterpret_cast<uint4*>(&sm.q[r * Sm::QS + v * 8]) = val;
  }

  // per-thread selection cursor for row `tid` (tid < TR)
  int my_cnt = 0, my_cur = 0;
  const int32_t* my_list = nullptr;
  if (tid < n_rows) {
    const int hq = sm.row_hq[tid], pos = sm.row_pos[tid];
    int64_t off;
    int row_index;
    if (video) {
      const int cc = pos / g.S;
      off = video_list_offset(a.capv, hq, g.S, cc, pos - cc * g.S);
      row_index = pos;
    } else {
      off = extra_list_offset(a.capv, g.Hq, a.n_extra, g.Nc, hq, pos);
      row_index = (a.has_video ? g.N : 0) + pos;
    }
    my_list = a.sel_idx + off;
    my_cnt = a.sel_count[(size_t)hq * a.rows_per_head + row_index];
    if (!video && chunk > 0) {  // first entry >= chunk start (lists are ascending)
      const int key = chunk * sc.extra_chunk_cubes;
      int lo = 0, hi = my_cnt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (my_list[mid] < key) lo = mid + 1; else hi = mid;
      }
      my_cur = lo;
    }
  }
  __syncthreads();

  const float qscale = kLog2e / sqrtf((float)D);  // scores kept in log2 units

  // ---- K/V block staging ------------------------------------------------------
  constexpr int KV_VECS = KB * VPR;                 // 16-byte vectors per K block
  constexpr int KV_PER_T = (KV_VECS + 255) / 256;
  uint4 kr[KV_PER_T], vr[KV_PER_T];
  auto fetch_kv = [&](const uint16_t* kbase, const uint16_t* vbase, size_t row_stride, int kc) {
#pragma unroll
    for (int u = 0; u < KV_PER_T; ++u) {
      const int e = tid + 256 * u;
      const int key = e / VPR, v = e % VPR;
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (e < KV_VECS && key < kc) {
        kr[u] = *reinterpret_cast<const uint4*>(kbase + key * row_stride + v * 8);
        vr[u] = *reinterpret_cast<const uint4*>(vbase + key * row_stride + v * 8);
      }
    }
  };
  auto store_kv = [&]() {
#pragma unroll
    for (int u = 0; u < KV_PER_T; ++u) {
      const int e = tid + 256 * u;
      if (e < KV_VECS) {
        const int key = e / VPR, v = e % VPR;
        *reinterpret_cast<uint4*>(&sm.k[key * Sm::KS + v * 8]) = kr[u];
        const uint32_t w[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm.vt[(v * 8 + 2 * i) * Sm::VS + key] = (uint16_t)(w[i] & 0xFFFFu);
          sm.vt[(v * 8 + 2 * i + 1) * Sm::VS + key] = (uint16_t)(w[i] >> 16);
        }
      }
    }
  };

  // ---- one key block for the rows listed in sm.rows[0..nr) ------------------
  // kc valid keys; causal: key index kbase_idx + kk must be <= row's token.
  auto compute_block = [&](int nr, int kc, bool causal, int kbase_idx) {
    const int nblk = (nr + 15) / 16;
    for (int blk = wave; blk < nblk; blk += 4) {
      const int slot = blk * 16 + li;
      const bool valid = slot < nr;
      const int row = sm.rows[valid ? slot : 0];
      // S^T = K Q^T : 4 key sub-blocks of 16
      f32x4 st[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const bf16x8 qb = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&sm.q[row * Sm::QS + 32 * s + 8 * lg]));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (kb * 16 < kc) {
            const bf16x8 ka = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4*>(&sm.k[(kb * 16 + li) * Sm::KS + 32 * s + 8 * lg]));
            st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb, st[kb], 0, 0, 0);
          }
        }
      }
      // online softmax for row `row` (lanes li, li+16, li+32, li+48 share it)
      const int rtok = causal ? sm.row_pos[row] : 0;
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb * 16 + 4 * lg + i;
          const bool ok = key < kc && (!causal || kbase_idx + key <= rtok);
          const float sv = ok ? st[kb][i] * qscale : -INFINITY;
          st[kb][i] = sv;
          mloc = fmaxf(mloc, sv);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
      const float m_old = sm.m[row];
      const float m_new = fmaxf(m_old, mloc);
      const float alpha = exp2_fast(m_old - m_new);
      float lsum = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = exp2_fast(st[kb][i] - m_new);
          const __bf16 pbv = f32_to_bf16(pv);
          lsum += (float)pbv;
          pb[kb / 2][(kb % 2) * 4 + i] = pbv;
        }
      lsum += __shfl_xor(lsum, 16, kWave);
      lsum += __shfl_xor(lsum, 32, kWave);
      // O^T = V^T P^T : D/16 d-blocks x 2 k-steps of 32 keys
      f32x4 ob[D / 16];
#pragma unroll
      for (int db = 0; db < D / 16; ++db) ob[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks * 32 < kc) {
#pragma unroll
          for (int db = 0; db < D / 16; ++db) {
            const uint16_t* vrow = &sm.vt[(db * 16 + li) * Sm::VS];
            const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (2 * ks) * 16 + 4 * lg);
            const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (2 * ks + 1) * 16 + 4 * lg);
            const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
            ob[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ks], ob[db], 0, 0, 0);
          }
        }
      }
      if (valid) {
        float* accrow = &sm.acc[row * Sm::AS];
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          float4* p = reinterpret_cast<float4*>(accrow + db * 16 + 4 * lg);
          float4 o = *p;
          o.x = fmaf(alpha, o.x, ob[db][0]);
          o.y = fmaf(alpha, o.y, ob[db][1]);
          o.z = fmaf(alpha, o.z, ob[db][2]);
          o.w = fmaf(alpha, o.w, ob[db][3]);
          *p = o;
        }
        if (lg == 0) {
          sm.l[row] = fmaf(alpha, sm.l[row], lsum);
          sm.m[row] = m_new;
        }
      }
    }
  };

  // rows of the tile selected by mask words w[0..MW) -> sm.rows; returns count
  auto build_rows_from_mask = [&](const uint32_t* w) {
    int total = 0;
    if (tid < TR) {
      const int word = tid / 32, bit = tid % 32;
      const uint32_t mw = w[word];
      if ((mw >> bit) & 1u) {
        int before = __builtin_popcount(mw & ((1u << bit) - 1u));
        for (int k = 0; k < word; ++k) before += __builtin_popcount(w[k]);
        sm.rows[before] = (int16_t)tid;
      }
    }
#pragma unroll
    for (int k = 0; k < Sm::MW; ++k) total += __builtin_popcount(w[k]);
    return total;
  };

  const int nkb_cube = (g.S + KB - 1) / KB;   // key blocks per cube
  const uint16_t* kg = (const uint16_t*)a.k_cube + (size_t)grp * g.N * D;
  const uint16_t* vg = (const uint16_t*)a.v_cube + (size_t)grp * g.N * D;

  // ---- own cube (video rows): every row of the tile, block-causal ------------
  if (video) {
    for (int t = tid; t < n_rows; t += 256) sm.rows[t] = (int16_t)t;
    for (int kb = 0; kb < nkb_cube; ++kb) {
      const int kc = min(KB, g.S - kb * KB);
      fetch_kv(kg + ((size_t)c * g.S + kb * KB) * D, vg + ((size_t)c * g.S + kb * KB) * D, D, kc);
      store_kv();
      __syncthreads();
      compute_block(n_rows, kc, false, 0);
      __syncthreads();
    }
  }

  // ---- text keys (extra rows with causal text K/V), chunk 0 only ------------
  if (!video && a.n_text_kv > 0 && chunk == 0) {
    const uint16_t* kt = (const uint16_t*)a.k_text + (size_t)grp * D;
    const uint16_t* vt = (const uint16_t*)a.v_text + (size_t)grp * D;
    const int ntb = (a.n_text_kv + KB - 1) / KB;
    for (int tb = 0; tb < ntb; ++tb) {
      const int kc = min(KB, a.n_text_kv - tb * KB);
      fetch_kv(kt + (size_t)tb * KB * g.Hkv * D, vt + (size_t)tb * KB * g.Hkv * D,
               (size_t)g.Hkv * D, kc);
      store_kv();
      // rows whose token reaches this block
      if (tid == 0) {
        int nr = 0;
        for (int t = 0; t < n_rows; ++t)
          if (sm.row_pos[t] >= tb * KB) sm.rows[nr++] = (int16_t)t;
        sm.n_cubes = nr;  // reused as a row count
      }
      __syncthreads();
      compute_block(sm.n_cubes, kc, true, tb * KB);
      __syncthreads();
    }
  }

  // ---- selected cubes ---------------------------------------------------------
  int cube_lo, cube_hi;
  if (video) {
    cube_lo = 0;
    cube_hi = c;
  } else {
    cube_lo = chunk * sc.extra_chunk_cubes;
    cube_hi = min(g.Nc, cube_lo + sc.extra_chunk_cubes);
  }
  for (int jb = cube_lo; jb < cube_hi; jb += PASS) {
    const int je = min(cube_hi, jb + PASS);
    for (int e = tid; e < PASS * Sm::MW; e += 256) sm.mask[e] = 0u;
    __syncthreads();
    if (tid < n_rows) {
      while (my_cur < my_cnt) {
        const int j = my_list[my_cur];
        if (j >= je) break;
        atomicOr(&sm.mask[(j - jb) * Sm::MW + tid / 32], 1u << (tid % 32));
        ++my_cur;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int jj = lane;
      bool any = false;
      if (jj < je - jb) {
#pragma unroll
        for (int k = 0; k < Sm::MW; ++k) any |= sm.mask[jj * Sm::MW + k] != 0u;
      }
      const uint64_t bal = __ballot(any);
      if (any) sm.cubes[lanes_below(bal)] = jj;
      if (lane == 0) sm.n_cubes = popc64(bal);
    }
    __syncthreads();
    const int ncub = sm.n_cubes;
    const int nblocks = ncub * nkb_cube;
    if (nblocks > 0) {
      {
        const int j = jb + sm.cubes[0];
        fetch_kv(kg + (size_t)j * g.S * D, vg + (size_t)j * g.S * D, D, min(KB, g.S));
      }
      for (int it = 0; it < nblocks; ++it) {
        const int ci = it / nkb_cube, kb = it - ci * nkb_cube;
        const int jl = sm.cubes[ci];
        const int kc = min(KB, g.S - kb * KB);
        store_kv();
        const int nr = build_rows_from_mask(&sm.mask[jl * Sm::MW]);
        __syncthreads();
        if (it + 1 < nblocks) {
          const int ci2 = (it + 1) / nkb_cube, kb2 = (it + 1) - ci2 * nkb_cube;
          const int j2 = jb + sm.cubes[ci2];
          const size_t off2 = ((size_t)j2 * g.S + kb2 * KB) * D;
          fetch_kv(kg + off2, vg + off2, D, min(KB, g.S - kb2 * KB));
        }
        compute_block(nr, kc, false, 0);
        __syncthreads();
      }
    }
  }

  // ---- epilogue -------------------------------------------------------------------
  const bool partial = !video && sc.extra_chunks > 1;
  if (partial) {
    const int tile = blockIdx.x / sc.extra_chunks;
    float* dst = a.partials + ((size_t)tile * sc.extra_chunks + chunk) * TR * (D + 2);
    for (int e = tid; e < n_rows * (D + 2); e += 256) {
      const int r = e / (D + 2), cc = e % (D + 2);
      float v;
      if (cc == 0) v = sm.m[r];
      else if (cc == 1) v = sm.l[r];
      else v = sm.acc[r * Sm::AS + cc - 2];
      dst[e] = v;
    }
    return;
  }
  for (int e = tid; e < n_rows * VPR; e += 256) {
    const int r = e / VPR, v = e % VPR;
    const int hq = sm.row_hq[r], pos = sm.row_pos[r];
    const float inv = 1.0f / sm.l[r];
    const float* ar = &sm.acc[r * Sm::AS + v * 8];
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_bits(ar[2 * i] * inv) |
             ((uint32_t)f32_to_bf16_bits(ar[2 * i + 1] * inv) << 16);
    uint16_t* dst;
    if (video) {
      const int cc = pos / g.S;
      const int n = raster_of(g, cc, pos - cc * g.S);
      dst = (uint16_t*)a.out_raster + ((size_t)n * g.Hq + hq) * D;
    } else {
      dst = (uint16_t*)a.out_extra + ((size_t)pos * g.Hq + hq) * D;
    }
    *reinterpret_cast<uint4*>(dst + v * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Merge split partial results of extra rows: one wave per row.
template <int D, int TR>
__global__ __launch_bounds__(256) void k_merge_bf16(AttnArgs a, AttnSched sc, int n_tiles) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = blockIdx.x * 4 + threadIdx.x / kWave;
  const int tile = wid / TR, r = wid % TR;
  if (tile >= n_tiles) return;
  const int grp = tile / sc.extra_tiles_per_group;
  const int rho = (tile - grp * sc.extra_tiles_per_group) * TR + r;
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  if (rho >= gsz * a.n_extra) return;
  const int slot = rho / a.n_extra;
  const int hq = a.hg.heads[a.hg.start[grp] + slot];
  const int m = rho - slot * a.n_extra;
  const float* base = a.partials + (size_t)tile * sc.extra_chunks * TR * (D + 2);
  float M = -INFINITY;
  for (int q = 0; q < sc.extra_chunks; ++q) M = fmaxf(M, base[((size_t)q * TR + r) * (D + 2)]);
  constexpr int PER = D / kWave;
  float o[PER] = {};
  float L = 0.f;
  for (int q = 0; q < sc.extra_chunks; ++q) {
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
  const float* vc = (const float*)a.v_cube + (size_t)grp * g.N * D;
  float M = -INFINITY, L = 0.f, o[PER] = {};
  // key sources: own cube (video), selected cubes, then causal text
  auto run_keys = [&](const float* kbase, const float* vbase, size_t stride, int nkeys) {
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
        for (int i = 0; i < PER; ++i) o[i] = fmaf(pk, vbase[(k0 + kk) * stride + lane * PER + i], o[i]);
      }
      M = Mn;
    }
  };
  if (video) run_keys(kc + (size_t)own * g.S * D, vc + (size_t)own * g.S * D, D, g.S);
  for (int t = 0; t < cnt; ++t) {
    const int j = list[t];
    run_keys(kc + (size_t)j * g.S * D, vc + (size_t)j * g.S * D, D, g.S);
  }
  if (!video && a.n_text_kv > 0)
    run_keys((const float*)a.k_text + (size_t)grp * D, (const float*)a.v_text + (size_t)grp * D,
             (size_t)g.Hkv * D, m + 1);
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
namespace {

// The union-tile kernel (attn_union.hip) is the default bf16 path; the
// gathered-row kernel in this file is kept for comparison and selected with
// ADAS_ATTN_KERNEL=gather.
bool use_gather_kernel() {
  static const int v = [] {
    const char* e = getenv("ADAS_ATTN_KERNEL");
    return (e != nullptr && e[0] == 'g') ? 1 : 0;
  }();
  return v != 0;
}

// rows per tile of the active bf16 kernel (sets the split-partials layout)
int attn_tr(const AttnArgs&) { return use_gather_kernel() ? 128 : union_tile_rows(); }
}  // namespace

void plan_attention(AttnArgs& a, adas_dtype dt) {
  a.extra_tiles_per_group = 0;
  a.extra_chunks = 1;
  a.extra_chunk_cubes = a.g.Nc;
  if (dt != ADAS_BF16 || a.n_extra == 0) return;
  const int TR = attn_tr(a);
  a.extra_tiles_per_group = (a.hg.gmax * a.n_extra + TR - 1) / TR;
  const int extra_tiles = a.g.Hkv * a.extra_tiles_per_group;
  const long video_wgs = a.has_video
      ? (long)a.g.Nc * a.g.Hkv * ((a.hg.gmax * a.g.S + 127) / 128) : 0;
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
  const int TR = attn_tr(a);
  return (size_t)a.g.Hkv * a.extra_tiles_per_group * a.extra_chunks * TR * (a.g.D + 2) * sizeof(float);
}

template <int D, int TR>
static hipError_t launch_bf16(const AttnArgs& a, hipStream_t s) {
  AttnSched sc;
  sc.video_tiles_per_group = a.has_video ? (a.hg.gmax * a.g.S + TR - 1) / TR : 0;
  sc.extra_tiles_per_group = a.extra_tiles_per_group;
  sc.extra_chunks = a.extra_chunks;
  sc.extra_chunk_cubes = a.extra_chunk_cubes;
  sc.n_extra_wgs = a.g.Hkv * sc.extra_tiles_per_group * sc.extra_chunks;
  const long blocks = sc.n_extra_wgs + (a.has_video ? (long)a.g.Nc * a.g.Hkv * sc.video_tiles_per_group : 0);
  if (blocks > 0) hipLaunchKernelGGL((k_attn_bf16<D, TR>), dim3((unsigned)blocks), dim3(256), 0, s, a, sc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_extra > 0 && sc.extra_chunks > 1) {
    const int n_tiles = a.g.Hkv * sc.extra_tiles_per_group;
    const int waves = n_tiles * TR;
    hipLaunchKernelGGL((k_merge_bf16<D, TR>), dim3((waves + 3) / 4), dim3(256), 0, s, a, sc, n_tiles);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_attention(const AttnArgs& a, adas_dtype dt, hipStream_t s) {
  if (dt == ADAS_BF16) {
    if (use_gather_kernel())
      return a.g.D == 128 ? launch_bf16<128, 128>(a, s) : launch_bf16<64, 128>(a, s);
    hipError_t e = a.g.D == 128 ? launch_union<128>(a, s) : launch_union<64>(a, s);
    if (e != hipSuccess) return e;
    if (a.n_extra > 0 && a.extra_chunks > 1) {
      AttnSched sc;
      sc.video_tiles_per_group = 0;
      sc.extra_tiles_per_group = a.extra_tiles_per_group;
      sc.extra_chunks = a.extra_chunks;
      sc.extra_chunk_cubes = a.extra_chunk_cubes;
      sc.n_extra_wgs = a.g.Hkv * sc.extra_tiles_per_group * sc.extra_chunks;
      const int n_tiles = a.g.Hkv * sc.extra_tiles_per_group;
      constexpr int TRU = 256;  // union_tile_rows()
      const int waves = n_tiles * TRU;
      if (a.g.D == 128)
        hipLaunchKernelGGL((k_merge_bf16<128, TRU>), dim3((waves + 3) / 4), dim3(256), 0, s, a, sc, n_tiles);
      else
        hipLaunchKernelGGL((k_merge_bf16<64, TRU>), dim3((waves + 3) / 4), dim3(256), 0, s, a, sc, n_tiles);
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
