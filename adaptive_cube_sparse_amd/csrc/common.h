// Shared device helpers and launch descriptors for the AdaS-Attn kernels
// (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adas.h"

namespace adas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Geometry as the kernels see it (all derived on the host).
struct KGeom {
  int T, H, W;
  int ct, ch, cw;
  int nT, nH, nW;
  int N;     // tokens
  int S;     // tokens per cube
  int Nc;    // cubes
  int Hq, Hkv, D;
  int NS;    // tokens per head in cube-layout buffers (capacity; N unless a cache is larger)
};

// Query heads grouped by the KV head they read.  Heads of group g are
// heads[start[g] .. start[g+1]).
struct HeadGroups {
  int16_t start[ADAS_MAX_HEADS + 1];
  uint8_t heads[ADAS_MAX_HEADS];
  int gmax;  // largest group
};

// ---------------------------------------------------------------------------
// cube geometry
// ---------------------------------------------------------------------------
// Raster token index of cube-layout position (c, r).
__device__ __forceinline__ int raster_of(const KGeom& g, int c, int r) {
  const int bx = c % g.nW;
  const int t1 = c / g.nW;
  const int by = t1 % g.nH;
  const int bt = t1 / g.nH;
  const int dx = r % g.cw;
  const int t2 = r / g.cw;
  const int dy = t2 % g.ch;
  const int dt = t2 / g.ch;
  const int f = bt * g.ct + dt, y = by * g.ch + dy, x = bx * g.cw + dx;
  return (f * g.H + y) * g.W + x;
}

// Offset of a video row's list in sel_idx (closed form, see adas.h).
__device__ __forceinline__ int64_t video_list_offset(int64_t capv, int hq, int S, int c, int r) {
  return (int64_t)hq * capv + (int64_t)S * c * (c - 1) / 2 + (int64_t)r * c;
}
__device__ __forceinline__ int64_t extra_list_offset(int64_t capv, int Hq, int n_extra, int Nc, int hq,
                                                     int m) {
  return (int64_t)Hq * capv + ((int64_t)hq * n_extra + m) * Nc;
}

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
// round to nearest even (inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ __bf16 f32_to_bf16(float f) {
  return __builtin_bit_cast(__bf16, f32_to_bf16_bits(f));
}

// ---------------------------------------------------------------------------
// wave64 reductions on DPP (no LDS traffic).  quad_perm, row_half_mirror and
// row_mirror fold each 16-lane row; row_bcast15 / row_bcast31 carry rows 0-2
// into row 3; lane 63 then holds the total, and readlane makes the result one
// wave-uniform scalar, so decisions taken on it are uniform.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float t) {
  t += dpp_f32<0xb1>(t, 0.f);        // quad_perm [1,0,3,2]
  t += dpp_f32<0x4e>(t, 0.f);        // quad_perm [2,3,0,1]
  t += dpp_f32<0x141>(t, 0.f);       // row_half_mirror
  t += dpp_f32<0x140>(t, 0.f);       // row_mirror
  t += dpp_f32<0x142, 0xa>(t, 0.f);  // row_bcast15 -> rows 1, 3
  t += dpp_f32<0x143, 0xc>(t, 0.f);  // row_bcast31 -> rows 2, 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), 63));
}
__device__ __forceinline__ float wave_max(float t) {
  t = fmaxf(t, dpp_f32<0xb1>(t, -INFINITY));
  t = fmaxf(t, dpp_f32<0x4e>(t, -INFINITY));
  t = fmaxf(t, dpp_f32<0x141>(t, -INFINITY));
  t = fmaxf(t, dpp_f32<0x140>(t, -INFINITY));
  t = fmaxf(t, dpp_f32<0x142, 0xa>(t, -INFINITY));
  t = fmaxf(t, dpp_f32<0x143, 0xc>(t, -INFINITY));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), 63));
}
// value of lane (lane ^ 32), via v_permlane32_swap
__device__ __forceinline__ float xor32_f32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? (unsigned)r[0] : (unsigned)r[1]);
}
__device__ __forceinline__ int popc64(uint64_t m) { return __builtin_popcountll(m); }
// number of set bits of m in lanes below this one
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// s_waitcnt immediate that waits until at most n vector memory operations are
// outstanding (n < 64; exp and lgkm counters not waited on)
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// 16 bytes per lane from base + voff + soff (a buffer of `bytes` bytes; reads
// past it return 0) into LDS at lds + 16 * lane (lds wave-uniform).  A buffer
// load (MUBUF) rather than global_load_lds: the compiler counts a pending FLAT
// load into LDS as an LDS access too and then answers every LDS operand read
// with lgkmcnt(0); a buffer load is counted on vmcnt only.  Kept out of
// lambdas: inside one, the builtin fails the host pass silently and the
// enclosing kernel loses its host stub.
__device__ __forceinline__ void buffer_load_lds16(void* base, int bytes, void* lds, uint32_t voff, uint32_t soff) {
  typedef __attribute__((address_space(3))) void lds_t;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ float fast_exp(float x) {
  // exp(x) = 2^(x*log2 e); v_exp_f32 is accurate to ~1 ulp on normal results.
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// ---------------------------------------------------------------------------
// Top-p on one row held by one wave (key design 2, the S_i equation).
//
// E[i] (lane L) is exp(z_j - max z) for candidate j = L + 64*i, or -1 for
// j >= n (padding), with n <= 64*NPL.  Z is the wave-uniform sum of the valid
// E.  Finds the Top-p set under the order (E descending, j ascending), writes
// its ids ascending to out[0..count) and returns count (wave-uniform).
// `scratch` is 64 floats of LDS private to the wave.
//
// Method: the selected set is {E > tau} plus the lowest-index ties at tau,
// where tau is the largest float with mass(E >= tau) >= p*Z.  tau is found by
// bisection on the float bit pattern (positive floats order like their bits):
//   1. on all candidates until at most 64 lie between the bounds [lo, hi);
//   2. those are gathered one per lane, the mass at or above hi is fixed, and
//      the bisection continues on single registers until one element (or one
//      bit pattern) is left.
// The loops are fully unrolled and branch-free over NPL, so NPL should be the
// smallest capacity that holds n.
// ---------------------------------------------------------------------------
template <int NPL>
__device__ int topp_select_row(const float (&E)[NPL], int n, float Z, float p,
                               int32_t* __restrict__ out, float* __restrict__ scratch) {
  const int lane = threadIdx.x & (kWave - 1);
  if (n <= 0) return 0;
  if (p >= 1.0f) {
    for (int j = lane; j < n; j += kWave) out[j] = j;
    return n;
  }
  const float target = p * Z;
  // mass(E >= lo) >= target > mass(E >= hi).  Initial lo: the n candidates
  // below x0 = (1 - p) Z / (2n) hold less than (1 - p) Z / 2, so mass(E >= x0)
  // > target; starting there skips the steps that only pass over tiny E.
  uint32_t lo = __float_as_uint(0.5f * (1.0f - p) * Z / (float)n), hi = 0x3F800001u;
  int cnt_lo = 0, cnt_hi = 0;
  {
    const float f0 = __uint_as_float(lo);
#pragma unroll
    for (int i = 0; i < NPL; ++i) cnt_lo += popc64(__ballot(E[i] >= f0));
  }
  float tau = 0.0f;
  bool found = false;
  // 1. full bisection
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
    ms = wave_sum(ms);
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
    float mhi = 0.0f;
    int base = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      mhi += E[i] >= fhi ? E[i] : 0.0f;
      const bool in = E[i] >= flo && E[i] < fhi;
      const uint64_t b = __ballot(in);
      if (in) scratch[base + lanes_below(b)] = E[i];
      base += popc64(b);
    }
    mhi = wave_sum(mhi);
    __builtin_amdgcn_wave_barrier();
    const float v = lane < base ? scratch[lane] : -1.0f;
    // 3. bisection on one value per lane; every gathered v is below the
    //    gather-time bound, whose mass (mhi) and count (cnt_hi0) stay fixed
    const int cnt_hi0 = cnt_hi;
    for (;;) {
      if (cnt_lo - cnt_hi == 1) {  // exactly one element in [lo, hi): the cut
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
  }
  // ties at tau; with at most one (the usual case) the set is {E >= tau}.
  // Otherwise the mass strictly above tau fixes how many of them to take.
  int ceq = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) ceq += popc64(__ballot(E[i] == tau));
  int keq = ceq;
  if (ceq > 1) {
    float mgt = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) mgt += E[i] > tau ? E[i] : 0.0f;
    mgt = wave_sum(mgt);
    const float need = (target - mgt) / tau;
    int k = (int)ceilf(need);
    if (k < 1) k = 1;
    if (k < keq) keq = k;
  }
  // ascending compaction: stripe i holds candidates 64*i .. 64*i+63
  int base = 0;
  if (keq == ceq) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const bool sel = E[i] >= tau;
      const uint64_t bs = __ballot(sel);
      if (sel) out[base + lanes_below(bs)] = lane + kWave * i;
      base += popc64(bs);
    }
    return base;
  }
  int eq_seen = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool eq = E[i] == tau;
    const uint64_t beq = __ballot(eq);
    const int eq_rank = eq_seen + lanes_below(beq);
    const bool sel = (E[i] > tau) || (eq && eq_rank < keq);
    const uint64_t bs = __ballot(sel);
    if (sel) out[base + lanes_below(bs)] = lane + kWave * i;
    base += popc64(bs);
    eq_seen += popc64(beq);
  }
  return base;
}

// ---------------------------------------------------------------------------
// Top-K on one row held by one wave (the fixed-budget strategy the AdaSpark
// listing compares with Top-p, Table 4): the k candidates of largest logit
// (P is monotone in the logit), equal logits lower index first.
//
// z[i] (lane L) is the logit of candidate j = L + 64*i, valid for j < n.
// Logits map to unsigned keys that order like the floats; the k-th largest
// key t is built bit by bit from the top (largest t with count(key >= t) >= k),
// then the keys above t and the lowest-index ties at t are compacted in
// ascending order.  Writes the ids to out[0..) and returns their count.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int NPL>
__device__ int topk_select_row(const float (&z)[NPL], int n, int k, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  if (n <= 0) return 0;
  if (k >= n) {
    for (int j = lane; j < n; j += kWave) out[j] = j;
    return n;
  }
  uint32_t u[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) u[i] = lane + kWave * i < n ? ordered_key(z[i]) : 0u;  // 0: padding
  uint32_t t = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) cnt += popc64(__ballot(u[i] >= cand));
    if (cnt >= k) t = cand;
  }
  int cgt = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) cgt += popc64(__ballot(u[i] > t));
  const int keq = k - cgt;  // ties at t to take, lowest index first
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool eq = u[i] == t;
    const uint64_t beq = __ballot(eq);
    const bool sel = u[i] > t || (eq && eq_seen + lanes_below(beq) < keq);
    const uint64_t bs = __ballot(sel);
    if (sel) out[base + lanes_below(bs)] = lane + kWave * i;
    base += popc64(bs);
    eq_seen += popc64(beq);
  }
  return base;
}

// Column of cube offset r in a value row of ADAS_LAYOUT_VT: bits 2 and 3 of r
// swapped inside every complete aligned group of 16 offsets, identity in a
// trailing partial group.  An involution.
__host__ __device__ inline int vt_column(int r, int S) {
  return r < (S & ~15) ? ((r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1)) : r;
}

// ---------------------------------------------------------------------------
// host-side launch entry points (defined in the .hip files)
// ---------------------------------------------------------------------------
hipError_t launch_partition(const KGeom& g, int elem_bytes, int nh, bool vt, const void* src,
                            void* dst, int32_t* perm, hipStream_t s);
hipError_t launch_mean_keys(const KGeom& g, adas_dtype dt, const void* k, float* kbar,
                            hipStream_t s);
hipError_t launch_partition_keys(const KGeom& g, adas_dtype dt, const void* src, void* dst, int32_t* perm,
                                 float* kbar, hipStream_t s);
hipError_t launch_cache_append(const KGeom& g, int f_lo, int f_hi, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, float* kbar, double* ksum, hipStream_t s);

struct SelectArgs {
  KGeom g;
  HeadGroups hg;
  const void* q_cube;   // may be null
  const void* q_extra;  // may be null
  const float* kbar;
  float* zbuf;  // workspace: extra-row logits [Hq*n_extra][Nc] (split selection)
  int n_extra;
  float p;
  int topk;  // > 0: Top-K selection of topk cubes instead of Top-p
  int32_t* sel_count;
  int32_t* sel_idx;
  int64_t capv;  // per-head video capacity (0 without video rows)
  int rows_per_head;  // Nv + n_extra
  int has_video;
  // optional (split path, Top-p): also write each extra row's selection as a
  // bitmap [Hq*n_extra][bits_words], bit j%32 of word j/32 for cube j
  uint32_t* extra_bits;
  int bits_words;
};
hipError_t launch_select(const SelectArgs& a, adas_dtype dt, hipStream_t s);
size_t select_workspace_bytes(const KGeom& g, adas_dtype dt, int n_extra, int gmax);
bool use_split_select(const KGeom& g, int n_extra, int gmax);

struct AttnArgs {
  KGeom g;
  HeadGroups hg;
  const void* q_cube;
  const void* k_cube;
  const void* v_cube;
  const void* q_extra;
  const void* k_text;
  const void* v_text;
  const int32_t* sel_count;
  const int32_t* sel_idx;
  void* out_raster;
  void* out_extra;
  float* partials;       // workspace: split extra-row partials (when chunked)
  float* lse;            // optional [Hq][rows_per_head]: natural log-sum-exp of each row's scaled scores
  uint32_t* extra_bits;  // workspace: selection bitmap of extra rows [Hq*n_extra][bits_words]
  int bits_words;        // ceil(Nc / 32)
  int bits_ready;        // the selection already wrote extra_bits (no bitmap launch)
  int n_extra;
  int n_text_kv;
  int64_t capv;
  int rows_per_head;
  int has_video;
  // schedule (filled by plan_attention)
  int extra_tiles_per_group;
  int extra_chunks;       // partial rows per tile row (chunks, times waves in decode mode)
  int extra_chunk_cubes;
  int decode_chunks;      // > 0: extra rows run in k_attn_decode with this many chunks per KV head
};
void plan_attention(AttnArgs& a, adas_dtype dt);
size_t attention_workspace_bytes(const AttnArgs& a, adas_dtype dt);
void bind_attention_workspace(AttnArgs& a, adas_dtype dt, void* ws);
hipError_t launch_attention(const AttnArgs& a, adas_dtype dt, hipStream_t s);
template <int D>
hipError_t launch_union(const AttnArgs& a, hipStream_t s);
int union_tile_rows();  // rows per tile of the union kernel
hipError_t launch_decode(const AttnArgs& a, hipStream_t s);
int decode_waves();     // waves per workgroup of the decode kernel
int decode_max_chunk_cubes();  // most cubes in one chunk of the decode kernel

// peak probes (probe.hip)
double probe_mfma_flops_per_wg(int iters);
hipError_t launch_probe_mfma(int wgs, int iters, float* sink, hipStream_t s);
hipError_t launch_probe_read(const void* src, long bytes, uint32_t* sink, int wgs, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, long bytes, int wgs, hipStream_t s);
double probe_attn_mix_flops_per_wg(int iters);
hipError_t launch_probe_attn_mix(int wgs, int iters, bool mix, const void* src, int src_bytes, float* sink,
                                 hipStream_t s);

}  // namespace adas
