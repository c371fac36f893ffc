// AdaS-FFN on gfx950 (AdaSpark, papernotes.org, key design 3; key design 4
// for the shared Top-p rule):
//   k_ffn_select   per cube: float64 L2 norm of every token, its share of the
//                  cube's summed norm, Top-p over the shares -> count + bitmask
//   k_ffn_emit     per cube: exclusive prefix of the counts (act_off) and the
//                  compact list of active raster tokens (act_rows)
//   k_ffn_gemm<1>  H = silu(X W_gate^T) * (X W_up^T) over the gathered active
//                  and text rows, bf16 MFMA, float32 accumulation, bf16 H
//   k_ffn_gemm<0>  F = H W_down^T, float32
//   k_ffn_combine  per cube: m_c = mean of F over its active rows; y = x + F
//                  for active tokens, x + m_c for skipped ones; text y = x + F
#include "common.h"
#include "ffn.h"

namespace adas {

typedef __bf16 gbf16x8 __attribute__((ext_vector_type(8)));
typedef float gf32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// selection: one workgroup (1024 threads, one wave per token at a time) per cube
// ---------------------------------------------------------------------------
constexpr int FSEL_T = 1024;
__global__ __launch_bounds__(FSEL_T) void k_ffn_select(KGeom g, int hidden, const uint16_t* __restrict__ x,
                                                    double p, int32_t* __restrict__ act_count,
                                                    uint32_t* __restrict__ act_mask, int mw) {
  __shared__ double s_norm[ADAS_FFN_MAX_S];
  __shared__ double s_sorted[ADAS_FFN_MAX_S];
  __shared__ int s_rank[ADAS_FFN_MAX_S];
  __shared__ double s_total;
  __shared__ int s_k;
  const int c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = g.S;
  const int nvec = hidden >> 3;  // 16-byte pieces per row

  // squared L2 norm of token r: bf16 values widened to float64, whose
  // products are exact; one wave per token, float64 butterfly at the end
  for (int r = wave; r < S; r += FSEL_T / 64) {
    const uint4* row = reinterpret_cast<const uint4*>(x + (size_t)raster_of(g, c, r) * hidden);
    double acc = 0.0;
    for (int v = lane; v < nvec; v += 64) {
      const uint4 q = row[v];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double lo = (double)__uint_as_float(w[e] << 16);
        const double hi = (double)__uint_as_float(w[e] & 0xFFFF0000u);
        acc = fma(lo, lo, acc);
        acc = fma(hi, hi, acc);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) s_norm[r] = sqrt(acc);
  }
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;  // summed in offset order
    for (int j = 0; j < S; ++j) t += s_norm[j];
    s_total = t;
  }
  __syncthreads();
  const double total = s_total;
  // share of token tid and its rank under (share descending, offset ascending)
  double P = 0.0;
  int rank = 0;
  if (tid < S) {
    P = total > 0.0 ? s_norm[tid] / total : 1.0 / S;
    for (int j = 0; j < S; ++j) {
      const double Pj = total > 0.0 ? s_norm[j] / total : 1.0 / S;
      rank += (Pj > P) || (Pj == P && j < tid);
    }
    s_sorted[rank] = P;
    s_rank[tid] = rank;
  }
  __syncthreads();
  if (tid == 0) {
    int k = S;  // a float sum that never reaches p keeps every token
    if (p < 1.0) {
      double run = 0.0;
      for (int m = 0; m < S; ++m) {
        run += s_sorted[m];
        if (run >= p) {
          k = m + 1;
          break;
        }
      }
    }
    s_k = k;
    act_count[c] = k;
  }
  __syncthreads();
  const bool active = tid < S && s_rank[tid] < s_k;
  const uint64_t bits = __ballot(active);
  if (lane == 0) {
    if (2 * wave < mw) act_mask[(size_t)c * mw + 2 * wave] = (uint32_t)bits;
    if (2 * wave + 1 < mw) act_mask[(size_t)c * mw + 2 * wave + 1] = (uint32_t)(bits >> 32);
  }
}

// ---------------------------------------------------------------------------
// offsets and compact rows: one workgroup per cube
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ffn_emit(KGeom g, const int32_t* __restrict__ act_count,
                                                  const uint32_t* __restrict__ act_mask, int mw,
                                                  int32_t* __restrict__ act_off, int32_t* __restrict__ act_rows) {
  __shared__ int s_part[4];
  const int c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int sum = 0;
  for (int j = tid; j < c; j += 256) sum += act_count[j];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) s_part[wave] = sum;
  __syncthreads();
  const int base = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  if (tid == 0) {
    act_off[c] = base;
    if (c == g.Nc - 1) act_off[g.Nc] = base + act_count[c];
  }
  const int r = tid;
  if (r < g.S) {
    const uint32_t* m = act_mask + (size_t)c * mw;
    const uint32_t w = m[r >> 5];
    if ((w >> (r & 31)) & 1u) {
      int slot = __builtin_popcount(w & ((1u << (r & 31)) - 1u));
      for (int i = 0; i < (r >> 5); ++i) slot += __builtin_popcount(m[i]);
      act_rows[base + slot] = raster_of(g, c, r);
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM: C[M][n] = A[M][K] . B[n][K]^T on v_mfma_f32_32x32x16_bf16.
// Workgroup tile 256 x 256 (gate/up: 128 gate + 128 up columns of the same
// output features), 8 waves in a 4 x 2 grid, 64 x 128 per wave (2 x 4 MFMA
// tiles).  K moves in stages of 64 through two LDS buffers per operand; each
// stage is 64 direct global -> LDS loads of 1 KB (8 rows of 128 bytes), 8 per
// wave.  Inside a 128-byte LDS row the 16-byte piece of k-chunk ch sits at
// slot ch ^ ((row >> 1) & 7), so a 16-lane group of MFMA fragment reads (16
// rows, one chunk) touches 16 distinct 16-byte bank groups.
// ---------------------------------------------------------------------------
constexpr int GBM = 256, GBN = 256, GBK = 64, GNT = 512, GROW = GBK * 2;

template <bool GU>
__global__ __launch_bounds__(GNT) void k_ffn_gemm(FfnGemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[GBM * GROW];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[GBM * GROW];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[GBN * GROW];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[GBN * GROW];
  typedef __attribute__((address_space(3))) void lds_void;

  // rows: active video tokens (act_off[Nc] of them) then the text tokens
  const int Mv = a.act_off[a.Nc];
  const int M = Mv + a.n_text;
  const int mtiles = (M + GBM - 1) / GBM;
  const int T = mtiles * a.n_tiles;
  // XCD-aware order: workgroup b runs on XCD b % 8; XCD x takes the x-th
  // contiguous share of the tiles, ordered in groups of 8 row tiles with the
  // column tiles inside a group, so the ~32 tiles an XCD holds at once share
  // 8 A and 4 B panels in its L2.
  const int per = (T + 7) >> 3;
  const int kk = blockIdx.x >> 3;
  if (kk >= per) return;
  const int t = (blockIdx.x & 7) * per + kk;
  if (t >= T) return;
  const int gsz = 8 * a.n_tiles;
  const int grp = t / gsz, first = grp * 8, gm = min(mtiles - first, 8), rem = t - grp * gsz;
  const int mt = first + rem % gm, nt = rem / gm;
  const int m0 = mt * GBM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // loader: wave wv moves rows 32*wv .. 32*wv+31 of both operands
  const char* ap[4];
  const char* bp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 32 * wv + 8 * q + (lane >> 3);
    const int ch = (lane & 7) ^ ((r >> 1) & 7);  // k-chunk this lane's slot holds
    const int m = m0 + r;
    const uint16_t* arow;
    if (GU)
      arow = m < Mv ? a.a + (size_t)a.rows[m] * a.K
                    : (m < M ? a.a_text + (size_t)(m - Mv) * a.K : a.a);  // past M: any valid row
    else
      arow = a.a + (size_t)m * a.K;  // H holds a multiple of 256 rows
    ap[q] = reinterpret_cast<const char*>(arow) + ch * 16;
    const uint16_t* brow;
    if (GU)
      brow = r < 128 ? a.b0 + (size_t)(nt * 128 + r) * a.K : a.b1 + (size_t)(nt * 128 + r - 128) * a.K;
    else
      brow = a.b0 + (size_t)(nt * GBN + r) * a.K;
    bp[q] = reinterpret_cast<const char*>(brow) + ch * 16;
  }
  auto issue = [&](int k0, auto bufc) __attribute__((always_inline)) {
    uint8_t* sa = decltype(bufc)::value ? sA1 : sA0;
    uint8_t* sb = decltype(bufc)::value ? sB1 : sB0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(ap[q] + 2 * k0),
                                       (lds_void*)(sa + (32 * wv + 8 * q) * GROW), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(bp[q] + 2 * k0),
                                       (lds_void*)(sb + (32 * wv + 8 * q) * GROW), 16, 0, 0);
  };

  // compute: wave (wm, wn) owns rows 64*wm .. +63 and four 32-row B panels
  const int wm = wave & 3, wn = wave >> 2;
  const int l32 = lane & 31, hi = lane >> 5;
  const int swz = (lane >> 1) & 7;  // ((row >> 1) & 7) of every row this lane reads
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = ((2 * ks + hi) ^ swz) << 4;
  const int aoff = (64 * wm + l32) * GROW;
  int boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int br = GU ? (j < 2 ? 64 * wn + 32 * j : 128 + 64 * wn + 32 * (j - 2)) : 128 * wn + 32 * j;
    boff[j] = (br + l32) * GROW;
  }
  gf32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // Fragments of k-step ks+1 are read while the MFMAs of k-step ks run: the
  // scheduling group barriers interleave one fragment read after each of the
  // first six MFMAs, so the reads are under way long before their data is
  // needed and the only wait on LDS is at the first k-step of a stage.
  auto compute = [&](auto bufc, auto nextc, int k_next) __attribute__((always_inline)) {
    const uint8_t* sa = decltype(bufc)::value ? sA1 : sA0;
    const uint8_t* sb = decltype(bufc)::value ? sB1 : sB0;
    gbf16x8 av[2][2], bv[2][4];
    auto load = [&](int ks, int set) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[set][i] = __builtin_bit_cast(gbf16x8, *reinterpret_cast<const uint4*>(sa + aoff + i * 32 * GROW + koff[ks]));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bv[set][j] = __builtin_bit_cast(gbf16x8, *reinterpret_cast<const uint4*>(sb + boff[j] + koff[ks]));
    };
    load(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) load(ks + 1, (ks + 1) & 1);
      if (ks == 0) issue(k_next, nextc);  // the next stage's loads go out under the first MFMAs
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks & 1][i], bv[ks & 1][j], acc[i][j], 0, 0, 0);
      if (ks == 0) {
#pragma unroll
        for (int r = 0; r < 6; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global -> LDS load
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      } else if (ks + 1 < 4) {
#pragma unroll
        for (int r = 0; r < 6; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  // Stage s lives in buffer s % 2; the barrier before stage s also tells every
  // wave that stage s-1 (the other buffer) is no longer read, so stage s+1
  // may land there; its loads are issued inside the first k-step of stage s.
  // Past the last stage the loads repeat it (in bounds, never read), so every
  // step has the same shape.  The host guarantees an even number of stages.
  const int nst = a.K / GBK;
  issue(0, C0{});
  for (int s = 0; s < nst; s += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of stage s
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    compute(C0{}, C1{}, (s + 1) * GBK);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    compute(C1{}, C0{}, min(s + 2, nst - 1) * GBK);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the repeated loads land before LDS is reused

  // accumulator element e of lane l: row 8*(e/4) + 4*(l/32) + e%4, column l%32
  if constexpr (GU) {
    // h = silu(gate) * up, bf16, through LDS (rows 0..127 in sA0, 128..255 in
    // sA1, 256 bytes each) so that the stores are whole 16-byte pieces
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * hi + (e & 3);
          const int col = 64 * wn + 32 * j + l32;
          const float gv = acc[i][j][e], uv = acc[i][j + 2][e];
          const float h = gv / (1.0f + __expf(-gv)) * uv;
          uint8_t* dst = (row < 128 ? sA0 + row * 256 : sA1 + (row - 128) * 256) + 2 * col;
          *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16_bits(h);
        }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    uint16_t* H = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = it * GNT + tid;
      const int row = idx >> 4, ch = idx & 15;
      if (m0 + row < M) {
        const uint4 v = *reinterpret_cast<const uint4*>((row < 128 ? sA0 + row * 256 : sA1 + (row - 128) * 256) +
                                                        16 * ch);
        *reinterpret_cast<uint4*>(H + (size_t)(m0 + row) * a.ldo + nt * 128 + 8 * ch) = v;
      }
    }
  } else {
    float* F = static_cast<float*>(a.out);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (row < M) {
#pragma unroll
          for (int j = 0; j < 4; ++j) F[(size_t)row * a.ldo + nt * GBN + 128 * wn + 32 * j + l32] = acc[i][j][e];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// mean compensation and residual.  Block (b, chunk) covers 1024 columns
// (256 threads x 4) of cube b, or of 16 text rows when b >= Nc; columns go 4
// at a time (float4 of F, 8 bytes of bf16 x and y).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ffn_combine(KGeom g, int hidden, const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ x_text, int n_text,
                                                     const float* __restrict__ F,
                                                     const int32_t* __restrict__ act_off,
                                                     const uint32_t* __restrict__ act_mask, int mw,
                                                     uint16_t* __restrict__ y, uint16_t* __restrict__ y_text) {
  const int nv = hidden >> 2;
  const int v = blockIdx.y * 256 + threadIdx.x;
  if (v >= nv) return;
  const float4* F4 = reinterpret_cast<const float4*>(F);
  auto add_store = [&](const uint16_t* xs, uint16_t* ys, float4 f) __attribute__((always_inline)) {
    const uint2 xv = *reinterpret_cast<const uint2*>(xs);
    const float x0 = __uint_as_float(xv.x << 16), x1 = __uint_as_float(xv.x & 0xFFFF0000u);
    const float x2 = __uint_as_float(xv.y << 16), x3 = __uint_as_float(xv.y & 0xFFFF0000u);
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_bits(x0 + f.x) | ((uint32_t)f32_to_bf16_bits(x1 + f.y) << 16);
    o.y = (uint32_t)f32_to_bf16_bits(x2 + f.z) | ((uint32_t)f32_to_bf16_bits(x3 + f.w) << 16);
    *reinterpret_cast<uint2*>(ys) = o;
  };
  const int b = blockIdx.x;
  if (b < g.Nc) {
    const int c = b;
    const int beg = act_off[c], cnt = act_off[c + 1] - beg;
    const uint32_t* mk = act_mask + (size_t)c * mw;
    // mean over the active rows, four partial sums for independent loads
    float4 p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    int j = 0;
    for (; j + 4 <= cnt; j += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 f = F4[(size_t)(beg + j + u) * nv + v];
        p[u].x += f.x; p[u].y += f.y; p[u].z += f.z; p[u].w += f.w;
      }
    }
    for (; j < cnt; ++j) {
      const float4 f = F4[(size_t)(beg + j) * nv + v];
      p[0].x += f.x; p[0].y += f.y; p[0].z += f.z; p[0].w += f.w;
    }
    const float inv = 1.0f / (float)cnt;
    const float4 m = make_float4(((p[0].x + p[1].x) + (p[2].x + p[3].x)) * inv,
                                 ((p[0].y + p[1].y) + (p[2].y + p[3].y)) * inv,
                                 ((p[0].z + p[1].z) + (p[2].z + p[3].z)) * inv,
                                 ((p[0].w + p[1].w) + (p[2].w + p[3].w)) * inv);
    int slot = 0;
    for (int r0 = 0; r0 < g.S; r0 += 32) {
      const uint32_t w = mk[r0 >> 5];
#pragma unroll 4
      for (int r = r0; r < min(r0 + 32, g.S); ++r) {
        const bool act = (w >> (r & 31)) & 1u;
        const size_t n = (size_t)raster_of(g, c, r);
        const float4 f = act ? F4[(size_t)(beg + slot) * nv + v] : m;
        slot += act;
        add_store(x + n * hidden + 4 * v, y + n * hidden + 4 * v, f);
      }
    }
  } else {
    const int Mv = act_off[g.Nc];
    const int t0 = (b - g.Nc) * 16;
    for (int t = t0; t < min(t0 + 16, n_text); ++t)
      add_store(x_text + (size_t)t * hidden + 4 * v, y_text + (size_t)t * hidden + 4 * v,
                F4[(size_t)(Mv + t) * nv + v]);
  }
}

// ---------------------------------------------------------------------------
// host launches
// ---------------------------------------------------------------------------
int ffn_mask_words(int S) { return (S + 31) / 32; }

size_t ffn_rows_cap(const KGeom& g, int n_text) {
  return ((size_t)g.N + n_text + GBM - 1) / GBM * GBM;
}

size_t ffn_workspace_bytes(const KGeom& g, int hidden, int inter, int n_text) {
  const size_t rows = ffn_rows_cap(g, n_text);
  return rows * inter * 2 + rows * hidden * 4 + 256;
}

hipError_t launch_ffn_select(const KGeom& g, int hidden, const void* x, double p, int32_t* act_count,
                             int32_t* act_off, int32_t* act_rows, uint32_t* act_mask, hipStream_t s) {
  const int mw = ffn_mask_words(g.S);
  hipLaunchKernelGGL(k_ffn_select, dim3(g.Nc), dim3(FSEL_T), 0, s, g, hidden,
                     static_cast<const uint16_t*>(x), p, act_count, act_mask, mw);
  hipLaunchKernelGGL(k_ffn_emit, dim3(g.Nc), dim3(256), 0, s, g, (const int32_t*)act_count,
                     (const uint32_t*)act_mask, mw, act_off, act_rows);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnArgs& f, hipStream_t s) {
  const KGeom& g = f.g;
  const size_t rows = ffn_rows_cap(g, f.n_text);
  uint16_t* H = static_cast<uint16_t*>(f.ws);
  float* F = reinterpret_cast<float*>(static_cast<char*>(f.ws) + rows * f.inter * 2);
  const int mt_cap = (int)(rows / GBM);

  FfnGemmArgs gu{};
  gu.a = static_cast<const uint16_t*>(f.x);
  gu.a_text = static_cast<const uint16_t*>(f.x_text);
  gu.rows = f.act_rows;
  gu.act_off = f.act_off;
  gu.Nc = g.Nc;
  gu.n_text = f.n_text;
  gu.K = f.hidden;
  gu.b0 = static_cast<const uint16_t*>(f.w_gate);
  gu.b1 = static_cast<const uint16_t*>(f.w_up);
  gu.n_tiles = f.inter / 128;
  gu.out = H;
  gu.ldo = f.inter;
  const int grid_gu = (mt_cap * gu.n_tiles + 7) / 8 * 8;
  hipLaunchKernelGGL(k_ffn_gemm<true>, dim3(grid_gu), dim3(GNT), 0, s, gu);

  FfnGemmArgs dn = gu;
  dn.a = H;
  dn.a_text = nullptr;
  dn.rows = nullptr;
  dn.K = f.inter;
  dn.b0 = static_cast<const uint16_t*>(f.w_down);
  dn.b1 = nullptr;
  dn.n_tiles = f.hidden / GBN;
  dn.out = F;
  dn.ldo = f.hidden;
  const int grid_dn = (mt_cap * dn.n_tiles + 7) / 8 * 8;
  hipLaunchKernelGGL(k_ffn_gemm<false>, dim3(grid_dn), dim3(GNT), 0, s, dn);

  const int mw = ffn_mask_words(g.S);
  hipLaunchKernelGGL(k_ffn_combine, dim3(g.Nc + (f.n_text + 15) / 16, (f.hidden / 4 + 255) / 256), dim3(256), 0, s,
                     g, f.hidden,
                     static_cast<const uint16_t*>(f.x), static_cast<const uint16_t*>(f.x_text), f.n_text,
                     (const float*)F, f.act_off, f.act_mask, mw, static_cast<uint16_t*>(f.y),
                     static_cast<uint16_t*>(f.y_text));
  return hipGetLastError();
}

}  // namespace adas
