// Gradients of the sparse attention (AdaSpark, papernotes.org, key design 2
// attention; the training strategy adapts the model to the sparse pattern by
// fine-tuning).  The Top-p sets are discrete and held fixed, so gradients
// flow into Q, K and V only.  For a row with attended set A, scale
// c = 1/sqrt(d) and the forward's log-sum-exp L:
//   p_j = exp(c q.k_j - L),  dp_j = do.v_j,  D = do.o,  ds_j = p_j (dp_j - D)
//   dq = c sum_j ds_j k_j,   dk_j += c ds_j q,   dv_j += p_j do
// Four launches:
//   k_bwd_prep   D per row, and each row's selection as a bitmap stored
//                word-major ([hq][word][row]) so that consecutive rows of one
//                word are contiguous;
//   k_bwd_dq     query-major union tiles (the forward's structure): per key
//                block S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T
//                on v_mfma_f32_32x32x16_bf16, dQ kept in registers;
//   k_bwd_lists  per (KV head, cube): the rows that attend it (own-cube rows,
//                later video rows and extra rows whose bit is set), compacted
//                in row order;
//   k_bwd_dkdv   key-major: per (KV head, key block) four waves share K and V
//                in LDS and each walks its own 32-row tiles of the block's row
//                list, with dK^T and dV^T (128 x 64 each) in AGPRs; the waves'
//                partial sums are added through LDS at the end.
// With causal text keys (a text prefill: text row m also attends text tokens
// 0..m), two more: k_bwd_text_dq adds the text keys' share to dq of the text
// rows, k_bwd_text_dkdv forms the text keys' dK and dV (float32 on the vector
// ALUs: the text part is a few hundred rows against as many keys).
#include <type_traits>

#include "attn_bwd.h"

namespace adas {

namespace {
typedef __bf16 bbf16x8 __attribute__((ext_vector_type(8)));
typedef float bf32x16 __attribute__((ext_vector_type(16)));
constexpr float kBLog2e = 1.4426950408889634f;
constexpr int BKB = 64;            // keys per block
constexpr int BNW = 8;             // waves per dQ workgroup
constexpr int BNT = 64 * BNW;
constexpr int BTR = 32 * BNW;      // rows per dQ tile
constexpr int BPASS = 512;         // cubes per bitmap pass
__device__ __forceinline__ float bex2(float x) { return __builtin_amdgcn_exp2f(x); }
}  // namespace

// ---------------------------------------------------------------------------
// prep: 16 threads per row
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_bwd_prep(BwdArgs a) {
  const KGeom& g = a.g;
  const int R = a.rows_per_head;
  const int row_id = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  if (row_id >= g.Hq * R) return;
  const int hq = row_id / R, rr = row_id - hq * R;
  const int Nv = a.has_video ? g.N : 0;
  const uint16_t *o, *dO;
  const int32_t* list;
  int cnt;
  if (rr < Nv) {
    const int c = rr / g.S;
    const size_t n = (size_t)raster_of(g, c, rr - c * g.S);
    o = a.out_raster + (n * g.Hq + hq) * D;
    dO = a.dout_raster + (n * g.Hq + hq) * D;
    list = a.sel_idx + video_list_offset(a.capv, hq, g.S, c, rr - c * g.S);
  } else {
    const int m = rr - Nv;
    o = a.out_extra + ((size_t)m * g.Hq + hq) * D;
    dO = a.dout_extra + ((size_t)m * g.Hq + hq) * D;
    list = a.sel_idx + extra_list_offset(a.capv, g.Hq, a.n_extra, g.Nc, hq, m);
  }
  cnt = a.sel_count[(size_t)hq * R + rr];
  // D = do . o: thread t takes elements t, t + 16, ...
  float acc = 0.f;
#pragma unroll
  for (int e = t; e < D; e += 16) acc = fmaf(bf16_bits_to_f32(o[e]), bf16_bits_to_f32(dO[e]), acc);
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 16);
  if (t == 0) a.delta[(size_t)hq * R + rr] = acc;
  // selection bitmap, word-major: thread t writes words t, t+16, ...
  for (int w = t; w < a.W; w += 16) {
    int lo = 0, hi = cnt;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (list[mid] < 32 * w) lo = mid + 1; else hi = mid;
    }
    uint32_t word = 0u;
    for (int i = lo; i < cnt && list[i] < 32 * w + 32; ++i) word |= 1u << (list[i] & 31);
    a.bits[((size_t)hq * a.W + w) * R + rr] = word;
  }
}

// ---------------------------------------------------------------------------
// dQ: union tiles of 256 rows sharing a KV head (extra rows first, then video
// tiles of consecutive rows from the last query cube down)
// ---------------------------------------------------------------------------
template <int D>
struct BSmem {
  static constexpr int KS = D + 8;    // bf16 stride of K / V token rows
  static constexpr int VS = BKB + 8;  // bf16 stride of a K^T row
};

template <int D>
__global__ __launch_bounds__(BNT, 1) void k_bwd_dq(BwdArgs a) {
  using Sm = BSmem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lk0[BKB * Sm::KS], lk1[BKB * Sm::KS];
  __shared__ __attribute__((aligned(16))) uint16_t lv0[BKB * Sm::KS], lv1[BKB * Sm::KS];
  __shared__ __attribute__((aligned(16))) uint16_t lt0[D * Sm::VS], lt1[D * Sm::VS];
  __shared__ uint32_t s_bits[BPASS * BNW];
  __shared__ uint16_t s_ulist[BPASS];
  __shared__ int s_nunion;
  auto kbuf = [&](auto c) __attribute__((always_inline)) { if constexpr (decltype(c)::value == 0) return lk0; else return lk1; };
  auto vbuf = [&](auto c) __attribute__((always_inline)) { if constexpr (decltype(c)::value == 0) return lv0; else return lv1; };
  auto tbuf = [&](auto c) __attribute__((always_inline)) { if constexpr (decltype(c)::value == 0) return lt0; else return lt1; };
  const KGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int R = a.rows_per_head;
  const int Nv = a.has_video ? g.N : 0;

  // ---- tile ----
  // video tiles: 256 consecutive video rows of a KV head, numbered query cube
  // by query cube from the last (head slot, offset), so a tile may span query
  // cubes; each row's own cube joins its bitmap in the passes below
  bool video;
  int grp, rho0, c = 0;
  int b = blockIdx.x;
  if (b < a.n_extra_tiles) {
    video = false;
    grp = b / a.extra_tiles_per_group;
    rho0 = (b - grp * a.extra_tiles_per_group) * BTR;
  } else {
    video = true;
    b -= a.n_extra_tiles;
    grp = b % g.Hkv;
    rho0 = (b / g.Hkv) * BTR;
  }
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  const int n_rows = min(BTR, (video ? gsz * g.N : gsz * a.n_extra) - rho0);
  if (n_rows <= 0) return;
  const int hstart = a.hg.start[grp];
  if (video) c = g.Nc - 1 - rho0 / (gsz * g.S);  // the tile's highest query cube
  const int t_row = wave * 32 + lr;
  const bool row_ok = t_row < n_rows;
  int hq = 0, pos = 0;
  if (row_ok) {
    const int rho = rho0 + t_row;
    if (video) {
      const int ci = rho / (gsz * g.S);
      const int rem = rho - ci * gsz * g.S;
      const int slot = rem / g.S;
      hq = a.hg.heads[hstart + slot];
      pos = (g.Nc - 1 - ci) * g.S + (rem - slot * g.S);
    } else {
      const int slot = rho / a.n_extra;
      hq = a.hg.heads[hstart + slot];
      pos = rho - slot * a.n_extra;
    }
  }
  const int rr = video ? pos : Nv + pos;  // row index within the head

  // operands: Q^T and dO^T (row lr, d = 16*ds + 8*lh + [0..8)), row's log2 LSE and D
  bbf16x8 qb[D / 16], db[D / 16];
  {
    const uint16_t* qs = video ? a.q_cube + ((size_t)hq * g.NS + pos) * D : a.q_extra + ((size_t)pos * g.Hq + hq) * D;
    const uint16_t* ds_;
    if (video) {
      const int cc = pos / g.S;
      const size_t n = (size_t)raster_of(g, cc, pos - cc * g.S);
      ds_ = a.dout_raster + (n * g.Hq + hq) * D;
    } else {
      ds_ = a.dout_extra + ((size_t)pos * g.Hq + hq) * D;
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0), w = make_uint4(0, 0, 0, 0);
      if (row_ok) {
        v = *reinterpret_cast<const uint4*>(qs + 16 * s + 8 * lh);
        w = *reinterpret_cast<const uint4*>(ds_ + 16 * s + 8 * lh);
      }
      qb[s] = __builtin_bit_cast(bbf16x8, v);
      db[s] = __builtin_bit_cast(bbf16x8, w);
    }
  }
  const float L2 = row_ok ? a.lse[(size_t)hq * R + rr] * kBLog2e : 0.f;
  const float Dr = row_ok ? a.delta[(size_t)hq * R + rr] : 0.f;
  const float qscale = kBLog2e / sqrtf((float)D);
  bf32x16 acc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[d][i] = 0.f;

  // one key block: K rows (A of S^T), V rows (A of dP^T), K^T rows (A of dQ^T)
  auto compute = [&](const uint16_t* kb, const uint16_t* vb, const uint16_t* tb, bool sel) __attribute__((always_inline)) {
    bf32x16 st[2], dp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) { st[h][i] = 0.f; dp[h][i] = 0.f; }
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bbf16x8 ka = __builtin_bit_cast(bbf16x8, *reinterpret_cast<const uint4*>(&kb[(32 * h + lr) * Sm::KS + 16 * s + 8 * lh]));
        st[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[s], st[h], 0, 0, 0);
      }
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bbf16x8 va = __builtin_bit_cast(bbf16x8, *reinterpret_cast<const uint4*>(&vb[(32 * h + lr) * Sm::KS + 16 * s + 8 * lh]));
        dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, db[s], dp[h], 0, 0, 0);
      }
    // dS^T in the PV operand order: slot 8*lh + e of k-step u holds key
    // 16*u + 8*(e/4) + 4*lh + (e%4), which K^T keeps in column 16*u + 8*lh + e
    bbf16x8 dsb[4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = sel ? bex2(fmaf(st[h][i], qscale, -L2)) : 0.f;
        dsb[2 * h + i / 8][i % 8] = (__bf16)(p * (dp[h][i] - Dr));
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const bbf16x8 ta = __builtin_bit_cast(bbf16x8, *reinterpret_cast<const uint4*>(&tb[(32 * d + lr) * Sm::VS + 16 * u + 8 * lh]));
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, dsb[u], acc[d], 0, 0, 0);
      }
  };

  // direct global -> LDS loads: K rows and V rows (D*2 bytes, 16-byte padded),
  // K^T rows (128 bytes, padded); the padding piece re-reads a valid address
  constexpr int KPR = D / 8 + 1, TPR = BKB / 8 + 1;
  constexpr int NKI = BKB * KPR / 64, NTI = D * TPR / 64;
  constexpr int NLI = 2 * NKI + NTI;
  constexpr int NLW = (NLI + BNW - 1) / BNW;
  static_assert(BKB * KPR % 64 == 0 && D * TPR % 64 == 0, "piece counts");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t dsrc[NLW], dlds[NLW];
  int dkind[NLW];  // 0: K, 1: V, 2: K^T, 3: none
#pragma unroll
  for (int m = 0; m < NLW; ++m) {
    const int t = wv + BNW * m;
    int q;
    if (t < NKI) { dkind[m] = 0; q = t; }
    else if (t < 2 * NKI) { dkind[m] = 1; q = t - NKI; }
    else if (t < NLI) { dkind[m] = 2; q = t - 2 * NKI; }
    else { dkind[m] = 3; q = 0; }
    const int e = 64 * q + lane;
    if (dkind[m] <= 1) {
      const int row = e / KPR, col = e % KPR;
      dsrc[m] = row * D * 2 + (col == KPR - 1 ? 0 : col * 16);
    } else {
      const int row = e / TPR, col = e % TPR;
      dsrc[m] = row * g.S * 2 + (col == TPR - 1 ? 0 : col * 16);
    }
    dlds[m] = q * 1024;
  }
  // buffer loads into LDS (counted on vmcnt only; see buffer_load_lds16), one
  // descriptor per KV head's K rows, V rows and K^T rows
  const int head_bytes = (int)((size_t)g.NS * D * 2);  // < 2^31 (checked at launch)
  void* const kgp = (void*)(a.k_cube + (size_t)grp * g.NS * D);
  void* const vgp = (void*)(a.v_tok + (size_t)grp * g.NS * D);
  void* const tgp = (void*)(a.k_vt + (size_t)grp * g.NS * D);
  // block i of a walk: cube j, key block kbi
  auto issue = [&](int j, int kbi, auto bufc) __attribute__((always_inline)) {
    const uint32_t kvo = (uint32_t)(((size_t)j * g.S + kbi * BKB) * D * 2);
    const uint32_t to = (uint32_t)((size_t)j * g.S * D * 2 + kbi * BKB * 2);
#pragma unroll
    for (int m = 0; m < NLW; ++m) {
      if (dkind[m] == 0)
        buffer_load_lds16(kgp, head_bytes, (char*)kbuf(bufc) + dlds[m], dsrc[m], kvo);
      else if (dkind[m] == 1)
        buffer_load_lds16(vgp, head_bytes, (char*)vbuf(bufc) + dlds[m], dsrc[m], kvo);
      else if (dkind[m] == 2)
        buffer_load_lds16(tgp, head_bytes, (char*)tbuf(bufc) + dlds[m], dsrc[m], to);
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  // nb blocks, block i = (cube cube_of(i), key block i % nkb); work(i, k, v, t)
  const int nkb = g.S / BKB;
  auto walk = [&](int nb, auto cube_of, auto work) __attribute__((always_inline)) {
    if (nb <= 0) return;
    __syncthreads();  // nobody reads either buffer any more
    issue(cube_of(0), 0 % nkb, C0{});
    for (int i = 0; i < nb; i += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (i + 1 < nb) issue(cube_of(i + 1), (i + 1) % nkb, C1{});
      work(i, kbuf(C0{}), vbuf(C0{}), tbuf(C0{}));
      if (i + 1 >= nb) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (i + 2 < nb) issue(cube_of(i + 2), (i + 2) % nkb, C0{});
      work(i + 1, kbuf(C1{}), vbuf(C1{}), tbuf(C1{}));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
  };

  // attended cubes (selected, and for video rows their own cubes): passes of
  // BPASS cubes over the word-major bitmap
  const int cube_hi = video ? c + 1 : g.Nc;
  const uint32_t* rbits = a.bits + (size_t)hq * a.W * R + rr;
  const int own_c = (video && row_ok) ? pos / g.S : -1;  // not in the lists: added here
  for (int jb = 0; jb < cube_hi; jb += BPASS) {
    const int je = min(cube_hi, jb + BPASS);
    const int span = je - jb;
    __syncthreads();
    for (int w0 = jb >> 5; w0 < (je + 31) >> 5; ++w0) {
      uint32_t word = (row_ok && lh == 0) ? rbits[(size_t)w0 * R] : 0u;
      if (lh == 0 && own_c >= 0 && (own_c >> 5) == w0) word |= 1u << (own_c & 31);
      for (int bit = 0; bit < 32; ++bit) {
        const int u = 32 * w0 + bit - jb;
        const uint32_t m = (uint32_t)__ballot((word >> bit) & 1u);
        if (u >= 0 && u < span && lane == 0) s_bits[BNW * u + wave] = m;
      }
    }
    __syncthreads();
    if (wave == 0) {
      int base = 0;
      for (int u0 = 0; u0 < span; u0 += 64) {
        const int u = u0 + lane;
        bool any = false;
        if (u < span) {
          uint32_t o = 0;
#pragma unroll
          for (int w = 0; w < BNW; ++w) o |= s_bits[BNW * u + w];
          any = o != 0u;
        }
        const uint64_t bal = __ballot(any);
        if (any) s_ulist[base + lanes_below(bal)] = (uint16_t)u;
        base += popc64(bal);
      }
      if (lane == 0) s_nunion = base;
    }
    __syncthreads();
    const int nb = s_nunion * nkb;
    walk(nb, [&](int i) { return jb + s_ulist[i / nkb]; },
         [&](int i, const uint16_t* kb, const uint16_t* vb, const uint16_t* tb) __attribute__((always_inline)) {
           const uint32_t mw = s_bits[BNW * s_ulist[i / nkb] + wave];
           if (mw == 0u) return;
           compute(kb, vb, tb, ((mw >> lr) & 1u) != 0u);
         });
  }

  // epilogue: dq = c * acc, acc[d][i] = (K^T dS^T)[32*d + 8*(i/4) + 4*lh + (i%4)][row]
  if (!row_ok) return;
  const float cs = 1.0f / sqrtf((float)D);
  float* dst;
  if (video) {
    const int cc = pos / g.S;
    const size_t n = (size_t)raster_of(g, cc, pos - cc * g.S);
    dst = a.dq_raster + (n * g.Hq + hq) * D;
  } else {
    dst = a.dq_extra + ((size_t)pos * g.Hq + hq) * D;
  }
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(dst + 32 * d + 8 * q + 4 * lh) =
          make_float4(acc[d][4 * q] * cs, acc[d][4 * q + 1] * cs, acc[d][4 * q + 2] * cs, acc[d][4 * q + 3] * cs);
}

// ---------------------------------------------------------------------------
// row lists: one workgroup per (KV head, cube); rows in order: own-cube rows
// (head slot, offset), later video rows (head slot, position), extra rows
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_lists(BwdArgs a) {
  __shared__ int s_wsum[4];
  const KGeom& g = a.g;
  const int grp = blockIdx.x / g.Nc, j = blockIdx.x - grp * g.Nc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.rows_per_head;
  const int Nv = a.has_video ? g.N : 0;
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  int32_t* out = a.lists + list_offset(a, grp, j);
  int base = 0;
  // candidate e of a head: own rows [0, S) -> pos j*S + e; later rows
  // (j+1)*S + ...; then extra rows
  const int own = a.has_video ? g.S : 0;
  const int later = a.has_video ? g.N - (j + 1) * g.S : 0;
  const int per_head = own + later + a.n_extra;
  const int wbit = j & 31;
  for (int s = 0; s < gsz; ++s) {
    const int hq = a.hg.heads[a.hg.start[grp] + s];
    const uint32_t* col = a.bits + ((size_t)hq * a.W + (j >> 5)) * R;
    for (int e0 = 0; e0 < per_head; e0 += 256) {
      const int e = e0 + tid;
      bool take = false;
      int rr = 0;
      if (e < per_head) {
        if (e < own) { rr = j * g.S + e; take = true; }
        else if (e < own + later) { rr = (j + 1) * g.S + (e - own); take = (col[rr] >> wbit) & 1u; }
        else { rr = Nv + (e - own - later); take = (col[rr] >> wbit) & 1u; }
      }
      const uint64_t bal = __ballot(take);
      if (lane == 0) s_wsum[wave] = popc64(bal);
      __syncthreads();
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += s_wsum[w];
      const int tot = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
      if (take) out[base + pre + lanes_below(bal)] = hq * R + rr;
      base += tot;
      __syncthreads();
    }
  }
  if (tid == 0) a.list_count[(size_t)grp * g.Nc + j] = base;
}

// ---------------------------------------------------------------------------
// dK / dV: one workgroup (4 waves, one per SIMD) per (KV head, cube, key block)
// ---------------------------------------------------------------------------
template <int D>
struct BKmem {
  static constexpr int KS = D + 8;   // K / V token rows
  static constexpr int TS = 32 + 8;  // transposed Q / dO tiles: [d][32 rows + pad]
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_bwd_dkdv(BwdArgs a) {
  using Sm = BKmem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lk[BKB * Sm::KS], lv[BKB * Sm::KS];
  __shared__ __attribute__((aligned(16))) uint16_t tq[4][D * Sm::TS], tdo[4][D * Sm::TS];
  __shared__ __attribute__((aligned(16))) float rinfo[4][2][32];  // per wave: log2 LSE and D of its tile rows
  const KGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int R = a.rows_per_head;
  const int Nv = a.has_video ? g.N : 0;
  const int nkb = g.S / BKB;
  // KV head by KV head, so that the rows gathered at any one time are those
  // of one head group (they then stay in the memory-side cache); within a
  // head heaviest first: ascending cube (earlier cubes are attended by more
  // rows)
  const int per_g = g.Nc * nkb;
  const int grp = blockIdx.x / per_g;
  const int rem = blockIdx.x - grp * per_g;
  const int j = rem / nkb, kbi = rem - j * nkb;
  const int key0 = j * g.S + kbi * BKB;  // first key (cube-layout position)
  // K and V rows of the block into LDS
  for (int e = tid; e < BKB * D / 8; e += 256) {
    const int key = e / (D / 8), ch = e - key * (D / 8);
    const size_t src = ((size_t)grp * g.NS + key0 + key) * D + 8 * ch;
    *reinterpret_cast<uint4*>(&lk[key * Sm::KS + 8 * ch]) = *reinterpret_cast<const uint4*>(a.k_cube + src);
    *reinterpret_cast<uint4*>(&lv[key * Sm::KS + 8 * ch]) = *reinterpret_cast<const uint4*>(a.v_tok + src);
  }
  __syncthreads();
  const int cnt = a.list_count[(size_t)grp * g.Nc + j];
  const int32_t* list = a.lists + list_offset(a, grp, j);
  const float qscale = kBLog2e / sqrtf((float)D);
  bf32x16 ak[D / 32][2], av[D / 32][2];  // dK^T, dV^T: [d tile][key tile]
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) { ak[d][h][i] = 0.f; av[d][h][i] = 0.f; }
  uint16_t* Tq = tq[wave];
  uint16_t* Tdo = tdo[wave];
  const int pcol = vt_column(lr, 32);  // transposed column of this lane's row
  const int ntiles = (cnt + 31) / 32;
  // Tile t's rows are list entries 32t..32t+31.  Lanes past the list take the
  // last entry (a valid row with finite values) and are given an infinite
  // log2 LSE (P = 0) and D = 0, so they add nothing; every load is therefore
  // unconditional and none waits before its value is used.  List entries run
  // two tiles ahead of the rows and rows one tile ahead of the compute.
  auto entry = [&](int t) __attribute__((always_inline)) {
    return list[min(t * 32 + lr, cnt - 1)];
  };
  uint4 qraw[D / 16], draw[D / 16];
  float lraw = 0.f, draw_d = 0.f;
  auto fetch = [&](int id) __attribute__((always_inline)) {
    const int hq = id / R, rr = id - hq * R;
    const uint16_t *qs, *ds_;
    if (rr < Nv) {
      const int c = rr / g.S;
      const size_t n = (size_t)raster_of(g, c, rr - c * g.S);
      qs = a.q_cube + ((size_t)hq * g.NS + rr) * D;
      ds_ = a.dout_raster + (n * g.Hq + hq) * D;
    } else {
      const int m = rr - Nv;
      qs = a.q_extra + ((size_t)m * g.Hq + hq) * D;
      ds_ = a.dout_extra + ((size_t)m * g.Hq + hq) * D;
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qraw[s] = *reinterpret_cast<const uint4*>(qs + 16 * s + 8 * lh);
      draw[s] = *reinterpret_cast<const uint4*>(ds_ + 16 * s + 8 * lh);
    }
    lraw = a.lse[(size_t)hq * R + rr];
    draw_d = a.delta[(size_t)hq * R + rr];
  };
  int idn = 0;
  if (ntiles > wave) {
    fetch(entry(wave));
    if (wave + 4 < ntiles) idn = entry(wave + 4);
  }
  for (int t = wave; t < ntiles; t += 4) {
    // the current tile's operands; the next tile's loads fly during its MFMAs
    bbf16x8 qa[D / 16], da[D / 16];
    uint4 qcur[D / 16], dcur[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qcur[s] = qraw[s];
      dcur[s] = draw[s];
      qa[s] = __builtin_bit_cast(bbf16x8, qcur[s]);
      da[s] = __builtin_bit_cast(bbf16x8, dcur[s]);
    }
    if (lh == 0) {
      const bool ok = t * 32 + lr < cnt;
      rinfo[wave][0][lr] = ok ? lraw * kBLog2e : INFINITY;
      rinfo[wave][1][lr] = ok ? draw_d : 0.f;
    }
    if (t + 4 < ntiles) {
      fetch(idn);
      if (t + 8 < ntiles) idn = entry(t + 8);
    }
    // transposed copies: T[d][pcol] = row value at d (16-bit halves taken
    // from the raw words)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t qw[4] = {qcur[s].x, qcur[s].y, qcur[s].z, qcur[s].w};
      const uint32_t dw[4] = {dcur[s].x, dcur[s].y, dcur[s].z, dcur[s].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = 16 * s + 8 * lh + i;
        Tq[d * Sm::TS + pcol] = (uint16_t)(qw[i / 2] >> (16 * (i % 2)));
        Tdo[d * Sm::TS + pcol] = (uint16_t)(dw[i / 2] >> (16 * (i % 2)));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes land before its reads
    // S = Q K^T and dP = dO V^T (rows x keys): element i of lane l is row
    // 8*(i/4) + 4*lh + (i%4), key 32*h + lr
    bf32x16 st[2], dp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) { st[h][i] = 0.f; dp[h][i] = 0.f; }
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bbf16x8 kf = __builtin_bit_cast(bbf16x8, *reinterpret_cast<const uint4*>(&lk[(32 * h + lr) * Sm::KS + 16 * s + 8 * lh]));
        st[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf, st[h], 0, 0, 0);
      }
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bbf16x8 vf = __builtin_bit_cast(bbf16x8, *reinterpret_cast<const uint4*>(&lv[(32 * h + lr) * Sm::KS + 16 * s + 8 * lh]));
        dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[s], vf, dp[h], 0, 0, 0);
      }
    // P and dS as B operands: slot 8*lh + e of row-step u holds row
    // 16*u + 8*(e/4) + 4*lh + (e%4), kept in transposed column 16*u + 8*lh + e
    bbf16x8 pb[2][2], sb[2][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 L4 = *reinterpret_cast<const float4*>(&rinfo[wave][0][8 * q + 4 * lh]);
      const float4 D4 = *reinterpret_cast<const float4*>(&rinfo[wave][1][8 * q + 4 * lh]);
      const float Lq[4] = {L4.x, L4.y, L4.z, L4.w}, Dq[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q + e;
          const float p = bex2(fmaf(st[h][i], qscale, -Lq[e]));
          pb[h][i / 8][i % 8] = (__bf16)p;
          sb[h][i / 8][i % 8] = (__bf16)(p * (dp[h][i] - Dq[e]));
        }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the two row-steps
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const bbf16x8 fo = __builtin_bit_cast(bbf16x8, *reinterpret_cast<const uint4*>(&Tdo[(32 * d + lr) * Sm::TS + 16 * u + 8 * lh]));
        const bbf16x8 fq = __builtin_bit_cast(bbf16x8, *reinterpret_cast<const uint4*>(&Tq[(32 * d + lr) * Sm::TS + 16 * u + 8 * lh]));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          av[d][h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fo, pb[h][u], av[d][h], 0, 0, 0);
          ak[d][h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq, sb[h][u], ak[d][h], 0, 0, 0);
        }
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of T done before the next tile's writes
  }
  // add the four waves' partials through LDS (the transposed tiles are free
  // now), one 32 KB matrix at a time, then wave 0 writes dK and dV
  float* red = reinterpret_cast<float*>(&tq[0][0]);
  static_assert(sizeof(tq) >= (size_t)D * BKB * 4, "reduction buffer");
  auto reduce = [&](bf32x16 (&acc)[D / 32][2]) __attribute__((always_inline)) {
    for (int src = 1; src < 4; ++src) {
      __syncthreads();
      if (wave == src) {
#pragma unroll
        for (int d = 0; d < D / 32; ++d)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) red[((d * 2 + h) * 16 + i) * 64 + lane] = acc[d][h][i];
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int d = 0; d < D / 32; ++d)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[d][h][i] += red[((d * 2 + h) * 16 + i) * 64 + lane];
      }
    }
  };
  reduce(av);
  reduce(ak);
  if (wave != 0) return;
  const float cs = 1.0f / sqrtf((float)D);
  // element i of [d][h]: d-row 32*d + 8*(i/4) + 4*lh + (i%4), key 32*h + lr
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key = kbi * BKB + 32 * h + lr;  // offset inside cube j
    const size_t n = (size_t)raster_of(g, j, key);
    float* dk = a.dk_raster + (n * g.Hkv + grp) * D;
    float* dv = a.dv_raster + (n * g.Hkv + grp) * D;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e0 = 32 * d + 8 * q + 4 * lh;
        *reinterpret_cast<float4*>(dk + e0) = make_float4(ak[d][h][4 * q] * cs, ak[d][h][4 * q + 1] * cs,
                                                          ak[d][h][4 * q + 2] * cs, ak[d][h][4 * q + 3] * cs);
        *reinterpret_cast<float4*>(dv + e0) = make_float4(av[d][h][4 * q], av[d][h][4 * q + 1],
                                                          av[d][h][4 * q + 2], av[d][h][4 * q + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// causal text keys: the text row's log-sum-exp L and D = do . o cover its
// selected cubes and its text keys together, so the text keys' share of the
// gradients separates:  p_j = exp(c q.k_j - L), ds_j = p_j (do.v_j - D),
// dq += c sum_j ds_j k_j, dk_j = c sum_rows ds_j q, dv_j = sum_rows p_j do.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kv_group_of(const HeadGroups& hg, int n_groups, int hq) {
  int grp = 0;
  for (int gg = 0; gg < n_groups; ++gg)
    for (int t = hg.start[gg]; t < hg.start[gg + 1]; ++t)
      if (hg.heads[t] == hq) grp = gg;
  return grp;
}

// 16-byte piece of 8 bf16 values as float32
__device__ __forceinline__ void bf16x8_to_f32(const uint16_t* src, float (&x)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// One wave per text row (hq, m).  Each round, lane l takes text key j0 + l
// (j <= m) and forms ds_j from full float32 dot products against the row's q
// and do (kept in LDS); then every lane adds ds_j k_j over the round's keys to
// its D/64 output dims.  dq_extra already holds the selected cubes' share.
template <int D>
__global__ __launch_bounds__(64) void k_bwd_text_dq(BwdArgs a) {
  constexpr int PER = D / kWave;
  __shared__ float s_q[D], s_do[D], s_ds[kWave];
  const KGeom& g = a.g;
  const int lane = threadIdx.x;
  const int hq = blockIdx.x / a.n_extra, m = blockIdx.x - hq * a.n_extra;
  const int grp = kv_group_of(a.hg, g.Hkv, hq);
  const int R = a.rows_per_head, Nv = a.has_video ? g.N : 0;
  const uint16_t* q = a.q_extra + ((size_t)m * g.Hq + hq) * D;
  const uint16_t* dO = a.dout_extra + ((size_t)m * g.Hq + hq) * D;
  for (int e = lane; e < D; e += kWave) {
    s_q[e] = bf16_bits_to_f32(q[e]);
    s_do[e] = bf16_bits_to_f32(dO[e]);
  }
  const float L = a.lse[(size_t)hq * R + Nv + m];
  const float Dr = a.delta[(size_t)hq * R + Nv + m];
  const float c = 1.0f / sqrtf((float)D);
  const size_t kstride = (size_t)g.Hkv * D;  // between consecutive text tokens
  const uint16_t* kt = a.k_text + (size_t)grp * D;
  const uint16_t* vt = a.v_text + (size_t)grp * D;
  __syncthreads();
  float acc[PER] = {};
  for (int j0 = 0; j0 <= m; j0 += kWave) {
    const int j = j0 + lane;
    float ds = 0.f;
    if (j <= m) {
      float sd = 0.f, dp = 0.f;
      for (int e = 0; e < D; e += 8) {
        float kx[8], vx[8];
        bf16x8_to_f32(kt + j * kstride + e, kx);
        bf16x8_to_f32(vt + j * kstride + e, vx);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          sd = fmaf(kx[i], s_q[e + i], sd);
          dp = fmaf(vx[i], s_do[e + i], dp);
        }
      }
      const float p = expf(c * sd - L);
      ds = p * (dp - Dr);
    }
    s_ds[lane] = ds;
    __syncthreads();
    const int nj = min(kWave, m + 1 - j0);
    for (int jj = 0; jj < nj; ++jj) {
      const float w = s_ds[jj];
      const uint16_t* kr = kt + (size_t)(j0 + jj) * kstride + lane * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, bf16_bits_to_f32(kr[i]), acc[i]);
    }
    __syncthreads();
  }
  float* dst = a.dq_extra + ((size_t)m * g.Hq + hq) * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[i] += c * acc[i];
}

// One wave per (KV head, text key j): lanes take the group's text rows m >= j
// (head slot by head slot) 64 at a time, form p and ds for key j, then every
// lane folds dv += p do and dk += ds q over the round's rows into its D/64
// dims.  Every (key, KV head) of the text is written once.
template <int D>
__global__ __launch_bounds__(64) void k_bwd_text_dkdv(BwdArgs a) {
  constexpr int PER = D / kWave;
  __shared__ float s_k[D], s_v[D], s_p[kWave], s_ds[kWave];
  __shared__ int s_row[kWave];
  const KGeom& g = a.g;
  const int lane = threadIdx.x;
  const int grp = blockIdx.x / a.n_extra, j = blockIdx.x - grp * a.n_extra;
  const int R = a.rows_per_head, Nv = a.has_video ? g.N : 0;
  const int hstart = a.hg.start[grp], gsz = a.hg.start[grp + 1] - hstart;
  const size_t kstride = (size_t)g.Hkv * D;
  for (int e = lane; e < D; e += kWave) {
    s_k[e] = bf16_bits_to_f32(a.k_text[j * kstride + (size_t)grp * D + e]);
    s_v[e] = bf16_bits_to_f32(a.v_text[j * kstride + (size_t)grp * D + e]);
  }
  const float c = 1.0f / sqrtf((float)D);
  const int per_head = a.n_extra - j;  // text rows j .. n_extra - 1 of each head
  const int nr = gsz * per_head;
  __syncthreads();
  float dk[PER] = {}, dv[PER] = {};
  for (int r0 = 0; r0 < nr; r0 += kWave) {
    const int r = r0 + lane;
    float p = 0.f, ds = 0.f;
    int hq = 0, m = 0;
    if (r < nr) {
      const int slot = r / per_head;
      m = j + (r - slot * per_head);
      hq = a.hg.heads[hstart + slot];
      const uint16_t* q = a.q_extra + ((size_t)m * g.Hq + hq) * D;
      const uint16_t* dO = a.dout_extra + ((size_t)m * g.Hq + hq) * D;
      float sd = 0.f, dp = 0.f;
      for (int e = 0; e < D; e += 8) {
        float qx[8], ox[8];
        bf16x8_to_f32(q + e, qx);
        bf16x8_to_f32(dO + e, ox);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          sd = fmaf(qx[i], s_k[e + i], sd);
          dp = fmaf(ox[i], s_v[e + i], dp);
        }
      }
      p = expf(c * sd - a.lse[(size_t)hq * R + Nv + m]);
      ds = p * (dp - a.delta[(size_t)hq * R + Nv + m]);
    }
    s_p[lane] = p;
    s_ds[lane] = ds;
    s_row[lane] = m * g.Hq + hq;
    __syncthreads();
    const int nrr = min(kWave, nr - r0);
    for (int rr = 0; rr < nrr; ++rr) {
      const size_t off = (size_t)s_row[rr] * D + lane * PER;
      const float pw = s_p[rr], dw = s_ds[rr];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        dv[i] = fmaf(pw, bf16_bits_to_f32(a.dout_extra[off + i]), dv[i]);
        dk[i] = fmaf(dw, bf16_bits_to_f32(a.q_extra[off + i]), dk[i]);
      }
    }
    __syncthreads();
  }
  float* dko = a.dk_text + (j * kstride + (size_t)grp * D) + lane * PER;
  float* dvo = a.dv_text + (j * kstride + (size_t)grp * D) + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    dko[i] = c * dk[i];
    dvo[i] = dv[i];
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
void plan_backward(BwdArgs& a) {
  const KGeom& g = a.g;
  a.W = (g.Nc + 31) / 32;
  a.video_tiles_per_group = a.has_video ? (int)(((int64_t)a.hg.gmax * g.N + BTR - 1) / BTR) : 0;
  a.extra_tiles_per_group = a.n_extra ? (a.hg.gmax * a.n_extra + BTR - 1) / BTR : 0;
  a.n_extra_tiles = g.Hkv * a.extra_tiles_per_group;
  a.list_cap_g = (int64_t)a.hg.gmax * ((a.has_video ? (int64_t)g.S * g.Nc * (g.Nc + 1) / 2 : 0) +
                                       (int64_t)g.Nc * a.n_extra);
}

size_t backward_workspace_bytes(const BwdArgs& a) {
  const KGeom& g = a.g;
  const size_t rows = (size_t)g.Hq * a.rows_per_head;
  size_t b = rows * 4;                       // delta
  b += (size_t)g.Hq * a.W * a.rows_per_head * 4;  // bitmap
  b += (size_t)g.Hkv * g.Nc * 4;             // list counts
  b += (size_t)g.Hkv * a.list_cap_g * 4;     // lists
  return b + 256;
}

void bind_backward_workspace(BwdArgs& a, void* ws) {
  const KGeom& g = a.g;
  char* p = static_cast<char*>(ws);
  const size_t rows = (size_t)g.Hq * a.rows_per_head;
  a.delta = reinterpret_cast<float*>(p);
  p += rows * 4;
  a.bits = reinterpret_cast<uint32_t*>(p);
  p += (size_t)g.Hq * a.W * a.rows_per_head * 4;
  a.list_count = reinterpret_cast<int32_t*>(p);
  p += (size_t)g.Hkv * g.Nc * 4;
  a.lists = reinterpret_cast<int32_t*>(p);
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  const KGeom& g = a.g;
  // buffer descriptors address one KV head's rows with 32-bit offsets
  if ((size_t)g.NS * g.D * 2 > 0x7fffffffu) return hipErrorInvalidValue;
  const int rows = g.Hq * a.rows_per_head;
  const int nkb = g.S / BKB;
  if (g.D == 128) {
    hipLaunchKernelGGL(k_bwd_prep<128>, dim3((rows + 15) / 16), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_bwd_dq<128>, dim3(a.n_extra_tiles + g.Hkv * a.video_tiles_per_group), dim3(BNT),
                       0, s, a);
    hipLaunchKernelGGL(k_bwd_lists, dim3(g.Hkv * g.Nc), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_bwd_dkdv<128>, dim3(g.Nc * g.Hkv * nkb), dim3(256), 0, s, a);
    if (a.n_text_kv > 0) {
      hipLaunchKernelGGL(k_bwd_text_dq<128>, dim3(g.Hq * a.n_extra), dim3(64), 0, s, a);
      hipLaunchKernelGGL(k_bwd_text_dkdv<128>, dim3(g.Hkv * a.n_extra), dim3(64), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL(k_bwd_prep<64>, dim3((rows + 15) / 16), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_bwd_dq<64>, dim3(a.n_extra_tiles + g.Hkv * a.video_tiles_per_group), dim3(BNT),
                       0, s, a);
    hipLaunchKernelGGL(k_bwd_lists, dim3(g.Hkv * g.Nc), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_bwd_dkdv<64>, dim3(g.Nc * g.Hkv * nkb), dim3(256), 0, s, a);
    if (a.n_text_kv > 0) {
      hipLaunchKernelGGL(k_bwd_text_dq<64>, dim3(g.Hq * a.n_extra), dim3(64), 0, s, a);
      hipLaunchKernelGGL(k_bwd_text_dkdv<64>, dim3(g.Hkv * a.n_extra), dim3(64), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace adas
