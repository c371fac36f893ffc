// Attention over the selected cubes plus the own cube (AdaSpark,
// papernotes.org, key design 2: attend to the Top-p cube set and always keep
// full attention to the own cube; one exact softmax, scale 1/sqrt(d_k)).
// bf16 MFMA kernel with union tiles.
//
// A workgroup (8 waves) owns a tile of 256 rows that read the same KV head:
// consecutive video rows, numbered query cube by query cube from the last (a
// tile may span two or more query cubes), or extra rows.  Each wave owns 32
// rows; their query operands and float32 output accumulators stay in
// registers for the whole tile.  The workgroup walks the union of the cubes
// its rows attend (selected cubes and, for video rows, their own cubes, in
// descending order; for text rows also the causal text keys), one key block of
// 64 keys at a time:
//   * K rows and V^T rows (values arrive cube-transposed, ADAS_LAYOUT_VT) of a
//     block are staged in LDS.  When every block is full (S a multiple of 64)
//     video blocks move global -> LDS with buffer_load_dwordx4 ... lds over
//     four buffers, two blocks ahead, one barrier per pair of blocks;
//     otherwise, and for text keys, through registers one block ahead with
//     one barrier per block;
//   * each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, applies a
//     per-row bit (row x cube bitmap built from the selection lists and the
//     rows' own cubes) as a +inf softmax bias, keeps the online softmax in log2
//     units with lazy rescaling, and accumulates O^T += V^T P^T.  On full
//     blocks the softmax unit is half a block (32 keys) and the units are
//     software-pipelined: the exp / convert instructions of one unit are
//     issued between the MFMAs of its neighbours.
// Rows spend MFMA work on every key block of the tile union; the masked part is
// the price of keeping accumulators in registers.
//
// Tile order: extra rows first (heaviest), then video tiles from the last
// query cube down.  When 8 is a multiple of the KV head count, workgroup b runs
// on XCD b % 8 (round-robin dispatch) and video tiles are dealt so that each
// XCD serves one KV head, letting concurrently resident tiles share K/V in L2.
#include <type_traits>

#include "common.h"

namespace adas {

typedef __bf16 bf16x8u __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4u __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2u __attribute__((ext_vector_type(2)));

namespace {
constexpr int UKB = 64;      // keys per key block
constexpr int UNW = 8;       // waves per workgroup
constexpr int UNT = 64 * UNW;
constexpr int UTR = 32 * UNW;  // rows per tile
constexpr int UPASS = 512;   // cubes per selection-bitmap pass (LDS budget)
constexpr float kLog2eU = 1.4426950408889634f;
constexpr float kLazy = 8.0f;  // rescale only when a block max exceeds the reference by 2^8
constexpr float kOver = 16777216.0f;  // 2^24: largest block sum accepted without a block max

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
// f(integral_constant<int, I>), ..., f(integral_constant<int, N - 1>)
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
}  // namespace

int union_tile_rows() { return UTR; }

struct USched {
  int video_tiles_per_group;  // video tiles per KV head (its rows over every query cube)
  int extra_tiles_per_group;
  int extra_chunks;
  int extra_chunk_cubes;
  int n_extra_wgs;
  int xcd_mode;  // 1: XCD-aware dealing of video tiles
};

template <int D>
struct USmem {
  static constexpr int KS = D + 8;    // bf16 stride of a K row (68 dwords: conflict-free b128 reads)
  static constexpr int VS = UKB + 8;  // bf16 stride of a V^T row (36 dwords: conflict-free b128 reads)
};

// FULL: every key block holds UKB valid keys (S a multiple of UKB), so the
// video phases never need per-key masks.
template <int D, bool FULL>
__global__ __launch_bounds__(UNT, 1) void k_attn_union(AttnArgs a, USched sc) {
  using Sm = USmem<D>;
  // Three K and three V^T block buffers as separate LDS objects, so that the
  // compiler can tell reads of one from asynchronous global->LDS loads into
  // another.
  __shared__ __attribute__((aligned(16))) uint16_t lk0[UKB * Sm::KS], lk1[UKB * Sm::KS], lk2[UKB * Sm::KS],
      lk3[UKB * Sm::KS];
  __shared__ __attribute__((aligned(16))) uint16_t lv0[D * Sm::VS], lv1[D * Sm::VS], lv2[D * Sm::VS],
      lv3[D * Sm::VS];
  __shared__ uint32_t s_bits[UPASS * UNW];  // [cube in pass][wave] -> rows of the wave that selected it
  __shared__ uint16_t s_ulist[UPASS];       // cubes of the pass selected by any row
  __shared__ int s_nunion;
  auto kbuf_rt = [&](int b) __attribute__((always_inline)) { return b == 0 ? lk0 : (b == 1 ? lk1 : lk2); };
  auto vbuf_rt = [&](int b) __attribute__((always_inline)) { return b == 0 ? lv0 : (b == 1 ? lv1 : lv2); };
  auto kbuf_c = [&](auto c) __attribute__((always_inline)) {
    if constexpr (decltype(c)::value == 0) return lk0;
    else if constexpr (decltype(c)::value == 1) return lk1;
    else if constexpr (decltype(c)::value == 2) return lk2;
    else return lk3;
  };
  auto vbuf_c = [&](auto c) __attribute__((always_inline)) {
    if constexpr (decltype(c)::value == 0) return lv0;
    else if constexpr (decltype(c)::value == 1) return lv1;
    else if constexpr (decltype(c)::value == 2) return lv2;
    else return lv3;
  };
  const KGeom& g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;  // row of this lane inside the wave
  const int lh = lane >> 5;  // lane half

  // ---- decode the tile ----------------------------------------------------------
  bool video;
  int grp, rho0, c = 0, chunk = 0, tile_e = 0;
  int b = blockIdx.x;
  if (b < sc.n_extra_wgs) {
    video = false;
    tile_e = b / sc.extra_chunks;
    chunk = b - tile_e * sc.extra_chunks;
    grp = tile_e / sc.extra_tiles_per_group;
    rho0 = (tile_e - grp * sc.extra_tiles_per_group) * UTR;
  } else {
    // video tile t of KV head grp: rows rho0 .. rho0 + UTR of the head's video
    // rows, numbered query cube by query cube from the last (head slot, offset
    // inside a cube), so a tile may span two or more query cubes
    video = true;
    b -= sc.n_extra_wgs;
    int t;
    if (sc.xcd_mode) {
      const int x = b & 7, i = b >> 3;
      grp = x % g.Hkv;
      t = x / g.Hkv + i * (8 / g.Hkv);
    } else {
      grp = b % g.Hkv;
      t = b / g.Hkv;
    }
    if (t >= sc.video_tiles_per_group) return;
    rho0 = t * UTR;
  }
  const int gsz = a.hg.start[grp + 1] - a.hg.start[grp];
  const int group_rows = video ? gsz * g.N : gsz * a.n_extra;
  const int n_rows = min(UTR, group_rows - rho0);
  if (n_rows <= 0) return;
  const int hstart = a.hg.start[grp];
  if (video) c = g.Nc - 1 - rho0 / (gsz * g.S);  // the tile's highest query cube

  // ---- this lane's row ------------------------------------------------------------
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
  const bool wave_has_rows = wave * 32 < n_rows;

  // Q^T operand: row lr, d = 16*ds + 8*lh + [0..8)
  bf16x8u qb[D / 16];
  {
    const uint16_t* src = video ? (const uint16_t*)a.q_cube + ((size_t)hq * g.NS + pos) * D
                                : (const uint16_t*)a.q_extra + ((size_t)pos * g.Hq + hq) * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *reinterpret_cast<const uint4*>(src + 16 * ds + 8 * lh);
      qb[ds] = __builtin_bit_cast(bf16x8u, v);
    }
  }
  const float qscale = kLog2eU / sqrtf((float)D);
  const bf16x2u kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

  // running softmax state of the lane's row (identical in both lane halves)
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // ---- K/V staging through registers -------------------------------------------------
  // K: 16-byte vector e = tid + UNT*u -> key e / VPR, chunk e % VPR (row-major copy).
  // V from ADAS_LAYOUT_VT (video cubes): 16-byte piece e = tid + UNT*u -> V^T
  //    row e / 8, keys 8*(e % 8) .. +8 of the block, already in V^T column
  //    order; a plain copy.
  // V from token-major text: thread (key pair kp, d-chunk vc) loads keys 2kp,
  //    2kp+1 and writes V^T rows 8vc..8vc+7 as 32-bit pairs.  The two lane
  //    halves of a wave take adjacent d-chunks (rows 8 apart = 32 banks apart),
  //    so a 64-lane store covers 64 distinct banks.
  // V^T column order: inside each group of 16 keys, key bits 2 and 3 are
  // swapped, so the 8 keys one lane feeds to a PV k-step are contiguous and
  // read as one b128 (the same order ADAS_LAYOUT_VT stores).
  constexpr int VPR = D / 8;
  constexpr int NK = UKB * VPR / UNT;       // K vectors per thread (2 for D = 128, 1 for D = 64)
  constexpr int NVT = D * (UKB / 8) / UNT;  // V^T pieces per thread (same counts)
  static_assert(NVT <= 2, "vr holds two vectors");
  const int kp = lane & 31;
  const int vc = 2 * wave + lh;
  const int vcol = (2 * kp & ~12) | ((2 * kp & 4) << 1) | ((2 * kp & 8) >> 1);  // V^T column of key 2kp
  const bool v_thread = vc < VPR;
  uint4 kr[NK], vr[2];
  // vt: V comes cube-transposed (row stride vstride = S elements); else
  // token-major with the K stride.
  auto fetch = [&](bool vt, const uint16_t* kb, const uint16_t* vb, size_t stride, int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int e = tid + UNT * u;
      const int key = e / VPR, ch = e % VPR;
      kr[u] = key < kc ? *reinterpret_cast<const uint4*>(kb + key * stride + ch * 8)
                       : make_uint4(0, 0, 0, 0);
    }
    if (vt) {
#pragma unroll
      for (int u = 0; u < NVT; ++u) {
        const int e = tid + UNT * u;
        const int row = e >> 3, c8 = e & 7;
        vr[u] = 8 * c8 < kc ? *reinterpret_cast<const uint4*>(vb + (size_t)row * g.S + 8 * c8)
                            : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = 2 * kp + u;
        vr[u] = (v_thread && key < kc) ? *reinterpret_cast<const uint4*>(vb + key * stride + vc * 8)
                                       : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stage = [&](bool vt, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int e = tid + UNT * u;
      const int key = e / VPR, ch = e % VPR;
      *reinterpret_cast<uint4*>(&kbuf_rt(buf)[key * Sm::KS + ch * 8]) = kr[u];
    }
    if (vt) {
#pragma unroll
      for (int u = 0; u < NVT; ++u) {
        const int e = tid + UNT * u;
        *reinterpret_cast<uint4*>(&vbuf_rt(buf)[(e >> 3) * Sm::VS + 8 * (e & 7)]) = vr[u];
      }
    } else if (v_thread) {
      const uint32_t w0[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};
      const uint32_t w1[4] = {vr[1].x, vr[1].y, vr[1].z, vr[1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (e & 1) ? (w0[e / 2] >> 16) : (w0[e / 2] & 0xFFFFu);
        const uint32_t hi = (e & 1) ? (w1[e / 2] & 0xFFFF0000u) : (w1[e / 2] << 16);
        *reinterpret_cast<uint32_t*>(&vbuf_rt(buf)[(8 * vc + e) * Sm::VS + vcol]) = lo | hi;
      }
    }
  };

  // ---- one key block from buffer `buf`: rowsel = this lane's row takes part --------
  // kc valid keys; causal: key kbase_idx + key must be <= the row's token index.
  // A lane whose row did not select the block gets bias +inf, i.e. P = 0.
  auto compute = [&](auto per_key_mask, const uint16_t* kbuf, const uint16_t* vbuf, bool rowsel, int kc, bool causal,
                     int kbase_idx) __attribute__((always_inline)) {
    constexpr bool PKM = decltype(per_key_mask)::value;
    f32x16 st[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[h2][i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        if (!PKM || 32 * h2 < kc) {
          const bf16x8u ka = __builtin_bit_cast(
              bf16x8u, *reinterpret_cast<const uint4*>(&kbuf[(32 * h2 + lr) * Sm::KS + 16 * ds + 8 * lh]));
          st[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[ds], st[h2], 0, 0, 0);
        }
      }
    }
    // keys of st[h2][i]: 32*h2 + 8*(i/4) + 4*lh + (i%4)
    if constexpr (PKM) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * h2 + 8 * (i / 4) + 4 * lh + (i % 4);
          const bool ok = key < kc && (!causal || kbase_idx + key <= pos);
          st[h2][i] = ok ? st[h2][i] : -INFINITY;
        }
    }
    // P in bf16 against the reference m_run; the row sum is taken over the
    // same bf16 values the PV product uses (two per v_dot2 against (1, 1)),
    // so numerator and denominator agree.
    bf16x8u pb[4];
    float ls = 0.f;
    auto make_p = [&](float bias) __attribute__((always_inline)) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i) pb[2 * h2 + i / 8][i % 8] = (__bf16)ex2(fmaf(st[h2][i], qscale, -bias));
      ls = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2u pair = {pb[u][2 * e], pb[u][2 * e + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, ls, false);
        }
      ls += xor32_f32(ls);
    };
    // Fast path: once a row has a reference, P is formed against it without
    // a block max; the block is accepted while every row's block sum stays
    // at most 2^kOver (no P above 2^kOver, nothing near overflow).  Otherwise
    // (a row's first block, or a block far above its reference) the block
    // max sets the reference first; it is raised only when it exceeds the
    // old one by more than 2^kLazy, so the accumulators are rescaled rarely.
    bool done = false;
    if (__ballot(rowsel && m_run == -INFINITY) == 0ull) {
      make_p(rowsel ? m_run : INFINITY);
      done = __ballot(!(ls <= kOver)) == 0ull;
    }
    if (!done) {
      float mb = fmaxf(st[0][0], st[1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mb = fmaxf(fmaxf(mb, st[0][i]), st[1][i]);  // v_max3
      mb = fmaxf(mb, xor32_f32(mb));
      const float mb_c = rowsel ? mb * qscale : -INFINITY;
      const bool grow = mb_c > m_run + kLazy;
      if (__ballot(grow) != 0ull) {
        // only growing lanes rescale (a lane still at -inf must not form -inf - -inf)
        const float alpha = grow ? ex2(m_run - mb_c) : 1.0f;  // 0 when m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        m_run = grow ? mb_c : m_run;
      }
      make_p((rowsel && m_run != -INFINITY) ? m_run : INFINITY);
    }
    l_run += ls;
    // O^T += V^T P^T over 4 k-steps of 16 keys; slot 8*lh + e of k-step u
    // holds key 16*u + 8*(e/4) + 4*lh + (e%4), which V^T keeps in column
    // 16*u + 8*lh + e.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!PKM || 16 * u < kc) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8u va = __builtin_bit_cast(
              bf16x8u, *reinterpret_cast<const uint4*>(&vbuf[(32 * db + lr) * Sm::VS + 16 * u + 8 * lh]));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[u], acc[db], 0, 0, 0);
        }
      }
    }
  };
  using kFull = std::integral_constant<bool, false>;
  using kMasked = std::integral_constant<bool, true>;

  // ---- software-pipelined full blocks (video walks when FULL) ---------------------------
  // The softmax unit is a half block of 32 keys; unit u of a call is half u % 2
  // of block u / 2.  S(u): its score MFMAs; sm(u): its softmax on the vector
  // ALUs; PV(u): its MFMAs into the output (D/16 each).  The units of one or two blocks
  // run as steps S(0); S(1)|sm(0); S(2) PV(0)|sm(1); S(3) PV(1)|sm(2);
  // PV(2)|sm(3); PV(3).  Within a step the order is fixed by scheduling
  // barriers: slot k issues the LDS operand read of MFMA k+3, MFMA k, then a
  // slice of the softmax, so the exp and convert instructions of one unit run
  // while the MFMAs of its neighbours execute.  The last three slots of a step
  // read the first three operands of the next step of the same blocks, so a
  // step starts with its operands in flight.  Scores and probabilities
  // alternate between two register slots (u % 2); S and PV MFMAs of a step
  // alternate, so consecutive MFMAs use different accumulators.
  f32x16 su[2];
  bf16x8u pu[2][2];
  uint4 fq[4];  // LDS operand fragments in flight: MFMA k of a step reads fq[k % 4]
  // operand read of MFMA k of a step with score unit sU and output unit pvU
  auto rd_op = [&](auto sUc, auto pvUc, auto kc, const uint16_t* kb, const uint16_t* vb)
                   __attribute__((always_inline)) {
    constexpr int sU = decltype(sUc)::value, pvU = decltype(pvUc)::value, k = decltype(kc)::value;
    constexpr bool HS = sU >= 0, HP = pvU >= 0;
    constexpr bool is_s = HS && (!HP || k % 2 == 0);
    constexpr int i = (HS && HP) ? k / 2 : k;
    constexpr int ND = D / 32;
    if constexpr (is_s)
      fq[k % 4] = *reinterpret_cast<const uint4*>(&kb[(32 * (sU & 1) + lr) * Sm::KS + 16 * i + 8 * lh]);
    else
      fq[k % 4] = *reinterpret_cast<const uint4*>(
          &vb[(32 * (i % ND) + lr) * Sm::VS + 16 * (2 * (pvU & 1) + i / ND) + 8 * lh]);
  };
  // run_step(S unit, PV unit, softmax unit, K / V^T buffers, rows selected,
  //          operands already read by the previous step, next step's S and PV
  //          units (UN, UN: none), next step's buffers)
  auto run_step = [&](auto sUc, auto pvUc, auto smUc, const uint16_t* kb, const uint16_t* vb,
                      bool sel, auto preC, auto nsUc, auto npvUc, const uint16_t* kbn,
                      const uint16_t* vbn) __attribute__((always_inline)) {
    constexpr int sU = decltype(sUc)::value, pvU = decltype(pvUc)::value, smU = decltype(smUc)::value;
    constexpr bool HS = sU >= 0, HP = pvU >= 0, HM = smU >= 0;
    constexpr int NO = D / 16;  // MFMAs of one S(u) (k-steps over d) and of one PV(u) (2 k-steps x D/32 tiles)
    constexpr int ND = D / 32;
    constexpr int NM = (HS ? NO : 0) + (HP ? NO : 0);
    constexpr int NNM = (decltype(nsUc)::value >= 0 ? NO : 0) + (decltype(npvUc)::value >= 0 ? NO : 0);
    static_assert(NM % 4 == 0, "a step's MFMA count keeps the fragment slots aligned");
    constexpr int ss = sU & 1, ps = pvU & 1, ms = smU & 1;
    auto is_s = [](auto kc) constexpr { return HS && (!HP || (decltype(kc)::value % 2) == 0); };
    auto op_i = [](auto kc) constexpr { return (HS && HP) ? decltype(kc)::value / 2 : decltype(kc)::value; };
    auto mf = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value, i = op_i(kc);
      const bf16x8u a8 = __builtin_bit_cast(bf16x8u, fq[k % 4]);
      if constexpr (is_s(kc)) {
        if constexpr (i == 0) {
          const f32x16 z = {};
          su[ss] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, qb[0], z, 0, 0, 0);
        } else {
          su[ss] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, qb[i], su[ss], 0, 0, 0);
        }
      } else {
        acc[i % ND] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, pu[ps][i / ND], acc[i % ND], 0, 0, 0);
      }
    };
    // softmax of unit smU in 8 pieces (pairs of exp / convert / row-sum),
    // against the row's current reference m_run with no unit max: while
    // every selected row has a reference and its unit sum stays below kOver,
    // that is exact.  Otherwise (a row's first unit, or a unit far above the
    // reference) the slow path after the step takes the unit max, raises the
    // reference lazily (only past 2^kLazy), rescales and forms P again.
    const float bias = sel ? m_run : INFINITY;
    float ls = 0.f;
    auto piece = [&](auto ic) __attribute__((always_inline)) {
      constexpr int e = decltype(ic)::value;
      const __bf16 p0 = (__bf16)ex2(fmaf(su[ms][2 * e], qscale, -bias));
      const __bf16 p1 = (__bf16)ex2(fmaf(su[ms][2 * e + 1], qscale, -bias));
      pu[ms][e / 4][2 * (e % 4)] = p0;
      pu[ms][e / 4][2 * (e % 4) + 1] = p1;
      const bf16x2u pair = {p0, p1};
      ls = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, ls, false);
    };
    if constexpr (!decltype(preC)::value) {
      rd_op(sUc, pvUc, std::integral_constant<int, 0>{}, kb, vb);
      rd_op(sUc, pvUc, std::integral_constant<int, 1>{}, kb, vb);
      rd_op(sUc, pvUc, std::integral_constant<int, 2>{}, kb, vb);
    }
    static_for<0, NM>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k + 3 < NM) rd_op(sUc, pvUc, std::integral_constant<int, k + 3>{}, kb, vb);
      else if constexpr (k + 3 - NM < NNM)
        rd_op(nsUc, npvUc, std::integral_constant<int, k + 3 - NM>{}, kbn, vbn);
      mf(kc);
      if constexpr (HM)
        static_for<0, 8>([&](auto ic) __attribute__((always_inline)) {
          if constexpr ((decltype(ic)::value * NM) / 8 == k) piece(ic);
        });
    });
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (HM) {
      float lsu = ls + xor32_f32(ls);
      if (__ballot(sel && (m_run == -INFINITY || !(lsu <= kOver))) != 0ull) {
        float mb = fmaxf(su[ms][0], su[ms][1]);
#pragma unroll
        for (int e = 2; e < 16; e += 2) mb = fmaxf(fmaxf(mb, su[ms][e]), su[ms][e + 1]);
        mb = fmaxf(mb, xor32_f32(mb));
        const float mb_c = sel ? mb * qscale : -INFINITY;
        const bool grow = mb_c > m_run + kLazy;
        // the accumulators already hold PV(smU - 1), formed against the old
        // reference, so rescaling them here is exact
        if (__ballot(grow) != 0ull) {
          const float alpha = grow ? ex2(m_run - mb_c) : 1.0f;  // 0 when m_run = -inf
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
          m_run = grow ? mb_c : m_run;
        }
        const float b2 = (sel && m_run != -INFINITY) ? m_run : INFINITY;
        float l2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 p0 = (__bf16)ex2(fmaf(su[ms][2 * e], qscale, -b2));
          const __bf16 p1 = (__bf16)ex2(fmaf(su[ms][2 * e + 1], qscale, -b2));
          pu[ms][e / 4][2 * (e % 4)] = p0;
          pu[ms][e / 4][2 * (e % 4) + 1] = p1;
          const bf16x2u pair = {p0, p1};
          l2 = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, l2, false);
        }
        lsu = l2 + xor32_f32(l2);
      }
      l_run += lsu;
    }
  };
  using UN = std::integral_constant<int, -1>;
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;
  using U2 = std::integral_constant<int, 2>;
  using U3 = std::integral_constant<int, 3>;
  // preC: whether the previous step already read the first operands
  using PF = std::false_type;
  using PT = std::true_type;
  // two full blocks
  auto block2 = [&](const uint16_t* kb0, const uint16_t* vb0, bool sel0, const uint16_t* kb1,
                    const uint16_t* vb1, bool sel1) __attribute__((always_inline)) {
    run_step(U0{}, UN{}, UN{}, kb0, vb0, sel0, PF{}, U1{}, UN{}, kb0, vb0);
    run_step(U1{}, UN{}, U0{}, kb0, vb0, sel0, PT{}, U2{}, U0{}, kb1, vb0);
    run_step(U2{}, U0{}, U1{}, kb1, vb0, sel0, PT{}, U3{}, U1{}, kb1, vb0);
    run_step(U3{}, U1{}, U2{}, kb1, vb0, sel1, PT{}, UN{}, U2{}, kb1, vb1);
    run_step(UN{}, U2{}, U3{}, kb1, vb1, sel1, PT{}, UN{}, U3{}, kb1, vb1);
    run_step(UN{}, U3{}, UN{}, kb1, vb1, sel1, PT{}, UN{}, UN{}, kb1, vb1);
  };

  // Register-staged walk over nb key blocks: source(i, kptr, vptr, stride, kc)
  // names block i (vt: values cube-transposed), work(i, buf, kc) computes it.
  // One barrier per block: staging into buffer i&1 is safe because every
  // wave finished block i-2 before the barrier of block i-1.
  auto pipeline = [&](bool vt, int nb, auto source, auto work) __attribute__((always_inline)) {
    if (nb <= 0) return;
    __syncthreads();  // the previous phase no longer reads either buffer
    const uint16_t *kp0, *vp0;
    size_t st0;
    int kc0;
    source(0, kp0, vp0, st0, kc0);
    fetch(vt, kp0, vp0, st0, kc0);
    int kc_cur = kc0;
    for (int i = 0; i < nb; ++i) {
      const int buf = i & 1;
      stage(vt, buf);
      int kc_next = 0;
      if (i + 1 < nb) {
        const uint16_t *kpn, *vpn;
        size_t stn;
        source(i + 1, kpn, vpn, stn, kc_next);
        fetch(vt, kpn, vpn, stn, kc_next);
      }
      __syncthreads();
      work(i, buf, kc_cur);
      kc_cur = kc_next;
    }
  };

  // ---- direct global->LDS staging of video blocks (FULL only) -----------------------
  // K rows (D*2 bytes) and V^T rows (UKB*2 bytes) land in LDS padded by 16 bytes;
  // each load instruction moves 64 pieces of 16 bytes to 64 consecutive LDS
  // slots, so the piece index e = 64*q + lane names (row, column) = divmod(e,
  // pieces per row); the padding column re-reads the row's first piece.
  constexpr int KPR = D / 8 + 1;             // pieces per padded K row
  constexpr int VPRp = UKB / 8 + 1;          // pieces per padded V^T row
  constexpr int NKI = UKB * KPR / 64;        // K instructions per block
  constexpr int NVI = D * VPRp / 64;         // V^T instructions per block
  constexpr int NLI = NKI + NVI;
  constexpr int NLW = (NLI + UNW - 1) / UNW; // instructions per wave (max)
  constexpr int NLMIN = NLI / UNW;           // instructions per wave (min)
  static_assert(UKB * KPR % 64 == 0 && D * VPRp % 64 == 0, "piece counts");
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  uint32_t dsrc[NLW];
  uint32_t dlds[NLW];
  bool disk[NLW], dok[NLW];
#pragma unroll
  for (int m = 0; m < NLW; ++m) {
    const int t = wv + UNW * m;
    dok[m] = t < NLI;
    disk[m] = t < NKI;
    const int q = disk[m] ? t : t - NKI;
    const int e = 64 * q + lane;
    if (disk[m]) {
      const int row = e / KPR, col = e % KPR;
      dsrc[m] = row * D * 2 + (col == KPR - 1 ? 0 : col * 16);
      dlds[m] = q * 1024;
    } else {
      const int row = e / VPRp, col = e % VPRp;
      dsrc[m] = row * g.S * 2 + (col == VPRp - 1 ? 0 : col * 16);
      dlds[m] = q * 1024;
    }
  }
  // issue this wave's loads of the block whose K rows start at kb and whose
  // V^T rows start at vb (bytes), into buffer buf
  // Buffer loads into LDS (buffer_load_lds16), one descriptor per KV head's K
  // rows and V^T rows; ko / vo are the block's byte offsets inside them.
  const int head_bytes = (int)((size_t)g.NS * D * 2);  // < 2^31 (checked at launch)
  void* const kbase = (void*)((const uint16_t*)a.k_cube + (size_t)grp * g.NS * D);
  void* const vbase = (void*)((const uint16_t*)a.v_cube + (size_t)grp * g.NS * D);
  auto issue = [&](uint32_t ko, uint32_t vo, auto bufc) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLW; ++m) {
      if (dok[m]) {
        if (disk[m])
          buffer_load_lds16(kbase, head_bytes, (char*)kbuf_c(bufc) + dlds[m], dsrc[m], ko);
        else
          buffer_load_lds16(vbase, head_bytes, (char*)vbuf_c(bufc) + dlds[m], dsrc[m], vo);
      }
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  // Four buffers, block b in buffer b % 4, one barrier per pair of blocks.
  // Blocks i, i+1 (i even) land while blocks i-2, i-1 are computed; at the
  // barrier before blocks i, i+1 every wave is done with blocks i-2, i-1, so
  // their buffers take blocks i+2, i+3.  The loop is unrolled over both
  // buffer pairs so that every buffer is named at compile time.
  // The union list and mask lookups run one pair ahead: at pair i the wave
  // reads the masks of blocks i+2, i+3 and the list entries of blocks i+4,
  // i+5, which it uses only at the next pair, so no LDS round trip sits
  // between the barrier and the first MFMA.  ul_read(i): list entry of block
  // i (any i; beyond the list it names an in-bounds stale entry, which is
  // never used to load); offs(i, ul, ko, vo): block i's byte offsets;
  // mask_read(ul): this wave's row mask of a list entry.
  auto dpipeline = [&](int nb, auto ul_read, auto offs, auto mask_read, auto work) __attribute__((always_inline)) {
    if (nb <= 0) return;
    __syncthreads();  // the previous phase no longer reads any buffer
    auto issue_ul = [&](int i, int ul, auto bufc) __attribute__((always_inline)) {
      if (i < nb) {
        uint32_t ko, vo;
        offs(i, ul, ko, vo);
        issue(ko, vo, bufc);
      }
    };
    const int ul0 = ul_read(0), ul1 = ul_read(1);
    int ua0 = ul_read(2), ua1 = ul_read(3);  // list entries of blocks i+2, i+3
    issue_ul(0, ul0, C0{});
    issue_ul(1, ul1, C1{});
    issue_ul(2, ua0, C2{});
    issue_ul(3, ua1, C3{});
    uint32_t mw0 = mask_read(ul0), mw1 = mask_read(ul1);  // masks of blocks i, i+1
    auto pair = [&](auto b0, auto b1, auto n0, auto n1, int i) __attribute__((always_inline)) {
      // blocks i, i+1 must have landed.  At i = 0 the loads of blocks 2 and 3
      // (those that exist) may stay in flight: a wave issues NLMIN or NLMIN+1
      // loads per block and loads complete in order, so allowing 2*NLMIN
      // pending loads (two blocks behind) or NLMIN (one block behind, nb == 3)
      // still covers every load of blocks 0 and 1.
      if (i == 0 && nb > 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NLMIN));
      else if (i == 0 && nb == 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NLMIN));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (i >= 2) {
        issue_ul(i + 2, ua0, n0);
        issue_ul(i + 3, ua1, n1);
      }
      const uint32_t nm0 = mask_read(ua0), nm1 = mask_read(ua1);
      const int nu0 = ul_read(i + 4), nu1 = ul_read(i + 5);
      work(i, kbuf_c(b0), vbuf_c(b0), kbuf_c(b1), vbuf_c(b1), mw0, i + 1 < nb ? mw1 : 0u);
      mw0 = nm0;
      mw1 = nm1;
      ua0 = nu0;
      ua1 = nu1;
    };
    for (int i = 0; i < nb; i += 4) {
      pair(C0{}, C1{}, C2{}, C3{}, i);
      if (i + 2 >= nb) break;
      pair(C2{}, C3{}, C0{}, C1{}, i + 2);
    }
  };

  const int nkb_cube = (g.S + UKB - 1) / UKB;
  const uint16_t* kg = (const uint16_t*)a.k_cube + (size_t)grp * g.NS * D;
  const uint16_t* vg = (const uint16_t*)a.v_cube + (size_t)grp * g.NS * D;  // [Nc][D][S] (ADAS_LAYOUT_VT)

  if constexpr (FULL) {
    // block buffers start zeroed, so a masked stand-in block reads finite values
    const uint4 z = make_uint4(0, 0, 0, 0);
    for (int e = tid; e < UKB * Sm::KS / 8; e += UNT) {
      reinterpret_cast<uint4*>(lk0)[e] = z;
      reinterpret_cast<uint4*>(lk1)[e] = z;
      reinterpret_cast<uint4*>(lk2)[e] = z;
      reinterpret_cast<uint4*>(lk3)[e] = z;
    }
    for (int e = tid; e < D * Sm::VS / 8; e += UNT) {
      reinterpret_cast<uint4*>(lv0)[e] = z;
      reinterpret_cast<uint4*>(lv1)[e] = z;
      reinterpret_cast<uint4*>(lv2)[e] = z;
      reinterpret_cast<uint4*>(lv3)[e] = z;
    }
  }

  // ---- causal text keys (extra rows of a text prefill), chunk 0 --------------------------
  if (!video && a.n_text_kv > 0 && chunk == 0) {
    const uint16_t* kt = (const uint16_t*)a.k_text + (size_t)grp * D;
    const uint16_t* vt = (const uint16_t*)a.v_text + (size_t)grp * D;
    pipeline(
        false, (a.n_text_kv + UKB - 1) / UKB,
        [&](int i, const uint16_t*& kp_, const uint16_t*& vp_, size_t& st_, int& kc_) __attribute__((always_inline)) {
          kp_ = kt + (size_t)i * UKB * g.Hkv * D;
          vp_ = vt + (size_t)i * UKB * g.Hkv * D;
          st_ = (size_t)g.Hkv * D;
          kc_ = min(UKB, a.n_text_kv - i * UKB);
        },
        [&](int i, int buf, int kc) __attribute__((always_inline)) {
          const bool sel = row_ok && pos >= i * UKB;
          if (__ballot(sel) != 0ull) compute(kMasked{}, kbuf_rt(buf), vbuf_rt(buf), sel, kc, true, i * UKB);
        });
  }

  // ---- selected cubes (video rows: and their own cubes) ---------------------------------
  // video rows: two threads per row walk the row's ascending list; the row's
  // own cube is one more bit of the same bitmap
  const int my_row = tid >> 1, my_half = tid & 1;
  const int32_t* my_list = nullptr;
  int my_cnt = 0, my_c = -1, my_lo = 0;
  if (video && my_row < n_rows) {
    const int rho = rho0 + my_row;
    const int ci = rho / (gsz * g.S);
    const int rem = rho - ci * gsz * g.S;
    const int slot = rem / g.S;
    const int hq2 = a.hg.heads[hstart + slot];
    const int r = rem - slot * g.S;
    my_c = g.Nc - 1 - ci;
    my_list = a.sel_idx + video_list_offset(a.capv, hq2, g.S, my_c, r);
    my_cnt = a.sel_count[(size_t)hq2 * a.rows_per_head + my_c * g.S + r];
  }
  int cube_lo, cube_hi;
  if (video) {
    cube_lo = 0;
    cube_hi = c + 1;
  } else {
    cube_lo = chunk * sc.extra_chunk_cubes;
    cube_hi = min(g.Nc, cube_lo + sc.extra_chunk_cubes);
  }
  // Passes and the cubes inside a pass run in descending order, so a video
  // row meets its own cube (the highest it attends) first and takes its
  // softmax reference there.
  const int n_pass = (cube_hi - cube_lo + UPASS - 1) / UPASS;
  for (int ps = n_pass - 1; ps >= 0; --ps) {
    const int jb = cube_lo + ps * UPASS;
    const int je = min(cube_hi, jb + UPASS);
    const int span = je - jb;
    __syncthreads();  // previous users of bits/ulist are done
    if (!video) {
      // extra rows: the selection bitmap (one word per 32 cubes, built before
      // this kernel) gives each (wave, cube) mask as one ballot over the
      // wave's 32 rows (lanes 0..31)
      const uint32_t* rbits = a.extra_bits + (size_t)(hq * a.n_extra + pos) * a.bits_words;
      for (int w0 = jb >> 5; w0 < (je + 31) >> 5; ++w0) {
        const uint32_t word = (row_ok && lh == 0) ? rbits[w0] : 0u;
        for (int bit = 0; bit < 32; ++bit) {
          const int u = 32 * w0 + bit - jb;
          const uint32_t m = (uint32_t)__ballot((word >> bit) & 1u);
          if (u >= 0 && u < span && lane == 0) s_bits[UNW * u + wave] = m;
        }
      }
    } else {
      for (int e = tid; e < span * UNW; e += UNT) s_bits[e] = 0u;
    }
    __syncthreads();
    if (video && my_row < n_rows) {
      // entries in [lo, lo2) lie in [jb, je) (lists are ascending).  Every
      // entry is below cube_hi and at least cube_lo = 0, and passes run
      // downwards, so a bound needs a binary search (dependent loads from
      // global memory) only inside the cube range: the upper one is the
      // previous pass's lower one.
      const int lo2 = je == cube_hi ? my_cnt : my_lo;
      int lo = 0;
      if (jb > cube_lo) {
        int hi = lo2;
        while (lo < hi) { const int mid = (lo + hi) >> 1; if (my_list[mid] < jb) lo = mid + 1; else hi = mid; }
      }
      my_lo = lo;
      const uint32_t bit = 1u << (my_row & 31);
      uint32_t* wbase = &s_bits[my_row >> 5];
      // eight list entries per thread in flight before their LDS updates
      for (int i0 = lo + my_half; i0 < lo2; i0 += 16) {
        int e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + 2 * u;
          e[u] = i < lo2 ? my_list[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (e[u] >= 0) atomicOr(wbase + UNW * (e[u] - jb), bit);
      }
      if (my_half == 0 && my_c >= jb && my_c < je) atomicOr(wbase + UNW * (my_c - jb), bit);
    }
    __syncthreads();
    if (wave == 0) {
      int base = 0;
      for (int u0 = 0; u0 < span; u0 += 64) {
        const int u = span - 1 - (u0 + lane);  // descending
        bool any = false;
        if (u >= 0) {
          uint32_t o = 0;
#pragma unroll
          for (int w = 0; w < UNW; ++w) o |= s_bits[UNW * u + w];
          any = o != 0u;
        }
        const uint64_t bal = __ballot(any);
        if (any) s_ulist[base + lanes_below(bal)] = (uint16_t)u;
        base += popc64(bal);
      }
      if (lane == 0) s_nunion = base;
    }
    __syncthreads();
    if constexpr (FULL) {
      const int nblk = s_nunion * nkb_cube;
      dpipeline(
          nblk,
          [&](int i) __attribute__((always_inline)) { return (int)s_ulist[min(i / nkb_cube, UPASS - 1)]; },
          [&](int i, int ul, uint32_t& ko, uint32_t& vo) __attribute__((always_inline)) {
            const int kbi = i - (i / nkb_cube) * nkb_cube;
            const int j = __builtin_amdgcn_readfirstlane(jb + ul);
            ko = (uint32_t)(((size_t)j * g.S + kbi * UKB) * D * 2);
            vo = (uint32_t)((size_t)j * g.S * D * 2 + kbi * UKB * 2);
          },
          [&](int ul) __attribute__((always_inline)) { return s_bits[UNW * min(ul, UPASS - 1) + wave]; },
          [&](int i, const uint16_t* kb0, const uint16_t* vb0, const uint16_t* kb1, const uint16_t* vb1,
              uint32_t mw0, uint32_t mw1) __attribute__((always_inline)) {
            // this wave's row masks of blocks i and i+1.  Every pair runs the
            // two-block path, with no skipping (in union tiles a wave whose 32
            // rows all pass over a block is rare): one code path keeps the
            // accumulators in place instead of copying them where paths meet.
            // An odd last block pairs with the other buffer's stale (finite,
            // zeroed at the start) contents, every row masked.  A wave that
            // holds no rows (possible in a head's last tile) skips every pair.
            if (!wave_has_rows) return;
            const bool sel0 = ((mw0 >> lr) & 1u) != 0u, sel1 = ((mw1 >> lr) & 1u) != 0u;
            block2(kb0, vb0, sel0, kb1, vb1, sel1);
          });
    } else {
    pipeline(
        true, s_nunion * nkb_cube,
        [&](int i, const uint16_t*& kp_, const uint16_t*& vp_, size_t& st_, int& kc_) __attribute__((always_inline)) {
          const int ci = i / nkb_cube, kb = i - ci * nkb_cube;
          const int j = jb + s_ulist[ci];
          const size_t off = ((size_t)j * g.S + kb * UKB) * D;
          kp_ = kg + off;
          vp_ = vg + (size_t)j * g.S * D + kb * UKB;
          st_ = D;
          kc_ = min(UKB, g.S - kb * UKB);
        },
        [&](int i, int buf, int kc) __attribute__((always_inline)) {
          const int ul = s_ulist[i / nkb_cube];
          const uint32_t mw = s_bits[UNW * ul + wave];
          if (mw == 0u) return;
          const bool sel = ((mw >> lr) & 1u) != 0u;
          if (FULL || kc == UKB) compute(kFull{}, kbuf_rt(buf), vbuf_rt(buf), sel, kc, false, 0);
          else compute(kMasked{}, kbuf_rt(buf), vbuf_rt(buf), sel, kc, false, 0);
        });
    }
  }

  // ---- epilogue ----------------------------------------------------------------------
  if (!row_ok) return;
  // acc[db][i] = O^T[d = 32*db + 8*(i/4) + 4*lh + (i%4)][row]
  if (!video && sc.extra_chunks > 1) {
    float* dst = a.partials + ((size_t)tile_e * sc.extra_chunks + chunk) * UTR * (D + 2) +
                 (size_t)t_row * (D + 2);
    if (lh == 0) {
      dst[0] = m_run;
      dst[1] = l_run;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float* p = dst + 2 + 32 * db + 8 * q + 4 * lh;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = acc[db][4 * q + e];
      }
    return;
  }
  const float inv = 1.0f / l_run;
  if (a.lse != nullptr && lh == 0)
    a.lse[(size_t)hq * a.rows_per_head + (video ? pos : (a.has_video ? g.N : 0) + pos)] =
        (m_run + __log2f(l_run)) * 0.69314718055994531f;
  uint16_t* dst;
  if (video) {
    const int cr = pos / g.S;
    const int n = raster_of(g, cr, pos - cr * g.S);
    dst = (uint16_t*)a.out_raster + ((size_t)n * g.Hq + hq) * D;
  } else {
    dst = (uint16_t*)a.out_extra + ((size_t)pos * g.Hq + hq) * D;
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x4u o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[db][4 * q + e] * inv);
      *reinterpret_cast<bf16x4u*>(dst + 32 * db + 8 * q + 4 * lh) = o4;
    }
}

template <int D>
hipError_t launch_union(const AttnArgs& a, hipStream_t s) {
  USched sc;
  sc.video_tiles_per_group = a.has_video ? (int)(((long)a.hg.gmax * a.g.N + UTR - 1) / UTR) : 0;
  sc.extra_tiles_per_group = a.extra_tiles_per_group;
  sc.extra_chunks = a.extra_chunks;
  sc.extra_chunk_cubes = a.extra_chunk_cubes;
  sc.n_extra_wgs = a.g.Hkv * sc.extra_tiles_per_group * sc.extra_chunks;
  sc.xcd_mode = (8 % a.g.Hkv) == 0 ? 1 : 0;
  long video_blocks = 0;
  if (a.has_video) {
    if (sc.xcd_mode) {
      const int per = 8 / a.g.Hkv;  // XCDs serving one KV head
      video_blocks = 8L * ((sc.video_tiles_per_group + per - 1) / per);
    } else {
      video_blocks = (long)a.g.Hkv * sc.video_tiles_per_group;
    }
  }
  const long blocks = sc.n_extra_wgs + video_blocks;
  // buffer descriptors address one KV head's K (or V^T) rows with 32-bit offsets
  if ((size_t)a.g.NS * D * 2 > 0x7fffffffu) return hipErrorInvalidValue;
  if (blocks > 0) {
    if (a.g.S % UKB == 0)
      hipLaunchKernelGGL((k_attn_union<D, true>), dim3((unsigned)blocks), dim3(UNT), 0, s, a, sc);
    else
      hipLaunchKernelGGL((k_attn_union<D, false>), dim3((unsigned)blocks), dim3(UNT), 0, s, a, sc);
  }
  return hipGetLastError();
}

template hipError_t launch_union<128>(const AttnArgs&, hipStream_t);
template hipError_t launch_union<64>(const AttnArgs&, hipStream_t);

}  // namespace adas
