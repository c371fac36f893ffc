// Attention for extra rows that fit one wave: decode steps (AdaSpark,
// papernotes.org, key design 2; a decode query attends to its Top-p cube set
// only).  When a KV head's extra rows number at most 32 (e.g. one decode token
// x 7 query heads), the bf16 path uses this kernel instead of union tiles.
//
// One workgroup (4 waves) per (KV head, chunk of cubes).  Every wave holds the
// same <= 32 rows (query operand and float32 accumulators in registers) and
// walks its own cubes of the chunk (cube c0 + wave, + 4, ...), skipping cubes no
// row selected.  Each wave owns one LDS block buffer: a key block (64 keys of
// K rows and V^T rows, values in ADAS_LAYOUT_VT) arrives there by buffer
// loads into LDS in 1 KB contiguous pieces, then feeds the MFMAs with
// the same conflict-free b128 fragment reads as the union kernel.  Waves share
// no data while they walk their cubes, so there is no barrier in the loop; the
// four waves of a CU overlap one another's loads and math.  At the end the
// waves' (max, sum, outputs) states are merged in LDS into one partial row per
// (chunk, row), and k_merge_bf16 combines the chunks.
#include "common.h"

namespace adas {

namespace {
typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));
typedef float df32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 dbf16x2 __attribute__((ext_vector_type(2)));
constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLazyD = 8.0f;  // rescale only when a block max exceeds the reference by 2^8
constexpr int DW = 4;           // waves per workgroup
constexpr int DMAXL = 128;      // cubes per wave and chunk (list capacity)
}  // namespace

int decode_waves() { return DW; }
int decode_max_chunk_cubes() { return DW * DMAXL; }

// Requires S % 64 == 0 and at most 32 rows per KV head (host checks).
template <int D>
__global__ __launch_bounds__(64 * DW, 1) void k_attn_decode(AttnArgs a) {
  const KGeom& g = a.g;
  const int n_chunks = a.decode_chunks;
  const int grp = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - grp * n_chunks;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int hstart = a.hg.start[grp];
  const int n_rows = (a.hg.start[grp + 1] - hstart) * a.n_extra;
  const bool row_ok = lr < n_rows;
  int hq = 0, m = 0;
  if (row_ok) {
    const int slot = lr / a.n_extra;
    hq = a.hg.heads[hstart + slot];
    m = lr - slot * a.n_extra;
  }
  dbf16x8 qb[D / 16];
  {
    const uint16_t* src = (const uint16_t*)a.q_extra + ((size_t)m * g.Hq + hq) * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *reinterpret_cast<const uint4*>(src + 16 * ds + 8 * lh);
      qb[ds] = __builtin_bit_cast(dbf16x8, v);
    }
  }
  const float qscale = kLog2eD / sqrtf((float)D);
  const dbf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float m_run = -INFINITY, l_run = 0.f;
  df32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // this wave's LDS block: K rows (D + 8 bf16) then V^T rows (64 + 8 bf16)
  constexpr int KS = D + 8, VS = 64 + 8;
  constexpr int KPR = D / 8 + 1;             // 16-byte pieces per padded K row
  constexpr int VPR = 64 / 8 + 1;            // pieces per padded V^T row
  constexpr int NKI = 64 * KPR / 64;         // K load instructions per block
  constexpr int NVI = D * VPR / 64;          // V^T load instructions per block
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[DW][64 * KS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[DW][D * VS];
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint16_t* mk = lds_k[wv];
  uint16_t* mv = lds_v[wv];

  const uint32_t* rbits = a.extra_bits + (size_t)(hq * a.n_extra + m) * a.bits_words;
  const int head_bytes = (int)((size_t)g.NS * D * 2);  // < 2^31 (checked at launch)
  void* const kg = (void*)((const uint16_t*)a.k_cube + (size_t)grp * g.NS * D);
  void* const vg = (void*)((const uint16_t*)a.v_cube + (size_t)grp * g.NS * D);  // [Nc][D][S]
  const int c0 = chunk * a.extra_chunk_cubes;
  const int c1 = min(g.Nc, c0 + a.extra_chunk_cubes);
  // This wave's cubes (c0 + wave, + DW, ...) that some row selected, with the
  // rows that selected them, listed in LDS private to the wave.
  __shared__ uint32_t s_cube[DW][DMAXL], s_rmask[DW][DMAXL];
  int n_list = 0;
  for (int j = c0 + wv; j < c1; j += DW) {
    const uint32_t bit = (row_ok && lh == 0) ? (rbits[j >> 5] >> (j & 31)) & 1u : 0u;
    const uint32_t mask = (uint32_t)__ballot(bit != 0u);  // rows of the wave that selected j
    if (mask != 0u) {
      if (lane == 0) {
        s_cube[wv][n_list] = (uint32_t)j;
        s_rmask[wv][n_list] = mask;
      }
      ++n_list;
    }
  }
  // Key blocks b = (list entry b / nkbc, block b % nkbc of its cube).  K and
  // V^T of block b + 1 are loaded while block b computes: K(b+1) as soon as the
  // score MFMAs have read K(b), V^T(b+1) once the output MFMAs have read
  // V^T(b).  Loads into LDS return in order, so "at most NVI loads pending"
  // after K(b), V(b) were issued means K(b) has landed, and "at most NKI
  // pending" after K(b+1) was issued means V(b) has landed.
  const int nkbc = g.S / 64;
  const int nb = n_list * nkbc;
  auto block_offsets = [&](int b, uint32_t& ko, uint32_t& vo) __attribute__((always_inline)) {
    const int e = b / nkbc, kb = (b - e * nkbc) * 64;
    const int j = __builtin_amdgcn_readfirstlane((int)s_cube[wv][e]);  // wave-uniform: scalar offsets
    ko = (uint32_t)(((size_t)j * g.S + kb) * D * 2);
    vo = (uint32_t)((size_t)j * g.S * D * 2 + kb * 2);
  };
  // piece e = 64*q + lane of the padded block; the padding column re-reads
  // the row's first piece
  auto issue_k = [&](uint32_t ko) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NKI; ++q) {
      const int e = 64 * q + lane;
      const int row = e / KPR, col = e % KPR;
      buffer_load_lds16(kg, head_bytes, (char*)mk + 1024 * q, row * D * 2 + (col == KPR - 1 ? 0 : col * 16), ko);
    }
  };
  auto issue_v = [&](uint32_t vo) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NVI; ++q) {
      const int e = 64 * q + lane;
      const int row = e / VPR, col = e % VPR;
      buffer_load_lds16(vg, head_bytes, (char*)mv + 1024 * q, row * g.S * 2 + (col == VPR - 1 ? 0 : col * 16), vo);
    }
  };
  if (nb > 0) {
    uint32_t ko, vo;
    block_offsets(0, ko, vo);
    issue_k(ko);
    issue_v(vo);
  }
  for (int b = 0; b < nb; ++b) {
    const bool rowsel = ((s_rmask[wv][b / nkbc] >> lr) & 1u) != 0u;
    const bool has_next = b + 1 < nb;
    uint32_t kon = 0, von = 0;
    if (has_next) block_offsets(b + 1, kon, von);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NVI));  // K(b) is in LDS
    {
      // S^T = K Q^T; keys of st[h2][i]: 32*h2 + 8*(i/4) + 4*lh + (i%4)
      df32x16 st[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) st[h2][i] = 0.f;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
          const dbf16x8 ka = __builtin_bit_cast(
              dbf16x8, *reinterpret_cast<const uint4*>(&mk[(32 * h2 + lr) * KS + 16 * ds + 8 * lh]));
          st[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[ds], st[h2], 0, 0, 0);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the K fragments are read
      if (has_next) issue_k(kon);
      // online softmax in log2 units with lazy rescaling
      float mb = fmaxf(st[0][0], st[1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mb = fmaxf(fmaxf(mb, st[0][i]), st[1][i]);
      mb = fmaxf(mb, xor32_f32(mb));
      const float mb_c = rowsel ? mb * qscale : -INFINITY;
      const bool grow = mb_c > m_run + kLazyD;
      if (__ballot(grow) != 0ull) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mb_c) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        m_run = grow ? mb_c : m_run;
      }
      const float bias = (rowsel && m_run != -INFINITY) ? m_run : INFINITY;
      dbf16x8 pb[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pb[2 * h2 + i / 8][i % 8] = (__bf16)__builtin_amdgcn_exp2f(fmaf(st[h2][i], qscale, -bias));
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const dbf16x2 pair = {pb[u][2 * e], pb[u][2 * e + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, ls, false);
        }
      ls += xor32_f32(ls);
      l_run += ls;
      if (has_next) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NKI));  // V^T(b) is in LDS
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      // O^T += V^T P^T; slot 8*lh + e of k-step u holds key 16*u + 8*(e/4) + 4*lh + (e%4),
      // kept by ADAS_LAYOUT_VT in column 16*u + 8*lh + e
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const dbf16x8 va = __builtin_bit_cast(
              dbf16x8, *reinterpret_cast<const uint4*>(&mv[(32 * db + lr) * VS + 16 * u + 8 * lh]));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[u], acc[db], 0, 0, 0);
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the V^T fragments are read
      if (has_next) issue_v(von);
    }
  }
  // The four waves' states are merged in LDS (the block buffers are free now)
  // into one partial row per (KV head, chunk): [grp][chunk][32 rows][D + 2].
  constexpr int RS = D + 2;
  static_assert(DW * 32 * RS * 4 <= DW * (64 * KS + D * VS) * 2, "merge area fits the block buffers");
  static_assert(NKI < 64 && NVI < 64, "vmcnt range");
  float* red = reinterpret_cast<float*>(&lds_k[0][0]);  // [wave][row][RS], spans lds_k then lds_v
  __syncthreads();  // every wave is done with its block buffer
  if (row_ok) {
    float* r = red + ((size_t)wave * 32 + lr) * RS;
    if (lh == 0) {
      r[0] = m_run;
      r[1] = l_run;
    }
    // acc[db][i] = O^T[d = 32*db + 8*(i/4) + 4*lh + (i%4)][row]
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) r[2 + 32 * db + 8 * q + 4 * lh + e] = acc[db][4 * q + e];
  }
  __syncthreads();
  // thread t: row t / 8, output dims 16*(t % 8) .. +16 (D = 128) or 8*(t % 8) .. +8 (D = 64)
  constexpr int PD = D / 8;
  const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
  if (row >= n_rows) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < DW; ++w) M = fmaxf(M, red[((size_t)w * 32 + row) * RS]);
  float L = 0.f, o[PD] = {};
#pragma unroll
  for (int w = 0; w < DW; ++w) {
    const float* r = red + ((size_t)w * 32 + row) * RS;
    const float wgt = r[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(r[0] - M);
    L = fmaf(wgt, r[1], L);
#pragma unroll
    for (int i = 0; i < PD; ++i) o[i] = fmaf(wgt, r[2 + PD * part + i], o[i]);
  }
  float* dst = a.partials + (((size_t)grp * a.extra_chunks + chunk) * 32 + row) * RS;
  if (part == 0) {
    dst[0] = M;
    dst[1] = L;
  }
#pragma unroll
  for (int i = 0; i < PD; ++i) dst[2 + PD * part + i] = o[i];
}

hipError_t launch_decode(const AttnArgs& a, hipStream_t s) {
  // buffer descriptors address one KV head's rows with 32-bit offsets
  if ((size_t)a.g.NS * a.g.D * 2 > 0x7fffffffu) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.g.Hkv * a.decode_chunks));
  if (a.g.D == 128)
    hipLaunchKernelGGL((k_attn_decode<128>), grid, dim3(64 * DW), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_decode<64>), grid, dim3(64 * DW), 0, s, a);
  return hipGetLastError();
}

}  // namespace adas
