// Backward of the sparse attention: launch arguments, workspace layout and
// host entry points (kernels in attn_bwd.hip).
#pragma once

#include "common.h"

namespace adas {

struct BwdArgs {
  KGeom g;
  HeadGroups hg;
  const uint16_t* q_cube;       // [Hq][NS][D] or null (no video rows)
  const uint16_t* q_extra;      // [n_extra][Hq][D]
  const uint16_t* k_cube;       // [Hkv][NS][D] (ADAS_LAYOUT_TOKENS)
  const uint16_t* v_tok;        // [Hkv][NS][D] V in ADAS_LAYOUT_TOKENS
  const uint16_t* k_vt;         // [Hkv][NS/S][D][S] K in ADAS_LAYOUT_VT
  const uint16_t* out_raster;   // forward outputs
  const uint16_t* out_extra;
  const uint16_t* dout_raster;  // their gradients
  const uint16_t* dout_extra;
  const float* lse;             // [Hq][rows_per_head] natural log-sum-exp
  const int32_t* sel_count;
  const int32_t* sel_idx;
  float* dq_raster;             // [N][Hq][D]
  float* dq_extra;              // [n_extra][Hq][D]
  float* dk_raster;             // [N][Hkv][D]
  float* dv_raster;             // [N][Hkv][D]
  const uint16_t* k_text;       // [n_text_kv][Hkv][D] causal text keys of a text prefill (or null)
  const uint16_t* v_text;
  float* dk_text;               // [n_text_kv][Hkv][D]
  float* dv_text;
  int n_text_kv;                // 0, or n_extra: text row m attends text tokens 0..m
  // workspace
  float* delta;                 // [Hq][rows_per_head]: do . o
  uint32_t* bits;               // [Hq][W][rows_per_head]: selection bitmap, word-major
  int32_t* list_count;          // [Hkv][Nc]
  int32_t* lists;               // per (KV head, cube): rows attending it (hq * rows_per_head + row)
  int W;
  int n_extra;
  int64_t capv;
  int rows_per_head;
  int has_video;
  int64_t list_cap_g;           // list entries per KV head
  int video_tiles_per_group, extra_tiles_per_group, n_extra_tiles;
};
// first entry of the row list of (KV head grp, cube j): each cube has room for
// every row of the largest head group that could attend it
__host__ __device__ inline int64_t list_offset(const BwdArgs& a, int grp, int j) {
  const int64_t hv = a.has_video ? 1 : 0;
  return (int64_t)grp * a.list_cap_g +
         (int64_t)a.hg.gmax * (hv * a.g.S * ((int64_t)j * a.g.Nc - (int64_t)j * (j - 1) / 2) + (int64_t)j * a.n_extra);
}
void plan_backward(BwdArgs& a);
size_t backward_workspace_bytes(const BwdArgs& a);
void bind_backward_workspace(BwdArgs& a, void* ws);
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);

}  // namespace adas
