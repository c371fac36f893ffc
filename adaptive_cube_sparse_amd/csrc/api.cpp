// Host side of the libadas C ABI: argument validation, geometry derivation,
// workspace sizing and kernel launch selection.  Nothing here touches device
// memory contents; every check runs before any launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "adas.h"
#include "adas_ffn.h"
#include "attn_bwd.h"
#include "common.h"
#include "ffn.h"

namespace {

thread_local char g_last_error[512] = "";

adas_status fail(adas_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

adas_status ok() {
  g_last_error[0] = '\0';
  return ADAS_OK;
}

// Validate the geometry and derive the kernel view plus head groups.
adas_status derive(const adas_geom* geom, adas::KGeom& g, adas::HeadGroups& hg) {
  if (geom == nullptr) return fail(ADAS_ERR_NULL, "geom is NULL");
  const adas_geom& s = *geom;
  if (s.T <= 0 || s.H <= 0 || s.W <= 0 || s.ct <= 0 || s.ch <= 0 || s.cw <= 0)
    return fail(ADAS_ERR_SHAPE, "grid and cube extents must be positive");
  if (s.T % s.ct || s.H % s.ch || s.W % s.cw)
    return fail(ADAS_ERR_SHAPE, "cube %dx%dx%d (t,h,w) does not divide grid %dx%dx%d", s.ct, s.ch,
                s.cw, s.T, s.H, s.W);
  const long long N = (long long)s.T * s.H * s.W;
  if (N > (1LL << 30)) return fail(ADAS_ERR_SHAPE, "too many tokens (%lld)", N);
  if (s.head_dim != 64 && s.head_dim != 128)
    return fail(ADAS_ERR_SHAPE, "head_dim must be 64 or 128 (got %d)", s.head_dim);
  if (s.n_q_heads <= 0 || s.n_kv_heads <= 0 || s.n_q_heads > ADAS_MAX_HEADS ||
      s.n_kv_heads > ADAS_MAX_HEADS)
    return fail(ADAS_ERR_SHAPE, "head counts must be in [1, %d]", ADAS_MAX_HEADS);
  g.T = s.T; g.H = s.H; g.W = s.W;
  g.ct = s.ct; g.ch = s.ch; g.cw = s.cw;
  g.nT = s.T / s.ct; g.nH = s.H / s.ch; g.nW = s.W / s.cw;
  g.N = (int)N;
  g.S = s.ct * s.ch * s.cw;
  g.Nc = g.nT * g.nH * g.nW;
  g.Hq = s.n_q_heads;
  g.Hkv = s.n_kv_heads;
  g.D = s.head_dim;
  if (s.cache_T != 0 && (s.cache_T < s.T || s.cache_T % s.ct))
    return fail(ADAS_ERR_SHAPE, "cache_T (%d) must be 0 or a multiple of ct (%d) that is >= T (%d)", s.cache_T,
                s.ct, s.T);
  const long long NS = (long long)(s.cache_T ? s.cache_T : s.T) * s.H * s.W;
  if (NS > (1LL << 30)) return fail(ADAS_ERR_SHAPE, "cache too large (%lld tokens)", NS);
  g.NS = (int)NS;
  int map[ADAS_MAX_HEADS];
  if (s.head_map == nullptr) {
    if (s.n_q_heads % s.n_kv_heads)
      return fail(ADAS_ERR_SHAPE, "n_kv_heads (%d) must divide n_q_heads (%d) without head_map",
                  s.n_kv_heads, s.n_q_heads);
    const int rep = s.n_q_heads / s.n_kv_heads;
    for (int h = 0; h < s.n_q_heads; ++h) map[h] = h / rep;
  } else {
    for (int h = 0; h < s.n_q_heads; ++h) {
      map[h] = s.head_map[h];
      if (map[h] < 0 || map[h] >= s.n_kv_heads)
        return fail(ADAS_ERR_VALUE, "head_map[%d] = %d out of range [0, %d)", h, map[h],
                    s.n_kv_heads);
    }
  }
  int k = 0;
  hg.gmax = 0;
  for (int gg = 0; gg < s.n_kv_heads; ++gg) {
    hg.start[gg] = (int16_t)k;
    for (int h = 0; h < s.n_q_heads; ++h)
      if (map[h] == gg) hg.heads[k++] = (uint8_t)h;
    const int sz = k - hg.start[gg];
    if (sz > hg.gmax) hg.gmax = sz;
  }
  hg.start[s.n_kv_heads] = (int16_t)k;
  return ADAS_OK;
}

adas_status check_dtype(adas_dtype dt) {
  if (dt != ADAS_BF16 && dt != ADAS_F32) return fail(ADAS_ERR_DTYPE, "unknown dtype %d", (int)dt);
  return ADAS_OK;
}

adas_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ADAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int64_t capv_of(const adas::KGeom& g, bool has_video) {
  return has_video ? (int64_t)g.S * g.Nc * (g.Nc - 1) / 2 : 0;
}

int64_t capacity_of(const adas::KGeom& g, bool has_video, int n_extra) {
  return (int64_t)g.Hq * capv_of(g, has_video) + (int64_t)g.Hq * n_extra * g.Nc;
}

}  // namespace

extern "C" {

adas_status adas_cube_partition(const adas_geom* geom, adas_dtype dtype, int32_t n_heads,
                                adas_layout layout, const void* x_raster, void* x_cube,
                                int32_t* perm, void* stream) {
  adas::KGeom g;
  adas::HeadGroups hg;
  adas_status st = derive(geom, g, hg);
  if (st != ADAS_OK) return st;
  if ((st = check_dtype(dtype)) != ADAS_OK) return st;
  if (layout != ADAS_LAYOUT_TOKENS && layout != ADAS_LAYOUT_VT)
    return fail(ADAS_ERR_VALUE, "layout must be ADAS_LAYOUT_TOKENS or ADAS_LAYOUT_VT");
  if (x_raster == nullptr || x_cube == nullptr) return fail(ADAS_ERR_NULL, "x_raster/x_cube is NULL");
  if (n_heads <= 0 || n_heads > ADAS_MAX_HEADS)
    return fail(ADAS_ERR_SHAPE, "n_heads must be in [1, %d]", ADAS_MAX_HEADS);
  const int eb = dtype == ADAS_BF16 ? 2 : 4;
  return hip_status(adas::launch_partition(g, eb, n_heads, layout == ADAS_LAYOUT_VT, x_raster,
                                           x_cube, perm, (hipStream_t)stream),
                    "adas_cube_partition launch");
}

adas_status adas_cube_mean_keys(const adas_geom* geom, adas_dtype dtype, const void* k_cube,
                                float* kbar, void* stream) {
  adas::KGeom g;
  adas::HeadGroups hg;
  adas_status st = derive(geom, g, hg);
  if (st != ADAS_OK) return st;
  if ((st = check_dtype(dtype)) != ADAS_OK) return st;
  if (k_cube == nullptr || kbar == nullptr) return fail(ADAS_ERR_NULL, "k_cube/kbar is NULL");
  return hip_status(adas::launch_mean_keys(g, dtype, k_cube, kbar, (hipStream_t)stream),
                    "adas_cube_mean_keys launch");
}

adas_status adas_cube_partition_keys(const adas_geom* geom, adas_dtype dtype, const void* k_raster,
                                     void* k_cube, int32_t* perm, float* kbar, void* stream) {
  adas::KGeom g;
  adas::HeadGroups hg;
  adas_status st = derive(geom, g, hg);
  if (st != ADAS_OK) return st;
  if ((st = check_dtype(dtype)) != ADAS_OK) return st;
  if (k_raster == nullptr || k_cube == nullptr || kbar == nullptr)
    return fail(ADAS_ERR_NULL, "k_raster/k_cube/kbar is NULL");
  return hip_status(adas::launch_partition_keys(g, dtype, k_raster, k_cube, perm, kbar, (hipStream_t)stream),
                    "adas_cube_partition_keys launch");
}

// Shared body of adas_select_topp / adas_select_topk (topk > 0 selects Top-K).
static adas_status select_common(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                 int32_t n_extra, const void* q_extra, const float* kbar, float p,
                                 int32_t topk, int32_t* sel_count, int32_t* sel_idx,
                                 int64_t sel_cap, void* ws, size_t ws_bytes, void* stream,
                                 const char* name) {
  adas::KGeom g;
  adas::HeadGroups hg;
  adas_status st = derive(geom, g, hg);
  if (st != ADAS_OK) return st;
  if ((st = check_dtype(dtype)) != ADAS_OK) return st;
  if (topk == 0 && !(p > 0.0f && p <= 1.0f))
    return fail(ADAS_ERR_VALUE, "p must be in (0, 1] (got %g)", (double)p);
  if (topk < 0) return fail(ADAS_ERR_VALUE, "k must be >= 1 (got %d)", topk);
  if (n_extra < 0) return fail(ADAS_ERR_SHAPE, "n_extra must be >= 0");
  if (q_cube == nullptr && n_extra == 0) return fail(ADAS_ERR_SHAPE, "no query rows");
  if (n_extra > 0 && q_extra == nullptr) return fail(ADAS_ERR_NULL, "q_extra is NULL");
  if (kbar == nullptr || sel_count == nullptr || sel_idx == nullptr)
    return fail(ADAS_ERR_NULL, "kbar/sel_count/sel_idx is NULL");
  if (g.Nc > ADAS_MAX_CUBES)
    return fail(ADAS_ERR_SHAPE, "%d cubes exceed the selection limit %d", g.Nc, ADAS_MAX_CUBES);
  const bool has_video = q_cube != nullptr;
  const int64_t need = capacity_of(g, has_video, n_extra);
  if (sel_cap < need)
    return fail(ADAS_ERR_CAPACITY, "sel_cap %lld < required %lld", (long long)sel_cap,
                (long long)need);
  const size_t ws_need = adas::select_workspace_bytes(g, dtype, n_extra, hg.gmax);
  if (ws_need > 0 && (ws == nullptr || ws_bytes < ws_need))
    return fail(ADAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, ws_need);
  adas::SelectArgs a{};
  a.g = g;
  a.zbuf = (float*)ws;
  a.hg = hg;
  a.q_cube = q_cube;
  a.q_extra = q_extra;
  a.kbar = kbar;
  a.n_extra = n_extra;
  a.p = topk > 0 ? 1.0f : p;
  a.topk = topk;
  a.sel_count = sel_count;
  a.sel_idx = sel_idx;
  a.capv = capv_of(g, has_video);
  a.rows_per_head = (has_video ? g.N : 0) + n_extra;
  a.has_video = has_video;
  return hip_status(adas::launch_select(a, dtype, (hipStream_t)stream), name);
}

adas_status adas_select_topp(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                             int32_t n_extra, const void* q_extra, const float* kbar, float p,
                             int32_t* sel_count, int32_t* sel_idx, int64_t sel_cap, void* ws,
                             size_t ws_bytes, void* stream) {
  return select_common(geom, dtype, q_cube, n_extra, q_extra, kbar, p, 0, sel_count, sel_idx,
                       sel_cap, ws, ws_bytes, stream, "adas_select_topp launch");
}

adas_status adas_select_topk(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                             int32_t n_extra, const void* q_extra, const float* kbar, int32_t k,
                             int32_t* sel_count, int32_t* sel_idx, int64_t sel_cap, void* ws,
                             size_t ws_bytes, void* stream) {
  if (k < 1) return fail(ADAS_ERR_VALUE, "k must be >= 1 (got %d)", k);
  return select_common(geom, dtype, q_cube, n_extra, q_extra, kbar, 1.0f, k, sel_count, sel_idx,
                       sel_cap, ws, ws_bytes, stream, "adas_select_topk launch");
}

static adas_status build_attn(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                              int32_t n_extra, int32_t n_text_kv, adas::AttnArgs& a) {
  a = adas::AttnArgs{};
  adas_status st = derive(geom, a.g, a.hg);
  if (st != ADAS_OK) return st;
  if ((st = check_dtype(dtype)) != ADAS_OK) return st;
  if (n_extra < 0) return fail(ADAS_ERR_SHAPE, "n_extra must be >= 0");
  if (n_text_kv != 0 && n_text_kv != n_extra)
    return fail(ADAS_ERR_SHAPE, "n_text_kv must be 0 or n_extra (%d), got %d", n_extra, n_text_kv);
  if (q_cube == nullptr && n_extra == 0) return fail(ADAS_ERR_SHAPE, "no query rows");
  if (a.g.Nc > ADAS_MAX_CUBES)  // selection lists exist only up to this many cubes
    return fail(ADAS_ERR_SHAPE, "%d cubes exceed the limit %d", a.g.Nc, ADAS_MAX_CUBES);
  a.has_video = q_cube != nullptr;
  a.n_extra = n_extra;
  a.n_text_kv = n_text_kv;
  a.capv = capv_of(a.g, a.has_video);
  a.rows_per_head = (a.has_video ? a.g.N : 0) + n_extra;
  adas::plan_attention(a, dtype);
  return ADAS_OK;
}

static adas_status attn_fwd(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                            const void* k_cube, const void* v_cube, int32_t n_extra,
                            int32_t n_text_kv, const void* q_extra, const void* k_text,
                            const void* v_text, const int32_t* sel_count,
                            const int32_t* sel_idx, void* out_raster, void* out_extra,
                            float* lse, void* ws, size_t ws_bytes, void* stream) {
  adas::AttnArgs a;
  adas_status st = build_attn(geom, dtype, q_cube, n_extra, n_text_kv, a);
  if (st != ADAS_OK) return st;
  if (k_cube == nullptr || v_cube == nullptr || sel_count == nullptr || sel_idx == nullptr)
    return fail(ADAS_ERR_NULL, "k_cube/v_cube/sel_count/sel_idx is NULL");
  if (q_cube != nullptr && out_raster == nullptr) return fail(ADAS_ERR_NULL, "out_raster is NULL");
  if (n_extra > 0 && (q_extra == nullptr || out_extra == nullptr))
    return fail(ADAS_ERR_NULL, "q_extra/out_extra is NULL");
  if (n_text_kv > 0 && (k_text == nullptr || v_text == nullptr))
    return fail(ADAS_ERR_NULL, "k_text/v_text is NULL");
  const size_t need = adas::attention_workspace_bytes(a, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(ADAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  a.q_cube = q_cube;
  a.k_cube = k_cube;
  a.v_cube = v_cube;
  a.q_extra = q_extra;
  a.k_text = k_text;
  a.v_text = v_text;
  a.sel_count = sel_count;
  a.sel_idx = sel_idx;
  a.out_raster = out_raster;
  a.out_extra = out_extra;
  a.lse = lse;
  adas::bind_attention_workspace(a, dtype, ws);
  return hip_status(adas::launch_attention(a, dtype, (hipStream_t)stream),
                    "adas_sparse_attn_fwd launch");
}


adas_status adas_sparse_attn_fwd(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                 const void* k_cube, const void* v_cube, int32_t n_extra,
                                 int32_t n_text_kv, const void* q_extra, const void* k_text,
                                 const void* v_text, const int32_t* sel_count,
                                 const int32_t* sel_idx, void* out_raster, void* out_extra,
                                 void* ws, size_t ws_bytes, void* stream) {
  return attn_fwd(geom, dtype, q_cube, k_cube, v_cube, n_extra, n_text_kv, q_extra, k_text, v_text,
                  sel_count, sel_idx, out_raster, out_extra, nullptr, ws, ws_bytes, stream);
}

adas_status adas_sparse_attn_fwd_lse(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                     const void* k_cube, const void* v_cube, int32_t n_extra,
                                     int32_t n_text_kv, const void* q_extra, const void* k_text,
                                     const void* v_text, const int32_t* sel_count,
                                     const int32_t* sel_idx, void* out_raster, void* out_extra,
                                     float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (lse == nullptr) return fail(ADAS_ERR_NULL, "lse is NULL");
  return attn_fwd(geom, dtype, q_cube, k_cube, v_cube, n_extra, n_text_kv, q_extra, k_text, v_text,
                  sel_count, sel_idx, out_raster, out_extra, lse, ws, ws_bytes, stream);
}

// Workspace of adas_decode_step: the attention's part first, then the
// selection's at a 256-byte aligned offset.
static adas_status decode_plan(const adas_geom* geom, adas_dtype dtype, int32_t n_extra, adas::AttnArgs& a,
                               size_t& attn_bytes, size_t& sel_off, size_t& total) {
  if (n_extra < 1) return fail(ADAS_ERR_SHAPE, "n_extra must be >= 1 (got %d)", n_extra);
  adas_status st = build_attn(geom, dtype, nullptr, n_extra, 0, a);
  if (st != ADAS_OK) return st;
  attn_bytes = adas::attention_workspace_bytes(a, dtype);
  sel_off = (attn_bytes + 255) & ~(size_t)255;
  total = sel_off + adas::select_workspace_bytes(a.g, dtype, n_extra, a.hg.gmax);
  return ADAS_OK;
}

adas_status adas_decode_step(const adas_geom* geom, adas_dtype dtype, int32_t n_extra, const void* q_extra,
                             const float* kbar, const void* k_cube, const void* v_cube, float p,
                             int32_t* sel_count, int32_t* sel_idx, int64_t sel_cap, void* out_extra,
                             void* ws, size_t ws_bytes, void* stream) {
  adas::AttnArgs a;
  size_t attn_bytes = 0, sel_off = 0, need = 0;
  adas_status st = decode_plan(geom, dtype, n_extra, a, attn_bytes, sel_off, need);
  if (st != ADAS_OK) return st;
  if (!(p > 0.0f && p <= 1.0f)) return fail(ADAS_ERR_VALUE, "p must be in (0, 1] (got %g)", (double)p);
  if (q_extra == nullptr || kbar == nullptr || k_cube == nullptr || v_cube == nullptr || sel_count == nullptr ||
      sel_idx == nullptr || out_extra == nullptr)
    return fail(ADAS_ERR_NULL, "q_extra/kbar/k_cube/v_cube/sel_count/sel_idx/out_extra is NULL");
  const int64_t cap = capacity_of(a.g, false, n_extra);
  if (sel_cap < cap)
    return fail(ADAS_ERR_CAPACITY, "sel_cap %lld < required %lld", (long long)sel_cap, (long long)cap);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(ADAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  a.k_cube = k_cube;
  a.v_cube = v_cube;
  a.q_extra = q_extra;
  a.sel_count = sel_count;
  a.sel_idx = sel_idx;
  a.out_extra = out_extra;
  adas::bind_attention_workspace(a, dtype, ws);
  adas::SelectArgs s{};
  s.g = a.g;
  s.hg = a.hg;
  s.q_extra = q_extra;
  s.kbar = kbar;
  s.zbuf = reinterpret_cast<float*>(static_cast<char*>(ws) + sel_off);
  s.n_extra = n_extra;
  s.p = p;
  s.sel_count = sel_count;
  s.sel_idx = sel_idx;
  s.capv = 0;
  s.rows_per_head = n_extra;
  s.has_video = 0;
  // the split selection writes the extra rows' bitmaps the attention reads,
  // so the attention skips its bitmap launch
  if (dtype == ADAS_BF16 && a.extra_bits != nullptr && adas::use_split_select(a.g, n_extra, a.hg.gmax)) {
    s.extra_bits = a.extra_bits;
    s.bits_words = a.bits_words;
    a.bits_ready = 1;
  }
  hipError_t e = adas::launch_select(s, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "adas_decode_step selection launch");
  return hip_status(adas::launch_attention(a, dtype, (hipStream_t)stream), "adas_decode_step attention launch");
}

static adas_status build_bwd(const adas_geom* geom, adas_dtype dtype, bool has_video, int32_t n_extra,
                             adas::BwdArgs& b) {
  b = adas::BwdArgs{};
  adas_status st = derive(geom, b.g, b.hg);
  if (st != ADAS_OK) return st;
  if (dtype != ADAS_BF16) return fail(ADAS_ERR_DTYPE, "the backward supports bf16 only");
  if (b.g.S != 64)
    return fail(ADAS_ERR_SHAPE, "the backward is enabled for cubes of 64 tokens only (S = %d)", b.g.S);
  if (b.g.Nc > ADAS_MAX_CUBES) return fail(ADAS_ERR_SHAPE, "%d cubes exceed the limit %d", b.g.Nc, ADAS_MAX_CUBES);
  if (n_extra < 0) return fail(ADAS_ERR_SHAPE, "n_extra must be >= 0");
  if (!has_video && n_extra == 0) return fail(ADAS_ERR_SHAPE, "no query rows");
  b.has_video = has_video;
  b.n_extra = n_extra;
  b.capv = capv_of(b.g, has_video);
  b.rows_per_head = (has_video ? b.g.N : 0) + n_extra;
  adas::plan_backward(b);
  return ADAS_OK;
}

adas_status adas_sparse_attn_bwd(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                 const void* k_cube, const void* v_tok, const void* k_vt, int32_t n_extra,
                                 const void* q_extra, const int32_t* sel_count, const int32_t* sel_idx,
                                 const void* out_raster, const void* out_extra, const float* lse,
                                 const void* dout_raster, const void* dout_extra, float* dq_raster,
                                 float* dq_extra, float* dk_raster, float* dv_raster, int32_t n_text_kv,
                                 const void* k_text, const void* v_text, float* dk_text, float* dv_text,
                                 void* ws, size_t ws_bytes, void* stream) {
  adas::BwdArgs b;
  adas_status st = build_bwd(geom, dtype, q_cube != nullptr, n_extra, b);
  if (st != ADAS_OK) return st;
  if (n_text_kv != 0 && n_text_kv != n_extra)
    return fail(ADAS_ERR_VALUE, "n_text_kv must be 0 or n_extra (%d), got %d", n_extra, n_text_kv);
  if (n_text_kv > 0 && (k_text == nullptr || v_text == nullptr || dk_text == nullptr || dv_text == nullptr))
    return fail(ADAS_ERR_NULL, "k_text/v_text/dk_text/dv_text is NULL");
  if (k_cube == nullptr || v_tok == nullptr || k_vt == nullptr || sel_count == nullptr || sel_idx == nullptr ||
      lse == nullptr || dk_raster == nullptr || dv_raster == nullptr)
    return fail(ADAS_ERR_NULL, "k_cube/v_tok/k_vt/sel_count/sel_idx/lse/dk_raster/dv_raster is NULL");
  if (q_cube != nullptr && (out_raster == nullptr || dout_raster == nullptr || dq_raster == nullptr))
    return fail(ADAS_ERR_NULL, "out_raster/dout_raster/dq_raster is NULL");
  if (n_extra > 0 && (q_extra == nullptr || out_extra == nullptr || dout_extra == nullptr || dq_extra == nullptr))
    return fail(ADAS_ERR_NULL, "q_extra/out_extra/dout_extra/dq_extra is NULL");
  const size_t need = adas::backward_workspace_bytes(b);
  if (ws == nullptr || ws_bytes < need)
    return fail(ADAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  b.q_cube = (const uint16_t*)q_cube;
  b.q_extra = (const uint16_t*)q_extra;
  b.k_cube = (const uint16_t*)k_cube;
  b.v_tok = (const uint16_t*)v_tok;
  b.k_vt = (const uint16_t*)k_vt;
  b.out_raster = (const uint16_t*)out_raster;
  b.out_extra = (const uint16_t*)out_extra;
  b.dout_raster = (const uint16_t*)dout_raster;
  b.dout_extra = (const uint16_t*)dout_extra;
  b.lse = lse;
  b.sel_count = sel_count;
  b.sel_idx = sel_idx;
  b.dq_raster = dq_raster;
  b.dq_extra = dq_extra;
  b.dk_raster = dk_raster;
  b.dv_raster = dv_raster;
  b.n_text_kv = n_text_kv;
  b.k_text = (const uint16_t*)k_text;
  b.v_text = (const uint16_t*)v_text;
  b.dk_text = dk_text;
  b.dv_text = dv_text;
  adas::bind_backward_workspace(b, ws);
  return hip_status(adas::launch_backward(b, (hipStream_t)stream), "adas_sparse_attn_bwd launch");
}

adas_status adas_cache_append(const adas_geom* geom, adas_dtype dtype, int32_t t0, int32_t n_frames,
                              const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              float* kbar, double* ksum, void* stream) {
  adas::KGeom g;
  adas::HeadGroups hg;
  adas_status st = derive(geom, g, hg);
  if (st != ADAS_OK) return st;
  if (dtype != ADAS_BF16) return fail(ADAS_ERR_DTYPE, "adas_cache_append supports bf16 only");
  const int cap = geom->cache_T ? geom->cache_T : geom->T;
  if (t0 < 0 || n_frames <= 0 || (long long)t0 + n_frames > cap)
    return fail(ADAS_ERR_SHAPE, "frames [%d, %d) outside the cache of %d frames", t0, t0 + n_frames, cap);
  if (k_new == nullptr || v_new == nullptr || k_cache == nullptr || v_cache == nullptr || kbar == nullptr ||
      ksum == nullptr)
    return fail(ADAS_ERR_NULL, "k_new/v_new/k_cache/v_cache/kbar/ksum is NULL");
  // kernels index the whole cache: its grid is the capacity
  g.T = cap;
  g.nT = cap / g.ct;
  g.N = g.NS;
  g.Nc = g.NS / g.S;
  return hip_status(adas::launch_cache_append(g, t0, t0 + n_frames, k_new, v_new, k_cache, v_cache, kbar, ksum,
                                              (hipStream_t)stream),
                    "adas_cache_append launch");
}

size_t adas_cache_sum_bytes(const adas_geom* geom) {
  adas::KGeom g;
  adas::HeadGroups hg;
  if (derive(geom, g, hg) != ADAS_OK) return 0;
  return (size_t)g.Hkv * g.nH * g.nW * g.D * sizeof(double);
}

size_t adas_workspace_bytes(const adas_geom* geom, adas_dtype dtype, adas_ws_kind kind,
                            int32_t has_video, int32_t n_extra) {
  if (kind == ADAS_WS_SELECT) {
    adas::KGeom g;
    adas::HeadGroups hg;
    if (derive(geom, g, hg) != ADAS_OK || check_dtype(dtype) != ADAS_OK) return 0;
    if (n_extra < 0) return 0;
    return adas::select_workspace_bytes(g, dtype, n_extra, hg.gmax);
  }
  if (kind == ADAS_WS_DECODE) {
    adas::AttnArgs a;
    size_t attn_bytes = 0, sel_off = 0, total = 0;
    if (has_video || decode_plan(geom, dtype, n_extra, a, attn_bytes, sel_off, total) != ADAS_OK) return 0;
    return total;
  }
  if (kind == ADAS_WS_BWD) {
    adas::BwdArgs b;
    if (build_bwd(geom, dtype, has_video != 0, n_extra, b) != ADAS_OK) return 0;
    return adas::backward_workspace_bytes(b);
  }
  adas::AttnArgs a;
  const int dummy = 1;
  if (build_attn(geom, dtype, has_video ? &dummy : nullptr, n_extra, 0, a) != ADAS_OK) return 0;
  size_t bytes = adas::attention_workspace_bytes(a, dtype);
  // the query does not know whether the extra rows will bring causal text
  // keys, and without video rows that changes the plan (text keys rule out
  // the decode kernel): size for the larger of the two plans
  if (!has_video && n_extra > 0 && build_attn(geom, dtype, nullptr, n_extra, n_extra, a) == ADAS_OK) {
    const size_t b2 = adas::attention_workspace_bytes(a, dtype);
    if (b2 > bytes) bytes = b2;
  }
  return bytes;
}

int64_t adas_sel_capacity(const adas_geom* geom, int32_t has_video, int32_t n_extra) {
  adas::KGeom g;
  adas::HeadGroups hg;
  if (derive(geom, g, hg) != ADAS_OK || n_extra < 0) return -1;
  return capacity_of(g, has_video != 0, n_extra);
}

// ---------------------------------------------------------------------------
// AdaS-FFN
// ---------------------------------------------------------------------------
static adas_status derive_ffn(const adas_ffn_geom* geom, adas::KGeom& g) {
  if (geom == nullptr) return fail(ADAS_ERR_NULL, "geom is NULL");
  const adas_ffn_geom& s = *geom;
  if (s.T <= 0 || s.H <= 0 || s.W <= 0 || s.ct <= 0 || s.ch <= 0 || s.cw <= 0)
    return fail(ADAS_ERR_SHAPE, "grid and cube extents must be positive");
  if (s.T % s.ct || s.H % s.ch || s.W % s.cw)
    return fail(ADAS_ERR_SHAPE, "cube %dx%dx%d (t,h,w) does not divide grid %dx%dx%d", s.ct, s.ch,
                s.cw, s.T, s.H, s.W);
  const long long N = (long long)s.T * s.H * s.W;
  if (N > (1LL << 28)) return fail(ADAS_ERR_SHAPE, "too many tokens (%lld)", N);
  const int S = s.ct * s.ch * s.cw;
  if (S > ADAS_FFN_MAX_S)
    return fail(ADAS_ERR_SHAPE, "%d tokens per cube exceed the limit %d", S, ADAS_FFN_MAX_S);
  if (s.hidden <= 0 || s.hidden % 256 || s.hidden > 65536)
    return fail(ADAS_ERR_SHAPE, "hidden must be a positive multiple of 256 up to 65536 (got %d)", s.hidden);
  if (s.inter <= 0 || s.inter % 128 || s.inter > 262144)
    return fail(ADAS_ERR_SHAPE, "inter must be a positive multiple of 128 up to 262144 (got %d)", s.inter);
  g = adas::KGeom{};
  g.T = s.T; g.H = s.H; g.W = s.W;
  g.ct = s.ct; g.ch = s.ch; g.cw = s.cw;
  g.nT = s.T / s.ct; g.nH = s.H / s.ch; g.nW = s.W / s.cw;
  g.N = (int)N;
  g.S = S;
  g.Nc = g.nT * g.nH * g.nW;
  return ADAS_OK;
}

adas_status adas_ffn_select(const adas_ffn_geom* geom, const void* x, double p,
                            int32_t* act_count, int32_t* act_off, int32_t* act_rows,
                            uint32_t* act_mask, void* stream) {
  adas::KGeom g;
  adas_status st = derive_ffn(geom, g);
  if (st != ADAS_OK) return st;
  if (!(p > 0.0 && p <= 1.0)) return fail(ADAS_ERR_VALUE, "p must be in (0, 1] (got %g)", p);
  if (x == nullptr || act_count == nullptr || act_off == nullptr || act_rows == nullptr ||
      act_mask == nullptr)
    return fail(ADAS_ERR_NULL, "x/act_count/act_off/act_rows/act_mask is NULL");
  return hip_status(adas::launch_ffn_select(g, geom->hidden, x, p, act_count, act_off, act_rows,
                                            act_mask, (hipStream_t)stream),
                    "adas_ffn_select launch");
}

adas_status adas_ffn_fwd(const adas_ffn_geom* geom, const void* x, int32_t n_text,
                         const void* x_text, const void* w_gate, const void* w_up,
                         const void* w_down, const int32_t* act_off, const int32_t* act_rows,
                         const uint32_t* act_mask, void* y, void* y_text, void* ws,
                         size_t ws_bytes, void* stream) {
  adas::KGeom g;
  adas_status st = derive_ffn(geom, g);
  if (st != ADAS_OK) return st;
  if (n_text < 0 || n_text > (1 << 24)) return fail(ADAS_ERR_SHAPE, "n_text out of range (%d)", n_text);
  if (x == nullptr || w_gate == nullptr || w_up == nullptr || w_down == nullptr ||
      act_off == nullptr || act_rows == nullptr || act_mask == nullptr || y == nullptr)
    return fail(ADAS_ERR_NULL, "x/weights/selection/y is NULL");
  if (n_text > 0 && (x_text == nullptr || y_text == nullptr))
    return fail(ADAS_ERR_NULL, "x_text/y_text is NULL");
  const size_t need = adas::ffn_workspace_bytes(g, geom->hidden, geom->inter, n_text);
  if (ws == nullptr || ws_bytes < need)
    return fail(ADAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  adas::FfnArgs f;
  f.g = g;
  f.hidden = geom->hidden;
  f.inter = geom->inter;
  f.n_text = n_text;
  f.x = x;
  f.x_text = x_text;
  f.w_gate = w_gate;
  f.w_up = w_up;
  f.w_down = w_down;
  f.act_off = act_off;
  f.act_rows = act_rows;
  f.act_mask = act_mask;
  f.y = y;
  f.y_text = y_text;
  f.ws = ws;
  return hip_status(adas::launch_ffn(f, (hipStream_t)stream), "adas_ffn_fwd launch");
}

size_t adas_ffn_workspace_bytes(const adas_ffn_geom* geom, int32_t n_text) {
  adas::KGeom g;
  if (derive_ffn(geom, g) != ADAS_OK || n_text < 0) return 0;
  return adas::ffn_workspace_bytes(g, geom->hidden, geom->inter, n_text);
}

const char* adas_status_string(adas_status s) {
  switch (s) {
    case ADAS_OK: return "ADAS_OK";
    case ADAS_ERR_NULL: return "ADAS_ERR_NULL: a required pointer is NULL";
    case ADAS_ERR_SHAPE: return "ADAS_ERR_SHAPE: inconsistent shape arguments";
    case ADAS_ERR_VALUE: return "ADAS_ERR_VALUE: argument value out of range";
    case ADAS_ERR_DTYPE: return "ADAS_ERR_DTYPE: unknown dtype";
    case ADAS_ERR_WORKSPACE: return "ADAS_ERR_WORKSPACE: workspace too small";
    case ADAS_ERR_CAPACITY: return "ADAS_ERR_CAPACITY: selection buffer too small";
    case ADAS_ERR_HIP: return "ADAS_ERR_HIP: HIP runtime error";
  }
  return "unknown adas_status";
}

const char* adas_last_error(void) { return g_last_error; }

const char* adas_version(void) { return "0.1"; }

adas_status adas_probe_mfma(int32_t workgroups, int32_t iters, float* sink, double* flops, void* stream) {
  if (workgroups < 1 || iters < 1) return fail(ADAS_ERR_VALUE, "workgroups and iters must be >= 1");
  if (sink == nullptr) return fail(ADAS_ERR_NULL, "sink is NULL");
  if (flops != nullptr) *flops = adas::probe_mfma_flops_per_wg(iters) * workgroups;
  return hip_status(adas::launch_probe_mfma(workgroups, iters, sink, (hipStream_t)stream), "adas_probe_mfma launch");
}

adas_status adas_probe_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups,
                                void* stream) {
  if (src == nullptr || sink == nullptr) return fail(ADAS_ERR_NULL, "src/sink is NULL");
  if (bytes <= 0 || bytes % 16) return fail(ADAS_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (workgroups < 1) workgroups = 8 * 256;
  return hip_status(adas::launch_probe_read(src, bytes, sink, workgroups, (hipStream_t)stream),
                    "adas_probe_hbm_read launch");
}

adas_status adas_probe_hbm_copy(const void* src, void* dst, int64_t bytes, int32_t workgroups, void* stream) {
  if (src == nullptr || dst == nullptr) return fail(ADAS_ERR_NULL, "src/dst is NULL");
  if (bytes <= 0 || bytes % 16) return fail(ADAS_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (workgroups < 1) workgroups = 8 * 256;
  return hip_status(adas::launch_probe_copy(src, dst, bytes, workgroups, (hipStream_t)stream),
                    "adas_probe_hbm_copy launch");
}

adas_status adas_probe_attn_mix(int32_t workgroups, int32_t iters, int32_t mix, const void* src, int64_t src_bytes,
                                float* sink, double* flops, void* stream) {
  if (workgroups < 1 || iters < 1) return fail(ADAS_ERR_VALUE, "workgroups and iters must be >= 1");
  if (mix != 0 && mix != 1) return fail(ADAS_ERR_VALUE, "mix must be 0 or 1 (got %d)", mix);
  if (sink == nullptr) return fail(ADAS_ERR_NULL, "sink is NULL");
  if (mix == 1) {
    if (src == nullptr) return fail(ADAS_ERR_NULL, "src is NULL");
    if (src_bytes < (2 << 20) || src_bytes >= 0x80000000LL)
      return fail(ADAS_ERR_SHAPE, "src_bytes must be in [2 MiB, 2 GiB)");
  }
  if (flops != nullptr) *flops = adas::probe_attn_mix_flops_per_wg(iters) * workgroups;
  return hip_status(adas::launch_probe_attn_mix(workgroups, iters, mix == 1, src, (int)src_bytes, sink,
                                                (hipStream_t)stream),
                    "adas_probe_attn_mix launch");
}

}  // extern "C"

namespace adas {
// Exact attention workspace of one call (0 when none is needed), for the
// allocation-free entry point; validates like the call itself.
adas_status attn_workspace_need(const adas_geom* geom, adas_dtype dtype, const void* q_cube, int32_t n_extra,
                                int32_t n_text_kv, size_t* need) {
  AttnArgs a;
  adas_status st = build_attn(geom, dtype, q_cube, n_extra, n_text_kv, a);
  if (st != ADAS_OK) return st;
  *need = attention_workspace_bytes(a, dtype);
  return ADAS_OK;
}
adas_status set_error(adas_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace adas
