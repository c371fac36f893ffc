// Allocation-free variant of adas_sparse_attn_fwd, for callers that cannot
// allocate device memory (work recorded under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  The attention's scratch
// (extra-row selection bitmaps and per-chunk partial rows) lives in a
// file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy of the array until the process ends.
// Host code never passes the array's name to a kernel: its device address
// is looked up once per device and kept.
#include <mutex>

#include "common.h"

namespace {

__device__ __align__(256) unsigned char scratch[ADAS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    g_lookup[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_lookup[dev] != hipSuccess) return g_lookup[dev];
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

namespace adas {
adas_status attn_workspace_need(const adas_geom* geom, adas_dtype dtype, const void* q_cube, int32_t n_extra,
                                int32_t n_text_kv, size_t* need);
adas_status set_error(adas_status s, const char* msg);
}  // namespace adas

extern "C" adas_status adas_sparse_attn_fwd_noalloc(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                                     const void* k_cube, const void* v_cube, int32_t n_extra,
                                                     int32_t n_text_kv, const void* q_extra, const void* k_text,
                                                     const void* v_text, const int32_t* sel_count,
                                                     const int32_t* sel_idx, void* out_raster, void* out_extra,
                                                     void* stream) {
  size_t need = 0;
  adas_status st = adas::attn_workspace_need(geom, dtype, q_cube, n_extra, n_text_kv, &need);
  if (st != ADAS_OK) return st;
  if (need > (size_t)ADAS_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu "
             "(use adas_sparse_attn_fwd with a workspace)",
             need, (size_t)ADAS_NOALLOC_SCRATCH_BYTES);
    return adas::set_error(ADAS_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) {
      char msg[200];
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
      return adas::set_error(ADAS_ERR_HIP, msg);
    }
  }
  return adas_sparse_attn_fwd(geom, dtype, q_cube, k_cube, v_cube, n_extra, n_text_kv, q_extra, k_text, v_text,
                              sel_count, sel_idx, out_raster, out_extra, ws, (size_t)ADAS_NOALLOC_SCRATCH_BYTES,
                              stream);
}
