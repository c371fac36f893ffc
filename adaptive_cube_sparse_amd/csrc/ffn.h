// Launch descriptors of the AdaS-FFN kernels (host and device views).
#pragma once
#include "adas_ffn.h"
#include "common.h"

namespace adas {

// One GEMM launch of the FFN: C[M][n] = A[M][K] . B[n][K]^T, M read on the
// device as act_off[Nc] + n_text.
struct FfnGemmArgs {
  const uint16_t* a;       // gate/up: video hidden states [N][K]; down: H [rows][K]
  const uint16_t* a_text;  // gate/up: text hidden states [n_text][K]
  const int32_t* rows;     // gate/up: raster row of each active video token
  const int32_t* act_off;  // [Nc + 1]
  int Nc, n_text;
  int K;
  const uint16_t* b0;      // gate/up: W_gate; down: W_down  ([n][K])
  const uint16_t* b1;      // gate/up: W_up
  int n_tiles;             // output column tiles
  void* out;               // gate/up: H bf16 [rows][inter]; down: F float [rows][hidden]
  int ldo;
};

struct FfnArgs {
  KGeom g;
  int hidden, inter, n_text;
  const void* x;
  const void* x_text;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const int32_t* act_off;
  const int32_t* act_rows;
  const uint32_t* act_mask;
  void* y;
  void* y_text;
  void* ws;
};

int ffn_mask_words(int S);
size_t ffn_workspace_bytes(const KGeom& g, int hidden, int inter, int n_text);
hipError_t launch_ffn_select(const KGeom& g, int hidden, const void* x, double p, int32_t* act_count,
                             int32_t* act_off, int32_t* act_rows, uint32_t* act_mask, hipStream_t s);
hipError_t launch_ffn(const FfnArgs& f, hipStream_t s);

}  // namespace adas
