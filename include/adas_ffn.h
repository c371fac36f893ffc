/*
 * adas_ffn.h -- C ABI of libadas, AdaS-FFN (adaptive token-selective FFN) on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (AdaSpark, CVPR 2026; papernotes.org summary, "关键设计" items
 * 3 and 4; thelatestinai.com listing, Figure 2 caption):
 *   1. inside every video cube, each token's importance is estimated from its
 *      L2 norm, and Top-p (the AdaS-Attn rule, the same threshold p) keeps the
 *      tokens that go through the FFN: the active set M_c;
 *   2. an active token gets y = x + FFN(x);
 *   3. a skipped token k of cube c gets y_k = x_k + m_c, with m_c the mean of
 *      FFN(x_j) over j in M_c (mean compensation);
 *   4. text tokens always go through the FFN.
 * Readings taken here (the pages leave them open):
 *   * the Top-p distribution of a cube is each token's share of the cube's
 *     summed L2 norm, P_r = ||x_r|| / sum_j ||x_j||; the active set is the
 *     shortest prefix of tokens ordered by (P descending, offset r ascending)
 *     whose sum reaches p; p = 1 keeps every token;
 *   * FFN(x) = W_down (silu(W_gate x) * (W_up x)) (the SwiGLU MLP of the
 *     Qwen2.5-VL backbones of the listing's Table 5), silu(t) = t/(1+e^-t).
 *
 * Conventions: as in adas.h (device pointers owned by the caller, no device
 * allocation, asynchronous on `stream`, host-side validation before any
 * launch, thread-local adas_last_error()).  Cube numbering and offsets r are
 * those of adas.h.  Every tensor is bfloat16 except where stated.
 */
#ifndef ADAS_FFN_H
#define ADAS_FFN_H

#include "adas.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ADAS_FFN_MAX_S 256   /* limit on tokens per cube for AdaS-FFN */

/* FFN problem geometry (host only). */
typedef struct {
  int32_t T, H, W;     /* video grid in tokens: frames, rows, columns          */
  int32_t ct, ch, cw;  /* cube extents t, h, w; each divides T, H, W           */
  int32_t hidden;      /* model width: a multiple of 256                       */
  int32_t inter;       /* FFN width: a multiple of 128                         */
} adas_ffn_geom;

/*
 * adas_ffn_select -- token importance and per-cube Top-p (papernotes.org, key
 * design 3 and 4).
 *   x         [N][hidden]   video hidden states, raster token order
 *   p         threshold in (0, 1] (double: the decisions are taken in float64)
 *   act_count [Nc] int32    output: |M_c|, at least 1
 *   act_off   [Nc+1] int32  output: exclusive prefix sums of act_count; cube
 *                           c's active tokens are rows act_off[c] ..
 *                           act_off[c+1]-1 of the compact token list, and
 *                           act_off[Nc] is the number of active video tokens
 *   act_rows  [N] int32     output: raster index of every active token, cube
 *                           by cube, ascending offset inside a cube; entries
 *                           from act_off[Nc] on are not written
 *   act_mask  [Nc][ceil(S/32)] uint32  output: bit r%32 of word r/32 of cube c
 *                           is set iff token r of cube c is active
 * Norms are summed in float64 from the bf16 values; shares, their order and
 * the running sums are float64 too.
 * Errors: NULL, SHAPE (grid/cube, S > ADAS_FFN_MAX_S, hidden), VALUE (p), HIP.
 */
adas_status adas_ffn_select(const adas_ffn_geom* geom, const void* x, double p,
                            int32_t* act_count, int32_t* act_off, int32_t* act_rows,
                            uint32_t* act_mask, void* stream);

/*
 * adas_ffn_fwd -- FFN of the active tokens, mean compensation of the skipped
 * ones, dense FFN of the text tokens (papernotes.org, key design 3).
 *   x        [N][hidden]          video hidden states, raster order
 *   n_text   text tokens (0 allowed); x_text [n_text][hidden] (NULL iff 0)
 *   w_gate, w_up [inter][hidden]  weights in the nn.Linear [out][in] layout
 *   w_down   [hidden][inter]
 *   act_off, act_rows, act_mask   the selection written by adas_ffn_select
 *   y        [N][hidden]          output, raster order (must not overlap x)
 *   y_text   [n_text][hidden]     output (NULL iff n_text == 0)
 *   ws, ws_bytes  workspace of at least adas_ffn_workspace_bytes(): the
 *            bf16 hidden activations silu(W_gate x) * (W_up x) and the
 *            float32 FFN outputs of the active and text tokens.
 * Products accumulate in float32; the hidden activation is rounded to bf16
 * before W_down (as a bf16 model stores it); y = x + FFN(x) or x + m_c is
 * formed in float32 and rounded once to bf16.  The active count is read on
 * the device; the host never waits for the selection.
 * Errors: NULL, SHAPE (hidden % 256, inter % 128, grid), WORKSPACE, HIP.
 */
adas_status adas_ffn_fwd(const adas_ffn_geom* geom, const void* x, int32_t n_text,
                         const void* x_text, const void* w_gate, const void* w_up,
                         const void* w_down, const int32_t* act_off, const int32_t* act_rows,
                         const uint32_t* act_mask, void* y, void* y_text, void* ws,
                         size_t ws_bytes, void* stream);

/* Bytes of workspace adas_ffn_fwd needs (host only).  0 for invalid geometry. */
size_t adas_ffn_workspace_bytes(const adas_ffn_geom* geom, int32_t n_text);

#ifdef __cplusplus
}
#endif
#endif /* ADAS_FFN_H */
