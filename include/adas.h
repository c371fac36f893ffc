/*
 * adas.h -- C ABI of libadas, AdaS-Attn (adaptive cube-selective attention)
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (AdaSpark, CVPR 2026; papernotes.org summary, "关键设计" items
 * 1, 2 and 4; thelatestinai.com listing, Figure 2 caption):
 *   1. video tokens on a T x H x W grid are cut into h x w x t cubes;
 *   2. every cube j gets a mean key kbar_j;
 *   3. a query in cube i scores the preceding cubes,
 *      P_i = softmax_j(q . kbar_j / sqrt(d_k)), j < i;
 *   4. it keeps the Top-p set S_i: the fewest cubes, highest P first (equal P:
 *      lower cube index first), whose probabilities sum to at least p;
 *   5. it attends, with one exact softmax, to the tokens of S_i plus all
 *      tokens of its own cube.
 * Text queries select among all video cubes and attend causally to the text
 * tokens up to themselves; decode queries select among all cubes of a video
 * KV cache and attend to the selected cubes only.
 *
 * Conventions shared by every call
 * ---------------------------------
 *  * Tensor arguments are DEVICE pointers owned by the caller.  The library
 *    allocates no device memory; scratch memory is the caller's workspace
 *    (ws, ws_bytes), sized by adas_workspace_bytes().
 *  * Every compute call is asynchronous on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream).  Arguments are validated on the host
 *    before anything is launched; on an error nothing is launched and the
 *    outputs are untouched.  A launch failure returns ADAS_ERR_HIP.  A
 *    thread-local message describing the last error is kept for
 *    adas_last_error().
 *  * Shapes: N = T*H*W tokens, S = ct*ch*cw tokens per cube, Nc = N / S cubes.
 *    Cube-layout buffers (q_cube, k_cube, v_cube, kbar, x_cube) hold
 *    NS = cT*H*W tokens (NS/S cubes) per head, cT = cache_T or T: head h
 *    starts at token h*NS.  Only the first N tokens (Nc cubes) of a head are
 *    read or written by a call.
 *    Cube c of raster token n = (f*H + y)*W + x is
 *    c = ((f/ct)*(H/ch) + y/ch)*(W/cw) + x/cw, its offset inside the cube is
 *    r = ((f%ct)*ch + y%ch)*cw + x%cw, and its cube-layout position is c*S + r.
 *  * dtype ADAS_BF16: bfloat16 Q/K/V/outputs, MFMA kernels, head_dim 64 or
 *    128, S a multiple of 16.  ADAS_F32: float32 throughout (reference-grade
 *    kernels for small problems), head_dim 64 or 128.
 *  * Grouped-query attention: query head hq reads KV head head_map[hq]
 *    (head_map NULL: hq / (Hq/Hkv), which needs Hkv | Hq).
 *  * The library keeps no state between calls and is re-entrant.
 */
#ifndef ADAS_H
#define ADAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADAS_VERSION_MAJOR 0
#define ADAS_VERSION_MINOR 1

#define ADAS_MAX_HEADS 128   /* limit on n_q_heads and n_kv_heads            */
#define ADAS_MAX_CUBES 4096  /* limit on Nc for selection (candidates/row)   */

typedef enum {
  ADAS_OK = 0,
  ADAS_ERR_NULL = 1,       /* a required pointer is NULL                      */
  ADAS_ERR_SHAPE = 2,      /* grid/cube/head/size arguments are inconsistent  */
  ADAS_ERR_VALUE = 3,      /* p outside (0, 1], head_map entry or layout bad  */
  ADAS_ERR_DTYPE = 4,      /* unknown dtype                                   */
  ADAS_ERR_WORKSPACE = 5,  /* ws_bytes smaller than adas_workspace_bytes()    */
  ADAS_ERR_CAPACITY = 6,   /* sel_cap smaller than adas_sel_capacity()        */
  ADAS_ERR_HIP = 7         /* a HIP launch or runtime call failed             */
} adas_status;

typedef enum { ADAS_BF16 = 0, ADAS_F32 = 1 } adas_dtype;

/* Problem geometry.  Passed by pointer; read on the host only. */
typedef struct {
  int32_t T, H, W;          /* frame grid in tokens: frames, rows, columns    */
  int32_t ct, ch, cw;       /* cube extents t, h, w; each divides T, H, W     */
  int32_t n_q_heads;        /* Hq                                             */
  int32_t n_kv_heads;       /* Hkv                                            */
  int32_t head_dim;         /* d_k (64 or 128)                                */
  const int32_t* head_map;  /* HOST array [Hq] -> kv head, or NULL            */
  int32_t cache_T;          /* frames each head of a cube-layout buffer holds:
                               0 = T; else a multiple of ct, >= T (a video KV
                               cache allocated for cache_T frames of which the
                               first T are filled, see adas_cache_append)     */
} adas_geom;

/* Which call a workspace is sized for. */
typedef enum { ADAS_WS_SELECT = 0, ADAS_WS_ATTN = 1, ADAS_WS_BWD = 2, ADAS_WS_DECODE = 3 } adas_ws_kind;

/* Storage of a cube-layout tensor (see adas_cube_partition). */
typedef enum { ADAS_LAYOUT_TOKENS = 0, ADAS_LAYOUT_VT = 1 } adas_layout;

/*
 * adas_cube_partition -- cube partition (papernotes.org, key design 1).
 * Copies a token-major tensor into the cube-contiguous, head-major layout
 * used by every other call.  Bit-exact copy.
 *   x_raster [N][n_heads][d]  input, raster token order (as a QKV projection
 *                             emits it)
 *   layout   ADAS_LAYOUT_TOKENS: x_cube [n_heads][N][d] with
 *                             x_cube[h][c*S + r] = x_raster[n][h]
 *            ADAS_LAYOUT_VT:  x_cube [n_heads][Nc][d][S], each cube stored
 *                             transposed: x_cube[h][c][e][pi(r)] =
 *                             x_raster[n][h][e], where pi swaps bits 2 and 3
 *                             of r inside every complete aligned group of 16
 *                             offsets (pi(r) = r in a trailing partial group).
 *                             This is the value layout adas_sparse_attn_fwd
 *                             reads.
 *   perm     [N] int32        optional output (may be NULL): perm[c*S+r] = n
 * Call once for Q and K (n_heads = Hq, Hkv; ADAS_LAYOUT_TOKENS) and once for
 * V (n_heads = Hkv; ADAS_LAYOUT_VT).
 * Errors: NULL (x_raster/x_cube), SHAPE, VALUE (unknown layout), DTYPE, HIP.
 */
adas_status adas_cube_partition(const adas_geom* geom, adas_dtype dtype, int32_t n_heads,
                                adas_layout layout, const void* x_raster, void* x_cube,
                                int32_t* perm, void* stream);

/*
 * adas_cube_mean_keys -- cube mean keys kbar_j (papernotes.org, key design 2).
 *   k_cube [Hkv][N][d]   keys in cube layout (ADAS_LAYOUT_TOKENS)
 *   kbar   [Hkv][Nc][d]  float32 output: (1/S) * sum of cube j's S keys,
 *                        accumulated in float64, rounded once to float32
 *                        (round to nearest even).
 * Errors: NULL, SHAPE, DTYPE, HIP.
 */
adas_status adas_cube_mean_keys(const adas_geom* geom, adas_dtype dtype, const void* k_cube,
                                float* kbar, void* stream);

/*
 * adas_cube_partition_keys -- adas_cube_partition of the keys
 * (ADAS_LAYOUT_TOKENS, n_heads = n_kv_heads) and adas_cube_mean_keys in one
 * pass, so K is read from memory once (papernotes.org, key designs 1 and 2).
 *   k_raster [N][Hkv][d]  keys, raster token order
 *   k_cube   [Hkv][N][d]  output, as adas_cube_partition
 *   perm     [N] int32    output (nullable), as adas_cube_partition
 *   kbar     [Hkv][Nc][d] float32 output, as adas_cube_mean_keys: float64
 *                        sums, rounded once.  The rows are added in another
 *                        order than adas_cube_mean_keys adds them, so the two
 *                        agree bit for bit whenever the float64 sums are
 *                        exact; with S <= 256 that holds when a cube's
 *                        nonzero key magnitudes lie within a factor 2^37
 *                        (bf16) or 2^21 (float32) of each other.
 * Errors: NULL, SHAPE, DTYPE, HIP.
 */
adas_status adas_cube_partition_keys(const adas_geom* geom, adas_dtype dtype, const void* k_raster,
                                     void* k_cube, int32_t* perm, float* kbar, void* stream);

/*
 * adas_select_topp -- selection softmax and Top-p cube sets (papernotes.org,
 * key design 2, the P_i and S_i equations; key design 4, one threshold p).
 *
 * Rows: video rows (hq, pos) for pos in [0, N) when q_cube != NULL, then
 * extra rows (hq, m) for m in [0, n_extra) (text or decode queries).
 * Video row candidates are cubes 0..c-1 of its own cube c; extra rows'
 * candidates are all Nc cubes.
 *   q_cube   [Hq][N][d]       video queries in cube layout, or NULL
 *   n_extra  number of extra query tokens (0 allowed)
 *   q_extra  [n_extra][Hq][d] extra queries, token-major (NULL iff n_extra==0)
 *   kbar     [Hkv][Nc][d]     float32 mean keys
 *   p        threshold in (0, 1]; p == 1 keeps every candidate
 *   sel_count [Hq][R] int32   output, R = (q_cube ? N : 0) + n_extra:
 *                             video row pos at [hq*R + pos], extra row m at
 *                             [hq*R + Nv + m] (Nv = N or 0)
 *   sel_idx  int32 [sel_cap]  output: each row's selected cube ids, ascending,
 *                             at a closed-form offset:
 *                               CapV = S*Nc*(Nc-1)/2 (0 without video rows)
 *                               video (hq, pos), c = pos/S, r = pos%S:
 *                                 hq*CapV + S*c*(c-1)/2 + r*c
 *                               extra (hq, m): Hq*CapV + (hq*n_extra + m)*Nc
 *                             Entries past a row's count are not written.
 *   sel_cap  capacity of sel_idx in entries (>= adas_sel_capacity()).
 *   ws, ws_bytes  workspace (adas_workspace_bytes(ADAS_WS_SELECT, ...)): the
 *            bf16 path keeps the extra rows' float32 logits there when a row
 *            has more than 1024 candidates and a KV head has at most 64
 *            extra rows (decode steps); otherwise none is needed and NULL/0
 *            is accepted.
 * Ordering: cubes are ranked by (P descending, cube index ascending); the
 * scores are computed to float32 accuracy from the float32 kbar.
 * Errors: NULL, SHAPE (Nc > ADAS_MAX_CUBES, no rows), VALUE (p, head_map),
 *         DTYPE, CAPACITY, WORKSPACE, HIP.
 */
adas_status adas_select_topp(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                             int32_t n_extra, const void* q_extra, const float* kbar, float p,
                             int32_t* sel_count, int32_t* sel_idx, int64_t sel_cap, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * adas_select_topk -- fixed-budget cube sets, the alternative the AdaSpark
 * listing (thelatestinai.com, Table 4, "Top-K" row) compares Top-p with.
 * Same rows, candidates, outputs and layout as adas_select_topp, but each
 * row keeps the k candidates of largest P (equivalently largest logit; equal
 * values lower cube index first), emitted ascending; a row with at most k
 * candidates keeps all of them.  Scores are computed as in adas_select_topp.
 *   k        budget, >= 1
 * Errors: as adas_select_topp, VALUE for k < 1.
 */
adas_status adas_select_topk(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                             int32_t n_extra, const void* q_extra, const float* kbar, int32_t k,
                             int32_t* sel_count, int32_t* sel_idx, int64_t sel_cap, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * adas_sparse_attn_fwd -- attention over the selected cubes plus the own cube
 * (papernotes.org, key design 2: always keep full attention to the own cube).
 *
 * One exact softmax (scale 1/sqrt(d)) per row over
 *   video row (hq, pos):  tokens of its selected cubes and all S tokens of
 *                         its own cube;
 *   extra row (hq, m):    tokens of its selected cubes, plus text tokens
 *                         0..m when n_text_kv > 0 (causal text).
 *   q_cube, k_cube          [Hq|Hkv][N][d], ADAS_LAYOUT_TOKENS (q_cube NULL: no
 *                           video rows, e.g. decode)
 *   v_cube                  [Hkv][Nc][d][S], ADAS_LAYOUT_VT
 *   n_extra, q_extra        as in adas_select_topp
 *   n_text_kv               0 (decode: no text keys) or n_extra (text prefill)
 *   k_text, v_text          [n_extra][Hkv][d] when n_text_kv > 0, else NULL
 *   sel_count, sel_idx      the selection (layout as adas_select_topp)
 *   out_raster [N][Hq][d]   video outputs in raster token order (NULL iff
 *                           q_cube is NULL)
 *   out_extra  [n_extra][Hq][d]  extra-row outputs (NULL iff n_extra == 0)
 *   ws, ws_bytes            workspace (adas_workspace_bytes(ADAS_WS_ATTN, ...))
 * Selected ids must be ascending, < the row's candidate count, and counts
 * must not exceed it; the host does not read device lists (undefined
 * behaviour otherwise).  Outputs are float32-accumulated, stored in dtype.
 * The bf16 path with extra rows keeps a per-row selection bitmap and, when it
 * splits the extra rows' cubes into chunks, their partial results in ws.
 * Errors: NULL, SHAPE (Nc > ADAS_MAX_CUBES, ...), VALUE, DTYPE, WORKSPACE, HIP.
 */
adas_status adas_sparse_attn_fwd(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                 const void* k_cube, const void* v_cube, int32_t n_extra,
                                 int32_t n_text_kv, const void* q_extra, const void* k_text,
                                 const void* v_text, const int32_t* sel_count,
                                 const int32_t* sel_idx, void* out_raster, void* out_extra,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * adas_sparse_attn_fwd_lse -- adas_sparse_attn_fwd that also stores each
 * row's log-sum-exp, the statistic adas_sparse_attn_bwd needs.
 *   lse  [Hq][R] float32 (R and row order as sel_count): natural log of
 *        sum_j exp(q.k_j / sqrt(d)) over the row's attended keys
 * Errors: as adas_sparse_attn_fwd; NULL for lse.
 */
adas_status adas_sparse_attn_fwd_lse(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                     const void* k_cube, const void* v_cube, int32_t n_extra,
                                     int32_t n_text_kv, const void* q_extra, const void* k_text,
                                     const void* v_text, const int32_t* sel_count,
                                     const int32_t* sel_idx, void* out_raster, void* out_extra,
                                     float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * adas_decode_step -- one decode step over a built KV cache: the selection of
 * adas_select_topp and the attention of adas_sparse_attn_fwd for n_extra
 * query tokens with no video rows and no text keys (papernotes.org, key
 * design 2; the AdaSpark listing, thelatestinai.com, Figure 2 caption: every
 * token query selects its own cubes), in one call.  Results equal those of
 * the two calls on the same inputs, bit for bit.  When the bf16 selection
 * runs its split path (more than 1024 cubes, at most 64 query rows per KV
 * head), it also writes each row's selection bitmap into ws, and the
 * attention reads it instead of building it in a launch of its own.
 *   n_extra  query tokens (>= 1)
 *   q_extra  [n_extra][Hq][d], token-major
 *   kbar     [Hkv][Nc][d] float32 mean keys of the cache
 *   k_cube   [Hkv][N][d] ADAS_LAYOUT_TOKENS; v_cube [Hkv][Nc][d][S] ADAS_LAYOUT_VT
 *   p        Top-p threshold in (0, 1]
 *   sel_count [Hq][n_extra], sel_idx [sel_cap]: the selection, laid out as
 *            adas_select_topp lays out extra rows (sel_cap >=
 *            adas_sel_capacity(geom, 0, n_extra))
 *   out_extra [n_extra][Hq][d]
 *   ws, ws_bytes  adas_workspace_bytes(ADAS_WS_DECODE, has_video = 0, n_extra)
 * Errors: NULL, SHAPE (n_extra < 1, Nc > ADAS_MAX_CUBES, ...), VALUE (p,
 *         head_map), DTYPE, CAPACITY, WORKSPACE, HIP.
 */
adas_status adas_decode_step(const adas_geom* geom, adas_dtype dtype, int32_t n_extra, const void* q_extra,
                             const float* kbar, const void* k_cube, const void* v_cube, float p,
                             int32_t* sel_count, int32_t* sel_idx, int64_t sel_cap, void* out_extra,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * adas_sparse_attn_bwd -- gradients of the sparse attention for fine-tuning
 * on the sparse pattern (papernotes.org, training strategy; key design 2
 * attention).  The selection is a discrete choice and is held fixed: no
 * gradient reaches it or the mean keys.  Rows: video rows (selected cubes +
 * own cube) and extra rows (selected cubes, and with n_text_kv = n_extra the
 * causal text keys of a text prefill, as the forward reads them).  bf16 only,
 * cubes of S = 64 tokens.
 *   q_cube, k_cube [h][NS][d]      ADAS_LAYOUT_TOKENS (q_cube NULL: no video rows)
 *   v_tok    [Hkv][NS][d]          V in ADAS_LAYOUT_TOKENS
 *   k_vt     [Hkv][NS/S][d][S]     K in ADAS_LAYOUT_VT
 *   n_extra, q_extra, sel_count, sel_idx   as adas_sparse_attn_fwd
 *   out_raster, out_extra, lse     the forward's outputs (adas_sparse_attn_fwd_lse)
 *   dout_raster [N][Hq][d], dout_extra [n_extra][Hq][d]   their gradients (bf16)
 *   dq_raster [N][Hq][d], dq_extra [n_extra][Hq][d],
 *   dk_raster, dv_raster [N][Hkv][d]   float32 outputs, raster token order;
 *            every element is written (keys no row attends get 0)
 *   n_text_kv  0, or n_extra for a text prefill whose extra rows are text
 *            tokens with causal text keys (the forward's n_text_kv)
 *   k_text, v_text [n_text_kv][Hkv][d]  the forward's text keys and values
 *   dk_text, dv_text [n_text_kv][Hkv][d]  float32 outputs, every element
 *            written (NULL, with k_text and v_text, when n_text_kv = 0)
 *   ws, ws_bytes  adas_workspace_bytes(ADAS_WS_BWD, ...): per-row D, the
 *            selections as bitmaps, and per cube the list of rows attending it
 * Errors: NULL, SHAPE (S != 64, Nc), VALUE (n_text_kv not 0 or n_extra),
 *         DTYPE (not bf16), WORKSPACE, HIP.
 */
adas_status adas_sparse_attn_bwd(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                 const void* k_cube, const void* v_tok, const void* k_vt, int32_t n_extra,
                                 const void* q_extra, const int32_t* sel_count, const int32_t* sel_idx,
                                 const void* out_raster, const void* out_extra, const float* lse,
                                 const void* dout_raster, const void* dout_extra, float* dq_raster,
                                 float* dq_extra, float* dk_raster, float* dv_raster, int32_t n_text_kv,
                                 const void* k_text, const void* v_text, float* dk_text, float* dv_text,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * adas_cache_append -- grow a video KV cache while decoding: frames arrive in
 * order and are written straight into the cube layout, and the mean key of
 * every cube is formed as soon as its last frame arrives (streaming extension
 * of key designs 1 and 2; selection needs a cube's mean key, so a cube is
 * selectable once its temporal block is complete).
 *   geom      the whole cache: T = frames the cache can hold (or cache_T);
 *             bf16 only
 *   t0        frames already in the cache (0 for the first call)
 *   n_frames  frames in this call; t0 + n_frames <= capacity
 *   k_new, v_new [n_frames*H*W][Hkv][d]  the new frames' keys and values,
 *             raster order within the new frames
 *   k_cache   [Hkv][NS][d] (ADAS_LAYOUT_TOKENS), v_cache [Hkv][NS/S][d][S]
 *             (ADAS_LAYOUT_VT), kbar [Hkv][NS/S][d] float32
 *   ksum      float64 running sums of the unfinished temporal block,
 *             adas_cache_sum_bytes() bytes, caller-owned, kept between calls
 *             (no initialisation needed: a block that starts in a call starts
 *             from zero)
 * After the call the first t0 + n_frames frames of the cache are laid out as
 * adas_cube_partition lays out the whole prefix, and kbar holds the mean
 * keys of every cube of the completed temporal blocks, bit-identical to
 * adas_cube_mean_keys.  Decode then uses a geometry with T = the completed
 * frames and cache_T = the capacity.
 * Errors: NULL, SHAPE (frame range, grid), DTYPE (not bf16), HIP.
 */
adas_status adas_cache_append(const adas_geom* geom, adas_dtype dtype, int32_t t0, int32_t n_frames,
                              const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              float* kbar, double* ksum, void* stream);

/* Bytes of the running-sum state adas_cache_append keeps (host only). */
size_t adas_cache_sum_bytes(const adas_geom* geom);

/* Bytes of workspace `kind` needs (host only, no device work).  has_video is
 * 1 when q_cube will be non-NULL.  Returns 0 for invalid geometry. */
size_t adas_workspace_bytes(const adas_geom* geom, adas_dtype dtype, adas_ws_kind kind,
                            int32_t has_video, int32_t n_extra);

/* Entries sel_idx must hold (host only).  Returns -1 for invalid geometry. */
int64_t adas_sel_capacity(const adas_geom* geom, int32_t has_video, int32_t n_extra);

/* Static description of a status code. */
const char* adas_status_string(adas_status s);

/* Message for the last error on the calling thread ("" if none). */
const char* adas_last_error(void);

/* "major.minor" */
const char* adas_version(void);

/* ---------------------------------------------------------------------------
 * adas_sparse_attn_fwd_noalloc: adas_sparse_attn_fwd without a workspace
 * argument, for callers that cannot allocate device memory (work recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, layouts, results and errors are those of
 * adas_sparse_attn_fwd; the call allocates nothing.
 *
 * Its scratch (extra-row selection bitmaps and per-chunk partial rows, the
 * memory adas_workspace_bytes(ADAS_WS_ATTN, ...) sizes) is a device array of
 * ADAS_NOALLOC_SCRATCH_BYTES (16 MiB) that each GPU holds from the library's
 * first use on it until the process ends.  A call whose scratch would exceed
 * that returns ADAS_ERR_WORKSPACE and launches nothing; calls that need no
 * scratch (video rows only) never touch it.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (on different streams, or
 * from different threads without ordering) race on it and give undefined
 * results.  Calls on one stream are ordered and safe.  The array needs no
 * clearing between calls: each call writes all of the scratch it reads.
 * The first call on a device looks up the array's device address
 * (hipGetSymbolAddress) with that device current; a failure there returns
 * ADAS_ERR_HIP.
 * ------------------------------------------------------------------------- */
#define ADAS_NOALLOC_SCRATCH_BYTES (16u << 20)
adas_status adas_sparse_attn_fwd_noalloc(const adas_geom* geom, adas_dtype dtype, const void* q_cube,
                                         const void* k_cube, const void* v_cube, int32_t n_extra,
                                         int32_t n_text_kv, const void* q_extra, const void* k_text,
                                         const void* v_text, const int32_t* sel_count,
                                         const int32_t* sel_idx, void* out_raster, void* out_extra,
                                         void* stream);

/* ---------------------------------------------------------------------------
 * Measurement helpers (not part of the method).  Peak probes give the ceiling
 * the hardware sustains in isolation, so every stage of the path can be
 * reported against a measured peak as well as the published one.  They are
 * asynchronous on `stream` like the compute calls; the caller times them.
 *
 * adas_probe_mfma: `workgroups` workgroups of 4 waves, each wave running
 *   `iters` loop trips of 16 v_mfma_f32_32x32x16_bf16 (4 independent chains)
 *   on register operands.  *flops (host pointer, may be NULL) receives the
 *   dense bf16 FLOPs issued.  sink: device float[workgroups], never written
 *   in practice (it keeps the loop alive).  ADAS_ERR_VALUE for workgroups or
 *   iters < 1.
 * adas_probe_hbm_read: streams `bytes` (a positive multiple of 16) of src
 *   once with 16-byte loads; sink: device uint32[workgroups] (never written in
 *   practice).  workgroups < 1 means 8 per compute unit.
 * adas_probe_hbm_copy: copies `bytes` (a positive multiple of 16) from src to
 *   dst with 16-byte loads and stores.
 * adas_probe_attn_mix: `workgroups` workgroups of 8 waves (two per SIMD, as in
 *   the union attention), each wave running `iters` trips of 32
 *   v_mfma_f32_32x32x16_bf16 on four accumulators, with bf16 operands of
 *   random mantissas and signs.  mix = 0: the MFMAs alone.  mix = 1: with the
 *   attention's side work per MFMA (a 16-byte LDS operand read, an exp2 of an
 *   fma, half a bf16 pack and half a dot2 row-sum step), four 1 KB
 *   global->LDS loads per wave and trip from a 2 MB window of src, and a
 *   barrier every second trip.  src: device buffer of src_bytes >= 2 MiB
 *   (read, contents irrelevant; needed for mix = 1, may be NULL for 0).
 *   *flops (host, may be NULL) receives the FLOPs issued; sink: device
 *   float[workgroups], never written in practice.  ADAS_ERR_VALUE for
 *   workgroups or iters < 1 or mix not 0/1; ADAS_ERR_SHAPE for src_bytes below
 *   2 MiB or at least 2^31 when mix = 1.
 * ------------------------------------------------------------------------- */
adas_status adas_probe_mfma(int32_t workgroups, int32_t iters, float* sink, double* flops, void* stream);
adas_status adas_probe_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups,
                                void* stream);
adas_status adas_probe_hbm_copy(const void* src, void* dst, int64_t bytes, int32_t workgroups, void* stream);
adas_status adas_probe_attn_mix(int32_t workgroups, int32_t iters, int32_t mix, const void* src, int64_t src_bytes,
                                float* sink, double* flops, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ADAS_H */
