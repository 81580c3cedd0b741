/*
 * libnanokv -- compressed-history attention (NanoKV) for AMD Instinct MI355X.
 *
 * The method (NanoKV: High-Ratio KV Cache Compression for Autoregressive
 * Video Generation) keeps the historical K/V cache of an autoregressive video
 * model as, per token and per branch (K or V):
 *   - the index of a shared cluster center (abstract; Figure 4(a)),
 *   - r joint head-channel residual coefficients in INT4 (Figure 4(b)),
 * with centers, encoder and decoder fitted separately per K/V branch
 * (Table 5 caption).  History is read either full-dimensionally (decode,
 * then ordinary attention; Figure 4(a)) or, in NanoKV-Fast, through a fixed
 * routing policy that sends part of the history to a low-dimensional read in
 * coefficient space whose result is LSE-merged with the rest (Figure 4(d)).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - W = H * d.  Channel h*d + j of a [*, W] row belongs to head h.
 *  - Every array is a DEVICE pointer, row-major and contiguous, owned by the
 *    caller; the library allocates nothing, creates no streams or events
 *    (the opt-in profiling aid below aside) and keeps no state between calls
 *    (apart from the thread-local error string and the testing switch
 *    nkv_force_generic).  Scratch memory is the caller's `ws` buffer, sized
 *    by the matching *_workspace_size call.  Every kernel of a call runs on
 *    the caller's `stream`, in order.
 *  - Token, query, center, encoder, decoder and output tensors have the
 *    element type `nkv_shape.dtype`: NKV_F32 (float) or NKV_BF16 (bfloat16
 *    bit patterns in uint16).
 *  - Compressed records: idx int32 [N]; codes uint8 [N, r/2] (two's
 *    complement INT4, coefficient 2j in the low nibble of byte j); scales
 *    uint16 [N, r/group] holding IEEE fp16 bit patterns.  A group is `group`
 *    consecutive coefficients of one token; scale = fp16 round-half-even of
 *    max|z|/7 and code = clamp(round-half-even(z/scale), -8, 7); a zero scale
 *    means all-zero codes.
 *  - LSE outputs are natural-log, float32 [Nq, H].  An empty key set gives
 *    O = 0 and LSE = -inf.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued asynchronously on it; arguments are validated synchronously
 *    before anything is enqueued.  A device fault surfaces at the caller's
 *    next synchronisation.
 *  - Errors: a non-zero nkv_status; nkv_last_error() (thread-local) gives a
 *    description.  No C++ exception crosses this interface.  Center indices
 *    outside [0, A) in the inputs are undefined behaviour.
 *
 * Supported set (validated; NKV_EUNSUPPORTED otherwise): 1 <= H; d in
 * {16, 32, 64, 128}; r even, r % group == 0, group in {8, 16, 32, 64}; for
 * the Fast read 0 < r_low <= r.  The tuned MFMA kernels serve NKV_BF16 with
 * d == 128 (r and r_low multiples of 16); every other supported shape runs
 * on the generic HIP kernels.
 */
#ifndef NANOKV_H_
#define NANOKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NKV_VERSION 1
#define NKV_MAX_SEGMENTS 64

typedef enum {
  NKV_OK = 0,
  NKV_EINVAL = 1,        /* malformed arguments (null pointer, bad size) */
  NKV_EUNSUPPORTED = 2,  /* well-formed but outside the supported set   */
  NKV_EWORKSPACE = 3,    /* ws too small (see *_workspace_size)         */
  NKV_EHIP = 4           /* a HIP launch or runtime call failed         */
} nkv_status;

typedef enum { NKV_F32 = 0, NKV_BF16 = 1 } nkv_dtype;

typedef enum { NKV_FULL = 0, NKV_LOW = 1 } nkv_route;

typedef struct {
  int32_t H;            /* heads                                         */
  int32_t d;            /* head dimension                                */
  int32_t r;            /* coefficients per token and branch             */
  int32_t group;        /* INT4 group size (consecutive coefficients)    */
  int32_t dtype;        /* nkv_dtype of tokens/queries/codec/outputs     */
  float softmax_scale;  /* tau multiplying every score; <= 0 -> 1/sqrt(d) */
} nkv_shape;

/* One compressed branch (K or V): Figure 4(b) of the NanoKV pages. */
typedef struct {
  const int32_t* idx;      /* [N_hist] center index per token           */
  const uint8_t* codes;    /* [N_hist, r/2] packed INT4                 */
  const uint16_t* scales;  /* [N_hist, r/group] fp16 bits               */
  const void* centers;     /* [A, W] shared cluster centers             */
  const void* decoder;     /* [W, r] linear decoder D                   */
  int32_t A;               /* number of centers                         */
} nkv_branch;

/* A half-open range [begin, end) of history positions and its read mode
 * (Figure 4(d): a fixed policy routes history to full- or low-dimensional
 * attention).  Segments must be disjoint and together cover [0, N_hist);
 * at most NKV_MAX_SEGMENTS ranges per mode after adjacent ranges of the same
 * mode are joined.  Host memory; read during the call only. */
typedef struct {
  int64_t begin;
  int64_t end;
  int32_t mode;            /* NKV_FULL or NKV_LOW */
} nkv_segment;

/* Bytes of workspace nkv_encode needs for N tokens and A centers (0 when
 * none); SIZE_MAX if the shape is invalid. */
size_t nkv_encode_workspace_size(const nkv_shape* shape, int64_t N, int32_t A);

/*
 * Encoder of one branch (NanoKV abstract and Figure 4(b)): for each token
 * x_t (row of x [N, W]):
 *   a_t = argmin_a ||x_t - centers[a]||^2   (squared L2, ties -> lowest a)
 *   z_t = encoder (x_t - centers[a_t])       (encoder [r, W])
 *   INT4-quantise z_t per group (format above).
 * Writes idx[t], codes[t, :], scales[t, :].  Appending to a history is
 * pointer arithmetic on these outputs.  N == 0 is a no-op (ws may be NULL).
 */
nkv_status nkv_encode(const nkv_shape* shape, const void* x, int64_t N,
                      const void* centers, int32_t A, const void* encoder,
                      int32_t* idx, uint8_t* codes, uint16_t* scales,
                      void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for nkv_attend_full / nkv_attend_fast with the same
 * arguments (route == NULL, n_seg == 0 means "everything full").  SIZE_MAX
 * if the arguments are invalid. */
size_t nkv_attend_workspace_size(const nkv_shape* shape, int32_t A_k,
                                 int32_t A_v, int64_t N_hist,
                                 const nkv_segment* route, int32_t n_seg,
                                 int32_t r_low, int64_t Nq, int64_t N_cur);

/*
 * NanoKV full-dimensional read (Figure 4(a)/(b)): decode every history token
 * of both branches (x_hat = centers[idx] + decoder * (code * scale)), then
 * softmax attention per head with scores tau * q_h . k_h over the decoded
 * history followed by the uncompressed current chunk cur_k/cur_v [N_cur, W]
 * (ignored, and may be NULL, when N_cur == 0).  q [Nq, W]; out [Nq, W] (shape dtype);
 * lse [Nq, H] float32.  Nq == 0 is a no-op after validation (ws may be NULL).
 */
nkv_status nkv_attend_full(const nkv_shape* shape, const nkv_branch* k,
                           const nkv_branch* v, int64_t N_hist,
                           const void* q, int64_t Nq, const void* cur_k,
                           const void* cur_v, int64_t N_cur, void* out,
                           float* lse, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * NanoKV-Fast mixed-dimensional read (Figure 4(d)).  History positions in
 * NKV_FULL segments and the current chunk are read as in nkv_attend_full.
 * Positions in NKV_LOW segments are read in coefficient space with the
 * leading r_low coefficients of both branches; per head h, with D_{X,h} the
 * rows h*d..h*d+d-1 of decoder X:
 *   q~_h   = D_{K,h}[:, :r_low]^T q_h                        (query reduction)
 *   s_t    = tau * (q~_h . c^K_t[:r_low] + q_h . centers_K[a^K_t, h])
 *   O_low  = (D_{V,h}[:, :r_low] sum_t p_t c^V_t[:r_low]
 *             + sum_t p_t centers_V[a^V_t, h]) / sum_t p_t   (restoration)
 * with p_t = exp(s_t - max s).  The two partial results are LSE-merged.
 */
nkv_status nkv_attend_fast(const nkv_shape* shape, const nkv_branch* k,
                           const nkv_branch* v, int64_t N_hist,
                           const nkv_segment* route, int32_t n_seg,
                           int32_t r_low, const void* q, int64_t Nq,
                           const void* cur_k, const void* cur_v,
                           int64_t N_cur, void* out, float* lse, void* ws,
                           size_t ws_bytes, void* stream);

/* Workspace bytes for nkv_attend_fast_heads with the same arguments;
 * SIZE_MAX if the arguments are invalid. */
size_t nkv_attend_heads_workspace_size(const nkv_shape* shape, int32_t A_k,
                                       int32_t A_v, int64_t N_hist,
                                       const nkv_segment* route, int32_t n_seg,
                                       const int32_t* r_low_h, int64_t Nq,
                                       int64_t N_cur);

/*
 * NanoKV-Fast with a low-dimensional width per head (the deployed
 * configurations mix heads read at 32, 64, 96 and 128 dimensions; Table 6 of
 * the NanoKV page): identical to nkv_attend_fast except that head h reads
 * the NKV_LOW segments with the leading r_low_h[h] coefficients.  r_low_h is
 * a host array of H ints, each in [1, r], read before the call returns; H
 * may be at most 128 (NKV_EUNSUPPORTED otherwise, or for a width outside
 * [1, r]).  Heads of equal width share one pass of the low-dimensional
 * kernels.
 */
nkv_status nkv_attend_fast_heads(const nkv_shape* shape, const nkv_branch* k,
                                 const nkv_branch* v, int64_t N_hist,
                                 const nkv_segment* route, int32_t n_seg,
                                 const int32_t* r_low_h, const void* q,
                                 int64_t Nq, const void* cur_k,
                                 const void* cur_v, int64_t N_cur, void* out,
                                 float* lse, void* ws, size_t ws_bytes,
                                 void* stream);

/* Query-reduction and output-restoration maps of the low-dimensional read
 * (Figure 4(d) reduces the queries and restores the output dimension;
 * Table 8 of the NanoKV page compares the analytical maps with adapted
 * ones).  Both are [W, ld] device arrays of the shape's dtype, row-major;
 * head h uses rows h*d..h*d+d-1 and the leading r_low_h[h] columns.  The
 * analytical maps are the decoders: q_map = D_K, o_map = D_V, ld = r. */
typedef struct {
  const void* q_map;
  const void* o_map;
  int32_t ld;              /* columns of both maps, >= every r_low_h[h] */
} nkv_low_maps;

/* Workspace bytes for nkv_attend_fast_maps with the same arguments;
 * SIZE_MAX if they are invalid. */
size_t nkv_attend_maps_workspace_size(const nkv_shape* shape, int32_t A_k,
                                      int32_t A_v, int64_t N_hist,
                                      const nkv_segment* route, int32_t n_seg,
                                      const int32_t* r_low_h,
                                      const nkv_low_maps* maps, int64_t Nq,
                                      int64_t N_cur);

/*
 * NanoKV-Fast with per-head widths and caller-given low-dimensional maps:
 * identical to nkv_attend_fast_heads except that, for head h with width
 * w = r_low_h[h] and M_X,h the block rows h*d..h*d+d-1, columns 0..w-1 of
 * map X,
 *   q~_h  = M_{q,h}^T q_h
 *   O_low = (M_{o,h} sum_t p_t c^V_t[:w] + sum_t p_t centers_V[a^V_t, h])
 *           / sum_t p_t.
 * The scores still use the stored K coefficients and centers.  With the
 * analytical maps the result equals nkv_attend_fast_heads.  The tuned
 * kernels need ld % 8 == 0 and 16-byte aligned maps; other maps run on the
 * generic kernels.
 */
nkv_status nkv_attend_fast_maps(const nkv_shape* shape, const nkv_branch* k,
                                const nkv_branch* v, int64_t N_hist,
                                const nkv_segment* route, int32_t n_seg,
                                const int32_t* r_low_h,
                                const nkv_low_maps* maps, const void* q,
                                int64_t Nq, const void* cur_k,
                                const void* cur_v, int64_t N_cur, void* out,
                                float* lse, void* ws, size_t ws_bytes,
                                void* stream);

/* Scratch bytes of nkv_encode_noalloc's fixed device array (32 MiB). */
#define NKV_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * nkv_encode without a workspace and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * results as nkv_encode (bit for bit: the same kernels run), with the
 * scratch taken from a fixed device array of NKV_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.
 * Limit: calls whose nkv_encode_workspace_size exceeds that size return
 * NKV_EUNSUPPORTED before touching the device (at W = 3072, A = 1024,
 * r = 384 a 4680-token chunk needs 22.3 MiB and about 6700 tokens fit;
 * split larger inputs into several calls).  Every call
 * on one GPU shares the array: calls that overlap on one GPU (several
 * streams or host threads) race and must be serialised by the caller.
 * Nothing of an earlier call's contents is read.
 */
nkv_status nkv_encode_noalloc(const nkv_shape* shape, const void* x, int64_t N,
                              const void* centers, int32_t A,
                              const void* encoder, int32_t* idx,
                              uint8_t* codes, uint16_t* scales, void* stream);

/*
 * LSE merge of two partial attentions over disjoint key sets (Figure 4(d)):
 *   L = log(exp(L_a) + exp(L_b)),  O = exp(L_a - L) O_a + exp(L_b - L) O_b.
 * o_a, o_b float32 [Nq, H*d]; lse_a, lse_b, lse_out float32 [Nq, H]; out
 * [Nq, H*d] of out_dtype.  A -inf partition contributes nothing; if both are
 * -inf, O = 0 and L = -inf.  Any d >= 1 (four channels per step when
 * d % 4 == 0 and the rows are 16-byte aligned, one otherwise).
 * Aliasing: with out_dtype == NKV_F32, `out` may be the very array o_a or
 * o_b, and lse_out may be lse_a or lse_b; any other overlap (a bf16 `out`
 * over a part's bytes, a shifted view) returns NKV_EINVAL.
 */
nkv_status nkv_lse_merge(int64_t Nq, int32_t H, int32_t d, const float* o_a,
                         const float* lse_a, const float* o_b,
                         const float* lse_b, void* out, int32_t out_dtype,
                         float* lse_out, void* stream);

/* Workspace bytes for nkv_fit_centers (never 0); SIZE_MAX if invalid. */
size_t nkv_fit_workspace_size(const nkv_shape* shape, int64_t N, int32_t A);

/*
 * Center fitting for one branch (the NanoKV page fits K and V centers
 * separately, Table 5 caption, without printing how; this is Lloyd's
 * k-means).  `centers` [A, W] holds the initial centers and receives the
 * fitted ones.  Each of `iters` iterations assigns every row of x [N, W] to
 * its nearest center exactly as nkv_encode does (squared L2, ties to the
 * lowest index), then replaces every center that received rows by their
 * mean, rounded once (half to even) to the shape dtype; a center that
 * received none keeps its value.  Optional outputs (NULL to skip): idx [N]
 * int32, each row's nearest center among the returned centers; counts [A]
 * int32, rows per returned center under that assignment.  iters == 0 only
 * assigns.  x must be 16-byte aligned (NKV_EINVAL otherwise).  Means are
 * summed in fp64 (see the implementation for when the sum is
 * order-independent).
 */
nkv_status nkv_fit_centers(const nkv_shape* shape, const void* x, int64_t N,
                           void* centers, int32_t A, int32_t iters,
                           int32_t* idx, int32_t* counts, void* ws,
                           size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Rollout support: per-layer routing policy, per-layer compressed cache and
 * storage accounting.  Every chunk of an autoregressive rollout attends, at
 * every layer, to that layer's history plus its own keys/values; once the
 * chunk is final its K and V are encoded and appended to the history
 * (Figure 4(a)/(b)).
 * ------------------------------------------------------------------------ */

/* Full-dimensional routing policy of one layer (Table 7 of the NanoKV page:
 * recent latent frames, one anchor per F older frames, sink frames, all of a
 * short history, full-layer fallback).  History positions form latent frames
 * of frame_tokens consecutive tokens, oldest first; a ragged last frame is a
 * frame.  With n_frames frames in the history, frame f is read NKV_FULL when
 *   layer_full != 0, or n_frames <= all_full_frames, or f < sink_frames,
 *   or f >= n_frames - recent_frames,
 *   or anchor_every > 0 and f % anchor_every == 0,
 * and NKV_LOW otherwise.  Counts are non-negative; frame_tokens > 0. */
typedef struct {
  int64_t frame_tokens;
  int32_t recent_frames;
  int32_t sink_frames;
  int32_t anchor_every;     /* 0: no anchors */
  int32_t all_full_frames;  /* 0: none */
  int32_t layer_full;       /* non-zero: the whole layer is read full */
} nkv_route_policy;

/* Segments of `policy` for a history of n_hist tokens, oldest first,
 * adjacent frames of one mode joined into one segment (n_hist == 0 gives no
 * segment).  Host-only: writes *n_out and, if *n_out <= max_out, the
 * segments to out (host memory).  NKV_EINVAL for a malformed policy, or when
 * more than max_out segments are needed (*n_out then holds the number
 * needed). */
nkv_status nkv_route_segments(const nkv_route_policy* policy, int64_t n_hist,
                              nkv_segment* out, int32_t max_out,
                              int32_t* n_out);

/* Persistent bytes of one layer's compressed history (Figure 8 of the NanoKV
 * page splits storage into cached data and resident operators; Table 1
 * reports the effective compression ratio against the uncompressed cache).
 *   cached    = idx (4 B) + codes (r/2 B) + scales (2 r/group B) per token,
 *               for both branches;
 *   resident  = centers [A_k + A_v, W] + encoders 2 x [r, W]
 *               + decoders 2 x [W, r] at the element size of shape->dtype;
 *   original  = K and V of the same tokens in bf16 (2 B per value). */
typedef struct {
  int64_t idx, codes, scales, cached;
  int64_t centers, encoders, decoders, resident;
  int64_t total;          /* cached + resident */
  int64_t original;
  double cr_effective;    /* original / total (0 when total == 0) */
  double cr_cached;       /* original / cached (0 when cached == 0) */
  double cr_nominal;      /* (W x 16 bit) / (r x 4 bit) */
} nkv_storage;

/* Host-only; NKV_EINVAL for a NULL or invalid argument. */
nkv_status nkv_storage_account(const nkv_shape* shape, int32_t A_k,
                               int32_t A_v, int64_t n_hist, nkv_storage* out);

/* One branch of a layer cache: history arrays with room for `capacity`
 * tokens (layout as for nkv_encode) and the branch's codec. */
typedef struct {
  int32_t* idx;            /* [capacity]                                  */
  uint8_t* codes;          /* [capacity, r/2]                             */
  uint16_t* scales;        /* [capacity, r/group]                         */
  const void* centers;     /* [A, W]                                      */
  const void* encoder;     /* [r, W]                                      */
  const void* decoder;     /* [W, r]                                      */
  int32_t A;
} nkv_cache_branch;

/* The compressed history of one layer.  Device arrays are the caller's;
 * n_hist is maintained by nkv_layer_append (host field, advanced when the
 * encode work is enqueued, so stream order keeps later reads consistent). */
typedef struct {
  nkv_cache_branch k, v;
  int64_t n_hist;
  int64_t capacity;
} nkv_layer_cache;

/* Workspace bytes for nkv_layer_attend with the same arguments; SIZE_MAX if
 * they are invalid. */
size_t nkv_layer_attend_workspace_size(const nkv_shape* shape,
                                       const nkv_layer_cache* cache,
                                       const nkv_route_policy* policy,
                                       const int32_t* r_low_h, int64_t Nq,
                                       int64_t N_cur);

/*
 * Attention of one layer for one chunk: the chunk's queries q [Nq, W] over
 * the layer's history routed by `policy` (nkv_route_segments) plus the
 * chunk's own cur_k/cur_v [N_cur, W].  When every history frame is routed
 * full this is nkv_attend_full, otherwise nkv_attend_fast_heads with the
 * per-head widths r_low_h (host array of H ints; may be NULL only when the
 * policy routes the whole current history full).  Outputs as nkv_attend_full.
 */
nkv_status nkv_layer_attend(const nkv_shape* shape,
                            const nkv_layer_cache* cache,
                            const nkv_route_policy* policy,
                            const int32_t* r_low_h, const void* q, int64_t Nq,
                            const void* cur_k, const void* cur_v,
                            int64_t N_cur, void* out, float* lse, void* ws,
                            size_t ws_bytes, void* stream);

/* Workspace bytes for nkv_layer_append of N tokens; SIZE_MAX if invalid. */
size_t nkv_layer_append_workspace_size(const nkv_shape* shape,
                                       const nkv_layer_cache* cache,
                                       int64_t N);

/*
 * Encode a finished chunk's K and V rows (k_new, v_new [N, W]) with the
 * layer's codecs (as nkv_encode) into positions [n_hist, n_hist + N) of the
 * cache, then advance cache->n_hist by N.  NKV_EINVAL, with nothing
 * enqueued and n_hist unchanged, if the arrays lack room
 * (n_hist + N > capacity).
 */
nkv_status nkv_layer_append(const nkv_shape* shape, nkv_layer_cache* cache,
                            const void* k_new, const void* v_new, int64_t N,
                            void* ws, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* nkv_status_string(nkv_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* nkv_last_error(void);
int nkv_version(void);

/* Testing aid: 1 routes every call through the generic HIP kernels even
 * where the tuned MFMA kernels apply; 0 (default) restores the dispatch. */
void nkv_force_generic(int on);

/* Profiling aid, off by default.  While enabled, each kernel stage of the
 * tuned path is bracketed by HIP events recorded on the call's stream; these
 * events are the only HIP objects the library ever creates (kept in a pool
 * for reuse until the process ends).  Calls from several host threads are
 * safe: one lock covers the record list.  nkv_profile_read waits for the
 * recorded events, writes up to max_entries per-stage totals (elapsed
 * milliseconds and number of launches) and clears them; it returns the
 * number of stages written, or -1 on a HIP error. */
typedef struct {
  char name[32];
  double ms;
  int32_t count;
} nkv_prof_entry;

void nkv_profile_enable(int on);
int nkv_profile_read(nkv_prof_entry* out, int32_t max_entries);

#ifdef __cplusplus
}
#endif

#endif /* NANOKV_H_ */
