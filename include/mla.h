/*
 * mla.h -- C ABI of libmla: a latent KV cache with absorbed multi-head latent
 * attention for chunked video-token rollouts, on AMD MI355X (gfx950).
 *
 * The operations follow the VideoMLA pages ("VideoMLA: Low-Rank Latent KV Cache
 * for Minute-Scale Autoregressive Video Diffusion"; abstract, and the technical
 * summary's sections "problem definition" and "method", items 1-4):
 *   - per cached layer and per token, only the pair (c^KV_t, k^R_t) is stored:
 *     a content latent shared by all heads, c = W^KV_down x  (method item 1),
 *     and one positional key shared by all heads, rotated by 3D-RoPE over
 *     (latent frame, grid row, grid column)                   (method item 3);
 *   - the cache is a fixed-size sliding window of whole latent frames
 *     (problem definition: a 21-latent-frame window);
 *   - attention rebuilds each head's content key and value from the latent
 *     with per-head up-projections W^K_up, W^V_up            (method item 2).
 *     This library computes that result in two ways (see mla_attend_path):
 *     in absorbed form - W^K_up folded into each head's query, softmax(.)·C
 *     accumulated in latent space, W^V_up applied afterwards (equal by
 *     associativity) - or, for long query chunks where it needs fewer
 *     products, by rebuilding every resident key's per-head key and value
 *     once per call and running per-head attention over them.
 * A dense per-head K/V cache (problem definition: every cached token stores
 * full keys and values for every head) is provided with the same conventions
 * as the in-run comparison.
 *
 * Conventions
 *   - All matrices are row-major; weights map column vectors, y = W x:
 *       w_dkr [d_c + d_rope][hidden]  rows < d_c: W^KV_down, rows >= d_c: W^KR
 *       w_uk  [n_h][d_nope][d_c]      k^nope_h = w_uk[h] c
 *       w_uv  [n_h][d_v][d_c]         v_h      = w_uv[h] c
 *       w_k, w_v (dense) [n_h*d_h][hidden], d_h = d_nope + d_rope
 *   - Tokens of a latent frame are row-major over the grid (row, column);
 *     token tau of frame f has global index f*T + tau, T = grid_h*grid_w, and
 *     position (f, tau / grid_w, tau % grid_w).
 *   - 3D-RoPE rotates adjacent element pairs (2p, 2p+1); the first
 *     rope_pairs_t pairs follow the frame axis, the next rope_pairs_h the row
 *     axis, the last rope_pairs_w the column axis; pair i of an axis group with
 *     P_a pairs turns by pos_axis * rope_base^(-i / P_a) radians.
 *   - Score scale is 1/sqrt(d_nope + d_rope); every resident token is a key
 *     (no mask inside the window).
 *   - Ring slot of token tau of frame f: (f mod window_frames)*T + tau; batch
 *     element b's rows start at b*window_frames*T.  Latent rows hold
 *     [c (d_c) | k^R rotated (d_rope)]; dense rows hold [K: n_h x d_h | V: n_h x d_h].
 *   - x, q and weights have the config's dtype (bf16 or fp32); the ring stores
 *     cache_dtype (fp32 with fp32 inputs; bf16 or fp16 with bf16 inputs: two
 *     bytes per stored scalar either way, the per-token count of method
 *     item 4 at the 2-byte width the problem definition's ~6.0 GB implies).
 *     On the absorbed path prepared queries and softmax weights enter the
 *     matrix units in the cache type; with a bf16 ring each of them is
 *     carried as two bf16 parts (the value and the bf16 rounding of its
 *     remainder; twice the matrix work), since bf16's 8 significant bits
 *     alone move the output by about 1e-3 of its size.  The expand path
 *     rebuilds fp16 per-head keys and values for every ring type and runs
 *     its attention on fp16 operands.  Every sum is fp32 and the attention
 *     output is fp32.
 *   - Range: an fp16 ring holds magnitudes up to 65504; a computed c or k^R
 *     value beyond that is stored as +-infinity (IEEE round to nearest),
 *     and attention over such a row returns NaN for its sequence.  bf16 and
 *     fp32 rings have the fp32 exponent range.
 *   - One-byte latent ring (MLA_E4M3; beyond the pages, which imply two-byte
 *     scalars): the OCP 8-bit float E4M3 ('fn': 4 significant bits, largest
 *     magnitude 448, subnormal quantum 2^-9, no infinities), rounded to
 *     nearest even; magnitudes that round past 448 are stored as +-448
 *     (saturation, never NaN or infinity).  The attention widens the stored
 *     values to fp16 (exactly) and computes as for an fp16 ring: the result
 *     is the attention over the stored E4M3 values.  Both attention paths:
 *     the expand-then-attend path widens the rows as it rebuilds the per-head
 *     keys and values, which it rounds to fp16 as for an fp16 ring.  No dense
 *     (mha_*) caches.
 *
 * Ownership: the caller owns every device buffer (ring storage, weights,
 * activations, outputs, workspace).  The library owns only the small host
 * handle and never allocates device memory.
 *
 * Errors: every check runs before anything is enqueued; on error the handle's
 * state and all memory are unchanged.  A failed kernel launch returns
 * MLA_ERR_HIP; faults inside kernels surface at the caller's next
 * synchronisation.  No C++ exception crosses this interface.
 *
 * Concurrency: a handle is not thread-safe.  Calls on one stream are ordered;
 * ordering across streams is the caller's job.  Device pointers must be
 * 16-byte aligned.  `stream` is a hipStream_t (NULL = the null stream).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,       /* bad config, null/misaligned pointer, bad size */
  MLA_ERR_STORAGE_TOO_SMALL = 2, /* storage_bytes < mla_cache_bytes(cfg)           */
  MLA_ERR_FULL = 3,              /* write would exceed the window's free frames    */
  MLA_ERR_NOT_CONTIGUOUS = 4,    /* write does not continue the newest frame       */
  MLA_ERR_EVICT_RANGE = 5,       /* evicting more frames than are resident         */
  MLA_ERR_EMPTY = 6,             /* attend on an empty window                      */
  MLA_ERR_WORKSPACE = 7,         /* workspace missing or smaller than required     */
  MLA_ERR_UNSUPPORTED = 8,       /* shape valid but not built for this dtype       */
  MLA_ERR_WRONG_KIND = 9,        /* latent call on a dense handle or vice versa    */
  MLA_ERR_HIP = 10,              /* kernel launch failed                           */
  MLA_ERR_SCRATCH = 11           /* call needs more than the static scratch        */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_F16 = 2, MLA_E4M3 = 3 } mla_dtype;

typedef struct {
  int32_t hidden;         /* layer input width                                  */
  int32_t n_heads;        /* n_h                                                */
  int32_t d_nope;         /* per-head content part of q.k                       */
  int32_t d_rope;         /* shared positional key width (even)                 */
  int32_t d_v;            /* per-head value width                               */
  int32_t d_c;            /* shared content latent width                        */
  int32_t grid_h, grid_w; /* tokens per latent frame T = grid_h*grid_w          */
  int32_t window_frames;  /* ring capacity W in whole latent frames             */
  int32_t batch;          /* B independent sequences on one schedule            */
  int32_t rope_pairs_t, rope_pairs_h, rope_pairs_w; /* sum = d_rope/2 (latent) */
  float rope_base;        /* frequency base, e.g. 10000                         */
  int32_t dtype;          /* inputs (x, q, weights): MLA_BF16 or MLA_F32         */
  int32_t cache_dtype;    /* ring storage: MLA_F32 with fp32 inputs; MLA_BF16 or
                             MLA_F16 with bf16 inputs (2 bytes per scalar);
                             MLA_E4M3 with bf16 inputs, latent caches only
                             (1 byte per scalar)                                */
} mla_layer_config;

typedef struct {
  int64_t oldest_frame;   /* first resident frame (== newest+1 when empty)      */
  int64_t newest_frame;   /* last resident frame                                */
  int32_t n_resident_frames;
  int32_t capacity_frames;
} mla_cache_info;

typedef struct mla_cache mla_cache; /* opaque host handle, one per cached layer */

/* Bytes of ring storage for one latent layer (method item 4: d_c + d_rope
 * scalars per token instead of 2 * n_h * d_h):
 * batch * window_frames * T * (d_c + d_rope) * sizeof(cache_dtype).  0 on a bad config. */
size_t mla_cache_bytes(const mla_layer_config* cfg);

/* Bytes of ring storage for one dense layer:
 * batch * window_frames * T * 2 * n_heads * (d_nope + d_rope) * sizeof(cache_dtype). */
size_t mha_cache_bytes(const mla_layer_config* cfg);

/* Create a latent-cache handle over caller-owned `storage` (device memory of at
 * least mla_cache_bytes(cfg)).  The window starts empty.  The storage content
 * is not touched. */
mla_status mla_cache_create(const mla_layer_config* cfg, void* storage, size_t storage_bytes,
                            mla_cache** out);

/* Same for a dense per-head K/V cache (the comparison path). */
mla_status mha_cache_create(const mla_layer_config* cfg, void* storage, size_t storage_bytes,
                            mla_cache** out);

/* Free the host handle only; the storage stays the caller's. NULL is ignored. */
void mla_cache_destroy(mla_cache* cache);

/* Fused cache write (method items 1 and 3): for n_frames whole latent frames
 * starting at global frame `frame0`, per token computes
 *   c = W^KV_down x,  k^R = RoPE3D(W^KR x, position),
 * rounds both to cache_dtype (nearest even) and stores [c | k^R] at the
 * token's ring slot.  x: [batch][n_frames*T][hidden]; w_dkr as above.
 * Needs frame0 == newest+1 unless the window is empty (MLA_ERR_NOT_CONTIGUOUS),
 * and n_frames <= capacity - resident (MLA_ERR_FULL): nothing is overwritten
 * silently.  The new frames become resident when the call returns. */
mla_status mla_cache_write(mla_cache* cache, const void* x, const void* w_dkr, int64_t frame0,
                           int32_t n_frames, void* stream);

/* Fused cache write with the latent RMS-normalised before it is stored:
 *   c = gamma * (W^KV_down x) / sqrt(mean((W^KV_down x)^2) + eps),
 *   k^R = RoPE3D(W^KR x, position) (not normalised),
 * otherwise as mla_cache_write.  The pages store the latent of method item 1
 * and print no normalisation of it; this is the normalisation an MLA layer
 * commonly applies to its latent before the up-projections, offered for
 * layers that have one.  gamma: [d_c] gain in the input dtype (bf16); eps >= 0.
 * MLA_ERR_UNSUPPORTED unless bf16 inputs and d_c + d_rope in {96, 160, 224}. */
mla_status mla_cache_write_norm(mla_cache* cache, const void* x, const void* w_dkr, const void* gamma,
                                float eps, int64_t frame0, int32_t n_frames, void* stream);

/* Dense comparison write: per head k_h = RoPE3D((w_k x)_h) over all d_h dims
 * (pairs split t/h/w as P - 2*floor(P/3), floor(P/3), floor(P/3), P = d_h/2),
 * v_h = (w_v x)_h, rounded to cache_dtype. Same window rules. */
mla_status mha_cache_write(mla_cache* cache, const void* x, const void* w_k, const void* w_v,
                           int64_t frame0, int32_t n_frames, void* stream);

/* Slide the window (abstract: a fixed-size sliding-window KV cache; problem
 * definition: a window of 21 latent frames): drop the n_frames oldest
 * resident frames (host-side bookkeeping only; launches nothing).  MLA_ERR_EVICT_RANGE if n_frames is
 * negative or larger than the resident count. Works on both handle kinds. */
mla_status mla_cache_evict(mla_cache* cache, int32_t n_frames);

/* Read the window state. */
mla_status mla_cache_query(const mla_cache* cache, mla_cache_info* info);

/* Restore a saved window state (resume from a snapshot of the storage).
 * Requires 0 <= oldest, newest >= oldest-1, newest-oldest+1 <= capacity. */
mla_status mla_cache_set_state(mla_cache* cache, int64_t oldest_frame, int64_t newest_frame);

/* Ring slot of token tau of frame `frame` (independent of residency), or -1 on
 * bad arguments.  Same for every batch element. */
int64_t mla_cache_slot(const mla_cache* cache, int64_t frame, int32_t tau);

/* Device workspace mla_attend needs for Lq queries with `key_splits` key
 * ranges (0 = the library's choice for this shape), on this handle's current
 * attend path: the largest over every number of resident frames, so one
 * buffer serves the window as it fills and slides. */
size_t mla_attend_workspace_bytes(const mla_cache* cache, int32_t Lq, int32_t key_splits);

/* Absorbed latent attention (method item 2 in absorbed form) of a query chunk
 * over every resident token of the window:
 *   q     [batch][Lq][n_h][d_nope + d_rope], per head [q^nope | q^R], q^R not yet
 *         rotated; query row i sits at global token q_token0 + i;
 *   out   [batch][Lq][n_h][d_v] fp32, out_h = W^V_up,h (sum_j p_j c_j),
 *         p = softmax_j((q^nope.W^K_up,h c_j + RoPE3D(q^R).k^R_j) / sqrt(d_nope+d_rope)).
 * The work is spread evenly over the compute units (stream-K); row groups
 * whose keys end up on several units are merged exactly by log-sum-exp.
 * key_splits = 0 lets the library choose; > 0 cuts every row group's key
 * range into about that many pieces.  workspace: device memory of at least
 * mla_attend_workspace_bytes(cache, Lq, key_splits).  MLA_ERR_EMPTY if no frame
 * is resident.
 * Graph capture: the call enqueues only kernels on `stream` (no memset, no
 * allocation, no host synchronisation), so it can be captured into a HIP
 * graph.  A captured call keeps its arguments and the window state of the
 * capture (resident key count, first slot, attend path): replay it for new
 * contents of the same buffers, and capture again after a write, an
 * eviction or a state change. */
mla_status mla_attend(mla_cache* cache, const void* q, int64_t q_token0, int32_t Lq,
                      const void* w_uk, const void* w_uv, float* out, int32_t key_splits,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Query-side RMS norm for later mla_attend calls on this latent handle (and
 * mla_attend_noalloc): each head's query row [q^nope | q^R] is replaced by
 *   gamma * q_h / sqrt(mean(q_h^2) + eps)   (mean over its d_nope + d_rope values)
 * before its rotation and the folding of W^K_up, the same gain for every head.
 * The pages print no normalisation (technical summary, method items 2-3); a
 * query norm leaves the absorption intact, while a norm of the per-head keys
 * would not (it acts on W^K_up,h c, after the up-projection), so the key-side
 * counterpart is the latent norm of mla_cache_write_norm.  gamma: device
 * pointer to [d_nope + d_rope] gains in the input dtype (bf16), 16-byte
 * aligned, owned by the caller and read by every attend while set; NULL
 * switches the norm off.  eps >= 0 and finite (with eps = 0 an all-zero query
 * row has no scale and its output is NaN).  Errors: MLA_ERR_INVALID_ARG
 * (null handle, misaligned gamma, bad eps), MLA_ERR_WRONG_KIND (dense
 * handle), MLA_ERR_UNSUPPORTED (fp32 handles).  While it is set,
 * mla_attend_block returns MLA_ERR_UNSUPPORTED (its folded projection never
 * forms the per-head queries). */
mla_status mla_cache_set_query_norm(mla_cache* cache, const void* gamma, float eps);

/* Allocation-free mla_attend, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation on the same path as mla_attend (the
 * handle's mla_attend_path for Lq and key_splits), with the workspace taken
 * from a static device array inside the library instead of the caller.  That
 * array holds mla_attend_noalloc_max_bytes() bytes (64 MiB) on every GPU the
 * library runs on, until the process ends; a call whose workspace in the
 * window's current state would exceed it returns MLA_ERR_SCRATCH and enqueues
 * nothing (decode-like calls of up to 16 queries fit at any batch up to 16).
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (different streams, different host threads) race and must
 * be ordered by the caller.  Other errors as mla_attend. */
mla_status mla_attend_noalloc(mla_cache* cache, const void* q, int64_t q_token0, int32_t Lq,
                              const void* w_uk, const void* w_uv, float* out, int32_t key_splits,
                              void* stream);

/* Size of mla_attend_noalloc's static scratch in bytes. */
size_t mla_attend_noalloc_max_bytes(void);

/* The attention block around the absorbed path, from the query tokens' layer
 * input to model width.  The layer's query projection gives each head
 * [q^nope | q^R] (method item 3: each head's q.k width split into content and
 * positional parts) and its output projection W^O maps the heads' outputs,
 * concatenated, to model width:
 *   w_q [n_h * (d_nope + d_rope)][hidden]   head h's rows [W^nope_q,h ; W^R_q,h]
 *   w_o [hidden][n_h * d_v]                 head h's columns take o_h
 * Folded at the weight level (once per weight set), W^K_up enters the query
 * projection and W^V_up the output projection:
 *   w_qf[h] = [W_uk,h^T W^nope_q,h ; W^R_q,h]     [n_h][d_c + d_rope][hidden]
 *   w_fo    = [W^O_1 W_uv,1 | ... | W^O_n W_uv,n]  [hidden][n_h * d_c]
 * each stored as two bf16 parts (the fp32 product rounded to bf16, then the
 * bf16 rounding of the remainder), so the folds keep 16 significant bits:
 * w_qf is [2][n_h][d_c + d_rope][hidden], w_fo is [2][hidden][n_h * d_c].
 * mla_fold_*_bytes give their sizes; the folds run on `stream`. */
size_t mla_fold_query_bytes(const mla_cache* cache);
size_t mla_fold_output_bytes(const mla_cache* cache);
mla_status mla_fold_query_weights(const mla_cache* cache, const void* w_q, const void* w_uk, void* w_qf,
                                  size_t w_qf_bytes, void* stream);
mla_status mla_fold_output_weights(const mla_cache* cache, const void* w_o, const void* w_uv, void* w_fo,
                                   size_t w_fo_bytes, void* stream);

/* Workspace of mla_attend_block (the largest over every number of resident
 * frames), 0 for handles without the block. */
size_t mla_attend_block_workspace_bytes(const mla_cache* cache, int32_t Lq, int32_t key_splits);

/* out = W_O [o_1; ...; o_n_h] for the queries q = W_q x of x [batch][Lq][hidden]
 * (row i at global token q_token0 + i), o_h the attention of mla_attend, in
 * absorbed form with the folded weights: [q_lat | q^R] from x in one product
 * (rotated and scaled in its epilogue), the latent core, the merged latent
 * outputs, then out [batch][Lq][hidden] fp32 = w_fo o_lat in one product.
 * MLA_ERR_UNSUPPORTED unless bf16 inputs, the absorbed core's head shapes,
 * hidden % 64 == 0 and n_h * d_c % 64 == 0, and while a query norm is set
 * (mla_cache_set_query_norm).  Other errors as mla_attend. */
mla_status mla_attend_block(mla_cache* cache, const void* x, int64_t q_token0, int32_t Lq,
                            const void* w_qf, const void* w_fo, float* out, int32_t key_splits,
                            void* workspace, size_t workspace_bytes, void* stream);

/* How mla_attend computes (mla_cache_set_attend_path / mla_attend_path).
 * MLA_PATH_ABSORBED: scores and value sums in the d_c-wide latent space with
 *   W^K_up folded into the queries and W^V_up applied after the softmax sum.
 * MLA_PATH_EXPAND: per-head keys [W^K_up,h c_j | k^R_j] and values W^V_up,h c_j
 *   of the whole window rebuilt once per call into the workspace, then plain
 *   per-head attention over them (method item 2 taken literally: the per-head
 *   keys and values are reconstructed from the latent on demand).  Needs fewer
 *   products per query than the absorbed form when d_c is large; the rebuild
 *   is a fixed cost per call, paid back from a few hundred queries on.
 * MLA_PATH_AUTO: the library picks: expand from 512 queries when the handle
 *   supports it, key_splits is 0 and the latent products per (query, key,
 *   head), 2 (d_c + d_rope) + 2 d_c, are at least 1.5 times the per-head ones,
 *   2 (d_nope + d_rope) + 2 d_v (d_c = 192 for the Wan head shape; not 128 or
 *   64, where the latent form is as fast or faster).  A bf16 ring, whose
 *   absorbed core issues every product twice, expands sooner: from 128
 *   queries when twice the latent products are at least 3 times the per-head
 *   ones (d_c = 192), from 256 when at least 2 times (d_c = 128), else from
 *   384 (d_c = 64).  Both paths compute the
 * same function; they differ in rounding.  Every ring type expands into
 * fp16 keys and values: a bf16 ring's rebuild multiplies its stored values on
 * bf16 matrix units (exact products, fp32 sums) and rounds the results to
 * fp16, so the expanded attention is as accurate as an fp16 ring's (the
 * split operands of the bf16 absorbed core are not needed) and has fp16's
 * range: a rebuilt key or value beyond 65504 in magnitude becomes
 * +-infinity and the sequence's output NaN. */
typedef enum { MLA_PATH_AUTO = 0, MLA_PATH_ABSORBED = 1, MLA_PATH_EXPAND = 2 } mla_attend_path_kind;

/* Selects the path of later mla_attend calls on this latent handle.
 * MLA_ERR_UNSUPPORTED for MLA_PATH_EXPAND unless the handle has bf16 inputs
 * (any two-byte or E4M3 ring), d_nope = 96, d_rope = 32, d_v = 128 and d_c in
 * {64, 128, 192}; MLA_ERR_WRONG_KIND on a dense handle. */
mla_status mla_cache_set_attend_path(mla_cache* cache, int32_t path);

/* Reuse of the expanded window across attends (enable = 1; 0 switches it off;
 * either call forgets the last expansion).  With reuse on, an expand-path
 * mla_attend skips rebuilding the per-head keys and values when the previous
 * expand-path attend on this handle used the same workspace pointer and the
 * same w_uk / w_uv pointers and no write, eviction or state change happened
 * since: several attends on one window state (denoising steps of a chunk,
 * several query chunks) then pay the rebuild once.  The caller guarantees
 * that it did not modify that workspace, the weights or the ring storage
 * outside this library in between, and orders the calls on one stream (or
 * synchronises between streams).  Off by default.  MLA_ERR_WRONG_KIND on a
 * dense handle. */
mla_status mla_cache_set_expand_reuse(mla_cache* cache, int32_t enable);

/* The path mla_attend takes for Lq queries and `key_splits` (MLA_PATH_ABSORBED
 * or MLA_PATH_EXPAND; -1 for bad arguments).  key_splits > 0 and fp32 handles
 * always take the absorbed path. */
int32_t mla_attend_path(const mla_cache* cache, int32_t Lq, int32_t key_splits);

/* Workspace for mha_attend (rotated, pre-scaled queries and key-range
 * partials), the largest over every number of resident frames. */
size_t mha_attend_workspace_bytes(const mla_cache* cache, int32_t Lq);

/* Dense comparison attention: per head, q rotated over all d_h dims,
 * softmax(q.k / sqrt(d_h)) . v over every resident token.
 * q [batch][Lq][n_h][d_h]; out [batch][Lq][n_h][d_h] fp32. */
mla_status mha_attend(mla_cache* cache, const void* q, int64_t q_token0, int32_t Lq, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Profiling hook: when `start`/`stop` are hipEvent_t handles (not NULL), each
 * later mla_attend / mha_attend on this handle records `start` on its stream
 * right before its main attention kernel and `stop` right after it, so a
 * caller can time that kernel alone with hipEventElapsedTime.  NULL, NULL
 * switches it off.  The events stay owned by the caller. */
mla_status mla_cache_set_profile_events(mla_cache* cache, void* start, void* stop);

/* Human-readable name of a status code (static string). */
const char* mla_status_str(mla_status status);

/* Library version string. */
const char* mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
