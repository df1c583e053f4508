// Host side of libmla: argument validation, sliding-window bookkeeping,
// workspace carving and kernel launches.  Implements include/mla.h.
//
// Window semantics (VideoMLA abstract: a fixed-size sliding-window KV cache;
// technical summary, problem definition: a window of latent frames): whole
// frames enter at the newest end and leave from the oldest end; token tau of
// frame f always lives at ring slot (f mod W)*T + tau.  Every check runs
// before anything is enqueued, so a failed call changes nothing.
#include <algorithm>
#include <functional>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/mla.h"
#include "mla_launch.h"

struct mla_cache {
  mla_layer_config cfg;
  bool dense;
  void* storage;
  size_t storage_bytes;
  int64_t oldest;  // first resident frame
  int64_t newest;  // last resident frame; empty when newest < oldest
  hipEvent_t prof_start;
  hipEvent_t prof_stop;
  int32_t attend_path;  // mla_attend_path: auto, absorbed or expand
  // Window generation: bumped by every write, eviction and state change.
  uint64_t gen;
  // mla_cache_set_expand_reuse: the last expansion (workspace, weights,
  // generation) may serve later expand-path attends while nothing changed.
  int32_t expand_reuse;
  bool ex_valid;
  const void* ex_ws;
  const void* ex_wuk;
  const void* ex_wuv;
  uint64_t ex_gen;
  uint64_t ex_token;  // the expansion's entry in the workspace record below
  // mla_cache_set_query_norm: gain (caller's device memory) and epsilon of the
  // RMS norm of each head's query row; null when off.
  const void* qn_gamma;
  float qn_eps;
};

namespace {

constexpr size_t kAlign = 256;

size_t elem_size(int32_t dtype) {
  if (dtype == MLA_E4M3) return 1;
  return (dtype == MLA_BF16 || dtype == MLA_F16) ? 2 : (dtype == MLA_F32 ? 4 : 0);
}

// Input / storage combinations with kernels: fp32 everywhere, or bf16 inputs
// with a 2-byte (bf16 or fp16) ring, or (latent caches only) a one-byte E4M3
// ring.
bool valid_types(const mla_layer_config* c, bool dense) {
  if (c->dtype == MLA_F32) return c->cache_dtype == MLA_F32;
  if (c->dtype == MLA_BF16)
    return c->cache_dtype == MLA_BF16 || c->cache_dtype == MLA_F16 ||
           (!dense && c->cache_dtype == MLA_E4M3);
  return false;
}

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t tokens_per_frame(const mla_layer_config& c) { return (int64_t)c.grid_h * c.grid_w; }

// Process-wide record of the workspace ranges that hold an expanded window:
// every attend on any handle first erases the entries its writes overlap, and
// an expansion then enters its own range under a fresh token.  A handle reuses
// an expansion only while that token is still on record, so a workspace
// written in between by another handle (or another attend of the same one)
// forces a rebuild.
struct WsRecord {
  uintptr_t lo, hi;
  uint64_t token;
};
std::mutex g_ws_mu;
std::vector<WsRecord> g_ws;
uint64_t g_ws_next_token = 1;

void ws_erase_if(const std::function<bool(const WsRecord&)>& pred) {
  g_ws.erase(std::remove_if(g_ws.begin(), g_ws.end(), pred), g_ws.end());
}

// The caller's next kernels write [p, p + n).
void ws_clobber(const void* p, size_t n) {
  const uintptr_t lo = (uintptr_t)p, hi = lo + n;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  ws_erase_if([&](const WsRecord& r) { return r.lo < hi && lo < r.hi; });
}

// [p, p + n) now holds a new expansion; returns its token.
uint64_t ws_enter(const void* p, size_t n) {
  const uintptr_t lo = (uintptr_t)p, hi = lo + n;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  ws_erase_if([&](const WsRecord& r) { return r.lo < hi && lo < r.hi; });
  const uint64_t t = g_ws_next_token++;
  g_ws.push_back({lo, hi, t});
  return t;
}

bool ws_holds(const void* p, size_t n, uint64_t token) {
  const uintptr_t lo = (uintptr_t)p, hi = lo + n;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (const WsRecord& r : g_ws)
    if (r.token == token) return r.lo == lo && r.hi == hi;
  return false;
}

void ws_forget(uint64_t token) {
  if (token == 0) return;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  ws_erase_if([&](const WsRecord& r) { return r.token == token; });
}

int64_t dense_width(const mla_layer_config& c) {
  return 2LL * c.n_heads * (c.d_nope + c.d_rope);
}

bool valid_config(const mla_layer_config* c, bool dense) {
  if (c == nullptr) return false;
  if (c->hidden <= 0 || c->n_heads <= 0 || c->d_nope < 0 || c->d_rope < 0 || c->d_v <= 0 ||
      c->d_c <= 0 || c->grid_h <= 0 || c->grid_w <= 0 || c->window_frames <= 0 || c->batch <= 0)
    return false;
  if (c->d_rope % 2 != 0 || c->d_nope + c->d_rope <= 0) return false;
  if (c->rope_pairs_t < 0 || c->rope_pairs_h < 0 || c->rope_pairs_w < 0) return false;
  if (!dense && c->rope_pairs_t + c->rope_pairs_h + c->rope_pairs_w != c->d_rope / 2) return false;
  if (dense && (c->d_nope + c->d_rope) % 2 != 0) return false;
  if (!(c->rope_base > 0.0f) || !isfinite(c->rope_base)) return false;
  if (!valid_types(c, dense)) return false;
  if (c->d_rope / 2 > mla::kMaxRopePairs) return false;
  if (dense && (c->d_nope + c->d_rope) / 2 > mla::kMaxRopePairs) return false;
  // ring rows, key counts and element offsets inside one sequence's ring are
  // kept in 32-bit integers inside the kernels
  const int64_t ring_rows = (int64_t)c->window_frames * tokens_per_frame(*c);
  if (ring_rows >= (1LL << 30)) return false;
  const int64_t row_elems = dense ? 2LL * c->n_heads * (c->d_nope + c->d_rope)
                                  : (int64_t)c->d_c + c->d_rope;
  if (ring_rows * row_elems >= (1LL << 31)) return false;
  return true;
}

mla::RopeTable make_rope(int pt, int ph, int pw, double base) {
  mla::RopeTable t;
  memset(&t, 0, sizeof(t));
  const int counts[3] = {pt, ph, pw};
  int p = 0;
  for (int axis = 0; axis < 3; ++axis)
    for (int i = 0; i < counts[axis]; ++i, ++p) {
      t.axis[p] = axis;
      t.inv_freq[p] = pow(base, -(double)i / (double)counts[axis]);
    }
  t.n_pairs = p;
  return t;
}

mla::RopeTable latent_rope(const mla_layer_config& c) {
  return make_rope(c.rope_pairs_t, c.rope_pairs_h, c.rope_pairs_w, (double)c.rope_base);
}

mla::RopeTable dense_rope(const mla_layer_config& c) {
  const int P = (c.d_nope + c.d_rope) / 2;
  return make_rope(P - 2 * (P / 3), P / 3, P / 3, (double)c.rope_base);
}

int64_t n_resident(const mla_cache* h) { return h->newest - h->oldest + 1; }

mla_status check_write(const mla_cache* h, int64_t frame0, int32_t n_frames) {
  if (n_frames <= 0 || frame0 < 0) return MLA_ERR_INVALID_ARG;
  const int64_t res = n_resident(h);
  if (res > 0 && frame0 != h->newest + 1) return MLA_ERR_NOT_CONTIGUOUS;
  if (res + n_frames > h->cfg.window_frames) return MLA_ERR_FULL;
  return MLA_OK;
}

void commit_write(mla_cache* h, int64_t frame0, int32_t n_frames) {
  if (n_resident(h) <= 0) h->oldest = frame0;
  h->newest = frame0 + n_frames - 1;
  ++h->gen;
}

// Schedule of the attention core (see mla::Schedule) for core shape `sh`
// whose key rows take `chunks_per_key` 16-byte LDS chunks.  Default: as many
// blocks as fit the device at once (one per compute unit for the widest shape),
// but no more than leave each at least kMinStepsPerBlock key tiles, so that
// partial writes stay small next to the work.  key_splits > 0 instead gives
// every row group key_splits blocks' worth of work, cutting its key range into
// about that many pieces.
constexpr int64_t kMinStepsPerBlock = 8;
// Cost of starting a segment, in key-tile steps (block finish times on the
// 4680-query chunk: a tail block's extra segments cost it about three steps
// each on the latent rows, about six on the shorter per-head steps).
constexpr int64_t kSegmentCostLatent = 3;
constexpr int64_t kSegmentCostDense = 6;

// chunks_per_key: 16-byte chunks of a cached key row; decode_chunks_per_key:
// those of the fp16 decode tile of a one-byte ring (0 otherwise).
mla::Schedule make_schedule(int64_t B, int64_t R, int64_t Lk, int32_t key_splits, int64_t cus,
                            mla::CoreShape sh, int chunks_per_key, int64_t seg_cost, bool split,
                            int decode_chunks_per_key = 0) {
  mla::Schedule s;
  sh = mla::core_shape_for_keys(sh, chunks_per_key);
  const int64_t br = (int64_t)sh.rows * sh.waves;
  const int64_t n_rg = (R + br - 1) / br;
  const int64_t n_kt = (Lk + sh.key_tile - 1) / sh.key_tile;
  const int64_t groups = B * n_rg;
  const int64_t total = groups * n_kt;
  int64_t nb;
  if (key_splits > 0) {
    nb = groups * key_splits;
  } else {
    const int64_t by_work = (total + kMinStepsPerBlock - 1) / kMinStepsPerBlock;
    const int64_t resident = cus * mla::core_blocks_per_cu(sh, chunks_per_key, split, decode_chunks_per_key);
    nb = resident < by_work ? resident : by_work;
  }
  if (nb < 1) nb = 1;
  const int64_t full = groups / nb;
  const int64_t rem = groups - full * nb;
  int64_t main_len = n_kt, tpb = 1;
  if (rem > 0) {
    main_len = (rem * n_kt + nb - 1) / nb;
    if (main_len > n_kt) main_len = n_kt;
    // A tail block starts a segment (queries in, tile ring drained, a partial
    // written) for every group its run touches - on average 1 + run / tail
    // length of them - and a main block once.  Counting seg_cost steps per
    // segment, move key tiles from the tail runs to the main blocks while that
    // lowers the larger of the two costs.
    auto cost = [&](int64_t ml) {
      const int64_t tail_len = n_kt - ml;
      if (tail_len <= 0 || nb <= rem) return (double)(ml + seg_cost);
      const int64_t run = (rem * tail_len + (nb - rem) - 1) / (nb - rem);
      const double tail_cost = run + seg_cost * (1.0 + (double)run / tail_len);
      return std::max((double)(ml + seg_cost), tail_cost);
    };
    while (main_len < n_kt && cost(main_len + 1) < cost(main_len)) ++main_len;
    const int64_t tail = rem * (n_kt - main_len);
    if (tail > 0) tpb = (tail + (nb - rem) - 1) / (nb - rem);
  }
  s.block_rows = (int)br;
  s.key_tile = sh.key_tile;
  s.stages = sh.stages;
  s.n_rg = (int)n_rg;
  s.n_kt = (int)n_kt;
  s.n_groups = (int)groups;
  s.n_blocks = (int)nb;
  s.full_rounds = (int)full;
  s.rem = (int)rem;
  s.main_len = (int)main_len;
  s.tail_per_block = (int)tpb;
  s.n_slots = (int)(main_len < n_kt ? 1 + (n_kt - main_len + tpb - 1) / tpb + 1 : 1);
  return s;
}

int64_t window_keys(const mla_cache* h) {
  const mla_layer_config& c = h->cfg;
  return n_resident(h) > 0 ? n_resident(h) * tokens_per_frame(c)
                           : (int64_t)c.window_frames * tokens_per_frame(c);
}

// A bf16 ring runs the attention core on split operands (query and
// probabilities as two bf16 parts; see mla_attn_core.h): bf16 keeps too few
// bits for them on their own.  fp16 rings and fp32 handles do not split.
bool split_operands(const mla_layer_config& c) { return c.cache_dtype == MLA_BF16; }

// The few-row core shapes (32-key tiles: up to 128 query rows per sequence)
// split each row's keys into many ranges, and their partial value sums are a
// large share of the call's memory traffic; with a 2-byte operand ring they
// are stored normalised as fp16 (half the bytes; values within the cache
// type's range).  Split-operand (bf16) rings keep fp32 partials.
bool fp16_partials(const mla_layer_config& c, const mla::Schedule& s) {
  return !split_operands(c) && c.dtype == MLA_BF16 && s.key_tile == 32 && c.d_v <= 256;
}

struct LatentLayout {
  mla::Schedule sched;
  size_t qcat_off, qlo_off, opart_off, ml_off, total;
  size_t ohi_off, olo_off;  // attention block: latent outputs in two bf16 parts
};

// Layouts for `Lk` resident keys (default: the handle's current window).
LatentLayout latent_layout(const mla_cache* h, int32_t Lq, int32_t key_splits, int64_t Lk = -1,
                           bool block = false) {
  const mla_layer_config& c = h->cfg;
  const int64_t R = (int64_t)Lq * c.n_heads;
  LatentLayout L;
  const bool split = split_operands(c);
  const bool f8 = c.cache_dtype == MLA_E4M3;  // one-byte rows, widened in the core
  const int row_chunks = (c.d_c + c.d_rope) / (f8 ? 16 : 8);
  L.sched = make_schedule(c.batch, R, Lk < 0 ? window_keys(h) : Lk, key_splits, mla::device_cu_count(),
                          mla::core_shape_for_rows(R, split), row_chunks, kSegmentCostLatent, split,
                          f8 ? (c.d_c + c.d_rope) / 8 : 0);
  const size_t width = (size_t)(c.d_c + c.d_rope);
  const size_t slots = (size_t)L.sched.n_slots;
  const size_t qbytes = round_up((size_t)c.batch * R * width * 2, kAlign);
  L.qcat_off = 0;
  L.qlo_off = qbytes;
  L.opart_off = split ? 2 * qbytes : qbytes;
  L.ml_off = L.opart_off + round_up(slots * c.batch * R * c.d_c * 4, kAlign);
  L.total = L.ml_off + round_up(slots * c.batch * R * 2 * 4, kAlign);
  L.ohi_off = L.olo_off = L.total;
  if (block) {
    const size_t obytes = round_up((size_t)c.batch * R * c.d_c * 2, kAlign);
    L.ohi_off = L.total;
    L.olo_off = L.ohi_off + obytes;
    L.total = L.olo_off + obytes;
  }
  return L;
}

struct DenseLayout {
  mla::Schedule sched;
  int lq_pad;
  size_t qrot_off, qlo_off, opart_off, ml_off, total;
};

// rebuilt: the per-head attention over an expanded (fp16) window, never on
// split operands whatever the ring type.
DenseLayout dense_layout(const mla_cache* h, int32_t Lq, int64_t Lk = -1, bool rebuilt = false) {
  const mla_layer_config& c = h->cfg;
  const int d_h = c.d_nope + c.d_rope;
  DenseLayout L;
  const bool split = !rebuilt && split_operands(c);
  const mla::CoreShape sh = mla::core_shape_for_rows(Lq, split);
  const int br = sh.rows * sh.waves;
  L.lq_pad = (Lq + br - 1) / br * br;
  const int64_t R = (int64_t)c.n_heads * L.lq_pad;
  L.sched = make_schedule(c.batch, R, Lk < 0 ? window_keys(h) : Lk, 0, mla::device_cu_count(), sh,
                          2 * d_h / 8, kSegmentCostDense, split);
  const size_t slots = (size_t)L.sched.n_slots;
  const size_t qbytes = round_up((size_t)c.batch * R * d_h * 2, kAlign);
  L.qrot_off = 0;
  L.qlo_off = qbytes;
  L.opart_off = split ? 2 * qbytes : qbytes;
  L.ml_off = L.opart_off + round_up(slots * c.batch * R * d_h * 4, kAlign);
  L.total = L.ml_off + round_up(slots * c.batch * R * 2 * 4, kAlign);
  return L;
}

// Expand-then-attend workspace: the expanded per-head keys and values of
// the window, then the per-head attention workspace of the dense path.
struct ExpandLayout {
  DenseLayout dense;
  size_t kv_off, base, total;
};

ExpandLayout expand_layout(const mla_cache* h, int32_t Lq, int64_t Lk = -1) {
  const mla_layer_config& c = h->cfg;
  ExpandLayout L;
  L.dense = dense_layout(h, Lq, Lk, true);
  L.kv_off = 0;
  L.base = L.kv_off + round_up((size_t)c.batch * c.window_frames * tokens_per_frame(c) * 2 *
                                    c.n_heads * (c.d_nope + c.d_rope) * 2,
                                kAlign);
  L.total = L.base + L.dense.total;
  return L;
}

// On automatic, a chunk takes the expand-then-attend path when it has at
// least kExpandMinQueries queries and the latent form's products per (query,
// key, head), 2 (d_c + d_rope) + 2 d_c, are at least kExpandFlopRatio times the
// per-head ones, 2 (d_nope + d_rope) + 2 d_v.  The rebuild of the window is a
// fixed cost per call, and the latent core does more work per cycle than the
// per-head one, so the expansion pays only when it saves enough products.
// Measured on the 21-frame window (32760 keys, 12 heads) for whole calls:
// d_c 192 (832 vs 512 FLOP): absorbed faster at 256 queries (0.14 vs 0.16 ms),
// expand faster from 1024 (0.32 vs 0.44 ms) up to 4680 (1.18 vs 1.47 ms);
// d_c 128 (576 vs 512): even or absorbed faster at every chunk length;
// d_c 64: absorbed faster throughout.
// A bf16 ring's absorbed core issues every product twice (split operands)
// while its expansion runs the plain fp16 per-head core, so the rebuild pays
// back much sooner; measured on the same window (whole calls, batch 1):
// d_c 192: absorbed 0.096 / expand 0.125 ms at 64 queries, 0.156 / 0.136 at
// 128; d_c 128: 0.109 / 0.134 at 128, 0.182 / 0.141 at 256; d_c 64: 0.133 /
// 0.131 at 256, 0.188 / 0.164 at 384 (batch 4: even near 350).  Split rings
// expand from 128 queries when the issued latent products are at least 3
// times the per-head ones, from 256 when at least 2 times, else from 384.
constexpr int32_t kExpandMinQueries = 512;
constexpr double kExpandFlopRatio = 1.5;
constexpr int32_t kSplitExpandMinQueries[3] = {128, 256, 384};

// The expansion serves fp16-ring handles of the dense core's head width whose
// expanded full window (every key, every head) keeps one sequence's offsets
// below 2^31 elements, like a dense cache.  The expanded window is sized for
// the full window so the workspace size does not change as frames arrive.
// Every ring with bf16 inputs expands into an fp16 window: an E4M3 value
// widens to fp16 exactly, a bf16 ring's products run on bf16 MFMA (exact
// products of the stored values).  Rounded to bf16 instead, the rebuilt keys
// and values (like the query and the probabilities) would each move the
// attention output by about 1e-3 of its size on Gaussian inputs; in fp16 the
// expansion is as accurate as an fp16 ring's, with fp16's range (the rebuilt
// values must stay below 65504 in magnitude).
bool expand_possible(const mla_cache* h) {
  const mla_layer_config& c = h->cfg;
  return c.dtype == MLA_BF16 &&
         (c.cache_dtype == MLA_F16 || c.cache_dtype == MLA_E4M3 || c.cache_dtype == MLA_BF16) &&
         mla::expand_supported(c.d_c, c.d_rope, c.d_nope, c.d_v) &&
         (int64_t)c.window_frames * tokens_per_frame(c) * 2 * c.n_heads * (c.d_nope + c.d_rope) <
             (1LL << 31);
}

// The path an attend of Lq queries takes (MLA_PATH_ABSORBED or MLA_PATH_EXPAND).
int32_t attend_path_for(const mla_cache* h, int32_t Lq, int32_t key_splits) {
  const mla_layer_config& c = h->cfg;
  if (!expand_possible(h) || key_splits > 0 || h->attend_path == MLA_PATH_ABSORBED) return MLA_PATH_ABSORBED;
  if (h->attend_path == MLA_PATH_EXPAND) return MLA_PATH_EXPAND;
  const double latent = 2.0 * (c.d_c + c.d_rope) + 2.0 * c.d_c;
  const double per_head = 2.0 * (c.d_nope + c.d_rope) + 2.0 * c.d_v;
  if (split_operands(c)) {
    const double issued = 2.0 * latent;
    const int32_t min_q = issued >= 3.0 * per_head   ? kSplitExpandMinQueries[0]
                          : issued >= 2.0 * per_head ? kSplitExpandMinQueries[1]
                                                     : kSplitExpandMinQueries[2];
    return Lq >= min_q ? MLA_PATH_EXPAND : MLA_PATH_ABSORBED;
  }
  return Lq >= kExpandMinQueries && latent >= kExpandFlopRatio * per_head ? MLA_PATH_EXPAND
                                                                          : MLA_PATH_ABSORBED;
}

// Rotation table of the expanded queries: the d_nope content dimensions stay
// as they are (zero angle), the positional pairs turn as in the latent path.
mla::RopeTable expand_rope(const mla_layer_config& c) {
  const mla::RopeTable lat = latent_rope(c);
  mla::RopeTable t;
  memset(&t, 0, sizeof(t));
  const int pn = c.d_nope / 2;
  for (int p = 0; p < pn; ++p) {
    t.axis[p] = 0;
    t.inv_freq[p] = 0.0;
  }
  for (int p = 0; p < lat.n_pairs; ++p) {
    t.axis[pn + p] = lat.axis[p];
    t.inv_freq[pn + p] = lat.inv_freq[p];
  }
  t.n_pairs = pn + lat.n_pairs;
  return t;
}

mla_status launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Projection arguments with every optional part off (one pass, no rotation
// skip, no normalisation, unit scale).
mla::CacheWriteArgs projection_defaults() {
  mla::CacheWriteArgs a;
  memset(&a, 0, sizeof(a));
  a.passes = 1;
  a.scale = 1.0f;
  a.rot_group = 1;
  return a;
}

// Latent attention of Lq queries at q_token0 over the current window.
mla::AttendArgs latent_attend_args(const mla_cache* h, const void* q, int64_t q_token0, int32_t Lq,
                                   const void* w_uk, const void* w_uv, float* out) {
  const mla_layer_config& c = h->cfg;
  mla::AttendArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.ring = h->storage;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  a.B = c.batch;
  a.Lq = Lq;
  a.n_h = c.n_heads;
  a.d_nope = c.d_nope;
  a.d_rope = c.d_rope;
  a.d_v = c.d_v;
  a.d_c = c.d_c;
  a.q_token0 = q_token0;
  a.T = (int)tokens_per_frame(c);
  a.grid_w = c.grid_w;
  a.ring_rows = (int64_t)c.window_frames * a.T;
  a.key_slot0 = (h->oldest % c.window_frames) * a.T;
  a.Lk = (int)(n_resident(h) * a.T);
  a.cache_type = c.cache_dtype;
  a.qscale = (float)(1.4426950408889634 / sqrt((double)(c.d_nope + c.d_rope)));
  a.qn_gamma = h->qn_gamma;
  a.qn_eps = h->qn_eps;
  a.ev_start = h->prof_start;
  a.ev_stop = h->prof_stop;
  a.rope = latent_rope(c);
  return a;
}

// The attention block's shapes: 2-byte rings of the absorbed core's head
// shapes, and projection widths the GEMM tiles (32 output columns, 64-element
// depth chunks).
bool block_supported(const mla_layer_config& c) {
  return c.dtype == MLA_BF16 && mla::attend_bf16_supported(c.d_c, c.d_rope, c.d_nope, c.d_v) &&
         c.hidden % 64 == 0 && (c.n_heads * (c.d_c + c.d_rope)) % 32 == 0 &&
         (c.n_heads * c.d_c) % 64 == 0;
}

// The latent cache write of n_frames frames from frame0.
mla::CacheWriteArgs latent_write_args(const mla_cache* h, const void* x, const void* w_dkr,
                                      int64_t frame0, int32_t n_frames) {
  const mla_layer_config& c = h->cfg;
  const int width = c.d_c + c.d_rope;
  mla::CacheWriteArgs a = projection_defaults();
  a.x = x;
  a.w = w_dkr;
  a.w2 = w_dkr;
  a.w_split = width;
  a.ring = h->storage;
  a.tokens_per_batch = (int)(n_frames * tokens_per_frame(c));
  a.M = (int64_t)c.batch * a.tokens_per_batch;
  a.hidden = c.hidden;
  a.width = width;
  a.rot_begin = c.d_c;
  a.rot_end = width;
  a.rot_group = c.d_rope > 0 ? c.d_rope : 1;
  a.T = (int)tokens_per_frame(c);
  a.grid_w = c.grid_w;
  a.W = c.window_frames;
  a.ring_rows = (int64_t)c.window_frames * a.T;
  a.frame0 = frame0;
  a.out_type = c.cache_dtype;
  a.rope = latent_rope(c);
  return a;
}

mla_status create(const mla_layer_config* cfg, void* storage, size_t storage_bytes, bool dense,
                  mla_cache** out) {
  if (out == nullptr) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (!valid_config(cfg, dense) || !aligned16(storage)) return MLA_ERR_INVALID_ARG;
  const size_t need = dense ? mha_cache_bytes(cfg) : mla_cache_bytes(cfg);
  if (storage_bytes < need) return MLA_ERR_STORAGE_TOO_SMALL;
  mla_cache* h = new (std::nothrow) mla_cache;
  if (h == nullptr) return MLA_ERR_INVALID_ARG;
  h->cfg = *cfg;
  h->dense = dense;
  h->storage = storage;
  h->storage_bytes = storage_bytes;
  h->oldest = 0;
  h->newest = -1;
  h->prof_start = nullptr;
  h->prof_stop = nullptr;
  h->attend_path = MLA_PATH_AUTO;
  h->gen = 0;
  h->expand_reuse = 0;
  h->ex_valid = false;
  h->qn_gamma = nullptr;
  h->qn_eps = 0.0f;
  h->ex_ws = h->ex_wuk = h->ex_wuv = nullptr;
  h->ex_gen = 0;
  h->ex_token = 0;
  *out = h;
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_cache_bytes(const mla_layer_config* cfg) {
  if (!valid_config(cfg, false)) return 0;
  return (size_t)cfg->batch * cfg->window_frames * tokens_per_frame(*cfg) *
         (cfg->d_c + cfg->d_rope) * elem_size(cfg->cache_dtype);
}

size_t mha_cache_bytes(const mla_layer_config* cfg) {
  if (!valid_config(cfg, true)) return 0;
  return (size_t)cfg->batch * cfg->window_frames * tokens_per_frame(*cfg) * dense_width(*cfg) *
         elem_size(cfg->cache_dtype);
}

mla_status mla_cache_create(const mla_layer_config* cfg, void* storage, size_t storage_bytes,
                            mla_cache** out) {
  return create(cfg, storage, storage_bytes, false, out);
}

mla_status mha_cache_create(const mla_layer_config* cfg, void* storage, size_t storage_bytes,
                            mla_cache** out) {
  return create(cfg, storage, storage_bytes, true, out);
}

void mla_cache_destroy(mla_cache* cache) {
  if (cache != nullptr) ws_forget(cache->ex_token);
  delete cache;
}

mla_status mla_cache_write(mla_cache* h, const void* x, const void* w_dkr, int64_t frame0,
                           int32_t n_frames, void* stream) {
  if (h == nullptr || !aligned16(x) || !aligned16(w_dkr)) return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  mla_status st = check_write(h, frame0, n_frames);
  if (st != MLA_OK) return st;
  const mla_layer_config& c = h->cfg;
  const int width = c.d_c + c.d_rope;
  if (c.dtype == MLA_BF16 && !mla::cache_write_bf16_supported(width, c.hidden))
    return MLA_ERR_UNSUPPORTED;
  const mla::CacheWriteArgs a = latent_write_args(h, x, w_dkr, frame0, n_frames);
  hipStream_t s = (hipStream_t)stream;
  st = launch_status(c.dtype == MLA_BF16 ? mla::launch_cache_write_bf16(a, s)
                                         : mla::launch_cache_write_f32(a, s));
  if (st == MLA_OK) commit_write(h, frame0, n_frames);
  return st;
}

mla_status mla_cache_write_norm(mla_cache* h, const void* x, const void* w_dkr, const void* gamma,
                                float eps, int64_t frame0, int32_t n_frames, void* stream) {
  if (h == nullptr || !aligned16(x) || !aligned16(w_dkr) || !aligned16(gamma) || !(eps >= 0.0f) ||
      !isfinite(eps))
    return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  mla_status st = check_write(h, frame0, n_frames);
  if (st != MLA_OK) return st;
  const mla_layer_config& c = h->cfg;
  const int width = c.d_c + c.d_rope;
  if (c.dtype != MLA_BF16 || !mla::cache_write_bf16_supported(width, c.hidden) ||
      (width != 96 && width != 160 && width != 224))
    return MLA_ERR_UNSUPPORTED;
  mla::CacheWriteArgs a = latent_write_args(h, x, w_dkr, frame0, n_frames);
  a.gamma = gamma;
  a.eps = eps;
  a.norm_cols = c.d_c;
  st = launch_status(mla::launch_projection_bf16(a, mla::PROJ_CACHE_NORM, (hipStream_t)stream));
  if (st == MLA_OK) commit_write(h, frame0, n_frames);
  return st;
}

mla_status mha_cache_write(mla_cache* h, const void* x, const void* w_k, const void* w_v,
                           int64_t frame0, int32_t n_frames, void* stream) {
  if (h == nullptr || !aligned16(x) || !aligned16(w_k) || !aligned16(w_v))
    return MLA_ERR_INVALID_ARG;
  if (!h->dense) return MLA_ERR_WRONG_KIND;
  mla_status st = check_write(h, frame0, n_frames);
  if (st != MLA_OK) return st;
  const mla_layer_config& c = h->cfg;
  const int d_h = c.d_nope + c.d_rope;
  const int width = (int)dense_width(c);
  if (c.dtype == MLA_BF16 && !mla::cache_write_bf16_supported(width, c.hidden))
    return MLA_ERR_UNSUPPORTED;
  mla::CacheWriteArgs a = projection_defaults();
  a.x = x;
  a.w = w_k;
  a.w2 = w_v;
  a.w_split = c.n_heads * d_h;
  a.ring = h->storage;
  a.tokens_per_batch = (int)(n_frames * tokens_per_frame(c));
  a.M = (int64_t)c.batch * a.tokens_per_batch;
  a.hidden = c.hidden;
  a.width = width;
  a.rot_begin = 0;
  a.rot_end = c.n_heads * d_h;
  a.rot_group = d_h;
  a.T = (int)tokens_per_frame(c);
  a.grid_w = c.grid_w;
  a.W = c.window_frames;
  a.ring_rows = (int64_t)c.window_frames * a.T;
  a.frame0 = frame0;
  a.out_type = c.cache_dtype;
  a.rope = dense_rope(c);
  hipStream_t s = (hipStream_t)stream;
  st = launch_status(c.dtype == MLA_BF16 ? mla::launch_cache_write_bf16(a, s)
                                         : mla::launch_cache_write_f32(a, s));
  if (st == MLA_OK) commit_write(h, frame0, n_frames);
  return st;
}

mla_status mla_cache_evict(mla_cache* h, int32_t n_frames) {
  if (h == nullptr) return MLA_ERR_INVALID_ARG;
  if (n_frames < 0 || n_frames > n_resident(h)) return MLA_ERR_EVICT_RANGE;
  h->oldest += n_frames;
  ++h->gen;
  return MLA_OK;
}

mla_status mla_cache_query(const mla_cache* h, mla_cache_info* info) {
  if (h == nullptr || info == nullptr) return MLA_ERR_INVALID_ARG;
  info->oldest_frame = h->oldest;
  info->newest_frame = h->newest;
  info->n_resident_frames = (int32_t)n_resident(h);
  info->capacity_frames = h->cfg.window_frames;
  return MLA_OK;
}

mla_status mla_cache_set_state(mla_cache* h, int64_t oldest, int64_t newest) {
  if (h == nullptr || oldest < 0 || newest < oldest - 1 ||
      newest - oldest + 1 > h->cfg.window_frames)
    return MLA_ERR_INVALID_ARG;
  h->oldest = oldest;
  h->newest = newest;
  ++h->gen;
  return MLA_OK;
}

int64_t mla_cache_slot(const mla_cache* h, int64_t frame, int32_t tau) {
  if (h == nullptr || frame < 0 || tau < 0 || tau >= tokens_per_frame(h->cfg)) return -1;
  return (frame % h->cfg.window_frames) * tokens_per_frame(h->cfg) + tau;
}

size_t mla_attend_workspace_bytes(const mla_cache* h, int32_t Lq, int32_t key_splits) {
  if (h == nullptr || h->dense || Lq <= 0 || key_splits < 0) return 0;
  if (h->cfg.dtype == MLA_F32) return 0;
  // The largest workspace over every number of resident frames (the
  // schedule, hence the count of key-range partials, depends on it), so a
  // buffer sized once serves the window as it fills and slides.
  const bool expand = attend_path_for(h, Lq, key_splits) == MLA_PATH_EXPAND;
  const int64_t T = tokens_per_frame(h->cfg);
  size_t need = 0;
  for (int64_t f = 1; f <= h->cfg.window_frames; ++f) {
    const size_t t = expand ? expand_layout(h, Lq, f * T).total : latent_layout(h, Lq, key_splits, f * T).total;
    need = t > need ? t : need;
  }
  return need;
}

mla_status mla_cache_set_expand_reuse(mla_cache* h, int32_t enable) {
  if (h == nullptr || (enable != 0 && enable != 1)) return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  h->expand_reuse = enable;
  h->ex_valid = false;
  ws_forget(h->ex_token);
  h->ex_token = 0;
  return MLA_OK;
}

int32_t mla_attend_path(const mla_cache* h, int32_t Lq, int32_t key_splits) {
  if (h == nullptr || h->dense || Lq <= 0 || key_splits < 0) return -1;
  return attend_path_for(h, Lq, key_splits);
}

mla_status mla_cache_set_attend_path(mla_cache* h, int32_t path) {
  if (h == nullptr || path < MLA_PATH_AUTO || path > MLA_PATH_EXPAND) return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  if (path == MLA_PATH_EXPAND && !expand_possible(h)) return MLA_ERR_UNSUPPORTED;
  h->attend_path = path;
  return MLA_OK;
}

mla_status mla_cache_set_query_norm(mla_cache* h, const void* gamma, float eps) {
  if (h == nullptr) return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  if (gamma == nullptr) {
    h->qn_gamma = nullptr;
    h->qn_eps = 0.0f;
    return MLA_OK;
  }
  if (!aligned16(gamma) || !(eps >= 0.0f) || !isfinite(eps)) return MLA_ERR_INVALID_ARG;
  if (h->cfg.dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  h->qn_gamma = gamma;
  h->qn_eps = eps;
  return MLA_OK;
}

mla_status mla_attend(mla_cache* h, const void* q, int64_t q_token0, int32_t Lq, const void* w_uk,
                      const void* w_uv, float* out, int32_t key_splits, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (h == nullptr || !aligned16(q) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(out) ||
      Lq <= 0 || key_splits < 0 || q_token0 < 0)
    return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  if (n_resident(h) <= 0) return MLA_ERR_EMPTY;
  const mla_layer_config& c = h->cfg;
  if ((int64_t)Lq * c.n_heads >= (1LL << 30)) return MLA_ERR_INVALID_ARG;
  const bool bf16 = c.dtype == MLA_BF16;
  const bool expand = bf16 && attend_path_for(h, Lq, key_splits) == MLA_PATH_EXPAND;
  if (bf16 && !expand && !mla::attend_bf16_supported(c.d_c, c.d_rope, c.d_nope, c.d_v))
    return MLA_ERR_UNSUPPORTED;
  mla::AttendArgs a = latent_attend_args(h, q, q_token0, Lq, w_uk, w_uv, out);
  hipStream_t s = (hipStream_t)stream;
  if (!bf16) return launch_status(mla::launch_attend_f32(a, s));
  if (expand) {
    const ExpandLayout X = expand_layout(h, Lq);
    if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0 || workspace_bytes < X.total)
      return MLA_ERR_WORKSPACE;
    char* ws = (char*)workspace;
    mla::ExpandArgs e;
    memset(&e, 0, sizeof(e));
    e.ring = h->storage;
    e.w_uk = w_uk;
    e.w_uv = w_uv;
    e.kv = ws + X.kv_off;
    e.B = c.batch;
    e.n_h = c.n_heads;
    e.d_nope = c.d_nope;
    e.d_rope = c.d_rope;
    e.d_c = c.d_c;
    e.d_v = c.d_v;
    e.ring_rows = a.ring_rows;
    e.key_slot0 = a.key_slot0;
    e.Lk = a.Lk;
    e.cache_type = c.cache_dtype;
    mla::MhaAttendArgs m;
    memset(&m, 0, sizeof(m));
    m.q = q;
    m.ring = e.kv;
    m.out = out;
    m.qrot = ws + X.base + X.dense.qrot_off;
    m.qrot_lo = nullptr;  // fp16 window: plain operands
    m.B = c.batch;
    m.Lq = Lq;
    m.n_h = c.n_heads;
    m.d_h = c.d_nope + c.d_rope;
    m.q_token0 = q_token0;
    m.T = a.T;
    m.grid_w = c.grid_w;
    m.ring_rows = a.Lk;
    m.key_slot0 = 0;
    m.Lk = a.Lk;
    m.cache_type = MLA_F16;  // the rebuilt window is fp16 for either ring
    m.qscale = a.qscale;
    m.qn_gamma = a.qn_gamma;
    m.qn_eps = a.qn_eps;
    m.ev_start = h->prof_start;
    m.ev_stop = h->prof_stop;
    m.rope = expand_rope(c);
    // The rebuilt window in this workspace is still current when reuse is on,
    // neither the window nor the weights changed since it was written, and no
    // attend on any handle has written over it since (several attends per
    // chunk, e.g. denoising steps).
    const size_t kv_bytes = X.base - X.kv_off;
    const bool reuse = h->expand_reuse && h->ex_valid && h->ex_ws == workspace &&
                       h->ex_wuk == w_uk && h->ex_wuv == w_uv && h->ex_gen == h->gen &&
                       ws_holds(ws + X.kv_off, kv_bytes, h->ex_token);
    if (!reuse) {
      h->ex_valid = false;
      ws_forget(h->ex_token);
      h->ex_token = 0;
      ws_clobber(ws, X.total);
      const hipError_t err = mla::launch_expand_kv(e, s);
      if (err != hipSuccess) return MLA_ERR_HIP;
      h->ex_valid = true;
      h->ex_ws = workspace;
      h->ex_wuk = w_uk;
      h->ex_wuv = w_uv;
      h->ex_gen = h->gen;
      h->ex_token = ws_enter(ws + X.kv_off, kv_bytes);
    }
    ws_clobber(ws + X.base, X.total - X.base);
    return launch_status(mla::launch_mha_attend_bf16_ws(m, (float*)(ws + X.base + X.dense.opart_off),
                                                        (float*)(ws + X.base + X.dense.ml_off),
                                                        X.dense.sched, s));
  }
  h->ex_valid = false;  // the absorbed path overwrites the workspace
  const LatentLayout L = latent_layout(h, Lq, key_splits);
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0 || workspace_bytes < L.total)
    return MLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  ws_clobber(ws, L.total);
  a.qcat = ws + L.qcat_off;
  a.qcat_lo = split_operands(c) ? ws + L.qlo_off : nullptr;
  a.opart = (float*)(ws + L.opart_off);
  a.ml = (float*)(ws + L.ml_off);
  a.sched = L.sched;
  a.part16 = fp16_partials(c, L.sched);
  return launch_status(mla::launch_attend_bf16(a, s));
}

mla_status mla_attend_noalloc(mla_cache* h, const void* q, int64_t q_token0, int32_t Lq,
                              const void* w_uk, const void* w_uv, float* out, int32_t key_splits,
                              void* stream) {
  if (h == nullptr || Lq <= 0 || key_splits < 0) return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  if (n_resident(h) <= 0) return MLA_ERR_EMPTY;
  if ((int64_t)Lq * h->cfg.n_heads >= (1LL << 30)) return MLA_ERR_INVALID_ARG;
  // The workspace this call needs in the window's current state.
  size_t need = 0;
  if (h->cfg.dtype != MLA_F32)
    need = attend_path_for(h, Lq, key_splits) == MLA_PATH_EXPAND ? expand_layout(h, Lq).total
                                                                 : latent_layout(h, Lq, key_splits).total;
  if (need > mla::kScratchBytes) return MLA_ERR_SCRATCH;
  void* ws = nullptr;
  if (mla::scratch_for_current_device(&ws) != hipSuccess || ws == nullptr) return MLA_ERR_HIP;
  return mla_attend(h, q, q_token0, Lq, w_uk, w_uv, out, key_splits, ws, mla::kScratchBytes, stream);
}

size_t mla_attend_noalloc_max_bytes(void) { return mla::kScratchBytes; }

size_t mla_fold_query_bytes(const mla_cache* h) {
  if (h == nullptr || h->dense) return 0;
  const mla_layer_config& c = h->cfg;
  return (size_t)2 * c.n_heads * (c.d_c + c.d_rope) * c.hidden * 2;
}

size_t mla_fold_output_bytes(const mla_cache* h) {
  if (h == nullptr || h->dense) return 0;
  const mla_layer_config& c = h->cfg;
  return (size_t)2 * c.hidden * c.n_heads * c.d_c * 2;
}

mla_status mla_fold_query_weights(const mla_cache* h, const void* w_q, const void* w_uk, void* w_qf,
                                  size_t w_qf_bytes, void* stream) {
  if (h == nullptr || !aligned16(w_q) || !aligned16(w_uk) || !aligned16(w_qf)) return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  if (!block_supported(h->cfg)) return MLA_ERR_UNSUPPORTED;
  if (w_qf_bytes < mla_fold_query_bytes(h)) return MLA_ERR_INVALID_ARG;
  const mla_layer_config& c = h->cfg;
  mla::FoldArgs f;
  memset(&f, 0, sizeof(f));
  f.w_q = w_q;
  f.w_uk = w_uk;
  f.out = w_qf;
  f.n_h = c.n_heads;
  f.d_nope = c.d_nope;
  f.d_rope = c.d_rope;
  f.d_v = c.d_v;
  f.d_c = c.d_c;
  f.hidden = c.hidden;
  return launch_status(mla::launch_fold_query(f, (hipStream_t)stream));
}

mla_status mla_fold_output_weights(const mla_cache* h, const void* w_o, const void* w_uv, void* w_fo,
                                   size_t w_fo_bytes, void* stream) {
  if (h == nullptr || !aligned16(w_o) || !aligned16(w_uv) || !aligned16(w_fo)) return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  if (!block_supported(h->cfg)) return MLA_ERR_UNSUPPORTED;
  if (w_fo_bytes < mla_fold_output_bytes(h)) return MLA_ERR_INVALID_ARG;
  const mla_layer_config& c = h->cfg;
  mla::FoldArgs f;
  memset(&f, 0, sizeof(f));
  f.w_o = w_o;
  f.w_uv = w_uv;
  f.out = w_fo;
  f.n_h = c.n_heads;
  f.d_nope = c.d_nope;
  f.d_rope = c.d_rope;
  f.d_v = c.d_v;
  f.d_c = c.d_c;
  f.hidden = c.hidden;
  return launch_status(mla::launch_fold_output(f, (hipStream_t)stream));
}

size_t mla_attend_block_workspace_bytes(const mla_cache* h, int32_t Lq, int32_t key_splits) {
  if (h == nullptr || h->dense || Lq <= 0 || key_splits < 0 || !block_supported(h->cfg)) return 0;
  const int64_t T = tokens_per_frame(h->cfg);
  size_t need = 0;
  for (int64_t f = 1; f <= h->cfg.window_frames; ++f) {
    const size_t t = latent_layout(h, Lq, key_splits, f * T, true).total;
    need = t > need ? t : need;
  }
  return need;
}

mla_status mla_attend_block(mla_cache* h, const void* x, int64_t q_token0, int32_t Lq, const void* w_qf,
                            const void* w_fo, float* out, int32_t key_splits, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (h == nullptr || !aligned16(x) || !aligned16(w_qf) || !aligned16(w_fo) || !aligned16(out) ||
      Lq <= 0 || key_splits < 0 || q_token0 < 0)
    return MLA_ERR_INVALID_ARG;
  if (h->dense) return MLA_ERR_WRONG_KIND;
  if (n_resident(h) <= 0) return MLA_ERR_EMPTY;
  const mla_layer_config& c = h->cfg;
  if ((int64_t)Lq * c.n_heads >= (1LL << 30)) return MLA_ERR_INVALID_ARG;
  if (!block_supported(c)) return MLA_ERR_UNSUPPORTED;
  // The block never forms the per-head queries the norm would act on (they
  // come out of the folded projection already absorbed).
  if (h->qn_gamma != nullptr) return MLA_ERR_UNSUPPORTED;
  const LatentLayout L = latent_layout(h, Lq, key_splits, -1, true);
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0 || workspace_bytes < L.total)
    return MLA_ERR_WORKSPACE;
  h->ex_valid = false;  // overwrites the workspace like an absorbed attend
  char* ws = (char*)workspace;
  ws_clobber(ws, L.total);
  const bool split = split_operands(c);
  mla::AttendArgs a = latent_attend_args(h, nullptr, q_token0, Lq, nullptr, nullptr, out);
  a.qcat = ws + L.qcat_off;
  a.qcat_lo = split ? ws + L.qlo_off : nullptr;
  a.opart = (float*)(ws + L.opart_off);
  a.ml = (float*)(ws + L.ml_off);
  a.sched = L.sched;
  a.part16 = fp16_partials(c, L.sched);
  hipStream_t s = (hipStream_t)stream;
  // 1. [q_lat | q^R] of every head straight from x with the folded weights
  //    (two parts), rotated at each query's position and scaled
  const int qw = c.n_heads * (c.d_c + c.d_rope);
  mla::CacheWriteArgs p = projection_defaults();
  p.x = x;
  p.w = w_qf;
  p.w2 = w_qf;
  p.w_split = qw;
  p.ring = a.qcat;
  p.M = (int64_t)c.batch * Lq;
  p.tokens_per_batch = Lq;
  p.hidden = c.hidden;
  p.width = qw;
  p.rot_begin = 0;
  p.rot_end = qw;
  p.rot_group = c.d_c + c.d_rope;
  p.rot_skip = c.d_c;
  p.T = a.T;
  p.grid_w = c.grid_w;
  p.W = c.window_frames;
  p.q_token0 = q_token0;
  p.out_type = c.cache_dtype == MLA_E4M3 ? MLA_F16 : c.cache_dtype;  // the core's operand type
  p.rope = latent_rope(c);
  p.passes = 2;
  p.w_part[1] = (int64_t)qw * c.hidden * 2;
  p.scale = a.qscale;
  p.out_lo = a.qcat_lo;
  hipError_t e = mla::launch_projection_bf16(p, mla::PROJ_QUERY, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  // 2. the absorbed core, 3. merged latent outputs in two parts
  e = mla::launch_attend_core_only(a, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  void* o_hi = ws + L.ohi_off;
  void* o_lo = ws + L.olo_off;
  e = mla::launch_merge_latent(a, o_hi, o_lo, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  // 4. model-width output with the folded output weights: three passes of the
  //    two-part operands (value x value, value x remainder, remainder x value)
  const int K = c.n_heads * c.d_c;
  mla::CacheWriteArgs o = projection_defaults();
  o.x = o_hi;
  o.w = w_fo;
  o.w2 = w_fo;
  o.w_split = c.hidden;
  o.ring = out;
  o.M = (int64_t)c.batch * Lq;
  o.tokens_per_batch = Lq;
  o.hidden = K;
  o.width = c.hidden;
  o.T = a.T;
  o.grid_w = c.grid_w;
  o.W = c.window_frames;
  o.out_type = MLA_BF16;
  o.passes = 3;
  o.w_part[1] = (int64_t)c.hidden * K * 2;
  o.x_part[2] = (int64_t)((char*)o_lo - (char*)o_hi);
  return launch_status(mla::launch_projection_bf16(o, mla::PROJ_OUT, s));
}

size_t mha_attend_workspace_bytes(const mla_cache* h, int32_t Lq) {
  if (h == nullptr || !h->dense || Lq <= 0) return 0;
  if (h->cfg.dtype == MLA_F32) return 0;
  // largest over every number of resident frames (see mla_attend_workspace_bytes)
  const int64_t T = tokens_per_frame(h->cfg);
  size_t need = 0;
  for (int64_t f = 1; f <= h->cfg.window_frames; ++f) {
    const size_t t = dense_layout(h, Lq, f * T).total;
    need = t > need ? t : need;
  }
  return need;
}

mla_status mha_attend(mla_cache* h, const void* q, int64_t q_token0, int32_t Lq, float* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (h == nullptr || !aligned16(q) || !aligned16(out) || Lq <= 0 || q_token0 < 0)
    return MLA_ERR_INVALID_ARG;
  if (!h->dense) return MLA_ERR_WRONG_KIND;
  if (n_resident(h) <= 0) return MLA_ERR_EMPTY;
  const mla_layer_config& c = h->cfg;
  const int d_h = c.d_nope + c.d_rope;
  if ((int64_t)Lq * c.n_heads >= (1LL << 30)) return MLA_ERR_INVALID_ARG;
  const bool bf16 = c.dtype == MLA_BF16;
  if (bf16 && !mla::mha_attend_bf16_supported(d_h)) return MLA_ERR_UNSUPPORTED;
  mla::MhaAttendArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.ring = h->storage;
  a.out = out;
  a.B = c.batch;
  a.Lq = Lq;
  a.n_h = c.n_heads;
  a.d_h = d_h;
  a.q_token0 = q_token0;
  a.T = (int)tokens_per_frame(c);
  a.grid_w = c.grid_w;
  a.ring_rows = (int64_t)c.window_frames * a.T;
  a.key_slot0 = (h->oldest % c.window_frames) * a.T;
  a.Lk = (int)(n_resident(h) * a.T);
  a.cache_type = c.cache_dtype;
  a.qscale = (float)(1.4426950408889634 / sqrt((double)d_h));
  a.ev_start = h->prof_start;
  a.ev_stop = h->prof_stop;
  a.rope = dense_rope(c);
  hipStream_t s = (hipStream_t)stream;
  if (!bf16) return launch_status(mla::launch_mha_attend_f32(a, s));
  const DenseLayout L = dense_layout(h, Lq);
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0 || workspace_bytes < L.total)
    return MLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  ws_clobber(ws, L.total);
  a.qrot = ws + L.qrot_off;
  a.qrot_lo = split_operands(c) ? ws + L.qlo_off : nullptr;
  return launch_status(mla::launch_mha_attend_bf16_ws(a, (float*)(ws + L.opart_off),
                                                      (float*)(ws + L.ml_off), L.sched, s));
}

mla_status mla_cache_set_profile_events(mla_cache* h, void* start, void* stop) {
  if (h == nullptr || ((start == nullptr) != (stop == nullptr))) return MLA_ERR_INVALID_ARG;
  h->prof_start = (hipEvent_t)start;
  h->prof_stop = (hipEvent_t)stop;
  return MLA_OK;
}

const char* mla_status_str(mla_status st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_STORAGE_TOO_SMALL: return "storage too small";
    case MLA_ERR_FULL: return "window full";
    case MLA_ERR_NOT_CONTIGUOUS: return "frames do not continue the newest resident frame";
    case MLA_ERR_EVICT_RANGE: return "evicting more frames than are resident";
    case MLA_ERR_EMPTY: return "window empty";
    case MLA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MLA_ERR_UNSUPPORTED: return "shape not supported for this dtype";
    case MLA_ERR_WRONG_KIND: return "latent call on a dense handle or vice versa";
    case MLA_ERR_HIP: return "kernel launch failed";
    case MLA_ERR_SCRATCH: return "call needs more workspace than the library's static scratch";
  }
  return "unknown status";
}

const char* mla_version(void) { return "libmla 0.1 (gfx950)"; }

}  // extern "C"
