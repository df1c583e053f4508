// Internal interface between the host library (validation, window bookkeeping,
// workspace carving) and the gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mla {

constexpr int kMaxRopePairs = 64;

// Per-pair rotation table of 3D-RoPE: pair p turns by
// pos[axis[p]] * inv_freq[p] radians (axis 0 = latent frame, 1 = grid row,
// 2 = grid column).
struct RopeTable {
  int n_pairs;
  int axis[kMaxRopePairs];
  double inv_freq[kMaxRopePairs];
};

// Projection y = W x for a run of tokens on the LDS-staged MFMA GEMM, with an
// epilogue per use:
//  * cache write (PROJ_CACHE): RoPE on the rotated columns, round to the
//    storage dtype, scatter each token's row to its ring slot;
//  * cache write with the latent RMS-normalised (PROJ_CACHE_NORM): the first
//    norm_cols columns scaled by gamma / rms before rounding;
//  * folded query projection (PROJ_QUERY): rows [q_lat | q^R] per head, RoPE
//    on the positional columns of every head at the query's position, scaled
//    by `scale`, written to token rows of the cache type (and the remainders'
//    rounding to out_lo for split operands);
//  * output projection (PROJ_OUT): fp32 token rows.
// The weights (and the inputs) may come in parts whose products are summed:
// pass p multiplies x part x_part[p] by weight part w_part[p] (byte offsets
// from x and from w / w2), so a weight carried as two bf16 parts (value and
// remainder) keeps 16 significant bits.
enum ProjMode { PROJ_CACHE = 0, PROJ_CACHE_NORM = 1, PROJ_QUERY = 2, PROJ_OUT = 3 };
constexpr int kProjMaxPasses = 3;
struct CacheWriteArgs {
  const void* x;          // [M][hidden], M = batch * tokens_per_batch
  const void* w;          // rows [0, w_split) of the [width][hidden] projection
  const void* w2;         // rows [w_split, width) (may alias w + w_split*hidden)
  int w_split;
  void* ring;             // cache: [batch][ring_rows][width]; query / out: [M][width]
  int64_t M;
  int tokens_per_batch;   // cache: n_frames * T; query / out: Lq
  int hidden;
  int width;              // output columns (latent: d_c + d_rope; dense: 2 * n_h * d_h)
  int rot_begin;          // first rotated column
  int rot_end;            // one past the last rotated column
  int rot_group;          // rotated columns restart their pair count every rot_group
  int rot_skip;           // columns below rot_skip within each group are not rotated
  int T, grid_w, W;
  int64_t ring_rows;      // W * T
  int64_t frame0;         // cache: first frame written
  int64_t q_token0;       // query: global token of row 0 of every sequence
  int out_type;           // output element type: 1 = bf16, 2 = fp16, 3 = E4M3 (cache writes)
  RopeTable rope;
  int passes;                             // 1 .. kProjMaxPasses
  int64_t x_part[kProjMaxPasses];         // byte offset of pass p's x part from x
  int64_t w_part[kProjMaxPasses];         // byte offset of pass p's weight part from w and w2
  const void* gamma;      // PROJ_CACHE_NORM: [norm_cols] gain, input dtype (bf16)
  float eps;
  int norm_cols;
  float scale;            // PROJ_QUERY: applied to every column
  void* out_lo;           // PROJ_QUERY with split operands: remainders (null otherwise)
};

#if defined(__HIPCC__)
#define MLA_HD __host__ __device__
#else
#define MLA_HD
#endif

// Shapes of the attention core: a block of `waves` waves owns 32 * waves rows
// and cycles `stages` LDS buffers of `key_tile` keys.  Many query rows (the
// chunk case) take the widest block, which reuses each staged key tile most;
// a few rows (cache-bound small-query shapes) take narrow blocks on short
// tiles with deeper buffer rings, to keep more key bytes in flight per CU.
// `rows` is the query rows per wave: 32 on 32x32x16 MFMAs, or 16 on
// 16x16x32 MFMAs for row units of at most 16 rows (one query per sequence
// over 12 heads, say), which then waste a quarter of the matrix work instead
// of five eighths.
struct CoreShape {
  int waves;
  int key_tile;
  int stages;
  int rows;
};
constexpr CoreShape kCoreShapes[] = {{8, 64, 3, 32}, {4, 32, 4, 32}, {1, 32, 2, 32}, {1, 32, 2, 16},
                                     {4, 32, 4, 16}};
// Chunk shape of split-operand cores (bf16 cache: query and probabilities
// carried as two bf16 parts, one wave per SIMD): four waves on 64-key tiles.
constexpr CoreShape kCoreShapeSplitChunk = {4, 64, 3, 32};

// Shape for `rows` query rows of one row unit (latent: Lq * n_h rows of a
// batch element; dense: Lq rows of one head).  `split`: split-operand core.
inline CoreShape core_shape_for_rows(int64_t rows, bool split = false) {
  if (rows <= 16) return kCoreShapes[3];
  if (rows <= 32) return kCoreShapes[2];
  if (rows <= 64) return kCoreShapes[4];
  if (rows <= 128) return kCoreShapes[1];
  return split ? kCoreShapeSplitChunk : kCoreShapes[0];
}

// Stages of a shape for key rows of `chunks_per_key` 16-byte chunks: the
// tile loads a wave keeps in flight behind the next tile (stages - 1 tiles of
// key_tile * chunks_per_key / 64 loads for a one-wave block) must fit the
// 63-count vector-memory counter.
inline CoreShape core_shape_for_keys(CoreShape sh, int chunks_per_key) {
  const int spans = sh.key_tile * chunks_per_key / 64 / sh.waves;
  const int max_stages = 1 + 63 / (spans > 0 ? spans : 1);
  if (sh.stages > max_stages) sh.stages = max_stages;
  return sh;
}

// Blocks of a shape that fit one compute unit at once: LDS (160 KiB per CU)
// holds `stages` key tiles of `chunks_per_key` 16-byte chunks per key (plus,
// for one-byte rows, one decode tile of `decode_chunks_per_key`), and the
// core's register use allows two waves per SIMD (eight per CU), or one (four
// per CU) for split operands.
inline int core_blocks_per_cu(CoreShape sh, int chunks_per_key, bool split = false,
                              int decode_chunks_per_key = 0) {
  const int lds = (sh.stages * chunks_per_key + decode_chunks_per_key) * sh.key_tile * 16;
  const int by_lds = (160 * 1024) / lds;
  const int by_waves = (split ? 4 : 8) / sh.waves;
  return by_lds < by_waves ? by_lds : by_waves;
}

// Work schedule of the attention core over (row group, key tile) steps, where a
// group is one batch element's block of block_rows rows:
//  * data-parallel rounds: while there are at least n_blocks groups left, each
//    block takes whole groups (all key tiles), all blocks in key-tile lockstep;
//  * the remaining `rem` groups (rem < n_blocks) are balanced stream-K style:
//    group j's "main" block (block j) walks key tiles [0, main_len) in lockstep
//    with the other main blocks, and the tail tiles [main_len, n_kt) of all
//    remaining groups - a short key range that stays L2-resident - are cut into
//    contiguous runs of tail_per_block steps for blocks rem .. n_blocks-1.
// A group whose tiles span several blocks leaves one partial (value sums, max,
// sum) per block, merged exactly by log-sum-exp: slot 0 = main block, slots
// 1.. = tail blocks in order.
struct Schedule {
  int block_rows;       // rows per group (rows per wave * waves of the core shape)
  int key_tile;         // keys per step
  int stages;           // LDS tile buffers of the core shape
  int n_rg;             // row groups per batch element
  int n_kt;             // key tiles in the window
  int n_groups;         // batch * n_rg
  int n_blocks;
  int full_rounds;      // data-parallel rounds of whole groups
  int rem;              // groups left for the balanced part
  int main_len;         // key tiles a remaining group's main block walks
  int tail_per_block;   // tail steps per tail block (>= 1)
  int n_slots;          // partial slots to provide per group (upper bound)
};

struct StepInfo {
  int grp, kt, slot;
  bool first, last;     // first / last step of this block's segment of grp
};

// Tail blocks (index into rem..n_blocks-1) touching remaining group j.
MLA_HD inline int sched_tail_first(const Schedule& s, int j) {
  return j * (s.n_kt - s.main_len) / s.tail_per_block;
}
MLA_HD inline int sched_tail_last(const Schedule& s, int j) {
  return ((j + 1) * (s.n_kt - s.main_len) - 1) / s.tail_per_block;
}

// Steps block g executes.
MLA_HD inline int sched_block_steps(const Schedule& s, int g) {
  int n = s.full_rounds * s.n_kt;
  if (s.rem > 0) {
    if (g < s.rem) {
      n += s.main_len;
    } else {
      const int tail = s.rem * (s.n_kt - s.main_len);
      const int t0 = (g - s.rem) * s.tail_per_block;
      const int t1 = t0 + s.tail_per_block < tail ? t0 + s.tail_per_block : tail;
      n += t1 > t0 ? t1 - t0 : 0;
    }
  }
  return n;
}

// Logical block of hardware workgroup hw.  Workgroups are dealt round-robin
// to the kDies accelerator dies (die hw % kDies), each with its own L2, so
// die x runs hardware workgroups P_x .. P_x + c_x - 1 in this count.  With no
// balanced tail, die x runs the contiguous logical blocks [P_x, P_x + c_x):
// consecutive row groups - the same head on the per-head path, whose blocks
// read the same key and value tiles in lockstep - share one L2 instead of
// spreading over all.  With a tail, the main blocks 0 .. rem - 1 and the tail
// blocks rem .. n_blocks - 1 are spread over the dies in proportion
// (die x: main blocks [P_x rem / n_blocks, P_{x+1} rem / n_blocks), and the
// tail blocks in the same proportion), so that a die's tail blocks finish the
// row groups its own main blocks started and their short tail key ranges are
// read through the L2 that already holds that head's tiles.
constexpr int kDies = 8;
MLA_HD inline int sched_block_of(const Schedule& s, int hw) {
  const int nb = s.n_blocks, q = nb / kDies, r = nb % kDies;
  const int x = hw % kDies, k = hw / kDies;
  const int start = x * q + (x < r ? x : r), cnt = q + (x < r ? 1 : 0);
  if (s.rem <= 0 || s.main_len >= s.n_kt) return start + k;
  const int m0 = (int)((int64_t)start * s.rem / nb);
  const int mc = (int)((int64_t)(start + cnt) * s.rem / nb) - m0;
  return k < mc ? m0 + k : s.rem + (start - m0) + (k - mc);
}

// Step i (0 <= i < sched_block_steps(s, g)) of block g.
MLA_HD inline StepInfo sched_decode(const Schedule& s, int g, int i) {
  StepInfo r;
  const int dp = s.full_rounds * s.n_kt;
  if (i < dp) {
    r.grp = g + (i / s.n_kt) * s.n_blocks;
    r.kt = i % s.n_kt;
    r.slot = 0;
    r.first = r.kt == 0;
    r.last = r.kt == s.n_kt - 1;
    return r;
  }
  const int i2 = i - dp;
  const int base = s.full_rounds * s.n_blocks;
  if (g < s.rem) {
    r.grp = base + g;
    r.kt = i2;
    r.slot = 0;
    r.first = i2 == 0;
    r.last = i2 == s.main_len - 1;
    return r;
  }
  const int tl = s.n_kt - s.main_len;
  const int t = (g - s.rem) * s.tail_per_block + i2;
  const int j = t / tl;
  r.grp = base + j;
  r.kt = s.main_len + (t - j * tl);
  r.slot = 1 + (g - s.rem) - sched_tail_first(s, j);
  r.first = i2 == 0 || r.kt == s.main_len;
  r.last = i2 == sched_block_steps(s, g) - dp - 1 || r.kt == s.n_kt - 1;
  return r;
}

// Incremental walk over block g's steps i = 0, 1, 2, ... with the same
// results as sched_decode(s, g, i), decoding the schedule (integer divisions)
// only where a segment starts.  n_steps = sched_block_steps(s, g).
struct SchedCursor {
  StepInfo si;  // step i
  int i;
  int left;     // steps of the same segment after step i
};

// Last key tile of the segment that contains step i (decoded as si).
MLA_HD inline int sched_segment_last_kt(const Schedule& s, int g, int i, const StepInfo& si,
                                        int n_steps) {
  if (i < s.full_rounds * s.n_kt) return s.n_kt - 1;
  if (g < s.rem) return s.main_len - 1;
  const int by_block = si.kt + (n_steps - 1 - i);
  return by_block < s.n_kt - 1 ? by_block : s.n_kt - 1;
}

MLA_HD inline void sched_cursor_seek(const Schedule& s, int g, int n_steps, int i, SchedCursor& c) {
  c.i = i;
  c.si = sched_decode(s, g, i);
  c.left = sched_segment_last_kt(s, g, i, c.si, n_steps) - c.si.kt;
}

// Advance to step c.i + 1; returns true when that step starts a new segment.
// Past the block's last step only the index moves (nothing is decoded).
MLA_HD inline bool sched_cursor_next(const Schedule& s, int g, int n_steps, SchedCursor& c) {
  if (c.i + 1 >= n_steps) {
    ++c.i;
    return false;
  }
  if (c.left > 0) {
    ++c.i;
    ++c.si.kt;
    c.si.first = false;
    --c.left;
    c.si.last = c.left == 0;
    return false;
  }
  sched_cursor_seek(s, g, n_steps, c.i + 1, c);
  return true;
}

// Partials left for group grp (its slots are 0 .. count-1).
MLA_HD inline int sched_group_slots(const Schedule& s, int grp) {
  const int base = s.full_rounds * s.n_blocks;
  if (grp < base || s.main_len >= s.n_kt) return 1;
  const int j = grp - base;
  return 1 + sched_tail_last(s, j) - sched_tail_first(s, j) + 1;
}

// Absorbed latent attention.
struct AttendArgs {
  const void* q;          // [B][Lq][n_h][d_nope + d_rope]
  const void* ring;       // [B][ring_rows][d_c + d_rope]
  const void* w_uk;       // [n_h][d_nope][d_c]
  const void* w_uv;       // [n_h][d_v][d_c]
  float* out;             // [B][Lq][n_h][d_v]
  void* qcat;             // workspace [B][R][d_c + d_rope] cache type, R = Lq * n_h
  void* qcat_lo;          // bf16 cache: the remainders of qcat (same layout); else null
  float* opart;           // workspace [n_split][B][R][d_c]
  float* ml;              // workspace [n_split][B][R][2]  (running max (log2 units), sum)
  int part16;             // partials stored normalised as fp16 (few-row core shapes)
  int B, Lq, n_h, d_nope, d_rope, d_v, d_c;
  int64_t q_token0;
  int T, grid_w;
  int64_t ring_rows;
  int64_t key_slot0;      // ring slot of resident key 0
  int Lk;                 // resident keys
  Schedule sched;
  int cache_type;         // 1 = bf16, 2 = fp16, 3 = E4M3 (widened to fp16); inputs are bf16
  float qscale;           // log2(e) / sqrt(d_nope + d_rope)
  const void* qn_gamma;   // optional RMS norm of each head's query row: gain [d_nope + d_rope] bf16; null = none
  float qn_eps;
  hipEvent_t ev_start;    // optional: recorded right before / after the core kernel
  hipEvent_t ev_stop;
  RopeTable rope;
};

// Dense per-head attention (comparison path).
struct MhaAttendArgs {
  const void* q;          // [B][Lq][n_h][d_h]
  const void* ring;       // [B][ring_rows][2][n_h][d_h]
  float* out;             // [B][Lq][n_h][d_h]
  void* qrot;             // workspace [B][n_h * Lq_pad][d_h] cache type (rotated, pre-scaled)
  void* qrot_lo;          // bf16 cache: the remainders of qrot (same layout); else null
  int B, Lq, n_h, d_h;
  int64_t q_token0;
  int T, grid_w;
  int64_t ring_rows;
  int64_t key_slot0;
  int Lk;
  int cache_type;
  float qscale;
  const void* qn_gamma;   // optional RMS norm of each query row over d_h: gain [d_h] bf16; null = none
  float qn_eps;
  hipEvent_t ev_start;
  hipEvent_t ev_stop;
  RopeTable rope;
};

// Expand-then-attend: per-head keys and values of the resident window rebuilt
// from the latent ring into the dense cache's layout.
struct ExpandArgs {
  const void* ring;       // [B][ring_rows][d_c + d_rope] cache type
  const void* w_uk;       // [n_h][d_nope][d_c] bf16
  const void* w_uv;       // [n_h][d_v][d_c] bf16
  void* kv;               // workspace [B][Lk][2][n_h][d_nope + d_rope] fp16
  int B, n_h, d_nope, d_rope, d_c, d_v;
  int64_t ring_rows;
  int64_t key_slot0;      // ring slot of resident key 0
  int Lk;
  int cache_type;         // ring: 1 = bf16, 2 = fp16, 3 = E4M3 (the rebuilt window is fp16 for each)
};

hipError_t launch_cache_write_bf16(const CacheWriteArgs& a, hipStream_t s);
// The other projection modes (PROJ_CACHE_NORM, PROJ_QUERY, PROJ_OUT) on the
// same GEMM; `mode` selects the epilogue.
hipError_t launch_projection_bf16(const CacheWriteArgs& a, int mode, hipStream_t s);
hipError_t launch_cache_write_f32(const CacheWriteArgs& a, hipStream_t s);
bool cache_write_bf16_supported(int width, int hidden);

hipError_t launch_attend_bf16(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_f32(const AttendArgs& a, hipStream_t s);
bool attend_bf16_supported(int d_c, int d_rope, int d_nope, int d_v);

// Dense path: rotated queries go to a.qrot ([B][n_h * Lq_pad][d_h], Lq_pad =
// Lq rounded up to the schedule's block_rows); opart/ml hold per-slot partials
// as in the latent path.
hipError_t launch_mha_attend_bf16_ws(const MhaAttendArgs& a, float* opart, float* ml,
                                     const Schedule& sched, hipStream_t s);

// Weight-level folds around the absorbed path (mla_block.hip), each written as
// two bf16 parts (value, remainder) of the fp32 product:
//  query:  w_qf[part][h][i][k] = sum_n w_uk[h][n][i] w_q[h*d_qk + n][k] (i < d_c),
//          w_q[h*d_qk + d_nope + i - d_c][k] (d_c <= i < d_c + d_rope);
//  output: w_fo[part][c][h*d_c + i] = sum_v w_o[c][h*d_v + v] w_uv[h][v][i].
struct FoldArgs {
  const void* w_q;   // [n_h * (d_nope + d_rope)][hidden] bf16
  const void* w_uk;  // [n_h][d_nope][d_c] bf16
  const void* w_o;   // [hidden][n_h * d_v] bf16
  const void* w_uv;  // [n_h][d_v][d_c] bf16
  void* out;         // [2][...] bf16
  int n_h, d_nope, d_rope, d_v, d_c, hidden;
};
hipError_t launch_fold_query(const FoldArgs& f, hipStream_t s);
hipError_t launch_fold_output(const FoldArgs& f, hipStream_t s);

// Attention block (mla_attend_block): the absorbed core's partials merged,
// normalised and written as the latent outputs o_lat [B*Lq][n_h*d_c] in two
// bf16 parts (o_hi, o_lo), the operand of the folded output projection.
hipError_t launch_attend_core_only(const AttendArgs& a, hipStream_t s);
hipError_t launch_merge_latent(const AttendArgs& a, void* o_hi, void* o_lo, hipStream_t s);

// Static device scratch of mla_attend_noalloc (mla_noalloc.hip): its size, and
// its address on the calling thread's current device (looked up once per
// device; hipErrorInvalidSymbol if the lookup gives nothing).
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_for_current_device(void** out);

// Compute units of the current device (queried once per device).
int device_cu_count();
hipError_t launch_mha_attend_f32(const MhaAttendArgs& a, hipStream_t s);
bool mha_attend_bf16_supported(int d_h);

// Expand-then-attend: the rebuild kernels (then launch_mha_attend_bf16_ws on
// the expanded buffer).
bool expand_supported(int d_c, int d_rope, int d_nope, int d_v);
hipError_t launch_expand_kv(const ExpandArgs& a, hipStream_t s);

}  // namespace mla
