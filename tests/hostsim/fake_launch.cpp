// Recording launcher for CPU tests of the host library: the kernels are
// replaced by functions that store their arguments (and can be told to fail),
// so window bookkeeping, validation and launch arguments run on any machine.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "mla_launch.h"

namespace {
mla::CacheWriteArgs g_write;
mla::AttendArgs g_attend;
mla::MhaAttendArgs g_mha;
mla::Schedule g_mha_sched;
mla::ExpandArgs g_expand;
float* g_mha_opart = nullptr;
float* g_mha_ml = nullptr;
// 1 write bf16, 2 write f32, 3 attend bf16, 4 attend f32, 5 mha bf16, 6 mha f32, 7 expand
int g_kind = 0;
int g_count = 0;
int g_fail = 0;
hipError_t rec(int kind) {
  g_kind = kind;
  ++g_count;
  if (g_fail) {
    g_fail = 0;
    return hipErrorLaunchFailure;
  }
  return hipSuccess;
}
}  // namespace

namespace mla {
bool cache_write_bf16_supported(int width, int hidden) {
  return width > 0 && width % 32 == 0 && hidden > 0 && hidden % 64 == 0;
}
bool attend_bf16_supported(int d_c, int d_rope, int d_nope, int d_v) {
  return (d_c == 64 || d_c == 128 || d_c == 192) && d_rope == 32 && d_nope % 16 == 0 && d_nope > 0 &&
         d_v % 32 == 0 && d_v > 0;
}
bool mha_attend_bf16_supported(int d_h) { return d_h == 128; }
int device_cu_count() { return 256; }
hipError_t launch_cache_write_bf16(const CacheWriteArgs& a, hipStream_t) { g_write = a; return rec(1); }
hipError_t launch_cache_write_f32(const CacheWriteArgs& a, hipStream_t) { g_write = a; return rec(2); }
hipError_t launch_attend_bf16(const AttendArgs& a, hipStream_t) { g_attend = a; return rec(3); }
hipError_t launch_attend_f32(const AttendArgs& a, hipStream_t) { g_attend = a; return rec(4); }
hipError_t launch_mha_attend_bf16_ws(const MhaAttendArgs& a, float* opart, float* ml,
                                     const Schedule& sc, hipStream_t) {
  g_mha = a;
  g_mha_sched = sc;
  g_mha_opart = opart;
  g_mha_ml = ml;
  return rec(5);
}
bool expand_supported(int d_c, int d_rope, int d_nope, int d_v) {
  return (d_c == 64 || d_c == 128 || d_c == 192) && d_nope == 96 && d_rope == 32 && d_v == 128;
}
hipError_t launch_expand_kv(const ExpandArgs& a, hipStream_t) { g_expand = a; return rec(7); }
hipError_t launch_mha_attend_f32(const MhaAttendArgs& a, hipStream_t) { g_mha = a; return rec(6); }
mla::CacheWriteArgs g_proj[2];  // the last query and output projections
int g_proj_mode = -1;
hipError_t launch_projection_bf16(const CacheWriteArgs& a, int mode, hipStream_t) {
  g_proj_mode = mode;
  if (mode == PROJ_CACHE_NORM) g_write = a;
  if (mode == PROJ_QUERY) g_proj[0] = a;
  if (mode == PROJ_OUT) g_proj[1] = a;
  return rec(10 + mode);
}
hipError_t launch_fold_query(const FoldArgs&, hipStream_t) { return rec(20); }
hipError_t launch_fold_output(const FoldArgs&, hipStream_t) { return rec(21); }
hipError_t launch_attend_core_only(const AttendArgs& a, hipStream_t) { g_attend = a; return rec(22); }
hipError_t launch_merge_latent(const AttendArgs&, void*, void*, hipStream_t) { return rec(23); }
// The static scratch stands at a fixed fake address (never dereferenced).
hipError_t scratch_for_current_device(void** out) {
  *out = (void*)(uintptr_t)(3ULL << 40);
  return hipSuccess;
}
}  // namespace mla

extern "C" {
int fake_kind() { return g_kind; }
// The last projection of `which` (0 query, 1 output): M, tokens_per_batch,
// hidden, width, rot_begin, rot_end, rot_group, rot_skip, passes, w_part[1],
// x_part[2], q_token0, ring pointer, out_lo pointer, x pointer.
void fake_proj_info(int which, long long* o) {
  const mla::CacheWriteArgs& a = mla::g_proj[which];
  long long v[15] = {a.M, a.tokens_per_batch, a.hidden, a.width, a.rot_begin, a.rot_end,
                     a.rot_group, a.rot_skip, a.passes, a.w_part[1], a.x_part[2], a.q_token0,
                     (long long)(intptr_t)a.ring, (long long)(intptr_t)a.out_lo, (long long)(intptr_t)a.x};
  memcpy(o, v, sizeof(v));
}
// Element types of the last cache write, latent attend and query projection.
void fake_type_info(int* o) {
  o[0] = g_write.out_type;
  o[1] = g_attend.cache_type;
  o[2] = mla::g_proj[0].out_type;
  o[3] = g_expand.cache_type;
  o[4] = g_mha.cache_type;
}
float fake_write_eps() { return g_write.eps; }
int fake_write_norm_cols() { return g_write.norm_cols; }
int fake_count() { return g_count; }
void fake_fail_next() { g_fail = 1; }
// frame0, M, tokens_per_batch, width, ring_rows, rot_begin, rot_end, rot_group, w_split, hidden
void fake_write_info(long long* o) {
  const mla::CacheWriteArgs& a = g_write;
  long long v[10] = {a.frame0, a.M, a.tokens_per_batch, a.width, a.ring_rows, a.rot_begin,
                     a.rot_end, a.rot_group, a.w_split, a.hidden};
  memcpy(o, v, sizeof(v));
}
// key_slot0, Lk, B, Lq, q_token0, ring_rows, n_h, d_c, then the schedule:
// n_rg, n_kt, n_groups, n_blocks, full_rounds, rem, main_len, tail_per_block, n_slots,
// block_rows, key_tile, stages
void fake_attend_info(long long* o) {
  const mla::AttendArgs& a = g_attend;
  const mla::Schedule& s = a.sched;
  long long v[20] = {a.key_slot0, a.Lk, a.B, a.Lq, a.q_token0, a.ring_rows, a.n_h, a.d_c,
                     s.n_rg, s.n_kt, s.n_groups, s.n_blocks, s.full_rounds, s.rem, s.main_len,
                     s.tail_per_block, s.n_slots, s.block_rows, s.key_tile, s.stages};
  memcpy(o, v, sizeof(v));
}
// The last (which = 0: latent, 1: dense) attend's schedule as the kernels decode it.
static const mla::Schedule& sched_of(int which) { return which ? g_mha_sched : g_attend.sched; }
int fake_sched_block_of(int which, int hw) { return mla::sched_block_of(sched_of(which), hw); }
int fake_sched_steps(int which, int g) { return mla::sched_block_steps(sched_of(which), g); }
void fake_sched_decode(int which, int g, int i, int* o) {
  const mla::StepInfo si = mla::sched_decode(sched_of(which), g, i);
  o[0] = si.grp;
  o[1] = si.kt;
  o[2] = si.slot;
  o[3] = si.first;
  o[4] = si.last;
}
// Walk every block of the last schedule with the incremental cursor and
// count the steps where it differs from sched_decode.
int fake_sched_cursor_mismatches(int which) {
  const mla::Schedule& s = sched_of(which);
  int bad = 0;
  for (int g = 0; g < s.n_blocks; ++g) {
    const int n = mla::sched_block_steps(s, g);
    if (n <= 0) continue;
    mla::SchedCursor c;
    mla::sched_cursor_seek(s, g, n, 0, c);
    for (int i = 0; i < n; ++i) {
      const mla::StepInfo d = mla::sched_decode(s, g, i);
      if (c.i != i || c.si.grp != d.grp || c.si.kt != d.kt || c.si.slot != d.slot ||
          c.si.first != d.first || c.si.last != d.last)
        ++bad;
      const bool seg = mla::sched_cursor_next(s, g, n, c);
      if (i + 1 < n && seg != mla::sched_decode(s, g, i + 1).first) ++bad;
    }
  }
  return bad;
}
int fake_sched_group_slots(int which, int grp) {
  return mla::sched_group_slots(sched_of(which), grp);
}
float fake_attend_qscale() { return g_attend.qscale; }
// Query norm the last latent (which = 0) or per-head (which = 1) attend
// carried: the gain pointer, and its epsilon through fake_qnorm_eps.
long long fake_qnorm_gamma(int which) {
  return (long long)(intptr_t)(which ? g_mha.qn_gamma : g_attend.qn_gamma);
}
float fake_qnorm_eps(int which) { return which ? g_mha.qn_eps : g_attend.qn_eps; }
// The last latent attend's workspace pointers: qcat, qcat_lo, opart, ml.
void fake_attend_ptrs(long long* o) {
  long long v[4] = {(long long)(intptr_t)g_attend.qcat, (long long)(intptr_t)g_attend.qcat_lo,
                    (long long)(intptr_t)g_attend.opart, (long long)(intptr_t)g_attend.ml};
  memcpy(o, v, sizeof(v));
}
// key_slot0, Lk, B, Lq, q_token0, n_rg, n_kt, n_groups, n_blocks, full_rounds, rem,
// main_len, tail_per_block, n_slots, block_rows, key_tile, stages
void fake_mha_info(long long* o) {
  const mla::Schedule& s = g_mha_sched;
  long long v[17] = {g_mha.key_slot0, g_mha.Lk, g_mha.B, g_mha.Lq, g_mha.q_token0, s.n_rg,
                     s.n_kt, s.n_groups, s.n_blocks, s.full_rounds, s.rem, s.main_len,
                     s.tail_per_block, s.n_slots, s.block_rows, s.key_tile, s.stages};
  memcpy(o, v, sizeof(v));
}
// The last expand: B, ring_rows, key_slot0, Lk, n_h, d_nope, d_rope, d_c, d_v,
// cache_type, then the kv, ring and w_uk pointers as integers.
void fake_expand_info(long long* o) {
  const mla::ExpandArgs& a = g_expand;
  long long v[13] = {a.B, a.ring_rows, a.key_slot0, a.Lk, a.n_h, a.d_nope, a.d_rope, a.d_c, a.d_v,
                     a.cache_type, (long long)(intptr_t)a.kv, (long long)(intptr_t)a.ring,
                     (long long)(intptr_t)a.w_uk};
  memcpy(o, v, sizeof(v));
}
// The last dense attend's ring_rows, d_h, ring, qrot, opart, ml, q, out pointers,
// qscale*1e6 and the qrot_lo pointer.
void fake_mha_ptrs(long long* o) {
  const mla::MhaAttendArgs& a = g_mha;
  long long v[10] = {a.ring_rows, a.d_h, (long long)(intptr_t)a.ring, (long long)(intptr_t)a.qrot,
                     (long long)(intptr_t)g_mha_opart, (long long)(intptr_t)g_mha_ml,
                     (long long)(intptr_t)a.q, (long long)(intptr_t)a.out,
                     (long long)llround((double)a.qscale * 1e6), (long long)(intptr_t)a.qrot_lo};
  memcpy(o, v, sizeof(v));
}
// which: 0 = last write, 1 = last attend, 2 = last dense attend
int fake_rope(int which, int* axis, double* inv_freq) {
  const mla::RopeTable& t = which == 0 ? g_write.rope : (which == 1 ? g_attend.rope : g_mha.rope);
  for (int p = 0; p < t.n_pairs; ++p) {
    axis[p] = t.axis[p];
    inv_freq[p] = t.inv_freq[p];
  }
  return t.n_pairs;
}
}
