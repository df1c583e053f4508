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

// Fused cache write: y = W x for every token of n whole frames, RoPE on the
// rotated columns, round to the storage dtype, scatter rows to ring slots.
struct CacheWriteArgs {
  const void* x;          // [M][hidden], M = batch * tokens_per_batch
  const void* w;          // rows [0, w_split) of the [width][hidden] projection
  const void* w2;         // rows [w_split, width) (may alias w + w_split*hidden)
  int w_split;
  void* ring;             // [batch][ring_rows][width]
  int64_t M;
  int tokens_per_batch;   // n_frames * T
  int hidden;
  int width;              // output columns (latent: d_c + d_rope; dense: 2 * n_h * d_h)
  int rot_begin;          // first rotated column
  int rot_end;            // one past the last rotated column
  int rot_group;          // rotated columns restart their pair count every rot_group
  int T, grid_w, W;
  int64_t ring_rows;      // W * T
  int64_t frame0;
  int out_type;           // ring element type: 1 = bf16, 2 = fp16 (2-byte path only)
  RopeTable rope;
};

// Absorbed latent attention.
struct AttendArgs {
  const void* q;          // [B][Lq][n_h][d_nope + d_rope]
  const void* ring;       // [B][ring_rows][d_c + d_rope]
  const void* w_uk;       // [n_h][d_nope][d_c]
  const void* w_uv;       // [n_h][d_v][d_c]
  float* out;             // [B][Lq][n_h][d_v]
  void* qcat;             // workspace [B][R][d_c + d_rope] cache type, R = Lq * n_h
  float* opart;           // workspace [n_split][B][R][d_c]
  float* ml;              // workspace [n_split][B][R][2]  (running max (log2 units), sum)
  int B, Lq, n_h, d_nope, d_rope, d_v, d_c;
  int64_t q_token0;
  int T, grid_w;
  int64_t ring_rows;
  int64_t key_slot0;      // ring slot of resident key 0
  int Lk;                 // resident keys
  int n_split;
  int keys_per_split;     // multiple of the key tile
  int cache_type;         // 1 = bf16, 2 = fp16 (2-byte path); inputs are bf16
  float qscale;           // log2(e) / sqrt(d_nope + d_rope)
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
  int B, Lq, n_h, d_h;
  int64_t q_token0;
  int T, grid_w;
  int64_t ring_rows;
  int64_t key_slot0;
  int Lk;
  int cache_type;
  float qscale;
  hipEvent_t ev_start;
  hipEvent_t ev_stop;
  RopeTable rope;
};

// Key tile of the attention kernels (keys staged in LDS per step).
constexpr int kKeyTile = 64;

hipError_t launch_cache_write_bf16(const CacheWriteArgs& a, hipStream_t s);
hipError_t launch_cache_write_f32(const CacheWriteArgs& a, hipStream_t s);
bool cache_write_bf16_supported(int width, int hidden);

hipError_t launch_attend_bf16(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_f32(const AttendArgs& a, hipStream_t s);
bool attend_bf16_supported(int d_c, int d_rope, int d_nope, int d_v);

// Dense path: rotated queries go to a.qrot ([B][n_h * mha_lq_pad(Lq)][d_h]
// bf16); opart/ml hold per-key-range partials as in the latent path.
int mha_lq_pad(int Lq);
hipError_t launch_mha_attend_bf16_ws(const MhaAttendArgs& a, float* opart, float* ml, int n_split,
                                     int keys_per_split, hipStream_t s);
hipError_t launch_mha_attend_f32(const MhaAttendArgs& a, hipStream_t s);
bool mha_attend_bf16_supported(int d_h);

}  // namespace mla
