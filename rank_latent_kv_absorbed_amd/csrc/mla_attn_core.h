// Flash-style attention core shared by the latent (absorbed) path and the
// dense comparison path, for gfx950 MFMA (fp16 or bf16 operands, fp32 sums).
//
// Rows are prepared query rows (cache type, pre-scaled by log2(e)/sqrt(d));
// keys are ring rows of the window.  A block of NW waves owns row groups of
// 32 * NW rows (32 per wave) and walks key tiles of KT keys (CoreShape: 8 x 64
// for many rows, narrower blocks on 32-key tiles for a few rows).  A wave whose
// 32 rows are all padding still loads its share of each tile but skips the
// arithmetic:
//
//  * Schedule (Schedule in mla_launch.h): whole row groups data-parallel
//    while they last, the remainder balanced stream-K style with main blocks
//    in key-tile lockstep and a short, L2-resident tail range shared by the
//    spare blocks, so every compute unit gets the same work however the row
//    count divides.  A block writes one partial (un-normalised value sums,
//    running max, running sum) per row-group segment; the merge kernels
//    combine a group's partials by log-sum-exp.
//  * Key tiles move HBM -> LDS with gfx950's direct 16-byte loads
//    (global_load_lds_dwordx4): each wave instruction fills one contiguous
//    KiB of LDS, lane l writing bytes [16l, 16l+16).  Rows are padded by one
//    16-byte chunk; padding lanes are switched off.  Two tile buffers (two
//    distinct LDS arrays, used alternately by an unrolled step pair so that
//    every access names its buffer): the next tile streams in while the
//    current one is consumed, one barrier per tile.
//  * Scores S^T[key][row] = sum_d K[key][d] Q[row][d] on 32x32x16 MFMA; a
//    segment's query fragments stay in registers.  In this orientation a lane
//    owns one row (MFMA column): the row's running max and sum live in the
//    lane, and one exchange with the other half-wave covers the whole tile.
//  * Values O^T[dim][row] += sum_key V^T[dim][key] P[row][key]: the V^T
//    operand is read straight from the key-major tile with the LDS transpose
//    read (ds_read_b64_tr_b16), so no transposed copy of V is stored.
//  * Online softmax in the exp2 domain with a lazy rescale: the running max
//    is raised (and O, l rescaled) only when a score exceeds it by more than
//    2^8, so most tiles skip the rescale; probabilities stay <= 256.
//
// Latent rows (SHARED_KV): K = [c | k^R] and V = c are one cached row, so the
// value operand reads the first DV columns of the key tile.  Dense rows: K and
// V of head h are separate slices of the cached row, both staged per key.
#pragma once

#include "mla_device.h"

namespace mla {

struct AttnCore {
  const void* qrows;     // [B][R][DQK] elements of the cache type
  const void* ring;      // [B][ring_rows][ring_stride]
  float* opart;          // [n_slots][B][R][DV]  un-normalised value sums
  float* ml;             // [n_slots][B][R][2]   running max (log2 units), sum
  int64_t ring_rows;
  int ring_stride;       // elements per cached token row
  int k_off, v_off;      // offsets of K and V of head 0 inside a cached row
  int head_stride;       // offset step per head (0 for the shared latent row)
  int R;                 // rows per batch element (dense: a multiple of the
                         // block rows per head; latent: ragged)
  int rows_per_head;     // rows of one head (latent: R)
  int valid_per_head;    // rows of a head that are real (rest is padding)
  int B, Lk;
  Schedule sched;
  int64_t key_slot0;     // ring slot of resident key 0
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS transpose read: within each 16-lane group, lane i receives element i%4
// of the 8-byte rows addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Direct 16-byte global -> LDS load (global_load_lds_dwordx4): lane l of the
// wave writes LDS bytes [lds + 16 l, lds + 16 l + 16); `lds` must be uniform.
__device__ __forceinline__ void global_to_lds16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}

// Raise-the-max threshold of the lazy rescale (log2 units).
constexpr float kRescaleThreshold = 8.0f;

// Register budget: two waves per SIMD whatever the block size, so that narrow
// blocks can share a compute unit.
template <typename E, int DQK, int DV, int NW, int KT, bool SHARED_KV>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_core_kernel(AttnCore a) {
  typedef typename Elem<E>::v8 V8;
  constexpr int NKS = DQK / 16;               // MFMA depth steps of the score product
  constexpr int NDT = DV / 32;                // 32-wide tiles of the value product
  constexpr int BR = NW * 32;                 // rows per row group
  constexpr int NKB = KT / 32;                // 32-key blocks per tile
  constexpr int KCH = DQK / 8;                // 16-byte chunks of K per key
  constexpr int CPK = SHARED_KV ? KCH : KCH + DV / 8;  // chunks staged per key
  constexpr int RCH = CPK + 1;                // chunks per padded LDS row
  constexpr int KSTR = RCH * 8;               // padded LDS row stride (elements)
  constexpr int VOFF = SHARED_KV ? 0 : DQK;   // V columns inside an LDS row
  constexpr int CHUNKS = KT * RCH;            // 16-byte chunks per tile
  constexpr int SPANS = (CHUNKS + 63) / 64;   // 1-KiB direct-load spans per tile
  constexpr int TILE = KT * KSTR;             // elements per tile buffer
  static_assert(KT == 32 || KT == 64, "key tiles are one or two 32-key MFMA blocks");
  static_assert(!SHARED_KV || DV <= DQK, "shared rows hold V inside K");

  __shared__ __attribute__((aligned(1024))) E kt0[TILE];
  __shared__ __attribute__((aligned(1024))) E kt1[TILE];

  const Schedule& sc = a.sched;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int g = blockIdx.x;
  const int n_steps = sched_block_steps(sc, g);

  // Issue the direct loads of key tile kt of batch element b into `dst`.  Keys
  // past the window re-load the last key (their scores are masked), so every
  // LDS row a wave reads holds finite cache data.
  auto load_tile = [&](int b, int rg, int kt, E* dst) {
    const E* ring = (const E*)a.ring + (size_t)b * a.ring_rows * a.ring_stride;
    const int head = (rg * BR) / a.rows_per_head;
    const int koff = a.k_off + head * a.head_stride;
    const int voff = a.v_off + head * a.head_stride;
#pragma unroll
    for (int sp = w; sp < SPANS; sp += NW) {
      const int c = sp * 64 + l;
      const int key = c / RCH, q = c - (c / RCH) * RCH;
      if (c < CHUNKS && q < CPK) {
        const int kg = min(kt * KT + key, a.Lk - 1);
        int64_t slot = a.key_slot0 + kg;
        if (slot >= a.ring_rows) slot -= a.ring_rows;
        const E* src = ring + slot * a.ring_stride + (q < KCH ? koff + q * 8 : voff + (q - KCH) * 8);
        global_to_lds16(src, dst + sp * 512);
      }
    }
  };

  // lane-constant parts of the transpose-read addresses
  const int tr_key = 4 * hi + ((l & 15) >> 2);           // key offset of this lane's row
  const int tr_col = 16 * ((l & 31) >> 4) + 4 * (l & 3);  // column offset in a 32-wide tile

  V8 qf[NKS];
  f32x16 o[NDT];
  float m = -INFINITY, lsum = 0.0f;
  int row = 0;
  bool live = false;  // this wave's rows include a real one (wave-uniform)

  // One step: `cur` holds the key tile of step i; prefetch step i+1 into `nxt`.
  auto step = [&](int i, const E* cur, E* nxt) {
    const StepInfo si = sched_decode(sc, g, i);
    const int b = si.grp / sc.n_rg;
    const int rg = si.grp - b * sc.n_rg;
    const int kt = si.kt;

    if (si.first) {  // new row-group segment: queries in, state reset
      row = rg * BR + w * 32 + lo;
      const int row0 = rg * BR + w * 32;  // rows of a wave never straddle a head
      live = row0 < a.R && (row0 % a.rows_per_head) < a.valid_per_head;
      const bool ok = row < a.R && (row % a.rows_per_head) < a.valid_per_head;
      const E* src = (const E*)a.qrows + ((size_t)b * a.R + (ok ? row : 0)) * DQK + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = ok ? ld8<E>(src + 16 * ks) : zero8<E>();
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
      m = -INFINITY;
      lsum = 0.0f;
    }
    if (i + 1 < n_steps) {
      const StepInfo sn = sched_decode(sc, g, i + 1);
      const int b1 = sn.grp / sc.n_rg;
      load_tile(b1, sn.grp - b1 * sc.n_rg, sn.kt, nxt);
    }

    if (live) {
      f32x16 sv[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[kb][r] = 0.0f;
        const E* krow = cur + (kb * 32 + lo) * KSTR + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sv[kb] = Elem<E>::mfma(ld8<E>(krow + 16 * ks), qf[ks], sv[kb]);
      }
      const int t0 = kt * KT;
      if (t0 + KT > a.Lk) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t0 + kb * 32 + acc_row(r, hi) >= a.Lk) sv[kb][r] = -INFINITY;
      }

      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // lazy rescale: raise the max only when a score passes it by > 2^8
      if (__ballot(mx > m + kRescaleThreshold)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = exp2_fast(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      V8 pf[NKB][2];
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(sv[kb][r] - m);
          ps += p;
          pf[kb][r >> 3][r & 7] = Elem<E>::from(p);
        }
      lsum += ps;

#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const E* vrow = cur + (kb * 32 + 16 * st + tr_key) * KSTR + VOFF + tr_col;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const i16x4 lo4 = lds_read_tr16(vrow + dt * 32);
            const i16x4 hi4 = lds_read_tr16(vrow + 8 * KSTR + dt * 32);
            const V8 va = __builtin_bit_cast(V8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            o[dt] = Elem<E>::mfma(va, pf[kb][st], o[dt]);
          }
        }

      if (si.last) {  // segment ends: write this block's partial
        const int slot = si.slot;
        const float ltot = lsum + __shfl_xor(lsum, 32);
        if (row < a.R) {
          const size_t prow = ((size_t)slot * a.B + b) * a.R + row;
          float* op = a.opart + prow * DV;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
              f32x4 v = {o[dt][4 * gg], o[dt][4 * gg + 1], o[dt][4 * gg + 2], o[dt][4 * gg + 3]};
              *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * gg + 4 * hi) = v;
            }
          if (hi == 0) {
            a.ml[prow * 2] = m;
            a.ml[prow * 2 + 1] = ltot;
          }
        }
      }
    }  // live
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (n_steps <= 0) return;
  {
    const StepInfo s0 = sched_decode(sc, g, 0);
    const int b = s0.grp / sc.n_rg;
    load_tile(b, s0.grp - b * sc.n_rg, s0.kt, kt0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = 0; i < n_steps; i += 2) {
    step(i, kt0, kt1);
    if (i + 1 < n_steps) step(i + 1, kt1, kt0);
  }
}

// Log-sum-exp merge of one row's partials into `acc` (n values from column
// c0, n a multiple of 4): acc = sum_k w_k O_k / sum_k w_k l_k with
// w_k = 2^(m_k - max_k m_k).
__device__ __forceinline__ void merge_row_partials(const AttnCore& a, int DV, int b, int row,
                                                   int c0, int n, float* acc) {
  const Schedule& sc = a.sched;
  const int n_part = sched_group_slots(sc, b * sc.n_rg + row / sc.block_rows);
  float M = -INFINITY;
  for (int k = 0; k < n_part; ++k) M = fmaxf(M, a.ml[(((size_t)k * a.B + b) * a.R + row) * 2]);
  for (int i = 0; i < n; ++i) acc[i] = 0.0f;
  float L = 0.0f;
  for (int k = 0; k < n_part; ++k) {
    const size_t prow = ((size_t)k * a.B + b) * a.R + row;
    const float wgt = exp2_fast(a.ml[prow * 2] - M);
    L += wgt * a.ml[prow * 2 + 1];
    const float* op = a.opart + prow * DV + c0;
    for (int i = 0; i < n; i += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(op + i);
      acc[i] += wgt * x[0];
      acc[i + 1] += wgt * x[1];
      acc[i + 2] += wgt * x[2];
      acc[i + 3] += wgt * x[3];
    }
  }
  const float inv = 1.0f / L;
  for (int i = 0; i < n; ++i) acc[i] *= inv;
}

}  // namespace mla
