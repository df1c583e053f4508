// Flash-style attention core shared by the latent (absorbed) path and the
// dense comparison path, for gfx950 MFMA (bf16 or fp16 operands, fp32 sums).
//
// Rows are prepared query rows (cache type, pre-scaled by log2(e)/sqrt(d)); keys are
// ring rows of the window.  A 256-thread block owns 128*RB rows (four waves of
// 32*RB rows) and one key range; it walks the range in tiles of kKeyTile keys
// staged in LDS twice: key-major for the score product and transposed
// (dim-major) for the value product.  The next tile's global loads are issued
// into registers before the current tile is consumed.
//
//   S^T[key][row] = sum_d K[key][d] Q[row][d]     (A = key tile, B = queries)
//   O^T[dim][row] += sum_key V^T[dim][key] P[row][key]
// With this orientation a lane owns one row (MFMA column), so the running max
// and sum of that row live in the lane; the other half-wave holds the row's
// other keys and one exchange combines them.
//
// Latent rows (SHARED_KV): K = [c | k^R] and V = c are the same cached row, so
// one global load feeds both LDS copies.  Dense rows: K and V of head h are
// separate slices of the cached row.
#pragma once

#include "mla_device.h"

namespace mla {

struct AttnCore {
  const void* qrows;     // [B][R][DQK] elements of the cache type
  const void* ring;      // [B][ring_rows][ring_stride]
  float* opart;          // [n_split][B][R][DV]   un-normalised value sums
  float* ml;             // [n_split][B][R][2]    running max (log2 units), sum
  int64_t ring_rows;
  int ring_stride;       // elements per cached token row
  int k_off, v_off;      // offsets of K and V of head 0 inside a cached row
  int head_stride;       // offset step per head (0 for the shared latent row)
  int R;                 // rows per batch element
  int rows_per_head;     // rows of one head (latent: R)
  int valid_per_head;    // rows of a head that are real (rest is padding)
  int B, Lk, n_split, keys_per_split;
  int64_t key_slot0;     // ring slot of resident key 0
};

// Position of key u (0..31 inside a 32-key group) in the transposed V tile:
// bits 2 and 3 swapped, so that a lane's eight consecutive positions are the
// eight keys its P fragment holds for one 16-deep MFMA step.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <typename E, int DQK, int DV, int RB, bool SHARED_KV>
__global__ __launch_bounds__(256) void attn_core_kernel(AttnCore a) {
  typedef typename Elem<E>::v8 V8;
  constexpr int NKS = DQK / 16;             // MFMA depth steps of the score product
  constexpr int NDT = DV / 32;              // 32-wide tiles of the value product
  constexpr int KT = kKeyTile;              // keys per LDS tile
  constexpr int KSTR = DQK + 8;             // padded key-row stride (elements)
  constexpr int VSTR = KT + 8;              // padded transposed-V row stride (elements)
  constexpr int KCH = DQK / 8;              // 16-byte chunks of K per key
  constexpr int CPK = SHARED_KV ? KCH : KCH + DV / 8;
  constexpr int NPRE = KT * CPK / 256;
  static_assert(KT * CPK % 256 == 0, "tile must split evenly over the block");
  static_assert(!SHARED_KV || DV <= DQK, "shared rows hold V inside K");

  __shared__ E kt[KT * KSTR];
  __shared__ E vt[DV * VSTR];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int b = blockIdx.z, split = blockIdx.y;
  const int blk_row0 = blockIdx.x * (128 * RB);
  const int row0 = blk_row0 + w * (32 * RB);
  const int head = blk_row0 / a.rows_per_head;
  const int k_begin = split * a.keys_per_split;
  const int k_end = min(a.Lk, k_begin + a.keys_per_split);

  V8 qf[RB][NKS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + rb * 32 + lo;
    const bool ok = row < a.R && (row % a.rows_per_head) < a.valid_per_head;
    const E* src = (const E*)a.qrows + ((size_t)b * a.R + (ok ? row : 0)) * DQK + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[rb][ks] = ok ? ld8<E>(src + 16 * ks) : zero8<E>();
  }

  f32x16 o[RB][NDT];
  float m[RB], lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    lsum[rb] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[rb][dt][r] = 0.0f;
  }

  const E* ring = (const E*)a.ring + (size_t)b * a.ring_rows * a.ring_stride;
  const int koff = a.k_off + head * a.head_stride;
  const int voff = a.v_off + head * a.head_stride;
  u32x4 pre[NPRE];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int c = tid + 256 * i;
      const int key = c % KT, q = c / KT;
      const int kg = t0 + key;
      if (kg < k_end) {
        int64_t slot = a.key_slot0 + kg;
        if (slot >= a.ring_rows) slot -= a.ring_rows;
        const E* src = ring + slot * a.ring_stride +
                            (q < KCH ? koff + q * 8 : voff + (q - KCH) * 8);
        pre[i] = *reinterpret_cast<const u32x4*>(src);
      } else {
        pre[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int c = tid + 256 * i;
      const int key = c % KT, q = c / KT;
      if (q < KCH) *reinterpret_cast<u32x4*>(kt + key * KSTR + q * 8) = pre[i];
      const int vq = SHARED_KV ? q : q - KCH;
      if (vq >= 0 && vq * 8 < DV) {
        const V8 v = __builtin_bit_cast(V8, pre[i]);
        const int pos = (key & ~31) | vt_pos(key & 31);
#pragma unroll
        for (int j = 0; j < 8; ++j) vt[(vq * 8 + j) * VSTR + pos] = v[j];
      }
    }
  };

  if (k_begin < k_end) {
    load_tile(k_begin);
    store_tile();
  }
  __syncthreads();

  for (int t0 = k_begin; t0 < k_end; t0 += KT) {
    const bool more = t0 + KT < k_end;
    if (more) load_tile(t0 + KT);

    f32x16 s[RB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[rb][kb][r] = 0.0f;
      const E* krow = kt + (kb * 32 + lo) * KSTR + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const V8 ka = ld8<E>(krow + 16 * ks);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kb] = Elem<E>::mfma(ka, qf[rb][ks], s[rb][kb]);
      }
    }
    if (t0 + KT > k_end) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (t0 + kb * 32 + acc_row(r, hi) >= k_end) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[rb][kb][r] = -INFINITY;
          }
        }
    }

    V8 pf[RB][2][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[rb], mx);
      const float alpha = exp2f(m[rb] - mnew);
      m[rb] = mnew;
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[rb][kb][r] - mnew);
          ps += p;
          pf[rb][kb][r >> 3][r & 7] = Elem<E>::from(p);
        }
      lsum[rb] = lsum[rb] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[rb][dt][r] *= alpha;
    }

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const V8 va = ld8<E>(vt + (dt * 32 + lo) * VSTR + kb * 32 + 16 * st + 8 * hi);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[rb][dt] = Elem<E>::mfma(va, pf[rb][kb][st], o[rb][dt]);
        }
      }

    __syncthreads();
    if (more) store_tile();
    __syncthreads();
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + rb * 32 + lo;
    if (row >= a.R) continue;
    const float ltot = lsum[rb] + __shfl_xor(lsum[rb], 32);
    const size_t prow = ((size_t)split * a.B + b) * a.R + row;
    float* op = a.opart + prow * DV;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {o[rb][dt][4 * g], o[rb][dt][4 * g + 1], o[rb][dt][4 * g + 2],
                   o[rb][dt][4 * g + 3]};
        *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * g + 4 * hi) = v;
      }
    if (hi == 0) {
      a.ml[prow * 2] = m[rb];
      a.ml[prow * 2 + 1] = ltot;
    }
  }
}

// Rows per block of the core kernel.
template <int RB>
constexpr int core_block_rows() { return 128 * RB; }

}  // namespace mla
