// Flash-style attention core shared by the latent (absorbed) path and the
// dense comparison path, for gfx950 MFMA (fp16 or bf16 operands, fp32 sums).
//
// Rows are prepared query rows (cache type, pre-scaled by log2(e)/sqrt(d));
// keys are ring rows of the window.  A block of NW waves owns NW*32*RB rows
// and one key range, which it walks in tiles of kKeyTile keys:
//
//  * Key tiles move HBM -> LDS with gfx950's direct 16-byte loads
//    (global_load_lds_dwordx4): each wave instruction fills one contiguous
//    KiB of LDS, lane l writing bytes [16l, 16l+16).  Rows are padded by one
//    16-byte chunk (no bank conflicts on the score reads); padding lanes are
//    switched off.  Two tile buffers: the next tile streams in while the
//    current one is consumed, with one barrier per tile.
//  * Scores S^T[key][row] = sum_d K[key][d] Q[row][d] on 32x32x16 MFMA; the
//    query fragments stay in registers for the whole key range.  In this
//    orientation a lane owns one row (MFMA column): the row's running max and
//    sum live in the lane, and one exchange with the other half-wave combines
//    the two halves of the key tile.
//  * Values O^T[dim][row] += sum_key V^T[dim][key] P[row][key]: the V^T
//    operand is read straight from the key-major tile with the LDS transpose
//    read (ds_read_b64_tr_b16), so no transposed copy of V is ever stored.
//  * Online softmax in the exp2 domain with a lazy rescale: the running max
//    is only raised (and O, l rescaled) when a new score exceeds it by more
//    than 2^8, so most tiles skip the rescale; probabilities stay <= 256.
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

template <typename E, int DQK, int DV, int RB, int NW, bool SHARED_KV>
__global__ __launch_bounds__(NW * 64) void attn_core_kernel(AttnCore a) {
  typedef typename Elem<E>::v8 V8;
  constexpr int NKS = DQK / 16;               // MFMA depth steps of the score product
  constexpr int NDT = DV / 32;                // 32-wide tiles of the value product
  constexpr int KT = kKeyTile;                // keys per LDS tile
  constexpr int KCH = DQK / 8;                // 16-byte chunks of K per key
  constexpr int CPK = SHARED_KV ? KCH : KCH + DV / 8;  // chunks staged per key
  constexpr int RCH = CPK + 1;                // chunks per padded LDS row
  constexpr int KSTR = RCH * 8;               // padded LDS row stride (elements)
  constexpr int VOFF = SHARED_KV ? 0 : DQK;   // V columns inside an LDS row
  constexpr int SPANS = KT * RCH / 64;        // 1-KiB direct-load spans per tile
  constexpr int TILE = KT * KSTR;             // elements per tile buffer
  static_assert(KT == 64, "one span per padded chunk column needs 64-key tiles");
  static_assert(!SHARED_KV || DV <= DQK, "shared rows hold V inside K");

  __shared__ __attribute__((aligned(1024))) E kt[2 * TILE];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int b = blockIdx.z, split = blockIdx.y;
  const int blk_row0 = blockIdx.x * (NW * 32 * RB);
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

  // Issue the direct loads of tile t0 into buffer `buf`.  Keys past the range
  // re-load the last valid key (their scores are masked), so every LDS row a
  // wave reads holds finite cache data.
  auto load_tile = [&](int t0, int buf) {
#pragma unroll
    for (int sp = w; sp < SPANS; sp += NW) {
      const int c = sp * 64 + l;
      const int key = c / RCH, q = c - (c / RCH) * RCH;
      if (q < CPK) {
        int kg = min(t0 + key, k_end - 1);
        int64_t slot = a.key_slot0 + kg;
        if (slot >= a.ring_rows) slot -= a.ring_rows;
        const E* src = ring + slot * a.ring_stride + (q < KCH ? koff + q * 8 : voff + (q - KCH) * 8);
        global_to_lds16(src, kt + buf * TILE + sp * 512);
      }
    }
  };

  if (k_begin < k_end) load_tile(k_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // lane-constant parts of the LDS addresses
  const int tr_key = 4 * hi + ((l & 15) >> 2);           // key offset of this lane's row
  const int tr_col = 16 * ((l & 31) >> 4) + 4 * (l & 3);  // column offset in a 32-wide tile

  int buf = 0;
  for (int t0 = k_begin; t0 < k_end; t0 += KT, buf ^= 1) {
    const bool more = t0 + KT < k_end;
    if (more) load_tile(t0 + KT, buf ^ 1);
    const E* tile = kt + buf * TILE;

    f32x16 s[RB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[rb][kb][r] = 0.0f;
      const E* krow = tile + (kb * 32 + lo) * KSTR + 8 * hi;
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
      // lazy rescale: raise the max only when a score passes it by > 2^8
      if (__ballot(mx > m[rb] + kRescaleThreshold)) {
        const float mnew = fmaxf(m[rb], mx);
        const float alpha = exp2f(m[rb] - mnew);
        m[rb] = mnew;
        lsum[rb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[rb][dt][r] *= alpha;
      }
      const float mc = m[rb];
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[rb][kb][r] - mc);
          ps += p;
          pf[rb][kb][r >> 3][r & 7] = Elem<E>::from(p);
        }
      lsum[rb] += ps;
    }

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const E* vrow = tile + (kb * 32 + 16 * st + tr_key) * KSTR + VOFF + tr_col;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const i16x4 lo4 = lds_read_tr16(vrow + dt * 32);
          const i16x4 hi4 = lds_read_tr16(vrow + 8 * KSTR + dt * 32);
          const V8 va = __builtin_bit_cast(V8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[rb][dt] = Elem<E>::mfma(va, pf[rb][kb][st], o[rb][dt]);
        }
      }

    __builtin_amdgcn_s_waitcnt(0);
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
template <int RB, int NW>
constexpr int core_block_rows() { return NW * 32 * RB; }

}  // namespace mla
