// Absorbed latent attention for gfx950 (VideoMLA technical summary, method
// item 2, computed in absorbed form).
//
// Three kernels run back to back on the caller's stream:
//  1. qprep:    q_lat,h = W^K_up,h^T q^nope_h and q^R rotated at the query's
//               position, both scaled by log2(e)/sqrt(d_nope + d_rope), written
//               as one row [q_lat | q^R_rot] of the cache type per (token, head)
//               pair (a bf16 cache also gets the row of remainders, the bf16
//               rounding of q - bf16(q), for the split-operand core).  With a
//               query norm set, each head's query row is RMS-normalised with
//               its gain first (before the rotation and the fold).
//  2. attend:   the shared flash-style core (mla_attn_core.h).  Rows are
//               (token, head) pairs; every row scores against the same cached
//               rows [c | k^R], so a key tile staged once in LDS serves all heads
//               and tokens of a block, and V = c is read from the same tile.
//               Each block covers one key range and writes un-normalised
//               partials (O_lat, max, sum).
//  3. epilogue: merges the key ranges by log-sum-exp, normalises, and applies
//               W^V_up,h, writing fp32 output.  Many rows: one lane per row,
//               bf16 MFMA on a hi/lo split of O_lat (keeps fp32 accuracy).  A
//               few rows with many key ranges each (small query chunks): one
//               block per row, partials spread over the block, plain fp32.
#include "mla_attn_core.h"

namespace mla {

namespace {

// ---------------------------------------------------------------------------
// 1. query prologue
// ---------------------------------------------------------------------------
// W^K_up,h is staged in LDS in its natural [d_nope][DC] layout; the MFMA
// operand A[m = latent dim i][k = n] = W[n][i] comes out of it with the LDS
// transpose read, which hands lane (i, half hi) the k-slots t = 0..7 as
// n = 16 ks + 8 (t / 4) + 4 hi + t % 4.  The query operand uses the same
// k-slot order: two 8-byte loads per step.
// Store v as the cache type; with SPLIT also the remainder's rounding at lo.
template <typename E, bool SPLIT>
__device__ __forceinline__ void store_q(E* hi, E* lo, float v) {
  const E h = Elem<E>::from(v);
  *hi = h;
  if constexpr (SPLIT) *lo = Elem<E>::from(v - (float)h);
}

// NORM (a query norm is set): the gained query g q^nope (exact in fp32) enters
// the products as two bf16 parts, its leading part and the bf16 rounding of
// the remainder, against the same weights; the row's 1 / rms, a scalar that
// commutes with the fold, scales the result with the score scale.
template <typename E, int DC, bool SPLIT, bool NORM = false>
__global__ __launch_bounds__(256) void qprep_bf16_kernel(AttendArgs a) {
  constexpr int NT = DC / 32;
  constexpr int WSTR = DC + 8;                 // padded LDS row (elements)
  extern __shared__ bf16_t wlds[];             // [d_nope][WSTR]
  __shared__ float inv_s[NORM ? 128 : 1];      // 1 / rms of the block's 128 tokens
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int d_qk = a.d_nope + a.d_rope;
  const int width = DC + a.d_rope;
  const int R = a.Lq * a.n_h;

  const bf16_t* wuk = (const bf16_t*)a.w_uk + (size_t)h * a.d_nope * DC;
  for (int c = tid; c < a.d_nope * (DC / 8); c += 256) {
    const int n = c / (DC / 8), i0 = (c % (DC / 8)) * 8;
    *reinterpret_cast<bf16x8*>(wlds + n * WSTR + i0) = ld_bf16x8(wuk + (size_t)n * DC + i0);
  }
  __syncthreads();

  const int tok = blockIdx.x * 128 + w * 32 + lo;
  const bool valid = tok < a.Lq;
  const bf16_t* qrow =
      (const bf16_t*)a.q + (((size_t)b * a.Lq + (valid ? tok : 0)) * a.n_h + h) * d_qk + 4 * hi;
  const int tr_key = 4 * hi + ((l & 15) >> 2);
  const int tr_col = 16 * ((l & 31) >> 4) + 4 * (l & 3);
  f32x16 acc[NT];
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[it][r] = 0.0f;
  const bf16_t* gam = (const bf16_t*)a.qn_gamma;
  float ss = 0.0f;  // NORM: the lane's share of the row's sum of squares
  for (int k0 = 0; k0 < a.d_nope; k0 += 16) {
    bf16x8 bq = zero_bf16x8();
    if (valid) {
      const bf16x4 q0 = *reinterpret_cast<const bf16x4*>(qrow + k0);
      const bf16x4 q1 = *reinterpret_cast<const bf16x4*>(qrow + k0 + 8);
      bq = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    bf16x8 bq_lo = zero_bf16x8();
    if constexpr (NORM) {
      const bf16x4 g0 = *reinterpret_cast<const bf16x4*>(gam + k0 + 4 * hi);
      const bf16x4 g1 = *reinterpret_cast<const bf16x4*>(gam + k0 + 8 + 4 * hi);
      const bf16x8 g8 = __builtin_shufflevector(g0, g1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float x = (float)bq[t], p = x * (float)g8[t];
        ss = fmaf(x, x, ss);
        bq[t] = to_bf16(p);
        bq_lo[t] = to_bf16(p - (float)bq[t]);
      }
    }
    const bf16_t* wrow = wlds + (k0 + tr_key) * WSTR + tr_col;
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      const i16x4 lo4 = lds_read_tr16(wrow + it * 32);
      const i16x4 hi4 = lds_read_tr16(wrow + 8 * WSTR + it * 32);
      const bf16x8 wa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[it] = mfma32(wa, bq, acc[it]);
      if constexpr (NORM) acc[it] = mfma32(wa, bq_lo, acc[it]);
    }
  }
  float inv = 1.0f;
  if constexpr (NORM) {
    // the rotary part's squares (this lane's half of the row), then the row
    if (valid) {
      const bf16_t* qr = (const bf16_t*)a.q + (((size_t)b * a.Lq + tok) * a.n_h + h) * d_qk + a.d_nope;
      for (int d = hi; d < a.d_rope; d += 2) {
        const float x = (float)qr[d];
        ss = fmaf(x, x, ss);
      }
    }
    ss += __shfl_xor(ss, 32);
    inv = 1.0f / sqrtf(ss / (float)d_qk + a.qn_eps);
    if (hi == 0) inv_s[w * 32 + lo] = inv;
  }
  const size_t orow = ((size_t)b * R + (size_t)tok * a.n_h + h) * width;
  E* out = (E*)a.qcat + orow;
  if (valid) {
    const float sc = a.qscale * inv;
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typename Elem<E>::v4 o, ol;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = acc[it][4 * g + j] * sc;
          o[j] = Elem<E>::from(v);
          ol[j] = Elem<E>::from(v - (float)o[j]);
        }
        *reinterpret_cast<typename Elem<E>::v4*>(out + it * 32 + 8 * g + 4 * hi) = o;
        if constexpr (SPLIT)
          *reinterpret_cast<typename Elem<E>::v4*>((E*)a.qcat_lo + orow + it * 32 + 8 * g + 4 * hi) = ol;
      }
  }
  // rotary part: lanes walk (token, pair) of this wave's 32 tokens
  // (NORM: the gain before the rotation, the row's 1 / rms after it)
  if constexpr (NORM) __syncthreads();
  const int P = a.d_rope / 2;
  for (int e = l; e < 32 * P; e += 64) {
    const int tt = blockIdx.x * 128 + w * 32 + e / P;
    const int p = e % P;
    if (tt >= a.Lq) continue;
    const bf16_t* qr =
        (const bf16_t*)a.q + (((size_t)b * a.Lq + tt) * a.n_h + h) * d_qk + a.d_nope + 2 * p;
    float x0 = (float)qr[0], x1 = (float)qr[1];
    float sc = a.qscale;
    if constexpr (NORM) {
      x0 *= (float)gam[a.d_nope + 2 * p];
      x1 *= (float)gam[a.d_nope + 2 * p + 1];
      sc *= inv_s[w * 32 + e / P];
    }
    rope_pair(a.rope, p, token_pos(a.q_token0 + tt, a.T, a.grid_w), x0, x1);
    const size_t off = ((size_t)b * R + (size_t)tt * a.n_h + h) * width + DC + 2 * p;
    E* lo = SPLIT ? (E*)a.qcat_lo + off : nullptr;
    store_q<E, SPLIT>((E*)a.qcat + off, lo, x0 * sc);
    store_q<E, SPLIT>((E*)a.qcat + off + 1, lo + 1, x1 * sc);
  }
}

// Query prologue for a few tokens per sequence (decode-like calls): one block
// per (head, batch element).  Thread (column chunk j, row group g) holds
// W^K_up,h[n][8 j .. 8 j + 7] for rows n = g, g + NG, ... in registers, all
// loaded up front straight from global memory (the product is too small to
// pay for staging), and forms its share of q_lat for every token; the row
// groups are summed through LDS.  The MFMA kernel above serves longer chunks.
constexpr int kQprepRowsMaxLq = 8;   // tokens per sequence
constexpr int kQprepRowsMaxK = 12;   // W rows per thread (d_nope <= NG * 12)

template <int DC>
constexpr int qprep_rows_max_nope() {
  return (256 / (DC / 8)) * kQprepRowsMaxK;
}

// NORM: the queries are gained and scaled by their row's 1 / rms in fp32 as
// they are staged; the rotary pairs likewise, the gain before the rotation.
template <typename E, int DC, bool SPLIT, bool NORM = false>
__global__ __launch_bounds__(256) void qprep_rows_kernel(AttendArgs a) {
  constexpr int CH = DC / 8;                      // 8-column chunks of a W row
  constexpr int NG = 256 / CH;                    // row groups
  constexpr int NMAX = NG * kQprepRowsMaxK;       // largest d_nope served
  constexpr int QPT = (kQprepRowsMaxLq * NMAX + 255) / 256;  // query elements per thread
  __shared__ float qs[kQprepRowsMaxLq * NMAX];    // [tok][n] fp32 queries
  __shared__ float red[NG][DC];                   // one token's row-group sums
  __shared__ float inv_s[NORM ? kQprepRowsMaxLq : 1];  // 1 / rms of each token's row
  const int tid = threadIdx.x;
  const int j = tid % CH, g = tid / CH;
  const bool active = g < NG;
  const int h = blockIdx.x, b = blockIdx.y;
  const int d_nope = a.d_nope, d_qk = d_nope + a.d_rope;
  const int width = DC + a.d_rope;
  const int R = a.Lq * a.n_h;
  const bf16_t* q = (const bf16_t*)a.q;

  // Loads are unconditional (indices clamped into range) so that they all
  // issue before the first wait; rows past d_nope meet a zero query below.
  const bf16_t* wuk = (const bf16_t*)a.w_uk + (size_t)h * d_nope * DC + 8 * j;
  bf16x8 w[kQprepRowsMaxK];
#pragma unroll
  for (int k = 0; k < kQprepRowsMaxK; ++k) {
    const int n = min(min(g, NG - 1) + NG * k, d_nope - 1);
    w[k] = ld_bf16x8(wuk + (size_t)n * DC);
  }
  const int nq = a.Lq * d_nope;
  float qv[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int e = min(tid + 256 * i, nq - 1);
    const int tok = e / d_nope, n = e - tok * d_nope;
    qv[i] = (float)q[(((size_t)b * a.Lq + tok) * a.n_h + h) * d_qk + n];
  }
  const bf16_t* gam = (const bf16_t*)a.qn_gamma;
  if constexpr (NORM) {
    // wave 0: each token's sum of squares over its d_nope + d_rope values
    if (tid < 64) {
      for (int tok = 0; tok < a.Lq; ++tok) {
        const bf16_t* qr = q + (((size_t)b * a.Lq + tok) * a.n_h + h) * d_qk;
        float ss = 0.0f;
        for (int d = tid; d < d_qk; d += 64) {
          const float x = (float)qr[d];
          ss = fmaf(x, x, ss);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        if (tid == 0) inv_s[tok] = 1.0f / sqrtf(ss / (float)d_qk + a.qn_eps);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int e = tid + 256 * i;
    if (e < nq) {
      if constexpr (NORM) {
        const int tok = e / d_nope, n = e - tok * d_nope;
        qs[e] = qv[i] * (float)gam[n] * inv_s[tok];
      } else {
        qs[e] = qv[i];
      }
    }
  }
  __syncthreads();

  for (int tok = 0; tok < a.Lq; ++tok) {
    float acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int k = 0; k < kQprepRowsMaxK; ++k) {
      const int n = g + NG * k;
      const float qn = n < d_nope ? qs[tok * d_nope + n] : 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = fmaf(qn, (float)w[k][t], acc[t]);
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < 8; ++t) red[g][8 * j + t] = acc[t];
    }
    __syncthreads();
    const size_t orow = ((size_t)b * R + (size_t)tok * a.n_h + h) * width;
    for (int c = tid; c < DC; c += 256) {
      float sum = 0.0f;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) sum += red[gg][c];
      store_q<E, SPLIT>((E*)a.qcat + orow + c, SPLIT ? (E*)a.qcat_lo + orow + c : nullptr, sum * a.qscale);
    }
    __syncthreads();
  }
  // rotary part: threads walk (token, pair)
  const int P = a.d_rope / 2;
  for (int e = tid; e < a.Lq * P; e += 256) {
    const int tok = e / P, p = e - tok * P;
    const bf16_t* qr = q + (((size_t)b * a.Lq + tok) * a.n_h + h) * d_qk + d_nope + 2 * p;
    float x0 = (float)qr[0], x1 = (float)qr[1];
    float sc = a.qscale;
    if constexpr (NORM) {
      x0 *= (float)gam[d_nope + 2 * p];
      x1 *= (float)gam[d_nope + 2 * p + 1];
      sc *= inv_s[tok];
    }
    rope_pair(a.rope, p, token_pos(a.q_token0 + tok, a.T, a.grid_w), x0, x1);
    const size_t off = ((size_t)b * R + (size_t)tok * a.n_h + h) * width + DC + 2 * p;
    E* lo = SPLIT ? (E*)a.qcat_lo + off : nullptr;
    store_q<E, SPLIT>((E*)a.qcat + off, lo, x0 * sc);
    store_q<E, SPLIT>((E*)a.qcat + off + 1, lo + 1, x1 * sc);
  }
}

// ---------------------------------------------------------------------------
// 3. merge of key ranges + W^V_up epilogue
// ---------------------------------------------------------------------------
template <int DC>
__global__ __launch_bounds__(64) void epilogue_bf16_kernel(AttendArgs a) {
  constexpr int NKS = DC / 16;
  const int l = threadIdx.x, lo = l & 31, hi = l >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tok = blockIdx.x * 32 + lo;
  const bool valid = tok < a.Lq;
  const int R = a.Lq * a.n_h;
  const int row = (valid ? tok : 0) * a.n_h + h;

  // log-sum-exp merge of the partials this row's row group left behind
  const int n_part = sched_group_slots(a.sched, b * a.sched.n_rg + row / a.sched.block_rows);
  float M = -INFINITY;
  for (int k = 0; k < n_part; ++k) M = fmaxf(M, a.ml[(((size_t)k * a.B + b) * R + row) * 2]);
  float v[NKS][8];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int t = 0; t < 8; ++t) v[ks][t] = 0.0f;
  float L = 0.0f;
  for (int k = 0; k < n_part; ++k) {
    const size_t prow = ((size_t)k * a.B + b) * R + row;
    const float wgt = exp2_fast(a.ml[prow * 2] - M);
    const float lk = a.ml[prow * 2 + 1];
    L += wgt * lk;
    const float wv = wgt;  // fp32 partials (fp16 ones are merged by the per-row epilogue)
    const size_t e0 = prow * DC + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f32x4 x0 = load_part4<false>(a.opart, e0 + 16 * ks);
      const f32x4 x1 = load_part4<false>(a.opart, e0 + 16 * ks + 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[ks][t] += wv * x0[t];
        v[ks][4 + t] += wv * x1[t];
      }
    }
  }
  const float inv = valid ? 1.0f / L : 0.0f;
  bf16x8 vh[NKS], vl[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float x = v[ks][t] * inv;
      const bf16_t xh = to_bf16(x);
      vh[ks][t] = xh;
      vl[ks][t] = to_bf16(x - (float)xh);
    }

  const bf16_t* wuv = (const bf16_t*)a.w_uv + (size_t)h * a.d_v * DC + 8 * hi;
  float* out = a.out + (((size_t)b * a.Lq + tok) * a.n_h + h) * a.d_v;
  for (int vt = 0; vt < a.d_v / 32; ++vt) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const bf16_t* wr = wuv + (size_t)(vt * 32 + lo) * DC;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 wa = ld_bf16x8(wr + 16 * ks);
      acc = mfma32(wa, vh[ks], acc);
      acc = mfma32(wa, vl[ks], acc);
    }
    if (valid) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 o4 = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        *reinterpret_cast<f32x4*>(out + vt * 32 + 8 * g + 4 * hi) = o4;
      }
    }
  }
}

// Few-row variant: one 256-thread block per (token, head) row, for rows with
// many key-range partials.  Every load the row needs is in flight at once
// before any of them is used: the thread's slice of W^V_up,h (one output
// dimension per thread), the slot maxima and sums (one slot per thread), and
// its first run of partials (thread (column chunk c4, slot lane j) sums slots
// j, j + LANES, ... of four columns).  The slot weights 2^(m_k - max) go
// through LDS; the lanes are added through LDS, normalised, and the
// W^V_up,h product runs in plain fp32.
// Above this many partial slots per row group the per-row epilogue is used.
constexpr int kLaneMergeMaxSlots = 4;
// With many rows in flight (more blocks than a couple per compute unit) the
// kernel is run lean instead: a shorter run of partial loads and W^V_up,h
// read after the merge, so that several blocks share a compute unit.
constexpr int kEpiWeights = 1024;    // slot weights kept in LDS
constexpr int kEpiMaxDv = 256;       // output dimensions (one per thread)
constexpr int kEpiLeanRows = 256;    // rows (blocks) from which the lean form runs

template <int DC, bool LEAN, bool P16>
__global__ __launch_bounds__(256) void epilogue_rows_kernel(AttendArgs a) {
  constexpr int kEpiRun = LEAN ? 8 : 26;  // partial loads in flight per thread
  constexpr int C4 = DC / 4;       // 4-column chunks of a partial row
  constexpr int LANES = 256 / C4;  // slot lanes
  constexpr int NW8 = DC / 8;      // 16-byte pieces of a W^V_up row
  __shared__ float wts[kEpiWeights];
  __shared__ float red[2][4];
  __shared__ float part[LANES][DC];
  __shared__ float olat[DC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x, b = blockIdx.y;  // row = tok * n_h + h
  const int R = a.Lq * a.n_h;
  const int tok = row / a.n_h, h = row - tok * a.n_h;
  const int n_part = sched_group_slots(a.sched, b * a.sched.n_rg + row / a.sched.block_rows);
  auto prow_of = [&](int k) { return ((size_t)k * a.B + b) * R + row; };
  constexpr bool p16 = P16;
  const int c4 = tid % C4, j = tid / C4;
  const bool lane_ok = j < LANES;

  // loads, all issued before the first use
  // (Indices are clamped into range instead of predicating the loads, so
  // that none of them waits for another; slots past n_part get weight 0.)
  const bool v_ok = tid < a.d_v;
  const bf16_t* wr = (const bf16_t*)a.w_uv + ((size_t)h * a.d_v + (v_ok ? tid : 0)) * DC;
  bf16x8 wv[LEAN ? 1 : NW8];
  if constexpr (!LEAN) {
#pragma unroll
    for (int i = 0; i < NW8; ++i) wv[i] = ld_bf16x8(wr + 8 * i);
  }
  const float2 ml2 = *reinterpret_cast<const float2*>(a.ml + prow_of(min(tid, n_part - 1)) * 2);
  f32x4 x[kEpiRun];
#pragma unroll
  for (int u = 0; u < kEpiRun; ++u) {
    const int k = min(j + LANES * u, n_part - 1);
    x[u] = load_part4<P16>(a.opart, prow_of(k) * DC + 4 * c4);
  }
  const float m0 = tid < n_part ? ml2.x : -INFINITY, l0 = ml2.y;
  // normalised fp16 partials: each slot's values also weighted by its sum

  // block maximum of the slot maxima (slots past the first 256 by a loop)
  float mx = m0;
  for (int k = tid + 256; k < n_part; k += 256) mx = fmaxf(mx, a.ml[prow_of(k) * 2]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  // weights and the weighted sum of the slot sums
  float ls = 0.0f;
  for (int k = tid; k < n_part; k += 256) {
    float mk = m0, lk = l0;
    if (k != tid) {
      mk = a.ml[prow_of(k) * 2];
      lk = a.ml[prow_of(k) * 2 + 1];
    }
    const float wk = exp2_fast(mk - M);
    if (k < kEpiWeights) wts[k] = p16 ? wk * lk : wk;
    ls += wk * lk;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
  if (lane == 0) red[1][wave] = ls;
  __syncthreads();
  const float inv = 1.0f / (red[1][0] + red[1][1] + red[1][2] + red[1][3]);
  auto weight = [&](int k) {
    if (k < kEpiWeights) return wts[k];
    const float wk = exp2_fast(a.ml[prow_of(k) * 2] - M);
    return p16 ? wk * a.ml[prow_of(k) * 2 + 1] : wk;
  };

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (lane_ok) {
#pragma unroll
    for (int u = 0; u < kEpiRun; ++u) {
      const int k = j + LANES * u;
      const float wk = k < n_part ? weight(k) : 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = fmaf(wk, x[u][t], acc[t]);
    }
    // slots past the first run, a run of loads at a time
    for (int k0 = j + LANES * kEpiRun; k0 < n_part; k0 += LANES * kEpiRun) {
#pragma unroll
      for (int u = 0; u < kEpiRun; ++u)
        x[u] = load_part4<P16>(a.opart, prow_of(min(k0 + LANES * u, n_part - 1)) * DC + 4 * c4);
#pragma unroll
      for (int u = 0; u < kEpiRun; ++u) {
        const int k = k0 + LANES * u;
        const float wk = k < n_part ? weight(k) : 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = fmaf(wk, x[u][t], acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) part[j][4 * c4 + t] = acc[t];
  }
  __syncthreads();
  for (int i = tid; i < DC; i += 256) {
    float sum = 0.0f;
#pragma unroll
    for (int jj = 0; jj < LANES; ++jj) sum += part[jj][i];
    olat[i] = sum * inv;
  }
  __syncthreads();

  if (v_ok) {
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NW8; ++i) {
      const bf16x8 w8 = LEAN ? ld_bf16x8(wr + 8 * i) : wv[i];
#pragma unroll
      for (int t = 0; t < 8; ++t) sum = fmaf((float)w8[t], olat[8 * i + t], sum);
    }
    a.out[(((size_t)b * a.Lq + tok) * a.n_h + h) * a.d_v + tid] = sum;
  }
}

// ---------------------------------------------------------------------------
// fp32 path (small shapes): one block per (token, head) row, exact two-pass
// softmax in the absorbed form, plain fp32 arithmetic.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attend_f32_kernel(AttendArgs a) {
  extern __shared__ float sm[];
  const int d_qk = a.d_nope + a.d_rope;
  const int width = a.d_c + a.d_rope;
  float* qlat = sm;                  // [d_c + d_rope]
  float* part = qlat + width;        // [256] reduction scratch
  float* pk = part + 256;            // [256] probabilities of one key chunk
  float* olat = pk + 256;            // [d_c]
  const int tid = threadIdx.x;
  const int row = blockIdx.x, b = blockIdx.y;
  const int tok = row / a.n_h, h = row % a.n_h;
  const float* q = (const float*)a.q + (((size_t)b * a.Lq + tok) * a.n_h + h) * d_qk;
  const float* wuk = (const float*)a.w_uk + (size_t)h * a.d_nope * a.d_c;
  const float* ring = (const float*)a.ring + (size_t)b * a.ring_rows * width;
  const float scale = a.qscale;  // log2(e)/sqrt(d_qk)

  for (int i = tid; i < a.d_c; i += 256) {
    float acc = 0.0f;
    for (int n = 0; n < a.d_nope; ++n) acc = fmaf(q[n], wuk[(size_t)n * a.d_c + i], acc);
    qlat[i] = acc * scale;
    olat[i] = 0.0f;
  }
  for (int p = tid; p < a.d_rope / 2; p += 256) {
    float x0 = q[a.d_nope + 2 * p], x1 = q[a.d_nope + 2 * p + 1];
    rope_pair(a.rope, p, token_pos(a.q_token0 + tok, a.T, a.grid_w), x0, x1);
    qlat[a.d_c + 2 * p] = x0 * scale;
    qlat[a.d_c + 2 * p + 1] = x1 * scale;
  }
  __syncthreads();
  auto key_row = [&](int j) {
    int64_t slot = a.key_slot0 + j;
    if (slot >= a.ring_rows) slot -= a.ring_rows;
    return ring + slot * width;
  };
  auto score = [&](int j) {
    const float* k = key_row(j);
    float s = 0.0f;
    for (int i = 0; i < width; ++i) s = fmaf(qlat[i], k[i], s);
    return s;
  };
  float mx = -INFINITY;
  for (int j = tid; j < a.Lk; j += 256) mx = fmaxf(mx, score(j));
  part[tid] = mx;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) part[tid] = fmaxf(part[tid], part[tid + st]);
    __syncthreads();
  }
  const float M = part[0];
  __syncthreads();
  float lacc = 0.0f;
  for (int j0 = 0; j0 < a.Lk; j0 += 256) {
    const int j = j0 + tid;
    float p = 0.0f;
    if (j < a.Lk) p = exp2f(score(j) - M);
    pk[tid] = p;
    lacc += p;
    __syncthreads();
    const int n = min(256, a.Lk - j0);
    for (int i = tid; i < a.d_c; i += 256) {
      float acc = olat[i];
      for (int jj = 0; jj < n; ++jj) acc = fmaf(pk[jj], key_row(j0 + jj)[i], acc);
      olat[i] = acc;
    }
    __syncthreads();
  }
  part[tid] = lacc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) part[tid] += part[tid + st];
    __syncthreads();
  }
  const float inv = 1.0f / part[0];
  const float* wuv = (const float*)a.w_uv + (size_t)h * a.d_v * a.d_c;
  float* out = a.out + (((size_t)b * a.Lq + tok) * a.n_h + h) * a.d_v;
  for (int vv = tid; vv < a.d_v; vv += 256) {
    float acc = 0.0f;
    for (int i = 0; i < a.d_c; ++i) acc = fmaf(wuv[(size_t)vv * a.d_c + i], olat[i], acc);
    out[vv] = acc * inv;
  }
}

// A bf16 cache runs the core on split operands (see mla_attn_core.h).
template <typename E>
constexpr bool kSplitOf = __is_same(E, bf16_t);

// Core launch for the schedule's shape (block rows, key tile, stages).
// F8: the ring holds one-byte E4M3 rows, widened to fp16 operands (E) in the
// core; the chunk shape then runs without the ping-pong wave groups.
template <typename E, int DC, bool F8 = false>
hipError_t launch_core(const AttnCore& c, hipStream_t s) {
  const Schedule& sc = c.sched;
  const dim3 grid((unsigned)sc.n_blocks);
  constexpr bool SPLIT = kSplitOf<E>;
#define MLA_SHAPE(NW, KT, NS, ROWS)                                                                  \
  if (sc.block_rows == ROWS * NW && sc.key_tile == KT && sc.stages == NS) {                         \
    hipLaunchKernelGGL(                                                                             \
        (attn_core_kernel<E, DC + 32, DC, NW, KT, NS, true, 1, (NW == 8 && !F8), ROWS, SPLIT, F8>), \
        grid, dim3(NW * 64), 0, s, c);                                                              \
    return hipGetLastError();                                                                       \
  }
  if constexpr (SPLIT) {
    MLA_SHAPE(4, 64, 3, 32)
  } else {
    MLA_SHAPE(8, 64, 3, 32)
  }
  MLA_SHAPE(4, 32, 4, 32)
  MLA_SHAPE(4, 32, 4, 16)
  MLA_SHAPE(1, 32, 2, 32)
  MLA_SHAPE(1, 32, 2, 16)
#undef MLA_SHAPE
  return hipErrorInvalidValue;
}

// The core over the prepared queries in a.qcat (profiling events around it).
template <typename E, int DC, bool F8 = false>
hipError_t launch_core_of(const AttendArgs& a, hipStream_t s) {
  AttnCore c;
  c.qrows = a.qcat;
  c.qrows_lo = a.qcat_lo;
  c.ring = a.ring;
  c.part16 = a.part16;
  c.opart = a.opart;
  c.ml = a.ml;
  c.ring_rows = a.ring_rows;
  c.ring_stride = DC + 32;
  c.k_off = 0;
  c.v_off = 0;
  c.head_stride = 0;
  c.R = a.Lq * a.n_h;
  c.rows_per_head = c.R;
  c.valid_per_head = c.R;
  c.B = a.B;
  c.Lk = a.Lk;
  c.sched = a.sched;
  c.key_slot0 = a.key_slot0;
  if (a.ev_start != nullptr) {
    hipError_t e = hipEventRecord(a.ev_start, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_core<E, DC, F8>(c, s);
  if (e != hipSuccess) return e;
  if (a.ev_stop != nullptr) e = hipEventRecord(a.ev_stop, s);
  return e;
}

// Latent outputs of the attention block: thread per (row, 8 latent columns)
// merges the row's partials by log-sum-exp, normalises, and writes the 8
// values as two bf16 parts (value, remainder) into token rows
// [B * Lq][n_h * DC] (row tok * n_h + h of sequence b is that token's head h).
template <int DC, bool P16>
__global__ __launch_bounds__(256) void merge_latent_kernel(AttendArgs a, bf16_t* o_hi, bf16_t* o_lo) {
  constexpr int C8 = DC / 8;
  const int R = a.Lq * a.n_h;
  const int64_t n = (int64_t)a.B * R * C8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int c8 = (int)(idx % C8);
  const int64_t br = idx / C8;
  const int b = (int)(br / R), row = (int)(br - (int64_t)b * R);
  AttnCore c;
  c.opart = a.opart;
  c.ml = a.ml;
  c.part16 = a.part16;
  c.R = R;
  c.B = a.B;
  c.sched = a.sched;
  float acc[8];
  merge_row_partials<P16>(c, DC, b, row, 8 * c8, 8, acc);
  bf16x8 h8, l8;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    h8[t] = to_bf16(acc[t]);
    l8[t] = to_bf16(acc[t] - (float)h8[t]);
  }
  const size_t off = (size_t)br * DC + 8 * c8;
  st_bf16x8(o_hi + off, h8);
  st_bf16x8(o_lo + off, l8);
}

template <typename E, int DC, bool F8 = false>
hipError_t launch_dc(const AttendArgs& a, hipStream_t s) {
  constexpr bool SPLIT = kSplitOf<E>;
  if ((a.qcat_lo != nullptr) != SPLIT) return hipErrorInvalidValue;
  const bool norm = a.qn_gamma != nullptr;
  if (a.Lq <= kQprepRowsMaxLq && a.d_nope <= qprep_rows_max_nope<DC>()) {
    const dim3 grid((unsigned)a.n_h, (unsigned)a.B);
    if (norm)
      hipLaunchKernelGGL((qprep_rows_kernel<E, DC, SPLIT, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((qprep_rows_kernel<E, DC, SPLIT>), grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const size_t lds = (size_t)a.d_nope * (DC + 8) * sizeof(bf16_t);
    dim3 grid((unsigned)((a.Lq + 127) / 128), (unsigned)a.n_h, (unsigned)a.B);
    if (norm)
      hipLaunchKernelGGL((qprep_bf16_kernel<E, DC, SPLIT, true>), grid, dim3(256), lds, s, a);
    else
      hipLaunchKernelGGL((qprep_bf16_kernel<E, DC, SPLIT>), grid, dim3(256), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    hipError_t e = launch_core_of<E, DC, F8>(a, s);
    if (e != hipSuccess) return e;
  }
  // Rows with many key-range partials each (narrow blocks on 32-key tiles,
  // or few row groups spread over the whole device) merge one row per block;
  // otherwise one lane per row, whose merge walks the partials one after
  // another.
  if ((a.sched.key_tile < 64 || a.sched.n_slots > kLaneMergeMaxSlots) &&
      a.d_v <= kEpiMaxDv) {
    const dim3 grid((unsigned)(a.Lq * a.n_h), (unsigned)a.B);
    const bool lean = grid.x * grid.y >= (unsigned)kEpiLeanRows;
    if (a.part16) {
      if (lean)
        hipLaunchKernelGGL((epilogue_rows_kernel<DC, true, true>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((epilogue_rows_kernel<DC, false, true>), grid, dim3(256), 0, s, a);
    } else {
      if (lean)
        hipLaunchKernelGGL((epilogue_rows_kernel<DC, true, false>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((epilogue_rows_kernel<DC, false, false>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.part16) return hipErrorInvalidValue;  // fp16 partials only reach the per-row epilogue
  {
    dim3 grid((unsigned)((a.Lq + 31) / 32), (unsigned)a.n_h, (unsigned)a.B);
    hipLaunchKernelGGL(epilogue_bf16_kernel<DC>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
  }
}

}  // namespace

bool attend_bf16_supported(int d_c, int d_rope, int d_nope, int d_v) {
  return (d_c == 64 || d_c == 128 || d_c == 192) && d_rope == 32 && d_nope > 0 &&
         d_nope % 16 == 0 && d_v > 0 && d_v % 32 == 0;
}

template <typename E, bool F8 = false>
hipError_t launch_typed(const AttendArgs& a, hipStream_t s) {
  switch (a.d_c) {
    case 64: return launch_dc<E, 64, F8>(a, s);
    case 128: return launch_dc<E, 128, F8>(a, s);
    case 192: return launch_dc<E, 192, F8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attend_core_only(const AttendArgs& a, hipStream_t s) {
  if (a.cache_type == 3) {
    if (a.qcat_lo != nullptr) return hipErrorInvalidValue;
    switch (a.d_c) {
      case 64: return launch_core_of<f16_t, 64, true>(a, s);
      case 128: return launch_core_of<f16_t, 128, true>(a, s);
      case 192: return launch_core_of<f16_t, 192, true>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  const bool f16 = a.cache_type == 2;
  if ((a.qcat_lo != nullptr) == f16) return hipErrorInvalidValue;
  switch (a.d_c) {
    case 64: return f16 ? launch_core_of<f16_t, 64>(a, s) : launch_core_of<bf16_t, 64>(a, s);
    case 128: return f16 ? launch_core_of<f16_t, 128>(a, s) : launch_core_of<bf16_t, 128>(a, s);
    case 192: return f16 ? launch_core_of<f16_t, 192>(a, s) : launch_core_of<bf16_t, 192>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge_latent(const AttendArgs& a, void* o_hi, void* o_lo, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.Lq * a.n_h * (a.d_c / 8);
  const dim3 grid((unsigned)((n + 255) / 256));
#define MLA_MERGE(DC)                                                                                  \
  if (a.part16)                                                                                        \
    hipLaunchKernelGGL((merge_latent_kernel<DC, true>), grid, dim3(256), 0, s, a, (bf16_t*)o_hi,       \
                       (bf16_t*)o_lo);                                                                 \
  else                                                                                                 \
    hipLaunchKernelGGL((merge_latent_kernel<DC, false>), grid, dim3(256), 0, s, a, (bf16_t*)o_hi,      \
                       (bf16_t*)o_lo);
  switch (a.d_c) {
    case 64: MLA_MERGE(64) break;
    case 128: MLA_MERGE(128) break;
    case 192: MLA_MERGE(192) break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_MERGE
  return hipGetLastError();
}

hipError_t launch_attend_bf16(const AttendArgs& a, hipStream_t s) {
  if (a.cache_type == 3) return launch_typed<f16_t, true>(a, s);
  return a.cache_type == 2 ? launch_typed<f16_t>(a, s) : launch_typed<bf16_t>(a, s);
}

hipError_t launch_attend_f32(const AttendArgs& a, hipStream_t s) {
  const size_t lds = (size_t)(a.d_c + a.d_rope + 512 + a.d_c) * sizeof(float);
  dim3 grid((unsigned)(a.Lq * a.n_h), (unsigned)a.B);
  hipLaunchKernelGGL(attend_f32_kernel, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace mla
