// Dense per-head attention over a dense K/V window: the comparison path (in
// the VideoMLA problem definition every cached token stores full keys and
// values for every head), and the second half of expand-then-attend, over
// the window rebuilt from the latent.  Queries are rotated over the whole head
// width (optionally RMS-normalised first) and pre-scaled, then the shared
// flash-style core runs per head with K and V as separate slices of the
// cached row, and a merge kernel normalises into fp32.
#include "mla_attn_core.h"

namespace mla {

namespace {

// q [B][Lq][n_h][d_h] -> qrot [B][n_h * Lq_pad][d_h] in the cache type
// (head-major rows), rotated and scaled; with SPLIT (bf16 cache) also the
// remainders' rounding into qrot_lo, for the split-operand core.  A block
// takes kQprepTokens tokens of one sequence: the rotation's cos/sin per
// (token, pair) are evaluated once
// into LDS and shared by every head; then each thread moves 8-element chunks
// (16-byte loads and stores).  Pairs whose frequency is 0 keep angle 0.
constexpr int kQprepTokens = 4;
constexpr int kQprepRun = 4;

// NORM (a query norm is set; d_h = 128): the 16 lanes that hold a row's 16
// chunks (a row starts at a multiple of 16 chunks, and every thread's chunks
// sit 256 apart) sum its squares by shuffles; each value is gained before
// the rotation and scaled by the row's 1 / rms with the score scale, in fp32.
template <typename E, bool SPLIT, bool NORM = false>
__global__ __launch_bounds__(256) void mha_qprep_bf16_kernel(MhaAttendArgs a, int lq_pad) {
  typedef typename Elem<E>::v8 V8;
  __shared__ float cs[kQprepTokens][kMaxRopePairs][2];
  const int P = a.d_h / 2;
  const int b = blockIdx.y;
  const int tok0 = blockIdx.x * kQprepTokens;
  for (int i = threadIdx.x; i < kQprepTokens * P; i += blockDim.x) {
    const int tt = i / P, p = i - tt * P;
    float c = 1.0f, s = 0.0f;
    if (tok0 + tt < a.Lq && a.rope.inv_freq[p] != 0.0)
      rope_cos_sin(pos_axis(token_pos(a.q_token0 + tok0 + tt, a.T, a.grid_w), a.rope.axis[p]) *
                       a.rope.inv_freq[p],
                   c, s);
    cs[tt][p][0] = c;
    cs[tt][p][1] = s;
  }
  __syncthreads();
  const int C = a.d_h / 8;
  const int per_tok = a.n_h * C;
  const int total = kQprepTokens * per_tok;
  // kQprepRun chunks per thread at a time, all loaded before any is stored
  // (a chunk past the block's tokens re-reads a valid one and is not stored)
  for (int i0 = threadIdx.x; i0 < total; i0 += kQprepRun * blockDim.x) {
    bf16x8 v[kQprepRun];
#pragma unroll
    for (int u = 0; u < kQprepRun; ++u) {
      const int i = i0 + u * blockDim.x;
      const int tt = i < total ? i / per_tok : 0, rem = i < total ? i - tt * per_tok : 0;
      const int h = rem / C, ch = rem - h * C;
      const int tok = tok0 + tt < a.Lq ? tok0 + tt : a.Lq - 1;
      v[u] = ld_bf16x8((const bf16_t*)a.q + (((size_t)b * a.Lq + tok) * a.n_h + h) * a.d_h + 8 * ch);
    }
    float rs[kQprepRun];  // NORM: each chunk's row 1 / rms (every lane takes part)
    if constexpr (NORM) {
#pragma unroll
      for (int u = 0; u < kQprepRun; ++u) {
        float ss = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) ss = fmaf((float)v[u][t], (float)v[u][t], ss);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o);
        rs[u] = 1.0f / sqrtf(ss / (float)a.d_h + a.qn_eps);
      }
    }
#pragma unroll
    for (int u = 0; u < kQprepRun; ++u) {
      const int i = i0 + u * blockDim.x;
      const int tt = i / per_tok, rem = i - tt * per_tok;
      const int h = rem / C, ch = rem - h * C;
      const int tok = tok0 + tt;
      if (i >= total || tok >= a.Lq) continue;
      float sc = a.qscale;
      bf16x8 g8;
      if constexpr (NORM) {
        g8 = ld_bf16x8((const bf16_t*)a.qn_gamma + 8 * ch);
        sc *= rs[u];
      }
      V8 o, ol;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float c = cs[tt][4 * ch + j][0], s = cs[tt][4 * ch + j][1];
        float x0 = (float)v[u][2 * j], x1 = (float)v[u][2 * j + 1];
        if constexpr (NORM) {
          x0 *= (float)g8[2 * j];
          x1 *= (float)g8[2 * j + 1];
        }
        const float y0 = (x0 * c - x1 * s) * sc, y1 = (x0 * s + x1 * c) * sc;
        o[2 * j] = Elem<E>::from(y0);
        o[2 * j + 1] = Elem<E>::from(y1);
        ol[2 * j] = Elem<E>::from(y0 - (float)o[2 * j]);
        ol[2 * j + 1] = Elem<E>::from(y1 - (float)o[2 * j + 1]);
      }
      const size_t off = ((size_t)b * a.n_h * lq_pad + (size_t)h * lq_pad + tok) * a.d_h + 8 * ch;
      *reinterpret_cast<V8*>((E*)a.qrot + off) = o;
      if constexpr (SPLIT) *reinterpret_cast<V8*>((E*)a.qrot_lo + off) = ol;
    }
  }
}

// Merge a row group's partials and normalise: one thread per (row, 4 dims).
__global__ __launch_bounds__(256) void mha_merge_kernel(MhaAttendArgs a, AttnCore c) {
  const int C4 = a.d_h / 4;
  const int64_t n = (int64_t)a.B * a.n_h * a.Lq * C4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int c4 = (int)(idx % C4);
  int64_t r = idx / C4;
  const int tok = (int)(r % a.Lq);
  r /= a.Lq;
  const int h = (int)(r % a.n_h);
  const int b = (int)(r / a.n_h);
  const int row = h * c.rows_per_head + tok;
  const Schedule& sc = c.sched;
  const int n_part = sched_group_slots(sc, b * sc.n_rg + row / sc.block_rows);
  f32x4 o;
  constexpr int kFew = 4;
  if (n_part <= kFew) {
    // Every slot's loads go out together (slots past n_part re-read slot 0
    // and get weight 0), then the log-sum-exp combination.
    f32x4 x[kFew];
    float2 ml[kFew];
#pragma unroll
    for (int k = 0; k < kFew; ++k) {
      const size_t prow = ((size_t)(k < n_part ? k : 0) * c.B + b) * c.R + row;
      x[k] = *reinterpret_cast<const f32x4*>(c.opart + prow * a.d_h + 4 * c4);
      ml[k] = *reinterpret_cast<const float2*>(c.ml + prow * 2);
    }
    float M = ml[0].x;
#pragma unroll
    for (int k = 1; k < kFew; ++k)
      if (k < n_part) M = fmaxf(M, ml[k].x);
    float L = 0.0f;
    o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kFew; ++k) {
      const float wgt = k < n_part ? exp2_fast(ml[k].x - M) : 0.0f;
      L += wgt * ml[k].y;
      o += wgt * x[k];
    }
    o *= 1.0f / L;
  } else {
    float acc[4];
    merge_row_partials(c, a.d_h, b, row, 4 * c4, 4, acc);
    o = {acc[0], acc[1], acc[2], acc[3]};
  }
  *reinterpret_cast<f32x4*>(a.out + (((size_t)b * a.Lq + tok) * a.n_h + h) * a.d_h + 4 * c4) = o;
}

// fp32 dense path (small shapes): one block per (token, head), exact two-pass softmax.
__global__ __launch_bounds__(256) void mha_attend_f32_kernel(MhaAttendArgs a) {
  extern __shared__ float sm[];
  float* qr = sm;            // [d_h]
  float* part = qr + a.d_h;  // [256]
  float* pk = part + 256;    // [256]
  float* acc = pk + 256;     // [d_h]
  const int tid = threadIdx.x;
  const int row = blockIdx.x, b = blockIdx.y;
  const int tok = row / a.n_h, h = row % a.n_h;
  const int stride = 2 * a.n_h * a.d_h;
  const float* q = (const float*)a.q + (((size_t)b * a.Lq + tok) * a.n_h + h) * a.d_h;
  const float* ring = (const float*)a.ring + (size_t)b * a.ring_rows * stride;
  for (int p = tid; p < a.d_h / 2; p += 256) {
    float x0 = q[2 * p], x1 = q[2 * p + 1];
    rope_pair(a.rope, p, token_pos(a.q_token0 + tok, a.T, a.grid_w), x0, x1);
    qr[2 * p] = x0 * a.qscale;
    qr[2 * p + 1] = x1 * a.qscale;
  }
  for (int d = tid; d < a.d_h; d += 256) acc[d] = 0.0f;
  __syncthreads();
  auto krow = [&](int j) {
    int64_t slot = a.key_slot0 + j;
    if (slot >= a.ring_rows) slot -= a.ring_rows;
    return ring + slot * stride + (size_t)h * a.d_h;
  };
  auto score = [&](int j) {
    const float* k = krow(j);
    float s = 0.0f;
    for (int d = 0; d < a.d_h; ++d) s = fmaf(qr[d], k[d], s);
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
    for (int d = tid; d < a.d_h; d += 256) {
      float s = acc[d];
      for (int jj = 0; jj < n; ++jj) s = fmaf(pk[jj], krow(j0 + jj)[a.n_h * a.d_h + d], s);
      acc[d] = s;
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
  float* out = a.out + (((size_t)b * a.Lq + tok) * a.n_h + h) * a.d_h;
  for (int d = tid; d < a.d_h; d += 256) out[d] = acc[d] * inv;
}

}  // namespace

bool mha_attend_bf16_supported(int d_h) { return d_h == 128; }

namespace {
template <typename E>
hipError_t launch_mha_typed(const MhaAttendArgs& a, float* opart, float* ml, const Schedule& sched,
                            hipStream_t s) {
  const int br = sched.block_rows;
  const int lq_pad = (a.Lq + br - 1) / br * br;
  // a bf16 cache runs the core on split operands (see mla_attn_core.h)
  constexpr bool SPLIT = __is_same(E, bf16_t);
  if ((a.qrot_lo != nullptr) != SPLIT) return hipErrorInvalidValue;
  {
    const dim3 grid((unsigned)((a.Lq + kQprepTokens - 1) / kQprepTokens), (unsigned)a.B);
    if (a.qn_gamma != nullptr) {
      // the norm's 16-lane row reduction needs 16 chunks per row
      if (a.d_h != 128) return hipErrorInvalidValue;
      hipLaunchKernelGGL((mha_qprep_bf16_kernel<E, SPLIT, true>), grid, dim3(256), 0, s, a, lq_pad);
    } else {
      hipLaunchKernelGGL((mha_qprep_bf16_kernel<E, SPLIT>), grid, dim3(256), 0, s, a, lq_pad);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  AttnCore c;
  c.qrows = a.qrot;
  c.qrows_lo = a.qrot_lo;
  c.ring = a.ring;
  c.part16 = 0;
  c.opart = opart;
  c.ml = ml;
  c.ring_rows = a.ring_rows;
  c.ring_stride = 2 * a.n_h * a.d_h;
  c.k_off = 0;
  c.v_off = a.n_h * a.d_h;
  c.head_stride = a.d_h;
  c.R = a.n_h * lq_pad;
  c.rows_per_head = lq_pad;
  c.valid_per_head = a.Lq;
  c.B = a.B;
  c.Lk = a.Lk;
  c.sched = sched;
  c.key_slot0 = a.key_slot0;
  {
    if (a.ev_start != nullptr) {
      hipError_t e = hipEventRecord(a.ev_start, s);
      if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)sched.n_blocks);
    bool launched = false;
#define MLA_SHAPE(NW, KT, NS, ROWS)                                                                   \
  if (!launched && br == ROWS * NW && sched.key_tile == KT && sched.stages == NS) {                  \
    hipLaunchKernelGGL((attn_core_kernel<E, 128, 128, NW, KT, NS, false, 1, (NW == 8), ROWS, SPLIT>), \
                       grid, dim3(NW * 64), 0, s, c);                                                \
    launched = true;                                                                                 \
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
    if (!launched) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev_stop != nullptr) {
      e = hipEventRecord(a.ev_stop, s);
      if (e != hipSuccess) return e;
    }
  }
  {
    const int64_t n = (int64_t)a.B * a.n_h * a.Lq * (a.d_h / 4);
    hipLaunchKernelGGL(mha_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, c);
    return hipGetLastError();
  }
}
}  // namespace

// The host carves the workspace into rotated queries (a.qrot), partial value
// sums (opart) and per-row max/sum (ml).
hipError_t launch_mha_attend_bf16_ws(const MhaAttendArgs& a, float* opart, float* ml,
                                     const Schedule& sched, hipStream_t s) {
  return a.cache_type == 2 ? launch_mha_typed<f16_t>(a, opart, ml, sched, s)
                           : launch_mha_typed<bf16_t>(a, opart, ml, sched, s);
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_mha_attend_f32(const MhaAttendArgs& a, hipStream_t s) {
  const size_t lds = (size_t)(2 * a.d_h + 512) * sizeof(float);
  hipLaunchKernelGGL(mha_attend_f32_kernel, dim3((unsigned)(a.Lq * a.n_h), (unsigned)a.B),
                     dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace mla
