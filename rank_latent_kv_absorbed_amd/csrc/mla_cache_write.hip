// Fused cache write for gfx950 (VideoMLA technical summary, method items 1
// and 3): one GEMM y = W x over every token of the written frames, 3D-RoPE on
// the positional columns, round to the storage dtype, scatter each token's row
// to its ring slot.  The same kernel serves the dense comparison cache (K and
// V of every head; K rotated per head).
//
// 2-byte path (bf16 inputs; bf16 or fp16 ring): a block computes one tile of
// 32 tokens x 32 output columns, its four waves each taking a quarter of the
// hidden dimension (so a tile's long dependent MFMA chain is four short ones
// running on four SIMDs, and four times as many waves hide the load latency);
// the quarters are summed through LDS and each wave finishes 8 of the tile's
// 32 columns.  The product is laid out transposed (columns on the MFMA M
// side, tokens on the N side) so that a lane holds one token and both
// elements of every rotary pair.
#include "mla_device.h"

#define MLA_INLINE __attribute__((always_inline))

namespace mla {

namespace {

constexpr int kSplitK = 4;     // waves per block = hidden-dimension quarters

template <typename E>
__global__ __launch_bounds__(kSplitK * 64) void cache_write_bf16_kernel(CacheWriteArgs a) {
  __shared__ float red[kSplitK][16][64];
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int ct = blockIdx.y;               // column tile
  const int64_t tok = (int64_t)blockIdx.x * 32 + lo;
  const bool valid = tok < a.M;
  const int col = ct * 32 + lo;            // W row this lane feeds
  // k-order: step 4g + s gives lane half hi the 8 elements
  // [64 g + 32 hi + 8 s, +8): over four steps a lane reads 64 contiguous
  // bytes of its row, and the wave covers whole 128-byte lines.
  const bf16_t* xrow = (const bf16_t*)a.x + (valid ? tok : 0) * a.hidden + 32 * hi;
  const bf16_t* wrow = (col < a.w_split ? (const bf16_t*)a.w + (int64_t)col * a.hidden
                                        : (const bf16_t*)a.w2 + (int64_t)(col - a.w_split) * a.hidden) +
                       32 * hi;
  const int ng = a.hidden / 64;            // groups of four 16-deep steps
  const int g0 = w * ng / kSplitK, g1 = (w + 1) * ng / kSplitK;  // this wave's groups

  // A ring of kDepth groups in flight: the loads of group g + kDepth - 1 go
  // out before the products of group g.
  constexpr int kDepth = 3;
  bf16x8 xf[kDepth][4], wf[kDepth][4];
  auto load_group = [&](int gi, int slot) MLA_INLINE {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      xf[slot][s4] = valid ? ld_bf16x8(xrow + gi * 64 + 8 * s4) : zero_bf16x8();
      wf[slot][s4] = ld_bf16x8(wrow + gi * 64 + 8 * s4);
    }
  };
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (g0 + d < g1) load_group(g0 + d, d);
  for (int gi = g0; gi < g1; gi += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (gi + d < g1) {
        if (gi + d + kDepth - 1 < g1) load_group(gi + d + kDepth - 1, (d + kDepth - 1) % kDepth);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) acc = mfma32(wf[d][s4], xf[d][s4], acc);
      }
    }
  }
  // Sum the quarters: every wave stores its partial tile; wave w then owns
  // accumulator group g = w (columns 8 g + 4 hi .. + 4 of every token).
#pragma unroll
  for (int r = 0; r < 16; ++r) red[w][r][l] = acc[r];
  __syncthreads();
  if (!valid) return;
  const int g = w;
  float v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < kSplitK; ++q) sum += red[q][4 * g + k][l];
    v[k] = sum;
  }

  const int64_t b = tok / a.tokens_per_batch;
  const int i = (int)(tok - b * a.tokens_per_batch);
  const int64_t frame = a.frame0 + i / a.T;
  const int tau = i % a.T;
  TokPos pos;
  pos.f = frame;
  pos.y = tau / a.grid_w;
  pos.x = tau - pos.y * a.grid_w;
  const int64_t slot = (frame % a.W) * a.T + tau;
  E* dst = (E*)a.ring + (b * a.ring_rows + slot) * a.width;
  const int c0 = ct * 32 + 8 * g + 4 * hi;
  if (c0 >= a.rot_begin && c0 < a.rot_end) {
    const int p0 = ((c0 - a.rot_begin) % a.rot_group) >> 1;
    rope_pair(a.rope, p0, pos, v[0], v[1]);
    rope_pair(a.rope, p0 + 1, pos, v[2], v[3]);
  }
  typename Elem<E>::v4 o;
  o[0] = Elem<E>::from(v[0]);
  o[1] = Elem<E>::from(v[1]);
  o[2] = Elem<E>::from(v[2]);
  o[3] = Elem<E>::from(v[3]);
  *reinterpret_cast<typename Elem<E>::v4*>(dst + c0) = o;
}

// fp32 path (small shapes): one thread per (token, column pair), plain fp32
// dot products, the same rotation and slot map.
__global__ __launch_bounds__(256) void cache_write_f32_kernel(CacheWriteArgs a) {
  const int64_t pairs = a.width / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.M * pairs) return;
  const int64_t tok = idx / pairs;
  const int c0 = (int)(idx - tok * pairs) * 2;
  const float* x = (const float*)a.x + tok * a.hidden;
  auto wrow = [&](int row) {
    return row < a.w_split ? (const float*)a.w + (int64_t)row * a.hidden
                           : (const float*)a.w2 + (int64_t)(row - a.w_split) * a.hidden;
  };
  const float* w0 = wrow(c0);
  const float* w1 = wrow(c0 + 1);
  float y0 = 0.0f, y1 = 0.0f;
  for (int k = 0; k < a.hidden; ++k) {
    y0 = fmaf(w0[k], x[k], y0);
    y1 = fmaf(w1[k], x[k], y1);
  }
  const int64_t b = tok / a.tokens_per_batch;
  const int i = (int)(tok - b * a.tokens_per_batch);
  const int64_t frame = a.frame0 + i / a.T;
  const int tau = i % a.T;
  if (c0 >= a.rot_begin && c0 < a.rot_end) {
    TokPos pos;
    pos.f = frame;
    pos.y = tau / a.grid_w;
    pos.x = tau - pos.y * a.grid_w;
    rope_pair(a.rope, ((c0 - a.rot_begin) % a.rot_group) >> 1, pos, y0, y1);
  }
  const int64_t slot = (frame % a.W) * a.T + tau;
  float* dst = (float*)a.ring + (b * a.ring_rows + slot) * a.width + c0;
  dst[0] = y0;
  dst[1] = y1;
}

template <typename E>
hipError_t launch_typed(const CacheWriteArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.M + 31) / 32), (unsigned)(a.width / 32));
  hipLaunchKernelGGL(cache_write_bf16_kernel<E>, grid, dim3(kSplitK * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool cache_write_bf16_supported(int width, int hidden) {
  return width > 0 && width % 32 == 0 && hidden > 0 && hidden % 64 == 0;
}

hipError_t launch_cache_write_bf16(const CacheWriteArgs& a, hipStream_t s) {
  return a.out_type == 2 ? launch_typed<f16_t>(a, s) : launch_typed<bf16_t>(a, s);
}

hipError_t launch_cache_write_f32(const CacheWriteArgs& a, hipStream_t s) {
  const int64_t n = a.M * (a.width / 2);
  hipLaunchKernelGGL(cache_write_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
