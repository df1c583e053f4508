// Fused cache write for gfx950 (VideoMLA technical summary, method items 1
// and 3): one GEMM y = W x over every token of the written frames, 3D-RoPE on
// the positional columns, round to the storage dtype, scatter each token's row
// to its ring slot.  The same kernel serves the dense comparison cache (K and
// V of every head; K rotated per head).
//
// 2-byte path (bf16 inputs; bf16 or fp16 ring): a 256-thread block owns 32 tokens x (32*CT) output columns.  The
// four waves split the hidden dimension four ways and each runs the MFMA
// product on its quarter; waves 1-3 hand their partial sums to wave 0 through
// LDS, and wave 0 adds them, rotates, rounds and stores.  The product is laid
// out transposed (columns on the MFMA M side, tokens on the N side) so that a
// lane holds one token and both elements of every rotary pair.
#include "mla_device.h"

namespace mla {

namespace {

constexpr int kWaves = 4;

template <typename E, int CT>
__global__ __launch_bounds__(256) void cache_write_bf16_kernel(CacheWriteArgs a) {
  extern __shared__ float red[];  // [kWaves - 1][CT][16][64]
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int64_t tok = (int64_t)blockIdx.x * 32 + lo;
  const bool valid = tok < a.M;
  const int col0 = blockIdx.y * CT * 32;
  const int kq = a.hidden / kWaves;
  const int kbeg = w * kq;

  const bf16_t* xrow = (const bf16_t*)a.x + (valid ? tok : 0) * a.hidden + 8 * hi;
  const bf16_t* wrow[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    int row = col0 + ct * 32 + lo;
    wrow[ct] = (row < a.w_split ? (const bf16_t*)a.w + (int64_t)row * a.hidden
                                : (const bf16_t*)a.w2 + (int64_t)(row - a.w_split) * a.hidden) +
               8 * hi;
  }

  f32x16 acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ct][r] = 0.0f;

  for (int k0 = kbeg; k0 < kbeg + kq; k0 += 16) {
    bf16x8 bx = valid ? ld_bf16x8(xrow + k0) : zero_bf16x8();
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma32(ld_bf16x8(wrow[ct] + k0), bx, acc[ct]);
  }

  if (w > 0) {
    float* dst = red + (size_t)(w - 1) * CT * 16 * 64;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(ct * 16 + r) * 64 + l] = acc[ct][r];
  }
  __syncthreads();
  if (w > 0 || !valid) return;

#pragma unroll
  for (int ww = 0; ww < kWaves - 1; ++ww) {
    const float* src = red + (size_t)ww * CT * 16 * 64;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ct][r] += src[(ct * 16 + r) * 64 + l];
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

#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c0 = col0 + ct * 32 + 8 * g + 4 * hi;
      float v[4] = {acc[ct][4 * g], acc[ct][4 * g + 1], acc[ct][4 * g + 2], acc[ct][4 * g + 3]};
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
  }
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

template <typename E, int CT>
hipError_t launch_ct(const CacheWriteArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.M + 31) / 32), (unsigned)(a.width / (32 * CT)));
  const size_t lds = (size_t)(kWaves - 1) * CT * 16 * 64 * sizeof(float);
  // more than the default 64 KB of dynamic LDS for the wider column groups
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)cache_write_bf16_kernel<E, CT>, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((cache_write_bf16_kernel<E, CT>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace

bool cache_write_bf16_supported(int width, int hidden) {
  return width > 0 && width % 32 == 0 && hidden > 0 && hidden % (16 * kWaves) == 0;
}

template <typename E>
hipError_t launch_typed(const CacheWriteArgs& a, hipStream_t s) {
  const int tiles = a.width / 32;
  if (tiles % 7 == 0) return launch_ct<E, 7>(a, s);
  if (tiles % 6 == 0) return launch_ct<E, 6>(a, s);
  if (tiles % 5 == 0) return launch_ct<E, 5>(a, s);
  if (tiles % 4 == 0) return launch_ct<E, 4>(a, s);
  if (tiles % 3 == 0) return launch_ct<E, 3>(a, s);
  if (tiles % 2 == 0) return launch_ct<E, 2>(a, s);
  return launch_ct<E, 1>(a, s);
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
