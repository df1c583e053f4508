// Weight-level folds of the attention block around the absorbed path (the
// layer's query projection and output projection on either side of VideoMLA's
// per-head rebuild, technical summary, method items 2 and 3): W^K_up folded
// into the query projection, so that each head's [q_lat | q^R] comes from the
// layer input in one product, and W^V_up folded into W^O, so that the output
// in model width comes from the latent outputs in one product.
//
// The folds run once per weight set (not per step): plain fp32 dot products,
// one thread per output element, each result written as two bf16 parts (the
// value rounded to bf16 and the bf16 rounding of the remainder), so that the
// folded products keep 16 significant bits.  A plain bf16 fold would round the
// folded query weights like the prepared queries themselves, which moves the
// attention output by about 1e-3 of its size (see the split operands of the
// attention core).
#include "mla_device.h"

namespace mla {

namespace {

__device__ __forceinline__ void store_parts(bf16_t* hi, bf16_t* lo, float v) {
  const bf16_t h = to_bf16(v);
  *hi = h;
  *lo = to_bf16(v - (float)h);
}

// w_qf[part][h][i][k], i < d_c + d_rope, k < hidden.
__global__ __launch_bounds__(256) void fold_query_kernel(FoldArgs f) {
  const int width = f.d_c + f.d_rope, d_qk = f.d_nope + f.d_rope;
  const int64_t n = (int64_t)f.n_h * width * f.hidden;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int k = (int)(idx % f.hidden);
  const int64_t hi_ = idx / f.hidden;
  const int i = (int)(hi_ % width), h = (int)(hi_ / width);
  const bf16_t* wq = (const bf16_t*)f.w_q + (size_t)h * d_qk * f.hidden + k;
  float v;
  if (i < f.d_c) {
    const bf16_t* wuk = (const bf16_t*)f.w_uk + (size_t)h * f.d_nope * f.d_c + i;
    v = 0.0f;
    for (int nn = 0; nn < f.d_nope; ++nn)
      v = fmaf((float)wuk[(size_t)nn * f.d_c], (float)wq[(size_t)nn * f.hidden], v);
  } else {
    v = (float)wq[(size_t)(f.d_nope + i - f.d_c) * f.hidden];
  }
  bf16_t* out = (bf16_t*)f.out;
  store_parts(out + idx, out + n + idx, v);
}

// w_fo[part][c][h * d_c + i], c < hidden.
__global__ __launch_bounds__(256) void fold_output_kernel(FoldArgs f) {
  const int K = f.n_h * f.d_c;
  const int64_t n = (int64_t)f.hidden * K;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int j = (int)(idx % K);
  const int c = (int)(idx / K);
  const int h = j / f.d_c, i = j - h * f.d_c;
  const bf16_t* wo = (const bf16_t*)f.w_o + (size_t)c * f.n_h * f.d_v + (size_t)h * f.d_v;
  const bf16_t* wuv = (const bf16_t*)f.w_uv + (size_t)h * f.d_v * f.d_c + i;
  float v = 0.0f;
  for (int vv = 0; vv < f.d_v; ++vv) v = fmaf((float)wo[vv], (float)wuv[(size_t)vv * f.d_c], v);
  bf16_t* out = (bf16_t*)f.out;
  store_parts(out + idx, out + n + idx, v);
}

}  // namespace

hipError_t launch_fold_query(const FoldArgs& f, hipStream_t s) {
  const int64_t n = (int64_t)f.n_h * (f.d_c + f.d_rope) * f.hidden;
  hipLaunchKernelGGL(fold_query_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, f);
  return hipGetLastError();
}

hipError_t launch_fold_output(const FoldArgs& f, hipStream_t s) {
  const int64_t n = (int64_t)f.hidden * f.n_h * f.d_c;
  hipLaunchKernelGGL(fold_output_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, f);
  return hipGetLastError();
}

}  // namespace mla
