// Expand-then-attend for large query chunks (VideoMLA technical summary,
// method item 2: per-head keys and values are rebuilt on demand from the
// cached latent, k^nope_h = W^K_up,h c and v_h = W^V_up,h c).  For a chunk of
// many queries, rebuilding the window's per-head keys and values once and then
// running per-head attention (d = d_nope + d_rope for scores, d_v for values)
// needs fewer products than the absorbed form, whose every score and value
// product runs in the d_c-wide latent space.
//
// Two kernels, then the per-head attention path of the dense cache:
//  1. weights_to_cache_kernel: [W^K_up,h ; W^V_up,h] (bf16) -> one matrix per
//     head in the ring's element type, [n_h][d_nope + d_v][d_c] (fp16 is exact
//     for these weights' range; bf16 is a copy).
//  2. expand_kv_kernel: for every resident key j and head h,
//       K[j][h] = [ W^K_up,h c_j | k^R_j ],   V[j][h] = W^V_up,h c_j,
//     written as [B][Lk][2][n_h][d_h] in the ring's element type - the layout
//     of the dense cache, so the same attention core reads it.  One GEMM per
//     32-key block: D[key][col] = c[key][:] . W[col][:], on 32x32x16 MFMA with
//     the latent rows (A operand) in registers and each 32-row weight tile
//     (B operand) staged in LDS by direct global->LDS loads, shared by the
//     four waves (four 32-key blocks) of a workgroup.
#include "mla_attn_core.h"

namespace mla {

namespace {

template <typename E>
__global__ __launch_bounds__(256) void weights_to_cache_kernel(ExpandArgs a) {
  const int rows = a.d_nope + a.d_v;
  const int64_t n = (int64_t)a.n_h * rows * a.d_c;
  const int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (idx >= n) return;
  const int i = (int)(idx % a.d_c);
  const int64_t hr = idx / a.d_c;
  const int r = (int)(hr % rows);
  const int h = (int)(hr / rows);
  const bf16_t* src = r < a.d_nope
                          ? (const bf16_t*)a.w_uk + ((size_t)h * a.d_nope + r) * a.d_c + i
                          : (const bf16_t*)a.w_uv + ((size_t)h * a.d_v + (r - a.d_nope)) * a.d_c + i;
  const bf16x8 v = ld_bf16x8(src);
  typename Elem<E>::v8 o;
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = Elem<E>::from((float)v[t]);
  *reinterpret_cast<typename Elem<E>::v8*>((E*)a.wx + idx) = o;
}

// DC: latent width.  A workgroup of 4 waves owns 128 keys (32 per wave) of one
// sequence and walks every 32-row weight tile of every head.
template <typename E, int DC>
__global__ __launch_bounds__(256) void expand_kv_kernel(ExpandArgs a) {
  typedef typename Elem<E>::v8 V8;
  constexpr int NKS = DC / 16;         // MFMA depth steps
  constexpr int CPR = DC / 8;          // 16-byte chunks per weight row
  constexpr int TILE = 32 * DC;        // elements per weight tile (32 rows)
  constexpr int SPANS = TILE * 2 / 1024;
  static_assert(DC % 64 == 0 && (TILE * 2) % 1024 == 0, "whole 1-KiB spans per tile");
  static_assert(CPR % 8 == 0, "the chunk permutation stays inside groups of 8");
  __shared__ __attribute__((aligned(1024))) E wt0[TILE];
  __shared__ __attribute__((aligned(1024))) E wt1[TILE];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int b = blockIdx.y;
  const int key0 = blockIdx.x * 128 + w * 32;
  const int d_h = a.d_nope + a.d_rope;
  const int tph = (a.d_nope + a.d_v) / 32;   // weight tiles per head
  const int n_tiles = a.n_h * tph;

  // This lane's latent row (A operand: key lo, depth 16 ks + 8 hi .. + 8).
  const int key = key0 + lo;
  const bool kvalid = key < a.Lk;
  int64_t slot = a.key_slot0 + (kvalid ? key : 0);
  if (slot >= a.ring_rows) slot -= a.ring_rows;
  const E* crow = (const E*)a.ring + ((size_t)b * a.ring_rows + slot) * (DC + a.d_rope);
  V8 cf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) cf[ks] = ld8<E>(crow + 16 * ks + 8 * hi);

  // Weight tile t = rows [32 t, 32 t + 32) of the converted [n_h * (d_nope +
  // d_v)][DC] matrix.  In LDS, chunk q of tile row r sits at q ^ ((r >> 1) & 7)
  // (inside aligned groups of 8 chunks): the 16 lanes of a B-operand read,
  // rows 0..15 at one chunk, then touch 64 distinct banks.  Lane l of span sp
  // fills LDS chunk c = 64 sp + l: row c / CPR, position c % CPR.
  auto load_tile = [&](int t, E* dst) __attribute__((always_inline)) {
    const E* src = (const E*)a.wx + (size_t)t * TILE;
#pragma unroll
    for (int j = 0; j < SPANS / 4; ++j) {
      const int sp = w + 4 * j;
      const int c = sp * 64 + l;
      const int r = c / CPR, p = c - r * CPR;
      const int q = p ^ ((r >> 1) & 7);
      global_to_lds16(src + r * DC + q * 8, dst + sp * 512);
    }
  };
  static_assert(SPANS % 4 == 0, "spans divide over the four waves");

  // B-operand read: lane (col lo, hi) takes chunk 2 ks + hi of row lo.
  const int rsw = (lo >> 1) & 7;

  auto tile_product = [&](const E* wt, int t) __attribute__((always_inline)) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const E* wrow = wt + lo * DC;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      acc = Elem<E>::mfma(cf[ks], ld8<E>(wrow + 8 * ((2 * ks + hi) ^ rsw)), acc);
    // D[key][col]: lane holds col lo of keys 8 (r / 4) + 4 hi + r % 4.
    const int h = t / tph;
    const int c0 = (t - h * tph) * 32;   // row of the head's [K nope ; V] block
    const bool kpart = c0 < a.d_nope;
    const int col = (kpart ? c0 : c0 - a.d_nope) + lo;
    E* base = (E*)a.kv + (((size_t)b * a.Lk) * 2 + (kpart ? 0 : 1)) * a.n_h * d_h + (size_t)h * d_h + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (kk < a.Lk) base[(size_t)kk * 2 * a.n_h * d_h] = Elem<E>::from(acc[r]);
    }
  };

  load_tile(0, wt0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; t += 2) {
    if (t + 1 < n_tiles) load_tile(t + 1, wt1);
    tile_product(wt0, t);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < n_tiles) {
      if (t + 2 < n_tiles) load_tile(t + 2, wt0);
      tile_product(wt1, t + 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // k^R of each key into every head's positional columns.
  if (kvalid) {
    const E* kr = crow + DC;
    E* dst = (E*)a.kv + ((size_t)b * a.Lk + key) * 2 * a.n_h * d_h + a.d_nope;
    for (int h = 0; h < a.n_h; ++h)
      for (int i = 8 * hi; i < a.d_rope; i += 16)
        *reinterpret_cast<V8*>(dst + (size_t)h * d_h + i) = ld8<E>(kr + i);
  }
}

template <typename E, int DC>
hipError_t launch_expand_dc(const ExpandArgs& a, hipStream_t s) {
  {
    const int64_t n = (int64_t)a.n_h * (a.d_nope + a.d_v) * a.d_c / 8;
    hipLaunchKernelGGL(weights_to_cache_kernel<E>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)((a.Lk + 127) / 128), (unsigned)a.B);
  hipLaunchKernelGGL((expand_kv_kernel<E, DC>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_expand_typed(const ExpandArgs& a, hipStream_t s) {
  switch (a.d_c) {
    case 64: return launch_expand_dc<E, 64>(a, s);
    case 128: return launch_expand_dc<E, 128>(a, s);
    case 192: return launch_expand_dc<E, 192>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool expand_supported(int d_c, int d_rope, int d_nope, int d_v) {
  return (d_c == 64 || d_c == 128 || d_c == 192) && d_nope + d_rope == 128 && d_v == 128 &&
         d_nope % 32 == 0 && d_rope % 8 == 0;
}

hipError_t launch_expand_kv(const ExpandArgs& a, hipStream_t s) {
  return a.cache_type == 2 ? launch_expand_typed<f16_t>(a, s) : launch_expand_typed<bf16_t>(a, s);
}

}  // namespace mla
