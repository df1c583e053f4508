// Fused cache write for gfx950 (VideoMLA technical summary, method items 1
// and 3): one GEMM y = W x over every token of the written frames, 3D-RoPE on
// the positional columns, round to the storage dtype, scatter each token's row
// to its ring slot.  The same kernel serves the dense comparison cache (K and
// V of every head; K rotated per head), and, with other epilogues, the steps
// on either side of the path (ProjMode in mla_launch.h): the cache write with
// the latent RMS-normalised, the query projection with W^K_up folded into its
// weights (each head's [q_lat | q^R] directly from the layer input), and the
// output projection with W^V_up folded into W^O.
//
// 2-byte path (bf16 inputs; bf16 or fp16 ring): a workgroup owns 32 tokens
// and NT <= 8 32-column tiles of the output, one tile per wave (a d_c = 192
// latent row [c | k^R] is 7 tiles: one workgroup of 7 when there are enough
// tokens to fill the chip, else two of 4).  The hidden dimension is walked in
// 64-element chunks through a ring of three LDS stages, each holding the
// chunk's 32 token rows and NT * 32 weight rows at 128 bytes per row, filled
// with direct global->LDS loads that cover whole 128-byte lines (the x tile
// is read from memory once, every weight row once per workgroup).  Products
// are D[col][token] = W[col][:] . x[token][:] on 32x32x16 MFMA with the
// weights as the A operand; the weight rows of a tile are staged in a
// permuted order so that lane (token lo, hi) ends up holding 16 consecutive
// output columns of its token, every rotary pair whole, which it rotates,
// rounds and writes as two 16-byte pieces of the token's ring row.  Weights
// carried in parts (value and remainder) run the hidden dimension once per
// part, into the same accumulators.

#include "mla_attn_core.h"

namespace mla {

namespace {

constexpr int kChunk = 64;  // hidden elements per staged chunk (128-byte rows)

template <typename E, int NT, int MODE = PROJ_CACHE, int NP = 1>
__global__ __launch_bounds__(NT * 64) void cache_write_bf16_kernel(CacheWriteArgs a) {
  constexpr int RB = kChunk * 2;              // staged bytes per row
  constexpr int ROWS = 32 + 32 * NT;          // token rows, then weight rows
  constexpr int SB = ROWS * RB;               // bytes per stage
  constexpr int SPANS = SB / 1024;            // 1-KiB load spans per stage (8 rows each)
  constexpr int SPW = (SPANS + NT - 1) / NT;  // spans per wave; surplus slots repeat the last span
  constexpr bool RING = MODE == PROJ_CACHE || MODE == PROJ_CACHE_NORM;
  static_assert(SB % 1024 == 0, "whole spans per stage");
  static_assert(NP >= 1 && NP <= kProjMaxPasses, "projection passes");
  __shared__ __attribute__((aligned(1024))) char st0[SB], st1[SB], st2[SB];
  __shared__ float2 rcs[32][kMaxRopePairs];  // cos, sin per (token, rotary pair)
  __shared__ int64_t rowoff[32];             // output row of each token (elements)
  __shared__ float nss[MODE == PROJ_CACHE_NORM ? 32 : 1][2 * NT];  // partial sums of squares
  const int tid = threadIdx.x;
  const int w = NT == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lo = l & 31, hi = l >> 5;
  const int64_t tok0 = (int64_t)blockIdx.x * 32;
  const int col0 = blockIdx.y * 32 * NT;

  // Staged row r, 16-byte slot s holds chunk s ^ ((r >> 1) & 7) of the row's
  // 128 bytes: the 16 lanes of an operand read (rows 0..15 at one chunk)
  // then touch 64 distinct banks.  Rows 0..31 are tokens tok0.. (past the
  // last token: the last token again, never written out); row 32 + 32 t + m
  // is weight row col0 + 32 t + 16 ((m >> 2) & 1) + 4 (m >> 3) + (m & 3).
  // Lane l of span sp fills row 8 sp + l / 8, slot l % 8.
  const bf16_t* const xg = (const bf16_t*)a.x;
  const char* src[SPW];
  bool wrow[SPW];  // the span's rows are weight rows (not token rows)
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int sp = w + j * NT < SPANS ? w + j * NT : SPANS - 1;
    const int row = 8 * sp + (l >> 3);
    const int q = (l & 7) ^ ((row >> 1) & 7);
    const bf16_t* p;
    wrow[j] = row >= 32;
    if (row < 32) {
      const int64_t t = tok0 + row < a.M ? tok0 + row : a.M - 1;
      p = xg + t * a.hidden;
    } else {
      const int m = row - 32, mm = m & 31;
      int col = col0 + (m & ~31) + 16 * ((mm >> 2) & 1) + 4 * (mm >> 3) + (mm & 3);
      col = col < a.width ? col : a.width - 1;  // tiles past the row: loaded, never written
      p = col < a.w_split ? (const bf16_t*)a.w + (int64_t)col * a.hidden
                          : (const bf16_t*)a.w2 + (int64_t)(col - a.w_split) * a.hidden;
    }
    src[j] = (const char*)(p + q * 8);
  }
  // Workgroups walk the chunks from different starting points: the rows
  // are hidden * 2 bytes apart, so one chunk of every weight row sits in a
  // few L2 channels, which workgroups in lockstep would all hit at once.
  // With several passes, chunk c of the walk is chunk c % NC of pass c / NC.
  const int NC = a.hidden / kChunk;
  const int NCT = NP * NC;
  const int rot = (int)(blockIdx.x % (unsigned)NC);
  auto issue = [&](int c, char* stg) MLA_INLINE {
    lds_char* const ls = (lds_char*)stg;
    const int pass = NP == 1 ? 0 : c / NC;
    const int cc = NP == 1 ? c : c - pass * NC;
    const int cr = cc + rot < NC ? cc + rot : cc + rot - NC;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int sp = w + j * NT < SPANS ? w + j * NT : SPANS - 1;
      const char* base = src[j];
      if constexpr (NP > 1) base += wrow[j] ? a.w_part[pass] : a.x_part[pass];
      global_to_lds16(base + cr * RB, ls + sp * 1024);
    }
  };

  // Operand reads for k-step ks of a chunk: chunk 2 ks + hi of token row lo
  // (B) and of the wave's weight row lo (A).
  const int sw = (lo >> 1) & 7;
  int xo[4], wo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    xo[ks] = lo * RB + 16 * ((2 * ks + hi) ^ sw);
    wo[ks] = (32 + 32 * w + lo) * RB + 16 * ((2 * ks + hi) ^ sw);
  }
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  auto compute = [&](const char* stg) MLA_INLINE {
    bf16x8 av[4], bv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      av[ks] = *reinterpret_cast<const bf16x8*>(stg + wo[ks]);
      bv[ks] = *reinterpret_cast<const bf16x8*>(stg + xo[ks]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma32(av[ks], bv[ks], acc);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Chunk c is computed from its stage; then, once this wave's loads of
  // chunk c + 1 are in (loads retire in order; chunk c + 2 stays in flight),
  // a barrier publishes every wave's loads of it and frees the stage just
  // read, which is refilled with chunk c + 3 (past the end: the last chunk
  // again, into a stage nobody reads any more).  Every step is the same
  // straight-line code and each stage is refilled right after it was read,
  // so the compiler's own tracking of the loads into LDS adds no waits.
  auto step = [&](int c, char* cur) MLA_INLINE {
    compute(cur);
    wait_vmem(SPW);
    lds_barrier();
    issue(c + 3 < NCT ? c + 3 : NCT - 1, cur);
  };
  issue(0, st0);
  issue(NCT > 1 ? 1 : 0, st1);
  issue(NCT > 2 ? 2 : 0, st2);
  // While the first chunks load: each token's output row, and cos / sin of
  // every rotary pair of every token (rotated columns c use pair
  // ((c - rot_begin) % rot_group - rot_skip) / 2).  Cache writes place token
  // i of a sequence at its ring slot and position (frame0 + i / T, i % T);
  // projections write token rows and take positions from q_token0 + i.
  const int npairs = a.rot_end > a.rot_begin ? (a.rot_group - a.rot_skip) / 2 : 0;
  for (int e = tid; e < 32 * (npairs + 1); e += NT * 64) {
    const int r = e & 31, p = (e >> 5) - 1;
    const int64_t t = tok0 + r < a.M ? tok0 + r : a.M - 1;
    const int64_t b = t / a.tokens_per_batch;
    const int i = (int)(t - b * a.tokens_per_batch);
    int64_t frame;
    int tau;
    if constexpr (RING) {
      frame = a.frame0 + i / a.T;
      tau = i % a.T;
    } else {
      const int64_t g = a.q_token0 + i;
      frame = g / a.T;
      tau = (int)(g - frame * a.T);
    }
    if (p < 0) {
      rowoff[r] = RING ? (b * a.ring_rows + (frame % a.W) * a.T + tau) * a.width : t * a.width;
    } else {
      TokPos pos;
      pos.f = frame;
      pos.y = tau / a.grid_w;
      pos.x = tau - pos.y * a.grid_w;
      float cs, sn;
      rope_cos_sin(pos_axis(pos, a.rope.axis[p]) * a.rope.inv_freq[p], cs, sn);
      rcs[r][p] = make_float2(cs, sn);
    }
  }
  wait_vmem(2 * SPW);
  lds_barrier();
  int c = 0;
  for (; c + 3 <= NCT; c += 3) {
    step(c, st0);
    step(c + 1, st1);
    step(c + 2, st2);
  }
  if (c < NCT) step(c, st0);
  if (c + 1 < NCT) step(c + 1, st1);
  // No load into LDS may still be in flight when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));

  // Lane (lo, hi) holds columns cb .. cb + 15 of token tok0 + lo.
  const int cb = col0 + 32 * w + 16 * hi;
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = acc[r];
  if constexpr (MODE == PROJ_CACHE_NORM) {
    // RMS of the token's first norm_cols columns: this workgroup holds the
    // token's whole row (one wave per 32-column tile), partial sums of squares
    // meet in LDS.
    float ss = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ss += cb + r < a.norm_cols ? v[r] * v[r] : 0.0f;
    nss[lo][2 * w + hi] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int k = 0; k < 2 * NT; ++k) tot += nss[lo][k];
    const float inv = 1.0f / sqrtf(tot / (float)a.norm_cols + a.eps);
    const bf16_t* gam = (const bf16_t*)a.gamma;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (cb + r < a.norm_cols) v[r] = v[r] * inv * (float)gam[cb + r];
  }
  if (tok0 + lo >= a.M || col0 + 32 * w >= a.width) return;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int c = cb + 2 * p;
    if (c >= a.rot_begin && c < a.rot_end) {
      const int k = (c - a.rot_begin) % a.rot_group;
      if (k >= a.rot_skip) {
        const float2 t = rcs[lo][(k - a.rot_skip) >> 1];
        const float ra = v[2 * p] * t.x - v[2 * p + 1] * t.y;
        const float rb = v[2 * p] * t.y + v[2 * p + 1] * t.x;
        v[2 * p] = ra;
        v[2 * p + 1] = rb;
      }
    }
  }
  if constexpr (MODE == PROJ_OUT) {
    float* dst = (float*)a.ring + rowoff[lo] + cb;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 o = {v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]};
      *reinterpret_cast<f32x4*>(dst + 4 * u) = o;
    }
    return;
  }
  if constexpr (MODE == PROJ_QUERY) {
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] *= a.scale;
  }
  E* dst = (E*)a.ring + rowoff[lo] + cb;
  if constexpr (__is_same(E, e4m3_t)) {
    // 16 one-byte codes: one 16-byte store (rows are multiples of 32 bytes)
    u32x4 o = {e4m3_pack4(v[0], v[1], v[2], v[3]), e4m3_pack4(v[4], v[5], v[6], v[7]),
               e4m3_pack4(v[8], v[9], v[10], v[11]), e4m3_pack4(v[12], v[13], v[14], v[15])};
    *reinterpret_cast<u32x4*>(dst) = o;
    return;
  } else {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    typename Elem<E>::v8 o, ol;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = Elem<E>::from(v[8 * u + e]);
      ol[e] = Elem<E>::from(v[8 * u + e] - (float)o[e]);
    }
    *reinterpret_cast<typename Elem<E>::v8*>(dst + 8 * u) = o;
    if constexpr (MODE == PROJ_QUERY)
      if (a.out_lo != nullptr) *reinterpret_cast<typename Elem<E>::v8*>((E*)a.out_lo + rowoff[lo] + cb + 8 * u) = ol;
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

template <typename E, int NT, int MODE, int NP>
hipError_t launch_nt(const CacheWriteArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.M + 31) / 32), (unsigned)((a.width / 32 + NT - 1) / NT));
  hipLaunchKernelGGL((cache_write_bf16_kernel<E, NT, MODE, NP>), grid, dim3(NT * 64), 0, s, a);
  return hipGetLastError();
}

// Tiles per workgroup: a row's 32-column tiles split over the fewest
// workgroups per token tile (at most 8 tiles each) that still give every
// compute unit a workgroup; the last workgroup of a row may own fewer tiles
// than waves.
int tiles_per_group(const CacheWriteArgs& a) {
  const int tiles = a.width / 32;
  const int64_t token_tiles = (a.M + 31) / 32;
  int groups = (tiles + 7) / 8;
  const int cus = device_cu_count();
  while (groups < tiles && token_tiles * groups < cus) ++groups;
  return (tiles + groups - 1) / groups;
}

template <typename E>
hipError_t launch_typed(const CacheWriteArgs& a, hipStream_t s) {
  switch (tiles_per_group(a)) {
    case 8: return launch_nt<E, 8, PROJ_CACHE, 1>(a, s);
    case 7: return launch_nt<E, 7, PROJ_CACHE, 1>(a, s);
    case 6: return launch_nt<E, 6, PROJ_CACHE, 1>(a, s);
    case 5: return launch_nt<E, 5, PROJ_CACHE, 1>(a, s);
    case 4: return launch_nt<E, 4, PROJ_CACHE, 1>(a, s);
    case 3: return launch_nt<E, 3, PROJ_CACHE, 1>(a, s);
    case 2: return launch_nt<E, 2, PROJ_CACHE, 1>(a, s);
    default: return launch_nt<E, 1, PROJ_CACHE, 1>(a, s);
  }
}

// The normalised cache write keeps a token's whole row in one workgroup (the
// row's sum of squares meets in LDS): latent rows of 96, 160 or 224 columns.
template <typename E>
hipError_t launch_norm(const CacheWriteArgs& a, hipStream_t s) {
  switch (a.width / 32) {
    case 7: return launch_nt<E, 7, PROJ_CACHE_NORM, 1>(a, s);
    case 5: return launch_nt<E, 5, PROJ_CACHE_NORM, 1>(a, s);
    case 3: return launch_nt<E, 3, PROJ_CACHE_NORM, 1>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Projections on two- or three-part operands take 1, 2, 4 or 8 tiles per
// workgroup (the fewest that fill the device, rounded up to a power of two).
template <typename E, int MODE, int NP>
hipError_t launch_parts(const CacheWriteArgs& a, hipStream_t s) {
  int nt = tiles_per_group(a);
  nt = nt > 4 ? 8 : (nt > 2 ? 4 : nt);
  switch (nt) {
    case 8: return launch_nt<E, 8, MODE, NP>(a, s);
    case 4: return launch_nt<E, 4, MODE, NP>(a, s);
    case 2: return launch_nt<E, 2, MODE, NP>(a, s);
    default: return launch_nt<E, 1, MODE, NP>(a, s);
  }
}

}  // namespace

bool cache_write_bf16_supported(int width, int hidden) {
  return width > 0 && width % 32 == 0 && hidden > 0 && hidden % 64 == 0;
}

hipError_t launch_cache_write_bf16(const CacheWriteArgs& a, hipStream_t s) {
  if (a.out_type == 3) return launch_typed<e4m3_t>(a, s);
  return a.out_type == 2 ? launch_typed<f16_t>(a, s) : launch_typed<bf16_t>(a, s);
}

hipError_t launch_projection_bf16(const CacheWriteArgs& a, int mode, hipStream_t s) {
  const bool f16 = a.out_type == 2;
  if (mode == PROJ_CACHE_NORM && a.passes == 1) {
    if (a.out_type == 3) return launch_norm<e4m3_t>(a, s);
    return f16 ? launch_norm<f16_t>(a, s) : launch_norm<bf16_t>(a, s);
  }
  if (a.out_type == 3) return hipErrorInvalidValue;  // projections write 2-byte operands
  if (mode == PROJ_QUERY && a.passes == 2)
    return f16 ? launch_parts<f16_t, PROJ_QUERY, 2>(a, s) : launch_parts<bf16_t, PROJ_QUERY, 2>(a, s);
  if (mode == PROJ_OUT && a.passes == 3) return launch_parts<bf16_t, PROJ_OUT, 3>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_cache_write_f32(const CacheWriteArgs& a, hipStream_t s) {
  const int64_t n = a.M * (a.width / 2);
  hipLaunchKernelGGL(cache_write_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
