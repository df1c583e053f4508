// Expand-then-attend for large query chunks (VideoMLA technical summary,
// method item 2: per-head keys and values are rebuilt on demand from the
// cached latent, k^nope_h = W^K_up,h c and v_h = W^V_up,h c).  For a chunk of
// many queries, rebuilding the window's per-head keys and values once and then
// running per-head attention (d = d_nope + d_rope for scores, d_v for values)
// needs fewer products than the absorbed form, whose every score and value
// product runs in the d_c-wide latent space.
//
// One kernel, then the per-head attention path of the dense cache:
//  expand_kv_kernel: for every resident key j and head h,
//       K[j][h] = [ W^K_up,h c_j | k^R_j ],   V[j][h] = W^V_up,h c_j,
//     written as [B][Lk][2][n_h][d_h] in fp16 - the layout of the dense
//     cache, so the same attention core reads it.  A workgroup owns one head
//     and a range of keys of one sequence: the head's whole [d_nope + d_v][d_c]
//     matrix is loaded into LDS once (converted from bf16 to fp16 on the way
//     for fp16 and one-byte E4M3 rings, the latter widening each latent row to
//     fp16 exactly as it is loaded; kept in bf16 for a bf16 ring, whose
//     products then run on bf16 MFMA - exact products of the stored values -
//     into the same fp16 window), then each wave independently walks 32-key
//     blocks:
//     latent rows into registers (MFMA A operand), D[key][col] =
//     c[key][:] . W[col][:] on 32x32x16 MFMA per 32-row weight tile (B
//     operand from LDS), the head's key and value blocks staged in the wave's
//     own LDS area and written out as whole 256-byte rows.
#include "mla_attn_core.h"

namespace mla {

namespace {

constexpr int kExpandWaves = 8;       // waves per workgroup (two per SIMD)
// Head shape of the rebuild: d_nope = 96 content and d_rope = 32 positional
// key columns, d_v = 128 value columns (the Wan shape); 7 weight tiles of 32
// rows per head, 3 of them for keys.
constexpr int kExpandNope = 96, kExpandRope = 32, kExpandDv = 128;
constexpr int kExpandKTiles = kExpandNope / 32, kExpandTiles = kExpandKTiles + kExpandDv / 32;

template <bool B, typename T, typename F>
struct Pick {
  typedef T type;
};
template <typename T, typename F>
struct Pick<false, T, F> {
  typedef F type;
};

// DC: latent width.  Workgroup (x, h, b): head h of sequence b, keys
// [x * keys_per_block, (x + 1) * keys_per_block).
// E: the rebuilt window's type (fp16).  F8: one-byte E4M3 ring.  BF: bf16
// ring (weights and latent rows stay bf16 as MFMA operands).
template <typename E, int DC, bool F8 = false, bool BF = false>
__global__ __launch_bounds__(kExpandWaves * 64) void expand_kv_kernel(ExpandArgs a, int keys_per_block) {
  static_assert(__is_same(E, f16_t), "the rebuilt keys and values are fp16");
  static_assert(!(F8 && BF), "one ring type");
  typedef typename Elem<E>::v8 V8;
  typedef typename Pick<BF, bf16_t, E>::type OP;  // operand type of the products
  typedef typename Elem<OP>::v8 OV8;
  constexpr int NKS = DC / 16;         // MFMA depth steps
  constexpr int CPR = DC / 8;          // 16-byte chunks per weight row
  constexpr int TILE = 32 * DC;        // elements per weight tile (32 rows)
  constexpr int DH = 128;              // per-head key width (d_nope + d_rope) and value width
  constexpr int WSPANS = kExpandTiles * TILE * 2 / 1024;
  static_assert(DC % 64 == 0 && (TILE * 2) % 1024 == 0, "whole 1-KiB spans per tile");
  static_assert(CPR % 8 == 0, "the chunk permutation stays inside groups of 8");
  static_assert(kExpandNope + kExpandRope == DH && kExpandDv == DH, "128-wide heads");
  __shared__ __attribute__((aligned(1024))) OP wts[kExpandTiles * TILE];
  __shared__ __attribute__((aligned(16))) E stg[kExpandWaves][32 * DH];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int kbeg = blockIdx.x * keys_per_block;
  const int kend = kbeg + keys_per_block < a.Lk ? kbeg + keys_per_block : a.Lk;
  E* st = stg[w];

  // The head's weight tiles: rows [32 t, 32 t + 32) of its [d_nope + d_v][d_c]
  // matrix, row m of a tile in LDS holding matrix row 32 t + 16 ((m >> 2) & 1)
  // + 4 (m >> 3) + (m & 3) (see the products below).  In LDS, chunk q of tile
  // row r sits at q ^ ((r >> 1) & 7) (inside aligned groups of 8 chunks): the
  // 16 lanes of an operand read, rows 0..15 at one chunk, then touch 64
  // distinct banks.  Lane l of span sp fills LDS chunk c = 64 sp + l: row
  // c / CPR, position c % CPR of the rows of all tiles.
  // The rows come straight from W^K_up,h and W^V_up,h (bf16), converted to
  // fp16 on the way unless the products run in bf16 (exact for magnitudes in
  // [6.1e-5, 65504]; smaller weights land in fp16's subnormal range with an
  // absolute quantum of 2^-24).
  {
    const bf16_t* src_k = (const bf16_t*)a.w_uk + (size_t)h * kExpandNope * DC;
    const bf16_t* src_v = (const bf16_t*)a.w_uv + (size_t)h * kExpandDv * DC;
    constexpr int SPW = (WSPANS + kExpandWaves - 1) / kExpandWaves;  // spans per wave
    auto chunk_src = [&](int sp) MLA_INLINE {
      const int c = sp * 64 + l;
      const int r = c / CPR, p = c - r * CPR;
      const int q = p ^ ((r >> 1) & 7);
      const int m = r & 31;
      const int wr = (r & ~31) + 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
      return (wr < kExpandNope ? src_k + wr * DC : src_v + (wr - kExpandNope) * DC) + q * 8;
    };
    {
      // every load of the wave first, then the conversions and LDS stores
      bf16x8 v[SPW];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int sp = w + j * kExpandWaves;
        v[j] = ld_bf16x8(chunk_src(sp < WSPANS ? sp : w));
      }
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int sp = w + j * kExpandWaves;
        if (sp < WSPANS) {
          OV8 o;
#pragma unroll
          for (int t = 0; t < 8; ++t) o[t] = Elem<OP>::from((float)v[j][t]);
          *reinterpret_cast<OV8*>(wts + (size_t)(sp * 64 + l) * 8) = o;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Products D[col][key] = W[col][:] . c[key][:] on 32x32x16 MFMA: weight
  // rows are the A operand (lane (lo, hi) reads chunk 2 ks + hi of LDS tile
  // row lo), latent rows the B operand.  Lane (lo, hi) receives D rows
  // 8 g + 4 hi + j (g, j < 4) of key lo; by the row order of the LDS tiles
  // those are output columns 16 hi + 4 g + j, so accumulator r holds column
  // 16 hi + r of the lane's key: 16 consecutive columns, staged as two 16-byte
  // LDS writes.
  const int rsw = (lo >> 1) & 7;
  // Staged block: key kk's 128 columns at st[kk * DH ..]; column chunk q
  // (8 columns) of key kk sits at chunk q ^ (kk & 15), so the 16-byte stores
  // of 16 consecutive keys and the key-row reads spread over the banks.
  auto stage_at = [&](int kk, int col) MLA_INLINE {
    return kk * DH + ((((col >> 3) ^ kk) & 15) << 3) + (col & 7);
  };
  auto mma = [&](int t, const OV8 (&c)[NKS]) MLA_INLINE {
    const OP* wrow = wts + t * TILE + lo * DC;
    OV8 wf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) wf[ks] = ld8<OP>(wrow + 8 * ((2 * ks + hi) ^ rsw));
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = Elem<OP>::mfma(wf[ks], c[ks], acc);
    return acc;
  };
  // Tile t's columns: key columns 32 t for t < 3, value columns 32 (t - 3).
  auto stage = [&](int t, const f32x16& acc) MLA_INLINE {
    const int c0 = t < kExpandKTiles ? 32 * t : 32 * (t - kExpandKTiles);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      V8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = Elem<E>::from(acc[8 * u + e]);
      *reinterpret_cast<V8*>(st + stage_at(lo, c0 + 16 * hi + 8 * u)) = o;
    }
  };
  // Output rows: key j of sequence b is a record of 2 parts x n_h heads x DH
  // elements.  Flush i of a staged block writes keys 4 i + l / 16, 16 bytes
  // at column chunk l % 16 per lane: a uniform base per (block, part, i) plus
  // one 32-bit lane offset (a sequence's expanded window stays below 2^31
  // elements, checked on the host).
  const size_t rec = (size_t)2 * a.n_h * DH;
  E* const kv_b = (E*)a.kv + (size_t)b * a.Lk * rec + (size_t)h * DH;
  const uint32_t fl_off = (uint32_t)(((l >> 4) * rec + (l & 15) * 8) * sizeof(E));
  auto flush = [&](int k0, int part) MLA_INLINE {
    const char* base = (const char*)(kv_b + (size_t)k0 * rec + (size_t)part * a.n_h * DH);
    const bool whole = k0 + 32 <= kend;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = 4 * i + (l >> 4), q = l & 15;
      const V8 v = *reinterpret_cast<const V8*>(st + kk * DH + ((q ^ kk) & 15) * 8);
      char* p = (char*)base + (size_t)i * 4 * rec * sizeof(E) + fl_off;
      if (whole || k0 + kk < kend) *reinterpret_cast<V8*>(p) = v;
    }
  };
  // This lane's latent row of the 32-key block at k0 (B operand: key lo,
  // depth 16 ks + 8 hi .. + 8, then k^R as 8-column pieces 8 hi + 16 j);
  // keys past the range load key k0's row (never written out).  Ring offsets
  // of one sequence fit 32 bits (checked when the cache is created).
  constexpr int NR = kExpandRope / 16;  // k^R pieces per lane
  constexpr int RW = DC + kExpandRope;  // elements per cached row
  constexpr int EB = F8 ? 1 : (int)sizeof(E);  // bytes per cached scalar
  const char* const ring_b = (const char*)a.ring + (size_t)b * a.ring_rows * RW * EB;
  const int rows = (int)a.ring_rows;
  auto load_row = [&](int k0, OV8 (&c)[NKS], V8 (&r)[NR]) MLA_INLINE {
    const int key = k0 + lo < kend ? k0 + lo : k0;
    int slot = (int)a.key_slot0 + key;
    slot = slot >= rows ? slot - rows : slot;
    if constexpr (F8) {
      // one-byte row: 8 codes per operand piece, widened to fp16
      const char* p8 = ring_b + ((uint32_t)slot * (uint32_t)RW + 8 * hi);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint2 raw = *reinterpret_cast<const uint2*>(p8 + 16 * ks);
        c[ks] = e4m3x8_to_f16(raw.x, raw.y);
      }
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const uint2 raw = *reinterpret_cast<const uint2*>(p8 + DC + 16 * j);
        r[j] = e4m3x8_to_f16(raw.x, raw.y);
      }
      return;
    }
    const char* p = ring_b + ((uint32_t)slot * (uint32_t)(RW * sizeof(E)) + 16 * hi);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) c[ks] = *reinterpret_cast<const OV8*>(p + 32 * ks);
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if constexpr (BF) {
        // k^R of a bf16 ring into the fp16 key rows
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(p + 2 * DC + 32 * j);
#pragma unroll
        for (int t = 0; t < 8; ++t) r[j][t] = (f16_t)(float)x[t];
      } else {
        r[j] = *reinterpret_cast<const V8*>(p + 2 * DC + 32 * j);
      }
    }
  };

  // Each wave walks its 32-key blocks with the next block's rows in flight.
  // The seven weight tiles run as a two-deep pipeline: tile t + 1's products
  // are issued before tile t's results are converted and staged.
  int k0 = kbeg + 32 * w;
  OV8 cf[NKS];
  V8 rf[NR];
  if (k0 < kend) load_row(k0, cf, rf);
  for (; k0 < kend; k0 += 32 * kExpandWaves) {
    OV8 cn[NKS];
    V8 rn[NR];
    const int k1 = k0 + 32 * kExpandWaves;
    if (k1 < kend) load_row(k1, cn, rn);
    // k^R into columns d_nope .. 127 of the staged key block
#pragma unroll
    for (int j = 0; j < NR; ++j)
      *reinterpret_cast<V8*>(st + stage_at(lo, kExpandNope + 16 * j + 8 * hi)) = rf[j];
    static_assert(kExpandTiles == 7 && kExpandKTiles == 3, "pipeline below is written for 3 + 4 tiles");
    // (Scheduling fences keep each tile's operand reads next to its
    // products; hoisted, the reads of all tiles would not fit in registers.)
    f32x16 acc0 = mma(0, cf);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc1 = mma(1, cf);
    stage(0, acc0);
    __builtin_amdgcn_sched_barrier(0);
    acc0 = mma(2, cf);
    stage(1, acc1);
    __builtin_amdgcn_sched_barrier(0);
    acc1 = mma(3, cf);
    stage(2, acc0);
    flush(k0, 0);
    __builtin_amdgcn_sched_barrier(0);
    acc0 = mma(4, cf);
    stage(3, acc1);
    __builtin_amdgcn_sched_barrier(0);
    acc1 = mma(5, cf);
    stage(4, acc0);
    __builtin_amdgcn_sched_barrier(0);
    acc0 = mma(6, cf);
    stage(5, acc1);
    __builtin_amdgcn_sched_barrier(0);
    stage(6, acc0);
    flush(k0, 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) cf[ks] = cn[ks];
#pragma unroll
    for (int j = 0; j < NR; ++j) rf[j] = rn[j];
  }
}

// Workgroups per (head, sequence): the key split with the fewest rounds of
// workgroups per unit of keys (one workgroup per compute unit at a time);
// measured faster than one round of longer key ranges, since each wave's
// key blocks run one after another.
int expand_splits(int n_h, int B, int Lk) {
  const int cus = device_cu_count();
  const int units = n_h * B;
  const int max_split = (Lk + 255) / 256;
  int best = 1;
  double best_cost = 1e30;
  for (int s = 1; s <= max_split && s <= 256; ++s) {
    const double rounds = (double)((units * s + cus - 1) / cus);
    const double cost = rounds / s;
    if (cost < best_cost - 1e-12) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

template <typename E, int DC, bool F8, bool BF>
hipError_t launch_expand_dc(const ExpandArgs& a, hipStream_t s) {
  const int splits = expand_splits(a.n_h, a.B, a.Lk);
  const int kpb = ((a.Lk + splits - 1) / splits + 31) / 32 * 32;
  dim3 grid((unsigned)((a.Lk + kpb - 1) / kpb), (unsigned)a.n_h, (unsigned)a.B);
  hipLaunchKernelGGL((expand_kv_kernel<E, DC, F8, BF>), grid, dim3(kExpandWaves * 64), 0, s, a, kpb);
  return hipGetLastError();
}

template <typename E, bool F8, bool BF>
hipError_t launch_expand_typed(const ExpandArgs& a, hipStream_t s) {
  switch (a.d_c) {
    case 64: return launch_expand_dc<E, 64, F8, BF>(a, s);
    case 128: return launch_expand_dc<E, 128, F8, BF>(a, s);
    case 192: return launch_expand_dc<E, 192, F8, BF>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool expand_supported(int d_c, int d_rope, int d_nope, int d_v) {
  return (d_c == 64 || d_c == 128 || d_c == 192) && d_nope == kExpandNope && d_rope == kExpandRope &&
         d_v == kExpandDv;
}

// Every 2-byte and one-byte ring expands into an fp16 window.
hipError_t launch_expand_kv(const ExpandArgs& a, hipStream_t s) {
  if (a.cache_type == 3) return launch_expand_typed<f16_t, true, false>(a, s);
  if (a.cache_type == 1) return launch_expand_typed<f16_t, false, true>(a, s);
  return a.cache_type == 2 ? launch_expand_typed<f16_t, false, false>(a, s) : hipErrorInvalidValue;
}

}  // namespace mla
