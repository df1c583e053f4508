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
//     written as [B][Lk][2][n_h][d_h] in the ring's element type - the layout
//     of the dense cache, so the same attention core reads it.  A workgroup
//     owns one head and a range of keys of one sequence: the head's whole
//     [d_nope + d_v][d_c] matrix is loaded into LDS once (direct
//     global->LDS loads for a bf16 ring, converted to fp16 on the way for an
//     fp16 ring), then each wave independently walks 32-key blocks:
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

// DC: latent width.  Workgroup (x, h, b): head h of sequence b, keys
// [x * keys_per_block, (x + 1) * keys_per_block).
template <typename E, int DC>
__global__ __launch_bounds__(kExpandWaves * 64) void expand_kv_kernel(ExpandArgs a, int keys_per_block) {
  typedef typename Elem<E>::v8 V8;
  constexpr int NKS = DC / 16;         // MFMA depth steps
  constexpr int CPR = DC / 8;          // 16-byte chunks per weight row
  constexpr int TILE = 32 * DC;        // elements per weight tile (32 rows)
  constexpr int DH = 128;              // per-head key width (d_nope + d_rope) and value width
  constexpr int WSPANS = kExpandTiles * TILE * 2 / 1024;
  static_assert(DC % 64 == 0 && (TILE * 2) % 1024 == 0, "whole 1-KiB spans per tile");
  static_assert(CPR % 8 == 0, "the chunk permutation stays inside groups of 8");
  static_assert(kExpandNope + kExpandRope == DH && kExpandDv == DH, "128-wide heads");
  __shared__ __attribute__((aligned(1024))) E wts[kExpandTiles * TILE];
  __shared__ __attribute__((aligned(16))) E stg[kExpandWaves][32 * DH];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int kbeg = blockIdx.x * keys_per_block;
  const int kend = kbeg + keys_per_block < a.Lk ? kbeg + keys_per_block : a.Lk;
  E* st = stg[w];

  // The head's weight tiles: rows [32 t, 32 t + 32) of its converted matrix.
  // In LDS, chunk q of tile row r sits at q ^ ((r >> 1) & 7) (inside aligned
  // groups of 8 chunks): the 16 lanes of a B-operand read, rows 0..15 at one
  // chunk, then touch 64 distinct banks.  Lane l of span sp fills LDS chunk
  // c = 64 sp + l: row c / CPR, position c % CPR of the rows of all tiles.
  // The rows come straight from W^K_up,h and W^V_up,h (bf16): a bf16 ring
  // copies them into LDS with direct loads, an fp16 ring converts them on the
  // way (exact for these weights' range).
  {
    const bf16_t* src_k = (const bf16_t*)a.w_uk + (size_t)h * kExpandNope * DC;
    const bf16_t* src_v = (const bf16_t*)a.w_uv + (size_t)h * kExpandDv * DC;
    lds_char* const wl = (lds_char*)wts;
    constexpr int SPW = (WSPANS + kExpandWaves - 1) / kExpandWaves;  // spans per wave
    auto chunk_src = [&](int sp) MLA_INLINE {
      const int c = sp * 64 + l;
      const int r = c / CPR, p = c - r * CPR;
      const int q = p ^ ((r >> 1) & 7);
      return (r < kExpandNope ? src_k + r * DC : src_v + (r - kExpandNope) * DC) + q * 8;
    };
    if constexpr (__is_same(E, bf16_t)) {
      for (int sp = w; sp < WSPANS; sp += kExpandWaves) global_to_lds16(chunk_src(sp), wl + sp * 1024);
    } else {
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
          V8 o;
#pragma unroll
          for (int t = 0; t < 8; ++t) o[t] = Elem<E>::from((float)v[j][t]);
          *reinterpret_cast<V8*>(wts + (size_t)(sp * 64 + l) * 8) = o;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // B-operand read: lane (col lo, hi) takes chunk 2 ks + hi of tile row lo.
  const int rsw = (lo >> 1) & 7;
  // Staged block: key kk's 128 columns at st[kk * DH ..]; column chunk q
  // (8 columns) of key kk sits at chunk q ^ (kk & 15), so the two half-waves
  // of a tile store (keys 4 apart) and the key-row reads spread over the banks.
  auto stage_at = [&](int kk, int col) __attribute__((always_inline)) {
    return kk * DH + ((((col >> 3) ^ kk) & 15) << 3) + (col & 7);
  };
  // Write the staged 32 x 128 block of keys k0.. as part `part` (0 keys,
  // 1 values): 16 lanes per key row, 16 bytes each.
  auto flush = [&](int k0, int part) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * 64 + l;
      const int kk = c >> 4, q = c & 15;
      const V8 v = *reinterpret_cast<const V8*>(st + kk * DH + ((q ^ kk) & 15) * 8);
      const int kg = k0 + kk;
      if (kg < kend)
        *reinterpret_cast<V8*>((E*)a.kv + ((((size_t)b * a.Lk + kg) * 2 + part) * a.n_h + h) * DH +
                               q * 8) = v;
    }
  };
  // This lane's latent row of the 32-key block at k0 (A operand: key lo,
  // depth 16 ks + 8 hi .. + 8, then k^R as 8-column pieces 8 hi + 16 j);
  // keys past the range load key k0's row (never written out).
  constexpr int NR = kExpandRope / 16;  // k^R pieces per lane
  auto load_row = [&](int k0, V8 (&c)[NKS], V8 (&r)[NR]) __attribute__((always_inline)) {
    const int key = k0 + lo < kend ? k0 + lo : k0;
    int64_t slot = a.key_slot0 + key;
    if (slot >= a.ring_rows) slot -= a.ring_rows;
    const E* crow = (const E*)a.ring + ((size_t)b * a.ring_rows + slot) * (DC + kExpandRope);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) c[ks] = ld8<E>(crow + 16 * ks + 8 * hi);
#pragma unroll
    for (int j = 0; j < NR; ++j) r[j] = ld8<E>(crow + DC + 16 * j + 8 * hi);
  };

  for (int k0 = kbeg + 32 * w; k0 < kend; k0 += 32 * kExpandWaves) {
    V8 cf[NKS], rf[NR];
    load_row(k0, cf, rf);

    // k^R into columns d_nope .. 127 of the staged key block
#pragma unroll
    for (int j = 0; j < NR; ++j)
      *reinterpret_cast<V8*>(st + stage_at(lo, kExpandNope + 16 * j + 8 * hi)) = rf[j];
#pragma unroll 1
    for (int t = 0; t < kExpandTiles; ++t) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
      const E* wrow = wts + t * TILE + lo * DC;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        acc = Elem<E>::mfma(cf[ks], ld8<E>(wrow + 8 * ((2 * ks + hi) ^ rsw)), acc);
      // D[key][col]: lane holds column c0 + lo of keys 8 (r / 4) + 4 hi + r % 4.
      const int c0 = t < kExpandKTiles ? 32 * t : 32 * (t - kExpandKTiles);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        st[stage_at(8 * (r >> 2) + 4 * hi + (r & 3), c0 + lo)] = Elem<E>::from(acc[r]);
      if (t == kExpandKTiles - 1) flush(k0, 0);
      if (t == kExpandTiles - 1) flush(k0, 1);
    }
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

template <typename E, int DC>
hipError_t launch_expand_dc(const ExpandArgs& a, hipStream_t s) {
  const int splits = expand_splits(a.n_h, a.B, a.Lk);
  const int kpb = ((a.Lk + splits - 1) / splits + 31) / 32 * 32;
  dim3 grid((unsigned)((a.Lk + kpb - 1) / kpb), (unsigned)a.n_h, (unsigned)a.B);
  hipLaunchKernelGGL((expand_kv_kernel<E, DC>), grid, dim3(kExpandWaves * 64), 0, s, a, kpb);
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
  return (d_c == 64 || d_c == 128 || d_c == 192) && d_nope == kExpandNope && d_rope == kExpandRope &&
         d_v == kExpandDv;
}

hipError_t launch_expand_kv(const ExpandArgs& a, hipStream_t s) {
  return a.cache_type == 2 ? launch_expand_typed<f16_t>(a, s) : launch_expand_typed<bf16_t>(a, s);
}

}  // namespace mla
