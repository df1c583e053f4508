// Flash-style attention core shared by the latent (absorbed) path and the
// dense comparison path, for gfx950 MFMA (fp16 or bf16 operands, fp32 sums).
//
// Rows are prepared query rows (cache type, pre-scaled by log2(e)/sqrt(d));
// keys are ring rows of the window.  A block of NW waves owns row groups of
// 32 * NW rows (32 per wave) and walks key tiles of KT keys (CoreShape: 8 x 64
// for many rows, narrower blocks on 32-key tiles for a few rows).  A wave whose
// 32 rows are all padding still loads its share of each tile but skips the
// arithmetic:
//
//  * Schedule (Schedule in mla_launch.h): whole row groups data-parallel
//    while they last, the remainder balanced stream-K style with main blocks
//    in key-tile lockstep and a short, L2-resident tail range shared by the
//    spare blocks, so every compute unit gets the same work however the row
//    count divides.  A block writes one partial (un-normalised value sums,
//    running max, running sum) per row-group segment; the merge kernels
//    combine a group's partials by log-sum-exp.
//  * Key tiles move HBM -> LDS with gfx950's direct 16-byte loads
//    (global_load_lds_dwordx4): each wave instruction fills one contiguous
//    KiB of LDS, lane l writing bytes [16l, 16l+16).  LDS rows are not padded;
//    instead the 16-byte chunks of a key row are XOR-permuted by the key index
//    (chunk q of key r sits at position q ^ swz(r), inside its aligned group of
//    4 chunks for latent rows, 16 for dense rows), so that the score and
//    transpose reads of 16 consecutive keys hit distinct LDS banks.  Every lane
//    of a load instruction is active and the lanes of each aligned 64-byte
//    group read one 64-byte piece of the ring (in permuted order), which the
//    memory pipeline coalesces like a straight copy.  NS tile buffers (distinct
//    LDS arrays, cycled by an NS-fold unrolled step loop so that every access
//    names its buffer) form a ring: NS - 1 tiles stream in while one is
//    consumed, one barrier per tile.  Each wave waits for its own loads of the
//    next tile with an exact vector-memory count (loads retire in order), then
//    the barrier publishes the tile to the block.  The chunk shape uses two
//    buffers (it is MFMA-bound); the narrow shapes use deeper rings, since a
//    few query rows leave them bound by the key bytes in flight.
//  * Scores S^T[key][row] = sum_d K[key][d] Q[row][d] on 32x32x16 MFMA; a
//    segment's query fragments stay in registers.  In this orientation a lane
//    owns one row (MFMA column): the row's running max and sum live in the
//    lane, and one exchange with the other half-wave covers the whole tile.
//  * Values O^T[dim][row] += sum_key V^T[dim][key] P[row][key]: the V^T
//    operand is read straight from the key-major tile with the LDS transpose
//    read (ds_read_b64_tr_b16), so no transposed copy of V is stored.
//  * Online softmax in the exp2 domain with a lazy rescale: the running max
//    is raised (and O, l rescaled) only when a score exceeds it by more than
//    2^8, so most tiles skip the rescale; probabilities stay <= 256.
//
// Latent rows (SHARED_KV): K = [c | k^R] and V = c are one cached row, so the
// value operand reads the first DV columns of the key tile.  Dense rows: K and
// V of head h are separate slices of the cached row, both staged per key.
//
// Split operands (SPLIT, used with a bf16 cache): bf16 keeps 8 significant
// bits, and the rounding of the prepared query and of the probabilities to
// bf16 does not average out over the window (keys and values come from the
// same cached rows, so the softmax's tilt carries it coherently into the
// output).  Each of the two is then carried as a pair of bf16 values, a
// leading part and the bf16 rounding of the remainder, and every product is
// issued for both parts with the same cached operand: 16 significant bits,
// at twice the matrix work.  The extra registers take the whole register
// file of a SIMD, so split blocks run one wave per SIMD.
//
// One-byte latent rows (F8, an E4M3 cache): the direct loads bring the raw
// tile (KT * DQK bytes, the ring rows as they are) into a staging buffer,
// half the bytes of a 2-byte tile; at the start of its step every lane widens
// its share to fp16 (exact) into one decode buffer in the layout above, keys
// past the window zeroed, and a barrier publishes it.  The staging buffer is
// refilled right after that barrier, so the next NS raw tiles stream in while
// the widened one is consumed.  Products then run on fp16 operands as for an
// fp16 cache.
// One-wave 16-row blocks widen differently: each lane widens the key
// fragments of its own score products into registers and writes only the
// value columns to the decode buffer (nothing is read back for the scores).
#pragma once

#include "mla_device.h"

namespace mla {

struct AttnCore {
  const void* qrows;     // [B][R][DQK] elements of the cache type
  const void* qrows_lo;  // split operands: the remainders, same layout
  const void* ring;      // [B][ring_rows][ring_stride]
  float* opart;          // [n_slots][B][R][DV]  un-normalised value sums
  float* ml;             // [n_slots][B][R][2]   running max (log2 units), sum
  int part16;            // partials stored normalised (O / l) as fp16 (see load_part4)
  int64_t ring_rows;
  int ring_stride;       // elements per cached token row
  int k_off, v_off;      // offsets of K and V of head 0 inside a cached row
  int head_stride;       // offset step per head (0 for the shared latent row)
  int R;                 // rows per batch element (dense: a multiple of the
                         // block rows per head; latent: ragged)
  int rows_per_head;     // rows of one head (latent: R)
  int valid_per_head;    // rows of a head that are real (rest is padding)
  int B, Lk;
  Schedule sched;
  int64_t key_slot0;     // ring slot of resident key 0
};

// Four values of a partial row at element `elem` as fp32.  Partials of the
// few-row shapes are stored normalised (O / l: a convex combination of cached
// values, so within the cache type's range) as fp16, half the bytes of the
// fp32 sums; readers then weight them by l as well.
template <bool P16>
__device__ __forceinline__ f32x4 load_part4(const float* opart, size_t elem) {
  if constexpr (P16) {
    const f16x4 h = *reinterpret_cast<const f16x4*>((const f16_t*)opart + elem);
    f32x4 r = {(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    return r;
  }
  return *reinterpret_cast<const f32x4*>(opart + elem);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS transpose read: within each 16-lane group, lane i receives element i%4
// of the 8-byte rows addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Direct 16-byte global -> LDS load (global_load_lds_dwordx4): lane l of the
// wave writes LDS bytes [lds + 16 l, lds + 16 l + 16); `lds` must be uniform.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ void global_to_lds16(const void* g, lds_char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#endif
}

// Lambdas of the kernel body are always inlined: one left out of line would
// turn its reference captures into loads through a stack frame.
#define MLA_INLINE __attribute__((always_inline))

// Accumulator fragment of one MFMA shape: 32x32 (16 values per lane) or
// 16x16 (4 values per lane).
template <int ROWS>
struct AccOf;
template <>
struct AccOf<32> {
  typedef f32x16 type;
};
template <>
struct AccOf<16> {
  typedef f32x4 type;
};

// Raise-the-max threshold of the lazy rescale (log2 units).
constexpr float kRescaleThreshold = 8.0f;

// s_waitcnt immediate that waits until at most n vector memory operations of
// this wave are outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima, i.e. not waited on).
#define MLA_VMCNT(n) ((((n)&15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))
#define MLA_VMCASE(n) \
  case n:             \
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(n)); \
    break;

__device__ __forceinline__ void wait_vmem(int n) {
  switch (n) {
    MLA_VMCASE(0) MLA_VMCASE(1) MLA_VMCASE(2) MLA_VMCASE(3) MLA_VMCASE(4) MLA_VMCASE(5)
    MLA_VMCASE(6) MLA_VMCASE(7) MLA_VMCASE(8) MLA_VMCASE(9) MLA_VMCASE(10) MLA_VMCASE(11)
    MLA_VMCASE(12) MLA_VMCASE(13) MLA_VMCASE(14) MLA_VMCASE(15) MLA_VMCASE(16) MLA_VMCASE(17)
    MLA_VMCASE(18) MLA_VMCASE(19) MLA_VMCASE(20) MLA_VMCASE(21) MLA_VMCASE(22) MLA_VMCASE(23)
    MLA_VMCASE(24) MLA_VMCASE(25) MLA_VMCASE(26) MLA_VMCASE(27) MLA_VMCASE(28) MLA_VMCASE(29)
    MLA_VMCASE(30) MLA_VMCASE(31) MLA_VMCASE(32) MLA_VMCASE(33) MLA_VMCASE(34) MLA_VMCASE(35)
    MLA_VMCASE(36) MLA_VMCASE(37) MLA_VMCASE(38) MLA_VMCASE(39) MLA_VMCASE(40) MLA_VMCASE(41)
    MLA_VMCASE(42) MLA_VMCASE(43) MLA_VMCASE(44) MLA_VMCASE(45) MLA_VMCASE(46) MLA_VMCASE(47)
    MLA_VMCASE(48) MLA_VMCASE(49) MLA_VMCASE(50) MLA_VMCASE(51) MLA_VMCASE(52) MLA_VMCASE(53)
    MLA_VMCASE(54) MLA_VMCASE(55) MLA_VMCASE(56) MLA_VMCASE(57) MLA_VMCASE(58) MLA_VMCASE(59)
    MLA_VMCASE(60) MLA_VMCASE(61) MLA_VMCASE(62)
    default: __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0)); break;
  }
}
#undef MLA_VMCASE

// Block barrier that waits only for this wave's LDS instructions: tile loads
// in flight stay in flight (the steps wait for the ones they need with
// wait_vmem first).  A memory fence here would also wait for every direct
// global->LDS load, since those write LDS.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Register budget: two waves per SIMD for one 32-row block per wave, so that
// narrow blocks can share a compute unit; one wave per SIMD (the whole
// register file, accumulators in AGPRs) when each wave owns RB > 1 row blocks.
template <typename E, int DQK, int DV, int NW, int KT, int NS, bool SHARED_KV, int RB = 1,
          bool PP = false, int ROWS = 32, bool SPLIT = false, bool F8 = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu((RB == 1 && !SPLIT) ? 2 : 1, (RB == 1 && !SPLIT) ? 2 : 1)))
void attn_core_kernel(AttnCore a) {
  typedef typename Elem<E>::v8 V8;
  // ROWS = 32: 32x32x16 MFMAs, a lane owns one row (MFMA column) with its two
  // half-waves splitting the keys.  ROWS = 16: 16x16x32 MFMAs, a row is shared
  // by the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48).
  constexpr bool R16 = ROWS == 16;
  typedef typename AccOf<ROWS>::type AccT;   // accumulator fragment
  constexpr int AV = R16 ? 4 : 16;            // accumulator values per lane
  constexpr int NKS = R16 ? DQK / 32 : DQK / 16;  // MFMA depth steps of the score product
  constexpr int NDT = R16 ? DV / 16 : DV / 32;    // MFMA column tiles of the value product
  constexpr int BR = NW * ROWS * RB;          // rows per row group (ROWS * RB per wave)
  constexpr int NKB = KT / ROWS;              // MFMA key blocks per tile
  constexpr int NPF = R16 ? 1 : 2 * NKB;      // probability operands per row block
  static_assert(ROWS == 32 || (ROWS == 16 && (NW == 1 || NW == 4) && KT == 32 && RB == 1 && !PP &&
                               DQK % 32 == 0 && DV % 16 == 0),
                "16-row waves: one- or four-wave blocks on 32-key tiles");
  constexpr int KCH = DQK / 8;                // 16-byte chunks of K per key
  constexpr int CPK = SHARED_KV ? KCH : KCH + DV / 8;  // chunks staged per key
  constexpr int KSTR = CPK * 8;               // LDS row stride (elements)
  constexpr int VOFF = SHARED_KV ? 0 : DQK;   // V columns inside an LDS row
  constexpr int CHUNKS = KT * CPK;            // 16-byte chunks per tile
  constexpr int SPANS = CHUNKS / 64;          // 1-KiB direct-load spans per tile
  constexpr int TILE = KT * KSTR;             // elements per tile buffer
  static_assert(KT == 32 || KT == 64, "key tiles are one or two 32-key MFMA blocks");
  static_assert(!SHARED_KV || DV <= DQK, "shared rows hold V inside K");
  static_assert(NS >= 2 && NS <= 5, "two to five tile buffers");
  static_assert(!PP || (NS == 3 && NW % 2 == 0 && NW >= 2), "ping-pong: two wave groups, three buffers");
  static_assert(!SPLIT || (NW <= 4 && RB == 1), "split operands: one wave per SIMD");
  constexpr int NQ = SPLIT ? 2 : 1;           // operand parts (leading, remainder)
  static_assert(!F8 || (SHARED_KV && __is_same(E, f16_t) && !PP && !SPLIT && RB == 1),
                "one-byte latent rows widen to fp16 operands");
  constexpr int SPANS8 = KT * DQK / 1024;     // 1-KiB direct-load spans of a raw one-byte tile
  static_assert(!F8 || (KT * DQK) % 1024 == 0, "raw tiles are whole 1-KiB spans");
  constexpr int SPL = F8 ? SPANS8 : SPANS;    // spans loaded per tile
  static_assert((SPL + NW - 1) / NW * (NS - 1) <= 63, "tile loads in flight fit the vmcnt counter");
  // Whole spans with every lane active (exact load counts per wave); the chunk
  // permutation stays inside aligned groups of a row.
  static_assert(CHUNKS % 64 == 0, "tiles are whole 1-KiB spans");
  static_assert(SHARED_KV ? (CPK % 4 == 0 && (CPK * 4) % 32 == 16)
                          : (CPK % 16 == 0 && KCH % 16 == 0),
                "row strides the swizzle was laid out for");

  // Tile buffers (raw one-byte tiles for F8: half the size) and, for F8, the
  // decode buffer the products read.
  constexpr int TB = F8 ? TILE / 2 : TILE;
  __shared__ __attribute__((aligned(1024))) E kt0[TB];
  __shared__ __attribute__((aligned(1024))) E kt1[TB];
  __shared__ __attribute__((aligned(1024))) E kt2[NS > 2 ? TB : 8];
  __shared__ __attribute__((aligned(1024))) E kt3[NS > 3 ? TB : 8];
  __shared__ __attribute__((aligned(1024))) E kt4[NS > 4 ? TB : 8];
  __shared__ __attribute__((aligned(1024))) E kd[F8 ? TILE : 8];

  const Schedule& sc = a.sched;
  const int tid = threadIdx.x;
  // The tile loads sit under per-wave span tests (sp < SPANS below) that the
  // compiler does not fold, even for one-wave blocks.  All waits for tile
  // loads are explicit (exact per-wave counts, then a barrier); loads the
  // compiler cannot count are ones it does not try to wait for itself.
  const int w = NW == 1 ? 0 : tid >> 6, l = tid & 63, lo = l & 31, hi = l >> 5;
  const int g = sched_block_of(sc, blockIdx.x);
  const int n_steps = sched_block_steps(sc, g);
  const int n_ld = (SPL - w + NW - 1) / NW;  // direct loads this wave issues per tile

  // Chunk permutation of key row r (it depends on r mod 16 only).  Latent
  // rows are 4 * CPK dwords long, an odd multiple of 16 dwords (mod 64), so
  // four consecutive keys start in four different 16-bank windows and the
  // XOR has to separate keys r, r + 4, r + 8, r + 12; this one also separates
  // the even (odd) keys among 8 consecutive ones.  Dense rows are a multiple
  // of 64 dwords: the permutation spreads 16 keys over 16 chunk slots and
  // puts keys 4j .. 4j + 3 in different 4-chunk groups.  With 64 banks of
  // 4 bytes, the 16 lanes of a score read and the 32 lanes of a transpose
  // read then touch every bank once.
  auto swz = [](int r) MLA_INLINE {
    return SHARED_KV ? (((r >> 2) ^ (r >> 1)) & 3) : (((r & 3) << 2) | ((r >> 2) & 3));
  };

  // Issue the direct loads of key tile kt of batch element b into `dst`.  Keys
  // past the window re-load the last key (their scores are masked), so every
  // LDS row a wave reads holds finite cache data.  Wave w issues spans w,
  // w + NW, ...; lane l of span sp fills LDS chunk c = 64 sp + l: key
  // c / CPK, position p = c % CPK, which holds chunk p ^ swz(key) of the key's
  // row.  Offsets within one sequence's ring fit 32 bits (checked when the
  // cache is created).
  constexpr int LPW = (SPANS + NW - 1) / NW;  // span slots per wave
  // Lane offset (elements) of span sp relative to the first key row of a
  // tile and the head's K columns (V columns sit at v_off - k_off from K).
  // For F8 the same offsets (ring_stride = DQK) address the 8 raw bytes of
  // the chunk a lane decodes in the staging buffer.
  // 16 keys fill CPK / 4 spans exactly and the chunk permutation repeats
  // every 16 keys, so span sp + CPK / 4 is span sp shifted by 16 key rows: a
  // one-wave block keeps the CPK / 4 distinct lane offsets, a wider block the
  // offsets of its own (at most four) spans.
  constexpr int PER = CPK / 4;
  static_assert((64 * PER) % CPK == 0 && 64 * PER / CPK == 16, "16 keys per span period");
  auto lane_offset = [&](int sp) MLA_INLINE {
    const int c = sp * 64 + l;
    const int key = c / CPK, q = (c - key * CPK) ^ swz(key);
    return key * a.ring_stride + (q < KCH ? q * 8 : a.v_off - a.k_off + (q - KCH) * 8);
  };
  constexpr int LKEEP = NW == 1 ? (PER < SPANS ? PER : SPANS) : LPW;
  int lane_off[LKEEP];
  uint32_t lane_bytes[LKEEP];  // the same in bytes (non-negative)
#pragma unroll
  for (int j = 0; j < LKEEP; ++j) {
    lane_off[j] = lane_offset(NW == 1 ? j : w + j * NW);
    lane_bytes[j] = (uint32_t)lane_off[j] * (uint32_t)sizeof(E);
  }
  auto load_tile = [&](int b, int head, int kt, E* dst) MLA_INLINE {
    const int rows = (int)a.ring_rows;
    int s0 = (int)a.key_slot0 + kt * KT;
    s0 = s0 >= rows ? s0 - rows : s0;
    if constexpr (F8) {
      // The raw tile is KT * DQK contiguous bytes of the ring (rows of DQK
      // bytes); lane l of span sp copies bytes [1024 sp + 16 l, + 16).  Past
      // the ring's end the bytes continue at its start.
      const char* base = (const char*)a.ring + ((size_t)b * rows + s0) * DQK;
      lds_char* const ldst = (lds_char*)dst;
      const int split = (rows - s0) * DQK, back = rows * DQK;
#pragma unroll
      for (int j = 0; j < (SPANS8 + NW - 1) / NW; ++j) {
        const int sp = w + j * NW;
        if (NW == 1 || sp < SPANS8) {
          int off = sp * 1024 + 16 * l;
          off = off >= split ? off - back : off;
          if (rows < KT)  // a ring shorter than the tile: keys past the window wrap again
            while (off >= split) off -= back;
          global_to_lds16(base + off, ldst + sp * 1024);
        }
      }
      return;
    }
    const E* ring = (const E*)a.ring + (size_t)b * a.ring_rows * a.ring_stride;
    const E* base = ring + ((size_t)s0 * a.ring_stride + a.k_off + head * a.head_stride);
    // Keys of a tile that crosses the ring's end continue at its start: the
    // lane offsets at or past the crossing move back by the ring size (as
    // often as needed when the ring holds fewer rows than a tile; such keys
    // are past the window, so only their addresses matter).
    // (Keys past the window still read ring rows - allocated, possibly stale
    // memory; the step that uses the tile clears them in LDS.)
    const bool wraps = s0 + KT > rows;
    // (The LDS address space is taken before any offset is added, so that
    // the buffer's address folds to a constant.)
    lds_char* const ldst = (lds_char*)dst;
    if (!wraps) {
      // Common case: a wave-uniform base per 16-key period plus the lane's
      // 32-bit byte offset, which maps onto the load's scalar-base form.
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int sp = w + j * NW;
        if (NW == 1 || sp < SPANS) {
          const char* pb = (const char*)(NW == 1 ? base + (j / PER) * 16 * a.ring_stride : base);
          global_to_lds16(pb + lane_bytes[NW == 1 ? j % PER : j], ldst + sp * 1024);
        }
      }
      return;
    }
    const int split = (rows - s0) * a.ring_stride, back = rows * a.ring_stride;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int sp = w + j * NW;
      if (NW == 1 || sp < SPANS) {
        int off = NW == 1 ? (j / PER) * 16 * a.ring_stride + lane_off[j % PER] : lane_off[j];
        off = off >= split ? off - back : off;
        if (rows < KT)  // a ring shorter than the tile: keys past the window wrap again
          while (off >= split) off -= back;
        global_to_lds16(base + off, ldst + sp * 1024);
      }
    }
  };

  // Zero the rows of keys past the window in a ragged last tile: their
  // scores are masked, and zero values keep the value product finite.
  auto scrub = [&](int kt, E* buf) MLA_INLINE {
    const int nk = a.Lk - kt * KT;  // keys of the tile inside the window (0 < nk < KT)
    f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = nk * CPK + w * 64 + l; c < KT * CPK; c += NW * 64)
      *reinterpret_cast<f32x4*>(buf + c * 8) = zero;
  };

  // F8: widen the raw tile in `stage` (key tile kt) into the decode buffer.
  // Lane l of span sp writes decode chunk c = 64 sp + l (key c / CPK, the
  // permuted position of the direct loads above) from the 8 raw bytes of the
  // key's chunk (c % CPK) ^ swz(key); keys past the window become zeros.
  auto decode = [&](const E* stage, int kt) MLA_INLINE {
    const char* src = (const char*)stage;
    const int nk = a.Lk - kt * KT;  // keys of the tile inside the window
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int sp = NW == 1 ? j : w + j * NW;
      if (NW == 1 || sp < SPANS) {
        const int off = NW == 1 ? (j / PER) * 16 * DQK + lane_off[j % PER] : lane_off[j];
        const uint2 raw = *reinterpret_cast<const uint2*>(src + off);
        f16x8 h = e4m3x8_to_f16(raw.x, raw.y);
        const int c = sp * 64 + l;
        if (nk < KT && c / CPK >= nk) h = zero8<f16_t>();
        *reinterpret_cast<f16x8*>(kd + c * 8) = h;
      }
    }
  };

  // Lane-constant parts of the LDS read addresses.  Score reads: lane (lo, hi)
  // reads chunk 2 ks + hi of key kb * 32 + lo.  Transpose reads: the lane
  // addresses key row tr_key (+ 8 for the second half) of a 16-key step and
  // the 8 bytes at chunk 4 dt + tr_c, half tr_h, of a 32-column tile.
  // (2 ks + hi) ^ s = 2 (ks ^ (s >> 1)) + (hi ^ (s & 1)); for latent rows
  // s < 4, so even and odd ks each need one lane offset.  Likewise
  // (4 dt + c) ^ s = 4 (dt ^ (s >> 2)) + (c ^ (s & 3)).
  const int k_sw = swz(lo);
  const int k_off0 = 8 * (hi ^ (k_sw & 1)) + 16 * (k_sw >> 1);        // even ks (latent)
  const int k_off1 = 8 * (hi ^ (k_sw & 1)) + 16 * ((k_sw >> 1) ^ 1);  // odd ks (latent)
  const int tr_key = 4 * hi + ((l & 15) >> 2);
  const int tr_c = 2 * ((l & 31) >> 4) + ((l & 3) >> 1);
  const int tr_h = 4 * (l & 1);
  const int tr_sw0 = swz(tr_key), tr_sw1 = swz(tr_key + 8);
  const int tr_off0 = tr_h + 8 * (tr_c ^ (tr_sw0 & 3)), tr_off1 = tr_h + 8 * (tr_c ^ (tr_sw1 & 3));
  const int tr_dt0 = tr_sw0 >> 2, tr_dt1 = tr_sw1 >> 2;  // 0 for latent rows
  // 16-row waves: lane (r16, g16) is MFMA row/column r16 of 16-lane group g16.
  // Score reads: chunk 4 s + g16 of key kb * 16 + r16.  Transpose reads: the
  // lane addresses key 4 g16 + t16 (+ 16 for the second key block) and the
  // 8 bytes of columns 4 c16 .. + 4 of a 16-column tile, so that lane i of the
  // group receives column i of keys 4 g16 .. 4 g16 + 3.
  const int r16 = l & 15, g16 = l >> 4;
  const int k_sw16 = swz(r16);
  const int t16 = r16 >> 2, c16 = r16 & 3;
  const int tsw16 = swz(4 * g16 + t16);

  // F8, one-wave 16-row blocks: each lane widens exactly the key fragments
  // its score products take (chunk 4 ks + g16 of key kb * 16 + r16, read from
  // the raw tile at its place in the ring row) and keeps them in registers;
  // only the value columns (the first DV of a row) go to the decode buffer,
  // at the permuted positions the transpose reads expect.  The wave's lanes
  // cover every chunk of the tile once, so nothing is read back for the
  // scores.  Keys past the window become zeros.
  auto decode_frags = [&](const E* stage, int kt, auto& kf) MLA_INLINE {
    const char* src = (const char*)stage;
    const int nk = a.Lk - kt * KT;  // keys of the tile inside the window
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int key = kb * 16 + r16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int q = 4 * ks + g16;
        const uint2 raw = *reinterpret_cast<const uint2*>(src + key * DQK + 8 * q);
        f16x8 h = e4m3x8_to_f16(raw.x, raw.y);
        if (key >= nk) h = zero8<f16_t>();
        kf[kb][ks] = h;
        if (ks < DV / 32) *reinterpret_cast<f16x8*>(kd + (key * CPK + (q ^ k_sw16)) * 8) = h;
      }
    }
  };

  // Per row block rb of the wave: query fragments, value sums, running max
  // and sum, the lane's row.  Each key fragment read from LDS feeds RB
  // products, so LDS traffic per product falls as 1 / RB.
  V8 qf[NQ][RB][NKS];
  AccT o[RB][NDT];
  float m[RB], lsum[RB];
  int row[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    lsum[rb] = 0.0f;
    row[rb] = 0;
  }
  bool live = false;  // this wave's rows include a real one (wave-uniform)

  // Tiles issued after tile i + 1 by the end of step i, counting the refill
  // of step i itself (the ring is short near the end of the block's steps).
  auto ahead = [&](int i) MLA_INLINE {
    const int a2 = n_steps - i - 2;
    return a2 < 0 ? 0 : (a2 < NS - 1 ? a2 : NS - 1);
  };
  // Block-uniform walks over the block's steps: `wc` is the step being
  // computed, `wi` the next tile to load (tiles are issued in step order).
  // Each keeps its segment's batch element and head.
  struct Walk {
    SchedCursor c;
    int b, head;
  };
  auto walk_segment = [&](Walk& x) MLA_INLINE {
    x.b = x.c.si.grp / sc.n_rg;
    x.head = ((x.c.si.grp - x.b * sc.n_rg) * BR) / a.rows_per_head;
  };
  auto walk_next = [&](Walk& x) MLA_INLINE {
    if (sched_cursor_next(sc, g, n_steps, x.c)) walk_segment(x);
  };
  Walk wc, wi;
  // Load the next tile of the block's walk into `dst`.
  auto issue = [&](E* dst) MLA_INLINE {
    load_tile(wi.b, wi.head, wi.c.si.kt, dst);
    walk_next(wi);
  };

  // New row-group segment: query fragments in (global loads, not waited on
  // here), running state reset.
  auto begin_segment = [&](int b, int rg) MLA_INLINE {
    const int row0 = rg * BR + w * ROWS * RB;  // rows of a wave never straddle a head
    live = row0 < a.R && (row0 % a.rows_per_head) < a.valid_per_head;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      row[rb] = row0 + ROWS * rb + (R16 ? r16 : lo);
      const int r = row[rb];
      const bool ok = r < a.R && (r % a.rows_per_head) < a.valid_per_head;
      const size_t qoff = ((size_t)b * a.R + (ok ? r : 0)) * DQK + (R16 ? 8 * g16 : 8 * hi);
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const E* src = (const E*)(u == 0 ? a.qrows : a.qrows_lo) + qoff;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[u][rb][ks] = ok ? ld8<E>(src + (R16 ? 32 : 16) * ks) : zero8<E>();
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < AV; ++q) o[rb][dt][q] = 0.0f;
      m[rb] = -INFINITY;
      lsum[rb] = 0.0f;
    }
  };

  // The three phases of a step on one key tile, for this wave's rows.
  // 16-row waves: the score products from the tile's key fragments (lane
  // (r16, g16) holds chunk 4 ks + g16 of key kb * 16 + r16), the two key
  // blocks' chains interleaved.
  auto score_products16 = [&](const auto& kf, auto& sv) MLA_INLINE {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < AV; ++r) sv[0][kb][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int u = 0; u < NQ; ++u) sv[0][kb] = Elem<E>::mfma16(kf[kb][ks], qf[u][0][ks], sv[0][kb]);
  };
  // Scores S^T = K Q^T of the tile in `cur`.
  auto scores = [&](const E* cur, AccT (&sv)[RB][NKB]) MLA_INLINE {
    if constexpr (R16) {
      // All key fragments of the tile first, then the products (the two key
      // blocks' chains interleaved): a narrow block has too few waves per
      // SIMD to hide one LDS round trip per product.
      V8 kf[NKB][NKS];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const E* krow = cur + (kb * 16 + r16) * KSTR;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) kf[kb][ks] = ld8<E>(krow + 8 * ((4 * ks + g16) ^ k_sw16));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
      score_products16(kf, sv);
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[rb][kb][r] = 0.0f;
        const E* krow = cur + (kb * 32 + lo) * KSTR;
        auto kptr = [&](int ks) MLA_INLINE {
          return SHARED_KV ? krow + 32 * (ks >> 1) + ((ks & 1) ? k_off1 : k_off0)
                           : krow + 8 * ((2 * ks + hi) ^ k_sw);
        };
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const V8 kf = ld8<E>(kptr(ks));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int u = 0; u < NQ; ++u) sv[rb][kb] = Elem<E>::mfma(kf, qf[u][rb][ks], sv[rb][kb]);
        }
      }
    }
  };
  // Online softmax of key tile kt: mask keys past the window, lazy rescale,
  // probabilities (in the cache type) into pf, running sums.
  // Key of accumulator value r of key block kb held by this lane.
  auto key_of = [&](int kb, int r) MLA_INLINE {
    return R16 ? kb * 16 + 4 * g16 + r : kb * 32 + acc_row(r, hi);
  };
  auto softmax = [&](int kt, AccT (&sv)[RB][NKB], V8 (&pf)[NQ][RB][NPF]) MLA_INLINE {
    const int t0 = kt * KT;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (t0 + KT > a.Lk) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < AV; ++r)
            if (t0 + key_of(kb, r) >= a.Lk) sv[rb][kb][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < AV; ++r) mx = fmaxf(mx, sv[rb][kb][r]);
      if constexpr (R16) mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // lazy rescale: raise the max only when a score passes it by > 2^8
      if (__ballot(mx > m[rb] + kRescaleThreshold)) {
        const float mnew = fmaxf(m[rb], mx);
        const float alpha = exp2_fast(m[rb] - mnew);
        m[rb] = mnew;
        lsum[rb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < AV; ++r) o[rb][dt][r] *= alpha;
      }
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < AV; ++r) {
          const float p = exp2_fast(sv[rb][kb][r] - m[rb]);
          ps += p;
          // 16-row waves: value-product slot 8 g16 + 4 kb + r is key
          // kb * 16 + 4 g16 + r, so the lane's own scores form its operand
          const E ph = Elem<E>::from(p);
          const int fi = R16 ? 0 : 2 * kb + (r >> 3), fe = R16 ? 4 * kb + r : (r & 7);
          pf[0][rb][fi][fe] = ph;
          if constexpr (SPLIT) pf[1][rb][fi][fe] = Elem<E>::from(p - (float)ph);
        }
      lsum[rb] += ps;
    }
  };
  // Value sums O^T += V^T P^T of the tile in `cur`.
  auto values = [&](const E* cur, const V8 (&pf)[NQ][RB][NPF]) MLA_INLINE {
    if constexpr (R16) {
      // slots 8 g16 .. + 3: keys 4 g16 + t (block 0); + 4 .. + 7: keys 16 + 4 g16 + t
      const E* v0 = cur + (4 * g16 + t16) * KSTR + VOFF + 4 * (c16 & 1);
      const E* v1 = v0 + 16 * KSTR;
      // all transpose reads first, then the products
      i16x4 lo4[NDT], hi4[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int q = (2 * dt + (c16 >> 1)) ^ tsw16;
        lo4[dt] = lds_read_tr16(v0 + 8 * q);
        hi4[dt] = lds_read_tr16(v1 + 8 * q);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const V8 va =
            __builtin_bit_cast(V8, __builtin_shufflevector(lo4[dt], hi4[dt], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int u = 0; u < NQ; ++u) o[0][dt] = Elem<E>::mfma16(va, pf[u][0][0], o[0][dt]);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const E* vrow = cur + (kb * 32 + 16 * st + tr_key) * KSTR + VOFF;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int d0 = SHARED_KV ? dt : (dt ^ tr_dt0), d1 = SHARED_KV ? dt : (dt ^ tr_dt1);
            const i16x4 lo4 = lds_read_tr16(vrow + 32 * d0 + tr_off0);
            const i16x4 hi4 = lds_read_tr16(vrow + 8 * KSTR + 32 * d1 + tr_off1);
            const V8 va = __builtin_bit_cast(V8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
              for (int u = 0; u < NQ; ++u) o[rb][dt] = Elem<E>::mfma(va, pf[u][rb][2 * kb + st], o[rb][dt]);
          }
        }
    }
  };
  // Segment end: write this block's partial of the row group (slot si.slot)
  // of batch element b.
  auto write_partial = [&](const StepInfo& si, int b) MLA_INLINE {
    if constexpr (R16) {
      // lane (r16, g16) holds columns 16 dt + 4 g16 .. + 4 of row r16
      float ltot = lsum[0] + __shfl_xor(lsum[0], 16);
      ltot += __shfl_xor(ltot, 32);
      if (row[0] < a.R) {
        const size_t prow = ((size_t)si.slot * a.B + b) * a.R + row[0];
        float* op = a.opart + prow * DV;
        if (a.part16) {
          const float inv = 1.0f / ltot;
          f16_t* oh = (f16_t*)a.opart + prow * DV;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            f16x4 hv = {(f16_t)(o[0][dt][0] * inv), (f16_t)(o[0][dt][1] * inv), (f16_t)(o[0][dt][2] * inv),
                        (f16_t)(o[0][dt][3] * inv)};
            *reinterpret_cast<f16x4*>(oh + 16 * dt + 4 * g16) = hv;
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g16) = o[0][dt];
        }
        if (g16 == 0) {
          a.ml[prow * 2] = m[0];
          a.ml[prow * 2 + 1] = ltot;
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float ltot = lsum[rb] + __shfl_xor(lsum[rb], 32);
        if (row[rb] < a.R) {
          const size_t prow = ((size_t)si.slot * a.B + b) * a.R + row[rb];
          float* op = a.opart + prow * DV;
          const float inv = 1.0f / ltot;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
              if (a.part16) {
                f16x4 hv = {(f16_t)(o[rb][dt][4 * gg] * inv), (f16_t)(o[rb][dt][4 * gg + 1] * inv),
                            (f16_t)(o[rb][dt][4 * gg + 2] * inv), (f16_t)(o[rb][dt][4 * gg + 3] * inv)};
                *reinterpret_cast<f16x4*>((f16_t*)a.opart + prow * DV + dt * 32 + 8 * gg + 4 * hi) = hv;
              } else {
                f32x4 v = {o[rb][dt][4 * gg], o[rb][dt][4 * gg + 1], o[rb][dt][4 * gg + 2],
                           o[rb][dt][4 * gg + 3]};
                *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * gg + 4 * hi) = v;
              }
            }
          if (hi == 0) {
            a.ml[prow * 2] = m[rb];
            a.ml[prow * 2 + 1] = ltot;
          }
        }
      }
    }
  };
  // Start of step i: clear the keys past the window of a ragged last tile;
  // a segment starting mid-block loads its queries.  Its query loads retire
  // in order behind the tiles in flight, so it waits for all of them (rare:
  // only blocks that cross from one row group to the next).
  auto step_begin = [&](const StepInfo& si, int b, int i, E* cur) MLA_INLINE {
    if (si.kt * KT + KT > a.Lk) {
      scrub(si.kt, cur);
      lds_barrier();
    }
    if (si.first && i > 0) {
      begin_segment(b, si.grp - b * sc.n_rg);
      asm volatile("" ::: "memory");  // keep the loads above the wait
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    }
  };

  if (n_steps <= 0) return;
  sched_cursor_seek(sc, g, n_steps, 0, wc.c);
  walk_segment(wc);
  wi = wc;
  const StepInfo s0 = wc.c.si;
  const int b0 = wc.b;

  if constexpr (F8) {
    // A step: widen the raw tile, publish it (the barrier also frees the raw
    // buffer, refilled at once with tile i + NS), compute on the decode
    // buffer, then wait for this wave's loads of tile i + 1 and meet the
    // other waves (nobody reads the decode buffer any more).
    constexpr bool DIRECT = NW == 1 && R16;
    static_assert(!DIRECT || DV % 32 == 0, "value columns are whole 32-column score steps");
    auto step8 = [&](int i, E* stage) MLA_INLINE {
      const StepInfo si = wc.c.si;
      const int b = wc.b;
      V8 kf[DIRECT ? NKB : 1][DIRECT ? NKS : 1];
      if constexpr (DIRECT)
        decode_frags(stage, si.kt, kf);
      else
        decode(stage, si.kt);
      lds_barrier();
      if (i + NS < n_steps) issue(stage);
      if (si.first && i > 0) {
        begin_segment(b, si.grp - b * sc.n_rg);
        asm volatile("" ::: "memory");  // keep the loads above the wait
        __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
      }
      if (live) {
        AccT sv[RB][NKB];
        V8 pf[NQ][RB][NPF];
        if constexpr (DIRECT)
          score_products16(kf, sv);
        else
          scores(kd, sv);
        softmax(si.kt, sv, pf);
        values(kd, pf);
        if (si.last) write_partial(si, b);
      }
      walk_next(wc);
      if (i + 1 < n_steps) {
        wait_vmem(n_ld * ahead(i));
        lds_barrier();
      }
    };
    issue(kt0);
    if (n_steps > 1) issue(kt1);
    if (NS > 2 && n_steps > 2) issue(kt2);
    if (NS > 3 && n_steps > 3) issue(kt3);
    if (NS > 4 && n_steps > 4) issue(kt4);
    begin_segment(b0, s0.grp - b0 * sc.n_rg);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    lds_barrier();
    for (int i = 0; i < n_steps; i += NS) {
      step8(i, kt0);
      if (i + 1 < n_steps) step8(i + 1, kt1);
      if constexpr (NS > 2) if (i + 2 < n_steps) step8(i + 2, kt2);
      if constexpr (NS > 3) if (i + 3 < n_steps) step8(i + 3, kt3);
      if constexpr (NS > 4) if (i + 4 < n_steps) step8(i + 4, kt4);
    }
    return;
  }

  if constexpr (PP) {
    // Two wave groups, one wave of each per SIMD, work half a step apart so
    // that one group's softmax (vector ALU) overlaps the other's products
    // (matrix units).  Every wave runs the same steps - scores, softmax,
    // values of tile k - with one barrier per step, but group A (waves
    // 0 .. NW/2 - 1) meets it after the values and group B before them.
    // Between barriers k - 1 and k, A runs scores, softmax and values of tile
    // k while B runs the values of tile k - 1 (its probabilities wait in
    // registers across the barrier), then scores and softmax of tile k.
    // Tiles k - 1 and k are read in that interval while tile k + 1 streams
    // in: three buffers.  At its barrier a wave waits for its own loads of
    // tile k + 1 first; after the barrier and its values of tile k, it issues
    // its loads of tile k + 2 into the buffer of tile k - 1, which both groups
    // are done with.
    const bool grp_b = w >= NW / 2;
    auto sync = [&](int k) MLA_INLINE {
      if (k + 1 < n_steps) {
        __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
        lds_barrier();
      }
    };
    auto step_pp = [&](int k, E* cur, E* refill) MLA_INLINE {
      const StepInfo si = wc.c.si;
      const int b = wc.b;
      step_begin(si, b, k, cur);
      V8 pf[NQ][RB][NPF];
      if (live) {
        AccT sv[RB][NKB];
        scores(cur, sv);
        softmax(si.kt, sv, pf);
      }
      if (grp_b) sync(k);
      if (live) {
        values(cur, pf);
        if (si.last) write_partial(si, b);
      }
      if (!grp_b) sync(k);
      // Group B issues its share of tile k + 2 after its values, so that the
      // loads are not in flight while it reads tile k.
      if (k + 2 < n_steps) issue(refill);
      walk_next(wc);
    };
    begin_segment(b0, s0.grp - b0 * sc.n_rg);
    issue(kt0);
    if (n_steps > 1) issue(kt1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    lds_barrier();
    for (int k = 0; k < n_steps; k += 3) {
      step_pp(k, kt0, kt2);
      if (k + 1 < n_steps) step_pp(k + 1, kt1, kt0);
      if (k + 2 < n_steps) step_pp(k + 2, kt2, kt1);
    }
    return;
  }

  // One step: `cur` holds the key tile of step i.  Once every wave is done
  // with it, tile i + NS is issued into the same buffer.  (Issuing at the end
  // of a step keeps each buffer's write after its read within one unrolled
  // loop pass; the compiler then adds no wait of its own for the tile loads.)
  auto step = [&](int i, E* cur) MLA_INLINE {
    const StepInfo si = wc.c.si;
    const int b = wc.b;
    step_begin(si, b, i, cur);
    if (live) {
      AccT sv[RB][NKB];
      V8 pf[NQ][RB][NPF];
      scores(cur, sv);
      softmax(si.kt, sv, pf);
      values(cur, pf);
      if (si.last) write_partial(si, b);
    }
    walk_next(wc);
    // After the last step nothing is read any more: no wait (the partial
    // stores above retire on their own; every tile load was waited for at
    // the end of the step before).
    if (i + 1 < n_steps) {
      if constexpr (NW == 1) {
        // one wave: refill `cur` before waiting for tile i + 1, so NS tiles
        // are in flight during the wait
        lds_barrier();
        if (i + NS < n_steps) issue(cur);
        wait_vmem(n_ld * ahead(i));
        lds_barrier();
      } else {
        // several waves: one barrier per step; the refill follows it
        wait_vmem(n_ld * (ahead(i) < NS - 2 ? ahead(i) : NS - 2));
        lds_barrier();
        if (i + NS < n_steps) issue(cur);
      }
    }
  };

  // Prologue: the block's first segment (queries) and one tile per buffer.
  // Every buffer access below names its LDS array directly, so that the
  // compiler can tell the tile being read from the tiles still being written.
  if constexpr (NW == 1) {
    // One tile per buffer, then the queries; one full wait covers them all.
    // The loop is entered with no tile load in flight: a load left in flight
    // here (say tile NS - 1 streaming in during step 0) makes the compiler's
    // own LDS-write tracking put a full vector-memory wait in front of the
    // first tile read of every pass of the step loop, which drains the ring
    // at every NS-th step.
    issue(kt0);
    if (n_steps > 1) issue(kt1);
    if (NS > 2 && n_steps > 2) issue(kt2);
    if (NS > 3 && n_steps > 3) issue(kt3);
    if (NS > 4 && n_steps > 4) issue(kt4);
    begin_segment(b0, s0.grp - b0 * sc.n_rg);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
  } else {
    begin_segment(b0, s0.grp - b0 * sc.n_rg);
    issue(kt0);
    if (n_steps > 1) issue(kt1);
    if (NS > 2 && n_steps > 2) issue(kt2);
    if (NS > 3 && n_steps > 3) issue(kt3);
    if (NS > 4 && n_steps > 4) issue(kt4);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
  }
  lds_barrier();
  for (int i = 0; i < n_steps; i += NS) {
    step(i, kt0);
    if (i + 1 < n_steps) step(i + 1, kt1);
    if constexpr (NS > 2) if (i + 2 < n_steps) step(i + 2, kt2);
    if constexpr (NS > 3) if (i + 3 < n_steps) step(i + 3, kt3);
    if constexpr (NS > 4) if (i + 4 < n_steps) step(i + 4, kt4);
  }
}

// Log-sum-exp merge of one row's partials into `acc` (n values from column
// c0, n a multiple of 4): acc = sum_k w_k O_k / sum_k w_k l_k with
// w_k = 2^(m_k - max_k m_k).
template <bool P16 = false>
__device__ __forceinline__ void merge_row_partials(const AttnCore& a, int DV, int b, int row,
                                                   int c0, int n, float* acc) {
  const Schedule& sc = a.sched;
  const int n_part = sched_group_slots(sc, b * sc.n_rg + row / sc.block_rows);
  float M = -INFINITY;
  for (int k = 0; k < n_part; ++k) M = fmaxf(M, a.ml[(((size_t)k * a.B + b) * a.R + row) * 2]);
  for (int i = 0; i < n; ++i) acc[i] = 0.0f;
  float L = 0.0f;
  for (int k = 0; k < n_part; ++k) {
    const size_t prow = ((size_t)k * a.B + b) * a.R + row;
    const float wgt = exp2_fast(a.ml[prow * 2] - M);
    const float lk = a.ml[prow * 2 + 1];
    L += wgt * lk;
    const float wv = P16 ? wgt * lk : wgt;
    for (int i = 0; i < n; i += 4) {
      const f32x4 x = load_part4<P16>(a.opart, prow * DV + c0 + i);
      acc[i] += wv * x[0];
      acc[i + 1] += wv * x[1];
      acc[i + 2] += wv * x[2];
      acc[i + 3] += wv * x[3];
    }
  }
  const float inv = 1.0f / L;
  for (int i = 0; i < n; ++i) acc[i] *= inv;
}

}  // namespace mla
