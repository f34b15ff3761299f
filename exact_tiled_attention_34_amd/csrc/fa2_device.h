// Device helpers for the gfx950 (CDNA4) attention kernels: MFMA wrappers,
// bf16 packing, fast exp2/log2, the LDS tile layout, asynchronous
// global->LDS tile loads and the two ways MFMA operands are read from LDS.
//
// MFMA lane layout (v_mfma_f32_32x32x16_bf16, one 64-lane wavefront):
//   A (32 x 16): lane l holds A[l % 32][8*(l/32) + j],  j = 0..7
//   B (16 x 32): lane l holds B[8*(l/32) + j][l % 32],  j = 0..7
//   C (32 x 32): lane l, register i holds C[8*(i/4) + 4*(l/32) + (i%4)][l % 32]
// so every lane owns one column of C and 16 of its rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> one word of two bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Exchange with the lane 32 positions away (the other half of the wavefront).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// Wait until this wavefront's outstanding vector-memory loads (including
// global->LDS loads) have completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Row-major tiles in LDS.
//
// A tile holds ROWS token rows of D bf16 features, in 16-byte chunks.  The
// chunk order inside a row is permuted per row so that both access patterns
// used by the kernels spread over the LDS banks:
//   (a) 16-byte reads of one chunk by 32 consecutive rows (MFMA operands
//       whose reduction index is the feature: Q K^T, dO V^T), and
//   (b) transposed reads of 8 rows x 4 chunks (operands whose reduction
//       index is the token: V^T, dO^T, Q^T, K^T).
// D = 128 (16 chunks) and D = 64 (8 chunks) use an XOR of the chunk index;
// D = 80 (10 chunks) pads every row to 11 chunk slots instead.
// ---------------------------------------------------------------------------
template <int D>
struct RowTile {
  static constexpr int CH = D / 8;
  static constexpr bool PADDED = (CH & (CH - 1)) != 0;
  static constexpr int SLOTS = PADDED ? CH + 1 : CH;
  static_assert(D % 16 == 0 && (PADDED || CH == 8 || CH == 16), "unsupported head dim");

  // XOR key of a row (an involution on the chunk index).
  __device__ __forceinline__ static int swz(int row) {
    if constexpr (PADDED) {
      return 0;
    } else if constexpr (CH == 16) {
      return (4 * (row & 3)) | ((row >> 2) & 3);
    } else {
      const int g = (row >> 1) & 7;
      return (4 * (g & 1)) | (g >> 1);
    }
  }
  // 16-byte slot index of (row, chunk) inside the tile.
  __device__ __forceinline__ static int slot(int row, int chunk) {
    return row * SLOTS + (PADDED ? chunk : (chunk ^ swz(row)));
  }
  // bf16 element offset of (row, col); col % 4 == 0.
  __device__ __forceinline__ static int elem(int row, int col) {
    return slot(row, col >> 3) * 8 + (col & 7);
  }
  // bf16 elements to reserve for a tile (transposed reads of the padded
  // feature block of D = 80 may run 8 elements past the last row).
  static constexpr int elems(int rows) { return rows * SLOTS * 8 + (PADDED ? 16 : 0); }
};

// One 16-byte global -> LDS load per lane.  `lds` must be the same for every
// lane of the wavefront; lane l's 16 bytes land at lds + 16*l bytes.
__device__ __forceinline__ void global_load_lds16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}

// Start loading rows [row0, row0 + ROWS) of one head (row-major, D features)
// into a RowTile in LDS.  Rows past n_rows are clamped to the last row (finite
// data that the caller masks or weights by zero).  Returns immediately;
// wait_vmem() + a workgroup barrier make the tile visible.
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void load_tile_async(uint16_t* tile, const uint16_t* head, int row0,
                                                int n_rows, int tid) {
  using L = RowTile<D>;
  constexpr int TOTAL = ROWS * L::SLOTS;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
#pragma unroll
  for (int t = 0; t < (TOTAL + THREADS - 1) / THREADS; ++t) {
    const int base = wave * 64 + t * THREADS;   // wavefront-uniform
    if (base >= TOTAL) break;
    const int s = base + lane;
    const int row = s / L::SLOTS;
    int chunk = s % L::SLOTS;
    if (L::PADDED) {
      if (chunk >= L::CH) chunk = 0;   // the pad slot gets a copy of chunk 0
    } else {
      chunk ^= L::swz(row);
    }
    const int grow = min(row0 + row, n_rows - 1);
    if (s < TOTAL) global_load_lds16(head + (size_t)grow * D + chunk * 8, tile + base * 8);
  }
}

// MFMA operand whose reduction index is the feature: lane l gets 8
// consecutive features [col, col+8) of tile row `row` (16-byte read).
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* tile, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(tile + RowTile<D>::elem(row, col));
}

// MFMA operand whose reduction index is the token: the transpose of a
// 16-token x 32-feature block starting at (tok0, col0).  Lane l gets feature
// col0 + l%32 and, in its 8 k-slots, tokens tok0 + 4h + {0..3} then
// tok0 + 8 + 4h + {0..3} (h = l/32) — the same token order in which an MFMA
// accumulator holds its rows, so a P or dS accumulator feeds the other
// operand directly.  Two ds_read_b64_tr_b16: inside each 16-lane group the
// instruction hands lane i element i%4 of source lane 4j + i/4 as its j-th
// value; source lane s therefore points at row base + s/4, features 4(s%4)+.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int tok0, int col0, int lane) {
  i16x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
  const int s = lane & 15;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  const int row = tok0 + 4 * (lane >> 5) + (s >> 2);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((lds_u16*)tile + RowTile<D>::elem(row, col)));
  hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((lds_u16*)tile + RowTile<D>::elem(row + 8, col)));
#else
  (void)tile; (void)tok0; (void)col0; (void)lane;
#endif
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// Transposed tiles in LDS.
//
// Operands whose reduction index is the token (V^T, K^T, Q^T, dO^T) need 8
// consecutive tokens per lane, i.e. a column of the row-major tile.  A
// transposed read instruction exists but costs several times a 16-byte read,
// so these tiles are transposed once, while being staged: each thread loads
// a 4-token x 8-feature block into registers, permutes it with v_perm into 8
// feature rows of 4 tokens and writes those (8 bytes each).  Feature rows hold
// 64 tokens (+ 8 elements of padding: rows 144 bytes apart, so 16 consecutive
// rows cover all 64 banks).  Inside each group of 16 tokens the middle two
// groups of four are swapped: an MFMA accumulator holds, in lane half h, the
// tokens {4h..4h+3, 8+4h..8+4h+3}, which then lie side by side, so the
// operand is one 16-byte read and P or dS feeds the other operand directly.
// Feature rows at or past D (the 80 -> 96 padding) stay zero.
// ---------------------------------------------------------------------------
template <int D, int TOK = 64>
struct TrTile {
  static_assert(TOK == 32 || TOK == 64, "tokens per transposed tile");
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int ROW = TOK + 8;                // bf16 per feature row
  static constexpr int ELEMS = DP * ROW;
  __device__ __forceinline__ static int pos(int tok) {   // swap groups 1 and 2 of each 16
    const int g = (tok >> 2) & 3;
    return (tok & ~15) | ((g == 1 ? 2 : g == 2 ? 1 : g) << 2) | (tok & 3);
  }
  __device__ __forceinline__ static int elem(int row, int tok) { return row * ROW + pos(tok); }
  // zero the padding rows [D, DP) (once; staging never writes them)
  __device__ __forceinline__ static void zero_pad(uint16_t* t, int tid, int nthreads) {
    if constexpr (DP != D)
      for (int i = tid; i < (DP - D) * ROW; i += nthreads) t[D * ROW + i] = 0;
  }
};

// Stager of one transposed tile of TOK tokens: load() issues the global loads
// into registers, store() (after the values are needed, typically once the
// current tile's compute is done) writes the transposed tile.  Thread t
// handles tokens 4(t%G)..+3 and features 8(t/G)..+7, G = TOK/4.
template <int D, int TOK = 64>
struct TrStage {
  static constexpr int CH = D / 8;
  static constexpr int G = TOK / 4;
  u32x4 r[4];
  __device__ __forceinline__ bool active(int tid) const { return tid < G * CH; }
  __device__ __forceinline__ void load(const uint16_t* head, int tok0, int n_rows, int tid) {
    if (!active(tid)) return;
    const int g = tid % G, ch = tid / G;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = min(tok0 + 4 * g + k, n_rows - 1);
      r[k] = ld_global16(head + (size_t)row * D + ch * 8);
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
    if (!active(tid)) return;
    const int g = tid % G, ch = tid / G;
    uint16_t* dst = tile + TrTile<D, TOK>::elem(8 * ch, 4 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      // feature 8 ch + e of tokens 4g..4g+3: low or high halves of word w
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2 out;
      out[0] = __builtin_amdgcn_perm(r[1][w], r[0][w], sel);
      out[1] = __builtin_amdgcn_perm(r[3][w], r[2][w], sel);
      *reinterpret_cast<u32x2*>(dst + e * TrTile<D, TOK>::ROW) = out;
    }
  }
};

// Per-lane LDS element offsets of the two operand reads, computed once per
// kernel.  The chunk permutation of a RowTile depends only on row % 16, so
// moving by whole 16-row groups (32-row operand blocks, 16-token chunks) adds
// a compile-time constant: every read in the hot loops is one precomputed
// register plus an immediate offset.
template <int D, int TOK = 64>
struct LaneOffsets {
  static constexpr int DK = D / 16;
  static constexpr int NDB = (D + 31) / 32;
  static constexpr int ROW16 = 16 * RowTile<D>::SLOTS * 8;   // elements per 16 rows
  static constexpr int TR32 = 32 * TrTile<D, TOK>::ROW;     // elements per 32 feature rows
  int row[DK];   // row-major tile: features 16 s + 8 h .. +7 of row lane % 32
  int tr;        // transposed tile: tokens {4h..4h+3, 8+4h..8+4h+3} of feature row lane % 32
  __device__ __forceinline__ void init(int lane) {
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int s = 0; s < DK; ++s) row[s] = RowTile<D>::elem(lr, s * 16 + 8 * lh);
    tr = lr * TrTile<D, TOK>::ROW + 8 * lh;   // + 16 c (token chunk) + TR32 mb (feature block)
  }
};

__device__ __forceinline__ bf16x8 lds_read16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposed operand from two precomputed addresses (see tr_operand).
__device__ __forceinline__ bf16x8 lds_read_tr(const uint16_t* lo_p, const uint16_t* hi_p) {
  i16x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const __attribute__((address_space(3))) uint16_t*)lo_p);
  hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const __attribute__((address_space(3))) uint16_t*)hi_p);
#else
  (void)lo_p; (void)hi_p;
#endif
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// bf16x8 B operand for 16 tokens (chunk c of a 32-row accumulator pair) from
// packed accumulator words w[0..7] (w[t] = rows 2t, 2t+1 of the accumulator).
__device__ __forceinline__ bf16x8 acc_chunk(const uint32_t* w, int half) {
  const u32x4 v = {w[4 * half + 0], w[4 * half + 1], w[4 * half + 2], w[4 * half + 3]};
  return as_bf16x8(v);
}

}  // namespace fa2
