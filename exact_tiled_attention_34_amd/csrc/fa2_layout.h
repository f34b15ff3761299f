// Index arithmetic of the attention kernels: LDS tile layouts, and which
// global bytes each lane moves into which LDS slot.
//
// Everything here is plain integer arithmetic, compiled both into the kernels
// (through fa2_device.h) and into a host program that enumerates every lane,
// pass, tile and sequence length of small cases and checks that every global
// address stays inside its tensor and every LDS slot receives the chunk the
// layout assigns to it.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FA2_HD __host__ __device__ __forceinline__
#else
#define FA2_HD inline
#endif

namespace fa2 {

// ---------------------------------------------------------------------------
// Row-major tiles in LDS.
//
// A tile holds ROWS token rows of D bf16 features, in 16-byte chunks.  The
// chunk order inside a row is permuted per row so that 16-byte reads of one
// chunk by 32 consecutive rows (the MFMA operands whose reduction index is
// the feature: Q K^T, dO V^T, K Q^T, V dO^T) spread over the LDS banks.
// D = 256 (32 chunks), D = 128 (16 chunks) and D = 64 (8 chunks) use an XOR
// of the chunk index (at D = 256 of its low four bits); D = 80 (10 chunks) and
// D = 96 (12 chunks) pad every row by one chunk slot instead (11 and 13 slots:
// 176- and 208-byte rows, whose first 16 rows start on 16 distinct 4-bank
// groups).
// ---------------------------------------------------------------------------
template <int D>
struct RowTile {
  static constexpr int CH = D / 8;
  static constexpr bool PADDED = (CH & (CH - 1)) != 0;
  static constexpr int SLOTS = PADDED ? CH + 1 : CH;
  static constexpr bool HAS_CONST = false;        // every slot is copied from the tensor
  static constexpr bool CONST_ZERO = false;
  static_assert(D % 16 == 0 && (PADDED || CH == 8 || CH == 16 || CH == 32), "unsupported head dim");

  // XOR key of a row (an involution on the chunk index); depends on row % 16.
  static FA2_HD int swz(int row) {
    if constexpr (PADDED) {
      return 0;
    } else if constexpr (CH >= 16) {
      return (4 * (row & 3)) | ((row >> 2) & 3);
    } else {
      const int g = (row >> 1) & 7;
      return (4 * (g & 1)) | (g >> 1);
    }
  }
  // 16-byte slot index of (row, chunk) inside the tile.
  static FA2_HD int slot(int row, int chunk) {
    return row * SLOTS + (PADDED ? chunk : (chunk ^ swz(row)));
  }
  // bf16 element offset of (row, col); col % 4 == 0.
  static FA2_HD int elem(int row, int col) { return slot(row, col >> 3) * 8 + (col & 7); }
  // Logical chunk stored in slot s (the pad slot of a padded row holds chunk 0).
  static FA2_HD int chunk_of_slot(int s) {
    const int row = s / SLOTS;
    const int c = s % SLOTS;
    if constexpr (PADDED) return c >= CH ? 0 : c;
    return c ^ swz(row);
  }
  // bf16 elements to reserve for a tile.
  static constexpr int elems(int rows) { return rows * SLOTS * 8; }
  // Elements per 16 rows (the period of the swizzle).
  static constexpr int ROWS16 = 16 * SLOTS * 8;
  // Row lr + 32 b, features 16 s + 8 h: the lane's block-0 offset for step
  // perm(s, b) (= s: the permutation repeats every 16 rows) plus block(b).
  static constexpr int perm(int s, int) { return s; }
  static constexpr int block(int b) { return b * 32 * SLOTS * 8; }
};

// ---------------------------------------------------------------------------
// Row-major tiles read transposed.
//
// ds_read_b64_tr_b16 (gfx950) reads 8 bytes per lane and transposes them
// within each group of 16 lanes: lane j of a group receives, for e = 0..3,
// 16-bit element j % 4 of the 8 bytes addressed by lane 4 e + j / 4 of its
// group.  So when lane 4 e + r of group g addresses row T0(g) + e, columns
// F0(g) + 4 r .. + 3 of a row-major tile, lane j receives column F0(g) + j of
// rows T0(g) .. T0(g) + 3.  Two such reads give the 8 tokens of an MFMA
// operand whose reduction index is the token (V^T, K^T, Q^T, dO^T): for the
// 16-token chunk c, feature block mb and read rd, group g addresses rows
// 16 c + 8 rd + 4 (g / 2) + e and columns 32 mb + 16 (g % 2) + 4 r, so lane
// l = 32 h + i receives feature 32 mb + i of tokens 16 c + 8 rd + 4 h + e:
// the tokens {4h..4h+3, 8+4h..8+4h+3} of an accumulator's lane half.
//
// Layouts, chosen so that each 32-lane half of such a read touches every
// LDS bank once (checked on the host): at D = 64, 128 and 256 the RowTile
// itself (its XOR swizzle); at D = 80 and 96 plain 12-slot rows (192 bytes).
// At D = 80 slots 10 and 11 of every row are not copied from the tensor:
// they hold features 80..95 of the padded feature blocks, set once to
// (1, 0, .., 0) and zeros, so that a product with the transposed tile also
// yields the sum of the other operand over its tokens (feature row 80).
// ---------------------------------------------------------------------------
template <int D>
struct TrRowTile {
  static constexpr int CH = D / 8;
  static constexpr bool LINEAR = D == 80 || D == 96;
  static constexpr bool PADDED = LINEAR;          // not a 16-row XOR period (DmaPlan)
  static constexpr int SLOTS = LINEAR ? 12 : CH;
  static constexpr bool HAS_CONST = D == 80;     // slots 10 and 11 are constant
  static constexpr bool CONST_ZERO = false;      // slot 10 is not zero
  static_assert(LINEAR || D == 64 || D == 128 || D == 256, "unsupported head dim");

  static FA2_HD int slot(int row, int chunk) {
    if constexpr (LINEAR) return row * SLOTS + chunk;
    else return RowTile<D>::slot(row, chunk);
  }
  static FA2_HD int elem(int row, int col) { return slot(row, col >> 3) * 8 + (col & 7); }
  // Chunk of the tensor row stored in slot s; -1 for a constant slot.
  static FA2_HD int chunk_of_slot(int s) {
    if constexpr (LINEAR) {
      const int c = s % SLOTS;
      return c < CH ? c : -1;
    } else {
      return RowTile<D>::chunk_of_slot(s);
    }
  }
  static constexpr int elems(int rows) { return rows * SLOTS * 8; }
  // Elements between 16-row groups: the swizzle repeats every 16 rows, so the
  // token chunk c of a read adds c * ROWS16.
  static constexpr int ROWS16 = 16 * SLOTS * 8;
};

// Element offset, in a tile of layout L, of the 8 bytes that lane `lane`
// addresses in transposed read rd of feature block mb, token chunk 0 (the
// token chunk c adds c * L::ROWS16).
template <class L>
FA2_HD int tr_lane_elem(int lane, int rd, int mb) {
  const int g = (lane >> 4) & 3, e = (lane >> 2) & 3, r = lane & 3;
  return L::elem(8 * rd + 4 * (g >> 1) + e, 32 * mb + 16 * (g & 1) + 4 * r);
}

// ---------------------------------------------------------------------------
// D = 80 and 96 features in 128-feature rows: the RowTile<128> layout (whose
// swizzle suits both 16-byte row reads and transposed reads), of which only
// the first D / 8 chunks of each row are copied from the tensor; the other
// slots (chunk -1 for the copy plan) hold zeros, which every copy stores
// (DmaPlan::stored_offset), and feed only padding rows of the feature blocks.
// ---------------------------------------------------------------------------
template <int D>
struct WideRowTile {
  using W = RowTile<128>;
  static constexpr int CH = 16;                  // chunk slots per row
  static constexpr int DCH = D / 8;              // chunks copied from the tensor
  static constexpr bool PADDED = false;
  static constexpr int SLOTS = 16;
  static constexpr bool HAS_CONST = DCH < 16;
  static constexpr bool CONST_ZERO = true;       // the constant slots hold zeros
  static_assert(D == 80 || D == 96, "wide rows for D = 80, 96");
  static FA2_HD int slot(int row, int chunk) { return W::slot(row, chunk); }
  static FA2_HD int elem(int row, int col) { return W::elem(row, col); }
  static FA2_HD int chunk_of_slot(int s) {
    const int c = W::chunk_of_slot(s);
    return c < DCH ? c : -1;
  }
  static constexpr int elems(int rows) { return W::elems(rows); }
  static constexpr int ROWS16 = 16 * SLOTS * 8;
  static constexpr int perm(int s, int b) { return W::perm(s, b); }
  static constexpr int block(int b) { return W::block(b); }
};

// ---------------------------------------------------------------------------
// Direct global -> LDS copy of a RowTile of ROWS rows by THREADS threads.
//
// Pass t moves slots [t*THREADS, (t+1)*THREADS); wavefront w's 64 lanes move
// the 64 consecutive slots starting at w*64 + t*THREADS (a load into LDS
// writes lane l's 16 bytes at its wavefront base + 16 l).  Rows of the source
// tensor lie R elements apart (R >= D, a multiple of 8: the row pitch, D for a
// contiguous [.., N, D] tensor).  The chunk swizzle repeats every 16 rows, so
// when a pass spans whole rows and PERIOD passes span a multiple of 16 rows
// (PERIODIC) a lane's source offset in pass t is that of pass t % PERIOD moved
// by whole rows, and PERIOD registers hold every offset (one at D = 64 and
// 128 with 256 or more threads; two at D = 256 with 256 threads, whose passes
// span 8 rows).
// ---------------------------------------------------------------------------
template <int D, int ROWS, int THREADS, class LT = RowTile<D>>
struct DmaPlan {
  using L = LT;
  static constexpr int TOTAL = ROWS * L::SLOTS;   // 16-byte slots per tile
  static constexpr int ITER = (TOTAL + THREADS - 1) / THREADS;
  static constexpr int RPP = THREADS / L::SLOTS;  // rows per pass (PERIODIC only)
  static constexpr bool PERIODIC =
      !L::PADDED && THREADS % L::SLOTS == 0 && RPP > 0 && (RPP % 16 == 0 || 16 % RPP == 0);
  static constexpr int PERIOD = !PERIODIC ? 1 : RPP % 16 == 0 ? 1 : 16 / RPP;   // passes
  static constexpr int NOFF = PERIODIC ? (PERIOD < ITER ? PERIOD : ITER) : ITER;
  static_assert(TOTAL % 64 == 0 && THREADS % 64 == 0, "whole wavefronts per pass");

  // First slot of pass t for wavefront `wave` (uniform); the pass exists for
  // that wavefront iff the result is < TOTAL.
  static FA2_HD int pass_slot(int wave, int t) { return wave * 64 + t * THREADS; }
  // Which stored offset serves pass t, and the first pass of its period.
  static FA2_HD int off_index(int t) { return PERIODIC ? t % PERIOD : t; }
  static FA2_HD int period_start(int t) { return PERIODIC ? t - t % PERIOD : 0; }

  // Row (from the first row of the tile) and byte offset of the source chunk
  // of lane `lane` in pass t, stored once per lane (t < NOFF).  A slot that
  // the layout keeps constant (chunk -1) is not copied: its offset is kSkip.
  static constexpr uint32_t kSkip = 0xFFFFFFFFu;
  static FA2_HD int lane_row(int wave, int lane, int t) { return (pass_slot(wave, t) + lane) / L::SLOTS; }
  static FA2_HD uint32_t lane_offset(int wave, int lane, int t, int R) {
    const int s = pass_slot(wave, t) + lane;
    const int c = L::chunk_of_slot(s);
    if constexpr (L::HAS_CONST) {
      if (c < 0) return kSkip;
    }
    return (uint32_t)((s / L::SLOTS) * R + c * 8) * 2u;
  }

  // The offset a copy stores for lane `lane` of pass t (t < NOFF): that of
  // its chunk, or for a constant slot kOutOfRange (past any tile, so the slot
  // is stored as zeros) when the layout's constants are zeros, else kSkip
  // (the lane does not load).
  static constexpr uint32_t kOutOfRange = 0x80000000u;
  static constexpr bool SKIP_BY_LANE = L::HAS_CONST && !L::CONST_ZERO;
  static FA2_HD uint32_t stored_offset(int wave, int lane, int t, int R) {
    const uint32_t o = lane_offset(wave, lane, t, R);
    return (o == kSkip && !SKIP_BY_LANE) ? kOutOfRange : o;
  }
  // The copy of a tile reads a byte range that starts at the tile's first
  // row: pass t of a lane reads the 16 bytes at lane_offset(off_index(t)) +
  // pass_offset(t) of it, and a read at or past tile_bytes() returns zeros.
  // Bytes between the stored pass off_index(t) and pass t:
  static FA2_HD uint32_t pass_offset(int t, int R) {
    return PERIODIC ? (uint32_t)(period_start(t) * RPP) * (uint32_t)R * 2u : 0u;
  }
  // Bytes of the range of a tile of which `rows` rows exist (0 .. ROWS): up
  // to the last feature of its last row.
  static FA2_HD uint32_t tile_bytes(int rows, int R) {
    return rows <= 0 ? 0u : (uint32_t)(rows - 1) * (uint32_t)R * 2u + (uint32_t)D * 2u;
  }
};

// Per-lane LDS element offsets of the row-major operand reads, computed once
// per kernel for the lane's row in the first 32-row block; the reads of other
// blocks and feature steps (L::perm, L::block) differ by compile-time
// constants: every such read in the hot loops is one precomputed register
// plus an immediate offset.
template <int D, class L = RowTile<D>>
struct LaneOffsets {
  static constexpr int DK = D / 16;
  static constexpr int NDB = (D + 31) / 32;
  // feature steps of the layout's rows (more than DK when D features are
  // stored in wider rows: L::perm may then name a step past DK)
  static constexpr int NROW = L::CH / 2;
  int row[NROW];   // row-major tile: features 16 s + 8 h .. +7 of row lane % 32
  FA2_HD void init(int lane) {
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int s = 0; s < NROW; ++s) row[s] = L::elem(lr, s * 16 + 8 * lh);
  }
  // row-major read of 32-row block b, feature step s
  FA2_HD int rd(int s, int b) const { return row[L::perm(s, b)] + L::block(b); }
};

}  // namespace fa2
