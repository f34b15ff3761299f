// Host check of the kernels' index arithmetic (fa2_layout.h), compiled with
// the system C++ compiler: for every lane, pass, tile and sequence length of
// small cases, every read a tile copy makes in range must lie inside its
// tensor and fetch the chunk the LDS layout assigns to the slot it lands in,
// and every slot that must hold zeros must be read out of range (check_dma);
// every slot of a tile must be written exactly once; every MFMA operand read
// must stay inside its LDS tile.  16-byte LDS reads are also checked for bank
// conflicts, taking 16 lanes per cycle (64 banks of 4 bytes: 16 groups of 4
// banks): every group of 16 lanes of an operand read must reach 16 distinct
// groups.  Transposed operand reads (ds_read_b64_tr_b16) are simulated lane
// by lane and checked for content and banks (check_tr_reads).
// Prints "ok" and exits 0, or prints the first violation and exits 1.
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <type_traits>
#include <vector>

#include "fa2_layout.h"

using namespace fa2;

static int failures = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      if (failures++ < 10) {                               \
        std::printf("FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
        std::printf(__VA_ARGS__);                          \
        std::printf("\n");                                 \
      }                                                    \
    }                                                      \
  } while (0)

// Rows of the source tensor lie R elements apart (R = D: contiguous rows;
// R > D: a strided view such as one head of a [B, N, H, D] tensor); the
// tensor's last byte is that of row n - 1's last feature.  A tile copy reads
// a byte range that starts at the tile's first row and ends tile_bytes()
// later; a lane's read at or past that end stores zeros (the buffer range
// check).  So: every chunk of a row that exists must be read in range, from
// that row and chunk, inside the tensor; every slot of a row past the end,
// and every zero-constant slot, must be read out of range; slots of other
// constants must be left out by lane; no offset may wrap 32 bits.  Tiles
// starting at or past the end (the copies after a last step) are covered.
template <int D, int ROWS, int THREADS, class LT = RowTile<D>>
void check_dma(int max_n, int R) {
  using P = DmaPlan<D, ROWS, THREADS, LT>;
  using L = LT;
  const long row_bytes = 2L * R;
  for (int n = 1; n <= max_n; ++n) {
    for (int row0 = 0; row0 < n + ROWS; row0 += ROWS) {
      const int rows = n - row0;
      const uint64_t bytes = P::tile_bytes(rows < ROWS ? rows : ROWS, R);
      CHECK(bytes < (1ull << 31) && bytes % 16 == 0, "D=%d R=%d range %llu", D, R, (unsigned long long)bytes);
      std::vector<int> written(P::TOTAL, 0);
      for (int wave = 0; wave < THREADS / 64; ++wave) {
        for (int t = 0; t < P::ITER; ++t) {
          const int first = P::pass_slot(wave, t);
          CHECK(P::TOTAL % THREADS != 0 || first < P::TOTAL, "D=%d full plan with a missing pass", D);
          if (first >= P::TOTAL) continue;
          for (int lane = 0; lane < 64; ++lane) {
            const int slot = first + lane;
            CHECK(slot < P::TOTAL, "D=%d slot %d", D, slot);
            if (slot >= P::TOTAL) continue;
            const uint32_t off = P::stored_offset(wave, lane, P::off_index(t), R);
            const int c = L::chunk_of_slot(slot);
            if (off == P::kSkip) {   // left out by lane
              CHECK(P::SKIP_BY_LANE && c < 0, "D=%d slot %d skipped", D, slot);
              continue;
            }
            written[slot]++;
            const uint64_t total = (uint64_t)off + P::pass_offset(t, R);
            CHECK(total < (1ull << 32) && total % 16 == 0, "D=%d R=%d t=%d offset %llu", D, R, t,
                  (unsigned long long)total);
            const bool in_range = total < bytes;
            const int row = row0 + slot / L::SLOTS;
            if (c < 0) {
              CHECK(L::CONST_ZERO && !in_range, "D=%d n=%d row0=%d constant slot %d read in range", D, n, row0,
                    slot);
              continue;
            }
            if (row >= n) {
              CHECK(!in_range, "D=%d R=%d n=%d row0=%d slot %d (row %d past the end) read in range", D, R, n,
                    row0, slot, row);
              continue;
            }
            CHECK(in_range, "D=%d R=%d THREADS=%d n=%d row0=%d t=%d slot %d out of range", D, R, THREADS, n,
                  row0, t, slot);
            const long addr = (long)row0 * row_bytes + (long)total;
            const long end = (n - 1) * row_bytes + 2L * D;
            CHECK(addr + 16 <= end && addr % row_bytes + 16 <= 2L * D,
                  "D=%d R=%d n=%d row0=%d t=%d wave=%d lane=%d addr=%ld of %ld", D, R, n, row0, t, wave, lane,
                  addr, end);
            CHECK(addr / row_bytes == row && (int)((addr % row_bytes) / 16) == c,
                  "D=%d n=%d row0=%d slot=%d: row %ld chunk %ld, want %d %d", D, n, row0, slot, addr / row_bytes,
                  (addr % row_bytes) / 16, row, c);
          }
        }
      }
      for (int s = 0; s < P::TOTAL; ++s)
        CHECK(written[s] == (P::SKIP_BY_LANE && L::chunk_of_slot(s) < 0 ? 0 : 1),
              "D=%d THREADS=%d slot %d written %d times", D, THREADS, s, written[s]);
    }
  }
}

// Operand reads: row-major tiles of TOK rows are read at row[s] + 2*b*ROW16
// (b = 32-row block, s = 16-feature chunk), 8 elements.  Each read must stay
// inside its tile and fetch the features the MFMA lane layout expects, and
// each 16 lanes must reach 16 distinct bank groups.
template <int D, int TOK = 64, class L = RowTile<D>>
void check_reads() {
  using O = LaneOffsets<D, L>;
  O lanes[64];
  for (int lane = 0; lane < 64; ++lane) lanes[lane].init(lane);
  // row-major reads: bank groups of each 16 lanes
  for (int b = 0; b < TOK / 32; ++b)
    for (int s = 0; s < O::DK; ++s)
      for (int l0 = 0; l0 < 64; l0 += 16) {
        int seen[16] = {0};
        for (int lane = l0; lane < l0 + 16; ++lane) seen[(lanes[lane].rd(s, b) / 8) % 16]++;
        for (int q = 0; q < 16; ++q)
          CHECK(seen[q] <= 1, "D=%d TOK=%d row read b=%d s=%d lanes %d..: bank group %d hit %d times", D, TOK, b,
                s, l0, q, seen[q]);
      }
  for (int lane = 0; lane < 64; ++lane) {
    const O& o = lanes[lane];
    const int lr = lane & 31, lh = lane >> 5;
    for (int b = 0; b < TOK / 32; ++b)
      for (int s = 0; s < O::DK; ++s) {
        const int e = o.rd(s, b);
        CHECK(e >= 0 && e + 8 <= L::elems(TOK), "D=%d row read out of tile", D);
        CHECK(e == L::elem(32 * b + lr, 16 * s + 8 * lh), "D=%d row read of lane %d b=%d s=%d", D, lane, b, s);
      }
  }
}

// Transposed reads (ds_read_b64_tr_b16) of a TrRowTile of ROWS rows: lane j
// of 16-lane group g receives, for e = 0..3, element j % 4 of the 8 bytes
// that lane 4e + j/4 of its group addresses (the instruction's lane layout on
// gfx950).  For token chunk c, feature block mb and read rd, lane l = 32h + i
// must receive feature 32 mb + i of tokens 16c + 8rd + 4h + e (at D = 80,
// features 80..95 come from the constant slots: 1 for feature 80, else 0);
// every address must lie in the tile, 8-byte aligned; each 32-lane half must
// reach each of the 64 banks once.
template <int D, int ROWS, class L = TrRowTile<D>>
void check_tr_reads() {
  constexpr bool ONES = std::is_same<L, TrRowTile<D>>::value && L::HAS_CONST;   // (1, 0, ..) in features D..
  const int NDB = (D + 31) / 32;
  // content of every element: 1000 * (row + 1) + col for tensor data,
  // -1 / -2 for the constant one / zero elements
  std::vector<int> tile(L::elems(ROWS), -3);
  for (int r = 0; r < ROWS; ++r) {
    for (int col = 0; col < D; ++col) tile[L::elem(r, col)] = 1000 * (r + 1) + col;
    if (ONES)
      for (int col = D; col < 96; ++col) tile[L::elem(r, col)] = col == D ? -1 : -2;
  }
  for (int c = 0; c < ROWS / 16; ++c)
    for (int mb = 0; mb < NDB; ++mb)
      for (int rd = 0; rd < 2; ++rd) {
        int addr[64];
        for (int lane = 0; lane < 64; ++lane) {
          addr[lane] = tr_lane_elem<L>(lane, rd, mb) + c * L::ROWS16;
          CHECK(addr[lane] >= 0 && addr[lane] + 4 <= L::elems(ROWS) && addr[lane] % 4 == 0,
                "D=%d tr read address of lane %d c=%d mb=%d rd=%d: %d", D, lane, c, mb, rd, addr[lane]);
        }
        for (int half = 0; half < 2; ++half) {
          int banks[64] = {0};
          for (int lane = 32 * half; lane < 32 * half + 32; ++lane)
            for (int w = 0; w < 2; ++w) banks[(addr[lane] / 2 + w) % 64]++;
          for (int b = 0; b < 64; ++b)
            CHECK(banks[b] <= 1, "D=%d tr read c=%d mb=%d rd=%d half %d: bank %d hit %d times", D, c, mb, rd, half,
                  b, banks[b]);
        }
        for (int lane = 0; lane < 64; ++lane) {
          const int g = lane >> 4, j = lane & 15, h = lane >> 5, i = lane & 31;
          for (int e = 0; e < 4; ++e) {
            const int src = 16 * g + 4 * e + (j >> 2);
            const int got = tile[addr[src] + (j & 3)];
            const int row = 16 * c + 8 * rd + 4 * h + e, col = 32 * mb + i;
            const int want = col < D ? 1000 * (row + 1) + col : (ONES ? (col == D ? -1 : -2) : -4);
            if (col < D || ONES)
              CHECK(got == want, "D=%d tr read lane %d c=%d mb=%d rd=%d e=%d: got %d want %d", D, lane, c, mb, rd,
                    e, got, want);
          }
        }
      }
}

int main() {
  const int max_n = 3 * 64 + 9;
  // row pitches: contiguous rows, a [B, N, H, D] head (R = H D), the q part of a
  // fused [B, N, 3, H, D] projection (R = 3 H D), and a pitch of D + 8
  for (int mult : {1, 2, 3}) {
    check_dma<64, 64, 256>(max_n, 64 * mult);
    check_dma<80, 64, 256>(max_n, 80 * mult);
    check_dma<96, 64, 256>(max_n, 96 * mult);
    check_dma<128, 64, 256>(max_n, 128 * mult);
    check_dma<64, 64, 512>(max_n, 64 * mult);
    check_dma<80, 64, 512>(max_n, 80 * mult);
    check_dma<96, 64, 512>(max_n, 96 * mult);
    check_dma<128, 64, 512>(max_n, 128 * mult);
    check_dma<64, 64, 768>(max_n, 64 * mult);
    check_dma<64, 128, 512>(max_n, 64 * mult);
    check_dma<96, 128, 768>(max_n, 96 * mult);
    check_dma<128, 128, 512>(max_n, 128 * mult);
    check_dma<80, 64, 768>(max_n, 80 * mult);
    check_dma<96, 64, 768>(max_n, 96 * mult);
    check_dma<128, 64, 768>(max_n, 128 * mult);
  }
  check_dma<128, 64, 256>(max_n, 136);
  check_dma<80, 64, 512>(max_n, 88);
  // 32-row tiles (the dQ kernel's key tile can be 32 keys for D = 64 and 128)
  for (int mult : {1, 3}) {
    check_dma<64, 32, 512>(max_n, 64 * mult);
    check_dma<128, 32, 512>(max_n, 128 * mult);
  }
  // head dim 256: 64-key K (forward, dQ) and V (dQ) tiles, 256 threads
  for (int mult : {1, 2, 3}) {
    check_dma<256, 64, 256>(max_n, 256 * mult);
  }
  check_dma<256, 64, 256>(max_n, 264);
  // V tiles of the forward (TrRowTile): the thread counts of its workgroups
  for (int mult : {1, 2, 3}) {
    check_dma<64, 64, 512, TrRowTile<64>>(max_n, 64 * mult);
    check_dma<64, 128, 512, TrRowTile<64>>(max_n, 64 * mult);
    check_dma<80, 64, 256, TrRowTile<80>>(max_n, 80 * mult);
    check_dma<96, 64, 768, TrRowTile<96>>(max_n, 96 * mult);
    check_dma<128, 64, 512, TrRowTile<128>>(max_n, 128 * mult);
    check_dma<256, 64, 256, TrRowTile<256>>(max_n, 256 * mult);
  }
  check_dma<256, 64, 256, TrRowTile<256>>(max_n, 264);
  check_dma<80, 64, 256, TrRowTile<80>>(max_n, 88);
  check_tr_reads<64, 64>();
  check_tr_reads<64, 128>();
  check_tr_reads<80, 64>();
  check_tr_reads<96, 64>();
  check_tr_reads<128, 64>();
  check_tr_reads<256, 64>();
  // Q and dO tiles of the dK/dV pass (copied, read row-wise and transposed)
  for (int mult : {1, 2, 3}) {
    check_dma<64, 64, 256, RowTile<64>>(max_n, 64 * mult);
    check_dma<80, 64, 256, WideRowTile<80>>(max_n, 80 * mult);
    check_dma<96, 64, 256, WideRowTile<96>>(max_n, 96 * mult);
    check_dma<128, 64, 256, RowTile<128>>(max_n, 128 * mult);
  }
  check_dma<80, 64, 256, WideRowTile<80>>(max_n, 88);
  // K and V tiles of the dQ pass (eight wavefronts)
  for (int mult : {1, 2, 3}) {
    check_dma<80, 64, 512, WideRowTile<80>>(max_n, 80 * mult);
    check_dma<96, 64, 512, WideRowTile<96>>(max_n, 96 * mult);
  }
  check_reads<80, 64, WideRowTile<80>>();
  check_reads<96, 64, WideRowTile<96>>();
  check_tr_reads<64, 64, RowTile<64>>();
  check_tr_reads<80, 64, WideRowTile<80>>();
  check_tr_reads<96, 64, WideRowTile<96>>();
  check_tr_reads<128, 64, RowTile<128>>();
  // Q and dO tiles of the head-dim-256 dK/dV pass (64 rows, four wavefronts)
  check_dma<256, 64, 256, RowTile<256>>(max_n, 256);
  check_dma<256, 64, 256, RowTile<256>>(max_n, 264);
  check_dma<256, 64, 256, RowTile<256>>(max_n, 768);
  // the largest row pitch the API accepts (2^20 elements): no offset wraps
  check_dma<128, 64, 256>(70, 1 << 20);
  check_dma<64, 128, 512>(140, 1 << 20);
  check_dma<96, 64, 256, WideRowTile<96>>(70, 1 << 20);
  check_dma<256, 64, 256, RowTile<256>>(70, 1 << 20);
  check_reads<256, 64, RowTile<256>>();
  check_tr_reads<256, 64, RowTile<256>>();
  check_reads<256, 32>();
  check_reads<64, 32>();
  check_reads<128, 32>();
  check_reads<64>();
  check_reads<80>();
  check_reads<96>();
  check_reads<128>();
  if (failures) {
    std::printf("%d violations\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
