// Forward pass of exact tiled attention on gfx950: O and the row logsumexp L.
//
// Work split ("FlashAttention-2" summary page, "How It Works" 1; glossary page
// "FlashAttention (v2)" on splitting a head along the sequence): one workgroup
// per (query row-block, batch*head).  Inside the workgroup each wavefront owns
// 32 query rows outright, so row maxima and sums never leave the wavefront
// (glossary page: warps re-partitioned to exchange less through shared memory).
//
// Per wavefront and K/V tile (64 keys):
//   S^T = K Q^T            bf16 MFMA 32x32x16; lane l then holds query l%32 and
//                          16 of the 64 keys, so the row max/sum is an in-lane
//                          reduction plus one exchange with lane l^32
//   causal / tail mask     only tiles crossing the diagonal or the end of the
//                          sequence are masked; tiles wholly above the diagonal
//                          are never visited ("FlashAttention-2: Faster
//                          Attention with Better Parallelism and Work
//                          Partitioning" page, closing sentence)
//   online softmax         m' = max(m, rowmax S); P = 2^(c S - c m'),
//                          c = scale*log2(e); l = 2^(c(m-m')) l + rowsum P;
//                          O *= 2^(c(m-m')).  The rescale of O is skipped for
//                          the whole wavefront when no row's max grew in this
//                          tile (then every factor is exactly 1), which after
//                          the first tiles is the common case
//                          ("FlashAttention-2" summary page, "How It Works" 2:
//                          scaling kept out of the inner loop).  The maximum
//                          pass itself is skipped while every P against the
//                          current m stays <= 2^8.
//   O^T += V^T P^T         bf16 MFMA; V^T is a transposed LDS tile, P^T comes
//                          straight from registers
// After the last tile, O is divided once by the row sum of P as rounded for
// the product ("FlashAttention-2" summary page, "How It Works" 2) and
// L = (c m + log2 l) ln 2 is stored.
//
// K and V tiles go global -> LDS directly (no registers), both row-major; the
// P V product reads V^T with transposing LDS reads.  Tiles are staged in
// stages of one or two tiles, double-buffered: the copies of stage J+1 are
// issued right after the barrier that opens stage J.
#include <type_traits>

#include "fa2_device.h"
#include "fa2_launch.h"


namespace fa2 {
namespace {

// Wavefronts per workgroup and workgroups per CU, chosen by timing on MI355X:
// a large workgroup (8 wavefronts at D = 64 and 128, 12 at D = 96) shares each
// staged K/V tile among more query rows; one per CU at D = 96 and 128, two at
// D = 64 (four wavefronts per SIMD in 124 VGPRs); at D = 80 two workgroups of
// 4 wavefronts are as fast as 12 wavefronts and 5 % faster than 8.  At D = 256
// a wavefront's Q operands (64 registers) and O accumulators (128) leave room
// for one wavefront per SIMD only: 4 wavefronts.  Its 64-key K and V tiles
// take 128 KiB of LDS double-buffered; against 32-key tiles, whose score
// products were one dependent chain of MFMAs per tile, B1 H16 N8192 d256
// causal forward -4.5 % on MI355X.
template <int D, bool CAUSAL = false>
struct FwdCfg {
  static constexpr int WAVES = D == 96 ? 12 : D == 80 || D == 256 ? 4 : 8;
  static constexpr int WGS_PER_CU = D == 64 || D == 80 ? 2 : 1;
  static constexpr int WAVES_PER_SIMD = WAVES * WGS_PER_CU / 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BR = 32 * WAVES;           // query rows per workgroup
  static constexpr int BC = 64;                   // keys per K/V tile
  static constexpr int KB = BC / 32;              // 32-key MFMA blocks per tile
  static constexpr int DP = (D + 31) / 32 * 32;   // O^T rows padded to whole 32-row MFMA blocks
  static constexpr int NDB = DP / 32;
  static constexpr int DK = D / 16;               // k-steps of K Q^T
  // Tiles per stage: a stage of SUB tiles is copied together and opened by one
  // workgroup barrier (half the barriers at SUB = 2).  Two at D = 64, where it also keeps
  // the non-causal kernel within 128 VGPRs (B8 H16 N2048 d64: -12 %; B4 H32
  // N4096 d64 causal: -1 %); at D = 96 and 128 it measured even or slower
  // (B1 H16 N16384 d128 causal: +1.5 %).
  static constexpr int SUB = D == 64 && !CAUSAL ? 2 : 1;
  static constexpr int STAGE = SUB * BC;          // keys per stage
  static constexpr int TILE = RowTile<D>::elems(STAGE);
  // V tiles: copied row-major like K and read transposed by the P V product
  // (TrRowTile).  Against staging them transposed through registers, which
  // competes with the softmax for the vector unit: forward B4 H32 N4096 d64
  // causal -4 %, B2 H32 N8192 d80 causal and B2 H24 N8192 d96 causal -2 %,
  // B1 H16 N16384 d128 causal -1.6 %, B8 H16 N2048 d128 -2.5 %, B1 H16 N8192
  // d256 causal -3 % (MI355X).
  using VL = TrRowTile<D>;
  static constexpr int VTILE = VL::elems(STAGE);
  // LDS operand reads kept in flight ahead of the MFMAs (the scheduling hint
  // of the P V products); fewer at D = 96, whose three wavefronts per SIMD
  // have 170 registers each
  static constexpr int READ_AHEAD = D == 96 ? 4 : 6;
  // stages of the S^T products whose K operands are read ahead (scores())
  static constexpr int SCORE_PF = 2;
  // D = 256: the Q operands (64 registers) sit in accumulator registers, as
  // MFMA B operands may, which leaves the vector registers room for operand
  // reads in flight (one wavefront per SIMD: nothing else hides them)
  static constexpr bool Q_IN_AGPR = D == 256;
  // When V^T is padded to whole 32-feature blocks (D = 80), its first padding
  // row holds ones: O^T row D then accumulates the row sum of the rounded P
  // (scaled with O by every rescale), at no cost, instead of a sum in the
  // vector unit.  That row sits in accumulator block D / 32, register
  // ONES_REG, of the lanes of half ONES_HALF.
  static constexpr bool ONES_ROW = DP != D;
  // The softmax step first tries P against the current reference maximum
  // (no maximum pass); the scores stay live until it knows whether the
  // maximum pass is due.  Forward time on MI355X: B1 H16 N16384 d128 causal
  // -7 %, B8 H16 N2048 d128 -7 %, B1 H16 N8192 d256 causal -19 %,
  // B4 H32 N4096 d64 causal -7 %.
  static constexpr bool LAZY = true;
  // With the lazy maximum, one softmax step per 32-key block instead of one
  // per tile, so that the exponentials of block 1 can run under the products
  // of block 0: B2 H32 N8192 d80 causal -6 %, B2 H24 N8192 d96 causal -5 %,
  // but B1 H16 N16384 d128 causal +6 %.  At D = 64 (four wavefronts per SIMD,
  // 128 registers) and 96 the whole-tile step spills.
  static constexpr bool BLOCK_STEPS = LAZY && KB == 2 && (D == 64 || D == 80 || D == 96);
  static constexpr int ONES_REG = 4 * ((D % 32) / 8) + D % 4;
  static constexpr int ONES_HALF = (D % 8) / 4;
};

// Bound on a lane's share of a row's P sum above which the softmax step moves
// the row's reference maximum (so every P stays at most 2^8).
constexpr float kLazyBound = 256.f;

template <int D, bool CAUSAL, class E>
struct FwdWave {
  using C = FwdCfg<D, CAUSAL>;
  u32x4 qf[C::DK];
  f32x16 oacc[C::NDB];
  f32x16 sc[1][C::KB];  // scores of the current tile
  // running max, running sum of P (for L) and running sum of P as rounded to
  // the storage type (the weights the P V product actually uses: O is divided
  // by this sum, so its rows are exact convex combinations of V's rows)
  float m_run, l_run, lr_run;
  int lane, lr, lh, q_wave, q_lane;
  int key_last;        // causal: last key this lane's query may see (q_lane + Nk - Nq)
  int key_last_wave;   // the same for the wavefront's last query row
  LaneOffsets<D> off;
  int vtr[2][C::NDB];  // TrRowTile offsets of the V^T reads 0 and 1 per feature block

  __device__ __forceinline__ void init_offsets() {
    off.init(lane);
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
      for (int mb = 0; mb < C::NDB; ++mb) vtr[rd][mb] = tr_lane_elem<typename C::VL>(lane, rd, mb);
  }

  // S^T (64 keys x this wave's 32 queries) of the K tile at kt: a fixed list
  // of DK stages, one k-step of every 32-key block each (the blocks' MFMA
  // chains interleaved), each stage's K operands read SCORE_PF stages ahead.
  // Left to the scheduler, the reads went out one at a time, each waited for
  // right before its MFMA, and the blocks' chains ran one after the other.
  __device__ __forceinline__ void scores(const uint16_t* kt, f32x16 (&sacc)[C::KB]) const {
    constexpr int PF = C::SCORE_PF;
    u32x4 rk[C::DK][C::KB];
    auto fetch = [&](int s) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) rk[s][kb] = lds_read16(kt + off.rd(s, kb));
    };
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < PF; ++s) fetch(s);
#pragma unroll
    for (int s = 0; s < C::DK; ++s) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) sacc[kb] = E::mfma(rk[s][kb], qf[s], sacc[kb]);
      if (s + PF < C::DK) fetch(s + PF);
      sched_fence();
    }
  }

  // P = 2^(c S - mc) for score blocks [KB0, KB0 + NKB), packed to the storage
  // type (pw), with the row sums of P in fp32 (rs) and of P as rounded (rsr).
  template <int KB0, int NKB>
  __device__ __forceinline__ void exps(const f32x16 (&sacc)[C::KB], uint32_t (&pw)[C::KB][8], float mc,
                                       float scale_log2, float& rs, float& rsr) const {
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int kb = KB0; kb < KB0 + NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = exp2_fast(__builtin_fmaf(sacc[kb][i], scale_log2, -mc));
        const float p1 = exp2_fast(__builtin_fmaf(sacc[kb][i + 1], scale_log2, -mc));
        const float pp = p0 + p1;
        r0 = kb == KB0 && i == 0 ? pp : r0 + pp;
        const uint32_t w = E::pack2(p0, p1);
        pw[kb][i >> 1] = w;
        if constexpr (!C::ONES_ROW) r1 = E::add_pair(w, r1);
      }
    rs = r0;
    rsr = r1;
  }

  // Scores of keys past the end of the sequence, and above the diagonal, to
  // -inf: applied to a whole tile that may hold such keys for some of this
  // wave's rows, as a run-time branch over the scores only (one tile body for
  // every tile, so the O accumulators keep one register assignment through the
  // loop).
  // Register i of block kb holds key key0 + 4 lh + (kb 32 + 8 (i / 4) + i % 4):
  // one per-lane bound on that constant offset covers both tests (one compare
  // with an inline constant per register instead of an add and two compares;
  // B4 H32 N4096 d64 causal forward -1.1 %, B1 H16 N16384 d128 causal -0.6 %
  // on MI355X).
  __device__ __forceinline__ void apply_mask(f32x16 (&sacc)[C::KB], int key0, int Nk) const {
    const int last = CAUSAL ? min(Nk - 1, key_last) : Nk - 1;   // last key the lane's row sees
    const int lim = last - key0 - 4 * lh;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) sacc[kb][i] = -INFINITY;
  }

  // Online-softmax step on score blocks [KB0, KB0 + NKB): P packed to the
  // storage type (pw), running sums updated.  Returns the factor that O must
  // be multiplied by; `any` tells whether some lane's factor differs from 1.
  //
  // LAZY: the reference m of a row need not be its running maximum; any m
  // works as long as no 2^(c (S - m)) overflows, and the final division by the
  // row sum cancels it ("FlashAttention-2" summary page, "How It Works" 2: the
  // scaling leaves the inner loop).  So P is first computed against the
  // current m, without a maximum pass over the scores, and kept if every
  // lane's share of the row sum is at most 2^8 (then so is every P, and no
  // rescale is due).  Otherwise (the first block, where m = -inf makes the sum
  // inf or NaN, or a score more than 8 / c above m) m moves to the row maximum
  // as below and P is recomputed.
  template <int KB0, int NKB>
  __device__ __forceinline__ float softmax(f32x16 (&sacc)[C::KB], uint32_t (&pw)[C::KB][8], bool& any,
                                           float scale_log2) {
    float rs, rsr;
    if constexpr (C::LAZY) {
      exps<KB0, NKB>(sacc, pw, m_run * scale_log2, scale_log2, rs, rsr);
      if (__all(rs <= kLazyBound)) {   // false for NaN
        l_run += rs;
        lr_run += rsr;
        any = false;
        return 1.f;
      }
    }
    float mx = fmaxf(sacc[KB0][0], sacc[KB0][1]);
#pragma unroll
    for (int kb = KB0; kb < KB0 + NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, swap_halves(mx));
    const bool grow = mx > m_run;
    // A masked tile can hide every key from a row (a query that precedes all
    // visible keys when Nq > Nk): its maximum stays -inf, and 0 stands in
    // for it so that P = 0 and alpha = 0 instead of NaN.
    const float m_new = grow ? mx : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_fast((m_run - m_use) * scale_log2);
    exps<KB0, NKB>(sacc, pw, m_use * scale_log2, scale_log2, rs, rsr);
    l_run = l_run * alpha + rs;
    lr_run = lr_run * alpha + rsr;
    m_run = m_new;
    any = __any(grow);
    return alpha;
  }

  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[mb][i] *= alpha;
  }

  // O^T (d x query) += V^T (d x 16 keys) P^T (16 keys x query) over the 16-key
  // chunks of score blocks [KB0, KB0 + NKB): V^T by two transposed reads of
  // the row-major V tile vt per operand.
  template <int KB0, int NKB>
  __device__ __forceinline__ void pv(const uint16_t* vt, const uint32_t (&pw)[C::KB][8]) {
#pragma unroll
    for (int c = 2 * KB0; c < 2 * (KB0 + NKB); ++c) {
      const u32x4 b = acc_chunk(pw[c >> 1], c & 1);
#pragma unroll
      for (int mb = 0; mb < C::NDB; ++mb) {
        const u32x4 a = lds_read_tr(vt + vtr[0][mb] + c * C::VL::ROWS16, vt + vtr[1][mb] + c * C::VL::ROWS16);
        oacc[mb] = E::mfma(a, b, oacc[mb]);
      }
    }
    mfma_pipeline_hint<2, 2 * NKB * C::NDB, 4 * NKB * C::NDB, C::READ_AHEAD, 2>();
  }

  // Softmax and O += V P over score blocks [KB0, KB0 + NKB) of the tile.
  template <int KB0, int NKB>
  __device__ __forceinline__ void softmax_pv(const uint16_t* vt, float scale_log2) {
    uint32_t pw[C::KB][8];
    bool any;
    const float alpha = softmax<KB0, NKB>(sc[0], pw, any, scale_log2);
    if (any) rescale(alpha);
    pv<KB0, NKB>(vt, pw);
  }
};

// Stage J (PAR = J % 2, a compile-time constant so that LDS buffers are
// immediate offsets) holds tiles J*SUB .. J*SUB + SUB - 1: issue the copies of
// stage J+1's K and V, then per tile scores, softmax, the rare rescale and
// O += V(j) P(j).  Tiles from n_full on are masked.
template <int D, bool CAUSAL, class E, int PAR>
__device__ __forceinline__ void fwd_stage(FwdWave<D, CAUSAL, E>& w,
                                          const TileDma<D, FwdCfg<D, CAUSAL>::STAGE, FwdCfg<D, CAUSAL>::THREADS>& kdma,
                                          const TileDma<D, FwdCfg<D, CAUSAL>::STAGE, FwdCfg<D, CAUSAL>::THREADS,
                                                        TrRowTile<D>>& vdma,
                                          uint16_t (*k_lds)[FwdCfg<D, CAUSAL>::TILE],
                                          uint16_t (*v_lds)[FwdCfg<D, CAUSAL>::VTILE],
                                          const uint16_t* Kh, const uint16_t* Vh, int J,
                                          int n_tiles, int n_full, int Nk, float scale_log2) {
  using C = FwdCfg<D, CAUSAL>;
  wait_vmem();
  __syncthreads();   // stage J is in LDS; every wave is done with the other buffer
  const int n_stages = (n_tiles + C::SUB - 1) / C::SUB;
  if (J + 1 < n_stages) {
    kdma.issue(k_lds[PAR ^ 1], Kh, (J + 1) * C::STAGE, Nk);
    vdma.issue(v_lds[PAR ^ 1], Vh, (J + 1) * C::STAGE, Nk);
  }
#pragma unroll
  for (int sub = 0; sub < C::SUB; ++sub) {
    const int j = J * C::SUB + sub;
    const bool mask = j >= n_full;
    // a wavefront whose rows all precede the tile's first key has nothing to do
    if (j < n_tiles && (!mask || !CAUSAL || j * C::BC <= w.key_last_wave)) {
      w.scores(k_lds[PAR] + sub * RowTile<D>::block(C::KB), w.sc[0]);
      if (mask) w.apply_mask(w.sc[0], j * C::BC, Nk);
      const uint16_t* vt = v_lds[PAR] + sub * (C::BC / 16) * C::VL::ROWS16;
      // With the lazy maximum each 32-key block is a softmax step of its own,
      // so the exponentials of block 1 can run under the products of block 0.
      if constexpr (C::BLOCK_STEPS) {
        w.template softmax_pv<0, 1>(vt, scale_log2);
        w.template softmax_pv<1, 1>(vt, scale_log2);
      } else {
        w.template softmax_pv<0, C::KB>(vt, scale_log2);
      }
    }
  }
}

template <int D, bool CAUSAL, class E>
__global__ __launch_bounds__((FwdCfg<D, CAUSAL>::THREADS), (FwdCfg<D, CAUSAL>::WAVES_PER_SIMD)) void fwd_kernel(CView Q, CView K, CView V, View O,
                                                     float* __restrict__ LSE, int BH, int H, int Nq,
                                                     int Nk, float scale_log2) {
  using C = FwdCfg<D, CAUSAL>;
  __shared__ __attribute__((aligned(256))) uint16_t k_lds[2][C::TILE];
  __shared__ __attribute__((aligned(256))) uint16_t v_lds[2][C::VTILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  if constexpr (C::VL::HAS_CONST) {
    // features 80..95 of every V row: (1, 0, .., 0) and zeros (slots 10, 11)
    for (int i = tid; i < 2 * C::STAGE; i += C::THREADS) {
      const u32x4 one = {(uint32_t)E::kOne, 0u, 0u, 0u}, zero = {0u, 0u, 0u, 0u};
      uint16_t* row = v_lds[i / C::STAGE] + C::VL::elem(i % C::STAGE, 80);
      *reinterpret_cast<u32x4*>(row) = one;
      *reinterpret_cast<u32x4*>(row + 8) = zero;
    }
  }

  // Linear workgroup id -> (row block, batch*head).  Consecutive ids take
  // different heads, so with the round-robin dispatch over the 8 XCDs all row
  // blocks of one head land on the same XCD (and its L2).  Causal: the longest
  // row blocks (most tiles) are dispatched first.
  const int nrb = (Nq + C::BR - 1) / C::BR;
  const int bh = blockIdx.x % BH;
  int rb = blockIdx.x / BH;
  if (CAUSAL) rb = nrb - 1 - rb;

  const uint16_t* Qh = Q.head(bh / H, bh % H);
  const uint16_t* Kh = K.head(bh / H, bh % H);
  const uint16_t* Vh = V.head(bh / H, bh % H);
  uint16_t* Oh = O.head(bh / H, bh % H);
  // causal: query i sees keys j <= i + koff (queries aligned to the end of the keys)
  const int koff = Nk - Nq;

  FwdWave<D, CAUSAL, E> w;
  w.lane = tid & 63;
  w.lr = w.lane & 31;
  w.lh = w.lane >> 5;
  w.q_wave = rb * C::BR + wave * 32;
  w.q_lane = w.q_wave + w.lr;
  w.key_last = w.q_lane + koff;
  w.key_last_wave = w.q_wave + 31 + koff;
  w.m_run = -INFINITY;
  w.l_run = 0.f;
  w.lr_run = 0.f;
  w.init_offsets();
#pragma unroll
  for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.oacc[mb][i] = 0.f;

  const int q_first = rb * C::BR;              // first query row of the workgroup
  int n_tiles = (Nk + C::BC - 1) / C::BC;
  if (CAUSAL) {
    const int last_key = q_first + C::BR - 1 + koff;   // last key any row of the block sees
    n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / C::BC + 1);
  }
  // tiles [0, n_full) hold only keys that every row of the block may see
  const int n_full = min(n_tiles, (CAUSAL ? max(0, min(q_first + koff + 1, Nk)) : Nk) / C::BC);

  // Stage 0 into LDS: K and V by direct copies.
  TileDma<D, C::STAGE, C::THREADS> kdma;
  TileDma<D, C::STAGE, C::THREADS, typename C::VL> vdma;
  kdma.init(tid, K.sr);
  vdma.init(tid, V.sr);
  if (n_tiles > 0) {
    kdma.issue(k_lds[0], Kh, 0, Nk);
    vdma.issue(v_lds[0], Vh, 0, Nk);
  }
  // Q fragments stay in registers for the whole pass (B operand of S^T = K Q^T).
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (w.q_lane < Nq) z = ld_global16(Qh + (size_t)w.q_lane * Q.sr + s * 16 + 8 * w.lh);
    w.qf[s] = z;
    if constexpr (C::Q_IN_AGPR) asm volatile("" : "+a"(w.qf[s]));
  }

  // Stage J uses buffer J % 2; unrolled by two so the buffer is an immediate.
  const int n_stages = (n_tiles + C::SUB - 1) / C::SUB;
  for (int J = 0; J < n_stages; J += 2) {
    fwd_stage<D, CAUSAL, E, 0>(w, kdma, vdma, k_lds, v_lds, Kh, Vh, J, n_tiles, n_full, Nk, scale_log2);
    if (J + 1 < n_stages)
      fwd_stage<D, CAUSAL, E, 1>(w, kdma, vdma, k_lds, v_lds, Kh, Vh, J + 1, n_tiles, n_full, Nk, scale_log2);
  }

  // Epilogue: one division by the row sum of the rounded P, then O (bf16) and
  // L (fp32, natural log, from the unrounded sum).  A row that saw no key
  // (l = 0) gets O = 0 and L = -inf.
  const float l_tot = w.l_run + swap_halves(w.l_run);
  float lr_tot;
  if constexpr (C::ONES_ROW) {
    const float own = w.oacc[D / 32][C::ONES_REG];
    const float other = swap_halves(own);
    lr_tot = w.lh == C::ONES_HALF ? own : other;
  } else {
    lr_tot = w.lr_run + swap_halves(w.lr_run);
  }
  if (w.q_lane < Nq) {
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    uint16_t* orow = Oh + (size_t)w.q_lane * O.sr;
#pragma unroll
    for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * w.lh;
        if (d0 < D) {
          u32x2 v = {E::pack2(w.oacc[mb][4 * g + 0] * inv, w.oacc[mb][4 * g + 1] * inv),
                     E::pack2(w.oacc[mb][4 * g + 2] * inv, w.oacc[mb][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = v;
        }
      }
    if (w.lh == 0)
      LSE[(size_t)bh * Nq + w.q_lane] =
          l_tot > 0.f ? (w.m_run * scale_log2 + log2_fast(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, class E>
hipError_t launch_fwd_t(const Strided& q, const Strided& k, const Strided& v, const Strided& o,
                        float* lse, int B, int H, int Nq, int Nk, float scale, hipStream_t stream) {
  using C = FwdCfg<D, CAUSAL>;
  const int BH = B * H;
  const int nrb = (Nq + C::BR - 1) / C::BR;
  fwd_kernel<D, CAUSAL, E><<<dim3((unsigned)(nrb * BH)), C::THREADS, 0, stream>>>(
      cview(q), cview(k), cview(v), view(o), lse, BH, H, Nq, Nk, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const Strided& q, const Strided& k, const Strided& v, const Strided& o,
                      float* lse, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      int dtype, hipStream_t stream) {
  return dispatch(d, causal, dtype, [&](auto dc, auto cc, auto ec) {
    return launch_fwd_t<decltype(dc)::value, decltype(cc)::value, decltype(ec)>(q, k, v, o, lse, B, H,
                                                                                 Nq, Nk, scale, stream);
  });
}

void fwd_tiles(int d, int* block_q, int* block_k, int* waves) {
  auto set = [&](auto cfg) {
    using C = decltype(cfg);
    *block_q = C::BR;
    *block_k = C::BC;
    *waves = C::WAVES;
  };
  if (d == 64) set(FwdCfg<64>{});
  else if (d == 80) set(FwdCfg<80>{});
  else if (d == 96) set(FwdCfg<96>{});
  else if (d == 256) set(FwdCfg<256>{});
  else set(FwdCfg<128>{});
}

}  // namespace fa2
