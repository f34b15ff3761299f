// Backward pass of exact tiled attention on gfx950.
//
// Three kernels, enqueued in order by fa2_bwd:
//   preprocess  for every query row: delta_i = sum_k dO_ik O_ik and L_i log2(e),
//               written to row-padded fp32 arrays (rows past Nq, and rows that saw
//               no key (L = -inf): delta 0 or its value, L +inf, which makes every
//               P of such a row exactly 0); HBM-bound, 8 lanes per row.
//   dkdv        one workgroup per (128-key column block, batch*head); each of its 4
//               wavefronts owns 32 keys and keeps K and V (as MFMA operands) and its
//               dK, dV accumulators in registers while walking the 64-query row
//               blocks that can see those keys (causal: from the diagonal on;
//               blocks wholly above it are never visited, diagonal ones are masked
//               element-wise).  Per block, with P recomputed from the stored L:
//                 S  = Q K^T          P  = 2^(c S - L log2 e),  c = scale log2 e
//                 dP = dO V^T         dS = P (dP - delta)
//                 dV^T += dO^T P      dK^T += Q^T dS
//               P and dS feed their MFMAs straight from registers; Q and dO are
//               copied row-major straight into LDS and read there both
//               row-wise and transposed (ds_read_b64_tr_b16).
//   dq          one workgroup of 8 wavefronts per (256-query row block, batch*head),
//               shaped like the forward: Q and dO stay in registers, K/V tiles are
//               copied into LDS (K is read there both row-wise and transposed):
//                 S^T = K Q^T   dP^T = V dO^T   dS^T = P^T (dP^T - delta)
//                 dQ^T += K^T dS^T
//               This second pass recomputes S and dP instead of adding partial dQ
//               with atomics (it needs no fp32 accumulator and no atomics).
// The softmax scale of dQ and dK is applied once, in the epilogues
// ("FlashAttention-2" summary page, "How It Works" 2).
#include <type_traits>

#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {

// Multiple of every query block size the backward kernels use (64 and 256).
#if !FA2_DQ256_UNIT
int bwd_rows_padded(int N) { return (N + 255) / 256 * 256; }
#endif

namespace {

// ---------------------------------------------------------------------------
// preprocess
// ---------------------------------------------------------------------------
// Lanes per row of the preprocess kernel: each lane reads 16-byte chunks
// sub, sub + 8, ... of its row of O and dO (D / 8 chunks: every lane busy at
// D = 64 and 128).
constexpr int kPreLanes = 8;
constexpr int kPreRows = 256 / kPreLanes;   // rows per workgroup

template <int D, class E>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(
    CView O, CView dO, const float* __restrict__ LSE, float* __restrict__ Delta,
    float* __restrict__ L2, int H, int N, int Npad, long rows_pad) {
  constexpr int CH = D / 8;
  constexpr int ITER = (CH + kPreLanes - 1) / kPreLanes;
  const long prow = (long)blockIdx.x * kPreRows + (threadIdx.x / kPreLanes);   // padded row index
  const int sub = threadIdx.x % kPreLanes;
  const long bh = prow / Npad;
  const int q = (int)(prow - bh * Npad);
  const bool valid = prow < rows_pad && q < N;
  const long row = bh * N + q;
  float acc = 0.f;
  if (valid) {
    const uint16_t* orow = O.head((int)(bh / H), (int)(bh % H)) + (size_t)q * O.sr;
    const uint16_t* grow = dO.head((int)(bh / H), (int)(bh % H)) + (size_t)q * dO.sr;
    // every load of the lane first, then the arithmetic
    u32x4 o[ITER], g[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int ch = sub + it * kPreLanes;
      if (ch < CH) {
        o[it] = ld_global16(orow + ch * 8);
        g[it] = ld_global16(grow + ch * 8);
      }
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      if (sub + it * kPreLanes < CH) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          acc += E::lo(o[it][w]) * E::lo(g[it][w]) + E::hi(o[it][w]) * E::hi(g[it][w]);
      }
    }
  }
#pragma unroll
  for (int off = kPreLanes / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (prow < rows_pad && sub == 0) {
    Delta[prow] = valid ? acc : 0.f;
    const float l = valid ? LSE[row] : -INFINITY;
    L2[prow] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
struct DkdvCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BKC = 32 * WAVES;          // keys per workgroup
  static constexpr int BQ = 64;                   // queries per step
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int NDB = DP / 32;
  static constexpr int DK = D / 16;
  static constexpr int NQB = BQ / 32;
  // Q and dO tiles are copied row-major straight into LDS (direct global ->
  // LDS loads, no registers) and read twice: row-wise for S and dP, and with
  // transposing reads (ds_read_b64_tr_b16) as Q^T and dO^T for the dV and dK
  // products.  RowTile's swizzle suits both kinds of read; D = 80 and 96 use
  // its 128-feature rows (WideRowTile).  Staging both tiles through
  // registers and writing them twice, row-major and transposed, measured
  // 2-4 % slower on MI355X (backward B4 H32 N4096 d64 causal -3.3 %,
  // B2 H32 N8192 d80 causal -1.4 %, B1 H16 N16384 d128 causal -1.5 %).
  using TileL = std::conditional_t<(D == 80 || D == 96), WideRowTile<D>, RowTile<D>>;
  static constexpr int TILE = TileL::elems(BQ);
  // passes of the copy of one tile (one per MFMA stage)
  static constexpr int NP = DmaPlan<D, BQ, THREADS, TileL>::ITER;
  static_assert(BQ == 64, "64 queries per step");
};

template <int D, bool CAUSAL, class E>
struct DkdvWave {
  using C = DkdvCfg<D>;
  u32x4 kf[C::DK], vf[C::DK];   // K and -V (B operands of S and of delta - dP)
  f32x16 dkacc[C::NDB], dvacc[C::NDB];
  int lane, lr, lh, key_w, key_lane;
  LaneOffsets<D, typename C::TileL> off;
  int tro[2][C::NDB];   // transposed reads 0 and 1 of feature block mb

  __device__ __forceinline__ void init_offsets() {
    off.init(lane);
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
      for (int mb = 0; mb < C::NDB; ++mb) tro[rd][mb] = tr_lane_elem<typename C::TileL>(lane, rd, mb);
  }

  // One 64-query step.  qt, dot: the row-major Q and dO tiles (read row-wise
  // and transposed); l2s, dls: the step's L log2 e and delta; kq0: the last
  // key the step's first query may see (causal); Nk: keys.  issue(t) runs at
  // the end of stage t (the caller's copies for the next step, spread out so
  // that they never go out in one burst).
  //
  // The step is a fixed sequence of MFMA stages, two MFMAs each:
  //   stage t <  NS:  S and dP of query half qb = t / DK, feature chunk s = t % DK
  //   stage NS + u:   dV and dK of 16-query chunk c = u / NDB, feature block mb = u % NDB
  // Each stage's two LDS operands are read PF stages ahead of it.  The softmax
  // of query half 0 runs under the S/dP MFMAs of half 1, and that of half 1
  // under the first dV/dK MFMAs (which only need half 0): with one wavefront
  // per SIMD this is the only way the matrix cores and the vector ALU overlap.
  template <bool MASK, class Issue>
  __device__ __forceinline__ void step(const uint16_t* qt, const uint16_t* dot, const float* l2s,
                                       const float* dls, int kq0, int Nk, float scale_log2, Issue&& issue) {
    static_assert(C::NQB == 2, "two 32-query halves per step");
    constexpr int NS = C::NQB * C::DK;
    constexpr int NT = (C::BQ / 16) * C::NDB;
    constexpr int NALL = NS + NT;
    // operand reads in flight: 2 stages at D = 128, whose registers are
    // the tightest (fewer spills to the accumulator registers: B1 H16 N16384
    // d128 causal dK/dV -0.8 %), else 3
    constexpr int PF = D == 128 ? 2 : 3;
    u32x4 ra[NALL], rb[NALL];
    auto fetch = [&](int t) {
      if (t < NS) {
        const int o = off.rd(t % C::DK, t / C::DK);
        ra[t] = lds_read16(qt + o);
        rb[t] = lds_read16(dot + o);
      } else {
        const int u = t - NS;
        const int c = u / C::NDB, mb = u % C::NDB;
        constexpr int R16 = C::TileL::ROWS16;
        ra[t] = lds_read_tr(dot + tro[0][mb] + c * R16, dot + tro[1][mb] + c * R16);
        rb[t] = lds_read_tr(qt + tro[0][mb] + c * R16, qt + tro[1][mb] + c * R16);
      }
    };
    // Row statistics of group (qb, g): lane (lr, lh) needs queries
    // qb*32 + 8g + 4lh + r.  sm_stage(qb, g) is the stage whose end runs the
    // group's softmax; its L log2 e is read LEAD stages earlier (from stage 0
    // on).  LDS reads complete in order, so a statistics read issued just
    // before its use would make the softmax also wait for the operand reads
    // prefetched ahead of it.
    f32x4 lv[C::NQB][4];
    auto sm_stage = [](int qb, int g) {
      return qb == 0 ? C::DK + 1 + g * (C::DK - 1) / 4 : NS + 1 + g * (2 * C::NDB - 1) / 4;
    };
    constexpr int LEAD = 4;
    auto stats_stage = [&](int qb, int g) { return max(0, sm_stage(qb, g) - LEAD); };
    auto load_stats = [&](int qb, int g) {
      lv[qb][g] = *reinterpret_cast<const f32x4*>(l2s + qb * 32 + 8 * g + 4 * lh);
    };

    // The dP accumulators start from delta: with V negated (the caller's
    // vf) the MFMAs leave delta - dP in them, so dS = -(P acc) takes one
    // multiply.  Half 0's delta is read before the step's operand reads,
    // half 1's LEAD stages before its first dP product.
    f32x16 sacc[C::NQB], pacc[C::NQB];
    auto load_delta = [&](int qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 d = *reinterpret_cast<const f32x4*>(dls + qb * 32 + 8 * g + 4 * lh);
#pragma unroll
        for (int r = 0; r < 4; ++r) pacc[qb][4 * g + r] = d[r];
      }
    };
    constexpr int DELTA1_STAGE = C::DK > LEAD ? C::DK - LEAD : 0;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int t = 0; t < 16; ++t) sacc[qb][t] = 0.f;
    load_delta(0);
    uint32_t pw[C::NQB][8], dsw[C::NQB][8];
    // P = 2^(c S - L log2 e) and dS = P (dP - delta) for 4 of a half's 16
    // registers (queries qb*32 + 8g + 4lh + r), packed to bf16.
    auto softmax_group = [&](int qb, int g) {
      float p[4], ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * g + r;
        // a masked score becomes -inf, so P = 2^-inf = 0: the exponential
        // stays unconditional (a test on its result became a branch per
        // group; B4 H32 N4096 d64 causal dK/dV -0.9 %, B1 H16 N16384 d128
        // causal -0.5 % on MI355X)
        float sv = sacc[qb][t];
        if (MASK && (key_lane >= Nk || (CAUSAL && key_lane > kq0 + qb * 32 + 8 * g + 4 * lh + r))) sv = -INFINITY;
        const float x = exp2_fast(__builtin_fmaf(sv, scale_log2, -lv[qb][g][r]));
        p[r] = x;
        ds[r] = -(x * pacc[qb][t]);
      }
      pw[qb][2 * g] = E::pack2(p[0], p[1]);
      pw[qb][2 * g + 1] = E::pack2(p[2], p[3]);
      dsw[qb][2 * g] = E::pack2(ds[0], ds[1]);
      dsw[qb][2 * g + 1] = E::pack2(ds[2], ds[3]);
    };

#pragma unroll
    for (int t = 0; t < PF; ++t) fetch(t);

    // S = Q K^T, delta - dP = delta + dO (-V)^T; softmax of half 0 from stage
    // DK + 1 on.
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int qb = t / C::DK, s = t % C::DK;
      sacc[qb] = E::mfma(ra[t], kf[s], sacc[qb]);
      pacc[qb] = E::mfma(rb[t], vf[s], pacc[qb]);
      if (t + PF < NALL) fetch(t + PF);
      if (t == DELTA1_STAGE) load_delta(1);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (t == stats_stage(0, g)) load_stats(0, g);
        if (t == stats_stage(1, g)) load_stats(1, g);
        if (t == sm_stage(0, g)) softmax_group(0, g);
      }
      issue(t);
      sched_fence();
    }
    // dV^T += dO^T P, dK^T += Q^T dS (16 queries per MFMA); softmax of half 1
    // under chunks 0 and 1.
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int t = NS + u, c = u / C::NDB, mb = u % C::NDB;
      dvacc[mb] = E::mfma(ra[t], acc_chunk(pw[c >> 1], c & 1), dvacc[mb]);
      dkacc[mb] = E::mfma(rb[t], acc_chunk(dsw[c >> 1], c & 1), dkacc[mb]);
      if (t + PF < NALL) fetch(t + PF);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (t == stats_stage(1, g)) load_stats(1, g);
        if (t == sm_stage(1, g)) softmax_group(1, g);
      }
      issue(t);
      sched_fence();
    }
  }
};

template <int D, bool CAUSAL, class E>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    CView Q, CView K, CView V, CView dO, const float* __restrict__ L2,
    const float* __restrict__ Delta, View dK, View dV, int BH, int H, int Nq, int Nk, int Npad,
    float scale, float scale_log2) {
  using C = DkdvCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[2][C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[2][C::TILE];
  __shared__ __attribute__((aligned(16))) float ld_lds[2][2 * C::BQ];   // [L log2e | delta]

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  // the constant slots of wide rows are zeros, which every copy stores
  static_assert(!C::TileL::HAS_CONST || C::TileL::CONST_ZERO, "copies store the constant slots");

  // Linear id -> (key block, batch*head); consecutive ids take different heads
  // (XCD round-robin keeps one head's blocks on one XCD).  Key block 0 sees the
  // most query blocks under a causal mask, so it is dispatched first.
  const int bh = blockIdx.x % BH;
  const int kblk = blockIdx.x / BH;
  const uint16_t* Qh = Q.head(bh / H, bh % H);
  const uint16_t* dOh = dO.head(bh / H, bh % H);
  const float* L2h = L2 + (size_t)bh * Npad;
  const float* Dh = Delta + (size_t)bh * Npad;
  // causal: query i sees keys j <= i + koff (queries aligned to the end of the keys)
  const int koff = Nk - Nq;

  const int key_wg = kblk * C::BKC;
  const int n_qblk = (Nq + C::BQ - 1) / C::BQ;
  // causal: the first query block holding a query that sees key key_wg (the
  // last query sees every key, so i_begin < n_qblk)
  const int i_begin = CAUSAL ? max(0, key_wg - koff) / C::BQ : 0;

  // L log2 e and delta of one query block: 2 x 64 floats, 16 bytes per lane.
  // (lanes 16..31 land 256 bytes after lanes 0..15, i.e. at the delta half)
  auto load_ld = [&](float* dst, int q0) {
    if (wave == 0) {
      const int lane = tid & 63;
      if (lane < C::BQ / 4)
        global_load_lds16(L2h + q0, 16u * lane, dst);
      else if (lane < C::BQ / 2)
        global_load_lds16(Dh + q0, 16u * (lane - C::BQ / 4), dst);
    }
  };
  // Q and dO: direct copies into the idle buffers.  Inside a step the next
  // step's copies go out one pass per MFMA stage (stages 0..NP-1 Q, then dO;
  // every step has at least 16 stages): issued as one burst before the step,
  // they measured slower.  After the last step the tiles have no rows: the
  // copies then only store zeros into buffers nobody reads again.
  TileDma<D, C::BQ, C::THREADS, typename C::TileL> qdma, dodma;
  qdma.init(tid, Q.sr);
  dodma.init(tid, dO.sr);
  i32x4 rq, rdo;   // the next step's tiles
  uint32_t dma_q = 0, dma_do = 0;   // LDS addresses of the idle buffers
  auto issue = [&](int t) {
    if (t < C::NP) qdma.issue_pass(t, dma_q, rq);
    else if (t < 2 * C::NP) dodma.issue_pass(t - C::NP, dma_do, rdo);
  };
  if (i_begin < n_qblk) {
    load_ld(ld_lds[0], i_begin * C::BQ);
    qdma.issue(q_lds[0], Qh, i_begin * C::BQ, Nq);
    dodma.issue(do_lds[0], dOh, i_begin * C::BQ, Nq);
  }

  DkdvWave<D, CAUSAL, E> w;
  w.lane = tid & 63;
  w.lr = w.lane & 31;
  w.lh = w.lane >> 5;
  w.key_w = key_wg + wave * 32;
  w.key_lane = w.key_w + w.lr;
  w.init_offsets();
  // K, V as B operands (lane: one key, 8 consecutive features per k-step).
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
    if (w.key_lane < Nk) {
      zk = ld_global16(K.head(bh / H, bh % H) + (size_t)w.key_lane * K.sr + s * 16 + 8 * w.lh);
      zv = ld_global16(V.head(bh / H, bh % H) + (size_t)w.key_lane * V.sr + s * 16 + 8 * w.lh);
    }
    w.kf[s] = zk;
    w.vf[s] = zv ^ 0x80008000u;   // -V: the dP products accumulate onto delta (DkdvWave::step)
    // K and V only ever feed MFMAs, which read operands from the accumulator
    // registers as well: keeping them there leaves the vector registers to
    // the S and dP products, which the softmax reads.
    asm volatile("" : "+a"(w.kf[s]));
    asm volatile("" : "+a"(w.vf[s]));
  }
#pragma unroll
  for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      w.dkacc[mb][t] = 0.f;
      w.dvacc[mb][t] = 0.f;
    }

  // Step i uses buffer (i - i_begin) % 2; unrolled by two so the buffer is a
  // compile-time offset of every LDS read.
  auto iteration = [&](auto buf_tag, int i) {
    constexpr int BUF = decltype(buf_tag)::value;
    wait_vmem();
    __syncthreads();   // step i is in LDS; every wave is done with the other buffer
    if (i + 1 < n_qblk) load_ld(ld_lds[BUF ^ 1], (i + 1) * C::BQ);
    rq = qdma.tile(Qh, (i + 1) * C::BQ, Nq);
    rdo = dodma.tile(dOh, (i + 1) * C::BQ, Nq);
    dma_q = lds_address(q_lds[BUF ^ 1]);
    dma_do = lds_address(do_lds[BUF ^ 1]);
    // kq0: the key position of the step's first query (its last visible key)
    const int kq0 = i * C::BQ + koff;
    const bool need_mask = (CAUSAL && w.key_w + 31 > kq0) || (w.key_w + 32 > Nk);
    const bool active = !CAUSAL || w.key_w <= kq0 + C::BQ - 1;
    if (!need_mask) {
      w.template step<false>(q_lds[BUF], do_lds[BUF], ld_lds[BUF], ld_lds[BUF] + C::BQ, kq0, Nk,
                             scale_log2, issue);
    } else if (active) {
      w.template step<true>(q_lds[BUF], do_lds[BUF], ld_lds[BUF], ld_lds[BUF] + C::BQ, kq0, Nk,
                            scale_log2, issue);
    } else {
      // a wavefront with no key this step can see still does its share of
      // copying the next one
#pragma unroll
      for (int t = 0; t < 2 * C::NP; ++t) issue(t);
    }
  };
  for (int i = i_begin; i < n_qblk; i += 2) {
    iteration(std::integral_constant<int, 0>{}, i);
    if (i + 1 < n_qblk) iteration(std::integral_constant<int, 1>{}, i + 1);
  }
  wait_vmem();   // the last step's copies: LDS must not be released under them

  // Epilogue: dK = scale * dS^T Q, dV = P^T dO (bf16).
  if (w.key_lane < Nk) {
    uint16_t* dkrow = dK.head(bh / H, bh % H) + (size_t)w.key_lane * dK.sr;
    uint16_t* dvrow = dV.head(bh / H, bh % H) + (size_t)w.key_lane * dV.sr;
#pragma unroll
    for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * w.lh;
        if (d0 < D) {
          u32x2 wk = {E::pack2(w.dkacc[mb][4 * g] * scale, w.dkacc[mb][4 * g + 1] * scale),
                      E::pack2(w.dkacc[mb][4 * g + 2] * scale, w.dkacc[mb][4 * g + 3] * scale)};
          u32x2 wv = {E::pack2(w.dvacc[mb][4 * g], w.dvacc[mb][4 * g + 1]),
                      E::pack2(w.dvacc[mb][4 * g + 2], w.dvacc[mb][4 * g + 3])};
          *reinterpret_cast<u32x2*>(dkrow + d0) = wk;
          *reinterpret_cast<u32x2*>(dvrow + d0) = wv;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV at head dimension 256
// ---------------------------------------------------------------------------
// The kernel above keeps K, V and the dK, dV accumulators of a wavefront's 32
// keys in its registers: at D = 256 that alone would be 384 registers.  Here
// each 32-key block is shared by a pair of wavefronts (waves p and p + PAIRS):
// both hold all of K and V (the S and dP products reduce over every feature),
// each accumulates dK and dV for one half of the features.  Per 64-query step:
//   phase 1  member h computes S = Q K^T and dP = dO V^T for query half h
//            (32 queries), then P and dS, which it keeps in registers and
//            writes to LDS for its partner;
//   barrier;
//   phase 2  member h accumulates dV^T += dO^T P and dK^T += Q^T dS for its
//            feature half over all 64 queries (its own half's P and dS from
//            registers, the partner's from LDS).
// One wavefront per SIMD (4 wavefronts, 64 keys per workgroup).  Q and dO are
// copied row-major straight into double-buffered LDS tiles (the copies of
// step i + 1 go out one pass per phase-1 MFMA stage of step i) and read
// row-wise in phase 1 and transposed (ds_read_b64_tr_b16) in phase 2.
template <int D>
struct DkdvSplitCfg {
  static constexpr int PAIRS = 2;
  static constexpr int WAVES = 2 * PAIRS;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BKC = 32 * PAIRS;          // keys per workgroup
  static constexpr int BQ = 64;                   // queries per step
  static constexpr int NDB = D / 32;              // 32-feature blocks
  static constexpr int NBH = NDB / 2;             // feature blocks per member
  static constexpr int DK = D / 16;               // k-steps of S and dP
  using TileL = RowTile<D>;                       // read row-wise and transposed
  static constexpr int TILE = TileL::elems(BQ);
  static constexpr int XV = 2 * 2 * 64;           // u32x4 per member: [P | dS][word quad][lane]
  static constexpr int NP = DmaPlan<D, BQ, THREADS, TileL>::ITER;   // copy passes per tile
  static_assert(D % 64 == 0, "feature halves made of whole 32-feature blocks");
  static_assert(2 * NP <= 2 * DK, "one copy pass per phase-1 stage");
  // Both phases are fixed stage lists, one MFMA (phase 1) or one pair
  // (phase 2) per stage with a scheduling fence after each: with one
  // wavefront per SIMD only reads kept in flight hide LDS latency.  Phase-1
  // row reads go P1_PF stages ahead, the statistics STAT_LEAD stages before
  // their use, phase-2 transposed reads P2_PF stages ahead.  Against the
  // scheduled loops (row reads mostly one ahead, each group's statistics read
  // right before its exponentials): B1 H16 N8192 d256 causal dK/dV 1.176 ->
  // 1.11 ms on MI355X.  Splitting each product's accumulator chain in two
  // measured 7 % slower.
  static constexpr int P1_PF = 4;
  static constexpr int STAT_LEAD = 4;
  static constexpr int P2_PF = 3;
};

template <int D, bool CAUSAL, class E>
struct DkdvSplitWave {
  using C = DkdvSplitCfg<D>;
  u32x4 kf[C::DK], vf[C::DK];
  f32x16 dkacc[C::NBH], dvacc[C::NBH];
  int lane, lr, lh, h, key_w, key_lane;
  int qrow[C::DK];          // row reads: features 16 s + 8 lh of query 32 h + lr
  // transposed reads rd of the member's feature block j, first 16-query chunk
  // of the own (o = 0) and the partner's (o = 1) query half
  int tro[2][2][C::NBH];

  __device__ __forceinline__ void init_offsets() {
    using L = typename C::TileL;
#pragma unroll
    for (int s = 0; s < C::DK; ++s) qrow[s] = L::elem(32 * h + lr, 16 * s + 8 * lh);
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int j = 0; j < C::NBH; ++j)
          tro[o][rd][j] = tr_lane_elem<L>(lane, rd, h * C::NBH + j) + 2 * (o ? 1 - h : h) * L::ROWS16;
  }

  // S and dP for query half h (row-major tiles qt, dot), then P (packed to the
  // storage type as soon as it is computed, under the dP products) and
  // dS = P (dP - delta) from that P.  l2s, dls: the step's L log2 e and delta;
  // kq0: the key position of the step's first query.  mask: some keys of the
  // block lie past the end or above the diagonal for some of the half's
  // queries (a run-time branch, so that one body serves every step).
  // issue(t) runs after stage t (the copies of the next step).
  template <class Issue>
  __device__ __forceinline__ void phase1(bool mask, const uint16_t* qt, const uint16_t* dot,
                                         const float* l2s, const float* dls, int kq0, int Nk,
                                         float scale_log2, uint32_t (&pw)[8], uint32_t (&dsw)[8],
                                         Issue&& issue) {
    constexpr int NS = 2 * C::DK;   // S (t < DK), then dP
    constexpr int PF = C::P1_PF;
    constexpr int SL = C::STAT_LEAD;
    u32x4 ra[NS];
    auto fetch = [&](int t) { ra[t] = lds_read16((t < C::DK ? qt : dot) + qrow[t % C::DK]); };
#pragma unroll
    for (int t = 0; t < PF; ++t) fetch(t);
    f32x16 sacc, pacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sacc[i] = 0.f;
      pacc[i] = 0.f;
    }
    // queries of register 4 g + r: 32 h + 8 g + 4 lh + r
    const float* l2h = l2s + 32 * h + 4 * lh;
    const float* dlh = dls + 32 * h + 4 * lh;
    f32x4 lv[4], dv[4];
    // a fixed list of stages (one MFMA each); the statistics of group g are
    // read SL stages before the stage that uses them
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (t < C::DK) sacc = E::mfma(ra[t], kf[t], sacc);
      else pacc = E::mfma(ra[t], vf[t - C::DK], pacc);
      if (t + PF < NS) fetch(t + PF);
      issue(t);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (t == C::DK + g * C::DK / 4 - SL) lv[g] = *reinterpret_cast<const f32x4*>(l2h + 8 * g);
        if (t == NS - 1 - SL) dv[g] = *reinterpret_cast<const f32x4*>(dlh + 8 * g);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (t == C::DK + g * C::DK / 4) {
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = exp2_fast(__builtin_fmaf(sacc[4 * g + r], scale_log2, -lv[g][r]));
          // (a -inf score for masked keys, as in the kernel above, measured
          // 6 % slower here: B1 H16 N8192 d256 causal)
          if (mask) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key_lane >= Nk || (CAUSAL && key_lane > kq0 + 32 * h + 8 * g + 4 * lh + r)) x[r] = 0.f;
          }
          pw[2 * g] = E::pack2(x[0], x[1]);
          pw[2 * g + 1] = E::pack2(x[2], x[3]);
        }
      }
      sched_fence();
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float p0 = E::lo(pw[2 * g]), p1 = E::hi(pw[2 * g]);
      const float p2 = E::lo(pw[2 * g + 1]), p3 = E::hi(pw[2 * g + 1]);
      dsw[2 * g] = E::pack2(p0 * (pacc[4 * g] - dv[g][0]), p1 * (pacc[4 * g + 1] - dv[g][1]));
      dsw[2 * g + 1] = E::pack2(p2 * (pacc[4 * g + 2] - dv[g][2]), p3 * (pacc[4 * g + 3] - dv[g][3]));
    }
  }

  // dV^T += dO^T P and dK^T += Q^T dS for the member's feature blocks over the
  // step's four 16-query chunks: the own half's two (B operands pw, dsw), then
  // the partner's two (px: its P and dS words in LDS).  qt, dot: the row-major
  // Q and dO tiles, read transposed.
  __device__ __forceinline__ void phase2(const uint16_t* qt, const uint16_t* dot, const u32x4* px,
                                         const uint32_t (&pw)[8], const uint32_t (&dsw)[8]) {
    u32x4 xp[2], xd[2];
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      xp[q4] = px[q4 * 64 + lane];
      xd[q4] = px[(2 + q4) * 64 + lane];
    }
    constexpr int NT = 4 * C::NBH;   // stage u: chunk k = u / NBH, block j = u % NBH
    constexpr int PF = C::P2_PF;
    u32x4 ra[NT], rb[NT];
    auto fetch = [&](int u) {
      const int k = u / C::NBH, j = u % C::NBH;
      const int o = k < 2 ? 0 : 1;
      const int c = (k % 2) * C::TileL::ROWS16;
      ra[u] = lds_read_tr(dot + tro[o][0][j] + c, dot + tro[o][1][j] + c);
      rb[u] = lds_read_tr(qt + tro[o][0][j] + c, qt + tro[o][1][j] + c);
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) fetch(u);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int k = u / C::NBH, j = u % C::NBH;
      const u32x4 bp = k < 2 ? acc_chunk(pw, k) : xp[k - 2];
      const u32x4 bd = k < 2 ? acc_chunk(dsw, k) : xd[k - 2];
      dvacc[j] = E::mfma(ra[u], bp, dvacc[j]);
      dkacc[j] = E::mfma(rb[u], bd, dkacc[j]);
      if (u + PF < NT) fetch(u + PF);
      sched_fence();
    }
  }
};

template <int D, bool CAUSAL, class E>
__global__ __launch_bounds__(DkdvSplitCfg<D>::THREADS, 1) void bwd_dkdv_split_kernel(
    CView Q, CView K, CView V, CView dO, const float* __restrict__ L2,
    const float* __restrict__ Delta, View dK, View dV, int BH, int H, int Nq, int Nk, int Npad,
    float scale, float scale_log2) {
  using C = DkdvSplitCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[2][C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[2][C::TILE];
  __shared__ __attribute__((aligned(16))) u32x4 x_lds[C::WAVES][C::XV];
  __shared__ __attribute__((aligned(16))) float ld_lds[2][2 * C::BQ];   // [L log2e | delta]

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  // Linear id -> (key block, batch*head), as in the kernel above.
  const int bh = blockIdx.x % BH;
  const int kblk = blockIdx.x / BH;
  const float* L2h = L2 + (size_t)bh * Npad;
  const float* Dh = Delta + (size_t)bh * Npad;
  const int koff = Nk - Nq;   // causal: query i sees keys j <= i + koff
  const int key_wg = kblk * C::BKC;
  const int n_qblk = (Nq + C::BQ - 1) / C::BQ;
  const int i_begin = CAUSAL ? max(0, key_wg - koff) / C::BQ : 0;

  auto load_ld = [&](float* dst, int q0) {
    if (wave == 0) {
      const int lane = tid & 63;
      if (lane < C::BQ / 4)
        global_load_lds16(L2h + q0, 16u * lane, dst);
      else if (lane < C::BQ / 2)
        global_load_lds16(Dh + q0, 16u * (lane - C::BQ / 4), dst);
    }
  };
  const uint16_t* Qh = Q.head(bh / H, bh % H);
  const uint16_t* dOh = dO.head(bh / H, bh % H);
  // Q and dO: direct copies into the idle buffers, one pass per phase-1 stage
  // (Q passes first, then dO).  After the last step the tiles have no rows:
  // the copies then only store zeros into buffers nobody reads again.
  TileDma<D, C::BQ, C::THREADS, typename C::TileL> qdma, dodma;
  qdma.init(tid, Q.sr);
  dodma.init(tid, dO.sr);
  i32x4 rq, rdo;   // the next step's tiles
  uint32_t dma_q = 0, dma_do = 0;   // LDS addresses of the idle buffers
  auto issue = [&](int t) {
    if (t < C::NP) qdma.issue_pass(t, dma_q, rq);
    else if (t < 2 * C::NP) dodma.issue_pass(t - C::NP, dma_do, rdo);
  };
  if (i_begin < n_qblk) {
    load_ld(ld_lds[0], i_begin * C::BQ);
    qdma.issue(q_lds[0], Qh, i_begin * C::BQ, Nq);
    dodma.issue(do_lds[0], dOh, i_begin * C::BQ, Nq);
  }

  DkdvSplitWave<D, CAUSAL, E> w;
  w.lane = tid & 63;
  w.lr = w.lane & 31;
  w.lh = w.lane >> 5;
  w.h = wave / C::PAIRS;
  w.key_w = key_wg + (wave % C::PAIRS) * 32;
  w.key_lane = w.key_w + w.lr;
  w.init_offsets();
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
    if (w.key_lane < Nk) {
      zk = ld_global16(K.head(bh / H, bh % H) + (size_t)w.key_lane * K.sr + s * 16 + 8 * w.lh);
      zv = ld_global16(V.head(bh / H, bh % H) + (size_t)w.key_lane * V.sr + s * 16 + 8 * w.lh);
    }
    w.kf[s] = zk;
    w.vf[s] = zv;
    // accumulator registers, as in the kernel above (here: 128 vector
    // registers left for the reads in flight; -2 % dK/dV time at B1 H16 N8192
    // d256 causal)
    asm volatile("" : "+a"(w.kf[s]));
    asm volatile("" : "+a"(w.vf[s]));
  }
#pragma unroll
  for (int j = 0; j < C::NBH; ++j)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      w.dkacc[j][t] = 0.f;
      w.dvacc[j][t] = 0.f;
    }
  u32x4* x_own = x_lds[wave];
  const u32x4* x_partner = x_lds[(wave + C::PAIRS) % C::WAVES];
  wait_vmem();
  __syncthreads();   // the first step's tiles and statistics are in LDS

  for (int i = i_begin; i < n_qblk; ++i) {
    const int buf = (i - i_begin) & 1;   // tile and statistics buffer of step i
    if (i + 1 < n_qblk) load_ld(ld_lds[buf ^ 1], (i + 1) * C::BQ);
    rq = qdma.tile(Qh, (i + 1) * C::BQ, Nq);
    rdo = dodma.tile(dOh, (i + 1) * C::BQ, Nq);
    dma_q = lds_address(q_lds[buf ^ 1]);
    dma_do = lds_address(do_lds[buf ^ 1]);
    const int kq0 = i * C::BQ + koff;   // key position of the step's first query
    // Every pair runs every step of the workgroup: a block whose keys all lie
    // above a step's queries (at most the first step of the second pair) is
    // masked to P = 0 rather than skipped, which keeps one straight-line body.
    const bool need_mask = (CAUSAL && w.key_w + 31 > kq0 + 32 * w.h) || (w.key_w + 32 > Nk);
    uint32_t pw[8], dsw[8];
    w.phase1(need_mask, q_lds[buf], do_lds[buf], ld_lds[buf], ld_lds[buf] + C::BQ, kq0, Nk, scale_log2, pw, dsw,
             issue);
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      x_own[q4 * 64 + w.lane] = acc_chunk(pw, q4);
      x_own[(2 + q4) * 64 + w.lane] = acc_chunk(dsw, q4);
    }
    __syncthreads();   // both members' P and dS visible
    w.phase2(q_lds[buf], do_lds[buf], x_partner, pw, dsw);
    wait_vmem();
    __syncthreads();   // tiles and statistics of step i + 1 in LDS; X and this step's tiles free
  }

  // Epilogue: dK = scale * dS^T Q, dV = P^T dO (bf16), the member's features.
  if (w.key_lane < Nk) {
    uint16_t* dkrow = dK.head(bh / H, bh % H) + (size_t)w.key_lane * dK.sr;
    uint16_t* dvrow = dV.head(bh / H, bh % H) + (size_t)w.key_lane * dV.sr;
    const int lh = (int)(__lane_id() >> 5);
#pragma unroll
    for (int j = 0; j < C::NBH; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = (w.h * C::NBH + j) * 32 + 8 * g + 4 * lh;
        u32x2 wk = {E::pack2(w.dkacc[j][4 * g] * scale, w.dkacc[j][4 * g + 1] * scale),
                    E::pack2(w.dkacc[j][4 * g + 2] * scale, w.dkacc[j][4 * g + 3] * scale)};
        u32x2 wv = {E::pack2(w.dvacc[j][4 * g], w.dvacc[j][4 * g + 1]),
                    E::pack2(w.dvacc[j][4 * g + 2], w.dvacc[j][4 * g + 3])};
        *reinterpret_cast<u32x2*>(dkrow + d0) = wk;
        *reinterpret_cast<u32x2*>(dvrow + d0) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
struct DqCfg {
  // At D = 256 the Q and dO operands (128 registers) and dQ accumulators (128)
  // leave room for one wavefront per SIMD: 4 wavefronts.  Its 64-key K and V
  // tiles take 128 KiB of LDS double-buffered (B1 H16 N8192 d256 causal dQ
  // -1 % against 32-key tiles on MI355X).
  static constexpr int WAVES = D == 256 ? 4 : 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BR = 32 * WAVES;           // query rows per workgroup
  static constexpr int BC = 64;                   // keys per K/V tile
  static constexpr int KB = BC / 32;              // 32-key MFMA blocks per tile
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int NDB = DP / 32;
  static constexpr int DK = D / 16;
  // K and V tiles are copied row-major straight into LDS and read row-wise
  // (S^T, dP^T); K is also read transposed (ds_read_b64_tr_b16) as K^T for
  // the dQ product.  RowTile's swizzle suits both kinds of read; D = 80 and
  // 96 use its 128-feature rows (WideRowTile).
  using TileL = std::conditional_t<(D == 80 || D == 96), WideRowTile<D>, RowTile<D>>;
  static constexpr int TILE = TileL::elems(BC);
  // Where registers allow, the dP^T products start from delta (16 registers
  // holding this lane's delta) with dO negated, leaving delta - dP^T: dS^T =
  // -(P^T acc) then takes one multiply instead of a subtraction and one
  // (B4 H32 N4096 d64 causal dQ -9.5 %, B2 H32 N8192 d80 causal -2.7 % on
  // MI355X).  At D = 128 it measured even (B1 H16 N16384 d128 causal) or 1 %
  // slower (B8 H16 N2048 d128).
  static constexpr bool DELTA_INIT = D != 128;
  // With one wavefront per SIMD (D = 256) nothing hides an LDS read's
  // latency, and left to the scheduler the products waited for their reads
  // (a third of the MFMAs behind a full wait): there tile() issues them as
  // explicit stage lists, the S^T and dP^T operands SCORE_PF k-steps ahead
  // and the K^T operands of the dQ products DQ_PF products ahead (B1 H16
  // N8192 d256 causal dQ -3.6 % on MI355X).  With two wavefronts per SIMD the
  // same lists measured even or up to 3 % slower than the scheduled loops,
  // whose LDS reads a scheduling hint keeps READ_AHEAD deep.
  static constexpr bool STAGED = D == 256;
  static constexpr int SCORE_PF = 2;
  static constexpr int DQ_PF = 2;
  static constexpr int READ_AHEAD = 6;
};

template <int D, bool CAUSAL, class E>
struct DqWave {
  using C = DqCfg<D>;
  // Also the stage lists at D = 64 without the causal mask: there the
  // scheduling hint did not take (each score operand read right before its
  // MFMA); B8 H16 N2048 d64 dQ -1.6 % on MI355X.
  static constexpr bool STAGED = C::STAGED || (D == 64 && !CAUSAL);
  u32x4 qf[C::DK], dof[C::DK];   // Q and dO (DELTA_INIT: -dO)
  f32x16 dqacc[C::NDB];
  f32x16 dl16;   // DELTA_INIT: dl in every register
  float l2, dl;
  int lane, lr, lh, q_wave, q_lane;
  int key_last;   // causal: last key this lane's query may see (q_lane + Nk - Nq)
  LaneOffsets<D, typename DqCfg<D>::TileL> off;
  int tro[2][C::NDB];   // transposed reads 0 and 1 of feature block mb

  __device__ __forceinline__ void init_offsets() {
    off.init(lane);
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
      for (int mb = 0; mb < C::NDB; ++mb) tro[rd][mb] = tr_lane_elem<typename C::TileL>(lane, rd, mb);
  }

  // kt, vt: row-major K and V tiles (K also read transposed).  mask: the tile
  // may hold keys past the end or above the diagonal for some of this wave's
  // rows.  It is a run-time branch that only sets such scores to -inf (so P
  // = 0): one tile body for every tile, so the dQ accumulators keep one
  // register assignment through the loop.
  __device__ __forceinline__ void tile(bool mask, const uint16_t* kt, const uint16_t* vt, int key0, int Nk,
                                       float scale_log2) {
    f32x16 sacc[C::KB], pacc[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[kb][i] = 0.f;
        pacc[kb][i] = C::DELTA_INIT ? dl16[i] : 0.f;
      }
    if constexpr (STAGED) {
      // DK stages, one k-step of every S^T and dP^T chain each
      constexpr int PF = C::SCORE_PF;
      u32x4 rk[C::DK][C::KB], rv[C::DK][C::KB];
      auto fetch = [&](int s) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          rk[s][kb] = lds_read16(kt + off.rd(s, kb));
          rv[s][kb] = lds_read16(vt + off.rd(s, kb));
        }
      };
#pragma unroll
      for (int s = 0; s < PF; ++s) fetch(s);
#pragma unroll
      for (int s = 0; s < C::DK; ++s) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          sacc[kb] = E::mfma(rk[s][kb], qf[s], sacc[kb]);
          pacc[kb] = E::mfma(rv[s][kb], dof[s], pacc[kb]);
        }
        if (s + PF < C::DK) fetch(s + PF);
        sched_fence();
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int s = 0; s < C::DK; ++s) {
          const int o = off.rd(s, kb);
          sacc[kb] = E::mfma(lds_read16(kt + o), qf[s], sacc[kb]);
          pacc[kb] = E::mfma(lds_read16(vt + o), dof[s], pacc[kb]);
        }
      mfma_pipeline_hint<1, 2 * C::KB * C::DK, 2 * C::KB * C::DK, C::READ_AHEAD>();
    }
    // dQ products t: 16-key chunk t / NDB of feature block t % NDB, K^T by two
    // transposed reads of the K tile (staged: the first ones go out before
    // the exponentials)
    constexpr int R16 = C::TileL::ROWS16;
    constexpr int NT = (C::BC / 16) * C::NDB;
    u32x4 rt[NT];
    auto fetch_t = [&](int t) {
      const int c = t / C::NDB, mb = t % C::NDB;
      rt[t] = lds_read_tr(kt + tro[0][mb] + c * R16, kt + tro[1][mb] + c * R16);
    };
    if constexpr (STAGED)
#pragma unroll
      for (int t = 0; t < C::DQ_PF; ++t) fetch_t(t);
    if (mask) {
      // register i of block kb: key key0 + 4 lh + (kb 32 + 8 (i / 4) + i % 4);
      // one per-lane bound on the constant offset covers both tests (B4 H32
      // N4096 d64 causal dQ -1.1 % on MI355X)
      const int last = CAUSAL ? min(Nk - 1, key_last) : Nk - 1;
      const int lim = last - key0 - 4 * lh;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) sacc[kb][i] = -INFINITY;
    }
    uint32_t dsw[C::KB][8];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2_fast(__builtin_fmaf(sacc[kb][i], scale_log2, -l2));
        pacc[kb][i] = C::DELTA_INIT ? -(p * pacc[kb][i]) : p * (pacc[kb][i] - dl);
      }
#pragma unroll
      for (int i = 0; i < 16; i += 2) dsw[kb][i >> 1] = E::pack2(pacc[kb][i], pacc[kb][i + 1]);
    }
    // dQ^T (d x query) += K^T (d x 16 keys) dS^T (16 keys x query)
    if constexpr (STAGED) {
      sched_fence();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int c = t / C::NDB;
        dqacc[t % C::NDB] = E::mfma(rt[t], acc_chunk(dsw[c >> 1], c & 1), dqacc[t % C::NDB]);
        if (t + C::DQ_PF < NT) fetch_t(t + C::DQ_PF);
        sched_fence();
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int c = t / C::NDB;
        fetch_t(t);
        dqacc[t % C::NDB] = E::mfma(rt[t], acc_chunk(dsw[c >> 1], c & 1), dqacc[t % C::NDB]);
      }
      mfma_pipeline_hint<2, NT, 2 * NT, C::READ_AHEAD, 2>();
    }
  }
};

template <int D, bool CAUSAL, class E>
__global__ __launch_bounds__(DqCfg<D>::THREADS, 1) void bwd_dq_kernel(
    CView Q, CView K, CView V, CView dO, const float* __restrict__ L2,
    const float* __restrict__ Delta, View dQ, int BH, int H, int Nq, int Nk, int Npad, float scale,
    float scale_log2) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][C::TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  // the constant slots of wide rows are zeros, which every copy stores
  static_assert(!C::TileL::HAS_CONST || C::TileL::CONST_ZERO, "copies store the constant slots");
  const int nrb = (Nq + C::BR - 1) / C::BR;
  const int bh = blockIdx.x % BH;
  int rb = blockIdx.x / BH;
  if (CAUSAL) rb = nrb - 1 - rb;

  const uint16_t* Kh = K.head(bh / H, bh % H);
  const uint16_t* Vh = V.head(bh / H, bh % H);
  const uint16_t* Qh = Q.head(bh / H, bh % H);
  const uint16_t* dOh = dO.head(bh / H, bh % H);
  // causal: query i sees keys j <= i + koff (queries aligned to the end of the keys)
  const int koff = Nk - Nq;

  DqWave<D, CAUSAL, E> w;
  w.lane = tid & 63;
  w.lr = w.lane & 31;
  w.lh = w.lane >> 5;
  w.q_wave = rb * C::BR + wave * 32;
  w.q_lane = w.q_wave + w.lr;
  w.key_last = w.q_lane + koff;
  w.init_offsets();

  const int q_first = rb * C::BR;
  int n_tiles = (Nk + C::BC - 1) / C::BC;
  if (CAUSAL) {
    const int last_key = q_first + C::BR - 1 + koff;   // last key any row of the block sees
    n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / C::BC + 1);
  }
  const int n_full = min(n_tiles, (CAUSAL ? max(0, min(q_first + koff + 1, Nk)) : Nk) / C::BC);

  // K and V are copied to LDS directly, in the same layout (one set of lane
  // offsets reads both row-wise).
  TileDma<D, C::BC, C::THREADS, typename C::TileL> kdma, vdma;
  kdma.init(tid, K.sr);
  vdma.init(tid, V.sr);
  if (n_tiles > 0) {
    kdma.issue(k_lds[0], Kh, 0, Nk);
    vdma.issue(v_lds[0], Vh, 0, Nk);
  }

  // Q and dO fragments stay in registers (B operands of K Q^T and V dO^T);
  // rows past Nq read as zero and have L = +inf in the padded L array.
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 zq = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
    if (w.q_lane < Nq) {
      zq = ld_global16(Qh + (size_t)w.q_lane * Q.sr + s * 16 + 8 * w.lh);
      zd = ld_global16(dOh + (size_t)w.q_lane * dO.sr + s * 16 + 8 * w.lh);
    }
    w.qf[s] = zq;
    w.dof[s] = C::DELTA_INIT ? zd ^ 0x80008000u : zd;
  }
  w.l2 = L2[(size_t)bh * Npad + w.q_lane];
  w.dl = Delta[(size_t)bh * Npad + w.q_lane];
#pragma unroll
  for (int i = 0; i < 16; ++i) w.dl16[i] = w.dl;
#pragma unroll
  for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.dqacc[mb][i] = 0.f;

  auto iteration = [&](auto buf_tag, int j) {
    constexpr int BUF = decltype(buf_tag)::value;
    wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) {
      kdma.issue(k_lds[BUF ^ 1], Kh, (j + 1) * C::BC, Nk);
      vdma.issue(v_lds[BUF ^ 1], Vh, (j + 1) * C::BC, Nk);
    }
    const int key0 = j * C::BC;
    // tiles from n_full on are masked; a wavefront whose rows all precede the
    // tile's first key has nothing to do.  Without the causal mask every tile
    // is visited; at D = 256 that is written as the same run-time test with a
    // bound past every key (Nq + Nk), because the straight-line loop the
    // compiler otherwise builds needs more than the 512 registers of a lane.
    const bool visit = CAUSAL ? (j < n_full || key0 <= w.q_wave + 31 + koff)
                              : (D != 256 || key0 <= w.q_wave + 31 + koff + Nq + Nk);
    if (visit) w.tile(j >= n_full, k_lds[BUF], v_lds[BUF], key0, Nk, scale_log2);
  };
  for (int j = 0; j < n_tiles; j += 2) {
    iteration(std::integral_constant<int, 0>{}, j);
    if (j + 1 < n_tiles) iteration(std::integral_constant<int, 1>{}, j + 1);
  }

  // Epilogue: dQ = scale * dS K (bf16).
  if (w.q_lane < Nq) {
    uint16_t* row = dQ.head(bh / H, bh % H) + (size_t)w.q_lane * dQ.sr;
#pragma unroll
    for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * w.lh;
        if (d0 < D) {
          u32x2 v = {E::pack2(w.dqacc[mb][4 * g] * scale, w.dqacc[mb][4 * g + 1] * scale),
                     E::pack2(w.dqacc[mb][4 * g + 2] * scale, w.dqacc[mb][4 * g + 3] * scale)};
          *reinterpret_cast<u32x2*>(row + d0) = v;
        }
      }
  }
}

template <int D, class E>
hipError_t launch_pre_t(const Strided& o, const Strided& dout, const float* lse, float* delta,
                        float* l2, int B, int H, int N, hipStream_t stream) {
  const int Npad = bwd_rows_padded(N);
  const long rows_pad = (long)B * H * Npad;
  bwd_preprocess_kernel<D, E><<<dim3((unsigned)((rows_pad + kPreRows - 1) / kPreRows)), 256, 0, stream>>>(
      cview(o), cview(dout), lse, delta, l2, H, N, Npad, rows_pad);
  return hipGetLastError();
}

template <int D, bool CAUSAL, class E>
hipError_t launch_dkdv_t(const Strided& q, const Strided& k, const Strided& v, const Strided& dout,
                         const float* l2, const float* delta, const Strided& dk, const Strided& dv,
                         int B, int H, int Nq, int Nk, float scale, hipStream_t stream) {
  if constexpr (D == 256) {
    using C = DkdvSplitCfg<D>;
    const int nkb = (Nk + C::BKC - 1) / C::BKC;
    bwd_dkdv_split_kernel<D, CAUSAL, E><<<dim3((unsigned)(nkb * B * H)), C::THREADS, 0, stream>>>(
        cview(q), cview(k), cview(v), cview(dout), l2, delta, view(dk), view(dv), B * H, H, Nq, Nk,
        bwd_rows_padded(Nq), scale, scale * kLog2e);
  } else {
    using C = DkdvCfg<D>;
    const int nkb = (Nk + C::BKC - 1) / C::BKC;
    bwd_dkdv_kernel<D, CAUSAL, E><<<dim3((unsigned)(nkb * B * H)), C::THREADS, 0, stream>>>(
        cview(q), cview(k), cview(v), cview(dout), l2, delta, view(dk), view(dv), B * H, H, Nq, Nk,
        bwd_rows_padded(Nq), scale, scale * kLog2e);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL, class E>
hipError_t launch_dq_t(const Strided& q, const Strided& k, const Strided& v, const Strided& dout,
                       const float* l2, const float* delta, const Strided& dq, int B, int H, int Nq,
                       int Nk, float scale, hipStream_t stream) {
  using C = DqCfg<D>;
  const int nrb = (Nq + C::BR - 1) / C::BR;
  bwd_dq_kernel<D, CAUSAL, E><<<dim3((unsigned)(nrb * B * H)), C::THREADS, 0, stream>>>(
      cview(q), cview(k), cview(v), cview(dout), l2, delta, view(dq), B * H, H, Nq, Nk,
      bwd_rows_padded(Nq), scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

#if FA2_DQ256_UNIT
// The dQ kernel at head dimension 256 (one wavefront per SIMD) is compiled in
// a unit of its own (fa2_bwd_dq256.hip), without the MFMA register form the
// other backward kernels are built with (build.py): its dQ accumulators are
// only ever MFMA operands and belong in the accumulator registers.
hipError_t launch_bwd_dq_d256(const Strided& q, const Strided& k, const Strided& v, const Strided& dout,
                              const float* l2, const float* delta, const Strided& dq, int B, int H,
                              int Nq, int Nk, float scale, int causal, int dtype, hipStream_t stream) {
  return dispatch(256, causal, dtype, [&](auto dc, auto cc, auto ec) {
    if constexpr (decltype(dc)::value == 256)
      return launch_dq_t<256, decltype(cc)::value, decltype(ec)>(q, k, v, dout, l2, delta, dq, B, H, Nq, Nk,
                                                               scale, stream);
    return hipErrorInvalidValue;
  });
}
#else
hipError_t launch_bwd_preprocess(const Strided& o, const Strided& dout, const float* lse,
                                 float* delta, float* l2, int B, int H, int N, int d, int dtype,
                                 hipStream_t stream) {
  return dispatch(d, 0, dtype, [&](auto dc, auto, auto ec) {
    return launch_pre_t<decltype(dc)::value, decltype(ec)>(o, dout, lse, delta, l2, B, H, N, stream);
  });
}

hipError_t launch_bwd_dkdv(const Strided& q, const Strided& k, const Strided& v,
                           const Strided& dout, const float* l2, const float* delta,
                           const Strided& dk, const Strided& dv, int B, int H, int Nq, int Nk,
                           int d, float scale, int causal, int dtype, hipStream_t stream) {
  return dispatch(d, causal, dtype, [&](auto dc, auto cc, auto ec) {
    return launch_dkdv_t<decltype(dc)::value, decltype(cc)::value, decltype(ec)>(
        q, k, v, dout, l2, delta, dk, dv, B, H, Nq, Nk, scale, stream);
  });
}

hipError_t launch_bwd_dq(const Strided& q, const Strided& k, const Strided& v, const Strided& dout,
                         const float* l2, const float* delta, const Strided& dq, int B, int H,
                         int Nq, int Nk, int d, float scale, int causal, int dtype,
                         hipStream_t stream) {
  if (d == 256) return launch_bwd_dq_d256(q, k, v, dout, l2, delta, dq, B, H, Nq, Nk, scale, causal, dtype, stream);
  return dispatch(d, causal, dtype, [&](auto dc, auto cc, auto ec) {
    if constexpr (decltype(dc)::value == 256) return hipErrorInvalidValue;   // launch_bwd_dq_d256
    else
      return launch_dq_t<decltype(dc)::value, decltype(cc)::value, decltype(ec)>(
          q, k, v, dout, l2, delta, dq, B, H, Nq, Nk, scale, stream);
  });
}

void bwd_tiles(int d, int* block_k, int* block_q, int* waves) {
  if (d == 256) {
    *block_k = DkdvSplitCfg<256>::BKC;
    *block_q = DkdvSplitCfg<256>::BQ;
    *waves = DkdvSplitCfg<256>::WAVES;
    return;
  }
  *block_k = DkdvCfg<128>::BKC;
  *block_q = DkdvCfg<128>::BQ;
  *waves = DkdvCfg<128>::WAVES;
}
#endif

}  // namespace fa2
