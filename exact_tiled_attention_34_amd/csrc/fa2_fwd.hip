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
//                          O *= 2^(c(m-m'))
//   O^T += V^T P^T         bf16 MFMA, P packed to bf16 straight from registers
// After the last tile, O is divided by l once ("FlashAttention-2" summary page,
// "How It Works" 2) and L = (c m + log2 l) ln 2 is stored.
//
// K/V tiles are staged global -> registers -> LDS, double-buffered so the
// loads of tile j+1 are in flight while tile j is multiplied.
#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BR = 32 * WAVES;           // query rows per workgroup
  static constexpr int BC = 64;                   // keys per K/V tile
  static constexpr int DP = (D + 31) / 32 * 32;   // O^T rows padded to whole 32-row MFMA blocks
  static constexpr int DK = D / 16;               // k-steps of Q K^T
  static constexpr int CH = D / 8;                // 16-byte chunks per row
  static constexpr int KROW = D + 8;              // bf16 per K row in LDS (16 B of padding)
  static constexpr int KBUF = BC * KROW;          // bf16 per K buffer
  static constexpr int VBUF = DP * BC;            // bf16 per V^T buffer
  static constexpr int KUNITS = BC * CH;          // 16-byte K loads per tile
  static constexpr int KLOADS = (KUNITS + THREADS - 1) / THREADS;
  static constexpr int VUNITS = (BC / 4) * CH;    // 4-key x 8-dim V blocks per tile
  static_assert(VUNITS <= THREADS, "one V block per thread");
  static_assert(D % 16 == 0, "head dim must be a multiple of 16");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int BH, int N, float scale_log2) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2 * C::KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2 * C::VBUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // Linear workgroup id -> (row block, batch*head).  Consecutive ids take
  // different heads, so with the round-robin dispatch over the 8 XCDs all row
  // blocks of one head land on the same XCD (and its L2).  Causal: the longest
  // row blocks (most tiles) are dispatched first.
  const int nrb = (N + C::BR - 1) / C::BR;
  const int bh = blockIdx.x % BH;
  int rb = blockIdx.x / BH;
  if (CAUSAL) rb = nrb - 1 - rb;

  const size_t head_off = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head_off;
  const uint16_t* Kh = K + head_off;
  const uint16_t* Vh = V + head_off;

  const int q_wave = rb * C::BR + wave * 32;   // first query row of this wavefront
  const int q_lane = q_wave + lr;              // the query row this lane owns

  // Q fragments stay in registers for the whole pass (B operand of S^T = K Q^T).
  bf16x8 qf[C::DK];
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (q_lane < N) z = ld_global16(Qh + (size_t)q_lane * D + s * 16 + 8 * lh);
    qf[s] = as_bf16x8(z);
  }

  int n_tiles = (N + C::BC - 1) / C::BC;
  if (CAUSAL) n_tiles = min(n_tiles, (rb * C::BR + C::BR - 1) / C::BC + 1);

  // Padding rows of V^T (d >= D, only when D is not a multiple of 32) stay zero.
  if (C::DP != D) {
    for (int i = tid; i < 2 * (C::DP - D) * C::BC; i += C::THREADS) {
      const int buf = i / ((C::DP - D) * C::BC);
      const int rem = i % ((C::DP - D) * C::BC);
      v_lds[buf * C::VBUF + (D + rem / C::BC) * C::BC + rem % C::BC] = 0;
    }
  }

  u32x4 kreg[C::KLOADS];
  u32x4 vreg[4];

  auto load_tile = [&](int j) {
    const int key0 = j * C::BC;
#pragma unroll
    for (int t = 0; t < C::KLOADS; ++t) {
      const int u = tid + t * C::THREADS;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (u < C::KUNITS) {
        const int row = u / C::CH, ch = u % C::CH;
        if (key0 + row < N) z = ld_global16(Kh + (size_t)(key0 + row) * D + ch * 8);
      }
      kreg[t] = z;
    }
    if (tid < C::VUNITS) {
      const int g = tid / C::CH, ch = tid % C::CH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 4 * g + r;
        u32x4 z = {0u, 0u, 0u, 0u};
        if (key < N) z = ld_global16(Vh + (size_t)key * D + ch * 8);
        vreg[r] = z;
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* kb = k_lds + buf * C::KBUF;
#pragma unroll
    for (int t = 0; t < C::KLOADS; ++t) {
      const int u = tid + t * C::THREADS;
      if (u < C::KUNITS) {
        const int row = u / C::CH, ch = u % C::CH;
        st_lds16(kb + row * C::KROW + ch * 8, kreg[t]);
      }
    }
    if (tid < C::VUNITS) {
      // 4 keys x 8 dims -> 8 rows of V^T, 4 keys (8 bytes) each.
      uint16_t* vb = v_lds + buf * C::VBUF;
      const int g = tid / C::CH, ch = tid % C::CH;
      const int pos = tok_perm(4 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t a0 = vreg[0][w], a1 = vreg[1][w], a2 = vreg[2][w], a3 = vreg[3][w];
        uint32_t lo, hi;
        if (e & 1) {
          lo = (a0 >> 16) | (a1 & 0xffff0000u);
          hi = (a2 >> 16) | (a3 & 0xffff0000u);
        } else {
          lo = (a0 & 0xffffu) | (a1 << 16);
          hi = (a2 & 0xffffu) | (a3 << 16);
        }
        u32x2 pr = {lo, hi};
        st_lds8(vb + tr64_offset(ch * 8 + e, pos), pr);
      }
    }
  };

  f32x16 oacc[C::DP / 32];
#pragma unroll
  for (int mb = 0; mb < C::DP / 32; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mb][i] = 0.f;
  float m_run = -INFINITY;   // running max of the raw scores q.k
  float l_run = 0.f;         // this lane's share of the running row sum

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    const int key0 = j * C::BC;
    // A wavefront whose rows all precede the tile's first key has nothing to do.
    const bool active = !CAUSAL || key0 <= q_wave + 31;
    if (active) {
      const uint16_t* kb = k_lds + buf * C::KBUF;
      const uint16_t* vb = v_lds + buf * C::VBUF;
      f32x16 sacc[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb2][i] = 0.f;
#pragma unroll
        for (int s = 0; s < C::DK; ++s) {
          const bf16x8 a = ld_lds16(kb + (kb2 * 32 + lr) * C::KROW + s * 16 + 8 * lh);
          sacc[kb2] = mfma32x32x16(a, qf[s], sacc[kb2]);
        }
      }
      const bool need_mask = (CAUSAL && key0 + C::BC - 1 > q_wave) || (key0 + C::BC > N);
      if (need_mask) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kb2 * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
            if (key >= N || (CAUSAL && key > q_lane)) sacc[kb2][i] = -INFINITY;
          }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb2][i]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast((m_run - m_new) * scale_log2);
      const float mc = m_new * scale_log2;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < C::DP / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] *= alpha;

      uint32_t pw[2][8];
      float rs = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = exp2_fast(__builtin_fmaf(sacc[kb2][i], scale_log2, -mc));
          const float p1 = exp2_fast(__builtin_fmaf(sacc[kb2][i + 1], scale_log2, -mc));
          rs += p0 + p1;
          pw[kb2][i >> 1] = pack_bf16x2(p0, p1);
        }
      l_run += rs;

      // O^T (d x query) += V^T (d x 16 keys) * P^T (16 keys x query), four key chunks.
#pragma unroll
      for (int c = 0; c < C::BC / 16; ++c) {
        u32x4 bw = {pw[c >> 1][(c & 1) * 4 + 0], pw[c >> 1][(c & 1) * 4 + 1],
                    pw[c >> 1][(c & 1) * 4 + 2], pw[c >> 1][(c & 1) * 4 + 3]};
        const bf16x8 b = as_bf16x8(bw);
#pragma unroll
        for (int mb = 0; mb < C::DP / 32; ++mb) {
          const bf16x8 a = ld_lds16(vb + tr64_offset(mb * 32 + lr, 16 * c + 8 * lh));
          oacc[mb] = mfma32x32x16(a, b, oacc[mb]);
        }
      }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: one division by the row sum, then O (bf16) and L (fp32, natural log).
  const float l_tot = l_run + swap_halves(l_run);
  if (q_lane < N) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = O + head_off + (size_t)q_lane * D;
#pragma unroll
    for (int mb = 0; mb < C::DP / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * lh;
        if (d0 < D) {
          u32x2 w = {pack_bf16x2(oacc[mb][4 * g + 0] * inv, oacc[mb][4 * g + 1] * inv),
                     pack_bf16x2(oacc[mb][4 * g + 2] * inv, oacc[mb][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      }
    if (lh == 0) LSE[(size_t)bh * N + q_lane] = (m_run * scale_log2 + log2_fast(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, float scale, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int BH = B * H;
  const int nrb = (N + C::BR - 1) / C::BR;
  const dim3 grid((unsigned)(nrb * BH));
  fwd_kernel<D, CAUSAL><<<grid, C::THREADS, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, BH, N, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  switch (d) {
    case 64:  return causal ? launch_fwd_t<64, true>(q, k, v, o, lse, B, H, N, scale, stream)
                            : launch_fwd_t<64, false>(q, k, v, o, lse, B, H, N, scale, stream);
    case 80:  return causal ? launch_fwd_t<80, true>(q, k, v, o, lse, B, H, N, scale, stream)
                            : launch_fwd_t<80, false>(q, k, v, o, lse, B, H, N, scale, stream);
    case 128: return causal ? launch_fwd_t<128, true>(q, k, v, o, lse, B, H, N, scale, stream)
                            : launch_fwd_t<128, false>(q, k, v, o, lse, B, H, N, scale, stream);
    default:  return hipErrorInvalidValue;
  }
}

void fwd_tiles(int d, int* block_q, int* block_k, int* waves) {
  (void)d;
  *block_q = FwdCfg<128>::BR;
  *block_k = FwdCfg<128>::BC;
  *waves = FwdCfg<128>::WAVES;
}

}  // namespace fa2
