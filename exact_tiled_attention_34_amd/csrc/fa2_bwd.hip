// Backward pass of exact tiled attention on gfx950.
//
// Three kernels, enqueued in order by fa2_bwd:
//   preprocess   delta_i = sum_k dO_ik O_ik (fp32) and the fp32 dQ accumulator
//                cleared; HBM-bound, 16 lanes per row.
//   dkdv         one workgroup per (key column-block of 128, batch*head); each
//                of its 4 wavefronts owns 32 keys and keeps K, V (as MFMA
//                operands) and the dK, dV accumulators in registers while it
//                walks the 64-query row-blocks that can see those keys
//                (causal: from the diagonal on; blocks wholly above it are
//                never visited, the diagonal ones are masked element-wise).
//                Per step, with P recomputed from the stored L:
//                  S  = Q K^T           P = 2^(c S - L log2 e), c = scale log2 e
//                  dP = dO V^T          dS = P (dP - delta)
//                  dV^T += dO^T P       dK^T += Q^T dS
//                  dQ  += dS K          (fp32 atomics into the accumulator)
//                dS is the only tile that must change orientation (the S
//                layout gives each lane one key; dQ needs 8 keys per lane), so
//                it makes one round trip through LDS.
//   dq_convert   dq = bf16(scale * accumulator): the softmax scale is applied
//                once at the end ("FlashAttention-2" summary page, "How It
//                Works" 2), as it is for dK in dkdv's epilogue.
#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {
namespace {

// ---------------------------------------------------------------------------
// preprocess
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    float* __restrict__ Delta, float* __restrict__ dQacc, long rows) {
  constexpr int CH = D / 8;
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    for (int ch = sub; ch < CH; ch += 16) {
      const u32x4 o = ld_global16(O + row * D + ch * 8);
      const u32x4 g = ld_global16(dO + row * D + ch * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        acc += bf16lo(o[w]) * bf16lo(g[w]) + bf16hi(o[w]) * bf16hi(g[w]);
      u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dQacc + row * D + ch * 8) = z;
      *reinterpret_cast<u32x4*>(dQacc + row * D + ch * 8 + 4) = z;
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && sub == 0) Delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV (+ atomic dQ)
// ---------------------------------------------------------------------------
template <int D>
struct BwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BKC = 32 * WAVES;          // keys per workgroup
  static constexpr int BQ = 64;                   // queries per step
  static constexpr int DP = (D + 31) / 32 * 32;   // feature rows padded to whole MFMA blocks
  static constexpr int DK = D / 16;               // k-steps over the head dimension
  static constexpr int CH = D / 8;                // 16-byte chunks per row
  static constexpr int QROW = D + 8;              // bf16 per Q / dO row in LDS
  static constexpr int SROW = BKC + 8;            // bf16 per dS row and per K^T row
  static constexpr int QBUF = BQ * QROW;
  static constexpr int TBUF = DP * BQ;            // Q^T / dO^T: DP rows of 64 queries
  static constexpr int SBUF = BQ * SROW;
  static constexpr int KTBUF = DP * SROW;
  static constexpr int QUNITS = (BQ / 4) * CH;    // 4-query x 8-dim blocks per step
  static constexpr int KTUNITS = (BKC / 4) * CH;  // 4-key x 8-dim blocks of K
  static constexpr int NQB = BQ / 32;
  static constexpr int NDB = DP / 32;
  static constexpr int DQBLOCKS = NQB * NDB;
  static_assert(QUNITS <= THREADS, "one Q/dO block per thread");
};

// Transpose a 4-token x 8-feature block (4 rows of 16 bytes) into feature row e
// (4 tokens, 8 bytes).
__device__ __forceinline__ u32x2 tr4x8_row(const u32x4* r, int e) {
  const int w = e >> 1;
  const uint32_t a0 = r[0][w], a1 = r[1][w], a2 = r[2][w], a3 = r[3][w];
  u32x2 out;
  if (e & 1) {
    out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
    out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
  } else {
    out[0] = (a0 & 0xffffu) | (a1 << 16);
    out[1] = (a2 & 0xffffu) | (a3 << 16);
  }
  return out;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const float* __restrict__ LSE,
    const uint16_t* __restrict__ dO, const float* __restrict__ Delta,
    float* __restrict__ dQacc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int BH, int N, float scale, float scale_log2) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[C::QBUF];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[C::QBUF];
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds[C::TBUF];
  __shared__ __attribute__((aligned(16))) uint16_t dot_lds[C::TBUF];
  __shared__ __attribute__((aligned(16))) uint16_t ds_lds[C::SBUF];
  __shared__ __attribute__((aligned(16))) uint16_t kt_lds[C::KTBUF];
  __shared__ __attribute__((aligned(16))) float l_lds[C::BQ];
  __shared__ __attribute__((aligned(16))) float dl_lds[C::BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // Linear id -> (key block, batch*head); consecutive ids take different heads
  // (XCD round-robin keeps one head's blocks on one XCD).  Key block 0 sees the
  // most query blocks under a causal mask, so it is dispatched first.
  const int bh = blockIdx.x % BH;
  const int kblk = blockIdx.x / BH;
  const size_t head_off = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head_off;
  const uint16_t* Kh = K + head_off;
  const uint16_t* Vh = V + head_off;
  const uint16_t* dOh = dO + head_off;
  const float* Lh = LSE + (size_t)bh * N;
  const float* Dh = Delta + (size_t)bh * N;
  float* dQh = dQacc + head_off;

  const int key_wg = kblk * C::BKC;
  const int key_w = key_wg + wave * 32;
  const int key_lane = key_w + lr;

  // K, V as B operands (lane: one key, 8 consecutive features per k-step).
  bf16x8 kf[C::DK], vf[C::DK];
#pragma unroll
  for (int s = 0; s < C::DK; ++s) {
    u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
    if (key_lane < N) {
      zk = ld_global16(Kh + (size_t)key_lane * D + s * 16 + 8 * lh);
      zv = ld_global16(Vh + (size_t)key_lane * D + s * 16 + 8 * lh);
    }
    kf[s] = as_bf16x8(zk);
    vf[s] = as_bf16x8(zv);
  }

  // K^T (feature rows, the workgroup's 128 keys in order) for dQ = dS K.
  for (int u = tid; u < C::KTUNITS; u += C::THREADS) {
    const int g = u / C::CH, ch = u % C::CH;
    u32x4 r[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = key_wg + 4 * g + t;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (key < N) z = ld_global16(Kh + (size_t)key * D + ch * 8);
      r[t] = z;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) st_lds8(kt_lds + (ch * 8 + e) * C::SROW + 4 * g, tr4x8_row(r, e));
  }
  if (C::DP != D) {
    // padded feature rows contribute zeros
    for (int i = tid; i < (C::DP - D) * C::SROW; i += C::THREADS) kt_lds[D * C::SROW + i] = 0;
    for (int i = tid; i < (C::DP - D) * C::BQ; i += C::THREADS) {
      qt_lds[D * C::BQ + i] = 0;
      dot_lds[D * C::BQ + i] = 0;
    }
  }

  f32x16 dkacc[C::NDB], dvacc[C::NDB];
#pragma unroll
  for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[mb][i] = 0.f;
      dvacc[mb][i] = 0.f;
    }

  const int n_qblk = (N + C::BQ - 1) / C::BQ;
  const int i_begin = CAUSAL ? key_wg / C::BQ : 0;

  u32x4 qreg[4], doreg[4];
  float lreg = 0.f, dreg = 0.f;
  auto load_step = [&](int i) {
    const int q0 = i * C::BQ;
    if (tid < C::QUNITS) {
      const int g = tid / C::CH, ch = tid % C::CH;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int q = q0 + 4 * g + t;
        u32x4 zq = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
        if (q < N) {
          zq = ld_global16(Qh + (size_t)q * D + ch * 8);
          zd = ld_global16(dOh + (size_t)q * D + ch * 8);
        }
        qreg[t] = zq;
        doreg[t] = zd;
      }
    }
    if (tid < C::BQ) {
      const int q = q0 + tid;
      // rows past the end get L = +inf, hence P = 0
      lreg = q < N ? Lh[q] * kLog2e : INFINITY;
      dreg = q < N ? Dh[q] : 0.f;
    }
  };
  auto store_step = [&]() {
    if (tid < C::QUNITS) {
      const int g = tid / C::CH, ch = tid % C::CH;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        st_lds16(q_lds + (4 * g + t) * C::QROW + ch * 8, qreg[t]);
        st_lds16(do_lds + (4 * g + t) * C::QROW + ch * 8, doreg[t]);
      }
      const int pos = tok_perm(4 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        st_lds8(qt_lds + tr64_offset(ch * 8 + e, pos), tr4x8_row(qreg, e));
        st_lds8(dot_lds + tr64_offset(ch * 8 + e, pos), tr4x8_row(doreg, e));
      }
    }
    if (tid < C::BQ) {
      l_lds[tid] = lreg;
      dl_lds[tid] = dreg;
    }
  };

  if (i_begin < n_qblk) load_step(i_begin);
  for (int i = i_begin; i < n_qblk; ++i) {
    __syncthreads();   // previous step's readers are done with every LDS tile
    store_step();
    __syncthreads();
    if (i + 1 < n_qblk) load_step(i + 1);

    const int q0 = i * C::BQ;
    const bool active = !CAUSAL || key_w <= q0 + C::BQ - 1;
    if (active) {
      f32x16 sacc[C::NQB], pacc[C::NQB];
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          sacc[qb][t] = 0.f;
          pacc[qb][t] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < C::DK; ++s) {
          const bf16x8 a = ld_lds16(q_lds + (qb * 32 + lr) * C::QROW + s * 16 + 8 * lh);
          sacc[qb] = mfma32x32x16(a, kf[s], sacc[qb]);
          const bf16x8 a2 = ld_lds16(do_lds + (qb * 32 + lr) * C::QROW + s * 16 + 8 * lh);
          pacc[qb] = mfma32x32x16(a2, vf[s], pacc[qb]);
        }
      }
      const bool need_mask = (CAUSAL && key_w + 31 > q0) || (key_w + 32 > N);
      uint32_t pw[C::NQB][8], dsw[C::NQB][8];
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = qb * 32 + 8 * g + 4 * lh;   // local index of 4 consecutive queries
          const float4 lv = *reinterpret_cast<const float4*>(l_lds + ql);
          const float4 dv = *reinterpret_cast<const float4*>(dl_lds + ql);
          const float lvs[4] = {lv.x, lv.y, lv.z, lv.w};
          const float dvs[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            float p = exp2_fast(__builtin_fmaf(sacc[qb][t], scale_log2, -lvs[r]));
            if (need_mask && (key_lane >= N || (CAUSAL && key_lane > q0 + ql + r))) p = 0.f;
            sacc[qb][t] = p;
            pacc[qb][t] = p * (pacc[qb][t] - dvs[r]);
          }
        }
#pragma unroll
        for (int t = 0; t < 16; t += 2) {
          pw[qb][t >> 1] = pack_bf16x2(sacc[qb][t], sacc[qb][t + 1]);
          dsw[qb][t >> 1] = pack_bf16x2(pacc[qb][t], pacc[qb][t + 1]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per MFMA.
#pragma unroll
      for (int c = 0; c < C::BQ / 16; ++c) {
        const int qb = c >> 1, h8 = (c & 1) * 4;
        u32x4 bp = {pw[qb][h8], pw[qb][h8 + 1], pw[qb][h8 + 2], pw[qb][h8 + 3]};
        u32x4 bs = {dsw[qb][h8], dsw[qb][h8 + 1], dsw[qb][h8 + 2], dsw[qb][h8 + 3]};
#pragma unroll
        for (int mb = 0; mb < C::NDB; ++mb) {
          const int off = tr64_offset(mb * 32 + lr, 16 * c + 8 * lh);
          dvacc[mb] = mfma32x32x16(ld_lds16(dot_lds + off), as_bf16x8(bp), dvacc[mb]);
          dkacc[mb] = mfma32x32x16(ld_lds16(qt_lds + off), as_bf16x8(bs), dkacc[mb]);
        }
      }
      // dS -> LDS, rows = queries, this wavefront's 32 key columns.
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int ql = qb * 32 + 8 * (t >> 2) + 4 * lh + (t & 3);
          const uint32_t w = dsw[qb][t >> 1];
          ds_lds[ql * C::SROW + wave * 32 + lr] = (t & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
        }
    } else {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int ql = qb * 32 + 8 * (t >> 2) + 4 * lh + (t & 3);
          ds_lds[ql * C::SROW + wave * 32 + lr] = 0;
        }
    }
    __syncthreads();

    // dQ (BQ x D) += dS (BQ x 128 keys) K (128 keys x D); unscaled, fp32 atomics.
    for (int b = wave; b < C::DQBLOCKS; b += C::WAVES) {
      const int qb = b / C::NDB, nb = b % C::NDB;
      f32x16 acc;
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[t] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::BKC / 16; ++ks) {
        const bf16x8 a = ld_lds16(ds_lds + (qb * 32 + lr) * C::SROW + ks * 16 + 8 * lh);
        const bf16x8 bb = ld_lds16(kt_lds + (nb * 32 + lr) * C::SROW + ks * 16 + 8 * lh);
        acc = mfma32x32x16(a, bb, acc);
      }
      const int dcol = nb * 32 + lr;
      if (dcol < D) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int q = q0 + qb * 32 + 8 * (t >> 2) + 4 * lh + (t & 3);
          if (q < N) unsafeAtomicAdd(dQh + (size_t)q * D + dcol, acc[t]);
        }
      }
    }
  }

  // Epilogue: dK = scale * dS^T Q, dV = P^T dO (bf16).
  if (key_lane < N) {
    uint16_t* dkrow = dK + head_off + (size_t)key_lane * D;
    uint16_t* dvrow = dV + head_off + (size_t)key_lane * D;
#pragma unroll
    for (int mb = 0; mb < C::NDB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * lh;
        if (d0 < D) {
          u32x2 wk = {pack_bf16x2(dkacc[mb][4 * g] * scale, dkacc[mb][4 * g + 1] * scale),
                      pack_bf16x2(dkacc[mb][4 * g + 2] * scale, dkacc[mb][4 * g + 3] * scale)};
          u32x2 wv = {pack_bf16x2(dvacc[mb][4 * g], dvacc[mb][4 * g + 1]),
                      pack_bf16x2(dvacc[mb][4 * g + 2], dvacc[mb][4 * g + 3])};
          *reinterpret_cast<u32x2*>(dkrow + d0) = wk;
          *reinterpret_cast<u32x2*>(dvrow + d0) = wv;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dQ convert: dq = bf16(scale * accumulator), 8 values per thread
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         uint16_t* __restrict__ dq, long n8,
                                                         float scale) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(acc + 8 * i);
    const u32x4 b = *reinterpret_cast<const u32x4*>(acc + 8 * i + 4);
    u32x4 out = {pack_bf16x2(__uint_as_float(a[0]) * scale, __uint_as_float(a[1]) * scale),
                 pack_bf16x2(__uint_as_float(a[2]) * scale, __uint_as_float(a[3]) * scale),
                 pack_bf16x2(__uint_as_float(b[0]) * scale, __uint_as_float(b[1]) * scale),
                 pack_bf16x2(__uint_as_float(b[2]) * scale, __uint_as_float(b[3]) * scale)};
    *reinterpret_cast<u32x4*>(dq + 8 * i) = out;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const void* q, const void* k, const void* v, const float* lse,
                         const void* dout, const float* delta, float* dq_accum, void* dk, void* dv,
                         int B, int H, int N, float scale, hipStream_t stream) {
  using C = BwdCfg<D>;
  const int BH = B * H;
  const int nkb = (N + C::BKC - 1) / C::BKC;
  bwd_dkdv_kernel<D, CAUSAL><<<dim3((unsigned)(nkb * BH)), C::THREADS, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), lse, static_cast<const uint16_t*>(dout), delta, dq_accum,
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), BH, N, scale, scale * kLog2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pre_t(const void* o, const void* dout, float* delta, float* dq_accum, long rows,
                        hipStream_t stream) {
  const unsigned blocks = (unsigned)((rows + 15) / 16);
  bwd_preprocess_kernel<D><<<dim3(blocks), 256, 0, stream>>>(
      static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), delta, dq_accum, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, float* dq_accum,
                                 int B, int H, int N, int d, hipStream_t stream) {
  const long rows = (long)B * H * N;
  switch (d) {
    case 64:  return launch_pre_t<64>(o, dout, delta, dq_accum, rows, stream);
    case 80:  return launch_pre_t<80>(o, dout, delta, dq_accum, rows, stream);
    case 128: return launch_pre_t<128>(o, dout, delta, dq_accum, rows, stream);
    default:  return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, const float* delta, float* dq_accum, void* dk,
                           void* dv, int B, int H, int N, int d, float scale, int causal,
                           hipStream_t stream) {
#define FA2_DKDV(DD)                                                                         \
  return causal ? launch_dkdv_t<DD, true>(q, k, v, lse, dout, delta, dq_accum, dk, dv, B, H, \
                                          N, scale, stream)                                  \
                : launch_dkdv_t<DD, false>(q, k, v, lse, dout, delta, dq_accum, dk, dv, B, H, \
                                           N, scale, stream)
  switch (d) {
    case 64:  FA2_DKDV(64);
    case 80:  FA2_DKDV(80);
    case 128: FA2_DKDV(128);
    default:  return hipErrorInvalidValue;
  }
#undef FA2_DKDV
}

hipError_t launch_bwd_dq_convert(const float* dq_accum, void* dq, int B, int H, int N, int d,
                                 float scale, hipStream_t stream) {
  const long n8 = (long)B * H * N * d / 8;
  long blocks = (n8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  dq_convert_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(
      dq_accum, static_cast<uint16_t*>(dq), n8, scale);
  return hipGetLastError();
}

void bwd_tiles(int d, int* block_k, int* block_q, int* waves) {
  (void)d;
  *block_k = BwdCfg<128>::BKC;
  *block_q = BwdCfg<128>::BQ;
  *waves = BwdCfg<128>::WAVES;
}

}  // namespace fa2
