// Internal launch interface between the C ABI (fa2_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fa2 {

// A bf16 [B, H, N, d] tensor with a contiguous last dimension: element
// (b, h, n, i) at p + b*batch + h*head + n*row + i (element strides).
struct Strided {
  const void* p;
  long long batch, head, row;
};
// The contiguous layout of [B, H, N, d].
inline Strided contiguous(const void* p, int H, int N, int d) {
  return Strided{p, (long long)H * N * d, (long long)N * d, d};
}

// Query rows Nq (q, o, lse, dout, dq, row arrays), key rows Nk (k, v, dk, dv).
// dtype: 0 = bfloat16, 1 = float16 (all 16-bit tensors of a call share it).
hipError_t launch_fwd(const Strided& q, const Strided& k, const Strided& v, const Strided& o,
                      float* lse, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      int dtype, hipStream_t stream);

// Rows per (batch, head) of the padded fp32 arrays the backward kernels read.
int bwd_rows_padded(int N);

hipError_t launch_bwd_preprocess(const Strided& o, const Strided& dout, const float* lse,
                                 float* delta, float* lse_log2, int B, int H, int N, int d,
                                 int dtype, hipStream_t stream);

hipError_t launch_bwd_dkdv(const Strided& q, const Strided& k, const Strided& v,
                           const Strided& dout, const float* lse_log2, const float* delta,
                           const Strided& dk, const Strided& dv, int B, int H, int Nq, int Nk,
                           int d, float scale, int causal, int dtype, hipStream_t stream);

hipError_t launch_bwd_dq(const Strided& q, const Strided& k, const Strided& v, const Strided& dout,
                         const float* lse_log2, const float* delta, const Strided& dq, int B, int H,
                         int Nq, int Nk, int d, float scale, int causal, int dtype,
                         hipStream_t stream);

// launch_bwd_dq at head dimension 256 (its own compilation unit)
hipError_t launch_bwd_dq_d256(const Strided& q, const Strided& k, const Strided& v, const Strided& dout,
                              const float* lse_log2, const float* delta, const Strided& dq, int B, int H,
                              int Nq, int Nk, float scale, int causal, int dtype, hipStream_t stream);

void fwd_tiles(int d, int* block_q, int* block_k, int* waves);
void bwd_tiles(int d, int* block_k, int* block_q, int* waves);

}  // namespace fa2
