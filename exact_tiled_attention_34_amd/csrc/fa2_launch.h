// Internal launch interface between the C ABI (fa2_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fa2 {

// Query rows Nq (q, o, lse, dout, dq, row arrays), key rows Nk (k, v, dk, dv).
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      hipStream_t stream);

// Rows per (batch, head) of the padded fp32 arrays the backward kernels read.
int bwd_rows_padded(int N);

hipError_t launch_bwd_preprocess(const void* o, const void* dout, const float* lse, float* delta,
                                 float* lse_log2, int B, int H, int N, int d, hipStream_t stream);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                           const float* lse_log2, const float* delta, void* dk, void* dv, int B,
                           int H, int Nq, int Nk, int d, float scale, int causal,
                           hipStream_t stream);

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                         const float* lse_log2, const float* delta, void* dq, int B, int H,
                         int Nq, int Nk, int d, float scale, int causal, hipStream_t stream);

void fwd_tiles(int d, int* block_q, int* block_k, int* waves);
void bwd_tiles(int d, int* block_k, int* block_q, int* waves);

}  // namespace fa2
