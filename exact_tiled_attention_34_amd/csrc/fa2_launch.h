// Internal launch interface between the C ABI (fa2_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fa2 {

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, float* dq_accum,
                                 int B, int H, int N, int d, hipStream_t stream);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, const float* delta, float* dq_accum, void* dk,
                           void* dv, int B, int H, int N, int d, float scale, int causal,
                           hipStream_t stream);

hipError_t launch_bwd_dq_convert(const float* dq_accum, void* dq, int B, int H, int N, int d,
                                 float scale, hipStream_t stream);

void fwd_tiles(int d, int* block_q, int* block_k, int* waves);
void bwd_tiles(int d, int* block_k, int* block_q, int* waves);

}  // namespace fa2
