// Dense bf16 MFMA rate this GPU sustains, with operands held in registers:
// every wavefront issues back-to-back v_mfma_f32_32x32x16_bf16 into 8 rotating
// accumulators, on all compute units (8192 workgroups of 4 wavefronts), once
// with all-zero operands and once with random bf16 operands drawn like the
// attention inputs (uniform in [-2, 2)).  No memory traffic and no other
// instruction competes, so the rate is the matrix cores' own under the power
// and clock behaviour of each operand kind: the practical ceiling against
// which the attention kernels' MFMA rates can be read (the published dense
// peak assumes the maximum clock).  Prints one JSON line; with an argument
// C > 0 it instead prints, random operands first (from an idle GPU), the rate
// of each of C chunks of 20 launches (about 50 ms each), to show that the rate
// holds over time.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

constexpr int kIters = 256;       // 16 MFMAs per iteration
constexpr int kGrid = 8192;       // workgroups of 256 threads
constexpr int kSets = 64;         // operand sets (workgroup id mod 64)

__global__ __launch_bounds__(256) void mfma_loop(const bf16x8* __restrict__ a, const bf16x8* __restrict__ b,
                                                 float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = (blockIdx.x % kSets) * 1024 + wave * 256 + lane;   // < kSets * 1024
  bf16x8 av[4], bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    av[i] = a[base + 64 * i];
    bv[i] = b[base + 64 * i];
  }
  f32x16 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m)
      acc[m % 8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[m % 4], bv[(m / 4) % 4], acc[m % 8], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int n = 0; n < 8; ++n) s += acc[n][0] + acc[n][15];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

int main(int argc, char** argv) {
  const int chunks = argc > 1 ? std::atoi(argv[1]) : 0;
  const size_t n_vec = (size_t)kSets * 1024;   // bf16x8 elements per operand buffer
  bf16x8 *a = nullptr, *b = nullptr;
  float* out = nullptr;
  CHECK(hipMalloc(&a, n_vec * 16));
  CHECK(hipMalloc(&b, n_vec * 16));
  CHECK(hipMalloc(&out, (size_t)kGrid * 256 * 4));
  std::vector<uint16_t> h(n_vec * 8);
  double tflops[2];
  for (int kk = 0; kk < 2; ++kk) {
    const int kind = chunks > 0 ? 1 - kk : kk;
    uint32_t x = 12345u;   // linear congruential draws, top 23 bits -> [-2, 2)
    for (size_t i = 0; i < h.size(); ++i) {
      x = x * 1664525u + 1013904223u;
      const float f = kind ? ((float)(x >> 9) * (1.0f / 8388608.0f) - 0.5f) * 4.f : 0.f;
      uint32_t u;
      std::memcpy(&u, &f, 4);
      h[i] = (uint16_t)(u >> 16);
    }
    CHECK(hipMemcpy(a, h.data(), n_vec * 16, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(b, h.data(), n_vec * 16, hipMemcpyHostToDevice));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const int reps = 20;
    const double chunk_flops = (double)reps * kGrid * 4 * kIters * 16 * (2.0 * 32 * 32 * 16);
    for (int c = 0; c < chunks; ++c) {
      CHECK(hipEventRecord(e0));
      for (int r = 0; r < reps; ++r) mfma_loop<<<kGrid, 256>>>(a, b, out);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0.f;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      std::printf("{\"operands\": \"%s\", \"chunk\": %d, \"ms\": %.2f, \"tflops\": %.1f}\n",
                  kind ? "random" : "zero", c, ms, chunk_flops / (ms * 1e-3) / 1e12);
    }
    if (chunks > 0) continue;
    for (int w = 0; w < 3; ++w) mfma_loop<<<kGrid, 256>>>(a, b, out);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < reps; ++r) mfma_loop<<<kGrid, 256>>>(a, b, out);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double flops = (double)reps * kGrid * 4 * kIters * 16 * (2.0 * 32 * 32 * 16);
    tflops[kind] = flops / (ms * 1e-3) / 1e12;
  }
  if (chunks > 0) return 0;
  std::printf("{\"mfma_bf16_32x32x16_tflops_zero_operands\": %.1f, "
              "\"mfma_bf16_32x32x16_tflops_random_operands\": %.1f}\n", tflops[0], tflops[1]);
  return 0;
}
