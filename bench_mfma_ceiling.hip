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

// One operand per MFMA from memory.  SRC 0: one 16-byte LDS read per MFMA;
// 1: one 16-byte LDS read per two MFMAs; 2: a 16-byte global load per MFMA (a
// 64 KiB window per workgroup, L1-resident after the first pass); 3: two
// transposing 8-byte LDS reads per MFMA (ds_read_b64_tr_b16, consecutive
// lanes 8 bytes apart).  Every address is masked into its buffer.
//
// PF = 0: the compiler schedules the reads (it issues a loop iteration's
// reads ahead of its MFMAs, so each iteration starts by waiting for a read).
// PF > 0: software-pipelined as the attention kernels do it: the operand of
// MFMA k is read right after MFMA k - PF is issued, into a ring of PF
// registers, across loop iterations, and a scheduling barrier after every
// MFMA keeps that order.
template <int SRC, int PF>
__device__ __forceinline__ bf16x8 fed_read(const char* lbase, const char* gbase, int lane, int wave, int k) {
  const int u = k & 15, it = k >> 4;
  if constexpr (SRC == 3) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const uint32_t o0 = (uint32_t)(lane * 8 + u * 1024 + wave * 4096 + it * 256) & 0xFFF8u;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lbase + o0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lbase + (o0 ^ 512u)));
    const s16x4 both[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, both);
  } else {
    const uint32_t off = (uint32_t)(lane * 16 + u * 1024 + wave * 4096 + it * 256) & 0xFFF0u;
    return SRC == 2 ? *reinterpret_cast<const bf16x8*>(gbase + off) : *reinterpret_cast<const bf16x8*>(lbase + off);
  }
}

template <int SRC, int PF>
__global__ __launch_bounds__(1024) void mfma_fed(const uint16_t* __restrict__ g, float* __restrict__ out, int iters) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[32768];   // 64 KiB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 32768; i += blockDim.x) lds[i] = g[i];
  __syncthreads();
  const bf16x8 b = *reinterpret_cast<const bf16x8*>(lds + 8 * lane);
  f32x16 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;
  const char* lbase = reinterpret_cast<const char*>(lds);
  const char* gbase = reinterpret_cast<const char*>(g) + (size_t)(blockIdx.x % 64) * 65536;
  constexpr int STEP = SRC == 1 ? 2 : 1;   // MFMAs per read
  if constexpr (PF == 0) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 16; u += STEP) {
        const bf16x8 a = fed_read<SRC, PF>(lbase, gbase, lane, wave, it * 16 + u);
        acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u & 3], 0, 0, 0);
        if (SRC == 1) acc[(u + 1) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[(u + 1) & 3], 0, 0, 0);
      }
    }
  } else {
    bf16x8 ring[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[p] = fed_read<SRC, PF>(lbase, gbase, lane, wave, p * STEP);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 16; u += STEP) {
        const int slot = (u / STEP) % PF;
        acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[slot], b, acc[u & 3], 0, 0, 0);
        if (SRC == 1)
          acc[(u + 1) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, ring[slot], acc[(u + 1) & 3], 0, 0, 0);
        ring[slot] = fed_read<SRC, PF>(lbase, gbase, lane, wave, it * 16 + u + PF * STEP);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) acc[0][p] += (float)ring[p][0];
  }
  float s = 0.f;
#pragma unroll
  for (int n = 0; n < 4; ++n) s += acc[n][0] + acc[n][15];
  out[blockIdx.x * blockDim.x + tid] = s;
}

// rates of mfma_fed: 256 workgroups (one per CU) of 4, 8 or 16 wavefronts
template <int SRC, int PF>
int run_fed_one(const char* name, const uint16_t* g, float* out, hipEvent_t e0, hipEvent_t e1) {
  const int iters = 2048;
  for (int waves : {4, 8, 16}) {
    float ms = 0.f;
    for (int rep = 0; rep < 3; ++rep) {   // the last of three runs is reported
      CHECK(hipEventRecord(e0));
      mfma_fed<SRC, PF><<<256, 64 * waves>>>(g, out, iters);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipEventElapsedTime(&ms, e0, e1));
    }
    const double flops = 256.0 * waves * iters * 16 * (2.0 * 32 * 32 * 16);
    std::printf("{\"operand_source\": \"%s\", \"reads_ahead\": %d, \"wavefronts_per_simd\": %d, \"ms\": %.3f, "
                "\"tflops\": %.1f}\n",
                name, PF, waves / 4, ms, flops / (ms * 1e-3) / 1e12);
    std::fflush(stdout);
  }
  return 0;
}

int run_fed() {
  const size_t n = (size_t)64 * 65536 / 2;   // bf16 elements: 64 windows of 64 KiB
  std::vector<uint16_t> h(n);
  uint32_t x = 12345u;
  for (size_t i = 0; i < n; ++i) {
    x = x * 1664525u + 1013904223u;
    const float f = ((float)(x >> 9) * (1.0f / 8388608.0f) - 0.5f) * 4.f;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    h[i] = (uint16_t)(u >> 16);
  }
  uint16_t* g = nullptr;
  float* out = nullptr;
  CHECK(hipMalloc(&g, n * 2));
  CHECK(hipMalloc(&out, (size_t)256 * 1024 * 4));
  CHECK(hipMemcpy(g, h.data(), n * 2, hipMemcpyHostToDevice));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const char* lds1 = "LDS read per MFMA";
  const char* lds2 = "LDS read per 2 MFMAs";
  const char* l1 = "L1 global load per MFMA";
  const char* tr = "two transposing 8-byte LDS reads per MFMA";
  if (run_fed_one<0, 0>(lds1, g, out, e0, e1) || run_fed_one<1, 0>(lds2, g, out, e0, e1) ||
      run_fed_one<2, 0>(l1, g, out, e0, e1) || run_fed_one<3, 0>(tr, g, out, e0, e1) ||
      run_fed_one<0, 2>(lds1, g, out, e0, e1) || run_fed_one<0, 4>(lds1, g, out, e0, e1) ||
      run_fed_one<1, 2>(lds2, g, out, e0, e1) || run_fed_one<3, 2>(tr, g, out, e0, e1) ||
      run_fed_one<3, 4>(tr, g, out, e0, e1))
    return 1;
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "fed") == 0) return run_fed();
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
