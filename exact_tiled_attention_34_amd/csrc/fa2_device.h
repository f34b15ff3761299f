// Device helpers for the gfx950 (CDNA4) attention kernels: MFMA wrappers,
// bf16 packing, fast exp2/log2, the LDS tile layout, asynchronous
// global->LDS tile loads and the two ways MFMA operands are read from LDS.
//
// MFMA lane layout (v_mfma_f32_32x32x16_bf16, one 64-lane wavefront):
//   A (32 x 16): lane l holds A[l % 32][8*(l/32) + j],  j = 0..7
//   B (16 x 32): lane l holds B[8*(l/32) + j][l % 32],  j = 0..7
//   C (32 x 32): lane l, register i holds C[8*(i/4) + 4*(l/32) + (i%4)][l % 32]
// so every lane owns one column of C and 16 of its rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa2_launch.h"
#include "fa2_layout.h"

namespace fa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The 16-bit storage types.  Operands travel as raw 32-bit words (u32x4: 8
// elements) and are reinterpreted only at the MFMA; P, dS and the outputs are
// rounded to the storage type to nearest-even.
struct BF16 {
  static constexpr int kId = 0;
  static constexpr uint16_t kOne = 0x3F80;   // 1.0
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> one word of two bf16 (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  // acc + lo(w) + hi(w) in one instruction (v_dot2c_f32_bf16 with (1, 1))
  static __device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
  }
};

struct F16 {
  static constexpr int kId = 1;
  static constexpr uint16_t kOne = 0x3C00;   // 1.0
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  // acc + lo(w) + hi(w) in one instruction (v_dot2c_f32_f16 with (1, 1))
  static __device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
  }
};

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Exchange with the lane 32 positions away (the other half of the wavefront).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// Wait until this wavefront's outstanding vector-memory loads (including
// global->LDS loads) have completed: s_waitcnt vmcnt(0) (expcnt and lgkmcnt
// fields at their maximum, i.e. not waited on).  Emitted through the builtin so
// that the compiler's own wait bookkeeping knows that nothing is pending after
// it; kernels call it at the end of their prologue as well, so the register
// operands loaded there are never waited for inside the main loop (where the
// wait would also cover the prefetch of the next tile).
__device__ __forceinline__ void wait_vmem() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0x0f70);
#endif
}

// Scheduling fence: the compiler may move no instruction across it.  Kernels
// that issue their LDS operand reads a fixed number of MFMA stages ahead put
// one between stages, so the distance they chose (and the interleaving of
// softmax arithmetic with matrix work) survives instruction scheduling.
__device__ __forceinline__ void sched_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
#endif
}

template <int SYNC, int N_MFMA, int N_READS, int RPM, int I, int READS>
__device__ __forceinline__ void mfma_pipeline_step() {
  if constexpr (I < N_MFMA) {
    constexpr int more = READS + RPM <= N_READS ? RPM : N_READS - READS;
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_group_barrier(0x008, 1, SYNC);                 // one MFMA
    if constexpr (more > 0) __builtin_amdgcn_sched_group_barrier(0x100, more, SYNC);  // its reads
#endif
    mfma_pipeline_step<SYNC, N_MFMA, N_READS, RPM, I + 1, READS + more>();
  }
}

// Scheduling hint for a run of N_MFMA MFMAs fed by N_READS LDS reads, RPM
// reads per MFMA: issue DEPTH reads first, then RPM more after each MFMA, so
// DEPTH operand loads stay in flight and the LDS latency hides behind the
// matrix cores instead of stalling every MFMA.  Emitted right after the code
// it describes, in the same basic block; SYNC tells independent hints apart.
template <int SYNC, int N_MFMA, int N_READS, int DEPTH, int RPM = 1>
__device__ __forceinline__ void mfma_pipeline_hint() {
  constexpr int first = DEPTH < N_READS ? DEPTH : N_READS;
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_group_barrier(0x100, first, SYNC);
#endif
  mfma_pipeline_step<SYNC, N_MFMA, N_READS, RPM, 0, first>();
}

// One 16-byte global -> LDS load per lane (global_load_lds_dwordx4 with a
// scalar base address and a per-lane 32-bit byte offset).  `lds` must be the
// same for every lane of the wavefront; lane l's 16 bytes land at
// lds + 16*l bytes (also when only some lanes are active).
//
// Issued as inline assembly on purpose: the compiler cannot tell which LDS
// bytes such a load writes, so for the builtin it waits for every outstanding
// vector-memory load before each later LDS read, which would make every tile
// wait for the prefetch of the next one.  The kernels order these loads
// themselves: wait_vmem() and a workgroup barrier before a tile is read, and
// no load into a buffer that a wavefront may still be reading.
__device__ __forceinline__ void global_load_lds16(const void* base, uint32_t byte_off, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  // M0 (the LDS base of the load) is a reserved register that the compiler
  // only ever sets immediately before an instruction that reads it; nothing
  // else in these kernels uses it, so clobbering it here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(byte_off), "s"(base), "s"(m0)
               : "memory", "m0");
#pragma clang diagnostic pop
#endif
}

// Resource descriptor of an untyped byte range [base, base + num_bytes) for
// the buffer loads below: a load whose byte offset (the per-lane offset plus
// the scalar one) reaches num_bytes is out of range and returns zeros, and
// into LDS it stores zeros (measured on MI355X).  Word 3 selects the 32-bit
// data format with no stride, swizzle or index: plain byte addressing.
__device__ __forceinline__ i32x4 raw_buffer(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)num_bytes);
  r[3] = 0x00020000;
  return r;
}

// The LDS byte address of a pointer into LDS.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// One 16-byte buffer -> LDS load per lane (buffer_load_dwordx4 ... lds) from
// byte voff + soff of the range `rsrc`; lane l's 16 bytes land at LDS byte
// address lds + 16*l, zeros when the offset is out of range.  Inline assembly
// for the reason given at global_load_lds16.
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(m0)
               : "memory", "m0");
#pragma clang diagnostic pop
#endif
}

// Copies ROWS-row tiles of one head (rows R elements apart, D features) into
// a RowTile (or a TrRowTile / WideRowTile: LT) in LDS with buffer -> LDS
// loads, following DmaPlan.  The per-lane byte offsets within a tile are
// computed once (init); a tile's resource (tile()) covers only its rows that
// exist, so the rows of a ragged last tile, and every row of a tile that
// starts at or past the end, arrive as zeros with no test in the kernel.  A
// pass then costs one scalar offset, the LDS address and the load.  Slots
// that the layout keeps at zero are loaded out of range (zeros again); slots
// holding other constants are left out by lane.  issue() returns at once;
// wait_vmem() and a workgroup barrier make the tile visible.
//
// Offsets stay below 2^31: the row pitch is at most 2^20 elements (checked by
// the API), so a tile spans at most 128 * 2^21 bytes.
template <int D, int ROWS, int THREADS, class LT = RowTile<D>>
struct TileDma {
  using P = DmaPlan<D, ROWS, THREADS, LT>;
  uint32_t off[P::NOFF];
  int wave, R;

  __device__ __forceinline__ void init(int tid, int row_pitch) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    R = row_pitch;
#pragma unroll
    for (int t = 0; t < P::NOFF; ++t) off[t] = P::stored_offset(wave, tid & 63, t, row_pitch);
  }
  // The resource of the tile whose first row is row0 (row0 >= 0): rows
  // row0 .. n_rows - 1 of it, none when row0 >= n_rows.
  __device__ __forceinline__ i32x4 tile(const uint16_t* head, int row0, int n_rows) const {
    row0 = __builtin_amdgcn_readfirstlane(row0);
    const int rows = n_rows - row0;
    return raw_buffer(head + (size_t)row0 * R, P::tile_bytes(rows < ROWS ? rows : ROWS, R));
  }
  // Pass t of the copy of the tile `rs` into the tile at LDS byte address `tile`.
  __device__ __forceinline__ void issue_pass(int t, uint32_t tile, i32x4 rs) const {
    const int first = P::pass_slot(wave, t);   // wavefront-uniform
    if (P::TOTAL % THREADS == 0 || first < P::TOTAL) {
      const uint32_t o = off[P::off_index(t)];
      const uint32_t soff = P::pass_offset(t, R);
      const uint32_t dst = tile + (uint32_t)first * 16u;
      if constexpr (P::SKIP_BY_LANE) {
        if (o != P::kSkip) buffer_load_lds16(rs, o, soff, dst);
      } else {
        buffer_load_lds16(rs, o, soff, dst);
      }
    }
  }
  // The whole tile at row0 (row0 >= 0; rows at or past n_rows arrive as zeros).
  __device__ __forceinline__ void issue(uint16_t* tile, const uint16_t* head, int row0,
                                        int n_rows) const {
    const i32x4 rs = this->tile(head, row0, n_rows);
    const uint32_t dst = lds_address(tile);
#pragma unroll
    for (int t = 0; t < P::ITER; ++t) issue_pass(t, dst, rs);
  }
};

// One bf16 [B, H, N, D] tensor addressed through element strides (the last
// dimension contiguous): element (b, h, n, i) is at p + b sb + h sh + n sr + i.
// sr is the row pitch R of the tile copies and stages.
struct CView {
  const uint16_t* p;
  long long sb, sh;
  int sr;
  __device__ __forceinline__ const uint16_t* head(int b, int h) const { return p + b * sb + h * sh; }
};
struct View {
  uint16_t* p;
  long long sb, sh;
  int sr;
  __device__ __forceinline__ uint16_t* head(int b, int h) const { return p + b * sb + h * sh; }
};

// Calls f(head dim, causal, element type) with compile-time values for the
// run-time (d, causal, dtype) of a launch: the one place that lists every
// kernel instantiation.
template <class F>
inline hipError_t dispatch(int d, int causal, int dtype, F&& f) {
  auto by_type = [&](auto dc, auto cc) -> hipError_t {
    if (dtype == 0) return f(dc, cc, BF16{});
    if (dtype == 1) return f(dc, cc, F16{});
    return hipErrorInvalidValue;
  };
  auto by_causal = [&](auto dc) -> hipError_t {
    return causal ? by_type(dc, std::true_type{}) : by_type(dc, std::false_type{});
  };
  switch (d) {
    case 64:  return by_causal(std::integral_constant<int, 64>{});
    case 80:  return by_causal(std::integral_constant<int, 80>{});
    case 96:  return by_causal(std::integral_constant<int, 96>{});
    case 128: return by_causal(std::integral_constant<int, 128>{});
    case 256: return by_causal(std::integral_constant<int, 256>{});
    default:  return hipErrorInvalidValue;
  }
}

inline CView cview(const Strided& t) {
  return CView{static_cast<const uint16_t*>(t.p), t.batch, t.head, (int)t.row};
}
inline View view(const Strided& t) {
  return View{static_cast<uint16_t*>(const_cast<void*>(t.p)), t.batch, t.head, (int)t.row};
}

__device__ __forceinline__ u32x4 lds_read16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// MFMA operand from two transposed reads of a row-major tile (TrRowTile):
// p0 and p1 are the lane's addresses of reads 0 and 1 (tokens 4h..4h+3 and
// 8+4h..8+4h+3 of the chunk, feature lane % 32 of the block).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 lds_read_tr(const uint16_t* p0, const uint16_t* p1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  const u32x4 v = {ua[0], ua[1], ub[0], ub[1]};
  return v;
}

// MFMA B operand for 16 tokens (chunk c of a 32-row accumulator pair) from
// packed accumulator words w[0..7] (w[t] = rows 2t, 2t+1 of the accumulator).
__device__ __forceinline__ u32x4 acc_chunk(const uint32_t* w, int half) {
  const u32x4 v = {w[4 * half + 0], w[4 * half + 1], w[4 * half + 2], w[4 * half + 3]};
  return v;
}

}  // namespace fa2
