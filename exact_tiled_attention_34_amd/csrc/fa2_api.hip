// C ABI entry points (include/fa2.h): argument validation, then kernel launches.
// Every check runs before the first HIP call, so a rejected call touches no
// device state.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "fa2.h"
#include "fa2_launch.h"

namespace {

thread_local char g_last_error[256] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA2_OK;
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e),
                hipGetErrorString(e));
  return FA2_ERR_HIP;
}

bool ptr_ok(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Sizes: B, H, N >= 1, d supported, element count small enough for the
// kernels' 32-bit row indices.
int check_sizes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA2_ERR_INVALID_ARG;
  if (d != 64 && d != 80 && d != 96 && d != 128 && d != 256) return FA2_ERR_UNSUPPORTED;
  const long long elems = (long long)B * H * N * d;
  if (elems >= (1LL << 31)) return FA2_ERR_INVALID_ARG;
  return FA2_OK;
}

// Query and key lengths: both must pass the checks above.
int check_sizes2(int B, int H, int Nq, int Nk, int d) {
  const int st = check_sizes(B, H, Nq, d);
  return st != FA2_OK ? st : check_sizes(B, H, Nk, d);
}

int check_scale_causal(float scale, int causal) {
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA2_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARG;
  return FA2_OK;
}

// No output span may overlap an input span or another output span.
bool disjoint(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], ins[j])) return false;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], outs[j])) return false;
  }
  return true;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Contiguous [B, H, N, d] tensors (the plain entry points).
fa2::Strided dense(const void* p, int H, int N, int d) { return fa2::contiguous(p, H, N, d); }

// A strided bf16 [B, H, N, d] tensor (s == NULL: contiguous).  Checks: 16-byte
// aligned base; strides >= 0 and multiples of 8 elements (every row starts on
// 16 bytes); one head's rows within 2^30 elements and a row stride of at most
// 2^20 elements (the kernels' 32-bit offsets: a 128-row tile stays below
// 2^31 bytes).  For an output, the element map must be one-to-one: ordered by
// stride, every dimension must step over everything inside it (the last
// dimension, d elements at stride 1, innermost).  On success *span is the
// byte range the tensor touches.
bool strided_view(const void* p, const fa2_strides* s, int B, int H, int N, int d, bool output,
                  fa2::Strided* t, Span* sp) {
  if (!ptr_ok(p)) return false;
  *t = s ? fa2::Strided{p, s->batch, s->head, s->row} : fa2::contiguous(p, H, N, d);
  // a dimension of extent 1 is never stepped over: its stride is ignored
  if (B == 1) t->batch = 0;
  if (H == 1) t->head = 0;
  if (N == 1) t->row = 0;
  const long long st[3] = {t->batch, t->head, t->row};
  const long long ext[3] = {B, H, N};
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] % 8 != 0) return false;
  if ((long long)(N - 1) * t->row + d > (1LL << 30) || t->row > (1LL << 20)) return false;
  const long long last = (B - 1) * t->batch + (long long)(H - 1) * t->head + (long long)(N - 1) * t->row + d;
  if (last > (1LL << 40)) return false;
  if (output) {
    // insertion-sort the dimensions of extent > 1 by stride, then check nesting
    long long sst[3], sex[3];
    int n = 0;
    for (int i = 0; i < 3; ++i) {
      if (ext[i] == 1) continue;
      int j = n++;
      while (j > 0 && sst[j - 1] > st[i]) {
        sst[j] = sst[j - 1];
        sex[j] = sex[j - 1];
        --j;
      }
      sst[j] = st[i];
      sex[j] = ext[i];
    }
    long long inner = d;   // elements spanned by everything inside the current dimension
    for (int i = 0; i < n; ++i) {
      if (sst[i] < inner) return false;
      inner = sst[i] * (sex[i] - 1) + inner;
    }
  }
  *sp = span(p, (size_t)last * 2);
  return true;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free backward (fa2_bwd_qk_noalloc): the two padded
// fp32 row arrays live in this fixed device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy for the life of
// the process.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// passed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on first use).
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return FA2_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return FA2_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA2_OK;
}

}  // namespace

extern "C" {

int fa2_fwd_strided(const void* q, const fa2_strides* sq, const void* k, const fa2_strides* sk,
                    const void* v, const fa2_strides* sv, void* o, const fa2_strides* so,
                    float* lse, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    int dtype, void* stream) {
  int st = check_sizes2(B, H, Nq, Nk, d);
  if (st != FA2_OK) return st;
  if ((st = check_scale_causal(scale, causal)) != FA2_OK) return st;
  if (dtype != FA2_BF16 && dtype != FA2_FP16) return FA2_ERR_INVALID_ARG;
  fa2::Strided tq, tk, tv, to;
  Span ins[3], outs[2];
  if (!strided_view(q, sq, B, H, Nq, d, false, &tq, &ins[0]) ||
      !strided_view(k, sk, B, H, Nk, d, false, &tk, &ins[1]) ||
      !strided_view(v, sv, B, H, Nk, d, false, &tv, &ins[2]) ||
      !strided_view(o, so, B, H, Nq, d, true, &to, &outs[0]) || !ptr_ok(lse))
    return FA2_ERR_INVALID_ARG;
  outs[1] = span(lse, (size_t)B * H * Nq * 4);
  if (!disjoint(outs, 2, ins, 3)) return FA2_ERR_INVALID_ARG;
  return hip_status(fa2::launch_fwd(tq, tk, tv, to, lse, B, H, Nq, Nk, d, scale, causal, dtype,
                                    as_stream(stream)));
}

int fa2_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Nq, int Nk, int d, float scale, int causal, void* stream) {
  int st = check_sizes2(B, H, Nq, Nk, d);
  if (st != FA2_OK) return st;
  if ((st = check_scale_causal(scale, causal)) != FA2_OK) return st;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o) || !ptr_ok(lse))
    return FA2_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * H * Nk * d * 2;
  const size_t lb = (size_t)B * H * Nq * 4;
  const Span ins[3] = {span(q, qb), span(k, kb), span(v, kb)};
  const Span outs[2] = {span(o, qb), span(lse, lb)};
  if (!disjoint(outs, 2, ins, 3)) return FA2_ERR_INVALID_ARG;
  return hip_status(fa2::launch_fwd(dense(q, H, Nq, d), dense(k, H, Nk, d), dense(v, H, Nk, d),
                                    dense(o, H, Nq, d), lse, B, H, Nq, Nk, d, scale, causal,
                                    FA2_BF16, as_stream(stream)));
}

int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
            int d, float scale, int causal, void* stream) {
  return fa2_fwd_qk(q, k, v, o, lse, B, H, N, N, d, scale, causal, stream);
}

int fa2_bwd_rows_padded(int N) { return N < 1 ? 0 : fa2::bwd_rows_padded(N); }

size_t fa2_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (check_sizes(B, H, N, d) != FA2_OK) return 0;
  const size_t rows = (size_t)B * H * fa2::bwd_rows_padded(N);
  return 2 * align256(rows * 4);
}

int fa2_bwd_preprocess(const void* o, const void* dout, const float* lse, float* delta,
                       float* lse_log2, int B, int H, int N, int d, void* stream) {
  int st = check_sizes(B, H, N, d);
  if (st != FA2_OK) return st;
  if (!ptr_ok(o) || !ptr_ok(dout) || !ptr_ok(lse) || !ptr_ok(delta) || !ptr_ok(lse_log2))
    return FA2_ERR_INVALID_ARG;
  const size_t tb = (size_t)B * H * N * d * 2, rows = (size_t)B * H * N;
  const size_t prow = (size_t)B * H * fa2::bwd_rows_padded(N);
  const Span ins[3] = {span(o, tb), span(dout, tb), span(lse, rows * 4)};
  const Span outs[2] = {span(delta, prow * 4), span(lse_log2, prow * 4)};
  if (!disjoint(outs, 2, ins, 3)) return FA2_ERR_INVALID_ARG;
  return hip_status(fa2::launch_bwd_preprocess(dense(o, H, N, d), dense(dout, H, N, d), lse, delta,
                                               lse_log2, B, H, N, d, FA2_BF16, as_stream(stream)));
}

// Shared checks of the two tile phases: 4 bf16 inputs (q, dout: Nq rows; k,
// v: Nk rows), the two padded row arrays (Nq rows), and one or two bf16
// outputs of out_rows rows.
static int check_tile_phase(const void* q, const void* k, const void* v, const void* dout,
                            const float* lse_log2, const float* delta, const void* out0,
                            const void* out1, int out_rows, int B, int H, int Nq, int Nk, int d,
                            float scale, int causal) {
  int st = check_sizes2(B, H, Nq, Nk, d);
  if (st != FA2_OK) return st;
  if ((st = check_scale_causal(scale, causal)) != FA2_OK) return st;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(dout) || !ptr_ok(lse_log2) ||
      !ptr_ok(delta) || !ptr_ok(out0) || (out1 != nullptr && !ptr_ok(out1)))
    return FA2_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * H * Nk * d * 2;
  const size_t ob = (size_t)B * H * out_rows * d * 2;
  const size_t prow = (size_t)B * H * fa2::bwd_rows_padded(Nq);
  const Span ins[6] = {span(q, qb), span(k, kb), span(v, kb), span(dout, qb),
                       span(lse_log2, prow * 4), span(delta, prow * 4)};
  const Span outs[2] = {span(out0, ob), span(out1, out1 ? ob : 0)};
  if (!disjoint(outs, out1 ? 2 : 1, ins, 6)) return FA2_ERR_INVALID_ARG;
  return FA2_OK;
}

int fa2_bwd_dkdv_qk(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse_log2, const float* delta, void* dk, void* dv, int B, int H,
                    int Nq, int Nk, int d, float scale, int causal, void* stream) {
  if (dv == nullptr) return FA2_ERR_INVALID_ARG;
  const int st = check_tile_phase(q, k, v, dout, lse_log2, delta, dk, dv, Nk, B, H, Nq, Nk, d,
                                  scale, causal);
  if (st != FA2_OK) return st;
  return hip_status(fa2::launch_bwd_dkdv(dense(q, H, Nq, d), dense(k, H, Nk, d), dense(v, H, Nk, d),
                                         dense(dout, H, Nq, d), lse_log2, delta, dense(dk, H, Nk, d),
                                         dense(dv, H, Nk, d), B, H, Nq, Nk, d, scale, causal,
                                         FA2_BF16, as_stream(stream)));
}

int fa2_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                 const float* lse_log2, const float* delta, void* dk, void* dv, int B, int H,
                 int N, int d, float scale, int causal, void* stream) {
  return fa2_bwd_dkdv_qk(q, k, v, dout, lse_log2, delta, dk, dv, B, H, N, N, d, scale, causal,
                         stream);
}

int fa2_bwd_dq_qk(const void* q, const void* k, const void* v, const void* dout,
                  const float* lse_log2, const float* delta, void* dq, int B, int H, int Nq,
                  int Nk, int d, float scale, int causal, void* stream) {
  const int st = check_tile_phase(q, k, v, dout, lse_log2, delta, dq, nullptr, Nq, B, H, Nq, Nk,
                                  d, scale, causal);
  if (st != FA2_OK) return st;
  return hip_status(fa2::launch_bwd_dq(dense(q, H, Nq, d), dense(k, H, Nk, d), dense(v, H, Nk, d),
                                       dense(dout, H, Nq, d), lse_log2, delta, dense(dq, H, Nq, d),
                                       B, H, Nq, Nk, d, scale, causal, FA2_BF16,
                                       as_stream(stream)));
}

int fa2_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
               const float* lse_log2, const float* delta, void* dq, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
  return fa2_bwd_dq_qk(q, k, v, dout, lse_log2, delta, dq, B, H, N, N, d, scale, causal, stream);
}

// Shared body of fa2_bwd_qk and fa2_bwd_strided: launches the three phases.
static int bwd_run(const fa2::Strided& tq, const fa2::Strided& tk, const fa2::Strided& tv,
                   const fa2::Strided& to, const float* lse, const fa2::Strided& tdo,
                   const fa2::Strided& tdq, const fa2::Strided& tdk, const fa2::Strided& tdv, int B,
                   int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                   void* workspace, void* stream) {
  const size_t prow = (size_t)B * H * fa2::bwd_rows_padded(Nq);
  float* delta = static_cast<float*>(workspace);
  float* lse_log2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(prow * 4));
  hipStream_t s = as_stream(stream);
  int st;
  if ((st = hip_status(fa2::launch_bwd_preprocess(to, tdo, lse, delta, lse_log2, B, H, Nq, d, dtype,
                                                  s))) != FA2_OK)
    return st;
  if ((st = hip_status(fa2::launch_bwd_dkdv(tq, tk, tv, tdo, lse_log2, delta, tdk, tdv, B, H, Nq, Nk,
                                            d, scale, causal, dtype, s))) != FA2_OK)
    return st;
  return hip_status(fa2::launch_bwd_dq(tq, tk, tv, tdo, lse_log2, delta, tdq, B, H, Nq, Nk, d, scale,
                                       causal, dtype, s));
}

int fa2_bwd_qk(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
               int d, float scale, int causal, void* workspace, size_t workspace_bytes,
               void* stream) {
  int st = check_sizes2(B, H, Nq, Nk, d);
  if (st != FA2_OK) return st;
  if ((st = check_scale_causal(scale, causal)) != FA2_OK) return st;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o) || !ptr_ok(lse) || !ptr_ok(dout) ||
      !ptr_ok(dq) || !ptr_ok(dk) || !ptr_ok(dv) || !ptr_ok(workspace))
    return FA2_ERR_INVALID_ARG;
  const size_t need = fa2_bwd_workspace_bytes(B, H, Nq, d);
  if (workspace_bytes < need) return FA2_ERR_WORKSPACE;
  const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * H * Nk * d * 2;
  const size_t rows = (size_t)B * H * Nq;
  const Span ins[6] = {span(q, qb), span(k, kb), span(v, kb),
                       span(o, qb), span(lse, rows * 4), span(dout, qb)};
  const Span outs[4] = {span(dq, qb), span(dk, kb), span(dv, kb), span(workspace, need)};
  if (!disjoint(outs, 4, ins, 6)) return FA2_ERR_INVALID_ARG;
  return bwd_run(dense(q, H, Nq, d), dense(k, H, Nk, d), dense(v, H, Nk, d), dense(o, H, Nq, d), lse,
                 dense(dout, H, Nq, d), dense(dq, H, Nq, d), dense(dk, H, Nk, d), dense(dv, H, Nk, d),
                 B, H, Nq, Nk, d, scale, causal, FA2_BF16, workspace, stream);
}

int fa2_bwd_qk_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                       int d, float scale, int causal, void* stream) {
  int st = check_sizes2(B, H, Nq, Nk, d);
  if (st != FA2_OK) return st;
  if ((st = check_scale_causal(scale, causal)) != FA2_OK) return st;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o) || !ptr_ok(lse) || !ptr_ok(dout) ||
      !ptr_ok(dq) || !ptr_ok(dk) || !ptr_ok(dv))
    return FA2_ERR_INVALID_ARG;
  if (fa2_bwd_workspace_bytes(B, H, Nq, d) > kScratchBytes) return FA2_ERR_WORKSPACE;
  const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * H * Nk * d * 2;
  const size_t rows = (size_t)B * H * Nq;
  const Span ins[6] = {span(q, qb), span(k, kb), span(v, kb),
                       span(o, qb), span(lse, rows * 4), span(dout, qb)};
  const Span outs[3] = {span(dq, qb), span(dk, kb), span(dv, kb)};
  if (!disjoint(outs, 3, ins, 6)) return FA2_ERR_INVALID_ARG;
  void* ws = nullptr;
  if ((st = current_scratch(&ws)) != FA2_OK) return st;
  return bwd_run(dense(q, H, Nq, d), dense(k, H, Nk, d), dense(v, H, Nk, d), dense(o, H, Nq, d), lse,
                 dense(dout, H, Nq, d), dense(dq, H, Nq, d), dense(dk, H, Nk, d), dense(dv, H, Nk, d),
                 B, H, Nq, Nk, d, scale, causal, FA2_BF16, ws, stream);
}

size_t fa2_bwd_noalloc_max_bytes(void) { return kScratchBytes; }

int fa2_bwd_strided(const void* q, const fa2_strides* sq, const void* k, const fa2_strides* sk,
                    const void* v, const fa2_strides* sv, const void* o, const fa2_strides* so,
                    const float* lse, const void* dout, const fa2_strides* sdo, void* dq,
                    const fa2_strides* sdq, void* dk, const fa2_strides* sdk, void* dv,
                    const fa2_strides* sdv, int B, int H, int Nq, int Nk, int d, float scale,
                    int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_sizes2(B, H, Nq, Nk, d);
  if (st != FA2_OK) return st;
  if ((st = check_scale_causal(scale, causal)) != FA2_OK) return st;
  if (dtype != FA2_BF16 && dtype != FA2_FP16) return FA2_ERR_INVALID_ARG;
  fa2::Strided tq, tk, tv, to, tdo, tdq, tdk, tdv;
  Span ins[6], outs[4];
  if (!strided_view(q, sq, B, H, Nq, d, false, &tq, &ins[0]) ||
      !strided_view(k, sk, B, H, Nk, d, false, &tk, &ins[1]) ||
      !strided_view(v, sv, B, H, Nk, d, false, &tv, &ins[2]) ||
      !strided_view(o, so, B, H, Nq, d, false, &to, &ins[3]) ||
      !strided_view(dout, sdo, B, H, Nq, d, false, &tdo, &ins[4]) ||
      !strided_view(dq, sdq, B, H, Nq, d, true, &tdq, &outs[0]) ||
      !strided_view(dk, sdk, B, H, Nk, d, true, &tdk, &outs[1]) ||
      !strided_view(dv, sdv, B, H, Nk, d, true, &tdv, &outs[2]) || !ptr_ok(lse) ||
      !ptr_ok(workspace))
    return FA2_ERR_INVALID_ARG;
  const size_t need = fa2_bwd_workspace_bytes(B, H, Nq, d);
  if (workspace_bytes < need) return FA2_ERR_WORKSPACE;
  ins[5] = span(lse, (size_t)B * H * Nq * 4);
  outs[3] = span(workspace, need);
  // each output against every input; the workspace against the three outputs.
  // The outputs themselves may interleave (for instance three head groups of
  // one buffer): that they touch disjoint elements is the caller's to ensure.
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], ins[j])) return FA2_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (overlaps(outs[i], outs[3])) return FA2_ERR_INVALID_ARG;
  return bwd_run(tq, tk, tv, to, lse, tdo, tdq, tdk, tdv, B, H, Nq, Nk, d, scale, causal, dtype,
                 workspace, stream);
}

int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
            float scale, int causal, void* workspace, size_t workspace_bytes, void* stream) {
  return fa2_bwd_qk(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, N, d, scale, causal, workspace,
                    workspace_bytes, stream);
}

const char* fa2_strerror(int status) {
  switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_INVALID_ARG: return "invalid argument (null/misaligned pointer, size, scale, causal flag or aliasing)";
    case FA2_ERR_UNSUPPORTED: return "unsupported head dimension (supported: 64, 80, 96, 128, 256)";
    case FA2_ERR_WORKSPACE: return "workspace too small (see fa2_bwd_workspace_bytes; fa2_bwd_qk_noalloc: fa2_bwd_noalloc_max_bytes)";
    case FA2_ERR_HIP: return "HIP launch error (see fa2_last_error)";
    default: return "unknown status";
  }
}

const char* fa2_last_error(void) { return g_last_error; }

int fa2_tile_config(int d, int* fwd_block_q, int* fwd_block_k, int* bwd_block_k, int* bwd_block_q,
                    int* fwd_waves, int* bwd_waves) {
  if (d != 64 && d != 80 && d != 96 && d != 128 && d != 256) return FA2_ERR_UNSUPPORTED;
  if (!fwd_block_q || !fwd_block_k || !bwd_block_k || !bwd_block_q || !fwd_waves || !bwd_waves)
    return FA2_ERR_INVALID_ARG;
  fa2::fwd_tiles(d, fwd_block_q, fwd_block_k, fwd_waves);
  fa2::bwd_tiles(d, bwd_block_k, bwd_block_q, bwd_waves);
  return FA2_OK;
}

}  // extern "C"
