/*
 * fa2.h — C ABI of an MI355X (gfx950) library for exact tiled softmax attention.
 *
 * What is computed.  Standard softmax attention and its gradient, exactly (up to
 * floating-point rounding order): the "FlashAttention (v2)" glossary page says
 * the method computes attention tile by tile in on-chip memory without
 * approximating the result and that its output matches standard attention, so
 * that adopting it is only a choice of backend.  Per (batch b, head h):
 *
 *     S    = scale * Q K^T                 (never written to memory)
 *     S_ij = -inf for key j > query i + Nk - Nq   when causal
 *     L_i  = log sum_j exp(S_ij)           natural-log logsumexp, fp32
 *     O    = softmax(S) V
 *
 * The plain entry points take one length N for queries and keys (Nq = Nk = N:
 * the causal mask keeps key j for query i iff j <= i).  The "_qk" entry points
 * take Nq query rows (q, o, lse, dout, dq) and Nk key rows (k, v, dk, dv); the
 * pages show the causal mask only for a sequence attending to itself, and for
 * Nq != Nk it is aligned bottom-right here: the queries are the last Nq
 * positions of the key sequence, as for a block of new tokens attending to a
 * key/value cache.  With Nq > Nk under causal, the first Nq - Nk queries see
 * no key: their O row is 0, their L is -inf and they add nothing to any
 * gradient.
 *
 * and, given dO, the gradient of sum(dO * O):  dV = P^T dO, dP = dO V^T,
 * D_i = sum_k dO_ik O_ik, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q,
 * with P = exp(S - L) recomputed from L.
 *
 * Work split ("FlashAttention-2" summary page, "How It Works" 1 and 3; the
 * glossary page on splitting one head across thread blocks): every call is
 * spread over (batch, head) AND over blocks of the sequence, so that a few long
 * heads still fill all 256 compute units.  With causal=1, key blocks lying
 * wholly above the diagonal are skipped and only blocks crossing it are masked
 * element by element ("FlashAttention-2: Faster Attention with Better
 * Parallelism and Work Partitioning" page, closing sentence).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are DEVICE pointers to contiguous row-major [B, H, N, d] arrays
 *    (d fastest), except in the two "_strided" entry points, which take the
 *    element strides of each bf16 tensor (fa2_strides).  q, k, v, o, dout, dq, dk, dv hold bfloat16 values stored as
 *    16-bit words.  lse is fp32 [B, H, N]; the backward's delta and lse_log2
 *    are fp32 [B, H, fa2_bwd_rows_padded(N)].
 *  - Supported: B, H, N >= 1 with B*H*N*d < 2^31; d in {64, 80, 96, 128, 256};
 *    causal in {0, 1}; scale finite and > 0 (the usual 1/sqrt(d)).
 *  - Every pointer must be non-null and 16-byte aligned.  Outputs must not
 *    overlap inputs or each other.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *    enqueue work and return; results are valid after the stream is
 *    synchronised.  The library allocates no memory, keeps no pointer after a
 *    call returns, and is re-entrant: calls on different streams may run
 *    concurrently (a workspace must not be shared by calls in flight).
 *  - Outputs are overwritten, never accumulated into.
 *  - Errors: every argument is checked before any HIP call; a failed check
 *    returns FA2_ERR_INVALID_ARG, FA2_ERR_UNSUPPORTED or FA2_ERR_WORKSPACE and
 *    writes nothing.  A failed kernel launch returns FA2_ERR_HIP; the HIP
 *    error text is kept per thread (fa2_last_error).  No C++ exception crosses
 *    this interface.
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa2_status {
    FA2_OK = 0,
    FA2_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, aliasing, bad scale/causal */
    FA2_ERR_UNSUPPORTED = 2, /* head dimension not in {64, 80, 96, 128, 256} */
    FA2_ERR_WORKSPACE = 3,   /* workspace too small */
    FA2_ERR_HIP = 4          /* a HIP launch failed; see fa2_last_error() */
} fa2_status;

/*
 * Element strides of a bf16 [B, H, N, d] tensor whose last dimension is
 * contiguous: element (b, h, n, i) lies at base + b*batch + h*head + n*row + i
 * (in elements, not bytes).  The contiguous [B,H,N,d] layout is
 * {H*N*d, N*d, d}; a [B, N, H, d] ("batch, sequence, head") tensor is
 * {N*H*d, d, H*d}; head group j of a fused [B, N, 3, H, d] projection is
 * base + j*H*d with {N*3*H*d, d, 3*H*d}.
 * Requirements (else FA2_ERR_INVALID_ARG): the base 16-byte aligned; every
 * stride >= 0 and a multiple of 8 (the stride of a dimension of extent 1 is
 * ignored); (N-1)*row + d <= 2^30 and row <= 2^20.  An output tensor
 * must also map its elements one to one: ordered by stride, every dimension
 * steps over everything inside it (the d contiguous elements innermost).
 */
typedef struct fa2_strides {
    long long batch, head, row;
} fa2_strides;

/* Storage type of the 16-bit tensors of a "_strided" call (q, k, v, o, dout,
 * dq, dk, dv share it; lse and the workspace stay fp32).  The other entry
 * points take bfloat16.  Both run the same kernels with the matching 16-bit
 * matrix instruction (v_mfma_f32_32x32x16_bf16 / _f16); P and dS are rounded
 * to the storage type (nearest even) before their products. */
typedef enum fa2_dtype { FA2_BF16 = 0, FA2_FP16 = 1 } fa2_dtype;

/*
 * Forward pass on strided tensors: as fa2_fwd_qk, with the layout of q, k, v
 * and o given by sq, sk, sv, so (NULL: contiguous) and their 16-bit storage
 * type by dtype (fa2_dtype; anything else is FA2_ERR_INVALID_ARG).  lse stays
 * contiguous fp32 [B,H,Nq].  o and lse must not overlap any input.
 */
int fa2_fwd_strided(const void* q, const fa2_strides* sq, const void* k, const fa2_strides* sk,
                    const void* v, const fa2_strides* sv, void* o, const fa2_strides* so,
                    float* lse, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    int dtype, void* stream);

/*
 * Backward pass on strided tensors: as fa2_bwd_qk, with the layout of every
 * 16-bit tensor given by its fa2_strides (NULL: contiguous) and their storage
 * type by dtype (fa2_dtype); lse is contiguous
 * fp32 [B,H,Nq]; workspace as for fa2_bwd_qk.  No output (dq, dk, dv, the
 * workspace) may overlap an input, and the workspace no output.  dq, dk and
 * dv may share one buffer (for instance the three head groups of a fused
 * [B, N, 3, H, d] gradient) as long as they write disjoint elements, which
 * the library does not check.
 */
int fa2_bwd_strided(const void* q, const fa2_strides* sq, const void* k, const fa2_strides* sk,
                    const void* v, const fa2_strides* sv, const void* o, const fa2_strides* so,
                    const float* lse, const void* dout, const fa2_strides* sdo, void* dq,
                    const fa2_strides* sdq, void* dk, const fa2_strides* sdk, void* dv,
                    const fa2_strides* sdv, int B, int H, int Nq, int Nk, int d, float scale,
                    int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward pass with separate query and key lengths (see the top of this file
 * for the causal alignment).
 *   q       : in,  bf16 [B,H,Nq,d];   k, v : in, bf16 [B,H,Nk,d]
 *   o       : out, bf16 [B,H,Nq,d]
 *   lse     : out, fp32 [B,H,Nq] (-inf for a query that sees no key)
 * Nq, Nk >= 1; every other convention as for fa2_fwd.
 */
int fa2_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream);

/*
 * Forward pass: O and L from Q, K, V.
 * One query row-block per workgroup, its rows split across the workgroup's
 * wavefronts; an online softmax runs over K/V tiles staged in LDS, and the
 * division by the row sum happens once, after the last tile ("FlashAttention-2"
 * summary page, "How It Works" 2).
 *   q, k, v : in,  bf16 [B,H,N,d]
 *   o       : out, bf16 [B,H,N,d]
 *   lse     : out, fp32 [B,H,N], natural-log logsumexp of the scaled masked scores
 */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int B, int H, int N, int d, float scale, int causal, void* stream);

/* Rows per (batch, head) of the padded fp32 row arrays used by the backward
 * phases: N rounded up to a multiple of 256.  Returns 0 for N < 1. */
int fa2_bwd_rows_padded(int N);

/* Bytes of device workspace fa2_bwd needs: delta then L*log2(e), each fp32
 * [B,H,fa2_bwd_rows_padded(N)] and 256-byte aligned.  Returns 0 for
 * unsupported or invalid sizes.  For fa2_bwd_qk pass N = Nq (the row arrays
 * have one entry per query row). */
size_t fa2_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass: dQ, dK, dV from Q, K, V, the forward's O and L, and dO.
 * Runs, on `stream`, fa2_bwd_preprocess, fa2_bwd_dkdv and fa2_bwd_dq below
 * (one call each), using `workspace` for the two padded row arrays.
 *   q, k, v, o, dout : in, bf16 [B,H,N,d];  lse : in, fp32 [B,H,N] from fa2_fwd
 *   dq, dk, dv       : out, bf16 [B,H,N,d]
 *   workspace        : device scratch of >= fa2_bwd_workspace_bytes(B,H,N,d)
 *                      bytes, owned by the caller; its contents on entry do not
 *                      matter and on return are unspecified.
 */
int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv,
            int B, int H, int N, int d, float scale, int causal,
            void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass with separate query and key lengths: as fa2_bwd, with q, o,
 * dout, dq bf16 [B,H,Nq,d], lse fp32 [B,H,Nq], k, v, dk, dv bf16 [B,H,Nk,d]
 * and a workspace of >= fa2_bwd_workspace_bytes(B,H,Nq,d) bytes.  Runs
 * fa2_bwd_preprocess (N = Nq), fa2_bwd_dkdv_qk and fa2_bwd_dq_qk. */
int fa2_bwd_qk(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv,
               int B, int H, int Nq, int Nk, int d, float scale, int causal,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass that allocates nothing and takes no workspace: as fa2_bwd_qk,
 * with the two padded row arrays kept in a fixed device-resident scratch array
 * inside the library (fa2_bwd_noalloc_max_bytes() bytes, held by every GPU the
 * library runs on until the process ends).  For callers that cannot allocate
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It calls no allocating routine.
 *   Sizes: fa2_bwd_workspace_bytes(B,H,Nq,d) must not exceed
 *   fa2_bwd_noalloc_max_bytes() (32 MiB: B*H*Nq up to about 4 million query
 *   rows), else FA2_ERR_WORKSPACE and nothing is written.
 *   The scratch of the CURRENT device is used: `stream` must belong to it.
 *   Every call on a GPU shares that GPU's scratch, which keeps the last call's
 *   contents (nothing in it needs to start at zero: every row the kernels read
 *   is written first by the same call).  Calls that overlap in time on one GPU
 *   (on different streams, or from different threads) race on it; serialise
 *   them, for example by issuing them on one stream.
 * Other conventions and errors as for fa2_bwd_qk; the first call on a device
 * looks up the scratch's device address (a failure returns FA2_ERR_HIP).
 */
int fa2_bwd_qk_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv,
                       int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream);

/* Bytes of device scratch behind fa2_bwd_qk_noalloc (its size limit). */
size_t fa2_bwd_noalloc_max_bytes(void);

/* Backward phase 1 (HBM-bound, elementwise): for every row i of every head,
 * delta_i = sum_k dout_ik * o_ik and lse_log2_i = lse_i * log2(e); rows from N
 * up to fa2_bwd_rows_padded(N) get delta 0 and lse_log2 +inf, and so does the
 * lse_log2 of a row whose lse is -inf (a query that saw no key).
 *   o, dout : in, bf16 [B,H,N,d];  lse : in, fp32 [B,H,N]
 *   delta, lse_log2 : out, fp32 [B,H,Np], Np = fa2_bwd_rows_padded(N) */
int fa2_bwd_preprocess(const void* o, const void* dout, const float* lse, float* delta,
                       float* lse_log2, int B, int H, int N, int d, void* stream);

/* Backward phase 2: dK and dV.  One key/value column-block per workgroup,
 * looping over the query row-blocks that can see it (causal: from the diagonal
 * on), recomputing P = exp(scale q k^T - L) from lse_log2.
 *   q, k, v, dout   : in, bf16 [B,H,N,d];  lse_log2, delta : in, from phase 1
 *   dk, dv          : out, bf16 [B,H,N,d] */
int fa2_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                 const float* lse_log2, const float* delta, void* dk, void* dv,
                 int B, int H, int N, int d, float scale, int causal, void* stream);

/* Phase 2 with separate lengths: q, dout [B,H,Nq,d]; k, v, dk, dv [B,H,Nk,d];
 * lse_log2, delta from fa2_bwd_preprocess with N = Nq.  (Under the causal
 * alignment every key is seen by at least the last query.) */
int fa2_bwd_dkdv_qk(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse_log2, const float* delta, void* dk, void* dv,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream);

/* Backward phase 3: dQ.  One query row-block per workgroup, looping over the
 * key tiles it can see, recomputing S and dP; no atomics, no accumulator.
 *   q, k, v, dout   : in, bf16 [B,H,N,d];  lse_log2, delta : in, from phase 1
 *   dq              : out, bf16 [B,H,N,d] */
int fa2_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
               const float* lse_log2, const float* delta, void* dq,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/* Phase 3 with separate lengths: q, dout, dq [B,H,Nq,d]; k, v [B,H,Nk,d];
 * lse_log2, delta from fa2_bwd_preprocess with N = Nq.  A query that sees no
 * key gets dQ = 0. */
int fa2_bwd_dq_qk(const void* q, const void* k, const void* v, const void* dout,
                  const float* lse_log2, const float* delta, void* dq,
                  int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream);

/* Static description of a status code (never NULL). */
const char* fa2_strerror(int status);

/* Text of the last HIP error seen by a call on this thread ("" if none). */
const char* fa2_last_error(void);

/* Tile geometry used for head dimension d, for reporting: rows of the query
 * block per forward workgroup, keys per forward K/V tile, keys per backward
 * workgroup, queries per backward step, wavefronts per workgroup (fwd, bwd).
 * Returns FA2_ERR_UNSUPPORTED for other d. */
int fa2_tile_config(int d, int* fwd_block_q, int* fwd_block_k, int* bwd_block_k,
                    int* bwd_block_q, int* fwd_waves, int* bwd_waves);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
