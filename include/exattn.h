/*
 * exattn.h -- C ABI of the exact block-wise attention library (libexattn.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation.  Attention is a weighted average of value rows whose
 * weights are the softmax of query-key dot products ("Training a Large Video
 * Model on a Single Machine in a Day", section 3, "Flash Attention"
 * paragraph).  With the scale inside the softmax, per (batch b, head h):
 *
 *     S   = scale * Q K^T                       (Nq x Nkv, never stored)
 *     LSE = ln sum_j exp(S_ij)                  (per query row, natural log)
 *     O   = exp(S - LSE) V                      (Nq x d)
 *
 * The library computes this block by block with an online softmax, so the
 * Nq x Nkv weight matrix is never written to memory (same page, sections 1
 * and 3: results of on-chip-sized blocks are combined into the final output;
 * memory falls from O(N^2) to O(N)).  The result is exact up to floating
 * point rounding, not an approximation.
 *
 * Conventions shared by every call:
 *  - Tensors are [B, H, N, d] with the d (head dimension) stride equal to 1;
 *    the B, H and N strides are free (in elements, see attn_tensor).  A
 *    key/value chunk is therefore a strided view, never a copy.
 *  - All data pointers are DEVICE pointers allocated and owned by the
 *    caller.  The library never allocates, frees, copies to or from the host,
 *    or synchronises.  Each call validates its arguments on the host,
 *    enqueues its kernels on `stream` (a hipStream_t; NULL means the default
 *    stream) and returns.  Results are ready when the stream reaches them.
 *  - Validation happens before anything is enqueued: a call that returns an
 *    error other than ATTN_E_HIP has enqueued no work and touched no memory.
 *  - ATTN_E_HIP means a kernel launch was rejected by the HIP runtime; work
 *    enqueued earlier in the same call may have run.
 *  - No call prints, throws or aborts, and none keeps global mutable state
 *    except attn_bwd_noalloc's per-GPU scratch (see there).  Calls on
 *    distinct streams may run concurrently from different host threads.
 *  - Supported: d in {64, 80, 128}; inputs all F32 or all BF16.  bf16 inputs
 *    use bf16 matrix-core products with fp32 accumulation; f32 inputs use
 *    genuine fp32 products and accumulation.  B*H (or sequences * H for
 *    packed sequences) at most 2^31 - 1, else ATTN_E_UNSUPPORTED.
 */
#ifndef EXATTN_H
#define EXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 1

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = 1,      /* null pointer, non-positive size, mixed dtypes */
  ATTN_E_UNSUPPORTED = 2,  /* valid but not served: d, stride, alignment   */
  ATTN_E_WORKSPACE = 3,    /* workspace missing or smaller than required   */
  ATTN_E_HIP = 4           /* the HIP runtime rejected a launch            */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* A [B, H, N, d] tensor: element (b, h, n, c) lives at
 * ptr + (b*sb + h*sh + n*sn + c) elements.  ptr must be 16-byte aligned and
 * sn, sh, sb multiples of 8 (BF16) or 4 (F32) elements, so that a row of d
 * values can be moved with 16-byte vector accesses.  The row stride sn may
 * span at most 16 MiB (tiles are addressed with 32-bit offsets); larger
 * strides are ATTN_E_UNSUPPORTED. */
typedef struct {
  void* ptr;
  int32_t dtype;           /* attn_dtype */
  int64_t sb, sh, sn;
} attn_tensor;

/* Problem shape.  scale multiplies Q K^T inside the softmax (1/sqrt(d) for
 * the usual attention).  It must be finite (else ATTN_E_INVALID) and
 * positive (scale <= 0 is ATTN_E_UNSUPPORTED: the bf16 kernels take the
 * running row maximum over unscaled scores).  Inputs are expected to keep
 * scale * q.k within the fp32 range; scores are accumulated in fp32. */
typedef struct {
  int32_t B, H, Nq, Nkv, d;
  float scale;
} attn_problem;

/* attn_bwd flags.
 * DQ_ACCUMULATE: dq is F32 and the gradient is ADDED to it.  Used for the
 *   backward over key/value chunks, where dQ is the sum of the chunks'
 *   contributions.
 * D_PRECOMPUTED: the workspace already holds D = rowsum(dO * O) for these o
 *   and dout (from attn_bwd_preprocess, or an earlier attn_bwd call with the
 *   same o, dout and workspace); the preprocess is skipped and o may be NULL.
 *   Lets the chunks of a chunked backward share one preprocess.
 * NO_DQ / NO_DKDV: skip dQ (dq may be NULL) or dK and dV (dk, dv may be
 *   NULL).  The two halves are independent given D, so a caller may run them
 *   on two streams. */
#define ATTN_BWD_DQ_ACCUMULATE 1u
#define ATTN_BWD_D_PRECOMPUTED 2u
#define ATTN_BWD_NO_DQ 4u
#define ATTN_BWD_NO_DKDV 8u

/*
 * attn_fwd -- forward pass: O and the per-row log-sum-exp.
 *
 *   q  [B,H,Nq,d], k and v [B,H,Nkv,d]: same dtype (F32 or BF16).
 *   o  [B,H,Nq,d]: the input dtype, or F32 for any input (a partial that is
 *      later merged by attn_lse_merge).  Written, never read.
 *   lse [B,H,Nq] contiguous fp32: LSE_i = ln sum_j exp(scale q_i . k_j),
 *      natural log, scale included.  Written, never read.
 *
 * The log-sum-exp is the one O(N) statistic the backward needs (weights are
 * recomputed from it, not stored: the memory argument of "Training a Large
 * Video Model on a Single Machine in a Day", section 4.1)
 * and the one that lets partial results over disjoint key sets be merged
 * exactly (attn_lse_merge).
 */
attn_status attn_fwd(const attn_problem* p, attn_tensor q, attn_tensor k,
                     attn_tensor v, attn_tensor o, float* lse, void* stream);

/*
 * attn_fwd_chunked -- forward pass over n_chunks key/value chunks in one
 * launch, producing the per-chunk partials that attn_lse_merge combines.
 *
 * Chunk c covers key rows [c*L, min((c+1)*L, Nkv)) with L = ceil(Nkv /
 * n_chunks); a chunk with no rows yields O = 0 and LSE = -inf.  Exactly the
 * same as n_chunks calls of attn_fwd on the chunk views with F32 outputs.
 *
 * This is the one-GPU share of the LV-XAttn setting (ICML 2025 poster
 * "LV-XAttn", abstract): a small query block against large key/value blocks
 * that stay where they are, each block producing a partial result.
 *
 *   q [B,H,Nq,d], k/v [B,H,Nkv,d] (F32 or BF16).
 *   o_parts   [n_chunks,B,H,Nq,d] fp32 contiguous.  Written.
 *   lse_parts [n_chunks,B,H,Nq]   fp32 contiguous.  Written.
 */
attn_status attn_fwd_chunked(const attn_problem* p, int32_t n_chunks,
                             attn_tensor q, attn_tensor k, attn_tensor v,
                             float* o_parts, float* lse_parts, void* stream);

/*
 * attn_lse_merge -- exact merge of partials over disjoint key/value sets.
 *
 * Because exp(LSE) of a union of key sets is the sum of the parts' exp(LSE):
 *     M   = max_c LSE_c
 *     LSE = M + ln sum_c exp(LSE_c - M)
 *     O   = sum_c exp(LSE_c - LSE) O_c
 * (the exact, output-preserving combination of the LV-XAttn abstract and
 * lay summary).  A partial with LSE_c = -inf contributes nothing; a row whose
 * partials are all -inf gets O = 0 and LSE = -inf.
 *
 *   o_parts   [n_parts,B,H,Nq,d] fp32 contiguous.  Read only.
 *   lse_parts [n_parts,B,H,Nq]   fp32 contiguous.  Read only.
 *   o   [B,H,Nq,d] F32 or BF16 (strided like any attn_tensor).  Written.
 *   lse [B,H,Nq] fp32 contiguous.  Written.
 * n_parts >= 1.  d must be a multiple of 4 (64, 80, 128 are).
 */
attn_status attn_lse_merge(int32_t n_parts, int32_t B, int32_t H, int32_t Nq,
                           int32_t d, const float* o_parts,
                           const float* lse_parts, attn_tensor o, float* lse,
                           void* stream);

/*
 * attn_bwd_workspace_bytes -- device workspace attn_bwd needs for problem p
 * and the given flags (0 if p is invalid): B*H*Nq floats for D, rounded up
 * to 256 bytes; then, when dQ is computed for a short query block against a
 * long key range (the dQ pass then splits the keys into ranges so that the
 * whole GPU is used), the fp32 partials of dQ, ranges*B*H*Nq*d floats
 * rounded up to 256 bytes.  The size depends on the shape only, not on the
 * dtype.  The caller allocates it; unless ATTN_BWD_D_PRECOMPUTED is passed
 * its contents on entry do not matter (the D part is then read; the rest is
 * always scratch).
 */
size_t attn_bwd_workspace_bytes(const attn_problem* p, uint32_t flags);

/*
 * attn_bwd_preprocess -- D_i = sum_c dO_ic O_ic, the per-row term of the
 * softmax Jacobian (equal to sum_j P_ij dP_ij for the full row), in fp32.
 *
 *   o [B,H,Nq,d] (F32 or BF16), dout [B,H,Nq,d] (F32 or BF16).  Read only.
 *   dsum [B,H,Nq] fp32 contiguous, 4-byte aligned.  Written.  Passing the
 *      attn_bwd workspace here and ATTN_BWD_D_PRECOMPUTED to attn_bwd skips
 *      attn_bwd's own preprocess.
 */
attn_status attn_bwd_preprocess(const attn_problem* p, attn_tensor o, attn_tensor dout,
                                float* dsum, void* stream);

/*
 * attn_bwd -- backward pass for the loss gradient dO, from the saved LSE.
 *
 * The weights are recomputed block by block from Q, K and the saved LSE,
 * never loaded (the memory-for-compute trade of the AVION page, section 4.1,
 * and the activation recomputation of the LV-XAttn abstract):
 *     P  = exp(scale Q K^T - LSE)
 *     dV = P^T dO,   dP = dO V^T,   D_i = dO_i . O_i,
 *     dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q.
 * dK and dV are computed key-block by key-block and dQ query-block by
 * query-block, each output row by exactly one workgroup: no atomics, and the
 * results are bitwise reproducible.
 *
 *   q, k, v, dout: the forward's inputs and the output gradient, one dtype.
 *   o [B,H,Nq,d]: the forward output (F32 or BF16).  Only D = rowsum(dO*O)
 *      is taken from it.
 *   lse [B,H,Nq] fp32 contiguous: the forward's log-sum-exp.
 *   o and lse must describe the FULL softmax row.  For a key/value chunk,
 *   pass the merged O and LSE: each chunk then yields exactly its rows of dK
 *   and dV, and its contribution to dQ (use ATTN_BWD_DQ_ACCUMULATE).
 *   dq [B,H,Nq,d], dk/dv [B,H,Nkv,d]: the input dtype, written; except dq
 *      under ATTN_BWD_DQ_ACCUMULATE, which must be F32 and is added to.
 *   workspace: device memory of at least attn_bwd_workspace_bytes(p, flags)
 *      bytes, 256-byte aligned: D = rowsum(dO * O) (see ATTN_BWD_D_PRECOMPUTED).
 *   flags: ATTN_BWD_* above; passing both NO_DQ and NO_DKDV is invalid.
 */
attn_status attn_bwd(const attn_problem* p, attn_tensor q, attn_tensor k,
                     attn_tensor v, attn_tensor o, attn_tensor dout,
                     const float* lse, attn_tensor dq, attn_tensor dk,
                     attn_tensor dv, void* workspace, size_t workspace_bytes,
                     uint32_t flags, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, flags, results and errors are those of attn_bwd, without the
 * workspace: the workspace is a device array inside the library, one copy
 * per GPU, ATTN_NOALLOC_SCRATCH_BYTES (96 MiB) long, held from the library's
 * first use on that GPU until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its first call on
 * a GPU looks up that GPU's copy (hipGetSymbolAddress) once.
 *
 *   A problem whose attn_bwd_workspace_bytes(p, flags) exceeds the scratch
 *   returns ATTN_E_WORKSPACE with nothing enqueued (e.g. the 8-way split dQ
 *   pass of 4 x 32 heads x 128 queries x d = 128 needs 64 MiB + 64 KiB and
 *   fits; D alone for B*H*Nq rows needs 4 bytes per row).
 *   ATTN_BWD_D_PRECOMPUTED means: the scratch holds D from the previous
 *   call on this GPU with the same o and dout (its contents are kept
 *   between calls; nothing in it needs to start at zero).
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (different streams or host threads) race on it and must
 *   be ordered by the caller.  ATTN_E_HIP if the scratch cannot be looked up.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

attn_status attn_bwd_noalloc(const attn_problem* p, attn_tensor q, attn_tensor k,
                             attn_tensor v, attn_tensor o, attn_tensor dout,
                             const float* lse, attn_tensor dq, attn_tensor dk,
                             attn_tensor dv, uint32_t flags, void* stream);

/*
 * Packed variable-length sequences ("THD" layout).
 *
 * n_seq sequences of different lengths concatenated along one token axis,
 * the sequence packing of mixed image / video batches (NeMo video-model
 * page, "Efficient multimodal dataloading": variable-length images and
 * videos packed up to a maximum sequence length instead of padded).  Each
 * sequence attends only to itself: its query tokens [cu_q[s], cu_q[s+1])
 * against its key/value tokens [cu_kv[s], cu_kv[s+1]), with the same
 * softmax, LSE and gradients as a separate attn_fwd / attn_bwd per sequence.
 *
 *   q, o, dout, dq: [total_q, H, d]; k, v, dk, dv: [total_kv, H, d], as
 *      attn_tensor with sb ignored: token t, head h at t*sn + h*sh.
 *   lse (and D in the workspace): [H, total_q] fp32 contiguous.
 *   cu_q, cu_kv: DEVICE int32 arrays of n_seq + 1 prefix sums, non-
 *      decreasing, cu[0] = 0, cu_q[n_seq] = total_q, cu_kv[n_seq] =
 *      total_kv.  A sequence may be empty on either side (no keys: O = 0,
 *      LSE = -inf, dQ = 0; no queries: dK = dV = 0).
 *   max_q, max_kv: host bounds (>= 1) on every sequence's query and key
 *      lengths; they size the launch.  The arrays are read on the device
 *      only, and each span is clamped there: rows outside [0, total_q) or
 *      [0, total_kv) are dropped, a length above its bound is cut to the
 *      bound, and a pair cu[s] > cu[s+1] is an empty sequence.  So arrays
 *      that break the rules above give wrong results but never address
 *      rows outside the tensors.  The arrays themselves must hold n_seq + 1
 *      readable entries each.
 * scale as in attn_problem (finite, > 0).
 * BF16 only (F32 is ATTN_E_UNSUPPORTED); d in {64, 80, 128}.  Sequences with
 * both lengths <= 32 take the packed-tile kernels, longer ones the general
 * kernels (the resident-query dK/dV and split-key dQ variants are not used).
 */
typedef struct {
  int32_t n_seq, H, d;
  int32_t max_q, max_kv;
  int64_t total_q, total_kv;
  float scale;
  const int32_t* cu_q;
  const int32_t* cu_kv;
} attn_varlen;

attn_status attn_fwd_varlen(const attn_varlen* p, attn_tensor q, attn_tensor k, attn_tensor v,
                            attn_tensor o, float* lse, void* stream);

/* Workspace of attn_bwd_varlen: H * total_q floats for D, rounded up to 256
 * bytes (0 if p is invalid).  With ATTN_BWD_D_PRECOMPUTED it must hold D =
 * rowsum(dO * O) in [H, total_q] order: attn_bwd_preprocess with the problem
 * {B = 1, H, Nq = total_q, Nkv = 1, d} on the packed o and dout writes it. */
size_t attn_bwd_varlen_workspace_bytes(const attn_varlen* p);

/* Backward of attn_fwd_varlen; arguments and flags as attn_bwd (dq F32 and
 * added to under ATTN_BWD_DQ_ACCUMULATE). */
attn_status attn_bwd_varlen(const attn_varlen* p, attn_tensor q, attn_tensor k, attn_tensor v,
                            attn_tensor o, attn_tensor dout, const float* lse, attn_tensor dq,
                            attn_tensor dk, attn_tensor dv, void* workspace,
                            size_t workspace_bytes, uint32_t flags, void* stream);

/* Human-readable name of a status code (static storage). */
const char* attn_status_string(attn_status st);

/* ATTN_ABI_VERSION of the library that was loaded. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXATTN_H */
