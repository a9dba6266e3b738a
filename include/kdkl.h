/* kdkl.h — C ABI of the fused chunked top-K KL distillation loss (MI355X / gfx950).
 *
 * What it computes.  The pages "Efficient Knowledge Distillation for LLMs:
 * Offline Top-K Logits and a Fused Chunked KL Loss" (abstract) and "Making
 * Knowledge Distillation Cheap Enough to Run at Scale" (section "Two systems
 * changes") describe a KL-divergence distillation loss whose student side is
 * the output projection of hidden states h[T,H] through the head weight
 * W[V,H], and whose teacher side is an offline cache of the teacher's top-K
 * logits per position.  The fused variant projects, reduces and discards one
 * chunk of logits at a time and recomputes each chunk in the backward pass,
 * so the T x V logit tensor is never stored.  With the readings this library
 * adopts (tau divides both sides, no tau^2 factor, mean over kept tokens):
 *
 *   q[t,v]  = softmax_v(S[t,:]/tau),  S = h W^T          (full vocabulary)
 *   p[t,k]  = softmax_k(teacher_logit[t,k]/tau)          (renormalised over K)
 *   P[t,v]  = sum_k p[t,k] [teacher_idx[t,k] == v]        (duplicates add)
 *   KL_t    = sum_v P[t,v] (log P[t,v] - log q[t,v])      (0 log 0 = 0)
 *   loss    = (1/N) sum_t mask_t KL_t,  N = sum_t mask_t  (loss = 0 if N = 0)
 *   dH      = G W,  dW = G^T h,  G[t,v] = mask_t (q[t,v] - P[t,v]) / (N tau)
 *
 * Precision: bf16 h and W, fp32 MFMA accumulation, fp32 exponentials and
 * logarithms, the logit gradient rounded once to bf16 (round to nearest
 * even) before the two gradient contractions, fp32 dH and dW.
 *
 * Memory: besides the caller's inputs and outputs the library touches only
 * the caller's workspace (see kd_topk_kl_workspace_size): two fixed
 * block_t x chunk_v bf16 gradient buffers (one when the call has a single
 * token block and vocabulary chunk, or with KD_FLAG_SEQ_CHUNK a single
 * vocabulary chunk), h^T of one token block (H x block_t
 * bf16), when H % 256 is 64 or 128 a copy of W's last H % 256 columns
 * ((H % 256) x V bf16, rounded up to 64 columns of V), plus
 * O(T*K + T*V/256) per-token state.  It allocates no device
 * memory, keeps no state between calls (except the optional timing
 * facility below and the static scratch of kd_topk_kl_fwd_bwd_noalloc) and
 * is reentrant across streams given distinct workspaces.
 */
#ifndef KDKL_H
#define KDKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kd_status {
  KD_OK = 0,
  KD_ERR_ARG = 1,          /* invalid argument (null pointer, bad size, tau <= 0 ...) */
  KD_ERR_UNSUPPORTED = 2,  /* valid but not supported: H % 64 != 0, K > 1024, bad alignment,
                              chunk_v / block_t not multiples of 256, or one chunk or block
                              too large for 32-bit offsets: chunk_v * H * 4, block_t * H * 4
                              and block_t * chunk_v * 2 must each be below 4 GiB, and
                              256 * block_t * 4 too with KD_FLAG_SEQ_CHUNK (the chunk
                              and block actually used, defaults included); or a launch
                              grid past 2^32 work-items (the limits on T, T * K and,
                              for pass 1, (block / 256) * ceil(V / 256) at most 2^24 - 8) */
  KD_ERR_WORKSPACE = 3,    /* workspace_bytes smaller than kd_topk_kl_workspace_size() */
  KD_ERR_INDEX = 4,        /* (KD_FLAG_VALIDATE) a kept row has a teacher id outside [0, V) */
  KD_ERR_NONFINITE = 5,    /* (KD_FLAG_VALIDATE) a kept row has a NaN/+inf logit or all -inf */
  KD_ERR_HIP = 6,          /* a HIP runtime call failed (no device, launch failure ...) */
  /* not a status: gives the enum the value range of int32_t, so any code
   * handed back to kd_status_string is a valid kd_status value in C++ too */
  KD_STATUS_RANGE_ = INT32_MIN
} kd_status;

/* Check teacher ids and logits of kept rows on the device, then synchronise
 * the stream and report KD_ERR_INDEX / KD_ERR_NONFINITE.  Without this flag
 * valid inputs are a precondition (out-of-range ids never fault: they read
 * zeros and give meaningless results). */
#define KD_FLAG_VALIDATE 1u
/* Gradient outputs: add to dH / dW instead of overwriting them (e.g. a
 * parameter gradient summed over micro-batches). */
#define KD_FLAG_ACCUMULATE_DH 2u
#define KD_FLAG_ACCUMULATE_DW 4u
/* dH and dW are bf16 (bit patterns) instead of fp32.  The contractions still
 * accumulate in fp32 inside the workspace (one token block of dH,
 * [block_t,H], and one chunk of dW, [chunk_v,H], or all of dW [V,H] when T
 * exceeds one token block; with KD_FLAG_SEQ_CHUNK all of dH [T,H]) and each
 * output element is rounded to bf16 once (to nearest
 * even), after its last contribution (with an accumulate flag: once, after
 * adding the previous bf16 value in fp32). */
#define KD_FLAG_GRAD_BF16 8u
/* kd_topk_kl_fwd_bwd only: the sequence-chunk schedule of the blog "Making
 * Knowledge Distillation Cheap Enough to Run at Scale" (section "Two systems
 * changes": one chunk of the sequence at a time).  The forward pass keeps a
 * token block's logits (fp32, block_t x V, in the workspace) and the backward
 * forms the logit gradient from them instead of recomputing the projection:
 * 6 T H V instead of 8 T H V flops, for block_t * V * 4 bytes of workspace
 * (block_t = 0 means 4096 here).  Same results up to fp32 rounding order.
 * kd_topk_kl_fwd / kd_topk_kl_bwd ignore it (size their workspaces without
 * it). */
#define KD_FLAG_SEQ_CHUNK 16u

typedef struct kd_problem {
  int64_t T;        /* tokens (rows of h); 0 allowed (loss = 0, dW = 0); at most
                       2^26 - 256, and T * K at most 2^32 - 256 */
  int64_t H;        /* hidden size; multiple of 64 */
  int64_t V;        /* vocabulary size; >= 1 */
  int32_t K;        /* cached teacher entries per token; 1 <= K <= min(V, 1024) */
  float tau;        /* temperature; finite, > 0 */
  int32_t chunk_v;  /* vocabulary chunk of the gradient pass, multiple of 256;
                       0 = 12288 for a token block of at most 4096, else 8192
                       (16384 with KD_FLAG_SEQ_CHUNK) */
  int32_t block_t;  /* token block of both passes, multiple of 256; 0 = 8192
                       (4096 with KD_FLAG_SEQ_CHUNK) */
  uint32_t flags;   /* KD_FLAG_* */
} kd_problem;

/* Bytes of device workspace kd_topk_kl_fwd_bwd and kd_topk_kl_bwd need for
 * this problem (flags included).  Synchronous, host only; returns
 * KD_ERR_ARG / KD_ERR_UNSUPPORTED for a problem the main call would reject. */
kd_status kd_topk_kl_workspace_size(const kd_problem* p, size_t* bytes);

/* The tiling kd_topk_kl_fwd_bwd / kd_topk_kl_bwd use for this problem (the
 * caller's chunk_v / block_t, else the defaults): tokens per block (T
 * rounded up to 256 when below one block), vocabulary rows per chunk, and
 * the number of bf16 gradient buffers (2 when the call has several (block,
 * chunk) units: unit i's contractions share a launch with unit i + 1's
 * pass 2).  Synchronous, host only. */
kd_status kd_topk_kl_tiling(const kd_problem* p, int64_t* block_t, int64_t* chunk_v, int32_t* gbufs);

/* Forward and backward of the loss above, enqueued on `stream`.
 *
 *   h             [T,H]  bf16 bit patterns, row-major, device, 16-byte aligned
 *   W             [V,H]  bf16 bit patterns, row-major, device, 16-byte aligned
 *   teacher_idx   [T,K]  int32 vocabulary ids, row-major, device
 *   teacher_logit [T,K]  fp32 cached teacher logits (any per-row shift; -inf = no mass)
 *   mask          [T]    uint8, nonzero = token counts; NULL = all tokens count
 *   loss          [1]    fp32, device, overwritten
 *   dH            [T,H]  fp32 (bf16 with KD_FLAG_GRAD_BF16), device, 16-byte aligned,
 *                        overwritten (added to with KD_FLAG_ACCUMULATE_DH); NULL = not computed
 *   dW            [V,H]  as dH (KD_FLAG_ACCUMULATE_DW); NULL = not computed
 *   row_loss      [T]    fp32 mask_t * KL_t (not divided by N), device; NULL = not written
 *   workspace     device memory of at least kd_topk_kl_workspace_size() bytes,
 *                 256-byte aligned; contents on entry are irrelevant
 *   stream        hipStream_t (NULL = the null stream)
 *
 * All pointers are borrowed: the caller owns every buffer, which must stay
 * valid until the stream reaches this call's end.  Argument errors are
 * returned synchronously before anything is enqueued; otherwise the call
 * returns KD_OK as soon as the work is enqueued (KD_FLAG_VALIDATE: after it
 * has finished).  With dH = dW = NULL only the loss pass runs. */
kd_status kd_topk_kl_fwd_bwd(const kd_problem* p,
                             const uint16_t* h, const uint16_t* W,
                             const int32_t* teacher_idx, const float* teacher_logit,
                             const uint8_t* mask,
                             float* loss, void* dH, void* dW, float* row_loss,
                             void* workspace, size_t workspace_bytes, void* stream);

/* kd_topk_kl_fwd_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: the library holds
 * one static device scratch array of KD_NOALLOC_SCRATCH_BYTES per GPU, from
 * its first use on that GPU until the process ends, and runs the same
 * kernels with the same tiling as kd_topk_kl_fwd_bwd (bitwise the same
 * results for the same problem) through one gradient buffer instead of two
 * (each unit's pass 2 and contractions in launches of their own).
 *
 *   Arguments as kd_topk_kl_fwd_bwd, minus workspace / workspace_bytes.  The
 *   stream must belong to the current device (KD_ERR_ARG otherwise).
 *   A problem whose single-buffer workspace (kd_topk_kl_workspace_size
 *   less one block_t x chunk_v bf16 gradient buffer when the call has more
 *   than one (block, chunk) unit) exceeds KD_NOALLOC_SCRATCH_BYTES returns
 *   KD_ERR_WORKSPACE before anything is enqueued; the gpt-oss-20b-like head
 *   (T 4096, H 2880, V 201088, K 64) fits with chunk_v = 8192 (114 MiB).
 *   The first call on a GPU looks up that GPU's scratch address
 *   (hipGetSymbolAddress); make it outside graph capture.
 *   Every call on one GPU uses the same scratch, which keeps the last call's
 *   contents (nothing in it is assumed zero on entry): calls ordered on one
 *   stream are safe, calls that may overlap on one GPU (different streams,
 *   other threads) race on it. */
#define KD_NOALLOC_SCRATCH_BYTES (128u << 20)
kd_status kd_topk_kl_fwd_bwd_noalloc(const kd_problem* p,
                                     const uint16_t* h, const uint16_t* W,
                                     const int32_t* teacher_idx, const float* teacher_logit,
                                     const uint8_t* mask,
                                     float* loss, void* dH, void* dW, float* row_loss,
                                     void* stream);

/* The same loss split into its two passes, for autograd-style callers (the
 * blog "Making Knowledge Distillation Cheap Enough to Run at Scale", section
 * "Two systems changes": the forward folds each chunk into the running loss
 * and discards it; the backward recomputes each chunk).
 *
 * kd_topk_kl_fwd runs the loss pass only and leaves in `saved` (caller-owned
 * device memory of kd_topk_kl_saved_size() bytes, 256-byte aligned) what the
 * backward needs: the per-token log-sum-exp (fp32 [T] at offset 0, log2
 * units as in kd_topk_kl_workspace_lse2) followed by the student logits at
 * the cached teacher ids.  Its workspace is kd_topk_kl_fwd_workspace_size()
 * bytes (no gradient buffer).  Arguments otherwise as kd_topk_kl_fwd_bwd.
 *
 * kd_topk_kl_bwd takes the same problem and inputs plus `saved` from a
 * kd_topk_kl_fwd call on them, and writes grad_loss * d(loss)/dH and
 * grad_loss * d(loss)/dW, where grad_loss is an fp32 scalar in device memory
 * (NULL = 1); the flags KD_FLAG_ACCUMULATE_* and KD_FLAG_GRAD_BF16 apply.
 * Its workspace is kd_topk_kl_workspace_size() bytes.  `saved` is only
 * read, so one forward can be followed by several backward calls. */
kd_status kd_topk_kl_saved_size(const kd_problem* p, size_t* bytes);
kd_status kd_topk_kl_fwd_workspace_size(const kd_problem* p, size_t* bytes);
kd_status kd_topk_kl_fwd(const kd_problem* p,
                         const uint16_t* h, const uint16_t* W,
                         const int32_t* teacher_idx, const float* teacher_logit,
                         const uint8_t* mask,
                         float* loss, float* row_loss, void* saved,
                         void* workspace, size_t workspace_bytes, void* stream);
kd_status kd_topk_kl_bwd(const kd_problem* p,
                         const uint16_t* h, const uint16_t* W,
                         const int32_t* teacher_idx, const float* teacher_logit,
                         const uint8_t* mask,
                         const void* saved, const float* grad_loss,
                         void* dH, void* dW,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Forward-chunked KL on materialised student logits.  The page "Making
 * Knowledge Distillation Cheap Enough to Run at Scale", section "Two systems
 * changes", describes this variant: the teacher stays sparse (its cached
 * top-K) while the student's logits Z[T,V] exist in full; the loss is the
 * same, and the gradient returned is the one with respect to the logits:
 *
 *   dZ[t,v] = mask_t (softmax_v(Z[t,:]/tau) - P[t,v]) / (N tau)
 *
 * It reads Z once for the log-sum-exp and once more for dZ (HBM-bound).
 */
#define KD_FLAG_LOGITS_F32 32u  /* Z and dZ are fp32 (default: bf16 bit patterns) */

typedef struct kd_logits_problem {
  int64_t T;        /* rows of Z; 0 allowed (loss = 0); below 2^23 */
  int64_t V;        /* vocabulary size; >= 1 */
  int32_t K;        /* cached teacher entries per row; 1 <= K <= min(V, 1024) */
  float tau;        /* temperature; finite, > 0 */
  uint32_t flags;   /* KD_FLAG_VALIDATE | KD_FLAG_LOGITS_F32 */
} kd_logits_problem;

kd_status kd_topk_kl_logits_workspace_size(const kd_logits_problem* p, size_t* bytes);

/*   Z             [T,V]  bf16 (or fp32) student logits, row-major, device, 16-byte aligned
 *   teacher_idx, teacher_logit, mask, loss, row_loss: as kd_topk_kl_fwd_bwd
 *   dZ            [T,V]  same type as Z, device, 16-byte aligned, overwritten; NULL = loss only
 * Rows whose byte length is not a multiple of 16 take a slower element-wise
 * path.  Same conventions (errors, ownership, asynchrony) as above. */
kd_status kd_topk_kl_logits(const kd_logits_problem* p, const void* Z,
                            const int32_t* teacher_idx, const float* teacher_logit,
                            const uint8_t* mask, float* loss, void* dZ, float* row_loss,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Top-K selection: the producer of the teacher cache (the page "Making
 * Knowledge Distillation Cheap Enough to Run at Scale", section "Two systems
 * changes": the teacher's K most likely tokens per position are computed
 * once and cached).  For every row of X[T,V] (teacher logits, bf16 bit
 * patterns, row-major, device, 16-byte aligned) it writes the ids of the K
 * largest values in descending order of value, equal values by ascending id
 * (so the result is unique; -0 counts as +0), and the values (exact, fp32).
 * Values are ordered as real numbers; NaN rows are a precondition violation.
 * v1 limits: V % 8 == 0 and V <= 2^30 - 1 (KD_ERR_UNSUPPORTED otherwise),
 * 1 <= K <= min(V, 1024).
 * No workspace; asynchronous on `stream`.
 */
typedef struct kd_topk_problem {
  int64_t T;        /* rows; 0 allowed; below 2^23 */
  int64_t V;        /* row length */
  int32_t K;        /* entries per row */
  uint32_t flags;   /* must be 0 */
} kd_topk_problem;

kd_status kd_topk_select(const kd_topk_problem* p, const uint16_t* X,
                         int32_t* idx, float* values, void* stream);

/* Device address, inside a workspace used by the last completed call with
 * problem p, of the per-token log-sum-exp of S/tau (natural log would be
 * value * ln 2: the array holds log2 of sum_v 2^(log2(e) S[t,v]/tau), fp32,
 * [T]).  NULL if p is invalid. */
const float* kd_topk_kl_workspace_lse2(const kd_problem* p, const void* workspace);

/* Static message for a status code. */
const char* kd_status_string(kd_status s);

/* ABI version (incremented on any change of the declarations above; 2 adds
 * the split forward / backward entry points and the gradient flags, 3 the
 * logits variant, the top-K selection and two more timing classes, 4 the
 * timing class mask, 5 the allocation-free fused call, the tiling query and
 * timing class 11). */
int kd_abi_version(void);

/* Optional per-kernel timing with HIP events recorded on the launch stream
 * around every launch of the library's kernels while enabled.  Intended for
 * benchmarks; the state is process-wide (calls from several threads add
 * their launches to one list, under a lock).  Kernel classes: 0 teacher, 1 gather,
 * 2 pass1, 3 lse, 4 loss, 5 pass2, 6 buckets (the teacher entries bucketed
 * by tile and their gradient values), 7 bwd, 8 other, 9 logits (the row kernel of
 * kd_topk_kl_logits), 10 topk (kd_topk_select), 11 bwd_pass2 (one unit's
 * contractions with the next unit's pass 2).
 * kd_timing_collect synchronises the recorded events, adds each class's
 * elapsed milliseconds and launch count to ms[12] / launches[12] (either may
 * be NULL) and releases the events. */
kd_status kd_timing_enable(int on);
kd_status kd_timing_collect(double* ms, int64_t* launches);
/* Restricts the timing to the classes whose bit (1 << class) is set in mask
 * (default: all); the other launches record no events, so that timing one
 * kernel adds no event traffic between the rest.  Bits of unknown classes
 * are ignored. */
kd_status kd_timing_classes(uint32_t mask);

#ifdef __cplusplus
}
#endif
#endif /* KDKL_H */
