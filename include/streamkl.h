/*
 * streamkl.h - C ABI of the fused attention KL-divergence library for AMD
 * MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   "StreamKL: Fast and Memory-Efficient KL Divergence for Boosting Attention
 *   Distillation" (gist.science technical summary):
 *     - Problem Statement: two attention distributions P1 = softmax(S1) (the
 *       teacher) and P2 = softmax(S2) (the student), both N_Q x N_K, compared
 *       row by row with the KL divergence KL(P1 || P2).
 *     - Methodology 1, Online Formulation: a single pass over key tiles keeps
 *       five running scalars per row (m1, m2, l1, l2, acc); the row loss is
 *       acc / l1 + LSE2 - LSE1 with LSE_t = m_t + log l_t.  Causal key tiles
 *       past the frontier are skipped.
 *     - Methodology 2, Recomputation Strategy: only KL, LSE1, LSE2 are saved;
 *       the backward regenerates P_t = exp(S_t - LSE_t) tile by tile, for
 *       Setting 1 (P1 fixed, gradients to Q2, K2) and Setting 2 (P2 fixed,
 *       gradients to Q1, K1); a fused kernel accumulates dQ with atomics,
 *       with separate kernels as the fallback.
 *     - Methodology 3, GPU Kernel Optimizations: a split-K variant divides
 *       the keys among workgroups when there are few queries (decode).
 *
 * Conventions shared by every entry point
 *   S_t = scale * Q_t K_t^T, t = 1, 2, one scale for both distributions.
 *   Logarithms are natural: KL in nats, LSE in nats.
 *   Layout: Q1, Q2 are [heads, n_q, head_dim], K1, K2 are [heads, n_k,
 *     head_dim], row-major, head_dim contiguous, base addresses 16-byte
 *     aligned.  (A batch dimension is folded into heads.)  All four inputs
 *     share one dtype.
 *   Causal: query i sees key j iff j <= i + (n_k - n_q) (bottom-right
 *     alignment); causal with n_q > n_k is rejected.
 *   Outputs are fp32: kl, lse1, lse2 are [heads, n_q]; gradients are
 *     [heads, n, head_dim] like the tensor they belong to.
 *   Pointers: every array argument is DEVICE memory owned by the caller.  The
 *     library keeps no pointer after the call returns and allocates no device
 *     memory of its own.
 *   Streams: all work is enqueued on `stream` (0 = the null stream); there is
 *     no host synchronisation.  Outputs are complete once the stream reaches
 *     the point after the call.
 *   Errors: arguments are validated before anything is enqueued; a negative
 *     status is returned and nothing runs.  A launch failure is reported as
 *     STREAMKL_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   Supported: head_dim 64 or 128; dtype bf16 or fp32; scale finite and >= 0;
 *     n_q, n_k, heads >= 1 with heads * n_q and heads * n_k below 2^31 rows.
 *   Thread safety: calls may be made from several host threads; calls that
 *     write the same outputs must be ordered by the caller.
 *   Environment (read once per process, at the first call that needs it; for
 *     experiments, the arguments stay the interface):
 *     STREAMKL_LOG=1     one line on stderr per compute call: its shape, what
 *                        was chosen (split count and its source, backward
 *                        path, workgroup counts) and the status returned.
 *     STREAMKL_SPLITS=n  the split count num_splits = 0 resolves to
 *                        (1 <= n <= 1024, then reduced to the non-empty key
 *                        ranges); streamkl_splitk_auto and
 *                        streamkl_workspace_bytes report it too.
 *     STREAMKL_BWD_PATH=fused|separate  the path STREAMKL_BWD_AUTO resolves
 *                        to in streamkl_bwd_set1/2 and streamkl_bwd_select
 *                        (fused falls back to separate where unsupported);
 *                        streamkl_bwd_both has no fused variant and ignores it.
 *     A value that does not parse is ignored with a warning on stderr.  Tile
 *     shapes are compile-time constants of the kernels and have no override.
 */
#ifndef STREAMKL_H
#define STREAMKL_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { STREAMKL_BF16 = 0, STREAMKL_FP32 = 1 } streamkl_dtype;

typedef enum {
  STREAMKL_BWD_AUTO = 0,      /* library chooses (see streamkl_bwd_select) */
  STREAMKL_BWD_FUSED = 1,     /* one kernel per (head, key block); dQ by fp32 atomics */
  STREAMKL_BWD_SEPARATE = 2,  /* a dK kernel and a dQ kernel, each recomputing P */
  STREAMKL_BWD_DK_ONLY = 3,   /* only the dK kernel of the separate path; dQ is not
                                 written and may be NULL (e.g. queries frozen) */
  STREAMKL_BWD_DQ_ONLY = 4    /* only the dQ kernel of the separate path; dK is not
                                 written and may be NULL (e.g. keys frozen) */
} streamkl_bwd_path;

enum {
  STREAMKL_OK = 0,
  STREAMKL_ERR_NULL = -1,         /* a required pointer is NULL */
  STREAMKL_ERR_SHAPE = -2,        /* n_q, n_k or heads < 1, too large, or causal with n_q > n_k */
  STREAMKL_ERR_UNSUPPORTED = -3,  /* head_dim, dtype, path or split count not supported */
  STREAMKL_ERR_SCALE = -4,        /* scale not finite or negative */
  STREAMKL_ERR_WORKSPACE = -5,    /* workspace NULL or smaller than streamkl_workspace_bytes */
  STREAMKL_ERR_HIP = -6,          /* a HIP launch reported an error */
  STREAMKL_ERR_ALIGN = -7,        /* an array is not 16-byte aligned */
  STREAMKL_ERR_TOO_LARGE = -8     /* streamkl_fwd_splitk_noalloc: the partial states would
                                     exceed STREAMKL_NOALLOC_SCRATCH_BYTES */
};

/*
 * Fused one-pass forward (Methodology 1, Online Formulation).
 * Inputs q1, k1, q2, k2 (dtype `dtype`, layout above).  Writes per row
 * kl[h, i] = KL(P1_i || P2_i), lse1[h, i], lse2[h, i] (fp32, [heads, n_q]).
 * Extra device memory: none beyond the three O(n_q) outputs.
 */
int streamkl_fwd(const void* q1, const void* k1, const void* q2, const void* k2,
                 int n_q, int n_k, int heads, int head_dim, int causal, float scale,
                 streamkl_dtype dtype, float* kl, float* lse1, float* lse2,
                 hipStream_t stream);

/*
 * Split-K forward (Methodology 3, Split-K Variant): the keys of every row are
 * divided into `num_splits` contiguous ranges processed by different
 * workgroups; each writes its partial (m1, l1, acc, m2, l2) state to
 * `workspace`, and a second kernel on the same stream merges the states and
 * writes kl, lse1, lse2 as streamkl_fwd does.  num_splits = 0 lets the
 * library choose (streamkl_splitk_auto); otherwise 1 <= num_splits <= 1024.
 * A call whose grid would reach 2^31 workgroups (heads x query blocks x
 * splits; a query block is 128 queries, or 32 when n_q <= 32) returns
 * STREAMKL_ERR_SHAPE.
 * workspace: device memory of at least
 *   streamkl_workspace_bytes(0, n_q, n_k, heads, head_dim, num_splits, 0)
 * bytes, owned by the caller; its contents on entry are ignored.
 */
int streamkl_fwd_splitk(const void* q1, const void* k1, const void* q2, const void* k2,
                        int n_q, int n_k, int heads, int head_dim, int causal, float scale,
                        streamkl_dtype dtype, int num_splits,
                        float* kl, float* lse1, float* lse2,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the fixed device scratch behind streamkl_fwd_splitk_noalloc. */
#define STREAMKL_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * Split-K forward that allocates nothing, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same operation, arguments
 * (minus the workspace), kernels and results as streamkl_fwd_splitk with the
 * same num_splits; the partial states go to a fixed scratch array of
 * STREAMKL_NOALLOC_SCRATCH_BYTES (8 MiB) in the library's device memory, one
 * per GPU, held until the process ends.  The partial states take
 * 20 * splits * heads * n_q bytes (splits as streamkl_workspace_bytes(0, ...)
 * counts them); a call that needs more returns STREAMKL_ERR_TOO_LARGE before
 * anything is enqueued.  The first call on a device looks the scratch up
 * (hipGetSymbolAddress) with that device current; no call allocates.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams, or different host threads without ordering)
 * race and must be serialised by the caller.  No clearing is needed between
 * calls: each call writes every partial state its combine reads.
 */
int streamkl_fwd_splitk_noalloc(const void* q1, const void* k1, const void* q2, const void* k2,
                                int n_q, int n_k, int heads, int head_dim, int causal, float scale,
                                streamkl_dtype dtype, int num_splits,
                                float* kl, float* lse1, float* lse2, hipStream_t stream);

/*
 * Backward, Setting 1 (Methodology 2: P1 fixed, gradients to the student).
 * With g = dkl (fp32 [heads, n_q]; NULL means all ones) the loss is
 * sum_i g_i KL_i, and dS2 = g (P2 - P1).  Writes dq2 = scale dS2 K2 and
 * dk2 = scale dS2^T Q2 (fp32, [heads, n_q, head_dim] and [heads, n_k,
 * head_dim]), overwriting them.  lse1, lse2 are the forward's outputs for the
 * same inputs.  `path` picks the fused or separate kernels (AUTO: the
 * library's choice); DK_ONLY / DQ_ONLY compute one of the two gradients.
 * Calling DK_ONLY then DQ_ONLY gives the same result as SEPARATE.
 * workspace: at least streamkl_workspace_bytes(1, ...) bytes (may be NULL
 * when that is 0, which it is for every shape today).
 */
int streamkl_bwd_set1(const void* q1, const void* k1, const void* q2, const void* k2,
                      int n_q, int n_k, int heads, int head_dim, int causal, float scale,
                      streamkl_dtype dtype, const float* lse1, const float* lse2,
                      const float* dkl, float* dq2, float* dk2, streamkl_bwd_path path,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward, Setting 2 (Methodology 2: P2 fixed, gradients to the teacher).
 * dS1 = g P1 ((S1 - LSE1) - (S2 - LSE2) - KL), the log ratio taken from
 * logits and saved LSEs (Methodology 3, Numerical Stability); kl is the
 * forward's per-row output.  Writes dq1 = scale dS1 K1, dk1 = scale dS1^T Q1.
 * Other arguments as for streamkl_bwd_set1.
 */
int streamkl_bwd_set2(const void* q1, const void* k1, const void* q2, const void* k2,
                      int n_q, int n_k, int heads, int head_dim, int causal, float scale,
                      streamkl_dtype dtype, const float* lse1, const float* lse2,
                      const float* kl, const float* dkl, float* dq1, float* dk1,
                      streamkl_bwd_path path, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Backward, both settings at once (Methodology 2, both gradient settings for
 * the same loss sum_i g_i KL_i): writes Setting 2's dq1 = scale dS1 K1,
 * dk1 = scale dS1^T Q1 and Setting 1's dq2 = scale dS2 K2, dk2 = scale dS2^T Q2
 * (fp32, overwritten), from one recomputation of S1, S2 and P1 per
 * (query, key) pair, where calling streamkl_bwd_set1 and streamkl_bwd_set2
 * recomputes them twice.  kl, lse1, lse2 are the forward's outputs; dkl as
 * for streamkl_bwd_set1 (NULL = all ones).  The four output arrays must not
 * overlap.  bf16 runs dedicated kernels (a dK kernel and a dQ kernel, one
 * wave per SIMD); fp32 runs the two settings' separate kernels one after the
 * other.  path: AUTO or SEPARATE (all four gradients), DK_ONLY (dk1, dk2;
 * dq1, dq2 untouched and may be NULL) or DQ_ONLY (dq1, dq2); FUSED is
 * STREAMKL_ERR_UNSUPPORTED.  Needs no workspace.
 */
int streamkl_bwd_both(const void* q1, const void* k1, const void* q2, const void* k2,
                      int n_q, int n_k, int heads, int head_dim, int causal, float scale,
                      streamkl_dtype dtype, const float* lse1, const float* lse2,
                      const float* kl, const float* dkl, float* dq1, float* dk1,
                      float* dq2, float* dk2, streamkl_bwd_path path, hipStream_t stream);

/*
 * Device workspace, in bytes, that an entry point needs:
 *   op 0 = streamkl_fwd_splitk (num_splits 0 = the automatic choice),
 *   op 1 = streamkl_bwd_set1, op 2 = streamkl_bwd_set2.
 * Returns 0 for an op that needs none, and (size_t)-1 for invalid arguments.
 */
size_t streamkl_workspace_bytes(int op, int n_q, int n_k, int heads, int head_dim,
                                int num_splits, streamkl_bwd_path path);

/* The split count streamkl_fwd_splitk uses when num_splits = 0 (the
 * heuristic, or STREAMKL_SPLITS when set). */
int streamkl_splitk_auto(int n_q, int n_k, int heads, int head_dim);

/* The backward path AUTO resolves to for this shape (STREAMKL_BWD_FUSED or
 * STREAMKL_BWD_SEPARATE).  The pages (Methodology 2, Recomputation Strategy,
 * its Kernel Fusion paragraph) prefer the fused kernel while the dQ buffer
 * fits the cache.  On MI355X the fused kernel moves 4 * head_dim / 128 bytes of
 * fp32 atomics per (query, key) pair and was measured slower than the separate
 * kernels at every size tried (64 to 16K queries against 128K keys, both
 * settings), so the result does not depend on the arguments: it is
 * STREAMKL_BWD_SEPARATE for every shape, unless STREAMKL_BWD_PATH is set.
 * The arguments are kept so that a shape-dependent rule can be added without
 * changing the ABI. */
int streamkl_bwd_select(int n_q, int n_k, int heads, int head_dim, int causal);

/* Static text for a status code. */
const char* streamkl_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* STREAMKL_H */
