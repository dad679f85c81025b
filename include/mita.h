/* MiTA (Mixture of Top-k Activations) attention forward pass on one AMD Instinct
 * MI355X (gfx950): C ABI.
 *
 * The operation is the one described on the three gist.science summaries of
 * "MiTA Attention: Efficient Fast-Weight Scaling via a Mixture of Top-k
 * Activations" (Arabic, Dutch and Hindi pages). Per (batch, head) slice, with
 * Q, K, V of shape [N, d] and no mask:
 *   1. landmark queries Q~ [m, d]: adaptive average pooling of Q
 *      (Arabic/Hindi section 2, "mechanism details"; Dutch "Kernconcepten" 1);
 *   2. shared expert V~ = softmax(Q~ K^T / sqrt d) V, Q~ also being its keys
 *      (Arabic/Hindi section 2; Dutch "Kernconcepten" 2, "Wiskundige Formulering");
 *   3. deformable experts I_i = the k tokens n with the largest q~_i . K_n
 *      (Arabic/Hindi section 2; Dutch "Kernconcepten" 3);
 *   4. routing: query q goes to the s landmarks with the largest q . q~_i
 *      (the pages leave the rule open; this dot-product top-s is the reading taken);
 *   5. output: softmax(q K*^T / sqrt d) V* with K* = [Q~, K_{I_e1}, .., K_{I_es}],
 *      V* = [V~, V_{I_e1}, .., V_{I_es}] (Dutch "Wiskundige Formulering").
 *      A token present in two of a query's experts is counted twice.
 * Ties in steps 3 and 4 go to the lower index.
 *
 * Conventions for every entry point
 *   - Tensors are device pointers, row-major and contiguous: Q, K, V and out are
 *     [B, H, N, d] with d fastest, all of the dtype named in the shape (bf16 as
 *     raw 16-bit patterns, or fp32). The caller allocates and owns every buffer;
 *     the library keeps no pointer after a call returns and allocates no device
 *     memory (mita_forward keeps one side stream and two events per device).
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously; the call returns without synchronising. Device faults show
 *     up at the caller's next synchronisation.
 *   - Arguments are checked before anything is enqueued. A failed check returns
 *     a negative status and enqueues nothing; mita_last_error() then describes it.
 *     No C++ exception crosses this interface.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef MITA_H
#define MITA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MITA_OK = 0,
  MITA_ERR_INVALID_ARG = -1, /* a size, pointer or shape field is out of range   */
  MITA_ERR_UNSUPPORTED = -2, /* valid request this build does not implement      */
  MITA_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small      */
  MITA_ERR_HIP = -4          /* a HIP runtime call failed; see mita_last_error() */
} mita_status;

typedef enum { MITA_F32 = 0, MITA_BF16 = 1 } mita_dtype;

/* Problem shape. Tokens lie on a row-major grid_h x grid_w grid (grid_h = 1 for a
 * 1D sequence) and are pooled separably to a row-major pool_h x pool_w grid of
 * landmarks, so m = pool_h * pool_w. Pooling window i of an axis of length L
 * pooled to M cells is [floor(i L / M), ceil((i + 1) L / M)).
 * Supported: d in {64, 128}; 1 <= pool_h <= grid_h; 1 <= pool_w <= grid_w;
 * grid_h * grid_w = N; m <= 4096; B * H * N * max(d, s) < 2^31. */
typedef struct {
  int32_t B, H, N, d;
  int32_t grid_h, grid_w;
  int32_t pool_h, pool_w;
  int32_t dtype; /* mita_dtype */
} mita_shape;

/* Bytes of device workspace that mita_forward and the step entry points need for
 * this shape and (m, k, s); 0 if the arguments are invalid. The workspace holds
 * every intermediate (landmarks, score-group maxima, top-k candidates, expert
 * sets, routing, buckets and partial outputs) and must be 256-byte aligned. */
size_t mita_workspace_bytes(const mita_shape* shape, int m, int k, int s);

/* Whole forward pass, steps 1-5: out = MiTA(Q, K, V) with m landmarks, experts of
 * k tokens and s routed experts per query. Requires 1 <= m <= N, 1 <= k <= N,
 * 1 <= s <= m. `out` has the input dtype ([B, H, N, d]); bf16 results are
 * rounded to nearest even. Equivalent to calling mita_pool, mita_landmark,
 * mita_topk, mita_route, mita_gather and mita_combine in that order on the same
 * workspace, except that routing (step 4, which needs only step 1) runs concurrently with
 * steps 2 and 3 on a side stream: per device the library keeps one stream
 * (default priority) and two events, created on the first call, and joins the
 * side stream back into `stream` before step 5 (so the call stays ordered on
 * `stream`, and may be captured into a graph). No device memory is allocated. */
mita_status mita_forward(const void* Q, const void* K, const void* V, int m, int k, int s, void* out,
                         const mita_shape* shape, void* workspace, size_t workspace_bytes, void* stream);

/* Step entry points, for per-step checks and timing. They run the steps of
 * mita_forward one at a time: each reads what the earlier steps left in the
 * workspace, so they must be called in this order (pool, landmark, topk, route,
 * gather, combine) with the same shape, (m, k, s) and workspace. Each may also
 * copy its result out for inspection; every `*_out` pointer may be NULL. */

/* Step 1 (pooling). Qt_out: fp64 [B, H, m, d], the landmark queries. */
mita_status mita_pool(const void* Q, int m, int k, int s, const mita_shape* shape, void* workspace,
                      size_t workspace_bytes, double* Qt_out, void* stream);

/* Step 2 (shared expert). Vt_out: fp32 [B, H, m, d], the shared expert V~
 * (copied from the workspace). The m x N score rows q~_i . K_n are not kept; the
 * step leaves maxima of groups of them and, derived from those, each row's
 * candidate threshold for step 3. S_out, when not NULL, is a
 * device buffer (fp32 [B, H, m, N], 16-byte aligned) that the kernel fills with
 * the unscaled scores as computed on the GPU (fp32 accumulation), for checking. */
mita_status mita_landmark(const void* K, const void* V, int m, int k, int s, const mita_shape* shape,
                          void* workspace, size_t workspace_bytes, float* Vt_out, float* S_out, void* stream);

/* Step 3 (deformable experts). I_out: int32 [B, H, m, k], each row the k token
 * ids of expert i in ascending order. Selection is exact: the scores are
 * recomputed and only those above a per-row threshold (set from the group
 * maxima of step 2, minus the error bound) are kept as candidates; candidates
 * whose fp32 score lies within a proven error bound of the k-th largest are
 * re-scored in fp64 before the cut. Rows with too many candidates (massive
 * ties) are selected from fp64 scores of the whole row. */
mita_status mita_topk(const void* K, int m, int k, int s, const mita_shape* shape, void* workspace,
                      size_t workspace_bytes, int32_t* I_out, void* stream);

/* Step 4 (routing). E_out: int32 [B, H, N, s], the routed landmarks of each
 * query. The set is exact in the same sense as step 3; the order among a
 * query's s entries is not specified (it does not change the output). Also
 * groups the (query, expert) pairs by expert (a counting sort) for step 5. */
mita_status mita_route(const void* Q, int m, int k, int s, const mita_shape* shape, void* workspace,
                       size_t workspace_bytes, int32_t* E_out, void* stream);

/* Step 5, routed part (output: Dutch "Wiskundige Formulering", the keys and
 * values of the experts a query is routed to): attention of each expert's bucket
 * of queries over the expert's k gathered key/value rows. With s = 1 and
 * m <= 64 the same kernel also attends the m shared-expert pairs and writes
 * `out` (mita_combine then does nothing); otherwise it leaves one partial
 * softmax per (query, slot) in the workspace and `out` is written by
 * mita_combine. */
mita_status mita_gather(const void* Q, const void* K, const void* V, int m, int k, int s, void* out,
                        const mita_shape* shape, void* workspace, size_t workspace_bytes, void* stream);

/* Step 5, shared-expert part and merge: attention of every query over the m
 * pairs (Q~, V~), merged with the s partial softmaxes mita_gather left, into
 * `out` ([B, H, N, d], input dtype). Call after mita_gather with the same
 * arguments; enqueues nothing when mita_gather already wrote `out`. */
mita_status mita_combine(const void* Q, int m, int k, int s, void* out, const mita_shape* shape, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Backward of the forward pass (bf16 inputs only): dQ, dK, dV (fp32 [B, H, N, d],
 * owned by the caller) of sum(dout * out), with the expert sets I and the
 * routing E held fixed (they are selections, not differentiable). The pages
 * report training through MiTA (Long Range Arena training wall-clock: Arabic/
 * Hindi section 4, Dutch "Resultaten") but give no backward; this is the chain
 * rule through the forward as defined: the final attention over
 * [Q~, K_{I_e1}, ..] / [V~, V_{I_e1}, ..] (a token in two of a query's experts
 * receives both contributions), the shared expert V~ = softmax(Q~ K^T / sqrt d) V,
 * and the pooling Q -> Q~.
 * Reads what mita_forward (or the step entry points through mita_combine) left
 * in `workspace` for the same Q, K, V, shape and (m, k, s): landmarks, V~, the
 * expert sets, the routing buckets and the softmax normalisers. `out` is that
 * forward's output and `dout` the gradient of the loss with respect to it, both
 * bf16 [B, H, N, d]. The forward workspace is not modified. `bwd_workspace`
 * (256-byte aligned, mita_backward_workspace_bytes bytes) holds the partial
 * gradients. Sums run in a fixed order (no float atomics): two calls on the same
 * inputs give bit-identical gradients. Errors as for mita_forward; fp32 inputs
 * give MITA_ERR_UNSUPPORTED. */
size_t mita_backward_workspace_bytes(const mita_shape* shape, int m, int k, int s);
mita_status mita_backward(const void* Q, const void* K, const void* V, const void* out, const void* dout, int m,
                          int k, int s, float* dQ, float* dK, float* dV, const mita_shape* shape,
                          const void* workspace, size_t workspace_bytes, void* bwd_workspace,
                          size_t bwd_workspace_bytes, void* stream);

/* Full softmax attention, out = softmax(Q K^T / sqrt d) V over all N keys of each
 * (batch, head) slice: the quadratic standard attention that MiTA replaces
 * (MiTA pages: introduction and problem statement; the pages' speed-ups are
 * quoted against it). Not part of the MiTA forward: a comparator on the same
 * inputs. Q, K, V, out: [B, H, N, d] in shape->dtype, contiguous, 16-byte
 * aligned device buffers owned by the caller; bf16 results are rounded to
 * nearest even. Only B, H, N, d and dtype of `shape` are read (d in {64, 128},
 * B * H * N * d < 2^31). Needs no workspace and allocates nothing; runs on
 * `stream`. Errors: MITA_ERR_INVALID_ARG for a NULL or misaligned pointer or a
 * bad size or dtype, MITA_ERR_UNSUPPORTED for another d, MITA_ERR_HIP if the
 * launch fails. */
mita_status mita_dense_attention(const void* Q, const void* K, const void* V, void* out, const mita_shape* shape,
                                 void* stream);

/* Size of the fixed scratch array behind mita_forward_noalloc (64 MiB per GPU). */
#define MITA_NOALLOC_SCRATCH_BYTES 67108864u

/* Whole forward pass like mita_forward, for callers that cannot allocate device
 * memory or hand over a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. The caller still passes Q, K, V and
 * `out` (same layout, dtype and checks as mita_forward); the intermediates live
 * in a fixed array of MITA_NOALLOC_SCRATCH_BYTES in the library's device code,
 * one per GPU, which each GPU the library runs on holds until the process ends.
 * Nothing is allocated and no stream or event is created: every step runs in
 * order on `stream`. Results are bit-identical to mita_forward's.
 * Limit: problems whose intermediates need more than the array (the same sizes as
 * mita_workspace_bytes, except that the exact top-k fallback keeps only its
 * fewest 64 score rows) are rejected with MITA_ERR_WORKSPACE before anything is
 * enqueued; small problems fit, e.g. B = H = 1, N = 1024, d = 64 with m = 16,
 * k = 64 takes under 2 MiB.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams or host threads, or a graph replay beside an
 * eager call) race and give wrong results; calls kept in order on one stream are
 * safe. Each call sets every part of the array it reads, so what an earlier call
 * left there does not matter. */
mita_status mita_forward_noalloc(const void* Q, const void* K, const void* V, int m, int k, int s, void* out,
                                 const mita_shape* shape, void* stream);

/* Short description of a status code (static storage). */
const char* mita_status_string(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* mita_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MITA_H */
