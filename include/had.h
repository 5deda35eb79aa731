/*
 * had.h - C ABI of the HAD (Hamming Attention Distillation) inference
 * attention library for AMD Instinct MI355X (gfx950).
 *
 * The method (Pith review of "Hamming Attention Distillation: Binarizing Keys
 * and Queries for Efficient Long-Context Transformers", section "What carries
 * the argument"): queries and keys are standardized by sigma_Q / sigma_K and
 * sign-binarized to {-1,+1}; the logits QK^T become +-1 dot products computed
 * as d - 2*popcount(q XOR k); a top-N mask keeps the largest logits of every
 * query row; softmax and the value accumulation run over that sparse set with
 * full-precision V.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major, contiguous [B, H, n, d] ("had_shape").
 *  - Every data pointer is a *device* pointer owned by the caller; the library
 *    never frees, keeps or allocates caller memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it and the call returns without synchronizing.
 *  - Host-side argument checks run first and synchronously; a failed check
 *    returns a status and enqueues nothing.  Launch failures return
 *    HAD_ERR_HIP.  No C++ exception crosses this interface.
 *  - had_last_error() returns a thread-local text for the last failure.
 *  - Results are deterministic: identical inputs give bit-identical outputs
 *    (no floating-point atomics anywhere).
 */
#ifndef HAD_H
#define HAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HAD_OK = 0,
  HAD_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad value */
  HAD_ERR_UNSUPPORTED = 2, /* valid request outside the library's limits */
  HAD_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} had_status;

typedef enum { HAD_F32 = 0, HAD_BF16 = 1 } had_dtype;

/* Device status word bits written by had_pack (see below). */
#define HAD_DEV_NAN_INPUT 1u

/* Limits: 1 <= d <= HAD_MAX_DIM; 1 <= n <= HAD_MAX_SEQ for the attention
   calls (had_pack accepts n up to HAD_MAX_DECODE_KEYS, to pack key caches). */
#define HAD_MAX_DIM 256
#define HAD_MAX_SEQ 65536

typedef struct {
  int64_t batch; /* B */
  int64_t heads; /* H */
  int64_t seq;   /* n: tokens per (batch, head) */
  int64_t dim;   /* d: features per token */
} had_shape;

/* Decoding against a key/value cache (had_decode). */
#define HAD_MAX_DECODE_Q 65536         /* new query rows per (batch, head) */
#define HAD_MAX_DECODE_KEYS (1 << 22)  /* rows of the cache (k_stride) */

typedef struct {
  int64_t batch;    /* B */
  int64_t heads;    /* H */
  int64_t n_q;      /* new query rows per (batch, head) */
  int64_t n_k;      /* valid rows of the key/value cache */
  int64_t k_stride; /* allocated rows of the cache per (batch, head), >= n_k */
  int64_t dim;      /* d */
} had_decode_shape;

/* Number of uint32 words holding the d sign bits of one row: ceil(d / 32). */
int64_t had_words_per_row(int64_t dim);

/* Workspace bytes that had_pack needs when it computes sigma. */
size_t had_pack_workspace_bytes(had_shape s);

/*
 * had_pack - standardize, sign-binarize and bit-pack Q or K.
 *
 * Defined by: Pith review, "What carries the argument" (standardization with
 * data-estimated sigma_Q, sigma_K, then sign quantization to {-1,+1}) and
 * referee minor comment 6 on Eq. 12 (sigma is the standard deviation over all
 * elements of the matrix).
 *
 *  x          [B,H,n,d] float32, device, 4-byte aligned (16-byte alignment
 *             takes the faster vector path).  Read once.
 *  xbits      [B,H,n,W] uint32, device, W = had_words_per_row(d).  Bit
 *             (c mod 32) of word floor(c/32) of a row is 1 exactly when
 *             x[c] < 0 (so +0.0 and -0.0 give 0, i.e. +1); unused high bits
 *             of the last word are 0.  Since sigma > 0 the bits of x/sigma
 *             equal the bits of x, so they never depend on a reduction.
 *  sigma      device float*, or NULL.  When non-NULL it receives the
 *             population standard deviation of all B*H*n*d elements
 *             (float64 accumulation, deterministic order, rounded to float).
 *  workspace  device memory of had_pack_workspace_bytes(s) bytes, 16-byte
 *             aligned, required when sigma != NULL (ignored otherwise).  It
 *             holds per-block partial sums; no initial contents are needed.
 *             Calls that may run at the same time need distinct workspaces.
 *  dev_status device uint32*, or NULL.  When non-NULL, HAD_DEV_NAN_INPUT is
 *             OR-ed into it if x holds a NaN (the bit value of a NaN element
 *             is then unspecified).  The library never clears it.
 *  Errors: HAD_ERR_INVALID_ARG for a null x/xbits, a non-positive shape
 *  field, or a missing/small workspace; HAD_ERR_UNSUPPORTED above the limits.
 */
had_status had_pack(const float* x, had_shape s, uint32_t* xbits, float* sigma,
                    void* workspace, size_t workspace_bytes,
                    uint32_t* dev_status, void* stream);

/*
 * Running sigma calibration (the per-layer estimate over many calibration
 * minibatches described for Eq. 12: Pith review, referee minor comment 6 and
 * "Assumptions & free parameters").  A had_sigma_state lives in device
 * memory; set it to zero (e.g. hipMemsetAsync) to start a calibration.
 * Each call merges its elements with the parallel-variance update, so the
 * state never differences large sums of squares.
 */
typedef struct {
  double count; /* elements seen */
  double mean;  /* their mean */
  double m2;    /* sum of squared deviations from the mean */
  double reserved;
} had_sigma_state;

/*
 * had_pack_calibrate - had_pack without a per-call sigma: packs x into xbits
 * and merges the element count, mean and squared deviations of x into *state
 * (device, 8-byte aligned).  Calls on one stream merge in stream order, so
 * the state is the same on every run.  workspace: had_pack_workspace_bytes(s) bytes,
 * 16-byte aligned.  Calls that may overlap need distinct workspaces and must
 * not share a state.
 */
had_status had_pack_calibrate(const float* x, had_shape s, uint32_t* xbits,
                              had_sigma_state* state, void* workspace,
                              size_t workspace_bytes, uint32_t* dev_status,
                              void* stream);

/* had_sigma_from_state - *sigma = population standard deviation of every
 * element added to *state so far (0 for an empty state), one device float. */
had_status had_sigma_from_state(const had_sigma_state* state, float* sigma, void* stream);

/*
 * had_attention - Hamming logits, top-N selection, softmax over the kept set
 * and value accumulation, fused; the n x n matrix is never written.
 *
 * Defined by: Pith review, "What carries the argument" (XNOR-plus-popcount
 * logits, top-N mask of the largest logits per row, softmax and value
 * accumulation on the sparse matrix) and referee major comment 3 (values in
 * full precision); Pith verdict record, "one_line_summary".
 *
 *  qbits, kbits  [B,H,n,W] uint32 sign words as written by had_pack.
 *  v             [B,H,n,d] values, device, float32 (v_dtype HAD_F32) or
 *                bfloat16 (HAD_BF16).  16-byte aligned.
 *  topn          N >= 1.  Row i keeps N_i = min(N, visible_i) keys.
 *  scale         finite and > 0.  The float logit is scale * s where s is
 *                the integer +-1 dot product; fold sigma_Q*sigma_K or
 *                1/sqrt(d) into it as wanted.
 *  causal        0: row i sees every key.  1: row i sees keys j <= i; the mask
 *                is applied before selection.
 *  out           [B,H,n,d] float32, device, 16-byte aligned.
 *
 *  Row i keeps S_i = {j visible : s_ij > t_i} plus the lowest-index keys with
 *  s_ij == t_i, where t_i is the N_i-th largest visible logit, so that
 *  |S_i| = N_i exactly; out_i = sum_{j in S_i} softmax_{S_i}(scale*s_ij) V_j.
 *  Precision: logits and selection are exact integers; the softmax weights
 *  are computed in float32 and applied with float32 accumulation (bf16 V:
 *  weights split into two bf16 terms, relative weight error below 2^-15).
 *  Errors: HAD_ERR_INVALID_ARG for null or misaligned pointers, non-positive
 *  sizes, topn < 1, non-finite or non-positive scale, unknown v_dtype;
 *  HAD_ERR_UNSUPPORTED above the limits.
 */
had_status had_attention(const uint32_t* qbits, const uint32_t* kbits,
                         const void* v, had_dtype v_dtype, had_shape s,
                         int64_t topn, float scale, int causal, float* out,
                         void* stream);

/* Workspace bytes that had_forward needs when it computes sigma. */
size_t had_forward_workspace_bytes(had_shape s);

/*
 * had_forward - the whole inference path in two kernel launches: the pack of
 * Q and of K in one launch, then the attention launch, which also finalizes
 * sigma_Q and sigma_K.  Every output equals that of had_pack(q),
 * had_pack(k) and had_attention(qbits, kbits, ...) called one after the other
 * with the same arguments (bits, sigma and out bit for bit).
 *
 * Defined by: the passages cited for had_pack and had_attention (Pith review,
 * "What carries the argument"; referee minor comment 6 on Eq. 12 and major
 * comment 3).
 *
 *  q, k        [B,H,n,d] float32, device, 4-byte aligned.  Read once each.
 *  qbits,kbits [B,H,n,W] uint32, device: receive the sign words (as had_pack)
 *              and are read by the attention launch.
 *  v, v_dtype, topn, scale, causal, out: as had_attention.
 *  sigma_q, sigma_k  device float*, or NULL each (as had_pack's sigma).
 *  workspace   device memory of had_forward_workspace_bytes(s) bytes, 16-byte
 *              aligned, required when a sigma is requested.  No initial
 *              contents needed; calls that may overlap need distinct ones.
 *  dev_status  as had_pack, for a NaN in q or k.
 *  Errors: those of had_pack and had_attention; nothing is enqueued then.
 */
had_status had_forward(const float* q, const float* k, const void* v,
                       had_dtype v_dtype, had_shape s, int64_t topn,
                       float scale, int causal, uint32_t* qbits,
                       uint32_t* kbits, float* out, float* sigma_q,
                       float* sigma_k, void* workspace,
                       size_t workspace_bytes, uint32_t* dev_status,
                       void* stream);

/*
 * had_forward_noalloc - had_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same two launches and the same results bit for bit,
 * with the sigma partials in a fixed device array inside the library instead
 * of a caller workspace.  The call allocates nothing; the caller still owns
 * q, k, v, qbits, kbits, out, sigma_q, sigma_k and dev_status (meanings as
 * had_forward).
 *
 *  Scratch: HAD_FORWARD_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the
 *  first call on that GPU until the process ends.  Shapes whose
 *  had_forward_workspace_bytes() exceeds it are rejected with
 *  HAD_ERR_UNSUPPORTED (the partials are capped at 256 pairs per tensor, so
 *  no valid shape needs more).  The array keeps the last call's contents and
 *  needs no initial contents.  All calls on one GPU share it: two calls that
 *  may overlap on the same GPU (different streams, or threads without
 *  ordering) race and may produce a wrong sigma.
 *  Errors: those of had_forward, and HAD_ERR_HIP if the array's device
 *  address cannot be looked up.
 */
#define HAD_FORWARD_NOALLOC_SCRATCH_BYTES 8192
had_status had_forward_noalloc(const float* q, const float* k, const void* v,
                               had_dtype v_dtype, had_shape s, int64_t topn,
                               float scale, int causal, uint32_t* qbits,
                               uint32_t* kbits, float* out, float* sigma_q,
                               float* sigma_k, uint32_t* dev_status,
                               void* stream);

/* Workspace bytes that had_backward needs for shape s (0 for an invalid
 * shape or d > 128). */
size_t had_backward_workspace_bytes(had_shape s);

/*
 * had_backward - the straight-through backward of had_attention, for the
 * training stages that finish the binarization with a straight-through
 * estimator.
 *
 * Defined by: Pith review, "What carries the argument" (a four-stage
 * annealing schedule: a scaled tanh approaching sign, then a straight-through
 * estimator finishing the binarization); the forward pass is had_attention's
 * path.  Readings: sign's derivative is taken as 1 on the standardized input
 * x / sigma (the plain straight-through estimator) with sigma a calibrated
 * constant, and the top-N selection, a discrete choice, is held fixed.  For
 * row i with kept set K_i (exactly had_attention's) and p_ij its softmax
 * weights:
 *   dP_ij = dout_i . V_j,  D_i = dout_i . out_i,
 *   dS_ij = scale * p_ij * (dP_ij - D_i) for j in K_i (0 elsewhere),
 *   dv_j  = sum_i p_ij dout_i,
 *   dq_i  = (sum_j dS_ij Bk_j) / sigma_q,  dk_j = (sum_i dS_ij Bq_i) / sigma_k,
 * with Bq, Bk the +-1 rows the sign words encode.
 *
 *  qbits, kbits, v, v_dtype, topn, scale, causal: as had_attention (the
 *               same values as the forward call).  d <= 128.
 *  out          [B,H,n,d] float32: had_attention's output for these inputs.
 *  dout         [B,H,n,d] float32: the gradient of the loss at out.
 *  sigma_q, sigma_k  device float* (had_pack's sigma), or NULL for 1
 *               (gradients with respect to the standardized inputs).
 *  dq, dk, dv   [B,H,n,d] float32 outputs, device; every element written.
 *  workspace    had_backward_workspace_bytes(s) bytes, 256-byte aligned (per
 *               row statistics; no initial contents needed).  Calls that may
 *               overlap need distinct workspaces.
 *  All pointers 4-byte aligned.  Precision: integer logits and selection;
 *  float32 weights, products and sums (no floating-point atomics: results are
 *  identical run to run).
 *  Errors: HAD_ERR_INVALID_ARG for null or misaligned pointers, bad sizes,
 *  topn < 1, bad scale, causal or v_dtype, a small workspace;
 *  HAD_ERR_UNSUPPORTED for d > 128 or n above HAD_MAX_SEQ.
 */
had_status had_backward(const uint32_t* qbits, const uint32_t* kbits,
                        const void* v, had_dtype v_dtype, had_shape s,
                        int64_t topn, float scale, int causal,
                        const float* out, const float* dout,
                        const float* sigma_q, const float* sigma_k,
                        float* dq, float* dk, float* dv, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Limit of the soft (scaled-tanh) forward: the logit block of 32 query rows
   and every key stays in registers. */
#define HAD_SOFT_MAX_SEQ 1024

/* Workspace bytes that had_soft_forward / had_soft_select need for shape s
 * (0 for an invalid shape, d > 128 or n > HAD_SOFT_MAX_SEQ). */
size_t had_soft_workspace_bytes(had_shape s);

/*
 * had_soft_forward - the attention path with the sign replaced by a scaled
 * tanh, for the training stages that approach the binarization smoothly.
 *
 * Defined by: Pith review, "What carries the argument" (a four-stage
 * annealing schedule whose first stages use a scaled tanh with a decaying
 * scale c that approaches the sign function); referee minor comment 1 (the
 * stage's Eqs. 13/15 are printed twice and never settled).  Reading: the soft
 * sign is B_c(x) = tanh(x / (sigma * c)), c > 0 (c -> 0 gives the sign path);
 * the logits are the real dot products s_ij = B_c(q_i) . B_c(k_j); row i keeps
 * its N_i = min(N, visible_i) largest logits (lower key index first among
 * equal float32 logits, causal mask first); out_i = softmax over the kept set
 * of scale * s_ij, times V.
 *
 *  q, k       [B,H,n,d] float32, device, 4-byte aligned.  n <= 1024, d <= 128.
 *             NaN inputs are outside the contract: the kept sets and outputs
 *             are then unspecified (every access stays in bounds).
 *  v, v_dtype as had_attention (float32 or bf16, 4-byte aligned).
 *  topn, scale, causal  as had_attention.
 *  c          the tanh scale, finite and > 0.
 *  sigma_q, sigma_k  device float* (had_pack's or had_sigma_from_state's
 *             sigma), or NULL for 1.  1 / (sigma * c) is taken as at most
 *             FLT_MAX (a sigma of 0 gives the sign, and 0 for x = 0).
 *  out        [B,H,n,d] float32, device; every element written.
 *  workspace  had_soft_workspace_bytes(s) bytes, 256-byte aligned (the soft
 *             key rows; no initial contents needed).  Calls that may overlap need
 *             distinct workspaces.
 *  Precision: float32 tanh, logits on the fp32 matrix cores, the kept set the
 *  exact top-N of those float32 logits, float32 weights, products and sums
 *  (no floating-point atomics: results are identical run to run).
 *  Errors: HAD_ERR_INVALID_ARG for null or misaligned pointers, bad sizes,
 *  topn < 1, bad scale, c, causal or v_dtype, a small workspace;
 *  HAD_ERR_UNSUPPORTED for d > 128 or n > HAD_SOFT_MAX_SEQ.
 */
had_status had_soft_forward(const float* q, const float* k, const void* v,
                            had_dtype v_dtype, had_shape s, int64_t topn,
                            float scale, float c, int causal,
                            const float* sigma_q, const float* sigma_k,
                            float* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * had_soft_select - inspection export of the kept sets of had_soft_forward
 * (same kernel code, same selection).
 *
 * Defined by: as had_soft_forward; the top-N rule of "What carries the
 * argument".
 *
 *  Arguments as had_soft_forward; slices bh in [bh_begin, bh_begin +
 *  bh_count) of the B*H slices, all n query rows.
 *  keep  [bh_count, n, n] uint8, device: 1 where row i keeps key j, else 0
 *        (cleared by the call).
 */
had_status had_soft_select(const float* q, const float* k, had_shape s,
                           int64_t topn, float c, int causal,
                           const float* sigma_q, const float* sigma_k,
                           int64_t bh_begin, int64_t bh_count, uint8_t* keep,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * had_logits - inspection export of the integer logits s = d - 2*Hamming
 * computed by the same logit stage as had_attention (no mask, every key).
 *
 * Defined by: Pith review, "What carries the argument" (QK^T by XNOR plus
 * popcount) and referee major comment 1 (the logits are integers).
 *
 *  Slices bh in [bh_begin, bh_begin + bh_count) of the B*H (batch, head)
 *  slices, query rows [row_begin, row_begin + row_count).
 *  s_out  [bh_count, row_count, n] int16, device.
 */
had_status had_logits(const uint32_t* qbits, const uint32_t* kbits, had_shape s,
                      int64_t bh_begin, int64_t bh_count, int64_t row_begin,
                      int64_t row_count, int16_t* s_out, void* stream);

/*
 * had_select - inspection export of the top-N sets chosen by had_attention's
 * selection stage (same kernel code, same tie rule).
 *
 * Defined by: Pith review, "What carries the argument" (top-N mask keeps only
 * the largest logits per row); lower key index wins among equal logits.
 *
 *  Slices bh in [bh_begin, bh_begin + bh_count), all n query rows.
 *  idx  [bh_count, n, topn] int32, device: row i holds its N_i kept key
 *       indices in ascending order, then -1 in the remaining topn - N_i slots.
 */
had_status had_select(const uint32_t* qbits, const uint32_t* kbits, had_shape s,
                      int64_t topn, int causal, int64_t bh_begin,
                      int64_t bh_count, int32_t* idx, void* stream);

/*
 * had_topn_mass - measurement: for every query row, the smallest N whose N
 * largest softmax weights (of scale * s over the visible keys) sum to at least
 * mass, from the same histogram stage as had_attention.
 *
 * Defined by: Pith verdict record, "concrete_test" (the fraction of softmax
 * mass captured by the top-N logits as n grows) and the Pith review's
 * Figure 4 (attention mass versus N); the top-N rule of "What carries the
 * argument".
 *
 *  Slices bh in [bh_begin, bh_begin + bh_count), all n rows; causal as
 *  had_attention.  mass in (0, 1]; mass >= 1 gives the visible count.
 *  n_out  [bh_count, n] int32, device.
 *  Precision: the weights exp(-2*scale*(h - h_min)) and their sums in float64;
 *  keys of one logit value share one weight, so N is exact up to that
 *  rounding.
 */
had_status had_topn_mass(const uint32_t* qbits, const uint32_t* kbits, had_shape s,
                         float scale, int causal, double mass, int64_t bh_begin,
                         int64_t bh_count, int32_t* n_out, void* stream);

/* Workspace bytes that had_decode needs for shape s. */
size_t had_decode_workspace_bytes(had_decode_shape s);

/*
 * had_decode - the attention of n_q new query rows against a cache of n_k
 * packed keys and their values: the decoding step of long-context inference.
 *
 * Defined by: the passages cited for had_attention (Pith review, "What
 * carries the argument"; referee major comment 3), with the query rows at
 * positions q_pos0 .. q_pos0 + n_q - 1 of the sequence whose first n_k rows
 * the cache holds.
 *
 *  qbits  [B,H,n_q,W] uint32 sign words of the new rows (had_pack output).
 *  kbits  [B,H,k_stride,W] uint32 sign words of the cache; rows >= n_k unused.
 *         4-byte aligned (with W even, 8- or 16-byte alignment lets key rows
 *         load as vectors).
 *  v      [B,H,k_stride,d] float32 (HAD_F32) or bfloat16 (HAD_BF16) values;
 *         rows >= n_k unused.  4-byte aligned.
 *  q_pos0 position of the first new row (>= 0).  causal = 1: row i sees the
 *         keys j <= q_pos0 + i (and j < n_k); causal = 0: every key.  With
 *         n_q = n_k and q_pos0 = 0 the call computes had_attention's outputs
 *         for the whole sequence by gathering only the kept V rows.
 *  topn, scale: as had_attention; row i keeps N_i = min(N, visible_i) keys,
 *         lower key index first among equal logits.
 *  out    [B,H,n_q,d] float32.
 *  workspace  device memory of had_decode_workspace_bytes(s) bytes, 256-byte
 *         aligned; no initial contents needed; calls that may overlap need
 *         distinct ones.
 *  Precision: exact integer logits and selection; weights exp(-2*scale*(h -
 *  h_min)) and sums in float32.  Only the kept V rows are read.
 *  Errors: HAD_ERR_INVALID_ARG for null or misaligned pointers, bad sizes,
 *  k_stride < n_k, q_pos0 < 0, topn < 1, bad scale, causal or v_dtype, a
 *  small workspace; HAD_ERR_UNSUPPORTED above the limits.
 */
had_status had_decode(const uint32_t* qbits, const uint32_t* kbits,
                      const void* v, had_dtype v_dtype, had_decode_shape s,
                      int64_t q_pos0, int64_t topn, float scale, int causal,
                      float* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * had_decode_forward - had_decode with the new rows given as float32: the
 * step "sign-binarize the new queries, then attend against the cache" in the
 * launches of had_decode (the first launch builds the rows' sign words).
 *
 * Defined by: the passages cited for had_pack (the sign of a standardized
 * row; no sigma is formed, since dividing by it changes no sign) and for
 * had_decode.
 *
 *  q      [B,H,n_q,d] float32 new rows, contiguous, 4-byte aligned.  Bit c of
 *         word w of a row is [q_{32w+c} < 0], pad bits 0: exactly the words
 *         had_pack writes, so the result equals had_pack followed by
 *         had_decode, bit for bit.  A NaN element gives a 0 bit and is not
 *         reported (call had_pack to have NaN input flagged).
 *  Every other argument, the workspace (the same had_decode_workspace_bytes;
 *  it also holds the rows' words), the precision and the errors are those of
 *  had_decode.
 */
had_status had_decode_forward(const float* q, const uint32_t* kbits,
                              const void* v, had_dtype v_dtype,
                              had_decode_shape s, int64_t q_pos0,
                              int64_t topn, float scale, int causal,
                              float* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* had_status_string(had_status st);

/* Thread-local description of the last failure on the calling thread. */
const char* had_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HAD_H */
