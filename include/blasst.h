/*
 * blasst.h - C ABI of the BLASST block-sparse attention library for AMD MI355X (gfx950).
 *
 * The method (pages about "BLASST: Dynamic BLocked Attention Sparsity via Softmax Thresholding",
 * arXiv 2512.12087):
 *   - attention is computed FlashAttention-style, visiting the KV blocks of a query tile left to
 *     right with an online softmax (running max m, running sum l, rescaled output)
 *     [xllm-io review, sections 解决方案概述 and 整体框架图];
 *   - block j is skipped when every row i of the query tile has m~_i - m_i < ln(lambda), where m~
 *     is the block-local row max and m the running max [xllm-io review, 核心公式 skip condition;
 *     gist.science (de), 2. Methodik / Kernidee];
 *   - a skipped block contributes nothing: its exp, its V load and its P.V product are elided
 *     [gist.science (de), Kernidee; fugumt.com English abstract];
 *   - lambda = a / L with L the context length, and a calibration model
 *     lambda * L = alpha * exp(beta * s) for a target sparsity s [xllm-io review, 核心公式
 *     threshold calibration and calibration model];
 *   - prefill keeps QK^T for every block and elides exp and P.V; decode elides the V load and
 *     decides at the K-load stage with batched loads [xllm-io review, 预填充内核优化 and
 *     解码内核优化].
 *
 * Conventions for every entry point:
 *   - All device buffers are owned by the caller.  The library allocates no device memory and keeps
 *     no pointer after a call returns.  Scratch space (decode with num_splits > 1) is passed in as
 *     a caller-owned workspace whose size the *_workspace_size query returns.
 *   - Work is enqueued on the caller's HIP stream (hipStream_t passed as void*; NULL = the default
 *     stream) and the call returns before the work completes.
 *   - Every argument check runs before the first HIP call, so invalid arguments are reported
 *     without touching the device.  Errors are returned as a status code; a message for the last
 *     error of the calling thread is available from blasst_last_error().  Nothing aborts or throws.
 *   - Numerics: bf16 or fp32 inputs, fp32 accumulation, natural-log units for lambda and for the
 *     critical values.  lambda must lie in [0, 1]; lambda = 0 (ln lambda = -inf) is dense.
 *   - Skip-mask bytes: 0 = kept, 1 = skipped, 2 = not live (no visible key for the whole tile).
 *   - Critical value of a live tile-block: max over the tile's rows of (m~_i - m_i) in logit units
 *     (softmax scale applied), with m the running max BEFORE the block (+inf for the first block of
 *     a split).  The block is skipped iff crit < ln(lambda).  NaN for blocks that are not live.
 */
#ifndef BLASST_H
#define BLASST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BLASST_OK = 0,
  BLASST_ERR_INVALID_ARG = 1,   /* a pointer, size, stride or threshold is invalid */
  BLASST_ERR_UNSUPPORTED = 2,   /* valid request, but no kernel for this head dim / block / dtype, or a
                                   problem whose workgroup count, context length or skip-mask size
                                   does not fit the kernels' 32-bit indexing */
  BLASST_ERR_HIP = 3,           /* a HIP call or kernel launch failed */
  BLASST_ERR_WORKSPACE = 4      /* workspace missing or smaller than *_workspace_size() */
} blasst_status;

typedef enum { BLASST_BF16 = 0, BLASST_FP32 = 1 } blasst_dtype;

typedef enum {
  BLASST_THR_LAMBDA = 0,   /* use `lambda` directly, must be in [0, 1] */
  BLASST_THR_A_OVER_L = 1, /* lambda = min(1, a / L), L = seqlen_k (prefill) or seq_lens[b] (decode) */
  BLASST_THR_NONE = 2      /* no threshold: every live block is kept (the result of lambda = 0), and
                              the bf16 prefill kernel for head dim 128, 128 x 128 blocks and an even
                              GQA group, and the GQA/MHA/MQA decode kernel, run without any decision
                              logic (no vote); used to measure the cost of the decisions.  skip_mask
                              and crit must be NULL and stats_only 0 (BLASST_ERR_INVALID_ARG
                              otherwise); counters count live blocks and no skipped ones.  lambda and
                              a are not read.  Other kernels (fp32 and paged prefill, latent decode)
                              run with lambda = 0. */
} blasst_threshold_mode;

typedef struct {
  int32_t mode;     /* blasst_threshold_mode */
  int32_t reserved; /* must be 0 */
  double lambda;    /* mode BLASST_THR_LAMBDA */
  double a;         /* mode BLASST_THR_A_OVER_L, a >= 0 */
} blasst_threshold;

/* V staging of the bf16 prefill (blasst_prefill_params.v_staging).  The result does not depend on
 * it: a skipped block never enters P.V.
 *   BLASST_V_KEPT (default): the V block of a key block is loaded only when a tile of the workgroup
 *     kept that block, so a skipped block costs neither V bytes nor V staging;
 *   BLASST_V_ALL: the V block of every live key block is loaded whether it is skipped or not, the
 *     pages' policy (xllm-io review, 预填充内核优化: the value block is still loaded from HBM so that
 *     prefetching stays regular), for measuring what skipping the V loads is worth.  Supported by
 *     the bf16 kernels; the fp32 kernel stages every V block anyway. */
typedef enum { BLASST_V_KEPT = 0, BLASST_V_ALL = 1 } blasst_v_staging;

/* Counter slots written (accumulated with atomics) when `counters` is not NULL; the caller zeroes
 * the buffer before the call if it wants per-call numbers. */
enum { BLASST_CNT_LIVE = 0, BLASST_CNT_SKIPPED = 1, BLASST_NUM_COUNTERS = 2 };

/*
 * Prefill: causal or full attention of seqlen_q queries over seqlen_k keys per (batch, q head).
 *
 * Layouts (element strides; the last dimension is contiguous):
 *   q [batch][num_q_heads][seqlen_q][head_dim_qk]    strides q_stride = {batch, head, token}
 *   k [batch][num_kv_heads][seqlen_k][head_dim_qk]   strides k_stride
 *   v [batch][num_kv_heads][seqlen_k][head_dim_v]    strides v_stride
 *   o [batch][num_q_heads][seqlen_q][head_dim_v]     strides o_stride, dtype out_dtype
 *   lse [batch][num_q_heads][seqlen_q] fp32 contiguous (natural log), nullable
 * Head mapping: q head h reads kv head h / (num_q_heads / num_kv_heads) (MHA, GQA, MQA).
 * Causal masking is bottom-right aligned: key k is visible to query row i iff
 *   k <= i + (seqlen_k - seqlen_q).
 * Query tile = block_q consecutive rows of one q head; KV block = block_k consecutive keys.
 * The live blocks of a tile are cut into num_splits contiguous chunks of ceil(J / num_splits)
 * blocks; the running max used by the skip rule restarts at -inf at every chunk, so the first block
 * of every chunk is kept.  The output is the softmax over the union of kept keys.
 * Diagnostics (nullable, device memory):
 *   skip_mask [batch][num_q_heads][ceil(seqlen_q/block_q)][ceil(seqlen_k/block_k)] uint8
 *   crit      same shape, fp32
 *   counters  BLASST_NUM_COUNTERS x uint64
 *   head_counters [batch][num_q_heads][BLASST_NUM_COUNTERS] uint64: the same counts per q head
 *             (accumulated with atomics like counters; the caller zeroes it), so that the sparsity
 *             one threshold gives each head can be read off directly (the pages' analysis of how
 *             sparsity varies across heads under a single threshold, "Sparsity distribution").
 * stats_only != 0: compute QK^T, block maxima, decisions, mask, crit and counters only; o and lse
 * are not written (calibration pass).
 * softmax_scale <= 0 selects 1/sqrt(head_dim_qk).
 * Supported kernels: bf16 in, bf16 or fp32 out, head_dim_qk == head_dim_v in {64, 128},
 * block_q == block_k in {64, 128}, k and v token strides in [head_dim, 2^22) elements (rows that do
 * not overlap); fp32 in/out, head_dim 64 or 128, block_q == block_k == 64.  All strides are
 * multiples of 16 bytes and the tensors 16-byte aligned (BLASST_ERR_UNSUPPORTED otherwise).
 */
typedef struct {
  size_t struct_size;        /* sizeof(blasst_prefill_params), for ABI checking */
  const void *q, *k, *v;
  void *o;
  float *lse;
  uint8_t *skip_mask;
  float *crit;
  unsigned long long *counters;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  blasst_threshold thr;
  int32_t in_dtype, out_dtype; /* blasst_dtype */
  int32_t batch, seqlen_q, seqlen_k, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v;
  int32_t causal, block_q, block_k, num_splits, stats_only;
  float softmax_scale;
  unsigned long long *head_counters; /* nullable, see above */
  int32_t v_staging;         /* blasst_v_staging: which V blocks the bf16 kernels stage in LDS */
} blasst_prefill_params;

/*
 * Chunked prefill against a paged KV cache: the seqlen_q query tokens of each sequence are its last
 * seqlen_q positions (their keys already written to the cache), and they attend to the sequence's
 * seq_lens[b] cached keys with the prefill's tiles, skip rule, splits and bottom-right causal mask:
 * query row i of sequence b sees keys k <= seq_lens[b] - seqlen_q + i.  The method serves prefill
 * and decode alike (xllm-io review, 核心思想 item 2); this is the prefill computation for a chunk
 * of a long prompt whose earlier keys sit in the same cache that decode reads.
 *
 * Layouts: q, o, lse, skip_mask, crit, counters as for blasst_prefill (seqlen_q rows, the mask's
 * key-block count is ceil(max_pages_per_seq * page_size / block_k)); k_cache, v_cache,
 * block_table and seq_lens as for blasst_decode (v_cache transposed inside each page).  A row that
 * sees no key (seq_lens[b] < seqlen_q) gets o = 0 and lse = -inf.  The threshold's L is seq_lens[b]
 * (per sequence, resolved on the device).
 * Supported: bf16 in, bf16 or fp32 out, head_dim_qk == head_dim_v == 128, block_q == block_k == 128,
 * page_size 16, causal only, seq_lens[b] >= 1, num_pages * num_kv_heads < 2^32 (a pool of at most
 * 16 TB per cache; larger values return BLASST_ERR_UNSUPPORTED).
 */
typedef struct {
  size_t struct_size;        /* sizeof(blasst_prefill_paged_params) */
  const void *q, *k_cache, *v_cache;
  const int32_t *block_table, *seq_lens;
  void *o;
  float *lse;
  uint8_t *skip_mask;
  float *crit;
  unsigned long long *counters;
  int64_t q_stride[3], o_stride[3];
  blasst_threshold thr;
  int32_t in_dtype, out_dtype;
  int32_t batch, seqlen_q, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v;
  int32_t page_size, max_pages_per_seq, num_pages;
  int32_t block_q, block_k, num_splits, stats_only;
  float softmax_scale;
} blasst_prefill_paged_params;

/*
 * Decode: the query tokens of each sequence attend to the keys of a paged KV cache, split along
 * the keys into num_splits chunks that run in parallel and are merged by a log-sum-exp combine.
 * With T = num_q_tokens (0 means 1) query tokens per sequence, they are the last T positions of
 * the sequence: token t sees keys k <= seq_lens[b] - T + t (bottom-right causal, as in prefill), so
 * T = 1 is ordinary decode and T > 1 serves a decode step that checks several tokens at once or a
 * chunk of prefill continued against the cache (the method serves both phases: xllm-io review,
 * 核心思想 item 2).  A token that sees no key (seq_lens[b] < T) gets o = 0 and lse = -inf.
 *
 * Layouts (contiguous):
 *   q           [batch][T][num_q_heads][head_dim_qk]
 *   k_cache     [num_pages][num_kv_heads][page_size][head_dim_qk]
 *   v_cache     [num_pages][num_kv_heads][head_dim_v][page_size]  (V transposed inside each page)
 *               NULL selects latent attention (MLA): V is the first head_dim_v channels of K.
 *   block_table [batch][max_pages_per_seq] int32 page ids; entries past a sequence's last page
 *               are never read
 *   seq_lens    [batch] int32, 0 <= seq_lens[b] <= max_pages_per_seq * page_size (an empty
 *               sequence reads no key: its rows get o = 0 and lse = -inf, its blocks are not live)
 *   o           [batch][T][num_q_heads][head_dim_v], dtype out_dtype
 *   lse         [batch][T][num_q_heads] fp32, nullable
 * Query tile = tile_rows q heads of one sequence that share a kv head (0 selects all
 * num_q_heads / num_kv_heads of them), for all T tokens: T * tile_rows rows, token-major, that
 * vote together; KV block = block_k keys (a multiple of page_size).
 * Diagnostics (nullable):
 *   skip_mask/crit [batch][num_kv_heads][G / tile_rows][ceil(max_pages_per_seq*page_size/block_k)]
 *   counters as for prefill.
 * workspace: needed when num_splits > 1, at least blasst_decode_workspace_size() bytes, device
 * memory, 256-byte aligned.
 * Supported kernels: bf16 in, bf16/fp32 out; page_size 16; block_k 64;
 *   GQA/MHA/MQA: head_dim_qk == head_dim_v == 128, T * tile_rows <= 16;
 *   latent (v_cache NULL): 128 q heads on 1 kv head, head_dim_qk == 576, head_dim_v == 512,
 *   T * tile_rows == 128 (128-row tiles: all heads of one token, or T = 2, 4 tokens x 64, 32 heads)
 *   or 64 (64-row tiles: T = 1, 2, 4 tokens x 64, 32, 16 heads).
 */
typedef struct {
  size_t struct_size;        /* sizeof(blasst_decode_params) */
  const void *q, *k_cache, *v_cache;
  const int32_t *block_table, *seq_lens;
  void *o;
  float *lse;
  uint8_t *skip_mask;
  float *crit;
  unsigned long long *counters;
  void *workspace;
  size_t workspace_bytes;
  blasst_threshold thr;
  int32_t in_dtype, out_dtype;
  int32_t batch, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v;
  int32_t page_size, max_pages_per_seq, num_pages;
  int32_t block_k, num_splits, tile_rows, stats_only;
  float softmax_scale;
  int32_t num_q_tokens;      /* T, query tokens per sequence; 0 or 1: one */
} blasst_decode_params;

/*
 * Prefill backward for sparsity-aware training: the gradients of the prefill forward with the
 * forward's skip decisions held fixed.  The pages' training extension runs the BLASST forward and
 * lets skipped blocks receive no gradient in the backward pass (xllm-io review, 训练流程 /
 * 稀疏感知训练); the function differentiated is, for each query row, softmax attention over the
 * visible keys of the key blocks its tile kept:
 *   O_i = sum_{k in K_i} softmax_k(scale * q_i . k_k) v_k,
 * so with P = exp(scale * Q K^T - LSE) on those pairs and D_i = sum_d dO_id O_id:
 *   dV = P^T dO, dP = dO V^T, dS = scale * P * (dP - D), dQ = dS K, dK = dS^T Q,
 * and a skipped or not-live tile-block adds nothing to dQ, dK or dV.
 *
 * Inputs (device memory, last dimension contiguous, element strides {batch, head, token}):
 *   q, k, v   as for the forward (bf16)
 *   o         the forward's output [batch][num_q_heads][seqlen_q][head_dim_v], dtype o_dtype (bf16 or
 *             fp32; it enters only D, where an fp32 output avoids the bf16 rounding of O)
 *   dout      dL/dO [batch][num_q_heads][seqlen_q][head_dim_v] (bf16)
 *   lse       the forward's LSE [batch][num_q_heads][seqlen_q] fp32 contiguous
 *   skip_mask the forward's skip mask [batch][num_q_heads][ceil(seqlen_q/block_q)]
 *             [ceil(seqlen_k/block_k)] uint8, from a forward with the same causal flag and blocks;
 *             NULL: every live block counts as kept (the backward of dense attention)
 * Outputs (overwritten, dtype grad_dtype):
 *   dq [batch][num_q_heads][seqlen_q][head_dim_qk], dk [batch][num_kv_heads][seqlen_k][head_dim_qk],
 *   dv [batch][num_kv_heads][seqlen_k][head_dim_v]; dk and dv sum over the q heads of each kv head.
 * workspace: device memory of at least blasst_prefill_backward_workspace_size() bytes (the row
 * sums D), 256-byte aligned; the library allocates nothing.
 * Rows without any kept key (LSE = -inf) get no gradient.
 * Supported: bf16 inputs, bf16 or fp32 gradients, head_dim_qk == head_dim_v == 128,
 * block_q == block_k == 128.
 */
typedef struct {
  size_t struct_size;        /* sizeof(blasst_prefill_backward_params) */
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  const uint8_t *skip_mask;
  void *dq, *dk, *dv;
  void *workspace;
  size_t workspace_bytes;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], dout_stride[3];
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  int32_t in_dtype, grad_dtype, o_dtype; /* blasst_dtype */
  int32_t batch, seqlen_q, seqlen_k, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v;
  int32_t causal, block_q, block_k;
  float softmax_scale;       /* <= 0 selects 1/sqrt(head_dim_qk); must match the forward */
} blasst_prefill_backward_params;

/* Prefill forward (see the struct comment).  stream: hipStream_t or NULL. */
blasst_status blasst_prefill(const blasst_prefill_params *params, void *stream);

/* Workspace bytes that blasst_prefill needs for these params: always 0, since one workgroup owns a
 * query tile for its whole key range (splits restart only the running max of the skip rule, and
 * their chunks accumulate in the same registers), so no partial results leave the kernel.  The query
 * exists so that callers can size buffers uniformly across entry points.  Returns 0 and sets the last
 * error when the params are invalid (pointers are not checked), 0 with the last error cleared
 * otherwise. */
size_t blasst_prefill_workspace_size(const blasst_prefill_params *params);

/* Chunked prefill against a paged cache (see the struct comment).  stream: hipStream_t or NULL. */
blasst_status blasst_prefill_paged(const blasst_prefill_paged_params *params, void *stream);

/* Prefill backward (see the struct comment).  stream: hipStream_t or NULL. */
blasst_status blasst_prefill_backward(const blasst_prefill_backward_params *params, void *stream);

/* Workspace bytes that blasst_prefill_backward needs for these params.  Returns 0 and sets the last
 * error when the params are invalid. */
size_t blasst_prefill_backward_workspace_size(const blasst_prefill_backward_params *params);

/* Paged split-KV decode forward (see the struct comment).  stream: hipStream_t or NULL. */
blasst_status blasst_decode(const blasst_decode_params *params, void *stream);

/* Workspace bytes that blasst_decode needs for these params (0 when num_splits == 1).  Returns 0
 * and sets the last error when the params are invalid. */
size_t blasst_decode_workspace_size(const blasst_decode_params *params);

/* Bytes of the scratch array behind blasst_decode_no_alloc (one array per GPU). */
#define BLASST_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * blasst_decode without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops or harnesses that forbid hipMalloc).  It computes exactly what
 * blasst_decode computes, with the same kernels; params->workspace and workspace_bytes are ignored.
 * The per-split partials go to a device array of BLASST_NO_ALLOC_SCRATCH_BYTES bytes that the
 * library holds on every GPU it runs on, until the process ends; params whose
 * blasst_decode_workspace_size() exceeds it are refused with BLASST_ERR_WORKSPACE before any HIP
 * call (GQA decode at batch 32, 32 q heads, 16 splits needs 8.5 MB; latent decode at batch 64 and 8
 * splits, 134 MB, is refused).  The call allocates nothing: on the first call on a device it looks
 * up that device's address of the array (hipGetSymbolAddress), and every later call reuses it.
 * Every call on one GPU shares that GPU's array and nothing in it needs clearing (every partial is
 * rewritten), so calls that may overlap on one GPU (two streams, or two host threads without
 * ordering) race on it: order them on one stream, or use blasst_decode with separate workspaces.
 */
blasst_status blasst_decode_no_alloc(const blasst_decode_params *params, void *stream);

/*
 * Host-only calibration [xllm-io review, 核心公式 calibration model lambda * L = alpha * exp(beta s);
 * 模型组件 calibration module: one forward pass over a sample].
 *
 * blasst_calib_quantile: from n critical values (host fp32 array, as written by a stats_only pass;
 * NaN entries are ignored, +inf entries count as never skippable), the ln(lambda) at which a
 * fraction target_s of them lies strictly below: with k = ceil(target_s * N) it is the midpoint of
 * the k-th and (k+1)-th smallest values, capped at 0 (lambda <= 1); target_s = 0 gives -inf.
 *
 * blasst_calibrate: ordinary least squares of y = ln(lambda_i * L_i) on x = s_i over n >= 2 points
 * (host arrays), giving alpha = exp(intercept), beta = slope and the rmse of y.  Requires
 * lambda_i > 0, L_i > 0 and at least two distinct s_i.
 *
 * blasst_lambda_for: the deployed threshold min(1, alpha * exp(beta * s) / L).
 */
blasst_status blasst_calib_quantile(const float *crit, int64_t n, double target_s, double *ln_lambda);
blasst_status blasst_calibrate(const double *L, const double *s, const double *lambda, int32_t n,
                               double *alpha, double *beta, double *rmse);
double blasst_lambda_for(double alpha, double beta, double s, double L);

/* Status text, last error message of the calling thread, library version (major*10000+minor*100+patch),
 * and the struct sizes the library was built with (for binding checks). */
const char *blasst_status_string(blasst_status status);
const char *blasst_last_error(void);
int32_t blasst_version(void);
size_t blasst_prefill_params_size(void);
size_t blasst_decode_params_size(void);
size_t blasst_prefill_backward_params_size(void);
size_t blasst_prefill_paged_params_size(void);

#ifdef __cplusplus
}
#endif

#endif /* BLASST_H */
