/*
 * fa.h -- C ABI of the exact tiled attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention,
 *
 *     O = softmax(scale * Q K^T + mask) V,
 *
 * one tile of queries against a stream of key/value tiles at a time, with an
 * online softmax that keeps a running row maximum and row sum, so the
 * seqlen_q x seqlen_k score matrix never reaches HBM.  The forward pass writes O
 * and the per-row natural-log log-sum-exp (LSE); the backward pass recomputes
 * the score tiles from Q, K and the LSE instead of storing probabilities.
 *
 * Sources (web pages, cited by title and section):
 *   [P4] "FlashAttention 实战指南:如何把训练内存省 20 倍、速度提 4 倍" (kwkr.cn):
 *        section "长序列注意力为什么会爆内存" -- the three steps of standard
 *        attention, tiling into on-chip memory, the online softmax that updates
 *        the row maximum and sum block by block, and recomputation in the
 *        backward pass; section "上手 FlashAttention 的三步走" -- tensors are
 *        (batch, seqlen, nheads, headdim) and causal=True for autoregressive
 *        use; section "进阶参数如何配置causal、window_size 与 MQA/GQA" --
 *        window_size (left, right) with -1 meaning unbounded, and K/V head
 *        counts that divide the Q head count (MQA/GQA).
 *   [P5] "AI模型推理优化Flash Attention原理" (52runoob.com), section
 *        "先搞清楚原理" -- scores are scaled by 1/sqrt(headdim) by default.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees, copies or synchronises; kernels are enqueued on
 *     the caller's HIP stream (hipStream_t passed as void*, NULL = null stream)
 *     and the call returns before they finish.
 *   - Layout: q, o, dout, dq are (batch, seqlen_q, nheads_q, headdim); k, v,
 *     dk, dv are (batch, seqlen_k, nheads_kv, headdim).  Strides are given in
 *     ELEMENTS for the batch, sequence and head axes; the headdim axis is
 *     contiguous (stride 1).  lse is a dense float32 array (batch, nheads_q,
 *     seqlen_q).
 *   - Masks: query i sees key j iff every active condition holds, with
 *     i' = i + seqlen_k - seqlen_q (the last query is aligned with the last key):
 *        causal                ->  j <= i'
 *        window_left  >= 0     ->  j >= i' - window_left
 *        window_right >= 0     ->  j <= i' + window_right
 *     A window bound of -1 is unbounded.  A query that sees no key gets O = 0,
 *     LSE = -inf and zero gradients.
 *   - MQA/GQA: query head h reads K/V head h / (nheads_q / nheads_kv).
 *   - Errors: every argument is validated on the host before any HIP call; a
 *     non-OK status is returned synchronously and fa_last_error() gives the
 *     detail (per thread).  No C++ exception crosses this boundary.  Kernel
 *     faults surface asynchronously on the stream like any HIP work.
 *   - Thread safety: the library keeps no mutable global state besides a
 *     per-device capability cache and the per-thread error string.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_VERSION 10000 /* 1.0.0 */

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* malformed input (sizes, null pointers, window < -1, ...) */
  FA_ERR_UNSUPPORTED = 2, /* valid input this build does not run (headdim, alignment, arch) */
  FA_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed */
} fa_status;

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/* The three stages of fa_bwd (see fa_bwd_stage). */
typedef enum {
  FA_BWD_PREPARE = 0, /* per-row statistics of the backward pass -> workspace */
  FA_BWD_DKDV = 1,    /* dk and dv, reading the workspace */
  FA_BWD_DQ = 2       /* dq, reading the workspace */
} fa_bwd_stage_id;

typedef struct {
  int64_t batch;
  int64_t seqlen_q, seqlen_k;
  int64_t nheads_q, nheads_kv; /* nheads_q must be a multiple of nheads_kv */
  int64_t headdim;             /* fp16/bf16: multiple of 8, 8..128; fp32: multiple of 4, 4..128 */
  /* (batch, seq, head) strides in elements; the headdim axis has stride 1.
   * In fa_bwd, dout uses o_strides, dq uses q_strides, dk uses k_strides and
   * dv uses v_strides. */
  int64_t q_strides[3], k_strides[3], v_strides[3], o_strides[3];
  fa_dtype dtype;       /* element type of q, k, v, o, dout, dq, dk, dv */
  float scale;          /* > 0 and finite; callers usually pass 1/sqrt(headdim) */
  int32_t causal;       /* 0 or 1 */
  int32_t window_left;  /* -1 = unbounded, else >= 0 */
  int32_t window_right; /* -1 = unbounded, else >= 0 */
  /* Score modifiers ([P4] section "进阶参数如何配置causal、window_size 与
   * MQA/GQA": alibi_slopes, a positional bias that decays scores with
   * distance; softcap, logits truncated to [-softcap, softcap]).  With
   * x = scale * q_i . k_j and i' = i + seqlen_k - seqlen_q, the logit fed to
   * the softmax is
   *     min(max(x, -softcap), softcap) - slope(b, h) * |i' - j|
   * (the clamp only when softcap > 0, the bias only when alibi_slopes is
   * given), and the mask is applied after.  The backward differentiates
   * this exactly: the clamp passes the gradient only where |x| < softcap. */
  const float* alibi_slopes;  /* NULL, or float32 DEVICE array: slope(b, h) at
                                 b * alibi_batch_stride + h, h < nheads_q */
  int64_t alibi_batch_stride; /* >= 0; 0 = the same slopes for every batch entry */
  float softcap;              /* 0 = off, else > 0 and finite */
  int32_t reserved_mod;       /* 0 */
} fa_params;

/*
 * Forward pass: o = softmax(scale * q k^T + mask) v and lse[b][h][i] =
 * natural-log log-sum-exp of row i's visible scaled scores ([P4] section
 * "长序列注意力为什么会爆内存"; the LSE is the final state of the online
 * softmax's running maximum and sum).
 *   q [in]  (batch, seqlen_q, nheads_q, headdim), dtype
 *   k [in]  (batch, seqlen_k, nheads_kv, headdim), dtype
 *   v [in]  same shape as k
 *   o [out] same shape as q (o_strides), dtype; must not alias q, k or v
 *   lse [out] float32 (batch, nheads_q, seqlen_q), dense
 *   stream  hipStream_t or NULL
 * Requirements: all pointers 16-byte aligned and every stride a multiple of
 * 16 bytes; sequence strides at most 2^22 elements and, when the sequence has
 * more than one row, at least headdim (else FA_ERR_UNSUPPORTED).  A sequence
 * of one row may carry any stride, 0 included.  Results are bitwise
 * repeatable for identical inputs and launch configuration.
 */
fa_status fa_fwd(const fa_params* params, const void* q, const void* k, const void* v,
                 void* o, float* lse, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these parameters: two float32
 * per-row arrays (D_i = sum_c dout[i,c] * o[i,c], and the LSE in base 2) of
 * batch * nheads_q * Nq_pad entries each, Nq_pad = seqlen_q rounded up to a
 * multiple of 128; the total is rounded up to 256 bytes.  Writes it to *bytes.
 */
fa_status fa_bwd_workspace_size(const fa_params* params, size_t* bytes);

/*
 * Backward pass: gradients of L = sum(o * dout) with respect to q, k and v,
 * recomputing the probability tiles from q, k and lse ([P4] section
 * "长序列注意力为什么会爆内存": the backward pass does not keep the attention
 * matrix and recomputes it when needed):
 *     dP = dout v^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
 *     dq = scale dS k,  dk = scale dS^T q,  dv = P^T dout,
 * with dk and dv summed over the query heads of a K/V head group.
 *   dout [in] same shape/layout as o (o_strides), dtype
 *   q, k, v [in] as in fa_fwd
 *   o [in]  the forward output (o_strides), dtype
 *   lse [in] the forward LSE, float32 (batch, nheads_q, seqlen_q)
 *   dq [out] shape of q (q_strides); dk, dv [out] shape of k (k_strides,
 *            v_strides).  Outputs are fully overwritten (no accumulation).
 *   workspace [scratch] device memory of at least fa_bwd_workspace_size bytes,
 *            256-byte aligned, owned by the caller; contents are clobbered.
 * The gradients are computed without atomics, so they are bitwise repeatable.
 */
fa_status fa_bwd(const fa_params* params, const void* dout, const void* q, const void* k,
                 const void* v, const void* o, const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * One stage of fa_bwd, with the same arguments and the same validation.
 * fa_bwd is exactly FA_BWD_PREPARE, FA_BWD_DKDV, FA_BWD_DQ on one stream;
 * the stages are exposed so that a caller can time them or order them
 * itself ([P4] section "长序列注意力为什么会爆内存" for the recomputation
 * each stage performs):
 *   FA_BWD_PREPARE  writes D_i = sum_c dout_ic o_ic and the forward LSE
 *                   (rescaled to base 2) of every query row into workspace;
 *                   reads dout, o, lse.  dq, dk, dv are not touched.
 *   FA_BWD_DKDV     writes dk and dv (fully overwritten); reads q, k, v,
 *                   dout and the workspace.
 *   FA_BWD_DQ       writes dq (fully overwritten); reads q, k, v, dout and
 *                   the workspace (and lse for fp32).
 * DKDV and DQ must run after PREPARE of the same params, inputs and
 * workspace has completed (stream order, or an event); they do not depend
 * on each other.  Every pointer argument is required exactly as for fa_bwd,
 * whichever stage runs.  An unknown stage is FA_ERR_INVALID_ARG.
 */
fa_status fa_bwd_stage(const fa_params* params, int stage, const void* dout, const void* q,
                       const void* k, const void* v, const void* o, const float* lse, void* dq,
                       void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight training or serving loops, harnesses
 * that forbid allocation).  Same arguments (minus the workspace), validation,
 * kernels and results as fa_bwd, bit for bit.  The backward's row statistics
 * go to a static scratch array inside the library instead: 16 MiB on each GPU
 * the library runs on, held until the process ends, enough for
 * batch * nheads_q * Nq_pad <= 2^21 rows (Nq_pad = seqlen_q rounded up to a
 * multiple of 128; e.g. batch 2 x 32 heads x 32768 queries).  Larger problems
 * return FA_ERR_UNSUPPORTED before any device work; use fa_bwd for them.
 * The call allocates nothing (the scratch's device address is looked up once
 * per device, on the first call made with that device current).  All calls
 * on one GPU share its scratch and it keeps the last call's contents:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be serialised by the caller.
 */
fa_status fa_bwd_noalloc(const fa_params* params, const void* dout, const void* q, const void* k,
                         const void* v, const void* o, const float* lse, void* dq, void* dk, void* dv,
                         void* stream);

/*
 * Packed variable-length batches ([P4] section "上手 FlashAttention 的三步走":
 * when the sequences of a batch differ in length, the varlen interfaces take
 * them packed one after another instead of padded).
 *
 * Sequence b (0 <= b < base.batch) is rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 * of q, o, dout, dq (each (total_q, nheads_q, headdim)) and rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k, v, dk, dv (each (total_k,
 * nheads_kv, headdim)).  Each sequence is attended on its own, exactly as one
 * batch entry of fa_fwd / fa_bwd with its own lengths (masks aligned to the
 * end of its own keys).
 *
 * base: batch = number of sequences; seqlen_q / seqlen_k = upper bounds of
 *   the sequence lengths (they size the launch; longer sequences are cut to
 *   them); the other fields as for fa_fwd.  strides[0] (the batch axis) is
 *   ignored; strides[1] is the row stride and strides[2] the head stride of
 *   the packed tensors.
 * total_q, total_k: rows of the packed tensors (at most 2^31 - 1).
 * cu_seqlens_q, cu_seqlens_k: int32 DEVICE arrays of batch + 1 prefix offsets,
 *   cu[0] = 0, nondecreasing, cu[batch] <= total.  They are read on the
 *   device: offsets are clamped to [0, total] and lengths to the bounds
 *   above, so inconsistent values give unspecified results but never an
 *   access outside the tensors.  Rows outside every sequence are not written.
 * lse: float32 (nheads_q, total_q): lse[h * total_q + row].
 */
typedef struct {
  fa_params base;
  int64_t total_q;
  int64_t total_k;
} fa_varlen_params;

/* Forward over a packed batch: o and lse as fa_fwd, per sequence. */
fa_status fa_fwd_varlen(const fa_varlen_params* params, const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o, float* lse,
                        void* stream);

/* Bytes of workspace fa_bwd_varlen needs: two float32 arrays of
 * nheads_q * (total_q + 128 * batch) entries, rounded up to 256 bytes. */
fa_status fa_bwd_varlen_workspace_size(const fa_varlen_params* params, size_t* bytes);

/* Backward over a packed batch: dq, dk, dv as fa_bwd, per sequence (dq has
 * q's strides, dk k's, dv v's, dout o's).  Key rows of sequences without
 * queries get zero gradients. */
fa_status fa_bwd_varlen(const fa_varlen_params* params, const void* dout, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Attention against a KV cache (incremental decoding, [P4] section
 * "增量解码场景flash_attn_with_kvcache": new keys and values are appended to
 * the cache in place, cache_seqlens gives each batch entry's valid length,
 * and the key range is split so that few queries against a long cache still
 * fill the GPU).
 *
 * base: batch; seqlen_q = Nq new queries per batch entry; seqlen_k = cache
 *   capacity in rows; nheads_q, nheads_kv, headdim (multiple of 8, <= 128); q_strides and
 *   o_strides for q and o (batch, Nq, nheads_q, headdim); k_strides and
 *   v_strides for the caches (batch, capacity, nheads_kv, headdim); dtype
 *   FA_F16 or FA_BF16; scale; causal and window as in fa_fwd.
 * knew_strides, vnew_strides: strides of k_new and v_new (batch, Nq,
 *   nheads_kv, headdim); ignored when k_new is NULL.
 * num_splits: parts of the key range per (batch, K/V head), >= 1, or 0 to
 *   let the library choose enough parts to fill the GPU; at most the
 *   capacity's count of 32-key tiles (and 1024) are used.  The visible key
 *   tiles of each block of queries are cut into that many equal runs.  The
 *   split only changes rounding, never the result's definition.
 */
typedef struct {
  fa_params base;
  int64_t knew_strides[3], vnew_strides[3];
  int32_t num_splits;
  int32_t reserved; /* 0 */
} fa_kvcache_params;

/* Bytes of workspace fa_fwd_kvcache needs: float32 partial outputs and LSEs
 * of every part, B * nheads_q * Nq * parts * (Dk + 1) floats, rounded up to
 * 256 bytes, where Dk = 64 for headdim <= 64 and 128 otherwise. */
fa_status fa_fwd_kvcache_workspace_size(const fa_kvcache_params* params, size_t* bytes);

/*
 * For each batch entry b with L = cache_seqlens[b] (clamped to [0, capacity]):
 *   if k_new is given, rows L .. L+Nq-1 of k_cache / v_cache are overwritten
 *   with k_new[b] / v_new[b] (rows past the capacity are dropped) and the
 *   queries see Lk = min(L + Nq, capacity) keys; otherwise Lk = L;
 *   o[b] = softmax(scale * q[b] K^T + mask) V over cache rows [0, Lk), with
 *   query i aligned to key i + Lk - Nq and the causal/window rule of fa_fwd;
 *   lse[b] is its float32 natural-log LSE (B, nheads_q, Nq).
 *   q [in] (batch, Nq, nheads_q, headdim), dtype
 *   k_cache, v_cache [in/out] (batch, capacity, nheads_kv, headdim), dtype
 *   cache_seqlens [in] int32 device array (batch); lengths are read on the
 *            device, so values outside [0, capacity] are clamped, not rejected
 *   k_new, v_new [in] both NULL (no append) or both given
 *   o [out] like q; lse [out] float32 (batch, nheads_q, Nq)
 *   workspace [scratch] fa_fwd_kvcache_workspace_size bytes, caller-owned
 * Rows with no visible key get o = 0 and lse = -inf.  fp32 returns
 * FA_ERR_UNSUPPORTED.  Asynchronous on stream.
 */
fa_status fa_fwd_kvcache(const fa_kvcache_params* params, const void* q, void* k_cache, void* v_cache,
                         const int32_t* cache_seqlens, const void* k_new, const void* v_new, void* o,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Static string naming a status code. */
const char* fa_status_string(fa_status status);

/* Detail message of the last non-OK status returned on this thread ("" if none). */
const char* fa_last_error(void);

/* FA_VERSION of the built library. */
int fa_version(void);

/*
 * Paged KV cache ([P4] section "增量解码场景flash_attn_with_kvcache": block_table
 * turns on a cache stored in fixed-size blocks, which makes swapping and
 * fragmentation easier to manage).  Everything is as in fa_fwd_kvcache except
 * where the cache rows live:
 *   k_cache, v_cache  pools of num_pages pages, (num_pages, page_size,
 *                     nheads_kv, headdim); base.k_strides / v_strides are the
 *                     (page, row, head) strides;
 *   block_table       int32 DEVICE array: row j of batch entry b is row
 *                     j % page_size of page block_table[b * block_table_stride
 *                     + j / page_size].  Page numbers are read on the device and
 *                     clamped to [0, num_pages), so a bad table gives wrong
 *                     results but no access outside the pools;
 *   base.seqlen_k     capacity of one entry, a whole number of pages
 *                     (pages per entry = seqlen_k / page_size <= block_table_stride);
 *   page_size         a positive multiple of 32 (a 32-key tile never spans pages).
 * The append writes the new rows into the pages the table names.  Workspace:
 * fa_fwd_kvcache_workspace_size.
 */
fa_status fa_fwd_kvcache_paged(const fa_kvcache_params* params, int32_t page_size, int64_t num_pages,
                               const int32_t* block_table, int64_t block_table_stride, const void* q, void* k_cache,
                               void* v_cache, const int32_t* cache_seqlens, const void* k_new, const void* v_new,
                               void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Packed Q/K/V ([P4] section "上手 FlashAttention 的三步走": q, k and v stored
 * in one tensor) need no entry point of their own: a (batch, seqlen, 3, nheads,
 * headdim) tensor gives q, k and v as strided views (head stride headdim,
 * sequence stride 3 * nheads * headdim) for fa_fwd / fa_bwd, and dq, dk, dv can
 * be the matching views of one packed gradient tensor. */

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* FA_H_ */
