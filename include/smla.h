/*
 * smla.h — C ABI of the MI355X (gfx950) library for sparse Multi-head Latent Attention with a
 * lightning indexer: indexer scoring -> per-query exact top-k -> sparse MLA over a shared
 * latent KV cache.
 *
 * What the pages define ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse on 16 H200", sections
 * "Why DP8 and TP8 fall short", "PCP: split tokens, not heads", "Why the numbers work"):
 *  - an indexer scores every earlier token for every query token and the 2,048 best are kept;
 *    its cost grows with the square of the prompt, sparse MLA's only linearly;
 *  - MLA's latent KV row is shared by all 64 heads, so one gathered row serves every head;
 *  - QK runs over 576 dims and PV over 512; queries and outputs are BF16; a KV row is 656 bytes
 *    of FP8 plus a 4-byte index;
 *  - partial attention results over disjoint row sets merge by log-sum-exp (section "DCP").
 * The indexer's formula is score(t, s) = sum_h w_h * ReLU(q_I[t,h] . k_I[s]) over s <= p(t),
 * on int8 inputs with exact int32 results; ties go to the lower token index.
 *
 * Conventions for every entry point
 *  - Pointers marked (device) are HIP device memory; (host) are host memory. The caller owns
 *    every buffer; the library keeps no pointer after a call returns.
 *  - GPU entry points are asynchronous on `stream` (a hipStream_t; NULL is the default stream)
 *    and never synchronise; buffers must stay valid until the stream reaches the work.
 *  - The library allocates no device memory: scratch comes from a caller workspace sized by the
 *    matching *_workspace_bytes function.
 *  - Return SMLA_OK (0) or a negative smla_status. Arguments are validated on the host before
 *    anything is enqueued; on error nothing is enqueued and smla_last_error() describes why.
 *  - Device pointers must be 16-byte aligned (q, kv, q_idx, k_idx, out, workspace: 256 bytes).
 *
 * Batch layout (all entry points): request b owns query tokens [Q_b, Q_b + n_q[b]) and latent
 * rows / indexer keys [R_b, R_b + kv_len[b]), Q and R being exclusive prefix sums. Query j of
 * request b sits at position p = kv_len[b] - n_q[b] + j (its own row is already in the cache)
 * and may use rows s <= p; s is local to the request. smla_batch_build_pos takes the positions
 * explicitly instead (a DCP shard's tokens, below).
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum smla_status {
  SMLA_OK = 0,
  SMLA_E_INVALID = -1,     /* null pointer, bad size, misaligned pointer, inconsistent batch */
  SMLA_E_UNSUPPORTED = -2, /* shape outside the supported families (see each entry point) */
  SMLA_E_WORKSPACE = -3,   /* workspace missing or smaller than *_workspace_bytes */
  SMLA_E_HIP = -4,         /* a HIP runtime call failed */
} smla_status;

typedef enum smla_kv_format {
  SMLA_KV_BF16 = 0,    /* row = D_qk bfloat16 values (2*D_qk bytes) */
  SMLA_KV_FP8_656 = 1, /* row = 656 bytes: [512 e4m3 (OCP E4M3FN) codes of dims 0..511]
                          [4 x fp32 scale, one per 128-dim block][64 x bf16 dims 512..575];
                          value = e4m3(code) * scale[d / 128]. Requires D_qk = 576, D_v = 512. */
} smla_kv_format;

/* Host-side summary of a batch; `table` points at the device table smla_batch_build wrote. */
typedef struct smla_batch {
  int32_t batch;      /* B >= 1 */
  int32_t total_q;    /* sum of n_q */
  int32_t max_q;      /* max n_q */
  int32_t n_items;    /* indexer work items in the table */
  int64_t max_kv;     /* max kv_len */
  int64_t total_rows; /* sum of kv_len */
  int64_t total_cand; /* sum over query tokens of (p + 1) */
  int64_t min_cand;   /* min over query tokens of (p + 1) */
  const void* table;  /* (device) table written by smla_batch_build */
  size_t table_bytes;
} smla_batch;

/* Device bytes smla_batch_build needs for a batch of `batch` requests and `total_q` tokens
 * (an upper bound that holds for any lengths). */
size_t smla_batch_table_bytes(int32_t batch, int32_t total_q, int64_t max_kv);

/*
 * Validate a batch and write its device table. n_q (host) [batch], kv_len (host) [batch] with
 * 1 <= n_q[b] <= kv_len[b] < 2^31 and total rows < 2^40. `table` (device, table_bytes from
 * smla_batch_table_bytes) receives the per-request, per-token and indexer work-item tables.
 * Blocking: returns after the table is on the device (smla_batch_build_pos with a staging
 * buffer does the same without waiting). `out` is filled on success.
 */
int smla_batch_build(int32_t batch, const int32_t* n_q, const int64_t* kv_len, void* table,
                     size_t table_bytes, void* stream, smla_batch* out);

/*
 * smla_batch_build with every query token's position given, and optionally without waiting.
 * pos (host, optional) [total_q]: token j of request b at pos[Q_b + j] with 0 <= pos <
 * kv_len[b], non-decreasing within a request; the token uses rows s <= pos (NULL: the default
 * positions kv_len - n_q + j). Under decode context parallelism ("Serving GLM-5.3 ... PCP, DCP,
 * Hybrid HiSparse", section "DCP") a shard holds every n-th row, so the consecutive global
 * positions of a request's tokens (MTP drafts) become local positions that repeat or step by
 * one: shard l of n gives global position P the local position floor((P - l) / n), which needs
 * P >= l. host_staging (host, optional, at least table_bytes): the table is assembled there and
 * copied to `table` on `stream` without waiting (pinned memory makes the copy truly
 * asynchronous); the caller keeps it unchanged until the stream has run the copy. NULL: the call
 * uses its own buffer and returns after the copy, as smla_batch_build does. Same table size
 * bound and contract otherwise.
 */
int smla_batch_build_pos(int32_t batch, const int32_t* n_q, const int64_t* kv_len,
                         const int64_t* pos, void* host_staging, void* table, size_t table_bytes,
                         void* stream, smla_batch* out);

/*
 * Indexer scores, full matrix (parity and debugging; O(total_q * max_kv) memory). The indexer
 * scores every earlier token of every query token ("Serving GLM-5.3 ... PCP, DCP, Hybrid
 * HiSparse", sections "Why DP8 and TP8 fall short" and "PCP: split tokens, not heads"; the
 * formula is in the file preamble).
 * q_idx (device) [total_q, H_I, D_I] int8; k_idx (device) [total_rows, D_I] int8;
 * w (device) [H_I] int32 with w_h >= 0 and sum_h w_h * 2^14 * D_I < 2^31 (so no score can
 * overflow; a violation gives wrong scores, never a fault).
 * scores (device) [total_q, max_kv] int32: score(t, s) for s <= p, -1 for p < s < max_kv.
 * Supported (H_I, D_I): (64, 128) on int8 MFMA, and H_I <= 16 with D_I a multiple of 4 up to
 * 256 on a generic kernel.
 */
int smla_indexer_scores(const smla_batch* b, const int8_t* q_idx, const int8_t* k_idx,
                        const int32_t* w, int32_t H_I, int32_t D_I, int32_t* scores, void* stream);

/*
 * Workspace for smla_indexer_scores_topk. Zero-fill it once after allocating it (for example
 * with hipMemsetAsync): the per-row histograms and counters it holds must be zero when a call
 * starts, and every call that returns SMLA_OK leaves them zero again, so the same workspace
 * serves any later call whose size fits. After a call that failed on the device, zero it again.
 * Calls that share one workspace must not overlap.
 */
size_t smla_indexer_topk_workspace_bytes(const smla_batch* b, int32_t H_I, int32_t D_I,
                                         int32_t top_k);

/*
 * Indexer scores followed by the exact per-query top-k (same inputs as smla_indexer_scores):
 * the 2,048 best earlier tokens of each query token that sparse MLA attends over ("Serving
 * GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why DP8 and TP8 fall short").
 * idx (device) [total_q, top_k] int32: the min(top_k, p+1) local row indices with the largest
 * scores, ties to the lower index (all s <= p when p+1 <= top_k), in ascending index order,
 * then -1 padding. score (device, optional) [total_q, top_k] int32: the score of each selected
 * index, -1 on padding. 1 <= top_k <= 2048; kv_len <= 8,388,608 (SMLA_E_UNSUPPORTED beyond).
 * ws: a workspace of smla_indexer_topk_workspace_bytes, zero-filled before its first use.
 */
int smla_indexer_scores_topk(const smla_batch* b, const int8_t* q_idx, const int8_t* k_idx,
                             const int32_t* w, int32_t H_I, int32_t D_I, int32_t top_k,
                             int32_t* idx, int32_t* score, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * Indexer scores over FP8 keys, full matrix (parity and debugging; O(total_q * max_kv) memory).
 * The pages' deployed indexer key is 128 E4M3 values plus one fp32 scale per token, 132 bytes
 * ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why the numbers work"):
 *   score(t, s) = k_scale[s] * sum_h w[t,h] * ReLU(sum_d q[t,h,d] * k[s,d])
 * q (device) [total_q, H_I, D_I] OCP E4M3 codes, 16-byte aligned; k (device) [total_rows, D_I]
 * E4M3 codes, 16-byte aligned; k_scale (device) [total_rows] fp32 >= 0; w (device)
 * [total_q, H_I] fp32 >= 0, per query token (a query's own scale folds into it).
 * The products are exact; each head's dot product is summed by the FP8 matrix cores, whose
 * sums are not IEEE-rounded fp32 (errors of order 2^-18 of the sum of |products| occur); the
 * head sum and the scale are fp32. scores (device, 16-byte aligned) [total_q, max_kv] fp32:
 * score(t, s) for s <= p, -1.0f for p < s < max_kv. Scores are >= +0 for valid inputs; NaN
 * codes (0x7F, 0xFF) or negative or non-finite w or k_scale give unspecified scores, never a
 * fault. Supported (H_I, D_I): (64, 128) only (SMLA_E_UNSUPPORTED otherwise).
 */
int smla_indexer_scores_fp8(const smla_batch* b, const uint8_t* q, const uint8_t* k,
                            const float* k_scale, const float* w, int32_t H_I, int32_t D_I,
                            float* scores, void* stream);

/*
 * FP8-key scores followed by the exact per-query top-k of those fp32 scores (larger score first,
 * ties to the lower index), with the contract of smla_indexer_scores_topk otherwise: idx
 * [total_q, top_k] ascending with -1 padding; score (optional) [total_q, top_k] fp32, -1.0f on
 * padding. ws: smla_indexer_topk_workspace_bytes(b, 64, 128, top_k) bytes, zero-filled before
 * its first use; one workspace serves both key formats (calls must not overlap).
 */
int smla_indexer_scores_topk_fp8(const smla_batch* b, const uint8_t* q, const uint8_t* k,
                                 const float* k_scale, const float* w, int32_t H_I, int32_t D_I,
                                 int32_t top_k, int32_t* idx, float* score, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Decode context parallelism on one GPU (the pages shard the KV cache round robin, every n-th
 * token to one GPU, and merge what the shards compute: "Serving GLM-5.3 ... PCP, DCP, Hybrid
 * HiSparse", section "DCP"). Shard l of n holds the tokens l, l + n, l + 2n, ... of every request,
 * so its local row j is global row j n + l. Each shard runs smla_indexer_scores_topk and a
 * sparse-MLA entry point on its own rows; these three calls merge the results.
 *
 * smla_topk_merge: the exact global top-k of each query token from the shards' lists. idx_lists
 * and score_lists (device) hold n_lists stacked [total_q, k_in] arrays, list l at element offset
 * l * list_stride (list_stride >= total_q * k_in): local indices (-1 padding) and their scores
 * (non-negative int32 with float_scores = 0; the bit patterns of non-negative fp32 scores, as
 * smla_indexer_scores_topk_fp8 returns them, with float_scores = 1). idx (device)
 * [total_q, top_k]: the top_k global indices by (score desc, index asc), in ascending index
 * order, -1 padded; score (device, optional) [total_q, top_k] likewise, -1 (-1.0f) on padding. The merge
 * is exact because a member of the global top-k is in its own shard's top-k. local_idx (device,
 * optional) [n_lists, total_q, top_k]: every shard's part of the merged selection, as
 * smla_dcp_local_indices would return it for n_shards = n_lists (ascending local indices, then -1),
 * written by the same launch; it needs n_lists <= 64 (SMLA_E_UNSUPPORTED otherwise).
 * 1 <= n_lists, 1 <= k_in, n_lists * k_in <= 16,384, 1 <= top_k <= 2,048; global indices must stay
 * below 2^31. Lists in the order the indexer's top-k returns them (each list's valid entries in
 * ascending local index, then only padding) take a sort-free path; any other order is accepted
 * and sorted.
 */
int smla_topk_merge(int32_t total_q, int32_t n_lists, int32_t k_in, const int32_t* idx_lists,
                    const int32_t* score_lists, int64_t list_stride, int32_t float_scores,
                    int32_t top_k, int32_t* idx, int32_t* score, int32_t* local_idx, void* stream);

/*
 * smla_dcp_local_indices: every shard's part of a global selection. idx (device)
 * [total_q, top_k] global indices (-1 padding); local_idx (device) [n_shards, total_q, top_k]:
 * for shard s, the entries g with g mod n_shards == s, as g div n_shards, in their order, then -1
 * (the order the sparse-MLA entry points read them in, padding last). 1 <= n_shards <= 65,535,
 * 1 <= top_k <= 2,048.
 */
int smla_dcp_local_indices(int32_t total_q, int32_t top_k, const int32_t* idx, int32_t n_shards,
                           int32_t* local_idx, void* stream);

/*
 * smla_lse_merge: partial attention results over disjoint row sets merged by log-sum-exp.
 * outs (device) [n_parts, total_q, H, D_v] bf16; lses (device) [n_parts, total_q, H] fp32,
 * natural log, -inf for a part that saw no row. out (device) [total_q, H, D_v] bf16:
 * sum_i w_i out_i / sum_i w_i with w_i = exp(lse_i - max lse); lse (device, optional)
 * [total_q, H]: max + log sum w_i (-inf and a zero output where no part saw a row).
 * 1 <= n_parts <= 64, 1 <= H, 1 <= D_v <= 4,096; bf16 arrays 2-byte aligned, fp32 4-byte.
 */
int smla_lse_merge(int32_t total_q, int32_t H, int32_t D_v, int32_t n_parts, const void* outs,
                   const float* lses, void* out, float* lse, void* stream);

/*
 * Hot-buffer resolve of a step's top-k under hybrid offload ("vLLM GLM 5.3 ... Hybrid
 * HiSparse", technical implementation: with mixed residency a request's older rows are in host
 * memory and only its tail is resident; the rows the indexer selects from the offloaded part are
 * served from a per-request GPU hot buffer of n_slots rows (the pages default to 2 x top_k),
 * managed least-recently-used; a miss copies one row from pinned host memory into an LRU slot).
 *
 * idx (device) [total_q, top_k]: the step's selections (local rows, -1 padding). Per request b
 * (device arrays of `batch` entries): resident_from[b] = first resident local row (rows below
 * it are offloaded; 0 = fully resident, nothing to do), at most p_0 + 1, p_0 the position of the
 * request's first query token (kv_len - n_q unless given to smla_batch_build_pos), so that every
 * query token of the request sees every offloaded row; hot_base[b] = local row of hot slot 0, with 0 <= hot_base and hot_base + n_slots <=
 * resident_from (the hot buffer sits in the request's released rows); host_row0[b] = host row
 * of the request's local row 0.
 * hot_tok / hot_age (device) [batch, n_slots]: the slots' token (-1 empty) and step of last use
 * (-1 never), initialised by the caller to -1 and updated in place; step >= 0 is this call's
 * and must grow from call to call for the least-recently-used order to hold.
 * host_rows (host, pinned: hipHostMalloc or a pinned torch tensor) [host_n_rows, row_bytes] is
 * read by the kernel directly; kv (device) rows of row_bytes (a multiple of 16), laid out as in
 * the batch; a miss of token u goes to kv row R_b + hot_base[b] + slot.
 *
 * Rule within one call (the pages fix none; this is the reading taken): the distinct offloaded
 * selections of the request's tokens, ascending; a selection whose token a slot holds is a hit
 * and that slot is used again; the misses, ascending, take the slots not hit in this call in
 * (last use, slot) order. Every used slot gets last use = step.
 * idx_out (device) [total_q, top_k], not aliasing idx: -1 for padding, resident rows as they
 * are, offloaded rows as hot_base[b] + slot — ready for the sparse-MLA entry points.
 * n_copied (device) [batch]: rows copied for request b, or (nothing changed, idx_out -1) -1 when
 * the distinct offloaded selections outnumber n_slots, -2 when resident_from / hot_base are
 * out of bounds, -3 when host rows [host_row0, host_row0 + resident_from) leave host_rows.
 * Limits: max n_q * top_k <= 8192, n_slots <= 4096. Calls for one request must be ordered.
 */
int smla_hot_resolve(const smla_batch* b, const int32_t* idx, int32_t top_k,
                     const int32_t* resident_from, const int32_t* hot_base, int32_t n_slots,
                     int32_t* hot_tok, int32_t* hot_age, int32_t step, const void* host_rows,
                     int64_t host_n_rows, const int64_t* host_row0, int32_t row_bytes, void* kv,
                     int32_t* idx_out, int32_t* n_copied, void* stream);

/* Workspace for the sparse-MLA entry points (decode needs split partials; prefill none). */
size_t smla_sparse_mla_workspace_bytes(const smla_batch* b, int32_t H, int32_t D_v,
                                       int32_t top_k, int32_t decode);

/*
 * Sparse MLA in MQA form: every head attends over the same selected rows ("Serving GLM-5.3 ...
 * PCP, DCP, Hybrid HiSparse", section "Why the numbers work": one latent row serves all 64
 * heads, QK over 576 dims and PV over 512, BF16 queries and outputs over 656-byte FP8 rows; the
 * split-KV merge of _decode is the log-sum-exp merge of section "DCP").
 * q (device) [total_q, H, D_qk] bf16; kv (device) [total_rows] rows of `kv_format`;
 * idx (device) [total_q, top_k] int32 local row indices (any order; -1 entries are skipped;
 * indices above the token's position p are treated like -1, so no row past p is ever read);
 * out (device) [total_q, H, D_v] bf16; lse (device, optional) [total_q, H] fp32 natural-log
 * log-sum-exp of the scaled logits (-inf and zero output for a token with no valid index).
 * logit_i = sm_scale * q_h . v_i over D_qk dims; output = softmax-weighted sum of v_i[0:D_v].
 * Supported: FP8_656 with (H, D_qk, D_v) = (64, 576, 512) on the matrix cores; BF16 rows with
 * H <= 16, D_qk <= 256, D_v <= D_qk on a generic fp32 kernel. top_k <= 2048.
 * FP8_656 arithmetic: the logits multiply q (bf16 as given) by the E4M3 codes and bf16 rope dims,
 * both exact in bf16, with fp32 accumulation; each 128-dim block's fp32 scale is applied to its
 * part of the logit in fp32, so any finite scale and the whole bf16 range of q are supported.
 * Softmax in fp32. The output products use P' = P * scale relative to a power of two chosen per
 * split: P and the relative scale each rounded to fp16 and multiplied in fp16 (11 significant
 * bits per rounding) while every row's scale stays within [2^-10, 2^3] of it, otherwise
 * P * scale in fp32 rounded to bf16 (the split is recomputed); fp32 accumulation; bf16 outputs. Intermediate sums
 * are fp32: finite results need |q . v| and |v| well inside the fp32 range (|v| < 2^90).
 * Entries that are -1 (or above p) never reach the output, whatever their placeholder row holds
 * (NaN codes or scales included).
 * _prefill runs one workgroup per query token; _decode also splits each token's rows across
 * workgroups and merges the partials by log-sum-exp (for few query tokens).
 */
int smla_sparse_mla_prefill(const smla_batch* b, const void* q, const void* kv, int32_t kv_format,
                            int32_t H, int32_t D_qk, int32_t D_v, const int32_t* idx,
                            int32_t top_k, float sm_scale, void* out, float* lse, void* ws,
                            size_t ws_bytes, void* stream);
int smla_sparse_mla_decode(const smla_batch* b, const void* q, const void* kv, int32_t kv_format,
                           int32_t H, int32_t D_qk, int32_t D_v, const int32_t* idx,
                           int32_t top_k, float sm_scale, void* out, float* lse, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * smla_sparse_mla_decode without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, results and errors are those of smla_sparse_mla_decode. The split partials live in
 * a scratch array built into the library: 512 (token, split) pairs, 33,685,504 bytes per GPU,
 * held from the first call on that GPU until the process ends. The split rule needs at most 510
 * pairs for the FP8_656 shape (and none from 256 query tokens up); a call whose partials would
 * not fit fails with SMLA_E_UNSUPPORTED. BF16 rows need no scratch. Allocates nothing.
 * Every call on one GPU shares that GPU's scratch: calls whose executions overlap on one GPU
 * (different streams, or threads without ordering) race and give wrong results; calls ordered
 * on one stream are safe. The scratch needs no clearing: each call writes the partials it reads.
 */
int smla_sparse_mla_decode_noalloc(const smla_batch* b, const void* q, const void* kv,
                                   int32_t kv_format, int32_t H, int32_t D_qk, int32_t D_v,
                                   const int32_t* idx, int32_t top_k, float sm_scale, void* out,
                                   float* lse, void* stream);

/*
 * New tokens into the caches (the step before scoring and attention in each decode or prefill
 * chunk): token i's latent row becomes row rows[i] of the FP8_656 latent cache, and its indexer
 * key row rows[i] of the key cache. The pages size the latent row at 656 bytes (FlashMLA's
 * fp8_ds_mla format; "Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why the numbers
 * work") and count those 656 bytes per token and layer in their cache budget.
 * latent (device) [n, 576] bf16: 512 value dims, then 64 rope dims.
 * rows (device) [n] int64: destination rows (distinct; the caller keeps them inside the caches).
 * kv (device) [R, 656] bytes: row r receives 512 E4M3 codes, 4 fp32 block scales (little-endian,
 *   value dims 128b..128b+127) and the 64 rope dims as given. Block scale = fp32(amax_b / 448)
 *   (1 for an all-zero block); code = E4M3(value / scale) with the quotient in fp64, rounded to
 *   nearest-even, saturated at 448. Values must be finite.
 * k_new (device, optional) [n, D_I] int8 and k_idx (device) [R, D_I] int8: key i is copied to row
 *   rows[i] of k_idx; D_I a multiple of 16, at most 1024.
 * n = 0 is a no-op. Alignment: latent, kv, k_new, k_idx 16 bytes; rows 8 bytes. Asynchronous on
 * `stream`; the caller owns every buffer.
 */
int smla_kv_append(int64_t n, const void* latent, const int8_t* k_new, int32_t D_I,
                   const int64_t* rows, void* kv, int8_t* k_idx, void* stream);

/*
 * Optional per-stage timing for benchmarks and profilers: while set, the GPU entry points record
 * begin[s] before and end[s] after the launches of stage s on the call's stream, for
 * s = 0 indexer scores, 1 top-k select, 2 sparse MLA, 3 split-KV combine (decode only).
 * begin/end (host arrays of n hipEvent_t, caller-owned; entries may be NULL) are read at each
 * call; pass n = 0 to stop. Process-wide setting: set it only while no other thread calls the
 * library.
 */
int smla_set_stage_events(void* const* begin, void* const* end, int32_t n);

/* Status name and the calling thread's last error message ("" if none). */
const char* smla_status_str(int status);
const char* smla_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t smla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SMLA_H */
