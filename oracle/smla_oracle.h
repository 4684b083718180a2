/*
 * smla_oracle.h — CPU oracle for the indexer -> top-k -> sparse-MLA path.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests, the package's smoke check and the benchmark's CPU
 * baseline may load this library. It shares no code with the GPU library.
 *
 * Plain, slow, obviously correct definitions:
 *  - Indexer score of query token t (at position p) against earlier token s <= p:
 *      score(t, s) = sum_h w_h * max(0, sum_d q_I[t,h,d] * k_I[s,d])   (int64, exact)
 *    The pages: an indexer scores every earlier token for every query to choose the 2,048 tokens
 *    sparse MLA attends ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why DP8 and
 *    TP8 fall short"); the formula itself is the workload definition of the tiny causal prefill.
 *  - Top-k: the min(k, p+1) tokens with the largest scores; ties go to the lower index; every
 *    s <= p is taken when p+1 <= k. Implemented as a sort by (score desc, s asc).
 *  - Sparse MLA (MQA form: all heads read the same selected latent rows; QK over 576 dims, PV
 *    over the first 512; section "Why the numbers work"): for each head h,
 *      l_i = sm_scale * sum_{d<D_qk} q[h,d] v_i[d],  m = max_i l_i,  e_i = exp(l_i - m),
 *      Z = sum_i e_i,  o[h,d] = sum_i (e_i / Z) v_i[d] for d < D_v,  lse[h] = m + log Z
 *    in fp64 over the dequantised rows.
 *  - Row dequantisation: bf16 rows decode exactly; 656-byte rows decode
 *      v[d] = e4m3(code[d]) * scale[d / 128] for d < 512 and v[d] = bf16(rope[d - 512]) otherwise.
 *  - Row encoding (appending a token to the cache), the inverse: a token's 576 bf16 latent values
 *    become its 656-byte row (the pages size the FP8 latent row at 656 bytes, in FlashMLA's
 *    fp8_ds_mla format: "Why the numbers work"; their per-token cache budget counts the same 656
 *    bytes per layer). For each 128-dim block b of the 512 value dims,
 *      scale_b = binary32(amax_b / 448)   (1 when the block is all zero)
 *      code_d  = E4M3(v_d / scale_b)      quotient in binary64, rounded to nearest-even,
 *                                         saturating at 448 (OCP E4M3FN has no infinity)
 *    then the four scales (little-endian binary32) and the 64 rope dims as stored.
 */
#ifndef SMLA_ORACLE_H
#define SMLA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OCP E4M3 ("FN") code -> value; NaN for S.1111.111. */
double smla_oracle_e4m3(uint8_t code);
/* bfloat16 bit pattern -> value. */
double smla_oracle_bf16(uint16_t bits);
/* Value -> OCP E4M3 ("FN") code, round to nearest-even on 3 mantissa bits (subnormals are
 * multiples of 2^-9), |v| >= 448 saturating to +-448; the sign of a zero is kept. */
uint8_t smla_oracle_e4m3_encode(double v);
/* One token's latent row (576 bf16 bit patterns: 512 value dims, then 64 rope dims) -> its
 * 656-byte FP8 row (layout above). */
int smla_oracle_fp8_row_encode(const uint16_t* latent, uint8_t* row);
/* Dequantise one latent row of `fmt` (0 bf16, 1 fp8-656) into D_qk doubles. */
int smla_oracle_dequant_row(const uint8_t* row, int32_t fmt, int32_t D_qk, double* out);

/* Scores of one query token (q_tok [H_I, D_I]) against keys [n, D_I]; out [n] int64.
 * Returns -1 when a score leaves [0, 2^31 - 1]. */
int smla_oracle_indexer_scores(const int8_t* q_tok, const int8_t* keys, const int32_t* w,
                               int32_t H_I, int32_t D_I, int64_t n, int64_t* out);

/* FP8 indexer keys (the pages' deployed key: 128 E4M3 values and one binary32 scale per token,
 * 132 bytes; "Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why the numbers work").
 * Scores of one query token (q_tok [H_I, D_I] E4M3 codes) against keys [n, D_I] (E4M3 codes)
 * with per-key scales k_scale [n] and per-head weights w [H_I] (binary32, >= 0):
 *   score(s) = k_scale[s] * sum_h w[h] * max(0, sum_d e4m3(q[h,d]) * e4m3(k[s,d]))
 * in binary64, where every dot product is exact. out [n]; abs_out [n] (optional) receives
 * k_scale[s] * sum_h w[h] * sum_d |e4m3(q[h,d]) * e4m3(k[s,d])|, the magnitude against which a
 * differently ordered or narrower accumulation is judged. Returns -1 on a NaN code or on a
 * weight or scale that is negative or not finite. */
int smla_oracle_indexer_scores_fp8(const uint8_t* q_tok, const uint8_t* keys, const float* k_scale,
                                   const float* w, int32_t H_I, int32_t D_I, int64_t n,
                                   double* out, double* abs_out);

/* Exact top-k of scores[0..n) by (score desc, index asc). idx/score [top_k], in that order;
 * slots past min(n, top_k) hold idx -1 and score -1. */
int smla_oracle_topk(const int64_t* scores, int64_t n, int32_t top_k, int32_t* idx,
                     int32_t* score);

/* DCP merges (the pages shard the KV cache round-robin, every n-th token to one GPU, and merge
 * what the shards compute: "Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "DCP").
 * Top-k merge of one query token: n_lists per-shard lists (idx_lists/score_lists
 * [n_lists][k_in], local indices, -1 padding), shard l holding the tokens l, l + n_lists, ...:
 * the top_k of the union by (score desc, global index asc), global = local * n_lists + l. The
 * result is in that order, -1 padded (as smla_oracle_topk). */
int smla_oracle_topk_merge(const int32_t* idx_lists, const int32_t* score_lists, int32_t n_lists,
                           int32_t k_in, int32_t top_k, int32_t* idx, int32_t* score);
/* LSE merge of n_parts partial attention results over disjoint row sets: outs [n][H][D_v],
 * lses [n][H] (natural log; -inf for a part with no row). m = max lse; w_i = exp(lse_i - m);
 * out = sum w_i out_i / sum w_i; lse = m + log sum w_i (-inf and a zero output when no part saw
 * a row). */
int smla_oracle_lse_merge(int32_t n_parts, int32_t H, int32_t D_v, const double* outs,
                          const double* lses, double* out, double* lse);

/* Hot-buffer resolve of one request (the pages' hybrid offload keeps the rows the indexer
 * selects in a GPU hot buffer with LRU replacement; a miss copies one row from pinned host
 * memory into an LRU slot: "vLLM GLM 5.3 ... Hybrid HiSparse", technical implementation).
 * idx [n_q, top_k]: the request's selections (local rows, -1 padding). Rows >= resident_from are
 * resident and read in place; the others must sit in the hot buffer of H slots, hot_tok[H]
 * (token or -1) and hot_age[H] (step of last use, -1 never), updated in place:
 *  - U = the distinct offloaded selections, ascending;
 *  - a token of U already in a slot is a hit: that slot's age becomes `step`;
 *  - the misses, ascending, take the slots not hit in this call in (age, slot) ascending order
 *    (least recently used first, ties to the lower slot); each gets the token and age `step`,
 *    and its row is to be copied from host memory (copy_src: pairs (token, slot), n_copy of them);
 *  - idx_out: -1 stays -1, a resident row stays, an offloaded row becomes hot_base + its slot.
 * Returns -2, with nothing changed, when the distinct offloaded rows outnumber the H slots.
 * kv_len >= 0 (the request's rows, its n_q query tokens last) also bounds the request: the
 * first token sits at position kv_len - n_q and attends only to rows up to it, so the offloaded
 * prefix must end there (resident_from <= kv_len - n_q + 1) and the hot buffer must lie inside
 * it (0 <= hot_base, hot_base + H <= resident_from); otherwise -3, nothing changed. kv_len < 0
 * skips these bounds (a request whose length is not given). */
int smla_oracle_hot_resolve(int32_t n_q, int32_t top_k, const int32_t* idx, int64_t kv_len,
                            int64_t resident_from, int32_t H, int32_t* hot_tok, int32_t* hot_age,
                            int32_t step, int64_t hot_base, int32_t* idx_out, int32_t* copy_src,
                            int32_t* n_copy);

/* Attention of one query token q_tok [H, D_qk] (bf16 bits) over rows[idx[i]] (row_bytes each),
 * skipping idx < 0; out [H, D_v], lse [H] (either may be NULL). Returns -1 if no row is valid. */
int smla_oracle_attend(const uint16_t* q_tok, const uint8_t* rows, int32_t fmt, int32_t row_bytes,
                       int32_t H, int32_t D_qk, int32_t D_v, const int32_t* idx, int32_t top_k,
                       double sm_scale, double* out, double* lse);

/*
 * Batched drivers over a list of query tokens, `nthreads` worker threads (<= 0: all cores).
 * Batch layout: request b owns query tokens [Q_b, Q_b + n_q[b]) and rows [R_b, R_b + kv_len[b])
 * with Q_b, R_b exclusive prefix sums of n_q and kv_len; its query j sits at position
 * p = kv_len[b] - n_q[b] + j and sees rows s <= p (s is local to the request).
 * Outputs are packed per listed token: idx_out/score_out [n_tokens, top_k],
 * out [n_tokens, H, D_v], lse [n_tokens, H]. `idx` for sparse MLA is [total_q, top_k] indexed by
 * the global token id.
 */
int smla_oracle_indexer_topk_batch(int32_t batch, const int32_t* n_q, const int64_t* kv_len,
                                   const int8_t* q_idx, const int8_t* k_idx, const int32_t* w,
                                   int32_t H_I, int32_t D_I, int32_t top_k, const int64_t* tokens,
                                   int64_t n_tokens, int32_t* idx_out, int32_t* score_out,
                                   int32_t nthreads);

int smla_oracle_sparse_mla_batch(int32_t batch, const int32_t* n_q, const int64_t* kv_len,
                                 const uint16_t* q, const uint8_t* kv, int32_t fmt,
                                 int32_t row_bytes, int32_t H, int32_t D_qk, int32_t D_v,
                                 const int32_t* idx, int32_t top_k, double sm_scale,
                                 const int64_t* tokens, int64_t n_tokens, double* out, double* lse,
                                 int32_t nthreads);

/* Worker threads used for nthreads <= 0. */
int32_t smla_oracle_default_threads(void);

#ifdef __cplusplus
}
#endif
#endif
