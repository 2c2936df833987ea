/*
 * pkv_oracle.h - plain, slow, CPU reference of the paged-KV decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This oracle exists to check the GPU library;
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header, table or helper with the GPU
 * path and never calls it.
 *
 * Conventions: bf16 values are passed as uint16 bit patterns; all caches
 * use the paged layout [num_blocks][block_size][num_kv_heads][head_dim]
 * (one layer's K or V pool, the per-layer view of the nano-vllm pool on its
 * "allocated kv cache" page).  Floating-point attention is done in fp64.
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of one physical block over all layers, K and V together
 * (nano-vllm "Model Runner" page, section "allocated kv cache"). */
int64_t oracle_block_bytes(int64_t num_layers, int64_t block_size,
                           int64_t num_kv_heads, int64_t head_dim,
                           int64_t itemsize);

/* Flat slot of logical position pos in one row's block table
 * (same page, the worked "token position 299" example): returns -1 if the
 * position's logical block is outside the table or the entry is negative. */
int64_t oracle_slot_for_position(const int32_t *block_table_row,
                                 int64_t table_len, int64_t pos,
                                 int64_t block_size);

/* Decode-step slot mapping: row b's new token sits at position n_b - 1
 * (nano-vllm page, section "prefill and decode"); n_b <= 0 gives -1. */
void oracle_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                         int64_t table_stride, const int32_t *context_lens,
                         int64_t batch, int64_t block_size);

/* Copy each token's K/V head rows (bit patterns) into the pools at its
 * slot; negative slots are skipped.  Returns 0, or -1 if a slot is beyond
 * the pool (nothing is written for that token then). */
int oracle_kv_store(uint16_t *k_cache, uint16_t *v_cache,
                    const uint16_t *k_new, const uint16_t *v_new,
                    const int32_t *slot_mapping, int64_t num_tokens,
                    int64_t num_kv_heads, int64_t head_dim,
                    int64_t block_size, int64_t num_blocks);

/* Single-query attention of one query head over positions 0..n-1 of one
 * row, gathering K/V rows through the block table; fp64 two-pass softmax.
 * n <= 0 gives the zero vector.  Returns 0, or -1 on a block id outside
 * [0, num_blocks). */
int oracle_decode_attention_head(double *out, const uint16_t *q_head,
                                 const uint16_t *k_cache,
                                 const uint16_t *v_cache,
                                 const int32_t *block_table_row,
                                 int64_t context_len, int64_t num_kv_heads,
                                 int64_t kv_head, int64_t head_dim,
                                 int64_t block_size, int64_t num_blocks,
                                 double scale);

/* All rows and query heads: out fp64 [batch][num_q_heads][head_dim].
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * scale <= 0 selects 1/sqrt(head_dim). */
int oracle_decode_attention(double *out, const uint16_t *q,
                            const uint16_t *k_cache, const uint16_t *v_cache,
                            const int32_t *block_tables, int64_t table_stride,
                            const int32_t *context_lens, int64_t batch,
                            int64_t num_q_heads, int64_t num_kv_heads,
                            int64_t head_dim, int64_t block_size,
                            int64_t num_blocks, double scale);

/* Attention over a contiguous cache [batch][max_len][num_kv_heads][head_dim]
 * (the nanochat (B, T, H, D) layout), for the paged == contiguous pin. */
int oracle_contiguous_attention(double *out, const uint16_t *q,
                                const uint16_t *k, const uint16_t *v,
                                const int32_t *context_lens, int64_t batch,
                                int64_t max_len, int64_t num_q_heads,
                                int64_t num_kv_heads, int64_t head_dim,
                                double scale);

/* Varlen multi-query paged attention (nano-vllm page, "prefix cache" and
 * "prefill and decode": a chunk of new tokens per sequence attends, with a
 * causal mask, to the sequence's cached tokens and to the new tokens up to
 * itself).  Sequence i has q_len = cu_seqlens_q[i+1] - cu_seqlens_q[i] new
 * tokens (rows cu_seqlens_q[i] .. of q and out) and k_len = cu_seqlens_k[i+1]
 * - cu_seqlens_k[i] >= q_len tokens in the cache (its block table covers
 * them; the new tokens' K/V are already stored).  New token j sits at
 * position k_len - q_len + j and attends to positions [0, k_len - q_len + j].
 * q uint16 (bf16 bits) [total_q][Hq][D]; out fp64 [total_q][Hq][D].
 * Returns 0, or -1 for a block id out of range or a bad length. */
int oracle_varlen_attention(double *out, const uint16_t *q,
                            const uint16_t *k_cache, const uint16_t *v_cache,
                            const int32_t *block_tables, int64_t table_stride,
                            const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int64_t batch,
                            int64_t num_q_heads, int64_t num_kv_heads,
                            int64_t head_dim, int64_t block_size,
                            int64_t num_blocks, double scale);

/* Slots of the new tokens of a varlen batch: token j of sequence i is at
 * position k_len - q_len + j of its block table (-1 where the table entry
 * is negative or the position is past the table). */
void oracle_varlen_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                                int64_t table_stride, const int32_t *cu_seqlens_q,
                                const int32_t *cu_seqlens_k, int64_t batch,
                                int64_t block_size);

/* Per-row sampler diagnostics. */
typedef struct {
    int32_t id;          /* sampled token id */
    int32_t greedy;      /* 1 if temperature <= 0 (argmax of raw logits) */
    int32_t kept;        /* size of the eligible set after top-k / top-p */
    int32_t topp_applied;/* 1 if the nucleus filter ran */
    float tau;           /* nucleus threshold on scaled logits (if applied) */
    float kth;           /* k-th largest scaled logit (if top-k applied) */
    double margin;       /* distance of 1-p from the nearest cumulative-mass
                            boundary around tau (normalised mass units);
                            0 when the cut had no crossing; +inf for
                            p <= 0 (the maxima: no mass is compared) */
} oracle_sample_info;

/* Next-token sampler for one row, in the Grok-1 runner's order
 * (chapter 8, section 8.3 and 8.3.1): scale by 1/T, top-k, nucleus cut,
 * then a Gumbel-max draw in logit space with the caller's noise.  Ties
 * resolve to the lowest index.  Returns the id (also stored in info). */
int32_t oracle_sample_row(const float *logits, const float *gumbel,
                          int64_t vocab, float temperature, float top_p,
                          int32_t top_k, oracle_sample_info *info);

/* The runner's extra sampler outputs (Grok-1 runner chapter, section 8.3:
 * the probability of the drawn token under the filtered distribution, and
 * the top-8 (TOP_K = 8) ids and probabilities for debugging). */
typedef struct {
    double chosen_prob;  /* softmax of the kept scaled logits at the drawn id */
    int32_t top_ids[8];  /* kept ids by (scaled logit desc, index asc), then
                            the lowest-index ids outside the kept set */
    double top_probs[8]; /* their probabilities (0 outside the kept set) */
} oracle_sample_extras;

/* oracle_sample_row with the vocabulary mask of section 8.3 (mask[i] == 0:
 * the scaled logit is replaced by -1e10 before the filters; NULL: no mask)
 * and, when extras is non-NULL, the extra outputs.  A non-positive
 * temperature is the greedy limit: the drawn id is the lowest index of the
 * largest masked raw logit, and the distribution is uniform over the tied
 * largest values. */
int32_t oracle_sample_row_ex(const float *logits, const float *gumbel,
                             const unsigned char *mask, int64_t vocab,
                             float temperature, float top_p, int32_t top_k,
                             oracle_sample_info *info,
                             oracle_sample_extras *extras);

void oracle_sample(int32_t *ids, oracle_sample_info *infos,
                   const float *logits, int64_t logits_stride,
                   const float *gumbel, int64_t gumbel_stride,
                   const float *temperature, const float *top_p,
                   const int32_t *top_k, int64_t batch, int64_t vocab);

#ifdef __cplusplus
}
#endif
#endif
