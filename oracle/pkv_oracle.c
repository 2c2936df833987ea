/*
 * pkv_oracle.c - plain, slow CPU reference of the paged-KV decode step.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the library.  Shares nothing with
 * the GPU path.  Built with -ffp-contract=off and without fast-math so that
 * every fp32 operation below is one IEEE-754 round-to-nearest-even step.
 *
 * Sources (web pages this follows; sections named per function):
 *   [grok]  "第 8 章 runners.py 推理引擎" (Grok-1 runners chapter)
 *   [nchat] "04 · Engine 推理与工具调用" (nanochat engine)
 *   [nvllm] "Model Runner" (nano-vllm model runner)
 */
#include "pkv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- bf16 ---------------------------------------------------------------- */

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- pool sizing and slots ([nvllm] "allocated kv cache") ---------------- */

int64_t oracle_block_bytes(int64_t num_layers, int64_t block_size,
                           int64_t num_kv_heads, int64_t head_dim,
                           int64_t itemsize)
{
    /* one block holds block_size tokens of K and of V in every layer */
    return 2 * num_layers * block_size * num_kv_heads * head_dim * itemsize;
}

int64_t oracle_slot_for_position(const int32_t *block_table_row,
                                 int64_t table_len, int64_t pos,
                                 int64_t block_size)
{
    if (pos < 0 || block_size <= 0)
        return -1;
    int64_t logical = pos / block_size;   /* which entry of the table */
    int64_t offset = pos % block_size;    /* token within the block */
    if (logical >= table_len)
        return -1;
    int64_t physical = block_table_row[logical];
    if (physical < 0)
        return -1;
    return physical * block_size + offset;
}

/* [nvllm] "prefill and decode": a decode step starts with n tokens, n-1 of
 * them cached; the new one is written at position n-1 and attention then
 * covers all n.  context_lens holds n. */
void oracle_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                         int64_t table_stride, const int32_t *context_lens,
                         int64_t batch, int64_t block_size)
{
    for (int64_t b = 0; b < batch; ++b) {
        int64_t n = context_lens[b];
        int64_t slot = -1;
        if (n > 0)
            slot = oracle_slot_for_position(block_tables + b * table_stride,
                                            table_stride, n - 1, block_size);
        slot_mapping[b] = (int32_t)slot;
    }
}

/* ---- KV store ([nvllm] "prepare Prefill"; [nchat] section 2) ------------- */

int oracle_kv_store(uint16_t *k_cache, uint16_t *v_cache,
                    const uint16_t *k_new, const uint16_t *v_new,
                    const int32_t *slot_mapping, int64_t num_tokens,
                    int64_t num_kv_heads, int64_t head_dim,
                    int64_t block_size, int64_t num_blocks)
{
    int rc = 0;
    int64_t row = num_kv_heads * head_dim;   /* elements per token */
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0)
            continue;
        if (slot >= num_blocks * block_size) {
            rc = -1;
            continue;
        }
        /* slot = block * block_size + offset, and the pool is laid out
         * [block][offset][head][dim], so the token row starts at slot*row */
        memcpy(k_cache + slot * row, k_new + t * row, (size_t)row * 2);
        memcpy(v_cache + slot * row, v_new + t * row, (size_t)row * 2);
    }
    return rc;
}

/* ---- attention ------------------------------------------------------------
 * [grok] 8.2.3: a decode step feeds one token whose query attends over all
 * cached K/V of its row; an inactive row (step 0) attends over nothing and
 * yields the zero vector.  [grok] 8.5: 48 query heads share 8 KV heads.
 * Plain definition: o = sum_j softmax_j(scale * q.k_j) v_j, computed here
 * as a straight two-pass softmax in fp64. */

static double dot_bf16(const uint16_t *a, const uint16_t *b, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += bf16_to_double(a[i]) * bf16_to_double(b[i]);
    return s;
}

static int attend_rows(double *out, const uint16_t *q_head,
                       const uint16_t *const *k_rows,
                       const uint16_t *const *v_rows, int64_t n,
                       int64_t head_dim, double scale)
{
    for (int64_t d = 0; d < head_dim; ++d)
        out[d] = 0.0;
    if (n <= 0)
        return 0;
    double *s = (double *)malloc((size_t)n * sizeof(double));
    if (!s)
        return -2;
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = scale * dot_bf16(q_head, k_rows[j], head_dim);
        if (s[j] > m)
            m = s[j];
    }
    double denom = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = exp(s[j] - m);
        denom += w;
        for (int64_t d = 0; d < head_dim; ++d)
            out[d] += w * bf16_to_double(v_rows[j][d]);
    }
    for (int64_t d = 0; d < head_dim; ++d)
        out[d] /= denom;
    free(s);
    return 0;
}

int oracle_decode_attention_head(double *out, const uint16_t *q_head,
                                 const uint16_t *k_cache,
                                 const uint16_t *v_cache,
                                 const int32_t *block_table_row,
                                 int64_t context_len, int64_t num_kv_heads,
                                 int64_t kv_head, int64_t head_dim,
                                 int64_t block_size, int64_t num_blocks,
                                 double scale)
{
    int64_t n = context_len > 0 ? context_len : 0;
    const uint16_t **kr = (const uint16_t **)malloc((size_t)(n + 1) * sizeof(*kr));
    const uint16_t **vr = (const uint16_t **)malloc((size_t)(n + 1) * sizeof(*vr));
    if (!kr || !vr) {
        free(kr);
        free(vr);
        return -2;
    }
    int rc = 0;
    for (int64_t j = 0; j < n; ++j) {
        /* position j lives in logical block j / block_size at offset
         * j % block_size ([nvllm] "allocated kv cache") */
        int64_t phys = block_table_row[j / block_size];
        if (phys < 0 || phys >= num_blocks) {
            rc = -1;
            break;
        }
        int64_t slot = phys * block_size + j % block_size;
        int64_t off = (slot * num_kv_heads + kv_head) * head_dim;
        kr[j] = k_cache + off;
        vr[j] = v_cache + off;
    }
    if (rc == 0)
        rc = attend_rows(out, q_head, kr, vr, n, head_dim, scale);
    free(kr);
    free(vr);
    return rc;
}

int oracle_decode_attention(double *out, const uint16_t *q,
                            const uint16_t *k_cache, const uint16_t *v_cache,
                            const int32_t *block_tables, int64_t table_stride,
                            const int32_t *context_lens, int64_t batch,
                            int64_t num_q_heads, int64_t num_kv_heads,
                            int64_t head_dim, int64_t block_size,
                            int64_t num_blocks, double scale)
{
    if (scale <= 0.0)
        scale = 1.0 / sqrt((double)head_dim);
    int64_t group = num_q_heads / num_kv_heads;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < num_q_heads; ++h) {
            int rc = oracle_decode_attention_head(
                out + (b * num_q_heads + h) * head_dim,
                q + (b * num_q_heads + h) * head_dim, k_cache, v_cache,
                block_tables + b * table_stride, context_lens[b],
                num_kv_heads, h / group, head_dim, block_size, num_blocks,
                scale);
            if (rc)
                return rc;
        }
    return 0;
}

int oracle_varlen_attention(double *out, const uint16_t *q,
                            const uint16_t *k_cache, const uint16_t *v_cache,
                            const int32_t *block_tables, int64_t table_stride,
                            const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int64_t batch,
                            int64_t num_q_heads, int64_t num_kv_heads,
                            int64_t head_dim, int64_t block_size,
                            int64_t num_blocks, double scale)
{
    if (scale <= 0.0)
        scale = 1.0 / sqrt((double)head_dim);
    int64_t group = num_q_heads / num_kv_heads;
    for (int64_t b = 0; b < batch; ++b) {
        int64_t q_len = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        int64_t k_len = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
        if (q_len < 0 || k_len < q_len)
            return -1;
        int64_t cached = k_len - q_len;
        for (int64_t j = 0; j < q_len; ++j) {
            int64_t row = cu_seqlens_q[b] + j;
            for (int64_t h = 0; h < num_q_heads; ++h) {
                /* causal: new token j sees every position up to its own */
                int rc = oracle_decode_attention_head(
                    out + (row * num_q_heads + h) * head_dim,
                    q + (row * num_q_heads + h) * head_dim, k_cache, v_cache,
                    block_tables + b * table_stride, cached + j + 1, num_kv_heads,
                    h / group, head_dim, block_size, num_blocks, scale);
                if (rc)
                    return rc;
            }
        }
    }
    return 0;
}

void oracle_varlen_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                                int64_t table_stride, const int32_t *cu_seqlens_q,
                                const int32_t *cu_seqlens_k, int64_t batch,
                                int64_t block_size)
{
    for (int64_t b = 0; b < batch; ++b) {
        int64_t q_len = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        int64_t k_len = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
        for (int64_t j = 0; j < q_len; ++j)
            slot_mapping[cu_seqlens_q[b] + j] = (int32_t)oracle_slot_for_position(
                block_tables + b * table_stride, table_stride, k_len - q_len + j, block_size);
    }
}

int oracle_contiguous_attention(double *out, const uint16_t *q,
                                const uint16_t *k, const uint16_t *v,
                                const int32_t *context_lens, int64_t batch,
                                int64_t max_len, int64_t num_q_heads,
                                int64_t num_kv_heads, int64_t head_dim,
                                double scale)
{
    if (scale <= 0.0)
        scale = 1.0 / sqrt((double)head_dim);
    int64_t group = num_q_heads / num_kv_heads;
    const uint16_t **kr = (const uint16_t **)malloc((size_t)(max_len + 1) * sizeof(*kr));
    const uint16_t **vr = (const uint16_t **)malloc((size_t)(max_len + 1) * sizeof(*vr));
    if (!kr || !vr) {
        free(kr);
        free(vr);
        return -2;
    }
    int rc = 0;
    for (int64_t b = 0; b < batch && rc == 0; ++b) {
        int64_t n = context_lens[b] < max_len ? context_lens[b] : max_len;
        for (int64_t h = 0; h < num_q_heads && rc == 0; ++h) {
            int64_t g = h / group;
            for (int64_t j = 0; j < n; ++j) {
                int64_t off = ((b * max_len + j) * num_kv_heads + g) * head_dim;
                kr[j] = k + off;
                vr[j] = v + off;
            }
            rc = attend_rows(out + (b * num_q_heads + h) * head_dim,
                             q + (b * num_q_heads + h) * head_dim, kr, vr, n,
                             head_dim, scale);
        }
    }
    free(kr);
    free(vr);
    return rc;
}

/* ---- sampler --------------------------------------------------------------
 * [grok] 8.3 sample_token: logits / T, then the nucleus filter, then a
 * categorical draw; 8.3.1.1: temperature is applied before the filter.
 * [nchat] section 3: top-k keeps the k largest before sampling.
 * [nvllm] "run model": divide by T, softmax, Gumbel-max picks the id.
 * The categorical draw is done as argmax(s_i + g_i) over the eligible set
 * with the caller's Gumbel noise g (same law as sampling softmax(s)). */

typedef struct {
    float v;
    int64_t i;
} val_idx;

/* larger value first; equal values by lower index first */
static int cmp_desc_value_asc_index(const void *pa, const void *pb)
{
    const val_idx *a = (const val_idx *)pa, *b = (const val_idx *)pb;
    if (a->v > b->v)
        return -1;
    if (a->v < b->v)
        return 1;
    return (a->i > b->i) - (a->i < b->i);
}

static int cmp_float_asc(const void *pa, const void *pb)
{
    float a = *(const float *)pa, b = *(const float *)pb;
    return (a > b) - (a < b);
}

/* Fills extras for the greedy limit: uniform over the tied maxima of v. */
static void greedy_extras(const float *v, int64_t vocab, float vmax, int64_t id,
                          oracle_sample_extras *x)
{
    int64_t ties = 0;
    for (int64_t i = 0; i < vocab; ++i)
        if (v[i] == vmax)
            ++ties;
    x->chosen_prob = 1.0 / (double)ties;
    (void)id;
    int r = 0;
    for (int64_t i = 0; i < vocab && r < 8; ++i)
        if (v[i] == vmax) {
            x->top_ids[r] = (int32_t)i;
            x->top_probs[r++] = 1.0 / (double)ties;
        }
    for (int64_t i = 0; i < vocab && r < 8; ++i)
        if (v[i] != vmax) {
            x->top_ids[r] = (int32_t)i;
            x->top_probs[r++] = 0.0;
        }
    for (; r < 8; ++r) {
        x->top_ids[r] = -1;
        x->top_probs[r] = 0.0;
    }
}

int32_t oracle_sample_row_ex(const float *logits, const float *gumbel,
                             const unsigned char *mask, int64_t vocab,
                             float temperature, float top_p, int32_t top_k,
                             oracle_sample_info *info, oracle_sample_extras *extras)
{
    oracle_sample_info local;
    if (!info)
        info = &local;
    memset(info, 0, sizeof *info);
    if (extras)
        memset(extras, 0, sizeof *extras);
    const float masked = -1e10f;   /* the runner's value for forbidden tokens */

    /* T = 0 is the greedy limit of temperature sampling ([grok] 8.1.1,
     * 8.3); a non-positive temperature is read as that limit.  The mask
     * still applies: forbidden tokens count as -1e10. */
    if (!(temperature > 0.0f)) {
        float *v = (float *)malloc((size_t)vocab * sizeof(float));
        if (!v) {
            info->id = -1;
            return -1;
        }
        for (int64_t i = 0; i < vocab; ++i)
            v[i] = (mask && !mask[i]) ? masked : logits[i];
        int64_t best = 0;
        for (int64_t i = 1; i < vocab; ++i)
            if (v[i] > v[best])
                best = i;
        info->id = (int32_t)best;
        info->greedy = 1;
        info->kept = 1;
        if (extras)
            greedy_extras(v, vocab, v[best], best, extras);
        free(v);
        return info->id;
    }

    float *s = (float *)malloc((size_t)vocab * sizeof(float));
    unsigned char *keep = (unsigned char *)malloc((size_t)vocab);
    val_idx *order = (val_idx *)malloc((size_t)vocab * sizeof(val_idx));
    float *asc = (float *)malloc((size_t)vocab * sizeof(float));
    double *cum = (double *)malloc((size_t)vocab * sizeof(double));
    if (!s || !keep || !order || !asc || !cum) {
        free(s); free(keep); free(order); free(asc); free(cum);
        info->id = -1;
        return -1;
    }

    /* 1. temperature: one IEEE fp32 division per logit; then the mask:
     * forbidden tokens get -1e10 (section 8.3, in that order) */
    for (int64_t i = 0; i < vocab; ++i) {
        s[i] = logits[i] / temperature;
        if (mask && !mask[i])
            s[i] = masked;
        keep[i] = 1;
    }

    /* 2. top-k: keep exactly k, ordered by value then index */
    if (top_k > 0 && top_k < vocab) {
        for (int64_t i = 0; i < vocab; ++i) {
            order[i].v = s[i];
            order[i].i = i;
        }
        qsort(order, (size_t)vocab, sizeof *order, cmp_desc_value_asc_index);
        memset(keep, 0, (size_t)vocab);
        for (int64_t r = 0; r < top_k; ++r)
            keep[order[r].i] = 1;
        info->kth = order[top_k - 1].v;
    }

    /* 3. nucleus ([grok] 8.3.1 top_p_filter): sort the eligible logits
     * ascending, softmax them, take the first position whose running sum
     * reaches 1 - p, and keep every logit >= the logit there. */
    if (top_p < 1.0f) {
        int64_t n = 0;
        for (int64_t i = 0; i < vocab; ++i)
            if (keep[i])
                asc[n++] = s[i];
        qsort(asc, (size_t)n, sizeof(float), cmp_float_asc);
        float tau;
        double margin = 0.0;
        if (!(top_p > 0.0f)) {
            /* p <= 0: only the maxima stay eligible; no mass is compared,
             * so no rounding can move the cut */
            tau = asc[n - 1];
            margin = INFINITY;
        } else {
            double mx = asc[n - 1];
            double z = 0.0;
            for (int64_t j = 0; j < n; ++j)
                z += exp((double)asc[j] - mx);
            double run = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                run += exp((double)asc[j] - mx) / z;
                cum[j] = run;
            }
            double target = 1.0 - (double)top_p;
            int64_t at = -1;
            for (int64_t j = 0; j < n; ++j)
                if (cum[j] >= target) {
                    at = j;
                    break;
                }
            if (at < 0) {
                /* rounding left the total below 1 - p: only a p so small
                 * that the exact rule keeps just the maxima */
                at = n - 1;
                margin = 0.0;
                tau = asc[at];
            } else {
                tau = asc[at];
                /* mass boundaries of tau's group of equal values */
                int64_t lo = at, hi = at;
                while (lo > 0 && asc[lo - 1] == tau)
                    --lo;
                while (hi + 1 < n && asc[hi + 1] == tau)
                    ++hi;
                double below = lo > 0 ? cum[lo - 1] : 0.0;
                double through = cum[hi];
                double m1 = target - below, m2 = through - target;
                margin = m1 < m2 ? m1 : m2;
            }
        }
        for (int64_t i = 0; i < vocab; ++i)
            if (keep[i] && !(s[i] >= tau))
                keep[i] = 0;
        info->topp_applied = 1;
        info->tau = tau;
        info->margin = margin;
    }

    /* 4. Gumbel-max over the eligible set: key = fl32(s + g) */
    int64_t best = -1;
    float best_key = 0.0f;
    int32_t kept = 0;
    for (int64_t i = 0; i < vocab; ++i) {
        if (!keep[i])
            continue;
        ++kept;
        float key = s[i] + gumbel[i];
        if (best < 0 || key > best_key) {
            best = i;
            best_key = key;
        }
    }
    info->id = (int32_t)best;
    info->kept = kept;

    /* 5. extras: softmax over the kept scaled logits (the filtered ones are
     * -1e10 on the page, exactly 0 after the softmax), the drawn id's
     * probability, and the top 8 by probability, ties to the lower index */
    if (extras) {
        double mx = -INFINITY;
        for (int64_t i = 0; i < vocab; ++i)
            if (keep[i] && (double)s[i] > mx)
                mx = s[i];
        double z = 0.0;
        for (int64_t i = 0; i < vocab; ++i)
            if (keep[i])
                z += exp((double)s[i] - mx);
        extras->chosen_prob = exp((double)s[best] - mx) / z;
        for (int64_t i = 0; i < vocab; ++i) {
            order[i].v = s[i];
            order[i].i = i;
        }
        qsort(order, (size_t)vocab, sizeof *order, cmp_desc_value_asc_index);
        int r = 0;
        for (int64_t j = 0; j < vocab && r < 8; ++j)
            if (keep[order[j].i]) {
                extras->top_ids[r] = (int32_t)order[j].i;
                extras->top_probs[r++] = exp((double)order[j].v - mx) / z;
            }
        for (int64_t i = 0; i < vocab && r < 8; ++i)
            if (!keep[i]) {
                extras->top_ids[r] = (int32_t)i;
                extras->top_probs[r++] = 0.0;
            }
        for (; r < 8; ++r) {
            extras->top_ids[r] = -1;
            extras->top_probs[r] = 0.0;
        }
    }
    free(s); free(keep); free(order); free(asc); free(cum);
    return info->id;
}

int32_t oracle_sample_row(const float *logits, const float *gumbel,
                          int64_t vocab, float temperature, float top_p,
                          int32_t top_k, oracle_sample_info *info)
{
    return oracle_sample_row_ex(logits, gumbel, NULL, vocab, temperature, top_p, top_k, info,
                                NULL);
}

void oracle_sample(int32_t *ids, oracle_sample_info *infos,
                   const float *logits, int64_t logits_stride,
                   const float *gumbel, int64_t gumbel_stride,
                   const float *temperature, const float *top_p,
                   const int32_t *top_k, int64_t batch, int64_t vocab)
{
    for (int64_t b = 0; b < batch; ++b)
        ids[b] = oracle_sample_row(logits + b * logits_stride,
                                   gumbel + b * gumbel_stride, vocab,
                                   temperature[b], top_p[b], top_k[b],
                                   infos ? infos + b : NULL);
}
