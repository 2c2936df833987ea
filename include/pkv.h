/*
 * pkv.h - C ABI of libpkv.so, the paged-KV decode step for AMD MI355X
 * (gfx950): slot mapping, KV store, split-KV paged GQA decode attention and
 * the next-token sampler.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers unless stated; the caller owns every
 *     buffer (pools, inputs, outputs, workspaces).  The library never
 *     allocates, frees or synchronises: each call only enqueues kernels on
 *     `stream` (NULL = the default stream) and returns.  Calls on one stream
 *     run in order, which gives the required store-before-attend order.
 *   - bf16 tensors are passed as raw 16-bit storage; they must be 16-byte
 *     aligned, and so must every row start implied by a stride.
 *   - Paged pool layout (one layer's K or V):
 *         [num_blocks][block_size][num_kv_heads][head_dim]   bf16
 *     i.e. the per-layer view of the nano-vllm pool (page "Model Runner",
 *     section "allocated kv cache").  A flat slot s addresses token row
 *     (s / block_size, s % block_size).
 *   - Return value: PKV_OK, or a negative pkv_status.  Argument errors are
 *     detected on the host before any HIP call and nothing is enqueued.
 *     PKV_ERR_HIP means a launch failed; pkv_last_error() has the text.
 *   - Device-side contents (slots, block ids, lengths) are a caller
 *     contract.  Kernels never access memory outside the buffers described
 *     by the size arguments: out-of-range slots are skipped, out-of-range
 *     block ids read block 0, over-long rows are truncated; results for such
 *     rows are unspecified.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or stride */
    PKV_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim) */
    PKV_ERR_WORKSPACE = -3,   /* workspace missing or too small */
    PKV_ERR_HIP = -4          /* a HIP launch failed */
} pkv_status;

/* Static text for a status code. */
const char *pkv_status_string(int status);

/* Text of the last failure on the calling host thread ("" if none). */
const char *pkv_last_error(void);

/* ---- device error word ----------------------------------------------------
 * Kernels cannot return a status, and device-side contents are only checked
 * on the device.  Rather than degrade silently (the "xAI native runtime"
 * article, section 4.2, asks for an explicit out-of-KV-slots error), the
 * kernels OR the bits below into a caller-owned device word when they meet
 * contents that break the contract stated with each entry point.  They keep
 * their in-bounds behaviour (skip the slot, read block 0, truncate the row),
 * so a set bit means the affected outputs are unspecified, never that memory
 * outside the buffers was touched.
 *
 * pkv_set_error_word(word): word is a device pointer to one uint32_t (4-byte
 * aligned), or NULL to stop reporting (the default).  The setting belongs to
 * the calling host thread and applies to the calls it makes afterwards
 * (kernels captured into a graph keep the word they were captured with).
 * The library never clears the word: the caller zeroes it (e.g. with a fill
 * kernel on the same stream) and reads it back when it wants the result. */
#define PKV_DEVERR_SLOT 0x1u        /* store: slot >= num_blocks * block_size */
#define PKV_DEVERR_BLOCK_ID 0x2u    /* a block id a row needs is < 0 or >= num_blocks */
#define PKV_DEVERR_CONTEXT_LEN 0x4u /* context length < 0, > max_context_len (or
                                       max_seqlen_k), or past the block table */
#define PKV_DEVERR_SEQLENS 0x8u     /* varlen: q_len < 0, k_len < q_len, or
                                       q_len > max_seqlen_q */
#define PKV_DEVERR_WAIT 0x10u       /* an in-kernel bounded wait gave up; the
                                       outputs of that launch are unreliable */

int pkv_set_error_word(uint32_t *word);
uint32_t *pkv_get_error_word(void);

/* Test hook: the iteration cap of the in-kernel bounded waits (varlen
 * attention's per-group step synchronisation), for the calling host thread.
 * 0 restores the default (2^22 polls, never reached in a correct run).  A
 * small cap makes the wait give up, which sets PKV_DEVERR_WAIT; addresses
 * never depend on the wait, so the launch still stays inside its buffers. */
int pkv_set_wait_limit(uint32_t polls);

/* ---- measurement helpers -----------------------------------------------------
 * Not part of the decode path: what the benchmark holds the kernels against
 * (the nanochat page's inference benchmark reports model bandwidth
 * utilisation against the device's bandwidth; these give the device's own
 * figures).
 *
 * Streaming-read probe: reads `bytes` of device memory at buf once, with the
 * 16-byte non-temporal vector loads the attention kernels stream K/V with,
 * over `workgroups` workgroups of 256 threads (0: 16 per compute unit), each
 * reading a contiguous share with eight loads in flight per thread.  sink: device uint32 [64], practically never written (it keeps the
 * loads from being optimised out).  Timing is the caller's (HIP events on
 * `stream`).  bytes: a multiple of 16; buf and sink 16- and 4-byte aligned. */
int pkv_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t workgroups,
                          hipStream_t stream);

/* Properties of a device, from the HIP runtime (hipGetDeviceProperties). */
typedef struct {
    char name[256];
    char arch[64];                  /* e.g. "gfx950:sramecc+:xnack-" */
    int32_t compute_units;
    int32_t clock_khz;              /* peak shader clock */
    int32_t memory_clock_khz;
    int32_t memory_bus_width_bits;
    int32_t l2_cache_bytes;
    int32_t lds_per_workgroup_bytes;
    int32_t wavefront_size;
    int32_t pad;
    uint64_t total_memory_bytes;
} pkv_device_info;

int pkv_get_device_info(int32_t device, pkv_device_info *out);

/* ---- slot mapping ---------------------------------------------------------
 * Decode-step slot of each row's new token (nano-vllm "Model Runner" page,
 * sections "allocated kv cache" and "prefill and decode"): a row whose
 * context holds n tokens (the new one included) writes position pos = n - 1
 * at
 *     slot = block_tables[b][pos / block_size] * block_size + pos % block_size
 * slot_mapping     int32 [batch]                      (out)
 * block_tables     int32 [batch][block_table_stride]  physical block ids
 * context_lens     int32 [batch]                      n per row
 * n <= 0, a logical block beyond the table, or a negative table entry gives
 * slot -1 (the store then skips the row).  block_size: power of two >= 1. */
int pkv_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                     int32_t block_table_stride, const int32_t *context_lens,
                     int32_t batch, int32_t block_size, hipStream_t stream);

/* ---- KV store -------------------------------------------------------------
 * Writes each token's new K and V head rows into the paged pools at its
 * slot, in place (nano-vllm page, section "prepare Prefill": the attention
 * path writes the new K/V at slot_mapping; nanochat engine page, section 2:
 * the cache is updated in place).  A bit copy.
 * k_cache, v_cache bf16 pools (layout above), num_blocks blocks each
 * k_new, v_new     bf16 [num_tokens][num_kv_heads][head_dim] rows; row t
 *                  starts at element t * new_token_stride (0 = packed)
 * slot_mapping     int32 [num_tokens]; slot < 0 or >= num_blocks*block_size
 *                  skips the token.  Slots of one call must be distinct.
 * head_dim: multiple of 8, <= 256.  block_size: power of two in [16, 4096]. */
int pkv_kv_store(void *k_cache, void *v_cache, const void *k_new,
                 const void *v_new, const int32_t *slot_mapping,
                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                 int64_t new_token_stride, int32_t block_size,
                 int64_t num_blocks, hipStream_t stream);

/* ---- paged decode attention ----------------------------------------------
 * Single-query GQA attention of each row over its own n_b cached positions,
 * gathered through its block table (Grok-1 runners chapter, sections 8.2.3
 * and 8.5: one new token attends over all cached K/V, 48 query heads share 8
 * KV heads; nano-vllm page, "prefill and decode": n_b includes the new
 * token, which must already be stored).  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads).  For each (b, h):
 *     o = sum_j softmax_j(scale * q . K_j) V_j,   j = 0 .. n_b - 1
 * and n_b == 0 (an inactive row, chapter 8.2.3) gives o = 0.
 *
 * The work is split: positions [s*split_tokens, (s+1)*split_tokens) of each
 * (row, KV head) form one partial (running max, sum and unnormalised
 * output, fp32, in the workspace); the reduce step merges a row's partials
 * with weights exp(m_s - M).  pkv_paged_decode_attention runs both steps;
 * the two steps are also exported separately.
 *
 * out            bf16 [batch][num_q_heads][head_dim], row b at b*out_stride
 * q              bf16 [batch][num_q_heads][head_dim], row b at b*q_stride
 *                (strides in elements; 0 = packed)
 * k_cache,v_cache bf16 pools, num_blocks blocks
 * block_tables   int32 [batch][block_table_stride]
 * context_lens   int32 [batch]; each must be <= max_context_len
 * head_dim       64 or 128;  block_size power of two in [16, 4096]
 * scale          softmax scale; <= 0 selects 1/sqrt(head_dim)
 * split_tokens   positions per partial: 0 = automatic, else a multiple of
 *                64 (see pkv_decode_split_tokens: the automatic choice
 *                depends on batch, heads and max_context_len only, never on
 *                device data, so a query and the launch always agree)
 * workspace      device scratch of at least pkv_decode_workspace_bytes(...)
 *                bytes, 256-byte aligned; contents on entry are ignored.
 * When the split geometry gives every row a single split, the combined
 * entry points (pkv_paged_decode_attention and its _store form) launch
 * only the partial step, which writes the normalised output itself; the
 * result is the same bit for bit as partial + reduce. */
int32_t pkv_decode_split_tokens(int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t max_context_len,
                                int32_t split_tokens);

size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_context_len,
                                  int32_t split_tokens);

int pkv_paged_decode_attention(void *out, int64_t out_stride, const void *q,
                               int64_t q_stride, const void *k_cache,
                               const void *v_cache,
                               const int32_t *block_tables,
                               int32_t block_table_stride,
                               const int32_t *context_lens, int32_t batch,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_context_len,
                               float scale, int32_t split_tokens,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Partial step only: fills the workspace. */
int pkv_decode_attention_partial(const void *q, int64_t q_stride,
                                 const void *k_cache, const void *v_cache,
                                 const int32_t *block_tables,
                                 int32_t block_table_stride,
                                 const int32_t *context_lens, int32_t batch,
                                 int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, int32_t max_context_len,
                                 float scale, int32_t split_tokens,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Reduce step only: reads a workspace filled by the partial step with the
 * same shape arguments and writes out. */
int pkv_decode_attention_reduce(void *out, int64_t out_stride,
                                const int32_t *context_lens, int32_t batch,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_table_stride,
                                int32_t block_size, int32_t max_context_len,
                                int32_t split_tokens, const void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ---- fused store + attention ---------------------------------------------
 * The decode step's store and attention in one pass, the way the pages'
 * attention kernels write the new K/V into the cache while attending
 * (nanochat engine page, section 2: the cache is written in place inside the
 * attention call; nano-vllm page, "prepare Prefill": the attention path
 * writes the new K/V at slot_mapping).  For each row b with
 * 1 <= n_b <= max_context_len, position n_b - 1 is the new token: its K/V
 * rows are taken from k_new/v_new (bf16 [batch][num_kv_heads][head_dim],
 * row b at b*new_token_stride elements, 0 = packed), written into the pools
 * at slot block_tables[b][(n_b-1)/block_size]*block_size + (n_b-1)%block_size
 * (skipped if that block id is outside [0, num_blocks)) by the workgroup
 * that attends to that position, before it streams its range.  The result
 * equals pkv_slot_mapping + pkv_kv_store + pkv_paged_decode_attention on the
 * same arguments.  Other arguments and the workspace are as for
 * pkv_paged_decode_attention. */
int pkv_paged_decode_attention_store(void *out, int64_t out_stride,
                                     const void *q, int64_t q_stride,
                                     void *k_cache, void *v_cache,
                                     const void *k_new, const void *v_new,
                                     int64_t new_token_stride,
                                     const int32_t *block_tables,
                                     int32_t block_table_stride,
                                     const int32_t *context_lens,
                                     int32_t batch, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int64_t num_blocks,
                                     int32_t max_context_len, float scale,
                                     int32_t split_tokens, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* The fused store + attention without a workspace argument, for callers
 * that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation).  The split-KV partials
 * go to a fixed device array inside the library, PKV_STATIC_SCRATCH_BYTES
 * long, of which each GPU holds its own copy for the life of the process;
 * no call allocates or frees anything.  The result equals
 * pkv_paged_decode_attention_store with the same arguments.
 * Limits: the partials must fit, i.e. pkv_decode_workspace_bytes(batch,
 * num_q_heads, num_kv_heads, head_dim, max_context_len, split_tokens) <=
 * PKV_STATIC_SCRATCH_BYTES, else PKV_ERR_WORKSPACE before any HIP call
 * (e.g. 64 rows x 16 heads at 4096 positions use about 4.3 MB).
 * Concurrency: every call on one GPU uses that GPU's single array, so calls
 * that overlap in time on one GPU (different streams, or other host
 * threads) race and give unspecified results; serialise them on one
 * stream.  Calls in order on one stream are safe (nothing in the array
 * needs clearing: each call fully writes what it reads). */
#define PKV_STATIC_SCRATCH_BYTES (32u << 20)

int pkv_paged_decode_attention_store_noalloc(void *out, int64_t out_stride,
                                             const void *q, int64_t q_stride,
                                             void *k_cache, void *v_cache,
                                             const void *k_new, const void *v_new,
                                             int64_t new_token_stride,
                                             const int32_t *block_tables,
                                             int32_t block_table_stride,
                                             const int32_t *context_lens,
                                             int32_t batch, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int64_t num_blocks,
                                             int32_t max_context_len, float scale,
                                             int32_t split_tokens, hipStream_t stream);

/* Partial step of the fused path only (store + partials); finish with
 * pkv_decode_attention_reduce. */
int pkv_decode_attention_partial_store(const void *q, int64_t q_stride,
                                       void *k_cache, void *v_cache,
                                       const void *k_new, const void *v_new,
                                       int64_t new_token_stride,
                                       const int32_t *block_tables,
                                       int32_t block_table_stride,
                                       const int32_t *context_lens,
                                       int32_t batch, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int64_t num_blocks,
                                       int32_t max_context_len, float scale,
                                       int32_t split_tokens, void *workspace,
                                       size_t workspace_bytes,
                                       hipStream_t stream);

/* ---- shared-prefix (cascade) decode --------------------------------------
 * Rows that begin with the same cached blocks, as after one prefill cloned
 * into N rows (nanochat engine page, section 3: one batch-1 prefill whose
 * cache is copied into every row of the decode batch; nano-vllm page,
 * "prefix cache": cached prefix blocks shared through block tables).  The
 * result equals pkv_paged_decode_attention over each row's whole context;
 * only the order of the work differs: the shared prefix, positions
 * [0, num_prefix_blocks*block_size), is read once per KV head for all the
 * rows (through prefix_blocks), each row's own positions after it through
 * its block table, and the two are merged by log-sum-exp.  Two launches:
 * one grid on the matrix cores for both parts (16 (row, query head) pairs
 * per prefix workgroup), then the split-KV reduce.
 *
 * prefix_blocks      int32 [num_prefix_blocks]: block ids of the shared
 *                    prefix, in position order.  Every row's first
 *                    num_prefix_blocks logical blocks are these; the
 *                    corresponding block-table entries are not read.
 * num_prefix_blocks  >= 1
 * context_lens       as for pkv_paged_decode_attention; a row shorter than
 *                    the prefix attends to its own first n_b prefix
 *                    positions only, and n_b = 0 gives a zero output.
 * workspace          at least pkv_cascade_workspace_bytes(...) bytes,
 *                    256-byte aligned; contents on entry are ignored.
 * Other arguments as for pkv_paged_decode_attention (split_tokens applies
 * to the positions after the prefix).  The new token's K/V is stored with
 * pkv_kv_store beforehand; it must not lie in a shared block. */
size_t pkv_cascade_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len,
                                   int32_t num_prefix_blocks,
                                   int32_t block_size, int32_t split_tokens);

int pkv_cascade_decode_attention(void *out, int64_t out_stride, const void *q,
                                 int64_t q_stride, const void *k_cache,
                                 const void *v_cache,
                                 const int32_t *prefix_blocks,
                                 int32_t num_prefix_blocks,
                                 const int32_t *block_tables,
                                 int32_t block_table_stride,
                                 const int32_t *context_lens, int32_t batch,
                                 int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, int32_t max_context_len,
                                 float scale, int32_t split_tokens,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* ---- varlen multi-query paged attention (chunked prefill) ----------------
 * The step before the decode path (nano-vllm page, "prefix cache" and
 * "prefill and decode": cu_seqlens_q / cu_seqlens_k over a paged cache,
 * the prompt's new tokens computed together, causally).  Sequence b has
 * q_len_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] new tokens, packed as rows
 * cu_seqlens_q[b] .. of q and out, and k_len_b = cu_seqlens_k[b+1] -
 * cu_seqlens_k[b] >= q_len_b tokens in the cache, the new ones last (their
 * K/V stored beforehand: pkv_varlen_slot_mapping + pkv_kv_store).  New
 * token j attends to positions [0, k_len_b - q_len_b + j] through the
 * sequence's block table.
 *
 * pkv_varlen_slot_mapping: slot_mapping int32 [total new tokens], the slot
 * of token j of sequence b at position k_len_b - q_len_b + j (-1 where the
 * table entry is negative or the position is past the table).
 * pkv_varlen_paged_attention:
 * out, q         bf16 [total_q][num_q_heads][head_dim]; token rows
 *                out_stride / q_stride elements apart (0 = packed);
 *                total_q = cu_seqlens_q[batch] (rows of q and out)
 * cu_seqlens_q, cu_seqlens_k  int32 [batch + 1], non-decreasing from 0
 * max_seqlen_q   >= every q_len_b (tokens past it are not computed)
 * max_seqlen_k   >= every k_len_b (positions past it or past the table
 *                are not attended)
 * head_dim 64 or 128; block_size a power of two in [16, 4096]; scale <= 0
 * selects 1/sqrt(head_dim).
 * split_tokens   positions per workgroup of a tile's causal range: 0 =
 *                automatic (pkv_varlen_split_tokens: from batch, heads and
 *                the maximum lengths only), else a positive multiple of
 *                256.  Ranges needing one split are written directly;
 *                longer ones go through fp32 partials in the workspace and
 *                a log-sum-exp merge.
 * workspace      >= pkv_varlen_workspace_bytes(...) bytes, 256-byte
 *                aligned; may be null when that size is 0 (every range fits
 *                one split).  Contents on entry are ignored.
 * A sequence with q_len_b = 0 or k_len_b < q_len_b writes nothing. */
int pkv_varlen_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                            int32_t block_table_stride,
                            const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t batch,
                            int32_t max_seqlen_q, int32_t block_size,
                            hipStream_t stream);

int32_t pkv_varlen_split_tokens(int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t max_seqlen_q,
                                int32_t max_seqlen_k, int32_t split_tokens);

size_t pkv_varlen_workspace_bytes(int32_t total_q, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seqlen_q,
                                  int32_t max_seqlen_k, int32_t split_tokens);

int pkv_varlen_paged_attention(void *out, int64_t out_stride, const void *q,
                               int64_t q_stride, const void *k_cache,
                               const void *v_cache,
                               const int32_t *block_tables,
                               int32_t block_table_stride,
                               const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, int32_t batch,
                               int32_t total_q, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               float scale, int32_t split_tokens,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ---- sampler --------------------------------------------------------------
 * Next token per row (Grok-1 runners chapter, section 8.3 and 8.3.1;
 * nanochat engine page, section 3; nano-vllm page, "run model").  Each row's
 * own settings decide what runs for it:
 *   temperature <= 0 (or NaN): greedy, the lowest index of max logits.
 *   otherwise, in this order:
 *     s_i = logits_i / T                      (IEEE fp32 division)
 *     top-k  if 0 < k < vocab: keep the k largest s, ties to lower index
 *            (k <= 0 or k >= vocab: off)
 *     top-p  if p < 1: over the kept set, keep every s_i >= tau where tau is
 *            the smallest value whose strictly-greater mass is <= p of the
 *            kept mass (the ascending-cumsum rule of the page, exact
 *            arithmetic); p <= 0 keeps only the maxima (p >= 1: off)
 *     id = argmax over kept i of fl32(s_i + gumbel_i), ties to lower index
 * The Gumbel noise is an input (standard Gumbel, fp32), so the draw is
 * reproducible.  Only the ids are written.  Three launches: one pass over
 * the logits (per-chunk maxima and candidate lists), a few workgroups per
 * row that bin the candidates below the row max (counts, exact masses, best
 * Gumbel keys), then one workgroup per row that resolves the cut exactly
 * inside its bin, or, when the candidates cannot be shown to hold the cut
 * (e.g. k larger than the candidate lists, or many tokens tied at the cut),
 * from the whole row read again (exact, slower).
 * out_ids      int32 [batch]
 * logits       fp32 [batch][vocab], row b at b*logits_stride (elements)
 * gumbel       fp32 [batch][vocab], row b at b*gumbel_stride; read for the
 *              candidates (about one token in eight of a nucleus row) and
 *              where a token is eligible (unused for greedy rows)
 * temperature, top_p  fp32 [batch];  top_k  int32 [batch]
 * vocab        1 .. 2^24;  batch <= 65535
 * workspace    >= pkv_sampler_workspace_bytes(batch, vocab), 256-B aligned;
 *              about 3 bytes per logit plus ~200 KB per filtered row
 *              (4.5 B per logit at 151,936); contents on entry are ignored */
size_t pkv_sampler_workspace_bytes(int32_t batch, int32_t vocab);

int pkv_sample_next_token(int32_t *out_ids, const float *logits,
                          int64_t logits_stride, const float *gumbel,
                          int64_t gumbel_stride, const float *temperature,
                          const float *top_p, const int32_t *top_k,
                          int32_t batch, int32_t vocab, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* The sampler with the runner's vocabulary mask and extra outputs (Grok-1
 * runners chapter, section 8.3: sample_token scales by 1/T, replaces the
 * logits of forbidden tokens by -1e10, filters, draws, and also returns the
 * drawn token's probability and the top 8 (TOP_K = 8) ids and
 * probabilities of the filtered distribution for debugging).
 * vocab_mask     uint8 [batch][vocab], row b at b*mask_stride (0 = packed);
 *                0 = forbidden: s_i = -1e10 after the scaling (greedy rows:
 *                the raw logit counts as -1e10).  NULL: no mask.
 * out_prob       fp32 [batch] or NULL: softmax over the kept s at the drawn
 *                id (greedy rows: 1 / number of tied maxima)
 * out_top_ids    int32 [batch][8] or NULL: the kept ids of largest s (ties
 *                to the lower index); fewer than 8 kept are followed by the
 *                lowest-index ids outside the kept set; -1 past vocab
 * out_top_probs  fp32 [batch][8] or NULL: their probabilities (0 outside
 *                the kept set)
 * When any output pointer is non-NULL one more workgroup per row reads the
 * row after the draw.  Everything else is as for pkv_sample_next_token,
 * which equals this call with NULL mask and outputs. */
int pkv_sample_next_token_ex(int32_t *out_ids, const float *logits,
                             int64_t logits_stride, const float *gumbel,
                             int64_t gumbel_stride, const uint8_t *vocab_mask,
                             int64_t mask_stride, const float *temperature,
                             const float *top_p, const int32_t *top_k,
                             int32_t batch, int32_t vocab,
                             float *out_prob, int32_t *out_top_ids,
                             float *out_top_probs, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
