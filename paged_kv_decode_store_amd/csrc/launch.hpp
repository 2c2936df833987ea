// Internal launchers behind the C ABI.  Arguments are already validated by
// the entry points in api.cpp; each launcher only enqueues kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// `err`: the device error word of the calling thread (null: no reporting).
hipError_t launch_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                               int32_t table_stride, const int32_t *context_lens,
                               int32_t batch, int32_t block_size, uint32_t *err,
                               hipStream_t stream);

hipError_t launch_kv_store(uint16_t *k_cache, uint16_t *v_cache, const uint16_t *k_new,
                           const uint16_t *v_new, const int32_t *slots, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int64_t new_stride,
                           int64_t total_slots, uint32_t *err, hipStream_t stream);

// Split-KV geometry shared by the partial and reduce steps.
struct SplitGeometry {
    int32_t split_tokens;  // positions per partial (multiple of 64)
    int32_t num_splits;    // partials per (row, query head)
    size_t part_o_bytes;   // fp32 [B][Hq][S][D]
    size_t part_ml_bytes;  // fp32 [B][Hq][S][2]
    size_t total_bytes;
};

int32_t auto_split_tokens(int32_t batch, int32_t num_kv_heads, int32_t max_context_len,
                          int32_t group);
SplitGeometry split_geometry(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                             int32_t max_context_len, int32_t split_tokens);

struct PartialArgs {
    float *part_o;
    float *part_ml;
    const uint16_t *q;
    int64_t q_stride;
    const uint16_t *k_cache;
    const uint16_t *v_cache;
    const int32_t *block_tables;
    int32_t table_stride;
    const int32_t *context_lens;
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;          // num_q_heads / num_kv_heads
    int32_t head_chunks;    // query-head chunks per KV head
    int32_t bs_log2;
    int64_t num_blocks;
    int32_t max_len;        // clamp of context_lens: min(max_context_len, stride*bs)
    int32_t split_tokens;
    int32_t num_splits;
    float c;                // softmax scale * log2(e)
    // fused store: when k_new is non-null, the workgroups whose range holds
    // a row's new position (context_lens[b] - 1) write its K/V rows from
    // k_new/v_new into the pools before streaming the range
    const uint16_t *k_new;
    const uint16_t *v_new;
    int64_t new_stride;     // elements between consecutive rows of k_new/v_new
    uint16_t *k_cache_w;    // same pools as k_cache/v_cache, written by the fused store
    uint16_t *v_cache_w;
    // shared-prefix (cascade) decode.  Tail launch: positions start at
    // pos_base and partial s goes to slot split_base + s.  Prefix launch:
    // one workgroup per (prefix split, KV head, chunk of virtual queries),
    // where the virtual queries of a KV head are the (row, query head) pairs
    // that use it, vq_per_kv = batch * group; positions [0, prefix_len) are
    // read once through prefix_blocks.
    // Cascade launch (both in one grid): the first prefix_wgs workgroups
    // are the prefix step with prefix_split positions per split, the rest
    // the tail step.
    int32_t pos_base;
    int32_t split_base;
    const int32_t *prefix_blocks;
    int32_t prefix_len;
    int32_t vq_per_kv;
    int32_t vchunks;        // virtual-query chunks per KV head
    int32_t prefix_split;   // positions per prefix split
    int32_t prefix_wgs;
    // varlen multi-query attention: sequence b's new tokens are rows
    // [cu_q[b], cu_q[b+1]) of q and out, its cache holds cu_k[b+1] - cu_k[b]
    // tokens (the new ones last); one workgroup per (chunk of 16 (token,
    // query head) pairs, KV head, sequence), bf16 output written directly
    const int32_t *cu_q;
    const int32_t *cu_k;
    uint16_t *out;
    int64_t out_stride;
    int32_t qchunks;        // chunks per sequence (from the longest one)
    int32_t total_q;        // rows of q / out (the merge step's grid)
    int32_t max_q;          // varlen: tokens past this in a sequence are not computed
    // device error word (PKV_DEVERR_* bits) or null, and the poll cap of
    // in-kernel bounded waits
    uint32_t *err;
    uint32_t wait_limit;
};

struct ReduceArgs {
    uint16_t *out;
    int64_t out_stride;
    const float *part_o;
    const float *part_ml;
    const int32_t *context_lens;
    int32_t batch;
    int32_t num_q_heads;
    int32_t max_len;
    int32_t split_tokens;
    int32_t num_splits;
    int32_t prefix_len;     // cascade: shared positions [0, prefix_len) ...
    int32_t prefix_splits;  // ... held in the first prefix_splits slots
};

hipError_t launch_decode_partial(const PartialArgs &a, int32_t head_dim, hipStream_t stream);
// Shared-prefix decode in one launch: the prefix step (prefix_blocks,
// prefix_len, prefix_split, vq_per_kv set) and the tail step (pos_base,
// split_base set) on the matrix cores, partials only.
hipError_t launch_decode_cascade_mfma(const PartialArgs &a, int32_t head_dim, hipStream_t stream);
hipError_t launch_decode_reduce(const ReduceArgs &a, int32_t head_dim, hipStream_t stream);
// Matrix-core partial step (up to 16 query heads per workgroup; head_chunks
// is derived).  The cascade decode runs on the same kernel
// (launch_decode_cascade_mfma; 16 virtual queries per prefix workgroup).
hipError_t launch_decode_partial_mfma(const PartialArgs &a, int32_t head_dim, hipStream_t stream);
// Varlen multi-query paged attention on the matrix-core kernel.
hipError_t launch_varlen_attention(const PartialArgs &a, int32_t head_dim, int32_t max_seqlen_q,
                                   hipStream_t stream);
hipError_t launch_varlen_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                                      int32_t table_stride, const int32_t *cu_seqlens_q,
                                      const int32_t *cu_seqlens_k, int32_t batch,
                                      int32_t max_seqlen_q, int32_t block_size,
                                      hipStream_t stream);
// Group sizes from which the partial step runs on the matrix cores (the VALU
// kernel is ALU-bound beyond group 2 on MI355X).
constexpr int32_t kMfmaMinGroup = 3;

// Streaming-read probe over `bytes` (a multiple of 16) of device memory with
// `workgroups` workgroups of 256 threads; sink: 64 uint32, almost never written.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t workgroups,
                              hipStream_t stream);

// The library's fixed device scratch array (PKV_STATIC_SCRATCH_BYTES) on
// the current device: its device address, resolved on first use per device.
hipError_t static_scratch(void **out);

// Sampler
size_t sampler_workspace_bytes(int32_t batch, int32_t vocab);
hipError_t launch_sampler(int32_t *out_ids, const float *logits, int64_t logits_stride,
                          const float *gumbel, int64_t gumbel_stride, const uint8_t *mask,
                          int64_t mask_stride, const float *temperature, const float *top_p,
                          const int32_t *top_k, int32_t batch, int32_t vocab, float *out_prob,
                          int32_t *out_top_ids, float *out_top_probs, void *workspace,
                          hipStream_t stream);

}  // namespace pkv
