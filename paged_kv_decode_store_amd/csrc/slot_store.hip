// Slot mapping and the paged KV store.
//
// The store is a scattered bit copy: each token's [num_kv_heads][head_dim]
// bf16 row goes to pool row `slot` (a pool row is contiguous in the
// [block][offset][head][dim] layout), one 16-byte chunk per lane.
#include "launch.hpp"
#include "pkv_device.hpp"

namespace pkv {

__global__ __launch_bounds__(256) void slot_mapping_kernel(int32_t *__restrict__ slot_mapping,
                                                           const int32_t *__restrict__ tables,
                                                           int32_t stride,
                                                           const int32_t *__restrict__ lens,
                                                           int32_t batch, int32_t bs_log2,
                                                           uint32_t *err)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const int n = lens[b];
    int32_t slot = -1;
    if (n > 0) {
        const int pos = n - 1;  // the new token is the last of the n positions
        const int logical = pos >> bs_log2;
        if (logical < stride) {
            const int phys = tables[(int64_t)b * stride + logical];
            const int64_t s = ((int64_t)phys << bs_log2) + (pos & ((1 << bs_log2) - 1));
            if (phys >= 0 && s <= INT32_MAX) slot = (int32_t)s;
            else report_error(err, PKV_DEVERR_BLOCK_ID);
        } else {
            report_error(err, PKV_DEVERR_CONTEXT_LEN);
        }
    } else if (n < 0) {
        report_error(err, PKV_DEVERR_CONTEXT_LEN);
    }
    slot_mapping[b] = slot;
}

hipError_t launch_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                               int32_t table_stride, const int32_t *context_lens, int32_t batch,
                               int32_t block_size, uint32_t *err, hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    const int bs_log2 = __builtin_ctz((unsigned)block_size);
    slot_mapping_kernel<<<(batch + 255) / 256, 256, 0, stream>>>(
        slot_mapping, block_tables, table_stride, context_lens, batch, bs_log2, err);
    return hipGetLastError();
}

// One lane per 16-byte chunk of a token's K row (and the same chunk of V).
__global__ __launch_bounds__(256) void kv_store_kernel(uint16_t *__restrict__ k_cache,
                                                       uint16_t *__restrict__ v_cache,
                                                       const uint16_t *__restrict__ k_new,
                                                       const uint16_t *__restrict__ v_new,
                                                       const int32_t *__restrict__ slots,
                                                       int32_t num_tokens, int32_t row_chunks,
                                                       int64_t new_stride, int64_t total_slots,
                                                       uint32_t *err)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t t = idx / row_chunks;
    if (t >= num_tokens) return;
    const int c = (int)(idx - t * row_chunks);
    const int64_t slot = slots[t];
    if (slot < 0) return;  // a skipped token
    if (slot >= total_slots) {
        if (c == 0) report_error(err, PKV_DEVERR_SLOT);
        return;
    }
    const int64_t row = (int64_t)row_chunks * 8;  // elements per pool row
    const uint4 kv = *reinterpret_cast<const uint4 *>(k_new + t * new_stride + c * 8);
    const uint4 vv = *reinterpret_cast<const uint4 *>(v_new + t * new_stride + c * 8);
    *reinterpret_cast<uint4 *>(k_cache + slot * row + c * 8) = kv;
    *reinterpret_cast<uint4 *>(v_cache + slot * row + c * 8) = vv;
}

hipError_t launch_kv_store(uint16_t *k_cache, uint16_t *v_cache, const uint16_t *k_new,
                           const uint16_t *v_new, const int32_t *slots, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int64_t new_stride,
                           int64_t total_slots, uint32_t *err, hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int32_t row_chunks = num_kv_heads * head_dim / 8;
    const int64_t lanes = (int64_t)num_tokens * row_chunks;
    const int64_t blocks = (lanes + 255) / 256;
    kv_store_kernel<<<(unsigned)blocks, 256, 0, stream>>>(k_cache, v_cache, k_new, v_new, slots,
                                                          num_tokens, row_chunks, new_stride,
                                                          total_slots, err);
    return hipGetLastError();
}

}  // namespace pkv
