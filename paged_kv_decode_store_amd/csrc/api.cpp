// C ABI entry points of libpkv.so: host-side argument checks, then the
// launchers.  Every check runs before any HIP call, so argument errors are
// reported without touching the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/pkv.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";
// device error word and bounded-wait cap of the calling host thread
thread_local uint32_t *g_err_word = nullptr;
thread_local uint32_t g_wait_limit = 0;
constexpr uint32_t kDefaultWaitLimit = 1u << 22;

uint32_t wait_limit() { return g_wait_limit ? g_wait_limit : kDefaultWaitLimit; }

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return PKV_OK;
    return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

#define REQUIRE(cond, status, ...)                  \
    do {                                            \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

int check_split(int32_t split_tokens)
{
    REQUIRE(split_tokens >= 0 && split_tokens % 64 == 0 && split_tokens <= (1 << 24),
            PKV_ERR_INVALID_ARG, "split_tokens must be 0 or a positive multiple of 64");
    return PKV_OK;
}

// Shape checks shared by the attention entry points.
int check_attention_shape(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t block_table_stride,
                          int32_t max_context_len)
{
    REQUIRE(batch >= 0, PKV_ERR_INVALID_ARG, "batch must be >= 0");
    REQUIRE(num_q_heads > 0 && num_kv_heads > 0, PKV_ERR_INVALID_ARG, "head counts must be > 0");
    REQUIRE(num_q_heads % num_kv_heads == 0, PKV_ERR_INVALID_ARG,
            "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", num_q_heads, num_kv_heads);
    REQUIRE(head_dim == 64 || head_dim == 128, PKV_ERR_UNSUPPORTED,
            "head_dim %d unsupported (64 or 128)", head_dim);
    REQUIRE(pow2(block_size) && block_size >= 16 && block_size <= 4096, PKV_ERR_UNSUPPORTED,
            "block_size %d unsupported (power of two in [16, 4096])", block_size);
    REQUIRE(block_table_stride > 0, PKV_ERR_INVALID_ARG, "block_table_stride must be > 0");
    REQUIRE(max_context_len >= 0, PKV_ERR_INVALID_ARG, "max_context_len must be >= 0");
    return PKV_OK;
}

// Largest divisor of the group size that is <= 8: query heads per workgroup.
int32_t heads_per_chunk(int32_t group)
{
    for (int g = 8; g >= 1; --g)
        if (group % g == 0) return g;
    return 1;
}

int32_t effective_split(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t max_context_len, int32_t split_tokens)
{
    if (split_tokens > 0) return split_tokens;
    const int32_t group = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 1;
    return pkv::auto_split_tokens(batch, num_kv_heads, max_context_len, group);
}

int32_t clamp_len(int32_t max_context_len, int32_t block_table_stride, int32_t block_size)
{
    const int64_t cap = (int64_t)block_table_stride * block_size;
    return (int32_t)(max_context_len < cap ? max_context_len : cap);
}

// Prefix launch shape: the matrix-core kernel takes 16 virtual queries per
// workgroup; the prefix is cut into splits so that about kPrefixGroups
// workgroups stream it (clone workload: 256 and 512 are equal, fewer is
// slower).
constexpr int kPrefixQ = 16;        // virtual queries per prefix workgroup
constexpr int kPrefixGroups = 256;  // prefix workgroups wanted

// Workspace geometry of the shared-prefix (cascade) decode: per (row, query
// head), prefix_splits partials of the shared prefix, then the partials of
// the row's own positions after it.
struct CascadeGeometry {
    int32_t prefix_len;
    int32_t prefix_split;    // positions per prefix partial
    int32_t prefix_splits;
    int32_t tail_split;      // positions per partial after the prefix
    int32_t num_splits;      // slots per (row, query head)
    int32_t vchunks;         // virtual-query chunks per KV head
    pkv::SplitGeometry ws;   // workspace sizes (split_tokens = tail_split)
};

CascadeGeometry cascade_geometry(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_len, int32_t num_prefix_blocks,
                                 int32_t block_size, int32_t split_tokens)
{
    CascadeGeometry g;
    const int32_t group = num_q_heads / num_kv_heads;
    g.prefix_len = num_prefix_blocks * block_size;
    // every (row, query head) of a KV head is one virtual query
    const int64_t vq = (int64_t)batch * group;
    g.vchunks = (int32_t)((vq + kPrefixQ - 1) / kPrefixQ);
    if (g.vchunks < 1) g.vchunks = 1;
    // prefix splits: enough workgroups (~512) to stream the prefix in parallel
    const int64_t per_split = (int64_t)num_kv_heads * g.vchunks;
    int64_t want = (kPrefixGroups + per_split - 1) / per_split;
    if (want < 1) want = 1;
    int64_t ps = (g.prefix_len + want - 1) / want;
    ps = (ps + 63) / 64 * 64;
    if (ps < 64) ps = 64;
    g.prefix_split = (int32_t)ps;
    g.prefix_splits = (int32_t)((g.prefix_len + ps - 1) / ps);
    const int32_t tail_len = max_len > g.prefix_len ? max_len - g.prefix_len : 0;
    g.tail_split = split_tokens > 0
                       ? split_tokens
                       : pkv::auto_split_tokens(batch, num_kv_heads, tail_len, group);
    const int32_t tail_splits = (tail_len + g.tail_split - 1) / g.tail_split;
    g.num_splits = g.prefix_splits + tail_splits;
    // workspace: the same layout as the plain split geometry with num_splits slots
    g.ws = pkv::split_geometry(batch, num_q_heads, head_dim, 0, g.tail_split);
    const size_t units = (size_t)batch * num_q_heads * g.num_splits;
    g.ws.num_splits = g.num_splits;
    g.ws.part_o_bytes = (units * head_dim * sizeof(float) + 255) & ~(size_t)255;
    g.ws.part_ml_bytes = (units * 2 * sizeof(float) + 255) & ~(size_t)255;
    g.ws.total_bytes = g.ws.part_o_bytes + g.ws.part_ml_bytes;
    return g;
}

}  // namespace

extern "C" {

const char *pkv_status_string(int status)
{
    switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char *pkv_last_error(void) { return g_last_error; }

int pkv_set_error_word(uint32_t *word)
{
    REQUIRE(aligned(word, 4), PKV_ERR_INVALID_ARG, "error word must be 4-byte aligned");
    g_err_word = word;
    return PKV_OK;
}

uint32_t *pkv_get_error_word(void) { return g_err_word; }

int pkv_set_wait_limit(uint32_t polls)
{
    g_wait_limit = polls;
    return PKV_OK;
}

int pkv_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t workgroups,
                          hipStream_t stream)
{
    REQUIRE(bytes % 16 == 0, PKV_ERR_INVALID_ARG, "bytes must be a multiple of 16");
    if (bytes == 0) return PKV_OK;
    REQUIRE(buf && sink, PKV_ERR_INVALID_ARG, "null pointer");
    REQUIRE(aligned(buf, 16) && aligned(sink, 4), PKV_ERR_INVALID_ARG, "misaligned buffer");
    REQUIRE(workgroups >= 0, PKV_ERR_INVALID_ARG, "workgroups must be >= 0");
    if (workgroups == 0) {
        int dev = 0, cus = 0;
        int rc = hip_status(hipGetDevice(&dev), "hipGetDevice");
        if (rc != PKV_OK) return rc;
        rc = hip_status(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                        "compute unit count");
        if (rc != PKV_OK) return rc;
        workgroups = 16 * cus;
    }
    return hip_status(pkv::launch_stream_read(buf, bytes, sink, workgroups, stream),
                      "stream read probe launch");
}

int pkv_get_device_info(int32_t device, pkv_device_info *out)
{
    REQUIRE(out, PKV_ERR_INVALID_ARG, "null pointer");
    hipDeviceProp_t p;
    const int rc = hip_status(hipGetDeviceProperties(&p, device), "hipGetDeviceProperties");
    if (rc != PKV_OK) return rc;
    memset(out, 0, sizeof(*out));
    snprintf(out->name, sizeof(out->name), "%s", p.name);
    snprintf(out->arch, sizeof(out->arch), "%s", p.gcnArchName);
    out->compute_units = p.multiProcessorCount;
    out->clock_khz = p.clockRate;
    out->memory_clock_khz = p.memoryClockRate;
    out->memory_bus_width_bits = p.memoryBusWidth;
    out->l2_cache_bytes = p.l2CacheSize;
    out->lds_per_workgroup_bytes = (int32_t)p.sharedMemPerBlock;
    out->wavefront_size = p.warpSize;
    out->total_memory_bytes = (uint64_t)p.totalGlobalMem;
    return PKV_OK;
}

int pkv_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                     int32_t block_table_stride, const int32_t *context_lens, int32_t batch,
                     int32_t block_size, hipStream_t stream)
{
    REQUIRE(batch >= 0, PKV_ERR_INVALID_ARG, "batch must be >= 0");
    if (batch == 0) return PKV_OK;
    REQUIRE(slot_mapping && block_tables && context_lens, PKV_ERR_INVALID_ARG, "null pointer");
    REQUIRE(aligned(slot_mapping, 4) && aligned(block_tables, 4) && aligned(context_lens, 4),
            PKV_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
    REQUIRE(block_table_stride > 0, PKV_ERR_INVALID_ARG, "block_table_stride must be > 0");
    REQUIRE(pow2(block_size) && block_size <= (1 << 20), PKV_ERR_UNSUPPORTED,
            "block_size %d must be a power of two", block_size);
    return hip_status(pkv::launch_slot_mapping(slot_mapping, block_tables, block_table_stride,
                                               context_lens, batch, block_size, g_err_word,
                                               stream),
                      "slot_mapping launch");
}

int pkv_kv_store(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                 const int32_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                 int32_t head_dim, int64_t new_token_stride, int32_t block_size,
                 int64_t num_blocks, hipStream_t stream)
{
    REQUIRE(num_tokens >= 0, PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
    REQUIRE(num_kv_heads > 0, PKV_ERR_INVALID_ARG, "num_kv_heads must be > 0");
    REQUIRE(head_dim > 0 && head_dim % 8 == 0 && head_dim <= 256, PKV_ERR_UNSUPPORTED,
            "head_dim %d unsupported (multiple of 8, <= 256)", head_dim);
    REQUIRE(pow2(block_size) && block_size >= 16 && block_size <= 4096, PKV_ERR_UNSUPPORTED,
            "block_size %d unsupported (power of two in [16, 4096])", block_size);
    REQUIRE(num_blocks > 0, PKV_ERR_INVALID_ARG, "num_blocks must be > 0");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    const int64_t stride = new_token_stride ? new_token_stride : row;
    REQUIRE(stride >= row && stride % 8 == 0, PKV_ERR_INVALID_ARG,
            "new_token_stride %lld must be >= %lld and a multiple of 8",
            (long long)new_token_stride, (long long)row);
    if (num_tokens == 0) return PKV_OK;
    REQUIRE(k_cache && v_cache && k_new && v_new && slot_mapping, PKV_ERR_INVALID_ARG,
            "null pointer");
    REQUIRE(aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(k_new, 16) &&
                aligned(v_new, 16),
            PKV_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
    REQUIRE(aligned(slot_mapping, 4), PKV_ERR_INVALID_ARG, "slot_mapping must be 4-byte aligned");
    return hip_status(pkv::launch_kv_store(static_cast<uint16_t *>(k_cache),
                                           static_cast<uint16_t *>(v_cache),
                                           static_cast<const uint16_t *>(k_new),
                                           static_cast<const uint16_t *>(v_new), slot_mapping,
                                           num_tokens, num_kv_heads, head_dim, stride,
                                           num_blocks * block_size, g_err_word, stream),
                      "kv_store launch");
}

int32_t pkv_decode_split_tokens(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t max_context_len, int32_t split_tokens)
{
    if (check_split(split_tokens) != PKV_OK) return 0;
    return effective_split(batch, num_q_heads, num_kv_heads, max_context_len, split_tokens);
}

size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_context_len,
                                  int32_t split_tokens)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len < 0 || check_split(split_tokens) != PKV_OK)
        return 0;
    const int32_t split = effective_split(batch, num_q_heads, num_kv_heads, max_context_len, split_tokens);
    return pkv::split_geometry(batch, num_q_heads, head_dim, max_context_len, split).total_bytes;
}

}  // extern "C"

namespace {

// Checks and fills the partial step's launch arguments; k_new == NULL selects
// the plain partial, otherwise the fused store + partial.
int setup_partial(pkv::PartialArgs &a, const void *q, int64_t q_stride, const void *k_cache,
                  const void *v_cache, const void *k_new, const void *v_new,
                  int64_t new_token_stride, const int32_t *block_tables,
                  int32_t block_table_stride, const int32_t *context_lens, int32_t batch,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int64_t num_blocks, int32_t max_context_len, float scale, int32_t split_tokens,
                  void *workspace, size_t workspace_bytes, bool fused,
                  const pkv::SplitGeometry *geometry = nullptr)
{
    // every field not set below is zero: in particular `out` stays null, so
    // the partial kernels write partials, not the direct output
    memset(&a, 0, sizeof a);
    a.err = g_err_word;
    a.wait_limit = wait_limit();
    int rc = check_attention_shape(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                   block_table_stride, max_context_len);
    if (rc) return rc;
    if ((rc = check_split(split_tokens))) return rc;
    REQUIRE(num_blocks > 0, PKV_ERR_INVALID_ARG, "num_blocks must be > 0");
    const int64_t qs = q_stride ? q_stride : (int64_t)num_q_heads * head_dim;
    REQUIRE(qs >= (int64_t)num_q_heads * head_dim && qs % 8 == 0, PKV_ERR_INVALID_ARG,
            "q_stride must be >= num_q_heads*head_dim and a multiple of 8");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    const int64_t ns = new_token_stride ? new_token_stride : row;
    if (fused) {
        REQUIRE(ns >= row && ns % 8 == 0, PKV_ERR_INVALID_ARG,
                "new_token_stride must be >= num_kv_heads*head_dim and a multiple of 8");
    }
    REQUIRE(isfinite(scale), PKV_ERR_INVALID_ARG, "scale must be finite");
    if (batch == 0) return PKV_OK;
    REQUIRE(q && k_cache && v_cache && block_tables && context_lens, PKV_ERR_INVALID_ARG,
            "null pointer");
    REQUIRE(aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16), PKV_ERR_INVALID_ARG,
            "bf16 tensors must be 16-byte aligned");
    if (fused) {
        REQUIRE(k_new && v_new, PKV_ERR_INVALID_ARG, "null pointer");
        REQUIRE(aligned(k_new, 16) && aligned(v_new, 16), PKV_ERR_INVALID_ARG,
                "bf16 tensors must be 16-byte aligned");
    }
    REQUIRE(aligned(block_tables, 4) && aligned(context_lens, 4), PKV_ERR_INVALID_ARG,
            "int32 arrays must be 4-byte aligned");
    const int32_t split =
        geometry ? geometry->split_tokens
                 : effective_split(batch, num_q_heads, num_kv_heads, max_context_len, split_tokens);
    const pkv::SplitGeometry g =
        geometry ? *geometry
                 : pkv::split_geometry(batch, num_q_heads, head_dim, max_context_len, split);
    REQUIRE(workspace && aligned(workspace, 256), PKV_ERR_WORKSPACE,
            "workspace must be non-null and 256-byte aligned");
    REQUIRE(workspace_bytes >= g.total_bytes, PKV_ERR_WORKSPACE,
            "workspace too small: %zu < %zu bytes", workspace_bytes, g.total_bytes);

    a.part_o = static_cast<float *>(workspace);
    a.part_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + g.part_o_bytes);
    a.q = static_cast<const uint16_t *>(q);
    a.q_stride = qs;
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.block_tables = block_tables;
    a.table_stride = block_table_stride;
    a.context_lens = context_lens;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.head_chunks = a.group / heads_per_chunk(a.group);
    a.bs_log2 = __builtin_ctz((unsigned)block_size);
    a.num_blocks = num_blocks;
    a.max_len = clamp_len(max_context_len, block_table_stride, block_size);
    a.split_tokens = split;
    a.num_splits = g.num_splits;
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)head_dim);
    a.c = sc * 1.4426950408889634f;
    a.k_new = fused ? static_cast<const uint16_t *>(k_new) : nullptr;
    a.v_new = fused ? static_cast<const uint16_t *>(v_new) : nullptr;
    a.new_stride = ns;
    a.k_cache_w = fused ? static_cast<uint16_t *>(const_cast<void *>(k_cache)) : nullptr;
    a.v_cache_w = fused ? static_cast<uint16_t *>(const_cast<void *>(v_cache)) : nullptr;
    a.pos_base = 0;
    a.split_base = 0;
    a.prefix_blocks = nullptr;
    a.prefix_len = 0;
    a.vq_per_kv = 0;
    a.vchunks = 1;
    return PKV_OK;
}

// Varlen attention: positions per split of a row tile's causal range.  Given
// a positive multiple of 256, that; otherwise only as many splits as bring
// the workgroup count up to about one per CU of the 256 on MI355X, assuming
// every sequence at the maximum lengths (the host never reads cu_seqlens),
// with at least 1024 positions per split.  Measured on the Qwen3-shaped
// chunk (256 row tiles already), splitting further costs more than it
// balances: 1024-position splits took 55.5 us + 13.9 us of merge against
// 48.3 us unsplit.  Never longer than max_seqlen_k needs (then one split:
// no workspace).
int32_t varlen_effective_split(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t split_tokens)
{
    const int64_t cap = ((int64_t)(max_seqlen_k > 0 ? max_seqlen_k : 1) + 255) / 256 * 256;
    int64_t spl = split_tokens;
    if (spl <= 0) {
        const int64_t g = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 1;
        const int64_t tiles = ((int64_t)max_seqlen_q * g + 127) / 128;
        const int64_t jobs = (int64_t)batch * num_kv_heads * tiles;
        spl = ((int64_t)max_seqlen_k * jobs + 255) / 256;
        if (spl < 1024) spl = 1024;
        spl = (spl + 1023) / 1024 * 1024;
    }
    if (spl > cap) spl = cap;
    return (int32_t)spl;
}

struct VarlenGeometry {
    int32_t split_tokens;
    int32_t num_splits;
    size_t part_o_bytes, total_bytes;
};

VarlenGeometry varlen_geometry(int32_t total_q, int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen_q,
                               int32_t max_len, int32_t split_tokens)
{
    VarlenGeometry g;
    g.split_tokens = varlen_effective_split(batch, num_q_heads, num_kv_heads, max_seqlen_q,
                                            max_len, split_tokens);
    const int64_t ml = max_len > 0 ? max_len : 0;
    g.num_splits = (int32_t)((ml + g.split_tokens - 1) / g.split_tokens);
    if (g.num_splits < 1) g.num_splits = 1;
    g.part_o_bytes = g.total_bytes = 0;
    if (g.num_splits > 1) {
        const size_t units = (size_t)(total_q > 0 ? total_q : 0) * num_q_heads * g.num_splits;
        g.part_o_bytes = (units * head_dim * sizeof(float) + 255) & ~(size_t)255;
        g.total_bytes = g.part_o_bytes + ((units * 2 * sizeof(float) + 255) & ~(size_t)255);
    }
    return g;
}

// Partial step then reduce step, or, when the split geometry gives every row
// a single split, only the partial step writing the normalised output
// itself (the reduce of one partial is that partial divided by its sum, so
// the result is the same bit for bit).  Every argument of both steps is
// checked before anything is enqueued.
int decode_attention_combined(void *out, int64_t out_stride, const void *q, int64_t q_stride,
                              const void *k_cache, const void *v_cache, const void *k_new,
                              const void *v_new, int64_t new_token_stride,
                              const int32_t *block_tables, int32_t block_table_stride,
                              const int32_t *context_lens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, int32_t max_context_len, float scale,
                              int32_t split_tokens, void *workspace, size_t workspace_bytes,
                              bool fused, hipStream_t stream, bool validate_only = false)
{
    const int64_t os = out_stride ? out_stride : (int64_t)num_q_heads * head_dim;
    if (batch > 0) {
        REQUIRE(out && aligned(out, 16), PKV_ERR_INVALID_ARG,
                "out must be non-null and 16-byte aligned");
    }
    REQUIRE(num_q_heads > 0 && (os >= (int64_t)num_q_heads * head_dim) && os % 8 == 0,
            PKV_ERR_INVALID_ARG, "out_stride must be >= num_q_heads*head_dim and a multiple of 8");
    pkv::PartialArgs a;
    int rc = setup_partial(a, q, q_stride, k_cache, v_cache, k_new, v_new, new_token_stride,
                           block_tables, block_table_stride, context_lens, batch, num_q_heads,
                           num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale,
                           split_tokens, workspace, workspace_bytes, fused);
    if (rc || batch == 0 || validate_only) return rc;
    if (a.num_splits == 1) {
        a.out = static_cast<uint16_t *>(out);
        a.out_stride = os;
        return hip_status(pkv::launch_decode_partial(a, head_dim, stream),
                          "decode attention (single split) launch");
    }
    rc = hip_status(pkv::launch_decode_partial(a, head_dim, stream), "decode partial launch");
    if (rc) return rc;
    return pkv_decode_attention_reduce(out, out_stride, context_lens, batch, num_q_heads,
                                       num_kv_heads, head_dim, block_table_stride, block_size,
                                       max_context_len, split_tokens, workspace, workspace_bytes,
                                       stream);
}

}  // namespace

extern "C" {

int pkv_decode_attention_partial(const void *q, int64_t q_stride, const void *k_cache,
                                 const void *v_cache, const int32_t *block_tables,
                                 int32_t block_table_stride, const int32_t *context_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                 int32_t max_context_len, float scale, int32_t split_tokens,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    pkv::PartialArgs a;
    int rc = setup_partial(a, q, q_stride, k_cache, v_cache, nullptr, nullptr, 0, block_tables,
                           block_table_stride, context_lens, batch, num_q_heads, num_kv_heads,
                           head_dim, block_size, num_blocks, max_context_len, scale,
                           split_tokens, workspace, workspace_bytes, false);
    if (rc || batch == 0) return rc;
    return hip_status(pkv::launch_decode_partial(a, head_dim, stream), "decode partial launch");
}

int pkv_decode_attention_partial_store(const void *q, int64_t q_stride, void *k_cache,
                                       void *v_cache, const void *k_new, const void *v_new,
                                       int64_t new_token_stride, const int32_t *block_tables,
                                       int32_t block_table_stride, const int32_t *context_lens,
                                       int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                       int32_t max_context_len, float scale,
                                       int32_t split_tokens, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream)
{
    pkv::PartialArgs a;
    int rc = setup_partial(a, q, q_stride, k_cache, v_cache, k_new, v_new, new_token_stride,
                           block_tables, block_table_stride, context_lens, batch, num_q_heads,
                           num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                           scale, split_tokens, workspace, workspace_bytes, true);
    if (rc || batch == 0) return rc;
    return hip_status(pkv::launch_decode_partial(a, head_dim, stream),
                      "decode partial (store) launch");
}

int pkv_decode_attention_reduce(void *out, int64_t out_stride, const int32_t *context_lens,
                                int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_table_stride, int32_t block_size,
                                int32_t max_context_len, int32_t split_tokens,
                                const void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_attention_shape(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                   block_table_stride, max_context_len);
    if (rc) return rc;
    if ((rc = check_split(split_tokens))) return rc;
    const int64_t os = out_stride ? out_stride : (int64_t)num_q_heads * head_dim;
    REQUIRE(os >= (int64_t)num_q_heads * head_dim && os % 8 == 0, PKV_ERR_INVALID_ARG,
            "out_stride must be >= num_q_heads*head_dim and a multiple of 8");
    if (batch == 0) return PKV_OK;
    REQUIRE(out && context_lens, PKV_ERR_INVALID_ARG, "null pointer");
    REQUIRE(aligned(out, 16), PKV_ERR_INVALID_ARG, "out must be 16-byte aligned");
    REQUIRE(aligned(context_lens, 4), PKV_ERR_INVALID_ARG, "context_lens must be 4-byte aligned");
    const int32_t split = effective_split(batch, num_q_heads, num_kv_heads, max_context_len, split_tokens);
    const pkv::SplitGeometry g =
        pkv::split_geometry(batch, num_q_heads, head_dim, max_context_len, split);
    REQUIRE(workspace && aligned(workspace, 256), PKV_ERR_WORKSPACE,
            "workspace must be non-null and 256-byte aligned");
    REQUIRE(workspace_bytes >= g.total_bytes, PKV_ERR_WORKSPACE,
            "workspace too small: %zu < %zu bytes", workspace_bytes, g.total_bytes);
    pkv::ReduceArgs a;
    a.out = static_cast<uint16_t *>(out);
    a.out_stride = os;
    a.part_o = static_cast<const float *>(workspace);
    a.part_ml = reinterpret_cast<const float *>(static_cast<const char *>(workspace) +
                                                g.part_o_bytes);
    a.context_lens = context_lens;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.max_len = clamp_len(max_context_len, block_table_stride, block_size);
    a.split_tokens = split;
    a.num_splits = g.num_splits;
    a.prefix_len = 0;
    a.prefix_splits = 0;
    return hip_status(pkv::launch_decode_reduce(a, head_dim, stream), "decode reduce launch");
}

int pkv_varlen_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                            int32_t block_table_stride, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                            int32_t block_size, hipStream_t stream)
{
    REQUIRE(batch >= 0 && max_seqlen_q >= 0, PKV_ERR_INVALID_ARG,
            "batch and max_seqlen_q must be >= 0");
    if (batch == 0 || max_seqlen_q == 0) return PKV_OK;
    REQUIRE(slot_mapping && block_tables && cu_seqlens_q && cu_seqlens_k, PKV_ERR_INVALID_ARG,
            "null pointer");
    REQUIRE(aligned(slot_mapping, 4) && aligned(block_tables, 4) && aligned(cu_seqlens_q, 4) &&
                aligned(cu_seqlens_k, 4),
            PKV_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
    REQUIRE(block_table_stride > 0, PKV_ERR_INVALID_ARG, "block_table_stride must be > 0");
    REQUIRE(pow2(block_size) && block_size <= (1 << 20), PKV_ERR_UNSUPPORTED,
            "block_size %d must be a power of two", block_size);
    return hip_status(pkv::launch_varlen_slot_mapping(slot_mapping, block_tables,
                                                      block_table_stride, cu_seqlens_q,
                                                      cu_seqlens_k, batch, max_seqlen_q,
                                                      block_size, stream),
                      "varlen slot mapping launch");
}

int32_t pkv_varlen_split_tokens(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t split_tokens)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seqlen_q < 0 ||
        max_seqlen_k < 0 || split_tokens < 0 || split_tokens % 256)
        return 0;
    return varlen_effective_split(batch, num_q_heads, num_kv_heads, max_seqlen_q, max_seqlen_k,
                                  split_tokens);
}

size_t pkv_varlen_workspace_bytes(int32_t total_q, int32_t batch, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen_q,
                                  int32_t max_seqlen_k, int32_t split_tokens)
{
    if (total_q < 0 || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_seqlen_q < 0 || max_seqlen_k < 0 || split_tokens < 0 || split_tokens % 256)
        return 0;
    return varlen_geometry(total_q, batch, num_q_heads, num_kv_heads, head_dim, max_seqlen_q,
                           max_seqlen_k, split_tokens)
        .total_bytes;
}

int pkv_varlen_paged_attention(void *out, int64_t out_stride, const void *q, int64_t q_stride,
                               const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, int32_t block_table_stride,
                               const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                               int32_t batch, int32_t total_q, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               float scale, int32_t split_tokens, void *workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_attention_shape(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                   block_table_stride, max_seqlen_k);
    if (rc) return rc;
    REQUIRE(max_seqlen_q >= 0 && total_q >= 0, PKV_ERR_INVALID_ARG,
            "max_seqlen_q and total_q must be >= 0");
    REQUIRE(split_tokens >= 0 && split_tokens % 256 == 0, PKV_ERR_INVALID_ARG,
            "split_tokens must be 0 or a positive multiple of 256");
    REQUIRE(num_blocks > 0, PKV_ERR_INVALID_ARG, "num_blocks must be > 0");
    REQUIRE((int64_t)max_seqlen_q * (num_q_heads / num_kv_heads) <= (1 << 30),
            PKV_ERR_UNSUPPORTED, "max_seqlen_q * group too large");
    const int64_t row = (int64_t)num_q_heads * head_dim;
    const int64_t qs = q_stride ? q_stride : row;
    const int64_t os = out_stride ? out_stride : row;
    REQUIRE(qs >= row && qs % 8 == 0 && os >= row && os % 8 == 0, PKV_ERR_INVALID_ARG,
            "q_stride / out_stride must be >= num_q_heads*head_dim and multiples of 8");
    REQUIRE(isfinite(scale), PKV_ERR_INVALID_ARG, "scale must be finite");
    if (batch == 0 || max_seqlen_q == 0 || total_q == 0) return PKV_OK;
    REQUIRE(out && q && k_cache && v_cache && block_tables && cu_seqlens_q && cu_seqlens_k,
            PKV_ERR_INVALID_ARG, "null pointer");
    REQUIRE(aligned(out, 16) && aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16),
            PKV_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
    REQUIRE(aligned(block_tables, 4) && aligned(cu_seqlens_q, 4) && aligned(cu_seqlens_k, 4),
            PKV_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
    const int32_t max_len = clamp_len(max_seqlen_k, block_table_stride, block_size);
    const VarlenGeometry g = varlen_geometry(total_q, batch, num_q_heads, num_kv_heads, head_dim,
                                             max_seqlen_q, max_len, split_tokens);
    if (g.num_splits > 1) {
        REQUIRE(workspace && aligned(workspace, 256), PKV_ERR_WORKSPACE,
                "workspace must be non-null and 256-byte aligned");
        REQUIRE(workspace_bytes >= g.total_bytes, PKV_ERR_WORKSPACE,
                "workspace too small: %zu < %zu bytes", workspace_bytes, g.total_bytes);
    }
    pkv::PartialArgs a;
    memset(&a, 0, sizeof a);
    a.err = g_err_word;
    a.wait_limit = wait_limit();
    a.q = static_cast<const uint16_t *>(q);
    a.q_stride = qs;
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.block_tables = block_tables;
    a.table_stride = block_table_stride;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.head_chunks = 1;
    a.bs_log2 = __builtin_ctz((unsigned)block_size);
    a.num_blocks = num_blocks;
    a.max_len = max_len;
    a.split_tokens = g.split_tokens;
    a.num_splits = g.num_splits;
    if (g.num_splits > 1) {
        a.part_o = static_cast<float *>(workspace);
        a.part_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + g.part_o_bytes);
    }
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)head_dim);
    a.c = sc * 1.4426950408889634f;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.out = static_cast<uint16_t *>(out);
    a.out_stride = os;
    a.total_q = total_q;
    return hip_status(pkv::launch_varlen_attention(a, head_dim, max_seqlen_q, stream),
                      "varlen attention launch");
}

size_t pkv_cascade_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t max_context_len,
                                   int32_t num_prefix_blocks, int32_t block_size,
                                   int32_t split_tokens)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        head_dim <= 0 || max_context_len < 0 || num_prefix_blocks <= 0 || !pow2(block_size) ||
        (int64_t)num_prefix_blocks * block_size > (1 << 30) || check_split(split_tokens) != PKV_OK)
        return 0;
    return cascade_geometry(batch, num_q_heads, num_kv_heads, head_dim, max_context_len,
                            num_prefix_blocks, block_size, split_tokens)
        .ws.total_bytes;
}

int pkv_cascade_decode_attention(void *out, int64_t out_stride, const void *q, int64_t q_stride,
                                 const void *k_cache, const void *v_cache,
                                 const int32_t *prefix_blocks, int32_t num_prefix_blocks,
                                 const int32_t *block_tables, int32_t block_table_stride,
                                 const int32_t *context_lens, int32_t batch,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks,
                                 int32_t max_context_len, float scale, int32_t split_tokens,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_attention_shape(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                   block_table_stride, max_context_len);
    if (rc) return rc;
    if ((rc = check_split(split_tokens))) return rc;
    REQUIRE(num_prefix_blocks > 0 && (int64_t)num_prefix_blocks * block_size <= (1 << 30),
            PKV_ERR_INVALID_ARG, "num_prefix_blocks must be > 0 (and the prefix < 2^30)");
    const int64_t os = out_stride ? out_stride : (int64_t)num_q_heads * head_dim;
    REQUIRE(os >= (int64_t)num_q_heads * head_dim && os % 8 == 0, PKV_ERR_INVALID_ARG,
            "out_stride must be >= num_q_heads*head_dim and a multiple of 8");
    const int32_t max_len = clamp_len(max_context_len, block_table_stride, block_size);
    const CascadeGeometry cg = cascade_geometry(batch, num_q_heads, num_kv_heads, head_dim, max_len,
                                                num_prefix_blocks, block_size, split_tokens);
    // the ordinary partial arguments cover the positions after the prefix
    pkv::SplitGeometry tail_geo = cg.ws;
    tail_geo.split_tokens = cg.tail_split;
    pkv::PartialArgs a;
    rc = setup_partial(a, q, q_stride, k_cache, v_cache, nullptr, nullptr, 0, block_tables,
                       block_table_stride, context_lens, batch, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, max_context_len, scale, split_tokens,
                       workspace, workspace_bytes, false, &tail_geo);
    if (rc || batch == 0) return rc;
    REQUIRE(out && prefix_blocks, PKV_ERR_INVALID_ARG, "null pointer");
    REQUIRE(aligned(out, 16), PKV_ERR_INVALID_ARG, "out must be 16-byte aligned");
    REQUIRE(aligned(prefix_blocks, 4), PKV_ERR_INVALID_ARG, "prefix_blocks must be 4-byte aligned");

    // one launch: the shared blocks, one workgroup per (prefix split, KV
    // head, query chunk), then each row's positions after the prefix
    a.prefix_blocks = prefix_blocks;
    a.prefix_len = cg.prefix_len;
    a.prefix_split = cg.prefix_split;
    a.vq_per_kv = batch * (num_q_heads / num_kv_heads);
    a.vchunks = cg.vchunks;
    a.pos_base = cg.prefix_len;
    a.split_base = cg.prefix_splits;
    rc = hip_status(pkv::launch_decode_cascade_mfma(a, head_dim, stream), "cascade launch");
    if (rc) return rc;
    pkv::ReduceArgs r;
    r.out = static_cast<uint16_t *>(out);
    r.out_stride = os;
    r.part_o = a.part_o;
    r.part_ml = a.part_ml;
    r.context_lens = context_lens;
    r.batch = batch;
    r.num_q_heads = num_q_heads;
    r.max_len = max_len;
    r.split_tokens = cg.tail_split;
    r.num_splits = cg.num_splits;
    r.prefix_len = cg.prefix_len;
    r.prefix_splits = cg.prefix_splits;
    return hip_status(pkv::launch_decode_reduce(r, head_dim, stream), "cascade reduce launch");
}

int pkv_paged_decode_attention(void *out, int64_t out_stride, const void *q, int64_t q_stride,
                               const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, int32_t block_table_stride,
                               const int32_t *context_lens, int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_context_len, float scale,
                               int32_t split_tokens, void *workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    return decode_attention_combined(out, out_stride, q, q_stride, k_cache, v_cache, nullptr,
                                     nullptr, 0, block_tables, block_table_stride, context_lens,
                                     batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                     num_blocks, max_context_len, scale, split_tokens, workspace,
                                     workspace_bytes, false, stream);
}

int pkv_paged_decode_attention_store(void *out, int64_t out_stride, const void *q,
                                     int64_t q_stride, void *k_cache, void *v_cache,
                                     const void *k_new, const void *v_new,
                                     int64_t new_token_stride, const int32_t *block_tables,
                                     int32_t block_table_stride, const int32_t *context_lens,
                                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                     int32_t max_context_len, float scale, int32_t split_tokens,
                                     void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return decode_attention_combined(out, out_stride, q, q_stride, k_cache, v_cache, k_new, v_new,
                                     new_token_stride, block_tables, block_table_stride,
                                     context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                     block_size, num_blocks, max_context_len, scale, split_tokens,
                                     workspace, workspace_bytes, true, stream);
}

int pkv_paged_decode_attention_store_noalloc(void *out, int64_t out_stride, const void *q,
                                             int64_t q_stride, void *k_cache, void *v_cache,
                                             const void *k_new, const void *v_new,
                                             int64_t new_token_stride,
                                             const int32_t *block_tables,
                                             int32_t block_table_stride,
                                             const int32_t *context_lens, int32_t batch,
                                             int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t block_size,
                                             int64_t num_blocks, int32_t max_context_len,
                                             float scale, int32_t split_tokens,
                                             hipStream_t stream)
{
    // the size of the partials, checked before any HIP call
    int rc = check_attention_shape(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                   block_table_stride, max_context_len);
    if (rc) return rc;
    if ((rc = check_split(split_tokens))) return rc;
    const int32_t split =
        effective_split(batch, num_q_heads, num_kv_heads, max_context_len, split_tokens);
    const size_t need =
        pkv::split_geometry(batch, num_q_heads, head_dim, max_context_len, split).total_bytes;
    REQUIRE(need <= PKV_STATIC_SCRATCH_BYTES, PKV_ERR_WORKSPACE,
            "partials need %zu bytes, more than the library's fixed %u-byte device array; "
            "use pkv_paged_decode_attention_store with a workspace",
            need, (unsigned)PKV_STATIC_SCRATCH_BYTES);
    // every other argument, checked before the first HIP call (the 256-byte
    // stand-in only passes the workspace checks; nothing is launched)
    rc = decode_attention_combined(out, out_stride, q, q_stride, k_cache, v_cache, k_new, v_new,
                                   new_token_stride, block_tables, block_table_stride,
                                   context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                   block_size, num_blocks, max_context_len, scale, split_tokens,
                                   reinterpret_cast<void *>(256), PKV_STATIC_SCRATCH_BYTES, true,
                                   stream, true);
    if (rc || batch == 0) return rc;
    void *scratch = nullptr;
    rc = hip_status(pkv::static_scratch(&scratch), "static scratch address");
    if (rc) return rc;
    return decode_attention_combined(out, out_stride, q, q_stride, k_cache, v_cache, k_new, v_new,
                                     new_token_stride, block_tables, block_table_stride,
                                     context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                     block_size, num_blocks, max_context_len, scale, split_tokens,
                                     scratch, PKV_STATIC_SCRATCH_BYTES, true, stream);
}

size_t pkv_sampler_workspace_bytes(int32_t batch, int32_t vocab)
{
    if (batch < 0 || vocab <= 0 || vocab > (1 << 24)) return 0;
    return pkv::sampler_workspace_bytes(batch, vocab);
}

int pkv_sample_next_token_ex(int32_t *out_ids, const float *logits, int64_t logits_stride,
                             const float *gumbel, int64_t gumbel_stride, const uint8_t *vocab_mask,
                             int64_t mask_stride, const float *temperature, const float *top_p,
                             const int32_t *top_k, int32_t batch, int32_t vocab,
                             float *out_prob, int32_t *out_top_ids, float *out_top_probs,
                             void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    REQUIRE(batch >= 0 && batch <= 65535, PKV_ERR_INVALID_ARG, "batch must be in [0, 65535]");
    REQUIRE(vocab > 0 && vocab <= (1 << 24), PKV_ERR_UNSUPPORTED,
            "vocab %d unsupported (1 .. 2^24)", vocab);
    const int64_t ls = logits_stride ? logits_stride : vocab;
    const int64_t gs = gumbel_stride ? gumbel_stride : vocab;
    const int64_t ms = mask_stride ? mask_stride : vocab;
    REQUIRE(ls >= vocab && gs >= vocab, PKV_ERR_INVALID_ARG, "row strides must be >= vocab");
    REQUIRE(!vocab_mask || ms >= vocab, PKV_ERR_INVALID_ARG, "mask_stride must be >= vocab");
    if (batch == 0) return PKV_OK;
    REQUIRE(out_ids && logits && gumbel && temperature && top_p && top_k, PKV_ERR_INVALID_ARG,
            "null pointer");
    REQUIRE(aligned(out_ids, 4) && aligned(logits, 4) && aligned(gumbel, 4) &&
                aligned(temperature, 4) && aligned(top_p, 4) && aligned(top_k, 4),
            PKV_ERR_INVALID_ARG, "arrays must be 4-byte aligned");
    REQUIRE((!out_prob || aligned(out_prob, 4)) && (!out_top_ids || aligned(out_top_ids, 4)) &&
                (!out_top_probs || aligned(out_top_probs, 4)),
            PKV_ERR_INVALID_ARG, "outputs must be 4-byte aligned");
    const size_t need = pkv::sampler_workspace_bytes(batch, vocab);
    REQUIRE(workspace && aligned(workspace, 256), PKV_ERR_WORKSPACE,
            "workspace must be non-null and 256-byte aligned");
    REQUIRE(workspace_bytes >= need, PKV_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes",
            workspace_bytes, need);
    return hip_status(pkv::launch_sampler(out_ids, logits, ls, gumbel, gs, vocab_mask, ms,
                                          temperature, top_p, top_k, batch, vocab, out_prob,
                                          out_top_ids, out_top_probs, workspace, stream),
                      "sampler launch");
}

int pkv_sample_next_token(int32_t *out_ids, const float *logits, int64_t logits_stride,
                          const float *gumbel, int64_t gumbel_stride, const float *temperature,
                          const float *top_p, const int32_t *top_k, int32_t batch, int32_t vocab,
                          void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return pkv_sample_next_token_ex(out_ids, logits, logits_stride, gumbel, gumbel_stride,
                                    nullptr, 0, temperature, top_p, top_k, batch, vocab, nullptr,
                                    nullptr, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"
