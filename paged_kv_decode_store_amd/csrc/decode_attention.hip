// Split-KV paged decode attention for gfx950.
//
// Partial step: one workgroup per (split, row, KV head, query-head chunk).
// Its four waves stream the split's cached positions in 16-position chunks
// (a chunk never straddles a block because block_size is a power of two
// >= 16).  Inside a wave, a lane group of D/8 lanes owns one position at a
// time and each lane holds 8 of its head dims (one 16-byte load of K and one
// of V), so every K/V byte is fetched from HBM exactly once and shared by
// all G query heads of the KV head.  q.k uses v_dot2_f32_bf16 on the packed
// bf16 pairs and a DPP butterfly inside the 16-lane row; each lane group
// keeps its own online-softmax state (max, sum, 8 output dims per lane),
// merged across groups with shuffles and across waves through LDS at the
// end.  The partial (max in log2 units, sum, unnormalised output) goes to
// the fp32 workspace.
//
// Shared-prefix (cascade) decode: the prefix launch (matrix-core kernel)
// writes one partial per (row, query head) and prefix split; this kernel,
// started at pos_base with its slots after the prefix ones, covers each
// row's own positions, and the reduce merges both kinds of partial alike.
//
// Reduce step: one wave per (row, query head) merges the row's partials,
// O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, and writes bf16.
#include <math.h>

#include <type_traits>

#include "launch.hpp"
#include "pkv_device.hpp"

namespace pkv {

constexpr int kWaves = 4;                 // waves per partial workgroup
constexpr int kChunk = 16;                // positions per wave iteration
constexpr int kRound = kWaves * kChunk;   // positions per workgroup iteration

template <int D, int G, bool FUSED>
__global__ __launch_bounds__(kWaves * 64) void decode_partial_kernel(const PartialArgs a)
{
    constexpr int LPT = D / 8;        // lanes per position
    constexpr int GPW = 64 / LPT;     // lane groups per wave
    constexpr int U = kChunk / GPW;   // positions per lane group per iteration
    static_assert(GPW * U == kChunk, "chunk geometry");

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int gi = lane / LPT;
    const int li = lane % LPT;

    // Consecutive workgroups go to different XCDs, so without a rotation
    // XCD j would stream only KV head j.  Heads sit at fixed offsets inside
    // each token row, and on MI355X some offsets stream measurably slower
    // (~25% for two of eight 256-byte offsets), which left the XCDs holding
    // those heads finishing last; rotating the head by the split index gives
    // every XCD every head.
    int x = blockIdx.x;
    const int hc = x % a.head_chunks;
    x /= a.head_chunks;
    const int kv_slot = x % a.num_kv_heads;
    x /= a.num_kv_heads;
    const int b = x % a.batch;
    const int s = x / a.batch;
    const int kvh = (kv_slot + s) % a.num_kv_heads;

    const int n_row = a.context_lens[b];
    const int n = min(max(n_row, 0), a.max_len);
    const int t_begin = a.pos_base + s * a.split_tokens;
    const int h0 = kvh * a.group + hc * G;
    // one workgroup per row reports a length outside [0, max_len]
    if (threadIdx.x == 0 && s == 0 && kv_slot == 0 && hc == 0 && n != n_row)
        report_error(a.err, PKV_DEVERR_CONTEXT_LEN);
    if (t_begin >= n) {
        // direct output (one split per row): an empty row's output is zero
        if (a.out && s == 0)
            for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64)
                a.out[(int64_t)b * a.out_stride + (int64_t)h0 * D + idx] = 0;
        return;
    }
    // fused store: the row's new position, if it lies inside the attended range
    const int pos_new = (FUSED && n_row >= 1 && n_row <= n) ? n_row - 1 : -1;
    const int t_end = min(n, t_begin + a.split_tokens);
    const float c = a.c;

    uint4 qv[G];
    {
        const uint16_t *qrow = a.q + (int64_t)b * a.q_stride + (int64_t)h0 * D + li * 8;
#pragma unroll
        for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const uint4 *>(qrow + h * D);
    }

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[h][d] = 0.f;
    }

    const int64_t tok_stride = (int64_t)a.num_kv_heads * D;
    const int64_t lane_off = (int64_t)kvh * D + li * 8 + (int64_t)(gi * U) * tok_stride;
    const int bs_mask = (1 << a.bs_log2) - 1;
    const int32_t *table = a.block_tables + (int64_t)b * a.table_stride;

    // Issue the K/V loads of the chunk starting at t0 (one block, U positions
    // per lane group, one 16-byte piece per lane and position).  A bad block
    // id is only noted here (a scalar flag, no branch in the loop) and
    // reported once after it.
    bool bad_block = false;
    auto load_chunk = [&](int t0, uint4 (&kr)[U], uint4 (&vr)[U]) {
        const int raw = load_block_id(table, uniform(t0 >> a.bs_log2));
        const bool blk_ok = raw >= 0 && raw < a.num_blocks;
        bad_block |= !blk_ok;
        const int blk = blk_ok ? raw : 0;
        const int64_t base =
            (((int64_t)blk << a.bs_log2) + (t0 & bs_mask)) * tok_stride + lane_off;
#pragma unroll
        for (int u = 0; u < U; ++u)
            kr[u] = load_stream16(a.k_cache + base + u * tok_stride);
#pragma unroll
        for (int u = 0; u < U; ++u)
            vr[u] = load_stream16(a.v_cache + base + u * tok_stride);
    };

    // Online softmax over one chunk.  The running max of a lane group only
    // moves when one of its scores exceeds it; the rescale of (l, o) is done
    // only in waves where some group's max moved (a wave-uniform branch).
    auto compute_chunk = [&](int t0, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
        const int tg = t0 + gi * U;
        float vf[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vf[u][0] = bf16_lo(vr[u].x);
            vf[u][1] = bf16_hi(vr[u].x);
            vf[u][2] = bf16_lo(vr[u].y);
            vf[u][3] = bf16_hi(vr[u].y);
            vf[u][4] = bf16_lo(vr[u].z);
            vf[u][5] = bf16_hi(vr[u].z);
            vf[u][6] = bf16_lo(vr[u].w);
            vf[u][7] = bf16_hi(vr[u].w);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float sc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float acc = dot2_bf16(qv[h].x, kr[u].x, 0.f);
                acc = dot2_bf16(qv[h].y, kr[u].y, acc);
                acc = dot2_bf16(qv[h].z, kr[u].z, acc);
                acc = dot2_bf16(qv[h].w, kr[u].w, acc);
                acc = group_sum<LPT>(acc);
                sc[u] = (tg + u < t_end) ? acc : -INFINITY;
            }
            float mx = m[h];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u]);
            if (__any(mx > m[h])) {
                const float ref = (mx == -INFINITY) ? 0.f : mx;
                const float alpha = __builtin_amdgcn_exp2f((m[h] - ref) * c);
                l[h] *= alpha;
#pragma unroll
                for (int d = 0; d < 8; ++d) o[h][d] *= alpha;
                m[h] = mx;
            }
            const float mc = (m[h] == -INFINITY) ? 0.f : m[h] * c;
            float p[U], psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = __builtin_amdgcn_exp2f(fmaf(sc[u], c, -mc));
                psum += p[u];
            }
            l[h] += psum;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                float acc = o[h][d];
#pragma unroll
                for (int u = 0; u < U; ++u) acc = fmaf(p[u], vf[u][d], acc);
                o[h][d] = acc;
            }
        }
    };

    if constexpr (FUSED) {
        // Fused store: the workgroup whose range holds the row's new position
        // first writes that position's K/V row (this KV head) into the pool,
        // then streams it back like every other position.  Every query-head
        // chunk of the KV head writes the same bytes.  The barrier orders the
        // stores before the other waves' loads: all waves of a workgroup run
        // on one CU and share its write-through vector L1.
        if (pos_new >= t_begin && pos_new < t_end) {
            const int raw = load_block_id(table, pos_new >> a.bs_log2);
            constexpr int PIECES = D / 8;
            if (raw >= 0 && raw < a.num_blocks && (int)threadIdx.x < 2 * PIECES) {
                const bool isv = (int)threadIdx.x >= PIECES;
                const int piece = (int)threadIdx.x - (isv ? PIECES : 0);
                const int64_t dst = (((int64_t)raw << a.bs_log2) + (pos_new & bs_mask)) * tok_stride +
                                    (int64_t)kvh * D + piece * 8;
                const int64_t src = (int64_t)b * a.new_stride + (int64_t)kvh * D + piece * 8;
                const uint4 v = *reinterpret_cast<const uint4 *>((isv ? a.v_new : a.k_new) + src);
                *reinterpret_cast<uint4 *>((isv ? a.v_cache_w : a.k_cache_w) + dst) = v;
            }
            __syncthreads();
        }
    }

    // One chunk per wave iteration: loads, then the online-softmax update.
    for (int t0 = t_begin + wave * kChunk; t0 < t_end; t0 += kRound) {
        uint4 ka[U], va[U];
        load_chunk(t0, ka, va);
        compute_chunk(t0, ka, va);
    }
    if (bad_block && lane == 0) report_error(a.err, PKV_DEVERR_BLOCK_ID);

    // merge the lane groups of this wave
#pragma unroll
    for (int xo = LPT; xo < 64; xo <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m2 = __shfl_xor(m[h], xo);
            const float l2 = __shfl_xor(l[h], xo);
            const float mn = fmaxf(m[h], m2);
            const float ref = (mn == -INFINITY) ? 0.f : mn;
            const float a1 = __builtin_amdgcn_exp2f((m[h] - ref) * c);
            const float a2 = __builtin_amdgcn_exp2f((m2 - ref) * c);
            l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
            for (int d = 0; d < 8; ++d) o[h][d] = o[h][d] * a1 + __shfl_xor(o[h][d], xo) * a2;
            m[h] = mn;
        }
    }

    // merge the waves through LDS and write the partial
    __shared__ float s_o[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];
    if (gi == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float4 *dst = reinterpret_cast<float4 *>(&s_o[wave][h][li * 8]);
            dst[0] = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
            dst[1] = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
            if (li == 0) {
                s_m[wave][h] = m[h];
                s_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();
    const int64_t pbase = ((int64_t)b * a.num_q_heads + h0) * a.num_splits + a.split_base + s;
    for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
        // a head whose waves all saw no position keeps M = -inf, l = 0, o = 0
        const float ref = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = __builtin_amdgcn_exp2f((s_m[w][h] - ref) * c);
            L += s_l[w][h] * e;
            O += s_o[w][h][d] * e;
        }
        if (a.out) {
            // direct output: the only split of the row is already the result
            a.out[(int64_t)b * a.out_stride + (int64_t)(h0 + h) * D + d] = (uint16_t)bf16_round(O / L);
            continue;
        }
        const int64_t pidx = pbase + (int64_t)h * a.num_splits;
        a.part_o[pidx * D + d] = O;
        if (d == 0) {
            a.part_ml[2 * pidx] = M * c;
            a.part_ml[2 * pidx + 1] = L;
        }
    }
}

template <int D, int SPEC>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const ReduceArgs a)
{
    constexpr int DPL = D / 64;  // output dims per lane
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= a.batch * a.num_q_heads) return;
    const int b = gw / a.num_q_heads;
    const int h = gw - b * a.num_q_heads;
    // The first kSpec slots' partials and every lane's (m, l) are requested
    // together with the row length, before it is known how many are in use
    // (slots past the row's count hold stale data inside the workspace and
    // are masked below): one memory round trip instead of three.  kSpec is
    // chosen by the launcher to cover the workspace's slots (8, 24 or 48):
    // more unrolled slots than there are cost time.
    constexpr int kSpec = SPEC;
    const int S = a.num_splits;
    const int64_t base = ((int64_t)b * a.num_q_heads + h) * S;
    const float *ml = a.part_ml + 2 * base;
    const float *po = a.part_o + base * D + lane * DPL;
    float mv = -INFINITY, lv = 0.f;
    if (lane < S) {
        mv = ml[2 * lane];
        lv = ml[2 * lane + 1];
    }
    float v[kSpec][DPL];
#pragma unroll
    for (int k = 0; k < kSpec; ++k)
#pragma unroll
        for (int j = 0; j < DPL; ++j) v[k][j] = k < S ? po[(int64_t)k * D + j] : 0.f;
    const int n = min(max(a.context_lens[b], 0), a.max_len);
    const int tail = max(n - a.prefix_len, 0);
    const int ns = n == 0 ? 0 : a.prefix_splits + (tail + a.split_tokens - 1) / a.split_tokens;
    uint16_t *orow = a.out + (int64_t)b * a.out_stride + (int64_t)h * D + lane * DPL;
    if (ns == 0) {
        // an inactive row attends over nothing: the output is the zero vector
#pragma unroll
        for (int j = 0; j < DPL; ++j) orow[j] = 0;
        return;
    }
    float M = lane < ns ? mv : -INFINITY;
    for (int s2 = lane + 64; s2 < ns; s2 += 64) M = fmaxf(M, ml[2 * s2]);
    M = wave_max(M);
    float L = lane < ns ? lv * __builtin_amdgcn_exp2f(mv - M) : 0.f;
    for (int s2 = lane + 64; s2 < ns; s2 += 64) L += ml[2 * s2 + 1] * __builtin_amdgcn_exp2f(ml[2 * s2] - M);
    L = wave_sum(L);
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
#pragma unroll
    for (int k = 0; k < kSpec; ++k) {
        const float mk = read_lane(mv, k);   // split k's max, held by lane k
        if (k < ns) {
            const float w = __builtin_amdgcn_exp2f(mk - M);
#pragma unroll
            for (int j = 0; j < DPL; ++j) acc[j] += w * v[k][j];
        }
    }
    // the remaining splits, eight per step so that their loads are in flight together
    int s = kSpec;
    for (; s + 8 <= ns; s += 8) {
        float w[8], u[8][DPL];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            w[k] = __builtin_amdgcn_exp2f(ml[2 * (s + k)] - M);
#pragma unroll
            for (int j = 0; j < DPL; ++j) u[k][j] = po[(int64_t)(s + k) * D + j];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int j = 0; j < DPL; ++j) acc[j] += w[k] * u[k][j];
    }
    for (; s < ns; ++s) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] += w * po[(int64_t)s * D + j];
    }
    if constexpr (DPL == 2) {
        const uint32_t lo = bf16_round(acc[0] / L), hi = bf16_round(acc[1] / L);
        *reinterpret_cast<uint32_t *>(orow) = lo | (hi << 16);
    } else {
        orow[0] = (uint16_t)bf16_round(acc[0] / L);
    }
}

// ---- host side ------------------------------------------------------------

int32_t auto_split_tokens(int32_t batch, int32_t num_kv_heads, int32_t max_context_len,
                          int32_t group)
{
    // Measured on MI355X: the VALU partial kernel runs best with roughly
    // 1-2k non-empty workgroups, about 9/32768 of B * Hkv * max_len
    // positions each (Qwen3-shaped, 3 repeats each: 88.4 us per layer at
    // 576 positions, 89.1 at 448, 90.5 at 512, 91.3 at 640, 92.2 at 768,
    // 5.0 TB/s at 1024).  The
    // matrix-core kernel (group >= kMfmaMinGroup) holds only two or three
    // workgroups per CU and streams best with long splits: 3/8192 of
    // B * Hkv * max_len positions each, at least 1024 (Grok-shaped, one
    // 2048-position row per KV head: 46 us at 1024 vs 50 at 2048 and 54 at
    // 512; long contexts: 576 us at 3072 vs 590 at 2048 and 626 at 1024).
    if (max_context_len <= 0 || batch <= 0 || num_kv_heads <= 0) return kRound;
    const bool mfma = group >= kMfmaMinGroup;
    const int64_t work = (int64_t)batch * num_kv_heads * max_context_len;
    int64_t split = mfma ? work * 3 / 8192 : work * 9 / 32768;
    const int64_t lo = mfma ? 1024 : 128;
    if (split < lo) split = lo;
    if (split > 8192) split = 8192;
    split = ((split + kRound - 1) / kRound) * kRound;
    // no longer than the longest row needs
    const int64_t cap = ((int64_t)max_context_len + kRound - 1) / kRound * kRound;
    if (split > cap) split = cap;
    return (int32_t)split;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SplitGeometry split_geometry(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                             int32_t max_context_len, int32_t split_tokens)
{
    SplitGeometry g;
    g.split_tokens = split_tokens;
    const int64_t ml = max_context_len > 0 ? max_context_len : 0;
    g.num_splits = (int32_t)((ml + split_tokens - 1) / split_tokens);
    if (g.num_splits < 1) g.num_splits = 1;
    const size_t units = (size_t)batch * num_q_heads * g.num_splits;
    g.part_o_bytes = align256(units * head_dim * sizeof(float));
    g.part_ml_bytes = align256(units * 2 * sizeof(float));
    g.total_bytes = g.part_o_bytes + g.part_ml_bytes;
    return g;
}

template <int D, int G>
static void launch_partial_g(const PartialArgs &a, hipStream_t stream)
{
    // splits after pos_base (all splits when pos_base = 0) x rows x KV heads x head chunks
    const int64_t grid =
        (int64_t)(a.num_splits - a.split_base) * a.batch * a.num_kv_heads * a.head_chunks;
    if (a.k_new)
        decode_partial_kernel<D, G, true><<<(unsigned)grid, kWaves * 64, 0, stream>>>(a);
    else
        decode_partial_kernel<D, G, false><<<(unsigned)grid, kWaves * 64, 0, stream>>>(a);
}

template <int D>
static hipError_t launch_partial_d(const PartialArgs &a, int G, hipStream_t stream)
{
    switch (G) {
    case 1: launch_partial_g<D, 1>(a, stream); break;
    case 2: launch_partial_g<D, 2>(a, stream); break;
    case 3: launch_partial_g<D, 3>(a, stream); break;
    case 4: launch_partial_g<D, 4>(a, stream); break;
    case 5: launch_partial_g<D, 5>(a, stream); break;
    case 6: launch_partial_g<D, 6>(a, stream); break;
    case 7: launch_partial_g<D, 7>(a, stream); break;
    case 8: launch_partial_g<D, 8>(a, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_partial(const PartialArgs &a, int32_t head_dim, hipStream_t stream)
{
    if (a.batch == 0 || a.num_splits <= a.split_base) return hipSuccess;
    if (a.group >= kMfmaMinGroup) return launch_decode_partial_mfma(a, head_dim, stream);
    const int G = a.group / a.head_chunks;
    if (head_dim == 128) return launch_partial_d<128>(a, G, stream);
    if (head_dim == 64) return launch_partial_d<64>(a, G, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_reduce(const ReduceArgs &a, int32_t head_dim, hipStream_t stream)
{
    if (a.batch == 0) return hipSuccess;
    const int64_t waves = (int64_t)a.batch * a.num_q_heads;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    auto go = [&](auto d) {
        constexpr int D = decltype(d)::value;
        if (a.num_splits <= 8)
            decode_reduce_kernel<D, 8><<<grid, 256, 0, stream>>>(a);
        else if (a.num_splits <= 24)
            decode_reduce_kernel<D, 24><<<grid, 256, 0, stream>>>(a);
        else
            decode_reduce_kernel<D, 48><<<grid, 256, 0, stream>>>(a);
    };
    if (head_dim == 128)
        go(std::integral_constant<int, 128>{});
    else if (head_dim == 64)
        go(std::integral_constant<int, 64>{});
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pkv
