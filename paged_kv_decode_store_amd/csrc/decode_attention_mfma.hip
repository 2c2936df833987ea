// Split-KV paged decode attention, partial step, on the matrix cores.
//
// For larger GQA groups the per-position work of the VALU kernel (a q.k
// dot product, a 16-lane reduction, the softmax update and the P.V
// accumulation, for every query head sharing the KV head) makes it ALU-bound
// instead of HBM-bound.  Here the two contractions of a 16-position chunk
// run as 16x16x16 bf16 MFMAs for up to 16 query heads at once:
//
//   S^T = K Q^T   A = K (16 positions x 16 dims), B = Q^T (16 dims x 16
//                 queries), accumulated over the head dims; the result
//                 layout gives lane l the scores of query l%16 at positions
//                 4*(l/16) + i, i < 4;
//   O  += P V     A = P (16 queries x 16 positions) -- exactly the layout
//                 S^T was produced in, so the probabilities feed the next
//                 MFMA without any exchange -- B = V (16 positions x 16
//                 dims), one MFMA per 16 output dims.
//
// The contraction index of each product may be permuted freely as long as
// both operands agree, which is used twice: for K lane l holds the 16-byte
// pieces 4*w + l/16 (w < D/32) of position l%16's row (and the same dims of
// its query), so each load instruction reads 64 contiguous bytes of every
// position of the chunk; for V it holds 8 (D 128) or 4 (D 64) contiguous
// dims of positions 4*(l/16) + j, so each instruction reads four whole
// rows.  A wave reads each chunk's K and V rows exactly once.
// P is split into a bf16 high part and a bf16 residual, both multiplied, so
// the probabilities keep about 16 significant bits.  The online softmax
// (max, rescale, sum) runs per query on four values per lane.
//
// Workgroup: 4 waves streaming the split's 16-position chunks in turn; the
// waves merge through LDS and write the same partials (max in log2 units,
// sum, unnormalised output) as the VALU kernel, so the reduce step is
// shared.  Query heads beyond 16 per KV head go to further workgroups.
#include <math.h>

#include "launch.hpp"
#include "pkv_device.hpp"

namespace pkv {

namespace {

typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

constexpr int kMWaves = 4;
constexpr int kMChunk = 16;                   // positions per wave iteration
constexpr int kMRound = kMWaves * kMChunk;    // positions per workgroup iteration
constexpr int kMQ = 16;                       // query heads per workgroup

__device__ __forceinline__ s4_t operand(uint32_t lo, uint32_t hi)
{
    return __builtin_bit_cast(s4_t, u2_t{lo, hi});
}

__device__ __forceinline__ f4_t mfma16(s4_t a, s4_t b, f4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}

__device__ __forceinline__ u2_t load_stream8(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u2_t *>(p));
}

// Select the low (H = 0) or high (H = 1) bf16 of x and of y into one pair.
template <int H>
__device__ __forceinline__ uint32_t pair_of(uint32_t x, uint32_t y)
{
    return __builtin_amdgcn_perm(y, x, H ? 0x07060302u : 0x05040100u);
}

// Launch modes of the kernel: the decode partial step, and the cascade's
// prefix and tail steps in one grid (prefix workgroups first).
enum : int { kDecode = 0, kCascade = 1 };

template <int D, bool FUSED, int MODE>
__global__ __launch_bounds__(kMWaves * 64) void decode_partial_mfma_kernel(const PartialArgs a)
{
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(!FUSED || MODE == kDecode, "only the decode step stores");
    // this workgroup runs the cascade's prefix step (always false, at compile
    // time, in the decode step)
    const bool PREFIX = MODE == kCascade && (int)blockIdx.x < a.prefix_wgs;
    constexpr int KD = D / 4;       // K dims per lane (one position)
    constexpr int KW = KD / 2;      // their packed words
    constexpr int KP = KD / 8;      // their 16-byte pieces: piece w is dims 8*(4*w + kb) + [0, 8)
    constexpr int QS = D / 16;      // S^T MFMA steps over the head dims
    constexpr int VD = D / 16;      // V dims per lane and position
    constexpr int NB = D / 16;      // O MFMAs (16 output dims each)

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int ln = lane & 15;       // query (S^T column) / position (K row) / dim block
    const int kb = lane >> 4;

    int x = (MODE == kCascade && !PREFIX) ? (int)blockIdx.x - a.prefix_wgs : (int)blockIdx.x;
    int hc, kvh, b, s;
    if (PREFIX) {
        hc = x % a.vchunks;
        x /= a.vchunks;
        kvh = x % a.num_kv_heads;
        s = x / a.num_kv_heads;
        b = 0;
    } else {
        hc = x % a.head_chunks;
        x /= a.head_chunks;
        kvh = x % a.num_kv_heads;
        x /= a.num_kv_heads;
        b = x % a.batch;
        s = x / a.batch;
        // the KV head rotates with the split: every XCD streams every head
        // (see the VALU partial kernel)
        kvh = (kvh + s) % a.num_kv_heads;
    }

    int n, t_begin, t_end, pos_new = -1;
    if (PREFIX) {
        t_begin = s * a.prefix_split;
        t_end = min(a.prefix_len, t_begin + a.prefix_split);
        n = t_end;
    } else {
        const int n_row = a.context_lens[b];
        n = min(max(n_row, 0), a.max_len);
        t_begin = a.pos_base + s * a.split_tokens;
        // one workgroup per row reports a length outside [0, max_len]
        if (threadIdx.x == 0 && s == 0 && hc == 0 && kvh == 0 && n != n_row)
            report_error(a.err, PKV_DEVERR_CONTEXT_LEN);
        if (t_begin >= n) {
            // direct output (one split per row): an empty row's output is zero
            if (a.out && s == 0) {
                const int nq0 = min(kMQ, a.group - hc * kMQ);
                const int64_t o0 = (int64_t)b * a.out_stride + (int64_t)(kvh * a.group + hc * kMQ) * D;
                for (int idx = threadIdx.x; idx < nq0 * D; idx += kMWaves * 64) a.out[o0 + idx] = 0;
            }
            return;
        }
        if (FUSED && n_row >= 1 && n_row <= n) pos_new = n_row - 1;
        t_end = min(n, t_begin + a.split_tokens);
    }
    const float c = a.c;

    // this lane's query: column ln of the workgroup's 16
    const int qv = hc * kMQ + ln;
    const bool qreal = PREFIX ? qv < a.vq_per_kv : qv < a.group;
    int qrow, qhead, lim;
    if (PREFIX) {
        qrow = qreal ? qv / a.group : 0;
        qhead = kvh * a.group + (qreal ? qv % a.group : 0);
        lim = qreal ? min(t_end, min(max(a.context_lens[qrow], 0), a.max_len)) : 0;
    } else {
        qrow = b;
        qhead = kvh * a.group + (qreal ? qv : 0);
        lim = qreal ? t_end : 0;
    }
    uint32_t q[KW];
    {
        const uint16_t *qp = a.q + (int64_t)qrow * a.q_stride + (int64_t)qhead * D + 8 * kb;
#pragma unroll
        for (int w = 0; w < KP; ++w) {
            const uint4 v = qreal ? *reinterpret_cast<const uint4 *>(qp + 32 * w)
                                  : make_uint4(0u, 0u, 0u, 0u);
            q[4 * w] = v.x;
            q[4 * w + 1] = v.y;
            q[4 * w + 2] = v.z;
            q[4 * w + 3] = v.w;
        }
    }

    f4_t o[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) o[j] = f4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;   // running max of query ln (same in its four lanes)
    float lsum = 0.f;      // this lane's share of query ln's sum

    const int64_t tok_stride = (int64_t)a.num_kv_heads * D;
    const int bs_mask = (1 << a.bs_log2) - 1;
    const int32_t *table = PREFIX ? a.prefix_blocks : a.block_tables + (int64_t)b * a.table_stride;

    if constexpr (FUSED) {
        // Fused store: the workgroup whose range holds the row's new position
        // first writes that position's K/V row (this KV head) into the pool,
        // then streams it back like every other position.  Every query chunk
        // of the KV head writes the same bytes.  The barrier orders the
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

    // a bad block id is noted in a scalar flag and reported after the loop
    bool bad_block = false;
    for (int t0 = t_begin + wave * kMChunk; t0 < t_end; t0 += kMRound) {
        const int raw = load_block_id(table, uniform(t0 >> a.bs_log2));
        const bool blk_ok = raw >= 0 && raw < a.num_blocks;
        bad_block |= !blk_ok;
        const int64_t base = (((int64_t)(blk_ok ? raw : 0) << a.bs_log2) + (t0 & bs_mask)) *
                                 tok_stride + (int64_t)kvh * D;
        // K: position t0 + ln, pieces 4*w + kb.  V: positions t0 + 4*kb + j,
        // dims [ln*VD, ln*VD + VD)
        uint32_t kw[KW];
        uint32_t vw[4][VD / 2];
        {
            const int64_t koff = base + ln * tok_stride + 8 * kb;
#pragma unroll
            for (int w = 0; w < KP; ++w) {
                const uint4 v = load_stream16(a.k_cache + koff + 32 * w);
                kw[4 * w] = v.x;
                kw[4 * w + 1] = v.y;
                kw[4 * w + 2] = v.z;
                kw[4 * w + 3] = v.w;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t off = base + (4 * kb + j) * tok_stride + ln * VD;
                if constexpr (VD == 8) {
                    const uint4 v = load_stream16(a.v_cache + off);
                    vw[j][0] = v.x;
                    vw[j][1] = v.y;
                    vw[j][2] = v.z;
                    vw[j][3] = v.w;
                } else {
                    const u2_t v = load_stream8(a.v_cache + off);
                    vw[j][0] = v.x;
                    vw[j][1] = v.y;
                }
            }
        }

        // scores of query ln at positions t0 + 4*kb + i
        f4_t st = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < QS; ++k)
            st = mfma16(operand(kw[2 * k], kw[2 * k + 1]), operand(q[2 * k], q[2 * k + 1]), st);
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = (t0 + 4 * kb + i < lim) ? st[i] : -INFINITY;

        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__any(mx > m)) {
            const float mn = fmaxf(m, mx);
            const float ref = (mn == -INFINITY) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f((m - ref) * c);
            lsum *= alpha;
            // output row i of this lane is query 4*kb + i, whose factor lives in lane 4*kb + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * kb + i);
#pragma unroll
                for (int j = 0; j < NB; ++j) o[j][i] *= ai;
            }
            m = mn;
        }
        const float mc = (m == -INFINITY) ? 0.f : m * c;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c, -mc));
        lsum += (p[0] + p[1]) + (p[2] + p[3]);
        // P as the A operand: row = query ln, columns = positions 4*kb + i
        const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
        const uint32_t r01 = pack_bf16(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
        const uint32_t r23 = pack_bf16(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
        const s4_t ph = operand(h01, h23), pr = operand(r01, r23);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            // column ln of output block j is dim ln*VD + j
            const int w = j >> 1;
            uint32_t b0, b1;
            if (j & 1) {
                b0 = pair_of<1>(vw[0][w], vw[1][w]);
                b1 = pair_of<1>(vw[2][w], vw[3][w]);
            } else {
                b0 = pair_of<0>(vw[0][w], vw[1][w]);
                b1 = pair_of<0>(vw[2][w], vw[3][w]);
            }
            const s4_t vb = operand(b0, b1);
            o[j] = mfma16(ph, vb, o[j]);
            o[j] = mfma16(pr, vb, o[j]);
        }
    }

    if (bad_block && lane == 0) report_error(a.err, PKV_DEVERR_BLOCK_ID);

    // merge the waves through LDS: o rows are queries 4*kb + i, columns dims
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    __shared__ float s_o[kMWaves][kMQ][D + 4];
    __shared__ float s_m[kMWaves][kMQ];
    __shared__ float s_l[kMWaves][kMQ];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[wave][4 * kb + i][ln * VD + j] = o[j][i];
    if (kb == 0) {
        s_m[wave][ln] = m;
        s_l[wave][ln] = lsum;
    }
    __syncthreads();
    const int nq = PREFIX ? min(kMQ, a.vq_per_kv - hc * kMQ) : min(kMQ, a.group - hc * kMQ);
    for (int idx = threadIdx.x; idx < nq * D; idx += kMWaves * 64) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kMWaves; ++w) M = fmaxf(M, s_m[w][h]);
        const float ref = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kMWaves; ++w) {
            const float e = __builtin_amdgcn_exp2f((s_m[w][h] - ref) * c);
            L += s_l[w][h] * e;
            O += s_o[w][h][d] * e;
        }
        const int v = hc * kMQ + h;
        if (!PREFIX && a.out) {
            // direct output: the only split of the row is already the result
            a.out[(int64_t)b * a.out_stride + (int64_t)(kvh * a.group + v) * D + d] =
                (uint16_t)bf16_round(O / L);
            continue;
        }
        int64_t pidx;
        if (PREFIX) {
            const int rb = v / a.group, rh = kvh * a.group + v % a.group;
            pidx = ((int64_t)rb * a.num_q_heads + rh) * a.num_splits + s;
        } else {
            pidx = ((int64_t)b * a.num_q_heads + kvh * a.group + v) * a.num_splits + a.split_base + s;
        }
        a.part_o[pidx * D + d] = O;
        if (d == 0) {
            a.part_ml[2 * pidx] = M * c;
            a.part_ml[2 * pidx + 1] = L;
        }
    }
}

template <int D, int MODE>
hipError_t launch_mfma_d(const PartialArgs &a, hipStream_t stream)
{
    PartialArgs m = a;
    if constexpr (MODE == kCascade) {
        m.vchunks = (a.vq_per_kv + kMQ - 1) / kMQ;
        m.head_chunks = (a.group + kMQ - 1) / kMQ;
        m.out = nullptr;
        const int64_t pre = (int64_t)((a.prefix_len + a.prefix_split - 1) / a.prefix_split) *
                            a.num_kv_heads * m.vchunks;
        const int64_t tail = (int64_t)(a.num_splits - a.split_base) * a.batch * a.num_kv_heads *
                             m.head_chunks;
        m.prefix_wgs = (int32_t)pre;
        decode_partial_mfma_kernel<D, false, kCascade>
            <<<(unsigned)(pre + tail), kMWaves * 64, 0, stream>>>(m);
    } else {
        m.head_chunks = (a.group + kMQ - 1) / kMQ;
        const int64_t grid = (int64_t)(a.num_splits - a.split_base) * a.batch * a.num_kv_heads *
                             m.head_chunks;
        if (a.k_new)
            decode_partial_mfma_kernel<D, true, kDecode><<<(unsigned)grid, kMWaves * 64, 0, stream>>>(m);
        else
            decode_partial_mfma_kernel<D, false, kDecode><<<(unsigned)grid, kMWaves * 64, 0, stream>>>(m);
    }
    return hipGetLastError();
}

// Slots of a varlen batch's new tokens: token j of sequence b is at position
// k_len - q_len + j of its block table.
__global__ void varlen_slot_mapping_kernel(int32_t *slots, const int32_t *block_tables,
                                           int32_t table_stride, const int32_t *cu_q,
                                           const int32_t *cu_k, int32_t batch, int32_t max_q,
                                           int32_t bs_log2)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)batch * max_q) return;
    const int b = (int)(t / max_q), j = (int)(t % max_q);
    const int q_len = cu_q[b + 1] - cu_q[b];
    if (j >= q_len) return;
    const int k_len = cu_k[b + 1] - cu_k[b];
    const int64_t pos = (int64_t)k_len - q_len + j;
    int32_t slot = -1;
    if (pos >= 0 && (pos >> bs_log2) < table_stride) {
        const int32_t blk = block_tables[(int64_t)b * table_stride + (pos >> bs_log2)];
        const int64_t sl = ((int64_t)blk << bs_log2) + (pos & ((1 << bs_log2) - 1));
        if (blk >= 0 && sl <= 0x7fffffff) slot = (int32_t)sl;
    }
    slots[cu_q[b] + j] = slot;
}

}  // namespace

hipError_t launch_decode_partial_mfma(const PartialArgs &a, int32_t head_dim, hipStream_t stream)
{
    if (a.batch == 0 || a.num_splits <= a.split_base) return hipSuccess;
    if (head_dim == 128) return launch_mfma_d<128, kDecode>(a, stream);
    if (head_dim == 64) return launch_mfma_d<64, kDecode>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_cascade_mfma(const PartialArgs &a, int32_t head_dim, hipStream_t stream)
{
    if (a.batch == 0 || a.prefix_len <= 0) return hipSuccess;
    if (head_dim == 128) return launch_mfma_d<128, kCascade>(a, stream);
    if (head_dim == 64) return launch_mfma_d<64, kCascade>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_varlen_slot_mapping(int32_t *slot_mapping, const int32_t *block_tables,
                                      int32_t table_stride, const int32_t *cu_seqlens_q,
                                      const int32_t *cu_seqlens_k, int32_t batch,
                                      int32_t max_seqlen_q, int32_t block_size,
                                      hipStream_t stream)
{
    if (batch == 0 || max_seqlen_q <= 0) return hipSuccess;
    const int64_t n = (int64_t)batch * max_seqlen_q;
    const unsigned grid = (unsigned)((n + 255) / 256);
    varlen_slot_mapping_kernel<<<grid, 256, 0, stream>>>(slot_mapping, block_tables, table_stride,
                                                         cu_seqlens_q, cu_seqlens_k, batch,
                                                         max_seqlen_q,
                                                         __builtin_ctz((unsigned)block_size));
    return hipGetLastError();
}

}  // namespace pkv
