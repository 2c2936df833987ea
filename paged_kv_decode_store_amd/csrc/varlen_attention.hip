// Varlen multi-query paged attention (chunked prefill over a cached prefix)
// on the gfx950 matrix cores.
//
// Sequence b has q_len new tokens (rows cu_q[b].. of q and out) at the end
// of its k_len cached positions; new token j attends causally to positions
// [0, k_len - q_len + j].  Rows of the computation are (token, query head)
// pairs of one KV head, token-major, so the GQA group's heads share every
// K/V tile.  A workgroup owns 128 such rows of one sequence and KV head and
// streams the causal range of its last token (or one split of it, below) in
// tiles of KT positions, staged through LDS.  Its eight waves form two groups of four
// (32 rows per wave) that take the even and the odd tiles, so each SIMD
// runs two waves whose memory, LDS and matrix-core latencies overlap; each
// group stages its own tiles and synchronises only its own four waves per
// step (an arrival counter in LDS), so the groups are not held in lock-step;
// their softmax states are merged through LDS at the end.
//
// Per tile and wave, two products on v_mfma_f32_32x32x16_bf16 (the gfx950
// double-rate bf16 form):
//
//   S^T = K Q^T   A = K (32 positions x 16 dims, key-major LDS rows), B =
//                 Q^T (16 dims x 32 queries, held in registers); lane l of
//                 the result holds query l%32 at positions 8q + 4(l/32) + r
//                 (item 4q + r);
//   O^T += V^T P^T  A = V^T (32 dims x 16 positions), B = P^T: the scores'
//                 result layout already gives lane l query l%32 at eight
//                 positions per 16-position step, which is exactly a B
//                 operand once the contraction index is permuted to match,
//                 so the probabilities need no exchange.  V is staged in
//                 LDS transposed into words of two adjacent positions at
//                 one dim, so each A operand is two 8-byte LDS reads.
//
// Long causal ranges are split over several workgroups (split_tokens
// positions each, like the split-KV decode): a row tile whose range needs
// one split writes its normalised output directly, the others write fp32
// partials (max in log2 units, sum, unnormalised output) that a merge
// kernel combines by log-sum-exp.  This keeps all CUs busy when few tiles
// carry long cached prefixes and balances tiles of unequal length.
//
// O^T leaves every query's running output in the lanes that own that
// query's scores, so the online-softmax rescale is lane-local.  It is also
// lazy: the reference max only moves when a row's max exceeds it by more
// than 2^8 in probability (or on the first tile), so the exponentials stay
// bounded by 256 and the rescale is rare.  P enters the product rounded to
// bf16, and the softmax sum adds the same rounded values (packed dot
// products with (1, 1)), so numerator and denominator use one P.
#include <math.h>

#include "launch.hpp"
#include "pkv_device.hpp"

namespace pkv {

namespace {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef float f4v_t __attribute__((ext_vector_type(4)));

constexpr int kVRowWaves = 4;                  // waves covering a tile's rows
constexpr int kVRowsW = 32;                    // rows (token, head) per wave
constexpr int kVRows = kVRowWaves * kVRowsW;   // rows per workgroup
constexpr int kVGroups = 2;                    // wave groups splitting the tiles
constexpr int kVGroupThreads = kVRowWaves * 64;
constexpr int kVThreads = kVGroups * kVGroupThreads;

__device__ __forceinline__ f16_t mfma32(bf8_t a, bf8_t b, f16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf8_t as_bf8(u4_t v) { return __builtin_bit_cast(bf8_t, v); }

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}

// max / sum of x over lanes l and l ^ 32.  v_permlane32_swap(x, x) yields
// (x[l], x[l^32]) for l < 32 and (x[l^32], x[l]) above, so one register
// exchange replaces an LDS permute; both lanes get the identical result.
__device__ __forceinline__ float xor32_max(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Low (H = 0) or high (H = 1) bf16 of x and of y as one packed pair.
template <int H>
__device__ __forceinline__ uint32_t pair16(uint32_t x, uint32_t y)
{
    return __builtin_amdgcn_perm(y, x, H ? 0x07060302u : 0x05040100u);
}

template <int D>
struct VarlenTile {
    static constexpr int KT = 8192 / D;           // positions per tile (64 at D 128)
    static constexpr int NKB = KT / 32;           // S^T blocks per tile
    static constexpr int QS = D / 16;             // S^T MFMA steps over the dims
    static constexpr int NOB = D / 32;            // O^T blocks (32 dims each)
    static constexpr int PIECES = D / 8;          // 16-byte pieces per K/V row
    static constexpr int KSTEP = kVGroupThreads / PIECES;  // positions between a thread's K pieces
    static constexpr int K_RS = D + 8;            // K row stride in LDS (bf16)
    // V^T rows (one per dim) of KT/2 position-pair words, padded to KT/2 + 2
    // words, with the word column XORed by V_XOR * (row / 32).  Found by an
    // exhaustive search over strides and swizzle tables under 64 banks of
    // 4 bytes (32 lanes per cycle for 8-byte accesses): both the operand
    // reads (32 lanes on 32 consecutive dims, one column) and the
    // transposing stores (lanes spread over dims and position pairs) are
    // then bank-conflict free.
    static constexpr int V_RS = KT / 2 + 2;
    static constexpr int V_XOR = D == 128 ? 4 : 8;
    static constexpr int K_BYTES = KT * K_RS * 2;
    static constexpr int V_BYTES = D * V_RS * 4;
    static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
    // staging (t = thread index inside its group, each group stages its own
    // tile): 4 K pieces (positions t/PIECES + i*KSTEP) and 4 V pieces
    // (positions 4*(t/PIECES) + i, dims 8*(t%PIECES) + [0, 8)) per thread
    static_assert(KT * PIECES == 4 * kVGroupThreads, "4 K pieces per thread");
    static_assert(V_XOR * (D / 32 - 1) < KT / 2 && V_XOR % 2 == 0, "swizzle stays inside a row");
};

// UB: every tile lies inside one block (block_size >= KT), so a tile's
// block id is one scalar and each staged load is that block's base plus a
// fixed per-lane offset.
template <int D, bool UB>
__global__ __launch_bounds__(kVThreads) void varlen_attention_kernel(const PartialArgs a)
{
    using T = VarlenTile<D>;
    constexpr int KT = T::KT, NKB = T::NKB, QS = T::QS, NOB = T::NOB, PIECES = T::PIECES;
    constexpr int KSTEP = T::KSTEP;
    // two stages, each holding one tile per wave group
    __shared__ __align__(16) unsigned char smem[2 * kVGroups * T::STAGE_BYTES];

    const int lane = threadIdx.x & 63;
    const int wgroup = uniform((int)threadIdx.x / kVGroupThreads);   // even / odd tiles
    const int tid = threadIdx.x - wgroup * kVGroupThreads;           // index inside the group
    const int wave = uniform(tid >> 6);
    const int c = lane & 31;          // query of this lane (S^T / O^T column)
    const int h = lane >> 5;          // half of the contraction slots

    // Grid order (fastest first): (sequence, KV head) pair, row tile from
    // the last one (longest causal range first), split.  Tiles of one pair
    // sit B*Hkv workgroups apart, i.e. on one XCD when B*Hkv % 8 == 0, so
    // they share that XCD's L2 copy of the pair's K/V.
    const int pairs = a.batch * a.num_kv_heads;
    const int pair = blockIdx.x % pairs;
    const int rest = (int)(blockIdx.x / pairs);
    const int tile = a.qchunks - 1 - rest % a.qchunks;
    const int sidx = rest / a.qchunks;    // split of the tile's causal range
    const int b = pair / a.num_kv_heads;
    const int kvh = pair - b * a.num_kv_heads;
    const int g = a.group;

    const int q0 = a.cu_q[b];
    const int q_len = a.cu_q[b + 1] - q0;
    const int k_len = a.cu_k[b + 1] - a.cu_k[b];
    // one workgroup per sequence reports lengths that break the contract
    if (threadIdx.x == 0 && kvh == 0 && rest == 0) {
        if (q_len < 0 || k_len < q_len || q_len > a.max_q) report_error(a.err, PKV_DEVERR_SEQLENS);
        if (k_len > a.max_len) report_error(a.err, PKV_DEVERR_CONTEXT_LEN);
    }
    if (q_len <= 0 || k_len < q_len) return;
    const int cached = k_len - q_len;
    const int row0 = tile * kVRows;
    if (row0 >= q_len * g) return;
    const int j_last = min(q_len - 1, (row0 + kVRows - 1) / g);
    const int t_full = min(cached + j_last + 1, a.max_len);   // the tile's causal range
    if (t_full <= 0) return;
    const int nsplit = (t_full + a.split_tokens - 1) / a.split_tokens;
    if (sidx >= nsplit) return;
    const int t_lo = sidx * a.split_tokens;                    // this split: [t_lo, t_end)
    const int t_end = min(t_full, t_lo + a.split_tokens);
    const int ntiles = (t_end - t_lo + KT - 1) / KT;
    const int nsteps = (ntiles + kVGroups - 1) / kVGroups;   // tiles per group

    // this lane's query row
    const int v = row0 + wave * kVRowsW + c;
    const bool real = v < q_len * g;
    const int jq = real ? v / g : 0;
    const int head = kvh * g + (real ? v - jq * g : 0);
    const int lim = real ? min(t_end, cached + jq + 1) : 0;
    int wave_lim = lim;
    for (int x = 32; x >= 1; x >>= 1) wave_lim = min(wave_lim, __shfl_xor(wave_lim, x));
    wave_lim = uniform(wave_lim);

    // Q^T operands: step w holds dims 8*(2w + h) + [0, 8) of query c
    u4_t qop[QS];
    {
        const uint16_t *qp = a.q + (int64_t)(q0 + jq) * a.q_stride + (int64_t)head * D + 8 * h;
#pragma unroll
        for (int w = 0; w < QS; ++w)
            qop[w] = real ? *reinterpret_cast<const u4_t *>(qp + 16 * w) : u4_t{0u, 0u, 0u, 0u};
    }

    const int tok_stride = a.num_kv_heads * D;
    const int bs_mask = (1 << a.bs_log2) - 1;
    const int32_t *table = a.block_tables + (int64_t)b * a.table_stride;
    const int piece = tid % PIECES;
    const int kq = tid / PIECES;                   // K: first position; V: position quad

    // byte offsets of this thread's staged pieces from its tile's first row
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        koff[i] = (uint32_t)(((kq + i * KSTEP) * tok_stride + piece * 8) * 2);
        voff[i] = (uint32_t)(((4 * kq + i) * tok_stride + piece * 8) * 2);
    }
    // a bad id reads block 0 and is noted (no branch) for one report at the end
    bool bad_block = false;
    auto valid_block = [&](int raw) {
        const bool ok = raw >= 0 && raw < a.num_blocks;
        bad_block |= !ok;
        return ok ? raw : 0;
    };

    // Block ids, read ahead and checked only where used (a range check at
    // the read would become a branch whose wait also drains the tile loads
    // in flight).  Table positions are clamped into [0, t_end).
    struct Ids {
        int blk;       // UB: the tile's block (wave-uniform)
        int kid[4];    // otherwise: per staged K position ...
        int vid;       // ... and per V quad
    };
    auto tile_ids = [&](int t0, Ids &ids) {
        if constexpr (UB) {
            ids.blk = load_block_id(table, min(t0, t_end - 1) >> a.bs_log2);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ids.kid[i] = table[min(t0 + kq + i * KSTEP, t_end - 1) >> a.bs_log2];
            ids.vid = table[min(t0 + 4 * kq, t_end - 1) >> a.bs_log2];
        }
    };
    // global -> registers (every address inside the pool: bad ids read
    // block 0); consumed only when the tile is written to LDS
    auto load_tile = [&](int t0, const Ids &ids, u4_t (&kr)[4], u4_t (&vr)[4]) {
        if constexpr (UB) {
            const int64_t base = ((((int64_t)valid_block(ids.blk)) << a.bs_log2) + (t0 & bs_mask)) *
                                     tok_stride + (int64_t)kvh * D;
            const char *kb = reinterpret_cast<const char *>(a.k_cache + base);
            const char *vb = reinterpret_cast<const char *>(a.v_cache + base);
#pragma unroll
            for (int i = 0; i < 4; ++i) kr[i] = *reinterpret_cast<const u4_t *>(kb + koff[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) vr[i] = *reinterpret_cast<const u4_t *>(vb + voff[i]);
        } else {
            auto addr = [&](int raw, int pos) -> int64_t {
                return ((((int64_t)valid_block(raw)) << a.bs_log2) + (pos & bs_mask)) * tok_stride +
                       (int64_t)kvh * D + piece * 8;
            };
#pragma unroll
            for (int i = 0; i < 4; ++i)
                kr[i] = *reinterpret_cast<const u4_t *>(a.k_cache + addr(ids.kid[i], t0 + kq + i * KSTEP));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vr[i] = *reinterpret_cast<const u4_t *>(a.v_cache + addr(ids.vid, t0 + 4 * kq + i));
        }
    };
    // registers -> LDS: K rows as they are, V transposed into words of two
    // adjacent positions (2kp, 2kp + 1) at one dim.
    auto store_tile = [&](unsigned char *base, int t0, const u4_t (&kr)[4], const u4_t (&vr_in)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u4_t *>(base + ((kq + i * KSTEP) * T::K_RS + piece * 8) * 2) = kr[i];
        u4_t vr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = vr_in[i];
        if (t0 + KT > t_end) {
            // V past t_end is zero (masked probabilities are exact zeros, but
            // the pool bytes there need not be finite); K there only feeds
            // scores that are masked by position anyway
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (t0 + 4 * kq + i >= t_end) vr[i] = u4_t{0u, 0u, 0u, 0u};
        }
        uint32_t *vs = reinterpret_cast<uint32_t *>(base + T::K_BYTES);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const int wi = d >> 1;
            uint32_t w0, w1;
            if (d & 1) {
                w0 = pair16<1>(vr[0][wi], vr[1][wi]);
                w1 = pair16<1>(vr[2][wi], vr[3][wi]);
            } else {
                w0 = pair16<0>(vr[0][wi], vr[1][wi]);
                w1 = pair16<0>(vr[2][wi], vr[3][wi]);
            }
            const int row = piece * 8 + d;
            const int col = (2 * kq) ^ (T::V_XOR * (row >> 5));
            *reinterpret_cast<u2_t *>(vs + row * T::V_RS + col) = u2_t{w0, w1};
        }
    };

    // LDS operand addresses (bytes from a stage's start): K row 32kb + c,
    // dims 8(2w + h); V^T row 32j + c, position-pair columns
    // (8u + 2h + 4e) ^ (V_XOR j).  The swizzle touches bits 2-3 of the word
    // column and 2h only bit 1, so the column is ((8u + 4e) ^ (V_XOR j)) +
    // 2h: a per-lane base plus a constant, i.e. an immediate offset.
    const int k_lds = (c * T::K_RS + 8 * h) * 2;
    const int v_lane = T::K_BYTES + (c * T::V_RS + 2 * h) * 4;
    auto v_lds = [&](int j, int u, int e) -> int {
        return v_lane + (32 * j * T::V_RS + ((8 * u + 4 * e) ^ (T::V_XOR * j))) * 4;
    };

    f16_t o[NOB];
#pragma unroll
    for (int j = 0; j < NOB; ++j) o[j] = f16_t{};
    float mr = -INFINITY;   // reference max of query c (raw score units)
    float lsum = 0.f;       // this lane's share of query c's sum
    const float cs = a.c;
    const float thr = 8.0f / cs;

    // Per-step synchronisation of one wave group only (its four waves stage
    // and read the group's own LDS slots), so that the two groups sharing
    // each SIMD are not held in lock-step by a workgroup-wide barrier.  An
    // arrival counter per group in LDS: each wave adds one and waits for
    // four arrivals per step so far.  The wait is bounded (every wave of a
    // group runs the same number of steps, so all arrive; the cap, 2^22
    // polls unless the caller set another, only guards against a defect
    // turning into a hang).  A wait that gives up is reported in the device
    // error word; no address depends on it.
    __shared__ uint32_t s_gbar[kVGroups];
    if (threadIdx.x < kVGroups) s_gbar[threadIdx.x] = 0;
    uint32_t gen = 0;
    bool gave_up = false;
    const uint32_t polls = a.wait_limit;
    auto group_sync = [&]() {
        ++gen;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_fetch_add(&s_gbar[wgroup], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t target = gen * kVRowWaves;
        bool met = false;
        for (uint32_t spin = 0; spin < polls; ++spin) {
            const uint32_t seen = __hip_atomic_load(&s_gbar[wgroup], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (__builtin_amdgcn_readfirstlane(seen) >= target) {
                met = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        gave_up |= !met;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };

    // stage st, this group's tile slot
    auto slot = [&](int st) { return smem + (st * kVGroups + wgroup) * T::STAGE_BYTES; };

    Ids ids;
    u4_t kr[4], vr[4];
    // group g's tiles are g, g + 2, g + 4, ...
    const int tfirst = t_lo + wgroup * KT;
    const int tlast = t_lo + (ntiles - 1) * KT;
    constexpr int TSTRIDE = kVGroups * KT;
    tile_ids(min(tfirst, tlast), ids);
    load_tile(tfirst, ids, kr, vr);
    if (nsteps > 1) tile_ids(min(tfirst + TSTRIDE, tlast), ids);
    if (tfirst < t_end) store_tile(slot(0), tfirst, kr, vr);
    __syncthreads();

    for (int it = 0; it < nsteps; ++it) {
        const int t0 = tfirst + it * TSTRIDE;
        const bool more = it + 1 < nsteps;
        if (more) {
            load_tile(t0 + TSTRIDE, ids, kr, vr);
            if (it + 2 < nsteps) tile_ids(min(t0 + 2 * TSTRIDE, tlast), ids);
        }
        const unsigned char *st_base = slot(it & 1);

        if (t0 < t_end) {
            // scores of the whole tile, the blocks' MFMA chains interleaved;
            // sts[kb] item 4q + r = query c at position t0 + 32kb + 8q + 4h + r
            f16_t sts[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sts[kb] = f16_t{};
#pragma unroll
            for (int w = 0; w < QS; ++w)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    sts[kb] = mfma32(as_bf8(*reinterpret_cast<const u4_t *>(
                                         st_base + k_lds + (32 * kb * T::K_RS + 16 * w) * 2)),
                                     as_bf8(qop[w]), sts[kb]);
            // causal mask (also covers every position past t_end)
            if (t0 + KT > wave_lim) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int pos = t0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
                        if (pos >= lim) sts[kb][i] = -INFINITY;
                    }
            }
            // one max per tile (tree reductions keep the chains short)
            float m8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                m8[i] = fmaxf(sts[0][2 * i], sts[0][2 * i + 1]);
#pragma unroll
                for (int kb = 1; kb < NKB; ++kb)
                    m8[i] = fmaxf(m8[i], fmaxf(sts[kb][2 * i], sts[kb][2 * i + 1]));
            }
#pragma unroll
            for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < w; ++i) m8[i] = fmaxf(m8[i], m8[i + w]);
            const float mx = xor32_max(m8[0]);
            if (__any(mx > mr + thr)) {
                const float mn = fmaxf(mr, mx);
                const float ref = (mn == -INFINITY) ? 0.f : mn;
                const float alpha = __builtin_amdgcn_exp2f((mr - ref) * cs);
                lsum *= alpha;
#pragma unroll
                for (int j = 0; j < NOB; ++j) o[j] *= alpha;
                mr = mn;
            }
            const float mc = (mr == -INFINITY) ? 0.f : mr * cs;

            // Branch-free from here, so block kb's P.V MFMAs and block kb+1's
            // exponentials share one scheduling region.  O^T += V^T P^T per
            // 16-position step u; slots (h, e) are position 16u + 8(e/4) +
            // 4h + e%4, i.e. word pairs 8u + 2h + {0,1} and 8u + 4 + 2h + {0,1}.
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float p[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sts[kb][i], cs, -mc));
                u4_t pw[2];
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        pw[half][m] = pack2_bf16(p[8 * half + 2 * m], p[8 * half + 2 * m + 1]);
                // the softmax sum, from the same bf16 values that enter P.V
                // (one dot product with the pair (1, 1), bits 0x3f803f80, per
                // packed pair; both operands are passed as 32-bit words: a
                // bf16-vector constant here made the compiler read one pair
                // four times)
                float ps[2] = {0.f, 0.f};
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int m = 0; m < 4; ++m) ps[half] = dot2_bf16(pw[half][m], 0x3f803f80u, ps[half]);
                lsum += ps[0] + ps[1];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int u = 2 * kb + half;
                    const bf8_t pb = as_bf8(pw[half]);
#pragma unroll
                    for (int j = 0; j < NOB; ++j) {
                        const u2_t lo = *reinterpret_cast<const u2_t *>(st_base + v_lds(j, u, 0));
                        const u2_t hi = *reinterpret_cast<const u2_t *>(st_base + v_lds(j, u, 1));
                        o[j] = mfma32(as_bf8(u4_t{lo.x, lo.y, hi.x, hi.y}), pb, o[j]);
                    }
                }
            }
        }

        if (more && t0 + TSTRIDE < t_end) store_tile(slot((it & 1) ^ 1), t0 + TSTRIDE, kr, vr);
        group_sync();
    }
    const bool any_bad = __any(bad_block);   // the whole wave votes, then one lane reports
    if (lane == 0) {
        if (any_bad) report_error(a.err, PKV_DEVERR_BLOCK_ID);
        if (gave_up) report_error(a.err, PKV_DEVERR_WAIT);
    }
    __syncthreads();   // both groups are done with their slots, which the merge reuses

    // merge the odd-tile group into the even-tile group: wave w + 4 holds
    // the same (query, dims) items as wave w, for the other tiles
    {
        // one odd-strided record per lane (NOB*16 outputs, max, sum): the 64
        // lanes of each access land in distinct banks
        float *xo = reinterpret_cast<float *>(smem) + (wave * 64 + lane) * (NOB * 16 + 3);
        if (wgroup == 1) {
#pragma unroll
            for (int j = 0; j < NOB; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) xo[j * 16 + i] = o[j][i];
            xo[NOB * 16] = mr;
            xo[NOB * 16 + 1] = lsum;
        }
        __syncthreads();
        if (wgroup == 1) return;
        const float m2 = xo[NOB * 16], l2 = xo[NOB * 16 + 1];
        const float mn = fmaxf(mr, m2);
        const float ref = (mn == -INFINITY) ? 0.f : mn;
        const float a1 = __builtin_amdgcn_exp2f((mr - ref) * cs);
        const float a2 = __builtin_amdgcn_exp2f((m2 - ref) * cs);
        lsum = lsum * a1 + l2 * a2;
#pragma unroll
        for (int j = 0; j < NOB; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[j][i] = o[j][i] * a1 + xo[j * 16 + i] * a2;
        mr = mn;   // (o, lsum) are now relative to the merged reference
    }

    // O^T block j item 4q + r = dim 32j + 8q + 4h + r
    lsum = xor32_sum(lsum);
    if (!real) return;
    if (nsplit > 1) {
        // partial of split sidx: output relative to 2^(mr * c), its sum, and
        // mr * c (log2 units; -inf when no position of the split is visible)
        const int64_t prow = ((int64_t)(q0 + jq) * a.num_q_heads + head) * a.num_splits + sidx;
        float *po = a.part_o + prow * D + 4 * h;
#pragma unroll
        for (int j = 0; j < NOB; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f4v_t *>(po + 32 * j + 8 * q) =
                    f4v_t{o[j][4 * q], o[j][4 * q + 1], o[j][4 * q + 2], o[j][4 * q + 3]};
        if (h == 0) {
            a.part_ml[2 * prow] = mr == -INFINITY ? -INFINITY : mr * cs;
            a.part_ml[2 * prow + 1] = lsum;
        }
        return;
    }
    // the only split: normalise and write bf16
    const float inv = 1.0f / lsum;
    uint16_t *orow = a.out + (int64_t)(q0 + jq) * a.out_stride + (int64_t)head * D + 4 * h;
#pragma unroll
    for (int j = 0; j < NOB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w0 = bf16_round(o[j][4 * q] * inv) | (bf16_round(o[j][4 * q + 1] * inv) << 16);
            const uint32_t w1 = bf16_round(o[j][4 * q + 2] * inv) | (bf16_round(o[j][4 * q + 3] * inv) << 16);
            *reinterpret_cast<u2_t *>(orow + 32 * j + 8 * q) = u2_t{w0, w1};
        }
}

// Merge of a split row tile's partials: one wave per (token row, query
// head).  The row's sequence is found by binary search in cu_q, its tile and
// causal range are recomputed exactly as the attention kernel derived them,
// and rows whose tile needed a single split (already written) are skipped.
// O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, bf16 (round to nearest
// even).
template <int D>
__global__ __launch_bounds__(256) void varlen_merge_kernel(const PartialArgs a)
{
    constexpr int DPL = D / 64;   // output dims per lane
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= (int64_t)a.total_q * a.num_q_heads) return;
    const int r = (int)(gw / a.num_q_heads);
    const int head = (int)(gw - (int64_t)r * a.num_q_heads);
    int lo = 0, hi = a.batch;   // the last b with cu_q[b] <= r
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu_q[mid] <= r) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int q0 = a.cu_q[b];
    const int q_len = a.cu_q[b + 1] - q0;
    const int k_len = a.cu_k[b + 1] - a.cu_k[b];
    if (q_len <= 0 || k_len < q_len || r - q0 >= q_len) return;
    const int g = a.group;
    const int v = (r - q0) * g + head % g;
    const int tile = v / kVRows;
    const int j_last = min(q_len - 1, (tile * kVRows + kVRows - 1) / g);
    const int t_full = min(k_len - q_len + j_last + 1, a.max_len);
    const int ns = t_full <= 0 ? 0 : (t_full + a.split_tokens - 1) / a.split_tokens;
    if (ns <= 1) return;
    const int64_t base = ((int64_t)r * a.num_q_heads + head) * a.num_splits;
    const float *ml = a.part_ml + 2 * base;
    float M = -INFINITY;
    for (int s2 = lane; s2 < ns; s2 += 64) M = fmaxf(M, ml[2 * s2]);
    M = wave_max(M);   // split 0 always holds position 0, so M is finite
    float L = 0.f;
    for (int s2 = lane; s2 < ns; s2 += 64) L += ml[2 * s2 + 1] * __builtin_amdgcn_exp2f(ml[2 * s2] - M);
    L = wave_sum(L);
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
    const float *po = a.part_o + base * D + lane * DPL;
    for (int s2 = 0; s2 < ns; ++s2) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * s2] - M);
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] += w * po[(int64_t)s2 * D + j];
    }
    uint16_t *orow = a.out + (int64_t)r * a.out_stride + (int64_t)head * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) orow[j] = (uint16_t)bf16_round(acc[j] / L);
}

template <int D>
hipError_t launch_varlen_d(const PartialArgs &a, hipStream_t stream)
{
    const int64_t grid = (int64_t)a.num_splits * a.qchunks * a.batch * a.num_kv_heads;
    if ((1 << a.bs_log2) >= VarlenTile<D>::KT)
        varlen_attention_kernel<D, true><<<(unsigned)grid, kVThreads, 0, stream>>>(a);
    else
        varlen_attention_kernel<D, false><<<(unsigned)grid, kVThreads, 0, stream>>>(a);
    if (a.num_splits > 1) {
        const int64_t rows = (int64_t)a.total_q * a.num_q_heads;
        varlen_merge_kernel<D><<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_varlen_attention(const PartialArgs &a, int32_t head_dim, int32_t max_seqlen_q,
                                   hipStream_t stream)
{
    if (a.batch == 0 || max_seqlen_q <= 0) return hipSuccess;
    PartialArgs m = a;
    m.qchunks = (int32_t)(((int64_t)max_seqlen_q * a.group + kVRows - 1) / kVRows);
    m.max_q = max_seqlen_q;
    if (head_dim == 128) return launch_varlen_d<128>(m, stream);
    if (head_dim == 64) return launch_varlen_d<64>(m, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
