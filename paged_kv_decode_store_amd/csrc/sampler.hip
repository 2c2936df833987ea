// Next-token sampler: temperature, top-k, nucleus (top-p) and a Gumbel-max
// draw, on fp32 logits [B][V].
//
// Row-parallel passes split each row into chunks of `chunk` logits, one
// 256-thread workgroup per (chunk, row).  Each thread first loads its whole
// share of the chunk into registers (float4 when rows are 16-byte aligned)
// and then recomputes s = z / T (IEEE division) and the order-preserving
// 32-bit key of s.  Thresholds come from a three-level radix select on the
// key (11 + 11 + 10 bits): a histogram pass counts the keys that match the
// prefix chosen so far into 2048 digits (global atomics), and a per-row
// select kernel (one workgroup per row) scans the histogram and fixes the
// next digit.  Top-k ranks by count; top-p accumulates the mass exp(s - max)
// in 2^-40 fixed point, so the sums are exact, independent of order and
// identical from run to run.  A top-k tie at the k-th key is cut by index
// with one more count pass.  The final pass takes the argmax of
// fl32(s + g) over the eligible logits as a 64-bit atomic max of
// (key, ~index), which resolves ties to the lowest index.
//
// Passes communicate only through kernel boundaries: no workgroup waits for
// or fences against another one inside a kernel.
#include <math.h>

#include "launch.hpp"
#include "pkv_device.hpp"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kDigits = 2048;
constexpr int kDigitsPerThread = kDigits / kThreads;
constexpr int kMaxPer = 32;  // logits per thread per chunk (chunk <= 8192)

enum : uint32_t { MODE_GREEDY = 1, MODE_TOPK = 2, MODE_TOPP = 4, MODE_TOPP_MAX = 8 };
enum : int { WHICH_K = 0, WHICH_P = 1 };

struct alignas(64) SampCtl {
    unsigned long long best;  // packed (key, ~index) of the draw
    unsigned long long Z;     // kept mass, 2^-40 units
    unsigned long long A;     // mass strictly above the current top-p bucket
    uint32_t max_key;         // key of max s
    uint32_t pad;
    uint32_t mode;
    uint32_t k_prefix;        // top-k: digits fixed so far
    uint32_t k_rank;          // rank still needed inside the prefix bucket
    uint32_t k_key;           // key of the k-th largest s
    uint32_t k_cut;           // last kept index among keys == k_key
    uint32_t k_tie;           // equal keys still to keep, when a cut is needed
    uint32_t p_prefix;        // top-p: digits fixed so far
    uint32_t p_key;           // key of tau
};
static_assert(sizeof(SampCtl) == 64, "control block");

struct SampLayout {
    int32_t chunk;
    int32_t nchunks;
    size_t ctl_off, cnt_off, mass_off, chunk_off, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SampLayout sampler_layout(int32_t batch, int32_t vocab)
{
    SampLayout L;
    // the largest chunk that still gives >= 1024 workgroups per pass
    int32_t chunk = 8192;
    while (chunk > 1024 && (int64_t)batch * ((vocab + chunk - 1) / chunk) < 1024) chunk >>= 1;
    L.chunk = chunk;
    L.nchunks = (vocab + chunk - 1) / chunk;
    size_t off = 0;
    L.ctl_off = off;
    off = align256(off + (size_t)batch * sizeof(SampCtl));
    L.cnt_off = off;
    off = align256(off + (size_t)batch * kDigits * sizeof(uint32_t));
    L.mass_off = off;
    off = align256(off + (size_t)batch * kDigits * sizeof(unsigned long long));
    L.chunk_off = off;
    off = align256(off + (size_t)batch * L.nchunks * sizeof(uint32_t));
    L.total = off;
    return L;
}

struct SampArgs {
    int32_t *out_ids;
    const float *logits;
    int64_t lstride;
    const float *gumbel;
    int64_t gstride;
    const float *temperature;
    const float *top_p;
    const int32_t *top_k;
    int32_t batch, vocab, chunk, nchunks;
    uint32_t flags;
    SampCtl *ctl;
    uint32_t *cnt;
    unsigned long long *mass;
    uint32_t *chunk_cnt;
};

__device__ __forceinline__ unsigned long long pack_key_index(uint32_t key, uint32_t i)
{
    return ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - i);
}

// exp(s - M) in 2^-40 fixed point; the fp32 rounding error of s - M is
// recovered exactly (TwoSum) and folded in to first order.
__device__ __forceinline__ unsigned long long mass_fixed(float s, float M)
{
    const float d = s - M;
    const float bb = d - s;
    const float e = (s - (d - bb)) + (-M - bb);
    float w = expf(d);
    w = fmaf(w, e, w);
    return (unsigned long long)(w * 1099511627776.0f);
}

template <typename T>
__device__ T block_sum(T v, T *scratch)
{
    __syncthreads();
    scratch[threadIdx.x] = v;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) scratch[threadIdx.x] += scratch[threadIdx.x + off];
        __syncthreads();
    }
    const T r = scratch[0];
    __syncthreads();
    return r;
}

template <typename T>
__device__ T block_max(T v, T *scratch)
{
    __syncthreads();
    scratch[threadIdx.x] = v;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off)
            scratch[threadIdx.x] = max(scratch[threadIdx.x], scratch[threadIdx.x + off]);
        __syncthreads();
    }
    const T r = scratch[0];
    __syncthreads();
    return r;
}

// Inclusive scan over threads, ascending (REVERSE = false) or descending.
template <typename T, bool REVERSE>
__device__ T block_scan_inclusive(T v, T *scratch)
{
    __syncthreads();
    const int t = REVERSE ? kThreads - 1 - (int)threadIdx.x : (int)threadIdx.x;
    scratch[t] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const T add = (t >= off) ? scratch[t - off] : T(0);
        __syncthreads();
        scratch[t] += add;
        __syncthreads();
    }
    const T r = scratch[t];
    __syncthreads();
    return r;
}

// Each thread's share of one chunk (chunk / 256 <= 32 logits), loaded into
// registers before any of it is used so that all loads of a pass are in
// flight together.  VEC4: consecutive threads read consecutive float4s
// (rows 16-byte aligned, vocab a multiple of 4); otherwise single floats.
template <bool VEC4>
struct Tile {
    float v[kMaxPer];

    __device__ __forceinline__ static int index(int i0, int j)
    {
        if constexpr (VEC4)
            return i0 + ((j >> 2) * kThreads + (int)threadIdx.x) * 4 + (j & 3);
        else
            return i0 + j * kThreads + (int)threadIdx.x;
    }

    __device__ __forceinline__ void load(const float *__restrict__ row, int i0, int i1, int per)
    {
        if constexpr (VEC4) {
#pragma unroll
            for (int q = 0; q < kMaxPer / 4; ++q) {
                const int i = index(i0, 4 * q);
                float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
                if (4 * q < per && i < i1) f = *reinterpret_cast<const float4 *>(row + i);
                v[4 * q] = f.x;
                v[4 * q + 1] = f.y;
                v[4 * q + 2] = f.z;
                v[4 * q + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j) {
                const int i = index(i0, j);
                v[j] = (j < per && i < i1) ? row[i] : 0.f;
            }
        }
    }
};

__global__ __launch_bounds__(kThreads) void samp_init_kernel(const SampArgs a)
{
    const int b = blockIdx.x;
    for (int d = threadIdx.x; d < kDigits; d += kThreads) {
        a.cnt[(int64_t)b * kDigits + d] = 0;
        a.mass[(int64_t)b * kDigits + d] = 0;
    }
    if (threadIdx.x == 0) {
        SampCtl c = {};
        const float T = a.temperature[b];
        if (!(T > 0.f)) {
            c.mode = MODE_GREEDY;
        } else {
            const int32_t k = a.top_k[b];
            if ((a.flags & 1u) && k > 0 && k < a.vocab) {
                c.mode |= MODE_TOPK;
                c.k_rank = (uint32_t)k;
            }
            const float p = a.top_p[b];
            if ((a.flags & 2u) && p < 1.f) c.mode |= (p > 0.f) ? MODE_TOPP : MODE_TOPP_MAX;
        }
        c.k_cut = 0xffffffffu;
        a.ctl[b] = c;
    }
}

// max key of s over the row (needed for top-p masses and the p <= 0 case)
template <bool VEC4>
__global__ __launch_bounds__(kThreads) void samp_max_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    if (!(ctl->mode & (MODE_TOPP | MODE_TOPP_MAX))) return;
    __shared__ uint32_t s_red[kThreads];
    const float T = a.temperature[b];
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    const int per = a.chunk / kThreads;
    Tile<VEC4> t;
    t.load(a.logits + (int64_t)b * a.lstride, i0, i1, per);
    uint32_t kmax = 0;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
        if (j < per && Tile<VEC4>::index(i0, j) < i1) kmax = max(kmax, float_key(t.v[j] / T));
    kmax = block_max(kmax, s_red);
    if (threadIdx.x == 0) atomicMax(&ctl->max_key, kmax);
}

// One radix level: histogram of the digit (key >> shift) & mask over the
// keys that match the prefix fixed so far.
template <int WHICH, bool VEC4>
__global__ __launch_bounds__(kThreads) void samp_hist_kernel(const SampArgs a, int level)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    const uint32_t mode = ctl->mode;
    if (WHICH == WHICH_K && !(mode & MODE_TOPK)) return;
    if (WHICH == WHICH_P && !(mode & MODE_TOPP)) return;

    __shared__ uint32_t s_cnt[kDigits];
    __shared__ unsigned long long s_mass[WHICH == WHICH_P ? kDigits : 1];
    __shared__ unsigned long long s_red[kThreads];

    const float T = a.temperature[b];
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    const int per = a.chunk / kThreads;
    Tile<VEC4> t;
    t.load(a.logits + (int64_t)b * a.lstride, i0, i1, per);

    for (int d = threadIdx.x; d < kDigits; d += kThreads) {
        s_cnt[d] = 0;
        if (WHICH == WHICH_P) s_mass[d] = 0;
    }
    __syncthreads();

    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const int width = level == 2 ? 10 : 11;
    const int hi = shift + width;
    const uint32_t dmask = (1u << width) - 1u;
    const uint32_t prefix = WHICH == WHICH_K ? ctl->k_prefix : ctl->p_prefix;
    const float M = key_float(ctl->max_key);
    const uint32_t kkey = ctl->k_key, kcut = ctl->k_cut;
    const bool topk = (mode & MODE_TOPK) != 0;

    unsigned long long zloc = 0;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
        const int i = Tile<VEC4>::index(i0, j);
        if (j >= per || i >= i1) continue;
        const float s = t.v[j] / T;
        const uint32_t key = float_key(s);
        if (hi < 32 && (key >> hi) != (prefix >> hi)) continue;
        if (WHICH == WHICH_P && topk && !(key > kkey || (key == kkey && (uint32_t)i <= kcut)))
            continue;
        const uint32_t d = (key >> shift) & dmask;
        atomicAdd(&s_cnt[d], 1u);
        if (WHICH == WHICH_P) {
            const unsigned long long w = mass_fixed(s, M);
            atomicAdd(&s_mass[d], w);
            zloc += w;
        }
    }
    __syncthreads();
    for (int d = threadIdx.x; d < kDigits; d += kThreads) {
        if (s_cnt[d]) {
            atomicAdd(&a.cnt[(int64_t)b * kDigits + d], s_cnt[d]);
            if (WHICH == WHICH_P) atomicAdd(&a.mass[(int64_t)b * kDigits + d], s_mass[d]);
        }
    }
    if (WHICH == WHICH_P && level == 0) {
        const unsigned long long zs = block_sum(zloc, s_red);
        if (threadIdx.x == 0 && zs) atomicAdd(&ctl->Z, zs);
    }
}

// One workgroup per row: pick the digit of the current level from the
// completed histogram, update the row's prefix, clear the histogram.
template <int WHICH>
__global__ __launch_bounds__(kThreads) void samp_select_kernel(const SampArgs a, int level)
{
    const int b = blockIdx.x;
    SampCtl *ctl = a.ctl + b;
    const uint32_t mode = ctl->mode;
    if (WHICH == WHICH_K && !(mode & MODE_TOPK)) return;
    if (WHICH == WHICH_P && !(mode & MODE_TOPP)) return;
    __shared__ unsigned long long s_red[kThreads];
    __shared__ int s_dstar;

    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const int d_lo = (int)threadIdx.x * kDigitsPerThread;
    uint32_t cnt[kDigitsPerThread];
    unsigned long long mass[kDigitsPerThread];
#pragma unroll
    for (int j = 0; j < kDigitsPerThread; ++j) {
        uint32_t *gc = &a.cnt[(int64_t)b * kDigits + d_lo + j];
        cnt[j] = *gc;
        *gc = 0;
        mass[j] = 0;
        if (WHICH == WHICH_P) {
            unsigned long long *gm = &a.mass[(int64_t)b * kDigits + d_lo + j];
            mass[j] = *gm;
            *gm = 0;
        }
    }
    if (threadIdx.x == 0) s_dstar = kDigits;

    if (WHICH == WHICH_K) {
        unsigned long long own = 0;
#pragma unroll
        for (int j = 0; j < kDigitsPerThread; ++j) own += cnt[j];
        // count in the digits above this thread's range
        unsigned long long above = block_scan_inclusive<unsigned long long, true>(own, s_red) - own;
        const unsigned long long r = ctl->k_rank;
#pragma unroll
        for (int j = kDigitsPerThread - 1; j >= 0; --j) {
            const unsigned long long cd = cnt[j];
            if (above < r && r <= above + cd) {
                // the unique digit holding the rank-th largest key
                const int d = d_lo + j;
                const uint32_t pre = ctl->k_prefix | ((uint32_t)d << shift);
                const uint32_t rank = (uint32_t)(r - above);
                ctl->k_prefix = pre;
                ctl->k_rank = rank;
                if (level == 2) {
                    ctl->k_key = pre;
                    if (rank < cd) ctl->k_tie = rank;  // keep only the lowest-index ties
                }
            }
            above += cd;
        }
    } else {
        unsigned long long own = 0;
#pragma unroll
        for (int j = 0; j < kDigitsPerThread; ++j) own += mass[j];
        unsigned long long above = block_scan_inclusive<unsigned long long, true>(own, s_red) - own;
        const unsigned long long A = ctl->A;
        const double limit = (double)a.top_p[b] * (double)ctl->Z;
        int cand = kDigits;
        unsigned long long cand_above = 0;
        // the lowest non-empty digit whose strictly-greater mass is within
        // the limit (that mass only grows as the digit falls)
#pragma unroll
        for (int j = kDigitsPerThread - 1; j >= 0; --j) {
            if ((double)(A + above) <= limit && cnt[j]) {
                cand = d_lo + j;
                cand_above = above;
            }
            above += mass[j];
        }
        if (cand < kDigits) atomicMin(&s_dstar, cand);
        __syncthreads();
        if (cand < kDigits && cand == s_dstar) {
            const uint32_t pre = ctl->p_prefix | ((uint32_t)cand << shift);
            ctl->A = A + cand_above;
            ctl->p_prefix = pre;
            if (level == 2) ctl->p_key = pre;
        }
    }
}

// top-k ties, count step: logits per chunk whose key equals k_key
template <bool VEC4>
__global__ __launch_bounds__(kThreads) void samp_tie_count_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    if (!(ctl->mode & MODE_TOPK) || ctl->k_tie == 0) return;
    __shared__ uint32_t s_red[kThreads];
    const float T = a.temperature[b];
    const uint32_t kkey = ctl->k_key;
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    const int per = a.chunk / kThreads;
    Tile<VEC4> t;
    t.load(a.logits + (int64_t)b * a.lstride, i0, i1, per);
    uint32_t eq = 0;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
        if (j < per && Tile<VEC4>::index(i0, j) < i1) eq += float_key(t.v[j] / T) == kkey;
    eq = block_sum(eq, s_red);
    if (threadIdx.x == 0) a.chunk_cnt[(int64_t)b * a.nchunks + blockIdx.x] = eq;
}

// top-k ties, cut step (one workgroup per row): keep only the k_tie
// lowest-index logits whose key equals k_key
__global__ __launch_bounds__(kThreads) void samp_tie_cut_kernel(const SampArgs a)
{
    const int b = blockIdx.x;
    SampCtl *ctl = a.ctl + b;
    if (!(ctl->mode & MODE_TOPK) || ctl->k_tie == 0) return;
    __shared__ uint32_t s_red[kThreads];
    __shared__ int s_chunk;
    __shared__ uint32_t s_rem;
    const float T = a.temperature[b];
    const uint32_t kkey = ctl->k_key;
    const float *z = a.logits + (int64_t)b * a.lstride;
    if (threadIdx.x == 0) {
        const uint32_t need = ctl->k_tie;
        uint32_t run = 0;
        int cstar = a.nchunks - 1;
        uint32_t rem = 1;
        for (int c = 0; c < a.nchunks; ++c) {
            const uint32_t v = a.chunk_cnt[(int64_t)b * a.nchunks + c];
            if (run + v >= need) {
                cstar = c;
                rem = need - run;
                break;
            }
            run += v;
        }
        s_chunk = cstar;
        s_rem = rem;
    }
    __syncthreads();
    // ordered scan of the chosen chunk: thread t owns a contiguous range
    const int per = a.chunk / kThreads;
    const int i0 = s_chunk * a.chunk + (int)threadIdx.x * per;
    const int i1 = min(a.vocab, i0 + per);
    uint32_t own = 0;
    for (int i = i0; i < i1; ++i) own += float_key(z[i] / T) == kkey;
    const uint32_t incl = block_scan_inclusive<uint32_t, false>(own, s_red);
    const uint32_t excl = incl - own;
    const uint32_t rem = s_rem;
    if (excl < rem && rem <= incl) {
        uint32_t seen = excl;
        for (int i = i0; i < i1; ++i) {
            if (float_key(z[i] / T) == kkey && ++seen == rem) {
                ctl->k_cut = (uint32_t)i;
                break;
            }
        }
    }
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void samp_final_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    __shared__ unsigned long long s_red[kThreads];
    const uint32_t mode = ctl->mode;
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    const int per = a.chunk / kThreads;
    Tile<VEC4> t;
    t.load(a.logits + (int64_t)b * a.lstride, i0, i1, per);
    unsigned long long best = 0;
    if (mode & MODE_GREEDY) {
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j) {
            const int i = Tile<VEC4>::index(i0, j);
            if (j < per && i < i1) best = max(best, pack_key_index(float_key(t.v[j]), (uint32_t)i));
        }
    } else {
        const float T = a.temperature[b];
        const float *g = a.gumbel + (int64_t)b * a.gstride;
        const bool topk = (mode & MODE_TOPK) != 0;
        const bool topp = (mode & (MODE_TOPP | MODE_TOPP_MAX)) != 0;
        if (!topk && !topp) {
            // every logit is eligible: stream the noise as a tile too
            Tile<VEC4> gt;
            gt.load(g, i0, i1, per);
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j) {
                const int i = Tile<VEC4>::index(i0, j);
                if (j < per && i < i1) {
                    const float kappa = t.v[j] / T + gt.v[j];
                    best = max(best, pack_key_index(float_key(kappa), (uint32_t)i));
                }
            }
        } else {
            const uint32_t kkey = ctl->k_key, kcut = ctl->k_cut;
            const uint32_t pkey = (mode & MODE_TOPP) ? ctl->p_key : ctl->max_key;
            uint32_t kept = 0;
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j) {
                const int i = Tile<VEC4>::index(i0, j);
                const float s = t.v[j] / T;
                const uint32_t key = float_key(s);
                bool ok = j < per && i < i1;
                if (topk) ok = ok && (key > kkey || (key == kkey && (uint32_t)i <= kcut));
                if (topp) ok = ok && key >= pkey;
                t.v[j] = s;
                kept |= (ok ? 1u : 0u) << j;
            }
            // noise only for the eligible logits, all loads issued together
            float gv[kMaxPer];
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j)
                gv[j] = ((kept >> j) & 1u) ? g[Tile<VEC4>::index(i0, j)] : 0.f;
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j)
                if ((kept >> j) & 1u)
                    best = max(best, pack_key_index(float_key(t.v[j] + gv[j]),
                                                    (uint32_t)Tile<VEC4>::index(i0, j)));
        }
    }
    best = block_max(best, s_red);
    if (threadIdx.x == 0 && best) atomicMax(&ctl->best, best);
}

__global__ __launch_bounds__(kThreads) void samp_write_ids_kernel(const SampArgs a)
{
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b >= a.batch) return;
    const unsigned long long v = a.ctl[b].best;
    a.out_ids[b] = (int32_t)(0xffffffffu - (uint32_t)(v & 0xffffffffull));
}

template <bool VEC4>
void launch_passes(const SampArgs &a, const dim3 grid, uint32_t flags, hipStream_t stream)
{
    if (flags & 2u) samp_max_kernel<VEC4><<<grid, kThreads, 0, stream>>>(a);
    if (flags & 1u) {
        for (int level = 0; level < 3; ++level) {
            samp_hist_kernel<WHICH_K, VEC4><<<grid, kThreads, 0, stream>>>(a, level);
            samp_select_kernel<WHICH_K><<<a.batch, kThreads, 0, stream>>>(a, level);
        }
        samp_tie_count_kernel<VEC4><<<grid, kThreads, 0, stream>>>(a);
        samp_tie_cut_kernel<<<a.batch, kThreads, 0, stream>>>(a);
    }
    if (flags & 2u)
        for (int level = 0; level < 3; ++level) {
            samp_hist_kernel<WHICH_P, VEC4><<<grid, kThreads, 0, stream>>>(a, level);
            samp_select_kernel<WHICH_P><<<a.batch, kThreads, 0, stream>>>(a, level);
        }
    samp_final_kernel<VEC4><<<grid, kThreads, 0, stream>>>(a);
    samp_write_ids_kernel<<<(a.batch + kThreads - 1) / kThreads, kThreads, 0, stream>>>(a);
}

}  // namespace

size_t sampler_workspace_bytes(int32_t batch, int32_t vocab)
{
    return sampler_layout(batch, vocab).total;
}

hipError_t launch_sampler(int32_t *out_ids, const float *logits, int64_t logits_stride,
                          const float *gumbel, int64_t gumbel_stride, const float *temperature,
                          const float *top_p, const int32_t *top_k, int32_t batch, int32_t vocab,
                          uint32_t flags, void *workspace, hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    const SampLayout L = sampler_layout(batch, vocab);
    char *ws = static_cast<char *>(workspace);
    SampArgs a;
    a.out_ids = out_ids;
    a.logits = logits;
    a.lstride = logits_stride;
    a.gumbel = gumbel;
    a.gstride = gumbel_stride;
    a.temperature = temperature;
    a.top_p = top_p;
    a.top_k = top_k;
    a.batch = batch;
    a.vocab = vocab;
    a.chunk = L.chunk;
    a.nchunks = L.nchunks;
    a.flags = flags;
    a.ctl = reinterpret_cast<SampCtl *>(ws + L.ctl_off);
    a.cnt = reinterpret_cast<uint32_t *>(ws + L.cnt_off);
    a.mass = reinterpret_cast<unsigned long long *>(ws + L.mass_off);
    a.chunk_cnt = reinterpret_cast<uint32_t *>(ws + L.chunk_off);

    const dim3 grid(L.nchunks, batch);
    samp_init_kernel<<<batch, kThreads, 0, stream>>>(a);
    const bool vec4 = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && logits_stride % 4 == 0 &&
                      (reinterpret_cast<uintptr_t>(gumbel) % 16 == 0) && gumbel_stride % 4 == 0 &&
                      vocab % 4 == 0;
    if (vec4)
        launch_passes<true>(a, grid, flags, stream);
    else
        launch_passes<false>(a, grid, flags, stream);
    return hipGetLastError();
}

}  // namespace pkv
