// Next-token sampler: temperature, top-k, nucleus (top-p) and a Gumbel-max
// draw, on fp32 logits [B][V].
//
// Every pass splits each row into chunks of `chunk` logits, one 256-thread
// workgroup per (chunk, row), and recomputes s = z / T (IEEE division) and
// its order-preserving 32-bit key.  Thresholds are found by a three-level
// radix select on the key (11 + 11 + 10 bits): each level histograms the
// keys that match the prefix chosen so far into 2048 digits, and the last
// workgroup of the row to finish (counted with an atomic ticket) scans the
// histogram and fixes the next digit.  Top-k ranks by count; top-p
// accumulates mass exp(s - max) in 40-bit fixed point, so the sums are
// exact, order independent and identical from run to run.  A top-k tie at
// the k-th key is cut by index with one more pass.  The final pass takes the
// argmax of fl32(s + g) over the eligible logits as one 64-bit atomic max of
// (key, ~index), which resolves ties to the lowest index.
#include <math.h>

#include "launch.hpp"
#include "pkv_device.hpp"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kDigits = 2048;
constexpr int kDigitsPerThread = kDigits / kThreads;

enum : uint32_t { MODE_GREEDY = 1, MODE_TOPK = 2, MODE_TOPP = 4, MODE_TOPP_MAX = 8 };
enum : int { WHICH_K = 0, WHICH_P = 1 };

struct alignas(64) SampCtl {
    unsigned long long best;  // packed (key, ~index) of the draw
    unsigned long long Z;     // kept mass, 2^-40 units
    unsigned long long A;     // mass strictly above the current top-p bucket
    uint32_t max_key;         // key of max s
    uint32_t done;            // last-workgroup ticket
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

// True in every thread of the one workgroup of row b that finishes last.
__device__ bool last_of_row(SampCtl *ctl, int *s_flag)
{
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) *s_flag = (atomicAdd(&ctl->done, 1u) == gridDim.x - 1) ? 1 : 0;
    __syncthreads();
    const bool last = *s_flag != 0;
    if (last) __threadfence();
    return last;
}

__global__ __launch_bounds__(kThreads) void samp_init_kernel(const SampArgs a)
{
    const int b = blockIdx.x;
    for (int d = threadIdx.x; d < kDigits; d += kThreads) {
        a.cnt[(int64_t)b * kDigits + d] = 0;
        a.mass[(int64_t)b * kDigits + d] = 0;
    }
    for (int c = threadIdx.x; c < a.nchunks; c += kThreads) a.chunk_cnt[(int64_t)b * a.nchunks + c] = 0;
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
__global__ __launch_bounds__(kThreads) void samp_max_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    if (!(ctl->mode & (MODE_TOPP | MODE_TOPP_MAX))) return;
    __shared__ uint32_t s_red[kThreads];
    const float T = a.temperature[b];
    const float *z = a.logits + (int64_t)b * a.lstride;
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    uint32_t kmax = 0;
    for (int i = i0 + threadIdx.x; i < i1; i += kThreads) kmax = max(kmax, float_key(z[i] / T));
    kmax = block_max(kmax, s_red);
    if (threadIdx.x == 0) atomicMax(&ctl->max_key, kmax);
}

template <int WHICH>
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
    __shared__ int s_flag;
    __shared__ int s_dstar;

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
    const float T = a.temperature[b];
    const float M = key_float(ctl->max_key);
    const uint32_t kkey = ctl->k_key, kcut = ctl->k_cut;
    const bool topk = (mode & MODE_TOPK) != 0;
    const float *z = a.logits + (int64_t)b * a.lstride;
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);

    unsigned long long zloc = 0;
    for (int i = i0 + threadIdx.x; i < i1; i += kThreads) {
        const float s = z[i] / T;
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
    if (!last_of_row(ctl, &s_flag)) return;

    // ---- last workgroup of the row: choose the digit ----
    for (int d = threadIdx.x; d < kDigits; d += kThreads) {
        uint32_t *gc = &a.cnt[(int64_t)b * kDigits + d];
        s_cnt[d] = __hip_atomic_load(gc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (WHICH == WHICH_P) {
            unsigned long long *gm = &a.mass[(int64_t)b * kDigits + d];
            s_mass[d] = __hip_atomic_load(gm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(gm, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (threadIdx.x == 0) s_dstar = kDigits;
    __syncthreads();

    const int d_hi = (int)threadIdx.x * kDigitsPerThread + kDigitsPerThread - 1;
    if (WHICH == WHICH_K) {
        unsigned long long own = 0;
        for (int j = 0; j < kDigitsPerThread; ++j) own += s_cnt[d_hi - j];
        // count in digits above this thread's range
        unsigned long long above = block_scan_inclusive<unsigned long long, true>(own, s_red) - own;
        const unsigned long long r = ctl->k_rank;
        for (int j = 0; j < kDigitsPerThread; ++j) {
            const int d = d_hi - j;
            const unsigned long long cd = s_cnt[d];
            if (above < r && r <= above + cd) {
                // unique digit holding the rank-th largest key
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
        for (int j = 0; j < kDigitsPerThread; ++j) own += s_mass[d_hi - j];
        unsigned long long above = block_scan_inclusive<unsigned long long, true>(own, s_red) - own;
        const unsigned long long A = ctl->A;
        const double limit = (double)a.top_p[b] * (double)ctl->Z;
        int cand = kDigits;
        unsigned long long cand_above = 0;
        for (int j = 0; j < kDigitsPerThread; ++j) {
            const int d = d_hi - j;
            // mass strictly above every key of digit d; grows as d falls
            if ((double)(A + above) > limit) break;
            if (s_cnt[d]) {
                cand = d;
                cand_above = above;
            }
            above += s_mass[d];
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
    if (threadIdx.x == 0) ctl->done = 0;
}

// top-k ties: keep only the k_tie lowest-index logits whose key equals k_key
__global__ __launch_bounds__(kThreads) void samp_tie_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    if (!(ctl->mode & MODE_TOPK) || ctl->k_tie == 0) return;
    __shared__ uint32_t s_red[kThreads];
    __shared__ int s_flag;
    __shared__ int s_chunk;
    __shared__ uint32_t s_rem;

    const float T = a.temperature[b];
    const uint32_t kkey = ctl->k_key;
    const float *z = a.logits + (int64_t)b * a.lstride;
    int i0 = blockIdx.x * a.chunk;
    int i1 = min(a.vocab, i0 + a.chunk);
    uint32_t eq = 0;
    for (int i = i0 + threadIdx.x; i < i1; i += kThreads) eq += float_key(z[i] / T) == kkey;
    eq = block_sum(eq, s_red);
    if (threadIdx.x == 0)
        __hip_atomic_store(&a.chunk_cnt[(int64_t)b * a.nchunks + blockIdx.x], eq, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (!last_of_row(ctl, &s_flag)) return;

    if (threadIdx.x == 0) {
        const uint32_t need = ctl->k_tie;
        uint32_t run = 0;
        int cstar = a.nchunks - 1;
        uint32_t rem = 1;
        for (int c = 0; c < a.nchunks; ++c) {
            const uint32_t v = __hip_atomic_load(&a.chunk_cnt[(int64_t)b * a.nchunks + c],
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    i0 = s_chunk * a.chunk + (int)threadIdx.x * per;
    i1 = min(a.vocab, i0 + per);
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
    if (threadIdx.x == 0) ctl->done = 0;
}

__global__ __launch_bounds__(kThreads) void samp_final_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    __shared__ unsigned long long s_red[kThreads];
    __shared__ int s_flag;
    const uint32_t mode = ctl->mode;
    const float *z = a.logits + (int64_t)b * a.lstride;
    const float *g = a.gumbel + (int64_t)b * a.gstride;
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    unsigned long long best = 0;
    if (mode & MODE_GREEDY) {
        for (int i = i0 + threadIdx.x; i < i1; i += kThreads)
            best = max(best, pack_key_index(float_key(z[i]), (uint32_t)i));
    } else {
        const float T = a.temperature[b];
        const bool topk = (mode & MODE_TOPK) != 0;
        const bool topp = (mode & (MODE_TOPP | MODE_TOPP_MAX)) != 0;
        const uint32_t kkey = ctl->k_key, kcut = ctl->k_cut;
        const uint32_t pkey = (mode & MODE_TOPP) ? ctl->p_key : ctl->max_key;
        for (int i = i0 + threadIdx.x; i < i1; i += kThreads) {
            const float s = z[i] / T;
            const uint32_t key = float_key(s);
            if (topk && !(key > kkey || (key == kkey && (uint32_t)i <= kcut))) continue;
            if (topp && key < pkey) continue;
            const float kappa = s + g[i];
            best = max(best, pack_key_index(float_key(kappa), (uint32_t)i));
        }
    }
    best = block_max(best, s_red);
    if (threadIdx.x == 0) atomicMax(&ctl->best, best);
    if (!last_of_row(ctl, &s_flag)) return;
    if (threadIdx.x == 0) {
        const unsigned long long v =
            __hip_atomic_load(&ctl->best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.out_ids[b] = (int32_t)(0xffffffffu - (uint32_t)(v & 0xffffffffull));
        ctl->done = 0;
    }
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
    if (flags & 2u) samp_max_kernel<<<grid, kThreads, 0, stream>>>(a);
    if (flags & 1u) {
        for (int level = 0; level < 3; ++level)
            samp_hist_kernel<WHICH_K><<<grid, kThreads, 0, stream>>>(a, level);
        samp_tie_kernel<<<grid, kThreads, 0, stream>>>(a);
    }
    if (flags & 2u)
        for (int level = 0; level < 3; ++level)
            samp_hist_kernel<WHICH_P><<<grid, kThreads, 0, stream>>>(a, level);
    samp_final_kernel<<<grid, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace pkv
