// Next-token sampler: temperature, top-k, nucleus (top-p) and a Gumbel-max
// draw, on fp32 logits [B][V].
//
// Row-parallel passes split each row into chunks of `chunk` logits, one
// 256-thread workgroup per (chunk, row).  Each thread first loads its whole
// share of the chunk into registers (float4 when rows are 16-byte aligned).
// The scaled logit is s = z / T, an IEEE fp32 division; since that division
// is monotone in z for T > 0, only the bins pass divides every logit.
//
// Rows with a top-k or nucleus filter take three passes over their logits:
//   max     the row max M of s, as (max allowed z) / T
//   bins    a histogram over 2048 value bins of width 1/32 below M
//           (bin = floor(fl(M - s) * 32), the last bin catching everything
//           >= 64 below M), with counts and the mass exp(s - M) in 2^-40
//           fixed point: exact, order independent and identical from run
//           to run
//   collect every logit in a bin above the threshold bin is eligible: its
//           Gumbel key fl32(s + g) joins a max of the packed 64-bit
//           (key, ~index) (ties to the lowest index); the logits of the
//           threshold bin itself are appended to a per-row candidate list.
//           Both classes are upper sets of z, so a logit is classified by
//           two thresholds on z that `select` finds by bisection, and s is
//           computed only for the logits that join the list.
// and two per-row kernels: `select` finds the threshold bin from the
// histogram, `resolve` ranks the candidates (by counting when there are at
// most 512, else by a bitonic sort in LDS) and fixes the exact cut inside
// that bin (by rank for top-k, by strictly-greater mass for the nucleus),
// then writes the id.  Top-k followed by the nucleus may need one more
// collect/resolve round when the nucleus cut lies above the top-k bin.  If a
// threshold bin holds more candidates than the list, `resolve` finds the cut
// exactly by scanning the row itself (radix select on the key).
//
// Greedy rows (T <= 0) and rows without a filter need only the collect pass.
// Passes communicate only through kernel boundaries: no workgroup waits for
// or fences against another one inside a kernel.  Per-chunk results (row
// max, best Gumbel key) go to per-chunk slots that the next kernel reduces,
// so no pass needs memory cleared beforehand except the histograms, which
// the max pass clears.
#include <math.h>

#include "launch.hpp"
#include "pkv_device.hpp"

namespace pkv {

namespace {

constexpr int kThreads = 256;           // row-parallel passes
constexpr int kRThreads = 512;          // per-row select / resolve
constexpr int kBins = 2048;             // value bins below the row max
constexpr float kBinsPerUnit = 32.f;    // bin width: 1/32 of a logit unit
constexpr int kCap = 4096;              // threshold-bin candidates kept per row
constexpr int kMaxPer = 32;             // logits per thread per chunk (bit masks: <= 32)
constexpr int kDigits = 2048;           // radix digits of the exact in-row fallback
constexpr int kMinGroups = 256;         // row-parallel workgroups wanted (one per CU)
constexpr int kList = 1024;             // compacted noise reads per collect workgroup
constexpr uint32_t kCandBit = 0x80000000u;
constexpr uint32_t kKeptBit = 0x40000000u;
constexpr uint32_t kIndexMask = 0x3fffffffu;  // vocab < 2^30
constexpr uint32_t kSlotMasked = 0x80000000u; // list entry of a forbidden logit

enum : uint32_t {
    MODE_GREEDY = 1,     // T <= 0: lowest index of the max raw logit
    MODE_PLAIN = 2,      // T > 0 and no filter: every token eligible
    MODE_TOPK = 4,
    MODE_TOPP = 8,
    MODE_TOPP_MAX = 16,  // p <= 0: only the maxima are eligible
    MODE_DONE = 32,      // id written
};

struct alignas(64) SampCtl {
    unsigned long long Z;     // eligible mass, 2^-40 units
    unsigned long long A;     // mass of the bins above the threshold bin
    uint32_t max_key;         // key of max s
    uint32_t mode;
    uint32_t k;               // top-k
    uint32_t jstar;           // threshold bin
    uint32_t rank;            // top-k: logits of the threshold bin to keep
    uint32_t ncand;           // logits of the threshold bin appended
    uint32_t round2;          // 1 while a second collect round is pending
    uint32_t tau;             // final cut: kept logits have key(s) >= tau (0: none)
    unsigned long long kpack; // top-k cut: kept have (key, ~index) >= kpack (0: none)
};
static_assert(sizeof(SampCtl) == 64, "control block");

struct SampLayout {
    int32_t chunk;
    int32_t nchunks;
    size_t ctl_off, cnt_off, mass_off, cand_off, kap_off, pmax_off, pbest_off, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SampLayout sampler_layout(int32_t batch, int32_t vocab)
{
    SampLayout L;
    // the largest chunk that still gives kMinGroups workgroups per pass
    int32_t chunk = kMaxPer * kThreads;
    while (chunk > 4 * kThreads && (int64_t)batch * ((vocab + chunk - 1) / chunk) < kMinGroups) chunk >>= 1;
    L.chunk = chunk;
    L.nchunks = (vocab + chunk - 1) / chunk;
    size_t off = 0;
    L.ctl_off = off;
    off = align256(off + (size_t)batch * sizeof(SampCtl));
    L.cnt_off = off;
    off = align256(off + (size_t)batch * kBins * sizeof(uint32_t));
    L.mass_off = off;
    off = align256(off + (size_t)batch * kBins * sizeof(unsigned long long));
    L.cand_off = off;
    off = align256(off + (size_t)batch * kCap * sizeof(unsigned long long));
    L.kap_off = off;
    off = align256(off + (size_t)batch * kCap * sizeof(uint32_t));
    L.pmax_off = off;
    off = align256(off + (size_t)batch * L.nchunks * sizeof(uint32_t));
    L.pbest_off = off;
    off = align256(off + (size_t)batch * L.nchunks * sizeof(unsigned long long));
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
    uint32_t *cnt;                 // [B][kBins]
    unsigned long long *mass;      // [B][kBins]
    unsigned long long *cand;      // [B][kCap]  (key << 32) | ~index
    uint32_t *kap;                 // [B][kCap]  key of fl32(s + g)
    uint32_t *part_max;            // [B][nchunks] key of the chunk max of s
    unsigned long long *part_best; // [B][nchunks] best packed Gumbel key of the chunk
    const uint8_t *mask;           // [B][V] (row b at b*mstride), 0 = forbidden; or null
    int64_t mstride;
    float *out_prob;               // [B] probability of the drawn id, or null
    int32_t *out_top_ids;          // [B][8], or null
    float *out_top_probs;          // [B][8], or null
};

// The runner's value for forbidden tokens (their scaled logit is replaced).
constexpr float kMasked = -1e10f;

// s = z / T, the IEEE fp32 quotient, by one double product: fl64(z) *
// fl64(1 / T) is within 2^-52 (relative) of z / T, while the quotient of two
// fp32 numbers, when not exactly an fp32 number, lies more than 2^-49
// (relative) from every fp32 rounding boundary, except for a tie in the
// subnormal range.  Rounding the product to fp32 therefore gives the
// correctly rounded quotient for every |z| >= 2^-125 T; below that the
// division itself runs (a branch that real logits essentially never take).
// Every place that computes s this way or by division gets the same value.
struct Scaler {
    float T, tiny;
    double inv;
    __device__ explicit Scaler(float t) : T(t), tiny(t * 0x1p-125f), inv(1.0 / (double)t) {}
    __device__ __forceinline__ float operator()(float z) const
    {
        float s = (float)((double)z * inv);
        if (__builtin_expect(fabsf(z) < tiny, 0)) s = z / T;
        return s;
    }
};

__device__ __forceinline__ unsigned long long pack_key_index(uint32_t key, uint32_t i)
{
    return ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - i);
}

__device__ __forceinline__ uint32_t unpack_index(unsigned long long v)
{
    return 0xffffffffu - (uint32_t)(v & 0xffffffffull);
}

// exp(s - M) in 2^-40 fixed point, by the hardware base-2 exponential.  The
// rounding errors of d = s - M (TwoSum) and of d * log2(e) (FMA residual)
// are recovered exactly and folded in to first order.  The fixed-point value
// is assembled from two 20-bit halves (w < 2, so w * 2^40 < 2^41).
__device__ __forceinline__ unsigned long long mass_fixed(float s, float M)
{
    constexpr float kLog2e = 1.44269504088896341f;
    constexpr float kLn2 = 0.693147180559945309f;
    const float d = s - M;
    const float bb = d - s;
    const float e = (s - (d - bb)) + (-M - bb);
    const float x = d * kLog2e;
    const float xe = fmaf(d, kLog2e, -x);
    float w = __builtin_amdgcn_exp2f(x);
    w = fmaf(w, fmaf(xe, kLn2, e), w);
    const float hi = floorf(w * 1048576.0f);             // w * 2^20, integer part
    const float lo = (w * 1048576.0f - hi) * 1048576.0f; // exact remainder, * 2^20
    return ((unsigned long long)(uint32_t)hi << 20) + (uint32_t)lo;
}

// Value bin below the row max M: monotone non-increasing in s (rounding of
// M - s is monotone, the scale is a power of two).
__device__ __forceinline__ int bin_of(float s, float M)
{
    const float d = (M - s) * kBinsPerUnit;
    return d < (float)(kBins - 1) ? (int)d : kBins - 1;
}

// One wave: the smallest z, in key order over the non-NaN floats, at which a
// monotone predicate (false below some z, true from there up) holds; -inf if
// it holds everywhere, NaN if nowhere.  64 probes per step narrow the key
// interval (lo, hi] about 64-fold, so a 32-bit key takes six steps.
template <typename Pred>
__device__ float wave_first_z(Pred pred)
{
    const float inf = __builtin_huge_valf();
    if (pred(-inf)) return -inf;
    if (!pred(inf)) return __builtin_nanf("");
    uint32_t lo = float_key(-inf), hi = float_key(inf);  // pred(lo) false, pred(hi) true
    const int lane = (int)threadIdx.x & 63;
    while (hi - lo > 1u) {
        const uint32_t probe = lo + (uint32_t)(((unsigned long long)(hi - lo) * (unsigned)(lane + 1)) >> 6);
        const unsigned long long t = __ballot(pred(key_float(probe)));  // lane 63 probes hi: true
        const int f = __builtin_ctzll(t);
        const uint32_t nlo = (uint32_t)__shfl((int)probe, f > 0 ? f - 1 : 0);
        hi = (uint32_t)__shfl((int)probe, f);
        if (f > 0) lo = nlo;
    }
    return key_float(hi);
}

// Thresholds on the raw logit z equivalent to "bin of z / T below j"
// (out[0]) and "bin of z / T at most j" (out[1]): division by T > 0 is
// monotone and bin_of is monotone in s, so each class is an upper set of z.
// (-0 and +0 fall in the same bin, so a float comparison with the threshold
// decides as the bin does.)  Wave 0 finds the first, wave 1 the second.
__device__ void z_thresholds(float T, float M, int j, float *out)
{
    const int w = (int)threadIdx.x >> 6;
    if (w > 1) return;
    const int lim = w == 0 ? j : j + 1;
    const float z0 = wave_first_z([=](float z) { return bin_of(z / T, M) < lim; });
    if ((threadIdx.x & 63) == 0) out[w] = z0;
}

// Block-wide reductions and scans: within each wave by lane shuffles, then
// one exchange of the per-wave results through `scratch` (>= NT / 64
// entries).  Every thread gets the result; `scratch` is free again on return.
template <typename T>
__device__ __forceinline__ T wave_sum_t(T v)
{
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_max_t(T v)
{
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v = max(v, __shfl_xor(v, m));
    return v;
}

// Sum over aligned groups of q consecutive lanes (q a power of two <= 64).
template <typename T>
__device__ __forceinline__ T group_sum_lanes(T v, int q)
{
    for (int m = 1; m < q; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

template <typename T, int NT>
__device__ T block_sum(T v, T *scratch)
{
    v = wave_sum_t(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r += scratch[w];
    __syncthreads();
    return r;
}

template <typename T, int NT>
__device__ T block_max(T v, T *scratch)
{
    v = wave_max_t(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r = max(r, scratch[w]);
    __syncthreads();
    return r;
}

// Inclusive scan over the threads in ascending order.
template <typename T, int NT>
__device__ T block_scan_inclusive(T v, T *scratch)
{
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T u = __shfl_up(v, (unsigned)off);
        if (lane >= off) v += u;
    }
    __syncthreads();
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
    T base = 0;
    for (int w = 0; w < wave; ++w) base += scratch[w];
    __syncthreads();
    return v + base;
}

// Each thread's share of one chunk (chunk / 256 <= 32 logits), loaded into
// registers before any of it is used so that all loads of a pass are in
// flight together.  VEC4: consecutive threads read consecutive float4s
// (rows 16-byte aligned, vocab a multiple of 4); otherwise single floats.
template <bool VEC4>
struct Tile {
    float v[kMaxPer];
    uint32_t ok = 0xffffffffu;  // bit j: element j is allowed by the mask

    // s of element j: z / T, or kMasked where the mask forbids it
    __device__ __forceinline__ float scaled(int j, const Scaler &sc) const
    {
        return ((ok >> j) & 1u) ? sc(v[j]) : kMasked;
    }
    // greedy value of element j: the raw logit, or kMasked
    __device__ __forceinline__ float raw(int j) const { return ((ok >> j) & 1u) ? v[j] : kMasked; }

    __device__ __forceinline__ void load_mask(const uint8_t *__restrict__ mrow, int i0, int i1,
                                              int per)
    {
        if (!mrow) return;
        uint32_t bits = 0;
        if constexpr (VEC4) {
#pragma unroll
            for (int q = 0; q < kMaxPer / 4; ++q) {
                const int i = index(i0, 4 * q);
                const uint32_t w = *reinterpret_cast<const uint32_t *>(mrow + ((4 * q < per && i < i1) ? i : i0));
#pragma unroll
                for (int k = 0; k < 4; ++k) bits |= (((w >> (8 * k)) & 0xffu) ? 1u : 0u) << (4 * q + k);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j) {
                const int i = index(i0, j);
                const uint8_t m = mrow[(j < per && i < i1) ? i : i0];
                bits |= (m ? 1u : 0u) << j;
            }
        }
        ok = bits;
    }

    __device__ __forceinline__ static int index(int i0, int j)
    {
        if constexpr (VEC4)
            return i0 + ((j >> 2) * kThreads + (int)threadIdx.x) * 4 + (j & 3);
        else
            return i0 + j * kThreads + (int)threadIdx.x;
    }

    // a chunk of kMaxPer logits per thread, all inside the row
    __device__ __forceinline__ static bool full(int i0, int i1, int per)
    {
        return per == kMaxPer && i1 - i0 == kMaxPer * kThreads;
    }

    // Every load is issued, in one straight run: an element outside the chunk
    // reads the chunk's first logits instead and is never used.  With no
    // branch between the loads and their use, each use waits only for its
    // own load.
    template <bool NT = false>
    __device__ __forceinline__ void load(const float *__restrict__ row, int i0, int i1, int per)
    {
        load_range<0, kMaxPer, NT>(row, i0, i1, per);
    }

    // elements [J0, J0 + NJ) only (multiples of 4)
    template <int J0, int NJ, bool NT = false>
    __device__ __forceinline__ void load_range(const float *__restrict__ row, int i0, int i1, int per)
    {
        if constexpr (VEC4) {
#pragma unroll
            for (int q = J0 / 4; q < (J0 + NJ) / 4; ++q) {
                const int i = index(i0, 4 * q);
                const int ic = (4 * q < per && i < i1) ? i : i0;
                typedef float f32x4 __attribute__((ext_vector_type(4)));
                const f32x4 *src = reinterpret_cast<const f32x4 *>(row + ic);
                const f32x4 f = NT ? __builtin_nontemporal_load(src) : *src;
                v[4 * q] = f.x;
                v[4 * q + 1] = f.y;
                v[4 * q + 2] = f.z;
                v[4 * q + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int j = J0; j < J0 + NJ; ++j) {
                const int i = index(i0, j);
                const float *src = row + ((j < per && i < i1) ? i : i0);
                v[j] = NT ? __builtin_nontemporal_load(src) : *src;
            }
        }
    }
};

// Calls f(j) for each element j of this thread's share of the chunk
// [i0, i1): without per-element range checks for a full chunk.
template <bool VEC4, typename F>
__device__ __forceinline__ void for_each_elem(int i0, int i1, int per, F f)
{
    if (Tile<VEC4>::full(i0, i1, per)) {
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j) f(j);
    } else {
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j)
            if (j < per && Tile<VEC4>::index(i0, j) < i1) f(j);
    }
}

// What a row needs, from its own settings and the enabled filters.
__device__ __forceinline__ uint32_t row_mode(const SampArgs &a, int b)
{
    const float T = a.temperature[b];
    if (!(T > 0.f)) return MODE_GREEDY;
    const int32_t k = a.top_k[b];
    const float p = a.top_p[b];
    uint32_t mode = 0;
    if ((a.flags & 1u) && k > 0 && k < a.vocab) mode |= MODE_TOPK;
    if ((a.flags & 2u) && p < 1.f) {
        if (!(p > 0.f)) return MODE_TOPP_MAX;  // the maxima are always in the top k
        mode |= MODE_TOPP;
    }
    return mode ? mode : MODE_PLAIN;
}

// First pass of filtered sampling: per-chunk max of s.  Chunk 0 of each row
// also sets up the row's control block, and the chunks of a filtered row
// clear its histogram between them.
template <bool VEC4, bool MASK>
__global__ __launch_bounds__(kThreads) void samp_max_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    const int per = a.chunk / kThreads;
    // issued before the row's settings are known, so that the two overlap
    Tile<VEC4> t;
    t.template load<true>(a.logits + (int64_t)b * a.lstride, i0, i1, per);
    t.load_mask(MASK ? a.mask + (int64_t)b * a.mstride : nullptr, i0, i1, per);
    const uint32_t mode = row_mode(a, b);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        SampCtl c = {};
        c.mode = mode;
        c.k = (uint32_t)a.top_k[b];
        c.jstar = kBins;
        a.ctl[b] = c;
    }
    if (!(mode & (MODE_TOPK | MODE_TOPP | MODE_TOPP_MAX))) return;
    if (mode & (MODE_TOPK | MODE_TOPP)) {
        for (int d = (int)(blockIdx.x * kThreads + threadIdx.x); d < kBins; d += (int)(gridDim.x * kThreads)) {
            a.cnt[(int64_t)b * kBins + d] = 0;
            a.mass[(int64_t)b * kBins + d] = 0;
        }
    }
    __shared__ uint32_t s_red[kThreads / 64];
    const float T = a.temperature[b];
    // Division by T > 0 is monotone, so the largest s = z / T is the largest
    // allowed z divided by T: one division per thread instead of per logit.
    // Forbidden logits count as kMasked.
    // The running max is a float select (a NaN z never wins it); float_key
    // maps -0 and +0 to one key, so this equals the max over keys of s for
    // every NaN-free row.
    float zmax = -__builtin_huge_valf();
    uint32_t seen = 0;  // bit j: element j is in the chunk
    for_each_elem<VEC4>(i0, i1, per, [&](int j) {
        const float z = ((t.ok >> j) & 1u) ? t.v[j] : -__builtin_huge_valf();
        zmax = z > zmax ? z : zmax;
        seen |= 1u << j;
    });
    uint32_t kmax = float_key(zmax / T);
    if (~t.ok & seen) kmax = max(kmax, float_key(kMasked));
    kmax = block_max<uint32_t, kThreads>(kmax, s_red);
    if (threadIdx.x == 0) a.part_max[(int64_t)b * a.nchunks + blockIdx.x] = kmax;
}

// Key of the row max of s, from the per-chunk maxima.
template <int NT>
__device__ uint32_t row_max_key(const SampArgs &a, int b, uint32_t *scratch)
{
    const uint32_t *pm = a.part_max + (int64_t)b * a.nchunks;
    uint32_t k = 0;
    for (int c = threadIdx.x; c < a.nchunks; c += NT) k = max(k, pm[c]);
    return block_max<uint32_t, NT>(k, scratch);
}

// Counts (and, for the nucleus, masses) per value bin below the row max.
template <bool VEC4, bool MASK>
__global__ __launch_bounds__(kThreads) void samp_bins_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    const int per = a.chunk / kThreads;
    // The chunk maxima are requested before the tile: loads complete in
    // order, so waiting for them then does not wait for the tile, whose
    // elements are used as they arrive.  (Clamped, not range-checked: a
    // repeated maximum changes no max.)
    const uint32_t *pm = a.part_max + (int64_t)b * a.nchunks;
    uint32_t kpm = pm[min((int)threadIdx.x, a.nchunks - 1)];
    Tile<VEC4> t;
    t.load(a.logits + (int64_t)b * a.lstride, i0, i1, per);
    t.load_mask(MASK ? a.mask + (int64_t)b * a.mstride : nullptr, i0, i1, per);
    const uint32_t mode = ctl->mode;
    if (!(mode & (MODE_TOPK | MODE_TOPP))) return;
    __shared__ uint32_t s_cnt[kBins];
    __shared__ unsigned long long s_mass[kBins];
    __shared__ unsigned long long s_red[kThreads / 64];
    const float T = a.temperature[b];
    const Scaler sc(T);
    for (int d = threadIdx.x; d < kBins; d += kThreads) {
        s_cnt[d] = 0;
        s_mass[d] = 0;
    }
    for (int c = threadIdx.x + kThreads; c < a.nchunks; c += kThreads) kpm = max(kpm, pm[c]);
    const float M = key_float(block_max<uint32_t, kThreads>(kpm, reinterpret_cast<uint32_t *>(s_red)));
    const bool want_mass = (mode & MODE_TOPP) != 0;
    const bool want_cnt = (mode & MODE_TOPK) != 0;  // nucleus-only rows need masses alone
    unsigned long long zloc = 0;
    uint32_t tail = 0;
    for_each_elem<VEC4>(i0, i1, per, [&](int j) {
        const float s = t.scaled(j, sc);
        const int bin = bin_of(s, M);
        // >= 64 below the max (the last bin): counted per thread, its mass
        // exp(-64) is below the fixed-point unit
        const bool last = bin == kBins - 1;
        tail += last ? 1u : 0u;
        if (!last) {
            if (want_cnt) atomicAdd(&s_cnt[bin], 1u);
            if (want_mass) {
                const unsigned long long w = mass_fixed(s, M);
                atomicAdd(&s_mass[bin], w);
                zloc += w;
            }
        }
    });
    __syncthreads();
    for (int d = threadIdx.x; d < kBins - 1; d += kThreads) {
        if (s_cnt[d]) atomicAdd(&a.cnt[(int64_t)b * kBins + d], s_cnt[d]);
        if (s_mass[d]) atomicAdd(&a.mass[(int64_t)b * kBins + d], s_mass[d]);
    }
    const unsigned long long tails = block_sum<unsigned long long, kThreads>(tail, s_red);
    if (threadIdx.x == 0 && tails)
        atomicAdd(&a.cnt[(int64_t)b * kBins + kBins - 1], (uint32_t)tails);
    if (want_mass) {
        const unsigned long long zs = block_sum<unsigned long long, kThreads>(zloc, s_red);
        if (threadIdx.x == 0 && zs) atomicAdd(&ctl->Z, zs);
    }
}

// One workgroup per row: the row max, and the threshold bin.  Top-k: the
// bin holding the k-th largest s, with the rank inside it.  Nucleus: the
// lowest non-empty bin whose strictly-greater mass is within p of the total;
// every bin above it is eligible in full.
__global__ __launch_bounds__(kRThreads) void samp_select_kernel(const SampArgs a)
{
    constexpr int BPT = kBins / kRThreads;
    const int b = blockIdx.x;
    SampCtl *ctl = a.ctl + b;
    const uint32_t mode = ctl->mode;
    if (!(mode & (MODE_TOPK | MODE_TOPP | MODE_TOPP_MAX))) return;
    __shared__ unsigned long long s_red[kRThreads / 64];
    // The histogram is requested before the row max is reduced, so that the
    // two round trips overlap; both arrays are read unconditionally (a
    // branch at a load makes the compiler wait for it), the counts are used
    // by top-k rows only and neither by p <= 0 rows.
    const int d0 = (int)threadIdx.x * BPT;
    const bool topk = (mode & MODE_TOPK) != 0;
    uint32_t cnt[BPT];
    unsigned long long mass[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        cnt[j] = a.cnt[(int64_t)b * kBins + d0 + j];
        mass[j] = a.mass[(int64_t)b * kBins + d0 + j];
    }
    const uint32_t max_key = row_max_key<kRThreads>(a, b, reinterpret_cast<uint32_t *>(s_red));
    if (threadIdx.x == 0) ctl->max_key = max_key;
    if (mode & MODE_TOPP_MAX) return;
    unsigned long long own_c = 0, own_m = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        if (!topk) cnt[j] = 0;
        own_c += cnt[j];
        own_m += mass[j];
    }
    unsigned long long above_m = block_scan_inclusive<unsigned long long, kRThreads>(own_m, s_red) - own_m;
    if (topk) {
        unsigned long long above_c = block_scan_inclusive<unsigned long long, kRThreads>(own_c, s_red) - own_c;
        const unsigned long long k = ctl->k;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            if (above_c < k && k <= above_c + cnt[j]) {
                ctl->jstar = (uint32_t)(d0 + j);
                ctl->rank = (uint32_t)(k - above_c);
                ctl->A = above_m;
            }
            above_c += cnt[j];
            above_m += mass[j];
        }
    } else {
        // Nucleus only (no counts kept): a bin whose logits all have mass 0
        // (below 2^-40 of the max's) has the whole Z above it, which exceeds
        // p Z for p < 1, so the non-empty bins that can qualify are exactly
        // those with mass.
        const double limit = (double)a.top_p[b] * (double)ctl->Z;
        long long cand = -1;
        unsigned long long cand_above = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            if (mass[j] && (double)above_m <= limit) {
                cand = d0 + j;
                cand_above = above_m;
            }
            above_m += mass[j];
        }
        const long long best = block_max<long long, kRThreads>(cand, reinterpret_cast<long long *>(s_red));
        if (cand >= 0 && cand == best) {
            ctl->jstar = (uint32_t)cand;
            ctl->A = cand_above;
        }
    }
}

// Eligible logits above the threshold bin join the Gumbel argmax; logits of
// the threshold bin are appended to the candidate list.  The noise is read
// only where it is needed: the (index, z) pairs that need it are compacted
// in LDS and their noise fetched together, kList pairs per round.  ROUND2:
// only rows waiting for a second round work.
template <bool VEC4, bool MASK, bool ROUND2>
__global__ __launch_bounds__(kThreads) void samp_collect_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    SampCtl *ctl = a.ctl + b;
    if (ROUND2 && !ctl->round2) return;
    __shared__ unsigned long long s_red[kThreads / 64];
    __shared__ uint32_t s_tot, s_base;
    __shared__ uint32_t s_idx[kList];   // index | kCandBit
    __shared__ float s_s[kList];
    __shared__ uint32_t s_slot[kList];
    const int i0 = blockIdx.x * a.chunk;
    const int i1 = min(a.vocab, i0 + a.chunk);
    const int per = a.chunk / kThreads;
    const float *g = a.gumbel + (int64_t)b * a.gstride;
    // the tile is requested before the row's settings are read, so that
    // the two overlap
    Tile<VEC4> t;
    t.template load<true>(a.logits + (int64_t)b * a.lstride, i0, i1, per);
    t.load_mask(MASK ? a.mask + (int64_t)b * a.mstride : nullptr, i0, i1, per);
    const uint32_t mode = a.flags ? ctl->mode : row_mode(a, b);
    unsigned long long best = 0;
    if (mode & MODE_GREEDY) {
        for_each_elem<VEC4>(i0, i1, per, [&](int j) {
            const uint32_t i = (uint32_t)Tile<VEC4>::index(i0, j);
            best = max(best, pack_key_index(float_key(t.raw(j)), i));
        });
    } else if (mode & MODE_PLAIN) {
        // every logit is eligible: stream the noise as a tile too, half a
        // tile at a time (fewer registers live)
        const float T = a.temperature[b];
        const Scaler sc(T);
        Tile<VEC4> gt;
        auto first_half = [&](int j) {
            if (j >= kMaxPer / 2) return;
            const float kappa = t.scaled(j, sc) + gt.v[j];
            best = max(best, pack_key_index(float_key(kappa), (uint32_t)Tile<VEC4>::index(i0, j)));
        };
        gt.template load_range<0, kMaxPer / 2>(g, i0, i1, per);
        for_each_elem<VEC4>(i0, i1, per, first_half);
        gt.template load_range<kMaxPer / 2, kMaxPer / 2>(g, i0, i1, per);
        for_each_elem<VEC4>(i0, i1, per, [&](int j) {
            if (j < kMaxPer / 2) return;
            const float kappa = t.scaled(j, sc) + gt.v[j];
            best = max(best, pack_key_index(float_key(kappa), (uint32_t)Tile<VEC4>::index(i0, j)));
        });
    } else {
        const float T = a.temperature[b];
        const Scaler sc(T);
        const uint32_t max_key = ctl->max_key;
        const float M = key_float(max_key);
        const int jstar = (int)ctl->jstar;
        const bool maxima = (mode & MODE_TOPP_MAX) != 0;
        uint32_t kept = 0, incand = 0;
        // The class bits are shifted in from the top element down, one
        // dependent step each, so no element's bit waits in a register of
        // its own.
        const bool full = Tile<VEC4>::full(i0, i1, per);
        if (maxima) {
            // p <= 0: the logits whose s equals the row max (t.v becomes s)
#pragma unroll
            for (int j = kMaxPer - 1; j >= 0; --j) {
                const bool in = full | ((j < per) & (Tile<VEC4>::index(i0, j) < i1));
                const float s = t.scaled(j, sc);
                t.v[j] = s;
                kept = (kept << 1) | ((in & (float_key(s) == max_key)) ? 1u : 0u);
            }
        } else {
            // The class of an allowed logit follows from z itself, so z / T
            // is computed only for the logits that go to the list (t.v stays
            // z).  The two thresholds are found while the tile loads are in
            // flight.  Forbidden logits (s = kMasked) and NaN ones (bin
            // kBins - 1) take their bin's class.
            __shared__ float s_zt[2];
            z_thresholds(T, M, jstar, s_zt);
            __syncthreads();
            const float z_elig = s_zt[0], z_cand = s_zt[1];
            const int bm = bin_of(kMasked, M);
            const bool ok_m = bm < jstar, c_m = bm == jstar;
            const bool ok_n = kBins - 1 < jstar, c_n = kBins - 1 == jstar;
#pragma unroll
            for (int j = kMaxPer - 1; j >= 0; --j) {
                const bool in = full | ((j < per) & (Tile<VEC4>::index(i0, j) < i1));
                const float z = t.v[j];
                const bool allowed = (t.ok >> j) & 1u;
                const bool nan = !(z == z);
                const bool ge_elig = z >= z_elig, ge_cand = z >= z_cand;
                const bool ok = !allowed ? ok_m : (nan ? ok_n : ge_elig);
                const bool c = !allowed ? c_m : (nan ? c_n : (!ge_elig & ge_cand));
                kept = (kept << 1) | ((in & ok) ? 1u : 0u);
                incand = (incand << 1) | ((in & c) ? 1u : 0u);
            }
        }
        const uint32_t need = kept | incand;
        const uint32_t nc = __popc(incand), nn = __popc(need);
        // candidates (high half) and noise reads (low half) before this thread;
        // both totals stay below 2^16
        const uint32_t incl = block_scan_inclusive<uint32_t, kThreads>((nc << 16) | nn,
                                                                       reinterpret_cast<uint32_t *>(s_red));
        // The last thread claims the workgroup's candidate slots; the claim's
        // result is needed only when the candidates are written, so its
        // latency overlaps the list building and the noise reads.
        uint32_t claimed = 0;
        if (threadIdx.x == kThreads - 1) {
            s_tot = incl;
            if (incl >> 16) claimed = atomicAdd(&ctl->ncand, incl >> 16);
        }
        __syncthreads();
        const uint32_t tot_n = s_tot & 0xffffu;
        unsigned long long *cand = a.cand + (int64_t)b * kCap;
        uint32_t *kap = a.kap + (int64_t)b * kCap;
        // s of a listed logit: z / T, or kMasked (the maxima rows hold s)
        auto scaled_entry = [&](float v, bool masked) {
            return maxima ? v : (masked ? kMasked : v / T);
        };
        // candidate `lc` of this workgroup: its key and Gumbel key go to slot cbase + lc
        auto put_cand = [&](uint32_t cs, float sv, uint32_t kk, uint32_t i) {
            if (cs < (uint32_t)kCap) {
                cand[cs] = pack_key_index(float_key(sv), i);
                kap[cs] = kk;
            }
        };
        uint32_t lc = (incl >> 16) - nc;  // this thread's first candidate, within the workgroup
        if (tot_n <= (uint32_t)kList) {
            // one list: this thread's entries take positions [pos0, pos0 + nn)
            uint32_t pos = (incl & 0xffffu) - nn;
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j) {
                if (!((need >> j) & 1u)) continue;
                const bool c = (incand >> j) & 1u;
                const uint32_t i = (uint32_t)Tile<VEC4>::index(i0, j);
                s_idx[pos] = i | (c ? kCandBit : 0u) | (((kept >> j) & 1u) ? kKeptBit : 0u);
                s_s[pos] = t.v[j];
                s_slot[pos] = lc | (((t.ok >> j) & 1u) ? 0u : kSlotMasked);
                ++pos;
                lc += c ? 1u : 0u;
            }
            __syncthreads();
            constexpr int R = kList / kThreads;
            float gv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t q = (uint32_t)(r * kThreads) + threadIdx.x;
                gv[r] = q < tot_n ? g[s_idx[q] & kIndexMask] : 0.f;
            }
            if (threadIdx.x == kThreads - 1) s_base = claimed;
            __syncthreads();
            const uint32_t cbase = s_base;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t q = (uint32_t)(r * kThreads) + threadIdx.x;
                if (q >= tot_n) continue;
                const uint32_t e = s_idx[q];
                const uint32_t i = e & kIndexMask;
                const uint32_t sq = s_slot[q];
                const float sv = scaled_entry(s_s[q], (sq & kSlotMasked) != 0);
                const uint32_t kk = float_key(sv + gv[r]);
                if (e & kKeptBit) best = max(best, pack_key_index(kk, i));
                if (e & kCandBit) put_cand(cbase + (sq & ~kSlotMasked), sv, kk, i);
            }
        } else {
            // more entries than the list holds: each thread reads the noise
            // of its own entries
            if (threadIdx.x == kThreads - 1) s_base = claimed;
            __syncthreads();
            const uint32_t cbase = s_base;
#pragma unroll
            for (int j = 0; j < kMaxPer; ++j) {
                if (!((need >> j) & 1u)) continue;
                const uint32_t i = (uint32_t)Tile<VEC4>::index(i0, j);
                const float sv = scaled_entry(t.v[j], !((t.ok >> j) & 1u));
                const uint32_t kk = float_key(sv + g[i]);
                if ((kept >> j) & 1u) best = max(best, pack_key_index(kk, i));
                if ((incand >> j) & 1u) put_cand(cbase + lc++, sv, kk, i);
            }
        }
    }
    best = block_max<unsigned long long, kThreads>(best, s_red);
    if (threadIdx.x == 0) a.part_best[(int64_t)b * a.nchunks + blockIdx.x] = best;
}

// ---- per-row resolution ---------------------------------------------------

struct ResolveShared {
    union {
        struct {
            unsigned long long key[kCap];  // candidates (sorted, descending, above kRThreads)
            uint32_t kap[kCap];
            unsigned long long w[kRThreads];  // masses of the kept few
        };
        struct {                           // exact in-row fallback
            uint32_t hcnt[kDigits];
            unsigned long long hmass[kDigits];
        };
    };
    unsigned long long scan[kRThreads];
};

// Descending bitonic sort of n (a power of two) packed keys with payload.
__device__ void bitonic_sort_desc(unsigned long long *key, uint32_t *pay, int n)
{
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += kRThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const unsigned long long x = key[i], y = key[ixj];
                    const bool first = (i & k) == 0;
                    if (first ? (x < y) : (x > y)) {
                        key[i] = y;
                        key[ixj] = x;
                        const uint32_t p = pay[i];
                        pay[i] = pay[ixj];
                        pay[ixj] = p;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// In-row exact machinery (used when the threshold bin overflows the
// candidate list).  The row is rescanned from memory; `sel` picks the logits
// that take part (in the threshold bin, maybe kept by top-k).
struct RowScan {
    const float *z;
    const uint8_t *m;   // mask row or null
    float T, M;
    int V;
    int jstar;
};

__device__ __forceinline__ bool in_bin(const RowScan &r, int i, float &s, uint32_t &key)
{
    s = (r.m && !r.m[i]) ? kMasked : r.z[i] / r.T;
    key = float_key(s);
    return bin_of(s, r.M) == r.jstar;
}

// Radix select, three levels of 11/11/10 key bits, over the logits of the
// threshold bin that pass `kept_k` (top-k cut: key > kkey or key == kkey and
// index <= kcut; kkey == 0 means no cut).  BY_MASS: the lowest digit whose
// strictly-greater mass stays within `limit` given mass `above` of keys
// above the bin; else: the digit holding the rank-th largest key.  Returns
// the exact key; for ranks, `rank_left` is how many of its ties to keep.
template <bool BY_MASS>
__device__ uint32_t radix_in_bin(const RowScan &r, ResolveShared &sh, uint32_t kkey, uint32_t kcut,
                                 unsigned long long above, double limit, uint32_t rank,
                                 uint32_t *rank_left)
{
    uint32_t prefix = 0;
    constexpr int DPT = kDigits / kRThreads;
    __shared__ int s_d;
    __shared__ unsigned long long s_above;
    __shared__ uint32_t s_rank;
    if (threadIdx.x == 0) {
        s_above = above;
        s_rank = rank;
    }
    __syncthreads();
    for (int level = 0; level < 3; ++level) {
        const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
        const int width = level == 2 ? 10 : 11;
        const int hi = shift + width;
        const unsigned long long rk = s_rank;   // read before any thread can update it
        const unsigned long long A = s_above;
        for (int d = threadIdx.x; d < kDigits; d += kRThreads) {
            sh.hcnt[d] = 0;
            sh.hmass[d] = 0;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < r.V; i += kRThreads) {
            float s;
            uint32_t key;
            if (!in_bin(r, i, s, key)) continue;
            if (kkey && !(key > kkey || (key == kkey && (uint32_t)i <= kcut))) continue;
            if (hi < 32 && (key >> hi) != (prefix >> hi)) continue;
            const uint32_t d = (key >> shift) & ((1u << width) - 1u);
            atomicAdd(&sh.hcnt[d], 1u);
            if (BY_MASS) atomicAdd(&sh.hmass[d], mass_fixed(s, r.M));
        }
        __syncthreads();
        // thread t owns digits [DPT t, DPT t + DPT); scan from the top digit down
        const int d_hi = (int)threadIdx.x * DPT + DPT - 1;
        unsigned long long own = 0;
        for (int j = 0; j < DPT; ++j) own += BY_MASS ? sh.hmass[d_hi - j] : sh.hcnt[d_hi - j];
        // exclusive sum over the digits above this thread's range
        __syncthreads();
        sh.scan[kRThreads - 1 - threadIdx.x] = own;
        __syncthreads();
        for (int off = 1; off < kRThreads; off <<= 1) {
            const int tt = kRThreads - 1 - (int)threadIdx.x;
            const unsigned long long add = tt >= off ? sh.scan[tt - off] : 0ull;
            __syncthreads();
            sh.scan[tt] += add;
            __syncthreads();
        }
        unsigned long long up = sh.scan[kRThreads - 1 - threadIdx.x] - own;
        if (threadIdx.x == 0) s_d = kDigits;
        __syncthreads();
        if (BY_MASS) {
            int cand = -1;
            unsigned long long cand_up = 0;
            for (int j = 0; j < DPT; ++j) {
                const int d = d_hi - j;
                if ((double)(A + up) > limit) break;
                if (sh.hcnt[d]) {
                    cand = d;
                    cand_up = up;
                }
                up += sh.hmass[d];
            }
            // the lowest qualifying digit
            if (cand >= 0) atomicMin(&s_d, cand);
            __syncthreads();
            if (cand >= 0 && cand == s_d) s_above = A + cand_up;
            __syncthreads();
            prefix |= (uint32_t)s_d << shift;
        } else {
            for (int j = 0; j < DPT; ++j) {
                const int d = d_hi - j;
                const unsigned long long c = sh.hcnt[d];
                if (up < rk && rk <= up + c) {
                    s_d = d;
                    s_rank = (uint32_t)(rk - up);
                }
                up += c;
            }
            __syncthreads();
            prefix |= (uint32_t)s_d << shift;
        }
        __syncthreads();
    }
    if (rank_left) *rank_left = s_rank;
    return prefix;
}

// Index of the `need`-th (1-based) logit of the threshold bin, in index
// order, whose key equals `key`.
__device__ uint32_t nth_tie_index(const RowScan &r, ResolveShared &sh, uint32_t key, uint32_t need)
{
    __shared__ uint32_t s_wave[kRThreads / 64];
    __shared__ uint32_t s_found;
    __shared__ uint32_t s_seen;
    if (threadIdx.x == 0) {
        s_found = 0xffffffffu;
        s_seen = 0;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int base = 0; base < r.V; base += kRThreads) {
        const int i = base + (int)threadIdx.x;
        bool hit = false;
        if (i < r.V) {
            float s;
            uint32_t k2;
            hit = in_bin(r, i, s, k2) && k2 == key;
        }
        const unsigned long long m = __ballot(hit);
        if (lane == 0) s_wave[wave] = __popcll(m);
        __syncthreads();
        uint32_t before = s_seen;
        for (int w = 0; w < wave; ++w) before += s_wave[w];
        const uint32_t below = __popcll(m & ((1ull << lane) - 1ull));
        if (hit && before + below + 1 == need) s_found = (uint32_t)i;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t tot = 0;
            for (int w = 0; w < kRThreads / 64; ++w) tot += s_wave[w];
            s_seen += tot;
        }
        __syncthreads();
        if (s_found != 0xffffffffu) break;
    }
    return s_found;
}

// Gumbel argmax over the threshold bin's logits that pass the final cut.
__device__ unsigned long long best_in_bin(const RowScan &r, const float *g, ResolveShared &sh,
                                          uint32_t kkey, uint32_t kcut, uint32_t tau)
{
    unsigned long long best = 0;
    for (int i = threadIdx.x; i < r.V; i += kRThreads) {
        float s;
        uint32_t key;
        if (!in_bin(r, i, s, key)) continue;
        if (kkey && !(key > kkey || (key == kkey && (uint32_t)i <= kcut))) continue;
        if (key < tau) continue;
        best = max(best, pack_key_index(float_key(s + g[i]), (uint32_t)i));
    }
    return block_max<unsigned long long, kRThreads>(best, sh.scan);
}

// Mass of the threshold bin's logits kept by the top-k cut.
__device__ unsigned long long kept_mass_in_bin(const RowScan &r, ResolveShared &sh, uint32_t kkey,
                                               uint32_t kcut)
{
    unsigned long long m = 0;
    for (int i = threadIdx.x; i < r.V; i += kRThreads) {
        float s;
        uint32_t key;
        if (!in_bin(r, i, s, key)) continue;
        if (!(key > kkey || (key == kkey && (uint32_t)i <= kcut))) continue;
        m += mass_fixed(s, r.M);
    }
    return block_sum<unsigned long long, kRThreads>(m, sh.scan);
}

// Second collect/resolve pass, set-up: the nucleus cut of a top-k row lies
// above its top-k bin.
// Every logit in bins above `jk` is in the top-k set, so the nucleus over
// that set is found like a plain nucleus with total mass Zk.
__device__ void setup_round2(const SampArgs &a, SampCtl *ctl, ResolveShared &sh, int b, int jk,
                             unsigned long long Zk)
{
    constexpr int BPT = kBins / kRThreads;
    const double limit = (double)a.top_p[b] * (double)Zk;
    const int d0 = (int)threadIdx.x * BPT;
    unsigned long long own = 0;
    for (int j = 0; j < BPT; ++j) own += a.mass[(int64_t)b * kBins + d0 + j];
    unsigned long long above = block_scan_inclusive<unsigned long long, kRThreads>(own, sh.scan) - own;
    long long cand = -1;
    unsigned long long cand_above = 0;
    for (int j = 0; j < BPT; ++j) {
        const int d = d0 + j;
        if (d < jk && a.cnt[(int64_t)b * kBins + d] && (double)above <= limit) {
            cand = d;
            cand_above = above;
        }
        above += a.mass[(int64_t)b * kBins + d];
    }
    const long long best = block_max<long long, kRThreads>(cand, reinterpret_cast<long long *>(sh.scan));
    if (cand >= 0 && cand == best) {
        ctl->jstar = (uint32_t)cand;
        ctl->A = cand_above;
        ctl->Z = Zk;
        ctl->mode = MODE_TOPP;
        ctl->ncand = 0;
        ctl->round2 = 1;
    }
}

template <bool ROUND2>
__global__ __launch_bounds__(kRThreads) void samp_resolve_kernel(const SampArgs a)
{
    __shared__ ResolveShared sh;
    const int b = blockIdx.x;
    SampCtl *ctl = a.ctl + b;
    // Everything the row may need is requested up front, so that the loads
    // overlap: the chunks' best keys, the first kRThreads list entries (in
    // bounds whatever the count; entries past it are ignored) and the
    // control block.
    const int i = (int)threadIdx.x;
    unsigned long long best = 0;
    {
        const unsigned long long *pb = a.part_best + (int64_t)b * a.nchunks;
        for (int c = i; c < a.nchunks; c += kRThreads) best = max(best, pb[c]);
    }
    const unsigned long long cand0 = a.cand[(int64_t)b * kCap + i];
    const uint32_t kap0 = a.kap[(int64_t)b * kCap + i];
    const double p = (double)a.top_p[b];
    SampCtl c = {};
    if (a.flags) c = *ctl;
    if (ROUND2 && !c.round2) return;
    const uint32_t mode = a.flags ? c.mode : row_mode(a, b);
    if (mode & MODE_DONE) return;
    // best eligible logit outside the threshold bin, over the chunks
    best = block_max<unsigned long long, kRThreads>(best, sh.scan);
    if (mode & (MODE_GREEDY | MODE_PLAIN | MODE_TOPP_MAX)) {
        if (threadIdx.x == 0) {
            a.out_ids[b] = (int32_t)unpack_index(best);
            if (a.flags) {
                ctl->mode = mode | MODE_DONE;
                ctl->tau = (mode & MODE_TOPP_MAX) ? c.max_key : 0u;
                ctl->kpack = 0;
            }
        }
        return;
    }
    // the final cut, kept for the extra outputs: key >= cut_tau and, for
    // top-k, (key, ~index) >= cut_k
    uint32_t cut_tau = 0;
    unsigned long long cut_k = 0;
    const bool topk = (mode & MODE_TOPK) != 0;
    const bool topp = (mode & MODE_TOPP) != 0;
    const uint32_t n = c.ncand;
    const float M = key_float(c.max_key);
    const unsigned long long A = c.A;
    const int jstar = (int)c.jstar;

    if (n <= (uint32_t)kRThreads) {
        // ---- few candidates: ranks and masses above by direct counting ----
        // q lanes (consecutive, q <= 64) share candidate e = i / q and split
        // the comparisons against all n candidates between them.
        int np = 1;
        while (np < (int)n) np <<= 1;
        const int q = min(64, kRThreads / np);
        const int e = i / q, part = i % q;
        sh.key[i] = i < (int)n ? cand0 : 0ull;
        sh.kap[i] = kap0;
        __syncthreads();
        const bool real = e < (int)n;
        const unsigned long long ke = real ? sh.key[e] : 0ull;
        const uint32_t se = (uint32_t)(ke >> 32);
        // top-k keeps the r largest (s, then lowest index); the nucleus runs
        // over what top-k keeps
        bool kept = real;
        if (topk) {
            uint32_t larger = 0;
            for (int j = part; j < (int)n; j += q) larger += sh.key[j] > ke ? 1u : 0u;
            larger = group_sum_lanes(larger, q);
            kept = real && larger < c.rank;
        }
        uint32_t tau = 0;
        if (topp) {
            __shared__ unsigned long long s_tot;
            const unsigned long long w = kept ? mass_fixed(key_float(se), M) : 0ull;
            if (part == 0 && real) sh.w[e] = w;
            const unsigned long long tot = block_sum<unsigned long long, kRThreads>(part == 0 ? w : 0ull, sh.scan);
            unsigned long long Zrow = c.Z;
            if (topk) {
                // the nucleus over the top-k set: total mass above the bin + kept candidates
                Zrow = A + tot;
                if ((double)A > p * (double)Zrow) {
                    setup_round2(a, ctl, sh, b, jstar, Zrow);
                    return;
                }
            }
            const double limit = p * (double)Zrow;
            // mass of kept candidates with a strictly larger s
            unsigned long long above = 0;
            for (int j = part; j < (int)n; j += q) above += (uint32_t)(sh.key[j] >> 32) > se ? sh.w[j] : 0ull;
            above = group_sum_lanes(above, q);
            // the smallest s whose strictly-larger mass fits the limit
            const uint32_t fit = (kept && (double)(A + above) <= limit) ? se : 0xffffffffu;
            tau = ~block_max<uint32_t, kRThreads>(~fit, reinterpret_cast<uint32_t *>(sh.scan));
        }
        if (part == 0 && kept && se >= tau) best = max(best, pack_key_index(sh.kap[e], unpack_index(ke)));
        best = block_max<unsigned long long, kRThreads>(best, sh.scan);
        cut_tau = tau;
        if (topk)  // the smallest packed key top-k keeps
            cut_k = ~block_max<unsigned long long, kRThreads>((part == 0 && kept) ? ~ke : 0ull, sh.scan);
    } else if (n <= (uint32_t)kCap) {
        // ---- sort the candidates of the threshold bin ----
        int np = 1;
        while (np < (int)n) np <<= 1;
        for (int i = threadIdx.x; i < np; i += kRThreads) {
            sh.key[i] = i < (int)n ? a.cand[(int64_t)b * kCap + i] : 0ull;
            sh.kap[i] = i < (int)n ? a.kap[(int64_t)b * kCap + i] : 0u;
        }
        __syncthreads();
        bitonic_sort_desc(sh.key, sh.kap, np);
        // thread t owns sorted positions [PT t, PT t + PT)
        constexpr int PT = kCap / kRThreads;
        const int i0 = (int)threadIdx.x * PT;
        // top-k keeps the first r; the nucleus runs over what top-k keeps
        const int r = topk ? (int)c.rank : (int)n;
        unsigned long long w[PT];
        unsigned long long own = 0;
        for (int j = 0; j < PT; ++j) {
            const int i = i0 + j;
            w[j] = (topp && i < r) ? mass_fixed(key_float((uint32_t)(sh.key[i] >> 32)), M) : 0ull;
            own += w[j];
        }
        const unsigned long long incl = block_scan_inclusive<unsigned long long, kRThreads>(own, sh.scan);
        const unsigned long long excl0 = incl - own;
        uint32_t tau = 0;
        if (topp) {
            unsigned long long Zrow = c.Z;
            if (topk) {
                // the nucleus over the top-k set: total mass above the bin + kept candidates
                __shared__ unsigned long long s_tot;
                if (threadIdx.x == kRThreads - 1) s_tot = incl;
                __syncthreads();
                Zrow = A + s_tot;
                if ((double)A > p * (double)Zrow) {
                    setup_round2(a, ctl, sh, b, jstar, Zrow);
                    return;
                }
            }
            const double limit = p * (double)Zrow;
            // the lowest group head whose strictly-greater mass fits the limit
            long long last = -1;
            unsigned long long run = excl0;
            for (int j = 0; j < PT; ++j) {
                const int i = i0 + j;
                if (i < r) {
                    const uint32_t k1 = (uint32_t)(sh.key[i] >> 32);
                    const bool head = i == 0 || (uint32_t)(sh.key[i - 1] >> 32) != k1;
                    if (head && (double)(A + run) <= limit) last = i;
                }
                run += w[j];
            }
            const long long lh = block_max<long long, kRThreads>(last, reinterpret_cast<long long *>(sh.scan));
            tau = lh >= 0 ? (uint32_t)(sh.key[lh] >> 32) : 0u;
        }
        // best Gumbel key over the kept candidates
        for (int j = 0; j < PT; ++j) {
            const int i = i0 + j;
            if (i < r && (uint32_t)(sh.key[i] >> 32) >= tau)
                best = max(best, pack_key_index(sh.kap[i], unpack_index(sh.key[i])));
        }
        best = block_max<unsigned long long, kRThreads>(best, sh.scan);
        cut_tau = tau;
        if (topk) cut_k = sh.key[r - 1];
    } else {
        // ---- the threshold bin overflowed the list: exact cut from the row ----
        RowScan rs;
        rs.z = a.logits + (int64_t)b * a.lstride;
        rs.m = a.mask ? a.mask + (int64_t)b * a.mstride : nullptr;
        rs.T = a.temperature[b];
        rs.M = M;
        rs.V = a.vocab;
        rs.jstar = jstar;
        const float *g = a.gumbel + (int64_t)b * a.gstride;
        uint32_t kkey = 0, kcut = 0xffffffffu, tau = 0;
        if (topk) {
            uint32_t left = 0;
            kkey = radix_in_bin<false>(rs, sh, 0, 0, 0, 0.0, c.rank, &left);
            // keep only the `left` lowest-index logits equal to the k-th key
            kcut = nth_tie_index(rs, sh, kkey, left);
        }
        if (topp) {
            unsigned long long Zrow = c.Z;
            if (topk) {
                Zrow = A + kept_mass_in_bin(rs, sh, kkey, kcut);
                if ((double)A > p * (double)Zrow) {
                    setup_round2(a, ctl, sh, b, jstar, Zrow);
                    return;
                }
            }
            tau = radix_in_bin<true>(rs, sh, kkey, kcut, A, p * (double)Zrow, 0, nullptr);
        }
        const unsigned long long bb = best_in_bin(rs, g, sh, kkey, kcut, tau);
        best = max(best, bb);
        cut_tau = tau;
        if (topk) cut_k = pack_key_index(kkey, kcut);
    }
    if (threadIdx.x == 0) {
        a.out_ids[b] = (int32_t)unpack_index(best);
        ctl->mode = mode | MODE_DONE;
        ctl->round2 = 0;
        ctl->tau = cut_tau;
        ctl->kpack = cut_k;
    }
}

// ---- extra outputs ---------------------------------------------------------

// One workgroup per row, after the draw: the drawn id's probability under
// the softmax of the kept scaled logits, and the 8 kept ids of largest s
// (ties to the lower index) with their probabilities; fewer than 8 kept ids
// are followed by the lowest-index ids outside the kept set (probability
// 0).  Greedy rows: the distribution is uniform over the tied maxima of the
// masked raw logits.  The row is read once (max, fp64 sum of exp(s - max)
// with running rescale, per-thread top 8), plus an ordered index scan when
// fewer than 8 ids are kept or for greedy ties.
__global__ __launch_bounds__(kRThreads) void samp_extras_kernel(const SampArgs a)
{
    const int b = blockIdx.x;
    const uint32_t mode = a.flags ? (a.ctl[b].mode & ~MODE_DONE) : row_mode(a, b);
    const bool greedy = (mode & MODE_GREEDY) != 0;
    const uint32_t tau = (a.flags && !greedy) ? a.ctl[b].tau : 0u;
    const unsigned long long kpack = (a.flags && !greedy) ? a.ctl[b].kpack : 0ull;
    const float T = a.temperature[b];
    const float *z = a.logits + (int64_t)b * a.lstride;
    const uint8_t *mk = a.mask ? a.mask + (int64_t)b * a.mstride : nullptr;
    const int V = a.vocab;
    const int id = a.out_ids[b];

    __shared__ unsigned long long s_red[kRThreads / 64];
    __shared__ double s_dred[kRThreads / 64];
    __shared__ unsigned long long s_top[8];
    __shared__ int s_idx[8];
    __shared__ int s_found;
    __shared__ uint32_t s_wave[kRThreads / 64];

    auto value = [&](int i) -> float {
        const bool ok = !mk || mk[i];
        return greedy ? (ok ? z[i] : kMasked) : (ok ? z[i] / T : kMasked);
    };
    auto kept = [&](int i, float v) -> bool {
        if (greedy) return true;
        const uint32_t k = float_key(v);
        return k >= tau && (kpack == 0 || pack_key_index(k, (uint32_t)i) >= kpack);
    };

    // one pass: running max and fp64 sum over the kept, per-thread top 8
    float mt = -INFINITY;
    double zt = 0.0;
    unsigned long long top[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) top[r] = 0;
    uint32_t nkept = 0;
    for (int i = threadIdx.x; i < V; i += kRThreads) {
        const float v = value(i);
        if (!kept(i, v)) continue;
        ++nkept;
        if (v > mt) {
            zt = (mt == -INFINITY) ? 1.0 : zt * (double)expf(mt - v) + 1.0;
            mt = v;
        } else {
            zt += (double)expf(v - mt);
        }
        const unsigned long long key = pack_key_index(float_key(v), (uint32_t)i);
        if (key > top[7]) {
            top[7] = key;
#pragma unroll
            for (int r = 7; r > 0; --r)
                if (top[r] > top[r - 1]) {
                    const unsigned long long x = top[r];
                    top[r] = top[r - 1];
                    top[r - 1] = x;
                }
        }
    }
    const float M = key_float(block_max<uint32_t, kRThreads>(
        mt == -INFINITY ? 0u : float_key(mt), reinterpret_cast<uint32_t *>(s_red)));
    const double Z = block_sum<double, kRThreads>(
        mt == -INFINITY ? 0.0 : zt * exp((double)mt - (double)M), s_dred);
    const uint32_t total_kept = (uint32_t)block_sum<unsigned long long, kRThreads>(nkept, s_red);

    // the top 8 over the block: 8 rounds of a block max, the owner pops
    for (int r = 0; r < 8; ++r) {
        const unsigned long long w = block_max<unsigned long long, kRThreads>(top[0], s_red);
        if (threadIdx.x == 0) s_top[r] = w;
        if (w != 0 && top[0] == w) {
#pragma unroll
            for (int k = 0; k < 7; ++k) top[k] = top[k + 1];
            top[7] = 0;
        }
    }
    __syncthreads();

    // first `need` indices (in index order) that satisfy pred, into s_idx[from..]
    auto first_indices = [&](int from, int need, auto pred) {
        if (threadIdx.x == 0) s_found = 0;
        __syncthreads();
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        for (int base = 0; base < V; base += kRThreads) {
            const int i = base + (int)threadIdx.x;
            const bool hit = i < V && pred(i);
            const unsigned long long bal = __ballot(hit);
            if (lane == 0) s_wave[wave] = (uint32_t)__popcll(bal);
            __syncthreads();
            int before = s_found;
            for (int w = 0; w < wave; ++w) before += (int)s_wave[w];
            const int rank = before + (int)__popcll(bal & ((1ull << lane) - 1ull));
            if (hit && rank < need) s_idx[from + rank] = i;
            __syncthreads();
            if (threadIdx.x == 0) {
                int tot = 0;
                for (int w = 0; w < kRThreads / 64; ++w) tot += (int)s_wave[w];
                s_found += tot;
            }
            __syncthreads();
            if (s_found >= need) break;
        }
    };

    if (greedy) {
        // uniform over the tied maxima: their first 8 indices, then the others
        const uint32_t ties = (uint32_t)block_sum<unsigned long long, kRThreads>(
            [&] {
                uint32_t c = 0;
                for (int i = threadIdx.x; i < V; i += kRThreads) c += value(i) == M ? 1u : 0u;
                return (unsigned long long)c;
            }(),
            s_red);
        const int nt = (int)min(ties, 8u);
        first_indices(0, nt, [&](int i) { return value(i) == M; });
        if (nt < 8) first_indices(nt, min(8, V) - nt, [&](int i) { return value(i) != M; });
        if (threadIdx.x < 8) {
            const int r = threadIdx.x;
            const bool real = r < min(8, V);
            const int idx = real ? s_idx[r] : -1;
            const float pr = (r < nt) ? (float)(1.0 / (double)ties) : 0.f;
            if (a.out_top_ids) a.out_top_ids[(int64_t)b * 8 + r] = idx;
            if (a.out_top_probs) a.out_top_probs[(int64_t)b * 8 + r] = real ? pr : 0.f;
        }
        if (threadIdx.x == 0 && a.out_prob) a.out_prob[b] = (float)(1.0 / (double)ties);
        return;
    }

    const int nk = (int)min(total_kept, 8u);
    if (nk < 8) first_indices(nk, min(8, V) - nk, [&](int i) { return !kept(i, value(i)); });
    if (threadIdx.x < 8) {
        const int r = threadIdx.x;
        int idx = -1;
        float pr = 0.f;
        if (r < nk) {
            idx = (int)unpack_index(s_top[r]);
            pr = (float)(exp((double)key_float((uint32_t)(s_top[r] >> 32)) - (double)M) / Z);
        } else if (r < min(8, V)) {
            idx = s_idx[r];
        }
        if (a.out_top_ids) a.out_top_ids[(int64_t)b * 8 + r] = idx;
        if (a.out_top_probs) a.out_top_probs[(int64_t)b * 8 + r] = pr;
    }
    if (threadIdx.x == 0 && a.out_prob) {
        const float v = value(id);
        a.out_prob[b] = (float)(exp((double)v - (double)M) / Z);
    }
}

// MASK: a vocabulary mask is given (without one, the row-parallel passes
// are compiled with every logit allowed).
template <bool VEC4, bool MASK>
void launch_passes(const SampArgs &a, const dim3 grid, uint32_t flags, hipStream_t stream)
{
    if (flags) {
        samp_max_kernel<VEC4, MASK><<<grid, kThreads, 0, stream>>>(a);
        samp_bins_kernel<VEC4, MASK><<<grid, kThreads, 0, stream>>>(a);
        samp_select_kernel<<<a.batch, kRThreads, 0, stream>>>(a);
    }
    samp_collect_kernel<VEC4, MASK, false><<<grid, kThreads, 0, stream>>>(a);
    samp_resolve_kernel<false><<<a.batch, kRThreads, 0, stream>>>(a);
    if ((flags & 3u) == 3u) {
        // top-k then nucleus: rows whose nucleus cut lies above their top-k bin
        samp_collect_kernel<VEC4, MASK, true><<<grid, kThreads, 0, stream>>>(a);
        samp_resolve_kernel<true><<<a.batch, kRThreads, 0, stream>>>(a);
    }
    if (a.out_prob || a.out_top_ids || a.out_top_probs)
        samp_extras_kernel<<<a.batch, kRThreads, 0, stream>>>(a);
}

}  // namespace

size_t sampler_workspace_bytes(int32_t batch, int32_t vocab)
{
    return sampler_layout(batch, vocab).total;
}

hipError_t launch_sampler(int32_t *out_ids, const float *logits, int64_t logits_stride,
                          const float *gumbel, int64_t gumbel_stride, const uint8_t *mask,
                          int64_t mask_stride, const float *temperature, const float *top_p,
                          const int32_t *top_k, int32_t batch, int32_t vocab, uint32_t flags,
                          float *out_prob, int32_t *out_top_ids, float *out_top_probs,
                          void *workspace, hipStream_t stream)
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
    a.cand = reinterpret_cast<unsigned long long *>(ws + L.cand_off);
    a.kap = reinterpret_cast<uint32_t *>(ws + L.kap_off);
    a.part_max = reinterpret_cast<uint32_t *>(ws + L.pmax_off);
    a.part_best = reinterpret_cast<unsigned long long *>(ws + L.pbest_off);
    a.mask = mask;
    a.mstride = mask_stride;
    a.out_prob = out_prob;
    a.out_top_ids = out_top_ids;
    a.out_top_probs = out_top_probs;

    const dim3 grid(L.nchunks, batch);
    const bool vec4 = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && logits_stride % 4 == 0 &&
                      (reinterpret_cast<uintptr_t>(gumbel) % 16 == 0) && gumbel_stride % 4 == 0 &&
                      (!mask || (reinterpret_cast<uintptr_t>(mask) % 4 == 0 && mask_stride % 4 == 0)) &&
                      vocab % 4 == 0;
    if (vec4)
        a.mask ? launch_passes<true, true>(a, grid, flags, stream)
               : launch_passes<true, false>(a, grid, flags, stream);
    else
        a.mask ? launch_passes<false, true>(a, grid, flags, stream)
               : launch_passes<false, false>(a, grid, flags, stream);
    return hipGetLastError();
}

}  // namespace pkv
