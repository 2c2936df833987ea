// Next-token sampler: temperature, top-k, nucleus (top-p) and a Gumbel-max
// draw, on fp32 logits [B][V], in three launches.
//
// scan   (one 256-thread workgroup per (chunk, row); the one pass over the
//        logits).  Greedy and unfiltered rows reduce their chunk to a best
//        packed key (the unfiltered ones read the noise too: every token is
//        eligible).  Filtered rows compute s = z / T, the chunk max M_c and
//        a histogram of 2048 value bins of width 1/32 below M_c, and from
//        it a candidate list: the tokens of the top bins, as many bins as
//        fit in the list (nucleus rows), or just enough to hold k (top-k)
//        or the maxima (p <= 0).  Every token of a listed bin is larger
//        than every unlisted one, so the chunk also records the largest
//        value it left out and, for nucleus rows, the mass of what it left
//        out (relative to M_c).
// hist   (up to kGroups 256-thread workgroups per filtered row, each over a
//        contiguous group of chunks).  With T* the largest value left out
//        by any chunk, the lists hold every token of the row with s > T*.
//        Each group bins its listed tokens above T* below the row max M
//        (1024 bins of width 1/32, the last one taking the rest): counts,
//        exact masses exp(s - M) (fp64, then 2^-38 fixed point: sums are
//        order independent and bit-reproducible) for nucleus rows, and the
//        best Gumbel key per bin (the noise of these tokens is read here);
//        prefix scans over the bins give each bin's offset and the best key
//        of the bins before it, and the tokens are written in bin order
//        with their noise.  The group's listed masses plus its chunks'
//        left-out masses give its share of Z.  Nothing is shared between
//        workgroups: each writes its own bins and totals.
// finish (one 1024-thread workgroup per row).  The groups' bins added up
//        give the bin holding the cut: the k-th largest (top-k) or the
//        deepest bin whose strictly-greater mass is within p of Z
//        (nucleus).  Every token in the bins before it is kept, and the
//        groups' prefix best keys give the best among them; only the cut
//        bin's tokens are read (from the groups' bin-sorted arrays) and the
//        exact cut among them is found in LDS.  This is valid when the cut
//        lies above T* (checked: at least k tokens above T*, or more than p
//        of the mass above T*).  Otherwise, and for top-k followed by a
//        nucleus, p <= 0 or a crowded cut bin, general selections (bins,
//        then radix selects by rank or by mass) run over the lists, or over
//        the whole row read again from memory when the cut may lie below
//        T* (slow but exact).
//
// Workgroups communicate only through kernel boundaries: no workgroup waits
// for or fences against another one, and no workspace memory needs clearing
// (every record, list, bin range and sorted array that a later launch reads
// is fully written earlier in the same call).
#include <math.h>

#include <type_traits>

#include "launch.hpp"
#include "pkv_device.hpp"

namespace pkv {

namespace {

constexpr int kThreads = 256;           // scan kernel
constexpr int kFThreads = 1024;         // finish kernel: one workgroup per row
constexpr int kRThreads = 512;          // extra outputs: one workgroup per row
constexpr int kBins = 512;              // scan: value bins below the chunk max ...
constexpr float kBinsPerUnit = 8.f;     // ... 1/8 of a logit unit wide
constexpr float kHBinsPerUnit = 32.f;   // finish-side bins: 1/32 of a unit
constexpr int kMaxPer = 16;             // logits per thread per chunk (more: register spills)
constexpr int kMinGroups = 512;         // scan workgroups wanted (two per CU)
constexpr int kListDiv = 8;             // list capacity per chunk: chunk / kListDiv
constexpr int kMaxChunks = 4096;        // vocab <= 2^24 in chunks of 4096
constexpr int kDigits = 4096;           // radix digits per level (<= 12 bits)
constexpr int kHBins = 1024;            // finish-side value bins (the last one takes the rest)
constexpr int kGroups = 8;              // histogram workgroups per row (at most)
constexpr int kGroupChunks = kMaxChunks / kGroups;   // chunks of one group (at most)
constexpr int kHThreads = 512;          // histogram kernel
constexpr int kHBatch = 8;              // list slots per thread whose loads are issued together
constexpr double kMassUnit = 0x1p38;    // fixed-point masses: 2^-38 of the row max's

enum : uint32_t {
    MODE_GREEDY = 1,     // T <= 0: lowest index of the max raw logit
    MODE_PLAIN = 2,      // T > 0 and no filter: every token eligible
    MODE_TOPK = 4,
    MODE_TOPP = 8,
    MODE_TOPP_MAX = 16,  // p <= 0: only the maxima are eligible
};

// One scan workgroup's result for its chunk.
struct alignas(32) ChunkRec {
    uint32_t mkey;             // key of the chunk max of s (filtered rows)
    uint32_t outkey;           // key of the largest s left out of the list (0: none)
    uint32_t n;                // tokens listed
    uint32_t pad;
    double zx;                 // mass of the tokens left out, exp(s - M_c) summed
    unsigned long long best;   // greedy / unfiltered rows: best packed key of the chunk
};
static_assert(sizeof(ChunkRec) == 32, "chunk record");

// The final cut of a row, for the extra outputs: kept tokens have
// key(s) >= tau and, for top-k, (key, ~index) >= kpack.
struct alignas(16) RowCut {
    uint32_t mode;
    uint32_t tau;
    unsigned long long kpack;
};

// Totals of one histogram workgroup's share of a row (integer sums: the
// row's totals do not depend on the order they are added in).
struct alignas(32) RowTot {
    unsigned long long Z;    // mass of its tokens (2^-38 units of the row max's)
    unsigned long long mu;   // mass of its listed tokens above T*
    uint32_t nu;             // its listed tokens above T*
    uint32_t kmax, tout;     // the row max's key and T*'s (the same in every group)
    uint32_t pad;
};
static_assert(sizeof(RowTot) == 32, "row totals");

// One histogram group's share of a finish-side value bin.
struct alignas(8) BinRec {
    uint32_t cnt;              // the group's listed tokens above T* in the bin
    uint32_t off;              // ... in the bins before it (where the bin starts
                               // in the group's bin-sorted tokens)
    unsigned long long mass;   // mass of the bin's tokens (nucleus rows)
    unsigned long long above;  // best Gumbel key of the group's tokens in the
                               // bins before it (0: none)
};
static_assert(sizeof(BinRec) == 24, "bin record");

// A listed token above T* with its noise, in a group's bin-sorted array.
struct alignas(16) SortedTok {
    unsigned long long packed;
    float g;
    uint32_t pad;
};

struct SampLayout {
    int32_t chunk, nchunks, cap, groups;
    int32_t gslots;   // bin-sorted tokens per group (at most)
    size_t rec_off, list_off, bins_off, sorted_off, tot_off, cut_off, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SampLayout sampler_layout(int32_t batch, int32_t vocab)
{
    SampLayout L;
    // the largest chunk that still gives kMinGroups scan workgroups
    int32_t chunk = kMaxPer * kThreads;
    while (chunk > 4 * kThreads && (int64_t)batch * ((vocab + chunk - 1) / chunk) < kMinGroups) chunk >>= 1;
    L.chunk = chunk;
    L.nchunks = (vocab + chunk - 1) / chunk;
    L.cap = chunk / kListDiv;
    L.groups = L.nchunks < kGroups ? L.nchunks : kGroups;
    const size_t slots = (size_t)batch * L.nchunks * L.cap;
    size_t off = 0;
    L.rec_off = off;
    off = align256(off + (size_t)batch * L.nchunks * sizeof(ChunkRec));
    L.list_off = off;
    off = align256(off + slots * sizeof(unsigned long long));
    // per row and histogram group: value bins, bin-sorted tokens, totals
    L.gslots = (L.nchunks + L.groups - 1) / L.groups * L.cap;
    L.bins_off = off;
    off = align256(off + (size_t)batch * L.groups * kHBins * sizeof(BinRec));
    L.sorted_off = off;
    off = align256(off + (size_t)batch * L.groups * L.gslots * sizeof(SortedTok));
    L.tot_off = off;
    off = align256(off + (size_t)batch * L.groups * sizeof(RowTot));
    L.cut_off = off;
    off = align256(off + (size_t)batch * sizeof(RowCut));
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
    int32_t batch, vocab, chunk, nchunks, cap, groups, gslots;
    ChunkRec *rec;                 // [B][nchunks]
    unsigned long long *list;      // [B][nchunks][cap]  (key << 32) | ~index
    BinRec *bins;                  // [B][groups][kHBins]
    SortedTok *sorted;             // [B][groups][gslots]
    RowTot *tot;                   // [B][groups]
    RowCut *cut;                   // [B]
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

// Value bin below the chunk max M: monotone non-increasing in s (rounding of
// M - s is monotone, the scale is a power of two); NaN lands in the last bin.
__device__ __forceinline__ int bin_of(float s, float M)
{
    const float d = (M - s) * kBinsPerUnit;
    return d < (float)(kBins - 1) ? (int)d : kBins - 1;
}

// The finish-side bin: as bin_of, with everything from kHBins - 1 bins down
// in the last one.
__device__ __forceinline__ int hbin_of(float s, float M)
{
    const float d = (M - s) * kHBinsPerUnit;
    return d < (float)(kHBins - 1) ? (int)d : kHBins - 1;
}

// exp(s - M) for s <= M, good to ~2e-7 relative however far s lies below M:
// s - M is exact in double, its base-2 exponent is split into an integer
// and a fraction in [0, 1) (both exact), and only the fraction goes through
// the fp32 exponential.  0 below 2^-200 (and for NaN).
__device__ __forceinline__ float mass_approx(float s, double M)
{
    // (-inf and NaN clamp to -200 too; 2^-200 and below round to 0 in fp32)
    const double x = fmax(((double)s - M) * 1.4426950408889634, -200.0);
    const double fl = floor(x);
    return ldexpf(__builtin_amdgcn_exp2f((float)(x - fl)), (int)fl);
}

// exp(s - M) for s <= M in fp64, to ~1e-14 relative: s - M is exact in
// double; with x = (s - M) log2(e) = e + j/64 + r (integers e, j in [0, 64),
// |r| <= 1/128), 2^x = 2^e * 2^(j/64) * exp(r ln 2), the middle factor from
// a 64-entry table of 2^(j/64) and the last from its Taylor series to the
// 6th power (remainder below 1e-19).  0 below 2^-1000 (and for NaN).
__device__ __forceinline__ double exp_below(double d, const double *tab)
{
    const double x = d * 1.4426950408889634;
    if (!(x > -1000.0)) return 0.0;
    const double k = rint(x * 64.0);
    const int ki = (int)k;
    const double y = (x - k * 0.015625) * 0.69314718055994531;
    double p = 1.0 + y * (1.0 / 6.0);
    p = 1.0 + y * (1.0 / 5.0) * p;
    p = 1.0 + y * (1.0 / 4.0) * p;
    p = 1.0 + y * (1.0 / 3.0) * p;
    p = 1.0 + y * (1.0 / 2.0) * p;
    p = 1.0 + y * p;
    return ldexp(tab[ki & 63] * p, ki >> 6);
}

// exp(s - M) in 2^-38 fixed point (round to nearest): each term within
// 2^-39 of exact, sums order independent.
__device__ __forceinline__ float value_of(unsigned long long packed)
{
    return key_float((uint32_t)(packed >> 32));
}

__device__ __forceinline__ unsigned long long mass_fixed(float s, double M, const double *tab)
{
    return (unsigned long long)(exp_below((double)s - M, tab) * kMassUnit + 0.5);
}

// Block-wide reductions and scans: within each wave by lane shuffles, then
// one exchange of the per-wave results through `scratch` (>= NT / 64
// entries).  Every thread gets the result; `scratch` is free again on return.
// Wave-wide sum and max: four DPP steps within each row of 16 lanes (quad
// permutations 1032 and 2301, half-row mirror, row mirror), then the four
// row results read as scalars.  Every lane of the wave must be active (all
// callers are in wave-uniform control flow); every lane gets the result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL, typename T>
__device__ __forceinline__ T dpp_t(T v)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lanes");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
    } else {
        const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
        const unsigned long long lo = dpp_u32<CTRL>((uint32_t)u);
        const unsigned long long hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
        return __builtin_bit_cast(T, (hi << 32) | lo);
    }
}

template <typename T>
__device__ __forceinline__ T readlane_t(T v, int lane)
{
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
    } else {
        const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
        const unsigned long long lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
        const unsigned long long hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
        return __builtin_bit_cast(T, (hi << 32) | lo);
    }
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce_t(T v, Op op)
{
    v = op(v, dpp_t<0xB1>(v));    // quad_perm 1,0,3,2
    v = op(v, dpp_t<0x4E>(v));    // quad_perm 2,3,0,1
    v = op(v, dpp_t<0x141>(v));   // row_half_mirror
    v = op(v, dpp_t<0x140>(v));   // row_mirror
    return op(op(readlane_t(v, 0), readlane_t(v, 16)), op(readlane_t(v, 32), readlane_t(v, 48)));
}

template <typename T>
__device__ __forceinline__ T wave_sum_t(T v)
{
    return wave_reduce_t(v, [](T x, T y) { return x + y; });
}

template <typename T>
__device__ __forceinline__ T wave_max_t(T v)
{
    return wave_reduce_t(v, [](T x, T y) { return max(x, y); });
}

template <typename T, int NT>
__device__ __forceinline__ T block_sum(T v, T *scratch)
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
__device__ __forceinline__ T block_max(T v, T *scratch)
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

// Inclusive scan over the threads in ascending order (REV: descending, i.e.
// thread t gets the sum over threads t .. NT-1).
// Two block-wide maxima of 32-bit values with one exchange.
template <int NT>
__device__ __forceinline__ void block_max2(uint32_t x, uint32_t y, unsigned long long *scratch,
                                           uint32_t &mx, uint32_t &my)
{
    x = wave_max_t(x);
    y = wave_max_t(y);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = ((unsigned long long)x << 32) | y;
    __syncthreads();
    mx = 0;
    my = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const unsigned long long s = scratch[w];
        mx = max(mx, (uint32_t)(s >> 32));
        my = max(my, (uint32_t)s);
    }
    __syncthreads();
}

template <int CTRL, typename T>
__device__ __forceinline__ T dpp_shift_t(T v)   // lanes with no source read 0
{
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
    } else {
        const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
        const unsigned long long lo =
            (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, true);
        const unsigned long long hi =
            (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
        return __builtin_bit_cast(T, (hi << 32) | lo);
    }
}

// Inclusive sum over the lanes of a wave in ascending order: row shifts by
// 1, 2, 4 and 8 within each row of 16 lanes, then the rows' totals read as
// scalars.  Every lane of the wave must be active.
template <typename T, typename Op>
__device__ __forceinline__ T wave_scan_op(T v, Op op)   // (op(x, 0) = x)
{
    v = op(v, dpp_shift_t<0x111>(v));   // row_shr:1
    v = op(v, dpp_shift_t<0x112>(v));   // row_shr:2
    v = op(v, dpp_shift_t<0x114>(v));   // row_shr:4
    v = op(v, dpp_shift_t<0x118>(v));   // row_shr:8
    const T r0 = readlane_t(v, 15), r1 = readlane_t(v, 31), r2 = readlane_t(v, 47);
    const int lane = threadIdx.x & 63;
    T add = 0;
    if (lane >= 16) add = op(add, r0);
    if (lane >= 32) add = op(add, r1);
    if (lane >= 48) add = op(add, r2);
    return op(v, add);
}

template <typename T>
__device__ __forceinline__ T wave_scan_incl(T v)
{
    return wave_scan_op(v, [](T x, T y) { return x + y; });
}

template <typename T, int NT, bool REV = false>
__device__ __forceinline__ T block_scan_inclusive(T v, T *scratch)
{
    const int tid = REV ? NT - 1 - (int)threadIdx.x : (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // lanes of a wave in scan order: REV reverses the lane order too
    if constexpr (REV) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const T u = __shfl_down(v, (unsigned)off);
            if (lane >= off) v += u;
        }
    } else {
        v = wave_scan_incl(v);
    }
    __syncthreads();
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
    T base = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {   // (all reads issued together)
        const T s = scratch[w];
        base += w < wave ? s : T(0);
    }
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

// Bit j set when element j of this thread's share lies in the chunk [i0, i1).
template <bool VEC4>
__device__ __forceinline__ uint32_t in_chunk_bits(int i0, int i1, int per)
{
    if (Tile<VEC4>::full(i0, i1, per)) return 0xffffffffu;
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
        bits |= ((j < per && Tile<VEC4>::index(i0, j) < i1) ? 1u : 0u) << j;
    return bits;
}

// What a row needs, from its own settings: 0 < k < V turns top-k on, p < 1
// the nucleus (p <= 0: the maxima only), T <= 0 (or NaN) means greedy.
struct RowSettings {
    uint32_t mode;
    int32_t k;
    float p, T;
};

__device__ __forceinline__ RowSettings row_settings(const SampArgs &a, int b)
{
    const float T = a.temperature[b];
    const int32_t k = a.top_k[b];
    const float p = a.top_p[b];
    uint32_t mode = 0;
    if (!(T > 0.f)) {
        mode = MODE_GREEDY;
    } else {
        if (k > 0 && k < a.vocab) mode |= MODE_TOPK;
        if (p < 1.f) mode |= (p > 0.f) ? MODE_TOPP : MODE_TOPP_MAX;
        if (!mode) mode = MODE_PLAIN;
    }
    return RowSettings{mode, k, p, T};
}

__device__ __forceinline__ uint32_t row_mode(const SampArgs &a, int b)
{
    return row_settings(a, b).mode;
}

// ---- scan ------------------------------------------------------------------

// Element j of this thread's share of a chunk starting at i0 (PER per
// thread; VEC4: float4 groups).
template <bool VEC4>
__device__ __forceinline__ int elem_index(int i0, int j)
{
    return Tile<VEC4>::index(i0, j);
}

// One scan workgroup's work on its chunk, PER logits per thread.  FULL: the
// chunk lies inside the row (no per-element range checks).
template <bool VEC4, bool MASK, int PER, bool FULL>
__device__ __forceinline__ void scan_chunk(const SampArgs &a, Tile<VEC4> &t, int b, int c, int i0,
                                           int i1, const RowSettings &rs)
{
    const uint32_t mode = rs.mode;
    __shared__ unsigned long long s_red[kThreads / 64];
    __shared__ uint32_t s_cnt[kBins];
    __shared__ uint32_t s_wkey[kThreads / 64];
    __shared__ float s_wzx[kThreads / 64];
    __shared__ uint32_t s_nlist;
    __shared__ uint32_t s_wtot[kThreads / 64];
    __shared__ int s_wfit[kThreads / 64], s_wneed[kThreads / 64];
    ChunkRec *rec = a.rec + (int64_t)b * a.nchunks + c;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    auto in = [&](int j) { return FULL || elem_index<VEC4>(i0, j) < i1; };

    if (mode & (MODE_GREEDY | MODE_PLAIN)) {
        unsigned long long best = 0;
        if (mode & MODE_GREEDY) {
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (in(j)) best = max(best, pack_key_index(float_key(t.raw(j)), (uint32_t)elem_index<VEC4>(i0, j)));
        } else {
            // every token is eligible: stream the noise too
            const Scaler sc(rs.T);
            Tile<VEC4> gt;
            gt.template load_range<0, PER>(a.gumbel + (int64_t)b * a.gstride, i0, i1, PER);
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (in(j))
                    best = max(best, pack_key_index(float_key(t.scaled(j, sc) + gt.v[j]),
                                                    (uint32_t)elem_index<VEC4>(i0, j)));
        }
        best = block_max<unsigned long long, kThreads>(best, s_red);
        if (threadIdx.x == 0) {
            ChunkRec r = {};
            r.best = best;
            *rec = r;
        }
        return;
    }

    // ---- filtered rows: s, the chunk max and the value histogram ----
    // Reductions run inside each wave and meet through small LDS arrays,
    // and list slots are claimed per wave (the list's order carries no
    // meaning).
    for (int d = threadIdx.x; d < kBins; d += kThreads) s_cnt[d] = 0;
    if (threadIdx.x == 0) s_nlist = 0;
    const Scaler sc(rs.T);
    // s = z / T by the double product for every element; a wave that holds
    // a logit small enough for a subnormal tie redoes those by division
    unsigned long long tiny = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) tiny |= __ballot(fabsf(t.v[j]) < sc.tiny);
    if (__builtin_expect(tiny != 0, 0)) {
#pragma unroll
        for (int j = 0; j < PER; ++j) t.v[j] = sc(t.v[j]);
    } else {
#pragma unroll
        for (int j = 0; j < PER; ++j) t.v[j] = (float)((double)t.v[j] * sc.inv);
    }
    float smax = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (MASK && !((t.ok >> j) & 1u)) t.v[j] = kMasked;
        // (fmaxf: NaN never wins)
        if (in(j)) smax = fmaxf(smax, t.v[j]);
    }
    {
        const uint32_t wk = wave_max_t(float_key(smax));
        if (lane == 0) s_wkey[wave] = wk;
    }
    __syncthreads();                                       // (1) also orders the clearing
    uint32_t kmax = s_wkey[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) kmax = max(kmax, s_wkey[w]);
    const float Mc = key_float(kmax);
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (in(j)) atomicAdd(&s_cnt[bin_of(t.v[j], Mc)], 1u);
    __syncthreads();                                       // (2)

    // Cut bin jc: the list holds the tokens of bins [0, jc).  cum(j) =
    // tokens in bins below j (non-decreasing, cum(kBins) = all).  j_fit: the
    // most bins whose tokens fit in the list; j_need: the fewest holding
    // `need` (top-k: k; p <= 0: the maxima, i.e. bin 0).  Thread t owns bins
    // [8t, 8t + 8); one exchange of wave totals, then each thread tests its
    // own bins and the results meet in LDS.
    int jc;
    {
        constexpr int BPT = kBins / kThreads;
        const int d0 = (int)threadIdx.x * BPT;
        uint32_t cnt[BPT];
        uint32_t own = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            cnt[j] = s_cnt[d0 + j];
            own += cnt[j];
        }
        uint32_t incl = own;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t u = __shfl_up(incl, (unsigned)off);
            if (lane >= off) incl += u;
        }
        if (lane == 63) s_wtot[wave] = incl;
        __syncthreads();                                   // (3a)
        uint32_t cum = incl - own;
        for (int w = 0; w < wave; ++w) cum += s_wtot[w];
        const uint32_t cap = (uint32_t)a.cap;
        uint32_t need = cap;                               // nucleus: as many as fit
        if (mode & MODE_TOPK) need = min((uint32_t)rs.k, cap);
        else if (mode & MODE_TOPP_MAX) need = 1;
        int fit = 0, nd = kBins;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            if (cum <= cap) fit = d0 + j;
            if (cum >= need) nd = min(nd, d0 + j);
            cum += cnt[j];
        }
        if (threadIdx.x == kThreads - 1) {                 // j = kBins: every token
            if (cum <= cap) fit = kBins;
            if (cum >= need) nd = min(nd, kBins);
        }
        const int wfit = wave_max_t(fit), wneed = -wave_max_t(-nd);
        if (lane == 0) {
            s_wfit[wave] = wfit;
            s_wneed[wave] = wneed;
        }
        __syncthreads();                                   // (3b)
        int j_fit = s_wfit[0], j_need = s_wneed[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) {
            j_fit = max(j_fit, s_wfit[w]);
            j_need = min(j_need, s_wneed[w]);
        }
        jc = (mode & (MODE_TOPK | MODE_TOPP_MAX)) ? min(j_fit, j_need) : j_fit;
    }

    // ---- classify: listed tokens, the largest left out, the left-out mass ----
    // Branch-free per element: a listed token enters the max and the mass
    // as -inf (mass exactly 0); the mass is computed only for nucleus rows
    // (a wave-uniform choice made once).
    uint32_t listed = 0;
    float omax = -__builtin_huge_valf();
    float zx = 0.f;
    bool any_nan_out = false;
    // bin_of(s, Mc) < jc reads (Mc - s) * kBinsPerUnit < jc for jc < kBins
    // (the truncated bin index of a non-negative d is below an integer jc
    // exactly when d is; NaN lands in the last bin either way)
    const bool all_listed = jc >= kBins;
    const float jcf = (float)jc;
    auto classify = [&](auto with_mass) {
        const double Md = (double)Mc;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const float s = t.v[j];
            const bool lj = in(j) && (all_listed || (Mc - s) * kBinsPerUnit < jcf);
            const bool oj = in(j) && !lj;
            listed |= (lj ? 1u : 0u) << j;
            const float so = oj ? s : -__builtin_huge_valf();
            omax = fmaxf(omax, so);
            any_nan_out |= oj && !(s == s);
            if (decltype(with_mass)::value) zx += mass_approx(so, Md);
        }
    };
    if ((mode & MODE_TOPP) && !(mode & MODE_TOPK))
        classify(std::true_type{});
    else
        classify(std::false_type{});
    {
        const uint32_t nl = __popc(listed);
        uint32_t incl = nl;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t u = __shfl_up(incl, (unsigned)off);
            if (lane >= off) incl += u;
        }
        uint32_t base = 0;
        if (lane == 63 && incl) base = atomicAdd(&s_nlist, incl);
        base = __shfl(base, 63);
        unsigned long long *lst = a.list + ((int64_t)b * a.nchunks + c) * a.cap;
        uint32_t pos = base + incl - nl;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if ((listed >> j) & 1u)
                lst[pos++] = pack_key_index(float_key(t.v[j]), (uint32_t)elem_index<VEC4>(i0, j));
        // a left-out NaN counts as the largest key (nothing is known above it)
        uint32_t ok_key = (omax == -__builtin_huge_valf()) ? 0u : float_key(omax);
        if (any_nan_out) ok_key = 0xffffffffu;
        const uint32_t wo = wave_max_t(ok_key);
        const float wz = wave_sum_t(zx);
        if (lane == 0) {
            s_wkey[wave] = wo;
            s_wzx[wave] = wz;
        }
    }
    __syncthreads();                                       // (4)
    if (threadIdx.x == 0) {
        ChunkRec r;
        r.mkey = kmax;
        r.outkey = s_wkey[0];
        double z = 0.0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            r.outkey = max(r.outkey, s_wkey[w]);
            z += (double)s_wzx[w];
        }
        r.n = s_nlist;
        r.pad = 0;
        r.zx = z;
        r.best = 0;
        *rec = r;
    }
}

template <bool VEC4, bool MASK, int PER>
__global__ __launch_bounds__(kThreads) void samp_scan_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    const int c = blockIdx.x;
    const int i0 = c * PER * kThreads;
    const int i1 = min(a.vocab, i0 + PER * kThreads);
    // the tile is requested before the row's settings are read, so that
    // the two overlap
    Tile<VEC4> t;
    t.template load_range<0, PER, true>(a.logits + (int64_t)b * a.lstride, i0, i1, PER);
    t.load_mask(MASK ? a.mask + (int64_t)b * a.mstride : nullptr, i0, i1, PER);
    const RowSettings rs = row_settings(a, b);
    if (i1 - i0 == PER * kThreads)
        scan_chunk<VEC4, MASK, PER, true>(a, t, b, c, i0, i1, rs);
    else
        scan_chunk<VEC4, MASK, PER, false>(a, t, b, c, i0, i1, rs);
}

// ---- histogram -------------------------------------------------------------

// Finish-side bins that can hold a token above T*: [0, nb).
__device__ __forceinline__ int bins_above(uint32_t tout, float M)
{
    return tout == 0u ? kHBins : hbin_of(key_float(tout), M) + 1;
}

// One workgroup per (group of chunks, row) of the filtered rows.  The
// group's listed tokens above T* get their noise and go into value bins
// below the row max M: counts, masses (nucleus rows) and the best Gumbel
// key per bin, from which each bin's count and best over the bins before it
// follow by prefix scans; the tokens are then written in bin order with
// their noise.  Every listed token's mass plus the chunks' left-out masses
// brought to M make the group's share of Z.  Everything is written for the
// group (no atomics across workgroups); the finish combines the groups.
// The first kHBatch list slots of each thread are requested together with
// the row's records, before anything is known of them (slots past a
// chunk's count hold stale data and are dropped once the counts arrive).
__global__ __launch_bounds__(kHThreads) void samp_hist_kernel(const SampArgs a)
{
    const int b = blockIdx.y;
    const int g = blockIdx.x;
    const uint32_t mode = row_mode(a, b);
    if (!(mode & (MODE_TOPK | MODE_TOPP))) return;   // greedy, plain, maxima: not needed
    __shared__ unsigned long long s_red[kHThreads / 64];
    __shared__ double s_tab[64];
    __shared__ uint32_t s_cnt[kHBins];
    __shared__ unsigned long long s_mass[kHBins];
    __shared__ unsigned long long s_best[kHBins];
    __shared__ unsigned long long s_sum[3][kHThreads / 64];
    __shared__ uint32_t s_n[kGroupChunks], s_mk[kGroupChunks];
    __shared__ double s_zx[kGroupChunks];
    const int c0 = (int)((int64_t)g * a.nchunks / a.groups);
    const int c1 = (int)((int64_t)(g + 1) * a.nchunks / a.groups);
    const unsigned long long *lgrp = a.list + ((int64_t)b * a.nchunks + c0) * a.cap;
    const int nslots = (c1 - c0) * a.cap;
    const int lc = __ffs(a.cap) - 1;   // cap is a power of two
    // ---- one round of loads: the first batch of slots and the records ----
    unsigned long long v[kHBatch];
#pragma unroll
    for (int j = 0; j < kHBatch; ++j) {
        const int f = (int)threadIdx.x + j * kHThreads;
        v[j] = lgrp[f < nslots ? f : 0];
    }
    const ChunkRec *rec = a.rec + (int64_t)b * a.nchunks;
    uint32_t km = 0, to = 0;
    for (int c = threadIdx.x; c < a.nchunks; c += kHThreads) {
        const ChunkRec r = rec[c];
        km = max(km, r.mkey);
        to = max(to, r.outkey);
        if (c >= c0 && c < c1) {
            s_n[c - c0] = r.n;
            s_mk[c - c0] = r.mkey;
            s_zx[c - c0] = r.zx;
        }
    }
    if (threadIdx.x < 64) s_tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
    for (int d = threadIdx.x; d < kHBins; d += kHThreads) {
        s_cnt[d] = 0;
        s_mass[d] = 0;
        s_best[d] = 0;
    }
    uint32_t kmax, tout;
    block_max2<kHThreads>(km, to, s_red, kmax, tout);   // (its barrier orders the fills)
    const float Mf = key_float(kmax);
    const double M = (double)Mf;
    const bool nucleus = (mode & MODE_TOPP) && !(mode & MODE_TOPK);
    const float *gn = a.gumbel + (int64_t)b * a.gstride;
    // slot f of the batch at f0, slot j: listed (live: and above T*)
    auto listed = [&](int f) {
        return f < nslots && (uint32_t)(f & (a.cap - 1)) < s_n[f < nslots ? f >> lc : 0];
    };
    auto live = [&](int f, unsigned long long p) { return listed(f) && (uint32_t)(p >> 32) > tout; };
    unsigned long long zl = 0, mu = 0, nu = 0;
    float gv[kHBatch];
    for (int f0 = threadIdx.x; f0 < nslots; f0 += kHBatch * kHThreads) {
        if (f0 != (int)threadIdx.x) {   // later batches
#pragma unroll
            for (int j = 0; j < kHBatch; ++j) {
                const int f = f0 + j * kHThreads;
                v[j] = lgrp[f < nslots ? f : 0];
            }
        }
#pragma unroll
        for (int j = 0; j < kHBatch; ++j) {   // (lanes with nothing to read issue no load)
            float gj = 0.f;
            if (live(f0 + j * kHThreads, v[j])) gj = gn[unpack_index(v[j])];
            gv[j] = gj;
        }
#pragma unroll
        for (int j = 0; j < kHBatch; ++j) {
            const int f = f0 + j * kHThreads;
            if (!listed(f)) continue;
            const float s = value_of(v[j]);
            const unsigned long long m = nucleus ? mass_fixed(s, M, s_tab) : 0ull;
            zl += m;
            if ((uint32_t)(v[j] >> 32) > tout) {
                const int d = hbin_of(s, Mf);
                const uint32_t i = unpack_index(v[j]);
                atomicAdd(&s_cnt[d], 1u);
                if (nucleus) atomicAdd(&s_mass[d], m);
                atomicMax(&s_best[d], pack_key_index(float_key(s + gv[j]), i));
                mu += m;
                ++nu;
            }
        }
    }
    if (nucleus)   // the chunks' left-out masses, brought from M_c to M
        for (int c = threadIdx.x; c < c1 - c0; c += kHThreads)
            if (s_zx[c] > 0.0)
                zl += (unsigned long long)(s_zx[c] * exp_below((double)key_float(s_mk[c]) - M, s_tab) *
                                           kMassUnit + 0.5);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    zl = wave_sum_t(zl);
    mu = wave_sum_t(mu);
    nu = wave_sum_t(nu);
    if (lane == 0) {
        s_sum[0][wave] = zl;
        s_sum[1][wave] = mu;
        s_sum[2][wave] = nu;
    }
    __syncthreads();   // the bins are complete

    // Exclusive prefix count and prefix max over the bins: thread t owns
    // bins [kPB t, kPB t + kPB).
    constexpr int kPB = kHBins / kHThreads;
    const int d0 = kPB * (int)threadIdx.x;
    uint32_t cnt[kPB];
    unsigned long long bst[kPB];
    uint32_t csum = 0;
    unsigned long long cmax = 0;
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
        cnt[j] = s_cnt[d0 + j];
        bst[j] = s_best[d0 + j];
        csum += cnt[j];
        cmax = max(cmax, bst[j]);
    }
    const uint32_t isum = wave_scan_incl(csum);
    const unsigned long long imax =
        wave_scan_op(cmax, [](unsigned long long x, unsigned long long y) { return max(x, y); });
    __shared__ unsigned long long s_wmax[kHThreads / 64];
    if (lane == 63) {   // (s_red is free: its last use was behind a barrier)
        s_red[wave] = isum;
        s_wmax[wave] = imax;
    }
    __syncthreads();
    uint32_t run = isum - csum;
    unsigned long long rmax = 0;
    {   // this thread's inclusive-exclusive conversion, plus the waves before
        const unsigned long long prev = __shfl_up(imax, 1u);
        rmax = lane > 0 ? prev : 0ull;
    }
#pragma unroll
    for (int w = 0; w < kHThreads / 64; ++w) {   // (all reads issued together)
        const uint32_t ws = (uint32_t)s_red[w];
        const unsigned long long wm = s_wmax[w];
        if (w < wave) {
            run += ws;
            rmax = max(rmax, wm);
        }
    }
    const int nb = bins_above(tout, Mf);
    const int64_t part = (int64_t)b * a.groups + g;
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
        const int d = d0 + j;
        if (d < nb) {
            BinRec r;
            r.cnt = cnt[j];
            r.off = run;
            r.mass = nucleus ? s_mass[d] : 0ull;
            r.above = rmax;
            a.bins[part * kHBins + d] = r;
        }
        s_cnt[d] = run;   // the bin's write cursor
        run += cnt[j];
        rmax = max(rmax, bst[j]);
    }
    __syncthreads();
    // the tokens in bin order, with their noise
    SortedTok *out = a.sorted + part * a.gslots;
    for (int f0 = threadIdx.x; f0 < nslots; f0 += kHBatch * kHThreads) {
        if (nslots > kHBatch * kHThreads) {   // several batches: read again
#pragma unroll
            for (int j = 0; j < kHBatch; ++j) {
                const int f = f0 + j * kHThreads;
                v[j] = lgrp[f < nslots ? f : 0];
            }
#pragma unroll
            for (int j = 0; j < kHBatch; ++j) {
                float gj = 0.f;
                if (live(f0 + j * kHThreads, v[j])) gj = gn[unpack_index(v[j])];
                gv[j] = gj;
            }
        }
#pragma unroll
        for (int j = 0; j < kHBatch; ++j) {
            if (!live(f0 + j * kHThreads, v[j])) continue;
            const uint32_t pos = atomicAdd(&s_cnt[hbin_of(value_of(v[j]), Mf)], 1u);
            SortedTok st;
            st.packed = v[j];
            st.g = gv[j];
            st.pad = 0;
            out[pos] = st;
        }
    }
    if (threadIdx.x == 0) {
        RowTot r = {};
#pragma unroll
        for (int w = 0; w < kHThreads / 64; ++w) {
            r.Z += s_sum[0][w];
            r.mu += s_sum[1][w];
            r.nu += (uint32_t)s_sum[2][w];
        }
        r.kmax = kmax;
        r.tout = tout;
        a.tot[part] = r;
    }
}

// ---- finish ----------------------------------------------------------------

constexpr int kCand = 1024;   // tokens of a threshold bin resolved in LDS
constexpr int kSmallCand = 128;   // up to this many, compared one by one directly
constexpr int kSubBins = 256;     // above: sub-ranges of their values ...
constexpr int kSubCand = 256;     // ... and candidates of one sub-range compared directly
// the counting cut gives each candidate q >= 1 lanes: at most one per thread
static_assert(kCand <= kFThreads, "cand_rank / cand_cut need a lane per candidate");
constexpr int kBatch = 8;     // list entries per thread whose loads are issued together

constexpr int kWaveCand = 256;     // cut-bin tokens one wave resolves (four per lane)
constexpr int kCutBins = 2048;   // the radix cut's widest level: 11 bits

// A token of a cut bin resolved by one wave (top-k: a = packed key;
// nucleus: a = value key, b = mass).
struct alignas(16) CandRec {
    unsigned long long a, b;
};
static_assert(kHBins <= kCutBins, "finish bins fit the radix arrays");

struct FinishShared {
    double tab[64];                       // 2^(j/64)
    uint32_t nlist[kMaxChunks];           // list sizes of the chunks
    uint32_t bcnt[kCutBins];              // value bins below the row max (kHBins) or
    unsigned long long bmass[kCutBins];   // one radix level: counts, masses (2^-38 units)
    unsigned long long ckey[kCand];       // one bin's tokens: packed keys ...
    unsigned long long cmass[kCand];      // ... masses
    float cgum[kCand];                    // ... and noise (one-pass draw)
    CandRec crec[kWaveCand];              // a cut bin resolved by one wave: its
    uint32_t wcnt[64];                    // sub-ranges' counts and masses, and the
    unsigned long long wmass[64];         // chosen sub-range's tokens (crec)
    RowTot gtot[kGroups];                 // the histogram groups' totals
    uint32_t goff[kGroups], gstart[kGroups + 1];   // the cut bin, per group
    uint32_t scnt[kSubBins];              // candidate sub-ranges: counts, masses,
    unsigned long long smass[kSubBins];
    unsigned long long skey[kSubCand], smas[kSubCand];   // ... the chosen one's tokens
    uint32_t hcnt[kDigits];               // radix digits (slow path)
    unsigned long long red[kFThreads / 64];
    uint32_t nc, sel, ssel, snc;
    unsigned long long up, pick;
    unsigned long long sup;               // sub-range search: what lies above it
};

// The row's listed tokens above T*, streamed from memory.  Thread t takes
// slot t % cap of chunks t / cap, t / cap + per, ... (per = kFThreads / cap;
// cap divides kFThreads), kBatch chunks' loads issued together.
struct ListSource {
    const unsigned long long *lrow;
    const uint32_t *nlist;   // LDS
    int cap, per, nch, slot, csub;
    uint32_t tout;
    double M;
    const double *tab;

    template <typename F>
    __device__ __forceinline__ void each(F f) const
    {
        for (int c0 = csub; c0 < nch; c0 += kBatch * per) {
            unsigned long long v[kBatch];
            bool ok[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int c = c0 + j * per;
                ok[j] = c < nch && slot < (int)nlist[c < nch ? c : 0];
                v[j] = lrow[(int64_t)(ok[j] ? c : 0) * cap + (ok[j] ? slot : 0)];
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (ok[j] && (uint32_t)(v[j] >> 32) > tout) f(v[j]);
        }
    }
    __device__ __forceinline__ unsigned long long mass(unsigned long long packed) const
    {
        return mass_fixed(value_of(packed), M, tab);
    }
};

// The whole row, read again from memory (s recomputed).
struct RowSource {
    const float *z;
    const uint8_t *m;
    Scaler sc;
    double M;
    int V;
    const double *tab;
    template <typename F>
    __device__ __forceinline__ void each(F f) const
    {
        for (int i = threadIdx.x; i < V; i += kFThreads) {
            const float s = (m && !m[i]) ? kMasked : sc(z[i]);
            f(pack_key_index(float_key(s), (uint32_t)i));
        }
    }
    __device__ __forceinline__ unsigned long long mass(unsigned long long packed) const
    {
        return mass_fixed(value_of(packed), M, tab);
    }
};

// The 56 significant bits of a packed key: the value key and the low 24 bits
// of ~index (vocab <= 2^24, so the top 8 bits of ~index are all ones).
__device__ __forceinline__ unsigned long long v56(unsigned long long packed)
{
    return ((packed >> 32) << 24) | (packed & 0xffffffull);
}

__device__ __forceinline__ unsigned long long packed_of_v56(unsigned long long v)
{
    return ((v >> 24) << 32) | 0xff000000ull | (v & 0xffffffull);
}

// Value-bin histogram (counts, and masses if MASS; bins below the row max
// M) of the tokens for which keep(packed) holds; returns their total mass.
template <bool MASS, typename Src, typename Keep>
__device__ __forceinline__ unsigned long long bin_hist(const Src &src, FinishShared &sh, float M, Keep keep)
{
    for (int d = threadIdx.x; d < kHBins; d += kFThreads) {
        sh.bcnt[d] = 0;
        sh.bmass[d] = 0;
    }
    __syncthreads();
    unsigned long long tot = 0;
    src.each([&](unsigned long long packed) {
        if (!keep(packed)) return;
        const int d = hbin_of(value_of(packed), M);
        atomicAdd(&sh.bcnt[d], 1u);
        if (MASS) {
            const unsigned long long m = src.mass(packed);
            atomicAdd(&sh.bmass[d], m);
            tot += m;
        }
    });
    return block_sum<unsigned long long, kFThreads>(tot, sh.red);
}

// Thread t owns bins [kFBins t, kFBins t + kFBins) (bin 0: largest values).
constexpr int kFBins = kHBins / kFThreads;
static_assert(kFBins >= 1 && kHBins % kFThreads == 0, "finish bins per thread");

// The bin holding the rank-th largest token, and the rank inside it.
__device__ __forceinline__ void bin_by_count(FinishShared &sh, uint32_t rank, int &bin, uint32_t &rank_in)
{
    const int d0 = kFBins * (int)threadIdx.x;
    uint32_t own = 0;
#pragma unroll
    for (int j = 0; j < kFBins; ++j) own += sh.bcnt[d0 + j];
    uint32_t above = (uint32_t)block_scan_inclusive<unsigned long long, kFThreads>(own, sh.red) - own;
#pragma unroll
    for (int j = 0; j < kFBins; ++j) {
        const uint32_t c = sh.bcnt[d0 + j];
        if (above < rank && rank <= above + c) {
            sh.sel = (uint32_t)(d0 + j);
            sh.up = above;
        }
        above += c;
    }
    __syncthreads();
    bin = (int)sh.sel;
    rank_in = rank - (uint32_t)sh.up;
    __syncthreads();
}

// The deepest non-empty bin whose strictly-greater mass is <= limit (the
// bin of the nucleus cut), and that mass.
__device__ __forceinline__ void bin_by_mass(FinishShared &sh, double limit, int &bin, unsigned long long &A)
{
    const int d0 = kFBins * (int)threadIdx.x;
    unsigned long long own = 0;
#pragma unroll
    for (int j = 0; j < kFBins; ++j) own += sh.bmass[d0 + j];
    unsigned long long above = block_scan_inclusive<unsigned long long, kFThreads>(own, sh.red) - own;
    int cand = -1;
    unsigned long long cand_a = 0;
#pragma unroll
    for (int j = 0; j < kFBins; ++j) {
        if (sh.bcnt[d0 + j] && (double)above <= limit) {
            cand = d0 + j;
            cand_a = above;
        }
        above += sh.bmass[d0 + j];
    }
    const int best =
        (int)block_max<unsigned long long, kFThreads>((unsigned long long)(cand + 1), sh.red) - 1;
    if (cand >= 0 && cand == best) sh.up = cand_a;
    __syncthreads();
    bin = best;
    A = sh.up;
    __syncthreads();
}

// Copies the tokens of bin `bin` passing keep, with their masses, into
// sh.ckey / sh.cmass; returns their number (only the first kCand stored).
template <typename Src, typename Keep>
__device__ __forceinline__ uint32_t compact_bin(const Src &src, FinishShared &sh, float M, int bin, Keep keep)
{
    if (threadIdx.x == 0) sh.nc = 0;
    __syncthreads();
    src.each([&](unsigned long long packed) {
        if (!keep(packed) || hbin_of(value_of(packed), M) != bin) return;
        const uint32_t slot = atomicAdd(&sh.nc, 1u);
        if (slot < (uint32_t)kCand) {
            sh.ckey[slot] = packed;
            sh.cmass[slot] = src.mass(packed);
        }
    });
    __syncthreads();
    const uint32_t n = sh.nc;
    __syncthreads();
    return n;
}

// Exact cut among n <= kCand candidates (keys, masses in LDS) by counting:
// q consecutive lanes (q a power of two) share one candidate and split the
// comparisons.  Top-k: the packed key of rank `rank` (1 = largest, by value
// then index).
__device__ __forceinline__ unsigned long long count_rank(FinishShared &sh, const unsigned long long *keys,
                                                         uint32_t n, uint32_t rank)
{
    uint32_t np = 1;
    while (np < n) np <<= 1;
    const uint32_t q = min(64u, (uint32_t)kFThreads / np);
    const uint32_t e = threadIdx.x / q, part = threadIdx.x % q;
    const bool real = e < n;
    const unsigned long long ke = real ? keys[e] : 0ull;
    uint32_t larger = 0;
    uint32_t j = part;
    for (; j + 7 * q < n; j += 8 * q) {   // eight LDS reads in flight
#pragma unroll
        for (int u = 0; u < 8; ++u) larger += keys[j + u * q] > ke ? 1u : 0u;
    }
    for (; j < n; j += q) larger += keys[j] > ke ? 1u : 0u;
    for (uint32_t m = 1; m < q; m <<= 1) larger += __shfl_xor(larger, (int)m);
    if (real && part == 0 && larger + 1 == rank) sh.pick = ke;
    __syncthreads();
    const unsigned long long r = sh.pick;
    __syncthreads();
    return r;
}

// Nucleus: the smallest candidate value whose strictly-greater mass (A from
// what lies above plus the candidates above) is <= limit.
__device__ __forceinline__ uint32_t count_cut(FinishShared &sh, const unsigned long long *keys,
                                              const unsigned long long *mass, uint32_t n,
                                              unsigned long long A, double limit)
{
    uint32_t np = 1;
    while (np < n) np <<= 1;
    const uint32_t q = min(64u, (uint32_t)kFThreads / np);
    const uint32_t e = threadIdx.x / q, part = threadIdx.x % q;
    const bool real = e < n;
    const uint32_t ke = real ? (uint32_t)(keys[e] >> 32) : 0u;
    unsigned long long above = 0;
    uint32_t j = part;
    for (; j + 7 * q < n; j += 8 * q) {   // eight LDS reads in flight
#pragma unroll
        for (int u = 0; u < 8; ++u)
            above += (uint32_t)(keys[j + u * q] >> 32) > ke ? mass[j + u * q] : 0ull;
    }
    for (; j < n; j += q) above += (uint32_t)(keys[j] >> 32) > ke ? mass[j] : 0ull;
    for (uint32_t m = 1; m < q; m <<= 1) above += __shfl_xor(above, (int)m);
    const bool fits = real && (double)(A + above) <= limit;
    // the smallest qualifying key: a max over complemented keys
    const uint32_t t =
        (uint32_t)block_max<unsigned long long, kFThreads>(fits ? (unsigned long long)(~ke) : 0ull, sh.red);
    return ~t;
}

// More than kSmallCand candidates: their value keys' range is cut into
// kSubBins sub-ranges; counts (and masses) per sub-range locate the one
// holding the cut, and only its candidates are compared one by one (all of
// them again if it holds more than kSubCand, e.g. many ties).  Sub-range of
// a value key: monotone in the key, so tied values share one.
__device__ __forceinline__ int sub_of(uint32_t k, uint32_t kmin, unsigned long long span)
{
    return (int)(((unsigned long long)(k - kmin) * kSubBins) / span);
}

// Fills sh.scnt (and sh.smass) over the candidates' sub-ranges; returns the
// key range through kmin / span.
__device__ __forceinline__ void sub_hist(FinishShared &sh, uint32_t n, bool with_mass, uint32_t &kmin,
                                         unsigned long long &span)
{
    if (threadIdx.x < kSubBins) {
        sh.scnt[threadIdx.x] = 0;
        sh.smass[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) sh.snc = 0;
    const bool real = threadIdx.x < n;
    const uint32_t k = real ? (uint32_t)(sh.ckey[threadIdx.x] >> 32) : 0u;
    uint32_t hi, nlo;
    block_max2<kFThreads>(real ? k : 0u, real ? ~k : 0u, sh.red, hi, nlo);   // (orders the clears)
    kmin = ~nlo;
    span = (unsigned long long)(hi - kmin) + 1;
    if (real) {
        const int s = sub_of(k, kmin, span);
        atomicAdd(&sh.scnt[s], 1u);
        if (with_mass) atomicAdd(&sh.smass[s], sh.cmass[threadIdx.x]);
    }
    __syncthreads();
}

// Copies the candidates of sub-range ssel (at most kSubCand) into sh.skey /
// sh.smas; returns their number.
__device__ __forceinline__ uint32_t sub_compact(FinishShared &sh, uint32_t n, uint32_t kmin,
                                                unsigned long long span)
{
    if (threadIdx.x < n) {
        const uint32_t k = (uint32_t)(sh.ckey[threadIdx.x] >> 32);
        if (sub_of(k, kmin, span) == (int)sh.ssel) {
            const uint32_t slot = atomicAdd(&sh.snc, 1u);
            if (slot < (uint32_t)kSubCand) {
                sh.skey[slot] = sh.ckey[threadIdx.x];
                sh.smas[slot] = sh.cmass[threadIdx.x];
            }
        }
    }
    __syncthreads();
    const uint32_t m = sh.snc;
    __syncthreads();
    return m;
}

// Top-k: the packed key of rank `rank` among the n candidates in LDS.
__device__ __forceinline__ unsigned long long cand_rank(FinishShared &sh, uint32_t n, uint32_t rank)
{
    if (n <= (uint32_t)kSmallCand) return count_rank(sh, sh.ckey, n, rank);
    uint32_t kmin;
    unsigned long long span;
    sub_hist(sh, n, false, kmin, span);
    if (threadIdx.x < 64) {   // wave 0: sub-ranges from the top, lane l owning 4
        const int lane = threadIdx.x;
        uint32_t c4[4], own = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c4[u] = sh.scnt[kSubBins - 1 - 4 * lane - u];
            own += c4[u];
        }
        uint32_t incl = own;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t v = (uint32_t)__shfl_up((int)incl, (unsigned)o);
            if (lane >= o) incl += v;
        }
        uint32_t before = incl - own;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (before < rank && rank <= before + c4[u]) {
                sh.ssel = (uint32_t)(kSubBins - 1 - 4 * lane - u);
                sh.sup = before;   // candidates in the sub-ranges above
            }
            before += c4[u];
        }
    }
    __syncthreads();
    const uint32_t r2 = rank - (uint32_t)sh.sup;
    const uint32_t m = sub_compact(sh, n, kmin, span);
    if (m > (uint32_t)kSubCand) return count_rank(sh, sh.ckey, n, rank);
    return count_rank(sh, sh.skey, m, r2);
}

// Nucleus: the smallest candidate value whose strictly-greater mass (A from
// the bins above plus the candidates above) is <= limit.
__device__ __forceinline__ uint32_t cand_cut(FinishShared &sh, uint32_t n, unsigned long long A, double limit)
{
    if (n <= (uint32_t)kSmallCand) return count_cut(sh, sh.ckey, sh.cmass, n, A, limit);
    uint32_t kmin;
    unsigned long long span;
    sub_hist(sh, n, true, kmin, span);
    if (threadIdx.x < 64) {   // wave 0: sub-ranges from the top, lane l owning 4
        const int lane = threadIdx.x;
        uint32_t c4[4];
        unsigned long long m4[4], own = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c4[u] = sh.scnt[kSubBins - 1 - 4 * lane - u];
            m4[u] = sh.smass[kSubBins - 1 - 4 * lane - u];
            own += m4[u];
        }
        unsigned long long incl = own;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long v = __shfl_up(incl, (unsigned)o);
            if (lane >= o) incl += v;
        }
        unsigned long long above = A + incl - own;
        // the deepest non-empty sub-range whose strictly-greater mass fits
        int deep = kSubBins;
        unsigned long long deep_a = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (c4[u] && (double)above <= limit) {
                deep = kSubBins - 1 - 4 * lane - u;
                deep_a = above;
            }
            above += m4[u];
        }
        const int best = -wave_max_t(-deep);
        if (deep == best && best < kSubBins) {
            sh.ssel = (uint32_t)best;
            sh.sup = deep_a;
        }
        if (lane == 0 && best == kSubBins) sh.ssel = 0xffffffffu;   // (none: cannot happen)
    }
    __syncthreads();
    if (sh.ssel == 0xffffffffu) return count_cut(sh, sh.ckey, sh.cmass, n, A, limit);
    const unsigned long long A2 = sh.sup;
    const uint32_t m = sub_compact(sh, n, kmin, span);
    if (m > (uint32_t)kSubCand) return count_cut(sh, sh.ckey, sh.cmass, n, A, limit);
    return count_cut(sh, sh.skey, sh.smas, m, A2, limit);
}

// Slow path of a bin with more than kCand tokens: radix select over the
// source restricted to that bin.  By count: the rank-th largest 56-bit value
// (11/11/10/12/12-bit levels).
template <typename Src, typename Keep>
__device__ __forceinline__ unsigned long long radix_rank(const Src &src, FinishShared &sh, uint32_t rank, Keep keep)
{
    constexpr int kShift[5] = {45, 34, 24, 12, 0};
    constexpr int kWidth[5] = {11, 11, 10, 12, 12};
    unsigned long long prefix = 0;
    for (int level = 0; level < 5; ++level) {
        const int shift = kShift[level], width = kWidth[level];
        const int hi = shift + width;
        const int nd = 1 << width;
        for (int d = threadIdx.x; d < nd; d += kFThreads) sh.hcnt[d] = 0;
        __syncthreads();
        src.each([&](unsigned long long packed) {
            if (!keep(packed)) return;
            const unsigned long long v = v56(packed);
            if (hi < 56 && (v >> hi) != (prefix >> hi)) return;
            atomicAdd(&sh.hcnt[(uint32_t)(v >> shift) & (uint32_t)(nd - 1)], 1u);
        });
        __syncthreads();
        const int dpt = nd / kFThreads;
        const int dlo = (int)threadIdx.x * dpt;
        unsigned long long own = 0;
        for (int j = 0; j < dpt; ++j) own += sh.hcnt[dlo + j];
        unsigned long long up =
            block_scan_inclusive<unsigned long long, kFThreads, true>(own, sh.red) - own;
        for (int j = dpt - 1; j >= 0; --j) {
            const unsigned long long cnt = sh.hcnt[dlo + j];
            if (up < rank && rank <= up + cnt) {
                sh.sel = (uint32_t)(dlo + j);
                sh.up = up;
            }
            up += cnt;
        }
        __syncthreads();
        prefix |= (unsigned long long)sh.sel << shift;
        rank -= (uint32_t)sh.up;
        __syncthreads();
    }
    return packed_of_v56(prefix);
}

// By mass on the value key (11/11/10-bit levels), above-mass starting at A:
// the smallest key whose strictly-greater mass is <= limit.
template <typename Src, typename Keep>
__device__ __forceinline__ uint32_t radix_cut(const Src &src, FinishShared &sh, unsigned long long A, double limit,
                              Keep keep)
{
    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kWidth[3] = {11, 11, 10};
    uint32_t prefix = 0;
    for (int level = 0; level < 3; ++level) {
        const int shift = kShift[level], width = kWidth[level];
        const int hi = shift + width;
        const int nd = 1 << width;
        for (int d = threadIdx.x; d < nd; d += kFThreads) {
            sh.bcnt[d] = 0;
            sh.bmass[d] = 0;
        }
        if (threadIdx.x == 0) sh.sel = 0xffffffffu;
        __syncthreads();
        src.each([&](unsigned long long packed) {
            if (!keep(packed)) return;
            const uint32_t key = (uint32_t)(packed >> 32);
            if (hi < 32 && (key >> hi) != (prefix >> hi)) return;
            const uint32_t d = (key >> shift) & (uint32_t)(nd - 1);
            atomicAdd(&sh.bcnt[d], 1u);
            atomicAdd(&sh.bmass[d], src.mass(packed));
        });
        __syncthreads();
        const int dpt = (nd + kFThreads - 1) / kFThreads;
        const int dlo = (int)threadIdx.x * dpt;
        unsigned long long own = 0;
        for (int j = 0; j < dpt; ++j)
            if (dlo + j < nd) own += sh.bmass[dlo + j];
        unsigned long long up =
            A + block_scan_inclusive<unsigned long long, kFThreads, true>(own, sh.red) - own;
        uint32_t cand = 0xffffffffu;
        unsigned long long cand_up = 0;
        for (int j = dpt - 1; j >= 0; --j) {
            const int d = dlo + j;
            if (d >= nd) continue;
            if ((double)up > limit) break;
            if (sh.bcnt[d]) {
                cand = (uint32_t)d;
                cand_up = up;
            }
            up += sh.bmass[d];
        }
        if (cand != 0xffffffffu) atomicMin(&sh.sel, cand);
        __syncthreads();
        if (cand != 0xffffffffu && cand == sh.sel) sh.up = cand_up;
        __syncthreads();
        prefix |= sh.sel << shift;
        A = sh.up;
        __syncthreads();
    }
    return prefix;
}

// Gumbel argmax over the kept tokens (packed >= kpack, key >= tau): per
// batch of list entries, the noise of the kept ones is requested together
// (a rejected entry reads element 0 and is ignored), so the gathers overlap.
__device__ __forceinline__ unsigned long long gumbel_best(const ListSource &src, FinishShared &sh, const float *g,
                                          unsigned long long kpack, uint32_t tau)
{
    unsigned long long best = 0;
    for (int c0 = src.csub; c0 < src.nch; c0 += kBatch * src.per) {
        unsigned long long v[kBatch];
        bool keep[kBatch];
        float gv[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int c = c0 + j * src.per;
            const bool ok = c < src.nch && src.slot < (int)src.nlist[c < src.nch ? c : 0];
            v[j] = src.lrow[(int64_t)(ok ? c : 0) * src.cap + (ok ? src.slot : 0)];
            const uint32_t key = (uint32_t)(v[j] >> 32);
            keep[j] = ok && key > src.tout && v[j] >= kpack && key >= tau;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) gv[j] = g[keep[j] ? unpack_index(v[j]) : 0u];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const unsigned long long cand =
                pack_key_index(float_key(value_of(v[j]) + gv[j]), unpack_index(v[j]));
            best = keep[j] ? max(best, cand) : best;
        }
    }
    return block_max<unsigned long long, kFThreads>(best, sh.red);
}

__device__ __forceinline__ unsigned long long gumbel_best(const RowSource &src, FinishShared &sh, const float *g,
                                          unsigned long long kpack, uint32_t tau)
{
    unsigned long long best = 0;
    src.each([&](unsigned long long packed) {
        const uint32_t key = (uint32_t)(packed >> 32);
        if (packed < kpack || key < tau) return;
        const uint32_t i = unpack_index(packed);
        best = max(best, pack_key_index(float_key(key_float(key) + g[i]), i));
    });
    return block_max<unsigned long long, kFThreads>(best, sh.red);
}

// Top-k, nucleus and the Gumbel argmax over one source; writes the id and
// the cut.  hist: sh.bcnt (and, for nucleus-only rows, sh.bmass) already
// hold the source's value bins.
template <typename Src>
__device__ __forceinline__ void select_and_draw(const SampArgs &a, FinishShared &sh, const Src &src, int b,
                                uint32_t mode, uint32_t kmax, unsigned long long Z, bool hist)
{
    const float M = key_float(kmax);
    const bool topk = (mode & MODE_TOPK) != 0;
    auto all = [](unsigned long long) { return true; };
    unsigned long long kpack = 0;
    if (topk) {
        const uint32_t k = (uint32_t)a.top_k[b];
        if (!hist) bin_hist<false>(src, sh, M, all);
        int jk;
        uint32_t r;
        bin_by_count(sh, k, jk, r);
        const uint32_t n = compact_bin(src, sh, M, jk, all);
        if (n <= (uint32_t)kCand)
            kpack = cand_rank(sh, n, r);
        else
            kpack = radix_rank(src, sh, r, [&](unsigned long long p) { return hbin_of(value_of(p), M) == jk; });
    }
    auto in_k = [=](unsigned long long packed) { return packed >= kpack; };
    uint32_t tau = 0;
    if (mode & MODE_TOPP_MAX) {
        tau = kmax;   // the maxima (top-k keeps the maximum too)
    } else if (mode & MODE_TOPP) {
        unsigned long long Zn = Z;
        // top-k then nucleus: the bins and total of the top-k set; over the
        // whole row the exact total replaces the lists' estimate
        if (topk || !hist) Zn = bin_hist<true>(src, sh, M, in_k);
        const double limit = (double)a.top_p[b] * (double)Zn;
        int js;
        unsigned long long A;
        bin_by_mass(sh, limit, js, A);
        const uint32_t n = compact_bin(src, sh, M, js, in_k);
        if (n <= (uint32_t)kCand)
            tau = cand_cut(sh, n, A, limit);
        else
            tau = radix_cut(src, sh, A, limit, [&](unsigned long long p) {
                return p >= kpack && hbin_of(value_of(p), M) == js;
            });
    }
    const unsigned long long best = gumbel_best(src, sh, a.gumbel + (int64_t)b * a.gstride, kpack, tau);
    if (threadIdx.x == 0) {
        a.out_ids[b] = (int32_t)unpack_index(best);
        RowCut cut;
        cut.mode = mode;
        cut.tau = tau;
        cut.kpack = kpack;
        a.cut[b] = cut;
    }
}

// The calling wave's LDS writes are complete before its later reads (LDS
// serves one wave's instructions in order): a wave-scope fence pair.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kWPer = kWaveCand / 64;      // tokens per lane of the resolving wave
constexpr int kWBins = kHBins / 64;        // bins per lane of that wave
static_assert(kHBins % 64 == 0 && kWaveCand % 64 == 0 && kWaveCand <= kCand, "wave fast path shape");

// Fast path of a row with one filter (top-k or nucleus): wave 0 finds the
// cut bin from the summed bins (16 per lane, a wave scan), the thread of
// that bin publishes where the bin's tokens lie in each group, and wave 0
// alone resolves the bin's tokens (at most kWaveCand) and draws, with no
// block-wide barrier after the publication (a larger bin, up to kCand
// tokens, is resolved by the whole workgroup).  False (the same in every
// thread) when the bin is empty or holds more than kCand tokens; then
// nothing has been written.

__device__ __forceinline__ bool one_pass_draw(const SampArgs &a, FinishShared &sh, const BinRec (&grp)[kGroups],
                                              int b, const RowSettings &rs, uint32_t kmax, unsigned long long Z)
{
    const uint32_t mode = rs.mode;
    const float M = key_float(kmax);
    const bool topk = (mode & MODE_TOPK) != 0;
    const uint32_t k = topk ? (uint32_t)rs.k : 0u;
    const double limit = topk ? 0.0 : (double)rs.p * (double)Z;
    if (threadIdx.x < 64) {
        const int lane = (int)threadIdx.x;
        const int d0 = lane * kWBins;
        uint32_t c[kWBins];
        unsigned long long m[kWBins];
        uint32_t csum = 0;
        unsigned long long msum = 0;
#pragma unroll
        for (int j = 0; j < kWBins; ++j) {
            c[j] = sh.bcnt[d0 + j];
            m[j] = topk ? 0ull : sh.bmass[d0 + j];
            csum += c[j];
            msum += m[j];
        }
        int found = -1;
        unsigned long long aux = 0;   // top-k: tokens in the bins before; nucleus: their mass
        if (topk) {
            uint32_t above = wave_scan_incl(csum) - csum;
#pragma unroll
            for (int j = 0; j < kWBins; ++j) {   // the bin holding rank k (one at most)
                if (above < k && k <= above + c[j]) {
                    found = d0 + j;
                    aux = above;
                }
                above += c[j];
            }
        } else {
            unsigned long long above = wave_scan_incl(msum) - msum;
#pragma unroll
            for (int j = 0; j < kWBins; ++j) {   // the deepest non-empty bin that fits
                if (c[j] && (double)above <= limit) {
                    found = d0 + j;
                    aux = above;
                }
                above += m[j];
            }
        }
        const int jc = wave_max_t(found);
        const unsigned long long own = __ballot(found == jc && jc >= 0);
        if (own) aux = readlane_t(aux, __ffsll((long long)own) - 1);
        if (lane == 0) {
            sh.sel = (uint32_t)jc;
            sh.pick = aux;
            sh.gstart[kGroups] = 0u;   // (no cut bin: nothing to resolve)
        }
    }
    __syncthreads();
    const int jc = (int)sh.sel;
    const unsigned long long aux = sh.pick;
    if ((int)threadIdx.x == jc) {   // the bin's tokens, group by group
        unsigned long long up = 0;
        uint32_t start = 0;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const bool in = g < a.groups;
            sh.goff[g] = in ? grp[g].off : 0u;
            sh.gstart[g] = start;
            start += in ? grp[g].cnt : 0u;
            up = in ? max(up, grp[g].above) : up;
        }
        sh.gstart[kGroups] = start;
        sh.up = up;
    }
    __syncthreads();
    const uint32_t n = sh.gstart[kGroups];
    if (n == 0u || n > (uint32_t)kCand) return false;   // (uniform)
    if (n > (uint32_t)kWaveCand) {   // a larger bin: every thread takes a token
        if (threadIdx.x < n) {
            int g = 0;
#pragma unroll
            for (int h = 1; h < kGroups; ++h) g = threadIdx.x >= sh.gstart[h] ? h : g;
            const SortedTok st = a.sorted[((int64_t)b * a.groups + g) * a.gslots + sh.goff[g] +
                                          (threadIdx.x - sh.gstart[g])];
            sh.ckey[threadIdx.x] = st.packed;
            sh.cgum[threadIdx.x] = st.g;
            sh.cmass[threadIdx.x] = topk ? 0ull : mass_fixed(value_of(st.packed), (double)M, sh.tab);
        }
        __syncthreads();
        unsigned long long kpack = 0;
        uint32_t tau = 0;
        if (topk)
            kpack = cand_rank(sh, n, k - (uint32_t)aux);
        else
            tau = cand_cut(sh, n, aux, limit);
        unsigned long long best = threadIdx.x == 0 ? sh.up : 0ull;
        if (threadIdx.x < n) {
            const unsigned long long v = sh.ckey[threadIdx.x];
            const bool keep = topk ? v >= kpack : (uint32_t)(v >> 32) >= tau;
            if (keep)
                best = max(best, pack_key_index(float_key(value_of(v) + sh.cgum[threadIdx.x]), unpack_index(v)));
        }
        best = block_max<unsigned long long, kFThreads>(best, sh.red);
        if (threadIdx.x == 0) {
            a.out_ids[b] = (int32_t)unpack_index(best);
            RowCut cut;
            cut.mode = mode;
            cut.tau = tau;
            cut.kpack = kpack;
            a.cut[b] = cut;
        }
        return true;
    }
    if (threadIdx.x >= 64) return true;

    // ---- wave 0 alone from here: lane l holds tokens l + 64 r of the bin ----
    const int lane = (int)threadIdx.x;
    unsigned long long key[kWPer], mass[kWPer];
    float gum[kWPer];
    uint32_t vlo = 0xffffffffu, vhi = 0u;
#pragma unroll
    for (int r = 0; r < kWPer; ++r) {
        const uint32_t e = (uint32_t)(lane + 64 * r);
        key[r] = 0;
        mass[r] = 0;
        gum[r] = 0.f;
        if (e < n) {
            int g = 0;
#pragma unroll
            for (int h = 1; h < kGroups; ++h) g = e >= sh.gstart[h] ? h : g;
            const SortedTok st =
                a.sorted[((int64_t)b * a.groups + g) * a.gslots + sh.goff[g] + (e - sh.gstart[g])];
            key[r] = st.packed;
            gum[r] = st.g;
            mass[r] = topk ? 0ull : mass_fixed(value_of(st.packed), (double)M, sh.tab);
            vlo = min(vlo, (uint32_t)(st.packed >> 32));
            vhi = max(vhi, (uint32_t)(st.packed >> 32));
        }
    }
    // Up to 16 tokens are compared directly.  Above that the bin's value
    // range is cut into 64 sub-ranges, lane l owning the (63 - l)-th so that
    // lanes run from the largest values down; their counts (and masses) in
    // LDS locate the sub-range holding the cut, and only its tokens are
    // compared one by one.  Tied values share a sub-range.
    const bool small = n <= 16u;
    uint32_t sub[kWPer] = {};
    uint32_t sel = 0;
    unsigned long long base = topk ? 0ull : aux;   // top-k: tokens in the sub-ranges above; nucleus: A plus their mass
    if (!small) {
        vlo = ~wave_max_t(~vlo);
        vhi = wave_max_t(vhi);
        const unsigned long long span = (unsigned long long)(vhi - vlo) + 1;
        sh.wcnt[lane] = 0;
        sh.wmass[lane] = 0;
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < kWPer; ++r) {
            if ((uint32_t)(lane + 64 * r) < n) {
                sub[r] = (uint32_t)(((unsigned long long)((uint32_t)(key[r] >> 32) - vlo) * 64) / span);
                atomicAdd(&sh.wcnt[sub[r]], 1u);
                if (!topk) atomicAdd(&sh.wmass[sub[r]], mass[r]);
            }
        }
        wave_lds_sync();
        const uint32_t cnt = sh.wcnt[63 - lane];
        if (topk) {
            const uint32_t rank = k - (uint32_t)aux;
            const uint32_t before = wave_scan_incl(cnt) - cnt;
            const unsigned long long bal = __ballot(before < rank && rank <= before + cnt);
            const int src = bal ? __ffsll((long long)bal) - 1 : 0;   // (one lane: rank <= n)
            sel = 63u - (uint32_t)src;
            base = readlane_t(before, src);
        } else {
            const unsigned long long ms = sh.wmass[63 - lane];
            const unsigned long long before = wave_scan_incl(ms) - ms;
            // the deepest non-empty sub-range whose strictly-greater mass fits
            // (the bin's top token always fits: its strictly-greater mass is A)
            const unsigned long long bal = __ballot(cnt != 0u && (double)(aux + before) <= limit);
            const int src = bal ? 63 - __clzll((long long)bal) : 0;
            sel = 63u - (uint32_t)src;
            base = aux + readlane_t(before, src);
        }
    }
    // the chosen sub-range's tokens, compacted into LDS records (top-k: the
    // packed key; nucleus: the value key and the mass)
    uint32_t m = 0;
    bool in[kWPer];
#pragma unroll
    for (int r = 0; r < kWPer; ++r) in[r] = (uint32_t)(lane + 64 * r) < n && (small || sub[r] == sel);
    if (!small) {
#pragma unroll
        for (int r = 0; r < kWPer; ++r) {
            const unsigned long long bal = __ballot(in[r]);
            const uint32_t pos = m + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (in[r]) sh.crec[pos] = topk ? CandRec{key[r], 0ull} : CandRec{key[r] >> 32, mass[r]};
            m += (uint32_t)__popcll(bal);
        }
        wave_lds_sync();
    }
    // each of them against every token of the sub-range (every lane reads
    // the same record: a broadcast), eight records in flight; a small bin's
    // tokens against each other through cross-lane reads
    uint32_t larger[kWPer] = {};
    unsigned long long above[kWPer] = {};
    uint32_t j = 0;
    auto visit = [&](const CandRec &rc) {
#pragma unroll
        for (int r = 0; r < kWPer; ++r) {
            if (topk)
                larger[r] += rc.a > key[r] ? 1u : 0u;
            else
                above[r] += rc.a > (key[r] >> 32) ? rc.b : 0ull;
        }
    };
    if (small) {   // one token per lane (lane < n), read across lanes
        for (; j < n; ++j) {
            if (topk) {
                larger[0] += readlane_t(key[0], (int)j) > key[0] ? 1u : 0u;
            } else {
                const uint32_t vj = readlane_t((uint32_t)(key[0] >> 32), (int)j);
                above[0] += vj > (uint32_t)(key[0] >> 32) ? readlane_t(mass[0], (int)j) : 0ull;
            }
        }
    } else {
        for (; j + 8 <= m; j += 8) {
            CandRec rc[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) rc[u] = sh.crec[j + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) visit(rc[u]);
        }
        for (; j < m; ++j) visit(sh.crec[j]);
    }
    unsigned long long kpack = 0;
    uint32_t tau = 0;
    if (topk) {
        const uint32_t rank_in = k - (uint32_t)aux - (uint32_t)base;
        unsigned long long pick = 0;
#pragma unroll
        for (int r = 0; r < kWPer; ++r)
            if (in[r] && larger[r] + 1 == rank_in) pick = key[r];
        kpack = wave_max_t(pick);   // (exactly one token has that rank)
    } else {
        // the smallest qualifying value: a max over complemented keys
        uint32_t nk = 0;
#pragma unroll
        for (int r = 0; r < kWPer; ++r)
            if (in[r] && (double)(base + above[r]) <= limit) nk = max(nk, ~(uint32_t)(key[r] >> 32));
        tau = ~wave_max_t(nk);
    }
    // the best of the bins before jc and of bin jc's kept tokens
    unsigned long long best = lane == 0 ? sh.up : 0ull;
#pragma unroll
    for (int r = 0; r < kWPer; ++r) {
        const unsigned long long v = key[r];
        if ((uint32_t)(lane + 64 * r) < n && (topk ? v >= kpack : (uint32_t)(v >> 32) >= tau))
            best = max(best, pack_key_index(float_key(value_of(v) + gum[r]), unpack_index(v)));
    }
    best = wave_max_t(best);
    if (lane == 0) {
        a.out_ids[b] = (int32_t)unpack_index(best);
        RowCut cut;
        cut.mode = mode;
        cut.tau = tau;
        cut.kpack = kpack;
        a.cut[b] = cut;
    }
    return true;
}

__global__ __launch_bounds__(kFThreads) void samp_finish_kernel(const SampArgs a)
{
    __shared__ FinishShared sh;
    const int b = blockIdx.x;
    const RowSettings rs = row_settings(a, b);   // (read once, before any barrier)
    const uint32_t mode = rs.mode;
    const ChunkRec *rec = a.rec + (int64_t)b * a.nchunks;
    const int nch = a.nchunks;
    if (mode & (MODE_GREEDY | MODE_PLAIN)) {
        unsigned long long best = 0;
        for (int c = threadIdx.x; c < nch; c += kFThreads) best = max(best, rec[c].best);
        best = block_max<unsigned long long, kFThreads>(best, sh.red);
        if (threadIdx.x == 0) {
            a.out_ids[b] = (int32_t)unpack_index(best);
            RowCut cut = {mode, 0u, 0ull};
            a.cut[b] = cut;
        }
        return;
    }
    const bool use_hist = (mode & (MODE_TOPK | MODE_TOPP)) != 0;
    const bool single = (mode == MODE_TOPK) || (mode == MODE_TOPP);

    // ---- one round of loads: the groups' records of this thread's bin
    // (requested blind: bins past the last one written hold stale data,
    // dropped once T* is known) and the groups' totals, which also carry the
    // row max and T*.  Rows without a histogram take those from the chunk
    // records.
    static_assert(kHBins == kFThreads, "one finish bin per thread");
    BinRec grp[kGroups];
    uint32_t kmax, tout;
    RowTot tot = {};
    if (use_hist) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g)   // (a missing group reads group 0, dropped below)
            grp[g] = a.bins[((int64_t)b * a.groups + (g < a.groups ? g : 0)) * kHBins + threadIdx.x];
        const RowTot t0 = a.tot[(int64_t)b * a.groups];
        if (threadIdx.x < (unsigned)a.groups) sh.gtot[threadIdx.x] = a.tot[(int64_t)b * a.groups + threadIdx.x];
        if (threadIdx.x < 64) sh.tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
        kmax = t0.kmax;
        tout = t0.tout;
        // the groups' bins and totals added up (the totals once the barrier
        // below has made them visible)
        const bool in = (int)threadIdx.x < bins_above(tout, key_float(kmax));
        uint32_t cnt = 0;
        unsigned long long mass = 0;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            if (!in || g >= a.groups) {
                grp[g].cnt = 0;
                grp[g].off = 0;
                grp[g].mass = 0;
                grp[g].above = 0;
            }
            cnt += grp[g].cnt;
            mass += grp[g].mass;
        }
        sh.bcnt[threadIdx.x] = cnt;
        sh.bmass[threadIdx.x] = mass;
        __syncthreads();
        for (int g = 0; g < a.groups; ++g) {
            tot.Z += sh.gtot[g].Z;
            tot.mu += sh.gtot[g].mu;
            tot.nu += sh.gtot[g].nu;
        }
    } else {
        uint32_t km = 0, to = 0;
        for (int c = threadIdx.x; c < nch; c += kFThreads) {
            const ChunkRec r = rec[c];
            km = max(km, r.mkey);
            to = max(to, r.outkey);
            sh.nlist[c] = r.n;
        }
        if (threadIdx.x < 64) sh.tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
        block_max2<kFThreads>(km, to, sh.red, kmax, tout);   // (its barrier orders the LDS fills)
    }
    const float Mf = key_float(kmax);
    const double M = (double)Mf;
    // The lists hold every token above T*; the cut must lie above T*.
    bool ok;
    if (mode & MODE_TOPK) ok = tot.nu >= (uint32_t)rs.k;
    else if (mode & MODE_TOPP) ok = (double)tot.mu > (double)rs.p * (double)tot.Z;
    else ok = tout < kmax;   // p <= 0: every maximum must be above T*
    if (ok && single && one_pass_draw(a, sh, grp, b, rs, kmax, tot.Z)) return;
    if (ok) {
        if (use_hist) {   // the lists' sizes (rows without a histogram have them)
            for (int c = threadIdx.x; c < nch; c += kFThreads) sh.nlist[c] = rec[c].n;
            __syncthreads();
        }
        ListSource src;
        src.lrow = a.list + (int64_t)b * nch * a.cap;
        src.nlist = sh.nlist;
        src.cap = a.cap;
        src.per = kFThreads / a.cap;
        src.nch = nch;
        src.slot = (int)threadIdx.x % a.cap;
        src.csub = (int)threadIdx.x / a.cap;
        src.tout = tout;
        src.M = M;
        src.tab = sh.tab;
        select_and_draw(a, sh, src, b, mode, kmax, tot.Z, use_hist);
    } else {
        RowSource rs{a.logits + (int64_t)b * a.lstride,
                     a.mask ? a.mask + (int64_t)b * a.mstride : nullptr,
                     Scaler(a.temperature[b]), M, a.vocab, sh.tab};
        select_and_draw(a, sh, rs, b, mode, kmax, tot.Z, false);
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
    const RowCut cut = a.cut[b];
    const uint32_t mode = cut.mode;
    const bool greedy = (mode & MODE_GREEDY) != 0;
    const uint32_t tau = greedy ? 0u : cut.tau;
    const unsigned long long kpack = greedy ? 0ull : cut.kpack;
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
        const float v = (id >= 0 && id < V) ? value(id) : __builtin_nanf("");
        a.out_prob[b] = (float)(exp((double)v - (double)M) / Z);
    }
}

// MASK: a vocabulary mask is given (without one, the scan is compiled with
// every logit allowed).
template <bool VEC4, bool MASK>
void launch_passes(const SampArgs &a, const dim3 grid, hipStream_t stream)
{
    switch (a.chunk / kThreads) {
    case 16: samp_scan_kernel<VEC4, MASK, 16><<<grid, kThreads, 0, stream>>>(a); break;
    case 8: samp_scan_kernel<VEC4, MASK, 8><<<grid, kThreads, 0, stream>>>(a); break;
    default: samp_scan_kernel<VEC4, MASK, 4><<<grid, kThreads, 0, stream>>>(a); break;
    }
    samp_hist_kernel<<<dim3(a.groups, a.batch), kHThreads, 0, stream>>>(a);
    samp_finish_kernel<<<a.batch, kFThreads, 0, stream>>>(a);
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
                          const int32_t *top_k, int32_t batch, int32_t vocab, float *out_prob,
                          int32_t *out_top_ids, float *out_top_probs, void *workspace,
                          hipStream_t stream)
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
    a.cap = L.cap;
    a.groups = L.groups;
    a.gslots = L.gslots;
    a.rec = reinterpret_cast<ChunkRec *>(ws + L.rec_off);
    a.list = reinterpret_cast<unsigned long long *>(ws + L.list_off);
    a.bins = reinterpret_cast<BinRec *>(ws + L.bins_off);
    a.sorted = reinterpret_cast<SortedTok *>(ws + L.sorted_off);
    a.tot = reinterpret_cast<RowTot *>(ws + L.tot_off);
    a.cut = reinterpret_cast<RowCut *>(ws + L.cut_off);
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
        a.mask ? launch_passes<true, true>(a, grid, stream)
               : launch_passes<true, false>(a, grid, stream);
    else
        a.mask ? launch_passes<false, true>(a, grid, stream)
               : launch_passes<false, false>(a, grid, stream);
    return hipGetLastError();
}

}  // namespace pkv
