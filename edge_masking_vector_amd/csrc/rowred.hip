// rowred.hip -- row reductions for gfx950: row sums and masked row maxima over row-major f32.
//
// Sources (web pages): Phobos docs "Slicing, bounds and masking" ("Loops over a dynamic extent":
// whole tiles unmasked plus one masked remainder; "Reductions over a ragged tile": the masked
// maximum takes -1.0e30 where iota(1) >= N - kt); teenygrad "Memory Coalescing and Tensor Layout"
// ("What it actually costs": the stride-1 row walk).
//
// Mapping.  A row is owned by a group of LPR consecutive lanes (W = 4 elements per 16-byte chunk,
// or 1 on the scalar path), so one column tile is one chunk per lane per step and the lanes of a
// group read consecutive chunks of the row: with LPR <= 64 a wave reads 64/LPR rows, LPR*W*4
// contiguous bytes each; with LPR > 64 a workgroup of LPR threads owns one row.  The host picks
// LPR from the row length and count (about 4 or 8 chunks per lane for short rows, a wave per long
// row, a whole workgroup per row when there are too few rows to fill the GPU).  The walk over column tiles is split in two: `nfull` whole tiles
// with no mask at all, issued 8 chunks at a time (32 single floats while as many remain) before
// any arithmetic (each workgroup starting at
// a different whole tile), then one remainder tile
// where a chunk element at tile-local column c is kept iff c < N - kt and otherwise replaced by the
// operator's fill (0 for a sum, -1.0e30f for a maximum).  Lane partials are folded in a fixed tree,
// then across the group with DPP row operations, ds_swizzle and readlane, and for LPR > 64 across
// the row's waves through LDS in wave order.  Rows past M re-read row
// M-1 (so every lane stays active for the cross-lane steps) and are not stored.
#include "device.hpp"
#include "launch.h"

namespace tmk {
namespace {

struct RowArgs {
    const float *x;
    float *out;         // sums / maxima; softmax statistics: m
    float *out2;        // softmax statistics: l
    int64_t ld, M, N;
    int64_t nfull;      // whole column tiles
    int64_t rem;        // live columns of the remainder tile (0 = no remainder tile)
    int64_t bc;         // column tile width
    int per_tile;       // chunks per lane per column tile
    int log_bc;         // log2(bc) (bc = LPR * W * per_tile, a power of two)
    uint32_t ngroups;   // row groups of kBlock / LPR rows
    uint64_t nf_c;      // multiply-high divisor of nfull (0: nfull too large, 64-bit modulo)
    uint32_t nf_d;
};

constexpr int kLoads = 8;   // chunks in flight per lane
constexpr int kAcc = 4;     // independent accumulators per lane
constexpr int kRemPrefetch = 4;  // remainder-tile chunks per lane loaded ahead of the whole tiles

template <class Op>
__device__ __forceinline__ float combine(float a, float b) { return Op::f(a, b); }
template <class Op>
__device__ __forceinline__ f4 combine(f4 a, f4 b) {
    f4 r;
    r.x = Op::f(a.x, b.x);
    r.y = Op::f(a.y, b.y);
    r.z = Op::f(a.z, b.z);
    r.w = Op::f(a.w, b.w);
    return r;
}

template <class Op>
__device__ __forceinline__ float lanes(float v) { return v; }
template <class Op>
__device__ __forceinline__ float lanes(f4 v) { return Op::f(Op::f(v.x, v.y), Op::f(v.z, v.w)); }

// Whole chunk of a whole tile.  When the LPR lanes of a row cover at least one 128-byte line per
// load instruction, it is streamed (non-temporal: every element is read exactly once).  Narrower
// groups read a line over several instructions, so the line must stay cached between them: with
// the non-temporal hint, 16-float rows read by one lane each took 11.5 us for 32 MB (held in the
// Infinity Cache) against 7.5 us with plain loads.
template <bool VEC, int LPR>
__device__ __forceinline__ auto load_whole(const float *p) {
    constexpr bool kStream = LPR * (VEC ? 16 : 4) >= 128;
    if constexpr (VEC)
        return kStream ? ld16_nt(p) : ld16(p);
    else
        return kStream ? ld4_nt(p) : *p;
}

// Chunk at p whose first `live` elements exist (live may be <= 0); the others take the fill.
template <class Op, bool VEC>
__device__ __forceinline__ auto load_fill(const float *p, int64_t live) {
    if constexpr (VEC) {
        if (live >= 4)
            return ld16(p);
        f4 r = f4(Op::kFill);
        if (live > 0)
            r.x = p[0];
        if (live > 1)
            r.y = p[1];
        if (live > 2)
            r.z = p[2];
        return r;
    } else {
        return live > 0 ? *p : Op::kFill;
    }
}

// SHIFT walks (rows off the 16-byte grid): the row is read from the 16-byte boundary `head`
// elements before its start, and the first `head` elements of its first chunk (not the row's)
// take the fill.
template <class Op>
__device__ __forceinline__ f4 head_fill(f4 v, int head) {
    v.x = head > 0 ? Op::kFill : v.x;
    v.y = head > 1 ? Op::kFill : v.y;
    v.z = head > 2 ? Op::kFill : v.z;
    return v;
}
template <class Op>
__device__ __forceinline__ float head_fill(float v, int head) { return v; }

// The row a lane walks: its start, its length and its split into whole tiles plus a remainder.
// SHIFT: from the 16-byte boundary at or before the row's start, with head masked elements in
// front (head = (start address / 4) mod 4), so that every chunk is a 16-byte vector; the split is
// then that of N + head elements.
struct RowSpan {
    const float *xr;
    int64_t N, nfull, rem;
    int head;
};
template <bool SHIFT>
__device__ __forceinline__ RowSpan row_span(const float *xr, int64_t N, int64_t nfull, int64_t rem, int log_bc) {
    RowSpan s{xr, N, nfull, rem, 0};
    if constexpr (SHIFT) {
        s.head = int((reinterpret_cast<uintptr_t>(xr) >> 2) & 3);
        s.xr = xr - s.head;
        s.N = N + s.head;
        s.nfull = s.N >> log_bc;
        s.rem = s.N - (s.nfull << log_bc);
    }
    return s;
}

// First whole tile of row group grp in the rotated walk: 7 * grp mod nfull, by multiply-high
// division (exact: fast_mod(grp) * 7 stays below 2^32 for the divisors the host passes).  A 64-bit
// modulo costs about a hundred scalar instructions, paid by every row group before its first
// load: it took 16M one-element row sums to 49 us.
__device__ __forceinline__ int64_t first_tile(uint32_t grp, const RowArgs &a) {
    if (a.nfull <= 1)
        return 0;
    if (a.nf_c != 0)
        return fast_mod(fast_mod(grp, a.nf_c, a.nf_d) * 7u, a.nf_c, a.nf_d);
    return static_cast<int64_t>(uint64_t(grp) * 7u % uint64_t(a.nfull));
}

// Threads per workgroup for LPR lanes per row: kBlock (several rows), or LPR (one row).
template <int LPR>
constexpr int block_threads() { return LPR > 64 ? LPR : kBlock; }

// The value of a row, from the per-lane values of its LPR lanes: the wave-level tree, then (LPR >
// 64) the row's waves in order through `wv` (LPR / 64 floats of LDS).  Every lane gets the
// result.  With LPR > 64 every thread of the workgroup must call it (it has barriers).
template <class Op, int LPR>
__device__ __forceinline__ float row_combine(float v, float *wv) {
    v = group_reduce<Op, (LPR < 64 ? LPR : 64)>(v);
    if constexpr (LPR > 64) {
        const int t = threadIdx.x;
        if ((t & 63) == 0)
            wv[t >> 6] = v;
        __syncthreads();
        v = wv[0];
#pragma unroll
        for (int k = 1; k < LPR / 64; ++k)
            v = Op::f(v, wv[k]);
        __syncthreads();  // wv is written again by the next combine
    }
    return v;
}

// PRE: the call has a remainder tile of at most kRemPrefetch chunks per lane, loaded ahead of the
// whole tiles (chosen on the host; without a remainder the plain walk is 2% faster).
//
// DEEP (4-byte chunks, at least 32 whole chunks per lane; chosen on the host): whole chunks go 32
// at a time while 32 remain, the bytes per lane in flight of the 16-byte path.  A separate instance,
// so that short walks keep the registers (and waves per SIMD) of the 8-deep loop.
// SHIFT (rows off the 16-byte grid, with VEC): see row_span; no rotation (the row pitch is not a
// multiple of 16 bytes, let alone of 4 KiB).
template <class Op, int LPR, bool VEC, bool PRE, bool DEEP, bool SHIFT = false>
__global__ __launch_bounds__(block_threads<LPR>()) void row_reduce(RowArgs a) {
    static_assert(!SHIFT || (VEC && !DEEP), "a shifted walk reads 16-byte chunks");
    using T = typename std::conditional<VEC, f4, float>::type;
    constexpr int W = VEC ? 4 : 1;
    constexpr int kRows = block_threads<LPR>() / LPR;  // rows per workgroup
    __shared__ float wv[LPR > 64 ? LPR / 64 : 1];
    constexpr int64_t kStep = int64_t(LPR) * W;  // columns a group covers per chunk step
    const int t = threadIdx.x;
    const int g = t % LPR;  // lane within the row group

    for (uint32_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x) {
        const int64_t row = int64_t(grp) * kRows + t / LPR;
        const int64_t rr = row < a.M ? row : a.M - 1;
        const RowSpan sp = row_span<SHIFT>(a.x + rr * a.ld, a.N, a.nfull, a.rem, a.log_bc);
        const float *xr = sp.xr;
        const float *p = xr + g * W;

        T acc[kAcc];
#pragma unroll
        for (int i = 0; i < kAcc; ++i)
            acc[i] = T(Op::kFill);

        // The remainder tile (columns kt .. N-1) is loaded first, so that its latency overlaps the
        // whole tiles instead of adding one more round trip after them (8.1 -> 7.6 us on the
        // 8192 x 1000 masked row max); it is still combined last.
        const int64_t kt = sp.nfull * a.bc;
        T rv[PRE ? kRemPrefetch : 1];
        if constexpr (PRE) {
#pragma unroll
            for (int f = 0; f < kRemPrefetch; ++f) {
                const int64_t c = int64_t(f) * kStep + g * W;  // tile-local column of the chunk
                rv[f] = f < a.per_tile ? load_fill<Op, VEC>(xr + kt + c, sp.N - kt - c) : T(Op::kFill);
                if (SHIFT && kt + c == 0)
                    rv[f] = head_fill<Op>(rv[f], sp.head);
            }
        }

        // Whole tiles: chunk k of this lane sits at column (k * LPR + g) * W; no masks.  Each
        // workgroup starts at a different whole tile (7 * group mod nfull) and wraps around: when the
        // row pitch is a multiple of 4 KiB, workgroups that all walked the tiles in the same order
        // would hit the same HBM channels at the same time.
        const int64_t main_chunks = sp.nfull * a.per_tile;
        const int64_t start = SHIFT ? 0 : first_tile(grp, a) * a.per_tile;
        // Chunk c feeds accumulator c mod kAcc in the same order at either depth: the same bits.
        int64_t k = 0;
        if constexpr (DEEP) {
            static_assert(!VEC, "the deep walk is for 4-byte chunks");
            constexpr int kDeep = 4 * kLoads;
            for (; k + kDeep <= main_chunks; k += kDeep) {
                float v[kDeep];
#pragma unroll
                for (int u = 0; u < kDeep; ++u) {
                    int64_t idx = k + u + start;
                    if (idx >= main_chunks)
                        idx -= main_chunks;
                    v[u] = load_whole<VEC, LPR>(p + idx * kStep);
                }
#pragma unroll
                for (int u = 0; u < kDeep; ++u)
                    acc[u % kAcc] = combine<Op>(acc[u % kAcc], v[u]);
            }
        }
        for (; k < main_chunks; k += kLoads) {
            T v[kLoads];
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                int64_t idx = k + u + start;
                if (idx >= main_chunks)
                    idx -= main_chunks;
                v[u] = (k + u < main_chunks) ? load_whole<VEC, LPR>(p + idx * kStep) : T(Op::kFill);
            }
            if constexpr (SHIFT) {
                if (k == 0 && g == 0)
                    v[0] = head_fill<Op>(v[0], sp.head);  // the chunk at the row's 16-byte boundary
            }
#pragma unroll
            for (int u = 0; u < kLoads; ++u)
                acc[u % kAcc] = combine<Op>(acc[u % kAcc], v[u]);
        }

        // The one remainder tile, starting at column kt: tile-local column c keeps its value iff
        // c < N - kt.
        if constexpr (PRE) {
#pragma unroll
            for (int f = 0; f < kRemPrefetch; ++f)
                if (f < a.per_tile)
                    acc[0] = combine<Op>(acc[0], rv[f]);
        } else if (sp.rem > 0) {
            for (int f = 0; f < a.per_tile; ++f) {
                const int64_t c = int64_t(f) * kStep + g * W;  // tile-local column of the chunk
                T v = load_fill<Op, VEC>(xr + kt + c, sp.N - kt - c);
                if (SHIFT && kt + c == 0)
                    v = head_fill<Op>(v, sp.head);
                acc[0] = combine<Op>(acc[0], v);
            }
        }

        // Fixed-order fold: accumulators pairwise, then the chunk's elements, then the lanes.
        T s = combine<Op>(combine<Op>(acc[0], acc[1]), combine<Op>(acc[2], acc[3]));
        float r = lanes<Op>(s);
        r = row_combine<Op, LPR>(r, wv);
        if (g == 0 && row < a.M)
            a.out[row] = r;
    }
}

// ---- softmax row statistics -------------------------------------------------------------------
// Per lane: a running maximum m and a running sum l of exp(s - m).  Each batch of chunks first
// raises m to the batch maximum b, then l = l * exp(m - b) + sum exp(s - b).  Masked and padding
// elements contribute nothing (they are skipped, not left to underflow).  The lanes of a row then
// combine: the group maximum M first, then the sum of l * exp(m - M).

__device__ __forceinline__ float sum_exp(float v, float b) { return exp_f32(v - b); }

template <class T>
__device__ __forceinline__ float chunk_max(T v) { return lanes<MaxOp>(v); }

__device__ __forceinline__ float sum_exp(f4 v, float b) {
    return (exp_f32(v.x - b) + exp_f32(v.y - b)) +
           (exp_f32(v.z - b) + exp_f32(v.w - b));
}

// Only the first `live` elements of the chunk exist.
__device__ __forceinline__ float sum_exp_live(float v, float b, int64_t live) {
    return live > 0 ? exp_f32(v - b) : 0.0f;
}
__device__ __forceinline__ float sum_exp_live(f4 v, float b, int64_t live) {
    if (live >= 4)
        return sum_exp(v, b);
    float acc = exp_f32(v.x - b);
    if (live > 1)
        acc += exp_f32(v.y - b);
    if (live > 2)
        acc += exp_f32(v.z - b);
    return acc;
}

// ---- rows read in one batch ---------------------------------------------------------------------
// Rows of a few hundred to a few thousand chunks: LPR lanes per row (16 to 64: kBlock / LPR rows per
// workgroup; 128 or 256: one row per workgroup of LPR threads, whose waves then meet in LDS in
// order) and K chunks per lane cover the row, lane g taking chunks g, g + LPR, ..., so a row costs
// one memory round trip.  The loads carry no control flow: every one is issued before any wait (a
// branch around each load had the compiler wait for each before the next, 8 round trips instead
// of 1: 7.9 against 6.9 us on 8192 x 1000).  A slot past the row loads the row's last chunk again
// and is then replaced by the fill.  The caller's column tile decides the masks ([SLICING] "Loops
// over a dynamic extent"): chunks below `whole` (the nfull whole tiles) are used as loaded;
// elements of the one remainder tile keep their value iff their column is below N and take the
// operator's fill otherwise ("Reductions over a ragged tile": -1.0e30 for the maximum).
//
// PART (16-byte chunks, N % 4 != 0): the chunk holding column N - 1 runs past the row, so every
// load goes through a buffer resource spanning exactly the row's N floats, whose range check
// returns 0 for each 4-byte word past the end (per word on gfx950) instead of reading it.
struct OnceArgs {
    const float *x;
    float *out;    // sums / maxima; softmax statistics: m
    float *out2;   // softmax statistics: l
    int64_t ld, M, N;
    int32_t whole;   // chunks of the whole tiles: nfull * bc / W
    int32_t last;    // the row's last chunk: ceil(N / W) - 1
};

// OPK: tmp::kRowSum, kRowMax or kRowSoftmax.
template <int OPK, int LPR, int K, bool VEC, bool PART>
__global__ __launch_bounds__(block_threads<LPR>()) void row_once(OnceArgs a) {
    using T = typename std::conditional<VEC, f4, float>::type;
    using Op = typename std::conditional<OPK == tmp::kRowSum, SumOp, MaxOp>::type;
    constexpr int W = VEC ? 4 : 1;
    static_assert(VEC || !PART, "4-byte chunks never straddle the row's end");
    __shared__ float wv[LPR > 64 ? LPR / 64 : 1];  // LPR > 64: the row's wave values
    const int t = threadIdx.x;
    const int g = t % LPR;
    const int64_t row = int64_t(blockIdx.x) * (block_threads<LPR>() / LPR) + t / LPR;
    const int64_t rr = row < a.M ? row : a.M - 1;  // rows past M re-read row M-1, never stored
    const float *xr = a.x + rr * a.ld;

    T v[K];
    if constexpr (PART) {
        const __amdgpu_buffer_rsrc_t rx = segment_rsrc(xr, int(a.N * 4));
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * LPR + g;
            v[k] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rx, (c < a.last ? c : a.last) * 16, 0,
                                                                               kPolicyStream));
        }
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * LPR + g;
            v[k] = load_whole<VEC, LPR>(xr + int64_t(c < a.last ? c : a.last) * W);
        }
    }
    // Masks of the remainder tile (and of the slots past the row): element e of chunk c is live
    // iff its column c * W + e is below N.
    auto live = [&](int c, int e) { return c < a.whole || int64_t(c) * W + e < a.N; };
    auto masked = [&](T x, int c, float fill) {
        if constexpr (VEC) {
            x.x = live(c, 0) ? x.x : fill;
            x.y = live(c, 1) ? x.y : fill;
            x.z = live(c, 2) ? x.z : fill;
            x.w = live(c, 3) ? x.w : fill;
            return x;
        } else {
            return live(c, 0) ? x : fill;
        }
    };
    if constexpr (OPK != tmp::kRowSoftmax) {
        // Chunk k is whole in every lane of the wave when (k + 1) * LPR <= whole, a test on kernel
        // arguments only: with 16-byte chunks such chunks skip their four selects (8192 x 1000
        // masked row maxima 7.17 -> 7.02 us).  4-byte chunks, and the softmax statistics, whose
        // code the second path doubles, measured no faster or slower that way.
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (!VEC || (k + 1) * LPR > a.whole)
                v[k] = masked(v[k], k * LPR + g, Op::kFill);
        // fixed-order fold: the K chunks pairwise, the chunk's elements, then the lanes
#pragma unroll
        for (int st = 1; st < K; st <<= 1)
#pragma unroll
            for (int i = 0; i + st < K; i += 2 * st)
                v[i] = combine<Op>(v[i], v[i + st]);
        const float r = row_combine<Op, LPR>(lanes<Op>(v[0]), wv);
        if (g == 0 && row < a.M)
            a.out[row] = r;
    } else {
        // m: the lane's maximum (the fill never exceeds a score); l: sum of exp(s - m) over the
        // live elements only; then the group maximum and the sum of l * exp(m - m_group).
        float m = kMaxFill;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            v[k] = masked(v[k], k * LPR + g, kMaxFill);
            m = __builtin_fmaxf(m, chunk_max(v[k]));
        }
        float l = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * LPR + g;
            if constexpr (VEC) {
                l += (live(c, 0) ? exp_f32(v[k].x - m) : 0.0f) + (live(c, 1) ? exp_f32(v[k].y - m) : 0.0f) +
                     (live(c, 2) ? exp_f32(v[k].z - m) : 0.0f) + (live(c, 3) ? exp_f32(v[k].w - m) : 0.0f);
            } else {
                l += live(c, 0) ? exp_f32(v[k] - m) : 0.0f;
            }
        }
        const float gm = row_combine<MaxOp, LPR>(m, wv);
        const float gl = row_combine<SumOp, LPR>(l * exp_f32(m - gm), wv);
        if (g == 0 && row < a.M) {
            a.out[row] = gm;
            a.out2[row] = gl;
        }
    }
}

// Sum of exp(s - b) over elements lo .. hi - 1 of a chunk (positions, not values, decide: a score
// may equal the fill).
__device__ __forceinline__ float sum_exp_range(f4 v, float b, int64_t lo, int64_t hi) {
    return ((lo <= 0 && 0 < hi ? exp_f32(v.x - b) : 0.0f) + (lo <= 1 && 1 < hi ? exp_f32(v.y - b) : 0.0f)) +
           ((lo <= 2 && 2 < hi ? exp_f32(v.z - b) : 0.0f) + (lo <= 3 && 3 < hi ? exp_f32(v.w - b) : 0.0f));
}
__device__ __forceinline__ float sum_exp_range(float v, float b, int64_t lo, int64_t hi) {
    return lo <= 0 && 0 < hi ? exp_f32(v - b) : 0.0f;
}

template <int LPR, bool VEC, bool PRE, bool SHIFT = false>
__global__ __launch_bounds__(block_threads<LPR>()) void row_softmax(RowArgs a) {
    static_assert(!SHIFT || VEC, "a shifted walk reads 16-byte chunks");
    using T = typename std::conditional<VEC, f4, float>::type;
    constexpr int W = VEC ? 4 : 1;
    constexpr int kRows = block_threads<LPR>() / LPR;
    __shared__ float wv[LPR > 64 ? LPR / 64 : 1];
    constexpr int64_t kStep = int64_t(LPR) * W;
    const int t = threadIdx.x;
    const int g = t % LPR;

    for (uint32_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x) {
        const int64_t row = int64_t(grp) * kRows + t / LPR;
        const int64_t rr = row < a.M ? row : a.M - 1;
        const RowSpan sp = row_span<SHIFT>(a.x + rr * a.ld, a.N, a.nfull, a.rem, a.log_bc);
        const float *xr = sp.xr;
        const float *p = xr + g * W;
        float m = kMaxFill, l = 0.0f;

        // The remainder tile's chunks are loaded ahead of the whole tiles (as in row_reduce) and
        // folded in after them.
        const int64_t kt = sp.nfull * a.bc;
        T rv[PRE ? kRemPrefetch : 1];
        if constexpr (PRE) {
#pragma unroll
            for (int f = 0; f < kRemPrefetch; ++f) {
                const int64_t c = int64_t(f) * kStep + g * W;
                rv[f] = f < a.per_tile ? load_fill<MaxOp, VEC>(xr + kt + c, sp.N - kt - c) : T(kMaxFill);
                if (SHIFT && kt + c == 0)
                    rv[f] = head_fill<MaxOp>(rv[f], sp.head);
            }
        }

        // Whole tiles, in the rotated order of row_reduce; no masks.
        const int64_t main_chunks = sp.nfull * a.per_tile;
        const int64_t start = SHIFT ? 0 : first_tile(grp, a) * a.per_tile;
        for (int64_t k = 0; k < main_chunks; k += kLoads) {
            T v[kLoads];
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                int64_t idx = k + u + start;
                if (idx >= main_chunks)
                    idx -= main_chunks;
                v[u] = (k + u < main_chunks) ? load_whole<VEC, LPR>(p + idx * kStep) : T(kMaxFill);
            }
            if constexpr (SHIFT) {
                if (k == 0 && g == 0)
                    v[0] = head_fill<MaxOp>(v[0], sp.head);  // its exp underflows to 0 below
            }
            float b = m;
#pragma unroll
            for (int u = 0; u < kLoads; ++u)
                b = __builtin_fmaxf(b, chunk_max(v[u]));  // padding is the fill: never above a score
            float acc = 0.0f;
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                if (SHIFT && u == 0 && k == 0 && g == 0)
                    acc += main_chunks > 0 ? sum_exp_range(v[0], b, sp.head, 4) : 0.0f;  // not the masked head
                else if (k + u < main_chunks)
                    acc += sum_exp(v[u], b);
            }
            l = l * exp_f32(m - b) + acc;
            m = b;
        }

        // The one remainder tile: only its first N - kt columns exist.
        if constexpr (PRE) {
#pragma unroll
            for (int f = 0; f < kRemPrefetch; ++f) {
                const int64_t c = int64_t(f) * kStep + g * W;
                const int64_t live = sp.N - kt - c;
                if (f < a.per_tile && live > 0) {
                    const float b = __builtin_fmaxf(m, chunk_max(rv[f]));
                    const float add = SHIFT && kt + c == 0 ? sum_exp_range(rv[f], b, sp.head, live)
                                                           : sum_exp_live(rv[f], b, live);
                    l = l * exp_f32(m - b) + add;
                    m = b;
                }
            }
        } else if (sp.rem > 0) {
            for (int f = 0; f < a.per_tile; ++f) {
                const int64_t c = int64_t(f) * kStep + g * W;
                const int64_t live = sp.N - kt - c;
                if (live > 0) {
                    T v = load_fill<MaxOp, VEC>(xr + kt + c, live);
                    const int64_t lo = SHIFT && kt + c == 0 ? sp.head : 0;  // masked head: not counted
                    if (lo > 0)
                        v = head_fill<MaxOp>(v, sp.head);
                    const float b = __builtin_fmaxf(m, chunk_max(v));
                    l = l * exp_f32(m - b) + (lo > 0 ? sum_exp_range(v, b, lo, live) : sum_exp_live(v, b, live));
                    m = b;
                }
            }
        }

        const float gm = row_combine<MaxOp, LPR>(m, wv);
        const float gl = row_combine<SumOp, LPR>(l * exp_f32(m - gm), wv);
        if (g == 0 && row < a.M) {
            a.out[row] = gm;
            a.out2[row] = gl;
        }
    }
}

// ---- split rows --------------------------------------------------------------------------------
// For a few long rows (the calls that bring a workspace): segment s of row i, columns
// [s*seg, min(N, (s+1)*seg)), is walked by one workgroup of kBlock threads, which writes the
// segment's partial -- its sum, its maximum, or its softmax pair (m, l) -- to the workspace at
// i*segs + s; a second kernel combines each row's partials in segment order.  Both are fixed-order
// folds, so results are deterministic.  A segment is kRowSegUnit * K elements: 4K per thread, as
// K 16-byte chunks or 4K single elements, at a stride of the workgroup's width so that a wave reads
// consecutive chunks.  Masked elements (past column N) take the operator's fill and contribute
// nothing to a softmax sum.
struct SplitArgs {
    const float *x;
    float *out;         // sums / maxima; softmax statistics: m
    float *out2;        // softmax statistics: l
    float *ws;          // partials: one float per segment, or (m, l) pairs
    int64_t ld, M, N;
    int64_t seg;        // elements per segment
    uint32_t segs;      // segments per row
    uint32_t nwork;     // M * segs
};

// v[0] = v[0] op v[1] op ... op v[C-1], pairwise in a fixed order (C a power of two).
template <class Op, int C, class T>
__device__ __forceinline__ T fold(T *v) {
#pragma unroll
    for (int st = 1; st < C; st <<= 1)
#pragma unroll
        for (int i = 0; i + st < C; i += 2 * st)
            v[i] = combine<Op>(v[i], v[i + st]);
    return v[0];
}

template <int OPK, bool VEC, int K>
__global__ __launch_bounds__(kBlock) void row_split_partial(SplitArgs a) {
    using T = typename std::conditional<VEC, f4, float>::type;
    using Op = typename std::conditional<OPK == tmp::kRowSum, SumOp, MaxOp>::type;
    constexpr int W = VEC ? 4 : 1;
    constexpr int C = tmp::kRowSegUnit / kBlock * K / W;  // chunks per thread
    constexpr int64_t kStride = int64_t(kBlock) * W;      // columns between a thread's chunks
    static_assert(C * kStride == int64_t(tmp::kRowSegUnit) * K, "segment = C chunks per thread");
    __shared__ float wv[kBlock / 64];
    const int t = threadIdx.x;

    for (uint32_t w = blockIdx.x; w < a.nwork; w += gridDim.x) {
        const uint32_t row = w / a.segs;
        const int64_t c0 = int64_t(w - row * a.segs) * a.seg;  // first column of the segment
        const float *p = a.x + int64_t(row) * a.ld + c0 + int64_t(t) * W;
        const int64_t live0 = a.N - c0 - int64_t(t) * W;     // columns from this thread's first chunk on
        const bool whole = c0 + a.seg <= a.N;                // uniform over the workgroup
        T v[C];
        if (whole) {
#pragma unroll
            for (int c = 0; c < C; ++c)
                v[c] = load_whole<VEC, kBlock>(p + c * kStride);
        } else {
#pragma unroll
            for (int c = 0; c < C; ++c)
                v[c] = load_fill<Op, VEC>(p + c * kStride, live0 - c * kStride);
        }
        if constexpr (OPK != tmp::kRowSoftmax) {
            const float r = row_combine<Op, kBlock>(lanes<Op>(fold<Op, C>(v)), wv);
            if (t == 0)
                a.ws[w] = r;
        } else {
            float m = kMaxFill;
#pragma unroll
            for (int c = 0; c < C; ++c)
                m = __builtin_fmaxf(m, chunk_max(v[c]));  // the fill never exceeds a score
            float l = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c)
                l += whole ? sum_exp(v[c], m)
                           : (live0 - c * kStride > 0 ? sum_exp_live(v[c], m, live0 - c * kStride) : 0.0f);
            const float gm = row_combine<MaxOp, kBlock>(m, wv);
            const float gl = row_combine<SumOp, kBlock>(l * exp_f32(m - gm), wv);
            if (t == 0) {
                a.ws[2 * int64_t(w)] = gm;
                a.ws[2 * int64_t(w) + 1] = gl;
            }
        }
    }
}

// One workgroup per row: thread t folds partials t, t + kBlock, ... in order, then the workgroup
// combines the threads in a fixed tree.
template <int OPK>
__global__ __launch_bounds__(kBlock) void row_split_finish(SplitArgs a) {
    __shared__ float wv[kBlock / 64];
    const int t = threadIdx.x;
    for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x) {
        if constexpr (OPK != tmp::kRowSoftmax) {
            using Op = typename std::conditional<OPK == tmp::kRowSum, SumOp, MaxOp>::type;
            const float *pp = a.ws + row * a.segs;
            float r = Op::kFill;
            for (uint32_t sg = t; sg < a.segs; sg += kBlock)
                r = Op::f(r, pp[sg]);
            r = row_combine<Op, kBlock>(r, wv);
            if (t == 0)
                a.out[row] = r;
        } else {
            const float *pp = a.ws + 2 * row * a.segs;
            float m = kMaxFill, l = 0.0f;
            for (uint32_t sg = t; sg < a.segs; sg += kBlock) {
                const float ms = pp[2 * sg], ls = pp[2 * sg + 1];
                const float b = __builtin_fmaxf(m, ms);
                l = l * exp_f32(m - b) + ls * exp_f32(ms - b);
                m = b;
            }
            const float gm = row_combine<MaxOp, kBlock>(m, wv);
            const float gl = row_combine<SumOp, kBlock>(l * exp_f32(m - gm), wv);
            if (t == 0) {
                a.out[row] = gm;
                a.out2[row] = gl;
            }
        }
    }
}

template <int OPK, bool VEC>
const void *pick_split_k(int log_k) {
    switch (log_k) {
    case 0: return reinterpret_cast<const void *>(&row_split_partial<OPK, VEC, 1>);
    case 1: return reinterpret_cast<const void *>(&row_split_partial<OPK, VEC, 2>);
    case 2: return reinterpret_cast<const void *>(&row_split_partial<OPK, VEC, 4>);
    case 3: return reinterpret_cast<const void *>(&row_split_partial<OPK, VEC, 8>);
    default: return reinterpret_cast<const void *>(&row_split_partial<OPK, VEC, 16>);
    }
}

template <int OPK>
const void *pick_split(const tmp::RowPlan &p) {
    return p.vec ? pick_split_k<OPK, true>(p.log_k) : pick_split_k<OPK, false>(p.log_k);
}

hipError_t launch_split(const tmp::RowPlan &p, hipStream_t stream) {
    static_assert(tmp::kRowSegMaxLogK == 4, "pick_split_k instantiates K = 1 .. 16");
    SplitArgs a;
    a.x = p.x;
    a.out = p.out;
    a.out2 = p.out2;
    a.ws = p.ws;
    a.ld = p.ld;
    a.M = p.M;
    a.N = p.N;
    a.seg = p.seg;
    a.segs = p.segs;
    a.nwork = p.nwork;
    void *args[] = {&a};
    const void *part = p.op == tmp::kRowMax       ? pick_split<tmp::kRowMax>(p)
                       : p.op == tmp::kRowSoftmax ? pick_split<tmp::kRowSoftmax>(p)
                                                  : pick_split<tmp::kRowSum>(p);
    const void *fin = p.op == tmp::kRowMax       ? reinterpret_cast<const void *>(&row_split_finish<tmp::kRowMax>)
                      : p.op == tmp::kRowSoftmax ? reinterpret_cast<const void *>(&row_split_finish<tmp::kRowSoftmax>)
                                                 : reinterpret_cast<const void *>(&row_split_finish<tmp::kRowSum>);
    hipError_t e = hipLaunchKernel(part, dim3(p.grid), dim3(kBlock), args, 0, stream);
    if (e != hipSuccess)
        return e;
    const uint32_t fgrid = static_cast<uint32_t>(p.M < (int64_t{1} << 20) ? p.M : (int64_t{1} << 20));
    return hipLaunchKernel(fin, dim3(fgrid), dim3(kBlock), args, 0, stream);
}

template <int LPR, bool PRE>
const void *pick_softmax_vec(const tmp::RowPlan &p) {
    if (p.shift)
        return reinterpret_cast<const void *>(&row_softmax<LPR, true, PRE, true>);
    return p.vec ? reinterpret_cast<const void *>(&row_softmax<LPR, true, PRE>)
                 : reinterpret_cast<const void *>(&row_softmax<LPR, false, PRE>);
}

template <bool PRE>
const void *pick_softmax(const tmp::RowPlan &p) {
    switch (p.lpr) {
    case 1: return pick_softmax_vec<1, PRE>(p);
    case 2: return pick_softmax_vec<2, PRE>(p);
    case 4: return pick_softmax_vec<4, PRE>(p);
    case 8: return pick_softmax_vec<8, PRE>(p);
    case 16: return pick_softmax_vec<16, PRE>(p);
    case 32: return pick_softmax_vec<32, PRE>(p);
    case 64: return pick_softmax_vec<64, PRE>(p);
    case 128: return pick_softmax_vec<128, PRE>(p);
    case 256: return pick_softmax_vec<256, PRE>(p);
    case 512: return pick_softmax_vec<512, PRE>(p);
    default: return pick_softmax_vec<1024, PRE>(p);
    }
}

template <class Op, bool VEC, bool PRE, bool DEEP, bool SHIFT = false>
const void *pick_lpr(int lpr) {
    switch (lpr) {
    case 1: return reinterpret_cast<const void *>(&row_reduce<Op, 1, VEC, PRE, DEEP, SHIFT>);
    case 2: return reinterpret_cast<const void *>(&row_reduce<Op, 2, VEC, PRE, DEEP, SHIFT>);
    case 4: return reinterpret_cast<const void *>(&row_reduce<Op, 4, VEC, PRE, DEEP, SHIFT>);
    case 8: return reinterpret_cast<const void *>(&row_reduce<Op, 8, VEC, PRE, DEEP, SHIFT>);
    case 16: return reinterpret_cast<const void *>(&row_reduce<Op, 16, VEC, PRE, DEEP, SHIFT>);
    case 32: return reinterpret_cast<const void *>(&row_reduce<Op, 32, VEC, PRE, DEEP, SHIFT>);
    case 64: return reinterpret_cast<const void *>(&row_reduce<Op, 64, VEC, PRE, DEEP, SHIFT>);
    case 128: return reinterpret_cast<const void *>(&row_reduce<Op, 128, VEC, PRE, DEEP, SHIFT>);
    case 256: return reinterpret_cast<const void *>(&row_reduce<Op, 256, VEC, PRE, DEEP, SHIFT>);
    case 512: return reinterpret_cast<const void *>(&row_reduce<Op, 512, VEC, PRE, DEEP, SHIFT>);
    default: return reinterpret_cast<const void *>(&row_reduce<Op, 1024, VEC, PRE, DEEP, SHIFT>);
    }
}

template <class Op, bool PRE>
const void *pick_vec(const tmp::RowPlan &p) {
    // 4-byte walks of at least 32 whole chunks per lane: 2048 x 8191 row sums 18.3 -> 14.9 us, 16
    // x 1000003 130 -> 110 us.  (One instance for every length had cost short walks up to 17%:
    // 8192 x 1000 at stride 1001 7.9 -> 9.3 us.)
    if (p.shift)
        return pick_lpr<Op, true, PRE, false, true>(p.lpr);
    if (p.vec)
        return pick_lpr<Op, true, PRE, false>(p.lpr);
    return p.nfull * p.per_tile >= 4 * kLoads ? pick_lpr<Op, false, PRE, true>(p.lpr)
                                              : pick_lpr<Op, false, PRE, false>(p.lpr);
}

template <bool PRE>
const void *pick_op(const tmp::RowPlan &p) {
    return p.op == tmp::kRowMax       ? pick_vec<MaxOp, PRE>(p)
           : p.op == tmp::kRowSoftmax ? pick_softmax<PRE>(p)
                                      : pick_vec<SumOp, PRE>(p);
}

template <int OPK, bool VEC, int K, bool PART>
const void *pick_once_lpr(int lpr) {
    switch (lpr) {
    case 16: return reinterpret_cast<const void *>(&row_once<OPK, 16, K, VEC, PART>);
    case 32: return reinterpret_cast<const void *>(&row_once<OPK, 32, K, VEC, PART>);
    case 64: return reinterpret_cast<const void *>(&row_once<OPK, 64, K, VEC, PART>);
    default: break;
    }
    if constexpr (VEC)  // 4-byte rows are planned with at most 64 lanes
        return lpr == 128 ? reinterpret_cast<const void *>(&row_once<OPK, 128, K, VEC, PART>)
                          : reinterpret_cast<const void *>(&row_once<OPK, 256, K, VEC, PART>);
    return nullptr;
}

template <int OPK>
const void *pick_once(const tmp::RowPlan &p) {
    if (!p.vec)
        return pick_once_lpr<OPK, false, tmp::kRowOnceKScalar, false>(p.lpr);
    return p.N % 4 != 0 ? pick_once_lpr<OPK, true, tmp::kRowOnceK, true>(p.lpr)
                        : pick_once_lpr<OPK, true, tmp::kRowOnceK, false>(p.lpr);
}

hipError_t launch_once(const tmp::RowPlan &p, hipStream_t stream) {
    OnceArgs a;
    a.x = p.x;
    a.out = p.out;
    a.out2 = p.out2;
    a.ld = p.ld;
    a.M = p.M;
    a.N = p.N;
    const int W = p.vec ? 4 : 1;
    a.whole = static_cast<int32_t>(p.nfull * (p.bc / W));
    a.last = static_cast<int32_t>((p.N + W - 1) / W - 1);
    const void *fn = p.op == tmp::kRowMax       ? pick_once<tmp::kRowMax>(p)
                     : p.op == tmp::kRowSoftmax ? pick_once<tmp::kRowSoftmax>(p)
                                                : pick_once<tmp::kRowSum>(p);
    if (fn == nullptr)
        return hipErrorInvalidConfiguration;
    void *args[] = {&a};
    return hipLaunchKernel(fn, dim3(p.grid), dim3(p.block), args, 0, stream);
}

}  // namespace

hipError_t launch_rows(const tmp::RowPlan &p, hipStream_t stream) {
    if (p.split)
        return launch_split(p, stream);
    if (p.once)
        return launch_once(p, stream);
    RowArgs a;
    a.x = p.x;
    a.out = p.out;
    a.out2 = p.out2;
    a.ld = p.ld;
    a.M = p.M;
    a.N = p.N;
    a.nfull = p.nfull;
    a.rem = p.rem;
    a.bc = p.bc;
    a.per_tile = p.per_tile;
    a.log_bc = tmp::ilog2(p.bc);
    const int64_t rows_per_wg = p.block / p.lpr;
    a.ngroups = static_cast<uint32_t>((p.M + rows_per_wg - 1) / rows_per_wg);
    // 7 * (grp mod nfull) < 2^32 keeps the two-step multiply-high modulo exact
    const bool small = p.nfull > 1 && p.nfull < int64_t{0xFFFFFFFF} / 7;
    const tmp::Div32 nf = small ? tmp::make_div32(static_cast<uint32_t>(p.nfull)) : tmp::Div32{};
    a.nf_c = small ? nf.c : 0;
    a.nf_d = nf.d;
    const bool pre = p.rem > 0 && p.per_tile <= kRemPrefetch;
    const void *fn = pre ? pick_op<true>(p) : pick_op<false>(p);
    void *args[] = {&a};
    return hipLaunchKernel(fn, dim3(p.grid), dim3(p.block), args, 0, stream);
}

}  // namespace tmk
