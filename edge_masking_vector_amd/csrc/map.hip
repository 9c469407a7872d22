// map.hip -- tiled element-wise maps for gfx950: y = fmaf(x, alpha, beta), y = alpha * x, the
// bitwise copy and the per-channel y = fmaf(x, scale[col], bias[col]), over TM x TN tiles of
// row-major f32 views.
//
// Sources (web pages): Phobos docs "@aligned" ("A minimal kernel", "What it changes"); Phobos docs
// "Slicing, bounds and masking" ("Masking", "Promising whole tiles with @aligned"); Mojo GPU
// puzzle 35 "Aligned Load & Store" ("The exercise", "Solution": the scalar, under-aligned and
// aligned variants); teenygrad "Memory Coalescing and Tensor Layout" ("Coalescing": consecutive
// lanes take consecutive addresses; "NCHW versus NHWC": per-channel scale and bias on an NC view).
//
// Mapping (the tile scheduler).  A tile holds TM rows of VR = TN/W chunks (W = 4 elements for the
// vector variants, 1 for scalar).  A workgroup takes one work item: R consecutive rows of G
// horizontally adjacent tiles of one tile row band, R*G*VR chunks, moved by 64 to 1024 threads
// with U chunks per thread (U = 4 for the 4-byte accesses AUTO falls back to, else 1: the vector
// variants and the one-element-per-thread scalar variant) at a stride of the workgroup size, all loads
// before any store.  Within a work-item row the lane-varying term of every address is the chunk
// index, so a wave reads consecutive chunks of a row.  Work items run with the tile groups
// fastest, then row strips, then tile rows, so workgroups dispatched together cover neighbouring
// memory.  The host picks the geometry (plan.cpp).  Views whose rows are contiguous in both
// tensors (row stride N) are planned as one row of M*N elements, except for the channel op, so
// that only the flat row's end can be ragged.  When rows start on 128-byte lines a work item
// is one wave's worth of chunks -- with 16-byte chunks, where the tile group allows, one 1 KiB
// row segment; else a strip of rows of a tile group with 512-byte row segments; when a whole
// item's output is one contiguous 1 KiB (a segment, or whole rows of contiguous rows) it is
// stored through a buffer resource with device scope and the streaming hint (sc1 nt) -- and
// otherwise it spans as many tiles as fit in 1024 threads across the row band, so that
// few 128-byte lines are shared by workgroups that may run on different XCDs (each XCD has its
// own L2 and would fetch a shared line again).  Whole chunks move with the non-temporal hint.  On
// gfx950 one 16-byte chunk per thread streamed faster than several chunks per thread, and
// one-wave workgroups at least as fast as 1024-thread ones (up to 11% faster on jobs of a few
// thousand workgroups, whose last round of workgroups is otherwise ragged).
//
// Paths.  aligned=1: no masks at all (the host checked whole tiles and 16-byte rows).
// aligned=0: a uniform per-tile test picks the same unmasked body for whole tiles; edge tiles
// take the masked body, where a chunk wholly inside the tensor still moves as one vector, a chunk
// straddling column N moves element by element, and elements past the edge read as 0 and are
// never stored.
#include "device.hpp"
#include "launch.h"

namespace tmk {
namespace {

struct MapArgs {
    const float *x;
    float *y;
    int64_t ldx, ldy, M, N;
    float alpha, beta;
    uint32_t tiles_n;    // tiles along N
    uint32_t group;      // G: tiles per work item along N
    uint32_t groups_n;   // tile groups along N: ceil(tiles_n / G)
    uint32_t nwork;      // work items: ceil(M / R) row strips * groups_n
    int log_tm, log_tn;
    int log_vr;          // chunks per tile row
    int log_gv;          // chunks per work-item row: G * VR
    int log_r;           // rows per work item
    int log_strips;      // work items per tile along M: TM / R
    int log_bs;          // threads per workgroup
    const float *scale;  // channel op: per-column scale (null: 1) and bias
    const float *bias;
    int cvec16;          // channel op: the column vectors are 16-byte aligned
    // Channel op over a flat view (rows of C contiguous channels planned as one row): the channel
    // of flat column col is col mod C.  chan_n = 0: the channel is the column.
    uint32_t chan_n;     // C
    uint32_t chan_step;  // (columns per work item) mod C
    uint64_t chan_c;     // multiply-high divisor of C
    // Element step inside an under-stated 4-element chunk.  Always 1; passed at run time so the
    // compiler cannot prove the four accesses adjacent and fuse them into one 16-byte access
    // (gfx950 accepts dwordx4 at 4-byte alignment, so a merely under-stated alignment would still
    // be vectorised).
    int64_t estep;
};

template <int ACC>
struct Chunk {
    using T = f4;
    static constexpr int W = 4;
};
template <>
struct Chunk<tmp::kScalar> {
    using T = float;
    static constexpr int W = 1;
};
template <>
struct Chunk<tmp::kScalar1> {
    using T = float;
    static constexpr int W = 1;
};

template <int OP>
__device__ __forceinline__ float apply1(float v, float a, float b) {
    if constexpr (OP == tmp::kAffine)
        return __builtin_fmaf(v, a, b);  // one rounding
    else if constexpr (OP == tmp::kScale)
        return a * v;                    // one IEEE multiply: -0 stays -0
    else
        return v;                        // register move: bits unchanged
}

template <int OP>
__device__ __forceinline__ float apply(float v, float a, float b) { return apply1<OP>(v, a, b); }
template <int OP>
__device__ __forceinline__ f4 apply(f4 v, float a, float b) {
    f4 r;
    r.x = apply1<OP>(v.x, a, b);
    r.y = apply1<OP>(v.y, a, b);
    r.z = apply1<OP>(v.z, a, b);
    r.w = apply1<OP>(v.w, a, b);
    return r;
}

// Channel op: per-column scale and bias of a chunk (the columns the chunk covers).  They are read
// by every row, so they are plain (cached) loads.  A missing scale is 1: fmaf(x, 1, b) is exactly
// the rounded sum x + b.
template <int ACC>
__device__ __forceinline__ typename Chunk<ACC>::T load_cvec(const float *v, int64_t col, int64_t live,
                                                             int vec16, float absent) {
    if constexpr (Chunk<ACC>::W == 1) {
        return v ? v[col] : absent;
    } else {
        f4 r = f4(absent);
        if (!v)
            return r;
        if (live >= 4 && vec16)
            return ld16(v + col);
        r.x = v[col];
        if (live > 1)
            r.y = v[col + 1];
        if (live > 2)
            r.z = v[col + 2];
        if (live > 3)
            r.w = v[col + 3];
        return r;
    }
}

// Flat channel view: element i of the chunk has channel (c0 + i) mod C (c0 < C).  With C % 4 == 0
// (and 16-byte aligned vectors) a 16-byte chunk's channels are one aligned vector chunk; otherwise
// they are gathered, wrapping at C.
template <int ACC>
__device__ __forceinline__ typename Chunk<ACC>::T load_cvec_flat(const float *v, uint32_t c0, uint32_t C,
                                                                  int vec16, float absent) {
    if constexpr (Chunk<ACC>::W == 1) {
        return v ? v[c0] : absent;
    } else {
        if (!v)
            return f4(absent);
        if (vec16)
            return ld16(v + c0);
        f4 r;
        uint32_t c = c0;
        r.x = v[c];
        c = c + 1 == C ? 0 : c + 1;
        r.y = v[c];
        c = c + 1 == C ? 0 : c + 1;
        r.z = v[c];
        c = c + 1 == C ? 0 : c + 1;
        r.w = v[c];
        return r;
    }
}

__device__ __forceinline__ float apply_channel(float v, float s, float b) { return __builtin_fmaf(v, s, b); }
__device__ __forceinline__ f4 apply_channel(f4 v, f4 s, f4 b) {
    f4 r;
    r.x = __builtin_fmaf(v.x, s.x, b.x);
    r.y = __builtin_fmaf(v.y, s.y, b.y);
    r.z = __builtin_fmaf(v.z, s.z, b.z);
    r.w = __builtin_fmaf(v.w, s.w, b.w);
    return r;
}

// Whole chunk at p, streamed (non-temporal: every element is touched exactly once).
template <int ACC>
__device__ __forceinline__ typename Chunk<ACC>::T load_chunk(const float *p, int64_t e) {
    if constexpr (ACC == tmp::kVec4) {
        return ld16_nt(p);
    } else if constexpr (ACC == tmp::kVec4Understated) {
        f4 r;
        r.x = ld4_nt(p);
        r.y = ld4_nt(p + e);
        r.z = ld4_nt(p + 2 * e);
        r.w = ld4_nt(p + 3 * e);
        return r;
    } else {
        return ld4_nt(p);
    }
}

template <int ACC>
__device__ __forceinline__ void store_chunk(float *p, typename Chunk<ACC>::T v, int64_t e) {
    if constexpr (ACC == tmp::kVec4) {
        st16_nt(p, v);
    } else if constexpr (ACC == tmp::kVec4Understated) {
        st4_nt(p, v.x);
        st4_nt(p + e, v.y);
        st4_nt(p + 2 * e, v.z);
        st4_nt(p + 3 * e, v.w);
    } else {
        st4_nt(p, v);
    }
}

// Chunk with n live elements (1 <= n): the first min(n, W) elements exist, the rest read as 0.
template <int ACC>
__device__ __forceinline__ typename Chunk<ACC>::T load_masked(const float *p, int64_t n, int64_t e) {
    if constexpr (Chunk<ACC>::W == 1) {
        return *p;
    } else {
        if (n >= 4)
            return load_chunk<ACC>(p, e);
        f4 r = {0.0f, 0.0f, 0.0f, 0.0f};
        r.x = p[0];
        if (n > 1)
            r.y = p[1];
        if (n > 2)
            r.z = p[2];
        return r;
    }
}

// Store only the first min(n, W) elements (1 <= n); the others are skipped.
template <int ACC>
__device__ __forceinline__ void store_masked(float *p, typename Chunk<ACC>::T v, int64_t n,
                                             int64_t e) {
    if constexpr (Chunk<ACC>::W == 1) {
        *p = v;
    } else {
        if (n >= 4) {
            store_chunk<ACC>(p, v, e);
            return;
        }
        p[0] = v.x;
        if (n > 1)
            p[1] = v.y;
        if (n > 2)
            p[2] = v.z;
    }
}

// Store of a whole chunk at byte `off` of a block addressed through a buffer resource, with the
// device-scope streaming policy.  Only for accesses whose every store instruction writes one
// contiguous run across the wave (16-byte or 4-byte chunks, lanes on consecutive chunks): the
// under-stated variant's four 4-byte stores per chunk each write every fourth word, and with
// this policy took the 1-D map from 5.2 to 9.7 us, so that variant keeps global stores.
template <int ACC>
__device__ __forceinline__ void store_seg(__amdgpu_buffer_rsrc_t r, int off, typename Chunk<ACC>::T v) {
    static_assert(ACC != tmp::kVec4Understated, "stores of every fourth word stay global");
    if constexpr (ACC == tmp::kVec4)
        st16_seg(r, off, v);
    else
        st4_seg(r, off, v);
}

// STREAM: every work item is one wave whose output is one contiguous block of
// tmp::kStreamSegmentBytes (one row segment, or whole rows of a view whose rows are contiguous;
// chosen on the host); whole items store it through a buffer resource with the device-scope
// streaming policy.
//
// SHARE (channel op, 4-byte chunks): every thread's U chunks lie in one column (the work item is no
// wider than the workgroup's chunks, G * VR <= threads; chunk q + u * threads then sits in the
// column of chunk q), so its channel vectors are read once, for the first chunk, and held in one
// register each (a live chunk implies its thread's first chunk is: rows grow with u).  Known when
// compiling, this keeps the scalar channel kernel's registers near the plain map's.
template <int OP, int ACC, bool ALIGNED, int U, bool GUARD, bool STREAM, bool SHARE>
__global__ __launch_bounds__(kMaxBlock) void map_tiles(MapArgs a) {
    using T = typename Chunk<ACC>::T;
    constexpr int W = Chunk<ACC>::W;
    const uint32_t t = threadIdx.x;
    const uint32_t vr_mask = (1u << a.log_vr) - 1u;
    const uint32_t gv_mask = (1u << a.log_gv) - 1u;
    const uint32_t strip_mask = (1u << a.log_strips) - 1u;
    const uint32_t chunks = 1u << (a.log_r + a.log_gv);  // chunks per work item
    const int64_t tm = int64_t(1) << a.log_tm, tn = int64_t(1) << a.log_tn;

    // The grid never exceeds the work count (the host caps it at nwork), so the first work item
    // needs no test; a grid smaller than the work loops.
    uint32_t w = blockIdx.x;
    do {
        // work item -> (tile row pm, row strip, tile group gi); tile groups vary fastest
        const uint32_t gi = w % a.groups_n;
        const uint32_t ps = w / a.groups_n;
        const uint32_t strip = ps & strip_mask;
        const uint32_t pm = ps >> a.log_strips;
        const int64_t row0 = (int64_t(pm) << a.log_tm) + (int64_t(strip) << a.log_r);
        const int64_t col0 = int64_t(gi) * a.group * tn;

        // Chunk q of the work item: row row0 + q / (G*VR); tile gq / VR of the group; chunk gq % VR.
        auto tile_col = [&](uint32_t q) { return col0 + int64_t((q & gv_mask) >> a.log_vr) * tn; };
        auto chunk_col = [&](uint32_t q) { return tile_col(q) + int64_t(q & vr_mask) * W; };
        auto chunk_row = [&](uint32_t q) { return row0 + int64_t(q >> a.log_gv); };

        // Channel vectors of the chunk at column col (live: its columns inside the tensor).  On a
        // flat view the channel of col is col mod C: col0 mod C = (gi mod C) * (columns per item
        // mod C) mod C (below C * C < 2^32), and col - col0 is below a work item's 4096 chunks.
        // A power-of-two C takes a mask instead (the 64-channel bias add paid 3% for the modulo).
        const bool chan_pow2 = (a.chan_n & (a.chan_n - 1)) == 0;
        auto chan_mod = [&](uint32_t v) {
            return chan_pow2 ? v & (a.chan_n - 1) : fast_mod(v, a.chan_c, a.chan_n);
        };
        uint32_t chan_base = 0;
        if constexpr (OP == tmp::kChannel) {
            if (a.chan_n != 0)
                chan_base = chan_mod(chan_mod(gi) * a.chan_step);
        }
        auto cvec = [&](const float *v, int64_t col, int64_t live, float absent) {
            if (a.chan_n != 0)
                return load_cvec_flat<ACC>(v, chan_mod(chan_base + uint32_t(col - col0)), a.chan_n, a.cvec16,
                                           absent);
            return load_cvec<ACC>(v, col, live, a.cvec16, absent);
        };
        constexpr int CV = SHARE ? 1 : U;  // channel vector registers per thread

        // Whole tiles (every tile, when the promise was checked; otherwise this work item's tiles
        // all lie inside the tensor): no masks.
        const bool item_whole = ALIGNED || ((int64_t(pm) + 1) * tm <= a.M &&
                                            col0 + int64_t(a.group) * tn <= a.N);
        if constexpr (STREAM) {
            static_assert(!GUARD, "a stream item is exactly one wave's chunks");
        }
        if (item_whole) {
            if constexpr (STREAM) {
                // The item's output block starts at (row0, col0); chunk q lies 4 W q bytes into it.
                const __amdgpu_buffer_rsrc_t ry = segment_rsrc(a.y + row0 * a.ldy + col0, tmp::kStreamSegmentBytes);
                T v[U], cs[CV], cb[CV];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t q = t + (uint32_t(u) << a.log_bs);
                    const int64_t row = chunk_row(q), col = chunk_col(q);
                    v[u] = load_chunk<ACC>(a.x + row * a.ldx + col, a.estep);
                    if constexpr (OP == tmp::kChannel) {
                        if (!SHARE || u == 0) {
                            cs[u] = cvec(a.scale, col, W, 1.0f);
                            cb[u] = cvec(a.bias, col, W, 0.0f);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t q = t + (uint32_t(u) << a.log_bs);
                    T r;
                    if constexpr (OP == tmp::kChannel)
                        r = apply_channel(v[u], cs[SHARE ? 0 : u], cb[SHARE ? 0 : u]);
                    else
                        r = apply<OP>(v[u], a.alpha, a.beta);
                    store_seg<ACC>(ry, int(q) * (4 * W), r);
                }
            } else {
                T v[U], cs[CV], cb[CV];
                int64_t yo[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t q = t + (uint32_t(u) << a.log_bs);
                    const int64_t row = chunk_row(q), col = chunk_col(q);
                    yo[u] = row * a.ldy + col;
                    if (!GUARD || q < chunks) {
                        v[u] = load_chunk<ACC>(a.x + row * a.ldx + col, a.estep);
                        if constexpr (OP == tmp::kChannel) {
                            if (!SHARE || u == 0) {
                                cs[u] = cvec(a.scale, col, W, 1.0f);
                                cb[u] = cvec(a.bias, col, W, 0.0f);
                            }
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!GUARD || t + (uint32_t(u) << a.log_bs) < chunks) {
                        T r;
                        if constexpr (OP == tmp::kChannel)
                            r = apply_channel(v[u], cs[SHARE ? 0 : u], cb[SHARE ? 0 : u]);
                        else
                            r = apply<OP>(v[u], a.alpha, a.beta);
                        store_chunk<ACC>(a.y + yo[u], r, a.estep);
                    }
                }
            }
        } else if constexpr (!ALIGNED) {
            // Edge tiles: an element past the tensor reads as 0 and its store is skipped; a chunk
            // of a whole tile still moves unmasked.
            T v[U], cs[CV], cb[CV];
            bool on[U], whole[U];
            int64_t live[U], yo[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t q = t + (uint32_t(u) << a.log_bs);
                const uint32_t pn = gi * a.group + ((q & gv_mask) >> a.log_vr);
                const int64_t row = chunk_row(q), col = chunk_col(q);
                live[u] = a.N - col;  // elements of the chunk inside the tensor
                whole[u] = row < a.M && tile_col(q) + tn <= a.N;
                on[u] = q < chunks && pn < a.tiles_n && row < a.M && live[u] > 0;
                yo[u] = row * a.ldy + col;
                v[u] = T(0.0f);  // a masked element reads as 0
                if (on[u]) {
                    const float *xp = a.x + row * a.ldx + col;
                    // (A live 4-byte chunk is always whole: one streamed access, whatever its tile.)
                    v[u] = W == 1 || whole[u] ? load_chunk<ACC>(xp, a.estep)
                                              : load_masked<ACC>(xp, live[u], a.estep);
                    if constexpr (OP == tmp::kChannel) {
                        if (!SHARE || u == 0) {
                            cs[u] = cvec(a.scale, col, live[u], 1.0f);
                            cb[u] = cvec(a.bias, col, live[u], 0.0f);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (on[u]) {  // a masked store is skipped
                    T r;
                    if constexpr (OP == tmp::kChannel)
                        r = apply_channel(v[u], cs[SHARE ? 0 : u], cb[SHARE ? 0 : u]);
                    else
                        r = apply<OP>(v[u], a.alpha, a.beta);
                    if (W == 1 || whole[u])
                        store_chunk<ACC>(a.y + yo[u], r, a.estep);
                    else
                        store_masked<ACC>(a.y + yo[u], r, live[u], a.estep);
                }
            }
        }
        w += gridDim.x;
    } while (w < a.nwork);
}

template <int OP, int ACC, bool GUARD, bool SHARE>
const void *pick_aligned(const tmp::MapPlan &p) {
    constexpr int U = ACC == tmp::kScalar ? tmp::kScalarChunksPerThread : 1;
    return p.aligned ? reinterpret_cast<const void *>(&map_tiles<OP, ACC, true, U, GUARD, false, SHARE>)
                     : reinterpret_cast<const void *>(&map_tiles<OP, ACC, false, U, GUARD, false, SHARE>);
}

template <int OP, int ACC, bool SHARE>
const void *pick_guard(const tmp::MapPlan &p) {
    constexpr int U = ACC == tmp::kScalar ? tmp::kScalarChunksPerThread : 1;
    if constexpr (ACC != tmp::kVec4Understated) {
        if (p.stream)
            return p.aligned ? reinterpret_cast<const void *>(&map_tiles<OP, ACC, true, U, false, true, SHARE>)
                             : reinterpret_cast<const void *>(&map_tiles<OP, ACC, false, U, false, true, SHARE>);
    }
    return p.guard ? pick_aligned<OP, ACC, true, SHARE>(p) : pick_aligned<OP, ACC, false, SHARE>(p);
}

template <int OP>
const void *pick_access(const tmp::MapPlan &p) {
    switch (p.access) {
    case tmp::kScalar:
        if constexpr (OP == tmp::kChannel) {
            if (p.share)
                return pick_guard<OP, tmp::kScalar, true>(p);
        }
        return pick_guard<OP, tmp::kScalar, false>(p);
    case tmp::kScalar1: return pick_guard<OP, tmp::kScalar1, false>(p);
    case tmp::kVec4Understated: return pick_guard<OP, tmp::kVec4Understated, false>(p);
    default: return pick_guard<OP, tmp::kVec4, false>(p);
    }
}

const void *pick(const tmp::MapPlan &p) {
    switch (p.op) {
    case tmp::kAffine: return pick_access<tmp::kAffine>(p);
    case tmp::kScale: return pick_access<tmp::kScale>(p);
    case tmp::kCopy: return pick_access<tmp::kCopy>(p);
    default: return pick_access<tmp::kChannel>(p);
    }
}

}  // namespace

hipError_t launch_map(const tmp::MapPlan &p, hipStream_t stream) {
    if (p.flat || p.rows)
        return launch_map_flat(p, stream);
    MapArgs a;
    a.x = p.x;
    a.y = p.y;
    a.ldx = p.ldx;
    a.ldy = p.ldy;
    a.M = p.M;
    a.N = p.N;
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.tiles_n = p.tiles_n;
    a.group = p.group;
    a.groups_n = p.groups_n;
    a.nwork = p.nwork;
    a.log_tm = p.log_tm;
    a.log_tn = p.log_tn;
    a.log_vr = p.log_vr;
    a.log_gv = p.log_gv;
    a.log_r = p.log_r;
    a.log_strips = p.log_strips;
    a.log_bs = p.log_bs;
    a.scale = p.scale;
    a.bias = p.bias;
    a.cvec16 = p.cvec16 ? 1 : 0;
    a.chan_n = p.chan_n;
    a.chan_step = p.chan_step;
    a.chan_c = p.chan.c;
    a.estep = 1;
    void *args[] = {&a};
    return hipLaunchKernel(pick(p), dim3(p.grid), dim3(1u << p.log_bs), args, 0, stream);
}

}  // namespace tmk
