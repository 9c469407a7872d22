// map.hip -- tiled element-wise maps for gfx950: y = fmaf(x, alpha, beta), y = alpha * x and the
// bitwise copy, over TM x TN tiles of row-major f32 views.
//
// Sources (web pages): Phobos docs "@aligned" ("A minimal kernel", "What it changes"); Phobos docs
// "Slicing, bounds and masking" ("Masking", "Promising whole tiles with @aligned"); Mojo GPU
// puzzle 35 "Aligned Load & Store" ("The exercise", "Solution": the scalar, under-aligned and
// aligned variants); teenygrad "Memory Coalescing and Tensor Layout" ("Coalescing": consecutive
// lanes take consecutive addresses).
//
// Mapping.  A tile holds TM*TN/W chunks (W = 4 elements for the vector variants, 1 for scalar),
// numbered along its rows.  One workgroup takes one block of BS = min(chunks, 1024) consecutive
// chunks of one tile (a tile of more than 1024 chunks spreads over several workgroups; one smaller
// than a wave leaves lanes idle) and every thread moves exactly one chunk: the lane-varying term of
// each address is the chunk index along a row, so a wave reads 64 consecutive chunks (1 KiB of
// 16-byte chunks) whenever the tile row is that wide.  Work items run row-major over tiles (pn
// fastest), so workgroups dispatched together cover neighbouring tiles of the same rows; a grid
// smaller than the work count loops.  Whole chunks move with the non-temporal hint.  On gfx950
// this one-chunk-per-thread shape with 1024-thread workgroups streamed faster than giving each
// thread several chunks or several tiles, and faster than remapping workgroups across XCDs.
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
    uint32_t tiles_n;   // tiles along N
    uint32_t slots;     // chunks per tile
    uint32_t nwork;     // workgroup work items: tiles * 2^log_sub
    int log_tm, log_tn, log_vr;
    int log_bs;         // threads per workgroup = chunks per work item
    int log_sub;        // work items per tile
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

template <int OP, int ACC, bool ALIGNED>
__global__ __launch_bounds__(kMaxBlock) void map_tiles(MapArgs a) {
    using T = typename Chunk<ACC>::T;
    constexpr int W = Chunk<ACC>::W;
    const uint32_t t = threadIdx.x;
    const uint32_t vr_mask = (1u << a.log_vr) - 1u;
    const uint32_t sub_mask = (1u << a.log_sub) - 1u;

    for (uint32_t w = blockIdx.x; w < a.nwork; w += gridDim.x) {
        const uint32_t tile = w >> a.log_sub;            // tile id, row-major over tiles
        const uint32_t s = ((w & sub_mask) << a.log_bs) + t;  // this thread's chunk in the tile
        const uint32_t pm = tile / a.tiles_n;            // tile (pm, pn): pm on rows, pn on columns
        const uint32_t pn = tile - pm * a.tiles_n;
        const int64_t row0 = int64_t(pm) << a.log_tm;
        const int64_t col0 = int64_t(pn) << a.log_tn;
        const uint32_t r = s >> a.log_vr;                // row within the tile
        const uint32_t c = (s & vr_mask) * W;            // first column of the chunk within the tile
        const float *xp = a.x + (row0 + r) * a.ldx + col0 + c;
        float *yp = a.y + (row0 + r) * a.ldy + col0 + c;
        const bool slot_ok = s < a.slots;                // false only for tiles smaller than a wave

        bool whole = true;
        int64_t rows_live = 0, cols_live = 0;
        if constexpr (!ALIGNED) {
            rows_live = a.M - row0;
            cols_live = a.N - col0;
            whole = rows_live >= (int64_t(1) << a.log_tm) && cols_live >= (int64_t(1) << a.log_tn);
        }
        if (whole) {
            // Unmasked: the chunk exists.
            if (slot_ok)
                store_chunk<ACC>(yp, apply<OP>(load_chunk<ACC>(xp, a.estep), a.alpha, a.beta), a.estep);
        } else if constexpr (!ALIGNED) {
            // Edge tile: elements past the tensor read as 0 and are never stored.
            const bool live = slot_ok && int64_t(r) < rows_live && int64_t(c) < cols_live;
            T v = T(0.0f);
            if (live)
                v = load_masked<ACC>(xp, cols_live - c, a.estep);
            if (live)
                store_masked<ACC>(yp, apply<OP>(v, a.alpha, a.beta), cols_live - c, a.estep);
        }
    }
}

template <int OP, int ACC>
const void *pick_aligned(const tmp::MapPlan &p) {
    return p.aligned ? reinterpret_cast<const void *>(&map_tiles<OP, ACC, true>)
                     : reinterpret_cast<const void *>(&map_tiles<OP, ACC, false>);
}

template <int OP>
const void *pick_access(const tmp::MapPlan &p) {
    switch (p.access) {
    case tmp::kScalar: return pick_aligned<OP, tmp::kScalar>(p);
    case tmp::kVec4Understated: return pick_aligned<OP, tmp::kVec4Understated>(p);
    default: return pick_aligned<OP, tmp::kVec4>(p);
    }
}

const void *pick(const tmp::MapPlan &p) {
    switch (p.op) {
    case tmp::kAffine: return pick_access<tmp::kAffine>(p);
    case tmp::kScale: return pick_access<tmp::kScale>(p);
    default: return pick_access<tmp::kCopy>(p);
    }
}

}  // namespace

hipError_t launch_map(const tmp::MapPlan &p, hipStream_t stream) {
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
    a.slots = p.slots;
    a.nwork = p.nwork;
    a.log_tm = p.log_tm;
    a.log_tn = p.log_tn;
    a.log_vr = p.log_vr;
    a.log_bs = p.log_bs;
    a.log_sub = p.log_sub;
    a.estep = 1;
    void *args[] = {&a};
    return hipLaunchKernel(pick(p), dim3(p.grid), dim3(1u << p.log_bs), args, 0, stream);
}

}  // namespace tmk
