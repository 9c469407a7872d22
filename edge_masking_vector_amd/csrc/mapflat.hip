// mapflat.hip -- the element-wise maps over one contiguous row, cut into 1 KiB work items: the
// case the tile scheduler reaches for every view whose rows are contiguous in both tensors (row
// stride N: the M x N elements are one row of M*N) and whose bases sit on 128-byte lines, with the
// affine map, the scale or the copy moved in 16-byte chunks or in 4-byte elements (map_flat).
// Also here: padded rows as one span of 1 KiB items on y's 1 KiB grid, columns past N masked per
// chunk (map_rows, map_rows_diff, map_rows_shift, map_rows_channel), and one contiguous row that
// map_flat cannot take, x at another 4-byte phase or a base off the line grid (map_flat_shift).
//
// Sources (web pages): Phobos docs "@aligned" ("A minimal kernel": the scale; "What it changes":
// no masks, 16-byte rows); Phobos docs "Slicing, bounds and masking" ("Masking": elements past the
// end read as 0 and are not stored; "Promising whole tiles with @aligned": the copy); Mojo GPU
// puzzle 35 "Aligned Load & Store" ("The exercise": a*2 + 1 over 1M elements); teenygrad "Memory
// Coalescing and Tensor Layout" ("Coalescing": lane t takes the t-th consecutive address).
//
// Why a kernel of its own.  These work items are short (one wave loads 1 KiB and stores 1 KiB),
// there are many of them (65,536 for a 4096 x 4096 map), and the HBM stream is only kept busy by
// how fast finished waves are replaced: on gfx950 an empty kernel of 65,536 one-wave workgroups
// already takes 14.7 us, and everything a wave does before its load lengthens its life.  The
// general tile kernel (map.hip) spends about 80 instructions and five scalar loads of a 400-byte
// argument block on tile arithmetic before its load; this one takes its six arguments preloaded
// into scalar registers (this file is compiled with kernel-argument preloading) and computes one
// address.  Measured on the 4096 x 4096 scale (kernel trace, 1 GiB of rotating buffers): 21.48 us
// for the general kernel, 20.84 us for this one.
//
// Work item w covers elements [256 w, 256 w + 256) of the row.  16-byte chunks: lane t of a wave
// moves elements 4t .. 4t + 3 of the item.  4-byte elements: lane t of a wave moves elements t,
// t + 64, t + 128 and t + 192, or (one element per thread) thread t of 256 moves element t;
// consecutive lanes take consecutive addresses either way.  Loads carry the non-temporal hint (touched
// once); a whole item's output, one contiguous 1 KiB, is stored through a buffer resource spanning
// exactly that block with the device-scope cache policy.  Only the last item can be ragged (the
// row's end): there an element past the end is neither read nor stored (what a masked element
// would read, 0, never reaches an output of a map).
#include "device.hpp"
#include "launch.h"

namespace tmk {
namespace {

constexpr int kItemFloats = 256;  // 1 KiB: one wave of 16-byte chunks
constexpr int kFlatStorePolicy = 16;  // sc1: device scope

template <int OP>
__device__ __forceinline__ float op1(float v, float a, float b) {
    if constexpr (OP == tmp::kAffine)
        return __builtin_fmaf(v, a, b);  // one rounding
    else if constexpr (OP == tmp::kScale)
        return a * v;                    // one IEEE multiply: -0 stays -0
    else
        return v;                        // register move: bits unchanged
}

template <int OP>
__device__ __forceinline__ f4 op4(f4 v, float a, float b) {
    f4 r;
    r.x = op1<OP>(v.x, a, b);
    r.y = op1<OP>(v.y, a, b);
    r.z = op1<OP>(v.z, a, b);
    r.w = op1<OP>(v.w, a, b);
    return r;
}

// How a work item's 256 elements are spread over the threads of its workgroup.
enum FlatMode {
    kChunk16 = 0,  // 64 threads, one 16-byte chunk each: lane t moves elements 4t .. 4t + 3
    kFour4 = 1,    // 64 threads, four 4-byte elements each: lane t moves t, t + 64, t + 128, t + 192
    kOne4 = 2      // 256 threads, one element each (the one-element-per-thread scalar variant)
};

template <int MODE>
constexpr int flat_threads() { return MODE == kOne4 ? 256 : 64; }

// Items [0, nwhole) are whole; when tail > 0, item nwhole holds the row's last `tail` elements
// (1 .. 255).  The host launches at most nwhole + (tail > 0) workgroups; a smaller grid loops.
template <int OP, int MODE>
__global__ __launch_bounds__(flat_threads<MODE>()) void map_flat(const float *__restrict__ x,
                                                                 float *__restrict__ y, float alpha,
                                                                 float beta, uint32_t nwhole,
                                                                 uint32_t tail) {
    const uint32_t t = threadIdx.x;
    uint32_t w = blockIdx.x;
    for (; w < nwhole; w += gridDim.x) {
        const size_t base = size_t(w) * kItemFloats;
        const __amdgpu_buffer_rsrc_t ry = segment_rsrc(y + base, kItemFloats * 4);
        if constexpr (MODE == kChunk16) {
            const f4 v = ld16_nt(x + base + 4 * t);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, op4<OP>(v, alpha, beta)), ry,
                                                   int(t) * 16, 0, kFlatStorePolicy);
        } else if constexpr (MODE == kFour4) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = ld4_nt(x + base + t + 64 * u);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, op1<OP>(v[u], alpha, beta)),
                                                      ry, int(t + 64 * u) * 4, 0, kFlatStorePolicy);
        } else {
            const float v = ld4_nt(x + base + t);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, op1<OP>(v, alpha, beta)), ry,
                                                  int(t) * 4, 0, kFlatStorePolicy);
        }
    }
    if (w != nwhole || tail == 0)
        return;
    // The row's ragged end, item nwhole: an element past the end is neither read nor stored.
    const float *xp = x + size_t(w) * kItemFloats;
    float *yp = y + size_t(w) * kItemFloats;
    if constexpr (MODE == kChunk16) {
        const int live = int(tail) - 4 * int(t);  // elements of chunk t inside the row
        if (live >= 4) {
            st16_nt(yp + 4 * t, op4<OP>(ld16_nt(xp + 4 * t), alpha, beta));
        } else if (live > 0) {
            yp[4 * t] = op1<OP>(xp[4 * t], alpha, beta);
            if (live > 1)
                yp[4 * t + 1] = op1<OP>(xp[4 * t + 1], alpha, beta);
            if (live > 2)
                yp[4 * t + 2] = op1<OP>(xp[4 * t + 2], alpha, beta);
        }
    } else if constexpr (MODE == kFour4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t e = t + 64 * u;
            if (e < tail)
                yp[e] = op1<OP>(xp[e], alpha, beta);
        }
    } else {
        if (t < tail)
            yp[t] = op1<OP>(xp[t], alpha, beta);
    }
}

// Padded rows in one span.  Element f of the span (f = 0 at y[0]) is row f / ld, column f % ld
// (ld: y's row stride), and live when that column is below N (the padding between rows is never
// stored).  Item w is the 1 KiB block of y's 1 KiB grid that starts 256 w - head floats from
// y[0]; lane t moves the 16-byte chunk of span elements q .. q + 3, q = 256 w + 4 t - head.  x's
// chunk for it starts at x index q + r dld (r: q's row; dld = ldx - ldy, 0 for one stride): on the
// 16-byte grid when x and y share their 16-byte phase, else (SHIFT) a 16-byte load from a 4-byte
// aligned address.  A chunk whose four elements are live is stored whole through a buffer
// resource spanning the block; at a row's end or the span's ends the live elements are stored one
// by one.  Every load holds a live element: loads are clamped to the chunks that hold y[0] and the
// span's last element (SHIFT: those two chunks load their live elements one by one), and with a
// line or more of padding (WIDE) a chunk wholly inside the padding between two rows loads the
// row's last live chunk instead (already read by another lane), so no line of padding alone is
// fetched, and a wave wholly inside the padding exits.  (Under a line of padding every line holds
// live elements, and the load is issued before the column is known.)  With different strides
// (DIFF) a chunk that crosses a row's end takes the next row's elements from a second load.
// Columns (and rows) come from a multiply-high division by ld (rows of at least 64 floats: at
// most one row boundary per chunk).
// The channel op (OP = kChannel) takes element (row, column c)'s channel c: y = fmaf(x, scale[c],
// bias[c]), scale 1 when absent; a whole chunk's four channels are one 16-byte load of each vector
// when cvec16 (both vectors 16-byte aligned and every chunk starting on a column divisible by 4).
template <int OP, bool WIDE, bool DIFF, bool SHIFT = false>
__device__ __forceinline__ void rows_body(const float *__restrict__ x, float *__restrict__ y, float alpha, float beta,
                                          uint32_t nwork, uint32_t head, uint32_t span, uint32_t ld, uint32_t N,
                                          uint64_t c_ld, const float *__restrict__ scale,
                                          const float *__restrict__ bias, uint32_t cvec16, int32_t dld,
                                          int32_t x_last) {
    const int t = threadIdx.x;
    const int32_t q_first = -int32_t(head & 3u);                         // the chunk holding y[0]
    const int32_t q_last = int32_t(span - 1) - int32_t((span - 1 + head) & 3u);  // ... the last element
    for (uint32_t w = blockIdx.x; w < nwork; w += gridDim.x) {
        const int32_t q = int32_t(w * 256u + 4u * t) - int32_t(head);
        f4 xv, xn;  // x's chunk for the span elements q .. q + 3; (DIFF) the next row's part
        if constexpr (!WIDE && !DIFF) {
            xv = ld16_nt(x + (q < q_first ? q_first : (q > q_last ? q_last : q)));
        }
        uint32_t r = 0, c = 0;  // row and column of element q (q >= 0)
        if (q > 0) {
            if constexpr (DIFF) {
                r = fast_div(uint32_t(q), c_ld, ld);
                c = uint32_t(q) - r * ld;
            } else {
                c = fast_mod(uint32_t(q), c_ld, ld);
            }
        }
        if constexpr (WIDE || DIFF) {
            // a wave whose chunks all lie in the padding between two rows (or past the span's
            // ends) neither loads nor stores
            const bool some_live = q + 3 >= 0 && q < int32_t(span) && (q < 0 || c < N || c + 3 >= ld);
            if (__builtin_amdgcn_ballot_w64(some_live) == 0)
                continue;
            // x index of the chunk: the span's own index shifted by dld per row (DIFF); a chunk
            // wholly inside y's padding loads the row's last live chunk; the span's ends clamp
            int32_t qa = q;
            if (q >= 0 && c >= N && c + 3 < ld) {
                const int32_t last = q - int32_t(c) + int32_t(N) - 1;
                qa = last - int32_t((uint32_t(last) + head) & 3u);
            }
            int32_t xa = DIFF ? qa + int32_t(r) * dld : qa;
            if constexpr (!SHIFT)
                xa = q < q_first ? q_first : (q > q_last ? (DIFF ? x_last : q_last) : xa);
            if constexpr (SHIFT) {
                // x at another 4-byte phase than y: x's chunk is the 16 bytes from x + xa, 4-byte
                // aligned.  The span's two end chunks (some element outside the span) load their
                // live elements one by one, so that no load leaves the view.
                const bool cross = q >= 0 && c + 3 >= ld && int64_t(q) - c + ld < int64_t(span);
                const int32_t xb = cross ? xa + dld : xa;
                if (cross && c >= N)
                    xa = xb;
                if (q >= 0 && q + 3 < int32_t(span)) {
                    xv = ld16u_nt(x + xa);
                    xn = xv;
                    if (dld != 0 && __builtin_amdgcn_ballot_w64(cross) != 0)
                        xn = ld16u_nt(x + xb);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int32_t f = q + i;
                        const uint32_t ci = q >= 0 ? c + i : uint32_t(f);
                        const bool nxt = q >= 0 && ci >= ld;
                        const uint32_t cl = nxt ? ci - ld : ci;
                        const int32_t row = int32_t(r) + (nxt ? 1 : 0);
                        xv[i] = f >= 0 && f < int32_t(span) && cl < N ? x[f + row * dld] : 0.0f;
                    }
                    xn = xv;
                }
            } else if constexpr (DIFF) {
                // elements past the row's end belong to the next row, dld further on in x; when
                // none of the chunk's elements is live in its own row, both loads take the next
                // row's chunk (x's padding past the row may hold no live element in its line)
                const bool cross = q >= 0 && c + 3 >= ld && int64_t(q) - c + ld < int64_t(span);
                const int32_t xb = cross ? xa + dld : xa;
                if (cross && c >= N)
                    xa = xb;
                xv = ld16_nt(x + xa);
                // the second load only in waves where a chunk crosses a row's end (a wave-uniform
                // test; chunks cross row ends only when y's rows start off the 16-byte grid)
                xn = xv;
                if (__builtin_amdgcn_ballot_w64(cross) != 0)
                    xn = ld16_nt(x + xb);
            } else {
                xv = ld16_nt(x + xa);
            }
        }
        const __amdgpu_buffer_rsrc_t ry = segment_rsrc(y + (int64_t(w) * 256 - head), kItemFloats * 4);
        const bool whole = q >= 0 && uint32_t(q) + 3 < span && c + 3 < N;
        uint32_t col[4];  // the chunk's columns (q < 0: f < 4, row 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ci = q >= 0 ? c + i : uint32_t(q + i);
            if constexpr (DIFF) {
                if (q >= 0 && ci >= ld)
                    xv[i] = xn[i];
            }
            col[i] = ci >= ld ? ci - ld : ci;
        }
        // The result of every lane is computed before the stores, whole or not: with the
        // arithmetic inside the masked branch, each lane there waited for its first element's
        // store before the next (the 4100 x 1000 map at row stride 1001: 8.1 against 7.5 us).
        f4 v;
        if constexpr (OP == tmp::kChannel) {
            f4 sv = f4(1.0f), bv;
            if (cvec16 && whole) {
                bv = ld16(bias + c);
                if (scale)
                    sv = ld16(scale + c);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t cc = col[i] < N ? col[i] : N - 1;  // a dead element reads a live channel
                    bv[i] = bias[cc];
                    if (scale)
                        sv[i] = scale[cc];
                }
            }
            v.x = __builtin_fmaf(xv.x, sv.x, bv.x);
            v.y = __builtin_fmaf(xv.y, sv.y, bv.y);
            v.z = __builtin_fmaf(xv.z, sv.z, bv.z);
            v.w = __builtin_fmaf(xv.w, sv.w, bv.w);
        } else {
            v = op4<OP>(xv, alpha, beta);
        }
        if (whole) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), ry, t * 16, 0, kFlatStorePolicy);
        } else {
            // the same buffer and policy as the whole chunks, which write the rest of these lines
            // (with plain stores here a 4100 x 1000 map at row stride 1001 took 13.6 us, against
            // 7.5 us)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t f = q + i;
                const float e = v[i];  // (a bit cast of the vector element itself stored element 0)
                if (f >= 0 && uint32_t(f) < span && col[i] < N)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), ry, (t * 4 + i) * 4, 0, kFlatStorePolicy);
            }
        }
    }
}

// The maps over one stride take ten arguments (the channel vectors and the second stride would
// add to every dispatch's argument block: three more cost these kernels 1-1.5%); the channel op
// and different strides have kernels of their own.
template <int OP, bool WIDE>
__global__ __launch_bounds__(64) void map_rows(const float *__restrict__ x, float *__restrict__ y, float alpha,
                                               float beta, uint32_t nwork, uint32_t head, uint32_t span,
                                               uint32_t ld, uint32_t N, uint64_t c_ld) {
    rows_body<OP, WIDE, false>(x, y, alpha, beta, nwork, head, span, ld, N, c_ld, nullptr, nullptr, 0u, 0, 0);
}

// One contiguous row (contiguous rows folded into one) that the flat kernel cannot take: x at
// another 4-byte phase than y, or a base off the 128-byte line grid.  Items on y's 1 KiB grid
// (item 0 starting `head` floats before y[0]); lane t moves the 16 bytes of y from element
// q = 256 w + 4 t - head, x's as one 4-byte aligned 16-byte load.  The row's two end chunks
// (some element outside it) move their elements one by one, so that no access leaves the row.
template <int OP>
__global__ __launch_bounds__(64) void map_flat_shift(const float *__restrict__ x, float *__restrict__ y, float alpha,
                                                     float beta, uint32_t nwork, uint32_t head, uint32_t n) {
    const int t = threadIdx.x;
    for (uint32_t w = blockIdx.x; w < nwork; w += gridDim.x) {
        const int32_t q = int32_t(w * 256u + 4u * t) - int32_t(head);
        const __amdgpu_buffer_rsrc_t ry = segment_rsrc(y + (int64_t(w) * 256 - head), kItemFloats * 4);
        if (q >= 0 && q + 4 <= int32_t(n)) {
            const f4 v = op4<OP>(ld16u_nt(x + q), alpha, beta);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), ry, t * 16, 0, kFlatStorePolicy);
        } else {
            f4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t f = q + i;
                v[i] = f >= 0 && f < int32_t(n) ? op1<OP>(x[f], alpha, beta) : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t f = q + i;
                const float e = v[i];
                if (f >= 0 && f < int32_t(n))
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), ry, (t * 4 + i) * 4, 0, kFlatStorePolicy);
            }
        }
    }
}

// x at another 4-byte phase than y (bases not a multiple of 16 bytes apart, or strides not a
// multiple of 4 floats apart; dld = ldx - ldy, 0 for one stride): 4-byte aligned 16-byte loads.
template <int OP>
__global__ __launch_bounds__(64) void map_rows_shift(const float *__restrict__ x, float *__restrict__ y, float alpha,
                                                     float beta, uint32_t nwork, uint32_t head, uint32_t span,
                                                     uint32_t ld, uint32_t N, uint64_t c_ld, int32_t dld) {
    rows_body<OP, true, true, true>(x, y, alpha, beta, nwork, head, span, ld, N, c_ld, nullptr, nullptr, 0u, dld, 0);
}

// Different strides (dld = ldx - ldy, a multiple of 4; x_last: x's index of the span's last chunk).
template <int OP>
__global__ __launch_bounds__(64) void map_rows_diff(const float *__restrict__ x, float *__restrict__ y, float alpha,
                                                    float beta, uint32_t nwork, uint32_t head, uint32_t span,
                                                    uint32_t ld, uint32_t N, uint64_t c_ld, int32_t dld,
                                                    int32_t x_last) {
    rows_body<OP, true, true>(x, y, alpha, beta, nwork, head, span, ld, N, c_ld, nullptr, nullptr, 0u, dld, x_last);
}

template <bool WIDE, bool DIFF, bool SHIFT>
__global__ __launch_bounds__(64) void map_rows_channel(const float *__restrict__ x, float *__restrict__ y,
                                                       uint32_t nwork, uint32_t head, uint32_t span, uint32_t ld,
                                                       uint32_t N, uint64_t c_ld, const float *__restrict__ scale,
                                                       const float *__restrict__ bias, uint32_t cvec16, int32_t dld,
                                                       int32_t x_last) {
    rows_body<tmp::kChannel, WIDE, DIFF, SHIFT>(x, y, 0.0f, 0.0f, nwork, head, span, ld, N, c_ld, scale, bias, cvec16,
                                               dld, x_last);
}

template <bool WIDE>
const void *pick_rows(int op) {
    return op == tmp::kAffine  ? reinterpret_cast<const void *>(&map_rows<tmp::kAffine, WIDE>)
           : op == tmp::kScale ? reinterpret_cast<const void *>(&map_rows<tmp::kScale, WIDE>)
                               : reinterpret_cast<const void *>(&map_rows<tmp::kCopy, WIDE>);
}

template <int OP>
const void *pick_flat(int mode) {
    switch (mode) {
    case kChunk16: return reinterpret_cast<const void *>(&map_flat<OP, kChunk16>);
    case kFour4: return reinterpret_cast<const void *>(&map_flat<OP, kFour4>);
    default: return reinterpret_cast<const void *>(&map_flat<OP, kOne4>);
    }
}

}  // namespace

hipError_t launch_map_flat(const tmp::MapPlan &p, hipStream_t stream) {
    const float *x = p.x;
    float *y = p.y;
    float alpha = p.alpha, beta = p.beta;
    if (p.rows) {
        uint32_t nwork = p.nwork, head = p.head, span = p.span, ld = p.ld_div.d, N = static_cast<uint32_t>(p.N);
        uint64_t c_ld = p.ld_div.c;
        int32_t dld = static_cast<int32_t>(p.ldx - p.ldy), x_last = p.x_last;
        const bool diff = dld != 0;
        const bool wide = p.ldy - p.N >= 32;
        if (p.op == tmp::kChannel) {
            const float *scale = p.scale, *bias = p.bias;
            uint32_t cvec16 = p.cvec16 ? 1u : 0u;
            void *cargs[] = {&x, &y, &nwork, &head, &span, &ld, &N, &c_ld, &scale, &bias, &cvec16, &dld, &x_last};
            const void *cfn = p.shift ? reinterpret_cast<const void *>(&map_rows_channel<true, true, true>)
                              : diff  ? reinterpret_cast<const void *>(&map_rows_channel<true, true, false>)
                              : wide  ? reinterpret_cast<const void *>(&map_rows_channel<true, false, false>)
                                      : reinterpret_cast<const void *>(&map_rows_channel<false, false, false>);
            return hipLaunchKernel(cfn, dim3(p.grid), dim3(64), cargs, 0, stream);
        }
        if (p.M == 1) {
            void *fargs[] = {&x, &y, &alpha, &beta, &nwork, &head, &span};
            const void *ffn = p.op == tmp::kAffine  ? reinterpret_cast<const void *>(&map_flat_shift<tmp::kAffine>)
                              : p.op == tmp::kScale ? reinterpret_cast<const void *>(&map_flat_shift<tmp::kScale>)
                                                    : reinterpret_cast<const void *>(&map_flat_shift<tmp::kCopy>);
            return hipLaunchKernel(ffn, dim3(p.grid), dim3(64), fargs, 0, stream);
        }
        if (p.shift) {
            void *sargs[] = {&x, &y, &alpha, &beta, &nwork, &head, &span, &ld, &N, &c_ld, &dld};
            const void *sfn = p.op == tmp::kAffine  ? reinterpret_cast<const void *>(&map_rows_shift<tmp::kAffine>)
                              : p.op == tmp::kScale ? reinterpret_cast<const void *>(&map_rows_shift<tmp::kScale>)
                                                    : reinterpret_cast<const void *>(&map_rows_shift<tmp::kCopy>);
            return hipLaunchKernel(sfn, dim3(p.grid), dim3(64), sargs, 0, stream);
        }
        if (diff) {
            void *dargs[] = {&x, &y, &alpha, &beta, &nwork, &head, &span, &ld, &N, &c_ld, &dld, &x_last};
            const void *dfn = p.op == tmp::kAffine  ? reinterpret_cast<const void *>(&map_rows_diff<tmp::kAffine>)
                              : p.op == tmp::kScale ? reinterpret_cast<const void *>(&map_rows_diff<tmp::kScale>)
                                                    : reinterpret_cast<const void *>(&map_rows_diff<tmp::kCopy>);
            return hipLaunchKernel(dfn, dim3(p.grid), dim3(64), dargs, 0, stream);
        }
        void *args[] = {&x, &y, &alpha, &beta, &nwork, &head, &span, &ld, &N, &c_ld};
        const void *fn = wide ? pick_rows<true>(p.op) : pick_rows<false>(p.op);
        return hipLaunchKernel(fn, dim3(p.grid), dim3(64), args, 0, stream);
    }
    uint32_t nwhole = p.flat_last == 256 ? p.nwork : p.nwork - 1;
    uint32_t tail = p.flat_last == 256 ? 0 : p.flat_last;
    void *args[] = {&x, &y, &alpha, &beta, &nwhole, &tail};
    const int mode = p.access == tmp::kVec4 ? kChunk16 : p.access == tmp::kScalar ? kFour4 : kOne4;
    const void *fn = p.op == tmp::kAffine ? pick_flat<tmp::kAffine>(mode)
                     : p.op == tmp::kScale ? pick_flat<tmp::kScale>(mode)
                                           : pick_flat<tmp::kCopy>(mode);
    return hipLaunchKernel(fn, dim3(p.grid), dim3(mode == kOne4 ? 256 : 64), args, 0, stream);
}

}  // namespace tmk
