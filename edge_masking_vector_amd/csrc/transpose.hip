// transpose.hip -- batched 2-D transpose for gfx950: y[b][j][i] = x[b][i][j], the layout
// conversion between NCHW and NHWC.
//
// Sources (web pages): teenygrad "Memory Coalescing and Tensor Layout" ("NCHW versus NHWC": a
// layout conversion costs one full pass over memory; "Seeing it in a real kernel" and "A
// checklist": load a tile once into fast memory, then read it in whatever order you like;
// "Strides, and reading an index expression"); Phobos docs "Slicing, bounds and masking"
// ("Masking": out-of-range elements read as 0 and their stores are skipped).
//
// Mapping.  A workgroup (512 threads) takes one SM x SN sub-tile of x (64 x 64; under the alignment
// promise the largest power of two up to 64 that divides the extent, which the caller's tile
// divides); sub-tiles are visited in diagonal order (see below).  It reads the sub-tile along x's rows -- lanes take consecutive chunks of a row,
// so the lane-varying term of the address is the column -- and stages it in LDS with a row stride
// of SN + 1 floats.  After a barrier it reads the staged tile down its columns and writes y's rows,
// again with consecutive lanes on consecutive chunks of a y row.  Both global sides are coalesced;
// only LDS sees the column order.  Chunks are 16 bytes when both tensors have 16-byte rows, else
// single elements.  Under the alignment promise every sub-tile is whole and no mask is evaluated.
// Diagonal order took the 4096 x 4096 transpose from 30.8 to 25.8 us, and 512 threads per
// workgroup to 24.4 us.
#include "device.hpp"
#include "launch.h"

namespace tmk {
namespace {

constexpr int kSub = 64;            // largest sub-tile edge
constexpr int kPad = kSub + 1;      // LDS row stride (floats) of the staged sub-tile
constexpr int kTrBlock = 512;       // threads per workgroup (2 x 16-byte chunks each per sub-tile)

struct TrArgs {
    const float *x;
    float *y;
    int64_t ldx, ldy, bsx, bsy;
    int64_t B, M, N;
    int sm, sn;                      // staged sub-tile extents (powers of two <= 64)
    uint32_t subs_m, subs_n;         // sub-tiles along M and N per batch
    uint64_t nwork;                  // B * subs_m * subs_n
};

template <bool VEC, bool ALIGNED, int BS>
__global__ __launch_bounds__(BS) void transpose_tiles(TrArgs a) {
    constexpr int W = VEC ? 4 : 1;
    constexpr int K = kSub * kSub / W / BS;   // chunks per thread for a full 64 x 64 sub-tile
    __shared__ float tile[kSub * kPad];
    const int t = threadIdx.x;
    const int cpr_x = a.sn / W;     // chunks per staged x row
    const int cpr_y = a.sm / W;     // chunks per y row
    const int nchunks = a.sm * a.sn / W;

    uint64_t w = blockIdx.x;
    do {
        const uint64_t per_b = uint64_t(a.subs_m) * a.subs_n;
        const uint64_t b = w / per_b;
        const uint64_t rest = w - b * per_b;
        // Diagonal order: consecutive work items step one sub-tile down AND one across, so the
        // workgroups running together read x and write y at different column offsets (in row-major
        // order they would all write y at one column offset, rows 64 * ldy apart, and crowd the
        // same HBM channels).  For each pm, q runs over every sub-tile column once.
        const uint64_t pm = rest % a.subs_m;
        const uint64_t q = rest / a.subs_m;
        const uint64_t pn = (q + pm) % a.subs_n;
        const int64_t row0 = int64_t(pm) * a.sm;   // x rows = y columns
        const int64_t col0 = int64_t(pn) * a.sn;   // x columns = y rows
        const float *xb = a.x + int64_t(b) * a.bsx;
        float *yb = a.y + int64_t(b) * a.bsy;
        const int64_t rows_live = a.M - row0, cols_live = a.N - col0;

        // Read x's sub-tile along its rows (all of this thread's chunks first); an element past
        // the tensor reads as 0.
        float v[K][W];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = t + k * BS;
            const int r = e / cpr_x, c = (e - r * cpr_x) * W;
            const float *p = xb + (row0 + r) * a.ldx + col0 + c;
            if (e < nchunks) {
                if (ALIGNED || (r < rows_live && c + W <= cols_live)) {
                    if constexpr (VEC) {
                        const f4 q = ld16_nt(p);
                        v[k][0] = q.x, v[k][1] = q.y, v[k][2] = q.z, v[k][3] = q.w;
                    } else {
                        v[k][0] = ld4_nt(p);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < W; ++i)
                        v[k][i] = (r < rows_live && c + i < cols_live) ? p[i] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = t + k * BS;
            const int r = e / cpr_x, c = (e - r * cpr_x) * W;
            if (e < nchunks) {
#pragma unroll
                for (int i = 0; i < W; ++i)
                    tile[r * kPad + c + i] = v[k][i];
            }
        }
        __syncthreads();

        // Write y's rows: y row j (x column col0 + j) takes the staged column j; a store past the
        // tensor is skipped.
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = t + k * BS;
            const int j = e / cpr_y, i = (e - j * cpr_y) * W;
            if (e < nchunks) {
#pragma unroll
                for (int q = 0; q < W; ++q)
                    v[k][q] = tile[(i + q) * kPad + j];
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = t + k * BS;
            const int j = e / cpr_y, i = (e - j * cpr_y) * W;
            float *q = yb + (col0 + j) * a.ldy + row0 + i;
            if (e < nchunks) {
                if (ALIGNED || (j < cols_live && i + W <= rows_live)) {
                    if constexpr (VEC)
                        st16_nt(q, f4{v[k][0], v[k][1], v[k][2], v[k][3]});
                    else
                        st4_nt(q, v[k][0]);
                } else if (j < cols_live) {
#pragma unroll
                    for (int z = 0; z < W; ++z)
                        if (i + z < rows_live)
                            q[z] = v[k][z];
                }
            }
        }
        __syncthreads();
        w += gridDim.x;
    } while (w < a.nwork);
}

}  // namespace

hipError_t launch_transpose(const tmp::TransposePlan &p, hipStream_t stream) {
    TrArgs a;
    a.x = p.x;
    a.y = p.y;
    a.ldx = p.ldx;
    a.ldy = p.ldy;
    a.bsx = p.bsx;
    a.bsy = p.bsy;
    a.B = p.B;
    a.M = p.M;
    a.N = p.N;
    a.sm = p.sm;
    a.sn = p.sn;
    a.subs_m = p.subs_m;
    a.subs_n = p.subs_n;
    a.nwork = p.nwork;
    const void *fn = p.vec ? (p.aligned ? reinterpret_cast<const void *>(&transpose_tiles<true, true, kTrBlock>)
                                        : reinterpret_cast<const void *>(&transpose_tiles<true, false, kTrBlock>))
                           : reinterpret_cast<const void *>(&transpose_tiles<false, false, kTrBlock>);
    void *args[] = {&a};
    return hipLaunchKernel(fn, dim3(p.grid), dim3(kTrBlock), args, 0, stream);
}

}  // namespace tmk
