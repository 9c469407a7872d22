// colred.hip -- column sums for gfx950 over row-major f32: the naive strided walk and the
// LDS-staged coalesced walk, both followed by a fixed-order pass over per-slab partials.
//
// Sources (web pages): teenygrad "Memory Coalescing and Tensor Layout" ("What it actually costs":
// the row and column walks of one 4096 x 4096 matrix, 65536 programs of 256 elements, column index
// varying fastest across programs; "Seeing it in a real kernel" and "A checklist": stage a tile in
// fast memory, then read it in any order); Phobos docs "Slicing, bounds and masking" ("Masking":
// out-of-range elements read as 0).
//
// Both walks cut the rows into slabs and write one partial per (slab, column) into the caller's
// workspace, column by column: ws[column * slabs + slab]; colsum_finish then adds each column's
// partials in a fixed order (a group of lanes per column, each taking every FL-th slab, then a
// lane tree), so the lanes of a column read consecutive floats.  Nothing uses atomics, so results
// are deterministic.
//
// Naive walk: slabs of the caller's TM rows; one workgroup per (slab, column), column fastest;
// lane t reads row slab*TM + t of that column.  The lane-varying term of the address is row * ld: every lane touches its own
// cache line.  In plain id order neighbouring columns run on different XCDs and every XCD fetches
// every line (8x the matrix on MI355X); the XCD-aware variant renumbers the workgroups so that
// each XCD walks a contiguous range of columns and shares its lines through one L2.
//
// LDS walk: slabs and strips of the walk's own size (256 rows or more, up to 128 columns; the
// caller's tile only states the promise); one workgroup per (slab, strip of TW columns), strip
// fastest.  LPR = TW / W lanes
// cover one row of the strip with consecutive 16-byte chunks (W = 4; W = 1 on the scalar path), so
// the 256 threads read RP = 256 / LPR rows at a time, fully coalesced, and each thread keeps
// running column partials in registers while walking down the slab.  The RP x TW partials are then
// staged in LDS row by row and read back column by column: thread c adds the RP values of column c
// in fixed order.  Writes into LDS are consecutive 16-byte chunks and reads are consecutive dwords,
// so neither side has bank conflicts and no padding is needed.
#include "device.hpp"
#include "launch.h"

namespace tmk {
namespace {

struct ColArgs {
    const float *x;
    float *ws;
    float *out;       // direct walk: the column sums
    int64_t ld, M, N;
    int log_tm;
    uint32_t strips;  // LDS walk: strips of TW columns; naive walk: N
    uint32_t slabs;
    int out16;        // direct walk: out is 16-byte aligned
};

// ---- naive walk ------------------------------------------------------------------------------

constexpr uint32_t kXcds = 8;  // MI355X: accelerator complex dies (XCDs), each with its own L2

// XCD: workgroup ids are dispatched to the XCDs in turn (id mod kXcds), so in plain column order
// the 32 workgroups whose columns share a 128-byte line run on different XCDs, each of which
// fetches the line into its own L2.  With XCD set, the ids are renumbered so that each XCD takes a
// contiguous range of work items (column order within it) and the line is fetched once.
template <bool XCD>
__global__ __launch_bounds__(kBlock) void col_naive(ColArgs a) {
    __shared__ float wave_sum[kBlock / 64];
    const int t = threadIdx.x;
    const int nwaves = blockDim.x / 64;
    const int64_t tm = int64_t(1) << a.log_tm;
    const uint64_t nwork = uint64_t(a.slabs) * uint64_t(a.N);
    uint64_t first = blockIdx.x;
    if constexpr (XCD) {
        // A bijection of [0, G): XCD x (the ids x, x + kXcds, ...) gets the contiguous range
        // starting at x * q + min(x, r), where G = q * kXcds + r.
        const uint32_t G = gridDim.x, q = G / kXcds, r = G % kXcds;
        const uint32_t x = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
        first = uint64_t(x) * q + (x < r ? x : r) + i;
    }
    for (uint64_t w = first; w < nwork; w += gridDim.x) {
        const uint64_t slab = w / uint64_t(a.N);
        const int64_t c = int64_t(w - slab * uint64_t(a.N));
        const int64_t row = int64_t(slab) * tm + t;
        float v = 0.0f;  // rows past the slab or past M read as 0
        if (t < tm && row < a.M)
            v = a.x[row * a.ld + c];
        v = group_reduce<SumOp, 64>(v);
        if ((t & 63) == 0)
            wave_sum[t >> 6] = v;
        __syncthreads();
        if (t == 0) {
            float s = wave_sum[0];
            for (int i = 1; i < nwaves; ++i)
                s += wave_sum[i];
            a.ws[c * int64_t(a.slabs) + int64_t(slab)] = s;
        }
        if (w + gridDim.x < nwork)
            __syncthreads();  // the next work item reuses wave_sum (uniform test)
    }
}

// ---- LDS-staged walk -------------------------------------------------------------------------

constexpr int kRowsInFlight = 16;  // rows each thread loads before adding
constexpr int kColAcc = 8;         // independent column accumulators per thread

template <bool VEC>
__device__ __forceinline__ auto chunk_or_zero(const float *p, int64_t live) {
    if constexpr (VEC) {
        if (live >= 4)
            return ld16u_nt(p);  // rows may be off the 16-byte grid
        f4 r = f4(0.0f);
        if (live > 0)
            r.x = p[0];
        if (live > 1)
            r.y = p[1];
        if (live > 2)
            r.z = p[2];
        return r;
    } else {
        return live > 0 ? ld4_nt(p) : 0.0f;
    }
}

template <bool VEC, bool ALIGNED, int LPR>
__global__ __launch_bounds__(kBlock) void col_lds(ColArgs a) {
    using T = typename std::conditional<VEC, f4, float>::type;
    constexpr int W = VEC ? 4 : 1;
    constexpr int RP = kBlock / LPR;  // rows read per step
    constexpr int TW = LPR * W;       // strip width in columns
    __shared__ float part[RP * TW];   // kBlock * W floats

    const int t = threadIdx.x;
    const int g = t % LPR;
    const int q = t / LPR;
    const int64_t tm = int64_t(1) << a.log_tm;
    const uint64_t nwork = uint64_t(a.slabs) * a.strips;

    for (uint64_t w = blockIdx.x; w < nwork; w += gridDim.x) {
        const uint64_t slab = w / a.strips;
        const int64_t strip = int64_t(w - slab * a.strips);
        const int64_t col0 = strip * TW;
        const int64_t row0 = int64_t(slab) << a.log_tm;
        const int64_t c = col0 + g * W;
        const int64_t live = a.N - c;  // elements of this thread's chunk inside the tensor
        const float *p = a.x + row0 * a.ld + c;
        const int64_t rows = ALIGNED ? tm : (a.M - row0 < tm ? a.M - row0 : tm);

        T acc[kColAcc];
#pragma unroll
        for (int u = 0; u < kColAcc; ++u)
            acc[u] = T(0.0f);
        for (int64_t r = q; r < rows; r += int64_t(RP) * kRowsInFlight) {
            T v[kRowsInFlight];
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u) {
                const int64_t rr = r + int64_t(u) * RP;
                v[u] = T(0.0f);
                if (rr < rows) {
                    if constexpr (ALIGNED)
                        v[u] = ld16u_nt(p + rr * a.ld);
                    else
                        v[u] = chunk_or_zero<VEC>(p + rr * a.ld, live);
                }
            }
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u)
                acc[u % kColAcc] += v[u];
        }
        // Fixed-order fold of the row accumulators.
        T s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));

        // Stage: row q of the partials, columns g*W .. g*W+W-1.
        if constexpr (VEC)
            *reinterpret_cast<f4 *>(&part[q * TW + g * W]) = s;
        else
            part[q * TW + g] = s;
        __syncthreads();
        // Read back by column: thread cl adds the RP partials of column cl in order.
        for (int cl = t; cl < TW; cl += kBlock) {
            float colsum = 0.0f;
            for (int k = 0; k < RP; ++k)
                colsum += part[k * TW + cl];
            if (col0 + cl < a.N)
                a.ws[(col0 + cl) * int64_t(a.slabs) + int64_t(slab)] = colsum;
        }
        if (w + gridDim.x < nwork)
            __syncthreads();  // the next work item reuses the LDS partials (uniform test)
    }
}

// ---- strip walk (wide matrices) -------------------------------------------------------------------
// A workgroup takes (slab, strip): tm rows by tmp::kColStripCols columns, strip fastest, so the
// workgroups running together read whole rows.  Lane t of each of its kColStripGroups waves owns
// 16-byte column chunk t of the strip; wave q adds rows [q tm / G, (q + 1) tm / G) of the slab
// down it, kStripBatch loads in flight into 4 accumulators folded in a fixed order, and the waves'
// sums meet in LDS in wave order: the slab's partial for the lane's four columns, stored as one
// 16-byte vector at ws[slab * N + column] (the workspace is 16-byte aligned and N % 4 == 0).  The
// loads carry no control flow: a row past M re-reads row M - 1 and a chunk past N re-reads the
// row's last chunk, and both are then replaced by 0 ([SLICING] "Masking": out-of-range elements
// read as 0).  WHOLE: the host found whole slabs and strips, so there is nothing to replace.  U:
// rows off the 16-byte grid (N a whole number of strips): chunks are 16-byte loads from 4-byte
// aligned addresses, which the GPU's unaligned access mode executes as one load.
constexpr int kStripBatch = 8;
constexpr int kStripGroups = tmp::kColStripGroups;
constexpr int kStripThreads = 64 * kStripGroups;
static_assert(tmp::kColStripCols == 64 * 4, "a strip is one 16-byte chunk per lane of a wave");
static_assert(tmp::kColRowSlab % (kStripGroups * kStripBatch) == 0, "whole batches per row group");

template <bool WHOLE, bool U>
__global__ __launch_bounds__(kStripThreads) void col_strip(ColArgs a) {
    __shared__ f4 part[kStripGroups][64];
    const int t = threadIdx.x % 64, q = threadIdx.x / 64;
    const uint32_t strip = blockIdx.x % a.strips, slab = blockIdx.x / a.strips;
    const int64_t nch = a.N / 4;                          // 16-byte chunks per row
    const int64_t ch = int64_t(strip) * 64 + t;           // this lane's column chunk
    const int64_t chc = ch < nch ? ch : nch - 1;
    const int64_t rg = (int64_t(1) << a.log_tm) / kStripGroups;  // rows per wave (tm >= 64)
    const int64_t row0 = (int64_t(slab) << a.log_tm) + q * rg;
    const float *p = a.x + chc * 4;
    f4 acc[4] = {f4(0.0f), f4(0.0f), f4(0.0f), f4(0.0f)};
    for (int64_t r0 = 0; r0 < rg; r0 += kStripBatch) {
        f4 v[kStripBatch];
#pragma unroll
        for (int u = 0; u < kStripBatch; ++u) {
            const int64_t row = row0 + r0 + u;
            const float *pr = p + (WHOLE || row < a.M ? row : a.M - 1) * a.ld;
            v[u] = U ? ld16u_nt(pr) : ld16_nt(pr);
        }
#pragma unroll
        for (int u = 0; u < kStripBatch; ++u) {
            if constexpr (!WHOLE)
                v[u] = row0 + r0 + u < a.M ? v[u] : f4(0.0f);
            acc[u % 4] += v[u];
        }
    }
    part[q][t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __syncthreads();
    if (q == 0 && (WHOLE || ch < nch)) {
        f4 s = part[0][t];
#pragma unroll
        for (int k = 1; k < kStripGroups; ++k)
            s += part[k][t];
        *reinterpret_cast<f4 *>(a.ws + int64_t(slab) * a.N + ch * 4) = s;
    }
}

// Pass 2 after the strip walk: workgroup b takes 16-byte column chunks 64 b .. 64 b + 63; wave w of
// its kFold waves adds slabs [w S / kFold, (w + 1) S / kFold) of its lane's chunk in order, 16
// coalesced loads in flight (consecutive lanes on consecutive chunks), and the waves' sums meet
// in LDS in wave order.  Fixed order throughout: the result is deterministic.  out need only be
// 4-byte aligned: its 16-byte stores go to 4-byte aligned addresses.
constexpr int kFold = 4;  // waves per workgroup
constexpr int kFoldBatch = 16;  // partials in flight per lane

__global__ __launch_bounds__(kFold * 64) void colsum_fold16(const float *ws, float *out, int64_t N,
                                                              uint32_t slabs) {
    __shared__ f4 wsum[kFold][64];
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    const int64_t nch = N / 4;
    const int64_t ch = int64_t(blockIdx.x) * 64 + lane;
    const int64_t chc = ch < nch ? ch : nch - 1;
    const uint32_t s_begin = uint32_t(uint64_t(slabs) * w / kFold);
    const uint32_t s_end = uint32_t(uint64_t(slabs) * (w + 1) / kFold);
    const f4 *p = reinterpret_cast<const f4 *>(ws) + chc;
    f4 acc = f4(0.0f);
    for (uint32_t s0 = s_begin; s0 < s_end; s0 += kFoldBatch) {
        f4 v[kFoldBatch];
#pragma unroll
        for (int u = 0; u < kFoldBatch; ++u) {
            const uint32_t s = s0 + u < s_end ? s0 + u : s_end - 1;
            v[u] = p[int64_t(s) * nch];
        }
#pragma unroll
        for (int u = 0; u < kFoldBatch; ++u)
            acc += s0 + u < s_end ? v[u] : f4(0.0f);
    }
    wsum[w][lane] = acc;
    __syncthreads();
    if (w == 0 && ch < nch) {
        f4 total = wsum[0][lane];
#pragma unroll
        for (int k = 1; k < kFold; ++k)
            total += wsum[k][lane];
        *reinterpret_cast<f4u *>(out + ch * 4) = total;
    }
}

// ---- direct walk ---------------------------------------------------------------------------------
// For few rows, or columns enough to fill the GPU by themselves: each thread owns one chunk of W
// columns and adds all M rows down it -- kRowsInFlight coalesced loads at a time (consecutive
// threads on consecutive chunks of a row) into kColAcc accumulators -- then folds the
// accumulators in a fixed order and stores the W sums.  One pass: no partials, no pass 2.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void col_direct(ColArgs a) {
    using T = typename std::conditional<VEC, f4, float>::type;
    constexpr int W = VEC ? 4 : 1;
    const int64_t nchunks = (a.N + W - 1) / W;
    for (int64_t q = int64_t(blockIdx.x) * kBlock + threadIdx.x; q < nchunks;
         q += int64_t(gridDim.x) * kBlock) {
        const int64_t c = q * W;
        const int64_t live = a.N - c;  // columns of this chunk inside the tensor
        const float *p = a.x + c;
        T acc[kColAcc];
#pragma unroll
        for (int u = 0; u < kColAcc; ++u)
            acc[u] = T(0.0f);
        for (int64_t r = 0; r < a.M; r += kRowsInFlight) {
            T v[kRowsInFlight];
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u)
                v[u] = r + u < a.M ? chunk_or_zero<VEC>(p + (r + u) * a.ld, live) : T(0.0f);
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u)
                acc[u % kColAcc] += v[u];
        }
        const T s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
        float *o = a.out + c;
        if constexpr (VEC) {
            if (live >= 4 && a.out16) {
                *reinterpret_cast<f4 *>(o) = s;
            } else {
                o[0] = s.x;
                if (live > 1)
                    o[1] = s.y;
                if (live > 2)
                    o[2] = s.z;
                if (live > 3)
                    o[3] = s.w;
            }
        } else {
            *o = s;
        }
    }
}

// ---- pass 2: fixed-order sum of the slab partials ---------------------------------------------

constexpr int kFinishBatch = tmp::kFinishBatchSlabs;  // partials loaded at once per lane, then added in slab order
constexpr int kFinishBlock = 256;  // threads per workgroup: kFinishBlock / FL columns

// FL lanes per column: lane f adds slabs f, f + FL, f + 2 FL, ... in order (batches of
// kFinishBatch loads in flight), then the FL lane values meet in a fixed DPP tree; past 64 lanes
// (2 or 4 waves per column) the waves' sums then meet in LDS in wave order.  Columns past N
// re-read column N - 1 so that every lane takes part in the tree; they are not stored.
template <int FL>
__global__ __launch_bounds__(kFinishBlock) void colsum_finish(const float *ws, float *out, int64_t N,
                                                            uint32_t slabs) {
    static_assert(FL <= kFinishBlock && kFinishBlock % FL == 0, "whole columns per workgroup");
    constexpr int kCols = kFinishBlock / FL;  // columns per workgroup and step
    constexpr int kWaves = FL > 64 ? FL / 64 : 1;  // waves per column
    __shared__ float wave_sum[kFinishBlock / 64];
    const int f = threadIdx.x % FL;
    for (int64_t j0 = int64_t(blockIdx.x) * kCols; j0 < N; j0 += int64_t(gridDim.x) * kCols) {
        const int64_t j = j0 + threadIdx.x / FL;
        const int64_t jc = j < N ? j : N - 1;
        float total = 0.0f;
        for (uint32_t s0 = f; s0 < slabs; s0 += uint32_t(FL) * kFinishBatch) {
            float v[kFinishBatch];
#pragma unroll
            for (int u = 0; u < kFinishBatch; ++u) {
                const uint32_t s = s0 + uint32_t(u) * FL;
                v[u] = s < slabs ? ws[jc * int64_t(slabs) + int64_t(s)] : 0.0f;
            }
            float blk = 0.0f;
#pragma unroll
            for (int u = 0; u < kFinishBatch; ++u)
                blk += v[u];
            total += blk;
        }
        if constexpr (kWaves == 1) {
            total = group_reduce<SumOp, FL>(total);
            if (f == 0 && j < N)
                out[j] = total;
        } else {
            total = group_reduce<SumOp, 64>(total);
            if (threadIdx.x % 64 == 0)
                wave_sum[threadIdx.x / 64] = total;
            __syncthreads();
            if (f == 0) {
                float s = wave_sum[threadIdx.x / 64];
#pragma unroll
                for (int w = 1; w < kWaves; ++w)
                    s += wave_sum[threadIdx.x / 64 + w];
                if (j < N)
                    out[j] = s;
            }
            __syncthreads();  // the next step reuses wave_sum (j0 is uniform over the workgroup)
        }
    }
}

const void *pick_finish(int fl) {
    switch (fl) {
    case 1: return reinterpret_cast<const void *>(&colsum_finish<1>);
    case 2: return reinterpret_cast<const void *>(&colsum_finish<2>);
    case 4: return reinterpret_cast<const void *>(&colsum_finish<4>);
    case 8: return reinterpret_cast<const void *>(&colsum_finish<8>);
    case 16: return reinterpret_cast<const void *>(&colsum_finish<16>);
    case 32: return reinterpret_cast<const void *>(&colsum_finish<32>);
    case 64: return reinterpret_cast<const void *>(&colsum_finish<64>);
    case 128: return reinterpret_cast<const void *>(&colsum_finish<128>);
    default: return reinterpret_cast<const void *>(&colsum_finish<256>);
    }
}

template <bool VEC, bool AL>
const void *pick_lpr(int lpr) {
    switch (lpr) {
    case 1: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 1>);
    case 2: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 2>);
    case 4: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 4>);
    case 8: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 8>);
    case 16: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 16>);
    case 32: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 32>);
    case 64: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 64>);
    case 128: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 128>);
    default: return reinterpret_cast<const void *>(&col_lds<VEC, AL, 256>);
    }
}

}  // namespace

hipError_t launch_cols(const tmp::ColPlan &p, hipStream_t stream) {
    constexpr uint32_t kGridCap = 1u << 20;
    if (p.direct) {
        ColArgs a;
        a.x = p.x;
        a.ws = nullptr;
        a.out = p.out;
        a.ld = p.ld;
        a.M = p.M;
        a.N = p.N;
        a.log_tm = 0;
        a.strips = 0;
        a.slabs = 0;
        a.out16 = p.out16 ? 1 : 0;
        void *args[] = {&a};
        const int64_t nchunks = (p.N + (p.vec ? 3 : 0)) / (p.vec ? 4 : 1);
        const int64_t blocks = (nchunks + kBlock - 1) / kBlock;
        const uint32_t grid = static_cast<uint32_t>(blocks < kGridCap ? blocks : kGridCap);
        const void *fn = p.vec ? reinterpret_cast<const void *>(&col_direct<true>)
                               : reinterpret_cast<const void *>(&col_direct<false>);
        return hipLaunchKernel(fn, dim3(grid), dim3(kBlock), args, 0, stream);
    }
    if (p.strip) {
        ColArgs a;
        a.x = p.x;
        a.ws = p.ws;
        a.out = p.out;
        a.out16 = 0;
        a.ld = p.ld;
        a.M = p.M;
        a.N = p.N;
        a.log_tm = p.log_tm;
        a.strips = p.strips;
        a.slabs = p.slabs;
        void *args[] = {&a};
        const void *fn = p.vec ? (p.whole ? reinterpret_cast<const void *>(&col_strip<true, false>)
                                          : reinterpret_cast<const void *>(&col_strip<false, false>))
                               : (p.whole ? reinterpret_cast<const void *>(&col_strip<true, true>)
                                          : reinterpret_cast<const void *>(&col_strip<false, true>));
        hipError_t err = hipLaunchKernel(fn, dim3(p.slabs * p.strips), dim3(kStripThreads), args, 0, stream);
        if (err != hipSuccess)
            return err;
        const float *ws = p.ws;
        float *out = p.out;
        int64_t N = p.N;
        uint32_t slabs = p.slabs;
        void *fargs[] = {&ws, &out, &N, &slabs};
        const uint32_t fgrid = static_cast<uint32_t>((p.N / 4 + 63) / 64);
        return hipLaunchKernel(reinterpret_cast<const void *>(&colsum_fold16), dim3(fgrid), dim3(kFold * 64),
                               fargs, 0, stream);
    }
    if (p.launch) {
        ColArgs a;
        a.x = p.x;
        a.ws = p.ws;
        a.out = p.out;
        a.out16 = 0;
        a.ld = p.ld;
        a.M = p.M;
        a.N = p.N;
        a.log_tm = p.log_tm;
        a.strips = p.strips;
        a.slabs = p.slabs;
        void *args[] = {&a};
        const uint64_t nwork = uint64_t(p.slabs) * p.strips;
        const uint32_t grid = static_cast<uint32_t>(nwork < kGridCap ? nwork : kGridCap);
        hipError_t err;
        if (p.walk == TM_COL_LDS) {
            const int W = p.vec ? 4 : 1;
            const int lpr = p.tw / W;
            // 16-byte chunks are only used when the host checked 16-byte rows; the unmasked body
            // only when it also found whole slabs and strips.
            const void *fn = p.vec ? (p.whole ? pick_lpr<true, true>(lpr) : pick_lpr<true, false>(lpr))
                                   : pick_lpr<false, false>(lpr);
            err = hipLaunchKernel(fn, dim3(grid), dim3(kBlock), args, 0, stream);
        } else {
            const void *fn = p.walk == TM_COL_NAIVE_XCD ? reinterpret_cast<const void *>(&col_naive<true>)
                                                        : reinterpret_cast<const void *>(&col_naive<false>);
            err = hipLaunchKernel(fn, dim3(grid), dim3(p.naive_block), args, 0, stream);
        }
        if (err != hipSuccess)
            return err;
    }
    if (p.finish) {
        const int64_t cols = kFinishBlock / p.fl;
        const int64_t blocks = (p.N + cols - 1) / cols;
        const uint32_t grid = static_cast<uint32_t>(blocks < kGridCap ? blocks : kGridCap);
        const float *ws = p.ws;
        float *out = p.out;
        int64_t N = p.N;
        uint32_t slabs = p.launch ? p.slabs : 0u;
        void *args[] = {&ws, &out, &N, &slabs};
        return hipLaunchKernel(pick_finish(p.fl), dim3(grid), dim3(kFinishBlock), args, 0, stream);
    }
    return hipSuccess;
}

}  // namespace tmk
