// transpose.hip -- batched 2-D transpose for gfx950: y[b][j][i] = x[b][i][j], the layout
// conversion between NCHW and NHWC.
//
// Sources (web pages): teenygrad "Memory Coalescing and Tensor Layout" ("NCHW versus NHWC": a
// layout conversion costs one full pass over memory; "Seeing it in a real kernel" and "A
// checklist": load a tile once into fast memory, then read it in whatever order you like;
// "Strides, and reading an index expression"); Phobos docs "Slicing, bounds and masking"
// ("Masking": out-of-range elements read as 0 and their stores are skipped).
//
// Mapping.  A workgroup (256 threads) takes one SM x SN sub-tile of x (32 x 32: a row segment is
// one 128-byte line; under the alignment promise the largest power of two up to 32 that divides
// the extent, which the caller's tile divides).  A narrow tensor -- fewer than 32 rows or columns,
// as the 3 channels of an RGB image in NCHW -> NHWC -- gets a sub-tile just as narrow and as much
// longer (4 x 256 for 3 channels), so that no lanes idle on rows that do not exist; sub-tiles
// hold at most 1024 elements.  Sub-tiles are visited in diagonal order (see
// below).  It reads the sub-tile along x's rows -- lanes take consecutive chunks of a row, so the
// lane-varying term of the address is the column -- and stages it in LDS with a row stride of
// SN + 1 floats.  After a barrier it reads the staged tile down its columns and writes y's rows,
// again with consecutive lanes on consecutive chunks of a y row.  Both global sides are coalesced;
// only LDS sees the column order.  Chunks are 16 bytes when both tensors have 16-byte rows, else
// single elements.  Under the alignment promise every sub-tile is whole and no mask is evaluated.
// Diagonal order took the 4096 x 4096 transpose from 30.8 to 25.8 us.  Sub-tile and workgroup
// size, measured on 4096 x 4096 and on NCHW -> NHWC of [32][64][3136]: 64 x 64 with 512 threads
// 24.6 / 10.6 us, 128 x 128 with 1024 threads 24.4 / -, 32 x 32 with 256 threads (one 16-byte
// chunk per thread) 24.2 / 9.7 us; in a standalone kernel on 4096 x 4096, longer row segments on
// one or both sides with 2-8 chunks per thread (32 x 64 up to 128 x 64, 256 threads) took
// 24.4-26.3 us against 23.9 us for 32 x 32.  Reading the staged tile by rows instead of columns
// (a timing-only variant) changed nothing: LDS bank conflicts do not limit this kernel.
#include "device.hpp"
#include "launch.h"

namespace tmk {
namespace {

constexpr int kSubElems = tmp::kTrSubElems;  // largest sub-tile (elements)
// LDS of a staged sub-tile: SM rows of stride SN + 1 floats, SM * SN <= SUB (the instance's
// largest sub-tile), so at most 2 * SUB floats (SN = 1: SUB rows of stride 2).
constexpr int kStage = 2 * kSubElems;
constexpr int kTrBlock = 256;       // threads per workgroup (one 16-byte chunk each per sub-tile)

// Kernel arguments: kept within 128 bytes so that one batch of scalar loads fetches them all
// before the first global load (a field past that was fetched by a second, dependent load).
struct TrArgs {
    const float *x;
    float *y;
    int64_t ldx, ldy, bsx, bsy;
    int64_t M, N;
    uint64_t nwork;                  // B * subs_m * subs_n
    uint64_t c_pb, c_m, c_n;         // multipliers of per_b, subs_m, subs_n for fast_div
    uint32_t subs_m, subs_n;         // sub-tiles along M and N per batch
    uint32_t per_b;                  // subs_m * subs_n (when the work count fits 32 bits)
    int log_sm, log_sn;              // staged sub-tile extents: 2^log_sm x 2^log_sn (<= kSubElems)
    int log_g;                       // batches per work item (whole matrices in one sub-tile)
    int64_t B;                       // batches
};
static_assert(sizeof(TrArgs) <= 128, "transpose arguments outgrew one scalar load batch");

// PACK: every matrix fits in one sub-tile, and a work item takes 2^log_g consecutive batches, each
// staged in its own LDS region (a 256-thread workgroup per 4 x 4 matrix left 240 threads idle).
// VX / VY: x's rows (the reads) / y's rows (the writes) move in 16-byte chunks, each side as its
// own rows allow (a 9163 x 1051 transpose with 16-byte x rows and 4-byte y rows took 42 us with
// 4-byte chunks on both sides).  The reads need no 16-byte grid: off it they are 16-byte loads from
// 4-byte aligned addresses (the GPU's unaligned access mode), and a chunk that crosses the view's
// edge moves element by element.
// SUB: the largest sub-tile (elements) the instance stages.
//
// Work item w -> (batch b, sub-tile row pm, sub-tile column pn) for work counts below 2^32.
// GROUPS (one matrix): vertical groups of G = 2^log_g items (pm = G r .. G r + G - 1; here log_g
// counts items, not batches) go to workgroups b, b + 8, ..., b + 8 (G - 1), which the dispatcher
// sends to the same XCD one after another: item w is group 8 (w / 8G) + (w mod 8), member
// (w / 8) mod G, groups numbered r fastest (per_b / c_pb hold the group rows, ceil(subs_m / G));
// an item past the last group has none (skip).  Otherwise the diagonal order, by multiply-high
// divisions.
template <bool GROUPS>
__device__ __forceinline__ void decode32(const TrArgs &a, uint32_t w32, uint32_t &b, uint32_t &pm, uint32_t &pn,
                                         bool &skip) {
    if constexpr (GROUPS) {
        // groups are numbered by group row fastest, then by column strip over all batches (batch
        // q / subs_n, strip q mod subs_n)
        const uint32_t grp = (w32 >> (3 + a.log_g)) * 8 + (w32 & 7u);
        const uint32_t member = (w32 >> 3) & ((1u << a.log_g) - 1u);
        const uint32_t q = fast_div(grp, a.c_pb, a.per_b);  // per_b: group rows
        b = fast_div(q, a.c_n, a.subs_n);
        pm = ((grp - q * a.per_b) << a.log_g) + member;    // < subs_m + 2^log_g <= 2^32
        pn = q - b * a.subs_n;
        skip = pm >= a.subs_m || int64_t(b) >= a.B;
    } else {
        const uint32_t b32 = fast_div(w32, a.c_pb, a.per_b);
        const uint32_t rest = w32 - b32 * a.per_b;
        const uint32_t q = fast_div(rest, a.c_m, a.subs_m);
        const uint32_t pm32 = rest - q * a.subs_m;
        b = b32;
        pm = pm32;
        pn = fast_mod(q + pm32, a.c_n, a.subs_n);  // q + pm32 < subs_n + subs_m < 2^32
        skip = false;
    }
}

template <bool VX, bool VY, bool ALIGNED, int BS, bool WIDE, bool PACK, int SUB = kSubElems>
__global__ __launch_bounds__(BS) void transpose_tiles(TrArgs a) {
    static_assert(!ALIGNED || (VX && VY), "the promise implies 16-byte rows on both sides");
    constexpr int LOG_WX = VX ? 2 : 0, LOG_WY = VY ? 2 : 0;
    constexpr int WX = 1 << LOG_WX, WY = 1 << LOG_WY;
    constexpr int KX = SUB / WX / BS;   // read chunks per thread for a full sub-tile
    constexpr int KY = SUB / WY / BS;   // write chunks per thread
    __shared__ float tile[2 * SUB];
    const int t = threadIdx.x;
    // Sub-tile extents are powers of two of at least the chunk width: chunk coordinates are shifts
    // and masks (run-time divisions per chunk took the 4096 x 4096 transpose from 25.5 to 27.5 us).
    const int lcx = a.log_sn - LOG_WX;  // log2 of the chunks per staged x row
    const int lcy = a.log_sm - LOG_WY;  // log2 of the chunks per y row
    const int ltx = a.log_sm + a.log_sn - LOG_WX;  // log2 of the read chunks of one sub-tile
    const int lty = a.log_sm + a.log_sn - LOG_WY;  // log2 of the write chunks of one sub-tile
    const int nx = 1 << (ltx + (PACK ? a.log_g : 0));  // read chunks of the work item
    const int ny = 1 << (lty + (PACK ? a.log_g : 0));  // write chunks of the work item
    const int sm = 1 << a.log_sm, sn = 1 << a.log_sn;
    const int pad = sn + 1;             // LDS row stride: odd for SN >= 2, so columns spread over banks
    const int stage = sm * pad;         // LDS floats of one staged sub-tile (PACK: one per batch)

    uint64_t w = blockIdx.x;
    do {
        // Diagonal order: consecutive work items step one sub-tile down AND one across, so the
        // workgroups running together read x and write y at different column offsets (in row-major
        // order they would all write y at one column offset, rows SN * ldy apart, and crowd the
        // same HBM channels).  For each pm, q runs over every sub-tile column once.
        uint64_t b, pm, pn;
        bool skip = false;
        if constexpr (!WIDE) {  // the work count fits 32 bits
            uint32_t b32, pm32, pn32;
            decode32<false>(a, static_cast<uint32_t>(w), b32, pm32, pn32, skip);
            b = b32;
            pm = pm32;
            pn = pn32;
        } else {
            const uint64_t per_b = uint64_t(a.subs_m) * a.subs_n;
            b = w / per_b;
            const uint64_t rest = w - b * per_b;
            pm = rest % a.subs_m;
            pn = (rest / a.subs_m + pm) % a.subs_n;
        }
        // (a skipped pair-order item still takes part in the barriers below: uniform, no loads)
        const int64_t row0 = int64_t(pm) * sm;     // x rows = y columns
        const int64_t col0 = int64_t(pn) * sn;     // x columns = y rows
        const int64_t rows_live = skip ? 0 : a.M - row0, cols_live = skip ? 0 : a.N - col0;
        // Chunk e of the work item belongs to batch b0 + (e >> lt) (PACK; else b) and is chunk
        // e & (2^lt - 1) of that batch's sub-tile (lt: ltx for reads, lty for writes).
        const int64_t b0 = PACK ? int64_t(b) << a.log_g : int64_t(b);
        auto batch_of = [&](int e, int lt) { return PACK ? b0 + (e >> lt) : b0; };
        auto in_tile = [&](int e, int lt) { return PACK ? e & ((1 << lt) - 1) : e; };

        // Read x's sub-tile along its rows (all of this thread's chunks first); an element past
        // the tensor reads as 0.
        float v[KX][WX];
#pragma unroll
        for (int k = 0; k < KX; ++k) {
            const int e = t + k * BS, et = in_tile(e, ltx);
            const int r = et >> lcx, c = (et & ((1 << lcx) - 1)) << LOG_WX;
            const int64_t bb = batch_of(e, ltx);
            const float *p = a.x + bb * a.bsx + (row0 + r) * a.ldx + col0 + c;
#pragma unroll
            for (int i = 0; i < WX; ++i)
                v[k][i] = 0.0f;
            if (e < nx && (!PACK || bb < a.B)) {
                if (ALIGNED || (r < rows_live && c + WX <= cols_live)) {
                    if constexpr (VX) {
                        const f4 q = ld16u_nt(p);  // x's rows may be off the 16-byte grid
                        v[k][0] = q.x, v[k][1] = q.y, v[k][2] = q.z, v[k][3] = q.w;
                    } else {
                        v[k][0] = ld4_nt(p);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < WX; ++i)
                        v[k][i] = (r < rows_live && c + i < cols_live) ? p[i] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < KX; ++k) {
            const int e = t + k * BS, et = in_tile(e, ltx);
            const int r = et >> lcx, c = (et & ((1 << lcx) - 1)) << LOG_WX;
            const int g = PACK ? e >> ltx : 0;
            if (e < nx) {
#pragma unroll
                for (int i = 0; i < WX; ++i)
                    tile[g * stage + r * pad + c + i] = v[k][i];
            }
        }
        __syncthreads();

        // Write y's rows: y row j (x column col0 + j) takes the staged column j; a store past the
        // tensor is skipped.
        float u[KY][WY];
#pragma unroll
        for (int k = 0; k < KY; ++k) {
            const int e = t + k * BS, et = in_tile(e, lty);
            const int j = et >> lcy, i = (et & ((1 << lcy) - 1)) << LOG_WY;
            const int g = PACK ? e >> lty : 0;
            if (e < ny) {
#pragma unroll
                for (int q = 0; q < WY; ++q)
                    u[k][q] = tile[g * stage + (i + q) * pad + j];
            }
        }
#pragma unroll
        for (int k = 0; k < KY; ++k) {
            const int e = t + k * BS, et = in_tile(e, lty);
            const int j = et >> lcy, i = (et & ((1 << lcy) - 1)) << LOG_WY;
            const int64_t bb = batch_of(e, lty);
            float *q = a.y + bb * a.bsy + (col0 + j) * a.ldy + row0 + i;
            if (e < ny && (!PACK || bb < a.B)) {
                if (ALIGNED || (j < cols_live && i + WY <= rows_live)) {
                    if constexpr (VY)
                        st16_nt(q, f4{u[k][0], u[k][1], u[k][2], u[k][3]});
                    else
                        st4_nt(q, u[k][0]);
                } else if (j < cols_live) {
#pragma unroll
                    for (int z = 0; z < WY; ++z)
                        if (i + z < rows_live)
                            q[z] = u[k][z];
                }
            }
        }
        w += gridDim.x;
        if (w >= a.nwork)
            break;  // uniform; no barrier after the last sub-tile (it would hold the workgroup
                    // until its stores complete)
        __syncthreads();  // the next sub-tile reuses the LDS tile
    } while (true);
}

// ---- y rows off the line grid: line-aligned y windows -------------------------------------------
// Matrices whose y rows miss the 128-byte line grid (a batch's windows are numbered with its
// column strips: strip q of B x subs_n is strip q mod subs_n of batch q / subs_n).  With
// sub-tiles, the sub-tiles above and below each other share the lines at the ends of their y-row
// pieces, and a line that two
// workgroups write in parts reaches memory as two partial writes unless both parts meet in one
// L2 first; HBM3E has no write mask, so each costs the controller a read-modify-write (written
// bytes rose only 11-13%, but 4096 x 4096 with y stride 4100 took 55.7 against 24.4 us).
// Here work item (pm, pn) writes, in each y row
// j of its 32 (x columns col0 + j), the 64 elements that start at the line boundary at or before
// y column row0 = 64 pm: a window [row0 - s_j, row0 - s_j + 64), s_j = the offset of y[col0 + j]
// [row0] inside its line (0 .. 31 floats).  The windows of pm and pm + 1 meet exactly, so every
// line of y is written by one work item (only a line that holds a row's end and the next row's
// start has two writers), and no line is written in parts from two XCDs, which HBM3E would
// serve as read-modify-writes.  A window starts on a line, so its chunks are 16-byte aligned
// whatever the row stride: y is written in 16-byte stores.  The windows of one item reach x rows
// row0 - 31 .. row0 + 63, so the item stages the band of x rows row0 - 32 .. row0 + 63 (the
// top 32 are also its upper neighbour's, which the group order runs on the same XCD just before:
// plain loads, so they are still in that L2).  ceil((M + 31) / 64) items along M cover every row.
// Loads are clamped into the view (row to 0 .. M - 1, chunk to the one holding the last live
// column); what a clamped load stages is never stored.  VX: x read in 16-byte chunks (16-byte
// loads from 4-byte aligned addresses when x's rows are off the 16-byte grid); the chunks at or
// past the one holding a row's last live column read the 16 bytes that end at that column.
template <bool VX>
__global__ __launch_bounds__(kTrBlock) void transpose_skew(TrArgs a) {
    constexpr int SM = 2 * tmp::kTrSub, SN = tmp::kTrSub, BAND = SM + SN, PAD = SN + 1;
    constexpr int WX = VX ? 4 : 1;
    constexpr int NXC = BAND * SN / WX;                 // read chunks of the band
    constexpr int KX = NXC / kTrBlock;                  // 3 (16-byte) or 12 (4-byte) per thread
    constexpr int KY = SN * (SM / 4) / kTrBlock;        // 2 16-byte write chunks per thread
    static_assert(NXC % kTrBlock == 0 && SN * (SM / 4) % kTrBlock == 0, "chunks divide the workgroup");
    __shared__ float tile[BAND * PAD];
    const int t = threadIdx.x;
    uint64_t w = blockIdx.x;
    do {
        uint32_t b, pm, pn;
        bool skip;
        decode32<true>(a, static_cast<uint32_t>(w), b, pm, pn, skip);
        const int64_t row0 = int64_t(pm) * SM, col0 = int64_t(pn) * SN;
        const int cols_live = skip ? 0 : static_cast<int>(a.N - col0 < SN ? a.N - col0 : SN);
        if (cols_live > 0) {  // uniform
            // band row r is x row row0 - SN + r; loads from clamped rows and chunks.  With 16-byte
            // reads a chunk at or past the one holding the last live column reads the 16 bytes
            // that end at that column (from a 4-byte aligned address: x's rows need no 16-byte
            // grid) and stages them there; threads that clamp alike stage the same values.
            float v[KX][WX];
            const int clast = (cols_live - 1) / WX;
            const int cend = cols_live - WX;  // 16-byte reads: the clamped chunk's first column
#pragma unroll
            for (int k = 0; k < KX; ++k) {
                const int e = t + k * kTrBlock;
                const int r = e / (SN / WX), c = e - r * (SN / WX);
                int64_t xr = row0 - SN + r;
                xr = xr < 0 ? 0 : (xr >= a.M ? a.M - 1 : xr);
                if constexpr (VX) {
                    const int cs = c < clast ? c * WX : cend;  // cend >= -3: col0 >= 32 when below 4
                    const f4 q = ld16u(a.x + int64_t(b) * a.bsx + xr * a.ldx + col0 + cs);
                    v[k][0] = q.x, v[k][1] = q.y, v[k][2] = q.z, v[k][3] = q.w;
                } else {
                    v[k][0] = a.x[int64_t(b) * a.bsx + xr * a.ldx + col0 + (c < clast ? c : clast)];
                }
            }
#pragma unroll
            for (int k = 0; k < KX; ++k) {
                const int e = t + k * kTrBlock;
                const int r = e / (SN / WX), c = e - r * (SN / WX);
                const int cs = VX && c >= clast ? cend : c * WX;
#pragma unroll
                for (int i = 0; i < WX; ++i)
                    if (!VX || cs + i >= 0)
                        tile[r * PAD + cs + i] = v[k][i];
            }
        }
        __syncthreads();
        if (cols_live > 0) {
#pragma unroll
            for (int k = 0; k < KY; ++k) {
                const int e = t + k * kTrBlock;
                const int j = e >> 4, c = e & 15;  // y row j, chunk c of its 64-element window
                if (j < cols_live) {
                    float *yr = a.y + int64_t(b) * a.bsy + (col0 + j) * a.ldy;
                    const int sft = static_cast<int>((reinterpret_cast<uintptr_t>(yr + row0) >> 2) & 31u);
                    const int64_t i0 = row0 - sft + 4 * c;  // y column (x row) of the chunk's first element
                    const int br = SN - sft + 4 * c;        // its band row
                    f4 u;
                    u.x = tile[(br + 0) * PAD + j];
                    u.y = tile[(br + 1) * PAD + j];
                    u.z = tile[(br + 2) * PAD + j];
                    u.w = tile[(br + 3) * PAD + j];
                    if (i0 >= 0 && i0 + 4 <= a.M) {
                        st16_nt(yr + i0, u);
                    } else {
                        if (i0 + 0 >= 0 && i0 + 0 < a.M) st4_nt(yr + i0 + 0, u.x);
                        if (i0 + 1 >= 0 && i0 + 1 < a.M) st4_nt(yr + i0 + 1, u.y);
                        if (i0 + 2 >= 0 && i0 + 2 < a.M) st4_nt(yr + i0 + 2, u.z);
                        if (i0 + 3 >= 0 && i0 + 3 < a.M) st4_nt(yr + i0 + 3, u.w);
                    }
                }
            }
        }
        w += gridDim.x;
        if (w >= a.nwork)
            break;  // uniform
        __syncthreads();  // the next item reuses the LDS band
    } while (true);
}

// ---- few channels, packed side -------------------------------------------------------------------
// NCHW -> NHWC with C < 32 channels (MODE 0: x = [C][P] rows, y = [P][C] with row stride C) writes
// each work item's output -- S positions of all C channels -- as one contiguous block of S*C
// floats; NHWC -> NCHW (MODE 1: x = [P][C] with row stride C, y = [C][P]) reads its input that way.
// The packed block moves in 16-byte chunks when it starts on 16-byte boundaries: element o of the
// block is position o / C, channel o % C (multiply-high division, then a wrapping step), staged
// through LDS as C rows of S positions with a row stride of S + 1 floats.  The strided side moves
// as C rows of S positions, in 16-byte chunks when its rows allow (V).  With rows of 3 floats the
// general kernel moved every element alone.
struct PackedArgs {
    const float *x;
    float *y;
    int64_t ldx, ldy, bsx, bsy;
    int64_t P;            // positions (H*W)
    uint64_t c_s, c_k;    // multiply-high divisors of subs and of C
    uint32_t subs;        // work items per batch: ceil(P / S)
    uint32_t k;           // C
    uint32_t nwork;       // B * subs
    int log_s;            // positions per work item: S = 2^log_s, S * 2^ceil(log2 C) <= kSubElems
    int flat16;           // the packed block starts on 16-byte boundaries
};

// CAP: the largest work item (elements): kSubElems for fewer than 32 channels, tmp::kTrPackBigElems
// for 32 to tmp::kTrPackBigC (16-byte strided rows only; items of 32 positions or more, so that
// each item's packed block starts and ends on a 128-byte line), whose LDS holds C rows of S + 1.
template <int CAP>
constexpr int packed_stage() { return CAP == kSubElems ? kStage : CAP + 2 * tmp::kTrPackBigC; }

template <int MODE, bool V, int CAP = kSubElems>
__global__ __launch_bounds__(kTrBlock) void transpose_packed(PackedArgs a) {
    static_assert(CAP == kSubElems || V, "large work items move the strided side in 16-byte chunks");
    constexpr int W = V ? 4 : 1;                       // strided side: elements per chunk
    constexpr int KS = CAP / W / kTrBlock;             // strided chunks per thread (at most)
    constexpr int KF = CAP / 4 / kTrBlock;             // packed 16-byte chunks per thread (at most)
    __shared__ float tile[packed_stage<CAP>()];
    const int t = threadIdx.x;
    const int S = 1 << a.log_s, pad = S + 1;
    const int lcs = a.log_s - (V ? 2 : 0);             // log2 of the strided chunks per channel row
    const int C = static_cast<int>(a.k);
    const int nstr = C << lcs;                         // strided chunks of a work item
    for (uint32_t w = blockIdx.x; w < a.nwork; w += gridDim.x) {
        const uint32_t b = fast_div(w, a.c_s, a.subs), ps = w - b * a.subs;
        const int64_t p0 = int64_t(ps) << a.log_s;
        const int L = static_cast<int>(a.P - p0 < S ? a.P - p0 : S);  // live positions
        const int nflat = L * C;                                       // live packed elements
        // strided side: channel row ch, positions p0 + pc .. (x rows in MODE 0, y rows in MODE 1)
        auto strided_at = [&](int ch, int pc) {
            if constexpr (MODE == 0)
                return a.x + int64_t(b) * a.bsx + int64_t(ch) * a.ldx + p0 + pc;
            else
                return a.y + int64_t(b) * a.bsy + int64_t(ch) * a.ldy + p0 + pc;
        };
        // packed side: the block of nflat floats at position p0
        auto packed_at = [&](int o) {
            if constexpr (MODE == 0)
                return a.y + int64_t(b) * a.bsy + p0 * C + o;
            else
                return a.x + int64_t(b) * a.bsx + p0 * C + o;
        };
        if constexpr (MODE == 0) {
            float v[KS][W];
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int e = t + k * kTrBlock;
                const int ch = e >> lcs, pc = (e & ((1 << lcs) - 1)) * W;
#pragma unroll
                for (int i = 0; i < W; ++i)
                    v[k][i] = 0.0f;
                if (e < nstr && pc < L) {
                    const float *p = strided_at(ch, pc);
                    if (V && pc + 4 <= L) {
                        const f4 q = ld16_nt(p);
                        v[k][0] = q.x, v[k][1] = q.y, v[k][2] = q.z, v[k][3] = q.w;
                    } else {
#pragma unroll
                        for (int i = 0; i < W; ++i)
                            if (pc + i < L)
                                v[k][i] = ld4_nt(p + i);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int e = t + k * kTrBlock;
                const int ch = e >> lcs, pc = (e & ((1 << lcs) - 1)) * W;
                if (e < nstr) {
#pragma unroll
                    for (int i = 0; i < W; ++i)
                        tile[ch * pad + pc + i] = v[k][i];
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                const int o = 4 * (t + k * kTrBlock);
                if (o < nflat) {
                    uint32_t j = fast_div(uint32_t(o), a.c_k, a.k);  // position
                    uint32_t i = uint32_t(o) - j * a.k;              // channel
                    float r[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        r[q] = tile[i * pad + j];
                        if (++i == a.k) {
                            i = 0;
                            ++j;
                        }
                    }
                    float *p = packed_at(o);
                    if (a.flat16 && o + 4 <= nflat) {
                        st16_nt(p, f4{r[0], r[1], r[2], r[3]});
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (o + q < nflat)
                                st4_nt(p + q, r[q]);
                    }
                }
            }
        } else {
            float r[KF][4];
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                const int o = 4 * (t + k * kTrBlock);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    r[k][q] = 0.0f;
                if (o < nflat) {
                    const float *p = packed_at(o);
                    if (a.flat16 && o + 4 <= nflat) {
                        const f4 f = ld16_nt(p);
                        r[k][0] = f.x, r[k][1] = f.y, r[k][2] = f.z, r[k][3] = f.w;
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (o + q < nflat)
                                r[k][q] = ld4_nt(p + q);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                const int o = 4 * (t + k * kTrBlock);
                if (o < nflat) {
                    uint32_t j = fast_div(uint32_t(o), a.c_k, a.k);
                    uint32_t i = uint32_t(o) - j * a.k;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (o + q < nflat)
                            tile[i * pad + j] = r[k][q];
                        if (++i == a.k) {
                            i = 0;
                            ++j;
                        }
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int e = t + k * kTrBlock;
                const int ch = e >> lcs, pc = (e & ((1 << lcs) - 1)) * W;
                if (e < nstr && pc < L) {
                    float *p = strided_at(ch, pc);
                    if (V && pc + 4 <= L) {
                        st16_nt(p, f4{tile[ch * pad + pc], tile[ch * pad + pc + 1], tile[ch * pad + pc + 2],
                                      tile[ch * pad + pc + 3]});
                    } else {
#pragma unroll
                        for (int i = 0; i < W; ++i)
                            if (pc + i < L)
                                st4_nt(p + i, tile[ch * pad + pc + i]);
                    }
                }
            }
        }
        if (w + gridDim.x < a.nwork)
            __syncthreads();  // the next work item reuses the LDS tile (uniform test)
    }
}

hipError_t launch_packed(const tmp::TransposePlan &p, hipStream_t stream) {
    PackedArgs a;
    a.x = p.x;
    a.y = p.y;
    a.ldx = p.ldx;
    a.ldy = p.ldy;
    a.bsx = p.bsx;
    a.bsy = p.bsy;
    const bool m0 = p.packed == 1;
    a.P = m0 ? p.N : p.M;
    a.k = static_cast<uint32_t>(m0 ? p.M : p.N);
    a.subs = m0 ? p.subs_n : p.subs_m;
    a.c_s = tmp::make_div32(a.subs).c;
    a.c_k = tmp::make_div32(a.k).c;
    a.nwork = static_cast<uint32_t>(p.nwork);
    a.log_s = tmp::ilog2(m0 ? p.sn : p.sm);
    a.flat16 = p.flat16 ? 1 : 0;
    void *args[] = {&a};
    const void *fn = p.pbig ? (m0 ? reinterpret_cast<const void *>(&transpose_packed<0, true, tmp::kTrPackBigElems>)
                                  : reinterpret_cast<const void *>(&transpose_packed<1, true, tmp::kTrPackBigElems>))
                     : m0 ? (p.pvec ? reinterpret_cast<const void *>(&transpose_packed<0, true>)
                                    : reinterpret_cast<const void *>(&transpose_packed<0, false>))
                          : (p.pvec ? reinterpret_cast<const void *>(&transpose_packed<1, true>)
                                    : reinterpret_cast<const void *>(&transpose_packed<1, false>));
    return hipLaunchKernel(fn, dim3(p.grid), dim3(kTrBlock), args, 0, stream);
}

template <bool WIDE, bool PACK>
const void *pick(const tmp::TransposePlan &p) {
    if constexpr (!PACK && !WIDE) {
        if (p.skew)  // y rows off the line grid: line-aligned y windows
            return p.vx ? reinterpret_cast<const void *>(&transpose_skew<true>)
                        : reinterpret_cast<const void *>(&transpose_skew<false>);
    }
    if (!PACK && !p.vy && p.sub == 2 * kSubElems)  // y rows off the 16-byte grid: 64 x 32 sub-tiles
        return p.vx ? reinterpret_cast<const void *>(&transpose_tiles<true, false, false, kTrBlock, WIDE, false, 2 * kSubElems>)
                    : reinterpret_cast<const void *>(&transpose_tiles<false, false, false, kTrBlock, WIDE, false, 2 * kSubElems>);
    if (p.vx && p.vy)
        return p.aligned ? reinterpret_cast<const void *>(&transpose_tiles<true, true, true, kTrBlock, WIDE, PACK>)
                         : reinterpret_cast<const void *>(&transpose_tiles<true, true, false, kTrBlock, WIDE, PACK>);
    if (p.vx)
        return reinterpret_cast<const void *>(&transpose_tiles<true, false, false, kTrBlock, WIDE, PACK>);
    if (p.vy)
        return reinterpret_cast<const void *>(&transpose_tiles<false, true, false, kTrBlock, WIDE, PACK>);
    return reinterpret_cast<const void *>(&transpose_tiles<false, false, false, kTrBlock, WIDE, PACK>);
}

}  // namespace

hipError_t launch_transpose(const tmp::TransposePlan &p, hipStream_t stream) {
    if (p.packed != 0)
        return launch_packed(p, stream);
    TrArgs a;
    a.x = p.x;
    a.y = p.y;
    a.ldx = p.ldx;
    a.ldy = p.ldy;
    a.bsx = p.bsx;
    a.bsy = p.bsy;
    a.M = p.M;
    a.N = p.N;
    a.log_sm = tmp::ilog2(p.sm);
    a.log_sn = tmp::ilog2(p.sn);
    a.subs_m = p.subs_m;
    a.subs_n = p.subs_n;
    a.per_b = p.per_b.d;
    a.c_pb = p.per_b.c;
    a.c_m = p.by_m.c;
    a.c_n = p.by_n.c;
    a.nwork = p.nwork;
    a.log_g = p.skew ? p.log_grp : p.log_g;
    a.B = p.B;
    const void *fn = p.log_g > 0 ? (p.wide ? pick<true, true>(p) : pick<false, true>(p))
                                 : (p.wide ? pick<true, false>(p) : pick<false, false>(p));
    void *args[] = {&a};
    return hipLaunchKernel(fn, dim3(p.grid), dim3(kTrBlock), args, 0, stream);
}

}  // namespace tmk
