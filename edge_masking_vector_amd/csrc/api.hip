// api.hip -- the extern "C" entry points of libtilemap.so (declared in include/tilemap.h).
//
// Every call validates on the host first (plan.cpp: argument checks, the alignment-promise check,
// the loop split and the tile schedule); only a valid plan with work reaches a launch.  A refused
// launch maps to TM_E_HIP.
#include <hip/hip_runtime_api.h>

#include "launch.h"
#include "plan.h"

#define TM_API extern "C" __attribute__((visibility("default")))

namespace {

int launched(hipError_t err) { return err == hipSuccess ? TM_OK : TM_E_HIP; }

int run_map(int op, const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
            float alpha, float beta, int TM, int TN, int aligned, int variant, void *stream) {
    tmp::MapPlan plan;
    const int st = tmp::plan_map(op, x, ldx, y, ldy, M, N, alpha, beta, TM, TN, aligned, variant,
                                 &plan);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_map(plan, static_cast<hipStream_t>(stream)));
}

}  // namespace

TM_API int tm_map_affine(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                         float alpha, float beta, int TM, int TN, int aligned, int variant,
                         void *stream) {
    return run_map(tmp::kAffine, x, ldx, y, ldy, M, N, alpha, beta, TM, TN, aligned, variant, stream);
}

TM_API int tm_scale2d(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                      float alpha, int TM, int TN, int aligned, int variant, void *stream) {
    return run_map(tmp::kScale, x, ldx, y, ldy, M, N, alpha, 0.0f, TM, TN, aligned, variant, stream);
}

TM_API int tm_copy2d(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                     int TM, int TN, int aligned, int variant, void *stream) {
    return run_map(tmp::kCopy, x, ldx, y, ldy, M, N, 0.0f, 0.0f, TM, TN, aligned, variant, stream);
}

TM_API int tm_channel_affine(const float *x, int64_t ldx, const float *scale, const float *bias,
                             float *y, int64_t ldy, int64_t M, int64_t N, int TM, int TN, int aligned,
                             int variant, void *stream) {
    tmp::MapPlan plan;
    const int st = tmp::plan_map(tmp::kChannel, x, ldx, y, ldy, M, N, 0.0f, 0.0f, TM, TN, aligned,
                                 variant, &plan, scale, bias);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_map(plan, static_cast<hipStream_t>(stream)));
}

TM_API int tm_rowsum(const float *x, int64_t ldx, float *out, int64_t M, int64_t N, int TM, int TN,
                     int aligned, void *stream) {
    tmp::RowPlan plan;
    const int st = tmp::plan_rows(tmp::kRowSum, x, ldx, out, M, N, TM, TN, aligned, &plan);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_rows(plan, static_cast<hipStream_t>(stream)));
}

TM_API int tm_rowmax_masked(const float *s, int64_t lds, float *out, int64_t M, int64_t N, int BR,
                            int BC, int aligned, void *stream) {
    tmp::RowPlan plan;
    const int st = tmp::plan_rows(tmp::kRowMax, s, lds, out, M, N, BR, BC, aligned, &plan);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_rows(plan, static_cast<hipStream_t>(stream)));
}

TM_API int tm_softmax_stats(const float *s, int64_t lds, float *m, float *l, int64_t M, int64_t N,
                            int BR, int BC, int aligned, void *stream) {
    tmp::RowPlan plan;
    const int st = tmp::plan_rows(tmp::kRowSoftmax, s, lds, m, M, N, BR, BC, aligned, &plan, l);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_rows(plan, static_cast<hipStream_t>(stream)));
}

TM_API size_t tm_rows_workspace_bytes(int64_t M, int64_t N) { return tmp::rows_ws_bytes(M, N); }

TM_API int tm_rowsum_ws(const float *x, int64_t ldx, float *out, int64_t M, int64_t N, int TM, int TN,
                        int aligned, void *ws, size_t ws_bytes, void *stream) {
    tmp::RowPlan plan;
    const int st = tmp::plan_rows(tmp::kRowSum, x, ldx, out, M, N, TM, TN, aligned, &plan, nullptr,
                                  true, ws, ws_bytes);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_rows(plan, static_cast<hipStream_t>(stream)));
}

TM_API int tm_rowmax_masked_ws(const float *s, int64_t lds, float *out, int64_t M, int64_t N, int BR,
                               int BC, int aligned, void *ws, size_t ws_bytes, void *stream) {
    tmp::RowPlan plan;
    const int st = tmp::plan_rows(tmp::kRowMax, s, lds, out, M, N, BR, BC, aligned, &plan, nullptr,
                                  true, ws, ws_bytes);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_rows(plan, static_cast<hipStream_t>(stream)));
}

TM_API int tm_softmax_stats_ws(const float *s, int64_t lds, float *m, float *l, int64_t M, int64_t N,
                               int BR, int BC, int aligned, void *ws, size_t ws_bytes, void *stream) {
    tmp::RowPlan plan;
    const int st = tmp::plan_rows(tmp::kRowSoftmax, s, lds, m, M, N, BR, BC, aligned, &plan, l, true,
                                  ws, ws_bytes);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_rows(plan, static_cast<hipStream_t>(stream)));
}

TM_API size_t tm_colsum_workspace_bytes(int64_t M, int64_t N, int TM, int TN, int walk) {
    return tmp::colsum_ws_bytes(M, N, TM, TN, walk);
}

TM_API int tm_colsum(const float *x, int64_t ldx, float *out, int64_t M, int64_t N, int TM, int TN,
                     int aligned, int walk, void *ws, size_t ws_bytes, void *stream) {
    tmp::ColPlan plan;
    const int st = tmp::plan_cols(x, ldx, out, M, N, TM, TN, aligned, walk, ws, ws_bytes, &plan);
    if (st != TM_OK || !plan.finish)
        return st;
    return launched(tmk::launch_cols(plan, static_cast<hipStream_t>(stream)));
}

TM_API int tm_col_walk(const void *x, int64_t ldx, const void *out, int64_t M, int64_t N, int TM, int TN,
                       int aligned, int walk, const void *ws, size_t ws_bytes, int *form, int64_t *slab_rows,
                       int64_t *strip_cols, int64_t *slabs, int64_t *strips) {
    if (form == nullptr || slab_rows == nullptr || strip_cols == nullptr || slabs == nullptr || strips == nullptr)
        return TM_E_INVAL;
    tmp::ColPlan plan;
    const int st = tmp::plan_cols(static_cast<const float *>(x), ldx, static_cast<float *>(const_cast<void *>(out)),
                                  M, N, TM, TN, aligned, walk, const_cast<void *>(ws), ws_bytes, &plan);
    if (st != TM_OK)
        return st;
    if (!plan.finish) {
        *form = TM_COLFORM_NONE;
        *slab_rows = *strip_cols = *slabs = *strips = 0;
    } else if (plan.direct) {
        *form = TM_COLFORM_ONE_PASS;
        *slab_rows = M;
        *strip_cols = plan.vec ? 4 : 1;
        *slabs = 1;
        *strips = (N + *strip_cols - 1) / *strip_cols;
    } else {
        *form = plan.strip ? TM_COLFORM_STRIPS : TM_COLFORM_TILES;
        *slab_rows = plan.launch ? int64_t{1} << plan.log_tm : 0;
        *strip_cols = plan.walk == TM_COL_LDS ? plan.tw : 1;
        *slabs = plan.launch ? int64_t(plan.slabs) : 0;
        *strips = int64_t(plan.strips);
    }
    return TM_OK;
}

TM_API int tm_transpose(const float *x, int64_t ldx, int64_t bsx, float *y, int64_t ldy, int64_t bsy,
                        int64_t B, int64_t M, int64_t N, int TM, int TN, int aligned, void *stream) {
    tmp::TransposePlan plan;
    const int st = tmp::plan_transpose(x, ldx, bsx, y, ldy, bsy, B, M, N, TM, TN, aligned, &plan);
    if (st != TM_OK || !plan.launch)
        return st;
    return launched(tmk::launch_transpose(plan, static_cast<hipStream_t>(stream)));
}

TM_API int tm_check_promise(int64_t M, int64_t N, int64_t ld_in, int64_t ld_out, int TM, int TN,
                            const void *in, const void *out) {
    return tmp::check_promise(M, N, ld_in, ld_out, TM, TN, in, out);
}

TM_API int tm_split(int64_t K, int64_t T, int64_t *nfull, int64_t *rem) {
    return tmp::split(K, T, nfull, rem);
}

TM_API int tm_row_walk(int64_t M, int64_t N, int64_t ld, int BR, int BC, int aligned, const void *x,
                       int64_t *bc, int64_t *nfull, int64_t *rem, int *lanes) {
    return tmp::row_walk_query(M, N, ld, BR, BC, aligned, x, bc, nfull, rem, lanes);
}

TM_API int tm_map_walk(int op, const void *x, int64_t ldx, const void *y, int64_t ldy, int64_t M, int64_t N,
                       int TM, int TN, int aligned, int variant, const void *bias, int *walk, int64_t *items) {
    if (op < tmp::kAffine || op > tmp::kChannel || walk == nullptr || items == nullptr)
        return TM_E_INVAL;
    tmp::MapPlan plan;
    const float *xf = static_cast<const float *>(x);
    float *yf = static_cast<float *>(const_cast<void *>(y));
    const int st = tmp::plan_map(op, xf, ldx, yf, ldy, M, N, 1.0f, 0.0f, TM, TN, aligned, variant, &plan, nullptr,
                                 op == tmp::kChannel ? static_cast<const float *>(bias) : nullptr);
    if (st != TM_OK)
        return st;
    // (the channel op over contiguous rows is one flat row too, its channel the flat column mod C)
    *walk = !plan.launch                    ? TM_MAP_NONE
            : plan.flat || plan.chan_n != 0 ? TM_MAP_FLAT
            : plan.rows                     ? TM_MAP_SPAN
                                            : TM_MAP_TILES;
    *items = plan.launch ? int64_t(plan.nwork) : 0;
    return TM_OK;
}

TM_API int tm_plan_tiles(int64_t M, int64_t N, int TM, int TN, int64_t *tiles_m, int64_t *tiles_n,
                         int64_t *whole) {
    return tmp::plan_tiles(M, N, TM, TN, tiles_m, tiles_n, whole);
}

TM_API int tm_pad_extents(int64_t M, int64_t N, int TM, int TN, int64_t *Mp, int64_t *Np,
                          int64_t *ldp) {
    return tmp::pad_extents(M, N, TM, TN, Mp, Np, ldp);
}

TM_API int tm_autotune_map(int op, const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M,
                           int64_t N, float alpha, float beta, int aligned, int variant, int reps,
                           void *ev_start, void *ev_stop, int *TM_best, int *TN_best, float *us_best,
                           float *table, void *stream) {
    if (op < tmp::kAffine || op > tmp::kCopy || reps < 1 || ev_start == nullptr ||
        ev_stop == nullptr || TM_best == nullptr || TN_best == nullptr || us_best == nullptr)
        return TM_E_INVAL;
    if (x != nullptr && x == y)
        return TM_E_INVAL;  // the op runs many times: it must read the same input each time
    constexpr int kRowsT = 9, kColsT = 11;  // TM = 2^0..2^8, TN = 2^0..2^10
    // Validate the shared arguments once, with a tile every call accepts.
    tmp::MapPlan plan;
    int st = tmp::plan_map(op, x, ldx, y, ldy, M, N, alpha, beta, 1, 4, 0, variant, &plan);
    if (st != TM_OK && st != TM_E_ALIGN && st != TM_E_UNSUPPORTED)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
    float best = -1.0f;
    int best_tm = 0, best_tn = 0;
    for (int i = 0; i < kRowsT; ++i) {
        for (int j = 0; j < kColsT; ++j) {
            const int TM = 1 << i, TN = 1 << j;
            float us = -1.0f;
            st = tmp::plan_map(op, x, ldx, y, ldy, M, N, alpha, beta, TM, TN, aligned, variant, &plan);
            if (st == TM_OK && plan.launch) {
                if (tmk::launch_map(plan, s) != hipSuccess)  // warm-up
                    return TM_E_HIP;
                if (hipEventRecord(e0, s) != hipSuccess)
                    return TM_E_HIP;
                for (int r = 0; r < reps; ++r)
                    if (tmk::launch_map(plan, s) != hipSuccess)
                        return TM_E_HIP;
                float ms = 0.0f;
                if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                    hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
                    return TM_E_HIP;
                us = ms * 1000.0f / reps;
                if (best < 0.0f || us < best) {
                    best = us;
                    best_tm = TM;
                    best_tn = TN;
                }
            } else if (st == TM_OK) {
                us = 0.0f;  // valid call with no work (M or N is 0)
                if (best < 0.0f) {
                    best = 0.0f;
                    best_tm = TM;
                    best_tn = TN;
                }
            }
            if (table != nullptr)
                table[i * kColsT + j] = us;
        }
    }
    if (best < 0.0f)
        return TM_E_ALIGN;  // no tile of the menu is accepted (under the promise: none keeps it)
    *TM_best = best_tm;
    *TN_best = best_tn;
    *us_best = best;
    return TM_OK;
}

TM_API const char *tm_status_string(int status) {
    switch (status) {
    case TM_OK: return "TM_OK";
    case TM_E_INVAL: return "TM_E_INVAL";
    case TM_E_ALIGN: return "TM_E_ALIGN";
    case TM_E_UNSUPPORTED: return "TM_E_UNSUPPORTED";
    case TM_E_WORKSPACE: return "TM_E_WORKSPACE";
    case TM_E_HIP: return "TM_E_HIP";
    default: return "unknown status";
    }
}
