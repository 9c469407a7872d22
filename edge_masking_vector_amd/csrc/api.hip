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

TM_API int tm_plan_tiles(int64_t M, int64_t N, int TM, int TN, int64_t *tiles_m, int64_t *tiles_n,
                         int64_t *whole) {
    return tmp::plan_tiles(M, N, TM, TN, tiles_m, tiles_n, whole);
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
