// qg_gemv_host.hpp -- launch of the VALU GEMV kernels (qgemv_lds_kernel,
// qgemv_kernel) for one batch width; instantiated per batch width in
// qg_gemv_b<B>.hip.
#pragma once

#include "qg_host.hpp"

namespace qg {
namespace host {

template <class F, int B, int US>
void launch_staged(const GemvParams &p, const Shape &s, size_t stage_bytes, hipStream_t st) {
    const int64_t per_iter = (int64_t)s.G * US;
    const int64_t iters = (p.rows + per_iter - 1) / per_iter;
    const int64_t xrounds = ((int64_t)B * p.cols + 32 * s.threads - 1) / (32 * s.threads);
    const int grid_xl =
        resident_grid((const void *)qgemv_lds_kernel<F, B, US, true>, s.threads, stage_bytes, iters);
    const int64_t blocks_per_wg = (iters + grid_xl - 1) / grid_xl;
    if (xrounds <= 1 || (xrounds <= QG_XL_ROUNDS && blocks_per_wg <= 2)) {
        hipLaunchKernelGGL((qgemv_lds_kernel<F, B, US, true>), dim3(grid_xl), dim3(s.threads),
                           stage_bytes, st, p);
    } else {
        const int grid = resident_grid((const void *)qgemv_lds_kernel<F, B, US, false>, s.threads,
                                       stage_bytes, iters);
        hipLaunchKernelGGL((qgemv_lds_kernel<F, B, US, false>), dim3(grid), dim3(s.threads),
                           stage_bytes, st, p);
    }
}

template <class F, int B, int U>
int launch_gemv(GemvParams p, hipStream_t st) {
    p.tiles = (int32_t)(p.cols / F::CPT);
    Shape s;
    if (!shape_for(p.tiles, &s))
        return fail(QG_EUNSUPPORTED, "qgemv: %u columns need %d lane tiles per row at batch %d; "
                                     "at most 512 are supported",
                    p.cols, p.tiles, B);
    // Batch 1 with one wave per row (64-lane groups): workgroups of two
    // waves, twice as many of them (Q4_K 4096 x 4096: 5.48 -> 5.39 us).
    if (B == 1 && s.S == 1 && s.lpr == 64) {
        s.G = 2;
        s.threads = 128;
    }
    p.lpr = s.lpr;
    p.S = s.S;
    p.G = s.G;
    // The stage holds kStageChunks 16-byte chunks per thread; a block of
    // G * US rows plus up to 15 bytes of leading alignment and the
    // realigning reads' extra dword past the last field must fit.  Four rows
    // per row group when they fit and the batch is at most 4 (more bytes in
    // flight per workgroup for long rows; at batch 8 the extra accumulators
    // cost occupancy), else two, else the unstaged kernel.
    const size_t stage_bytes = (size_t)kStageChunks * 16 * s.threads;
    auto fits = [&](int us) {
        return QG_STAGE && (size_t)s.G * us * p.row_bytes + 15 + 4 <= stage_bytes;
    };
    if (B <= 4 && fits(4)) {
        launch_staged<F, B, 4>(p, s, stage_bytes, st);
    } else if (fits(2)) {
        launch_staged<F, B, 2>(p, s, stage_bytes, st);
    } else {
        const int64_t per_iter = (int64_t)s.G * U;
        const int64_t iters = (p.rows + per_iter - 1) / per_iter;
        const int grid = resident_grid((const void *)qgemv_kernel<F, B, U>, s.threads, 0, iters);
        hipLaunchKernelGGL((qgemv_kernel<F, B, U>), dim3(grid), dim3(s.threads), 0, st, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ELAUNCH, "qgemv: launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

template <int B>
int dispatch_gemv_b(int fmt, bool aligned, int cpt, const GemvParams &p, hipStream_t st) {
    constexpr int U = B == 1 ? QG_U_B1 : QG_U_BN;
    constexpr int K45 = lw_k45(B), Q6 = lw_q6k(B), Q8 = lw_q80(B), Q4 = lw_q40(B);
    constexpr int FM = lw_f32max(B);
    // at batch >= 2 the block formats run on the matrix cores (qgemv); this
    // kernel takes F32 rows there
    if constexpr (B > 1) {
        if (fmt != QG_F32) return fail(QG_EUNSUPPORTED, "qgemv: internal: format %d at batch %d",
                                       fmt, B);
        if (cpt == FM) return launch_gemv<FmtF32<FM>, B, U>(p, st);
        if constexpr (FM > 8)
            if (cpt == FM / 2) return launch_gemv<FmtF32<FM / 2>, B, U>(p, st);
        if (cpt == 8) return launch_gemv<FmtF32<8>, B, U>(p, st);
        return launch_gemv<FmtF32<4>, B, U>(p, st);
    } else {
        switch (fmt) {
        case QG_Q4_K:
            return aligned ? launch_gemv<FmtQ4K<K45, false>, B, U>(p, st)
                           : launch_gemv<FmtQ4K<K45, true>, B, U>(p, st);
        case QG_Q5_K:
            return aligned ? launch_gemv<FmtQ5K<K45, false>, B, U>(p, st)
                           : launch_gemv<FmtQ5K<K45, true>, B, U>(p, st);
        case QG_Q6_K: return launch_gemv<FmtQ6K<Q6>, B, U>(p, st);
        case QG_Q8_0: return launch_gemv<FmtQ80<Q8>, B, U>(p, st);
        case QG_Q4_0: return launch_gemv<FmtQ40<Q4>, B, U>(p, st);
        case QG_F32:
            if (cpt == FM) return launch_gemv<FmtF32<FM>, B, U>(p, st);
            if constexpr (FM > 8)
                if (cpt == FM / 2) return launch_gemv<FmtF32<FM / 2>, B, U>(p, st);
            if constexpr (FM > 16)
                if (cpt == FM / 4) return launch_gemv<FmtF32<FM / 4>, B, U>(p, st);
            if (cpt == 8) return launch_gemv<FmtF32<8>, B, U>(p, st);
            return launch_gemv<FmtF32<4>, B, U>(p, st);
        default: return fail(QG_EUNSUPPORTED, "qgemv: unknown format %d", fmt);
        }
    }
}

// The int8-activation variant (batch 1): the format's tiles with q8a

}  // namespace host
}  // namespace qg
