// qg_moe_host.hpp -- launch of the MoE FFN's gate/up + SwiGLU and down +
// residual kernels for one format (shared by the exact and the
// int8-activation translation units).
#pragma once

#include "qg_host.hpp"

namespace qg {
namespace host {

template <class F>
int launch_gateup(MoeParams p, hipStream_t st) {
    constexpr int U = QG_MOE_GU_U;
    Shape s;
    p.gu_tiles = p.H / F::CPT;
    if (!shape_for(p.gu_tiles, &s))
        return fail(QG_EUNSUPPORTED, "moe_ffn: hidden %d too wide for the gate/up kernel", p.H);
    if (QG_MOE_GU_T128 && s.S == 1 && s.G >= 2) {
        s.G /= 2;
        s.threads = 128;
    }
    p.gu_lpr = s.lpr;
    p.gu_S = s.S;
    p.gu_G = s.G;
    const int64_t tasks = (int64_t)p.K * p.F, per = (int64_t)s.G * U;
    const int64_t iters = (tasks + per - 1) / per;
    const size_t lds = (size_t)kStageChunks * 16 * s.threads;
    const int grid = resident_grid((const void *)moe_gateup_kernel<F, U>, s.threads, lds, iters);
    hipLaunchKernelGGL((moe_gateup_kernel<F, U>), dim3(grid), dim3(s.threads), lds, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "moe_ffn: gate/up launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

template <class F>
int launch_down(MoeParams p, hipStream_t st) {
    constexpr int U = QG_MOE_DN_U;
    Shape s;
    p.dn_tiles_per_slot = p.F / F::CPT;
    p.dn_tiles = p.K * p.dn_tiles_per_slot;
    if (!shape_for(p.dn_tiles, &s))
        return fail(QG_EUNSUPPORTED, "moe_ffn: top_k * expert_dim too wide for the down kernel");
    if (QG_MOE_DN_T128 && s.S * s.G * 64 > 128 && s.G >= 2) {
        s.G /= 2;
        s.threads /= 2;
    }
    p.dn_lpr = s.lpr;
    p.dn_S = s.S;
    p.dn_G = s.G;
    const int64_t per = (int64_t)s.G * U;
    const int64_t iters = (p.H + per - 1) / per;
    const size_t lds = (size_t)kStageChunks * 16 * s.threads;
    // one grid row per token (blockIdx.y), the resident workgroups shared
    const int64_t cap = (int64_t)device_cus() *
                        resident_per_cu((const void *)moe_down_kernel<F, U>, s.threads, lds);
    int64_t gx = cap / p.T;
    gx = gx < 1 ? 1 : (gx > iters ? iters : gx);
    hipLaunchKernelGGL((moe_down_kernel<F, U>), dim3((unsigned)gx, (unsigned)p.T), dim3(s.threads),
                       lds, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "moe_ffn: down launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace host
}  // namespace qg
