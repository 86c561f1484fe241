// qg_moe.hip -- launch of the MoE FFN kernels (gate/up + SwiGLU, down +
// residual; several-token gate/up).
#include "qg_moe_host.hpp"

namespace qg {
namespace host {

// Several tokens: B activation vectors per tile (tokens past T are zero),
// tile widths of the batch-B GEMV.
template <class F, int B>
int launch_gateup_tokens(MoeParams p, hipStream_t st) {
    constexpr int U = 2;
    Shape s;
    p.gu_tiles = p.H / F::CPT;
    if (p.H % F::CPT != 0 || !shape_for(p.gu_tiles, &s))
        return fail(QG_EUNSUPPORTED, "moe_ffn_tokens: hidden %d does not fit the gate/up kernel",
                    p.H);
    p.gu_lpr = s.lpr;
    p.gu_S = s.S;
    p.gu_G = s.G;
    // at most T * K distinct experts
    const int64_t tasks = (int64_t)p.T * p.K * p.F, per = (int64_t)s.G * U;
    const int64_t iters = (tasks + per - 1) / per;
    const size_t lds = (size_t)kStageChunks * 16 * s.threads;
    const int grid =
        resident_grid((const void *)moe_gateup_tokens_kernel<F, B, U>, s.threads, lds, iters);
    hipLaunchKernelGGL((moe_gateup_tokens_kernel<F, B, U>), dim3(grid), dim3(s.threads), lds, st,
                       p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "moe_ffn_tokens: gate/up launch failed: %s",
                    hipGetErrorString(e));
    return QG_OK;
}

template <int B>
int dispatch_gateup_tokens_b(int fmt, const MoeParams &p, hipStream_t st) {
    constexpr int K45 = lw_k45(B), Q6 = lw_q6k(B), Q8 = lw_q80(B), Q4 = lw_q40(B);
    switch (fmt) {
    case QG_Q4_K: return launch_gateup_tokens<FmtQ4K<K45, true>, B>(p, st);
    case QG_Q5_K: return launch_gateup_tokens<FmtQ5K<K45, true>, B>(p, st);
    case QG_Q6_K: return launch_gateup_tokens<FmtQ6K<Q6, false>, B>(p, st);
    case QG_Q8_0: return launch_gateup_tokens<FmtQ80<Q8>, B>(p, st);
    case QG_Q4_0: return launch_gateup_tokens<FmtQ40<Q4>, B>(p, st);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn_tokens: gate/up format %d", fmt);
    }
}

// Tokens in groups of at most four, each group one launch of the B = 4
// kernel (its own routing, distinct experts and activations).  At B = 8 the
// tile is narrower (two waves per row group, one row per group and
// iteration) and the kernel ran 5x slower than two B = 4 groups, whose
// second pass re-reads the experts the groups share.
int dispatch_gateup_tokens(int fmt, const MoeParams &p0, hipStream_t st) {
    for (int t0 = 0; t0 < p0.T; t0 += 4) {
        MoeParams p = p0;
        p.T = p0.T - t0 < 4 ? p0.T - t0 : 4;
        p.x += (int64_t)t0 * p.H;
        p.logits += (int64_t)t0 * p.E;
        p.ws_sel += (int64_t)t0 * p.K;
        p.ws_w += (int64_t)t0 * p.K;
        p.act += (int64_t)t0 * p.K * p.F;
        if (p.sel_out) p.sel_out += (int64_t)t0 * p.K;
        if (p.w_out) p.w_out += (int64_t)t0 * p.K;
        const int rc = dispatch_gateup_tokens_b<4>(fmt, p, st);
        if (rc != QG_OK) return rc;
    }
    return QG_OK;
}

int dispatch_gateup(int fmt, const MoeParams &p, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_gateup<FmtQ4K<32, true>>(p, st);
    case QG_Q5_K: return launch_gateup<FmtQ5K<32, true>>(p, st);
    case QG_Q6_K: return launch_gateup<FmtQ6K<16, false>>(p, st);
    case QG_Q8_0: return launch_gateup<FmtQ80<32>>(p, st);
    case QG_Q4_0: return launch_gateup<FmtQ40<16>>(p, st);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn: gate/up format %d", fmt);
    }
}

int dispatch_down(int fmt, const MoeParams &p, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_down<FmtQ4K<32, true>>(p, st);
    case QG_Q5_K: return launch_down<FmtQ5K<32, true>>(p, st);
    case QG_Q6_K: return launch_down<FmtQ6K<16, false>>(p, st);
    case QG_Q8_0: return launch_down<FmtQ80<32>>(p, st);
    case QG_Q4_0: return launch_down<FmtQ40<16>>(p, st);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn: down format %d", fmt);
    }
}

}  // namespace host
}  // namespace qg
