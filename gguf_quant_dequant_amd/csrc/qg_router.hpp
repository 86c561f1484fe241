// qg_router.hpp -- the router kernels of the MoE FFN and the stand-alone
// routing kernel.  These kernels are not templates, so this header is
// included by the one translation unit that launches them (qg_api.hip).
#pragma once

#include "qg_kernels.hpp"

namespace qg {

__global__ void __launch_bounds__(64) route_topk_kernel(const double *logits, int E, int k,
                                                        int *sel, float *w) {
    __shared__ RouteLds s_rt;
    route_topk_wave(logits, E, k, sel, w, &s_rt);
}

// The routing of T tokens ahead of the grouped gate/up products on the
// matrix cores, once for all their workgroups (at more than four tokens the
// workgroups outnumber what the device holds at once, and routing in each
// of them would repeat it): workgroup t, one wave, routes token t (the
// single-token routing, bit for bit) and writes its routes and weights to
// the workspace and the optional outputs.
__global__ void __launch_bounds__(64) moe_route_tokens_kernel(const double *logits, int E, int K,
                                                              int *sel, float *w, int *sel_out,
                                                              float *w_out) {
    __shared__ RouteLds s_rt;
    __shared__ int s_sel[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    const int64_t t = blockIdx.x;
    const int lane = threadIdx.x;
    route_topk_wave(logits + t * E, E, K, s_sel, s_w, &s_rt);
    __syncthreads();
    if (lane < K) {
        const int64_t i = t * K + lane;
        sel[i] = s_sel[lane];
        w[i] = s_w[lane];
        if (sel_out) sel_out[i] = s_sel[lane];
        if (w_out) w_out[i] = s_w[lane];
    }
}

// ------------------------------------------------------------------ MoE K1

// logits[e] = sum_i R[e][i] * x[i]: every f32*f32 product is exact in f64
// and the sum is f64 in a fixed order.  One workgroup of RW waves per
// expert row: wave w takes the w-th of RW equal column ranges (whole
// multiples of 256 columns) in rounds of 2048 columns, all loads of a round
// issued before its FMAs, reduces across its lanes with a fixed tree, and
// the RW partial sums are added in wave order.  RW = 1 (one wave per
// expert) is the default: spreading the 128-expert router's rows over 2, 4
// or 8 waves made the MoE chain slower (21.6 -> 21.7 / 21.9 / 22.1 us per
// token), so the router's time is not its per-wave chain of loads and FMAs.
template <int RW>
__global__ void __launch_bounds__(64 * RW) moe_router_kernel(const float *__restrict__ R,
                                                             const float *__restrict__ x, int H,
                                                             double *__restrict__ logits) {
    __shared__ double part[RW];
    const int e = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const rsrc_t rr = make_rsrc(R + (int64_t)e * H, 4u * (uint32_t)H);
    const rsrc_t rx = make_rsrc(x, 4u * (uint32_t)H);
    const int hw = (H + 256 * RW - 1) / (256 * RW) * 256;  // columns per wave
    const int cb = wave * hw, ce = cb + hw < H ? cb + hw : H;
    double acc = 0.0;
    // columns past H (and past the wave's range) read as zero through the
    // resources, or are skipped by the guard below
    for (int c0 = cb; c0 < ce; c0 += 2048) {
        uint32_t a[8][4], b[8][4];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int c = c0 + 256 * i + 4 * lane;
            const uint32_t off = c < ce ? 4u * (uint32_t)c : 0xFFFFFFF0u;
            load_dw<4, QG_ROUTER_AUX>(rr, off, a[i]);
            load_dw<4>(rx, off, b[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
                acc = fma((double)__builtin_bit_cast(float, a[i][j]),
                          (double)__builtin_bit_cast(float, b[i][j]), acc);
    }
    acc = wave_sum_d(acc);
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double sum = part[0];
#pragma unroll
        for (int w = 1; w < RW; w++) sum += part[w];
        logits[e] = sum;
    }
}

// ------------------------------------------------------- MoE K1, with norm
//
// Fused residual add + RMSNorm + router (web page: docs.rs, crate
// ferrox-cuda 0.14.0, src/gpu.rs, FUSED_ADD_RMSNORM_KERNEL_SRC; the
// aprender-serve page's moe_layer runs the norm before its router).  One
// wave per expert, as moe_router_kernel.  Every wave forms h = a + b (f32)
// and reduces sum h^2 in f64 with the same fixed tree, so all waves hold
// the same inv = 1 / sqrt(sum / H + eps) without a grid-wide step; then
// xn = (h * inv) * gamma in f64, rounded to f32, and
// logits[e] = sum_i R[e][i] * xn[i] in f64.  Wave 0 also stores xn (to the
// workspace, and to xn_out when given).
__global__ void __launch_bounds__(64) moe_norm_router_kernel(
    const float *__restrict__ R, const float *__restrict__ a, const float *__restrict__ b,
    const float *__restrict__ gamma, double eps, int H, double *__restrict__ logits,
    float *__restrict__ xn_ws, float *__restrict__ xn_out) {
    const int e = blockIdx.x, lane = threadIdx.x;
    const uint32_t hb = 4u * (uint32_t)H;
    const rsrc_t rr = make_rsrc(R + (int64_t)e * H, hb);
    const rsrc_t ra = make_rsrc(a, hb), rb = make_rsrc(b, hb), rg = make_rsrc(gamma, hb);
    double acc = 0.0;
    if (H <= 2048) {
        // one round: every load of the wave (router row, both inputs, the
        // norm weight) goes out before the first use; columns past H read
        // as zero through the resources
        uint32_t vr[8][4], va[8][4], vb[8][4], vg[8][4];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t c = 256u * i + 4u * lane;
            load_dw<4>(ra, 4u * c, va[i]);
            load_dw<4>(rb, 4u * c, vb[i]);
            load_dw<4>(rr, 4u * c, vr[i]);
            load_dw<4>(rg, 4u * c, vg[i]);
        }
        float h[8][4];
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                h[i][j] =
                    __builtin_bit_cast(float, va[i][j]) + __builtin_bit_cast(float, vb[i][j]);
                ss = fma((double)h[i][j], (double)h[i][j], ss);
            }
        ss = wave_sum_d(ss);
        const double inv = 1.0 / sqrt(ss / (double)H + eps);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int c = 256 * i + 4 * lane;
            float xn[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                xn[j] = (float)(((double)h[i][j] * inv) *
                                (double)__builtin_bit_cast(float, vg[i][j]));
                acc = fma((double)__builtin_bit_cast(float, vr[i][j]), (double)xn[j], acc);
            }
            if (e == 0 && c < H) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    xn_ws[c + j] = xn[j];
                    if (xn_out) xn_out[c + j] = xn[j];
                }
            }
        }
    } else {
        // sum of squares over rounds of 2048 columns, then the router dot
        // over rounds of 1024 (the inputs are read twice, from cache)
        double ss = 0.0;
        for (int c0 = 0; c0 < H; c0 += 2048) {
            uint32_t va[8][4], vb[8][4];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int c = c0 + 256 * i + 4 * lane;
                load_dw<4>(ra, 4u * c, va[i]);
                load_dw<4>(rb, 4u * c, vb[i]);
            }
#pragma unroll
            for (int i = 0; i < 8; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float h = __builtin_bit_cast(float, va[i][j]) +
                                    __builtin_bit_cast(float, vb[i][j]);
                    ss = fma((double)h, (double)h, ss);
                }
        }
        ss = wave_sum_d(ss);
        const double inv = 1.0 / sqrt(ss / (double)H + eps);
        for (int c0 = 0; c0 < H; c0 += 1024) {
            uint32_t vr[4][4], va[4][4], vb[4][4], vg[4][4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int c = c0 + 256 * i + 4 * lane;
                load_dw<4>(rr, 4u * c, vr[i]);
                load_dw<4>(ra, 4u * c, va[i]);
                load_dw<4>(rb, 4u * c, vb[i]);
                load_dw<4>(rg, 4u * c, vg[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int c = c0 + 256 * i + 4 * lane;
                float xn[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float h = __builtin_bit_cast(float, va[i][j]) +
                                    __builtin_bit_cast(float, vb[i][j]);
                    xn[j] = (float)(((double)h * inv) *
                                    (double)__builtin_bit_cast(float, vg[i][j]));
                    acc = fma((double)__builtin_bit_cast(float, vr[i][j]), (double)xn[j], acc);
                }
                if (e == 0 && c < H) {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        xn_ws[c + j] = xn[j];
                        if (xn_out) xn_out[c + j] = xn[j];
                    }
                }
            }
        }
    }
    acc = wave_sum_d(acc);
    if (lane == 0) logits[e] = acc;
}

// logits[t][e] = sum_i R[e][i] * x[t][i] in f64: one wave per expert; the
// router row is read once for all T tokens.
__global__ void __launch_bounds__(64) moe_router_tokens_kernel(const float *__restrict__ R,
                                                               const float *__restrict__ x,
                                                               int T, int H, int E,
                                                               double *__restrict__ logits) {
    const int e = blockIdx.x, lane = threadIdx.x;
    const rsrc_t rr = make_rsrc(R + (int64_t)e * H, 4u * (uint32_t)H);
    // one resource per token, each ending at its token's last column, so a
    // column past H reads zero and never the next token's activations
    rsrc_t rx[8];
#pragma unroll
    for (int t = 0; t < 8; t++) rx[t] = make_rsrc(x + (int64_t)(t < T ? t : 0) * H, 4u * (uint32_t)H);
    double acc[8];
#pragma unroll
    for (int t = 0; t < 8; t++) acc[t] = 0.0;
    // rounds of 1024 columns: the router row's and all T tokens' loads of a
    // round are issued before its FMAs; columns past H read as zero (H is a
    // multiple of 4, so a 16-byte load is either wholly inside or outside)
    for (int c0 = 0; c0 < H; c0 += 1024) {
        uint32_t a[4][4], b[8][4][4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t c = (uint32_t)c0 + 256u * i + 4u * lane;
            load_dw<4>(rr, 4u * c, a[i]);
#pragma unroll
            for (int t = 0; t < 8; t++)
                if (t < T) load_dw<4>(rx[t], 4u * c, b[t][i]);
        }
#pragma unroll
        for (int t = 0; t < 8; t++)
            if (t < T)
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        acc[t] = fma((double)__builtin_bit_cast(float, a[i][j]),
                                     (double)__builtin_bit_cast(float, b[t][i][j]), acc[t]);
    }
#pragma unroll
    for (int t = 0; t < 8; t++) {
        if (t < T) {
            const double v = wave_sum_d(acc[t]);
            if (lane == 0) logits[(int64_t)t * E + e] = v;
        }
    }
}

}  // namespace qg
