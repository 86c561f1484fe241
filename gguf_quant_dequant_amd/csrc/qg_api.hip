// qg_api.hip -- host side of the C ABI declared in include/qgemv.h:
// argument validation (before any HIP call), kernel selection and launch on
// the caller's stream.  No allocation, no host synchronisation.  The kernel
// launches live in qg_gemv_b*.hip, qg_gemv_q8.hip, qg_mx_b*.hip and
// qg_moe.hip.
#include "qg_host.hpp"
#include "qg_router.hpp"

using namespace qg;
using namespace qg::host;

namespace {

// Streaming read of `bytes` bytes (a multiple of 16): every thread issues
// its kLoads 16-byte non-temporal loads of a round before using any, the
// same cache policy as the GEMVs' weight streams; the XOR of everything
// read is stored per workgroup so the loads cannot be dropped.
constexpr int kStreamThreads = 512, kStreamLoads = 4;

__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const uint8_t *buf,
                                                                     uint64_t bytes,
                                                                     uint32_t *out) {
    const uint64_t per_round = (uint64_t)gridDim.x * kStreamThreads * kStreamLoads * 16;
    uint32_t acc = 0;
    for (uint64_t base = (uint64_t)blockIdx.x * kStreamThreads * kStreamLoads * 16; base < bytes;
         base += per_round) {
        const uint64_t rem = bytes - base;
        const rsrc_t r = make_rsrc(buf + base, rem > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)rem);
        uint32_t v[kStreamLoads][4];
#pragma unroll
        for (int j = 0; j < kStreamLoads; j++) {
            const auto w = __builtin_amdgcn_raw_buffer_load_b128(
                r, 16u * (uint32_t)(j * kStreamThreads + (int)threadIdx.x), 0, kStream);
            v[j][0] = w[0]; v[j][1] = w[1]; v[j][2] = w[2]; v[j][3] = w[3];
        }
#pragma unroll
        for (int j = 0; j < kStreamLoads; j++) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    // one word per workgroup: the XOR over its threads
    __shared__ uint32_t red[kStreamThreads / 64];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = 0;
        for (int w = 0; w < kStreamThreads / 64; w++) a ^= red[w];
        out[blockIdx.x] = a;
    }
}

// The matrix-core GEMV with the whole row's activation image in LDS
// (qg_mfma.hpp): batch-1 rows too wide for the VALU kernel, and batch 2..4
// on rows of at most 1024 columns, where the batched kernel splits a row
// over too few waves (at batch 2: Q6_K 4096 x 1024 5.9 us against 8.7,
// Q4_K 4096 x 1024 5.9 against 7.3).  Wider rows at batch 2..4 are faster
// on the batched kernels (at batch 2: Q4_K 4096 x 4096 10.9 -> 7.9 us,
// Q8_0 4096 x 4096 16.7 -> 8.6, Q6_K 4096 x 4096 12.7 -> 9.4, Q4_0 4096 x
// 14336 84 -> 18.3, Q4_K 2048 x 2048 7.5 -> 7.4; Q5_K 4096 x 4096 at
// batch 3 12.7 -> 8.3).  *done = false when the shape does not fit.
int try_mx(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
           int batch, int64_t rb, hipStream_t st, bool *done) {
    *done = false;
    if (fmt == QG_F32 || batch > 4) return QG_OK;
    if (batch >= 2 && cols > 1024) return QG_OK;
    if (batch == 1) {
        if (tiles_fit(fmt, 1, cols)) return QG_OK;
        return try_mx_b<1>(fmt, W, rows, cols, X, Y, batch, rb, st, done);
    }
    if (batch <= 2) return try_mx_b<2>(fmt, W, rows, cols, X, Y, batch, rb, st, done);
    return try_mx_b<4>(fmt, W, rows, cols, X, Y, batch, rb, st, done);
}

int dispatch_gemv(int fmt, int B, bool aligned, int64_t cols, const GemvParams &p,
                  hipStream_t st) {
    const int cpt = gemv_cpt(fmt, B, cols);
    switch (B) {
    case 1: return dispatch_gemv_b<1>(fmt, aligned, cpt, p, st);
    case 2: return dispatch_gemv_b<2>(fmt, aligned, cpt, p, st);
    case 3: return dispatch_gemv_b<3>(fmt, aligned, cpt, p, st);
    case 4: return dispatch_gemv_b<4>(fmt, aligned, cpt, p, st);
    case 5: return dispatch_gemv_b<5>(fmt, aligned, cpt, p, st);
    case 6: return dispatch_gemv_b<6>(fmt, aligned, cpt, p, st);
    case 7: return dispatch_gemv_b<7>(fmt, aligned, cpt, p, st);
    case 8: return dispatch_gemv_b<8>(fmt, aligned, cpt, p, st);
    default: return fail(QG_EUNSUPPORTED, "qgemv: batch %d outside 1..8", B);
    }
}

}  // namespace

// ========================================================================= ABI

namespace {

// The fused add + RMSNorm in front of the chain (moe_ffn_norm): x and
// residual are then attn_out and hidden_in, the router kernel normalises.
struct NormStep {
    const float *gamma;
    double eps;
    float *normed;  // may be NULL
};

int moe_ffn_impl(const char *who, const float *x, const float *residual, float *y,
                 const float *router, int gate_fmt, const void *gate, int up_fmt, const void *up,
                 int down_fmt, const void *down, int64_t hidden, int64_t n_experts,
                 int64_t top_k, int64_t expert_dim, int32_t *sel_experts, float *sel_weights,
                 void *workspace, size_t workspace_bytes, void *stream, const NormStep *norm,
                 int64_t tokens = 1, bool q8 = false) {
    if (tokens < 1) return fail(QG_EINVAL, "%s: tokens must be positive", who);
    if (tokens > kMaxTokens)
        return fail(QG_EUNSUPPORTED, "%s: tokens must be in 1..%d", who, kMaxTokens);
    if (tokens > 1 && top_k > 0 && tokens * top_k > kMaxRoutes)
        return fail(QG_EUNSUPPORTED, "%s: tokens * top_k must be <= %d", who, kMaxRoutes);
    if (!x || !residual || !y || !router || !gate || !up || !down || !workspace)
        return fail(QG_EINVAL, "%s: x, residual, y, router, gate, up, down and workspace "
                               "must be non-NULL", who);
    if (hidden <= 0 || n_experts <= 0 || top_k <= 0 || expert_dim <= 0)
        return fail(QG_EINVAL, "%s: sizes must be positive", who);
    if (top_k > n_experts) return fail(QG_EINVAL, "%s: top_k %lld > n_experts %lld", who,
                                       (long long)top_k, (long long)n_experts);
    if (n_experts > kMaxExperts || top_k > kMaxTopK)
        return fail(QG_EUNSUPPORTED, "%s: n_experts <= %d and top_k <= %d", who, kMaxExperts,
                    kMaxTopK);
    if (hidden > 65536 || expert_dim > 65536)
        return fail(QG_EUNSUPPORTED, "%s: hidden and expert_dim must be <= 65536", who);
    const Geom gg = geom(gate_fmt), gu = geom(up_fmt), gd = geom(down_fmt);
    if (gg.elems == 0 || gu.elems == 0 || gd.elems == 0 || gate_fmt == QG_F32 ||
        up_fmt == QG_F32 || down_fmt == QG_F32)
        return fail(QG_EUNSUPPORTED, "%s: expert stacks must use a block format", who);
    if (gate_fmt != up_fmt)
        return fail(QG_EUNSUPPORTED, "%s: gate (%s) and up (%s) must share a format", who,
                    fmt_name(gate_fmt), fmt_name(up_fmt));
    if (hidden % gg.elems != 0 || expert_dim % gd.elems != 0)
        return fail(QG_EUNSUPPORTED, "%s: hidden must be a multiple of %d and expert_dim "
                                     "of %d", who, gg.elems, gd.elems);
    if (!aligned_to(gate, 2) || !aligned_to(up, 2) || !aligned_to(down, 2))
        return fail(QG_EINVAL, "%s: weight stacks must be 2-byte aligned", who);
    if (!aligned_to(x, 4) || !aligned_to(residual, 4) || !aligned_to(y, 4) ||
        !aligned_to(router, 4) || (sel_experts && !aligned_to(sel_experts, 4)) ||
        (sel_weights && !aligned_to(sel_weights, 4)))
        return fail(QG_EINVAL, "%s: float and int32 arrays must be 4-byte aligned", who);
    if (!aligned_to(workspace, 16)) return fail(QG_EINVAL, "%s: workspace not 16-byte aligned", who);
    if (!norm && y == x) return fail(QG_EINVAL, "%s: y must not alias x", who);
    if (norm) {
        if (!norm->gamma) return fail(QG_EINVAL, "%s: norm_weight must be non-NULL", who);
        if (!aligned_to(norm->gamma, 4) || (norm->normed && !aligned_to(norm->normed, 4)))
            return fail(QG_EINVAL, "%s: float arrays must be 4-byte aligned", who);
        if (!(norm->eps >= 0.0) || !std::isfinite(norm->eps))
            return fail(QG_EINVAL, "%s: eps must be finite and >= 0", who);
        const float *nd = norm->normed;
        if (nd && (nd == x || nd == residual || nd == y || nd == norm->gamma || nd == router))
            return fail(QG_EINVAL, "%s: normed must not alias another argument", who);
    }
    const WsLayout wl = ws_layout(n_experts, top_k, expert_dim, tokens);
    const size_t ws_need = wl.total + (norm ? align16(4 * (size_t)hidden) : 0);
    if (workspace_bytes < ws_need)
        return fail(QG_EINVAL, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes,
                    ws_need);
    const int64_t rbg = qg_row_bytes(gate_fmt, hidden), rbd = qg_row_bytes(down_fmt, expert_dim);
    const uint64_t gate_bytes = (uint64_t)n_experts * expert_dim * rbg;
    const uint64_t down_bytes = (uint64_t)n_experts * hidden * rbd;
    // stacks are addressed with 32-bit offsets below kOorRow (4 GiB - 64 KiB)
    if (gate_bytes > kOorRow - 16u || down_bytes > kOorRow - 16u)
        return fail(QG_EUNSUPPORTED, "%s: each expert stack must be under 4 GiB - 64 KiB", who);
    if (hidden % moe_cpt(gate_fmt) != 0 || expert_dim % moe_cpt(down_fmt) != 0)
        return fail(QG_EUNSUPPORTED, "%s: sizes do not tile", who);
    if (hidden / moe_cpt(gate_fmt) > 512 || top_k * (expert_dim / moe_cpt(down_fmt)) > 512)
        return fail(QG_EUNSUPPORTED, "%s: hidden or top_k * expert_dim too large", who);

    uint8_t *ws = (uint8_t *)workspace;
    MoeParams p{};
    p.x = x;
    p.residual = residual;
    p.y = y;
    p.gate = (const uint8_t *)gate;
    p.up = (const uint8_t *)up;
    p.down = (const uint8_t *)down;
    p.gate_bytes = gate_bytes;
    p.up_bytes = gate_bytes;
    p.down_bytes = down_bytes;
    p.rb_gate = (uint32_t)rbg;
    p.rb_down = (uint32_t)rbd;
    p.H = (int32_t)hidden;
    p.E = (int32_t)n_experts;
    p.K = (int32_t)top_k;
    p.F = (int32_t)expert_dim;
    p.T = (int32_t)tokens;
    p.logits = (const double *)(ws + wl.logits);
    p.ws_sel = (int32_t *)(ws + wl.sel);
    p.ws_w = (float *)(ws + wl.w);
    p.act = (float *)(ws + wl.act);
    p.sel_out = sel_experts;
    p.w_out = sel_weights;

    hipStream_t st = (hipStream_t)stream;
    if (const int rc0 = no_pending_error(who)) return rc0;
    if (norm) {
        // x = attn_out, residual = hidden_in: the router kernel forms
        // h = x + residual and its norm, the experts read xn (workspace),
        // the down kernel adds h = residual + x
        float *xn = (float *)(ws + wl.total);
        p.x = xn;
        p.residual2 = x;
        hipLaunchKernelGGL(moe_norm_router_kernel, dim3((unsigned)n_experts), dim3(64), 0, st,
                           router, x, residual, norm->gamma, norm->eps, (int)hidden,
                           (double *)(ws + wl.logits), xn, norm->normed);
    } else if (tokens > 1) {
        hipLaunchKernelGGL(moe_router_tokens_kernel, dim3((unsigned)n_experts), dim3(64), 0, st,
                           router, x, (int)tokens, (int)hidden, (int)n_experts,
                           (double *)(ws + wl.logits));
    } else {
        hipLaunchKernelGGL(moe_router_kernel<QG_ROUTER_WAVES>, dim3((unsigned)n_experts),
                           dim3(64 * QG_ROUTER_WAVES), 0, st, router, x, (int)hidden,
                           (double *)(ws + wl.logits));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ELAUNCH, "%s: router launch failed: %s", who,
                                     hipGetErrorString(e));
    int rc;
    if (tokens > 1) {
        // several tokens: the distinct experts' gate and up rows on the
        // matrix cores with the tokens as the batch (each row read once per
        // call).  Up to four tokens every gate/up workgroup routes them; above
        // that the grid outnumbers the workgroups the device holds at once,
        // and a small kernel of one wave per token routes ahead (per call,
        // routed in the workgroups / ahead: 4 tokens 48.4 / 50.0 us, 8 tokens
        // 76.5 / 74.9 us).
        const bool routed = tokens > 4;
        if (routed) {
            hipLaunchKernelGGL(moe_route_tokens_kernel, dim3((unsigned)tokens), dim3(64), 0, st,
                               (const double *)(ws + wl.logits), (int)n_experts, (int)top_k,
                               p.ws_sel, p.ws_w, sel_experts, sel_weights);
            e = hipGetLastError();
            if (e != hipSuccess) return fail(QG_ELAUNCH, "%s: routing launch failed: %s", who,
                                             hipGetErrorString(e));
        }
        rc = moe_gateup_ws(gate_fmt, p.gate, p.up, p.gate_bytes, p.rb_gate, p.H, p.F, p.K, p.T,
                           p.E, p.x, p.logits, routed, p.ws_sel, p.ws_w, sel_experts, sel_weights,
                           p.act, st);
    } else {
        rc = q8 ? dispatch_gateup_q8(gate_fmt, p, st) : dispatch_gateup(gate_fmt, p, st);
    }
    if (rc != QG_OK) return rc;
    rc = q8 ? dispatch_down_q8(down_fmt, p, st) : dispatch_down(down_fmt, p, st);
    if (rc != QG_OK) return rc;
    return ok();
}


}  // namespace

extern "C" {

int qg_block_elems(int fmt) { return geom(fmt).elems; }

int qg_block_bytes(int fmt) { return geom(fmt).bytes; }

int64_t qg_row_bytes(int fmt, int64_t cols) {
    const Geom g = geom(fmt);
    if (g.elems == 0 || cols <= 0 || cols % g.elems != 0) return -1;
    return (cols / g.elems) * g.bytes;
}

const char *qg_last_error(void) { return g_err; }

const char *qg_last_kernel(void) { return g_kernel; }

// Block formats: batch >= 2 on the matrix cores in launches of up to 32
// rows; F32 above 8 as groups of 8 (see qgemv).
constexpr int kMaxBatch = 64;

// The argument checks qgemv and qgemv_ws share.
static int check_gemv(const char *who, int fmt, const void *W, int64_t rows, int64_t cols,
                      const float *X, const float *Y, int batch) {
    const Geom g = geom(fmt);
    if (g.elems == 0) return fail(QG_EUNSUPPORTED, "%s: unknown format %d", who, fmt);
    if (!W || !X || !Y) return fail(QG_EINVAL, "%s: W, X and Y must be non-NULL", who);
    if (rows <= 0 || cols <= 0)
        return fail(QG_EINVAL, "%s: rows (%lld) and cols (%lld) must be positive", who,
                    (long long)rows, (long long)cols);
    if (cols % g.elems != 0)
        return fail(QG_EUNSUPPORTED, "%s: %s needs cols to be a multiple of %d (got %lld)", who,
                    fmt_name(fmt), g.elems, (long long)cols);
    if (batch < 1 || batch > kMaxBatch)
        return fail(QG_EUNSUPPORTED, "%s: batch %d outside 1..%d", who, batch, kMaxBatch);
    if (!aligned_to(W, fmt == QG_F32 ? 4 : 2))
        return fail(QG_EINVAL, "%s: W is not %d-byte aligned", who, fmt == QG_F32 ? 4 : 2);
    if (!aligned_to(X, 4) || !aligned_to(Y, 4))
        return fail(QG_EINVAL, "%s: X and Y must be 4-byte aligned", who);
    if (rows >= ((int64_t)1 << 31)) return fail(QG_EUNSUPPORTED, "%s: rows must be < 2^31", who);
    if (cols > 65536) return fail(QG_EUNSUPPORTED, "%s: cols must be <= 65536", who);
    if (fmt == QG_F32 && cols % 4 != 0)
        return fail(QG_EUNSUPPORTED, "%s: F32 rows must be a multiple of 4 floats", who);
    return QG_OK;
}

int qgemv(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
          int batch, void *stream) {
    if (const int rcv = check_gemv("qgemv", fmt, W, rows, cols, X, Y, batch)) return rcv;
    const int64_t rb = qg_row_bytes(fmt, cols);
    hipStream_t st = (hipStream_t)stream;
    if (const int rc0 = no_pending_error("qgemv")) return rc0;
    bool done = false;
    const uint64_t wbytes = (uint64_t)rows * (uint64_t)rb;
    if (QG_Q6_MX && fmt == QG_Q6_K &&
        (batch == 1 || (batch <= QG_Q6_MX_ROWS && wbytes >= QG_Q6_MX_ROWS_BYTES) ||
         (batch <= QG_Q6_MX_PAIRS && wbytes >= QG_Q6_MX_PAIRS_BYTES))) {
        // batch 1, and batch 2 on matrices of 16 MiB or more: the int8
        // digit-plane kernel, at batch 2 with both rows' planes against each
        // tile's codes (A/B on one box, batch 2: lm_head 151936 x 2048 117
        // us on the bf16 kernel, 86.5 as two batch-1 launches, 48.5; 32768
        // x 2048 26.1 -> 16.8; 14336 x 4096 21.5 -> 20.2; smaller matrices
        // keep the other kernels: 4096 x 4096 9.4 against 11.2); on the
        // lm_head's class batch 3-4 as launches of two rows and one
        for (int b0 = 0; b0 < batch; b0 += 2) {
            const int nb = batch - b0 < 2 ? batch - b0 : 2;
            GemvParams p{};
            p.W = (const uint8_t *)W;
            p.X = X + (int64_t)b0 * cols;
            p.Y = Y + (int64_t)b0 * rows;
            p.rows = rows;
            p.w_bytes = wbytes;
            p.row_bytes = (uint32_t)rb;
            p.cols = (uint32_t)cols;
            p.batch_x = 1;
            // the shape decides whether the kernel takes it, for one row
            // and two alike
            const int qrc = try_q6mx(p, nb, st, &done);
            if (!done) break;
            if (qrc != QG_OK) return qrc;
        }
        if (done) {
            g_kernel = "mfma_i8_q6k";
            return ok();
        }
    }
    if (gemm_ks2_fits(fmt, rows, cols, batch)) {
        // tall matrices at batch 2-32: activation operands shared through
        // LDS by a workgroup's 4 tiles, two column ranges per workgroup
        // (Q5_K 14336 x 4096: batch 4 19.5 -> 16.7 us against the f16
        // kernel, batch 8 24.6 -> 18.1 us against qgemm8_kernel, batch 16
        // 36.9 -> 24.6 us against qgemm_kernel)
        const int rc = gemm_ks2(fmt, W, rows, cols, X, Y, batch, rb, st);
        if (rc != QG_OK) return rc;
        g_kernel = "gemm_ks2_bf16";
        return ok();
    }
    const int mrc = try_mx(fmt, W, rows, cols, X, Y, batch, rb, st, &done);
    if (done) {
        if (mrc != QG_OK) return mrc;
        g_kernel = "mx_f16";
        return ok();
    }
    if (fmt != QG_F32 && batch >= 2) {
        // block formats at batch >= 2: the batched matrix-core kernel, up to
        // 32 batch rows per launch (the weights are read once per launch)
        // (tall matrices: each launch of 2-32 rows on the two-range kernel)
        bool ks2_all = true;
        for (int b0 = 0; b0 < batch; b0 += 32) {
            const int nb = batch - b0 < 32 ? batch - b0 : 32;
            const float *Xb = X + (int64_t)b0 * cols;
            float *Yb = Y + (int64_t)b0 * rows;
            int rc;
            if (gemm_ks2_fits(fmt, rows, cols, nb)) {
                rc = gemm_ks2(fmt, W, rows, cols, Xb, Yb, nb, rb, st);
            } else {
                ks2_all = false;
                rc = nb <= 16 ? gemm_b<1>(fmt, W, rows, cols, Xb, Yb, nb, rb, st)
                              : gemm_b<2>(fmt, W, rows, cols, Xb, Yb, nb, rb, st);
            }
            if (rc != QG_OK) return rc;
        }
        g_kernel = ks2_all ? "gemm_ks2_bf16" : "gemm_bf16";
        return ok();
    }
    if (batch > 8) {
        // F32 rows at batch > 8: groups of up to 8 activation rows, one after
        // another on the stream
        for (int b0 = 0; b0 < batch; b0 += 8) {
            const int nb = batch - b0 < 8 ? batch - b0 : 8;
            const int rc = qgemv(fmt, W, rows, cols, X + (int64_t)b0 * cols,
                                 Y + (int64_t)b0 * rows, nb, stream);
            if (rc != QG_OK) return rc;
        }
        return ok();
    }
    // Batches too wide for VGPR-resident activations run as several narrower
    // launches over column slices of X and Y.
    int chunk = batch;
    while (chunk > 1 && !tiles_fit(fmt, chunk, cols)) chunk = chunk > 4 ? 4 : chunk / 2;
    if (!tiles_fit(fmt, chunk, cols))
        return fail(QG_EUNSUPPORTED, "qgemv: %lld columns of %s exceed the kernel's row width",
                    (long long)cols, fmt_name(fmt));
    const bool aligned = aligned_to(W, 4) && rb % 4 == 0;
    for (int b0 = 0; b0 < batch; b0 += chunk) {
        const int nb = batch - b0 < chunk ? batch - b0 : chunk;
        GemvParams p{};
        p.W = (const uint8_t *)W;
        p.X = X + (int64_t)b0 * cols;
        p.Y = Y + (int64_t)b0 * rows;
        p.rows = rows;
        p.w_bytes = (uint64_t)rows * (uint64_t)rb;
        p.row_bytes = (uint32_t)rb;
        p.cols = (uint32_t)cols;
        p.batch_x = (uint32_t)nb;
        const int rc = dispatch_gemv(fmt, nb, aligned, cols, p, st);
        if (rc != QG_OK) return rc;
    }
    g_kernel = (fmt == QG_Q6_K && batch == 1) ? "valu_q6k_int" : "valu_f32";
    return ok();
}

size_t qgemv_ws_bytes(int fmt, int64_t rows, int64_t cols, int batch) {
    const Geom g = geom(fmt);
    if (g.elems == 0 || fmt == QG_F32 || rows <= 0 || cols <= 0 || cols % g.elems != 0 ||
        batch < 2 || batch > kMaxBatch || rows >= ((int64_t)1 << 31) || cols > 65536)
        return 0;
    if (ws_uses_qgemv(rows, cols, batch)) return 0;
    // the largest [kg][batch rows][rows] partial-sum block of the call's
    // launches (up to 32 batch rows each; 0 when no launch splits columns
    // across workgroups)
    size_t need = 0;
    for (int b0 = 0; b0 < batch; b0 += 32) {
        const int nb = batch - b0 < 32 ? batch - b0 : 32;
        const int kg = ws_kg(rows, cols, nb);
        const size_t n = kg > 1 ? (size_t)kg * (size_t)nb * (size_t)rows * sizeof(float) : 0;
        if (n > need) need = n;
    }
    return need;
}

int qgemv_ws(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
             int batch, void *workspace, size_t workspace_bytes, void *stream) {
    if (const int rcv = check_gemv("qgemv_ws", fmt, W, rows, cols, X, Y, batch)) return rcv;
    // no batched matrix-core work, or a shape where qgemv's kernels are
    // faster: qgemv, no workspace
    if (fmt == QG_F32 || batch == 1 || ws_uses_qgemv(rows, cols, batch))
        return qgemv(fmt, W, rows, cols, X, Y, batch, stream);
    const size_t need = qgemv_ws_bytes(fmt, rows, cols, batch);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(QG_EINVAL, "qgemv_ws: the workspace holds %zu bytes; this call needs %zu "
                               "(qgemv_ws_bytes)", workspace ? workspace_bytes : (size_t)0, need);
    if (need > 0 && !aligned_to(workspace, 16))
        return fail(QG_EINVAL, "qgemv_ws: the workspace must be 16-byte aligned");
    const int64_t rb = qg_row_bytes(fmt, cols);
    hipStream_t st = (hipStream_t)stream;
    if (const int rc0 = no_pending_error("qgemv_ws")) return rc0;
    // launches of up to 32 batch rows, each reading the weights once; they
    // run one after another on the stream and reuse the workspace
    for (int b0 = 0; b0 < batch; b0 += 32) {
        const int nb = batch - b0 < 32 ? batch - b0 : 32;
        const int rc = gemm_ws(fmt, W, rows, cols, X + (int64_t)b0 * cols,
                               Y + (int64_t)b0 * rows, nb, rb, (float *)workspace, st);
        if (rc != QG_OK) return rc;
    }
    g_kernel = "gemm_ws_bf16";
    return ok();
}

int qgemv_q8act(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
                void *stream) {
    const Geom g = geom(fmt);
    if (g.elems == 0 || fmt == QG_F32)
        return fail(QG_EUNSUPPORTED, "qgemv_q8act: format %d has no int8 path", fmt);
    if (!W || !X || !Y) return fail(QG_EINVAL, "qgemv_q8act: W, X and Y must be non-NULL");
    if (rows <= 0 || cols <= 0)
        return fail(QG_EINVAL, "qgemv_q8act: rows (%lld) and cols (%lld) must be positive",
                    (long long)rows, (long long)cols);
    if (cols % g.elems != 0)
        return fail(QG_EUNSUPPORTED, "qgemv_q8act: %s needs cols to be a multiple of %d (got %lld)",
                    fmt_name(fmt), g.elems, (long long)cols);
    if (!aligned_to(W, 2)) return fail(QG_EINVAL, "qgemv_q8act: W is not 2-byte aligned");
    if (!aligned_to(X, 4) || !aligned_to(Y, 4))
        return fail(QG_EINVAL, "qgemv_q8act: X and Y must be 4-byte aligned");
    if (rows >= ((int64_t)1 << 31))
        return fail(QG_EUNSUPPORTED, "qgemv_q8act: rows must be < 2^31");
    if (cols > 65536 || !tiles_fit(fmt, 1, cols))
        return fail(QG_EUNSUPPORTED, "qgemv_q8act: %lld columns of %s exceed the kernel's row "
                                     "width", (long long)cols, fmt_name(fmt));
    const int64_t rb = qg_row_bytes(fmt, cols);
    GemvParams p{};
    p.W = (const uint8_t *)W;
    p.X = X;
    p.Y = Y;
    p.rows = rows;
    p.w_bytes = (uint64_t)rows * (uint64_t)rb;
    p.row_bytes = (uint32_t)rb;
    p.cols = (uint32_t)cols;
    p.batch_x = 1;
    if (const int rc0 = no_pending_error("qgemv_q8act")) return rc0;
    const int rc = dispatch_gemv_q8(fmt, aligned_to(W, 4) && rb % 4 == 0, p, (hipStream_t)stream);
    if (rc != QG_OK) return rc;
    g_kernel = "valu_q8act";
    return ok();
}

size_t moe_ffn_workspace_bytes(int64_t n_experts, int64_t top_k, int64_t expert_dim) {
    if (n_experts <= 0 || top_k <= 0 || expert_dim <= 0 || top_k > n_experts) return 0;
    return ws_layout(n_experts, top_k, expert_dim).total;
}

int qg_route_topk(const double *logits, int64_t n_experts, int64_t top_k, int32_t *sel_experts,
                  float *sel_weights, void *stream) {
    if (!logits || !sel_experts || !sel_weights)
        return fail(QG_EINVAL, "qg_route_topk: logits, sel_experts and sel_weights are required");
    if (n_experts <= 0 || top_k <= 0 || top_k > n_experts)
        return fail(QG_EINVAL, "qg_route_topk: need 0 < top_k <= n_experts");
    if (n_experts > kMaxExperts || top_k > kMaxTopK)
        return fail(QG_EUNSUPPORTED, "qg_route_topk: n_experts <= %d and top_k <= %d",
                    kMaxExperts, kMaxTopK);
    if (!aligned_to(logits, 8) || !aligned_to(sel_experts, 4) || !aligned_to(sel_weights, 4))
        return fail(QG_EINVAL, "qg_route_topk: misaligned pointer");
    if (const int rc0 = no_pending_error("qg_route_topk")) return rc0;
    hipLaunchKernelGGL(route_topk_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, logits,
                       (int)n_experts, (int)top_k, (int *)sel_experts, sel_weights);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "qg_route_topk: launch failed: %s", hipGetErrorString(e));
    return ok();
}

int qg_stream_read(const void *buf, size_t bytes, uint32_t *out, int grid, void *stream) {
    if (!buf || !out) return fail(QG_EINVAL, "qg_stream_read: buf and out must be non-NULL");
    if (bytes == 0 || bytes % 16 != 0 || !aligned_to(buf, 16) || !aligned_to(out, 4))
        return fail(QG_EINVAL, "qg_stream_read: bytes must be a positive multiple of 16 and buf "
                               "16-byte aligned");
    const uint64_t per_wg = (uint64_t)kStreamThreads * kStreamLoads * 16;
    const uint64_t need = (bytes + per_wg - 1) / per_wg;
    if (grid <= 0) grid = (int)(need < 2048 ? need : 2048);
    if ((uint64_t)grid > need) grid = (int)need;
    if (const int rc0 = no_pending_error("qg_stream_read")) return rc0;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0,
                       (hipStream_t)stream, (const uint8_t *)buf, (uint64_t)bytes, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "qg_stream_read: launch failed: %s", hipGetErrorString(e));
    return ok();
}

int moe_ffn(const float *x, const float *residual, float *y, const float *router, int gate_fmt,
            const void *gate, int up_fmt, const void *up, int down_fmt, const void *down,
            int64_t hidden, int64_t n_experts, int64_t top_k, int64_t expert_dim,
            int32_t *sel_experts, float *sel_weights, void *workspace, size_t workspace_bytes,
            void *stream) {
    return moe_ffn_impl("moe_ffn", x, residual, y, router, gate_fmt, gate, up_fmt, up, down_fmt,
                        down, hidden, n_experts, top_k, expert_dim, sel_experts, sel_weights,
                        workspace, workspace_bytes, stream, nullptr);
}

int moe_ffn_q8act(const float *x, const float *residual, float *y, const float *router,
                  int gate_fmt, const void *gate, int up_fmt, const void *up, int down_fmt,
                  const void *down, int64_t hidden, int64_t n_experts, int64_t top_k,
                  int64_t expert_dim, int32_t *sel_experts, float *sel_weights, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return moe_ffn_impl("moe_ffn_q8act", x, residual, y, router, gate_fmt, gate, up_fmt, up,
                        down_fmt, down, hidden, n_experts, top_k, expert_dim, sel_experts,
                        sel_weights, workspace, workspace_bytes, stream, nullptr, 1, true);
}

size_t moe_ffn_tokens_workspace_bytes(int64_t tokens, int64_t n_experts, int64_t top_k,
                                      int64_t expert_dim) {
    if (tokens <= 0 || n_experts <= 0 || top_k <= 0 || expert_dim <= 0 || top_k > n_experts)
        return 0;
    return ws_layout(n_experts, top_k, expert_dim, tokens).total;
}

int moe_ffn_tokens(const float *x, const float *residual, float *y, const float *router,
                   int gate_fmt, const void *gate, int up_fmt, const void *up, int down_fmt,
                   const void *down, int64_t tokens, int64_t hidden, int64_t n_experts,
                   int64_t top_k, int64_t expert_dim, int32_t *sel_experts, float *sel_weights,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return moe_ffn_impl("moe_ffn_tokens", x, residual, y, router, gate_fmt, gate, up_fmt, up,
                        down_fmt, down, hidden, n_experts, top_k, expert_dim, sel_experts,
                        sel_weights, workspace, workspace_bytes, stream, nullptr, tokens);
}

size_t moe_ffn_norm_workspace_bytes(int64_t hidden, int64_t n_experts, int64_t top_k,
                                    int64_t expert_dim) {
    if (hidden <= 0 || n_experts <= 0 || top_k <= 0 || expert_dim <= 0 || top_k > n_experts)
        return 0;
    return ws_layout(n_experts, top_k, expert_dim).total + align16(4 * (size_t)hidden);
}

int moe_ffn_norm(const float *attn_out, const float *hidden_in, float *hidden_out,
                 const float *norm_weight, float eps, float *normed, const float *router,
                 int gate_fmt, const void *gate, int up_fmt, const void *up, int down_fmt,
                 const void *down, int64_t hidden, int64_t n_experts, int64_t top_k,
                 int64_t expert_dim, int32_t *sel_experts, float *sel_weights, void *workspace,
                 size_t workspace_bytes, void *stream) {
    const NormStep ns{norm_weight, (double)eps, normed};
    return moe_ffn_impl("moe_ffn_norm", attn_out, hidden_in, hidden_out, router, gate_fmt, gate,
                        up_fmt, up, down_fmt, down, hidden, n_experts, top_k, expert_dim,
                        sel_experts, sel_weights, workspace, workspace_bytes, stream, &ns);
}

}  // extern "C"

