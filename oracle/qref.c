/*
 * qref.c -- the CPU oracle for GGUF block dequantisation, the fused
 * dequantise-and-dot GEMV and the stacked-expert MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * Style: plain, slow, single-threaded, obviously correct.  Every weight is
 * decoded element by element from its own index formula into a double,
 * every dot product is accumulated in double in ascending column order.
 * Built with -ffp-contract=off so no fused multiply-add changes a rounding.
 *
 * Sources (web pages; the item named is where the definition sits):
 *   [gpu.rs]   docs.rs, crate ferrox-cuda 0.14.0, source src/gpu.rs
 *   [wm.rs]    docs.rs, ferrox-core 0.16.0, src/ferrox_core/weight_matrix.rs
 *   [moe.rs]   docs.rs, crate aprender-serve 0.70.2, source
 *              src/gguf/cuda/forward_qwen3_moe_resident.rs
 *
 * Parity pins for every function are in tests/test_oracle_*.py.  Readings
 * taken where the pages are silent are marked READING below.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Format tags: ggml's numeric type ids for the five block formats plus F32
 * ([wm.rs] QuantKind / quant_kind_for map GGUF dtypes onto these kinds). */
#define QREF_F32 0
#define QREF_Q4_0 2
#define QREF_Q8_0 8
#define QREF_Q4_K 12
#define QREF_Q5_K 13
#define QREF_Q6_K 14

#define QREF_OK 0
#define QREF_EINVAL 1
#define QREF_EUNSUPPORTED 2

/* Elements per block and bytes per block.
 * [gpu.rs] Q8_0_MATVEC_KERNEL_SRC: 34-byte blocks of 32 values.
 * [gpu.rs] Q4_0_MATVEC_KERNEL_SRC: 18-byte blocks of 32 values.
 * [gpu.rs] Q4_K_MATVEC_KERNEL_SRC: 144-byte super-blocks of 256 values.
 * [gpu.rs] Q5_K_MATVEC_KERNEL_SRC: 176-byte super-blocks of 256 values.
 * [gpu.rs] Q6_K_MATVEC_KERNEL_SRC: 210-byte super-blocks of 256 values.
 * F32 is one 4-byte value per element. */
int qref_block_elems(int fmt) {
    switch (fmt) {
    case QREF_F32: return 1;
    case QREF_Q4_0: return 32;
    case QREF_Q8_0: return 32;
    case QREF_Q4_K: return 256;
    case QREF_Q5_K: return 256;
    case QREF_Q6_K: return 256;
    default: return 0;
    }
}

int qref_block_bytes(int fmt) {
    switch (fmt) {
    case QREF_F32: return 4;
    case QREF_Q4_0: return 18;
    case QREF_Q8_0: return 34;
    case QREF_Q4_K: return 144;
    case QREF_Q5_K: return 176;
    case QREF_Q6_K: return 210;
    default: return 0;
    }
}

/* Bytes of one row: whole blocks, no padding ([wm.rs] block_bytes_per_row).
 * Returns -1 when cols is not a positive multiple of the block size. */
int64_t qref_row_bytes(int fmt, int64_t cols) {
    int qk = qref_block_elems(fmt);
    if (qk == 0 || cols <= 0 || cols % qk != 0) return -1;
    return (cols / qk) * (int64_t)qref_block_bytes(fmt);
}

/* IEEE binary16 -> double, written from the bit layout.
 * [gpu.rs] ferrox_f16_to_f32: sign bit 15, 5-bit exponent, 10-bit fraction;
 * exponent 0 is subnormal (fraction * 2^-24), exponent 31 is infinity when
 * the fraction is 0 and NaN otherwise, any other exponent gives
 * (1024 + fraction) * 2^(exponent - 25).  The sign is applied last. */
double qref_f16(uint16_t h) {
    unsigned sign = (h >> 15) & 1u;
    unsigned expo = (h >> 10) & 31u;
    unsigned frac = h & 1023u;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024u + frac), (int)expo - 25);
    }
    return sign ? -v : v;
}

/* Little-endian 16-bit field at byte offset off of a block. */
static uint16_t le16(const uint8_t *p, int off) {
    return (uint16_t)(p[off] | (p[off + 1] << 8));
}

/* Q4_K / Q5_K 6-bit (scale, min) pair of sub-block s (0..7) from the 12
 * packed bytes S.  [gpu.rs] ferrox_q4_k_scale_min: for s < 4 the low six
 * bits of S[s] and S[s+4]; for s >= 4 the low nibble (scale) or high nibble
 * (min) of S[s+4] supplies bits 0..3 and the top two bits of S[s-4] (scale)
 * or S[s] (min) supply bits 4..5. */
static void kquant_scale_min(const uint8_t *S, int s, int *sc, int *m) {
    if (s < 4) {
        *sc = S[s] & 63;
        *m = S[s + 4] & 63;
    } else {
        *sc = (S[s + 4] & 15) + 16 * (S[s - 4] >> 6);
        *m = (S[s + 4] >> 4) + 16 * (S[s] >> 6);
    }
}

/* Dequantise one block of format fmt into out[block_elems]. */
int qref_dequant_block(int fmt, const uint8_t *blk, double *out) {
    int e;
    switch (fmt) {
    case QREF_F32: {
        float f;
        memcpy(&f, blk, 4);
        out[0] = (double)f;
        return QREF_OK;
    }
    case QREF_Q8_0: {
        /* [gpu.rs] Q8_0_MATVEC_KERNEL_SRC: f16 scale d at bytes 0..1, then
         * 32 signed bytes; value i = d * q_i. */
        double d = qref_f16(le16(blk, 0));
        for (e = 0; e < 32; e++) out[e] = d * (double)(int8_t)blk[2 + e];
        return QREF_OK;
    }
    case QREF_Q4_0: {
        /* [gpu.rs] Q4_0_MATVEC_KERNEL_SRC: f16 d at 0..1, 16 packed bytes
         * from byte 2; element j < 16 is the low nibble of byte j, element
         * j + 16 the high nibble; value = d * (nibble - 8). */
        double d = qref_f16(le16(blk, 0));
        for (e = 0; e < 32; e++) {
            uint8_t byte = blk[2 + (e % 16)];
            int nib = (e < 16) ? (byte & 15) : (byte >> 4);
            out[e] = d * (double)(nib - 8);
        }
        return QREF_OK;
    }
    case QREF_Q4_K: {
        /* [gpu.rs] Q4_K_MATVEC_KERNEL_SRC: d (f16) at 0, dmin (f16) at 2,
         * 12 scale bytes at 4, 128 quant bytes at 16.  Element e belongs to
         * sub-block s = e/32 with its own (sc, m).  Its 4-bit code lives in
         * qs[32*(e/64) + e%32]: the low nibble for the first 32 elements of
         * each 64, the high nibble for the second 32.
         * value = d*sc*q - dmin*m.  READING: the code (8 sub-blocks of 32)
         * decides over the page's prose that speaks of 4 sub-blocks of 64. */
        double d = qref_f16(le16(blk, 0));
        double dmin = qref_f16(le16(blk, 2));
        const uint8_t *S = blk + 4, *qs = blk + 16;
        for (e = 0; e < 256; e++) {
            int s = e / 32, sc, m;
            int p = e / 64, hi = (e % 64) / 32, l = e % 32;
            uint8_t byte = qs[32 * p + l];
            int q = hi ? (byte >> 4) : (byte & 15);
            kquant_scale_min(S, s, &sc, &m);
            out[e] = d * (double)sc * (double)q - dmin * (double)m;
        }
        return QREF_OK;
    }
    case QREF_Q5_K: {
        /* [gpu.rs] Q5_K_MATVEC_KERNEL_SRC: as Q4_K, with 32 high-bit bytes
         * qh at 16 and the 128 quant bytes at 48.  The fifth bit of element
         * e is bit (2*(e/64) + (e%64)/32) of qh[e%32]; q = nibble + 16*bit. */
        double d = qref_f16(le16(blk, 0));
        double dmin = qref_f16(le16(blk, 2));
        const uint8_t *S = blk + 4, *qh = blk + 16, *qs = blk + 48;
        for (e = 0; e < 256; e++) {
            int s = e / 32, sc, m;
            int p = e / 64, hi = (e % 64) / 32, l = e % 32;
            uint8_t byte = qs[32 * p + l];
            int nib = hi ? (byte >> 4) : (byte & 15);
            int bit = (qh[l] >> (2 * p + hi)) & 1;
            int q = nib + 16 * bit;
            kquant_scale_min(S, s, &sc, &m);
            out[e] = d * (double)sc * (double)q - dmin * (double)m;
        }
        return QREF_OK;
    }
    case QREF_Q6_K: {
        /* [gpu.rs] Q6_K_MATVEC_KERNEL_SRC: ql[128] at 0, qh[64] at 128,
         * sixteen signed int8 scales at 192, f16 d at 208.  The block is two
         * halves of 128; within half h element e has t = (e%128)/32 and
         * l = e%32.  Its low four bits are nibble (t/2) of
         * ql[64h + 32*(t%2) + l], its top two bits are bits 2t..2t+1 of
         * qh[32h + l]; q = low + 16*top; value = d * sc[e/16] * (q - 32),
         * the scale read as SIGNED (the page records that an unsigned read
         * was a bug). */
        double d = qref_f16(le16(blk, 208));
        const uint8_t *ql = blk, *qh = blk + 128;
        const int8_t *sc = (const int8_t *)(blk + 192);
        for (e = 0; e < 256; e++) {
            int h = e / 128, t = (e % 128) / 32, l = e % 32;
            uint8_t lb = ql[64 * h + 32 * (t % 2) + l];
            int low = (t / 2) ? (lb >> 4) : (lb & 15);
            int top = (qh[32 * h + l] >> (2 * t)) & 3;
            int q = low + 16 * top;
            out[e] = d * (double)sc[e / 16] * (double)(q - 32);
        }
        return QREF_OK;
    }
    default:
        return QREF_EUNSUPPORTED;
    }
}

/* Dequantise one row of cols elements. */
int qref_dequant_row(int fmt, const uint8_t *row, int64_t cols, double *out) {
    int64_t rb = qref_row_bytes(fmt, cols);
    int qk = qref_block_elems(fmt), bb = qref_block_bytes(fmt);
    int64_t b;
    if (rb < 0) return qref_block_elems(fmt) ? QREF_EINVAL : QREF_EUNSUPPORTED;
    for (b = 0; b < cols / qk; b++) {
        int rc = qref_dequant_block(fmt, row + b * bb, out + b * qk);
        if (rc) return rc;
    }
    return QREF_OK;
}

/* One output element: sum over c of w[c] * x[c] in double, ascending c, and
 * the sum of |w[c] * x[c]| for the tolerance.  With the scales drawn in the
 * synthetic workloads' ranges each decoded weight has at most 24 significant
 * bits, so its product with an f32 activation is exact in double and the
 * only rounding is in the sum. */
static void dot_f64(const double *w, const float *x, int64_t cols, double *y,
                    double *yabs) {
    double acc = 0.0, aabs = 0.0;
    int64_t c;
    for (c = 0; c < cols; c++) {
        double p = w[c] * (double)x[c];
        acc += p;
        aabs += fabs(p);
    }
    *y = acc;
    *yabs = aabs;
}

/* GEMV over selected rows: Y[b*nidx + i] = sum_c deq(W)[row_idx[i]][c] *
 * X[b*cols + c] for b < batch.  Layout: W row-major [rows][row_bytes],
 * X [batch][cols], Y and Yabs [batch][nidx] ([wm.rs] apply / apply_batch:
 * activations and outputs are batch-major).  Yabs may be NULL. */
int qref_gemv_rows(int fmt, const void *W, int64_t rows, int64_t cols,
                   const float *X, int batch, const int64_t *row_idx,
                   int64_t nidx, double *Y, double *Yabs) {
    int64_t rb = qref_row_bytes(fmt, cols), i;
    double *w;
    int b, rc = QREF_OK;
    if (rb < 0) return qref_block_elems(fmt) ? QREF_EINVAL : QREF_EUNSUPPORTED;
    if (!W || !X || !Y || rows <= 0 || batch <= 0 || nidx < 0) return QREF_EINVAL;
    w = (double *)malloc(sizeof(double) * (size_t)cols);
    if (!w) return QREF_EINVAL;
    for (i = 0; i < nidx; i++) {
        int64_t r = row_idx[i];
        if (r < 0 || r >= rows) { rc = QREF_EINVAL; break; }
        rc = qref_dequant_row(fmt, (const uint8_t *)W + r * rb, cols, w);
        if (rc) break;
        for (b = 0; b < batch; b++) {
            double y, ya;
            dot_f64(w, X + (int64_t)b * cols, cols, &y, &ya);
            Y[(int64_t)b * nidx + i] = y;
            if (Yabs) Yabs[(int64_t)b * nidx + i] = ya;
        }
    }
    free(w);
    return rc;
}

/* Full GEMV: every row, Y and Yabs [batch][rows]. */
int qref_gemv(int fmt, const void *W, int64_t rows, int64_t cols,
              const float *X, int batch, double *Y, double *Yabs) {
    int64_t *idx, r;
    int rc;
    if (rows <= 0) return QREF_EINVAL;
    idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)rows);
    if (!idx) return QREF_EINVAL;
    for (r = 0; r < rows; r++) idx[r] = r;
    rc = qref_gemv_rows(fmt, W, rows, cols, X, batch, idx, rows, Y, Yabs);
    free(idx);
    return rc;
}

/* Rank order of experts: a comes before b when its logit is larger; equal
 * logits go to the lower index; a NaN logit ranks below every number
 * (READING: the routing function's body is not on the pages; the lower-index
 * tie-break is the stated rule, NaN placement is ours). */
static int ranks_before(const double *l, int a, int b) {
    int na = isnan(l[a]), nb = isnan(l[b]);
    if (na != nb) return nb; /* the non-NaN one first */
    if (!na && l[a] != l[b]) return l[a] > l[b];
    return a < b;
}

/* Routing: softmax over all E logits, top-k, renormalise over the chosen k
 * ([moe.rs] module doc: router GEMV, then softmax, top-k, renormalise; the
 * routes are reported as (expert, weight) pairs in rank order, see
 * last_routes).  READING: the choice is made on the logits, which orders the
 * experts exactly as the exact softmax probabilities do (exp is strictly
 * increasing) and cannot merge two distinct values the way rounded
 * probabilities could.  Weights: p = softmax(l) in double with the maximum
 * subtracted, w_s = p[sel_s] / sum over the k chosen of p.
 * sel[k] int32, w[k] double, both in rank order. */
int qref_route(const double *logits, int n_experts, int top_k, int32_t *sel,
               double *w) {
    int i, j, s;
    double mx = -INFINITY, denom = 0.0, ssum = 0.0;
    double *p;
    if (!logits || !sel || !w || n_experts <= 0 || top_k <= 0 || top_k > n_experts)
        return QREF_EINVAL;
    /* selection by repeated "best not yet taken" scan: O(k * E) */
    for (s = 0; s < top_k; s++) {
        int best = -1;
        for (i = 0; i < n_experts; i++) {
            int taken = 0;
            for (j = 0; j < s; j++)
                if (sel[j] == i) taken = 1;
            if (taken) continue;
            if (best < 0 || ranks_before(logits, i, best)) best = i;
        }
        sel[s] = best;
    }
    p = (double *)malloc(sizeof(double) * (size_t)n_experts);
    if (!p) return QREF_EINVAL;
    for (i = 0; i < n_experts; i++)
        if (logits[i] > mx) mx = logits[i];
    for (i = 0; i < n_experts; i++) {
        p[i] = exp(logits[i] - mx);
        denom += p[i];
    }
    for (i = 0; i < n_experts; i++) p[i] /= denom;
    for (s = 0; s < top_k; s++) ssum += p[sel[s]];
    for (s = 0; s < top_k; s++) w[s] = p[sel[s]] / ssum;
    free(p);
    return QREF_OK;
}

/* SiLU, in double.  [gpu.rs] SILU_MUL_KERNEL_SRC: silu(g) = g / (1 + e^-g),
 * and SwiGLU is silu(gate) * up. */
double qref_silu(double g) { return g / (1.0 + exp(-g)); }

/* The stacked-expert MoE FFN for one token ([moe.rs] moe_layer and the
 * module doc):
 *   logits[e] = sum_i R[e][i] * x[i]                 (router, F32 weights)
 *   (sel, w)  = route(logits, k)
 *   for each slot s in rank order, expert e = sel[s]:
 *     g = G[e] x,  u = U[e] x                        (rows F, cols H)
 *     act[s][j] = w_s * silu(g_j) * u_j              (weight folded into the
 *                                                     activation before the
 *                                                     linear down GEMV)
 *   y = residual + sum_s D[e] act[s]                  (down: rows H, cols F)
 * Expert e of a stack starts at base + e * rows * row_bytes ([moe.rs]
 * ExpertStack::expert).  Outputs (any may be NULL except y): logits[E],
 * sel[k], w[k], act[k][F], bound[H] = |residual| + sum_s sum_j |D act|. */
int qref_moe_ffn(const float *x, const float *residual, const float *router,
                 int gate_fmt, const void *gate, int up_fmt, const void *up,
                 int down_fmt, const void *down, int64_t hidden,
                 int64_t n_experts, int64_t top_k, int64_t expert_dim,
                 double *y, double *bound, double *logits_out,
                 int32_t *sel_out, double *w_out, double *act_out) {
    int64_t H = hidden, E = n_experts, K = top_k, F = expert_dim;
    int64_t rb_g = qref_row_bytes(gate_fmt, H), rb_u = qref_row_bytes(up_fmt, H);
    int64_t rb_d = qref_row_bytes(down_fmt, F);
    int64_t e, s, j, r;
    int rc = QREF_OK;
    double *logits, *w, *act, *row, *g, *u;
    int32_t *sel;
    if (!x || !residual || !router || !gate || !up || !down || !y) return QREF_EINVAL;
    if (H <= 0 || E <= 0 || K <= 0 || F <= 0 || K > E) return QREF_EINVAL;
    if (rb_g < 0 || rb_u < 0 || rb_d < 0) return QREF_EUNSUPPORTED;
    logits = (double *)malloc(sizeof(double) * (size_t)E);
    w = (double *)malloc(sizeof(double) * (size_t)K);
    sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    act = (double *)malloc(sizeof(double) * (size_t)(K * F));
    row = (double *)malloc(sizeof(double) * (size_t)(H > F ? H : F));
    g = (double *)malloc(sizeof(double) * (size_t)F);
    u = (double *)malloc(sizeof(double) * (size_t)F);
    if (!logits || !w || !sel || !act || !row || !g || !u) { rc = QREF_EINVAL; goto done; }

    /* router GEMV: F32 weights [E][H] */
    for (e = 0; e < E; e++) {
        double yabs;
        rc = qref_dequant_row(QREF_F32, (const uint8_t *)router + e * H * 4, H, row);
        if (rc) goto done;
        dot_f64(row, x, H, &logits[e], &yabs);
    }
    rc = qref_route(logits, (int)E, (int)K, sel, w);
    if (rc) goto done;

    /* gate, up, SwiGLU times the route weight */
    for (s = 0; s < K; s++) {
        const uint8_t *gb = (const uint8_t *)gate + (int64_t)sel[s] * F * rb_g;
        const uint8_t *ub = (const uint8_t *)up + (int64_t)sel[s] * F * rb_u;
        for (j = 0; j < F; j++) {
            double yabs;
            rc = qref_dequant_row(gate_fmt, gb + j * rb_g, H, row);
            if (rc) goto done;
            dot_f64(row, x, H, &g[j], &yabs);
            rc = qref_dequant_row(up_fmt, ub + j * rb_u, H, row);
            if (rc) goto done;
            dot_f64(row, x, H, &u[j], &yabs);
        }
        for (j = 0; j < F; j++) act[s * F + j] = w[s] * qref_silu(g[j]) * u[j];
    }

    /* down GEMV per slot, added into the residual in rank order */
    for (r = 0; r < H; r++) {
        double acc = (double)residual[r], aabs = fabs((double)residual[r]);
        for (s = 0; s < K; s++) {
            const uint8_t *db = (const uint8_t *)down + (int64_t)sel[s] * H * rb_d;
            rc = qref_dequant_row(down_fmt, db + r * rb_d, F, row);
            if (rc) goto done;
            for (j = 0; j < F; j++) {
                double p = row[j] * act[s * F + j];
                acc += p;
                aabs += fabs(p);
            }
        }
        y[r] = acc;
        if (bound) bound[r] = aabs;
    }
    if (logits_out) memcpy(logits_out, logits, sizeof(double) * (size_t)E);
    if (sel_out) memcpy(sel_out, sel, sizeof(int32_t) * (size_t)K);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)K);
    if (act_out) memcpy(act_out, act, sizeof(double) * (size_t)(K * F));
done:
    free(logits); free(w); free(sel); free(act); free(row); free(g); free(u);
    return rc;
}

/* Fused residual add + RMSNorm, the step that feeds the router.
 * [gpu.rs] FUSED_ADD_RMSNORM_KERNEL_SRC: out[i] = (x[i] + residual[i]) /
 * sqrt(mean((x + residual)^2) + eps) * weight[i]; [moe.rs] moe_layer runs
 * rmsnorm(hidden, ffn_norm) before the router and the experts, and adds the
 * expert outputs back into hidden.
 *   h[i]  = x[i] + residual[i]           f32 addition (the kernel's float v)
 *   ms    = sum_i h[i]^2 / n             double, ascending i
 *   inv   = 1 / sqrt(ms + eps)           double
 *   xn[i] = (h[i] * inv) * weight[i]     double, rounded once to f32
 * READING: the page's kernel computes the norm in f32 with rsqrtf; here it
 * is computed in double and rounded to f32 once, so that the value handed
 * to the router is the exactly rounded one.  h_out and xn_out may be NULL. */
int qref_add_rmsnorm(const float *x, const float *residual, const float *weight, double eps,
                     int64_t n, float *h_out, float *xn_out) {
    int64_t i;
    double ss = 0.0, inv;
    if (!x || !residual || !weight || n <= 0) return QREF_EINVAL;
    for (i = 0; i < n; i++) {
        float h = x[i] + residual[i];
        ss += (double)h * (double)h;
    }
    inv = 1.0 / sqrt(ss / (double)n + eps);
    for (i = 0; i < n; i++) {
        float h = x[i] + residual[i];
        if (h_out) h_out[i] = h;
        if (xn_out) xn_out[i] = (float)(((double)h * inv) * (double)weight[i]);
    }
    return QREF_OK;
}

/* The MoE FFN behind the fused add + RMSNorm ([moe.rs] moe_layer):
 *   h  = attn_out + hidden_in, xn = rmsnorm(h) * norm_weight   (above)
 *   y  = h + sum_s D[e_s] act[s], the experts and the router reading xn.
 * Outputs as qref_moe_ffn, plus h_out[H] and xn_out[H] (either may be NULL). */
int qref_moe_ffn_norm(const float *attn_out, const float *hidden_in, const float *norm_weight,
                      double eps, const float *router, int gate_fmt, const void *gate,
                      int up_fmt, const void *up, int down_fmt, const void *down,
                      int64_t hidden, int64_t n_experts, int64_t top_k, int64_t expert_dim,
                      double *y, double *bound, double *logits_out, int32_t *sel_out,
                      double *w_out, double *act_out, float *h_out, float *xn_out) {
    int rc;
    float *h, *xn;
    if (hidden <= 0) return QREF_EINVAL;
    h = (float *)malloc(sizeof(float) * (size_t)hidden);
    xn = (float *)malloc(sizeof(float) * (size_t)hidden);
    if (!h || !xn) { free(h); free(xn); return QREF_EINVAL; }
    rc = qref_add_rmsnorm(attn_out, hidden_in, norm_weight, eps, hidden, h, xn);
    if (!rc)
        rc = qref_moe_ffn(xn, h, router, gate_fmt, gate, up_fmt, up, down_fmt, down, hidden,
                          n_experts, top_k, expert_dim, y, bound, logits_out, sel_out, w_out,
                          act_out);
    if (!rc && h_out) memcpy(h_out, h, sizeof(float) * (size_t)hidden);
    if (!rc && xn_out) memcpy(xn_out, xn, sizeof(float) * (size_t)hidden);
    free(h);
    free(xn);
    return rc;
}

/* Activation quantisation of the int8-activation GEMV variant.
 * [gpu.rs] (module notes) and [wm.rs] cpu_int_dot_enabled describe the fast
 * variant only in words: quantise the activation to int8, take integer dot
 * products against the weight codes, convert to float once per block.
 * READING (the pages give no layout): groups of 16 consecutive columns of
 * each activation row; per group, in f32,
 *   amax = max |x|,  d = amax / 127,  id = 1 / d,
 *   q    = rint(x * id)  (round half to even), 0 for every element when
 *          amax = 0, clamped to [-127, 127];
 * the quantised activation is q * d.  A group holding a non-finite value
 * gets d = NaN and q = 0.  cols must be a multiple of 16.  q[cols] int8,
 * d[cols / 16] f32 per activation row. */
int qref_quantize_q8(const float *x, int64_t cols, int8_t *q, float *d) {
    int64_t g, j;
    if (!x || !q || !d || cols <= 0 || cols % 16 != 0) return QREF_EINVAL;
    for (g = 0; g < cols / 16; g++) {
        const float *xg = x + 16 * g;
        float amax = 0.0f, dg;
        int finite = 1;
        for (j = 0; j < 16; j++) {
            float a = fabsf(xg[j]);
            if (!(a <= FLT_MAX)) finite = 0;
            else if (a > amax) amax = a;
        }
        if (!finite) {
            d[g] = NAN;
            for (j = 0; j < 16; j++) q[16 * g + j] = 0;
            continue;
        }
        dg = amax / 127.0f;
        d[g] = dg;
        for (j = 0; j < 16; j++) {
            float id = amax == 0.0f ? 0.0f : 1.0f / dg;
            float v = rintf(xg[j] * id);
            if (v > 127.0f) v = 127.0f;
            if (v < -127.0f) v = -127.0f;
            q[16 * g + j] = (int8_t)v;
        }
    }
    return QREF_OK;
}

/* The GEMV on quantised activations: Y[b][r] = sum_c deq(W)[r][c] *
 * (q[b][c] * d[b][c / 16]), in double, ascending c (each product is exact:
 * a decoded weight times a 7-bit integer times an f32 scale), with the
 * sum of |products| in Yabs (may be NULL).  Layouts as qref_gemv. */
int qref_gemv_q8act(int fmt, const void *W, int64_t rows, int64_t cols, const float *X,
                    int batch, double *Y, double *Yabs) {
    int64_t rb = qref_row_bytes(fmt, cols), r, c;
    double *w = NULL, *xq = NULL;
    int8_t *q = NULL;
    float *d = NULL;
    int b, rc = QREF_OK;
    if (rb < 0) return qref_block_elems(fmt) ? QREF_EINVAL : QREF_EUNSUPPORTED;
    if (!W || !X || !Y || rows <= 0 || batch <= 0 || cols % 16 != 0) return QREF_EINVAL;
    w = (double *)malloc(sizeof(double) * (size_t)cols);
    xq = (double *)malloc(sizeof(double) * (size_t)(cols * batch));
    q = (int8_t *)malloc((size_t)cols);
    d = (float *)malloc(sizeof(float) * (size_t)(cols / 16));
    if (!w || !xq || !q || !d) { rc = QREF_EINVAL; goto done; }
    for (b = 0; b < batch; b++) {
        rc = qref_quantize_q8(X + (int64_t)b * cols, cols, q, d);
        if (rc) goto done;
        for (c = 0; c < cols; c++) xq[(int64_t)b * cols + c] = (double)q[c] * (double)d[c / 16];
    }
    for (r = 0; r < rows; r++) {
        rc = qref_dequant_row(fmt, (const uint8_t *)W + r * rb, cols, w);
        if (rc) goto done;
        for (b = 0; b < batch; b++) {
            double acc = 0.0, aabs = 0.0;
            const double *xb = xq + (int64_t)b * cols;
            for (c = 0; c < cols; c++) {
                double p = w[c] * xb[c];
                acc += p;
                aabs += fabs(p);
            }
            Y[(int64_t)b * rows + r] = acc;
            if (Yabs) Yabs[(int64_t)b * rows + r] = aabs;
        }
    }
done:
    free(w); free(xq); free(q); free(d);
    return rc;
}

/* Bound on how far the int8-activation MoE FFN may depart from the exact
 * one (qref_moe_ffn), per output row.  The variant quantises x, and each
 * slot's f32 SwiGLU activations, per group of 16 columns with the step
 * d = max|v| / 127, so every quantised value is within d / 2 of its input
 * (weight_matrix.rs page, cpu_int_dot_enabled: int8 activations; the group
 * and scale are the reading stated in qref_quantize_q8).  Propagated through
 * the chain of qref_moe_ffn (routes unchanged: the router reads x itself):
 *   dg_j <= sum_c |G_jc| d_x(c) / 2 + 1e-5 sum_c |G_jc x_c|, du_j alike;
 *   da_j <= w (|silu(g_j)| + L dg_j) du_j + w L dg_j |u_j| + 1e-5 |a_j|,
 *           L = 1.1 >= max |silu'|;
 *   the slot's group step as the variant forms it is at most
 *   dq = (max over the group of |a_j| + da_j) / 127;
 *   |dy_r| <= sum_s sum_j |D_rj| (da_j + dq / 2).
 * The 1e-5 terms cover the f32 sums of g, u and a; every half step is
 * widened by 1e-3 for the f32 arithmetic that forms the codes.  A
 * non-finite x gives NaN bounds. */
int qref_moe_q8act_bound(const float *x, const float *residual, const float *router,
                         int gate_fmt, const void *gate, int up_fmt, const void *up,
                         int down_fmt, const void *down, int64_t hidden, int64_t n_experts,
                         int64_t top_k, int64_t expert_dim, double *qbound) {
    const double half = 0.5 * (1.0 + 1e-3), L = 1.1;
    int64_t H = hidden, E = n_experts, K = top_k, F = expert_dim;
    int64_t rb_g = qref_row_bytes(gate_fmt, H), rb_u = qref_row_bytes(up_fmt, H);
    int64_t rb_d = qref_row_bytes(down_fmt, F);
    int64_t e, s, j, r, c;
    int rc = QREF_OK;
    double *logits = NULL, *w = NULL, *row = NULL, *dx = NULL, *da = NULL, *dq = NULL;
    int32_t *sel = NULL;
    if (!x || !residual || !router || !gate || !up || !down || !qbound) return QREF_EINVAL;
    if (H <= 0 || E <= 0 || K <= 0 || F <= 0 || K > E || H % 16 || F % 16) return QREF_EINVAL;
    if (rb_g < 0 || rb_u < 0 || rb_d < 0) return QREF_EUNSUPPORTED;
    logits = (double *)malloc(sizeof(double) * (size_t)E);
    w = (double *)malloc(sizeof(double) * (size_t)K);
    sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    row = (double *)malloc(sizeof(double) * (size_t)(H > F ? H : F));
    dx = (double *)malloc(sizeof(double) * (size_t)H);
    da = (double *)malloc(sizeof(double) * (size_t)(K * F));
    dq = (double *)malloc(sizeof(double) * (size_t)(K * F));
    if (!logits || !w || !sel || !row || !dx || !da || !dq) { rc = QREF_EINVAL; goto done; }

    /* the group step of x at every column */
    for (c = 0; c < H; c += 16) {
        double amax = 0.0;
        for (j = 0; j < 16; j++) {
            double a = fabs((double)x[c + j]);
            amax = (a > amax || a != a) ? a : amax;
        }
        for (j = 0; j < 16; j++) dx[c + j] = amax / 127.0;
    }
    for (e = 0; e < E; e++) {
        double yabs;
        rc = qref_dequant_row(QREF_F32, (const uint8_t *)router + e * H * 4, H, row);
        if (rc) goto done;
        dot_f64(row, x, H, &logits[e], &yabs);
    }
    rc = qref_route(logits, (int)E, (int)K, sel, w);
    if (rc) goto done;

    for (s = 0; s < K; s++) {
        const uint8_t *gb = (const uint8_t *)gate + (int64_t)sel[s] * F * rb_g;
        const uint8_t *ub = (const uint8_t *)up + (int64_t)sel[s] * F * rb_u;
        for (j = 0; j < F; j++) {
            double g = 0, u = 0, gs = 0, us = 0, ga = 0, ua = 0, a, dg, du;
            rc = qref_dequant_row(gate_fmt, gb + j * rb_g, H, row);
            if (rc) goto done;
            for (c = 0; c < H; c++) {
                g += row[c] * (double)x[c];
                gs += fabs(row[c]) * dx[c];
                ga += fabs(row[c] * (double)x[c]);
            }
            rc = qref_dequant_row(up_fmt, ub + j * rb_u, H, row);
            if (rc) goto done;
            for (c = 0; c < H; c++) {
                u += row[c] * (double)x[c];
                us += fabs(row[c]) * dx[c];
                ua += fabs(row[c] * (double)x[c]);
            }
            dg = half * gs + 1e-5 * ga;
            du = half * us + 1e-5 * ua;
            a = w[s] * qref_silu(g) * u;
            da[s * F + j] = w[s] * (fabs(qref_silu(g)) + L * dg) * du + w[s] * L * dg * fabs(u) +
                            1e-5 * fabs(a);
            dq[s * F + j] = fabs(a);  /* |a|, turned into the group step below */
        }
        for (j = 0; j < F; j += 16) {
            double m = 0.0;
            int64_t t;
            for (t = 0; t < 16; t++) {
                double v = dq[s * F + j + t] + da[s * F + j + t];
                m = (v > m || v != v) ? v : m;
            }
            for (t = 0; t < 16; t++) dq[s * F + j + t] = m / 127.0;
        }
    }
    for (r = 0; r < H; r++) {
        double b = 0.0;
        for (s = 0; s < K; s++) {
            const uint8_t *db = (const uint8_t *)down + (int64_t)sel[s] * H * rb_d;
            rc = qref_dequant_row(down_fmt, db + r * rb_d, F, row);
            if (rc) goto done;
            for (j = 0; j < F; j++)
                b += fabs(row[j]) * (da[s * F + j] + half * dq[s * F + j]);
        }
        qbound[r] = b;
    }
done:
    free(logits); free(w); free(sel); free(row); free(dx); free(da); free(dq);
    return rc;
}

/* The int8-activation MoE FFN (the MoE chain of qref_moe_ffn with the
 * expert GEMVs on int8 activations; weight_matrix.rs page,
 * cpu_int_dot_enabled; grouping and scale as qref_quantize_q8):
 *   logits, (sel, w)  as qref_moe_ffn (the router reads x itself);
 *   xq = q d from qref_quantize_q8(x);  g = G xq,  u = U xq  (f64);
 *   a[s] = (float)(w_s silu(g) u), the f32 vector the down GEMV reads;
 *   aq[s] = q d from qref_quantize_q8(a[s]);
 *   y = residual + sum_s D aq[s]   (f64, slots in rank order);
 *   bound[r] = |residual[r]| + sum_s sum_j |D_rj aq_j|.
 * tie[r] (may be NULL): sum of |D_rj| d over the slot elements whose scaled
 * value a / d lies within `window` of a rounding tie (an integer + 1/2) --
 * the most that a one-step change of those codes, as another f32 rounding
 * of a could cause, moves row r. */
int qref_moe_ffn_q8act(const float *x, const float *residual, const float *router,
                       int gate_fmt, const void *gate, int up_fmt, const void *up,
                       int down_fmt, const void *down, int64_t hidden, int64_t n_experts,
                       int64_t top_k, int64_t expert_dim, double window, double *y,
                       double *bound, double *tie, int32_t *sel_out, double *w_out) {
    int64_t H = hidden, E = n_experts, K = top_k, F = expert_dim;
    int64_t rb_g = qref_row_bytes(gate_fmt, H), rb_u = qref_row_bytes(up_fmt, H);
    int64_t rb_d = qref_row_bytes(down_fmt, F);
    int64_t e, s, j, r, c;
    int rc = QREF_OK;
    double *logits = NULL, *w = NULL, *row = NULL, *xq = NULL, *aq = NULL, *near = NULL;
    float *a = NULL, *d = NULL;
    int8_t *q = NULL;
    int32_t *sel = NULL;
    if (!x || !residual || !router || !gate || !up || !down || !y) return QREF_EINVAL;
    if (H <= 0 || E <= 0 || K <= 0 || F <= 0 || K > E || H % 16 || F % 16) return QREF_EINVAL;
    if (rb_g < 0 || rb_u < 0 || rb_d < 0) return QREF_EUNSUPPORTED;
    logits = (double *)malloc(sizeof(double) * (size_t)E);
    w = (double *)malloc(sizeof(double) * (size_t)K);
    sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    row = (double *)malloc(sizeof(double) * (size_t)(H > F ? H : F));
    xq = (double *)malloc(sizeof(double) * (size_t)H);
    aq = (double *)malloc(sizeof(double) * (size_t)(K * F));
    near = (double *)malloc(sizeof(double) * (size_t)(K * F));
    a = (float *)malloc(sizeof(float) * (size_t)F);
    q = (int8_t *)malloc((size_t)(H > F ? H : F));
    d = (float *)malloc(sizeof(float) * (size_t)((H > F ? H : F) / 16));
    if (!logits || !w || !sel || !row || !xq || !aq || !near || !a || !q || !d) {
        rc = QREF_EINVAL;
        goto done;
    }
    for (e = 0; e < E; e++) {
        double yabs;
        rc = qref_dequant_row(QREF_F32, (const uint8_t *)router + e * H * 4, H, row);
        if (rc) goto done;
        dot_f64(row, x, H, &logits[e], &yabs);
    }
    rc = qref_route(logits, (int)E, (int)K, sel, w);
    if (rc) goto done;
    rc = qref_quantize_q8(x, H, q, d);
    if (rc) goto done;
    for (c = 0; c < H; c++) xq[c] = (double)q[c] * (double)d[c / 16];

    for (s = 0; s < K; s++) {
        const uint8_t *gb = (const uint8_t *)gate + (int64_t)sel[s] * F * rb_g;
        const uint8_t *ub = (const uint8_t *)up + (int64_t)sel[s] * F * rb_u;
        for (j = 0; j < F; j++) {
            double g = 0.0, u = 0.0;
            rc = qref_dequant_row(gate_fmt, gb + j * rb_g, H, row);
            if (rc) goto done;
            for (c = 0; c < H; c++) g += row[c] * xq[c];
            rc = qref_dequant_row(up_fmt, ub + j * rb_u, H, row);
            if (rc) goto done;
            for (c = 0; c < H; c++) u += row[c] * xq[c];
            a[j] = (float)(w[s] * qref_silu(g) * u);
        }
        rc = qref_quantize_q8(a, F, q, d);
        if (rc) goto done;
        for (j = 0; j < F; j++) {
            const double dj = (double)d[j / 16];
            const double t = dj > 0.0 ? (double)a[j] / dj : 0.0;
            const double frac = t - floor(t);
            aq[s * F + j] = (double)q[j] * dj;
            near[s * F + j] = fabs(frac - 0.5) < window ? dj : 0.0;
        }
    }
    for (r = 0; r < H; r++) {
        double acc = (double)residual[r], aabs = fabs((double)residual[r]), tb = 0.0;
        for (s = 0; s < K; s++) {
            const uint8_t *db = (const uint8_t *)down + (int64_t)sel[s] * H * rb_d;
            rc = qref_dequant_row(down_fmt, db + r * rb_d, F, row);
            if (rc) goto done;
            for (j = 0; j < F; j++) {
                double p = row[j] * aq[s * F + j];
                acc += p;
                aabs += fabs(p);
                tb += fabs(row[j]) * near[s * F + j];
            }
        }
        y[r] = acc;
        if (bound) bound[r] = aabs;
        if (tie) tie[r] = tb;
    }
    if (sel_out) memcpy(sel_out, sel, sizeof(int32_t) * (size_t)K);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)K);
done:
    free(logits); free(w); free(sel); free(row); free(xq); free(aq); free(near);
    free(a); free(q); free(d);
    return rc;
}
