/*
 * qgemv.h -- C ABI of the MI355X (gfx950) fused dequantise-and-dot library.
 *
 * Two operations, both computed entirely by HIP kernels on the caller's
 * stream:
 *
 *   qgemv    Y = deq(W) * X for a GGUF block-quantised weight matrix W and a
 *            small batch of f32 activation vectors.
 *   moe_ffn  the stacked-expert mixture-of-experts FFN of one decode token:
 *            F32 router GEMV, softmax / top-k / renormalise, then for every
 *            routed expert a gate GEMV, an up GEMV, SwiGLU scaled by the
 *            route weight, and a down GEMV added into the residual.
 *   moe_ffn_norm  the same FFN behind the fused residual add + RMSNorm
 *            that feeds its router.
 *   moe_ffn_tokens  the same FFN for up to 8 decode tokens at once, each
 *            routed on its own, the expert GEMVs grouped by expert.
 *   qgemv_q8act  qgemv at batch 1 on int8-quantised activations (integer
 *            dot products; the pages' lossy fast variant).
 *
 * Sources (web pages):
 *   docs.rs, crate ferrox-cuda 0.14.0, source src/gpu.rs -- block layouts
 *     (the *_MATVEC_KERNEL_SRC kernels), the f16 decoder, SwiGLU
 *     (SILU_MUL_KERNEL_SRC), per-format launch wrappers launch_q*_matvec.
 *   docs.rs, ferrox-core 0.16.0, weight_matrix.rs -- WeightMatrix::apply /
 *     apply_batch (batch-major activations and outputs), block_bytes_per_row.
 *   docs.rs, crate aprender-serve 0.70.2, source
 *     src/gguf/cuda/forward_qwen3_moe_resident.rs -- the module doc's op
 *     order, ExpertStack (expert e at base + e * stride), moe_layer,
 *     last_routes.
 *
 * Conventions common to every entry point:
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The
 *     library allocates nothing, frees nothing and never synchronises the
 *     host; work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and is complete when that stream is.
 *   - Arguments are validated on the host before any HIP call.  On error
 *     nothing is launched, the return value is a QG_E* code and
 *     qg_last_error() names the reason.  Input the kernels do not support is
 *     refused, never computed approximately.
 *   - The entry points hold no global mutable state except the thread-local
 *     error string: calls from several host threads are safe.  Calls that
 *     share an output buffer or a workspace must be ordered by the caller.
 *   - Results are deterministic: no atomics take part in any sum, so the
 *     same inputs on the same stream give the same bits.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats: ggml's numeric type ids (the pages map GGUF dtypes onto
 * their own kinds in weight_matrix.rs quant_kind_for).  Block geometry
 * (elements / bytes): Q4_0 32 / 18, Q8_0 32 / 34, Q4_K 256 / 144,
 * Q5_K 256 / 176, Q6_K 256 / 210.  F32 is one little-endian float per
 * element and is accepted for the MoE router and for qgemv. */
enum qg_format {
    QG_F32 = 0,
    QG_Q4_0 = 2,
    QG_Q8_0 = 8,
    QG_Q4_K = 12,
    QG_Q5_K = 13,
    QG_Q6_K = 14
};

/* Return codes. */
enum qg_status {
    QG_OK = 0,
    QG_EINVAL = 1,       /* a NULL pointer, a non-positive size, k > E, a
                            workspace too small, a weight pointer that is
                            not 2-byte aligned, a float pointer that is not
                            4-byte aligned */
    QG_EUNSUPPORTED = 2, /* an unknown format, cols not a multiple of the
                            block size, batch outside 1..8, a size beyond the
                            kernels' limits, a router that is not F32 */
    QG_ELAUNCH = 3       /* the HIP runtime reported an error at launch */
};

/* Elements per block of fmt, or 0 for an unknown format. */
int qg_block_elems(int fmt);

/* Bytes per block of fmt, or 0 for an unknown format. */
int qg_block_bytes(int fmt);

/* Bytes of one row of cols elements: (cols / block_elems) * block_bytes,
 * rows are packed with no padding (weight_matrix.rs block_bytes_per_row).
 * Returns -1 for an unknown format or cols not a positive multiple of the
 * block size. */
int64_t qg_row_bytes(int fmt, int64_t cols);

/* Reason for the last non-QG_OK return on the calling thread ("" if none).
 * The string stays valid until the next call on the same thread. */
const char *qg_last_error(void);

/*
 * qgemv: Y[b][r] = sum_c deq(W)[r][c] * X[b][c]   for b < batch, r < rows.
 *
 *   fmt    one of enum qg_format.
 *   W      rows * qg_row_bytes(fmt, cols) bytes, row-major, GGUF blocks
 *          exactly as stored in the file (no repacking).  2-byte aligned.
 *   rows   > 0.
 *   cols   > 0, a multiple of qg_block_elems(fmt).
 *   X      float [batch][cols], 4-byte aligned.
 *   Y      float [batch][rows], 4-byte aligned; must not overlap W or X.
 *   batch  1..64.  Up to 8, every weight byte is read from memory once and
 *          used for all batch rows (weight_matrix.rs apply_batch).  Above 8
 *          the rows run as groups of 8, one after another on the stream,
 *          and each group streams the weights again (prefill-sized batches;
 *          results per row as at batch <= 8).
 *   stream hipStream_t or NULL.
 *
 * Dequantisation per element follows the block layouts of the gpu.rs page
 * kernels.  At batch 1 products are formed and accumulated in f32 on the
 * vector ALUs and reduced across lanes with a fixed tree; Q6_K is the
 * exception: its codes meet the activations in exact int32 dot products,
 * each run of 16 activation columns represented as integers X = rint(x *
 * 2^s) with max|X| in [2^21, 2^22), so a run's product sum is off by at
 * most 2^-22 * max|x| * sum|w| over the run (within the tolerance
 * 1e-4 * sum|w x| unless a run's largest |x| exceeds its typical |x| by
 * more than ~400x where the weights meet the large values with small
 * codes).  At batch >= 2 (and for batch-1 rows wider than 512 lane tiles)
 * the block formats run on the matrix cores: codes are exact f16 values
 * (codes at a format's zero point are exact zeros), each 256-column chunk
 * of X is split into f16 hi + lo parts after a power-of-two scaling
 * (relative error < 2^-21 per element), sums are f32.  Results are
 * deterministic run to run.  Limits: rows < 2^31, cols <= 65536; rows that fit neither
 * kernel (e.g. more than ~64 chunks of 256 columns at batch 1 beyond 512
 * lane tiles) return QG_EUNSUPPORTED.  Allocates nothing.
 */
int qgemv(int fmt, const void *W, int64_t rows, int64_t cols, const float *X,
          float *Y, int batch, void *stream);

/*
 * qgemv_q8act: the int8-activation variant of qgemv at batch 1 -- the
 * pages' fast variant, named there only in words (gpu.rs page, module
 * notes: llama.cpp's integer dp4a dot product that converts to float once
 * per block; weight_matrix.rs page, cpu_int_dot_enabled: quantise the
 * activation to int8 and run the integer vec_dot, faster and below the f32
 * reference's precision).
 *
 *   X is quantised per group of 16 consecutive columns: d = max|x| / 127,
 *   id = 1 / d, q = rint(x * id), all f32 (round half to even; 0 for an
 *   all-zero group; a group holding a non-finite value gives NaN outputs).  Then
 *   Y[r] = sum_c deq(W)[r][c] * q[c] * d[c / 16], with the code products
 *   summed exactly in int32 (v_dot4_i32_i8) per group and one f32 multiply
 *   per group.  The result differs from qgemv's by the quantisation of X:
 *   at most sum_c |deq(W)[r][c]| * d[c / 16] / 2 per row.
 *
 *   fmt    a block format (F32 is refused).  W, rows, cols, X [cols],
 *          Y [rows] and stream as qgemv at batch 1; rows of more than 512
 *          lane tiles (32768 columns for the K-quants, 16384 for Q8_0 and
 *          Q4_0) are refused.  Allocates nothing.
 */
int qgemv_q8act(int fmt, const void *W, int64_t rows, int64_t cols,
                const float *X, float *Y, void *stream);

/* Bytes of caller-owned device workspace moe_ffn needs for these sizes
 * (f64 router logits, the k routes, the k SwiGLU activations).  Returns 0
 * for invalid sizes. */
size_t moe_ffn_workspace_bytes(int64_t n_experts, int64_t top_k,
                               int64_t expert_dim);

/*
 * moe_ffn: one token through a Qwen3-MoE-style routed-expert FFN
 * (forward_qwen3_moe_resident.rs, module doc and moe_layer):
 *
 *   logits[e] = sum_i router[e][i] * x[i]            router F32 [E][H],
 *                                                    accumulated in f64
 *   (sel, w)  = top_k of softmax(logits), renormalised over the k chosen;
 *               experts ranked by logit (descending), ties to the lower
 *               index; rank order is also weight order
 *   for each slot s < k, expert e = sel[s]:
 *     g = gate[e] x,  u = up[e] x                     [F][H] stacks
 *     a[s] = w[s] * silu(g) * u,  silu(v) = v / (1 + exp(-v))
 *   y = residual + sum_s down[e] a[s]                 down: [E][H][F]
 *
 *   x, residual   float [H].  y float [H]; y may alias residual (the pages
 *                 update the hidden state in place); y must not alias x.
 *   router        float [E][H] (F32 only).
 *   gate, up      stacks of E matrices [F][H], expert e at
 *                 base + e * F * qg_row_bytes(fmt, H) (ExpertStack::expert);
 *                 formats gate_fmt / up_fmt, any block format.
 *   down          stack of E matrices [H][F], format down_fmt.
 *   hidden H, n_experts E, top_k k, expert_dim F: positive, k <= E,
 *                 k <= 32, E <= 1024, H and F multiples of the block sizes.
 *   sel_experts   int32 [k] or NULL: the chosen experts in rank order.
 *   sel_weights   float [k] or NULL: their renormalised weights.
 *   workspace     device memory of at least
 *                 moe_ffn_workspace_bytes(E, k, F) bytes, 16-byte aligned.
 *                 Its first E doubles hold the router logits after the call.
 *                 Overwritten by every call; no initial contents needed.
 *   stream        hipStream_t or NULL.
 *
 * Three kernels are enqueued (router; routing + gate/up + SwiGLU; down +
 * residual).  No host round trip takes place between them.
 */
int moe_ffn(const float *x, const float *residual, float *y,
            const float *router, int gate_fmt, const void *gate, int up_fmt,
            const void *up, int down_fmt, const void *down, int64_t hidden,
            int64_t n_experts, int64_t top_k, int64_t expert_dim,
            int32_t *sel_experts, float *sel_weights, void *workspace,
            size_t workspace_bytes, void *stream);

/*
 * moe_ffn_noalloc: moe_ffn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, semantics, kernels, results and errors are those
 * of moe_ffn, without the workspace: the library keeps one scratch array
 * of 1 MiB (1,048,576 bytes) in device memory, per GPU it runs on, for the
 * life of the process, and uses it as the workspace.  Sizes whose
 * moe_ffn_workspace_bytes exceed it are refused with QG_EUNSUPPORTED.  The
 * device current on the calling thread must be the device of `stream`.
 * Calls no allocating routine.  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents (its first E doubles hold the
 * router logits of the last call): calls that overlap on one GPU race.
 */
int moe_ffn_noalloc(const float *x, const float *residual, float *y,
                    const float *router, int gate_fmt, const void *gate, int up_fmt,
                    const void *up, int down_fmt, const void *down, int64_t hidden,
                    int64_t n_experts, int64_t top_k, int64_t expert_dim,
                    int32_t *sel_experts, float *sel_weights, void *stream);

/* Bytes of caller-owned device workspace moe_ffn_tokens needs for T tokens
 * (f64 logits [T][E], the routes [T][k], the activations [T][k][F]).
 * Returns 0 for invalid sizes. */
size_t moe_ffn_tokens_workspace_bytes(int64_t tokens, int64_t n_experts,
                                      int64_t top_k, int64_t expert_dim);

/*
 * moe_ffn_tokens: moe_ffn for T decode tokens at once, each routed on its
 * own (forward_qwen3_moe_resident.rs, moe_layer, per token):
 *
 *   y[t] = residual[t] + sum_s down[e_{t,s}] a[t][s]   for t < T,
 *
 * with every quantity as moe_ffn defines it for token t.  The expert GEMVs
 * are grouped by expert: within each group of up to four tokens, the gate
 * and up rows of every expert that a token of the group selected are read
 * once and dotted with the group's activations (weight_matrix.rs
 * apply_batch semantics), and each token that chose the expert receives
 * its own SwiGLU activation.  The down GEMVs run per token.
 *
 *   x, residual, y  float [T][H]; y may alias residual, not x.
 *   tokens       T, 1..8, with T * top_k <= 64.
 *   sel_experts  int32 [T][k] or NULL, sel_weights float [T][k] or NULL.
 *   workspace    moe_ffn_tokens_workspace_bytes(T, E, k, F) bytes, 16-byte
 *                aligned; its first T * E doubles hold the logits [T][E].
 *   Other arguments as moe_ffn.  T = 1 runs the moe_ffn kernels.
 *   Results per token equal moe_ffn's on that token to the moe_ffn
 *   tolerance (the expert dot products are summed with the batch-B tile
 *   widths, a different order); the routing is identical.
 */
int moe_ffn_tokens(const float *x, const float *residual, float *y,
                   const float *router, int gate_fmt, const void *gate,
                   int up_fmt, const void *up, int down_fmt, const void *down,
                   int64_t tokens, int64_t hidden, int64_t n_experts,
                   int64_t top_k, int64_t expert_dim, int32_t *sel_experts,
                   float *sel_weights, void *workspace, size_t workspace_bytes,
                   void *stream);

/* Bytes of caller-owned device workspace moe_ffn_norm needs: the moe_ffn
 * workspace plus the H normed activations.  Returns 0 for invalid sizes. */
size_t moe_ffn_norm_workspace_bytes(int64_t hidden, int64_t n_experts,
                                    int64_t top_k, int64_t expert_dim);

/*
 * moe_ffn_norm: moe_ffn behind the fused residual add + RMSNorm that feeds
 * the router (gpu.rs page, FUSED_ADD_RMSNORM_KERNEL_SRC: out = (x + r) /
 * sqrt(mean((x + r)^2) + eps) * weight; forward_qwen3_moe_resident.rs page,
 * moe_layer: rmsnorm(hidden, ffn_norm) feeds the router and the experts,
 * whose outputs are added back into hidden):
 *
 *   h[i]   = attn_out[i] + hidden_in[i]            f32 addition
 *   inv    = 1 / sqrt(sum_i h[i]^2 / H + eps)      f64
 *   xn[i]  = (h[i] * inv) * norm_weight[i]         f64, rounded once to f32
 *   hidden_out = h + sum_s down[e_s] a[s]          the moe_ffn chain on x = xn
 *
 *   attn_out, hidden_in, norm_weight  float [H] (device), 4-byte aligned.
 *   eps          the norm's epsilon (>= 0, finite).
 *   hidden_out   float [H]; may alias attn_out or hidden_in (each element
 *                is read and then written by the same thread).
 *   normed       float [H] or NULL: receives xn.  Must not alias any input.
 *   The other arguments are those of moe_ffn; the workspace must hold
 *   moe_ffn_norm_workspace_bytes(H, E, k, F) bytes, 16-byte aligned.
 *
 * Three kernels are enqueued: add + norm + router (every workgroup reduces
 * the sum of squares itself, in f64, so no extra launch or grid-wide sync
 * is needed); routing + gate/up + SwiGLU on xn; down + the residual add
 * h = attn_out + hidden_in.  Errors as moe_ffn, plus QG_EINVAL for a
 * negative or non-finite eps.
 */
int moe_ffn_norm(const float *attn_out, const float *hidden_in,
                 float *hidden_out, const float *norm_weight, float eps,
                 float *normed, const float *router, int gate_fmt,
                 const void *gate, int up_fmt, const void *up, int down_fmt,
                 const void *down, int64_t hidden, int64_t n_experts,
                 int64_t top_k, int64_t expert_dim, int32_t *sel_experts,
                 float *sel_weights, void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * qg_route_topk: the routing step of moe_ffn on its own, on given logits
 * (forward_qwen3_moe_resident.rs module doc: softmax, top-k, renormalise).
 *
 *   logits       double [n_experts] (device).
 *   sel_experts  int32 [top_k], sel_weights float [top_k] (device): the
 *                chosen experts in rank order and their weights; both
 *                required.
 *   n_experts 1..1024, top_k 1..min(32, n_experts).
 *
 * One workgroup; the same device code moe_ffn uses, so a test can check the
 * selection bit for bit on identical logits.
 */
int qg_route_topk(const double *logits, int64_t n_experts, int64_t top_k,
                  int32_t *sel_experts, float *sel_weights, void *stream);

/*
 * qg_stream_read: a measurement helper, not a step of the method.  Reads
 * `bytes` bytes of `buf` once with coalesced 16-byte non-temporal loads
 * (the cache policy of the GEMVs' weight streams) and stores the XOR of
 * what each workgroup read to out[workgroup].  Its time is the streaming
 * floor of a kernel that must read that many bytes, against which the
 * GEMVs' batch-1 times are read (weight_matrix.rs page, apply_batch notes:
 * reading the weights is the bottleneck, not the arithmetic).
 *
 *   buf    device memory, 16-byte aligned; bytes a positive multiple of 16.
 *   out    uint32 [grid] (device).
 *   grid   workgroups of 512 threads (each takes 32 KiB per round, all of a
 *          round's loads in flight together); <= 0 picks
 *          min(ceil(bytes / 32 KiB), 2048).  A grid above that count is
 *          reduced to it.
 *   stream hipStream_t or NULL.
 */
int qg_stream_read(const void *buf, size_t bytes, uint32_t *out, int grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
