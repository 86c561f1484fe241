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
 *   qgemv_ws  qgemv at batch >= 2 with a caller-provided workspace (the
 *            activations shared through LDS; qgemv_ws_bytes sizes it).
 *   qgemv_q8act  qgemv at batch 1 on int8-quantised activations (integer
 *            dot products; the pages' lossy fast variant).
 *   moe_ffn_q8act  moe_ffn with its expert GEMVs on int8-quantised
 *            activations.
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
    QG_ELAUNCH = 3       /* the HIP runtime reported an error at launch, or
                            still held one from earlier work on the calling
                            thread when the call was about to launch (then
                            nothing is launched; the error is cleared) */
};

/* Elements per block of fmt, or 0 for an unknown format: 32 for Q8_0 and
 * Q4_0, 256 for the K-quants (the super-block of the gpu.rs page's
 * *_MATVEC_KERNEL_SRC kernels), 1 for F32. */
int qg_block_elems(int fmt);

/* Bytes per block of fmt, or 0 for an unknown format: Q8_0 34, Q4_0 18,
 * Q4_K 144, Q5_K 176, Q6_K 210 (the block layouts of the same kernels),
 * F32 4. */
int qg_block_bytes(int fmt);

/* Bytes of one row of cols elements: (cols / block_elems) * block_bytes,
 * rows are packed with no padding (weight_matrix.rs block_bytes_per_row).
 * Returns -1 for an unknown format or cols not a positive multiple of the
 * block size. */
int64_t qg_row_bytes(int fmt, int64_t cols);

/* Reason for the last non-QG_OK return on the calling thread ("" if none).
 * Every refusal names its reason, as the aprender-serve page's `refuse`
 * does for the resident MoE path.  The string stays valid until the next
 * call on the same thread. */
const char *qg_last_error(void);

/* The arithmetic of the last qgemv, qgemv_ws or qgemv_q8act call on the calling
 * thread that returned QG_OK ("" before any):
 *   "valu_f32"      f32 products and sums on the vector ALUs;
 *   "valu_q6k_int"  Q6_K at batch 1: integer activation digits, exact int32
 *                   dot products, f32 per run (see qgemv);
 *   "mfma_i8_q6k"   the same arithmetic with the int32 products on the
 *                   matrix cores (Q6_K batch-1 rows of up to 4096 columns);
 *   "mx_f16"        matrix cores, f16 codes x f16 hi + lo activation parts;
 *   "gemm_bf16"     matrix cores, bf16 codes x bf16 hi + lo activation parts;
 *   "gemm_ws_bf16"  the same arithmetic, activation operands shared through
 *                   LDS (qgemv_ws);
 *   "gemm_ks2_bf16" the same arithmetic, activation operands shared through
 *                   LDS by 4 row tiles, two column ranges per workgroup
 *                   added in LDS (qgemv, batch 2-8, tall matrices);
 *   "valu_q8act"    int8 codes x int8 activations (qgemv_q8act).
 * A static string; reporting only, no effect on any call. */
const char *qg_last_kernel(void);

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
 *   batch  1..64.  Block formats: every weight byte is read from memory
 *          once per launch and used for all batch rows of the launch
 *          (weight_matrix.rs apply_batch); a launch takes up to 32 rows, so
 *          batches of 33..64 read the weights twice.  F32: up to 8 rows per
 *          launch, larger batches as groups of 8.
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
 * codes); rows of 256..2048 columns (any multiple of 256) or of 512..4096
 * (any multiple of 512) form those int32 products on the matrix cores
 * (v_mfma_i32_16x16x64_i8, 16 weight rows per instruction), the same sums
 * bit for bit in int32.  Q6_K matrices of 16 MiB or more run the same
 * kernel at batch 2, both rows against each tile's codes (the weights read
 * once; each row's result bit-identical to its batch-1 result), and those
 * of 128 MiB or more at batch 3..4 as launches of two rows and one.  At
 * batch >= 2 (and for batch-1 rows wider than 512 lane tiles)
 * the block formats run on the matrix cores with the codes as exact
 * integers (codes at a format's zero point are exact zeros) and f32 sums:
 * at batch 2..4 on rows of at most 1024 columns when the activations fit
 * in LDS (and the matrix is not tall enough for the shared-activation
 * kernel below), and for the over-wide batch-1 rows, as f16 codes with each 256-column chunk of X
 * split into f16 hi + lo parts after a power-of-two scaling (relative
 * error < 2^-21 per element); otherwise as bf16 codes with X split into
 * bf16 hi + lo parts (relative error <= 2^-16 per element).  Matrices of
 * at least 192 groups of 4 row tiles (12,241 rows or more) and 4 or more
 * 256-column chunks run each launch of 2..32 batch rows (Q8_0: 2..16) on a
 * kernel whose workgroups share each activation chunk between 4 row tiles
 * through LDS and add two column ranges in LDS ("gemm_ks2_bf16", no
 * workspace).  qg_last_kernel() names the
 * arithmetic a call used.  Results are
 * deterministic run to run.  Limits: rows < 2^31, cols <= 65536; rows that fit neither
 * kernel (e.g. more than ~64 chunks of 256 columns at batch 1 beyond 512
 * lane tiles) return QG_EUNSUPPORTED.  Allocates nothing.
 */
int qgemv(int fmt, const void *W, int64_t rows, int64_t cols, const float *X,
          float *Y, int batch, void *stream);

/*
 * qgemv_ws: qgemv with a caller-provided workspace, for batch >= 2.
 *
 * Same arguments, result and tolerance as qgemv (weight_matrix.rs
 * apply_batch: each weight row's bytes read once per launch of up to 32
 * batch rows and dotted with every activation of the batch), with the
 * block formats at batch 2..64 on a kernel that loads each activation
 * chunk once per workgroup of 8 row tiles and shares it through LDS.  A
 * row's columns are split over several workgroups; their partial sums go
 * to the workspace and a second kernel adds them per output in a fixed
 * order, so results are deterministic run to run (they differ from
 * qgemv's in rounding only).  At batch 2..16 the matrices on which qgemv
 * runs "gemm_ks2_bf16" (4 row tiles per workgroup, two column ranges added
 * in LDS) take that kernel here too, with no workspace (qgemv_ws_bytes 0).
 * F32, batch 1, and batch 2..8 on rows of at most 16 chunks of 256 columns
 * that this kernel would split over several workgroups (there qgemv's
 * kernels are faster) run qgemv itself, with no workspace.
 *
 *   workspace        device memory of at least qgemv_ws_bytes(fmt, rows,
 *                    cols, batch) bytes, 16-byte aligned, owned by the
 *                    caller; no initial contents needed.  May be NULL when
 *                    that size is 0.  Calls that overlap in time on one
 *                    workspace race.
 *   workspace_bytes  its size.
 *
 * Errors as qgemv; QG_EINVAL for a missing, short or misaligned workspace.
 * qg_last_kernel() reports "gemm_ws_bf16" for the batched kernel.
 * Allocates nothing.
 */
int qgemv_ws(int fmt, const void *W, int64_t rows, int64_t cols, const float *X,
             float *Y, int batch, void *workspace, size_t workspace_bytes,
             void *stream);

/* Workspace bytes qgemv_ws needs for these arguments: 0 when none is needed
 * (F32, batch 1, no row split over several workgroups, the calls that run
 * qgemv itself) and for arguments
 * qgemv_ws refuses.  Depends only on the arguments, not on the device. */
size_t qgemv_ws_bytes(int fmt, int64_t rows, int64_t cols, int batch);

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
 * (f64 router logits, the k routes, the k SwiGLU activations): the
 * per-layer device buffers of the aprender-serve page's `Scratch`, owned
 * here by the caller.  Returns 0 for invalid sizes. */
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
 * (f64 logits [T][E], the routes [T][k] and their weights, the activations
 * [T][k][F], each section 16-byte aligned).  Returns 0 for invalid sizes. */
size_t moe_ffn_tokens_workspace_bytes(int64_t tokens, int64_t n_experts,
                                      int64_t top_k, int64_t expert_dim);

/*
 * moe_ffn_tokens: moe_ffn for T decode tokens at once, each routed on its
 * own (forward_qwen3_moe_resident.rs, moe_layer, per token):
 *
 *   y[t] = residual[t] + sum_s down[e_{t,s}] a[t][s]   for t < T,
 *
 * with every quantity as moe_ffn defines it for token t.  The expert GEMVs
 * are grouped by expert: the gate and up rows of every expert that any of
 * the T tokens selected are read once per call and dotted with all T
 * tokens' activations (weight_matrix.rs apply_batch semantics) on the
 * matrix cores, as qgemv does at batch 2..8 (bf16 codes, each activation
 * split into bf16 hi + lo parts, f32 sums), and each token that chose the
 * expert receives its own SwiGLU activation.
 * The down GEMVs run per token.
 *
 *   x, residual, y  float [T][H]; y may alias residual, not x.
 *   tokens       T, 1..8, with T * top_k <= 64.
 *   sel_experts  int32 [T][k] or NULL, sel_weights float [T][k] or NULL.
 *   workspace    moe_ffn_tokens_workspace_bytes(T, E, k, F) bytes, 16-byte
 *                aligned; its first T * E doubles hold the logits [T][E].
 *   Other arguments as moe_ffn.  T = 1 runs the moe_ffn kernels.
 *   Results per token equal moe_ffn's on that token to the moe_ffn
 *   tolerance (the gate and up dot products are formed as above, in a
 *   different order); the routing is identical.
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
 * moe_ffn_q8act: moe_ffn with the expert GEMVs on int8-quantised
 * activations -- the pages' fast variant (gpu.rs page, module notes on the
 * integer dp4a dot product; weight_matrix.rs page, cpu_int_dot_enabled)
 * carried into the MoE chain, whose routing the aprender-serve page pins to
 * the float kernels until its effect on the routes is measured
 * (with_max_seq_len, the Q4kVariant / Q6kVariant pin).
 *
 *   The router GEMV, the routing and the residual add are moe_ffn's (the
 *   router reads the unquantised x, so the routes of this call are
 *   moe_ffn's bit for bit).  The gate and up GEMVs read x quantised as in
 *   qgemv_q8act (groups of 16 columns, d = max|x| / 127, q = rint(x / d)
 *   formed as x * (1 / d) in f32); the down GEMV reads each slot's f32
 *   activations a[s] = w[s] * silu(g) * u quantised the same way.  Integer
 *   code products summed exactly per group, one f32 multiply per group.
 *   Versus moe_ffn the output moves by the quantisation of x (through g, u
 *   and SwiGLU) and of a[s]: per row at most
 *   sum_s sum_j |down[e_s][r][j]| * (|da[s][j]| + d_a[s][j] / 2), where da
 *   is the change of a[s] that the gate/up quantisation causes.
 *
 *   Arguments, layouts, workspace (moe_ffn_workspace_bytes) and errors as
 *   moe_ffn.  Allocates nothing.
 */
int moe_ffn_q8act(const float *x, const float *residual, float *y,
                  const float *router, int gate_fmt, const void *gate,
                  int up_fmt, const void *up, int down_fmt, const void *down,
                  int64_t hidden, int64_t n_experts, int64_t top_k,
                  int64_t expert_dim, int32_t *sel_experts, float *sel_weights,
                  void *workspace, size_t workspace_bytes, void *stream);

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
