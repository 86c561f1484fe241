// qg_gemm_ws.hpp -- the batched dequantise-and-dot product with the
// activation operands shared through LDS (qgemv_ws).
//
// The batched kernel of qg_gemm.hpp gives every wave its own copy of the
// activations it multiplies: a 16-row tile re-reads its batch rows'
// activations for every chunk, several times the weight bytes, and that
// stream sets its time (with the activation loads removed it ran 1.7-2.3x
// faster).  Here a workgroup of 8 waves takes 8 tiles (128 rows) over one
// column range, and each chunk's activations are loaded once per workgroup
// with coalesced 16-byte loads, split into bf16 hi and lo parts, and
// written to LDS in the matrix core's operand order; every wave then reads
// its A operands from there.  The column ranges of a row are spread over
// workgroups, so the partial sums go to a caller-provided workspace and a
// second kernel adds them per output in a fixed order (deterministic).
//
// Numbers and the operand layout are those of qg_gemm.hpp: codes exact in
// bf16, each activation x = hi + lo with |x - hi - lo| <= 2^-16 |x|,
// v_mfma_f32_16x16x32_bf16 with lane l holding A[l % 16][8 (l / 16) + j],
// B[8 (l / 16) + j][l % 16] (j < 8) and D[4 (l / 16) + i][l % 16] (i < 4).
// MODE 0 (at most 8 batch rows): hi of batch row b in A row b and its lo in
// row 8 + b, one instruction per block.  MODE 1 (up to 16) and 2 (up to
// 32): separate hi and lo operands per block of 16 batch rows.
#pragma once

#include "qg_gemm.hpp"
#include "qg_kernels.hpp"

namespace qg {
namespace gw {

using gm::Blk;
using gm::bf16x2;
using gm::f32x4;
using gm::kChunk;
using gm::kTileRows;
using gm::mfma;
using gm::u32x4;

constexpr int kWaves = 8;  // tiles per workgroup, one per wave
constexpr int kThreads = 64 * kWaves;

struct WsParams {
    const uint8_t *W;
    const float *X;  // [batch][cols]
    float *Y;        // [batch][rows]
    float *part;     // [kg][batch][rows] partial sums (kg > 1)
    int64_t rows;
    uint64_t w_bytes;   // rows * row_bytes
    uint32_t row_bytes;
    uint32_t cols;
    int32_t batch;      // batch rows of this launch (<= 8, 16 or 32 by MODE)
    int32_t nchunks;    // ceil(cols / 256)
    int32_t last_nkb;   // 32-column blocks in the last chunk (1..8)
    int32_t tiles;      // ceil(rows / 16)
    int32_t kg;         // column ranges (workgroups per group of 8 tiles)
    int32_t nu;         // 16-byte units staged per row segment
    uint32_t slot;      // LDS bytes per staged row (odd multiple of 16)
    // the grouped gate/up products of several MoE tokens (MOE kernels): W is
    // the gate stack, W2 the up stack (w_bytes each), X the T = batch tokens'
    // activations, logits their router logits [T][E]; the routes and route
    // weights [T][K] are written to sel and rw (and sel_out, w_out when
    // given), the SwiGLU activations [T][K][F] to act.  With routed set the
    // routing has been done (moe_route_tokens_kernel) and sel and rw hold it
    const uint8_t *W2;
    int32_t routed;
    const double *logits;
    int32_t *sel, *sel_out;
    float *rw, *w_out;
    float *act;
    int32_t E, F, K, tpe;  // experts, expert rows, routes per token, 16-row tiles per expert
};

// Operand planes per image: MODE 0 one (hi and lo packed), 1 two (hi, lo),
// 2 four (hi, lo of each block of 16 batch rows).  An image plane holds the
// 8 blocks' operands of one chunk, 64 lanes x 16 bytes each.
// KS: column ranges inside a workgroup.  With KS = 2 the workgroup holds 4
// tiles, waves 0-3 take the first half of each row's chunks and waves 4-7
// the second, each half with its own activation images, and the halves'
// sums are added through LDS at the end (no workspace).
template <int MODE, int KS = 1>
struct Mode {
    static constexpr int PLANES = MODE == 0 ? 1 : MODE == 1 ? 2 : 4;
    static constexpr int MAXB = MODE == 0 ? 8 : MODE == 1 ? 16 : 32;
    static constexpr int TH = kThreads / KS;                    // threads per column range
    static constexpr int XU = (MAXB * 64 + TH - 1) / TH;        // activation units per thread
    static constexpr uint32_t IMG_U32 = PLANES * 8 * 64 * 4;   // one image, in dwords
};

// Bytes of LDS a workgroup uses: two activation images per column range,
// the waves' weight slots.
template <int MODE, int KS = 1>
__host__ __device__ constexpr size_t ws_lds_bytes(uint32_t slot) {
    return 2 * KS * (size_t)Mode<MODE>::IMG_U32 * 4 + (size_t)kWaves * kTileRows * slot;
}

// MOE: the tiles are the gate and up rows of the tokens' distinct experts,
// in pairs (wave 2i a gate tile, wave 2i + 1 the up tile of the
// same 16 rows), and the epilogue forms the SwiGLU activations of every
// token that chose the expert instead of storing Y.
template <class F, int MODE, bool RA, int UNITS, int KS = 1, bool MOE = false>
__global__ void __launch_bounds__(kThreads) qgemm_ws_kernel(WsParams p) {
    using M = Mode<MODE, KS>;
    static_assert(KS == 1 || KS == 2, "one or two column ranges per workgroup");
    static_assert(!MOE || (KS == 1 && MODE == 0), "MoE tokens: batch <= 8, one range");
    constexpr int TPG = kWaves / KS;  // tiles per workgroup
    // MOE: every workgroup routes the T tokens (wave t routes token t, as
    // the single-token chain does; workgroup 0 publishes the routes for the
    // down kernel) or, when routed ahead, reads their routes, and one wave
    // lists the distinct experts in route order with each one's slot per
    // token
    __shared__ int s_sel[MOE ? kMaxRoutes : 1];
    __shared__ float s_rw[MOE ? kMaxRoutes : 1];
    __shared__ RouteLds s_rl[MOE ? kWaves : 1];
    __shared__ int s_uexp[MOE ? kMaxRoutes : 1];
    __shared__ int s_uslot[MOE ? kMaxRoutes : 1][kMaxTokens];
    __shared__ int s_nu;
    int nu = 0;
    if constexpr (MOE) {
        const int tid0 = threadIdx.x, w0 = tid0 >> 6;
        for (int i = tid0; i < kMaxRoutes * kMaxTokens; i += kThreads) (&s_uslot[0][0])[i] = -1;
        if (p.routed) {
            // routed ahead (one workgroup per token): the routes and weights
            for (int i = tid0; i < p.batch * p.K; i += kThreads) {
                s_sel[i] = p.sel[i];
                s_rw[i] = p.rw[i];
            }
            __syncthreads();
        } else {
            __syncthreads();
            if (w0 < p.batch)
                route_topk_wave(p.logits + (int64_t)w0 * p.E, p.E, p.K, s_sel + w0 * p.K,
                                s_rw + w0 * p.K, &s_rl[w0]);
            __syncthreads();
            if (blockIdx.x == 0 && tid0 < p.batch * p.K) {
                p.sel[tid0] = s_sel[tid0];
                p.rw[tid0] = s_rw[tid0];
                if (p.sel_out) p.sel_out[tid0] = s_sel[tid0];
                if (p.w_out) p.w_out[tid0] = s_rw[tid0];
            }
        }
        if (w0 == 0) {
            // the dynamic LDS is free until the main loop: the experts' first routes
            extern __shared__ __attribute__((aligned(16))) int s_dyn[];
            const int n =
                distinct_experts(s_sel, p.batch * p.K, p.K, p.E, s_dyn, s_uexp, s_uslot);
            if ((tid0 & 63) == 0) s_nu = n;
        }
        __syncthreads();
        // workgroups past the distinct experts' tiles have nothing more to do
        nu = s_nu;
        if ((int64_t)blockIdx.x * (TPG / 2) >= (int64_t)nu * p.tpe) return;
    }
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave / TPG;          // this wave's column range in the workgroup
    const int htid = tid - half * M::TH;  // thread index inside that range's waves
    uint32_t *img = (uint32_t *)smem + (uint32_t)half * 2 * M::IMG_U32;  // [2][PLANES][8][64][4]
    const int r = lane & 15, q = lane >> 4;
    const int group = (int)(blockIdx.x / (uint32_t)p.kg);
    const int kgi = (int)(blockIdx.x % (uint32_t)p.kg);
    int64_t tile = (int64_t)group * TPG + wave % TPG;
    bool has_tile = tile < p.tiles;
    int moe_u = 0, moe_j = 0;
    if constexpr (MOE) {
        const int pair = (int)blockIdx.x * (TPG / 2) + wave / 2;
        moe_u = pair / p.tpe;
        moe_j = pair - moe_u * p.tpe;
        has_tile = moe_u < nu;
    }
    // column range kgi * KS + half of kg * KS; every range of the workgroup
    // runs the same number of steps (the longest range's), so that the
    // barriers match
    const int nr = p.kg * KS, ri = kgi * KS + half;
    const int c0 = (int)((int64_t)ri * p.nchunks / nr);
    const int c1 = (int)((int64_t)(ri + 1) * p.nchunks / nr);
    const int nsteps = (p.nchunks + nr - 1) / nr;
    uint8_t *stage = smem + 2 * KS * (size_t)M::IMG_U32 * 4 + (size_t)wave * kTileRows * p.slot;

    // zero the images: rows past the batch are never written and read as 0
    for (uint32_t i = (uint32_t)tid; i < 2 * KS * M::IMG_U32 / 4; i += kThreads)
        ((u32x4 *)smem)[i] = u32x4{0u, 0u, 0u, 0u};

    // ---- activations: unit u of a chunk is four columns of one batch row
    const rsrc_t rx = make_rsrc(p.X, 4u * p.cols * (uint32_t)p.batch);
    // every chunk issues the same loads, none under a branch: a chunk past
    // the range (valid false) reads zeros from an out-of-range offset (a
    // count that differs between paths made the compiler wait for all loads)
    auto x_issue = [&](int c, uint32_t (&x)[M::XU][4], bool valid) {
#pragma unroll
        for (int j = 0; j < M::XU; j++) {
            const int u = htid + M::TH * j;
            const int b = u >> 6;
            const uint32_t col = (uint32_t)c * kChunk + 4u * (uint32_t)(u & 63);
            const uint32_t off = (valid && b < p.batch && col < p.cols)
                                     ? 4u * ((uint32_t)b * p.cols + col) : 0x80000000u;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
            x[j][0] = v[0];
            x[j][1] = v[1];
            x[j][2] = v[2];
            x[j][3] = v[3];
        }
    };
    // the units' hi and lo parts into image `buf` at their operand places
    auto x_commit = [&](int buf, const uint32_t (&x)[M::XU][4]) {
#pragma unroll
        for (int j = 0; j < M::XU; j++) {
            const int u = htid + M::TH * j;
            const int b = u >> 6;
            if (b < p.batch) {
                const int c4 = 4 * (u & 63);
                const int kb = c4 >> 5, qq = (c4 >> 3) & 3, h2 = (c4 >> 2) & 1;
                uint32_t hd[2], ld[2];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const float x0 = __builtin_bit_cast(float, x[j][2 * i]);
                    const float x1 = __builtin_bit_cast(float, x[j][2 * i + 1]);
                    const bf16x2 hv = {(__bf16)x0, (__bf16)x1};
                    hd[i] = __builtin_bit_cast(uint32_t, hv);
                    const float h0 = __builtin_bit_cast(float, hd[i] << 16);
                    const float h1 = __builtin_bit_cast(float, hd[i] & 0xFFFF0000u);
                    const bf16x2 lv = {(__bf16)(x0 - h0), (__bf16)(x1 - h1)};
                    ld[i] = __builtin_bit_cast(uint32_t, lv);
                }
                int ph, pl, lh, ll;
                if constexpr (MODE == 0) {
                    ph = pl = 0;
                    lh = b + 16 * qq;
                    ll = b + 8 + 16 * qq;
                } else {
                    const int jb = b >> 4;
                    ph = 2 * jb;
                    pl = 2 * jb + 1;
                    lh = ll = (b & 15) + 16 * qq;
                }
                uint32_t *base = img + (uint32_t)buf * M::IMG_U32;
                uint32_t *dh = base + ((ph * 8 + kb) * 64 + lh) * 4 + 2 * h2;
                uint32_t *dl = base + ((pl * 8 + kb) * 64 + ll) * 4 + 2 * h2;
                dh[0] = hd[0];
                dh[1] = hd[1];
                dl[0] = ld[0];
                dl[1] = ld[1];
            }
        }
    };

    // ---- weights: the wave's tile, staged chunk by chunk into its slot
    uint64_t tb = (uint64_t)(has_tile ? tile : 0) * kTileRows * p.row_bytes;
    const uint8_t *gp = p.W + tb;
    if constexpr (MOE) {
        const uint32_t e = has_tile ? (uint32_t)s_uexp[moe_u] : 0u;
        tb = ((uint64_t)e * p.F + (uint64_t)moe_j * kTileRows) * p.row_bytes;
        gp = ((wave & 1) ? p.W2 : p.W) + tb;
    }
    const uint8_t *al = (const uint8_t *)((uintptr_t)gp & ~(uintptr_t)15);
    const uint32_t d0 = (uint32_t)(gp - al);
    const uint64_t rem = (p.w_bytes - tb + d0 + 15) & ~(uint64_t)15;
    const rsrc_t rw = make_rsrc(al, rem > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)rem);
    const int nunits = kTileRows * p.nu;
    uint32_t u_row[UNITS], u_off[UNITS];
#pragma unroll
    for (int j = 0; j < UNITS; j++) {
        const int u = lane + 64 * j, uu = u < nunits ? u : 0;
        const int rr = uu / p.nu;
        u_row[j] = (uint32_t)rr;
        u_off[j] = 16u * (uint32_t)(uu - rr * p.nu);
    }
    // branch-free: units past the tile's segments (and every unit of a wave
    // without a tile) read zeros from an out-of-range offset; loads under a
    // branch were each followed by a wait for all loads
    auto w_issue = [&](int c, u32x4 (&w)[UNITS], bool valid) {
#pragma unroll
        for (int j = 0; j < UNITS; j++) {
            const uint32_t base = (d0 + u_row[j] * p.row_bytes + (uint32_t)c * F::CHUNK) & ~15u;
            const uint32_t off =
                valid && has_tile && lane + 64 * j < nunits ? base + u_off[j] : 0xFFFFFFF0u;
            w[j] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kStream));
        }
    };
    auto w_store = [&](const u32x4 (&w)[UNITS]) {
#pragma unroll
        for (int j = 0; j < UNITS; j++)
            if (has_tile && lane + 64 * j < nunits)
                *(u32x4 *)(stage + u_row[j] * p.slot + u_off[j]) = w[j];
    };

    constexpr int NBB = MODE == 2 ? 2 : 1;  // blocks of 16 batch rows
    f32x4 acc[NBB];
#pragma unroll
    for (int j = 0; j < NBB; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const uint32_t keep_lo = q < 2 ? 0xFFFFFFFFu : 0u;  // Q6_K: lanes of the first group

    // chunk c: its weights into the slot (the buffer then takes chunk c + 2),
    // the products from image c & 1, then the next chunk's activations into
    // the other image (its reads ended at the previous barrier) and a
    // barrier.  GUARD: the row's last chunk may hold fewer than 8 blocks.
    auto chunk = [&](int c, u32x4 (&wc)[UNITS], uint32_t (&xn)[M::XU][4], auto guard_tag) {
        constexpr bool GUARD = decltype(guard_tag)::value;
        const bool live = !GUARD || c < c1;  // a step past a shorter range computes nothing
        if (live) w_store(wc);
        w_issue(c + 2, wc, c + 2 < c1);
        if (has_tile && live) {
            const int nkb = GUARD && c == p.nchunks - 1 ? p.last_nkb : 8;
            const uint32_t delta =
                (d0 + (uint32_t)r * p.row_bytes + (uint32_t)c * F::CHUNK) & 15u;
            const mx::RowRd<RA> rd = mx::make_rowrd<RA>(stage + r * p.slot, delta, 0);
            const typename F::Head hd = F::template head<RA>(rd, q);
            const u32x4 *im = (const u32x4 *)(img + (uint32_t)(c & 1) * M::IMG_U32);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 8; kb++) {
                if (!GUARD || kb < nkb) {
                    const Blk bk = F::template block<RA, MODE == 0>(rd, hd, kb, q);
                    u32x4 ca = bk.c, cb = bk.c;
                    if constexpr (F::TWO) {
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            ca[i] = bk.c[i] & keep_lo;
                            cb[i] = bk.c[i] & ~keep_lo;
                        }
                    }
#pragma unroll
                    for (int j = 0; j < NBB; j++) {
                        if constexpr (MODE == 0) {
                            const u32x4 a = im[kb * 64 + lane];
                            if constexpr (F::TWO) {
                                const f32x4 da = mfma(a, ca, z), db = mfma(a, cb, z);
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    acc[0][i] = fmaf(bk.s2, db[i], fmaf(bk.s, da[i], acc[0][i]));
                            } else {
                                const f32x4 d = mfma(a, bk.c, z);
                                f32x4 sm = z;
                                if constexpr (F::MINS) sm = mfma(a, ones, z);
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    acc[0][i] = fmaf(bk.s, gm::off128<F, MODE == 0>(d[i], sm[i]), acc[0][i]);
                                if constexpr (F::MINS) {
#pragma unroll
                                    for (int i = 0; i < 4; i++)
                                        acc[0][i] = fmaf(-bk.dm, sm[i], acc[0][i]);
                                }
                            }
                        } else {
                            const u32x4 ah = im[((2 * j) * 8 + kb) * 64 + lane];
                            const u32x4 al2 = im[((2 * j + 1) * 8 + kb) * 64 + lane];
                            if constexpr (F::TWO) {
                                f32x4 da = mfma(ah, ca, z);
                                da = mfma(al2, ca, da);
                                f32x4 db = mfma(ah, cb, z);
                                db = mfma(al2, cb, db);
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    acc[j][i] = fmaf(bk.s2, db[i], fmaf(bk.s, da[i], acc[j][i]));
                            } else {
                                f32x4 d = mfma(ah, bk.c, z);
                                d = mfma(al2, bk.c, d);
                                f32x4 sm = z;
                                if constexpr (F::MINS) {
                                    sm = mfma(ah, ones, z);
                                    sm = mfma(al2, ones, sm);
                                }
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    acc[j][i] = fmaf(bk.s, gm::off128<F, MODE == 0>(d[i], sm[i]), acc[j][i]);
                                if constexpr (F::MINS) {
#pragma unroll
                                    for (int i = 0; i < 4; i++)
                                        acc[j][i] = fmaf(-bk.dm, sm[i], acc[j][i]);
                                }
                            }
                        }
                    }
                }
            }
        }
        if (c + 1 < c1) x_commit((c + 1) & 1, xn);
        x_issue(c + 3, xn, c + 3 < c1);
        __syncthreads();
    };

    // prologue: chunk c0's and c0 + 1's loads, c0's activations into image
    // c0 & 1, c0 + 2's activations in flight
    uint32_t xA[M::XU][4], xB[M::XU][4];
    u32x4 wA[UNITS], wB[UNITS];
    x_issue(c0, xA, c0 < c1);
    w_issue(c0, wA, c0 < c1);
    x_issue(c0 + 1, xB, c0 + 1 < c1);
    w_issue(c0 + 1, wB, c0 + 1 < c1);
    __syncthreads();  // the images are zero
    if (c0 < c1) x_commit(c0 & 1, xA);
    x_issue(c0 + 2, xA, c0 + 2 < c1);
    __syncthreads();
    // chunk c's successor's activations are in xB for even c - c0, xA for
    // odd; the weights of c in wA for even c - c0, wB for odd.  The last one
    // or two steps take the variant that checks for the end of the range and
    // for a partial last chunk.
    int s = 0;
    for (; s + 2 < nsteps; s += 2) {
        chunk(c0 + s, wA, xB, std::false_type{});
        chunk(c0 + s + 1, wB, xA, std::false_type{});
    }
    if (s + 1 == nsteps) {
        chunk(c0 + s, wA, xB, std::true_type{});
    } else {
        chunk(c0 + s, wA, xB, std::true_type{});
        chunk(c0 + s + 1, wB, xA, std::true_type{});
    }

    if constexpr (MODE == 0) {
        // lane (r, q + 2) holds the lo parts' sums of the batch rows whose hi
        // parts' sums lane (r, q) holds
#pragma unroll
        for (int i = 0; i < 4; i++) acc[0][i] += __shfl_xor(acc[0][i], 32);
    }
    if constexpr (KS == 2) {
        // the second range's waves hand their sums to the first range's
        // waves of the same tile through LDS (the images are free after the
        // last step's barrier), which add them in range order
        f32x4 *xch = (f32x4 *)smem + ((wave % TPG) * NBB) * 64 + lane;
        if (half == 1) {
#pragma unroll
            for (int j = 0; j < NBB; j++) xch[j * 64] = acc[j];
        }
        __syncthreads();
        if (half == 1) return;
#pragma unroll
        for (int j = 0; j < NBB; j++) {
            const f32x4 o = xch[j * 64];
#pragma unroll
            for (int i = 0; i < 4; i++) acc[j][i] += o[i];
        }
    }
    if constexpr (MOE) {
        // the up tile's sums go to the gate tile's wave through LDS (the
        // images are free after the last step's barrier), which forms
        // w * silu(g) * u for each token that chose the expert
        f32x4 *xch = (f32x4 *)smem + (wave / 2) * 64 + lane;
        if (wave & 1) xch[0] = acc[0];
        __syncthreads();
        if ((wave & 1) || !has_tile || q >= 2) return;
        const f32x4 up = xch[0];
        const int row = moe_j * kTileRows + r;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int b = 4 * q + i;
            const int sl = b < p.batch ? s_uslot[moe_u][b] : -1;
            if (sl >= 0) {
                const float g = acc[0][i];
                p.act[((int64_t)b * p.K + sl) * p.F + row] =
                    s_rw[b * p.K + sl] * (g / (1.0f + expf(-g))) * up[i];
            }
        }
        return;
    }
    const int64_t row = tile * kTileRows + r;
    if (has_tile && row < p.rows && (MODE != 0 || q < 2)) {
        float *out = p.kg > 1 ? p.part + (size_t)kgi * p.batch * p.rows : p.Y;
#pragma unroll
        for (int j = 0; j < NBB; j++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int b = 16 * j + 4 * q + i;
                if (b < p.batch) out[(int64_t)b * p.rows + row] = acc[j][i];
            }
    }
}

// Y[b][r] = sum over g < kg of part[g][b][r], in order of g.  The partial
// sums come from other XCDs' caches or memory, so each thread issues eight
// loads before it adds any of them.
__global__ void __launch_bounds__(256) ws_reduce_kernel(const float *__restrict__ part,
                                                        float *__restrict__ Y, int64_t n, int kg) {
    constexpr int G = 8;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * 256) {
        float s = 0.f;
        for (int g0 = 0; g0 < kg; g0 += G) {
            float v[G];
#pragma unroll
            for (int j = 0; j < G; j++)
                v[j] = g0 + j < kg ? part[(int64_t)(g0 + j) * n + i] : 0.f;
#pragma unroll
            for (int j = 0; j < G; j++)
                if (g0 + j < kg) s = g0 + j == 0 ? v[j] : s + v[j];
        }
        Y[i] = s;
    }
}

}  // namespace gw
}  // namespace qg
