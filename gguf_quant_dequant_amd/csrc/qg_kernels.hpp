// qg_kernels.hpp -- the gfx950 kernels: the batched dequantise-and-dot GEMV
// and the three kernels of the stacked-expert MoE FFN.
//
// GEMV work layout.  A "row group" of lanes covers one weight row: lane g of
// the group owns tile g (a fixed column set, see qg_formats.hpp), holds its
// activations for all B batch columns in VGPRs, and walks rows.  A group is
// `lpr` lanes of one wave (a power of two <= 64) or S whole waves.  Every
// iteration a workgroup takes G*U consecutive rows, group g rows
// [g*U, g*U+U): all U rows' loads are issued before any is used.  Partial
// sums are reduced inside the wave with DPP / swizzle / bpermute and, for
// S > 1, across the group's waves through LDS, in a fixed order.
//
// MoE (web page: docs.rs, crate aprender-serve 0.70.2, source
// src/gguf/cuda/forward_qwen3_moe_resident.rs -- module doc and moe_layer):
//   K1 moe_router_kernel   logits[e] = R[e] . x in f64, one wave per expert
//   K2 moe_gateup_kernel   every workgroup ranks the logits (softmax, top-k,
//                          renormalise, ties to the lower index); then row
//                          tasks (slot s, row j) compute g = G[e_s][j] . x
//                          and u = U[e_s][j] . x and store
//                          a[s][j] = w_s * silu(g) * u
//   K3 moe_down_kernel     y[r] = residual[r] + sum_s D[e_s][r] . a[s]; the
//                          lanes of a row group own (slot, tile) pairs
#pragma once

#include "qg_formats.hpp"

// Cache policy of the router rows (read once per token, whole lines per
// wave instruction).
#ifndef QG_ROUTER_AUX
#define QG_ROUTER_AUX 0
#endif

namespace qg {

struct GemvParams {
    const uint8_t *W;
    const float *X;
    float *Y;
    int64_t rows;
    uint64_t w_bytes;    // rows * row_bytes
    uint32_t row_bytes;
    uint32_t cols;
    uint32_t batch_x;    // X rows present (>= B is not required: B <= batch_x)
    int32_t tiles;       // tiles per row
    int32_t lpr;         // lanes per row group inside a wave (S == 1)
    int32_t S;           // waves per row group
    int32_t G;           // row groups per workgroup
};

// Row offset of a load that is not wanted: every resource built by
// rows_rsrc ends at or below it, so the load reads zeros and touches no
// memory.  Loads under a branch would wait for each other (a realigning
// load uses its data at once and the compiler keeps it inside the branch),
// so unwanted rows are loaded from here instead of being skipped.
constexpr uint32_t kOorRow = 0xFFFF0000u;

// Buffer resource for the weight bytes from byte `start` of W to the end
// (w_bytes): base rounded down to 4 bytes, *delta = bytes between that base
// and W + start.  The record count is rounded up to a whole dword: a dword
// that only partly overlaps the array is read whole (its other bytes lie in
// the same page), while the hardware returns zero for a dword that overlaps
// the record range only in part.
__device__ __forceinline__ rsrc_t rows_rsrc(const uint8_t *W, uint64_t w_bytes, uint64_t start,
                                            uint32_t *delta) {
    const uint8_t *base = W + start;
    const uint8_t *abase = (const uint8_t *)((uintptr_t)base & ~(uintptr_t)3);
    *delta = (uint32_t)(base - abase);
    const uint64_t rem = (w_bytes - start + *delta + 3) & ~(uint64_t)3;
    return make_rsrc(abase, rem > kOorRow ? kOorRow : (uint32_t)rem);
}

template <class F, int B, int U>
__device__ __forceinline__ void gemv_issue(const GemvParams &p, int64_t it, int grp, bool active,
                                           const typename F::Lane &L,
                                           typename F::Raw (&raw)[U]) {
    const int64_t r0 = it * ((int64_t)p.G * U);
    uint32_t delta;
    const rsrc_t rs = rows_rsrc(p.W, p.w_bytes, (uint64_t)r0 * p.row_bytes, &delta);
    const int64_t rg = r0 + (int64_t)grp * U;
#pragma unroll
    for (int u = 0; u < U; u++)
        F::load(BufReader{rs},
                active && rg + u < p.rows ? delta + (uint32_t)(grp * U + u) * p.row_bytes : kOorRow,
                L, raw[u]);
}

// Dequantise-and-dot of one block of rows already loaded into raw, then the
// reduction across the row group and the stores.
template <class F, int B, int U>
__device__ __forceinline__ void gemv_finish(const GemvParams &p, int64_t it, int grp, int lig,
                                            int lane, int wave, bool active,
                                            const typename F::Lane &L,
                                            const typename F::Raw (&raw)[U],
                                            const typename F::template XTile<B> &xt,
                                            float (*red)[U * B]) {
    const int64_t rg = it * ((int64_t)p.G * U) + (int64_t)grp * U;
    float acc[U * B];
#pragma unroll
    for (int u = 0; u < U; u++) {
        float a[B];
#pragma unroll
        for (int b = 0; b < B; b++) a[b] = 0.f;
        if (active && rg + u < p.rows) F::template dot<B>(raw[u], L, xt, a);
#pragma unroll
        for (int b = 0; b < B; b++) acc[u * B + b] = a[b];
    }
    group_sum_all(acc, p.S == 1 ? p.lpr : 64);
    if (p.S == 1) {
        if (lig == 0) {
#pragma unroll
            for (int u = 0; u < U; u++)
                if (rg + u < p.rows)
#pragma unroll
                    for (int b = 0; b < B; b++) p.Y[b * p.rows + rg + u] = acc[u * B + b];
        }
    } else {
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < U * B; i++) red[wave][i] = acc[i];
        }
        __syncthreads();
        if (wave % p.S == 0 && lane < U * B) {
            float s = 0.f;
            for (int w = 0; w < p.S; w++) s += red[wave + w][lane];
            const int u = lane / B, b = lane % B;
            if (rg + u < p.rows) p.Y[b * p.rows + rg + u] = s;
        }
        __syncthreads();
    }
}

// Row blocks are double-buffered: the loads of the next block are issued
// before the current one is dequantised, so memory latency overlaps compute.
// The first block's loads go out before the activations are read.
template <class F, int B, int U>
__global__ void __launch_bounds__(512) qgemv_kernel(GemvParams p) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int grp, lig;
    if (p.S == 1) {
        grp = wave * (64 / p.lpr) + lane / p.lpr;
        lig = lane & (p.lpr - 1);
    } else {
        grp = wave / p.S;
        lig = (wave % p.S) * 64 + lane;
    }
    const bool active = lig < p.tiles;
    const typename F::Lane L = F::init(active ? lig : 0);
    const int64_t rpi = (int64_t)p.G * U;
    const int64_t step = gridDim.x;

    typename F::Raw ra[U], rb[U];
    int64_t it = blockIdx.x;
    if (it * rpi < p.rows) gemv_issue<F, B, U>(p, it, grp, active, L, ra);

    typename F::template XTile<B> xt;
    {
        const rsrc_t rx = make_rsrc(p.X, 4u * p.cols * (uint32_t)B);
        float x[B][F::CPT];
        load_tile_x<F, B>(rx, p.cols, L, active, x);
        F::template prep<B>(x, xt);
    }

    __shared__ float red[8][U * B];
    while (it * rpi < p.rows) {
        if ((it + step) * rpi < p.rows) gemv_issue<F, B, U>(p, it + step, grp, active, L, rb);
        gemv_finish<F, B, U>(p, it, grp, lig, lane, wave, active, L, ra, xt, red);
        it += step;
        if (it * rpi >= p.rows) break;
        if ((it + step) * rpi < p.rows) gemv_issue<F, B, U>(p, it + step, grp, active, L, ra);
        gemv_finish<F, B, U>(p, it, grp, lig, lane, wave, active, L, rb, xt, red);
        it += step;
    }
}

// ----------------------------------------------------- LDS-staged variant
//
// Each iteration a workgroup takes G*U consecutive rows.  Their bytes are
// read with 16-byte buffer loads in which thread t fetches chunks t,
// t + nthr, ... of the block (each wave instruction reads one contiguous
// KiB, every cache line is requested once), held in VGPRs, and written to
// LDS; after a barrier each lane reads its tile's fields from LDS and
// proceeds as in qgemv_kernel.  The loads of block i+1 are issued before
// block i is dequantised, so the copy overlaps the arithmetic.
//
// Copies start at the 16-byte boundary at or below the block's first byte.
// Every thread issues kStageChunks loads per block; a chunk past the array
// end is out of range (reads zero, no memory access), and the record count
// is rounded up to 16 bytes, so a chunk that overlaps the array is read
// whole (its extra bytes lie in the same page).

constexpr int kStageChunks = 8;  // 16-byte chunks per thread per block

struct StageBlock {
    rsrc_t rs;
    uint32_t d16;  // offset of the block's first byte in the stage
    uint32_t nch;  // 16-byte chunks that hold the block
};

__device__ __forceinline__ StageBlock stage_block(const GemvParams &p, int64_t it, int64_t rpi) {
    const int64_t r0 = it * rpi;
    const uint8_t *g0 = p.W + (uint64_t)r0 * p.row_bytes;
    const uint8_t *g16 = (const uint8_t *)((uintptr_t)g0 & ~(uintptr_t)15);
    const int64_t nrows = p.rows - r0 < rpi ? p.rows - r0 : rpi;
    StageBlock b;
    b.d16 = (uint32_t)(g0 - g16);
    b.nch = (b.d16 + (uint32_t)nrows * p.row_bytes + 15u) >> 4;
    const uint64_t rem = (p.w_bytes - (uint64_t)r0 * p.row_bytes + b.d16 + 15) & ~(uint64_t)15;
    b.rs = make_rsrc(g16, rem > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)rem);
    return b;
}

__device__ __forceinline__ void stage_fetch(const StageBlock &b, int tid, uint32_t nthr,
                                            uint32_t (&reg)[kStageChunks][4]) {
#pragma unroll
    for (int j = 0; j < kStageChunks; j++) {
        // chunks past the block read from an out-of-range offset: zeros,
        // no memory traffic
        const uint32_t c = j * nthr + (uint32_t)tid;
        const uint32_t off = c < b.nch ? 16u * c : 0xFFFFFFF0u;
        auto v = __builtin_amdgcn_raw_buffer_load_b128(b.rs, off, 0, kStream);
        reg[j][0] = v[0]; reg[j][1] = v[1]; reg[j][2] = v[2]; reg[j][3] = v[3];
    }
}

__device__ __forceinline__ void stage_store(uint32_t *stage, int tid, uint32_t nthr,
                                            const uint32_t (&reg)[kStageChunks][4]) {
#pragma unroll
    for (int j = 0; j < kStageChunks; j++) {
        uint32_t *d = stage + 4 * (j * nthr + (uint32_t)tid);
        d[0] = reg[j][0]; d[1] = reg[j][1]; d[2] = reg[j][2]; d[3] = reg[j][3];
    }
}

// Activations through LDS.  Loading a lane's tile straight from global
// memory makes every load instruction touch one cache line per lane (the
// tiles of neighbouring lanes lie CPT floats apart), which costs more than
// the weight stream on small matrices.  Instead the workgroup copies
// X[b][c0, c0 + n) into the stage buffer with coalesced 16-byte loads and
// each lane then reads its runs from LDS.  16-byte chunk j of a round is
// stored at chunk j ^ ((j >> 4) & 15): the lanes of one LDS read phase then
// fall on distinct banks for every tile layout used here (at most two-way
// conflicts).  X is copied as one flat array of B * cols floats, in rounds
// of up to 32 floats per thread (the stage's size, a multiple of 2048).
// Every run of a tile starts at a multiple of RUNLEN, and RUNLEN divides
// both cols and the round size, so no run straddles two rounds.

__device__ __forceinline__ uint32_t xs_pos(uint32_t j) { return j ^ ((j >> 4) & 15u); }

// Loads 16-byte chunks tid, tid + nthr, ... of a round that starts at byte
// `off` of X and holds n4 chunks; chunks past n4 read from an out-of-range
// offset (zeros, no memory access).
__device__ __forceinline__ void xs_fetch(rsrc_t rx, uint32_t off, uint32_t n4, int tid,
                                         uint32_t nthr, uint32_t (&reg)[kStageChunks][4]) {
#pragma unroll
    for (int j = 0; j < kStageChunks; j++) {
        const uint32_t c = j * nthr + (uint32_t)tid;
        const uint32_t o = c < n4 ? off + 16u * c : 0xFFFFFFF0u;
        auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0);
        reg[j][0] = v[0]; reg[j][1] = v[1]; reg[j][2] = v[2]; reg[j][3] = v[3];
    }
}

// Every chunk is written, zeros past the round included: xs_pos permutes
// chunks inside aligned groups of 16 and the stage holds 8 * nthr chunks, a
// multiple of 16, so all writes stay inside the stage.  (Stores under a
// predicate would let the compiler sink the loads behind the weight loads.)
__device__ __forceinline__ void xs_commit(uint32_t *stage, int tid, uint32_t nthr,
                                          const uint32_t (&reg)[kStageChunks][4]) {
#pragma unroll
    for (int j = 0; j < kStageChunks; j++) {
        uint32_t *d = stage + 4 * xs_pos(j * nthr + (uint32_t)tid);
        d[0] = reg[j][0]; d[1] = reg[j][1]; d[2] = reg[j][2]; d[3] = reg[j][3];
    }
}

// Copies the runs of this lane's tile that lie in floats [f0, f0 + n) of
// the flat array X into x; tile b starts at float xbase[b] of X.
template <class F, int B>
__device__ __forceinline__ void xs_read(const uint32_t *stage, uint32_t f0, uint32_t n,
                                        const uint32_t (&xbase)[B], const typename F::Lane &L,
                                        bool active, float (&x)[B][F::CPT]) {
#pragma unroll
    for (int b = 0; b < B; b++)
#pragma unroll
        for (int r = 0; r < F::NRUN; r++) {
            const uint32_t rel = xbase[b] + (uint32_t)F::col0(L, r) - f0;
            if (active && rel < n) {
#pragma unroll
                for (int k = 0; k < F::RUNLEN / 4; k++) {
                    const uint32_t *q = stage + 4 * xs_pos(rel / 4 + k);
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        x[b][r * F::RUNLEN + 4 * k + i] = __builtin_bit_cast(float, q[i]);
                }
            }
        }
}

// Stages the xtot floats of X round by round and fills x.  The
// caller has already issued the first round's loads into xr (so that they
// can go out ahead of its other loads).  Ends with a barrier: the stage is
// free again on return.
template <class F, int B>
__device__ __forceinline__ void xs_stage(uint32_t *stage, rsrc_t rx, uint32_t xtot,
                                         const uint32_t (&xbase)[B], const typename F::Lane &L,
                                         bool active, int tid, uint32_t nthr,
                                         const uint32_t (&xr)[kStageChunks][4],
                                         float (&x)[B][F::CPT]) {
    const uint32_t xcap = 32u * nthr;
#pragma unroll
    for (int b = 0; b < B; b++)
#pragma unroll
        for (int c = 0; c < F::CPT; c++) x[b][c] = 0.f;
    xs_commit(stage, tid, nthr, xr);
    __syncthreads();
    xs_read<F, B>(stage, 0u, xtot < xcap ? xtot : xcap, xbase, L, active, x);
    // further rounds (their loads wait for everything issued before them)
    for (uint32_t f0 = xcap; f0 < xtot; f0 += xcap) {
        const uint32_t n = xtot - f0 < xcap ? xtot - f0 : xcap;
        uint32_t yr[kStageChunks][4];
        __syncthreads();
        xs_fetch(rx, 4u * f0, n / 4u, tid, nthr, yr);
        xs_commit(stage, tid, nthr, yr);
        __syncthreads();
        xs_read<F, B>(stage, f0, n, xbase, L, active, x);
    }
    __syncthreads();
}

template <class F, int B, int U, bool XL>
__global__ void __launch_bounds__(512) qgemv_lds_kernel(GemvParams p) {
    extern __shared__ __attribute__((aligned(16))) uint32_t stage[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int grp, lig;
    if (p.S == 1) {
        grp = wave * (64 / p.lpr) + lane / p.lpr;
        lig = lane & (p.lpr - 1);
    } else {
        grp = wave / p.S;
        lig = (wave % p.S) * 64 + lane;
    }
    const bool active = lig < p.tiles;
    const typename F::Lane L = F::init(active ? lig : 0);
    const int64_t rpi = (int64_t)p.G * U;
    const uint32_t nthr = blockDim.x;

    // With XL the first activation round's loads go out first, then the
    // first block's weight loads (every workgroup has a first block: the
    // grid is never larger than the number of blocks), so the activations
    // are staged while the weights are still in flight.  Without XL each
    // lane reads its tile straight from global memory.
    int64_t it = blockIdx.x;
    const uint32_t xtot = p.cols * (uint32_t)B;
    const rsrc_t rx = make_rsrc(p.X, 4u * xtot);
    const uint32_t xcap = 32u * nthr;  // floats per round: the stage's size
    uint32_t xr[kStageChunks][4];
    if constexpr (XL) xs_fetch(rx, 0u, (xtot < xcap ? xtot : xcap) / 4u, tid, nthr, xr);
    uint32_t reg[kStageChunks][4];
    StageBlock cur = stage_block(p, it, rpi);
    stage_fetch(cur, tid, nthr, reg);

    typename F::template XTile<B> xt;
    {
        float x[B][F::CPT];
        if constexpr (XL) {
            uint32_t xbase[B];
#pragma unroll
            for (int b = 0; b < B; b++) xbase[b] = (uint32_t)b * p.cols;
            xs_stage<F, B>(stage, rx, xtot, xbase, L, active, tid, nthr, xr, x);
        } else {
            load_tile_x<F, B>(rx, p.cols, L, active, x);
        }
        F::template prep<B>(x, xt);
    }
    __shared__ float red[8][U * B];

    for (; it * rpi < p.rows; it += gridDim.x) {
        stage_store(stage, tid, nthr, reg);
        __syncthreads();
        const uint32_t d16 = cur.d16;
        if ((it + gridDim.x) * rpi < p.rows) {
            cur = stage_block(p, it + gridDim.x, rpi);
            stage_fetch(cur, tid, nthr, reg);
        }

        const LdsReader rd{stage};
        const int64_t rg = it * rpi + (int64_t)grp * U;
        float acc[U * B];
#pragma unroll
        for (int u = 0; u < U; u++) {
            float a[B];
#pragma unroll
            for (int b = 0; b < B; b++) a[b] = 0.f;
            if (active && rg + u < p.rows) {
                typename F::Raw raw;
                F::load(rd, d16 + (uint32_t)(grp * U + u) * p.row_bytes, L, raw);
                F::template dot<B>(raw, L, xt, a);
            }
#pragma unroll
            for (int b = 0; b < B; b++) acc[u * B + b] = a[b];
        }
        group_sum_all(acc, p.S == 1 ? p.lpr : 64);
        if (p.S == 1) {
            if (lig == 0) {
#pragma unroll
                for (int u = 0; u < U; u++)
                    if (rg + u < p.rows)
#pragma unroll
                        for (int b = 0; b < B; b++) p.Y[b * p.rows + rg + u] = acc[u * B + b];
            }
        } else {
            if (lane == 0) {
#pragma unroll
                for (int i = 0; i < U * B; i++) red[wave][i] = acc[i];
            }
            __syncthreads();
            if (wave % p.S == 0 && lane < U * B) {
                float sum = 0.f;
                for (int w = 0; w < p.S; w++) sum += red[wave + w][lane];
                const int u = lane / B, b = lane % B;
                if (rg + u < p.rows) p.Y[b * p.rows + rg + u] = sum;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ routing

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

// Order-preserving map of a double onto an unsigned 64-bit key, returned as
// (hi, lo) halves: larger logits give larger keys, -0.0 and +0.0 share a
// key, and NaN maps to 0, below every number (-inf included).  Rank order:
// a larger key first, equal keys to the lower expert index.
__device__ __forceinline__ void order_key(double v, uint32_t *hi, uint32_t *lo) {
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    b = (v == 0.0) ? 0ull : b;
    uint64_t k = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
    k = __builtin_isnan(v) ? 0ull : k;
    *hi = (uint32_t)(k >> 32);
    *lo = (uint32_t)k;
}

__device__ __forceinline__ bool key_before(uint32_t ah, uint32_t al, int ai, uint32_t bh,
                                           uint32_t bl, int bi) {
    return (ah > bh) | ((ah == bh) & ((al > bl) | ((al == bl) & (ai < bi))));
}

// The logit of an order key (inverse of order_key; a NaN's key 0 maps back
// to a NaN, -0.0 to +0.0).
__device__ __forceinline__ double key_value(uint32_t hi, uint32_t lo) {
    const uint64_t k = ((uint64_t)hi << 32) | lo;
    const uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    return __builtin_bit_cast(double, b);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_u<CTRL>((uint32_t)b), hi = dpp_u<CTRL>((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// A double of lane `src` (uniform), read half by half (readlane returns a
// signed int: each half is widened as unsigned).
__device__ __forceinline__ double readlane_d(double v, int src) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over each aligned group of 32 lanes (fixed tree); every lane of a
// group receives its group's sum.
__device__ __forceinline__ double group_sum32_d(double v) {
    v += dpp_d<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_d<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_d<0x141>(v);  // row_half_mirror
    v += dpp_d<0x140>(v);  // row_mirror
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = swz16_u((uint32_t)b), hi = swz16_u((uint32_t)(b >> 32));
    return v + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// LDS one routing wave gathers its chosen keys in: per chosen key its high
// half, low half and expert index.
struct RouteLds {
    uint32_t e[kMaxTopK][4];
};

__device__ __forceinline__ uint64_t ballot64(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// One wave: softmax / top-k / renormalise over E <= 1024 f64 logits (the
// module doc's routing on the aprender-serve page).  Lane l holds the
// order keys of experts l, l + 64, ... (PER slots); a slot past E holds
// key 0, as a NaN does.  Selection:
//   1. the k-th largest high key half T, two bits at a time from the top:
//      of T | 3 << b, T | 2 << b and T | 1 << b the largest that at least
//      k high halves reach is kept (ballots and population counts; every
//      threshold tried is >= 1, so the zero keys of slots past E never
//      count);
//   2. keys above T are chosen; among the keys equal to T the same descent
//      on the low halves picks the rest, and among fully equal keys the
//      lowest expert indices (expert l + 64 i orders by slot, then lane);
//   3. the chosen keys are gathered in expert order into LDS; lane s < k
//      takes the s-th and counts the gathered keys that rank before it
//      (larger key, or equal key and lower index): that count is its rank.
// Weights: lane s forms exp(l_s - l_0) in f64 (l_0 the logit of rank 0),
// the sum over the k chosen keys is a fixed tree in f64 over lanes
// 0 .. k-1, and w = exp(l_s - l_0) / sum, the softmax probabilities
// renormalised over the chosen set.  The lane of rank r writes sel[r] and
// wout[r] (any memory space).
template <int PER>
__device__ __forceinline__ void route_topk_per(const double *__restrict__ logits, int E, int k,
                                               int *sel, float *wout, RouteLds *lds) {
    const int lane = __lane_id();
    uint32_t kh[PER], kl[PER];
    bool valid[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int e = lane + 64 * i;
        valid[i] = e < E;
        order_key(logits[valid[i] ? e : 0], &kh[i], &kl[i]);
        kh[i] = valid[i] ? kh[i] : 0u;
        kl[i] = valid[i] ? kl[i] : 0u;
    }
    // 1. k-th largest high half.  T only grows and at least k high halves
    // reach it; once exactly k do, those k are the chosen set and the
    // remaining bits cannot change it, so the descent stops there.
    uint32_t T = 0;
#pragma unroll 1
    for (int b = 30; b >= 0; b -= 2) {
        const uint32_t c1 = T | (1u << b), c2 = T | (2u << b), c3 = T | (3u << b);
        int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            n1 += __popcll(ballot64(kh[i] >= c1));
            n2 += __popcll(ballot64(kh[i] >= c2));
            n3 += __popcll(ballot64(kh[i] >= c3));
        }
        T = n3 >= k ? c3 : (n2 >= k ? c2 : (n1 >= k ? c1 : T));
        if ((n3 == k) | ((n3 < k) & (n2 == k)) | ((n2 < k) & (n1 == k))) break;
    }
    // 2. the chosen set, as one ballot mask per slot
    uint64_t msel[PER];
    int ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const uint64_t gt = ballot64(kh[i] > T);
        const uint64_t eq = ballot64(valid[i] && kh[i] == T);
        ngt += __popcll(gt);
        neq += __popcll(eq);
        msel[i] = gt | eq;
    }
    const int need = k - ngt;
    if (neq > need) {
        // several keys share the high half T: descend on the low halves of
        // those keys (the others take low half 0, below every threshold)
        uint32_t lt[PER];
#pragma unroll
        for (int i = 0; i < PER; i++) lt[i] = (valid[i] && kh[i] == T) ? kl[i] : 0u;
        uint32_t TL = 0;
#pragma unroll 1
        for (int b = 30; b >= 0; b -= 2) {
            const uint32_t c1 = TL | (1u << b), c2 = TL | (2u << b), c3 = TL | (3u << b);
            int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
            for (int i = 0; i < PER; i++) {
                n1 += __popcll(ballot64(lt[i] >= c1));
                n2 += __popcll(ballot64(lt[i] >= c2));
                n3 += __popcll(ballot64(lt[i] >= c3));
            }
            TL = n3 >= need ? c3 : (n2 >= need ? c2 : (n1 >= need ? c1 : TL));
        }
        uint64_t g2[PER], e2[PER];
        int n2 = 0;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const bool eqT = valid[i] && kh[i] == T;
            g2[i] = ballot64(eqT && kl[i] > TL);
            e2[i] = ballot64(eqT && kl[i] == TL);
            n2 += __popcll(g2[i]);
        }
        int rest = need - n2;  // fully equal keys still to take, lowest index first
#pragma unroll
        for (int i = 0; i < PER; i++) {
            uint64_t m = e2[i], keep = 0;
            while (rest > 0 && m) {
                const uint64_t low = m & (~m + 1);
                keep |= low;
                m &= m - 1;
                rest--;
            }
            msel[i] = ballot64(kh[i] > T) | g2[i] | keep;
        }
    }
    // 3. gather the chosen keys in expert order, then rank them
    int base = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int pos = base + lanes_below(msel[i]);
        if (((msel[i] >> lane) & 1ull) && pos < kMaxTopK) {
            lds->e[pos][0] = kh[i];
            lds->e[pos][1] = kl[i];
            lds->e[pos][2] = (uint32_t)(lane + 64 * i);
        }
        base += __popcll(msel[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool mine = lane < k;
    const int s = mine ? lane : 0;
    const uint32_t oh = lds->e[s][0], ol = lds->e[s][1];
    const int oi = (int)lds->e[s][2];
    // eight gathered keys per round, all read before any is compared
    // (entries past k are read but not counted)
    int rank = 0;
#pragma unroll 1
    for (int j0 = 0; j0 < k; j0 += 8) {
        uint32_t v[8][3];
#pragma unroll
        for (int u = 0; u < 8; u++)
#pragma unroll
            for (int q = 0; q < 3; q++) v[u][q] = lds->e[j0 + u][q];
#pragma unroll
        for (int u = 0; u < 8; u++)
            rank += (j0 + u < k && key_before(v[u][0], v[u][1], (int)v[u][2], oh, ol, oi)) ? 1 : 0;
    }
    // weights
    const uint64_t m0 = ballot64(mine && rank == 0);
    const int j0 = m0 ? (int)__builtin_ctzll(m0) : 0;
    const uint32_t h0 = (uint32_t)__builtin_amdgcn_readlane((int)oh, j0);
    const uint32_t lo0 = (uint32_t)__builtin_amdgcn_readlane((int)ol, j0);
    const double ex = mine ? exp(key_value(oh, ol) - key_value(h0, lo0)) : 0.0;
    const double den = readlane_d(group_sum32_d(ex), 0);  // k <= 32: lanes 0 .. 31
    if (mine) {
        sel[rank] = oi;
        wout[rank] = (float)(ex / den);
    }
}

// Each lane holds ceil(E/64) keys, rounded up to a power of two, so the k
// selection rounds scan only as many slots as the expert count needs.
// `lds` is this wave's own gathering area.
__device__ __forceinline__ void route_topk_wave(const double *__restrict__ logits, int E, int k,
                                                int *sel, float *wout, RouteLds *lds) {
    static_assert(kMaxExperts == 64 * 16, "slot dispatch covers up to 16 keys per lane");
    if (E <= 64)
        route_topk_per<1>(logits, E, k, sel, wout, lds);
    else if (E <= 128)
        route_topk_per<2>(logits, E, k, sel, wout, lds);
    else if (E <= 256)
        route_topk_per<4>(logits, E, k, sel, wout, lds);
    else if (E <= 512)
        route_topk_per<8>(logits, E, k, sel, wout, lds);
    else
        route_topk_per<16>(logits, E, k, sel, wout, lds);
}




struct MoeParams {
    const float *x;
    const float *residual;
    const float *residual2;  // optional: the residual is residual + residual2 (f32)
    float *y;
    const uint8_t *gate;
    const uint8_t *up;
    const uint8_t *down;
    uint64_t gate_bytes, up_bytes, down_bytes;  // whole stacks
    uint32_t rb_gate;   // row bytes of a gate / up row (H columns)
    uint32_t rb_down;   // row bytes of a down row (F columns)
    int32_t H, E, K, F;
    const double *logits;  // workspace
    int32_t *ws_sel;       // workspace
    float *ws_w;           // workspace
    float *act;            // workspace [K][F]
    int32_t *sel_out;      // optional
    float *w_out;          // optional
    // gate/up kernel geometry
    int32_t gu_tiles, gu_lpr, gu_S, gu_G;
    // down kernel geometry
    int32_t dn_tiles_per_slot, dn_tiles, dn_lpr, dn_S, dn_G;
    // tokens (moe_ffn_tokens): x, residual, y are [T][H], the routes and
    // activations [T][K] and [T][K][F]; the down kernel takes its token
    // from blockIdx.y
    int32_t T;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// ------------------------------------------------------------------ MoE K2

template <class F, int U>
__global__ void __launch_bounds__(512) moe_gateup_kernel(MoeParams p) {
    __shared__ int s_sel[kMaxTopK];
    __shared__ RouteLds s_rt[1];
    __shared__ float s_w[kMaxTopK];
    __shared__ float red[8][2 * U];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int grp, lig;
    if (p.gu_S == 1) {
        grp = wave * (64 / p.gu_lpr) + lane / p.gu_lpr;
        lig = lane & (p.gu_lpr - 1);
    } else {
        grp = wave / p.gu_S;
        lig = (wave % p.gu_S) * 64 + lane;
    }
    const bool active = lig < p.gu_tiles;
    const typename F::Lane L = F::init(active ? lig : 0);
    // x is staged through LDS (coalesced loads) while wave 0 routes; the
    // staging's closing barrier also publishes s_sel and s_w
    extern __shared__ __attribute__((aligned(16))) uint32_t xst[];
    const uint32_t nthr = blockDim.x, xcap = 32u * nthr, H = (uint32_t)p.H;
    const rsrc_t rx = make_rsrc(p.x, 4u * H);
    uint32_t xr[kStageChunks][4];
    xs_fetch(rx, 0u, (H < xcap ? H : xcap) / 4u, tid, nthr, xr);
    if (wave == 0) route_topk_wave(p.logits, p.E, p.K, s_sel, s_w, &s_rt[0]);
    typename F::template XTile<1> xt;
    {
        const uint32_t xbase[1] = {0u};
        float x[1][F::CPT];
        xs_stage<F, 1>(xst, rx, H, xbase, L, active, tid, nthr, xr, x);
        F::template prep<1>(x, xt);
    }
    if (blockIdx.x == 0 && tid < p.K) {
        p.ws_sel[tid] = s_sel[tid];
        p.ws_w[tid] = s_w[tid];
        if (p.sel_out) p.sel_out[tid] = s_sel[tid];
        if (p.w_out) p.w_out[tid] = s_w[tid];
    }

    uint32_t dg, du;
    const rsrc_t rg = rows_rsrc(p.gate, p.gate_bytes, 0, &dg);
    const rsrc_t ru = rows_rsrc(p.up, p.up_bytes, 0, &du);
    const int64_t tasks = (int64_t)p.K * p.F;
    const int64_t tpi = (int64_t)p.gu_G * U;
    for (int64_t it = blockIdx.x; it * tpi < tasks; it += gridDim.x) {
        const int64_t t0 = it * tpi + (int64_t)grp * U;
        typename F::Raw rawg[U], rawu[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t t = t0 + u;
            const bool want = active && t < tasks;
            const int s = want ? (int)(t / p.F) : 0, j = want ? (int)(t % p.F) : 0;
            const uint32_t off = ((uint32_t)s_sel[s] * (uint32_t)p.F + (uint32_t)j) * p.rb_gate;
            F::load(BufReader{rg}, want ? dg + off : kOorRow, L, rawg[u]);
            F::load(BufReader{ru}, want ? du + off : kOorRow, L, rawu[u]);
        }
        float ag[U][1], au[U][1];
#pragma unroll
        for (int u = 0; u < U; u++) {
            ag[u][0] = au[u][0] = 0.f;
            if (active && t0 + u < tasks) {
                F::template dot<1>(rawg[u], L, xt, ag[u]);
                F::template dot<1>(rawu[u], L, xt, au[u]);
            }
        }
        {
            float v[2 * U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                v[2 * u] = ag[u][0];
                v[2 * u + 1] = au[u][0];
            }
            group_sum_all(v, p.gu_S == 1 ? p.gu_lpr : 64);
#pragma unroll
            for (int u = 0; u < U; u++) {
                ag[u][0] = v[2 * u];
                au[u][0] = v[2 * u + 1];
            }
        }
        if (p.gu_S == 1) {
            if (lig == 0) {
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const int64_t t = t0 + u;
                    if (t < tasks) {
                        const int s = (int)(t / p.F);
                        p.act[t] = s_w[s] * silu_f(ag[u][0]) * au[u][0];
                    }
                }
            }
        } else {
            if (lane == 0) {
#pragma unroll
                for (int u = 0; u < U; u++) {
                    red[wave][2 * u] = ag[u][0];
                    red[wave][2 * u + 1] = au[u][0];
                }
            }
            __syncthreads();
            if (wave % p.gu_S == 0 && lane < U) {
                float g = 0.f, v = 0.f;
                for (int w = 0; w < p.gu_S; w++) {
                    g += red[wave + w][2 * lane];
                    v += red[wave + w][2 * lane + 1];
                }
                const int64_t t = t0 + lane;
                if (t < tasks) {
                    const int s = (int)(t / p.F);
                    p.act[t] = s_w[s] * silu_f(g) * v;
                }
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------- MoE, several tokens
//
// moe_ffn_tokens: T <= 8 decode tokens, each routed on its own (the
// aprender-serve page's moe_layer per token), with the expert GEMVs grouped
// by expert so that every selected expert's gate and up rows are read once
// for all the tokens of a group that chose it (the batch semantics of the
// weight_matrix.rs page's apply_batch, applied per expert).  The host runs
// the gate/up kernel once per group of up to four tokens.


// The distinct experts among the T*K routes, in route order (token-major,
// then rank), and for each the slot every token holds it in (-1: none).
// One wave; lane i holds route i (T*K <= 64).  s_first is LDS scratch of E
// words: the lowest route index of each expert, found with one LDS minimum
// per route (the LDS operations of one wave take effect in program order).
constexpr int kMaxTokens = 8;
constexpr int kMaxRoutes = 64;

__device__ __forceinline__ int distinct_experts(const int *s_sel, int nroutes, int K, int E,
                                                int *s_first, int *s_uexp,
                                                int (*s_uslot)[kMaxTokens]) {
    const int lane = __lane_id();
    for (int i = lane; i < E; i += 64) s_first[i] = 64;
    const int e = lane < nroutes ? s_sel[lane] : -1;
    if (e >= 0) atomicMin(&s_first[e], lane);
    const int first = e >= 0 ? s_first[e] : lane;  // lowest route index holding e
    const bool lead = lane < nroutes && first == lane;
    const unsigned long long m = __ballot(lead);
    const int u_lead = __popcll(m & ((1ull << lane) - 1ull));
    const int u = __shfl(u_lead, first);
    if (lead) s_uexp[u] = e;
    if (lane < nroutes) s_uslot[u][lane / K] = lane % K;
    return __popcll(m);
}

// ------------------------------------------------------------------ MoE K3

template <class F, int U>
__global__ void __launch_bounds__(512) moe_down_kernel(MoeParams p) {
    __shared__ float red[8][U];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int grp, lig;
    if (p.dn_S == 1) {
        grp = wave * (64 / p.dn_lpr) + lane / p.dn_lpr;
        lig = lane & (p.dn_lpr - 1);
    } else {
        grp = wave / p.dn_S;
        lig = (wave % p.dn_S) * 64 + lane;
    }
    const bool active = lig < p.dn_tiles;
    const int slot = active ? lig / p.dn_tiles_per_slot : 0;
    const int tile = active ? lig % p.dn_tiles_per_slot : 0;
    const typename F::Lane L = F::init(tile);
    // this workgroup's token: its activations, routes, residual and output
    const int64_t tok = blockIdx.y;
    p.act += tok * p.K * p.F;
    p.ws_sel += tok * p.K;
    p.y += tok * p.H;
    p.residual += tok * p.H;
    if (p.residual2) p.residual2 += tok * p.H;
    // the activations of all K slots, staged through LDS (coalesced loads)
    extern __shared__ __attribute__((aligned(16))) uint32_t xst[];
    const uint32_t nthr = blockDim.x, xcap = 32u * nthr;
    const uint32_t xtot = (uint32_t)p.K * (uint32_t)p.F;
    const rsrc_t ra = make_rsrc(p.act, 4u * xtot);
    uint32_t xr[kStageChunks][4];
    xs_fetch(ra, 0u, (xtot < xcap ? xtot : xcap) / 4u, tid, nthr, xr);
    const uint32_t expert_off =
        active ? (uint32_t)p.ws_sel[slot] * (uint32_t)p.H * p.rb_down : 0u;
    uint32_t dd;
    const rsrc_t rd = rows_rsrc(p.down, p.down_bytes, 0, &dd);
    const int64_t rpi = (int64_t)p.dn_G * U;
    // the first rows' weight loads go out as soon as the routes are in,
    // ahead of the activation staging; each later round's loads are issued
    // at the end of the round before
    typename F::Raw raw[U];
    auto issue = [&](int64_t it) {
        const int64_t r0 = it * rpi + (int64_t)grp * U;
#pragma unroll
        for (int u = 0; u < U; u++)
            F::load(BufReader{rd},
                    active && r0 + u < p.H ? dd + expert_off + (uint32_t)(r0 + u) * p.rb_down
                                           : kOorRow,
                    L, raw[u]);
    };
    // the residual rows each writing lane adds, loaded with the weights:
    // U rows r0 + u for a row group's lane 0 (one-wave rows), row r0 + lane
    // for lanes below U of a group's first wave (rows over several waves);
    // rows past H read as zero.  With the norm step's residual add fused
    // here the residual is residual + residual2, added in f32.
    const uint32_t hb = 4u * (uint32_t)p.H;
    const rsrc_t rres = make_rsrc(p.residual, hb);
    const rsrc_t rres2 = make_rsrc(p.residual2 ? p.residual2 : p.residual, hb);
    auto fetch_res = [&](int64_t it, float (&rv)[U]) {
        const int64_t r0 = it * rpi + (int64_t)grp * U;
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t r = p.dn_S == 1 ? r0 + u : r0 + lane;
            const uint32_t off = r < p.H ? 4u * (uint32_t)r : 0xFFFFFFF0u;
            const float a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rres, off, 0, 0));
            const float b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rres2, off, 0, 0));
            rv[u] = p.residual2 ? a + b : a;
        }
    };
    float resv[U];
    if ((int64_t)blockIdx.x * rpi < p.H) {
        issue(blockIdx.x);
        fetch_res(blockIdx.x, resv);
    }
    typename F::template XTile<1> xt;
    {
        const uint32_t xbase[1] = {(uint32_t)slot * (uint32_t)p.F};
        float x[1][F::CPT];
        xs_stage<F, 1>(xst, ra, xtot, xbase, L, active, tid, nthr, xr, x);
        F::template prep<1>(x, xt);
    }
    for (int64_t it = blockIdx.x; it * rpi < p.H; it += gridDim.x) {
        const int64_t r0 = it * rpi + (int64_t)grp * U;
        float acc[U][1];
#pragma unroll
        for (int u = 0; u < U; u++) {
            acc[u][0] = 0.f;
            if (active && r0 + u < p.H) F::template dot<1>(raw[u], L, xt, acc[u]);
        }
        float resn[U];
        if ((it + gridDim.x) * rpi < p.H) {
            issue(it + gridDim.x);
            fetch_res(it + gridDim.x, resn);
        }
        {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; u++) v[u] = acc[u][0];
            group_sum_all(v, p.dn_S == 1 ? p.dn_lpr : 64);
#pragma unroll
            for (int u = 0; u < U; u++) acc[u][0] = v[u];
        }
        if (p.dn_S == 1) {
            if (lig == 0) {
#pragma unroll
                for (int u = 0; u < U; u++)
                    if (r0 + u < p.H) p.y[r0 + u] = resv[u] + acc[u][0];
            }
        } else {
            if (lane == 0) {
#pragma unroll
                for (int u = 0; u < U; u++) red[wave][u] = acc[u][0];
            }
            __syncthreads();
            if (wave % p.dn_S == 0 && lane < U) {
                float s = 0.f;
                for (int w = 0; w < p.dn_S; w++) s += red[wave + w][lane];
                const int64_t r = r0 + lane;
                if (r < p.H) p.y[r] = resv[0] + s;
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < U; u++) resv[u] = resn[u];
    }
}

}  // namespace qg
