// qg_q6mx.hpp -- the batch-1 Q6_K GEMV with its integer products on the
// matrix cores (v_mfma_i32_16x16x64_i8).
//
// Q6_K layout (web page: docs.rs, crate ferrox-cuda 0.14.0, src/gpu.rs,
// Q6_K_MATVEC_KERNEL_SRC): a 210-byte block holds 256 codes as ql[128]
// (low four bits), qh[64] (top two bits), sc[16] (signed sub-block scales)
// and d (f16).  Code i of half h (i = 128h + 32g + l, group g < 4, l < 32)
// is q = (ql[64h + l + 32(g & 1)] >> 4(g >> 1) & 15) | (qh[32h + l] >> 2g
// & 3) << 4, its weight d * sc[8h + 2g + l / 16] * (q - 32).
//
// The activations are the digit planes of the batch-1 VALU kernel: each
// run of 16 columns (one group g of one 16-wide l range) is scaled by a
// power of two 2^s so that its largest |x| 2^s lies in [2^21, 2^22), and
// X = rint(x 2^s) = 65536 p2 + 256 p1 + p0 with signed bytes p0, p1, p2.
// A code meets every plane in int32 exactly; the plane sums are combined
// once in f32 and scaled by d * sc * 2^-s (the same arithmetic, and the
// same error bound, as that kernel).
//
// Matrix-core mapping.  A tile is 64 columns of a row: super-block sb,
// half h, l0 in {0, 16}, i.e. the four groups' 16 codes at l0 .. l0 + 15.
// One MFMA takes 16 weight rows x one tile (K = 64):
//   B (codes): lane (n, kg) = (lane % 16, lane / 16) holds the signed code
//     bytes 4(q - 32) of weight row n at l = l0 + 4kg .. l0 + 4kg + 3, dword
//     g for group g (the same assembly as the VALU kernel's);
//   A (activations): lane (m, kg) holds, for m = 4r + p with p < 3, digit
//     plane p of the same four columns of group r in dword r and zeros in
//     the other dwords (m = 4r + 3 is all zero);
//   D: lane (n, j) = (lane % 16, lane / 16) receives in register p the sum
//     over group j's 16 codes of row n against plane p
// (D[m][n] = sum over lane groups and bytes of A(16 g + m) B(16 g + n),
// checked on the device).  Lane (n, j) then applies row n's scales for
// group j, which it has loaded itself (kg = j).
//
// Work layout.  A workgroup has W = tiles / TPW waves; wave w owns tiles
// w TPW .. w TPW + TPW - 1 of every row, so its A operands (TPW x 4 VGPRs)
// and run scales are built once.  Blocks of 16 rows are staged through LDS
// as in qgemv_lds_kernel (16-byte coalesced loads, the next block's loads
// in flight while the current one is computed); each wave accumulates its
// tiles' contributions per lane, the four groups are added across lanes,
// the W waves' partial sums in LDS in wave order.
#pragma once

#include "qg_kernels.hpp"

namespace qg {
namespace q6mx {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kRows = 16;  // weight rows per block (the instruction's N)

// Digit planes of four consecutive activations whose run maximum (as the
// bit pattern of |x|) is mb: p[k] holds digit k of the four values (value
// i in byte i); f = 2^-s, or NaN for a non-finite run.
__device__ __forceinline__ void digits4(const float (&x)[4], uint32_t mb, uint32_t (&pl)[3],
                                        float *f) {
    int s = 22 - __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, mb));
    s = s > 126 ? 126 : s;
    const float up = __builtin_bit_cast(float, (uint32_t)(s + 127) << 23);
    *f = mb < 0x7F800000u ? __builtin_bit_cast(float, (uint32_t)(127 - s) << 23)
                          : __builtin_nanf("");
    // y = X + 0x8080: bytes 0 and 1 of y are p0 + 128 and p1 + 128, byte 2
    // (sign-extended) is p2
    uint32_t y[4];
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = (uint32_t)((int)__builtin_rintf(x[i] * up) + 32896);
    const uint32_t a = __builtin_amdgcn_perm(y[1], y[0], 0x05040100u);
    const uint32_t b = __builtin_amdgcn_perm(y[3], y[2], 0x05040100u);
    pl[0] = __builtin_amdgcn_perm(b, a, 0x06040200u) ^ 0x80808080u;
    pl[1] = __builtin_amdgcn_perm(b, a, 0x07050301u) ^ 0x80808080u;
    const uint32_t c = __builtin_amdgcn_perm(y[1], y[0], 0x0C0C0602u);
    const uint32_t e = __builtin_amdgcn_perm(y[3], y[2], 0x0C0C0602u);
    pl[2] = __builtin_amdgcn_perm(e, c, 0x05040100u);
}

// A lane's fields of one tile of its row (staged in LDS): the two ql
// dwords and the qh dword as two aligned dwords each with their realigning
// selector, and d * sc / 4 of the lane's group (the codes carry a factor 4).
struct Fields {
    uint32_t a0, a1, b0, b1, h0, h1, sel;
    float ds;
};

// Tile i of wave `wave` (super-block wave * TPW / 4 + i / 4, half (i / 2) %
// 2, l0 = 16 (i % 2)) of the row staged at byte `rowoff`; the lane's code
// bytes start 4kg bytes into each field.  Staged bytes keep their offset
// mod 4, so a field at 2 mod 4 is realigned from two dwords.
template <int TPW>
__device__ __forceinline__ void fetch(const uint32_t *stage, uint32_t rowoff, int wave, int kg,
                                      int i, Fields &f) {
    const int sb = wave * (TPW / 4) + (i >> 2), h = (i >> 1) & 1, l0 = (i & 1) * 16;
    const uint32_t blk = rowoff + 210u * (uint32_t)sb;
    const uint32_t qoff = blk + 4u * (uint32_t)kg;
    const uint32_t *q = stage + (qoff >> 2);
    const int fa = (64 * h + l0) / 4;         // ql, groups 0 and 2
    const int fb = fa + 8;                    // ql, groups 1 and 3
    const int fh = (128 + 32 * h + l0) / 4;   // qh
    f.a0 = q[fa];
    f.a1 = q[fa + 1];
    f.b0 = q[fb];
    f.b1 = q[fb + 1];
    f.h0 = q[fh];
    f.h1 = q[fh + 1];
    f.sel = (qoff & 2u) ? 0x05040302u : 0x03020100u;
    // d and the sub-block scale sc[8h + 2kg + l0 / 16] of row n, group kg
    const int8_t *st8 = reinterpret_cast<const int8_t *>(stage);
    const float sc = (float)st8[blk + 2u * (uint32_t)kg + (uint32_t)(192 + 8 * h + l0 / 16)];
    const float d = (float)*reinterpret_cast<const _Float16 *>(st8 + blk + 208u);
    f.ds = d * 0.25f * sc;
}

// The codes 4(q - 32) of the lane's four groups as signed bytes: low four
// bits to bits 2..5, the two top bits to bits 6..7 with the upper one
// flipped.
__device__ __forceinline__ v4i codes(const Fields &f) {
    const uint32_t qa = __builtin_amdgcn_perm(f.a1, f.a0, f.sel);
    const uint32_t qb = __builtin_amdgcn_perm(f.b1, f.b0, f.sel);
    const uint32_t hx = __builtin_amdgcn_perm(f.h1, f.h0, f.sel) ^ 0xAAAAAAAAu;
    v4i B;
    B[0] = (int)(((qa << 2) & 0x3C3C3C3Cu) | ((hx << 6) & 0xC0C0C0C0u));
    B[1] = (int)(((qb << 2) & 0x3C3C3C3Cu) | ((hx << 4) & 0xC0C0C0C0u));
    B[2] = (int)(((qa >> 2) & 0x3C3C3C3Cu) | ((hx << 2) & 0xC0C0C0C0u));
    B[3] = (int)(((qb >> 2) & 0x3C3C3C3Cu) | (hx & 0xC0C0C0C0u));
    return B;
}

// NB batch rows (2): the rows of X lie one after another (cols floats each)
// and are staged together; every tile's codes are assembled once and
// meet each row's digit planes in an instruction of its own.
template <int TPW, int NB>
__device__ __forceinline__ void q6k_mx_body(const GemvParams &p) {
    extern __shared__ __attribute__((aligned(16))) uint32_t stage[];
    __shared__ float red[NB][8][kRows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = (int)(blockDim.x >> 6);
    const int n = lane & 15, kg = lane >> 4;  // B and D roles: row n, l quad / group kg
    const int ar = n >> 2, ap = n & 3;        // A role: group ar, plane ap (3: none)
    const uint32_t nthr = blockDim.x;

    // the activations' loads, then the first block's weight loads
    const uint32_t xtot = p.cols * (uint32_t)NB;
    const rsrc_t rx = make_rsrc(p.X, 4u * xtot);
    uint32_t xr[kStageChunks][4];
    xs_fetch(rx, 0u, xtot / 4u, tid, nthr, xr);
    int64_t it = blockIdx.x;
    uint32_t reg[kStageChunks][4];
    StageBlock cur = stage_block(p, it, kRows);
    stage_fetch(cur, tid, nthr, reg);

    // A operands and run scales of this wave's tiles
    xs_commit(stage, tid, nthr, xr);
    __syncthreads();
    v4i A[NB][TPW];
    float fr[NB][TPW];  // 2^-s of run (tile, group kg) of batch row b
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
    for (int i = 0; i < TPW; i++) {
        const int t = wave * TPW + i;
        const int sb = t >> 2, h = (t >> 1) & 1, l0 = (t & 1) * 16;
        const uint32_t c = (uint32_t)b * p.cols +
                           (uint32_t)(256 * sb + 128 * h + 32 * ar + l0 + 4 * kg);
        const uint32_t *q4 = stage + 4 * xs_pos(c / 4u);
        float x[4];
        uint32_t mb = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            x[j] = __builtin_bit_cast(float, q4[j]);
            const uint32_t a = q4[j] & 0x7FFFFFFFu;
            mb = a > mb ? a : mb;
        }
        // the run's 16 columns lie in lanes n, n + 16, n + 32, n + 48
        uint32_t o = (uint32_t)__shfl_xor((int)mb, 16);
        mb = o > mb ? o : mb;
        o = (uint32_t)__shfl_xor((int)mb, 32);
        mb = o > mb ? o : mb;
        uint32_t pl[3];
        float f;
        digits4(x, mb, pl, &f);
        const uint32_t mine = ap == 0 ? pl[0] : ap == 1 ? pl[1] : ap == 2 ? pl[2] : 0u;
        A[b][i][0] = (int)(ar == 0 ? mine : 0u);
        A[b][i][1] = (int)(ar == 1 ? mine : 0u);
        A[b][i][2] = (int)(ar == 2 ? mine : 0u);
        A[b][i][3] = (int)(ar == 3 ? mine : 0u);
        // the scale of run (t, kg) is held by lane 4 kg (group kg, plane 0)
        fr[b][i] = __shfl(f, 4 * kg);
    }
    __syncthreads();

    const v4i zero = {0, 0, 0, 0};
    for (; it * kRows < p.rows; it += gridDim.x) {
        // every wave has finished reading the previous block (the barrier
        // after its red writes), so the stage can be overwritten
        stage_store(stage, tid, nthr, reg);
        __syncthreads();
        const uint32_t d16 = cur.d16;
        if ((it + gridDim.x) * kRows < p.rows) {
            cur = stage_block(p, it + gridDim.x, kRows);
            stage_fetch(cur, tid, nthr, reg);
        }
        const uint32_t rowoff = d16 + (uint32_t)n * p.row_bytes;
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; b++) acc[b] = 0.f;
        // tile i's fields, read one tile ahead of its instruction; a
        // tile's scaling waits for the next tile's instruction to issue
        Fields fd[TPW];
        fetch<TPW>(stage, rowoff, wave, kg, 0, fd[0]);
        v4i Dp[NB];
#pragma unroll
        for (int b = 0; b < NB; b++) Dp[b] = zero;
#pragma unroll
        for (int i = 0; i < TPW; i++) {
            if (i + 1 < TPW) fetch<TPW>(stage, rowoff, wave, kg, i + 1, fd[i + 1]);
            const v4i Bc = codes(fd[i]);
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[b][i], Bc, zero, 0, 0, 0);
                if (i > 0)
                    acc[b] = fmaf(fd[i - 1].ds * fr[b][i - 1],
                                  digits_sum(Dp[b][0], Dp[b][1], Dp[b][2]), acc[b]);
                Dp[b] = D;
            }
        }
        // the four groups of row n (lanes n, n + 16, n + 32, n + 48), then
        // the waves in order
#pragma unroll
        for (int b = 0; b < NB; b++) {
            acc[b] = fmaf(fd[TPW - 1].ds * fr[b][TPW - 1],
                          digits_sum(Dp[b][0], Dp[b][1], Dp[b][2]), acc[b]);
            acc[b] += __shfl_xor(acc[b], 16);
            acc[b] += __shfl_xor(acc[b], 32);
            if (lane < kRows) red[b][wave][lane] = acc[b];
        }
        __syncthreads();
        // red is rewritten only after the next block's first barrier, which
        // these threads reach after reading it
        const int64_t r0 = it * kRows;
        if (tid < NB * kRows) {
            const int b = tid / kRows, rr = tid % kRows;
            if (r0 + rr < p.rows) {
                float s = red[b][0][rr];
                for (int w = 1; w < nw; w++) s += red[b][w][rr];
                p.Y[(int64_t)b * p.rows + r0 + rr] = s;
            }
        }
    }
}

// One batch row: the same steps written out for a single row (compiled
// through the two-row body it took 0.5 us longer on the lm_head).
template <int TPW>
__global__ void __launch_bounds__(512) q6k_mx1_kernel(GemvParams p) {
    extern __shared__ __attribute__((aligned(16))) uint32_t stage[];
    __shared__ float red[8][kRows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = (int)(blockDim.x >> 6);
    const int n = lane & 15, kg = lane >> 4;  // B and D roles: row n, l quad / group kg
    const int ar = n >> 2, ap = n & 3;        // A role: group ar, plane ap (3: none)
    const uint32_t nthr = blockDim.x;

    // the activations' loads, then the first block's weight loads
    const uint32_t xtot = p.cols;
    const rsrc_t rx = make_rsrc(p.X, 4u * xtot);
    uint32_t xr[kStageChunks][4];
    xs_fetch(rx, 0u, xtot / 4u, tid, nthr, xr);
    int64_t it = blockIdx.x;
    uint32_t reg[kStageChunks][4];
    StageBlock cur = stage_block(p, it, kRows);
    stage_fetch(cur, tid, nthr, reg);

    // A operands and run scales of this wave's tiles
    xs_commit(stage, tid, nthr, xr);
    __syncthreads();
    v4i A[TPW];
    float fr[TPW];  // 2^-s of run (tile, group kg)
#pragma unroll
    for (int i = 0; i < TPW; i++) {
        const int t = wave * TPW + i;
        const int sb = t >> 2, h = (t >> 1) & 1, l0 = (t & 1) * 16;
        const uint32_t c = (uint32_t)(256 * sb + 128 * h + 32 * ar + l0 + 4 * kg);
        const uint32_t *q4 = stage + 4 * xs_pos(c / 4u);
        float x[4];
        uint32_t mb = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            x[j] = __builtin_bit_cast(float, q4[j]);
            const uint32_t a = q4[j] & 0x7FFFFFFFu;
            mb = a > mb ? a : mb;
        }
        // the run's 16 columns lie in lanes n, n + 16, n + 32, n + 48
        uint32_t o = (uint32_t)__shfl_xor((int)mb, 16);
        mb = o > mb ? o : mb;
        o = (uint32_t)__shfl_xor((int)mb, 32);
        mb = o > mb ? o : mb;
        uint32_t pl[3];
        float f;
        digits4(x, mb, pl, &f);
        const uint32_t mine = ap == 0 ? pl[0] : ap == 1 ? pl[1] : ap == 2 ? pl[2] : 0u;
        A[i][0] = (int)(ar == 0 ? mine : 0u);
        A[i][1] = (int)(ar == 1 ? mine : 0u);
        A[i][2] = (int)(ar == 2 ? mine : 0u);
        A[i][3] = (int)(ar == 3 ? mine : 0u);
        // the scale of run (t, kg) is held by lane 4 kg (group kg, plane 0)
        fr[i] = __shfl(f, 4 * kg);
    }
    __syncthreads();

    const v4i zero = {0, 0, 0, 0};
    for (; it * kRows < p.rows; it += gridDim.x) {
        // every wave has finished reading the previous block (the barrier
        // after its red writes), so the stage can be overwritten
        stage_store(stage, tid, nthr, reg);
        __syncthreads();
        const uint32_t d16 = cur.d16;
        if ((it + gridDim.x) * kRows < p.rows) {
            cur = stage_block(p, it + gridDim.x, kRows);
            stage_fetch(cur, tid, nthr, reg);
        }
        const uint32_t rowoff = d16 + (uint32_t)n * p.row_bytes;
        float acc = 0.f;
        // tile i's fields, read one tile ahead of its instruction; a
        // tile's scaling waits for the next tile's instruction to issue
        Fields fd[TPW];
        fetch<TPW>(stage, rowoff, wave, kg, 0, fd[0]);
        v4i Dp = zero;
#pragma unroll
        for (int i = 0; i < TPW; i++) {
            if (i + 1 < TPW) fetch<TPW>(stage, rowoff, wave, kg, i + 1, fd[i + 1]);
            const v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[i], codes(fd[i]), zero, 0, 0, 0);
            if (i > 0) acc = fmaf(fd[i - 1].ds * fr[i - 1], digits_sum(Dp[0], Dp[1], Dp[2]), acc);
            Dp = D;
        }
        acc = fmaf(fd[TPW - 1].ds * fr[TPW - 1], digits_sum(Dp[0], Dp[1], Dp[2]), acc);
        // the four groups of row n (lanes n, n + 16, n + 32, n + 48), then
        // the waves in order
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        if (lane < kRows) red[wave][lane] = acc;
        __syncthreads();
        // red is rewritten only after the next block's first barrier, which
        // these threads reach after reading it
        const int64_t r0 = it * kRows;
        if (tid < kRows && r0 + tid < p.rows) {
            float s = red[0][tid];
            for (int w = 1; w < nw; w++) s += red[w][tid];
            p.Y[r0 + tid] = s;
        }
    }
}

// Two batch rows: the weights are read once for both.
template <int TPW>
__global__ void __launch_bounds__(512) q6k_mx2_kernel(GemvParams p) {
    q6k_mx_body<TPW, 2>(p);
}

}  // namespace q6mx
}  // namespace qg
