// qg_gemm.hpp -- the batched dequantise-and-dot product (batch 2..32 per
// launch) on the gfx950 matrix cores: v_mfma_f32_16x16x32_bf16 with the
// activations as the A operand (M = 16 batch rows) and the weight codes as
// the B operand (N = 16 weight rows), K = 32 columns per instruction.
//
// Operand layout (checked on the device): lane l holds A[l % 16][8 (l / 16)
// + j] and B[8 (l / 16) + j][l % 16] for j < 8, and D[4 (l / 16) + i][l % 16]
// for i < 4.  So lane (r = l % 16, q = l / 16) supplies the activations of
// batch row r and the codes of weight row r, both for columns 8q .. 8q + 7
// of the 32-column block, and receives the sums of weight row r for batch
// rows 4q .. 4q + 3: the row's scales are decoded by the lane that uses
// them, with no cross-lane traffic.
//
// Numbers.  Codes are small integers, exact in bf16: Q8_0's q, Q4_0's
// 16 (q - 8), Q6_K's 4 (q - 32), the K-quants' q (Q4_K's high nibbles as
// 16 q); the constant factors go into the scales.  A code at its format's
// zero point is an exact 0.  Each activation x is split into two bf16
// parts, hi = RNE(x) and lo = RNE(x - hi) (the subtraction is exact), so
// |x - hi - lo| <= 2^-16 |x|: per output the representation error is at most
// 2^-16 sum |w x|.  Two MFMAs (hi, lo) accumulate sum code * (hi + lo) over
// a 32-column block in f32; the block's scale multiplies that sum in f32.
// The K-quants' min term dmin * m * sum(x) takes its sums from two more
// MFMAs against a B operand of ones.  Q6_K has two scale groups per block:
// its codes go in twice, each time with the other group's half zeroed.
//
// Work layout.  A wave owns one tile of 16 weight rows and a contiguous
// range of 256-column chunks; a workgroup of 8 waves holds 8 / KS tiles,
// each split over KS waves along the columns, whose partial sums are added
// through LDS in wave order at the end (deterministic).  A chunk's 16 row
// segments are copied with coalesced 16-byte loads into a private LDS slot
// of the wave, issued one chunk ahead, and read from there; the activations
// are loaded per lane in the matrix core's operand order, one step ahead (a
// step is a chunk at up to 16 batch rows, half a chunk at 17..32).
#pragma once

#include <type_traits>

#include "qg_kernels.hpp"
#include "qg_mfma.hpp"

namespace qg {
namespace gm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;     // waves per workgroup
constexpr int kTileRows = 16; // weight rows per tile
constexpr int kChunk = 256;   // columns per chunk

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Eight activations -> bf16 hi and lo parts (four dwords each, column order).
__device__ __forceinline__ void split_bf16(const uint32_t (&x)[8], u32x4 &hi, u32x4 &lo) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float x0 = __builtin_bit_cast(float, x[2 * i]);
        const float x1 = __builtin_bit_cast(float, x[2 * i + 1]);
        const bf16x2 h = {(__bf16)x0, (__bf16)x1};
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const float h0 = __builtin_bit_cast(float, hb << 16);
        const float h1 = __builtin_bit_cast(float, hb & 0xFFFF0000u);
        const bf16x2 l = {(__bf16)(x0 - h0), (__bf16)(x1 - h1)};
        hi[i] = hb;
        lo[i] = __builtin_bit_cast(uint32_t, l);
    }
}

// Two f32 values that are small integers -> one dword of two bf16 (their
// high halves; the low halves are zero).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                                 0x07060302u);
}

// Eight signed / unsigned code bytes (two dwords) -> eight bf16.
__device__ __forceinline__ u32x4 codes_s8(uint32_t v0, uint32_t v1) {
    u32x4 c;
    c[0] = pack2(sbyte<0>(v0), sbyte<1>(v0));
    c[1] = pack2(sbyte<2>(v0), sbyte<3>(v0));
    c[2] = pack2(sbyte<0>(v1), sbyte<1>(v1));
    c[3] = pack2(sbyte<2>(v1), sbyte<3>(v1));
    return c;
}

__device__ __forceinline__ u32x4 codes_u8(uint32_t v0, uint32_t v1) {
    v0 = opaque(v0);
    v1 = opaque(v1);
    u32x4 c;
    c[0] = pack2(ubyte<0>(v0), ubyte<1>(v0));
    c[1] = pack2(ubyte<2>(v0), ubyte<3>(v0));
    c[2] = pack2(ubyte<0>(v1), ubyte<1>(v1));
    c[3] = pack2(ubyte<2>(v1), ubyte<3>(v1));
    return c;
}

// Eight unsigned code bytes below 128 (two dwords) -> the eight bf16
// values 128 + n: the byte n becomes the mantissa under the bf16 pattern of
// 128 (0x4300), one byte permute per two codes.  The caller removes the 128
// offset with the block's sum of activations.
__device__ __forceinline__ u32x4 codes_u7_off128(uint32_t v0, uint32_t v1) {
    u32x4 c;
    c[0] = __builtin_amdgcn_perm(0x43434343u, v0, 0x04010400u);
    c[1] = __builtin_amdgcn_perm(0x43434343u, v0, 0x04030402u);
    c[2] = __builtin_amdgcn_perm(0x43434343u, v1, 0x04010400u);
    c[3] = __builtin_amdgcn_perm(0x43434343u, v1, 0x04030402u);
    return c;
}

// ---------------------------------------------------------------- formats
//
// Each format decodes, for its lane (row r, column quarter q) and 32-column
// block kb of a chunk: the eight codes (u32x4 of bf16), the block's scale
// s (and, for Q6_K, the second group's scale s2; for the K-quants the min
// factor dm = dmin * m).  Byte offsets are relative to the chunk's first
// byte in the staged row.  Layouts: web page docs.rs, crate ferrox-cuda
// 0.14.0, source src/gpu.rs, the *_MATVEC_KERNEL_SRC kernels.

struct Blk {
    u32x4 c;
    float s, s2, dm;
};

// Q8_0: eight 34-byte blocks per chunk; f16 d at 0, int8 q at 2.
struct GQ80 {
    static constexpr int CHUNK = 272;
    static constexpr bool MINS = false, TWO = false, OFF128 = false;
    struct Head {};
    template <bool RA>
    __device__ static Head head(const mx::RowRd<RA> &, int) { return {}; }
    template <bool RA, bool OFF>
    __device__ static Blk block(const mx::RowRd<RA> &rd, const Head &, int kb, int q) {
        Blk b;
        const int o = 34 * kb;
        b.c = codes_s8(rd.dw(o + 2 + 8 * q), rd.dw(o + 6 + 8 * q));
        b.s = f16_lo(rd.dw(o));
        b.s2 = b.dm = 0.f;
        return b;
    }
};

// Q4_0: eight 18-byte blocks; f16 d at 0, 16 bytes at 2 (element j < 16 the
// low nibble of byte j, element j + 16 the high nibble); value d (q - 8).
// Codes: nibble ^ 8 moved to the top of its byte, the signed 16 (q - 8).
struct GQ40 {
    static constexpr int CHUNK = 144;
    static constexpr bool MINS = false, TWO = false, OFF128 = false;
    struct Head {};
    template <bool RA>
    __device__ static Head head(const mx::RowRd<RA> &, int) { return {}; }
    template <bool RA, bool OFF>
    __device__ static Blk block(const mx::RowRd<RA> &rd, const Head &, int kb, int q) {
        Blk b;
        const int o = 18 * kb;
        const uint32_t sh = q < 2 ? 4u : 0u;
        const uint32_t v0 = ((rd.dw(o + 2 + 8 * (q & 1)) ^ 0x88888888u) << sh) & 0xF0F0F0F0u;
        const uint32_t v1 = ((rd.dw(o + 6 + 8 * (q & 1)) ^ 0x88888888u) << sh) & 0xF0F0F0F0u;
        b.c = codes_s8(opaque(v0), opaque(v1));
        b.s = f16_lo(rd.dw(o)) * 0.0625f;
        b.s2 = b.dm = 0.f;
        return b;
    }
};

// Q4_K / Q5_K: one super-block per chunk; d, dmin at 0, twelve bytes of
// packed 6-bit (scale, min) at 4 (ferrox_q4_k_scale_min); Q4_K qs[128] at
// 16, Q5_K qh[32] at 16 and qs[128] at 48.  Block g = 2p + u: nibble u of
// qs[32p + l] (Q5_K: plus 16 * bit g of qh[l]); value d sc q - dmin m.
// With OFF the codes enter as 128 + q (codes_u7_off128, four byte permutes
// where the plain conversion takes twelve operations); the kernel then takes
// the block's sum of (128 + q) x minus 128 times its sum of x before
// scaling (off128), so a block of zero codes still gives exactly 0: the two
// matrix-core sums differ by the factor 128 exactly.  That costs one fma per
// output and block, which pays where one weight block meets few activation
// rows.
template <bool FIVE>
struct GK45 {
    static constexpr int CHUNK = FIVE ? 176 : 144;
    static constexpr bool MINS = true, TWO = false, OFF128 = true;
    static constexpr int QS = FIVE ? 48 : 16;
    struct Head {
        float d, dmin;
        uint32_t s0, s1, s2;
        uint32_t h0, h1;  // Q5_K: qh bytes 8q .. 8q + 7
    };
    template <bool RA>
    __device__ static Head head(const mx::RowRd<RA> &rd, int q) {
        Head h;
        const uint32_t w = rd.dw(0);
        h.d = f16_lo(w);
        h.dmin = f16_hi(w);
        h.s0 = rd.dw(4);
        h.s1 = rd.dw(8);
        h.s2 = rd.dw(12);
        h.h0 = h.h1 = 0;
        if constexpr (FIVE) {
            h.h0 = rd.dw(16 + 8 * q);
            h.h1 = rd.dw(20 + 8 * q);
        }
        return h;
    }
    template <bool RA, bool OFF>
    __device__ static Blk block(const mx::RowRd<RA> &rd, const Head &h, int g, int q) {
        Blk b;
        const int p = g >> 1, u = g & 1;
        const uint32_t a0 = rd.dw(QS + 32 * p + 8 * q), a1 = rd.dw(QS + 32 * p + 4 + 8 * q);
        uint32_t s, mm;
        if (g < 4) {
            s = h.s0 >> (8 * g);
            mm = h.s1 >> (8 * g);
        } else {
            const int j = g - 4;
            s = ((h.s2 >> (8 * j)) & 15u) | (((h.s0 >> (8 * j)) >> 6) << 4);
            mm = ((h.s2 >> (8 * j + 4)) & 15u) | (((h.s1 >> (8 * j)) >> 6) << 4);
        }
        const float sc = (float)(s & 63u), m = (float)(mm & 63u);
        if constexpr (FIVE || OFF) {
            uint32_t n0 = u ? (a0 >> 4) & 0x0F0F0F0Fu : a0 & 0x0F0F0F0Fu;
            uint32_t n1 = u ? (a1 >> 4) & 0x0F0F0F0Fu : a1 & 0x0F0F0F0Fu;
            if constexpr (FIVE) {
                n0 |= ((h.h0 >> g) & 0x01010101u) << 4;
                n1 |= ((h.h1 >> g) & 0x01010101u) << 4;
            }
            b.c = OFF ? codes_u7_off128(n0, n1) : codes_u8(n0, n1);
            b.s = h.d * sc;
        } else {
            const uint32_t mk = u ? 0xF0F0F0F0u : 0x0F0F0F0Fu;  // high nibbles in place: 16 q
            b.c = codes_u8(a0 & mk, a1 & mk);
            b.s = h.d * sc * (u ? 0.0625f : 1.0f);
        }
        b.dm = h.dmin * m;
        b.s2 = 0.f;
        return b;
    }
};

// Q6_K: one super-block per chunk; ql[128] at 0, qh[64] at 128, int8 sc[16]
// at 192, f16 d at 208.  Block kb = 4h + t covers elements 128h + 32t + l:
// low bits nibble t/2 of ql[64h + 32(t%2) + l], top bits 2t..2t+1 of
// qh[32h + l]; scale sc[8h + 2t + l/16], so lanes q < 2 and q >= 2 hold the
// two scale groups.  Codes are the signed bytes 4 (q - 32).
struct GQ6K {
    static constexpr int CHUNK = 210;
    static constexpr bool MINS = false, TWO = true, OFF128 = false;
    struct Head {
        float d4;
    };
    template <bool RA>
    __device__ static Head head(const mx::RowRd<RA> &rd, int) {
        return {f16_lo(rd.dw(208)) * 0.25f};
    }
    template <bool RA, bool OFF>
    __device__ static Blk block(const mx::RowRd<RA> &rd, const Head &hd, int kb, int q) {
        Blk b;
        const int h = kb >> 2, t = kb & 3;
        const int ol = 64 * h + 32 * (t & 1) + 8 * q, oh = 128 + 32 * h + 8 * q;
        uint32_t c2[2];
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const uint32_t a = rd.dw(ol + 4 * k), hx = rd.dw(oh + 4 * k) ^ 0xAAAAAAAAu;
            const uint32_t lo = t < 2 ? (a << 2) & 0x3C3C3C3Cu : (a >> 2) & 0x3C3C3C3Cu;
            const uint32_t hi = (t == 0 ? hx << 6 : t == 1 ? hx << 4 : t == 2 ? hx << 2 : hx) &
                                0xC0C0C0C0u;
            c2[k] = opaque(lo | hi);
        }
        b.c = codes_s8(c2[0], c2[1]);
        // the dword holding sc[8h + 2t] and sc[8h + 2t + 1]
        const uint32_t sw = rd.dw(192 + 8 * h + 4 * (t >> 1));
        const int sb = 2 * (t & 1);
        b.s = hd.d4 * (float)(int8_t)(sw >> (8 * sb));
        b.s2 = hd.d4 * (float)(int8_t)(sw >> (8 * sb + 8));
        b.dm = 0.f;
        return b;
    }
};

// Cache policy of the batched kernels' weight loads: the default (0), not
// the non-temporal policy of the contiguous batch-1 streams.  A 16-row tile
// reads 144-272-byte row segments chunk by chunk, and consecutive chunks
// share the lines at their boundaries; with non-temporal loads those lines
// were fetched twice.  Measured at batch 8 (cold weights): Q4_0 4096 x 14336
// 44.2 -> 39.4 MB read, 23.0 -> 22.7 us; Q5_K 14336 x 4096 44.7 -> 43.4 MB,
// 25.1 -> 24.7 us.  (The shared-operand kernel keeps the non-temporal
// policy: there it read fewer bytes but ran no faster, Q4_0 slower.)
#ifndef QG_GEMM_AUX
#define QG_GEMM_AUX 0
#endif

// ---------------------------------------------------------------- kernel

// A block's product sum with the codes' 128 offset removed (formats with
// OFF128, blocks decoded with OFF): sum (128 + q) x - 128 sum x, exact for
// zero codes.
template <class F, bool OFF>
__device__ __forceinline__ float off128(float d, float sm) {
    if constexpr (F::OFF128 && OFF) return fmaf(-128.0f, sm, d);
    return d;
}

template <int N>
__device__ __forceinline__ void zero(f32x4 (&a)[N]) {
#pragma unroll
    for (int j = 0; j < N; j++) a[j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

struct GemmParams {
    const uint8_t *W;
    const float *X;  // [batch][cols] (this launch's batch rows)
    float *Y;        // [batch][rows]
    int64_t rows;
    uint64_t w_bytes;   // rows * row_bytes
    uint32_t row_bytes;
    uint32_t cols;
    int32_t batch;      // batch rows of this launch (<= 16 NB)
    int32_t nchunks;    // ceil(cols / 256)
    int32_t last_nkb;   // 32-column blocks in the last chunk (1..8)
    int32_t tiles;      // ceil(rows / 16)
    int32_t ks;         // waves per tile (1, 2, 4, 8), splitting the chunks
    int32_t nu;         // 16-byte units staged per row segment
    uint32_t slot;      // LDS bytes per staged row (odd multiple of 16)
};

// NB: batch blocks of 16 (1 or 2).  RA: row segments may start at 2 mod 4
// in LDS and are realigned.  UNITS: 16-byte stage loads per lane.
template <class F, int NB, bool RA, int UNITS>
__global__ void __launch_bounds__(512) qgemm_kernel(GemmParams p) {
    constexpr int XK = 8 / NB, NS = 8 / XK;  // blocks per step, steps per chunk
#ifndef QG_OFF_NB
#define QG_OFF_NB 2
#endif
    // 128-offset codes while a weight block meets at most two blocks of 16
    // activation rows (the per-output fma then costs less than the decode
    // it saves)
    constexpr bool OFF = NB <= QG_OFF_NB;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r = lane & 15, q = lane >> 4;
    const int tpw = kWaves / p.ks;
    const int64_t tile = (int64_t)blockIdx.x * tpw + wave / p.ks;
    const int ksi = wave % p.ks;
    const int c0 = (int)((int64_t)ksi * p.nchunks / p.ks);
    const int c1 = (int)((int64_t)(ksi + 1) * p.nchunks / p.ks);
    uint8_t *stage = smem + wave * kTileRows * p.slot;
    float *red = (float *)(smem + kWaves * kTileRows * p.slot);

    f32x4 acc[NB];
    zero(acc);
    if (tile < p.tiles && c0 < c1) {
        // weight rows of this tile: resource from the 16-byte boundary at or
        // below the tile's first byte to the end of W (rounded up to 16)
        const uint64_t tb = (uint64_t)tile * kTileRows * p.row_bytes;
        const uint8_t *gp = p.W + tb;
        const uint8_t *al = (const uint8_t *)((uintptr_t)gp & ~(uintptr_t)15);
        const uint32_t d0 = (uint32_t)(gp - al);
        const uint64_t rem = (p.w_bytes - tb + d0 + 15) & ~(uint64_t)15;
        const rsrc_t rw = make_rsrc(al, rem > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)rem);
        // stage unit map: load j of this lane copies unit lane + 64 j of the
        // 16 * nu units (row u / nu, unit u % nu of the row's segment)
        const int nunits = kTileRows * p.nu;
        uint32_t u_row[UNITS], u_off[UNITS];
#pragma unroll
        for (int j = 0; j < UNITS; j++) {
            const int u = lane + 64 * j, uu = u < nunits ? u : 0;
            const int rr = uu / p.nu;
            u_row[j] = (uint32_t)rr;
            u_off[j] = 16u * (uint32_t)(uu - rr * p.nu);
        }
        u32x4 wreg[UNITS];
        // branch-free: a unit past the tile's segments reads an out-of-range
        // offset (zeros, no memory access); loads under a branch were each
        // followed by a wait for all loads
        auto w_issue = [&](int c) {
#pragma unroll
            for (int j = 0; j < UNITS; j++) {
                const uint32_t base =
                    (d0 + u_row[j] * p.row_bytes + (uint32_t)c * F::CHUNK) & ~15u;
                const uint32_t off = lane + 64 * j < nunits ? base + u_off[j] : 0xFFFFFFF0u;
                wreg[j] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, QG_GEMM_AUX));
            }
        };
        // the chunk's rows into the wave's LDS slot (the previous chunk's
        // reads are done: the LDS accesses of a wave are in order)
        auto w_store = [&]() {
#pragma unroll
            for (int j = 0; j < UNITS; j++)
                if (lane + 64 * j < nunits)
                    *(u32x4 *)(stage + u_row[j] * p.slot + u_off[j]) = wreg[j];
        };
        // activations: lane (r, q) reads batch row 16 j + r, columns 8q..8q+7
        // of each block; rows past the batch read as zero
        const rsrc_t rx = make_rsrc(p.X, 4u * p.cols * (uint32_t)p.batch);
        uint32_t xraw[XK][NB][8];
        auto x_issue = [&](int c, int step) {
#pragma unroll
            for (int k = 0; k < XK; k++)
#pragma unroll
                for (int j = 0; j < NB; j++) {
                    const int b = 16 * j + r;
                    const uint32_t col = (uint32_t)c * kChunk + 32u * (step * XK + k) + 8u * q;
                    const uint32_t off = (b < p.batch && col < p.cols)
                                             ? 4u * ((uint32_t)b * p.cols + col) : 0x80000000u;
                    const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
                    const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u, 0, 0);
                    xraw[k][j][0] = v0[0]; xraw[k][j][1] = v0[1];
                    xraw[k][j][2] = v0[2]; xraw[k][j][3] = v0[3];
                    xraw[k][j][4] = v1[0]; xraw[k][j][5] = v1[1];
                    xraw[k][j][6] = v1[2]; xraw[k][j][7] = v1[3];
                }
        };
        const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        const uint32_t keep_lo = q < 2 ? 0xFFFFFFFFu : 0u;  // Q6_K: lanes of the first group

        // one chunk.  GUARD: the chunk may be the wave's last (no further
        // loads) or the row's last (fewer than 8 blocks), checked at run
        // time; without it the chunk is one branch-free block of code, so the
        // compiler can overlap the matrix core's latency with the next
        // block's decode.
        auto chunk = [&](int c, auto guard_tag) {
            constexpr bool GUARD = decltype(guard_tag)::value;
            const bool more = !GUARD || c + 1 < c1;
            const int nkb = GUARD && c == p.nchunks - 1 ? p.last_nkb : 8;
            const uint32_t delta = (d0 + (uint32_t)r * p.row_bytes + (uint32_t)c * F::CHUNK) & 15u;
            const mx::RowRd<RA> rd = mx::make_rowrd<RA>(stage + r * p.slot, delta, 0);
            const typename F::Head hd = F::template head<RA>(rd, q);
#pragma unroll
            for (int step = 0; step < NS; step++) {
                u32x4 xh[XK][NB], xl[XK][NB];
#pragma unroll
                for (int k = 0; k < XK; k++)
#pragma unroll
                    for (int j = 0; j < NB; j++) split_bf16(xraw[k][j], xh[k][j], xl[k][j]);
                if (step + 1 < NS) x_issue(c, step + 1);
                else if (more) x_issue(c + 1, 0);
                if (step == 0 && more) w_issue(c + 1);
#pragma unroll
                for (int k = 0; k < XK; k++) {
                    const int kb = step * XK + k;
                    if (!GUARD || kb < nkb) {
                        const Blk b = F::template block<RA, OFF>(rd, hd, kb, q);
                        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                        if constexpr (F::TWO) {
                            u32x4 ca, cb;
#pragma unroll
                            for (int i = 0; i < 4; i++) {
                                ca[i] = b.c[i] & keep_lo;
                                cb[i] = b.c[i] & ~keep_lo;
                            }
#pragma unroll
                            for (int j = 0; j < NB; j++) {
                                f32x4 da = mfma(xh[k][j], ca, z);
                                da = mfma(xl[k][j], ca, da);
                                f32x4 db = mfma(xh[k][j], cb, z);
                                db = mfma(xl[k][j], cb, db);
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    acc[j][i] = fmaf(b.s2, db[i], fmaf(b.s, da[i], acc[j][i]));
                            }
                        } else {
#pragma unroll
                            for (int j = 0; j < NB; j++) {
                                f32x4 d = mfma(xh[k][j], b.c, z);
                                d = mfma(xl[k][j], b.c, d);
                                f32x4 sm;
                                if constexpr (F::MINS) {
                                    sm = mfma(xh[k][j], ones, z);
                                    sm = mfma(xl[k][j], ones, sm);
                                }
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    acc[j][i] = fmaf(b.s, off128<F, OFF>(d[i], sm[i]), acc[j][i]);
                                if constexpr (F::MINS) {
#pragma unroll
                                    for (int i = 0; i < 4; i++)
                                        acc[j][i] = fmaf(-b.dm, sm[i], acc[j][i]);
                                }
                            }
                        }
                    }
                }
            }
            if (more) w_store();
        };
        x_issue(c0, 0);
        w_issue(c0);
        w_store();
        if constexpr (NB == 1) {
            for (int c = c0; c < c1 - 1; c++) chunk(c, std::false_type{});
            chunk(c1 - 1, std::true_type{});
        } else {
            // at 17..32 batch rows the branch-free form needs more registers
            // than a wave has (spills)
            for (int c = c0; c < c1; c++) chunk(c, std::true_type{});
        }
    }

    // partial sums of the ks waves of a tile, added in wave order
    const int64_t row = tile * kTileRows + r;
    if (p.ks > 1) {
#pragma unroll
        for (int j = 0; j < NB; j++)
#pragma unroll
            for (int i = 0; i < 4; i++) red[((wave * NB + j) * 4 + i) * 64 + lane] = acc[j][i];
        __syncthreads();
        if (ksi == 0 && tile < p.tiles) {
            for (int w = 1; w < p.ks; w++)
#pragma unroll
                for (int j = 0; j < NB; j++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[j][i] += red[(((wave + w) * NB + j) * 4 + i) * 64 + lane];
        }
    }
    if (ksi == 0 && tile < p.tiles && row < p.rows) {
#pragma unroll
        for (int j = 0; j < NB; j++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int b = 16 * j + 4 * q + i;
                if (b < p.batch) p.Y[(int64_t)b * p.rows + row] = acc[j][i];
            }
    }
}

// ------------------------------------------------ batch 1..8: packed parts
//
// At most 8 batch rows.  The hi and lo parts share one A operand: row b
// holds hi of batch row b and row 8 + b its lo, so one instruction per
// block does the work of the two above, and lane (r, q + 2) ends with the
// lo parts' sums of the batch rows whose hi parts' sums lane (r, q) holds.
//
// The activations are the kernel's largest stream (a 16-row tile re-reads
// its batch rows' activations, 8 KB per chunk at batch 8, for ~2.3-2.8 KB
// of weights), and each chunk waits for them: with no activation loads at
// all the batch-8 Q5_K 14336 x 4096 GEMV took 15.7 us instead of 27.6 us.
// So both streams run two chunks ahead here.  Lane (r, q) loads four of
// the eight columns of its block (r < 8 the first four of batch row r,
// r >= 8 the last four of batch row r - 8: 16 bytes per lane and block),
// splits them into hi and lo parts and trades the half its partner needs
// (lane r +- 8, the same row of 16 lanes) with one DPP rotation.  The
// weights of a chunk are staged into the wave's LDS slot at the start of
// the chunk, and that register buffer is refilled at once with the chunk
// two ahead.
template <class F, bool RA, int UNITS>
__global__ void __launch_bounds__(512) qgemm8_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r = lane & 15, q = lane >> 4;
    const int tpw = kWaves / p.ks;
    const int64_t tile = (int64_t)blockIdx.x * tpw + wave / p.ks;
    const int ksi = wave % p.ks;
    const int c0 = (int)((int64_t)ksi * p.nchunks / p.ks);
    const int c1 = (int)((int64_t)(ksi + 1) * p.nchunks / p.ks);
    uint8_t *stage = smem + wave * kTileRows * p.slot;
    float *red = (float *)(smem + kWaves * kTileRows * p.slot);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tile < p.tiles && c0 < c1) {
        const uint64_t tb = (uint64_t)tile * kTileRows * p.row_bytes;
        const uint8_t *gp = p.W + tb;
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
        // Every chunk issues the same loads, and none sits under a branch:
        // a unit past the tile's segments, or a chunk past the wave's range
        // (valid false), reads zeros from an out-of-range offset.  Loads
        // under a branch, or a count that differs between paths, made the
        // compiler wait for all loads, and the chunks ahead were no longer in
        // flight.
        auto w_issue = [&](int c, u32x4 (&w)[UNITS], bool valid) {
#pragma unroll
            for (int j = 0; j < UNITS; j++) {
                const uint32_t base =
                    (d0 + u_row[j] * p.row_bytes + (uint32_t)c * F::CHUNK) & ~15u;
                const uint32_t off =
                    valid && lane + 64 * j < nunits ? base + u_off[j] : 0xFFFFFFF0u;
                w[j] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, QG_GEMM_AUX));
            }
        };
        auto w_store = [&](const u32x4 (&w)[UNITS]) {
#pragma unroll
            for (int j = 0; j < UNITS; j++)
                if (lane + 64 * j < nunits)
                    *(u32x4 *)(stage + u_row[j] * p.slot + u_off[j]) = w[j];
        };
        const rsrc_t rx = make_rsrc(p.X, 4u * p.cols * (uint32_t)p.batch);
        const int b = r & 7, hh = r >> 3;
        // (plain arrays: this compiler mis-evaluated the element-wise bf16
        // split when the four values were taken from a vector type by a
        // loop index, using the first value for the second)
        auto x_issue = [&](int c, uint32_t (&x)[8][4], bool valid) {
#pragma unroll
            for (int kb = 0; kb < 8; kb++) {
                const uint32_t col = (uint32_t)c * kChunk + 32u * kb + 8u * q + 4u * hh;
                const uint32_t off = (valid && b < p.batch && col < p.cols)
                                         ? 4u * ((uint32_t)b * p.cols + col) : 0x80000000u;
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
                x[kb][0] = v[0];
                x[kb][1] = v[1];
                x[kb][2] = v[2];
                x[kb][3] = v[3];
            }
        };
        // the operand of lane (r, q) for one block from its four values
        auto xop = [&](const uint32_t (&v)[4]) {
            uint32_t h[2], l[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const float x0 = __builtin_bit_cast(float, v[2 * i]);
                const float x1 = __builtin_bit_cast(float, v[2 * i + 1]);
                const bf16x2 hv = {(__bf16)x0, (__bf16)x1};
                h[i] = __builtin_bit_cast(uint32_t, hv);
                const float h0 = __builtin_bit_cast(float, h[i] << 16);
                const float h1 = __builtin_bit_cast(float, h[i] & 0xFFFF0000u);
                const bf16x2 lv = {(__bf16)(x0 - h0), (__bf16)(x1 - h1)};
                l[i] = __builtin_bit_cast(uint32_t, lv);
            }
            // r < 8 keeps its hi parts and takes the partner's hi parts of
            // the last four columns; r >= 8 keeps its lo parts and takes the
            // partner's lo parts of the first four
            const uint32_t t0 = dpp_u<0x128>(hh ? h[0] : l[0]);  // row_ror:8
            const uint32_t t1 = dpp_u<0x128>(hh ? h[1] : l[1]);
            u32x4 a;
            a[0] = hh ? t0 : h[0];
            a[1] = hh ? t1 : h[1];
            a[2] = hh ? l[0] : t0;
            a[3] = hh ? l[1] : t1;
            return a;
        };
        const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        const uint32_t keep_lo = q < 2 ? 0xFFFFFFFFu : 0u;  // Q6_K: lanes of the first group

        auto chunk = [&](int c, uint32_t (&xc)[8][4], u32x4 (&wc)[UNITS], auto guard_tag) {
            constexpr bool GUARD = decltype(guard_tag)::value;
            const int nkb = GUARD && c == p.nchunks - 1 ? p.last_nkb : 8;
            // chunk c's weights into the slot (the previous chunk's reads of
            // it are done: a wave's LDS accesses are in order), then the
            // buffer takes chunk c + 2
            w_store(wc);
            w_issue(c + 2, wc, c + 2 < c1);
            u32x4 a[8];
#pragma unroll
            for (int kb = 0; kb < 8; kb++) a[kb] = xop(xc[kb]);
            x_issue(c + 2, xc, c + 2 < c1);
            const uint32_t delta = (d0 + (uint32_t)r * p.row_bytes + (uint32_t)c * F::CHUNK) & 15u;
            const mx::RowRd<RA> rd = mx::make_rowrd<RA>(stage + r * p.slot, delta, 0);
            const typename F::Head hd = F::template head<RA>(rd, q);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 8; kb++) {
                if (!GUARD || kb < nkb) {
                    const Blk bk = F::template block<RA, true>(rd, hd, kb, q);
                    if constexpr (F::TWO) {
                        u32x4 ca, cb;
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            ca[i] = bk.c[i] & keep_lo;
                            cb[i] = bk.c[i] & ~keep_lo;
                        }
                        const f32x4 da = mfma(a[kb], ca, z);
                        const f32x4 db = mfma(a[kb], cb, z);
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[i] = fmaf(bk.s2, db[i], fmaf(bk.s, da[i], acc[i]));
                    } else {
                        const f32x4 d = mfma(a[kb], bk.c, z);
                        f32x4 sm = z;
                        if constexpr (F::MINS) sm = mfma(a[kb], ones, z);
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[i] = fmaf(bk.s, off128<F, true>(d[i], sm[i]), acc[i]);
                        if constexpr (F::MINS) {
#pragma unroll
                            for (int i = 0; i < 4; i++) acc[i] = fmaf(-bk.dm, sm[i], acc[i]);
                        }
                    }
                }
            }
        };
        uint32_t xA[8][4], xB[8][4];
        u32x4 wA[UNITS], wB[UNITS];
        x_issue(c0, xA, true);
        w_issue(c0, wA, true);
        x_issue(c0 + 1, xB, c0 + 1 < c1);
        w_issue(c0 + 1, wB, c0 + 1 < c1);
        // chunks in pairs (buffers A, B) while neither is the wave's last;
        // the last chunk checks the row's block count
        int c = c0;
        for (; c + 2 < c1; c += 2) {
            chunk(c, xA, wA, std::false_type{});
            chunk(c + 1, xB, wB, std::false_type{});
        }
        if (c + 1 == c1) {
            chunk(c, xA, wA, std::true_type{});
        } else {
            chunk(c, xA, wA, std::false_type{});
            chunk(c + 1, xB, wB, std::true_type{});
        }
    }
    // lane (r, q + 2) holds the lo parts' sums of the batch rows whose hi
    // parts' sums lane (r, q) holds
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] += __shfl_xor(acc[i], 32);

    // partial sums of the ks waves of a tile, added in wave order
    const int64_t row = tile * kTileRows + r;
    if (p.ks > 1) {
#pragma unroll
        for (int i = 0; i < 4; i++) red[(wave * 4 + i) * 64 + lane] = acc[i];
        __syncthreads();
        if (ksi == 0 && tile < p.tiles) {
            for (int w = 1; w < p.ks; w++)
#pragma unroll
                for (int i = 0; i < 4; i++) acc[i] += red[((wave + w) * 4 + i) * 64 + lane];
        }
    }
    if (ksi == 0 && tile < p.tiles && row < p.rows && q < 2) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int bo = 4 * q + i;
            if (bo < p.batch) p.Y[(int64_t)bo * p.rows + row] = acc[i];
        }
    }
}

}  // namespace gm
}  // namespace qg
