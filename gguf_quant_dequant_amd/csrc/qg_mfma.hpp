// qg_mfma.hpp -- the batched dequantise-and-dot GEMV on the gfx950 matrix
// cores: v_mfma_f32_32x32x16_f16 with the weight codes as one operand and
// the activations as the other.
//
// Numbers.  Codes enter the matrix core as exact f16 values.  Unsigned
// K-quant codes n (< 256) are widened to 16 bits and used as an IEEE
// binary16 bit pattern, i.e. the subnormal n * 2^-24, which the matrix core
// multiplies exactly.  Codes with a zero point (Q6_K's q - 32, Q8_0's signed
// q, Q4_0's q - 8) are turned into the signed integers themselves: the code
// byte u (an unsigned 0..255 form) becomes the low byte of the f16 pattern
// 0x64uu = 1024 + u, and a packed f16 subtraction of 1024 + offset leaves
// u - offset, exactly (every integer up to 2048 is an f16 value).  A code at
// its zero point is therefore an exact 0 and contributes nothing.  Each
// 256-column chunk of each activation row is scaled by a power of two 2^e,
// chosen so its largest magnitude lies in [2^13, 2^14), and split into
// hi = RTZ_f16(x') and lo = RTZ_f16(x' - hi), so that
// |x' - hi - lo| < 2^-21 |x'|.  The matrix core sums code * hi and
// code * lo over 16 columns in f32.  The group's scale (d * sc; for the
// signed codes times 2^-24, for the K-quants the min term d_min * m *
// sum(x') is carried beside it as an accumulator seed -sum(x') * 2^-24)
// multiplies the group sum in f32, and 2^(24 - e) takes each chunk back to
// the activations' units.
//
// Work layout.  A tile is 32 consecutive weight rows (the MFMA's n); lane l
// of a wave feeds row l % 32 and the half kh = l / 32 of each 16-column
// sub-group (columns 8 kh .. 8 kh + 7).  A workgroup has 8 waves; KS of
// them share a tile and take its chunks round-robin, the rest take other
// tiles; partial sums of a tile are added in LDS in wave order.  Each wave
// streams its chunks through a private LDS slot: the chunk's bytes for the
// 32 rows are read with coalesced 16-byte loads into VGPRs one chunk ahead,
// then written to the slot, so the next chunk's loads are in flight while
// the current one is decoded.  The activations are converted once per
// workgroup into an LDS image laid out as the MFMA reads it.
//
// MFMA register use (verified on the device): lane l holds A[m][k] for
// m = l % 32 and B[k][n] for n = l % 32 over the same eight k of half
// l / 32, and D[m][n] for n = l % 32, m = 8 (i / 4) + 4 (l / 32) + i % 4 in
// register i.  The activations use A rows m = b (hi of batch row b) and
// m = 8 + b (lo of b), so lane (n, kh) receives hi and lo of batch rows
// 4 kh .. 4 kh + 3 in registers 0..3 and 4..7.
#pragma once

#include "qg_device.hpp"

namespace qg {
namespace mx {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 32;    // weight rows per tile
constexpr int kChunk = 256;  // columns per chunk
constexpr int kSubs = 16;    // 16-column sub-groups per chunk
constexpr int kWaves = 8;    // waves per workgroup

// batch rows per lane, lane halves that carry batch rows, image bytes
constexpr int nb_of(int B) { return B < 4 ? B : 4; }
constexpr int kh_of(int B) { return B > 4 ? 2 : 1; }
// Activation image of one chunk: A operands [sub-group][slot][16] f16 with
// slot = hl * B + b (1024 B bytes), accumulator seeds [sub-group][kh][8]
// f32 (seed of batch rows 4 kh + i, then four zeros), and the chunk's
// scale-back factors [kh][4] f32.
constexpr int ximg_a(int B) { return 1024 * B; }
constexpr int ximg_c(int B) { return 512 * kh_of(B); }
constexpr int ximg_rec(int B) { return ximg_a(B) + ximg_c(B) + 16 * kh_of(B); }

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                   __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// Eight code bytes (two dwords) -> eight 16-bit lanes, in byte order.
__device__ __forceinline__ u32x4 widen2(uint32_t c0, uint32_t c1) {
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(0u, c0, 0x0C010C00u);
    r[1] = __builtin_amdgcn_perm(0u, c0, 0x0C030C02u);
    r[2] = __builtin_amdgcn_perm(0u, c1, 0x0C010C00u);
    r[3] = __builtin_amdgcn_perm(0u, c1, 0x0C030C02u);
    return r;
}

typedef _Float16 half2 __attribute__((ext_vector_type(2)));

// Eight code bytes u (two dwords) -> eight f16 lanes holding the integers
// u - OFF, in byte order: v_perm_b32 pairs each byte with 0x64 (the f16
// 1024 + u), then one packed f16 subtraction of 1024 + OFF per two codes.
// Both steps are exact for u < 256 and OFF <= 255.
template <int OFF>
__device__ __forceinline__ u32x4 widen2s(uint32_t c0, uint32_t c1) {
    constexpr uint32_t kHi = 0x64646464u;
    const half2 sub = {(_Float16)(-(1024 + OFF)), (_Float16)(-(1024 + OFF))};
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(kHi, c0, 0x04010400u);
    r[1] = __builtin_amdgcn_perm(kHi, c0, 0x04030402u);
    r[2] = __builtin_amdgcn_perm(kHi, c1, 0x04010400u);
    r[3] = __builtin_amdgcn_perm(kHi, c1, 0x04030402u);
#pragma unroll
    for (int i = 0; i < 4; i++)
        r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2, (uint32_t)r[i]) + sub);
    return r;
}

template <int S>
__device__ __forceinline__ uint32_t shl(uint32_t v) {
    if constexpr (S >= 0) return v << S;
    else return v >> (-S);
}

__device__ __forceinline__ float sbyte_at(uint32_t v, int j) { return (float)(int8_t)(v >> (8 * j)); }
__device__ __forceinline__ float ubyte_at(uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xFFu); }

template <int W>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (W >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
    if constexpr (W >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
    if constexpr (W >= 8) v = fmaxf(v, dpp_f<0x141>(v));
    if constexpr (W >= 16) v = fmaxf(v, dpp_f<0x140>(v));
    if constexpr (W >= 32) v = fmaxf(v, xor16_f(v));
    if constexpr (W >= 64) v = fmaxf(v, xor32_f(v));
    return v;
}

// ------------------------------------------------------------ activations

// Builds the activation image of all nc chunks in LDS (ximg), one wave per
// (chunk, batch row).  Batch row b starts at float b * xstride of X (X may
// be a column slice of a wider activation matrix; xbytes bounds the reads).
// With SEEDS (the K-quants) each code group's accumulator seed
// coff * sum(x') is stored beside the operands (coff = -2^-24, the min
// term); glanes = lanes per code group (4 for 16-column groups, 8 for 32).
// Batch rows >= batch and columns >= cols read as zero.
template <int B, bool SEEDS>
__device__ void build_ximg(const float *__restrict__ X, uint32_t cols, uint32_t xstride,
                           uint32_t xbytes, int batch, int nc, float coff, int glanes,
                           uint8_t *ximg) {
    constexpr int KH = kh_of(B), REC = ximg_rec(B);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const rsrc_t rx = make_rsrc(X, xbytes);
    // the wave's units in rounds of XK: all loads of a round are issued
    // before the first is converted (one load and its wait per unit left a
    // memory latency per unit on the workgroup's start)
    constexpr int XK = 8;
    const int nu = nc * B;
    for (int u0 = wave; u0 < nu; u0 += kWaves * XK) {
        uint32_t wv[XK][4];
#pragma unroll
        for (int k = 0; k < XK; k++) {
            const int u = u0 + k * kWaves;
            const int c = u / B, b = u - c * B;
            const uint32_t col = (uint32_t)c * kChunk + 4u * lane;
            // units past the last, columns past the row and batch rows past
            // `batch` read as zero (an out-of-range offset reads zeros
            // without a memory access)
            const uint32_t xo = (u < nu && b < batch && col < cols)
                                    ? 4u * ((uint32_t)b * xstride + col) : 0xFFFFFFF0u;
            const auto w = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
            wv[k][0] = w[0];
            wv[k][1] = w[1];
            wv[k][2] = w[2];
            wv[k][3] = w[3];
        }
#pragma unroll
        for (int k = 0; k < XK; k++) {
            const int u = u0 + k * kWaves;
            if (u >= nu) break;
            const int c = u / B, b = u - c * B;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; j++) v[j] = __builtin_bit_cast(float, wv[k][j]);
            float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
            am = group_max<64>(am);
            int e = 0;
            if (am > 0.f && am <= 3.4028234663852886e38f) {
                e = 14 - __builtin_amdgcn_frexp_expf(am);
                e = e < -64 ? -64 : (e > 64 ? 64 : e);
            }
            float xs[4], r[4];
#pragma unroll
            for (int j = 0; j < 4; j++) xs[j] = __builtin_amdgcn_ldexpf(v[j], e);
            const auto h01 = __builtin_amdgcn_cvt_pkrtz(xs[0], xs[1]);
            const auto h23 = __builtin_amdgcn_cvt_pkrtz(xs[2], xs[3]);
            r[0] = xs[0] - (float)h01[0];
            r[1] = xs[1] - (float)h01[1];
            r[2] = xs[2] - (float)h23[0];
            r[3] = xs[3] - (float)h23[1];
            const auto l01 = __builtin_amdgcn_cvt_pkrtz(r[0], r[1]);
            const auto l23 = __builtin_amdgcn_cvt_pkrtz(r[2], r[3]);
            uint8_t *rec = ximg + (size_t)c * REC;
            const int g = lane >> 2, pos = 4 * (lane & 3);
            u32x2 hv, lv;
            hv[0] = __builtin_bit_cast(uint32_t, h01);
            hv[1] = __builtin_bit_cast(uint32_t, h23);
            lv[0] = __builtin_bit_cast(uint32_t, l01);
            lv[1] = __builtin_bit_cast(uint32_t, l23);
            *(u32x2 *)(rec + 2 * ((g * 2 * B + b) * 16 + pos)) = hv;
            *(u32x2 *)(rec + 2 * ((g * 2 * B + B + b) * 16 + pos)) = lv;
            if constexpr (SEEDS) {
                float s = (xs[0] + xs[1]) + (xs[2] + xs[3]);
                s = glanes == 8 ? group_sum<8>(s) : group_sum<4>(s);
                if ((lane & (glanes - 1)) == 0) {
                    float *cp = (float *)(rec + ximg_a(B)) + (g * KH + b / 4) * 8;
                    cp[b & 3] = coff * s;
                    cp[4 + (b & 3)] = 0.f;
                }
            }
            if (lane == 0)
                ((float *)(rec + ximg_a(B) + ximg_c(B)))[4 * (b / 4) + (b & 3)] =
                    __builtin_amdgcn_ldexpf(1.0f, 24 - e);
        }
    }
}

// Per-lane byte offsets into a chunk's activation image.
struct XLane {
    uint32_t a;  // A operand of sub-group 0 (sub-group g adds 64 B g)
    uint32_t c;  // accumulator seed of sub-group 0 (g adds 32 KH g)
    uint32_t e;  // scale-back factors
};

template <int B>
__device__ __forceinline__ XLane make_xlane(int lane) {
    const int mm = lane & 15, kh = (lane >> 5) & 1;
    const int hl = mm >> 3;
    int b = mm & 7;
    b = b < B ? b : B - 1;  // rows of unused slots never reach an output
    const int khp = B > 4 ? kh : 0;
    XLane x;
    x.a = (uint32_t)(2 * ((hl * B + b) * 16 + kh * 8));
    x.c = (uint32_t)(ximg_a(B) + khp * 32);
    x.e = (uint32_t)(ximg_a(B) + ximg_c(B) + khp * 16);
    return x;
}

template <int B>
__device__ __forceinline__ u32x4 a_op(const uint8_t *rec, const XLane &xl, int g) {
    return *(const u32x4 *)(rec + xl.a + 64 * B * g);
}

// Seeds (-2^-24 * sum(x') of the code group starting at sub-group g, the
// K-quant min term) of this lane's batch rows.
template <int B>
__device__ __forceinline__ f32x4 c_vals(const uint8_t *rec, const XLane &xl, int g) {
    return *(const f32x4 *)(rec + xl.c + 32 * kh_of(B) * g);
}

// ---------------------------------------------------------- weight rows

// A row's chunk bytes in the LDS slot.  p0 points at the dword holding the
// chunk's first byte, sh is that byte's position in it (0 or 2; 0 when not
// RA).  Fields at byte offsets 0 mod 4 are read from p0 with shift sh,
// those at 2 mod 4 from p2 = p0 + sh/2 with shift (sh + 2) mod 4.  Code
// pieces add this lane's 8-byte half (kd = 2 kh dwords).
template <bool RA>
struct RowRd {
    const uint32_t *p0, *p2;
    uint32_t s0, s2;
    int kd;

    __device__ __forceinline__ uint32_t dw(int o) const {
        if (!RA && (o & 3) == 0) return p0[o >> 2];
        const uint32_t *p = (o & 3) ? p2 : p0;
        const uint32_t s = RA ? ((o & 3) ? s2 : s0) : 2u;
        const int i = o >> 2;
        return __builtin_amdgcn_alignbyte(p[i + 1], p[i], s);
    }
    // eight bytes at offset o + 8 kh
    __device__ __forceinline__ void piece(int o, uint32_t (&v)[2]) const {
        if (!RA && (o & 7) == 0) {
            const u32x2 w = *(const u32x2 *)(p0 + kd + (o >> 2));
            v[0] = w[0];
            v[1] = w[1];
            return;
        }
        if (!RA && (o & 3) == 0) {
            v[0] = p0[kd + (o >> 2)];
            v[1] = p0[kd + (o >> 2) + 1];
            return;
        }
        const uint32_t *p = ((o & 3) ? p2 : p0) + kd + (o >> 2);
        const uint32_t s = RA ? ((o & 3) ? s2 : s0) : 2u;
        const uint32_t w0 = p[0], w1 = p[1], w2 = p[2];
        v[0] = __builtin_amdgcn_alignbyte(w1, w0, s);
        v[1] = __builtin_amdgcn_alignbyte(w2, w1, s);
    }
};

template <bool RA>
__device__ __forceinline__ RowRd<RA> make_rowrd(const uint8_t *row, uint32_t delta, int kh) {
    RowRd<RA> r;
    const uint32_t *b = (const uint32_t *)(row + (delta & ~3u));
    const uint32_t sh = RA ? (delta & 3u) : 0u;
    r.p0 = b;
    r.p2 = b + (sh >> 1);
    r.s0 = sh;
    r.s2 = (sh + 2u) & 3u;
    r.kd = 2 * kh;
    return r;
}

// ------------------------------------------------------------ formats
//
// Each format decodes halves h0 .. h1 - 1 (of two) of one 256-column chunk
// of its lane's row and adds, for each of the lane's NB batch rows, the sum
// over those columns of weight * x' * 2^-24 into r.  CHUNK = bytes per
// chunk, SC = 16-byte units per row slot (odd, which spreads the rows over
// LDS banks), GW = code-group width, SEEDS = the image carries per-group
// accumulator seeds (the K-quant min term).

// Q6_K (web page: docs.rs, crate ferrox-cuda 0.14.0, source src/gpu.rs,
// Q6_K_MATVEC_KERNEL_SRC): 210-byte blocks, ql[128] at 0, qh[64] at 128,
// sixteen int8 scales at 192, f16 d at 208; element 128 h + 32 t + l has low
// bits nibble t/2 of ql[64 h + 32 (t%2) + l], top bits 2t..2t+1 of
// qh[32 h + l], value d * sc[e/16] * (q - 32).  Sub-group G = 8h + 2t + u
// holds l = 16u .. 16u+15 of quarter t.
struct MQ6K {
    static constexpr int CHUNK = 210, SC = 15, GW = 16;
    static constexpr bool SEEDS = false;

    template <int B, bool RA>
    static __device__ __forceinline__ void chunk(const RowRd<RA> &rd, const uint8_t *rec,
                                                 const XLane &xl, float (&r)[nb_of(B)], int,
                                                 int h0, int h1) {
        constexpr int NB = nb_of(B);
        uint32_t S[4];
#pragma unroll
        for (int j = 0; j < 4; j++) S[j] = rd.dw(192 + 4 * j);
        const float d = f16_lo(rd.dw(208)) * 0x1p-24f;  // codes are integers q - 32
        const f32x16 z = {};
#pragma unroll
        for (int h = 0; h < 2; h++) {
            if (h < h0 || h >= h1) continue;
#pragma unroll
            for (int u = 0; u < 2; u++) {
                uint32_t H[2];
                rd.piece(128 + 32 * h + 16 * u, H);
#pragma unroll
                for (int pp = 0; pp < 2; pp++) {
                    uint32_t A[2];
                    rd.piece(64 * h + 32 * pp + 16 * u, A);
                    uint32_t cl[2], ch[2];
#pragma unroll
                    for (int k = 0; k < 2; k++) {
                        const uint32_t hl = pp ? shl<2>(H[k]) : shl<4>(H[k]);
                        const uint32_t hh = pp ? shl<-2>(H[k]) : H[k];
                        cl[k] = (A[k] & 0x0F0F0F0Fu) | (hl & 0x30303030u);
                        ch[k] = ((A[k] >> 4) & 0x0F0F0F0Fu) | (hh & 0x30303030u);
                    }
#pragma unroll
                    for (int half = 0; half < 2; half++) {
                        const int G = 8 * h + 2 * (pp + 2 * half) + u;
                        const u32x4 bw =
                            half ? widen2s<32>(ch[0], ch[1]) : widen2s<32>(cl[0], cl[1]);
                        const f32x16 D = mfma(a_op<B>(rec, xl, G), bw, z);
                        const float s = d * sbyte_at(S[G >> 2], G & 3);
#pragma unroll
                        for (int i = 0; i < NB; i++) r[i] = fmaf(s, D[i] + D[4 + i], r[i]);
                    }
                }
            }
        }
    }
};

// Q4_K (same page, Q4_K_MATVEC_KERNEL_SRC) and Q5_K (Q5_K_MATVEC_KERNEL_SRC):
// d, dmin (f16) at 0 and 2, twelve bytes of 6-bit (scale, min) pairs at 4;
// Q4_K has qs[128] at 16, Q5_K has qh[32] at 16 and qs[128] at 48.  Group
// G (32 columns) takes nibble G%2 of qs[32 (G/2) + l]; Q5_K's fifth bit is
// bit G of qh[l].  Value d * sc * q - dmin * m.  Q4_K's high nibbles are
// used in place (16 q) and their group sums scaled by 1/16.
template <bool FIVE>
struct MK45 {
    static constexpr int CHUNK = FIVE ? 176 : 144, SC = FIVE ? 13 : 11, GW = 32;
    static constexpr bool SEEDS = true;  // seeds hold -sum(x') * 2^-24 for the min term
    static constexpr int QS = FIVE ? 48 : 16;

    template <int B, bool RA>
    static __device__ __forceinline__ void chunk(const RowRd<RA> &rd, const uint8_t *rec,
                                                 const XLane &xl, float (&r)[nb_of(B)], int,
                                                 int h0, int h1) {
        constexpr int NB = nb_of(B);
        const uint32_t w0 = rd.dw(0);
        const float d = f16_lo(w0), dmin = f16_hi(w0);
        const uint32_t S0 = rd.dw(4), S1 = rd.dw(8), S2 = rd.dw(12);
        const uint32_t sc[2] = {S0 & 0x3F3F3F3Fu,
                                (S2 & 0x0F0F0F0Fu) | ((S0 >> 2) & 0x30303030u)};
        const uint32_t mn[2] = {S1 & 0x3F3F3F3Fu,
                                ((S2 >> 4) & 0x0F0F0F0Fu) | ((S1 >> 2) & 0x30303030u)};
        uint32_t H[2][2];
        if constexpr (FIVE) {
            rd.piece(16, H[0]);
            rd.piece(32, H[1]);
        }
        float as[NB], ah[NB], am[NB];
#pragma unroll
        for (int i = 0; i < NB; i++) as[i] = ah[i] = am[i] = 0.f;
#pragma unroll
        for (int p = 0; p < 4; p++) {
            if (p < 2 * h0 || p >= 2 * h1) continue;
            f32x16 dl, dh;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                uint32_t A[2];
                rd.piece(QS + 32 * p + 16 * j, A);
                uint32_t cl[2], ch[2];
#pragma unroll
                for (int k = 0; k < 2; k++) {
                    if constexpr (FIVE) {
                        const uint32_t hb = H[j][k];
                        uint32_t bl, bh;
                        if (p == 0) { bl = hb << 4; bh = hb << 3; }
                        else if (p == 1) { bl = hb << 2; bh = hb << 1; }
                        else if (p == 2) { bl = hb; bh = hb >> 1; }
                        else { bl = hb >> 2; bh = hb >> 3; }
                        cl[k] = (A[k] & 0x0F0F0F0Fu) | (bl & 0x10101010u);
                        ch[k] = ((A[k] >> 4) & 0x0F0F0F0Fu) | (bh & 0x10101010u);
                    } else {
                        cl[k] = A[k] & 0x0F0F0F0Fu;
                        ch[k] = A[k] & 0xF0F0F0F0u;
                    }
                }
                const int gl = 2 * (2 * p) + j, gh = 2 * (2 * p + 1) + j;
                const f32x16 z = {};
                dl = mfma(a_op<B>(rec, xl, gl), widen2(cl[0], cl[1]), j ? dl : z);
                dh = mfma(a_op<B>(rec, xl, gh), widen2(ch[0], ch[1]), j ? dh : z);
            }
            const int G0 = 2 * p, G1 = 2 * p + 1;
            const float s0 = ubyte_at(sc[G0 >> 2], G0 & 3), s1 = ubyte_at(sc[G1 >> 2], G1 & 3);
            const float m0 = ubyte_at(mn[G0 >> 2], G0 & 3), m1 = ubyte_at(mn[G1 >> 2], G1 & 3);
            const f32x4 c0 = c_vals<B>(rec, xl, 2 * G0), c1 = c_vals<B>(rec, xl, 2 * G1);
#pragma unroll
            for (int i = 0; i < NB; i++) {
                as[i] = fmaf(s0, dl[i] + dl[4 + i], as[i]);
                ah[i] = fmaf(s1, dh[i] + dh[4 + i], ah[i]);
                am[i] = fmaf(m0, c0[i], am[i]);
                am[i] = fmaf(m1, c1[i], am[i]);
            }
        }
        const float hs = FIVE ? 1.f : 0.0625f;
#pragma unroll
        for (int i = 0; i < NB; i++) r[i] += d * fmaf(hs, ah[i], as[i]) + dmin * am[i];
    }
};

// Q8_0 (same page, Q8_0_MATVEC_KERNEL_SRC): 34-byte blocks of 32 columns,
// f16 d at 0, int8 codes at 2; value d * q.  Eight blocks per chunk (fewer
// in a row's last chunk when the row is not a multiple of 256 columns).
// The int8 q is flipped to q + 128 and widened back to the integer q.
struct MQ80 {
    static constexpr int CHUNK = 272, SC = 19, GW = 32;
    static constexpr bool SEEDS = false;

    template <int B, bool RA>
    static __device__ __forceinline__ void chunk(const RowRd<RA> &rd, const uint8_t *rec,
                                                 const XLane &xl, float (&r)[nb_of(B)],
                                                 int nblk, int h0, int h1) {
        constexpr int NB = nb_of(B);
        const f32x16 z = {};
#pragma unroll
        for (int blk = 0; blk < 8; blk++) {
            if (blk < nblk && blk >= 4 * h0 && blk < 4 * h1) {
                const float d = f16_lo(rd.dw(34 * blk)) * 0x1p-24f;
                f32x16 D;
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    uint32_t A[2];
                    rd.piece(34 * blk + 2 + 16 * j, A);
                    const u32x4 bw = widen2s<128>(A[0] ^ 0x80808080u, A[1] ^ 0x80808080u);
                    const int g = 2 * blk + j;
                    D = mfma(a_op<B>(rec, xl, g), bw, j ? D : z);
                }
#pragma unroll
                for (int i = 0; i < NB; i++) r[i] = fmaf(d, D[i] + D[4 + i], r[i]);
            }
        }
    }
};

// Q4_0 (same page, Q4_0_MATVEC_KERNEL_SRC): 18-byte blocks of 32 columns,
// f16 d at 0, 16 bytes at 2; element j < 16 is the low nibble of byte j,
// element j + 16 the high nibble; value d * (q - 8).
struct MQ40 {
    static constexpr int CHUNK = 144, SC = 11, GW = 32;
    static constexpr bool SEEDS = false;

    template <int B, bool RA>
    static __device__ __forceinline__ void chunk(const RowRd<RA> &rd, const uint8_t *rec,
                                                 const XLane &xl, float (&r)[nb_of(B)],
                                                 int nblk, int h0, int h1) {
        constexpr int NB = nb_of(B);
        const f32x16 z = {};
#pragma unroll
        for (int blk = 0; blk < 8; blk++) {
            if (blk < nblk && blk >= 4 * h0 && blk < 4 * h1) {
                const float d = f16_lo(rd.dw(18 * blk)) * 0x1p-24f;
                uint32_t A[2];
                rd.piece(18 * blk + 2, A);
                const int g = 2 * blk;
                f32x16 D = mfma(a_op<B>(rec, xl, g),
                                widen2s<8>(A[0] & 0x0F0F0F0Fu, A[1] & 0x0F0F0F0Fu), z);
                D = mfma(a_op<B>(rec, xl, g + 1),
                         widen2s<8>((A[0] >> 4) & 0x0F0F0F0Fu, (A[1] >> 4) & 0x0F0F0F0Fu), D);
#pragma unroll
                for (int i = 0; i < NB; i++) r[i] = fmaf(d, D[i] + D[4 + i], r[i]);
            }
        }
    }
};

// ---------------------------------------------------------------- kernel
//
// A workgroup of 8 waves works on one tile (32 rows) at a time.  The columns
// of a tile are taken in phases of P chunks; a stage is the tile's bytes for
// one phase.  The 512 threads copy a stage with 16-byte loads taken row
// segment by row segment (consecutive lanes read consecutive bytes of a row,
// so every cache line is requested whole), write it to an LDS buffer and,
// after a barrier, the waves decode it: work item i of the stage is half
// (i % NPART) of chunk i / NPART (NPART = 1 or 2), and wave w takes items
// w, w + 8.  The next stage's loads are in flight while a stage is decoded
// (two LDS buffers; one barrier per stage orders the copies against the
// reads); with two workgroups per CU one decodes while the other waits.
// After a tile's last phase the 8 partial sums of each row are added in LDS
// in wave order; the results stay in LDS until the workgroup's last stage
// and are then stored with coalesced writes.

struct MxParams {
    const uint8_t *W;
    const float *X;
    float *Y;
    int64_t rows;
    uint64_t w_bytes;     // rows * row_bytes
    int64_t tiles;        // ceil(rows / 32)
    uint32_t row_bytes;
    uint32_t cols;
    uint32_t ximg_bytes;  // nc * record bytes
    uint32_t slot;        // bytes per row segment in a stage buffer (odd multiple of 16)
    uint32_t stage_bytes; // 32 * slot
    uint32_t out_off;     // byte offset of the output buffer in LDS
    int32_t batch;
    int32_t nc;           // chunks per row
    int32_t P;            // chunks per phase
    int32_t nph;          // phases per tile
    int32_t npart;        // parts per chunk (1 or 2)
    int32_t nu;           // 16-byte units copied per row segment
    int32_t nbuf;         // stage buffers (1 or 2)
    int32_t last_nblk;    // 32-column blocks in a row's last chunk (block formats)
    float coff;           // seed factor of the K-quant min term: -2^-24
    // column slices: W and X point at the slice's first column, rows keep
    // their full strides; the slice's sums are added to Y when accumulate
    uint32_t x_stride;    // floats between batch rows of X
    uint32_t x_bytes;     // readable bytes from X
    int32_t accumulate;
};

// ROW16: row_bytes and CHUNK are multiples of 16, so every row segment of a
// stage starts at the weight base's offset mod 16.  RA: some field starts
// at 2 mod 4 in LDS and is realigned.  TLD: 16-byte loads per thread per
// stage (upper bound).
template <class F, int B, bool RA, bool ROW16, int TLD>
__global__ void __launch_bounds__(512) qgemv_mx_kernel(MxParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NB = nb_of(B), REC = ximg_rec(B);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int n = lane & 31, kh = lane >> 5;
    uint8_t *bufs = smem + p.ximg_bytes;
    float *red = (float *)(bufs + p.nbuf * p.stage_bytes);
    float *outb = (float *)(smem + p.out_off);  // [tile k][batch b][32 rows]

    // unit map: load j of this thread copies unit q = tid + 512 j (when
    // q < nq), unit u of row r = q / nu
    const int nq = kRows * p.nu;
    uint32_t s_src[TLD], s_u[TLD], s_dst[TLD];
#pragma unroll
    for (int j = 0; j < TLD; j++) {
        const int q = tid + 512 * j, qq = q < nq ? q : 0;
        const int r = qq / p.nu, u = qq - r * p.nu;
        s_src[j] = ROW16 ? (uint32_t)r * p.row_bytes + 16u * u : (uint32_t)r * p.row_bytes;
        s_u[j] = 16u * u;
        s_dst[j] = (uint32_t)r * p.slot + 16u * u;
    }
    auto tile_rsrc = [&](int64_t t, uint32_t *d0) -> rsrc_t {
        const uint64_t tb = (uint64_t)t * kRows * p.row_bytes;
        const uint8_t *gp = p.W + tb;
        const uint8_t *al = (const uint8_t *)((uintptr_t)gp & ~(uintptr_t)15);
        *d0 = (uint32_t)(gp - al);
        const uint64_t rem = (p.w_bytes - tb + *d0 + 15) & ~(uint64_t)15;
        return make_rsrc(al, rem > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)rem);
    };

    // this workgroup's stages: s -> (tile, phase)
    const int64_t nt = p.tiles > (int64_t)blockIdx.x
                           ? (p.tiles - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
    const int64_t ns = nt * p.nph;
    auto tile_of = [&](int64_t s) { return (int64_t)blockIdx.x + (s / p.nph) * gridDim.x; };

    u32x4 stg[TLD];
    auto issue = [&](int64_t s) {
        uint32_t d0;
        const rsrc_t rs = tile_rsrc(tile_of(s), &d0);
        const uint32_t K0 = (uint32_t)((int)(s % p.nph) * p.P) * F::CHUNK;
#pragma unroll
        for (int j = 0; j < TLD; j++) {
            if (tid + 512 * j < nq) {
                const uint32_t off =
                    ROW16 ? s_src[j] + K0 : ((s_src[j] + K0 + d0) & ~15u) + s_u[j];
                stg[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kStream);
            }
        }
    };

    // A workgroup with one stage starts its weight loads before reading the
    // activations; a streaming one converts the activations first.
    if (p.nbuf == 1) {
        if (ns > 0) issue(0);
        build_ximg<B, F::SEEDS>(p.X, p.cols, p.x_stride, p.x_bytes, p.batch, p.nc, p.coff,
                                F::GW / 4, smem);
    } else {
        build_ximg<B, F::SEEDS>(p.X, p.cols, p.x_stride, p.x_bytes, p.batch, p.nc, p.coff,
                                F::GW / 4, smem);
        if (ns > 0) issue(0);
    }
    const XLane xl = make_xlane<B>(lane);

    float acc[NB];
#pragma unroll
    for (int i = 0; i < NB; i++) acc[i] = 0.f;
    const int items = p.P * p.npart;

    for (int64_t s = 0; s < ns; s++) {
        uint8_t *buf = bufs + (p.nbuf == 2 ? (int)(s & 1) : 0) * p.stage_bytes;
#pragma unroll
        for (int j = 0; j < TLD; j++)
            if (tid + 512 * j < nq) *(u32x4 *)(buf + s_dst[j]) = stg[j];
        if (s + 1 < ns) issue(s + 1);
        __syncthreads();

        const int64_t t = tile_of(s);
        const int ph = (int)(s % p.nph);
        uint32_t d0;
        (void)tile_rsrc(t, &d0);
        const uint32_t K0 = (uint32_t)(ph * p.P) * F::CHUNK;
        const uint32_t delta = ROW16 ? d0 : (((uint32_t)n * p.row_bytes + K0 + d0) & 15u);
        const uint8_t *seg = buf + n * p.slot;
        for (int it = wave; it < items; it += kWaves) {
            const int c = p.npart == 2 ? it >> 1 : it;
            const int ca = ph * p.P + c;
            if (ca >= p.nc) break;
            const int h0 = p.npart == 2 ? (it & 1) : 0, h1 = p.npart == 2 ? h0 + 1 : 2;
            const RowRd<RA> rd = make_rowrd<RA>(seg, delta + (uint32_t)c * F::CHUNK, kh);
            const uint8_t *rec = smem + (size_t)ca * REC;
            float rv[NB];
#pragma unroll
            for (int i = 0; i < NB; i++) rv[i] = 0.f;
            F::template chunk<B, RA>(rd, rec, xl, rv, ca == p.nc - 1 ? p.last_nblk : 8, h0, h1);
            const f32x4 ub = *(const f32x4 *)(rec + xl.e);
#pragma unroll
            for (int i = 0; i < NB; i++) acc[i] = fmaf(ub[i], rv[i], acc[i]);
        }
        if (p.nbuf == 1) __syncthreads();
        if (ph == p.nph - 1) {
            // partial sums of the 8 waves, added in wave order
#pragma unroll
            for (int i = 0; i < NB; i++) red[(wave * 64 + lane) * NB + i] = acc[i];
            __syncthreads();
            if (wave == 0) {
                for (int w = 1; w < kWaves; w++)
#pragma unroll
                    for (int i = 0; i < NB; i++) acc[i] += red[(w * 64 + lane) * NB + i];
                const int k = (int)(s / p.nph);
#pragma unroll
                for (int i = 0; i < NB; i++) {
                    const int b = 4 * kh + i;
                    if (b < B) outb[(k * B + b) * kRows + n] = acc[i];
                }
            }
#pragma unroll
            for (int i = 0; i < NB; i++) acc[i] = 0.f;
            __syncthreads();
        }
    }

    // results of this workgroup's tiles, row-contiguous per batch row
    const int tot = (int)nt * B * kRows;
    for (int idx = tid; idx < tot; idx += 512) {
        const int k = idx / (B * kRows), rem = idx - k * B * kRows;
        const int b = rem / kRows, r = rem - b * kRows;
        const int64_t row = tile_of((int64_t)k * p.nph) * kRows + r;
        if (b < p.batch && row < p.rows) {
            float *y = p.Y + (int64_t)b * p.rows + row;
            *y = p.accumulate ? *y + outb[idx] : outb[idx];
        }
    }
}

}  // namespace mx
}  // namespace qg
