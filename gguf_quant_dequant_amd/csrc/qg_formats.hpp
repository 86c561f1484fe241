// qg_formats.hpp -- per-format lane tiles for the fused dequantise-and-dot
// kernels on gfx950.
//
// A "tile" is the part of one weight row a lane owns: a fixed set of
// columns, the same in every row the lane visits, so the matching
// activations stay in VGPRs for the whole kernel.  Each format struct says
//   CPT     columns per tile; the tile is NRUN runs of RUNLEN consecutive
//           columns, run r starting at column col0(L, r);
//   Lane    per-lane constants derived from the tile index;
//   Raw     the registers one row's tile occupies after loading;
//   load    buffer loads of the tile's bytes for one row;
//   dot     dequantise the tile and accumulate sum_c w[c] * x[b][c] in f32
//           for b < B, into acc[b].
//
// Block layouts (web page: docs.rs, crate ferrox-cuda 0.14.0, source
// src/gpu.rs -- the kernel sources Q8_0_MATVEC_KERNEL_SRC,
// Q4_0_MATVEC_KERNEL_SRC, Q4_K_MATVEC_KERNEL_SRC with ferrox_q4_k_scale_min,
// Q5_K_MATVEC_KERNEL_SRC, Q6_K_MATVEC_KERNEL_SRC):
//   Q8_0  34 B / 32:  f16 d @0, int8 q[32] @2;            w = d*q
//   Q4_0  18 B / 32:  f16 d @0, qs[16] @2, element j low nibble of qs[j],
//                     element j+16 high nibble;           w = d*(nib-8)
//   Q4_K 144 B / 256: f16 d @0, f16 dmin @2, 12 packed 6-bit scale/min
//                     bytes @4, qs[128] @16; element e: sub-block e/32,
//                     nibble ((e%64)/32) of qs[32*(e/64) + e%32];
//                     w = d*sc*q - dmin*m
//   Q5_K 176 B / 256: as Q4_K with qh[32] @16 (bit 2*(e/64)+(e%64)/32 of
//                     qh[e%32] adds 16) and qs @48
//   Q6_K 210 B / 256: ql[128] @0, qh[64] @128, int8 sc[16] @192, f16 d @208;
//                     half h = e/128, t = (e%128)/32, l = e%32: low bits
//                     nibble t/2 of ql[64h + 32(t%2) + l], top bits 2t..2t+1
//                     of qh[32h + l]; w = d*sc[e/16]*(q-32)
//
// Conversions are exact: codes become small integers in f32 (signed codes
// through v_cvt_f32_i32 with byte sign extension, offset codes re-centred
// bitwise first), so the only rounding is in the f32 products and sums.
#pragma once

#include <type_traits>

#include "qg_device.hpp"

namespace qg {

// Activation tile of the f32 decoders: the tile's floats and, for the
// formats with a min term, per-run sums.
template <int CPT, int NSUM, int B>
struct XF32 {
    float x[B][CPT];
    float sx[B][NSUM];
};

template <class F, int B>
__device__ __forceinline__ void prep_f32(const float (&x)[B][F::CPT],
                                         XF32<F::CPT, F::NSUM, B> &t) {
#pragma unroll
    for (int b = 0; b < B; b++) {
#pragma unroll
        for (int c = 0; c < F::CPT; c++) t.x[b][c] = x[b][c];
#pragma unroll
        for (int s = 0; s < F::NSUM; s++) {
            float a = 0.f;
            if constexpr (F::NEEDS_SUM) {
#pragma unroll
                for (int j = 0; j < F::RUNLEN; j++) a += x[b][s * F::RUNLEN + j];
            }
            t.sx[b][s] = a;
        }
    }
}

// Activation tile as base-256 digits, for exact integer dot products.
// Each run of RUNLEN columns gets its own power-of-two scale 2^s, chosen so
// that the largest |x| * 2^s lies in [2^21, 2^22).  X = rint(x * 2^s) (the
// scaling is exact, the rounding is to nearest, so |X - x 2^s| <= 1/2) is
// split into digits X = 65536 p2 + 256 p1 + p0 with p0, p1 in [-128, 127]
// and |p2| <= 64.  Plane k holds digit k of four consecutive columns per
// dword (column c in byte c % 4), so v_dot4 of four int8 codes with a plane
// dword is an exact partial sum.  f = 2^-s, or NaN when the run holds a
// non-finite value.  Error: every activation is represented to within
// 2^-s / 2 <= 2^-22 max|x| of the run, so a run's product sum is off by at
// most 2^-22 * max|x| * sum |w| over the run (w the dequantised weights).
template <int CPT, int NRUN, int B>
struct XI8 {
    uint32_t p[B][3][CPT / 4];
    float f[B][NRUN];
};

template <int RL>
__device__ __forceinline__ void digits_run(const float *x, uint32_t *p0, uint32_t *p1,
                                           uint32_t *p2, float *f) {
    uint32_t mb = 0;
#pragma unroll
    for (int j = 0; j < RL; j++) {
        const uint32_t a = __builtin_bit_cast(uint32_t, x[j]) & 0x7FFFFFFFu;
        mb = a > mb ? a : mb;
    }
    // frexp exponent e: max in [2^(e-1), 2^e); 0 for a zero maximum
    int s = 22 - __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, mb));
    s = s > 126 ? 126 : s;
    const float up = __builtin_bit_cast(float, (uint32_t)(s + 127) << 23);
    *f = mb < 0x7F800000u ? __builtin_bit_cast(float, (uint32_t)(127 - s) << 23)
                          : __builtin_nanf("");
#pragma unroll
    for (int q = 0; q < RL / 4; q++) {
        // y = X + 0x8080: bytes 0 and 1 of y are p0 + 128 and p1 + 128,
        // byte 2 (sign-extended) is p2
        uint32_t y[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            y[i] = (uint32_t)((int)__builtin_rintf(x[4 * q + i] * up) + 32896);
        const uint32_t a = __builtin_amdgcn_perm(y[1], y[0], 0x05040100u);
        const uint32_t b = __builtin_amdgcn_perm(y[3], y[2], 0x05040100u);
        p0[q] = __builtin_amdgcn_perm(b, a, 0x06040200u) ^ 0x80808080u;
        p1[q] = __builtin_amdgcn_perm(b, a, 0x07050301u) ^ 0x80808080u;
        const uint32_t c = __builtin_amdgcn_perm(y[1], y[0], 0x0C0C0602u);
        const uint32_t e = __builtin_amdgcn_perm(y[3], y[2], 0x0C0C0602u);
        p2[q] = __builtin_amdgcn_perm(e, c, 0x05040100u);
    }
}

// Sum of an exact digit-plane dot product: 65536 s2 + 256 s1 + s0, rounded
// once to f32.
__device__ __forceinline__ float digits_sum(int s0, int s1, int s2) {
    return fmaf((float)((s2 << 8) + s1), 256.0f, (float)s0);
}


// ---------------------------------------------------------------- Q4_K / Q5_K
//
// Tile = (super-block sb, pair p of sub-blocks 2p and 2p+1, byte range
// [l0, l0+LW) of the 32 quant bytes of that pair): low nibbles are columns
// 256sb + 64p + l0 + i (sub-block 2p), high nibbles the same + 32
// (sub-block 2p+1).  LW in {8, 16, 32}.

// Unpack (sc, m) of sub-blocks 2p and 2p+1 from header dwords h1 = S[0..3],
// h2 = S[4..7], h3 = S[8..11] (see ferrox_q4_k_scale_min): returns
// sc(2p) | sc(2p+1) << 8 in *sc and the same for the mins in *mn.
__device__ __forceinline__ void kquant_pair_scales(uint32_t h1, uint32_t h2, uint32_t h3, int p,
                                                   uint32_t *sc, uint32_t *mn) {
    const uint32_t sh = (p & 1) ? 16u : 0u;
    const uint32_t a = h1 >> sh, b = h2 >> sh, c = h3 >> sh;
    if (p < 2) {
        *sc = a & 0x3F3Fu;
        *mn = b & 0x3F3Fu;
    } else {
        *sc = (c & 0x0F0Fu) | ((a >> 2) & 0x3030u);
        *mn = ((c >> 4) & 0x0F0Fu) | ((b >> 2) & 0x3030u);
    }
}

template <int LW, bool RA, bool FIVE>
struct FmtK45 {
    static_assert(LW == 8 || LW == 16 || LW == 32, "tile width");
    static constexpr int QK = 256;
    static constexpr int BB = FIVE ? 176 : 144;
    static constexpr int QS_OFF = FIVE ? 48 : 16;
    static constexpr int CPT = 2 * LW;
    static constexpr int NRUN = 2, RUNLEN = LW;
    static constexpr int NSUM = 2;           // per-run sums of x (min term)
    static constexpr bool NEEDS_SUM = true;
    static constexpr int TPS = 4 * (32 / LW);  // tiles per super-block
    static constexpr int ND = LW / 4;        // quant dwords per tile

    struct Lane {
        uint32_t hoff, qoff, qhoff;
        int p, col0;
    };
    __device__ static Lane init(int t) {
        const int sb = t / TPS, w = t % TPS;
        const int p = w / (32 / LW), l0 = (w % (32 / LW)) * LW;
        Lane L;
        L.hoff = (uint32_t)(sb * BB);
        L.qoff = (uint32_t)(sb * BB + QS_OFF + 32 * p + l0);
        L.qhoff = (uint32_t)(sb * BB + 16 + l0);
        L.p = p;
        L.col0 = sb * QK + 64 * p + l0;
        return L;
    }
    __device__ static int col0(const Lane &L, int run) { return L.col0 + 32 * run; }

    struct Raw {
        uint32_t h[4];
        uint32_t q[ND];
        uint32_t qh[FIVE ? ND : 1];
    };
    template <class Rd>
    __device__ static void load(const Rd &r, uint32_t row, const Lane &L, Raw &w) {
        r.template span<4, RA>(row + L.hoff, w.h);
        if constexpr (FIVE) r.template span<ND, RA>(row + L.qhoff, w.qh);
        r.template span<ND, RA>(row + L.qoff, w.q);
    }

    template <int B> using XTile = XF32<CPT, NSUM, B>;
    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        prep_f32<FmtK45, B>(x, t);
    }

    template <int B>
    __device__ static void dot(const Raw &w, const Lane &L, const XTile<B> &t,
                               float (&acc)[B]) {
        const auto &x = t.x;
        const auto &sx = t.sx;
        const float d = f16_lo(w.h[0]), dmin = f16_hi(w.h[0]);
        uint32_t sc, mn;
        kquant_pair_scales(w.h[1], w.h[2], w.h[3], L.p, &sc, &mn);
        float alo[B], ahi[B];
#pragma unroll
        for (int b = 0; b < B; b++) alo[b] = ahi[b] = 0.f;
#pragma unroll
        for (int k = 0; k < ND; k++) {
            uint32_t lo, hi;
            if constexpr (FIVE) {
                const uint32_t bl = (w.qh[k] >> (2 * L.p)) & 0x01010101u;
                const uint32_t bh = (w.qh[k] >> (2 * L.p + 1)) & 0x01010101u;
                lo = opaque((w.q[k] & 0x0F0F0F0Fu) | (bl << 4));
                hi = opaque(((w.q[k] >> 4) & 0x0F0F0F0Fu) | (bh << 4));
            } else {
                lo = opaque(w.q[k] & 0x0F0F0F0Fu);
                hi = opaque(w.q[k] & 0xF0F0F0F0u);  // 16 * nibble
            }
            const float l[4] = {ubyte<0>(lo), ubyte<1>(lo), ubyte<2>(lo), ubyte<3>(lo)};
            const float h[4] = {ubyte<0>(hi), ubyte<1>(hi), ubyte<2>(hi), ubyte<3>(hi)};
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int b = 0; b < B; b++) {
                    alo[b] = fmaf(l[j], x[b][4 * k + j], alo[b]);
                    ahi[b] = fmaf(h[j], x[b][LW + 4 * k + j], ahi[b]);
                }
        }
        const float hscale = FIVE ? 1.0f : 0.0625f;
        const float ds0 = d * (float)(sc & 0xFFu), ds1 = d * (float)(sc >> 8) * hscale;
        const float dm0 = dmin * (float)(mn & 0xFFu), dm1 = dmin * (float)(mn >> 8);
#pragma unroll
        for (int b = 0; b < B; b++)
            acc[b] += ds0 * alo[b] + ds1 * ahi[b] - (dm0 * sx[b][0] + dm1 * sx[b][1]);
    }
};

template <int LW, bool RA> using FmtQ4K = FmtK45<LW, RA, false>;
template <int LW, bool RA> using FmtQ5K = FmtK45<LW, RA, true>;

// ------------------------------------------------------------------- Q6_K
//
// Tile = (super-block sb, half h, byte range [l0, l0+LW) of the 32-byte
// groups): run t (t = 0..3) is columns 256sb + 128h + 32t + l0 + i.  Its
// codes come from ql[64h + l0 + i] (t = 0 low nibble, t = 2 high nibble),
// ql[64h + 32 + l0 + i] (t = 1 low, t = 3 high) and bits 2t..2t+1 of
// qh[32h + l0 + i].  Scale of run t, element i: sc[8h + 2t + (l0+i)/16].
// LW in {4, 8, 16, 32}.  Blocks are 210 B, so every span is realigned.

template <int LW, bool IX = true>
struct FmtQ6K {
    static_assert(LW == 4 || LW == 8 || LW == 16 || LW == 32, "tile width");
    static constexpr int QK = 256, BB = 210;
    static constexpr int CPT = 4 * LW;
    static constexpr int NRUN = 4, RUNLEN = LW;
    static constexpr int NSUM = 1;            // unused
    static constexpr bool NEEDS_SUM = false;
    static constexpr int TPS = 2 * (32 / LW);
    static constexpr int ND = LW / 4;
    static constexpr int NG = LW == 32 ? 2 : 1;  // scale groups per run

    struct Lane {
        uint32_t qa, qb, qh, sc, d;
        uint32_t sbyte0;  // index of run 0's first scale inside sc[8h..8h+7]
        int col0;
    };
    __device__ static Lane init(int t) {
        const int sb = t / TPS, w = t % TPS;
        const int h = w / (32 / LW), l0 = (w % (32 / LW)) * LW;
        const int blk = sb * BB;
        Lane L;
        L.qa = (uint32_t)(blk + 64 * h + l0);
        L.qb = L.qa + 32u;
        L.qh = (uint32_t)(blk + 128 + 32 * h + l0);
        L.sc = (uint32_t)(blk + 192 + 8 * h);
        L.d = (uint32_t)(blk + 208);
        L.sbyte0 = (uint32_t)(l0 / 16);
        L.col0 = sb * QK + 128 * h + l0;
        return L;
    }
    __device__ static int col0(const Lane &L, int run) { return L.col0 + 32 * run; }

    struct Raw {
        uint32_t a[ND], b[ND], h[ND];
        uint32_t sc[2];
        uint32_t d;
    };
    template <class Rd>
    __device__ static void load(const Rd &r, uint32_t row, const Lane &L, Raw &w) {
        r.template span<ND, true>(row + L.qa, w.a);
        r.template span<ND, true>(row + L.qb, w.b);
        r.template span<ND, true>(row + L.qh, w.h);
        r.template span<2, true>(row + L.sc, w.sc);
        w.d = r.u16(row + L.d);
    }

    // Codes of runs 0..3 for quant dword k, each as the signed byte 4*(q-32):
    // the low four bits go to bits 2..5 and the two top bits to bits 6..7
    // with their upper bit flipped (qh ^ 0xAA once per dword), so that the
    // byte read as two's complement is 4*q - 128.
    __device__ static void codes(const Raw &w, int k, uint32_t (&q)[4]) {
        const uint32_t a = w.a[k], bq = w.b[k], hx = w.h[k] ^ 0xAAAAAAAAu;
        q[0] = opaque(((a << 2) & 0x3C3C3C3Cu) | ((hx << 6) & 0xC0C0C0C0u));
        q[1] = opaque(((bq << 2) & 0x3C3C3C3Cu) | ((hx << 4) & 0xC0C0C0C0u));
        q[2] = opaque(((a >> 2) & 0x3C3C3C3Cu) | ((hx << 2) & 0xC0C0C0C0u));
        q[3] = opaque(((bq >> 2) & 0x3C3C3C3Cu) | (hx & 0xC0C0C0C0u));
    }

    // d / 4 (the codes carry a factor 4) and the sub-block scale of run r,
    // group g: byte 2r + g + l0/16 of sc[8h..8h+7]
    __device__ static float scales(const Raw &w, const Lane &L, float (&sc)[4][NG]) {
        const uint32_t s0 = w.sc[0] >> (8 * L.sbyte0), s1 = w.sc[1] >> (8 * L.sbyte0);
        if constexpr (NG == 1) {
            sc[0][0] = sbyte<0>(s0);
            sc[1][0] = sbyte<2>(s0);
            sc[2][0] = sbyte<0>(s1);
            sc[3][0] = sbyte<2>(s1);
        } else {
            sc[0][0] = sbyte<0>(w.sc[0]);
            sc[0][1] = sbyte<1>(w.sc[0]);
            sc[1][0] = sbyte<2>(w.sc[0]);
            sc[1][1] = sbyte<3>(w.sc[0]);
            sc[2][0] = sbyte<0>(w.sc[1]);
            sc[2][1] = sbyte<1>(w.sc[1]);
            sc[3][0] = sbyte<2>(w.sc[1]);
            sc[3][1] = sbyte<3>(w.sc[1]);
        }
        return f16_lo(w.d) * 0.25f;
    }

    // IX: activations as digit planes and v_dot4 on the codes (the products
    // accumulate exactly in int32 per run and scale group); otherwise f32
    // activations and one FMA per code.  The planes cost a conversion of
    // the tile once per kernel, which pays off when a lane visits many rows.
    template <int B>
    using XTile = std::conditional_t<IX, XI8<CPT, NRUN, B>, XF32<CPT, NSUM, B>>;

    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        if constexpr (IX) {
#pragma unroll
            for (int b = 0; b < B; b++)
#pragma unroll
                for (int r = 0; r < NRUN; r++)
                    digits_run<RUNLEN>(&x[b][r * RUNLEN], &t.p[b][0][r * ND], &t.p[b][1][r * ND],
                                       &t.p[b][2][r * ND], &t.f[b][r]);
        } else {
            prep_f32<FmtQ6K, B>(x, t);
        }
    }

    template <int B>
    __device__ static void dot(const Raw &w, const Lane &L, const XTile<B> &t,
                               float (&acc)[B]) {
        if constexpr (IX) {
            int s0[4][NG][B], s1[4][NG][B], s2[4][NG][B];
#pragma unroll
            for (int r = 0; r < 4; r++)
#pragma unroll
                for (int g = 0; g < NG; g++)
#pragma unroll
                    for (int b = 0; b < B; b++) s0[r][g][b] = s1[r][g][b] = s2[r][g][b] = 0;
#pragma unroll
            for (int k = 0; k < ND; k++) {
                uint32_t q[4];
                codes(w, k, q);
                const int g = (4 * k) / 16 < NG ? (4 * k) / 16 : 0;
#pragma unroll
                for (int r = 0; r < 4; r++)
#pragma unroll
                    for (int b = 0; b < B; b++) {
                        const int qi = (int)q[r], o = r * ND + k;
                        s0[r][g][b] = __builtin_amdgcn_sdot4(qi, (int)t.p[b][0][o], s0[r][g][b], false);
                        s1[r][g][b] = __builtin_amdgcn_sdot4(qi, (int)t.p[b][1][o], s1[r][g][b], false);
                        s2[r][g][b] = __builtin_amdgcn_sdot4(qi, (int)t.p[b][2][o], s2[r][g][b], false);
                    }
            }
            float sc[4][NG];
            const float d = scales(w, L, sc);
#pragma unroll
            for (int r = 0; r < 4; r++)
#pragma unroll
                for (int g = 0; g < NG; g++) {
                    const float ds = d * sc[r][g];
#pragma unroll
                    for (int b = 0; b < B; b++)
                        acc[b] = fmaf(ds * t.f[b][r],
                                      digits_sum(s0[r][g][b], s1[r][g][b], s2[r][g][b]), acc[b]);
                }
        } else {
            float at[4][NG][B];
#pragma unroll
            for (int r = 0; r < 4; r++)
#pragma unroll
                for (int g = 0; g < NG; g++)
#pragma unroll
                    for (int b = 0; b < B; b++) at[r][g][b] = 0.f;
#pragma unroll
            for (int k = 0; k < ND; k++) {
                uint32_t q[4];
                codes(w, k, q);
                const int g = (4 * k) / 16 < NG ? (4 * k) / 16 : 0;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float f[4] = {sbyte<0>(q[r]), sbyte<1>(q[r]), sbyte<2>(q[r]),
                                        sbyte<3>(q[r])};
#pragma unroll
                    for (int j = 0; j < 4; j++)
#pragma unroll
                        for (int b = 0; b < B; b++)
                            at[r][g][b] = fmaf(f[j], t.x[b][r * LW + 4 * k + j], at[r][g][b]);
                }
            }
            float sc[4][NG];
            const float d = scales(w, L, sc);
#pragma unroll
            for (int r = 0; r < 4; r++)
#pragma unroll
                for (int g = 0; g < NG; g++) {
                    const float ds = d * sc[r][g];
#pragma unroll
                    for (int b = 0; b < B; b++) acc[b] = fmaf(ds, at[r][g][b], acc[b]);
                }
        }
    }
};

// ------------------------------------------------------------------- Q8_0
//
// Tile = LW consecutive codes of one block (LW in {8, 16, 32}): columns
// 32blk + o + i.

template <int LW>
struct FmtQ80 {
    static_assert(LW == 8 || LW == 16 || LW == 32, "tile width");
    static constexpr int QK = 32, BB = 34;
    static constexpr int CPT = LW;
    static constexpr int NRUN = 1, RUNLEN = LW;
    static constexpr int NSUM = 1;  // unused
    static constexpr bool NEEDS_SUM = false;
    static constexpr int TPB = 32 / LW;
    static constexpr int ND = LW / 4;

    struct Lane {
        uint32_t q, d;
        int col0;
    };
    __device__ static Lane init(int t) {
        const int blk = t / TPB, o = (t % TPB) * LW;
        Lane L;
        L.q = (uint32_t)(blk * BB + 2 + o);
        L.d = (uint32_t)(blk * BB);
        L.col0 = blk * QK + o;
        return L;
    }
    __device__ static int col0(const Lane &L, int) { return L.col0; }

    struct Raw {
        uint32_t q[ND];
        uint32_t d;
    };
    template <class Rd>
    __device__ static void load(const Rd &r, uint32_t row, const Lane &L, Raw &w) {
        r.template span<ND, true>(row + L.q, w.q);
        w.d = r.u16(row + L.d);
    }

    template <int B> using XTile = XF32<CPT, NSUM, B>;
    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        prep_f32<FmtQ80, B>(x, t);
    }

    template <int B>
    __device__ static void dot(const Raw &w, const Lane &, const XTile<B> &t,
                               float (&acc)[B]) {
        const auto &x = t.x;
        float a[B];
#pragma unroll
        for (int b = 0; b < B; b++) a[b] = 0.f;
#pragma unroll
        for (int k = 0; k < ND; k++) {
            const uint32_t v = w.q[k];
            const float f[4] = {sbyte<0>(v), sbyte<1>(v), sbyte<2>(v), sbyte<3>(v)};
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int b = 0; b < B; b++) a[b] = fmaf(f[j], x[b][4 * k + j], a[b]);
        }
        const float d = f16_lo(w.d);
#pragma unroll
        for (int b = 0; b < B; b++) acc[b] = fmaf(d, a[b], acc[b]);
    }
};

// ------------------------------------------------------------------- Q4_0
//
// Tile = quant bytes [o, o+LW) of one block (LW in {8, 16}): low nibbles
// are columns 32blk + o + i, high nibbles 32blk + 16 + o + i.

template <int LW>
struct FmtQ40 {
    static_assert(LW == 8 || LW == 16, "tile width");
    static constexpr int QK = 32, BB = 18;
    static constexpr int CPT = 2 * LW;
    static constexpr int NRUN = 2, RUNLEN = LW;
    static constexpr int NSUM = 1;  // unused
    static constexpr bool NEEDS_SUM = false;
    static constexpr int TPB = 16 / LW;
    static constexpr int ND = LW / 4;

    struct Lane {
        uint32_t q, d;
        int col0;
    };
    __device__ static Lane init(int t) {
        const int blk = t / TPB, o = (t % TPB) * LW;
        Lane L;
        L.q = (uint32_t)(blk * BB + 2 + o);
        L.d = (uint32_t)(blk * BB);
        L.col0 = blk * QK + o;
        return L;
    }
    __device__ static int col0(const Lane &L, int run) { return L.col0 + 16 * run; }

    struct Raw {
        uint32_t q[ND];
        uint32_t d;
    };
    template <class Rd>
    __device__ static void load(const Rd &r, uint32_t row, const Lane &L, Raw &w) {
        r.template span<ND, true>(row + L.q, w.q);
        w.d = r.u16(row + L.d);
    }

    template <int B> using XTile = XF32<CPT, NSUM, B>;
    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        prep_f32<FmtQ40, B>(x, t);
    }

    template <int B>
    __device__ static void dot(const Raw &w, const Lane &, const XTile<B> &t,
                               float (&acc)[B]) {
        const auto &x = t.x;
        // nibble ^ 8 is nibble - 8 in 4-bit two's complement; moved to the
        // top of its byte it converts as the signed byte 16 * (nibble - 8)
        float a[B];
#pragma unroll
        for (int b = 0; b < B; b++) a[b] = 0.f;
#pragma unroll
        for (int k = 0; k < ND; k++) {
            const uint32_t v = w.q[k] ^ 0x88888888u;
            const uint32_t lo = opaque((v << 4) & 0xF0F0F0F0u);
            const uint32_t hi = opaque(v & 0xF0F0F0F0u);
            const float l[4] = {sbyte<0>(lo), sbyte<1>(lo), sbyte<2>(lo), sbyte<3>(lo)};
            const float h[4] = {sbyte<0>(hi), sbyte<1>(hi), sbyte<2>(hi), sbyte<3>(hi)};
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int b = 0; b < B; b++) {
                    a[b] = fmaf(l[j], x[b][4 * k + j], a[b]);
                    a[b] = fmaf(h[j], x[b][LW + 4 * k + j], a[b]);
                }
        }
        const float d = f16_lo(w.d) * 0.0625f;
#pragma unroll
        for (int b = 0; b < B; b++) acc[b] = fmaf(d, a[b], acc[b]);
    }
};

// -------------------------------------------------------------------- F32
//
// Tile = LW consecutive floats (LW in {8, 16, 32}).

template <int LW>
struct FmtF32 {
    static constexpr int QK = 1, BB = 4;
    static constexpr int CPT = LW;
    static constexpr int NRUN = 1, RUNLEN = LW;
    static constexpr int NSUM = 1;  // unused
    static constexpr bool NEEDS_SUM = false;
    static constexpr int ND = LW;

    struct Lane {
        uint32_t off;
        int col0;
    };
    __device__ static Lane init(int t) {
        Lane L;
        L.off = (uint32_t)(t * LW * 4);
        L.col0 = t * LW;
        return L;
    }
    __device__ static int col0(const Lane &L, int) { return L.col0; }

    struct Raw {
        uint32_t v[ND];
    };
    template <class Rd>
    __device__ static void load(const Rd &r, uint32_t row, const Lane &L, Raw &w) {
        r.template dw<ND>(row + L.off, w.v);
    }

    template <int B> using XTile = XF32<CPT, NSUM, B>;
    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        prep_f32<FmtF32, B>(x, t);
    }

    template <int B>
    __device__ static void dot(const Raw &w, const Lane &, const XTile<B> &t,
                               float (&acc)[B]) {
        const auto &x = t.x;
#pragma unroll
        for (int i = 0; i < ND; i++) {
            const float f = __builtin_bit_cast(float, w.v[i]);
#pragma unroll
            for (int b = 0; b < B; b++) acc[b] = fmaf(f, x[b][i], acc[b]);
        }
    }
};

// Activations of one tile: x[b][run * RUNLEN + j] = X[b * xstride +
// col0(L, run) + j] read through the buffer resource rx (4-byte-aligned
// dword loads).  Lanes without a tile hold zeros.
template <class F, int B>
__device__ __forceinline__ void load_tile_x(rsrc_t rx, uint32_t xstride,
                                            const typename F::Lane &L, bool active,
                                            float (&x)[B][F::CPT]) {
#pragma unroll
    for (int b = 0; b < B; b++) {
#pragma unroll
        for (int r = 0; r < F::NRUN; r++) {
            uint32_t v[F::RUNLEN];
            if (active) {
                load_dw<F::RUNLEN>(rx, 4u * (b * xstride + (uint32_t)F::col0(L, r)), v);
            } else {
#pragma unroll
                for (int j = 0; j < F::RUNLEN; j++) v[j] = 0u;
            }
#pragma unroll
            for (int j = 0; j < F::RUNLEN; j++)
                x[b][r * F::RUNLEN + j] = __builtin_bit_cast(float, v[j]);
        }
    }
}

}  // namespace qg
