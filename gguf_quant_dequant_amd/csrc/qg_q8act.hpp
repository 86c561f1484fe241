// qg_q8act.hpp -- the int8-activation variant of the batch-1 GEMV: the
// activations are quantised to int8 and every weight code meets them in an
// integer dot product (v_dot4_i32_i8); each 16-column group converts to
// float once.
//
// Web pages: docs.rs, crate ferrox-cuda 0.14.0, src/gpu.rs, module notes
// (llama.cpp's K-quant kernels take an integer dp4a dot product and convert
// to float once per block); docs.rs, ferrox-core 0.16.0, weight_matrix.rs,
// cpu_int_dot_enabled (quantise the activation to int8 and run the integer
// vec_dot; faster, and it perturbs results below the f32 reference's
// precision).  The pages give no layout for the quantised activation; the
// one used here: groups of 16 consecutive columns, d = max|x| / 127,
// id = 1 / d and q = rint(x * id) in f32 (0 for an all-zero group; a group
// holding a non-finite value gets d = NaN).  One division per group.  Every
// lane quantises the groups of its own tile once per kernel: a tile is
// whole 16-column groups in every format at batch 1.
//
// Each format wrapper keeps the format's tile, loads and field decoding and
// replaces the activation tile and the dot product.
#pragma once

#include <cfloat>

#include "qg_formats.hpp"

namespace qg {
namespace q8a {

// int8 codes of the tile's columns (four per dword, in tile order), and per
// 16-column group the scale and the sum of the codes.
template <int CPT>
struct XQ8 {
    uint32_t q[CPT / 4];
    float d[CPT / 16];
    int s[CPT / 16];
};

template <int CPT>
__device__ __forceinline__ void quantize_tile(const float (&x)[CPT], XQ8<CPT> &t) {
#pragma unroll
    for (int g = 0; g < CPT / 16; g++) {
        float amax = 0.f;
        bool fin = true;
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const float a = fabsf(x[16 * g + j]);
            fin = fin && a <= FLT_MAX;
            amax = a > amax ? a : amax;
        }
        const float d = amax / 127.0f;
        const bool zero = !fin || amax == 0.f;
        const float id = zero ? 0.f : 1.0f / d;
        int sum = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            uint32_t packed = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float v = zero ? 0.f : __builtin_rintf(x[16 * g + 4 * k + i] * id);
                v = v > 127.f ? 127.f : (v < -127.f ? -127.f : v);
                const int qi = (int)v;
                sum += qi;
                packed |= ((uint32_t)qi & 0xFFu) << (8 * i);
            }
            t.q[4 * g + k] = packed;
        }
        t.d[g] = fin ? d : __builtin_nanf("");
        t.s[g] = sum;
    }
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

template <class F>
struct Q8A;

// Q4_K / Q5_K, 64-column tiles: run 0 (low nibbles, sub-block 2p) is
// groups 0 and 1, run 1 (high nibbles, sub-block 2p+1) groups 2 and 3.
template <bool RA, bool FIVE>
struct Q8A<FmtK45<32, RA, FIVE>> : FmtK45<32, RA, FIVE> {
    using Base = FmtK45<32, RA, FIVE>;
    using typename Base::Lane;
    using typename Base::Raw;
    static constexpr int CPT = Base::CPT;
    template <int B> using XTile = XQ8<CPT>;
    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        static_assert(B == 1, "batch 1");
        quantize_tile<CPT>(x[0], t);
    }
    template <int B>
    __device__ static void dot(const Raw &w, const Lane &L, const XTile<B> &t, float (&acc)[B]) {
        const float d = f16_lo(w.h[0]), dmin = f16_hi(w.h[0]);
        uint32_t sc, mn;
        kquant_pair_scales(w.h[1], w.h[2], w.h[3], L.p, &sc, &mn);
        int is[4] = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < Base::ND; k++) {
            uint32_t lo = w.q[k] & 0x0F0F0F0Fu, hi = (w.q[k] >> 4) & 0x0F0F0F0Fu;
            if constexpr (FIVE) {
                lo |= ((w.qh[k] >> (2 * L.p)) & 0x01010101u) << 4;
                hi |= ((w.qh[k] >> (2 * L.p + 1)) & 0x01010101u) << 4;
            }
            is[k / 4] = dot4(lo, t.q[k], is[k / 4]);
            is[2 + k / 4] = dot4(hi, t.q[8 + k], is[2 + k / 4]);
        }
        const float ds0 = d * (float)(sc & 0xFFu), ds1 = d * (float)(sc >> 8);
        const float dm0 = dmin * (float)(mn & 0xFFu), dm1 = dmin * (float)(mn >> 8);
        const float q0 = (float)is[0] * t.d[0] + (float)is[1] * t.d[1];
        const float q1 = (float)is[2] * t.d[2] + (float)is[3] * t.d[3];
        const float m0 = (float)t.s[0] * t.d[0] + (float)t.s[1] * t.d[1];
        const float m1 = (float)t.s[2] * t.d[2] + (float)t.s[3] * t.d[3];
        acc[0] += ds0 * q0 + ds1 * q1 - (dm0 * m0 + dm1 * m1);
    }
};

// Q6_K, 64-column tiles of four 16-column runs: run r is group r.  The
// codes are the signed bytes 4 (q - 32) of the format's decoder.
template <>
struct Q8A<FmtQ6K<16, false>> : FmtQ6K<16, false> {
    using Base = FmtQ6K<16, false>;
    template <int B> using XTile = XQ8<CPT>;
    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        static_assert(B == 1, "batch 1");
        quantize_tile<CPT>(x[0], t);
    }
    template <int B>
    __device__ static void dot(const Raw &w, const Lane &L, const XTile<B> &t, float (&acc)[B]) {
        int is[4] = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < ND; k++) {
            uint32_t q[4];
            codes(w, k, q);
#pragma unroll
            for (int r = 0; r < 4; r++) is[r] = dot4(q[r], t.q[4 * r + k], is[r]);
        }
        float sc[4][NG];
        const float d4 = scales(w, L, sc);  // d / 4: the codes carry a factor 4
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < 4; r++) a = fmaf(sc[r][0] * t.d[r], (float)is[r], a);
        acc[0] = fmaf(d4, a, acc[0]);
    }
};

// Q8_0, 32-column tiles (one block): groups 0 and 1.
template <>
struct Q8A<FmtQ80<32>> : FmtQ80<32> {
    template <int B> using XTile = XQ8<CPT>;
    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        static_assert(B == 1, "batch 1");
        quantize_tile<CPT>(x[0], t);
    }
    template <int B>
    __device__ static void dot(const Raw &w, const Lane &, const XTile<B> &t, float (&acc)[B]) {
        int is[2] = {0, 0};
#pragma unroll
        for (int k = 0; k < ND; k++) is[k / 4] = dot4(w.q[k], t.q[k], is[k / 4]);
        acc[0] = fmaf(f16_lo(w.d), (float)is[0] * t.d[0] + (float)is[1] * t.d[1], acc[0]);
    }
};

// Q4_0, 32-column tiles (one block): low nibbles are group 0, high nibbles
// group 1; the value is nibble - 8, so 8 * (sum of the group's codes)
// comes off the integer sum.
template <>
struct Q8A<FmtQ40<16>> : FmtQ40<16> {
    template <int B> using XTile = XQ8<CPT>;
    template <int B>
    __device__ static void prep(const float (&x)[B][CPT], XTile<B> &t) {
        static_assert(B == 1, "batch 1");
        quantize_tile<CPT>(x[0], t);
    }
    template <int B>
    __device__ static void dot(const Raw &w, const Lane &, const XTile<B> &t, float (&acc)[B]) {
        int i0 = 0, i1 = 0;
#pragma unroll
        for (int k = 0; k < ND; k++) {
            i0 = dot4(w.q[k] & 0x0F0F0F0Fu, t.q[k], i0);
            i1 = dot4((w.q[k] >> 4) & 0x0F0F0F0Fu, t.q[4 + k], i1);
        }
        i0 -= 8 * t.s[0];
        i1 -= 8 * t.s[1];
        acc[0] = fmaf(f16_lo(w.d), (float)i0 * t.d[0] + (float)i1 * t.d[1], acc[0]);
    }
};

}  // namespace q8a
}  // namespace qg
