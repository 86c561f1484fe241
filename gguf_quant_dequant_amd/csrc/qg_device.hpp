// qg_device.hpp -- device helpers for the gfx950 GEMV and MoE kernels:
// buffer-resource loads that realign 2-byte-aligned fields, f16 decode,
// byte-to-float conversions and wave-level reductions.
//
// Every weight byte is read through a raw buffer resource whose base is the
// 4-byte-aligned address at or below the first byte a workgroup needs and
// whose record count ends exactly at the end of the weight array.  Loads are
// always issued at 4-byte-aligned offsets at or above the base; a load that
// starts at or beyond the end of the array is out of range and reads as zero
// without touching memory, and every dword that is read shares a page with
// at least one byte of the array.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kWave = 64;

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// Keeps the optimiser from re-deriving a masked value byte by byte, so that
// byte extraction maps onto v_cvt_f32_ubyte{0..3}.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// Cache policy of the coalesced weight streams (the staged copies, where a
// wave instruction reads whole consecutive lines): non-temporal (the nt
// bit).  Every weight byte is read once per launch.  Measured with cold
// weights: Q4_K 4096 x 4096 5.78 -> 5.46 us, Q6_K 151936 x 2048 51.5 ->
// 49.4 us.  Per-lane tile loads (BufReader) keep the default policy: there
// neighbouring lanes read parts of the same lines, and with nt the MoE
// chain went from 25.0 to 28.9 us per token.
constexpr int kStream = 2;

// n consecutive dwords from a 4-byte-aligned buffer offset (cache policy AUX).
template <int N, int AUX = 0>
__device__ __forceinline__ void load_dw(rsrc_t r, uint32_t off, uint32_t *out) {
    int i = 0;
#pragma unroll
    for (; i + 4 <= N; i += 4) {
        auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, AUX);
        out[i] = v[0]; out[i + 1] = v[1]; out[i + 2] = v[2]; out[i + 3] = v[3];
    }
    if constexpr (N % 4 == 3) {
        auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 4 * i, 0, AUX);
        out[i] = v[0]; out[i + 1] = v[1]; out[i + 2] = v[2];
    } else if constexpr (N % 4 == 2) {
        auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * i, 0, AUX);
        out[i] = v[0]; out[i + 1] = v[1];
    } else if constexpr (N % 4 == 1) {
        out[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, AUX);
    }
}

// N dwords of a byte span starting at a 2-byte-aligned offset.  With
// REALIGN the window starts at off & ~3: N dwords are read with wide loads
// (they never reach past the span's last byte) and one more dword with a
// load of its own; each output dword is then assembled with v_perm_b32 from
// a pair of window dwords (bytes 2..5 of the pair when off is 2 mod 4,
// bytes 0..3 when off is 0 mod 4).  The extra dword either straddles the
// span's end, or starts past it, where it is part of the array or starts
// out of range (read as zero, no memory access).  Without REALIGN off must
// be a multiple of 4.
template <int N, bool REALIGN, int AUX = 0>
__device__ __forceinline__ void load_span(rsrc_t r, uint32_t off, uint32_t *out) {
    if constexpr (!REALIGN) {
        load_dw<N, AUX>(r, off, out);
    } else {
        uint32_t w[N + 1];
        const uint32_t base = off & ~3u;
        load_dw<N, AUX>(r, base, w);
        w[N] = __builtin_amdgcn_raw_buffer_load_b32(r, base + 4u * N, 0, AUX);
        const uint32_t sel = (off & 2u) ? 0x05040302u : 0x03020100u;
#pragma unroll
        for (int i = 0; i < N; i++) out[i] = __builtin_amdgcn_perm(w[i + 1], w[i], sel);
    }
}

// Readers of weight bytes.  The format decoders are written against this
// interface so the same code reads fields straight from global memory
// (buffer loads) or from a copy of the rows staged in LDS.
struct BufReader {
    rsrc_t r;
    template <int N>
    __device__ __forceinline__ void dw(uint32_t off, uint32_t *out) const { load_dw<N>(r, off, out); }
    template <int N, bool REALIGN>
    __device__ __forceinline__ void span(uint32_t off, uint32_t *out) const {
        load_span<N, REALIGN>(r, off, out);
    }
    __device__ __forceinline__ uint32_t u16(uint32_t off) const {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
};

// Bytes staged in LDS: `base` is 16-byte aligned and byte offsets keep the
// same value mod 4 as in global memory, so the same realignment applies.
// Every read is of whole aligned dwords.
struct LdsReader {
    const uint32_t *base;
    template <int N>
    __device__ __forceinline__ void dw(uint32_t off, uint32_t *out) const {
        const uint32_t *p = base + (off >> 2);
#pragma unroll
        for (int i = 0; i < N; i++) out[i] = p[i];
    }
    template <int N, bool REALIGN>
    __device__ __forceinline__ void span(uint32_t off, uint32_t *out) const {
        const uint32_t *p = base + (off >> 2);
        if constexpr (!REALIGN) {
#pragma unroll
            for (int i = 0; i < N; i++) out[i] = p[i];
        } else {
            uint32_t w[N + 1];
#pragma unroll
            for (int i = 0; i <= N; i++) w[i] = p[i];
            const uint32_t sel = (off & 2u) ? 0x05040302u : 0x03020100u;
#pragma unroll
            for (int i = 0; i < N; i++) out[i] = __builtin_amdgcn_perm(w[i + 1], w[i], sel);
        }
    }
    __device__ __forceinline__ uint32_t u16(uint32_t off) const {
        const uint32_t v = base[off >> 2];
        return (off & 2u) ? (v >> 16) : (v & 0xFFFFu);
    }
};

// A little-endian 16-bit field at a 2-byte-aligned offset.
__device__ __forceinline__ uint32_t load_u16(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// IEEE binary16 bits (low 16 bits of v) to f32, by the hardware convert.
__device__ __forceinline__ float f16_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}

// Byte j of v as an unsigned / signed value converted to f32.
template <int J>
__device__ __forceinline__ float ubyte(uint32_t v) {
    return (float)((v >> (8 * J)) & 0xFFu);
}
template <int J>
__device__ __forceinline__ float sbyte(uint32_t v) {
    return (float)(int8_t)(v >> (8 * J));
}

// --------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t swz16_u(uint32_t v) {
    // ds_swizzle bit mode: and 0x1F, or 0, xor 0x10 (within 32-lane halves)
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}
__device__ __forceinline__ float xor16_f(float v) {
    // ds_swizzle bit mode: and 0x1F, or 0, xor 0x10 (within 32-lane halves)
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                 0x401F));
}
__device__ __forceinline__ float xor32_f(float v) {
    const int lane = __lane_id();
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2,
                                                                  __builtin_bit_cast(int, v)));
}

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of
// a group receives the group sum.  The tree is fixed, so results do not
// depend on scheduling.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (W >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
    if constexpr (W >= 16) v += dpp_f<0x140>(v); // row_mirror
    if constexpr (W >= 32) v += xor16_f(v);
    if constexpr (W >= 64) v += xor32_f(v);
    return v;
}

template <int W, int N>
__device__ __forceinline__ void group_sum_all(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; i++) v[i] = group_sum<W>(v[i]);
}

// group_sum over an array with a width known only at run time (uniform
// across the workgroup): one scalar branch picks the compile-time tree.
template <int N>
__device__ __forceinline__ void group_sum_all(float (&v)[N], int width) {
    switch (width) {
    case 2: group_sum_all<2>(v); break;
    case 4: group_sum_all<4>(v); break;
    case 8: group_sum_all<8>(v); break;
    case 16: group_sum_all<16>(v); break;
    case 32: group_sum_all<32>(v); break;
    case 64: group_sum_all<64>(v); break;
    default: break;
    }
}

__device__ __forceinline__ double shfl_xor_d(double v, int mask) {
    const int lane = __lane_id();
    const long long bits = __builtin_bit_cast(long long, v);
    int lo = (int)(bits & 0xFFFFFFFFll), hi = (int)(bits >> 32);
    lo = __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, lo);
    hi = __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, hi);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ int shfl_xor_i(int v, int mask) {
    const int lane = __lane_id();
    return __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, v);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += shfl_xor_d(v, m);
    return v;
}

}  // namespace qg
