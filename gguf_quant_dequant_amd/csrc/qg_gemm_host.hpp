// qg_gemm_host.hpp -- planning and launch of the batched matrix-core kernel
// (gm::qgemm_kernel); instantiated per batch block count in qg_gemm_b<NB>.hip.
#pragma once

#include "qg_gemm.hpp"
#include "qg_host.hpp"

// Waves per tile along the columns (0: chosen from the shape).
#ifndef QG_GEMM_KS
#define QG_GEMM_KS 0
#endif
// 1: at most 8 batch rows run on gm::qgemm8_kernel (packed hi and lo parts,
// both streams two chunks ahead).
#ifndef QG_GEMM8
#define QG_GEMM8 1
#endif

namespace qg {
namespace host {

// 16-byte units staged per row segment of a chunk: the chunk's bytes plus
// up to 15 bytes of leading misalignment.
constexpr int gemm_nu(int chunk) { return (chunk + 15 + 15) / 16; }
constexpr int gemm_units(int chunk) { return (16 * gemm_nu(chunk) + 63) / 64; }

template <class F, int NB, bool RA>
int launch_gemm_t(const gm::GemmParams &p, int grid, size_t lds, hipStream_t st) {
    constexpr int U = gemm_units(F::CHUNK);
    if constexpr (NB == 1) {
        if (QG_GEMM8 && p.batch <= 8) {
            hipLaunchKernelGGL((gm::qgemm8_kernel<F, RA, U>), dim3(grid), dim3(64 * gm::kWaves),
                               lds, st, p);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return fail(QG_ELAUNCH, "qgemv: launch failed: %s", hipGetErrorString(e));
            return QG_OK;
        }
    }
    hipLaunchKernelGGL((gm::qgemm_kernel<F, NB, RA, U>), dim3(grid), dim3(64 * gm::kWaves), lds,
                       st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ELAUNCH, "qgemv: launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

template <class F, int NB>
int launch_gemm(const void *W, int64_t rows, int64_t cols, const float *X, float *Y, int batch,
                int64_t rb, hipStream_t st) {
    gm::GemmParams p{};
    p.W = (const uint8_t *)W;
    p.X = X;
    p.Y = Y;
    p.rows = rows;
    p.w_bytes = (uint64_t)rows * (uint64_t)rb;
    p.row_bytes = (uint32_t)rb;
    p.cols = (uint32_t)cols;
    p.batch = batch;
    p.nchunks = (int32_t)((cols + gm::kChunk - 1) / gm::kChunk);
    p.last_nkb = (int32_t)(((cols - 1) % gm::kChunk) / 32 + 1);
    p.tiles = (int32_t)((rows + gm::kTileRows - 1) / gm::kTileRows);
    // Waves per tile: a wave's chunks run one after another, each waiting
    // for its loads, so the columns are split until the waves cover the
    // chip's SIMDs about one and a half times over (measured: Q4_K
    // 4096 x 4096 at batch 32 took 63 / 34 / 20 us at 1 / 2 / 4 waves per
    // tile), each wave keeping at least two chunks.
    int ks = QG_GEMM_KS;
    if (ks == 0) {
        const int64_t target = 6LL * device_cus();
        ks = 1;
        while (ks < gm::kWaves && (int64_t)p.tiles * ks < target && p.nchunks >= 4 * ks) ks *= 2;
    }
    while (ks > 1 && ks > p.nchunks) ks /= 2;
    p.ks = ks;
    p.nu = gemm_nu(F::CHUNK);
    p.slot = 16u * (uint32_t)(p.nu | 1);
    const int tpw = gm::kWaves / ks;
    const int64_t grid = ((int64_t)p.tiles + tpw - 1) / tpw;
    const size_t lds = (size_t)gm::kWaves * gm::kTileRows * p.slot +
                       (ks > 1 ? (size_t)gm::kWaves * NB * 4 * 64 * 4 : 0);
    // 4-byte-aligned fields in LDS when every row and chunk starts at a
    // multiple of 4 bytes
    const bool ra = !(F::CHUNK % 4 == 0 && rb % 4 == 0 && aligned_to(W, 4));
    if constexpr (F::CHUNK % 4 == 0) {
        if (!ra) return launch_gemm_t<F, NB, false>(p, (int)grid, lds, st);
    }
    return launch_gemm_t<F, NB, true>(p, (int)grid, lds, st);
}

template <int NB>
int gemm_b(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
           int batch, int64_t rb, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_gemm<gm::GK45<false>, NB>(W, rows, cols, X, Y, batch, rb, st);
    case QG_Q5_K: return launch_gemm<gm::GK45<true>, NB>(W, rows, cols, X, Y, batch, rb, st);
    case QG_Q6_K: return launch_gemm<gm::GQ6K, NB>(W, rows, cols, X, Y, batch, rb, st);
    case QG_Q8_0: return launch_gemm<gm::GQ80, NB>(W, rows, cols, X, Y, batch, rb, st);
    case QG_Q4_0: return launch_gemm<gm::GQ40, NB>(W, rows, cols, X, Y, batch, rb, st);
    default: return fail(QG_EUNSUPPORTED, "qgemv: format %d has no matrix-core path", fmt);
    }
}

}  // namespace host
}  // namespace qg
