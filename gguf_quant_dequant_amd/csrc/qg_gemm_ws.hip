// qg_gemm_ws.hip -- planning and launch of the batched GEMV with shared
// activation operands (gw::qgemm_ws_kernel, qg_gemm_ws.hpp) behind qgemv_ws.
#include "qg_gemm_host.hpp"
#include "qg_gemm_ws.hpp"
#include "qg_mx_host.hpp"

// Workgroups a launch may have: one per CU of a 256-CU part.  A CU that
// holds two workgroups finishes last (measured on Q5_K 14336 x 4096 at batch
// 8: 224 workgroups 20.0 us, 336 25.4 us, 560-896 24.6-25.6 us), so the
// column split stops before the grid exceeds this; the fewest chunks a
// column range keeps.
#ifndef QG_WS_WGS
#define QG_WS_WGS 256
#endif
#ifndef QG_WS_MIN_CHUNKS
#define QG_WS_MIN_CHUNKS 2
#endif

namespace qg {
namespace host {

// Column ranges per group of 8 tiles: as many as keep the grid within
// QG_WS_WGS workgroups.  Independent of the device, so the workspace size is
// known on the host before any call.
int ws_kg(int64_t rows, int64_t cols) {
    const int64_t tiles = (rows + gm::kTileRows - 1) / gm::kTileRows;
    const int64_t groups = (tiles + gw::kWaves - 1) / gw::kWaves;
    const int64_t nchunks = (cols + gm::kChunk - 1) / gm::kChunk;
    int64_t kg = QG_WS_WGS / groups;
    const int64_t cap = nchunks / QG_WS_MIN_CHUNKS;
    if (kg > cap) kg = cap;
    if (kg < 1) kg = 1;
    return (int)kg;
}

namespace {

template <class F, int MODE, bool RA>
int launch_ws_t(const gw::WsParams &p, hipStream_t st) {
    constexpr int U = gemm_units(F::CHUNK);
    auto kern = gw::qgemm_ws_kernel<F, MODE, RA, U>;
    const size_t lds = gw::ws_lds_bytes<MODE>(p.slot);
    if (lds > (size_t)device_lds_max())
        return fail(QG_EUNSUPPORTED, "qgemv_ws: %zu bytes of LDS per workgroup exceed the "
                                     "device's %d", lds, device_lds_max());
    static std::atomic<bool> attr{false};
    if (lds > 65536 && !attr.load(std::memory_order_relaxed)) {
        (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  device_lds_max());
        (void)hipGetLastError();
        attr.store(true, std::memory_order_relaxed);
    }
    const int64_t groups = ((int64_t)p.tiles + gw::kWaves - 1) / gw::kWaves;
    hipLaunchKernelGGL(kern, dim3((unsigned)(groups * p.kg)), dim3(gw::kThreads), lds, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "qgemv_ws: launch failed: %s", hipGetErrorString(e));
    if (p.kg > 1) {
        const int64_t n = (int64_t)p.batch * p.rows;
        const int64_t blocks = (n + 255) / 256;
        const int grid = (int)(blocks < 4096 ? blocks : 4096);
        hipLaunchKernelGGL(gw::ws_reduce_kernel, dim3(grid), dim3(256), 0, st, p.part, p.Y, n,
                           p.kg);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(QG_ELAUNCH, "qgemv_ws: launch failed: %s", hipGetErrorString(e));
    }
    return QG_OK;
}

template <class F>
int launch_ws(const void *W, int64_t rows, int64_t cols, const float *X, float *Y, int batch,
              int64_t rb, float *part, hipStream_t st) {
    gw::WsParams p{};
    p.W = (const uint8_t *)W;
    p.X = X;
    p.Y = Y;
    p.part = part;
    p.rows = rows;
    p.w_bytes = (uint64_t)rows * (uint64_t)rb;
    p.row_bytes = (uint32_t)rb;
    p.cols = (uint32_t)cols;
    p.batch = batch;
    p.nchunks = (int32_t)((cols + gm::kChunk - 1) / gm::kChunk);
    p.last_nkb = (int32_t)(((cols - 1) % gm::kChunk) / 32 + 1);
    p.tiles = (int32_t)((rows + gm::kTileRows - 1) / gm::kTileRows);
    p.kg = ws_kg(rows, cols);
    p.nu = gemm_nu(F::CHUNK);
    p.slot = 16u * (uint32_t)(p.nu | 1);
    // 4-byte-aligned fields in LDS when every row and chunk starts at a
    // multiple of 4 bytes
    const bool ra = !(F::CHUNK % 4 == 0 && rb % 4 == 0 && aligned_to(W, 4));
    if constexpr (F::CHUNK % 4 == 0) {
        if (!ra) {
            if (batch <= 8) return launch_ws_t<F, 0, false>(p, st);
            if (batch <= 16) return launch_ws_t<F, 1, false>(p, st);
            return launch_ws_t<F, 2, false>(p, st);
        }
    }
    if (batch <= 8) return launch_ws_t<F, 0, true>(p, st);
    if (batch <= 16) return launch_ws_t<F, 1, true>(p, st);
    return launch_ws_t<F, 2, true>(p, st);
}

}  // namespace

int gemm_ws(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
            int batch, int64_t rb, float *part, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_ws<gm::GK45<false>>(W, rows, cols, X, Y, batch, rb, part, st);
    case QG_Q5_K: return launch_ws<gm::GK45<true>>(W, rows, cols, X, Y, batch, rb, part, st);
    case QG_Q6_K: return launch_ws<gm::GQ6K>(W, rows, cols, X, Y, batch, rb, part, st);
    case QG_Q8_0: return launch_ws<gm::GQ80>(W, rows, cols, X, Y, batch, rb, part, st);
    case QG_Q4_0: return launch_ws<gm::GQ40>(W, rows, cols, X, Y, batch, rb, part, st);
    default: return fail(QG_EUNSUPPORTED, "qgemv_ws: format %d has no matrix-core path", fmt);
    }
}

}  // namespace host
}  // namespace qg
