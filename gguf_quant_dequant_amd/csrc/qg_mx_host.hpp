// qg_mx_host.hpp -- planning and launch of the matrix-core GEMV
// (mx::qgemv_mx_kernel); instantiated per batch tile in qg_mx_b<B>.hip.
#pragma once

#include "qg_host.hpp"
#include "qg_mfma.hpp"

namespace qg {
namespace host {

// ------------------------------------------------------- matrix-core GEMV

inline int device_lds_max() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v) return v;
    int dev = 0, n = 65536;
    if (hipGetDevice(&dev) == hipSuccess) {
        int m = 0;
        if (hipDeviceGetAttribute(&m, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
                hipSuccess && m > 0)
            n = m;
    }
    cached.store(n, std::memory_order_relaxed);
    return n;
}



struct MxPlan {
    mx::MxParams p;
    size_t lds;
    int grid;
    int tld;
    bool ra, row16;
};

// Stage shape for the matrix-core kernel.  When every tile has a workgroup
// of its own, a workgroup takes its whole tile (up to 16 chunks) in one
// stage.  Otherwise workgroups stream phases of up to 4 chunks (each chunk
// split between two waves) through two buffers, sized so that two
// workgroups share a CU where the activation image allows.
template <class F, int B>
bool mx_plan(const void *W, int64_t rows, int64_t cols, int batch, int64_t rb, MxPlan *pl) {
    constexpr int REC = mx::ximg_rec(B), NB = mx::nb_of(B);
    const bool row16 = rb % 16 == 0 && F::CHUNK % 16 == 0;
    const bool ra = F::CHUNK % 4 != 0 || !(row16 && aligned_to(W, 16));
    const int64_t nc = (cols + mx::kChunk - 1) / mx::kChunk;
    const int64_t tiles = (rows + mx::kRows - 1) / mx::kRows;
    const size_t lds_max = (size_t)device_lds_max();
    const size_t ximg = (size_t)nc * REC, red = (size_t)mx::kWaves * 64 * NB * 4;
    const size_t out_tile = (size_t)B * mx::kRows * 4;
    const int cus = device_cus();
    auto seg_units = [&](int P) { return (P * F::CHUNK + (row16 && !ra ? 0 : 14) + 15) / 16; };
    auto slot_of = [&](int nu) { return 16 * (nu | 1); };

    int P = 0, npart = 1, nbuf = 1, nu = 0, tld = 16;
    int64_t grid = 0;
    size_t stage = 0, lds = 0;
    if (nc <= 16 && tiles <= 2 * cus) {
        P = (int)nc;
        npart = nc >= 8 ? 1 : 2;
        nu = seg_units(P);
        stage = (size_t)mx::kRows * slot_of(nu);
        lds = ximg + stage + red + out_tile;
        grid = tiles;
        if (lds > lds_max || mx::kRows * nu > 512 * 16) P = 0;
    }
    if (P == 0) {
        nbuf = 2;
        tld = 8;
        npart = 2;
        for (int per_cu = 2; per_cu >= 1 && P == 0; per_cu--) {
            for (int Pm = nc < 4 ? (int)nc : 4; Pm >= 1; Pm >>= 1) {
                nu = seg_units(Pm);
                stage = (size_t)mx::kRows * slot_of(nu);
                grid = (int64_t)cus * per_cu;
                if (grid > tiles) grid = tiles;
                const size_t out = (size_t)((tiles + grid - 1) / grid) * out_tile;
                lds = ximg + 2 * stage + red + out;
                if (lds * per_cu <= lds_max && mx::kRows * nu <= 512 * 8) {
                    P = Pm;
                    break;
                }
            }
        }
        if (P == 0) return false;
    }
    mx::MxParams &p = pl->p;
    p = mx::MxParams{};
    p.W = (const uint8_t *)W;
    p.rows = rows;
    p.w_bytes = (uint64_t)rows * (uint64_t)rb;
    p.tiles = tiles;
    p.row_bytes = (uint32_t)rb;
    p.cols = (uint32_t)cols;
    p.ximg_bytes = (uint32_t)ximg;
    p.slot = (uint32_t)slot_of(nu);
    p.stage_bytes = (uint32_t)stage;
    p.out_off = (uint32_t)(ximg + nbuf * stage + red);
    p.batch = batch;
    p.nc = (int32_t)nc;
    p.P = P;
    p.nph = (int32_t)((nc + P - 1) / P);
    p.npart = npart;
    p.nu = nu;
    p.nbuf = nbuf;
    p.last_nblk = (int32_t)(((cols - 1) % mx::kChunk) / 32 + 1);
    p.coff = -0x1p-24f;
    p.x_stride = (uint32_t)cols;
    p.x_bytes = (uint32_t)(4 * cols * batch);
    p.accumulate = 0;
    pl->lds = lds;
    pl->ra = ra;
    pl->row16 = row16;
    pl->grid = (int)grid;
    // 16-byte loads per thread and stage: the smallest instantiated count
    const int units = mx::kRows * nu;
    pl->tld = units <= 512 * 4 ? 4 : (units <= 512 * 8 ? 8 : 16);
    (void)tld;
    return true;
}

template <class F, int B, bool RA, bool ROW16, int TLD>
int launch_mx(const MxPlan &pl, hipStream_t st) {
    auto kern = mx::qgemv_mx_kernel<F, B, RA, ROW16, TLD>;
    static std::atomic<bool> attr{false};
    if (pl.lds > 65536 && !attr.load(std::memory_order_relaxed)) {
        (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  device_lds_max());
        (void)hipGetLastError();
        attr.store(true, std::memory_order_relaxed);
    }
    hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(512), pl.lds, st, pl.p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ELAUNCH, "qgemv: launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

template <class F, int B, bool RA, bool ROW16>
int launch_mx_t(const MxPlan &pl, hipStream_t st) {
    switch (pl.tld) {
    case 4: return launch_mx<F, B, RA, ROW16, 4>(pl, st);
    case 8: return launch_mx<F, B, RA, ROW16, 8>(pl, st);
    default: return launch_mx<F, B, RA, ROW16, 16>(pl, st);
    }
}

// Runs the matrix-core kernel when the shape fits; *done = false otherwise.
template <class F, int B>
int try_mx_f(const void *W, int64_t rows, int64_t cols, const float *X, float *Y, int batch,
             int64_t rb, hipStream_t st, bool *done) {
    MxPlan pl;
    *done = false;
    auto launch = [&](const MxPlan &q) {
        if constexpr (F::CHUNK % 4 != 0) return launch_mx_t<F, B, true, false>(q, st);
        else {
            if (!q.ra) return launch_mx_t<F, B, false, true>(q, st);
            return launch_mx_t<F, B, true, false>(q, st);
        }
    };
    if (mx_plan<F, B>(W, rows, cols, batch, rb, &pl)) {
        pl.p.X = X;
        pl.p.Y = Y;
        *done = true;
        return launch(pl);
    }
    return QG_OK;
}

template <int B>
int try_mx_b(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
             int batch, int64_t rb, hipStream_t st, bool *done) {
    switch (fmt) {
    case QG_Q4_K: return try_mx_f<mx::MK45<false>, B>(W, rows, cols, X, Y, batch, rb, st, done);
    case QG_Q5_K: return try_mx_f<mx::MK45<true>, B>(W, rows, cols, X, Y, batch, rb, st, done);
    case QG_Q6_K: return try_mx_f<mx::MQ6K, B>(W, rows, cols, X, Y, batch, rb, st, done);
    case QG_Q8_0: return try_mx_f<mx::MQ80, B>(W, rows, cols, X, Y, batch, rb, st, done);
    case QG_Q4_0: return try_mx_f<mx::MQ40, B>(W, rows, cols, X, Y, batch, rb, st, done);
    default: *done = false; return QG_OK;
    }
}

}  // namespace host
}  // namespace qg
