// qg_q6mx.hip -- launch of the batch-1 Q6_K GEMV on the matrix cores
// (q6mx::q6k_mx1_kernel, and q6k_mx2_kernel for two batch rows,
// qg_q6mx.hpp).
#include "qg_host.hpp"
#include "qg_q6mx.hpp"

namespace qg {
namespace host {

namespace {

template <int TPW, int NB>
int launch_q6mx(const GemvParams &p, int waves, hipStream_t st) {
    const int threads = 64 * waves;
    const size_t lds = (size_t)kStageChunks * 16 * threads;
    const int64_t blocks = (p.rows + q6mx::kRows - 1) / q6mx::kRows;
    const auto kern = NB == 1 ? q6mx::q6k_mx1_kernel<TPW> : q6mx::q6k_mx2_kernel<TPW>;
    const int grid = resident_grid((const void *)kern, threads, lds, blocks);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ELAUNCH, "qgemv: launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace

// Rows of 64 * TPW * W columns with TPW = 8 or 4 tiles per wave and W <= 8
// waves (every multiple of 512 columns up to 4096, every multiple of 256 up
// to 2048).  The stage of 128 bytes per thread then holds a block of 16
// rows with its leading alignment and the realigning reads' extra dword,
// and the activations (nb = 1 or 2 rows of X, cols floats each) fit one
// round of it.
int try_q6mx(const GemvParams &p, int nb, hipStream_t st, bool *done) {
    *done = false;
    if (p.cols % 256 != 0) return QG_OK;
    const int64_t tiles = p.cols / 64;
    int tpw = 0;
    if (tiles % 8 == 0 && tiles / 8 <= 8)
        tpw = 8;
    else if (tiles % 4 == 0 && tiles / 4 <= 8)
        tpw = 4;
    if (tpw == 0) return QG_OK;
    const int waves = (int)(tiles / tpw);
    const size_t cap = (size_t)kStageChunks * 16 * 64 * waves;
    if (nb < 1 || nb > 2 || (size_t)q6mx::kRows * p.row_bytes + 15 + 4 > cap ||
        (uint64_t)nb * p.cols > 32u * 64u * (uint64_t)waves)
        return QG_OK;
    *done = true;
    if (nb == 2)
        return tpw == 8 ? launch_q6mx<8, 2>(p, waves, st) : launch_q6mx<4, 2>(p, waves, st);
    return tpw == 8 ? launch_q6mx<8, 1>(p, waves, st) : launch_q6mx<4, 1>(p, waves, st);
}

}  // namespace host
}  // namespace qg
