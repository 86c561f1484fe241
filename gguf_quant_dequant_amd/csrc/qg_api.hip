// qg_api.hip -- host side of the C ABI declared in include/qgemv.h:
// argument validation (before any HIP call), kernel selection and launch on
// the caller's stream.  No allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <map>
#include <mutex>
#include <tuple>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/qgemv.h"
#include "qg_kernels.hpp"
#include "qg_mfma.hpp"
#include "qg_q8act.hpp"

using namespace qg;

// Launch tuning (compile-time): rows per row group per iteration for batch 1
// and for larger batches.
#ifndef QG_U_B1
#define QG_U_B1 2
#endif
#ifndef QG_U_BN
#define QG_U_BN 2
#endif
// The staged GEMV copies the activations through LDS when they take one
// round of the stage's size, or up to this many when each workgroup stages
// at most two row blocks; otherwise each lane loads its tile of X from
// global memory.
#ifndef QG_XL_ROUNDS
#define QG_XL_ROUNDS 4
#endif
// 1: GEMV rows are staged through LDS with coalesced 16-byte loads;
// 0: each lane loads its tile's fields straight from global memory.
#ifndef QG_STAGE
#define QG_STAGE 1
#endif
// Block formats at batch >= QG_MX_MIN_BATCH run on the matrix cores when the
// activation image and the stage buffers fit in LDS (0 disables).  At batch
// 1 the VALU kernels are as fast or faster on the measured shapes.
// Rows per row group and iteration in the MoE gate/up and down kernels.
#ifndef QG_MOE_GU_U
#define QG_MOE_GU_U 2
#endif
#ifndef QG_MOE_DN_U
#define QG_MOE_DN_U 2
#endif
// 1: workgroups of half the threads (half the row groups) in the MoE
// gate/up or down kernel.
#ifndef QG_MOE_GU_T128
#define QG_MOE_GU_T128 0
#endif
#ifndef QG_MOE_DN_T128
#define QG_MOE_DN_T128 0
#endif
#ifndef QG_MX_MIN_BATCH
#define QG_MX_MIN_BATCH 2
#endif

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return QG_OK;
}

struct Geom {
    int elems, bytes;
};

Geom geom(int fmt) {
    switch (fmt) {
    case QG_F32: return {1, 4};
    case QG_Q4_0: return {32, 18};
    case QG_Q8_0: return {32, 34};
    case QG_Q4_K: return {256, 144};
    case QG_Q5_K: return {256, 176};
    case QG_Q6_K: return {256, 210};
    default: return {0, 0};
    }
}

const char *fmt_name(int fmt) {
    switch (fmt) {
    case QG_F32: return "F32";
    case QG_Q4_0: return "Q4_0";
    case QG_Q8_0: return "Q8_0";
    case QG_Q4_K: return "Q4_K";
    case QG_Q5_K: return "Q5_K";
    case QG_Q6_K: return "Q6_K";
    default: return "unknown";
    }
}

// Workgroups per launch: enough to cover every CU several times over; the
// kernels loop over the rest.
int device_cus() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v) return v;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            cus = n;
    }
    cached.store(cus, std::memory_order_relaxed);
    return cus;
}

// Workgroups of kernel fn (threads, dynamic LDS) that fit on one CU at once,
// from the occupancy calculator; cached per configuration.
int resident_per_cu(const void *fn, int threads, size_t lds) {
    static std::mutex mu;
    static std::map<std::tuple<const void *, int, size_t>, int> cache;
    std::lock_guard<std::mutex> g(mu);
    const auto key = std::make_tuple(fn, threads, lds);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess || n < 1)
        n = 1;
    cache[key] = n;
    return n;
}

// A grid-stride kernel's grid: one workgroup per block of work, at most as
// many as are resident on the whole chip at once, so that no workgroup
// waits for a slot while others run (every workgroup does about the same
// work; a second partial round would run at a fraction of the occupancy).
int resident_grid(const void *fn, int threads, size_t lds, int64_t blocks) {
    const int64_t cap = (int64_t)device_cus() * resident_per_cu(fn, threads, lds);
    return (int)(blocks < cap ? blocks : cap);
}

bool aligned_to(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Row-group shape for `tiles` tiles per row: lanes per group inside one wave
// (power of two), or S whole waves; G groups per workgroup; block threads.
struct Shape {
    int lpr, S, G, threads;
};

bool shape_for(int tiles, Shape *s) {
    if (tiles <= 64) {
        s->lpr = next_pow2(tiles);
        s->S = 1;
        s->G = 256 / s->lpr;
        s->threads = 256;
        return true;
    }
    const int S = (tiles + 63) / 64;
    if (S > 8) return false;
    s->lpr = 64;
    s->S = S;
    s->G = S >= 4 ? 1 : 4 / S;
    s->threads = 64 * S * s->G;
    return true;
}

// ------------------------------------------------------------------- qgemv

// Tile widths per format at batch B: the activations of a tile stay in
// VGPRs, so columns-per-tile * B is kept at or below 128.
constexpr int lw_k45(int B) { return B == 1 ? 32 : (B <= 4 ? 16 : 8); }  // CPT = 2 LW
constexpr int lw_q6k(int B) { return B == 1 ? 16 : (B <= 4 ? 8 : 4); }   // CPT = 4 LW
constexpr int lw_q80(int B) { return B <= 4 ? 32 : 16; }                 // CPT = LW
constexpr int lw_q40(int B) { return B <= 4 ? 16 : 8; }                  // CPT = 2 LW
constexpr int lw_f32max(int B) { return B == 1 ? 32 : (B <= 4 ? 16 : 8); }

// Columns per tile for format fmt at batch B; F32 takes the widest tile
// (<= its maximum) that divides cols.  0 if none.
int gemv_cpt(int fmt, int B, int64_t cols) {
    switch (fmt) {
    case QG_Q4_K:
    case QG_Q5_K: return 2 * (B == 1 ? lw_k45(1) : (B <= 4 ? lw_k45(4) : lw_k45(8)));
    case QG_Q6_K: return 4 * (B == 1 ? lw_q6k(1) : (B <= 4 ? lw_q6k(4) : lw_q6k(8)));
    case QG_Q8_0: return B <= 4 ? lw_q80(4) : lw_q80(8);
    case QG_Q4_0: return 2 * (B <= 4 ? lw_q40(4) : lw_q40(8));
    case QG_F32: {
        const int maxw = B == 1 ? lw_f32max(1) : (B <= 4 ? lw_f32max(4) : lw_f32max(8));
        for (int w = maxw; w >= 4; w >>= 1)
            if (cols % w == 0) return w;
        return 0;
    }
    default: return 0;
    }
}

// The staged kernel with US rows per row group and stage: activations
// through LDS when they fit one round of the stage's size, or a few rounds
// in a workgroup that stages few row blocks (each further round adds a load
// latency to the workgroup's start, which many blocks amortise less well
// than the per-lane loads' uncoalesced reads).
template <class F, int B, int US>
void launch_staged(const GemvParams &p, const Shape &s, size_t stage_bytes, hipStream_t st) {
    const int64_t per_iter = (int64_t)s.G * US;
    const int64_t iters = (p.rows + per_iter - 1) / per_iter;
    const int64_t xrounds = ((int64_t)B * p.cols + 32 * s.threads - 1) / (32 * s.threads);
    const int grid_xl =
        resident_grid((const void *)qgemv_lds_kernel<F, B, US, true>, s.threads, stage_bytes, iters);
    const int64_t blocks_per_wg = (iters + grid_xl - 1) / grid_xl;
    if (xrounds <= 1 || (xrounds <= QG_XL_ROUNDS && blocks_per_wg <= 2)) {
        hipLaunchKernelGGL((qgemv_lds_kernel<F, B, US, true>), dim3(grid_xl), dim3(s.threads),
                           stage_bytes, st, p);
    } else {
        const int grid = resident_grid((const void *)qgemv_lds_kernel<F, B, US, false>, s.threads,
                                       stage_bytes, iters);
        hipLaunchKernelGGL((qgemv_lds_kernel<F, B, US, false>), dim3(grid), dim3(s.threads),
                           stage_bytes, st, p);
    }
}

template <class F, int B, int U>
int launch_gemv(GemvParams p, hipStream_t st) {
    p.tiles = (int32_t)(p.cols / F::CPT);
    Shape s;
    if (!shape_for(p.tiles, &s))
        return fail(QG_EUNSUPPORTED, "qgemv: %u columns need %d lane tiles per row at batch %d; "
                                     "at most 512 are supported",
                    p.cols, p.tiles, B);
    // Batch 1 with one wave per row (64-lane groups): workgroups of two
    // waves, twice as many of them (Q4_K 4096 x 4096: 5.48 -> 5.39 us).
    if (B == 1 && s.S == 1 && s.lpr == 64) {
        s.G = 2;
        s.threads = 128;
    }
    p.lpr = s.lpr;
    p.S = s.S;
    p.G = s.G;
    // The stage holds kStageChunks 16-byte chunks per thread; a block of
    // G * US rows plus up to 15 bytes of leading alignment and the
    // realigning reads' extra dword past the last field must fit.  Four rows
    // per row group when they fit and the batch is at most 4 (more bytes in
    // flight per workgroup for long rows; at batch 8 the extra accumulators
    // cost occupancy), else two, else the unstaged kernel.
    const size_t stage_bytes = (size_t)kStageChunks * 16 * s.threads;
    auto fits = [&](int us) {
        return QG_STAGE && (size_t)s.G * us * p.row_bytes + 15 + 4 <= stage_bytes;
    };
    if (B <= 4 && fits(4)) {
        launch_staged<F, B, 4>(p, s, stage_bytes, st);
    } else if (fits(2)) {
        launch_staged<F, B, 2>(p, s, stage_bytes, st);
    } else {
        const int64_t per_iter = (int64_t)s.G * U;
        const int64_t iters = (p.rows + per_iter - 1) / per_iter;
        const int grid = resident_grid((const void *)qgemv_kernel<F, B, U>, s.threads, 0, iters);
        hipLaunchKernelGGL((qgemv_kernel<F, B, U>), dim3(grid), dim3(s.threads), 0, st, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ELAUNCH, "qgemv: launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

template <int B>
int dispatch_gemv_b(int fmt, bool aligned, int cpt, const GemvParams &p, hipStream_t st) {
    constexpr int U = B == 1 ? QG_U_B1 : QG_U_BN;
    constexpr int K45 = lw_k45(B), Q6 = lw_q6k(B), Q8 = lw_q80(B), Q4 = lw_q40(B);
    constexpr int FM = lw_f32max(B);
    switch (fmt) {
    case QG_Q4_K:
        return aligned ? launch_gemv<FmtQ4K<K45, false>, B, U>(p, st)
                       : launch_gemv<FmtQ4K<K45, true>, B, U>(p, st);
    case QG_Q5_K:
        return aligned ? launch_gemv<FmtQ5K<K45, false>, B, U>(p, st)
                       : launch_gemv<FmtQ5K<K45, true>, B, U>(p, st);
    case QG_Q6_K: return launch_gemv<FmtQ6K<Q6>, B, U>(p, st);
    case QG_Q8_0: return launch_gemv<FmtQ80<Q8>, B, U>(p, st);
    case QG_Q4_0: return launch_gemv<FmtQ40<Q4>, B, U>(p, st);
    case QG_F32:
        if (cpt == FM) return launch_gemv<FmtF32<FM>, B, U>(p, st);
        if constexpr (FM > 8)
            if (cpt == FM / 2) return launch_gemv<FmtF32<FM / 2>, B, U>(p, st);
        if constexpr (FM > 16)
            if (cpt == FM / 4) return launch_gemv<FmtF32<FM / 4>, B, U>(p, st);
        if (cpt == 8) return launch_gemv<FmtF32<8>, B, U>(p, st);
        return launch_gemv<FmtF32<4>, B, U>(p, st);
    default: return fail(QG_EUNSUPPORTED, "qgemv: unknown format %d", fmt);
    }
}

// The int8-activation variant (batch 1): the format's tiles with q8a
// activation tiles and integer dot products.
int dispatch_gemv_q8(int fmt, bool aligned, const GemvParams &p, hipStream_t st) {
    constexpr int U = QG_U_B1;
    switch (fmt) {
    case QG_Q4_K:
        return aligned ? launch_gemv<q8a::Q8A<FmtQ4K<32, false>>, 1, U>(p, st)
                       : launch_gemv<q8a::Q8A<FmtQ4K<32, true>>, 1, U>(p, st);
    case QG_Q5_K:
        return aligned ? launch_gemv<q8a::Q8A<FmtQ5K<32, false>>, 1, U>(p, st)
                       : launch_gemv<q8a::Q8A<FmtQ5K<32, true>>, 1, U>(p, st);
    case QG_Q6_K: return launch_gemv<q8a::Q8A<FmtQ6K<16, false>>, 1, U>(p, st);
    case QG_Q8_0: return launch_gemv<q8a::Q8A<FmtQ80<32>>, 1, U>(p, st);
    case QG_Q4_0: return launch_gemv<q8a::Q8A<FmtQ40<16>>, 1, U>(p, st);
    default: return fail(QG_EUNSUPPORTED, "qgemv_q8act: format %d has no int8 path", fmt);
    }
}

int dispatch_gemv(int fmt, int B, bool aligned, int64_t cols, const GemvParams &p,
                  hipStream_t st) {
    const int cpt = gemv_cpt(fmt, B, cols);
    switch (B) {
    case 1: return dispatch_gemv_b<1>(fmt, aligned, cpt, p, st);
    case 2: return dispatch_gemv_b<2>(fmt, aligned, cpt, p, st);
    case 3: return dispatch_gemv_b<3>(fmt, aligned, cpt, p, st);
    case 4: return dispatch_gemv_b<4>(fmt, aligned, cpt, p, st);
    case 5: return dispatch_gemv_b<5>(fmt, aligned, cpt, p, st);
    case 6: return dispatch_gemv_b<6>(fmt, aligned, cpt, p, st);
    case 7: return dispatch_gemv_b<7>(fmt, aligned, cpt, p, st);
    case 8: return dispatch_gemv_b<8>(fmt, aligned, cpt, p, st);
    default: return fail(QG_EUNSUPPORTED, "qgemv: batch %d outside 1..8", B);
    }
}

bool tiles_fit(int fmt, int B, int64_t cols) {
    const int cpt = gemv_cpt(fmt, B, cols);
    if (cpt == 0) return false;
    return (cols / cpt) <= 512;
}

// ------------------------------------------------------- matrix-core GEMV

int device_lds_max() {
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
    p.coff = -F::OFF * 0x1p-24f;
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
    // The activation image of the whole row does not fit in LDS: split the
    // columns into the fewest slices of whole 256-column chunks whose plans
    // fit (batch >= 3 only, where the VALU kernel is compute-bound), and run
    // them in order, each adding its sums to Y.  Every weight byte is still
    // read once.
    // Each slice is a launch of its own over all row tiles, so slices pay
    // only when the tiles fill the chip (4096 rows = 128 tiles ran slower
    // in slices than on the VALU kernel).
    if (batch < 3 || (rows + mx::kRows - 1) / mx::kRows < device_cus()) return QG_OK;
    const int64_t nc = (cols + mx::kChunk - 1) / mx::kChunk;
    constexpr int kMaxSlices = 8;
    for (int64_t ns = 2; ns <= kMaxSlices && ns <= nc; ns++) {
        const int64_t per = (nc + ns - 1) / ns * mx::kChunk;  // columns per slice
        MxPlan sl[kMaxSlices];
        int n = 0;
        bool fit = true;
        for (int64_t c0 = 0; c0 < cols; c0 += per, n++) {
            const int64_t pc = cols - c0 < per ? cols - c0 : per;
            const int64_t woff = rb * c0 / cols;  // bytes of c0 columns (whole blocks)
            const uint8_t *Wp = (const uint8_t *)W + woff;
            if (!mx_plan<F, B>(Wp, rows, pc, batch, rb, &sl[n])) {
                fit = false;
                break;
            }
            mx::MxParams &q = sl[n].p;
            q.w_bytes = (uint64_t)rows * (uint64_t)rb - (uint64_t)woff;
            q.X = X + c0;
            q.x_stride = (uint32_t)cols;
            q.x_bytes = (uint32_t)(4 * (cols * batch - c0));
            q.Y = Y;
            q.accumulate = n > 0;
        }
        if (!fit) continue;
        *done = true;
        for (int i = 0; i < n; i++) {
            const int rc = launch(sl[i]);
            if (rc != QG_OK) return rc;
        }
        return QG_OK;
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

int try_mx(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
           int batch, int64_t rb, hipStream_t st, bool *done) {
    *done = false;
    if (QG_MX_MIN_BATCH == 0 || fmt == QG_F32) return QG_OK;
    // below the threshold only rows too wide for the VALU kernels go here
    if (batch < QG_MX_MIN_BATCH && tiles_fit(fmt, batch, cols)) return QG_OK;
    if (batch == 1) return try_mx_b<1>(fmt, W, rows, cols, X, Y, batch, rb, st, done);
    if (batch <= 2) return try_mx_b<2>(fmt, W, rows, cols, X, Y, batch, rb, st, done);
    if (batch <= 4) return try_mx_b<4>(fmt, W, rows, cols, X, Y, batch, rb, st, done);
    return try_mx_b<8>(fmt, W, rows, cols, X, Y, batch, rb, st, done);
}


// ------------------------------------------------------------------- MoE

size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

struct WsLayout {
    size_t logits, sel, w, act, total;
};

// Sections for T tokens: f64 logits [T][E], int32 routes [T][K], f32
// weights [T][K], f32 activations [T][K][F], each 16-byte aligned.
WsLayout ws_layout(int64_t E, int64_t K, int64_t F, int64_t T = 1) {
    WsLayout l;
    l.logits = 0;
    l.sel = align16(8 * (size_t)(T * E));
    l.w = l.sel + align16(4 * (size_t)(T * K));
    l.act = l.w + align16(4 * (size_t)(T * K));
    l.total = l.act + align16(4 * (size_t)(T * K) * (size_t)F);
    return l;
}

// columns per tile for the B = 1 kernels of the MoE chain
int moe_cpt(int fmt) {
    switch (fmt) {
    case QG_Q4_K:
    case QG_Q5_K:
    case QG_Q6_K: return 64;
    case QG_Q8_0:
    case QG_Q4_0: return 32;
    default: return 0;
    }
}

template <class F>
int launch_gateup(MoeParams p, hipStream_t st) {
    constexpr int U = QG_MOE_GU_U;
    Shape s;
    p.gu_tiles = p.H / F::CPT;
    if (!shape_for(p.gu_tiles, &s))
        return fail(QG_EUNSUPPORTED, "moe_ffn: hidden %d too wide for the gate/up kernel", p.H);
    if (QG_MOE_GU_T128 && s.S == 1 && s.G >= 2) {
        s.G /= 2;
        s.threads = 128;
    }
    p.gu_lpr = s.lpr;
    p.gu_S = s.S;
    p.gu_G = s.G;
    const int64_t tasks = (int64_t)p.K * p.F, per = (int64_t)s.G * U;
    const int64_t iters = (tasks + per - 1) / per;
    const size_t lds = (size_t)kStageChunks * 16 * s.threads;
    const int grid = resident_grid((const void *)moe_gateup_kernel<F, U>, s.threads, lds, iters);
    hipLaunchKernelGGL((moe_gateup_kernel<F, U>), dim3(grid), dim3(s.threads), lds, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "moe_ffn: gate/up launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

template <class F>
int launch_down(MoeParams p, hipStream_t st) {
    constexpr int U = QG_MOE_DN_U;
    Shape s;
    p.dn_tiles_per_slot = p.F / F::CPT;
    p.dn_tiles = p.K * p.dn_tiles_per_slot;
    if (!shape_for(p.dn_tiles, &s))
        return fail(QG_EUNSUPPORTED, "moe_ffn: top_k * expert_dim too wide for the down kernel");
    if (QG_MOE_DN_T128 && s.S * s.G * 64 > 128 && s.G >= 2) {
        s.G /= 2;
        s.threads /= 2;
    }
    p.dn_lpr = s.lpr;
    p.dn_S = s.S;
    p.dn_G = s.G;
    const int64_t per = (int64_t)s.G * U;
    const int64_t iters = (p.H + per - 1) / per;
    const size_t lds = (size_t)kStageChunks * 16 * s.threads;
    // one grid row per token (blockIdx.y), the resident workgroups shared
    const int64_t cap = (int64_t)device_cus() *
                        resident_per_cu((const void *)moe_down_kernel<F, U>, s.threads, lds);
    int64_t gx = cap / p.T;
    gx = gx < 1 ? 1 : (gx > iters ? iters : gx);
    hipLaunchKernelGGL((moe_down_kernel<F, U>), dim3((unsigned)gx, (unsigned)p.T), dim3(s.threads),
                       lds, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "moe_ffn: down launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

// Several tokens: B activation vectors per tile (tokens past T are zero),
// tile widths of the batch-B GEMV.
template <class F, int B>
int launch_gateup_tokens(MoeParams p, hipStream_t st) {
    constexpr int U = 2;
    Shape s;
    p.gu_tiles = p.H / F::CPT;
    if (p.H % F::CPT != 0 || !shape_for(p.gu_tiles, &s))
        return fail(QG_EUNSUPPORTED, "moe_ffn_tokens: hidden %d does not fit the gate/up kernel",
                    p.H);
    p.gu_lpr = s.lpr;
    p.gu_S = s.S;
    p.gu_G = s.G;
    // at most T * K distinct experts
    const int64_t tasks = (int64_t)p.T * p.K * p.F, per = (int64_t)s.G * U;
    const int64_t iters = (tasks + per - 1) / per;
    const size_t lds = (size_t)kStageChunks * 16 * s.threads;
    const int grid =
        resident_grid((const void *)moe_gateup_tokens_kernel<F, B, U>, s.threads, lds, iters);
    hipLaunchKernelGGL((moe_gateup_tokens_kernel<F, B, U>), dim3(grid), dim3(s.threads), lds, st,
                       p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "moe_ffn_tokens: gate/up launch failed: %s",
                    hipGetErrorString(e));
    return QG_OK;
}

template <int B>
int dispatch_gateup_tokens_b(int fmt, const MoeParams &p, hipStream_t st) {
    constexpr int K45 = lw_k45(B), Q6 = lw_q6k(B), Q8 = lw_q80(B), Q4 = lw_q40(B);
    switch (fmt) {
    case QG_Q4_K: return launch_gateup_tokens<FmtQ4K<K45, true>, B>(p, st);
    case QG_Q5_K: return launch_gateup_tokens<FmtQ5K<K45, true>, B>(p, st);
    case QG_Q6_K: return launch_gateup_tokens<FmtQ6K<Q6, false>, B>(p, st);
    case QG_Q8_0: return launch_gateup_tokens<FmtQ80<Q8>, B>(p, st);
    case QG_Q4_0: return launch_gateup_tokens<FmtQ40<Q4>, B>(p, st);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn_tokens: gate/up format %d", fmt);
    }
}

// Tokens in groups of at most four, each group one launch of the B = 4
// kernel (its own routing, distinct experts and activations).  At B = 8 the
// tile is narrower (two waves per row group, one row per group and
// iteration) and the kernel ran 5x slower than two B = 4 groups, whose
// second pass re-reads the experts the groups share.
int dispatch_gateup_tokens(int fmt, const MoeParams &p0, hipStream_t st) {
    for (int t0 = 0; t0 < p0.T; t0 += 4) {
        MoeParams p = p0;
        p.T = p0.T - t0 < 4 ? p0.T - t0 : 4;
        p.x += (int64_t)t0 * p.H;
        p.logits += (int64_t)t0 * p.E;
        p.ws_sel += (int64_t)t0 * p.K;
        p.ws_w += (int64_t)t0 * p.K;
        p.act += (int64_t)t0 * p.K * p.F;
        if (p.sel_out) p.sel_out += (int64_t)t0 * p.K;
        if (p.w_out) p.w_out += (int64_t)t0 * p.K;
        const int rc = dispatch_gateup_tokens_b<4>(fmt, p, st);
        if (rc != QG_OK) return rc;
    }
    return QG_OK;
}

int dispatch_gateup(int fmt, const MoeParams &p, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_gateup<FmtQ4K<32, true>>(p, st);
    case QG_Q5_K: return launch_gateup<FmtQ5K<32, true>>(p, st);
    case QG_Q6_K: return launch_gateup<FmtQ6K<16, false>>(p, st);
    case QG_Q8_0: return launch_gateup<FmtQ80<32>>(p, st);
    case QG_Q4_0: return launch_gateup<FmtQ40<16>>(p, st);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn: gate/up format %d", fmt);
    }
}

int dispatch_down(int fmt, const MoeParams &p, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_down<FmtQ4K<32, true>>(p, st);
    case QG_Q5_K: return launch_down<FmtQ5K<32, true>>(p, st);
    case QG_Q6_K: return launch_down<FmtQ6K<16, false>>(p, st);
    case QG_Q8_0: return launch_down<FmtQ80<32>>(p, st);
    case QG_Q4_0: return launch_down<FmtQ40<16>>(p, st);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn: down format %d", fmt);
    }
}

}  // namespace

// ========================================================================= ABI

namespace {

// The fused add + RMSNorm in front of the chain (moe_ffn_norm): x and
// residual are then attn_out and hidden_in, the router kernel normalises.
struct NormStep {
    const float *gamma;
    double eps;
    float *normed;  // may be NULL
};

int moe_ffn_impl(const char *who, const float *x, const float *residual, float *y,
                 const float *router, int gate_fmt, const void *gate, int up_fmt, const void *up,
                 int down_fmt, const void *down, int64_t hidden, int64_t n_experts,
                 int64_t top_k, int64_t expert_dim, int32_t *sel_experts, float *sel_weights,
                 void *workspace, size_t workspace_bytes, void *stream, const NormStep *norm,
                 int64_t tokens = 1) {
    if (tokens < 1) return fail(QG_EINVAL, "%s: tokens must be positive", who);
    if (tokens > kMaxTokens)
        return fail(QG_EUNSUPPORTED, "%s: tokens must be in 1..%d", who, kMaxTokens);
    if (tokens > 1 && top_k > 0 && tokens * top_k > kMaxRoutes)
        return fail(QG_EUNSUPPORTED, "%s: tokens * top_k must be <= %d", who, kMaxRoutes);
    if (!x || !residual || !y || !router || !gate || !up || !down || !workspace)
        return fail(QG_EINVAL, "%s: x, residual, y, router, gate, up, down and workspace "
                               "must be non-NULL", who);
    if (hidden <= 0 || n_experts <= 0 || top_k <= 0 || expert_dim <= 0)
        return fail(QG_EINVAL, "%s: sizes must be positive", who);
    if (top_k > n_experts) return fail(QG_EINVAL, "%s: top_k %lld > n_experts %lld", who,
                                       (long long)top_k, (long long)n_experts);
    if (n_experts > kMaxExperts || top_k > kMaxTopK)
        return fail(QG_EUNSUPPORTED, "%s: n_experts <= %d and top_k <= %d", who, kMaxExperts,
                    kMaxTopK);
    if (hidden > 65536 || expert_dim > 65536)
        return fail(QG_EUNSUPPORTED, "%s: hidden and expert_dim must be <= 65536", who);
    const Geom gg = geom(gate_fmt), gu = geom(up_fmt), gd = geom(down_fmt);
    if (gg.elems == 0 || gu.elems == 0 || gd.elems == 0 || gate_fmt == QG_F32 ||
        up_fmt == QG_F32 || down_fmt == QG_F32)
        return fail(QG_EUNSUPPORTED, "%s: expert stacks must use a block format", who);
    if (gate_fmt != up_fmt)
        return fail(QG_EUNSUPPORTED, "%s: gate (%s) and up (%s) must share a format", who,
                    fmt_name(gate_fmt), fmt_name(up_fmt));
    if (hidden % gg.elems != 0 || expert_dim % gd.elems != 0)
        return fail(QG_EUNSUPPORTED, "%s: hidden must be a multiple of %d and expert_dim "
                                     "of %d", who, gg.elems, gd.elems);
    if (!aligned_to(gate, 2) || !aligned_to(up, 2) || !aligned_to(down, 2))
        return fail(QG_EINVAL, "%s: weight stacks must be 2-byte aligned", who);
    if (!aligned_to(x, 4) || !aligned_to(residual, 4) || !aligned_to(y, 4) ||
        !aligned_to(router, 4) || (sel_experts && !aligned_to(sel_experts, 4)) ||
        (sel_weights && !aligned_to(sel_weights, 4)))
        return fail(QG_EINVAL, "%s: float and int32 arrays must be 4-byte aligned", who);
    if (!aligned_to(workspace, 16)) return fail(QG_EINVAL, "%s: workspace not 16-byte aligned", who);
    if (!norm && y == x) return fail(QG_EINVAL, "%s: y must not alias x", who);
    if (norm) {
        if (!norm->gamma) return fail(QG_EINVAL, "%s: norm_weight must be non-NULL", who);
        if (!aligned_to(norm->gamma, 4) || (norm->normed && !aligned_to(norm->normed, 4)))
            return fail(QG_EINVAL, "%s: float arrays must be 4-byte aligned", who);
        if (!(norm->eps >= 0.0) || !std::isfinite(norm->eps))
            return fail(QG_EINVAL, "%s: eps must be finite and >= 0", who);
        const float *nd = norm->normed;
        if (nd && (nd == x || nd == residual || nd == y || nd == norm->gamma || nd == router))
            return fail(QG_EINVAL, "%s: normed must not alias another argument", who);
    }
    const WsLayout wl = ws_layout(n_experts, top_k, expert_dim, tokens);
    const size_t ws_need = wl.total + (norm ? align16(4 * (size_t)hidden) : 0);
    if (workspace_bytes < ws_need)
        return fail(QG_EINVAL, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes,
                    ws_need);
    const int64_t rbg = qg_row_bytes(gate_fmt, hidden), rbd = qg_row_bytes(down_fmt, expert_dim);
    const uint64_t gate_bytes = (uint64_t)n_experts * expert_dim * rbg;
    const uint64_t down_bytes = (uint64_t)n_experts * hidden * rbd;
    if (gate_bytes > 0xFFFFFFFFull || down_bytes > 0xFFFFFFFFull)
        return fail(QG_EUNSUPPORTED, "%s: each expert stack must be under 4 GiB", who);
    if (hidden % moe_cpt(gate_fmt) != 0 || expert_dim % moe_cpt(down_fmt) != 0)
        return fail(QG_EUNSUPPORTED, "%s: sizes do not tile", who);
    if (hidden / moe_cpt(gate_fmt) > 512 || top_k * (expert_dim / moe_cpt(down_fmt)) > 512)
        return fail(QG_EUNSUPPORTED, "%s: hidden or top_k * expert_dim too large", who);
    // several tokens: the gate/up tiles are the batch-4 GEMV's
    if (tokens > 1) {
        const int cpt4 = gemv_cpt(gate_fmt, 4, hidden);
        if (cpt4 == 0 || hidden % cpt4 != 0 || hidden / cpt4 > 512)
            return fail(QG_EUNSUPPORTED, "%s: hidden %lld too wide for several tokens", who,
                        (long long)hidden);
    }

    uint8_t *ws = (uint8_t *)workspace;
    MoeParams p{};
    p.x = x;
    p.residual = residual;
    p.y = y;
    p.gate = (const uint8_t *)gate;
    p.up = (const uint8_t *)up;
    p.down = (const uint8_t *)down;
    p.gate_bytes = gate_bytes;
    p.up_bytes = gate_bytes;
    p.down_bytes = down_bytes;
    p.rb_gate = (uint32_t)rbg;
    p.rb_down = (uint32_t)rbd;
    p.H = (int32_t)hidden;
    p.E = (int32_t)n_experts;
    p.K = (int32_t)top_k;
    p.F = (int32_t)expert_dim;
    p.T = (int32_t)tokens;
    p.logits = (const double *)(ws + wl.logits);
    p.ws_sel = (int32_t *)(ws + wl.sel);
    p.ws_w = (float *)(ws + wl.w);
    p.act = (float *)(ws + wl.act);
    p.sel_out = sel_experts;
    p.w_out = sel_weights;

    hipStream_t st = (hipStream_t)stream;
    if (norm) {
        // x = attn_out, residual = hidden_in: the router kernel forms
        // h = x + residual and its norm, the experts read xn (workspace),
        // the down kernel adds h = residual + x
        float *xn = (float *)(ws + wl.total);
        p.x = xn;
        p.residual2 = x;
        hipLaunchKernelGGL(moe_norm_router_kernel, dim3((unsigned)n_experts), dim3(64), 0, st,
                           router, x, residual, norm->gamma, norm->eps, (int)hidden,
                           (double *)(ws + wl.logits), xn, norm->normed);
    } else if (tokens > 1) {
        hipLaunchKernelGGL(moe_router_tokens_kernel, dim3((unsigned)n_experts), dim3(64), 0, st,
                           router, x, (int)tokens, (int)hidden, (int)n_experts,
                           (double *)(ws + wl.logits));
    } else {
        hipLaunchKernelGGL(moe_router_kernel, dim3((unsigned)n_experts), dim3(64), 0, st, router,
                           x, (int)hidden, (double *)(ws + wl.logits));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ELAUNCH, "%s: router launch failed: %s", who,
                                     hipGetErrorString(e));
    int rc = tokens > 1 ? dispatch_gateup_tokens(gate_fmt, p, st) : dispatch_gateup(gate_fmt, p, st);
    if (rc != QG_OK) return rc;
    rc = dispatch_down(down_fmt, p, st);
    if (rc != QG_OK) return rc;
    return ok();
}


}  // namespace

extern "C" {

int qg_block_elems(int fmt) { return geom(fmt).elems; }

int qg_block_bytes(int fmt) { return geom(fmt).bytes; }

int64_t qg_row_bytes(int fmt, int64_t cols) {
    const Geom g = geom(fmt);
    if (g.elems == 0 || cols <= 0 || cols % g.elems != 0) return -1;
    return (cols / g.elems) * g.bytes;
}

const char *qg_last_error(void) { return g_err; }

// Batches above 8 run as groups of 8 (see qgemv).
constexpr int kMaxBatch = 64;

int qgemv(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
          int batch, void *stream) {
    const Geom g = geom(fmt);
    if (g.elems == 0) return fail(QG_EUNSUPPORTED, "qgemv: unknown format %d", fmt);
    if (!W || !X || !Y) return fail(QG_EINVAL, "qgemv: W, X and Y must be non-NULL");
    if (rows <= 0 || cols <= 0)
        return fail(QG_EINVAL, "qgemv: rows (%lld) and cols (%lld) must be positive",
                    (long long)rows, (long long)cols);
    if (cols % g.elems != 0)
        return fail(QG_EUNSUPPORTED, "qgemv: %s needs cols to be a multiple of %d (got %lld)",
                    fmt_name(fmt), g.elems, (long long)cols);
    if (batch < 1 || batch > kMaxBatch)
        return fail(QG_EUNSUPPORTED, "qgemv: batch %d outside 1..%d", batch, kMaxBatch);
    if (!aligned_to(W, fmt == QG_F32 ? 4 : 2))
        return fail(QG_EINVAL, "qgemv: W is not %d-byte aligned", fmt == QG_F32 ? 4 : 2);
    if (!aligned_to(X, 4) || !aligned_to(Y, 4))
        return fail(QG_EINVAL, "qgemv: X and Y must be 4-byte aligned");
    if (rows >= ((int64_t)1 << 31)) return fail(QG_EUNSUPPORTED, "qgemv: rows must be < 2^31");
    if (cols > 65536) return fail(QG_EUNSUPPORTED, "qgemv: cols must be <= 65536");
    if (fmt == QG_F32 && cols % 4 != 0)
        return fail(QG_EUNSUPPORTED, "qgemv: F32 rows must be a multiple of 4 floats");
    const int64_t rb = qg_row_bytes(fmt, cols);
    hipStream_t st = (hipStream_t)stream;
    if (batch > 8) {
        // groups of up to 8 activation rows, one after another on the
        // stream; each group streams the weights again
        for (int b0 = 0; b0 < batch; b0 += 8) {
            const int nb = batch - b0 < 8 ? batch - b0 : 8;
            const int rc = qgemv(fmt, W, rows, cols, X + (int64_t)b0 * cols,
                                 Y + (int64_t)b0 * rows, nb, stream);
            if (rc != QG_OK) return rc;
        }
        return ok();
    }
    bool done = false;
    const int mrc = try_mx(fmt, W, rows, cols, X, Y, batch, rb, st, &done);
    if (done) return mrc == QG_OK ? ok() : mrc;
    // Batches too wide for VGPR-resident activations run as several narrower
    // launches over column slices of X and Y.
    int chunk = batch;
    while (chunk > 1 && !tiles_fit(fmt, chunk, cols)) chunk = chunk > 4 ? 4 : chunk / 2;
    if (!tiles_fit(fmt, chunk, cols))
        return fail(QG_EUNSUPPORTED, "qgemv: %lld columns of %s exceed the kernel's row width",
                    (long long)cols, fmt_name(fmt));
    const bool aligned = aligned_to(W, 4) && rb % 4 == 0;
    for (int b0 = 0; b0 < batch; b0 += chunk) {
        const int nb = batch - b0 < chunk ? batch - b0 : chunk;
        GemvParams p{};
        p.W = (const uint8_t *)W;
        p.X = X + (int64_t)b0 * cols;
        p.Y = Y + (int64_t)b0 * rows;
        p.rows = rows;
        p.w_bytes = (uint64_t)rows * (uint64_t)rb;
        p.row_bytes = (uint32_t)rb;
        p.cols = (uint32_t)cols;
        p.batch_x = (uint32_t)nb;
        const int rc = dispatch_gemv(fmt, nb, aligned, cols, p, st);
        if (rc != QG_OK) return rc;
    }
    return ok();
}

int qgemv_q8act(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
                void *stream) {
    const Geom g = geom(fmt);
    if (g.elems == 0 || fmt == QG_F32)
        return fail(QG_EUNSUPPORTED, "qgemv_q8act: format %d has no int8 path", fmt);
    if (!W || !X || !Y) return fail(QG_EINVAL, "qgemv_q8act: W, X and Y must be non-NULL");
    if (rows <= 0 || cols <= 0)
        return fail(QG_EINVAL, "qgemv_q8act: rows (%lld) and cols (%lld) must be positive",
                    (long long)rows, (long long)cols);
    if (cols % g.elems != 0)
        return fail(QG_EUNSUPPORTED, "qgemv_q8act: %s needs cols to be a multiple of %d (got %lld)",
                    fmt_name(fmt), g.elems, (long long)cols);
    if (!aligned_to(W, 2)) return fail(QG_EINVAL, "qgemv_q8act: W is not 2-byte aligned");
    if (!aligned_to(X, 4) || !aligned_to(Y, 4))
        return fail(QG_EINVAL, "qgemv_q8act: X and Y must be 4-byte aligned");
    if (rows >= ((int64_t)1 << 31))
        return fail(QG_EUNSUPPORTED, "qgemv_q8act: rows must be < 2^31");
    if (cols > 65536 || !tiles_fit(fmt, 1, cols))
        return fail(QG_EUNSUPPORTED, "qgemv_q8act: %lld columns of %s exceed the kernel's row "
                                     "width", (long long)cols, fmt_name(fmt));
    const int64_t rb = qg_row_bytes(fmt, cols);
    GemvParams p{};
    p.W = (const uint8_t *)W;
    p.X = X;
    p.Y = Y;
    p.rows = rows;
    p.w_bytes = (uint64_t)rows * (uint64_t)rb;
    p.row_bytes = (uint32_t)rb;
    p.cols = (uint32_t)cols;
    p.batch_x = 1;
    const int rc = dispatch_gemv_q8(fmt, aligned_to(W, 4) && rb % 4 == 0, p, (hipStream_t)stream);
    return rc == QG_OK ? ok() : rc;
}

size_t moe_ffn_workspace_bytes(int64_t n_experts, int64_t top_k, int64_t expert_dim) {
    if (n_experts <= 0 || top_k <= 0 || expert_dim <= 0 || top_k > n_experts) return 0;
    return ws_layout(n_experts, top_k, expert_dim).total;
}

int qg_route_topk(const double *logits, int64_t n_experts, int64_t top_k, int32_t *sel_experts,
                  float *sel_weights, void *stream) {
    if (!logits || !sel_experts || !sel_weights)
        return fail(QG_EINVAL, "qg_route_topk: logits, sel_experts and sel_weights are required");
    if (n_experts <= 0 || top_k <= 0 || top_k > n_experts)
        return fail(QG_EINVAL, "qg_route_topk: need 0 < top_k <= n_experts");
    if (n_experts > kMaxExperts || top_k > kMaxTopK)
        return fail(QG_EUNSUPPORTED, "qg_route_topk: n_experts <= %d and top_k <= %d",
                    kMaxExperts, kMaxTopK);
    if (!aligned_to(logits, 8) || !aligned_to(sel_experts, 4) || !aligned_to(sel_weights, 4))
        return fail(QG_EINVAL, "qg_route_topk: misaligned pointer");
    hipLaunchKernelGGL(route_topk_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, logits,
                       (int)n_experts, (int)top_k, (int *)sel_experts, sel_weights);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "qg_route_topk: launch failed: %s", hipGetErrorString(e));
    return ok();
}

int moe_ffn(const float *x, const float *residual, float *y, const float *router, int gate_fmt,
            const void *gate, int up_fmt, const void *up, int down_fmt, const void *down,
            int64_t hidden, int64_t n_experts, int64_t top_k, int64_t expert_dim,
            int32_t *sel_experts, float *sel_weights, void *workspace, size_t workspace_bytes,
            void *stream) {
    return moe_ffn_impl("moe_ffn", x, residual, y, router, gate_fmt, gate, up_fmt, up, down_fmt,
                        down, hidden, n_experts, top_k, expert_dim, sel_experts, sel_weights,
                        workspace, workspace_bytes, stream, nullptr);
}

size_t moe_ffn_tokens_workspace_bytes(int64_t tokens, int64_t n_experts, int64_t top_k,
                                      int64_t expert_dim) {
    if (tokens <= 0 || n_experts <= 0 || top_k <= 0 || expert_dim <= 0 || top_k > n_experts)
        return 0;
    return ws_layout(n_experts, top_k, expert_dim, tokens).total;
}

int moe_ffn_tokens(const float *x, const float *residual, float *y, const float *router,
                   int gate_fmt, const void *gate, int up_fmt, const void *up, int down_fmt,
                   const void *down, int64_t tokens, int64_t hidden, int64_t n_experts,
                   int64_t top_k, int64_t expert_dim, int32_t *sel_experts, float *sel_weights,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return moe_ffn_impl("moe_ffn_tokens", x, residual, y, router, gate_fmt, gate, up_fmt, up,
                        down_fmt, down, hidden, n_experts, top_k, expert_dim, sel_experts,
                        sel_weights, workspace, workspace_bytes, stream, nullptr, tokens);
}

size_t moe_ffn_norm_workspace_bytes(int64_t hidden, int64_t n_experts, int64_t top_k,
                                    int64_t expert_dim) {
    if (hidden <= 0 || n_experts <= 0 || top_k <= 0 || expert_dim <= 0 || top_k > n_experts)
        return 0;
    return ws_layout(n_experts, top_k, expert_dim).total + align16(4 * (size_t)hidden);
}

int moe_ffn_norm(const float *attn_out, const float *hidden_in, float *hidden_out,
                 const float *norm_weight, float eps, float *normed, const float *router,
                 int gate_fmt, const void *gate, int up_fmt, const void *up, int down_fmt,
                 const void *down, int64_t hidden, int64_t n_experts, int64_t top_k,
                 int64_t expert_dim, int32_t *sel_experts, float *sel_weights, void *workspace,
                 size_t workspace_bytes, void *stream) {
    const NormStep ns{norm_weight, (double)eps, normed};
    return moe_ffn_impl("moe_ffn_norm", attn_out, hidden_in, hidden_out, router, gate_fmt, gate,
                        up_fmt, up, down_fmt, down, hidden, n_experts, top_k, expert_dim,
                        sel_experts, sel_weights, workspace, workspace_bytes, stream, &ns);
}

}  // extern "C"
