// qg_host.hpp -- host-side helpers shared by the translation units of
// libqgemv.so: error reporting, block geometry, occupancy-capped grids, row
// group shapes, tile widths, and the entry points each unit defines.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "../../include/qgemv.h"
#include "qg_kernels.hpp"


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
// Waves per expert row in the MoE router kernel (1, 2, 4 or 8).
#ifndef QG_ROUTER_WAVES
#define QG_ROUTER_WAVES 1
#endif
// 1: batch-1 Q6_K rows of up to 4096 columns run on the matrix cores
// (int8 digit-plane products, qg_q6mx.hpp); 0: on the VALU kernel.
#ifndef QG_Q6_MX
#define QG_Q6_MX 1
#endif
// Batch rows up to which Q6_K runs that kernel (two rows: the weights read
// once for both), on matrices of at least QG_Q6_MX_ROWS_BYTES.
#ifndef QG_Q6_MX_ROWS
#define QG_Q6_MX_ROWS 2
#endif
#ifndef QG_Q6_MX_ROWS_BYTES
#define QG_Q6_MX_ROWS_BYTES (16ull << 20)
#endif
// Batch rows up to which Q6_K matrices of at least QG_Q6_MX_PAIRS_BYTES run
// it as launches of two rows (and one).
#ifndef QG_Q6_MX_PAIRS
#define QG_Q6_MX_PAIRS 4
#endif
#ifndef QG_Q6_MX_PAIRS_BYTES
#define QG_Q6_MX_PAIRS_BYTES (128ull << 20)
#endif

namespace qg {
namespace host {

inline thread_local char g_err[512] = "";
// The arithmetic of the last qgemv / qgemv_q8act call on this thread that
// enqueued work (qg_last_kernel).
inline thread_local const char *g_kernel = "";

inline int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

inline int ok() {
    g_err[0] = '\0';
    return QG_OK;
}

// Called by every entry point after its validation, before its first
// launch: an error the HIP runtime still holds from earlier work on this
// thread is reported (and thereby cleared) as that, with nothing launched,
// instead of surfacing after this call's launch as if the launch had failed.
inline int no_pending_error(const char *who) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "%s: nothing launched: the HIP runtime holds an error from earlier "
                                "work on this thread: %s",
                    who, hipGetErrorString(e));
    return QG_OK;
}

struct Geom {
    int elems, bytes;
};

inline Geom geom(int fmt) {
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

inline const char *fmt_name(int fmt) {
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
inline int device_cus() {
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
inline int resident_per_cu(const void *fn, int threads, size_t lds) {
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
inline int resident_grid(const void *fn, int threads, size_t lds, int64_t blocks) {
    const int64_t cap = (int64_t)device_cus() * resident_per_cu(fn, threads, lds);
    return (int)(blocks < cap ? blocks : cap);
}

inline bool aligned_to(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Row-group shape for `tiles` tiles per row: lanes per group inside one wave
// (power of two), or S whole waves; G groups per workgroup; block threads.
struct Shape {
    int lpr, S, G, threads;
};

inline bool shape_for(int tiles, Shape *s) {
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
inline int gemv_cpt(int fmt, int B, int64_t cols) {
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

inline bool tiles_fit(int fmt, int B, int64_t cols) {
    const int cpt = gemv_cpt(fmt, B, cols);
    if (cpt == 0) return false;
    return (cols / cpt) <= 512;
}

// ------------------------------------------------------------------- MoE

inline size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

struct WsLayout {
    size_t logits, sel, w, act, total;
};

// Sections for T tokens: f64 logits [T][E], int32 routes [T][K], f32
// weights [T][K], f32 activations [T][K][F], each 16-byte aligned.
inline WsLayout ws_layout(int64_t E, int64_t K, int64_t F, int64_t T = 1) {
    WsLayout l;
    l.logits = 0;
    l.sel = align16(8 * (size_t)(T * E));
    l.w = l.sel + align16(4 * (size_t)(T * K));
    l.act = l.w + align16(4 * (size_t)(T * K));
    l.total = l.act + align16(4 * (size_t)(T * K) * (size_t)F);
    return l;
}

// columns per tile for the B = 1 kernels of the MoE chain
inline int moe_cpt(int fmt) {
    switch (fmt) {
    case QG_Q4_K:
    case QG_Q5_K:
    case QG_Q6_K: return 64;
    case QG_Q8_0:
    case QG_Q4_0: return 32;
    default: return 0;
    }
}

// Defined in their own translation units (compiled in parallel).
template <int B>
int dispatch_gemv_b(int fmt, bool aligned, int cpt, const GemvParams &p, hipStream_t st);
int dispatch_gemv_q8(int fmt, bool aligned, const GemvParams &p, hipStream_t st);
template <int B>
int try_mx_b(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
             int batch, int64_t rb, hipStream_t st, bool *done);
template <int NB>
int gemm_b(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
           int batch, int64_t rb, hipStream_t st);
int dispatch_gateup(int fmt, const MoeParams &p, hipStream_t st);
int dispatch_down(int fmt, const MoeParams &p, hipStream_t st);
int dispatch_gateup_q8(int fmt, const MoeParams &p, hipStream_t st);
int dispatch_down_q8(int fmt, const MoeParams &p, hipStream_t st);
int try_q6mx(const GemvParams &p, int nb, hipStream_t st, bool *done);
int ws_kg(int64_t rows, int64_t cols, int batch);
bool gemm_ks2_fits(int fmt, int64_t rows, int64_t cols, int batch);
bool ws_uses_qgemv(int64_t rows, int64_t cols, int batch);
int moe_gateup_ws(int fmt, const uint8_t *gate, const uint8_t *up, uint64_t stack_bytes,
                  int64_t rb, int H, int F, int K, int T, int E, const float *x,
                  const double *logits, bool routed, int32_t *sel, float *rw,
                  int32_t *sel_out, float *w_out, float *act, hipStream_t st);
int gemm_ks2(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
             int batch, int64_t rb, hipStream_t st);
int gemm_ws(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
            int batch, int64_t rb, float *part, hipStream_t st);

}  // namespace host
}  // namespace qg
