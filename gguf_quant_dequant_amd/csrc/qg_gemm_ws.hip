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

// Two column ranges inside each workgroup of 4 tiles (added in LDS) for
// tall matrices (qgemv at batch 2..32, qgemv_ws at 2..16): at least QG_KS2_MIN_WGS such
// workgroups (one per CU of a 256-CU part, and more) and 4 chunks per row,
// so that no range is split across workgroups.  Measured at batch 4 / 8,
// cold weights: Q5_K 14336 x 4096 18.4 / 18.9 us with 8 tiles per
// workgroup and two ranges across workgroups, 16.7 / 18.0 us with the two
// ranges inside; Q4_0 4096 x 14336 (64 such workgroups) slower with them,
// 18.6 / 18.7 -> 18.9 / 20.5 us, so short matrices keep the split across
// workgroups.
#ifndef QG_KS2_MIN_WGS
#define QG_KS2_MIN_WGS 192
#endif
// The batch rows up to which qgemv_ws takes the two-range kernel on such
// matrices (qgemv takes it for every launch of up to 32 rows).  Above 8
// rows the operands need two or four planes per image, which raises the
// kernel to ~155 (16 rows) and ~235 VGPRs (32 rows); against qgemm_kernel
// it still wins (Q5_K 14336 x 4096 at batch 12 / 16 / 24 / 32: 32.2 /
// 36.9 / 53.6 / 63.1 -> 23.3 / 24.6 / 34.0 / 36.8 us; lm_head 151936 x
// 2048 at batch 16 / 32: 183 / 309 -> 158 / 227 us), and against the split
// across workgroups up to 16 rows (batch 12 / 16: 23.8 / 25.1 -> 23.1 /
// 24.6 us; batch 32: 34.8 -> 36.9 us).
#ifndef QG_KS2_WS_MAXB
#define QG_KS2_WS_MAXB 16
#endif
static bool ks2_shape(int64_t rows, int64_t cols) {
    const int64_t tiles = (rows + gm::kTileRows - 1) / gm::kTileRows;
    const int64_t groups = (tiles + gw::kWaves / 2 - 1) / (gw::kWaves / 2);
    const int64_t nchunks = (cols + gm::kChunk - 1) / gm::kChunk;
    return QG_KS2_MIN_WGS > 0 && groups >= QG_KS2_MIN_WGS && nchunks >= 4;
}
static int ws_ks(int64_t rows, int64_t cols, int batch) {
    return batch <= QG_KS2_WS_MAXB && ks2_shape(rows, cols) ? 2 : 1;
}

// Column ranges across workgroups per group of tiles: as many as keep the
// grid within QG_WS_WGS workgroups.  Independent of the device, so the
// workspace size is known on the host before any call.
int ws_kg(int64_t rows, int64_t cols, int batch) {
    const int ks = ws_ks(rows, cols, batch), tpg = gw::kWaves / ks;
    const int64_t tiles = (rows + gm::kTileRows - 1) / gm::kTileRows;
    const int64_t groups = (tiles + tpg - 1) / tpg;
    const int64_t nchunks = (cols + gm::kChunk - 1) / gm::kChunk;
    int64_t kg = QG_WS_WGS / groups;
    const int64_t cap = nchunks / (QG_WS_MIN_CHUNKS * ks);
    if (kg > cap) kg = cap;
    if (kg < 1) kg = 1;
    return (int)kg;
}

namespace {

template <class F, int MODE, bool RA, int KS = 1>
int launch_ws_t(const gw::WsParams &p, hipStream_t st) {
    constexpr int U = gemm_units(F::CHUNK);
    auto kern = gw::qgemm_ws_kernel<F, MODE, RA, U, KS>;
    const size_t lds = gw::ws_lds_bytes<MODE, KS>(p.slot);
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
    const int64_t groups = ((int64_t)p.tiles + gw::kWaves / KS - 1) / (gw::kWaves / KS);
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

// KS = 2: two column ranges inside each workgroup of 4 tiles and no split
// across workgroups (no workspace; batch <= 32).
template <class F, int KS = 1>
int launch_ws(const void *W, int64_t rows, int64_t cols, const float *X, float *Y, int batch,
              int64_t rb, float *part, int kg, hipStream_t st) {
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
    p.kg = kg;
    p.nu = gemm_nu(F::CHUNK);
    p.slot = 16u * (uint32_t)(p.nu | 1);
    // 4-byte-aligned fields in LDS when every row and chunk starts at a
    // multiple of 4 bytes
    const bool ra = !(F::CHUNK % 4 == 0 && rb % 4 == 0 && aligned_to(W, 4));
    if constexpr (KS == 2) {
        if constexpr (F::CHUNK % 4 == 0) {
            if (!ra) {
                if (batch <= 8) return launch_ws_t<F, 0, false, 2>(p, st);
                if (batch <= 16) return launch_ws_t<F, 1, false, 2>(p, st);
                return launch_ws_t<F, 2, false, 2>(p, st);
            }
        }
        if (batch <= 8) return launch_ws_t<F, 0, true, 2>(p, st);
        if (batch <= 16) return launch_ws_t<F, 1, true, 2>(p, st);
        return launch_ws_t<F, 2, true, 2>(p, st);
    }
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

// qgemv takes the two-range kernel where qgemv_ws would (no workspace is
// needed there); shorter matrices keep qgemm8_kernel.
// qgemv_ws at batch 2..8 runs qgemv's kernels instead when its own kernel
// would split rows of at most 16 chunks across workgroups: there the
// second kernel that adds the column ranges costs more than qgemm8_kernel
// loses by sharing no activations (A/B on one box, batch 2 / 8: Q4_K 4096 x
// 4096 10.1 / 10.6 us against 7.9 / 8.8, Q6_K 9.9 / 12.5 against 9.4 /
// 10.1, Q8_0 11.2 / 11.8 against 8.5 / 9.4); with more chunks the shared
// activations win (Q4_0 4096 x 14336, 56 chunks: 17.0 / 17.7 against 18.3
// / 22.8 us).
bool ws_uses_qgemv(int64_t rows, int64_t cols, int batch) {
    const int64_t nchunks = (cols + gm::kChunk - 1) / gm::kChunk;
    return batch <= 8 && nchunks <= 16 && ws_ks(rows, cols, batch) == 1 &&
           ws_kg(rows, cols, batch) > 1;
}

// LDS of the two-range kernel for a format and batch: at 17-32 rows four
// operand planes per image (128 KiB of images) leave too little room for
// the weight slots of some formats (Q8_0).
static size_t ks2_lds(int fmt, int batch) {
    int chunk = 0;
    switch (fmt) {
    case QG_Q4_K: chunk = gm::GK45<false>::CHUNK; break;
    case QG_Q5_K: chunk = gm::GK45<true>::CHUNK; break;
    case QG_Q6_K: chunk = gm::GQ6K::CHUNK; break;
    case QG_Q8_0: chunk = gm::GQ80::CHUNK; break;
    case QG_Q4_0: chunk = gm::GQ40::CHUNK; break;
    default: return ~(size_t)0;
    }
    const uint32_t slot = 16u * (uint32_t)(gemm_nu(chunk) | 1);
    return batch <= 8 ? gw::ws_lds_bytes<0, 2>(slot)
                      : batch <= 16 ? gw::ws_lds_bytes<1, 2>(slot) : gw::ws_lds_bytes<2, 2>(slot);
}

bool gemm_ks2_fits(int fmt, int64_t rows, int64_t cols, int batch) {
    return fmt != QG_F32 && batch >= 2 && batch <= 32 && ks2_shape(rows, cols) &&
           ks2_lds(fmt, batch) <= (size_t)device_lds_max();
}

int gemm_ks2(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
             int batch, int64_t rb, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_ws<gm::GK45<false>, 2>(W, rows, cols, X, Y, batch, rb, nullptr, 1, st);
    case QG_Q5_K: return launch_ws<gm::GK45<true>, 2>(W, rows, cols, X, Y, batch, rb, nullptr, 1, st);
    case QG_Q6_K: return launch_ws<gm::GQ6K, 2>(W, rows, cols, X, Y, batch, rb, nullptr, 1, st);
    case QG_Q8_0: return launch_ws<gm::GQ80, 2>(W, rows, cols, X, Y, batch, rb, nullptr, 1, st);
    case QG_Q4_0: return launch_ws<gm::GQ40, 2>(W, rows, cols, X, Y, batch, rb, nullptr, 1, st);
    default: return fail(QG_EUNSUPPORTED, "qgemv: format %d has no matrix-core path", fmt);
    }
}

// The gate and up products of T <= 8 MoE tokens on the shared-activation
// kernel: every workgroup routes the tokens (or, when routed, reads the
// routes done ahead), then takes 4 pairs of gate / up tiles of the distinct experts
// (at most T * K of them) with SwiGLU in the epilogue.
template <class F>
int launch_moe_ws(const uint8_t *gate, const uint8_t *up, uint64_t stack_bytes, int64_t rb,
                  int H, int F_, int K, int T, int E, const float *x, const double *logits,
                  bool routed, int32_t *sel, float *rw, int32_t *sel_out, float *w_out,
                  float *act, hipStream_t st) {
    gw::WsParams p{};
    p.W = gate;
    p.W2 = up;
    p.X = x;
    p.w_bytes = stack_bytes;
    p.row_bytes = (uint32_t)rb;
    p.cols = (uint32_t)H;
    p.batch = T;
    p.nchunks = (int32_t)((H + gm::kChunk - 1) / gm::kChunk);
    p.last_nkb = (int32_t)(((H - 1) % gm::kChunk) / 32 + 1);
    p.kg = 1;
    p.nu = gemm_nu(F::CHUNK);
    p.slot = 16u * (uint32_t)(p.nu | 1);
    p.logits = logits;
    p.routed = routed ? 1 : 0;
    p.sel = sel;
    p.rw = rw;
    p.sel_out = sel_out;
    p.w_out = w_out;
    p.act = act;
    p.E = E;
    p.F = F_;
    p.K = K;
    p.tpe = F_ / gm::kTileRows;
    // every distinct expert's gate and up tiles, for the largest possible
    // count of distinct experts; workgroups past the actual count return
    const int64_t pairs = (int64_t)T * K * p.tpe;
    p.tiles = (int32_t)(2 * pairs);
    const int64_t grid = (pairs + gw::kWaves / 2 - 1) / (gw::kWaves / 2);
    const bool ra = !(F::CHUNK % 4 == 0 && rb % 4 == 0 && aligned_to(gate, 4) && aligned_to(up, 4));
    constexpr int U = gemm_units(F::CHUNK);
    auto kern = ra ? gw::qgemm_ws_kernel<F, 0, true, U, 1, true>
                   : gw::qgemm_ws_kernel<F, 0, F::CHUNK % 4 != 0, U, 1, true>;
    // the dynamic LDS doubles as the routing's E words of scratch
    const size_t lds = std::max(gw::ws_lds_bytes<0, 1>(p.slot), (size_t)4 * E);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(gw::kThreads), lds, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(QG_ELAUNCH, "moe_ffn_tokens: gate/up launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

int moe_gateup_ws(int fmt, const uint8_t *gate, const uint8_t *up, uint64_t stack_bytes,
                  int64_t rb, int H, int F, int K, int T, int E, const float *x,
                  const double *logits, bool routed, int32_t *sel, float *rw,
                  int32_t *sel_out, float *w_out, float *act, hipStream_t st) {
#define QG_MOE_WS_CASE(FM)                                                                   \
    return launch_moe_ws<FM>(gate, up, stack_bytes, rb, H, F, K, T, E, x, logits, routed, sel,   \
                             rw, sel_out, w_out, act, st)
    switch (fmt) {
    case QG_Q4_K: QG_MOE_WS_CASE(gm::GK45<false>);
    case QG_Q5_K: QG_MOE_WS_CASE(gm::GK45<true>);
    case QG_Q6_K: QG_MOE_WS_CASE(gm::GQ6K);
    case QG_Q8_0: QG_MOE_WS_CASE(gm::GQ80);
    case QG_Q4_0: QG_MOE_WS_CASE(gm::GQ40);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn_tokens: gate/up format %d", fmt);
    }
#undef QG_MOE_WS_CASE
}

int gemm_ws(int fmt, const void *W, int64_t rows, int64_t cols, const float *X, float *Y,
            int batch, int64_t rb, float *part, hipStream_t st) {
    const int kg = ws_kg(rows, cols, batch);
    const bool two = ws_ks(rows, cols, batch) == 2;
#define QG_WS_CASE(F)                                                                        \
    return two ? launch_ws<F, 2>(W, rows, cols, X, Y, batch, rb, part, kg, st)              \
               : launch_ws<F, 1>(W, rows, cols, X, Y, batch, rb, part, kg, st)
    switch (fmt) {
    case QG_Q4_K: QG_WS_CASE(gm::GK45<false>);
    case QG_Q5_K: QG_WS_CASE(gm::GK45<true>);
    case QG_Q6_K: QG_WS_CASE(gm::GQ6K);
    case QG_Q8_0: QG_WS_CASE(gm::GQ80);
    case QG_Q4_0: QG_WS_CASE(gm::GQ40);
    default: return fail(QG_EUNSUPPORTED, "qgemv_ws: format %d has no matrix-core path", fmt);
    }
#undef QG_WS_CASE
}

}  // namespace host
}  // namespace qg
