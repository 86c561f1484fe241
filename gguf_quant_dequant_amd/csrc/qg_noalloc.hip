// qg_noalloc.hip -- moe_ffn_noalloc: moe_ffn with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The kernels are moe_ffn's.
//
// `scratch` below is a device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code
// its name is only a host-side stand-in, so it is never passed to a kernel
// or a copy directly.  The first call on a device looks up that device's
// address with hipGetSymbolAddress (with the device current) and keeps it;
// every later call on that device passes the kept address as moe_ffn's
// workspace.  moe_ffn needs no initial contents in its workspace, so
// nothing is cleared.  All calls on one GPU share the array and it keeps the
// last call's contents: calls that overlap on one GPU (different streams,
// or different host threads without ordering) race on it.
#include <mutex>

#include "qg_host.hpp"

namespace {

// Largest workspace a call may use: 1 MiB.  The Qwen3-30B-A3B MoE shape
// (128 experts, top 8, expert_dim 768) needs 26,240 bytes.
constexpr size_t kScratchBytes = (size_t)1 << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (g_mu)

// Address of this device's copy of `scratch` (the device current on the
// calling thread, which must be the device of the caller's stream).
int scratch_address(void **out) {
    int dev = -1;
    const hipError_t e0 = hipGetDevice(&dev);
    if (e0 != hipSuccess)
        return qg::host::fail(QG_ELAUNCH, "moe_ffn_noalloc: hipGetDevice failed: %s",
                              hipGetErrorString(e0));
    if (dev < 0 || dev >= kMaxDevices)
        return qg::host::fail(QG_EUNSUPPORTED, "moe_ffn_noalloc: device %d beyond the %d "
                                               "supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return qg::host::fail(QG_ELAUNCH, "moe_ffn_noalloc: hipGetSymbolAddress of the "
                                              "scratch array failed on device %d: %s",
                                  dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QG_OK;
}

}  // namespace

extern "C" int moe_ffn_noalloc(const float *x, const float *residual, float *y,
                               const float *router, int gate_fmt, const void *gate, int up_fmt,
                               const void *up, int down_fmt, const void *down, int64_t hidden,
                               int64_t n_experts, int64_t top_k, int64_t expert_dim,
                               int32_t *sel_experts, float *sel_weights, void *stream) {
    const size_t need = moe_ffn_workspace_bytes(n_experts, top_k, expert_dim);
    if (need > kScratchBytes)
        return qg::host::fail(QG_EUNSUPPORTED,
                              "moe_ffn_noalloc: n_experts %lld, top_k %lld, expert_dim %lld need "
                              "%zu bytes of workspace; the library's scratch array holds %zu",
                              (long long)n_experts, (long long)top_k, (long long)expert_dim,
                              need, kScratchBytes);
    // need == 0: invalid sizes, refused by moe_ffn's own validation below
    void *ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != QG_OK) return rc;
    return moe_ffn(x, residual, y, router, gate_fmt, gate, up_fmt, up, down_fmt, down, hidden,
                   n_experts, top_k, expert_dim, sel_experts, sel_weights, ws, kScratchBytes,
                   stream);
}
