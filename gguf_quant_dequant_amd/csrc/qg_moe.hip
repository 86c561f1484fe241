// qg_moe.hip -- launch of the MoE FFN kernels (gate/up + SwiGLU, down +
// residual).
#include "qg_moe_host.hpp"

namespace qg {
namespace host {

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

}  // namespace host
}  // namespace qg
