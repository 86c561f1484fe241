// qg_moe_q8.hip -- the MoE FFN kernels on int8-quantised activations
// (moe_ffn_q8act): the gate/up and down kernels of qg_moe.hip with each
// format wrapped by q8a::Q8A, so a lane quantises its tile of x (gate/up)
// or of the SwiGLU activations (down) per 16-column group and meets the
// weight codes in integer dot products.
#include "qg_moe_host.hpp"
#include "qg_q8act.hpp"

namespace qg {
namespace host {

int dispatch_gateup_q8(int fmt, const MoeParams &p, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_gateup<q8a::Q8A<FmtQ4K<32, true>>>(p, st);
    case QG_Q5_K: return launch_gateup<q8a::Q8A<FmtQ5K<32, true>>>(p, st);
    case QG_Q6_K: return launch_gateup<q8a::Q8A<FmtQ6K<16, false>>>(p, st);
    case QG_Q8_0: return launch_gateup<q8a::Q8A<FmtQ80<32>>>(p, st);
    case QG_Q4_0: return launch_gateup<q8a::Q8A<FmtQ40<16>>>(p, st);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn_q8act: gate/up format %d", fmt);
    }
}

int dispatch_down_q8(int fmt, const MoeParams &p, hipStream_t st) {
    switch (fmt) {
    case QG_Q4_K: return launch_down<q8a::Q8A<FmtQ4K<32, true>>>(p, st);
    case QG_Q5_K: return launch_down<q8a::Q8A<FmtQ5K<32, true>>>(p, st);
    case QG_Q6_K: return launch_down<q8a::Q8A<FmtQ6K<16, false>>>(p, st);
    case QG_Q8_0: return launch_down<q8a::Q8A<FmtQ80<32>>>(p, st);
    case QG_Q4_0: return launch_down<q8a::Q8A<FmtQ40<16>>>(p, st);
    default: return fail(QG_EUNSUPPORTED, "moe_ffn_q8act: down format %d", fmt);
    }
}

}  // namespace host
}  // namespace qg
