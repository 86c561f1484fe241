// qg_gemv_q8.hip -- the int8-activation GEMV kernels (batch 1).
#include "qg_gemv_host.hpp"
#include "qg_q8act.hpp"

namespace qg {
namespace host {

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

}  // namespace host
}  // namespace qg
