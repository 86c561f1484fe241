// qg_gemv_b1.hip -- the VALU GEMV kernels at batch 1.
#include "qg_gemv_host.hpp"

namespace qg {
namespace host {
template int dispatch_gemv_b<1>(int, bool, int, const GemvParams &, hipStream_t);
}  // namespace host
}  // namespace qg
