// qg_gemv_b6.hip -- the VALU GEMV kernels at batch 6.
#include "qg_gemv_host.hpp"

namespace qg {
namespace host {
template int dispatch_gemv_b<6>(int, bool, int, const GemvParams &, hipStream_t);
}  // namespace host
}  // namespace qg
