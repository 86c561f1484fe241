// qg_gemv_b5.hip -- the VALU GEMV kernels at batch 5.
#include "qg_gemv_host.hpp"

namespace qg {
namespace host {
template int dispatch_gemv_b<5>(int, bool, int, const GemvParams &, hipStream_t);
}  // namespace host
}  // namespace qg
