// qg_gemv_b8.hip -- the VALU GEMV kernels at batch 8.
#include "qg_gemv_host.hpp"

namespace qg {
namespace host {
template int dispatch_gemv_b<8>(int, bool, int, const GemvParams &, hipStream_t);
}  // namespace host
}  // namespace qg
