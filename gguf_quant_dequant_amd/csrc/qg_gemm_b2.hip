// qg_gemm_b2.hip -- the batched matrix-core kernel for 32 batch rows or fewer per launch.
#include "qg_gemm_host.hpp"

namespace qg {
namespace host {
template int gemm_b<2>(int, const void *, int64_t, int64_t, const float *, float *, int, int64_t,
                       hipStream_t);
}  // namespace host
}  // namespace qg
