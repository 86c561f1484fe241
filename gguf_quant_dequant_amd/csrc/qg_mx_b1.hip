// qg_mx_b1.hip -- the matrix-core GEMV kernels for batch tiles of 1.
#include "qg_mx_host.hpp"

namespace qg {
namespace host {
template int try_mx_b<1>(int, const void *, int64_t, int64_t, const float *, float *, int,
                          int64_t, hipStream_t, bool *);
}  // namespace host
}  // namespace qg
