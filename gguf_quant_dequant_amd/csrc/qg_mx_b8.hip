// qg_mx_b8.hip -- the matrix-core GEMV kernels for batch tiles of 8.
#include "qg_mx_host.hpp"

namespace qg {
namespace host {
template int try_mx_b<8>(int, const void *, int64_t, int64_t, const float *, float *, int,
                          int64_t, hipStream_t, bool *);
}  // namespace host
}  // namespace qg
