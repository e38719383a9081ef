// Packed Q1 matmul kernels for 1 activation row.
#include "q1_gemv.inc"

namespace q1 {
template hipError_t launch_gemv_m<1>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
}  // namespace q1
