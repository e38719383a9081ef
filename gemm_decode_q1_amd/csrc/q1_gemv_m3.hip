// Packed Q1 matmul kernels for 3 activation rows.
#include "q1_gemv.inc"

namespace q1 {
template hipError_t launch_gemv_m<3>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
}  // namespace q1
