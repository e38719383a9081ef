// Packed Q1 matmul kernels for 6 activation rows.
#include "q1_gemv.inc"

namespace q1 {
template hipError_t launch_gemv_m<6>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
}  // namespace q1
