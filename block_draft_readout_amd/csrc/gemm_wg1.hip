// Instantiation of the shared-visit workgroup GEMM kernel (fp32 operands) for
// waves holding 1 A row tile(s).
#include "gemm_kernels.h"

namespace bdr {

hipError_t launch_wg_mtw1(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
  return p.nt == 8 ? launch_wg_one<float, 1, 8>(p, sa, st) : hipErrorInvalidValue;
}

}  // namespace bdr
