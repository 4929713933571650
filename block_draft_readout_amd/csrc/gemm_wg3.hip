// Instantiations of the workgroup streaming GEMM kernel for waves holding
// 3 A row tile(s).
#include "gemm_kernels.h"

namespace bdr {

hipError_t launch_wg_mtw3(const GemmPlan& p, const StreamArgs& sa, bool bf16, hipStream_t st) {
  if (!bf16) return p.nt == 8 ? launch_wg_one<float, 3, 8>(p, sa, st) : hipErrorInvalidValue;
  switch (p.nt) {
    case 8: return launch_wg_one<uint16_t, 3, 8>(p, sa, st);
    case 12: return launch_wg_one<uint16_t, 3, 12>(p, sa, st);
    default: return hipErrorInvalidValue;   // no instantiation for this tile count
  }
}

}  // namespace bdr
