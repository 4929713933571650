// Instantiations of the workgroup streaming GEMM kernel for waves holding
// 1 A row tile(s).
#include "gemm_kernels.h"

namespace bdr {

hipError_t launch_wg_mtw1(const GemmPlan& p, const StreamArgs& sa, bool bf16, hipStream_t st) {
  if (!bf16) return p.nt == 8 ? launch_wg_one<float, 1, 8>(p, sa, st) : hipErrorInvalidValue;
  switch (p.nt) {
    case 8: return launch_wg_one<uint16_t, 1, 8>(p, sa, st);
    case 16: return launch_wg_one<uint16_t, 1, 16>(p, sa, st);
    case 24: return launch_wg_one<uint16_t, 1, 24>(p, sa, st);
    case 32: return launch_wg_one<uint16_t, 1, 32>(p, sa, st);
    case 40: return launch_wg_one<uint16_t, 1, 40>(p, sa, st);
    default: return hipErrorInvalidValue;   // no instantiation for this tile count
  }
}

}  // namespace bdr
