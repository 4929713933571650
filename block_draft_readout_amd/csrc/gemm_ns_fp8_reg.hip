// Instantiations of the row-split workgroup GEMM (gemm_ns.h) with the register
// ring for fp8 (E4M3) weights, row-major with per-row scales (K-split plans:
// the fc): every A row-tile count from kNsRegMinMt (5) on with each ring depth
// of kNsLeanRings.
#include "gemm_ns.h"

namespace bdr {

hipError_t launch_ns_fp8_reg(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
#define BDR_NS(MT, R) \
  if (p.mt == MT && p.ring == R) return launch_ns_one<uint8_t, MT, R, true>(p, sa, st);
  BDR_NS(5, 6) BDR_NS(5, 5) BDR_NS(5, 3)
  BDR_NS(6, 6) BDR_NS(6, 5) BDR_NS(6, 3)
  BDR_NS(7, 5) BDR_NS(7, 3)
  BDR_NS(8, 5) BDR_NS(8, 3)
  BDR_NS(9, 4) BDR_NS(9, 3)
  BDR_NS(10, 3)
#undef BDR_NS
  return hipErrorInvalidValue;
}

}  // namespace bdr
