// Instantiations of the row-split workgroup GEMM (gemm_ns.h) with the LDS ring
// for fp8 (E4M3) weights with per-row scales: every A row-tile count with each
// ring depth of kNsLeanRings.
#include "gemm_ns.h"

namespace bdr {

hipError_t launch_ns_fp8(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
  if (p.reg) return launch_ns_fp8_reg(p, sa, st);   // the register ring (gemm_ns_fp8_reg.hip)
#define BDR_NS(MT, R) \
  if (p.mt == MT && p.ring == R) return launch_ns_one<uint8_t, MT, R>(p, sa, st);
  BDR_NS(2, 8) BDR_NS(2, 5) BDR_NS(2, 3)
  BDR_NS(3, 7) BDR_NS(3, 5) BDR_NS(3, 3)
  BDR_NS(4, 6) BDR_NS(4, 5) BDR_NS(4, 3)
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
