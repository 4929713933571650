// Instantiations of the row-split workgroup GEMM (gemm_ns.h) with the register
// ring, for bf16 weights in the packed layout: every A row-tile count from
// kNsRegMinMt (5) on with each ring depth of kNsLeanRings (fewer row tiles
// take the LDS ring, gemm_ns_bf16.hip).
#include "gemm_ns.h"

namespace bdr {

hipError_t launch_ns_bf16_packed(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
#define BDR_NS(MT, R) \
  if (p.mt == MT && p.ring == R) return launch_ns_one<uint16_t, MT, R, true>(p, sa, st);
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
