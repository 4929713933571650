// Instantiations of the row-split workgroup GEMM (gemm_ns.h) for fp8 (E4M3) weights with per-row scales.
#include "gemm_ns.h"

namespace bdr {

hipError_t launch_ns_fp8(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
  switch (p.mt) {
    case 2: return launch_ns_one<uint8_t, 2, 0>(p, sa, st);
    case 3: return launch_ns_one<uint8_t, 3, 0>(p, sa, st);
    case 4: return launch_ns_one<uint8_t, 4, 0>(p, sa, st);
    case 5: return launch_ns_one<uint8_t, 5, 0>(p, sa, st);
    case 6: return launch_ns_one<uint8_t, 6, 0>(p, sa, st);
    case 7: return launch_ns_one<uint8_t, 7, 0>(p, sa, st);
    case 8: return launch_ns_one<uint8_t, 8, 0>(p, sa, st);
    case 9: return launch_ns_one<uint8_t, 9, 0>(p, sa, st);
    case 10: return launch_ns_one<uint8_t, 10, 0>(p, sa, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bdr
