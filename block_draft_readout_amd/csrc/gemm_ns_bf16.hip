// Instantiations of the row-split workgroup GEMM (gemm_ns.h) for bf16 weights.
#include "gemm_ns.h"

namespace bdr {

hipError_t launch_ns_bf16(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
  switch (p.mt) {
    case 2: return launch_ns_one<uint16_t, 2>(p, sa, st);
    case 3: return launch_ns_one<uint16_t, 3>(p, sa, st);
    case 4: return launch_ns_one<uint16_t, 4>(p, sa, st);
    case 5: return launch_ns_one<uint16_t, 5>(p, sa, st);
    case 6: return launch_ns_one<uint16_t, 6>(p, sa, st);
    case 7: return launch_ns_one<uint16_t, 7>(p, sa, st);
    case 8: return launch_ns_one<uint16_t, 8>(p, sa, st);
    case 9: return launch_ns_one<uint16_t, 9>(p, sa, st);
    case 10: return launch_ns_one<uint16_t, 10>(p, sa, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bdr
