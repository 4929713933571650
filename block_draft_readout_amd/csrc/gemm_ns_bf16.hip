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

// the fc (mt1 = mt0 or mt0 + 1 row tiles) beside the LM head (mt0 row tiles)
hipError_t launch_ns_pair_bf16(int mt0, int mt1, const StreamArgs& a0, const StreamArgs& a1,
                               unsigned n0, unsigned n1, hipStream_t st) {
  const bool same = mt1 == mt0;
  if (!same && mt1 != mt0 + 1) return hipErrorInvalidValue;
#define BDR_PAIR(m)                                                                    \
  case m:                                                                              \
    return same ? launch_ns_pair_one<uint16_t, m, m>(a0, a1, n0, n1, st)               \
                : launch_ns_pair_one<uint16_t, m, m + 1>(a0, a1, n0, n1, st);
  switch (mt0) {
    BDR_PAIR(2)
    BDR_PAIR(3)
    BDR_PAIR(4)
    BDR_PAIR(5)
    BDR_PAIR(6)
    BDR_PAIR(7)
    BDR_PAIR(8)
    case 9:
      return same ? launch_ns_pair_one<uint16_t, 9, 9>(a0, a1, n0, n1, st) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;   // (ten row tiles: launched one by one)
  }
#undef BDR_PAIR
}

}  // namespace bdr
