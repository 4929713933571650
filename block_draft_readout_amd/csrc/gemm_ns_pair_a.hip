// Instantiations of the two-problem row-split launch (gemm_ns.h) with the LDS
// ring, bf16 weights (row-major or packed), LM head with 2 to 4 A row tiles:
// the LM head (mt0 tiles, ring r0 of kNsLeanRings) beside the fc (mt0 or
// mt0 + 1 tiles, ring 3).
#include "gemm_ns.h"

namespace bdr {

hipError_t launch_ns_pair_bf16_a(int mt0, int r0, int mt1, const StreamArgs& a0,
                                 const StreamArgs& a1, unsigned n0, unsigned n1, hipStream_t st) {
#define BDR_PAIR(M0, R0)                                                                   \
  if (mt0 == M0 && r0 == R0) {                                                           \
    if (mt1 == M0) return launch_ns_pair_one<uint16_t, M0, R0, M0, 3>(a0, a1, n0, n1, st); \
    if (mt1 == M0 + 1)                                                                   \
      return launch_ns_pair_one<uint16_t, M0, R0, M0 + 1, 3>(a0, a1, n0, n1, st);         \
  }
  BDR_PAIR(2, 8) BDR_PAIR(2, 5) BDR_PAIR(2, 3)
  BDR_PAIR(3, 7) BDR_PAIR(3, 5) BDR_PAIR(3, 3)
  BDR_PAIR(4, 6) BDR_PAIR(4, 5) BDR_PAIR(4, 3)
#undef BDR_PAIR
  return hipErrorInvalidValue;
}

}  // namespace bdr
