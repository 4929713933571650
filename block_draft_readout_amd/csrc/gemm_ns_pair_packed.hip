// Instantiations of the two-problem row-split launch (gemm_ns.h) with the
// register ring, bf16 weights in the packed layout: the LM head with 5 to 9 A
// row tiles (ring r0 of kNsLeanRings) beside the fc (mt0 or mt0 + 1 tiles, at
// most 9, ring 3).  Fewer row tiles take the LDS ring (gemm_ns_pair_a.hip).
#include "gemm_ns.h"

namespace bdr {

hipError_t launch_ns_pair_bf16_packed(int mt0, int r0, int mt1, const StreamArgs& a0,
                                      const StreamArgs& a1, unsigned n0, unsigned n1,
                                      hipStream_t st) {
#define BDR_PAIR(M0, R0)                                                                         \
  if (mt0 == M0 && r0 == R0) {                                                                 \
    if (mt1 == M0) return launch_ns_pair_one<uint16_t, M0, R0, M0, 3, true>(a0, a1, n0, n1, st); \
    if (mt1 == M0 + 1)                                                                         \
      return launch_ns_pair_one<uint16_t, M0, R0, M0 + 1, 3, true>(a0, a1, n0, n1, st);         \
  }
  BDR_PAIR(5, 6) BDR_PAIR(5, 5) BDR_PAIR(5, 3)
  BDR_PAIR(6, 6) BDR_PAIR(6, 5) BDR_PAIR(6, 3)
  BDR_PAIR(7, 5) BDR_PAIR(7, 3)
  BDR_PAIR(8, 5) BDR_PAIR(8, 3)
#undef BDR_PAIR
  if (mt0 == 9 && mt1 == 9) {
    if (r0 == 4) return launch_ns_pair_one<uint16_t, 9, 4, 9, 3, true>(a0, a1, n0, n1, st);
    if (r0 == 3) return launch_ns_pair_one<uint16_t, 9, 3, 9, 3, true>(a0, a1, n0, n1, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace bdr
