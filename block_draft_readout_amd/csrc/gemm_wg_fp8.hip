// Instantiations of the workgroup streaming GEMM kernel for fp8 (E4M3) weights
// with per-row scales and bf16 A (16 < M <= 160).
#include "gemm_kernels.h"

namespace bdr {

hipError_t launch_wg_fp8(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
  switch (p.mtw * 100 + p.nt) {
    case 108: return launch_wg_one<uint8_t, 1, 8>(p, sa, st);
    case 116: return launch_wg_one<uint8_t, 1, 16>(p, sa, st);
    case 124: return launch_wg_one<uint8_t, 1, 24>(p, sa, st);
    case 132: return launch_wg_one<uint8_t, 1, 32>(p, sa, st);
    case 140: return launch_wg_one<uint8_t, 1, 40>(p, sa, st);
    case 208: return launch_wg_one<uint8_t, 2, 8>(p, sa, st);
    case 216: return launch_wg_one<uint8_t, 2, 16>(p, sa, st);
    case 220: return launch_wg_one<uint8_t, 2, 20>(p, sa, st);
    case 308: return launch_wg_one<uint8_t, 3, 8>(p, sa, st);
    case 312: return launch_wg_one<uint8_t, 3, 12>(p, sa, st);
    default: return hipErrorInvalidValue;   // no instantiation for this shape
  }
}

}  // namespace bdr
