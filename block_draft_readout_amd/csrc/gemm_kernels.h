// Weight-streaming GEMM kernels shared by the gemm translation units (gfx950).
// C[M, N] = A[M, K] * W[N, K]^T with A given as segments laid side by side
// along K; see gemm.hip for the plans that choose between them.
#pragma once

#include <algorithm>
#include <type_traits>
#include <utility>

#include "bdr_device.h"
#include "bdr_internal.h"

namespace bdr {

struct GemmArgs {
  const void* a[BDR_MAX_TAPS];  // A segments, each [M, seg]
  int64_t seg;
  int64_t M, N, K;              // K = n_seg * seg
  const void* w;                // [N, K]
  void* out;                    // final [M, N] or fp32 partials [ksplit, M, N]
  int out_kind;                 // OutKind of a final output
  int partial;                  // 1: write fp32 partials [split, M, N]
  int64_t steps_per_split;      // K steps handled by one workgroup along K
  const float* w_scale;         // fp8 weights: one scale per W row [N]; else unused
  int w_packed;                 // 1: W in the packed layout (row-split kernel only)
};

// Segment base pointer chosen with scalar selects (t is uniform), so the
// pointer array is never indexed dynamically.
__device__ __forceinline__ const void* seg_base(const GemmArgs& g, int t) {
  const void* p = g.a[0];
#pragma unroll
  for (int c = 1; c < BDR_MAX_TAPS; ++c)
    if (t == c) p = g.a[c];
  return p;
}

struct StreamArgs {
  GemmArgs g;
  int64_t n_waves;      // workgroups along N (balanced row ranges)
  int64_t kblocks;      // K blocks per row (the last may be partial)
  int64_t kb_per_split; // K blocks per workgroup along K
};

// Output of one workgroup, read out of the kernel arguments once: fp32
// partials of K split `split` ([ksplit, M, N]), or the final fp32 / bf16 C.
struct OutRef {
  float* f32;
  uint16_t* bf16;   // non-null: final bf16 output
  int64_t M, N;
  __device__ __forceinline__ OutRef(const GemmArgs& g, unsigned split) : M(g.M), N(g.N) {
    if (g.partial) {
      f32 = static_cast<float*>(g.out) + static_cast<int64_t>(split) * g.M * g.N;
      bf16 = nullptr;
    } else if (g.out_kind == OUT_BF16) {
      f32 = nullptr;
      bf16 = static_cast<uint16_t*>(g.out);
    } else {
      f32 = static_cast<float*>(g.out);
      bf16 = nullptr;
    }
  }
  __device__ __forceinline__ void put(int64_t m, int64_t n, float v) const {
    if (bf16)
      bf16[m * N + n] = f32_to_bf16(v);
    else
      f32[m * N + n] = v;
  }
};

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, every index a compile-time constant
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Explicit waits on buffer-to-LDS loads (gfx9 encoding: vmcnt <= n, lgkmcnt
// <= l, expcnt free).  The empty assembly statement with a memory clobber and
// the scheduling barrier keep loads and stores from moving across.
#define BDR_WAIT_VM_LGKM(n, l)                                                          \
  do {                                                                                  \
    __builtin_amdgcn_s_waitcnt(((n)&0xF) | (0x7 << 4) | (((l)&0xF) << 8) |               \
                               ((((n) >> 4) & 3) << 14));                               \
    asm volatile("" ::: "memory");                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                  \
  } while (0)
#define BDR_WG_BARRIER()                 \
  do {                                   \
    asm volatile("s_barrier" ::: "memory"); \
    __builtin_amdgcn_sched_barrier(0);   \
  } while (0)

// fp8 weights (row-split kernel): S = uint8_t means E4M3 codes with one fp32
// scale per W row against bf16 A
template <typename S> constexpr bool kIsFp8 = std::is_same_v<S, uint8_t>;

// 16 E4M3 codes (little-endian bytes of q) -> bf16 operands of elements 0..7 (lo)
// and 8..15 (hi); exact, every E4M3 value being a bf16 value
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4_t q, u32x4_t& lo, u32x4_t& hi) {
  lo.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false));
  lo.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true));
  lo.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false));
  lo.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true));
  hi.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.z, 1.0f, false));
  hi.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.z, 1.0f, true));
  hi.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.w, 1.0f, false));
  hi.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.w, 1.0f, true));
}

// tiled variant for many rows (gemm_tile.hip)
hipError_t launch_gemm_tile(const GemmPlan& p, const GemmArgs& g, hipStream_t stream);
int tile_cols(int shape);   // output columns of a tiled-variant workgroup tile
// fp8 (E4M3) weights with per-row scales, bf16 A: one-wave streaming kernel
// (gemm_fp8.hip)
hipError_t launch_stream_fp8(const GemmPlan& p, const GemmArgs& g, hipStream_t st);
// row-split workgroup kernel (gemm_ns.h): bf16 and fp8 weights, bf16 A
hipError_t launch_ns_bf16(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
hipError_t launch_ns_fp8(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
hipError_t launch_ns_fp8_reg(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
// the LM head (mt0 row tiles, ring r0) beside the fc (mt1 = mt0 or mt0 + 1 row
// tiles, ring 3) in one launch: mt0 2..4 (gemm_ns_pair_a.hip), 5..9 (_b)
hipError_t launch_ns_pair_bf16_a(int mt0, int r0, int mt1, const StreamArgs& a0,
                                 const StreamArgs& a1, unsigned n0, unsigned n1, hipStream_t st);
hipError_t launch_ns_pair_bf16_b(int mt0, int r0, int mt1, const StreamArgs& a0,
                                 const StreamArgs& a1, unsigned n0, unsigned n1, hipStream_t st);
// the same with the register ring, for bf16 weights in the packed layout with
// at least kNsRegMinMt A row tiles (gemm_ns_packed.hip, gemm_ns_pair_packed.hip)
hipError_t launch_ns_bf16_packed(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
hipError_t launch_ns_pair_bf16_packed(int mt0, int r0, int mt1, const StreamArgs& a0,
                                      const StreamArgs& a1, unsigned n0, unsigned n1,
                                      hipStream_t st);

}  // namespace bdr
