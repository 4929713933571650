// Weight-streaming GEMM with fp8 weights for gfx950:
// C[m, n] = scale[n] * sum_k A[m, k] * e4m3(Wq[n, k]).
//
// The drafter checkpoints are published under fp8 names ("docs(vllm):
// Qwen3.8-27B DFlash drafter recipe", summary and "Published artifacts"); the
// weights are read here as OCP E4M3 codes with one fp32 scale per output row,
// and the activations stay bf16 (the taps are bf16 whatever the weights'
// storage: Qwen3.8-27B-DSpark model card, "Target quantisation").  Streaming
// one byte per weight instead of two halves the bytes of the LM head and the
// fc, which bound the whole block-step.
//
// ws_gemm_stream_fp8_kernel (M <= 16) keeps the organisation of the bf16
// streaming kernel: one-wave workgroups, each owning a balanced range of W
// rows and a range of K blocks; 16 rows x 1 KB of codes per visit copied to
// LDS with buffer-to-LDS loads (double-buffered, padded rows), the A slice of
// a K block held in registers and reused by every tile of the range.  A K
// block is 1024 reduction elements (one byte each).  Per 64-element step a
// lane reads the 16 codes k = 64*st + 16*grp + e (e < 16) of its row, widens
// them with v_cvt_scalef32_pk_bf16_fp8 (scale 1: exact, every E4M3 value is a
// bf16 value) into two bf16 operands, and issues two 16x16x32 bf16 MFMAs
// against the A elements with the same k: the reduction order is permuted
// identically on both sides.  The row scale multiplies the fp32 sum once in
// the epilogue (and each K split's partial before the ordered reduction).
//
// A segments (the taps of the fc) need only be multiples of 64 elements: the
// A slice of a block is loaded step by step, each step from the segment it
// falls in.

#include <algorithm>

#include "gemm_kernels.h"

namespace bdr {

constexpr int kF8KB = 1024;             // codes (= bytes) of each W row per visit
constexpr int kF8PadRow = kF8KB + 32;   // LDS row stride (bank-conflict-free reads, as kPadRow)
constexpr int kF8Steps = kF8KB / 64;    // 64-element steps per visit

// NT: 16-row tiles per workgroup (compile time; the last ones may be empty)
template <int NT>
__global__ __launch_bounds__(64) void ws_gemm_stream_fp8_kernel(const StreamArgs sa) {
  constexpr int STEPS = kF8Steps;
  const GemmArgs& g = sa.g;
  __shared__ __attribute__((aligned(16))) char lds[2][16 * kF8PadRow];
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const int64_t n_lo = static_cast<int64_t>(blockIdx.x) * g.N / sa.n_waves;
  const int64_t n_hi = static_cast<int64_t>(blockIdx.x + 1) * g.N / sa.n_waves;
  const int ntiles = static_cast<int>((n_hi - n_lo + 15) / 16);
  const uint32_t kb_lo = static_cast<uint32_t>(blockIdx.y * sa.kb_per_split);
  const uint32_t kb_hi = static_cast<uint32_t>(min<int64_t>(sa.kblocks, kb_lo + sa.kb_per_split));
  if (ntiles <= 0 || kb_lo >= kb_hi) return;
  const OutRef out(g, blockIdx.y);
  const uint32_t K = static_cast<uint32_t>(g.K);          // = W row bytes
  const uint32_t seg = static_cast<uint32_t>(g.seg);
  const int last_seg = static_cast<int>(g.K / g.seg) - 1;

  const rsrc_t rw = make_rsrc(static_cast<const uint8_t*>(g.w) + n_lo * g.K,
                              static_cast<uint32_t>(n_hi - n_lo) * K);
  const uint32_t abytes = static_cast<uint32_t>(g.M) * seg * 2;
  const uint32_t lane16 = static_cast<uint32_t>(lane) * 16;
  const uint32_t a_lane = static_cast<uint32_t>(r16) * seg * 2 + static_cast<uint32_t>(grp) * 32;
  const uint32_t lds_rd = static_cast<uint32_t>(r16 * kF8PadRow + grp * 16);

  f32x4_t acc[NT];
  static_for<NT>([&](auto t) { acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f}; });
  u32x4_t a[STEPS][2];

  // 16 rows of tile t, K block kb -> LDS buffer b (rows past the range and
  // codes past a row read zeros)
  auto dma = [&](uint32_t kb, int t, int b) __attribute__((always_inline)) {
    const uint32_t k0 = kb * kF8KB;
    const uint32_t lo = k0 + lane16 < K ? lane16 : kOOB;
    const uint32_t base = static_cast<uint32_t>(16 * t) * K + k0;
    char* dst = &lds[b][0];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(dst + r * kF8PadRow), 16,
          lo + base + static_cast<uint32_t>(r) * K, 0, 0, 2);
  };
  // A slice of K block kb: step st holds elements 64*st + 16*grp + [0, 8) and
  // + [8, 16) of row r16 (rows >= M and steps past K read zeros); each step
  // reads the segment it falls in (segments are multiples of 64 elements)
  auto load_a = [&](uint32_t kb, u32x4_t(&av)[STEPS][2]) __attribute__((always_inline)) {
    const uint32_t k0 = kb * kF8KB;
    int ts = static_cast<int>(k0 / seg);
    uint32_t kin = k0 - static_cast<uint32_t>(ts) * seg;
    static_for<STEPS>([&](auto st) {
      const bool live = k0 + 64 * st < K;
      const rsrc_t ra = make_rsrc(seg_base(g, min(ts, last_seg)), abytes);
      const uint32_t off = live ? a_lane + 2 * kin : kOOB;
      av[st][0] = bload16(ra, off);
      av[st][1] = bload16(ra, off + 16);
      kin += 64;
      if (kin == seg) {
        kin = 0;
        ++ts;
      }
    });
  };
  auto compute = [&](auto t, int b, const u32x4_t(&av)[STEPS][2], int nsteps) __attribute__((always_inline)) {
    const char* src = &lds[b][0] + lds_rd;
    static_for<STEPS>([&](auto st) {
      if (st < nsteps) {
        const u32x4_t q = *reinterpret_cast<const u32x4_t*>(src + st * 64);
        u32x4_t lo, hi;
        e4m3x16_to_bf16(q, lo, hi);
        acc[t] = mma16(av[st][0], lo, acc[t], uint16_t());
        acc[t] = mma16(av[st][1], hi, acc[t], uint16_t());
      }
    });
  };

  int buf = 0;
  // one K block: visit every tile, prefetching the next visit before waiting
  // on the current one.  The only memory operations issued after a visit's 16
  // loads are the next visit's 16 (and, at a block's first visit, the A slice
  // loads issued before those), hence "vmcnt <= 16" before reading it.  The A
  // slice is single-buffered (two slices do not fit the registers): the next
  // block's is loaded once the last tile of this one is multiplied, while the
  // next block's first visit is already in flight.
  auto block = [&](uint32_t kb) __attribute__((always_inline)) {
    const int nsteps = static_cast<int>(min<uint32_t>(STEPS, (K - kb * kF8KB) / 64));
    static_for<NT>([&](auto t) {
      if (t < ntiles) {
        const bool last = t + 1 == ntiles;
        if (!last) {
          dma(kb, t + 1, buf ^ 1);
          BDR_WAIT_VM(16);
        } else if (kb + 1 < kb_hi) {
          dma(kb + 1, 0, buf ^ 1);
          BDR_WAIT_VM(16);
        } else {
          BDR_WAIT_VM(0);
        }
        compute(t, buf, a, nsteps);
        buf ^= 1;
        if (last && kb + 1 < kb_hi) load_a(kb + 1, a);
      }
    });
  };

  load_a(kb_lo, a);
  dma(kb_lo, 0, 0);
  for (uint32_t kb = kb_lo; kb < kb_hi; ++kb) block(kb);

  static_for<NT>([&](auto t) {
    const int64_t n = n_lo + 16 * t + r16;
    if (t < ntiles && n < n_hi) {
      const float s = g.w_scale[n];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = 4 * grp + i;
        if (m < out.M) out.put(m, n, acc[t][i] * s);
      }
    }
  });
}

hipError_t launch_stream_fp8(const GemmPlan& p, const GemmArgs& g, hipStream_t st) {
  const StreamArgs sa{g, p.n_waves, p.kblocks, p.kb_per_split};
  const dim3 grid(static_cast<unsigned>(p.n_waves), static_cast<unsigned>(p.ksplit));
  const int64_t tiles = ((g.N + p.n_waves - 1) / p.n_waves + 15) / 16;
  if (tiles <= 1) hipLaunchKernelGGL((ws_gemm_stream_fp8_kernel<1>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 2) hipLaunchKernelGGL((ws_gemm_stream_fp8_kernel<2>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 4) hipLaunchKernelGGL((ws_gemm_stream_fp8_kernel<4>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 8) hipLaunchKernelGGL((ws_gemm_stream_fp8_kernel<8>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 10) hipLaunchKernelGGL((ws_gemm_stream_fp8_kernel<10>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 12) hipLaunchKernelGGL((ws_gemm_stream_fp8_kernel<12>), grid, dim3(64), 0, st, sa);
  else return hipErrorInvalidValue;   // the plan keeps ranges to <= 12 tiles
  return hipGetLastError();
}

}  // namespace bdr
