// Weight-streaming MFMA GEMM for gfx950: C[M, N] = A[M, K] * W[N, K]^T.
//
// Serves the drafter fc (A = the tapped hidden states, concatenated along K
// segment by segment; W = fc.weight [H, T*H]) and the LM head (A = the block's
// hidden states; W = [V, H]).  Both are dense contractions with few rows
// (M = 4..144) against a large weight read exactly once, so the kernel is
// organised around streaming W from HBM:
//   * each wave owns JN 16-column tiles of W and all MT*16 rows of A;
//   * every lane moves 16 contiguous bytes of one W row per load (4 lanes
//     cover 64 contiguous bytes of a row), with PF steps of loads in flight;
//   * the WK waves of a workgroup interleave K steps so that neighbouring
//     waves read neighbouring bytes of the same W rows, and their partial sums
//     are combined in LDS in a fixed order;
//   * when N alone gives too few workgroups (the fc: N = H) K is also split
//     across workgroups, each writing fp32 partials that a second kernel sums
//     in a fixed order -- the result is deterministic.
// Inputs are bf16 (v_mfma_f32_16x16x32_bf16) or fp32 (v_mfma_f32_16x16x4_f32),
// accumulation is fp32.

#include <algorithm>

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
  int partial;                  // 1: write fp32 partials indexed by blockIdx.y
  int64_t steps_per_split;      // K steps handled by one workgroup along K
};

template <typename S, int MT, int JN, int WK, int PF>
__global__ __launch_bounds__(256) void ws_gemm_kernel(const GemmArgs g) {
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  constexpr int WN = 4 / WK;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % WN;
  const int wk = wave / WN;
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (WN * 16 * JN) + wn * (16 * JN);
  const int64_t m0 = static_cast<int64_t>(blockIdx.z) * (MT * 16);
  const int64_t total_steps = (g.K + KS - 1) / KS;
  const int64_t s_lo = static_cast<int64_t>(blockIdx.y) * g.steps_per_split;
  const int64_t s_hi = min(total_steps, s_lo + g.steps_per_split);

  const S* wrow[JN];
  bool nok[JN];
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int64_t n = n0 + 16 * j + r16;
    nok[j] = n < g.N;
    wrow[j] = static_cast<const S*>(g.w) + (nok[j] ? n : 0) * g.K + grp * E;
  }
  int64_t arow[MT];
  bool mok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t m = m0 + 16 * mt + r16;
    mok[mt] = m < g.M;
    arow[mt] = (mok[mt] ? m : 0) * g.seg + grp * E;
  }

  f32x4_t acc[MT][JN];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < JN; ++j) acc[mt][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t bb[PF][JN];
  u32x4_t aa[PF][MT];

  // Next step to load, with its A segment and offset inside the segment.
  int64_t sl = s_lo + wk;
  int tl = 0;
  int64_t hl = 0;
  if (sl < s_hi) {
    const int64_t kb = sl * KS;
    tl = static_cast<int>(kb / g.seg);
    hl = kb - static_cast<int64_t>(tl) * g.seg;
  }

  auto load_step = [&](u32x4_t(&b)[JN], u32x4_t(&a)[MT]) {
    const int64_t kb = sl * KS;
    const bool kok = kb + grp * E < g.K;
#pragma unroll
    for (int j = 0; j < JN; ++j) b[j] = (nok[j] && kok) ? load16(wrow[j] + kb) : zero;
    const S* abase = static_cast<const S*>(g.a[tl]) + hl;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = (mok[mt] && kok) ? load16(abase + arow[mt]) : zero;
    hl += WK * KS;
    while (hl >= g.seg) {
      hl -= g.seg;
      ++tl;
    }
  };

#pragma unroll
  for (int d = 0; d < PF; ++d) {
    if (sl < s_hi) load_step(bb[d], aa[d]);
    sl += WK;
  }

  for (int64_t sc = s_lo + wk; sc < s_hi; sc += PF * WK) {
#pragma unroll
    for (int d = 0; d < PF; ++d) {
      if (sc + d * WK < s_hi) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < JN; ++j) acc[mt][j] = mma16(aa[d][mt], bb[d][j], acc[mt][j], S());
        if (sl < s_hi) load_step(bb[d], aa[d]);
        sl += WK;
      }
    }
  }

  if constexpr (WK > 1) {
    __shared__ float red[(WK - 1) * WN * MT * JN * 4 * 64];
    auto ridx = [&](int w, int mt, int j, int i) {
      return ((((w * WN + wn) * MT + mt) * JN + j) * 4 + i) * 64 + lane;
    };
    if (wk > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < JN; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[ridx(wk - 1, mt, j, i)] = acc[mt][j][i];
    }
    __syncthreads();
    if (wk != 0) return;
    for (int w = 0; w < WK - 1; ++w) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < JN; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][j][i] += red[ridx(w, mt, j, i)];
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 16 * mt + 4 * grp + i;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int64_t n = n0 + 16 * j + r16;
        if (n >= g.N) continue;
        const float v = acc[mt][j][i];
        if (g.partial) {
          static_cast<float*>(g.out)[(static_cast<int64_t>(blockIdx.y) * g.M + m) * g.N + n] = v;
        } else if (g.out_kind == OUT_BF16) {
          static_cast<uint16_t*>(g.out)[m * g.N + n] = f32_to_bf16(v);
        } else {
          static_cast<float*>(g.out)[m * g.N + n] = v;
        }
      }
    }
  }
}

// out[i] = sum_p part[p][i] in order p = 0, 1, ...
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int ksplit, int64_t mn, void* out,
                                                            int out_kind) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < mn;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    float s = 0.f;
    for (int p = 0; p < ksplit; ++p) s += part[p * mn + i];
    if (out_kind == OUT_BF16)
      static_cast<uint16_t*>(out)[i] = f32_to_bf16(s);
    else
      static_cast<float*>(out)[i] = s;
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

static void pick_tiles(int mt, int* jn, int* wk) {
  if (mt <= 2) {
    *jn = 4;
    *wk = 4;
  } else {
    *jn = 2;
    *wk = 4;
  }
}

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bdr_dtype dt, bool allow_split) {
  GemmPlan p;
  const int ks = dt == BDR_BF16 ? Elem<uint16_t>::KSTEP : Elem<float>::KSTEP;
  const int esize = dt == BDR_BF16 ? 2 : 4;
  const int64_t mtiles = std::max<int64_t>(1, (M + 15) / 16);
  if (mtiles <= 9) {
    p.mt = static_cast<int>(mtiles);
    p.m_groups = 1;
  } else {
    p.mt = 8;
    p.m_groups = static_cast<int>((mtiles + 7) / 8);
  }
  pick_tiles(p.mt, &p.jn, &p.wk);
  const int64_t cols = (4 / p.wk) * 16 * p.jn;
  p.n_wg = (N + cols - 1) / cols;
  const int64_t steps = (K + ks - 1) / ks;
  int64_t split = 1;
  if (allow_split) {
    const int64_t target_wgs = 2048;
    const int64_t base = p.n_wg * p.m_groups;
    split = (target_wgs + base - 1) / base;
    split = std::min<int64_t>(split, std::max<int64_t>(1, steps / (p.wk * 4)));
    // keep partial-sum traffic (write + read, fp32) under ~8% of the weight bytes
    const int64_t cap = std::max<int64_t>(
        1, static_cast<int64_t>(0.08 * static_cast<double>(K) * esize / (8.0 * std::max<int64_t>(M, 1))));
    split = std::max<int64_t>(1, std::min<int64_t>({split, cap, 64}));
  }
  p.steps_per_split = (steps + split - 1) / split;
  p.ksplit = static_cast<int>((steps + p.steps_per_split - 1) / p.steps_per_split);
  p.workspace = p.ksplit > 1 ? align256(static_cast<size_t>(p.ksplit) * M * N * 4) : 0;
  return p;
}

template <typename S, int MT>
static void launch_mt(const GemmPlan& p, const GemmArgs& g, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.n_wg), static_cast<unsigned>(p.ksplit),
                  static_cast<unsigned>(p.m_groups));
  // tile shapes per MT as chosen by pick_tiles()
  if constexpr (MT <= 2)
    hipLaunchKernelGGL((ws_gemm_kernel<S, MT, 4, 4, 2>), grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((ws_gemm_kernel<S, MT, 2, 4, 2>), grid, dim3(256), 0, st, g);
}

template <typename S>
static void launch_typed(const GemmPlan& p, const GemmArgs& g, hipStream_t st) {
  switch (p.mt) {
    case 1: launch_mt<S, 1>(p, g, st); break;
    case 2: launch_mt<S, 2>(p, g, st); break;
    case 3: launch_mt<S, 3>(p, g, st); break;
    case 4: launch_mt<S, 4>(p, g, st); break;
    case 5: launch_mt<S, 5>(p, g, st); break;
    case 6: launch_mt<S, 6>(p, g, st); break;
    case 7: launch_mt<S, 7>(p, g, st); break;
    case 8: launch_mt<S, 8>(p, g, st); break;
    default: launch_mt<S, 9>(p, g, st); break;
  }
}

hipError_t launch_gemm(const GemmPlan& p, bdr_dtype dt, const void* const* a, int n_seg,
                       int64_t seg, int64_t M, int64_t N, const void* w, void* out,
                       OutKind out_kind, void* workspace, hipStream_t stream) {
  GemmArgs g{};
  for (int t = 0; t < n_seg; ++t) g.a[t] = a[t];
  g.seg = seg;
  g.M = M;
  g.N = N;
  g.K = seg * n_seg;
  g.w = w;
  g.out_kind = out_kind;
  g.steps_per_split = p.steps_per_split;
  const bool split = p.ksplit > 1;
  g.partial = split ? 1 : 0;
  g.out = split ? workspace : out;
  if (dt == BDR_BF16)
    launch_typed<uint16_t>(p, g, stream);
  else
    launch_typed<float>(p, g, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  const int64_t mn = M * N;
  const int64_t blocks = std::min<int64_t>((mn + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const float*>(workspace), p.ksplit, mn, out,
                     static_cast<int>(out_kind));
  return hipGetLastError();
}

}  // namespace bdr
