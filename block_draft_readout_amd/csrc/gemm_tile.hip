// Tiled bf16 GEMM for many rows (the prefill-shaped fc: M in the thousands)
// on gfx950.
//
// C[M, N] = A[M, K] * W[N, K]^T with A given as tap segments along K (each
// [M, seg]), bf16 operands, fp32 accumulation.  With thousands of rows the
// product is bound by the matrix cores (about 2 M N K flops over
// 2 (M + N) K bytes, far above the bf16 ridge), so everything serves the MFMA
// issue rate:
//  * a workgroup of four waves owns a 256 x 160 tile of C; waves are 2 x 2,
//    each 128 x 80 = 8 x 5 MFMA tiles of 16 x 16 (160 fp32 accumulators per
//    lane, 40 v_mfma_f32_16x16x32_bf16 per 13 operand reads);
//  * K advances 64 elements per step.  A step's A slice (256 x 64) and W slice
//    (160 x 64) are copied global -> LDS by buffer-to-LDS loads (1 KB each, 13
//    per wave) into a ring of three 53 KB stages, two steps ahead of the one
//    being multiplied; one workgroup barrier per step;
//  * each step is multiplied in two halves of K = 32; the loads of step s + 2
//    and the second half's operand reads are spread over the first half's
//    MFMAs (measured: the copies issued back to back, before the MFMAs, were
//    the largest cost of the step);
//  * an LDS row holds one row's 64 elements (128 bytes) with its eight
//    16-byte chunks XOR-swizzled by the row index, so an operand read
//    (ds_read_b128: 16 rows x 4 chunks) touches 32 distinct banks per 8 lanes;
//    the loads place the chunks swizzled by choosing which chunk each lane
//    fetches;
//  * W rows are the MFMA's first operand, so each lane ends with 4
//    consecutive output columns of one row: one 8-byte bf16 store per tile;
//  * workgroup b runs on XCD b % 8; the tiles are numbered in bands of four
//    tile rows and every XCD takes a contiguous run of them, so the
//    workgroups resident on one XCD share A and W slices in its L2;
//  * optional split K (blockIdx.y) into fp32 partials, summed in fixed order
//    by the reduce kernel of gemm.hip.

#include "gemm_kernels.h"

namespace bdr {

// Shape of a workgroup tile: 2 x WN waves of WTM x WTN 16 x 16 MFMA tiles,
// K steps of 64 elements, STAGES LDS stages (loads run STAGES - 1 steps ahead).
template <int WTM, int WTN, int WN, int STAGES>
struct TileShape {
  static constexpr int WAVES = 2 * WN;
  static constexpr int BM = 32 * WTM;
  static constexpr int BN = 16 * WN * WTN;
  static constexpr int ROWS = BM + BN;               // LDS rows per stage (128 bytes each)
  static constexpr int STAGE_BYTES = ROWS * 128;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LOADS_A = BM / 8 / WAVES;     // 1 KB loads (8 rows) per wave: A rows
  static constexpr int LOADS = ROWS / 8 / WAVES;     // per wave, A then W rows
  static constexpr int NR = WTM + WTN;               // operand reads per wave per half step
  static constexpr int NM = 2 * WTM * WTN;           // MFMAs per wave per step
  static constexpr int MFMA_PER_LOAD = NM * 2 / 3 / LOADS;   // loads placed in the first 2/3
  static_assert(ROWS % (8 * WAVES) == 0 && BM % (8 * WAVES) == 0, "loads split evenly over the waves");
  static_assert(MFMA_PER_LOAD >= 1 && LDS_BYTES <= 160 * 1024, "tile fits");
};

struct TileArgs {
  GemmArgs g;
  int tiles_m, tiles_n;
  int per_xcd;          // tiles per XCD (grid.x = 8 * per_xcd)
  int ksteps;           // K steps of 64 per split
  int total_steps;      // K / 64
};

template <int WTM, int WTN, int WN, int STAGES>
__global__ __launch_bounds__(128 * WN) void gemm_tile_kernel(const TileArgs ta) {
  using TS = TileShape<WTM, WTN, WN, STAGES>;
  const GemmArgs& g = ta.g;
  extern __shared__ __attribute__((aligned(16))) char lds[];   // [STAGES][ROWS][128]
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  // tile of this workgroup: XCD-major runs of band-ordered tiles
  const int T = ta.tiles_m * ta.tiles_n;
  const int t = static_cast<int>(blockIdx.x % 8) * ta.per_xcd + static_cast<int>(blockIdx.x / 8);
  if (t >= T) return;   // whole workgroup
  const int band = t / (4 * ta.tiles_n);
  const int bh = min(4, ta.tiles_m - 4 * band);
  const int bidx = t - 4 * ta.tiles_n * band;
  const int tm = 4 * band + bidx % bh;
  const int tn = bidx / bh;
  const int64_t m0 = static_cast<int64_t>(tm) * TS::BM;
  const int64_t n0 = static_cast<int64_t>(tn) * TS::BN;
  const int s_lo = static_cast<int>(blockIdx.y) * ta.ksteps;
  const int nsteps = min(ta.total_steps, s_lo + ta.ksteps) - s_lo;
  if (nsteps <= 0) return;

  const uint32_t segbytes = static_cast<uint32_t>(g.seg * 2);
  const uint32_t kbytes = static_cast<uint32_t>(g.K * 2);
  const uint32_t rows_a = static_cast<uint32_t>(min<int64_t>(TS::BM, g.M - m0));
  const uint32_t rows_w = static_cast<uint32_t>(min<int64_t>(TS::BN, g.N - n0));
  // rows past M or N read zeros (offsets beyond the resource)
  const rsrc_t rw = make_rsrc(static_cast<const uint16_t*>(g.w) + n0 * g.K, rows_w * kbytes);
  // buffer-to-LDS lane mapping: row lane / 8 of a load, LDS chunk lane % 8
  // holding global chunk (lane % 8) ^ (row % 8)
  const uint32_t lrow = static_cast<uint32_t>(lane >> 3);
  const uint32_t lchunk_b = ((static_cast<uint32_t>(lane) & 7u) ^ lrow) * 16u;

  // Loads of one step: where (stage, tap resource, offsets) is prepared once
  // into the ld_* variables; load q of this wave is issued by dma_one.  A step
  // >= s_lo + nsteps reads zeros into its (free) stage, so every step issues
  // the same loads and the waits count alike.
  rsrc_t ld_ra;
  uint32_t ld_koff_a = 0, ld_koff_w = 0;
  char* ld_dst = lds;
  bool ld_live = false;
  auto dma_prep = [&](int step, int buf) {
    ld_live = step < s_lo + nsteps;
    const uint32_t kel = static_cast<uint32_t>(ld_live ? step : s_lo) * 64u;
    const uint32_t tap = kel / static_cast<uint32_t>(g.seg);   // a step never straddles taps
    ld_ra = make_rsrc(static_cast<const uint16_t*>(seg_base(g, static_cast<int>(tap))) + m0 * g.seg,
                      rows_a * segbytes);
    ld_koff_a = (kel - tap * static_cast<uint32_t>(g.seg)) * 2u + lchunk_b;
    ld_koff_w = kel * 2u + lchunk_b;
    ld_dst = lds + buf * TS::STAGE_BYTES;
  };
  auto dma_one = [&](auto qc) {
    constexpr int q = decltype(qc)::value;
    const int i = wave + TS::WAVES * q;   // load index in the stage; A rows for q < LOADS_A
    if constexpr (q < TS::LOADS_A) {
      const uint32_t row = static_cast<uint32_t>(8 * i) + lrow;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ld_ra, (__attribute__((address_space(3))) void*)(ld_dst + i * 1024), 16,
          ld_live ? row * segbytes + ld_koff_a : kOOB, 0, 0, 0);
    } else {
      const uint32_t row = static_cast<uint32_t>(8 * (i - TS::WAVES * TS::LOADS_A)) + lrow;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(ld_dst + i * 1024), 16,
          ld_live ? row * kbytes + ld_koff_w : kOOB, 0, 0, 0);
    }
  };
  auto dma_step = [&](int step, int buf) {
    dma_prep(step, buf);
    static_for<TS::LOADS>([&](auto q) { dma_one(q); });
  };

  f32x4_t acc[WTM][WTN];
  static_for<WTM>([&](auto i) {
    static_for<WTN>([&](auto j) { acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f}; });
  });
  // operand reads: row r16 of each 16-row tile, chunk (4 * half + grp) swizzled by r16 % 8
  const uint32_t rd_a = static_cast<uint32_t>(wm * 16 * WTM + r16) * 128u;
  const uint32_t rd_w = static_cast<uint32_t>(TS::BM + wn * 16 * WTN + r16) * 128u;
  const uint32_t sw = static_cast<uint32_t>(lane & 7);
  typedef u32x4_t FragA[WTM];
  typedef u32x4_t FragW[WTN];
  // operands of half `half` (K 32 * half .. + 31) of the step in stage `buf`
  auto read_frags = [&](int buf, int half, FragA& af, FragW& bw) {
    const char* base = lds + buf * TS::STAGE_BYTES;
    const uint32_t cb = ((static_cast<uint32_t>(4 * half + grp)) ^ sw) * 16u;
    static_for<WTM>([&](auto i) {
      af[i] = *reinterpret_cast<const u32x4_t*>(base + rd_a + i * 16 * 128 + cb);
    });
    static_for<WTN>([&](auto j) {
      bw[j] = *reinterpret_cast<const u32x4_t*>(base + rd_w + j * 16 * 128 + cb);
    });
  };
  // MFMA e of the step: half e / (WTM * WTN), tile (i, j) of that half
  auto mma_one = [&](auto ec, const FragA& a0, const FragW& b0, const FragA& a1,
                     const FragW& b1) {
    constexpr int e = decltype(ec)::value;
    constexpr int NH = WTM * WTN;
    constexpr int i = (e % NH) / WTN;
    constexpr int j = (e % NH) % WTN;
    if constexpr (e < NH)
      acc[i][j] = mma16(b0[j], a0[i], acc[i][j], uint16_t());
    else
      acc[i][j] = mma16(b1[j], a1[i], acc[i][j], uint16_t());
  };

  // Per step: the operand reads of both halves, then the MFMAs with one
  // buffer-to-LDS load of step s + STAGES - 1 after every MFMA_PER_LOAD-th
  // (all within the first two thirds).  The loads write LDS (the compiler
  // keeps them in program order with the LDS reads and does not hoist them
  // into the MFMAs by itself), so the interleaving is written out and pinned
  // with scheduling groups; spreading the loads keeps the texture path busy
  // while the matrix cores run (issued back to back, before the MFMAs, they
  // were the largest cost of the step).
  constexpr int MPL = TS::MFMA_PER_LOAD;
  static_for<STAGES - 1>([&](auto c) { dma_step(s_lo + decltype(c)::value, decltype(c)::value); });
  dma_prep(s_lo + STAGES - 1, STAGES - 1);
  FragA a0, a1;
  FragW b0, b1;
  int buf = 0;
  for (int s = 0; s < nsteps; ++s) {
    // this wave's loads of step s are done when at most those of the
    // STAGES - 2 steps after it remain
    BDR_WAIT_VM_LGKM((STAGES - 2) * TS::LOADS, 0);
    // every wave's loads of step s have landed, and every wave is done with
    // the stage the next loads overwrite (step s - 1's)
    BDR_WG_BARRIER();
    if constexpr (WN == 2) {
      // one wave per SIMD: both halves' operands read up front, so the
      // second half's reads are in flight during the first half's MFMAs
      read_frags(buf, 0, a0, b0);
      read_frags(buf, 1, a1, b1);
      static_for<TS::NM>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        mma_one(ec, a0, b0, a1, b1);
        if constexpr (e % MPL == MPL - 1 && e / MPL < TS::LOADS)
          dma_one(std::integral_constant<int, e / MPL>{});
      });
      // keep that order through scheduling
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * TS::NR, 0);
      static_for<TS::LOADS>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, MPL, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      });
      __builtin_amdgcn_sched_group_barrier(0x008, TS::NM - MPL * TS::LOADS, 0);
    } else {
      // two waves per SIMD (registers for one half's operands): each half's
      // reads just before its MFMAs, the other wave covering their latency;
      // the loads go into the first half
      constexpr int NH = WTM * WTN;
      constexpr int MPL1 = NH / TS::LOADS;
      static_assert(MPL1 >= 1, "loads fit in the first half");
      read_frags(buf, 0, a0, b0);
      static_for<NH>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        mma_one(ec, a0, b0, a0, b0);
        if constexpr (e % MPL1 == MPL1 - 1 && e / MPL1 < TS::LOADS)
          dma_one(std::integral_constant<int, e / MPL1>{});
      });
      read_frags(buf, 1, a0, b0);
      static_for<NH>([&](auto ec) {
        mma_one(std::integral_constant<int, decltype(ec)::value>{}, a0, b0, a0, b0);
      });
      __builtin_amdgcn_sched_group_barrier(0x100, TS::NR, 0);
      static_for<TS::LOADS>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, MPL1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      });
      __builtin_amdgcn_sched_group_barrier(0x008, NH - MPL1 * TS::LOADS, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, TS::NR, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NH, 0);
    }
    buf = buf + 1 == STAGES ? 0 : buf + 1;
    // where step s + STAGES goes (the stage of step s): prepared while the MFMAs drain
    dma_prep(s_lo + s + STAGES, buf == 0 ? STAGES - 1 : buf - 1);
  }
  BDR_WAIT_VM_LGKM(0, 0);   // the trailing zero-filling loads

  // epilogue: lane holds C[m][n .. n+3] of each tile (N % 4 == 0 here)
  const bool partial = g.partial != 0;
  float* pf = partial ? static_cast<float*>(g.out) + static_cast<int64_t>(blockIdx.y) * g.M * g.N
                      : static_cast<float*>(g.out);
  uint16_t* pb = static_cast<uint16_t*>(g.out);
  const bool to_bf16 = !partial && g.out_kind == OUT_BF16;
  static_for<WTM>([&](auto i) {
    const int64_t m = m0 + wm * 16 * WTM + decltype(i)::value * 16 + r16;
    static_for<WTN>([&](auto j) {
      const int64_t n = n0 + wn * 16 * WTN + decltype(j)::value * 16 + 4 * grp;
      if (m < g.M && n < g.N) {
        const f32x4_t v = acc[i][j];
        if (to_bf16) {
          const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(v[0])) |
                              (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
          const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(v[2])) |
                              (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
          *reinterpret_cast<uint2*>(pb + m * g.N + n) = uint2{lo, hi};
        } else {
          *reinterpret_cast<f32x4_t*>(pf + m * g.N + n) = v;
        }
      }
    });
  });
}

template <int WTM, int WTN, int WN, int STAGES>
static hipError_t launch_tile_shape(const TileArgs& ta, unsigned splits, hipStream_t stream) {
  using TS = TileShape<WTM, WTN, WN, STAGES>;
  static bool attr_set = false;   // per shape
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_tile_kernel<WTM, WTN, WN, STAGES>),
        hipFuncAttributeMaxDynamicSharedMemorySize, TS::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid(static_cast<unsigned>(8 * ta.per_xcd), splits);
  hipLaunchKernelGGL((gemm_tile_kernel<WTM, WTN, WN, STAGES>), grid, dim3(128 * WN),
                     TS::LDS_BYTES, stream, ta);
  return hipGetLastError();
}

int tile_cols(int shape) { return shape == 1 ? 320 : 160; }

hipError_t launch_gemm_tile(const GemmPlan& p, const GemmArgs& g, hipStream_t stream) {
  TileArgs ta{};
  ta.g = g;
  ta.tiles_m = p.tiles_m;
  ta.tiles_n = p.tiles_n;
  ta.per_xcd = (p.tiles_m * p.tiles_n + 7) / 8;
  ta.ksteps = static_cast<int>(p.kb_per_split);
  ta.total_steps = static_cast<int>(p.kblocks);
  const unsigned splits = static_cast<unsigned>(p.ksplit);
  if (p.tile_shape == 1) return launch_tile_shape<8, 5, 4, 2>(ta, splits, stream);
  return launch_tile_shape<8, 5, 2, 3>(ta, splits, stream);
}

}  // namespace bdr
