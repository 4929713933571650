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

constexpr int kTileBM = 256;
constexpr int kTileBN = 160;
constexpr int kTileWTM = 8;                          // 16-row tiles per wave
constexpr int kTileWTN = 5;                          // 16-column tiles per wave
constexpr int kTileStages = 3;
constexpr int kTileRows = kTileBM + kTileBN;         // LDS rows per stage
constexpr int kTileStageBytes = kTileRows * 128;     // 53248
constexpr int kTileLoadsA = kTileBM / 8;             // 1 KB loads (8 rows each) per step
constexpr int kTileLoads = kTileRows / 8;
constexpr int kTileLoadsPerWave = kTileLoads / 4;    // 13
static_assert(kTileLoads % 4 == 0 && kTileLoadsA % 4 == 0, "loads split evenly over the waves");
static_assert(2 * kTileWTM * 16 == kTileBM && 2 * kTileWTN * 16 == kTileBN, "2 x 2 waves");

struct TileArgs {
  GemmArgs g;
  int tiles_m, tiles_n;
  int per_xcd;          // tiles per XCD (grid.x = 8 * per_xcd)
  int ksteps;           // K steps of 64 per split
  int total_steps;      // K / 64
};

size_t gemm_tile_lds_bytes() { return static_cast<size_t>(kTileStages) * kTileStageBytes; }

__global__ __launch_bounds__(256) void gemm_tile_kernel(const TileArgs ta) {
  const GemmArgs& g = ta.g;
  extern __shared__ __attribute__((aligned(16))) char lds[];   // [kTileStages][kTileRows][128]
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
  const int64_t m0 = static_cast<int64_t>(tm) * kTileBM;
  const int64_t n0 = static_cast<int64_t>(tn) * kTileBN;
  const int s_lo = static_cast<int>(blockIdx.y) * ta.ksteps;
  const int nsteps = min(ta.total_steps, s_lo + ta.ksteps) - s_lo;
  if (nsteps <= 0) return;

  const uint32_t segbytes = static_cast<uint32_t>(g.seg * 2);
  const uint32_t kbytes = static_cast<uint32_t>(g.K * 2);
  const uint32_t rows_a = static_cast<uint32_t>(min<int64_t>(kTileBM, g.M - m0));
  const uint32_t rows_w = static_cast<uint32_t>(min<int64_t>(kTileBN, g.N - n0));
  // rows past M or N read zeros (offsets beyond the resource)
  const rsrc_t rw = make_rsrc(static_cast<const uint16_t*>(g.w) + n0 * g.K, rows_w * kbytes);
  // buffer-to-LDS lane mapping: row lane / 8 of a load, LDS chunk lane % 8
  // holding global chunk (lane % 8) ^ (row % 8)
  const uint32_t lrow = static_cast<uint32_t>(lane >> 3);
  const uint32_t lchunk_b = ((static_cast<uint32_t>(lane) & 7u) ^ lrow) * 16u;

  auto dma_step = [&](int step, int buf) {
    const uint32_t kel = static_cast<uint32_t>(step) * 64u;
    const uint32_t tap = kel / static_cast<uint32_t>(g.seg);   // a step never straddles taps
    const rsrc_t ra = make_rsrc(static_cast<const uint16_t*>(seg_base(g, static_cast<int>(tap))) +
                                    m0 * g.seg,
                                rows_a * segbytes);
    const uint32_t koff_a = (kel - tap * static_cast<uint32_t>(g.seg)) * 2u + lchunk_b;
    const uint32_t koff_w = kel * 2u + lchunk_b;
    char* dst = lds + buf * kTileStageBytes;
#pragma unroll
    for (int q = 0; q < kTileLoadsPerWave; ++q) {
      const int i = wave + 4 * q;   // load index in the stage; A for q < 8 (compile-time)
      if (q < kTileLoadsA / 4) {
        const uint32_t row = static_cast<uint32_t>(8 * i) + lrow;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
            row * segbytes + koff_a, 0, 0, 0);
      } else {
        const uint32_t row = static_cast<uint32_t>(8 * (i - kTileLoadsA)) + lrow;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
            row * kbytes + koff_w, 0, 0, 0);
      }
    }
  };

  f32x4_t acc[kTileWTM][kTileWTN];
  static_for<kTileWTM>([&](auto i) {
    static_for<kTileWTN>([&](auto j) { acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f}; });
  });
  // operand reads: row r16 of each 16-row tile, chunk (4 * half + grp) swizzled by r16 % 8
  const uint32_t rd_a = static_cast<uint32_t>(wm * 128 + r16) * 128u;
  const uint32_t rd_w = static_cast<uint32_t>(kTileBM + wn * 80 + r16) * 128u;
  const uint32_t sw = static_cast<uint32_t>(lane & 7);
  auto compute = [&](int buf) {
    const char* base = lds + buf * kTileStageBytes;
    static_for<2>([&](auto half) {
      const uint32_t cb = ((static_cast<uint32_t>(4 * decltype(half)::value + grp)) ^ sw) * 16u;
      u32x4_t af[kTileWTM], bw[kTileWTN];
      static_for<kTileWTM>([&](auto i) {
        af[i] = *reinterpret_cast<const u32x4_t*>(base + rd_a + i * 16 * 128 + cb);
      });
      static_for<kTileWTN>([&](auto j) {
        bw[j] = *reinterpret_cast<const u32x4_t*>(base + rd_w + j * 16 * 128 + cb);
      });
      static_for<kTileWTM>([&](auto i) {
        static_for<kTileWTN>([&](auto j) {
          acc[i][j] = mma16(bw[j], af[i], acc[i][j], uint16_t());
        });
      });
      __builtin_amdgcn_sched_group_barrier(0x100, kTileWTM + kTileWTN, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, kTileWTM * kTileWTN, 0);
    });
  };

  dma_step(s_lo, 0);
  if (nsteps > 1) dma_step(s_lo + 1, 1);
  int buf = 0;
  for (int s = 0; s < nsteps; ++s) {
    // this wave's loads of step s are done when at most the next step's remain
    if (s + 1 < nsteps)
      BDR_WAIT_VM_LGKM(kTileLoadsPerWave, 0);
    else
      BDR_WAIT_VM_LGKM(0, 0);
    // every wave's loads of step s have landed, and every wave is done with
    // the stage the next loads overwrite (step s - 1's)
    BDR_WG_BARRIER();
    if (s + 2 < nsteps) dma_step(s_lo + s + 2, buf == 0 ? 2 : buf - 1);
    compute(buf);
    buf = buf == 2 ? 0 : buf + 1;
  }

  // epilogue: lane holds C[m][n .. n+3] of each tile (N % 4 == 0 here)
  const bool partial = g.partial != 0;
  float* pf = partial ? static_cast<float*>(g.out) + static_cast<int64_t>(blockIdx.y) * g.M * g.N
                      : static_cast<float*>(g.out);
  uint16_t* pb = static_cast<uint16_t*>(g.out);
  const bool to_bf16 = !partial && g.out_kind == OUT_BF16;
  static_for<kTileWTM>([&](auto i) {
    const int64_t m = m0 + wm * 128 + decltype(i)::value * 16 + r16;
    static_for<kTileWTN>([&](auto j) {
      const int64_t n = n0 + wn * 80 + decltype(j)::value * 16 + 4 * grp;
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

hipError_t launch_gemm_tile(const GemmPlan& p, const GemmArgs& g, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tile_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(gemm_tile_lds_bytes()));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  TileArgs ta{};
  ta.g = g;
  ta.tiles_m = p.tiles_m;
  ta.tiles_n = p.tiles_n;
  ta.per_xcd = (p.tiles_m * p.tiles_n + 7) / 8;
  ta.ksteps = static_cast<int>(p.kb_per_split);
  ta.total_steps = static_cast<int>(p.kblocks);
  const dim3 grid(static_cast<unsigned>(8 * ta.per_xcd), static_cast<unsigned>(p.ksplit));
  hipLaunchKernelGGL(gemm_tile_kernel, grid, dim3(256), gemm_tile_lds_bytes(), stream, ta);
  return hipGetLastError();
}

}  // namespace bdr
