// Host-side interface of the GEMM kernels: plans and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bdr.h"

namespace bdr {

// ----------------------------------------------------------------------------
// Weight-streaming GEMM: C[M, N] = A[M, K] * W[N, K]^T with fp32 accumulation.
// A is given as n_seg row-major segments [M, seg] laid side by side along K
// (the fc's tap concatenation; one segment for the LM head).
// ----------------------------------------------------------------------------
struct GemmPlan {
  int mt = 1;             // 16-row tiles per workgroup (1..9)
  int m_groups = 1;       // workgroups along M
  int jn = 4;             // 16-column tiles per workgroup (one wave)
  int64_t n_wg = 1;       // workgroups along N
  int ksplit = 1;         // workgroups along K (partials reduced by a second kernel)
  int64_t steps_per_split = 0;
  size_t workspace = 0;   // bytes of split-K partials
  // streaming variants: balanced row ranges x K-block ranges; one wave per
  // range (M <= 16) or a four-wave workgroup per range (ns, 16 < M <= 160)
  bool stream = false;
  bool ns = false;        // row-split workgroup kernel (gemm_ns.h), mt = A row tiles
  int64_t n_waves = 0;    // row ranges (workgroups along N)
  int64_t kblocks = 0;
  int64_t kb_per_split = 0;
  int ring = 0;           // ns: LDS ring slots per wave (kNsLeanRings)
  bool reg = false;       // ns: the register ring (kNsRegMinMt)
  // tiled variant for many rows (bf16, M > 160): 256 x 160 output tiles,
  // K steps of 64 (kblocks / kb_per_split count steps)
  bool tile = false;
  int tile_shape = 0;     // 0: 256 x 160 tiles, 3 LDS stages; 1: 256 x 320, 2 stages
  int tiles_m = 0, tiles_n = 0;
  // packed bf16 weights: always the row-split kernel (mt >= 2), over slabs of
  // `slab` rows when M is larger (0: one slab)
  bool packed = false;
  int64_t slab = 0;
};

// Storage of activations and outputs under a weight dtype: the packed layout
// holds bf16 weights and takes bf16 activations.
inline bdr_dtype act_dtype(bdr_dtype dt) { return dt == BDR_BF16_PACKED ? BDR_BF16 : dt; }

// Rows per slab of a GEMM with packed weights (the row-split kernel's maximum).
constexpr int64_t kPackedSlabRows = 160;

// Bytes of the packed copy of a bf16 [rows, cols] weight (0: not packable).
size_t packed_weight_bytes(int64_t rows, int64_t cols);
hipError_t launch_pack_weight(const void* w, int64_t rows, int64_t cols, void* packed,
                              hipStream_t stream);

// Compute units of a gfx950 part (MI350X / MI355X); fixed so that workspace
// queries and launches always plan identically.
constexpr int kNumCU = 256;

// Row-split kernel (gemm_ns.h, bf16 and fp8 weights): per A row-tile count, the
// accumulator tiles one pass can hold, and the ring depths built (deepest
// first; 0 = none).  A deep ring keeps more loads in flight, a shallow one
// wastes fewer slots on waves with few tiles.
constexpr int kNsLeanNtwMax[11] = {0, 0, 16, 14, 12, 9, 8, 6, 5, 4, 3};
// bf16 weights in the packed layout, and fp8 codes in K-split plans (the fc),
// take the register ring from this many A row tiles on (the same ring depths;
// one group of R tiles per pass); fewer row tiles stream faster through the
// LDS ring
constexpr int kNsRegMinMt = 5;
constexpr int kNsLeanRings[11][3] = {{0, 0, 0}, {0, 0, 0}, {8, 5, 3}, {7, 5, 3}, {6, 5, 3},
                                     {6, 5, 3}, {6, 5, 3}, {5, 3, 0},  {5, 3, 0}, {4, 3, 0},
                                     {3, 0, 0}};

enum OutKind { OUT_F32 = 0, OUT_BF16 = 1 };

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bdr_dtype dt, bool allow_split,
                   int n_seg = 1);

// Row-split plans (bf16 and fp8 weights, 16 < M <= 160) take these values in
// place of their own where non-zero: the ring depth, the row ranges
// and the K splits (bounded by the shape).  Process-wide; the two-problem
// launch is not planned while any is set.
void set_row_split_override(int ring, int64_t workgroups, int ksplit);

hipError_t launch_gemm(const GemmPlan& p, bdr_dtype dt, const void* const* a, int n_seg,
                       int64_t seg, int64_t M, int64_t N, const void* w, void* out,
                       OutKind out_kind, void* workspace, hipStream_t stream);

// Two bf16 GEMMs in one launch of the row-split kernel: problem 0 (the LM
// head: no K split) and problem 1 (the drafter fc: n_seg1 segments, optional
// K split) share the chip, each workgroup taking part of one of them.  ok is
// false when either shape does not take the row-split kernel or their row tile
// counts differ by more than one.
struct PairPlan {
  bool ok = false;
  GemmPlan p0, p1;        // n_waves = workgroups along N; p1.ksplit along K
  unsigned n0 = 0, n1 = 0;
  size_t workspace = 0;   // problem 1's split-K partials
  int64_t M0 = 0, N0 = 0, K0 = 0, M1 = 0, N1 = 0, K1 = 0;
};
PairPlan plan_gemm_pair(int64_t M0, int64_t N0, int64_t K0, int64_t M1, int64_t N1, int64_t K1,
                        int n_seg1, bool packed = false);
hipError_t launch_gemm_pair(const PairPlan& pp, const void* a0, const void* w0, float* out0,
                            const void* const* a1, int n_seg1, int64_t seg1, const void* w1,
                            void* out1, void* workspace, bool packed, hipStream_t stream);

// hyper-connection stream average of each tap: dst[t][r, h] = mean_s src[t][s*ss + r*rs + h]
hipError_t launch_hc_average(const void* const* src, void* const* dst, int n_taps, int hc,
                             int64_t rows, int64_t hidden, int64_t stream_stride,
                             int64_t row_stride, bdr_dtype dt, hipStream_t stream);

// fp8 (E4M3) weights [N, K] with one fp32 scale per row, bf16 A segments
// (multiples of 64 elements); plan.stream == false means the shape is not
// supported.
GemmPlan plan_gemm_fp8(int64_t M, int64_t N, int64_t K, bool allow_split, int n_seg = 1);
hipError_t launch_gemm_fp8(const GemmPlan& p, const void* const* a, int n_seg, int64_t seg,
                           int64_t M, int64_t N, const uint8_t* w_q, const float* w_scale,
                           void* out, OutKind out_kind, void* workspace, hipStream_t stream);

}  // namespace bdr
