// Host-side interface between the C ABI layer and the kernel launchers.
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
  // range (M <= 16) or a four-wave workgroup per range (wg, 16 < M <= 192)
  bool stream = false;
  bool wg = false;
  bool ns = false;        // row-split workgroup kernel (gemm_ns.h), mt = A row tiles
  int kbb = 1024;         // W bytes per row per visit
  int mtw = 1;            // A row tiles per wave (wg)
  int nt = 1;             // 16-row W tiles per range (compile-time bound)
  int64_t n_waves = 0;    // row ranges (workgroups along N)
  int64_t kblocks = 0;
  int64_t kb_per_split = 0;
  // tiled variant for many rows (bf16, M > 160): 256 x 160 output tiles,
  // K steps of 64 (kblocks / kb_per_split count steps)
  bool tile = false;
  int tile_shape = 0;     // 0: 256 x 160 tiles, 3 LDS stages; 1: 256 x 320, 2 stages
  int tiles_m = 0, tiles_n = 0;
};

// Compute units of a gfx950 part (MI350X / MI355X); fixed so that workspace
// queries and launches always plan identically.
constexpr int kNumCU = 256;

enum OutKind { OUT_F32 = 0, OUT_BF16 = 1 };

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bdr_dtype dt, bool allow_split,
                   int n_seg = 1);

hipError_t launch_gemm(const GemmPlan& p, bdr_dtype dt, const void* const* a, int n_seg,
                       int64_t seg, int64_t M, int64_t N, const void* w, void* out,
                       OutKind out_kind, void* workspace, hipStream_t stream);

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

// ----------------------------------------------------------------------------
// Markov bias + semi-autoregressive argmax over k positions.
// ----------------------------------------------------------------------------
size_t markov_workspace(int64_t B, int k);
hipError_t launch_markov(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                         const void* w1, const void* w2, int rank, const int32_t* prev,
                         int32_t* draft, void* workspace, int n_cu, hipStream_t stream);

// ----------------------------------------------------------------------------
// Greedy verification.
// ----------------------------------------------------------------------------
int verify_chunks(int64_t B, int k, int64_t V);
size_t verify_workspace(int64_t B, int k, int64_t V);
hipError_t launch_verify(const void* Y, bdr_dtype dt, int64_t B, int k, int64_t V,
                         const int32_t* draft, const float* conf, float threshold,
                         int32_t* block_len, int32_t* accepted, int32_t* bonus,
                         int32_t* target_argmax, int64_t* acc, int64_t* prop,
                         void* workspace, hipStream_t stream);

// ----------------------------------------------------------------------------
// Probabilistic drafting and rejection-sampling verification.
// ----------------------------------------------------------------------------
// noise[(b * k + i) * V + v] = Gumbel noise of stream stream_id at (b, i, v)
hipError_t launch_gumbel_noise(float* noise, int64_t B, int k, int64_t V, uint64_t seed,
                               uint32_t stream_id, hipStream_t stream);
size_t markov_sample_workspace(int64_t B, int k, int64_t V);
hipError_t launch_markov_sample(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                                const void* w1, const void* w2, int rank, const int32_t* prev,
                                float inv_t, uint64_t seed, int32_t* draft, float* xout,
                                void* workspace, int n_cu, hipStream_t stream);
size_t sample_verify_workspace(int64_t B, int k, int64_t V);
hipError_t launch_verify_sample(const void* Y, bdr_dtype dt, int64_t B, int k, int64_t V,
                                const int32_t* draft, const float* X, const float* conf,
                                float threshold, float inv_t, uint64_t seed, int32_t* block_len,
                                int32_t* accepted, int32_t* bonus, int64_t* acc, int64_t* prop,
                                void* workspace, hipStream_t stream);

// ----------------------------------------------------------------------------
// Closing the loop: commit a verified block; the fc on gathered rows.
// ----------------------------------------------------------------------------
hipError_t launch_commit(const int32_t* draft, const int32_t* accepted, const int32_t* bonus,
                         const int32_t* block_len, int64_t B, int k, int32_t* next_prev,
                         int32_t* emitted, int32_t* draft_list, int32_t* row_index,
                         int32_t* row_count, int32_t* row_offsets, hipStream_t stream);
size_t fc_rows_workspace(int64_t max_rows, int64_t hidden, int n_taps, bdr_dtype dt);
hipError_t launch_fc_rows(const void* const* taps, int n_taps, int64_t rows, int64_t hidden,
                          bdr_dtype dt, const int32_t* row_index, const int32_t* row_count,
                          int64_t max_rows, const void* fc_w, void* out, void* workspace,
                          hipStream_t stream);
size_t fc_rows_fp8_workspace(int64_t max_rows, int64_t hidden, int n_taps);
hipError_t launch_fc_rows_fp8(const void* const* taps, int n_taps, int64_t rows, int64_t hidden,
                              const int32_t* row_index, const int32_t* row_count,
                              int64_t max_rows, const uint8_t* fc_q, const float* fc_scale,
                              void* out, void* workspace, hipStream_t stream);

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace bdr
