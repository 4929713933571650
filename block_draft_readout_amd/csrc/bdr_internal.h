// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bdr.h"
#include "gemm_plan.h"

namespace bdr {

// ----------------------------------------------------------------------------
// Markov bias + semi-autoregressive argmax over k positions.
// ----------------------------------------------------------------------------
size_t markov_workspace(int64_t B, int k);
hipError_t launch_markov(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                         const void* w1, const void* w2, int rank, const int32_t* prev,
                         int32_t* draft, int32_t* status, void* workspace, int n_cu,
                         hipStream_t stream);
// process-wide limit of the chain's bounded waits (negative / non-finite: default)
void set_poll_timeout_us(double us);
void set_forced_time_out(bool on);

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
                                const float* conf, float threshold, int32_t* status,
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
