// Host side of probabilistic DSpark drafting: the draft noise, then the Markov
// chain in sampling mode (each position's token is drawn from the biased
// distribution by the Gumbel-max rule and becomes the next position's context).

#include "markov_kernels.h"

namespace bdr {

// noise [B, k, V] fp32 | Markov workspace (its error word stays in the last 256 bytes)
size_t markov_sample_workspace(int64_t B, int k, int64_t V) {
  return align256(static_cast<size_t>(B) * k * V * 4) + markov_workspace(B, k);
}

hipError_t launch_markov_sample(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                                const void* w1, const void* w2, int rank, const int32_t* prev,
                                float inv_t, uint64_t seed, int32_t* draft, float* xout,
                                int32_t* status, void* workspace, int n_cu, hipStream_t stream) {
  float* noise = static_cast<float*>(workspace);
  void* mws = static_cast<char*>(workspace) + align256(static_cast<size_t>(B) * k * V * 4);
  hipError_t e = launch_gumbel_noise(noise, B, k, V, seed, kStreamDraft, stream);
  if (e != hipSuccess) return e;
  MarkovArgs g = markov_args(logits, B, k, V, w1, w2, rank, prev, draft, status, mws);
  g.noise = noise;
  g.xout = xout;
  g.inv_t = inv_t;
  return markov_dispatch<true>(g, wdt, n_cu, stream);
}

}  // namespace bdr
