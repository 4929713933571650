// Host side of probabilistic DSpark drafting: the Markov chain in sampling mode
// (each position's token is drawn from the biased distribution by the
// Gumbel-max rule and becomes the next position's context; the chain generates
// the draws' noise itself).

#include <cmath>

#include "markov_kernels.h"

namespace bdr {

// the Markov workspace (its error word in the last 256 bytes)
size_t markov_sample_workspace(int64_t B, int k, int64_t V) {
  (void)V;
  return markov_workspace(B, k);
}

hipError_t launch_markov_sample(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                                const void* w1, const void* w2, int rank, const int32_t* prev,
                                float inv_t, uint64_t seed, int32_t* draft, float* xout,
                                const float* conf, float threshold, int32_t* status,
                                void* workspace, int n_cu, hipStream_t stream) {
  MarkovArgs g = markov_args(logits, B, k, V, w1, w2, rank, prev, draft, status, workspace);
  g.seed_lo = static_cast<uint32_t>(seed);
  g.seed_hi = static_cast<uint32_t>(seed >> 32);
  g.xout = xout;
  g.inv_t = inv_t;
  g.conf = conf;
  g.th = threshold;
  g.use_conf = (conf != nullptr && !std::isnan(threshold)) ? 1 : 0;
  return markov_dispatch<true>(g, wdt, n_cu, stream);
}

}  // namespace bdr
