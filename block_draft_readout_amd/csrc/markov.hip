// Host side of the DSpark Markov-biased semi-autoregressive argmax: workspace
// layout and dispatch to the chain or per-position schedule.

#include "markov_kernels.h"

namespace bdr {

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

// keys | slots | tokens | completion counter | error word
static size_t keys_bytes(int64_t B, int k) {
  return align256(static_cast<size_t>(B) * k * kArriveGroups * 8);
}
static size_t slots_bytes(int64_t B, int k) {
  return align256(static_cast<size_t>(B) * k * kChainSlots * kSlotStride * 8);
}
static size_t tokens_bytes(int64_t B, int k) {
  return align256(static_cast<size_t>(B) * k * kTokenStride * 8);
}

size_t markov_workspace(int64_t B, int k) {
  return keys_bytes(B, k) + slots_bytes(B, k) + tokens_bytes(B, k) + 256 + 256;
}

MarkovArgs markov_args(const float* logits, int64_t B, int k, int64_t V, const void* w1,
                       const void* w2, int rank, const int32_t* prev, int32_t* draft,
                       void* workspace) {
  MarkovArgs g{};
  g.logits = logits;
  g.B = B;
  g.V = V;
  g.k = k;
  g.r = (w1 && w2) ? rank : 0;
  g.w1 = w1;
  g.w2 = w2;
  g.prev = prev;
  char* ws = static_cast<char*>(workspace);
  size_t off = 0;
  g.keys = reinterpret_cast<unsigned long long*>(ws + off);
  off += keys_bytes(B, k);
  g.slots = reinterpret_cast<unsigned long long*>(ws + off);
  off += slots_bytes(B, k);
  g.tokens = reinterpret_cast<unsigned long long*>(ws + off);
  off += tokens_bytes(B, k);
  g.done = reinterpret_cast<unsigned*>(ws + off);
  off += 256;
  g.err = reinterpret_cast<unsigned*>(ws + off);   // the last 256 bytes
  g.draft = draft;
  g.vtiles = (V + 15) / 16;
  return g;
}

hipError_t launch_markov(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                         const void* w1, const void* w2, int rank, const int32_t* prev,
                         int32_t* draft, void* workspace, int n_cu, hipStream_t stream) {
  const MarkovArgs g = markov_args(logits, B, k, V, w1, w2, rank, prev, draft, workspace);
  return markov_dispatch<false>(g, wdt, n_cu, stream);
}

}  // namespace bdr
