// DSpark Markov bigram bias + semi-autoregressive full-vocabulary argmax (gfx950).
//
// For each row b the context token p starts at the accepted bonus token of the
// previous step and, position after position, becomes the biased argmax just
// taken (llm-scaler PR #620, DSpark port notes: dflash.py and qwen3_dflash.py).
// One kernel launch handles one position for every row:
//   * the low-rank bias of 16 rows for 16 vocabulary entries is one MFMA tile:
//     A = markov_w1 rows of the 16 contexts ([16, r]), B = markov_w2 rows of the
//     16 entries ([r, 16]); r = 32/64 is one or two 16-byte loads per lane;
//   * the fp32 logits of the position are added and each lane keeps a running
//     (value, index) maximum over the entries it visits in increasing order;
//   * the running maxima are packed into order-preserving uint64 keys (value,
//     then lower index), reduced across lanes and waves, and folded into one
//     key per row with a device-scope atomic max -- max is order-independent,
//     so the result is deterministic;
//   * the next launch reads the previous position's key as its context and
//     writes the previous position's token out.
// Positions are separate launches because position i+1 needs the whole-vocab
// argmax of position i; the stream order provides that grid-wide dependency.

#include <algorithm>

#include "bdr_device.h"
#include "bdr_internal.h"

namespace bdr {

struct MarkovArgs {
  const float* logits;           // [B, k, V]
  int64_t B, V;
  int k, r;
  const void* w1;                // [V, r] embedding of the context token
  const void* w2;                // [V, r] projection to the vocabulary
  const int32_t* prev;           // [B] context of position 0
  unsigned long long* keys;      // [k, B] per-position argmax keys (zeroed first)
  int32_t* draft;                // [B, k]
  int64_t vtiles;                // ceil(V / 16)
};

__global__ __launch_bounds__(256) void markov_init_kernel(unsigned long long* keys, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    keys[i] = 0ull;
}

template <typename S, int RKS>
__global__ __launch_bounds__(256) void markov_pass_kernel(const MarkovArgs g, int pos) {
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * 16;

  // Context token of A-operand row r16.
  const int64_t brow = b0 + r16;
  int32_t p = -1;
  if (brow < g.B)
    p = pos == 0 ? g.prev[brow] : key_index(g.keys[static_cast<int64_t>(pos - 1) * g.B + brow]);
  if (pos > 0 && blockIdx.x == 0 && threadIdx.x < 16 && brow < g.B)
    g.draft[brow * g.k + (pos - 1)] = p;

  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t ef[RKS > 0 ? RKS : 1];
  if constexpr (RKS > 0) {
    const bool pok = p >= 0 && static_cast<int64_t>(p) < g.V;  // out-of-range context: no bias
#pragma unroll
    for (int c = 0; c < RKS; ++c) {
      const int j = c * KS + grp * E;
      ef[c] = (pok && j < g.r)
                  ? load16(static_cast<const S*>(g.w1) + static_cast<int64_t>(p) * g.r + j)
                  : zero;
    }
  }

  float bv[4];
  uint32_t bi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bv[i] = -INFINITY;
    bi[i] = 0xFFFFFFFFu;
  }
  // rows of the D tile held by this lane: b = b0 + 4*grp + i
  const float* zrow[4];
  bool bok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t b = b0 + 4 * grp + i;
    bok[i] = b < g.B;
    zrow[i] = g.logits + ((bok[i] ? b : 0) * g.k + pos) * g.V;
  }

  for (int64_t vt = static_cast<int64_t>(blockIdx.x) * 4 + wave; vt < g.vtiles;
       vt += static_cast<int64_t>(gridDim.x) * 4) {
    const int64_t v = vt * 16 + r16;
    const bool vok = v < g.V;
    f32x4_t bias = {0.f, 0.f, 0.f, 0.f};
    if constexpr (RKS > 0) {
      u32x4_t wf[RKS];
#pragma unroll
      for (int c = 0; c < RKS; ++c) {
        const int j = c * KS + grp * E;
        wf[c] = (vok && j < g.r) ? load16(static_cast<const S*>(g.w2) + v * g.r + j) : zero;
      }
#pragma unroll
      for (int c = 0; c < RKS; ++c) bias = mma16(ef[c], wf[c], bias, S());
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (vok && bok[i]) {
        const float s = zrow[i][v] + bias[i];
        if (s > bv[i]) {
          bv[i] = s;
          bi[i] = static_cast<uint32_t>(v);
        }
      }
    }
  }

  __shared__ unsigned long long sk[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned long long key = bi[i] != 0xFFFFFFFFu ? pack_key(bv[i], bi[i]) : 0ull;
    key = rowgroup_max16(key);
    if (r16 == 0) sk[wave][4 * grp + i] = key;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    unsigned long long key = umax64(umax64(sk[0][threadIdx.x], sk[1][threadIdx.x]),
                                    umax64(sk[2][threadIdx.x], sk[3][threadIdx.x]));
    const int64_t b = b0 + threadIdx.x;
    if (b < g.B && key != 0ull) atomicMax(&g.keys[static_cast<int64_t>(pos) * g.B + b], key);
  }
}

__global__ void markov_finalize_kernel(const unsigned long long* keys, int64_t B, int k,
                                       int32_t* draft) {
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; b < B;
       b += static_cast<int64_t>(gridDim.x) * 256)
    draft[b * k + (k - 1)] = key_index(keys[static_cast<int64_t>(k - 1) * B + b]);
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

size_t markov_workspace(int64_t B, int k) {
  return align256(static_cast<size_t>(B) * static_cast<size_t>(k) * 8);
}

template <typename S, int RKS>
static void launch_passes(const MarkovArgs& g, dim3 grid, hipStream_t st) {
  for (int pos = 0; pos < g.k; ++pos)
    hipLaunchKernelGGL((markov_pass_kernel<S, RKS>), grid, dim3(256), 0, st, g, pos);
}

template <typename S>
static void launch_typed(const MarkovArgs& g, int rks, dim3 grid, hipStream_t st) {
  switch (rks) {
    case 0: launch_passes<S, 0>(g, grid, st); break;
    case 1: launch_passes<S, 1>(g, grid, st); break;
    case 2: launch_passes<S, 2>(g, grid, st); break;
    case 3: launch_passes<S, 3>(g, grid, st); break;
    case 4: launch_passes<S, 4>(g, grid, st); break;
    case 5: launch_passes<S, 5>(g, grid, st); break;
    case 6: launch_passes<S, 6>(g, grid, st); break;
    case 7: launch_passes<S, 7>(g, grid, st); break;
    default: launch_passes<S, 8>(g, grid, st); break;
  }
}

hipError_t launch_markov(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                         const void* w1, const void* w2, int rank, const int32_t* prev,
                         int32_t* draft, void* workspace, hipStream_t stream) {
  MarkovArgs g{};
  g.logits = logits;
  g.B = B;
  g.V = V;
  g.k = k;
  g.r = (w1 && w2) ? rank : 0;
  g.w1 = w1;
  g.w2 = w2;
  g.prev = prev;
  g.keys = static_cast<unsigned long long*>(workspace);
  g.draft = draft;
  g.vtiles = (V + 15) / 16;
  const int ks = wdt == BDR_BF16 ? Elem<uint16_t>::KSTEP : Elem<float>::KSTEP;
  const int rks = (g.r + ks - 1) / ks;

  const int64_t nkeys = B * k;
  hipLaunchKernelGGL(markov_init_kernel,
                     dim3(static_cast<unsigned>(std::min<int64_t>((nkeys + 255) / 256, 1024))),
                     dim3(256), 0, stream, g.keys, nkeys);
  const int64_t wgs = std::min<int64_t>((g.vtiles + 3) / 4, 512);
  const dim3 grid(static_cast<unsigned>(wgs), static_cast<unsigned>((B + 15) / 16));
  if (wdt == BDR_BF16)
    launch_typed<uint16_t>(g, rks, grid, stream);
  else
    launch_typed<float>(g, rks, grid, stream);
  hipLaunchKernelGGL(markov_finalize_kernel,
                     dim3(static_cast<unsigned>(std::min<int64_t>((B + 255) / 256, 1024))),
                     dim3(256), 0, stream, g.keys, B, k, draft);
  return hipGetLastError();
}

}  // namespace bdr
