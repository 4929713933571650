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

// TPW vocabulary tiles of 16 per wave; all their loads are issued before any
// is consumed, so one pass costs about one memory round trip per wave.
template <typename S, int RKS, int TPW>
__global__ __launch_bounds__(256) void markov_pass_kernel(const MarkovArgs g, int pos) {
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  constexpr int ES = static_cast<int>(sizeof(S));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * 16;
  const int64_t nb = min<int64_t>(16, g.B - b0);

  // Context token of A-operand row r16.
  const int64_t brow = b0 + r16;
  int32_t p = -1;
  if (brow < g.B)
    p = pos == 0 ? g.prev[brow] : key_index(g.keys[static_cast<int64_t>(pos - 1) * g.B + brow]);
  if (pos > 0 && blockIdx.x == 0 && threadIdx.x < 16 && brow < g.B)
    g.draft[brow * g.k + (pos - 1)] = p;

  const uint32_t wbytes = static_cast<uint32_t>(g.V * g.r * ES);
  u32x4_t ef[RKS > 0 ? RKS : 1];
  if constexpr (RKS > 0) {
    const rsrc_t r1 = make_rsrc(g.w1, wbytes);
    const bool pok = p >= 0 && static_cast<int64_t>(p) < g.V;  // out-of-range context: no bias
#pragma unroll
    for (int c = 0; c < RKS; ++c) {
      const int j = c * KS + grp * E;
      ef[c] = bload16(r1, (pok && j < g.r)
                              ? static_cast<uint32_t>((static_cast<int64_t>(p) * g.r + j) * ES)
                              : kOOB);
    }
  }
  const rsrc_t r2 = make_rsrc(g.w2, wbytes);
  // logits of this position for rows b0..b0+nb-1 (row stride k*V floats)
  const rsrc_t rz = make_rsrc(g.logits + (b0 * g.k + pos) * g.V,
                              static_cast<uint32_t>(((nb - 1) * g.k * g.V + g.V) * 4));
  uint32_t zrow[4];
  bool bok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rb = 4 * grp + i;
    bok[i] = rb < nb;
    zrow[i] = static_cast<uint32_t>(rb * g.k * g.V * 4);
  }

  float bv[4];
  uint32_t bi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bv[i] = -INFINITY;
    bi[i] = 0xFFFFFFFFu;
  }

  const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 4 + wave; base < g.vtiles;
       base += nw * TPW) {
    u32x4_t wf[TPW][RKS > 0 ? RKS : 1];
    float zv[TPW][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int64_t v = (base + u * nw) * 16 + r16;
      const bool vok = v < g.V;
      if constexpr (RKS > 0) {
#pragma unroll
        for (int c = 0; c < RKS; ++c) {
          const int j = c * KS + grp * E;
          wf[u][c] = bload16(r2, (vok && j < g.r) ? static_cast<uint32_t>((v * g.r + j) * ES) : kOOB);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        zv[u][i] = bload_f32(rz, (vok && bok[i]) ? zrow[i] + static_cast<uint32_t>(v * 4) : kOOB);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int64_t v = (base + u * nw) * 16 + r16;
      f32x4_t bias = {0.f, 0.f, 0.f, 0.f};
      if constexpr (RKS > 0) {
#pragma unroll
        for (int c = 0; c < RKS; ++c) bias = mma16(ef[c], wf[u][c], bias, S());
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = zv[u][i] + bias[i];
        if (v < g.V && bok[i] && s > bv[i]) {
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
static void launch_passes(const MarkovArgs& g, hipStream_t st) {
  constexpr int TPW = RKS <= 2 ? 8 : (RKS <= 4 ? 4 : 2);
  const int64_t wgs = std::min<int64_t>((g.vtiles + 4 * TPW - 1) / (4 * TPW), 1024);
  const dim3 grid(static_cast<unsigned>(wgs), static_cast<unsigned>((g.B + 15) / 16));
  for (int pos = 0; pos < g.k; ++pos)
    hipLaunchKernelGGL((markov_pass_kernel<S, RKS, TPW>), grid, dim3(256), 0, st, g, pos);
}

template <typename S>
static void launch_typed(const MarkovArgs& g, int rks, hipStream_t st) {
  switch (rks) {
    case 0: launch_passes<S, 0>(g, st); break;
    case 1: launch_passes<S, 1>(g, st); break;
    case 2: launch_passes<S, 2>(g, st); break;
    case 3: launch_passes<S, 3>(g, st); break;
    case 4: launch_passes<S, 4>(g, st); break;
    case 5: launch_passes<S, 5>(g, st); break;
    case 6: launch_passes<S, 6>(g, st); break;
    case 7: launch_passes<S, 7>(g, st); break;
    default: launch_passes<S, 8>(g, st); break;
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
  if (wdt == BDR_BF16)
    launch_typed<uint16_t>(g, rks, stream);
  else
    launch_typed<float>(g, rks, stream);
  hipLaunchKernelGGL(markov_finalize_kernel,
                     dim3(static_cast<unsigned>(std::min<int64_t>((B + 255) / 256, 1024))),
                     dim3(256), 0, stream, g.keys, B, k, draft);
  return hipGetLastError();
}

}  // namespace bdr
