// DSpark Markov bigram bias + semi-autoregressive full-vocabulary argmax (gfx950).
//
// For each row b the context token p starts at the accepted bonus token of the
// previous step and, position after position, becomes the biased argmax just
// taken (llm-scaler PR #620, DSpark port notes: dflash.py and qwen3_dflash.py).
//
// Arithmetic of one position, for 16 rows at a time:
//   * the low-rank bias of 16 rows for 16 vocabulary entries is one MFMA tile:
//     A = markov_w1 rows of the 16 contexts ([16, r]), B = markov_w2 rows of
//     the 16 entries ([r, 16]); r = 32/64 is one or two 16-byte operand chunks;
//   * the fp32 logits of the position are added and each lane keeps a running
//     (value, index) maximum over the entries it visits in increasing order;
//   * maxima are packed into order-preserving uint64 keys (value, then lower
//     index) and folded across lanes, waves and workgroups with max, which is
//     order-independent: the result is deterministic.
//
// Two schedules:
//   chain  -- one persistent launch for all k positions.  One workgroup per
//             compute unit keeps its slice of markov_w2 in LDS for the whole
//             chain; positions are separated by a grid barrier with two-level
//             arrival counters (the last arriver writes that position's tokens,
//             and the final one returns the workspace to zero).  All
//             workgroups must be resident at once: the grid is at most the
//             number of compute units and each workgroup fits in one.  The spin
//             on the barrier is bounded; a time-out sets the error word of the
//             workspace instead of hanging.
//   passes -- one launch per position (used when the markov_w2 slice does not
//             fit in LDS); stream order provides the grid-wide dependency.
// Workgroup w folds its keys into group slot w % 16 (atomic max; 16-way at
// most), and readers take the max over the 16 group slots.
//
// Workspace (zero-filled before first use; every call leaves it zeroed):
//   keys[k][16][B] uint64 | group counters [k][16] | top counters [k]
//   (one 128-byte line each) | error uint32

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
  unsigned long long* keys;      // [k, 16, B] per-position argmax keys per arrival group
  unsigned* gcnt;                // [k][16] group arrival counters (128-byte stride)
  unsigned* tcnt;                // [k] top arrival counters (128-byte stride)
  unsigned* err;                 // error word
  int32_t* draft;                // [B, k]
  int64_t vtiles;                // ceil(V / 16)
};

constexpr unsigned kSpinLimit = 1u << 22;   // ~0.2 s of polling before giving up

// final key of row b at position pos: max over the 16 group slots
__device__ __forceinline__ unsigned long long final_key(const MarkovArgs& g, int pos, int64_t b) {
  const unsigned long long* p = g.keys + static_cast<int64_t>(pos) * kArriveGroups * g.B + b;
  unsigned long long k = 0ull;
#pragma unroll
  for (int i = 0; i < kArriveGroups; ++i) k = umax64(k, fetch_u64(p + i * g.B));
  return k;
}

// E fragments: markov_w1 rows of the contexts of rows b0 + (lane & 15)
template <typename S, int RKS>
__device__ __forceinline__ void context_frags(const MarkovArgs& g, int64_t b0, int pos, int r16,
                                              int grp, u32x4_t (&ef)[RKS > 0 ? RKS : 1]) {
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  constexpr int ES = static_cast<int>(sizeof(S));
  const int64_t brow = b0 + r16;
  int32_t p = -1;
  if (brow < g.B)
    p = pos == 0 ? g.prev[brow] : key_index(final_key(g, pos - 1, brow));
  if constexpr (RKS > 0) {
    const rsrc_t r1 = make_rsrc(g.w1, static_cast<uint32_t>(g.V * g.r * ES));
    const bool pok = p >= 0 && static_cast<int64_t>(p) < g.V;  // out-of-range context: no bias
#pragma unroll
    for (int c = 0; c < RKS; ++c) {
      const int j = c * KS + grp * E;
      ef[c] = bload16(r1, (pok && j < g.r)
                              ? static_cast<uint32_t>((static_cast<int64_t>(p) * g.r + j) * ES)
                              : kOOB);
    }
  }
}

// Fold the per-lane maxima of 16 rows into the position's keys.
__device__ __forceinline__ void publish_rows(const MarkovArgs& g, int64_t b0, int pos, int wave,
                                             int r16, int grp, const float (&bv)[4],
                                             const uint32_t (&bi)[4],
                                             unsigned long long (&sk)[4][16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned long long key = bi[i] != 0xFFFFFFFFu ? pack_key(bv[i], bi[i]) : 0ull;
    key = rowgroup_max16(key);
    if (r16 == 0) sk[wave][4 * grp + i] = key;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const unsigned long long key = umax64(umax64(sk[0][threadIdx.x], sk[1][threadIdx.x]),
                                          umax64(sk[2][threadIdx.x], sk[3][threadIdx.x]));
    const int64_t b = b0 + threadIdx.x;
    const int64_t slot = (static_cast<int64_t>(pos) * kArriveGroups + blockIdx.x % kArriveGroups) * g.B;
    if (b < g.B && key != 0ull) atomicMax(&g.keys[slot + b], key);
  }
  BDR_WAIT_ALL_MEM();  // the key updates are performed before this workgroup arrives
  __syncthreads();
}

// ----------------------------------------------------------------------------
// chain: persistent, all positions in one launch
// ----------------------------------------------------------------------------
template <typename S, int RKS, int MAXT>
__global__ __launch_bounds__(256) void markov_chain_kernel(const MarkovArgs g) {
  extern __shared__ u32x4_t w2s[];   // [tile][chunk][lane] operand chunks of markov_w2
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  constexpr int ES = static_cast<int>(sizeof(S));
  constexpr int NC = RKS > 0 ? RKS : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const unsigned G = gridDim.x;
  const int64_t t_lo = static_cast<int64_t>(blockIdx.x) * g.vtiles / G;
  const int64_t t_hi = static_cast<int64_t>(blockIdx.x + 1) * g.vtiles / G;
  const int ntl = static_cast<int>(t_hi - t_lo);   // wave w owns tiles w, w+4, ... (< 4*MAXT)

  __shared__ unsigned long long sk[4][16];
  __shared__ int last_flag;

  // stage this workgroup's markov_w2 rows in operand layout (lane l's 16 bytes
  // of chunk q land at w2s[q*64 + l])
  if constexpr (RKS > 0) {
    const rsrc_t r2 = make_rsrc(g.w2, static_cast<uint32_t>(g.V * g.r * ES));
    for (int q = wave; q < ntl * RKS; q += 4) {
      const int tile = q / RKS;
      const int c = q - tile * RKS;
      const int64_t v = (t_lo + tile) * 16 + r16;
      const int j = c * KS + grp * E;
      const uint32_t off = (v < g.V && j < g.r) ? static_cast<uint32_t>((v * g.r + j) * ES) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r2, (__attribute__((address_space(3))) void*)(&w2s[q * 64]), 16, off, 0, 0, 0);
    }
    BDR_WAIT_VM(0);
  }
  __syncthreads();

  // logits of position pos, rows b0.., for this wave's tiles
  float zv[MAXT][4];
  auto load_z = [&](int pos, int64_t b0) {
    const int64_t nb = min<int64_t>(16, g.B - b0);
    const rsrc_t rz = make_rsrc(g.logits + (b0 * g.k + pos) * g.V,
                                static_cast<uint32_t>(((nb - 1) * g.k * g.V + g.V) * 4));
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int tile = wave + 4 * u;
      const int64_t v = (t_lo + tile) * 16 + r16;
      const bool vok = tile < ntl && v < g.V;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rb = 4 * grp + i;
        zv[u][i] = bload_f32(rz, (vok && rb < nb)
                                     ? static_cast<uint32_t>((rb * g.k * g.V + v) * 4)
                                     : kOOB);
      }
    }
  };

  for (int pos = 0; pos < g.k; ++pos) {
    for (int64_t b0 = 0; b0 < g.B; b0 += 16) {
      load_z(pos, b0);  // independent of the context: in flight while the context is fetched
      u32x4_t ef[NC];
      context_frags<S, RKS>(g, b0, pos, r16, grp, ef);
      const int64_t nb = min<int64_t>(16, g.B - b0);
      float bv[4];
      uint32_t bi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bv[i] = -INFINITY;
        bi[i] = 0xFFFFFFFFu;
      }
#pragma unroll
      for (int u = 0; u < MAXT; ++u) {
        const int tile = wave + 4 * u;
        if (tile < ntl) {
          const int64_t v = (t_lo + tile) * 16 + r16;
          f32x4_t bias = {0.f, 0.f, 0.f, 0.f};
          if constexpr (RKS > 0) {
#pragma unroll
            for (int c = 0; c < RKS; ++c) bias = mma16(ef[c], w2s[(tile * RKS + c) * 64 + lane], bias, S());
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float s = zv[u][i] + bias[i];
            if (v < g.V && 4 * grp + i < nb && s > bv[i]) {
              bv[i] = s;
              bi[i] = static_cast<uint32_t>(v);
            }
          }
        }
      }
      publish_rows(g, b0, pos, wave, r16, grp, bv, bi, sk);
    }
    // grid barrier for this position; its last arriver writes the tokens
    if (threadIdx.x == 0) {
      last_flag = 0;
      if (arrive_group(g.gcnt + pos * kArriveGroups * kLineWords, blockIdx.x, G))
        last_flag = arrive_top(g.tcnt + pos * kLineWords, G) ? 1 : 0;
      if (!last_flag && pos + 1 < g.k) {
        const unsigned ng = arrive_groups(G);
        unsigned it = 0;
        while (fetch_u32(g.tcnt + pos * kLineWords) < ng) {
          __builtin_amdgcn_s_sleep(1);
          if (++it > kSpinLimit) {
            atomicOr(g.err, 1u);
            break;
          }
        }
      }
    }
    __syncthreads();
    if (last_flag) {
      for (int64_t b = threadIdx.x; b < g.B; b += blockDim.x)
        g.draft[b * g.k + pos] = key_index(final_key(g, pos, b));
      if (pos + 1 == g.k) {  // everyone has passed every barrier: return the workspace to zero
        __syncthreads();
        const int64_t nkeys = static_cast<int64_t>(g.k) * kArriveGroups * g.B;
        for (int64_t i = threadIdx.x; i < nkeys; i += blockDim.x) g.keys[i] = 0ull;
        for (int i = threadIdx.x; i < g.k * kArriveGroups; i += blockDim.x) g.gcnt[i * kLineWords] = 0u;
        for (int i = threadIdx.x; i < g.k; i += blockDim.x) g.tcnt[i * kLineWords] = 0u;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// passes: one launch per position
// ----------------------------------------------------------------------------
template <typename S, int RKS, int TPW>
__global__ __launch_bounds__(256) void markov_pass_kernel(const MarkovArgs g, int pos) {
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  constexpr int ES = static_cast<int>(sizeof(S));
  constexpr int NC = RKS > 0 ? RKS : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * 16;
  const int64_t nb = min<int64_t>(16, g.B - b0);
  __shared__ unsigned long long sk[4][16];

  if (pos > 0 && blockIdx.x == 0 && threadIdx.x < 16 && b0 + r16 < g.B)
    g.draft[(b0 + r16) * g.k + (pos - 1)] = key_index(final_key(g, pos - 1, b0 + r16));
  u32x4_t ef[NC];
  context_frags<S, RKS>(g, b0, pos, r16, grp, ef);

  const rsrc_t r2 = make_rsrc(g.w2, static_cast<uint32_t>(g.V * g.r * ES));
  const rsrc_t rz = make_rsrc(g.logits + (b0 * g.k + pos) * g.V,
                              static_cast<uint32_t>(((nb - 1) * g.k * g.V + g.V) * 4));
  uint32_t zrow[4];
  bool bok[4];
  float bv[4];
  uint32_t bi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rb = 4 * grp + i;
    bok[i] = rb < nb;
    zrow[i] = static_cast<uint32_t>(rb * g.k * g.V * 4);
    bv[i] = -INFINITY;
    bi[i] = 0xFFFFFFFFu;
  }

  const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 4 + wave; base < g.vtiles;
       base += nw * TPW) {
    u32x4_t wf[TPW][NC];
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
  publish_rows(g, b0, pos, wave, r16, grp, bv, bi, sk);
}

// last position's tokens; then the keys go back to zero
__global__ __launch_bounds__(256) void markov_finalize_kernel(MarkovArgs g) {
  for (int64_t b = threadIdx.x; b < g.B; b += blockDim.x)
    g.draft[b * g.k + (g.k - 1)] = key_index(final_key(g, g.k - 1, b));
  __syncthreads();
  const int64_t nkeys = static_cast<int64_t>(g.k) * kArriveGroups * g.B;
  for (int64_t i = threadIdx.x; i < nkeys; i += blockDim.x) g.keys[i] = 0ull;
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

// keys | group counters | top counters | error word
static size_t keys_bytes(int64_t B, int k) {
  return align256(static_cast<size_t>(B) * k * kArriveGroups * 8);
}
static size_t gcnt_bytes(int k) { return align256(static_cast<size_t>(k) * kArriveGroups * 128); }
static size_t tcnt_bytes(int k) { return align256(static_cast<size_t>(k) * 128); }

size_t markov_workspace(int64_t B, int k) {
  return keys_bytes(B, k) + gcnt_bytes(k) + tcnt_bytes(k) + 256;
}

constexpr size_t kChainLdsMax = 150 * 1024;

template <typename S, int RKS, int MAXT>
static hipError_t launch_chain_t(const MarkovArgs& g, unsigned G, size_t lds, hipStream_t st) {
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&markov_chain_kernel<S, RKS, MAXT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kChainLdsMax));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((markov_chain_kernel<S, RKS, MAXT>), dim3(G), dim3(256), lds, st, g);
  return hipSuccess;
}

// MAXT: 16-entry vocabulary tiles per wave (the workgroup's tiles / 4, rounded up)
template <typename S, int RKS>
static hipError_t launch_chain(const MarkovArgs& g, unsigned G, size_t lds, int64_t tiles_per_wg,
                               hipStream_t st) {
  const int64_t per_wave = (tiles_per_wg + 3) / 4;
  if (per_wave <= 2) return launch_chain_t<S, RKS, 2>(g, G, lds, st);
  if (per_wave <= 4) return launch_chain_t<S, RKS, 4>(g, G, lds, st);
  if (per_wave <= 8) return launch_chain_t<S, RKS, 8>(g, G, lds, st);
  if (per_wave <= 12) return launch_chain_t<S, RKS, 12>(g, G, lds, st);
  return launch_chain_t<S, RKS, 16>(g, G, lds, st);
}

template <typename S, int RKS>
static void launch_passes(const MarkovArgs& g, hipStream_t st) {
  constexpr int TPW = RKS <= 2 ? 8 : (RKS <= 4 ? 4 : 2);
  const int64_t wgs = std::min<int64_t>((g.vtiles + 4 * TPW - 1) / (4 * TPW), 1024);
  const dim3 grid(static_cast<unsigned>(wgs), static_cast<unsigned>((g.B + 15) / 16));
  for (int pos = 0; pos < g.k; ++pos)
    hipLaunchKernelGGL((markov_pass_kernel<S, RKS, TPW>), grid, dim3(256), 0, st, g, pos);
  hipLaunchKernelGGL(markov_finalize_kernel, dim3(1), dim3(256), 0, st, g);
}

template <typename S>
static hipError_t launch_typed(const MarkovArgs& g, int rks, int n_cu, hipStream_t st) {
  const unsigned G = static_cast<unsigned>(std::min<int64_t>(std::max(n_cu, 1), g.vtiles));
  const int64_t tiles = (g.vtiles + G - 1) / G;
  const size_t lds = static_cast<size_t>(tiles) * rks * 64 * 16;
  if (lds <= kChainLdsMax && tiles <= 64) {
    switch (rks) {
      case 0: return launch_chain<S, 0>(g, G, lds, tiles, st);
      case 1: return launch_chain<S, 1>(g, G, lds, tiles, st);
      case 2: return launch_chain<S, 2>(g, G, lds, tiles, st);
      case 3: return launch_chain<S, 3>(g, G, lds, tiles, st);
      case 4: return launch_chain<S, 4>(g, G, lds, tiles, st);
      default: break;  // larger fp32 ranks: per-position launches
    }
  }
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
  return hipSuccess;
}

hipError_t launch_markov(const float* logits, int64_t B, int k, int64_t V, bdr_dtype wdt,
                         const void* w1, const void* w2, int rank, const int32_t* prev,
                         int32_t* draft, void* workspace, int n_cu, hipStream_t stream) {
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
  g.keys = reinterpret_cast<unsigned long long*>(ws);
  g.gcnt = reinterpret_cast<unsigned*>(ws + keys_bytes(B, k));
  g.tcnt = reinterpret_cast<unsigned*>(ws + keys_bytes(B, k) + gcnt_bytes(k));
  g.err = reinterpret_cast<unsigned*>(ws + keys_bytes(B, k) + gcnt_bytes(k) + tcnt_bytes(k));
  g.draft = draft;
  g.vtiles = (V + 15) / 16;
  const int ks = wdt == BDR_BF16 ? Elem<uint16_t>::KSTEP : Elem<float>::KSTEP;
  const int rks = (g.r + ks - 1) / ks;
  hipError_t e = wdt == BDR_BF16 ? launch_typed<uint16_t>(g, rks, n_cu, stream)
                                 : launch_typed<float>(g, rks, n_cu, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace bdr
