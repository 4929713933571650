#pragma once

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
//             chain.  At each position every workgroup stores its local
//             maxima, tagged with the position, into its own slots (a plain
//             store, no read-modify-write), and the contexts of the next
//             position are formed from the slots:
//               B <= 2: every workgroup polls all slots until every tag is
//                       current and reduces them itself;
//               B > 2:  workgroup b % G reduces row b, stores the row's tagged
//                       token, and every workgroup polls the B tokens.
//             All workgroups must be resident at once: the grid is at most the
//             number of compute units and each workgroup fits in one.  Polls
//             are bounded in time (wall clock); a poll that gives up sets the
//             error word of the workspace, and the token it was waiting for
//             becomes -1 (no Markov bias as a later context) instead of the
//             kernel hanging.  The last workgroup to finish (a completion
//             counter) returns the slots to zero and moves the error word to
//             the caller's status word when one is given.
//   passes -- one launch per position (used when the markov_w2 slice does not
//             fit in LDS); stream order provides the grid-wide dependency, and
//             workgroup w folds its keys into group slot w % 16 (atomic max;
//             readers take the max over the 16 group slots).
//
// Workspace (zero-filled before first use; every call leaves it zeroed, except
// the error word when the caller passes no status word):
//   keys[k][16][B] uint64 (passes) | slots[k][B][256] uint64 (chain, per
//   workgroup, kSlotStride words apart) | tokens[k][B] uint64, each on its
//   own 128-byte line (chain,
//   B > 2) | completion counter (128 bytes) | error uint32 (the last 256
//   bytes)

#include <algorithm>

#include "bdr_device.h"
#include "bdr_internal.h"

namespace bdr {

// x of the sampling chain is written once and read once by verification:
// streaming (non-temporal) stores keep it from displacing the hand-off lines
__device__ __forceinline__ void xstore16(f32x4_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, 2);
}
__device__ __forceinline__ void xstore_f32(float v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 2);
}

struct MarkovArgs {
  const float* logits;           // [B, k, V]
  int64_t B, V;
  int k, r;
  const void* w1;                // [V, r] embedding of the context token
  const void* w2;                // [V, r] projection to the vocabulary
  const int32_t* prev;           // [B] context of position 0
  unsigned long long* keys;      // passes: [k, 16, B] per-position argmax keys per group
  unsigned long long* slots;     // chain: [k, B, kChainSlots] tagged local maxima, kSlotStride apart
  unsigned long long* tokens;    // chain: [k, B] tagged tokens (B > 2), kTokenStride apart
  unsigned* done;                // chain: completion counter
  unsigned* err;                 // error word
  int32_t* status;               // optional: receives the error word at the end (then cleared)
  unsigned long long poll_ticks; // wall-clock ticks a poll waits before giving up
  uint32_t forced_time_out;      // nonzero: every wait disregards what it reads (error-path tests)
  int32_t* draft;                // [B, k]
  int64_t vtiles;                // ceil(V / 16)
  // sampling (probabilistic drafting): the token of a position is the argmax
  // of x * inv_t + G, x = logits + bias, and x is stored; G is the standard
  // Gumbel variate of entry v of (row b, position i) from Philox4x32-10 keyed
  // by the seed, counter (v / 4, b, i, kStreamDraft), word v % 4 -- generated here, where
  // it is used, rather than read from memory
  uint32_t seed_lo, seed_hi;     // Philox key
  float* xout;                   // [B, k, V] biased logits x (the draft distribution)
  float inv_t;                   // 1 / temperature
  // x only for the positions verification reads: j < L_b, L_b the block length
  // by confidence (conf [B, k] and threshold th, when use_conf)
  const float* conf;
  float th;
  int use_conf;
};

// positions of row b whose x is stored
__device__ __forceinline__ int markov_x_len(const MarkovArgs& g, int64_t b) {
  return g.use_conf ? truncated_length<BDR_MAX_K>(g.conf + b * g.k, g.th, g.k) : g.k;
}

constexpr int kChainSlots = kNumCU;   // workgroups of the chain (at most)
constexpr int kChainMaxB = 256;       // rows the chain keeps contexts of in LDS
constexpr int kSinglePhaseB = 2;      // up to this many rows every workgroup reduces all slots
// Tokens sit one per 128-byte line: stores from many workgroups into one line
// are merged one after another at the memory side, which had made the token
// hand-off of 16 rows ~0.9 us slower per position.
constexpr int kTokenStride = 16;      // uint64 words
// Slots two words apart: eight writers per line instead of sixteen, at twice
// the bytes per poll (measured: one word 27.4 us for the B = 1 chain, two 26.4,
// four 26.8, sixteen 29.1; no change at B = 16 for two, worse for more).
constexpr int kSlotStride = 2;        // uint64 words


// final key of row b at position pos: max over the 16 group slots
__device__ __forceinline__ unsigned long long final_key(const MarkovArgs& g, int pos, int64_t b) {
  const unsigned long long* p = g.keys + static_cast<int64_t>(pos) * kArriveGroups * g.B + b;
  unsigned long long k = 0ull;
#pragma unroll
  for (int i = 0; i < kArriveGroups; ++i) k = umax64(k, fetch_u64(p + i * g.B));
  return k;
}

// Tagged keys of the chain hand-off: ordered value bits (32) | 0x1FFFFF - index
// (21) | tag (11), tag = position + 1.  Max order is the packed-key order
// (value, then lower index) among keys of one tag; a slot is current for a
// position iff its tag matches, and "no candidate" is the bare tag, below every
// real key.  Requires V <= 2^21.
constexpr int kTagBits = 11;
constexpr unsigned long long kTagMask = (1ull << kTagBits) - 1;
__device__ __forceinline__ unsigned long long tag_key(unsigned long long key, unsigned tag) {
  if (key == 0ull) return tag;
  const unsigned long long low = 0x1FFFFFull - key_index(key);
  return (key & 0xFFFFFFFF00000000ull) | (low << kTagBits) | tag;
}
__device__ __forceinline__ int32_t tagged_index(unsigned long long t) {
  return static_cast<int32_t>(0x1FFFFFu - static_cast<uint32_t>((t >> kTagBits) & 0x1FFFFFull));
}
// token of a reduced tagged key; a bare tag (no candidate: a poll that gave up)
// is -1, outside every vocabulary (a finite maximum never has zero value bits)
__device__ __forceinline__ int32_t tagged_token(unsigned long long t) {
  return (t >> 32) == 0ull ? -1 : tagged_index(t);
}

// Bounded wait: false once a poll that started failing at *t0 has waited
// longer than the workspace's limit (the first failed attempt starts the clock).
__device__ __forceinline__ bool keep_polling(const MarkovArgs& g, unsigned long long& t0,
                                             bool& started) {
  const unsigned long long now = static_cast<unsigned long long>(wall_clock64());
  if (!started) {
    started = true;
    t0 = now;
    return true;
  }
  return now - t0 <= g.poll_ticks;
}

// E fragments: markov_w1 row of context token p (the lane's row; p < 0 or
// p >= V: no bias)
template <typename S, int RKS>
__device__ __forceinline__ void context_frags(const MarkovArgs& g, int32_t p, int grp,
                                              u32x4_t (&ef)[RKS > 0 ? RKS : 1]) {
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  constexpr int ES = static_cast<int>(sizeof(S));
  if constexpr (RKS > 0) {
    const rsrc_t r1 = make_rsrc(g.w1, static_cast<uint32_t>(g.V * g.r * ES));
    const bool pok = p >= 0 && static_cast<int64_t>(p) < g.V;
#pragma unroll
    for (int c = 0; c < RKS; ++c) {
      const int j = c * KS + grp * E;
      ef[c] = bload16(r1, (pok && j < g.r)
                              ? static_cast<uint32_t>((static_cast<int64_t>(p) * g.r + j) * ES)
                              : kOOB);
    }
  }
}

// context token of row b at position pos for the passes schedule
__device__ __forceinline__ int32_t pass_context(const MarkovArgs& g, int pos, int64_t b) {
  if (b >= g.B) return -1;
  return pos == 0 ? g.prev[b] : key_index(final_key(g, pos - 1, b));
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

// Poll `n` <= kChainSlots tagged slots (stride `stride` from `base`) with one
// wave until all carry `tag`; returns their max (0 if the poll timed out, after
// setting the error word).  Every lane issues its kChainSlots / 64 loads back
// to back (addresses clamped into range, surplus lanes count as current), so
// one attempt costs one round trip.  Called by all 64 lanes of one wave.
__device__ __forceinline__ unsigned long long poll_max(const MarkovArgs& g,
                                                       const unsigned long long* base,
                                                       int64_t stride, int n, unsigned tag,
                                                       int lane) {
  constexpr int PL = kChainSlots / 64;
  unsigned long long t0 = 0;
  bool started = false;
  for (;;) {
    unsigned long long t[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int i = lane + 64 * j;
      t[j] = fetch_u64(base + static_cast<int64_t>(i < n ? i : n - 1) * stride);
    }
    unsigned long long m = 0ull;
    bool ok = true;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const bool cur = lane + 64 * j >= n || (t[j] & kTagMask) == tag;
      ok = ok & cur;
      m = umax64(m, t[j]);
    }
    if (__all(ok) && !g.forced_time_out) return wave_max64(m);
    if (!keep_polling(g, t0, started)) {
      if (lane == 0) atomicOr(g.err, 1u);
      return 0ull;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not its global loads, so prefetched loads stay in flight across it.
#define BDR_LDS_BARRIER()                              \
  do {                                                 \
    __builtin_amdgcn_s_waitcnt(0xC07F);  /* lgkmcnt(0) */ \
    asm volatile("s_barrier" ::: "memory");            \
    __builtin_amdgcn_sched_barrier(0);                 \
  } while (0)

// Waves of a chain workgroup: wave 0 for the hand-off and four compute waves,
// each with a quarter of the workgroup's vocabulary tiles (sampling: the
// compute waves generate the next position's noise while wave 0 waits).  W4:
// four waves, wave 0 also taking the hand-off once its tiles are compared,
// each within 168 registers (three waves' worth), so that a batched fc wave
// of up to 344 registers fits beside the chain on every SIMD and that GEMM
// runs beside it (with five waves one SIMD holds two chain waves).  Built
// for greedy drafting with ranks up to 64 and at most ten tiles a wave (more
// would spill), and launched from kChainW4MinB rows on (for fewer rows the fc
// runs in one launch with the LM head, and wave 0's own logits prefetch,
// which its polls retire behind, made the chain slower).
constexpr int kChainW4MinB = 8;
template <bool W4>
constexpr int chain_waves() {
  return W4 ? 4 : 5;
}

template <typename S, int RKS, int MAXT, bool SAMPLE, bool ONE, bool W4 = false>
__global__ __launch_bounds__(64 * chain_waves<W4>(), W4 ? 3 : 2)
void markov_chain_kernel(const MarkovArgs g) {
  static_assert(!W4 || (!SAMPLE && RKS <= 2 && MAXT <= 10), "four-wave chain: greedy, small");
  extern __shared__ u32x4_t w2s[];   // [tile][chunk][lane] operand chunks of markov_w2
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  constexpr int ES = static_cast<int>(sizeof(S));
  constexpr int NC = RKS > 0 ? RKS : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  constexpr int NW = chain_waves<W4>();
  const int cw = W4 ? wave : wave - 1;   // compute wave index, -1 for a hand-off-only wave 0
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const unsigned G = gridDim.x;
  const int64_t t_lo = static_cast<int64_t>(blockIdx.x) * g.vtiles / G;
  const int64_t t_hi = static_cast<int64_t>(blockIdx.x + 1) * g.vtiles / G;
  const int ntl = static_cast<int>(t_hi - t_lo);   // compute wave c owns tiles c, c+4, ... (< 4*MAXT)
  const bool single = g.B <= kSinglePhaseB;

  __shared__ unsigned long long sk[4][4][16];      // [compute wave][lane group][row]
  __shared__ int32_t ctx[kChainMaxB];              // context token of every row
  __shared__ int xlen[SAMPLE ? kChainMaxB : 1];    // sampling: positions of x stored per row
  __shared__ int last_flag;

  // stage this workgroup's markov_w2 rows in operand layout (lane l's 16 bytes
  // of chunk q land at w2s[q*64 + l])
  if constexpr (RKS > 0) {
    const rsrc_t r2 = make_rsrc(g.w2, static_cast<uint32_t>(g.V * g.r * ES));
    for (int q = wave; q < ntl * RKS; q += NW) {
      const int tile = q / RKS;
      const int c = q - tile * RKS;
      const int64_t v = (t_lo + tile) * 16 + r16;
      const int j = c * KS + grp * E;
      const uint32_t off = (v < g.V && j < g.r) ? static_cast<uint32_t>((v * g.r + j) * ES) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r2, (__attribute__((address_space(3))) void*)(&w2s[q * 64]), 16, off, 0, 0, 0);
    }
  }
  for (int64_t b = threadIdx.x; b < g.B; b += blockDim.x) {
    ctx[b] = g.prev[b];
    if constexpr (SAMPLE) xlen[b] = markov_x_len(g, b);
  }

  // logits of position pos, row b0 + r16, vocabulary entries 16 * tile + 4 * grp
  // .. + 3 of this compute wave's tiles: one 16-byte load per tile (entries
  // past V are masked when compared).  Indices fit 32 bits (V <= 2^21, k <= 16,
  // operands < 2^31 bytes).
  const int V32 = static_cast<int>(g.V);
  const int vbase = static_cast<int>(t_lo) * 16 + 4 * grp;   // + 16 * tile
  const uint32_t zrow = static_cast<uint32_t>(g.k) * static_cast<uint32_t>(g.V) * 4u;
  u32x4_t zv[MAXT];
  u32x4_t gv[SAMPLE ? MAXT : 1];   // sampling: the draws' Gumbel noise, same layout
  // bytes of the [nb rows][k][V] fp32 block a row group's position spans
  auto block_bytes = [&](int64_t b0) {
    const int nb = static_cast<int>(min<int64_t>(16, g.B - b0));
    return static_cast<uint32_t>(nb - 1) * zrow + static_cast<uint32_t>(V32) * 4u;
  };
  // cwo / ntlo / vbo: this wave's first tile, the workgroup's tile count and
  // the lane's first entry, passed in opaque per position (see below)
  auto load_z = [&](int pos, int64_t b0, int cwo, int ntlo, int vbo) {
    const int nb = static_cast<int>(min<int64_t>(16, g.B - b0));
    const int64_t first = (b0 * g.k + pos) * g.V;
    const rsrc_t rz = make_rsrc(g.logits + first, block_bytes(b0));
    const uint32_t lane_off = static_cast<uint32_t>(r16) * zrow;
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int tile = cwo + 4 * u;
      const int v0 = vbo + 16 * tile;
      const uint32_t off = (tile < ntlo && v0 < V32 && r16 < nb)
                               ? lane_off + static_cast<uint32_t>(v0) * 4u
                               : kOOB;
      zv[u] = bload16(rz, off);
    }
  };
  // sampling: the Gumbel variates of the lane's quads (entries v0 .. v0 + 3 of
  // row b0 + r16 are words 0..3 of one Philox call); ALU work, done while the
  // hand-off waits
  auto gen_noise = [&](int pos, int64_t b0, int cwo, int ntlo, int vbo) {
    if constexpr (SAMPLE) {
      const uint32_t row = static_cast<uint32_t>(b0 + r16);
#pragma unroll
      for (int u = 0; u < MAXT; ++u) {
        const int tile = cwo + 4 * u;
        const int v0 = vbo + 16 * tile;
        if (tile < ntlo && v0 < V32 && row < g.B) {
          const u32x4_t x = philox4x32_10(
              u32x4_t{static_cast<uint32_t>(v0) >> 2, row, static_cast<uint32_t>(pos), kStreamDraft},
              g.seed_lo, g.seed_hi);
#pragma unroll
          for (int w = 0; w < 4; ++w) gv[u][w] = __float_as_uint(gumbel_of(bits_to_uniform(x[w])));
        }
      }
    }
  };
  // One row (B == 1): the product is taken the other way round, D[row][entry]
  // = context embeddings x markov_w2 rows, so lane (r16, grp) holds entry
  // 16 * tile + r16 of row 4 * grp (the batch's row in grp 0 lanes) and each
  // tile costs one compare per lane instead of four.  z1 / n1: the lane's
  // logit and noise of each of its tiles.
  float z1[ONE ? MAXT : 1];
  float n1[ONE && SAMPLE ? MAXT : 1];
  uint32_t x1[ONE && SAMPLE ? MAXT : 1];   // where the lane stores x of the entry (kOOB: nowhere)
  const int vbase1 = static_cast<int>(t_lo) * 16 + r16;   // + 16 * tile
  auto load_z1 = [&](int pos, int cwo, int ntlo, int vbo) {
    const int64_t first = static_cast<int64_t>(pos) * g.V;
    const uint32_t bytes = static_cast<uint32_t>(V32) * 4u;
    const rsrc_t rz = make_rsrc(g.logits + first, bytes);
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int tile = cwo + 4 * u;
      const int v = vbo + 16 * tile;
      const uint32_t off = (grp == 0 && tile < ntlo && v < V32) ? static_cast<uint32_t>(v) * 4u : kOOB;
      z1[u] = bload_f32(rz, off);
      if constexpr (SAMPLE) x1[u] = off;
    }
  };
  // sampling, one row: the lane's entry v is word v % 4 (= r16 % 4) of the
  // Philox call of its quad
  auto gen_noise1 = [&](int pos, int cwo, int ntlo, int vbo) {
    if constexpr (ONE && SAMPLE) {
      const int w = r16 & 3;
#pragma unroll
      for (int u = 0; u < MAXT; ++u) {
        const int tile = cwo + 4 * u;
        const int v = vbo + 16 * tile;
        if (grp == 0 && tile < ntlo && v < V32) {
          const u32x4_t x = philox4x32_10(
              u32x4_t{static_cast<uint32_t>(v) >> 2, 0u, static_cast<uint32_t>(pos), kStreamDraft},
              g.seed_lo, g.seed_hi);
          const uint32_t bits = w == 0 ? x[0] : w == 1 ? x[1] : w == 2 ? x[2] : x[3];
          n1[u] = gumbel_of(bits_to_uniform(bits));
        }
      }
    }
  };
  if (cw >= 0) {
    if constexpr (ONE) {
      load_z1(0, cw, ntl, vbase1);
      gen_noise1(0, cw, ntl, vbase1);
    } else {
      load_z(0, 0, cw, ntl, vbase);
      gen_noise(0, 0, cw, ntl, vbase);
    }
  }
  BDR_WAIT_VM(0);
  __syncthreads();

  for (int pos = 0; pos < g.k; ++pos) {
    const unsigned tag = static_cast<unsigned>(pos) + 1;
    for (int64_t b0 = 0; b0 < g.B; b0 += 16) {
      const int64_t nb = min<int64_t>(16, g.B - b0);
      const bool last_group = b0 + 16 >= g.B;
      if (cw >= 0) {
        // per-tile indices are recomputed each position from opaque copies
        // instead of being kept live (in registers) across the whole chain
        int cwo = cw, ntlo = ntl, vbo = ONE ? vbase1 : vbase;
        asm volatile("" : "+s"(cwo), "+s"(ntlo), "+v"(vbo));
        if constexpr (ONE) {
          u32x4_t ef[NC];
          context_frags<S, RKS>(g, r16 == 0 ? ctx[0] : -1, grp, ef);
          // entries past the workgroup's range or the vocabulary get logit
          // -inf (their key is -inf or NaN, which never wins), set here while
          // the context embedding is in flight rather than in the compare loop
#pragma unroll
          for (int u = 0; u < MAXT; ++u) {
            const int tile = cwo + 4 * u;
            if (!(tile < ntlo && vbo + 16 * tile < V32)) z1[u] = -INFINITY;
          }
          float bv = -INFINITY;
          int bu = -1;   // tile slot u of the lane's maximum
          rsrc_t rx;
          bool xl = false;   // x of this position is stored
          if constexpr (SAMPLE) {
            rx = make_rsrc(g.xout + static_cast<int64_t>(pos) * g.V, static_cast<uint32_t>(V32) * 4u);
            xl = pos < xlen[0];
          }
#pragma unroll
          for (int u = 0; u < MAXT; ++u) {
            const int tile = cwo + 4 * u;
            const int tile_rd = tile < ntlo ? tile : ntlo - 1;
            f32x4_t d = {0.f, 0.f, 0.f, 0.f};
            if constexpr (RKS > 0) {
#pragma unroll
              for (int c = 0; c < RKS; ++c)
                d = mma16(ef[c], w2s[(tile_rd * RKS + c) * 64 + lane], d, S());
            }
            const float sv = z1[u] + d[0];
            float key = sv;
            if constexpr (SAMPLE) {
              key = sv * g.inv_t + n1[u];
              xstore_f32(sv, rx, xl ? x1[u] : kOOB);
            }
            if (key > bv) {
              bv = key;
              bu = u;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if (pos + 1 < g.k) load_z1(pos + 1, cwo, ntlo, vbo);
          // the row's maximum over the 16 lanes of grp 0, then over the waves
          unsigned long long key =
              bu >= 0 ? pack_key(bv, static_cast<uint32_t>(vbo + 16 * (cwo + 4 * bu))) : 0ull;
          key = rowgroup_max16(key);
          if (lane == 0) sk[cw][0][0] = key;
        } else {
          if (b0 > 0) {   // the first row group's logits (and noise) were prefetched
            load_z(pos, b0, cwo, ntlo, vbo);
            gen_noise(pos, b0, cwo, ntlo, vbo);
          }
          u32x4_t ef[NC];
          context_frags<S, RKS>(g, b0 + r16 < g.B ? ctx[b0 + r16] : -1, grp, ef);
          // entries past the workgroup's range or the vocabulary get logit
          // -inf (never winning), set while the context embeddings are in
          // flight; rows past the batch are never published and need no mask
#pragma unroll
          for (int u = 0; u < MAXT; ++u) {
            const int tile = cwo + 4 * u;
            const int lim = tile < ntlo ? V32 - (vbo + 16 * tile) : 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (!(i < lim)) zv[u][i] = 0xFF800000u;
          }
          // bias tile D[vocab 4 * grp + i][row r16] = markov_w2 rows x context
          // embeddings; each lane keeps the running maximum of its row r16 over
          // the entries it visits in increasing order (bs: slot 4 u + i of it).
          // Reads past the workgroup's last tile repeat it (no branch).
          float bv = -INFINITY;
          int bs = -1;
          const bool row_ok = r16 < nb;
          bool x_ok = false;   // x of row r16 at this position is stored
          if constexpr (SAMPLE) x_ok = row_ok && pos < xlen[row_ok ? b0 + r16 : 0];
          rsrc_t rx;
          f32x4_t xt = {0.f, 0.f, 0.f, 0.f};
          uint32_t toff = kOOB;
          if constexpr (SAMPLE) rx = make_rsrc(g.xout + (b0 * g.k + pos) * g.V, block_bytes(b0));
#pragma unroll
          for (int u = 0; u < MAXT; ++u) {
            const int tile = cwo + 4 * u;
            const int tile_rd = tile < ntlo ? tile : ntlo - 1;
            f32x4_t bias = {0.f, 0.f, 0.f, 0.f};
            if constexpr (RKS > 0) {
#pragma unroll
              for (int c = 0; c < RKS; ++c)
                bias = mma16(w2s[(tile_rd * RKS + c) * 64 + lane], ef[c], bias, S());
            }
            f32x4_t xs;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float s = __uint_as_float(zv[u][i]) + bias[i];
              float key = s;
              if constexpr (SAMPLE) {
                xs[i] = s;
                key = s * g.inv_t + __uint_as_float(gv[u][i]);
              }
              if (key > bv) {
                bv = key;
                bs = 4 * u + i;
              }
            }
            if constexpr (SAMPLE) {
              // entries of the lane's quad that exist (<= 0: none)
              const int v0 = vbo + 16 * tile;
              const int lim = (x_ok && tile < ntlo) ? V32 - v0 : 0;
              // x of the lane's four entries in one 16-byte store; the quad that
              // straddles the end of the row (at most one per lane) is kept for
              // element stores after the loop
              const uint32_t off = static_cast<uint32_t>(r16) * zrow + static_cast<uint32_t>(v0) * 4u;
              xstore16(xs, rx, lim >= 4 ? off : kOOB);
              const bool part = lim > 0 && lim < 4;
              xt = part ? xs : xt;
              toff = part ? off : toff;
            }
          }
          if constexpr (SAMPLE) {
            const int tn = V32 & 3;   // entries of a straddling quad
            if (toff != kOOB) {
#pragma unroll
              for (int i = 0; i < 3; ++i) xstore_f32(xt[i], rx, i < tn ? toff + 4u * i : kOOB);
            }
          }
          // the next position's first logits: independent of the hand-off below
          // (kept after the compares so the two logits sets are never live together)
          __builtin_amdgcn_sched_barrier(0);
          if (last_group && pos + 1 < g.k) load_z(pos + 1, 0, cwo, ntlo, vbo);
          // row r16's maximum over the lane groups and waves, taken from LDS
          sk[cw][grp][r16] =
              bs >= 0 ? pack_key(bv, static_cast<uint32_t>(vbo + 16 * (cwo + 4 * (bs >> 2)) + (bs & 3)))
                      : 0ull;
        }
      }
      BDR_LDS_BARRIER();
      // this workgroup's maxima of rows b0.. -> its tagged slots
      if (threadIdx.x < nb) {
        unsigned long long key = 0ull;
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int q = 0; q < (ONE ? 1 : 4); ++q) key = umax64(key, sk[w][q][threadIdx.x]);
        publish_u64(g.slots + ((pos * g.B + b0 + threadIdx.x) * kChainSlots + blockIdx.x) * kSlotStride,
                    tag_key(key, tag));
      }
      if (!last_group) BDR_LDS_BARRIER();   // sk is rewritten by the next row group
    }
    // sampling: the next position's noise, while wave 0 waits for the hand-off
    if constexpr (SAMPLE) {
      if (cw >= 0 && pos + 1 < g.k) {
        int cwo = cw, ntlo = ntl, vbo = ONE ? vbase1 : vbase;
        asm volatile("" : "+s"(cwo), "+s"(ntlo), "+v"(vbo));
        if constexpr (ONE)
          gen_noise1(pos + 1, cwo, ntlo, vbo);
        else
          gen_noise(pos + 1, 0, cwo, ntlo, vbo);
      }
    }
    // contexts of the next position (and this position's tokens)
    if (wave == 0) {
      // row b's slots of this position are adjacent: [pos][b][workgroup]
      const unsigned long long* pos_slots =
          g.slots + static_cast<int64_t>(pos) * g.B * kChainSlots * kSlotStride;
      if (single) {
        for (int64_t b = 0; b < g.B; ++b) {
          const int32_t tok =
              tagged_token(poll_max(g, pos_slots + b * kChainSlots * kSlotStride, kSlotStride,
                                    static_cast<int>(G), tag, lane));
          if (lane == 0) {
            ctx[b] = tok;
            if (blockIdx.x == 0) g.draft[b * g.k + pos] = tok;
          }
        }
      } else {
        unsigned long long* toks = g.tokens + static_cast<int64_t>(pos) * g.B * kTokenStride;
        for (int64_t b = blockIdx.x; b < g.B; b += G) {   // rows this workgroup reduces
          const unsigned long long t =
              poll_max(g, pos_slots + b * kChainSlots * kSlotStride, kSlotStride,
                       static_cast<int>(G), tag, lane);
          if (lane == 0) {
            g.draft[b * g.k + pos] = tagged_token(t);
            publish_u64(toks + b * kTokenStride, (t & ~kTagMask) | tag);
          }
        }
        for (int64_t b0 = 0; b0 < g.B; b0 += 64) {
          const int n = static_cast<int>(min<int64_t>(64, g.B - b0));
          unsigned long long t0 = 0;
          bool started = false;
          for (;;) {
            unsigned long long t = fetch_u64(toks + (b0 + (lane < n ? lane : n - 1)) * kTokenStride);
            const bool cur = (t & kTagMask) == tag;
            if (__all(lane >= n || cur) && !g.forced_time_out) {
              if (lane < n) ctx[b0 + lane] = tagged_token(t);
              break;
            }
            if (!keep_polling(g, t0, started)) {
              // rows whose token never came get no Markov context
              if (lane < n) ctx[b0 + lane] = cur ? tagged_token(t) : -1;
              if (lane == 0) atomicOr(g.err, 1u);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
      }
    }
    BDR_LDS_BARRIER();
  }

  // the last workgroup to finish returns the slots to zero (every other one has
  // finished reading them)
  if (threadIdx.x == 0) {
    BDR_WAIT_ALL_MEM();
    last_flag = atomicAdd(g.done, 1u) + 1 == G ? 1 : 0;
  }
  __syncthreads();
  if (last_flag) {
    const int64_t nslots = static_cast<int64_t>(g.k) * kChainSlots * g.B;
    for (int64_t i = threadIdx.x; i < nslots; i += blockDim.x) g.slots[i * kSlotStride] = 0ull;
    if (!single)
      for (int64_t i = threadIdx.x; i < static_cast<int64_t>(g.k) * g.B; i += blockDim.x)
        g.tokens[i * kTokenStride] = 0ull;
    if (threadIdx.x == 0) {
      *g.done = 0u;
      // every workgroup's error report precedes its arrival on the counter
      if (g.status) {
        g.status[0] = static_cast<int32_t>(fetch_u32(g.err));
        __hip_atomic_store(g.err, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// passes: one launch per position
// ----------------------------------------------------------------------------
template <typename S, int RKS, int TPW, bool SAMPLE>
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
  context_frags<S, RKS>(g, pass_context(g, pos, b0 + r16), grp, ef);

  const rsrc_t r2 = make_rsrc(g.w2, static_cast<uint32_t>(g.V * g.r * ES));
  const uint32_t blk = static_cast<uint32_t>(((nb - 1) * g.k * g.V + g.V) * 4);
  const rsrc_t rz = make_rsrc(g.logits + (b0 * g.k + pos) * g.V, blk);
  rsrc_t rx;
  if constexpr (SAMPLE) rx = make_rsrc(g.xout + (b0 * g.k + pos) * g.V, blk);
  uint32_t zrow[4];
  bool bok[4];
  bool xok[4];   // sampling: x of the row at this position is stored
  float bv[4];
  uint32_t bi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rb = 4 * grp + i;
    bok[i] = rb < nb;
    xok[i] = SAMPLE && bok[i] && pos < markov_x_len(g, b0 + rb);
    zrow[i] = static_cast<uint32_t>(rb * g.k * g.V * 4);
    bv[i] = -INFINITY;
    bi[i] = 0xFFFFFFFFu;
  }

  const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 4 + wave; base < g.vtiles;
       base += nw * TPW) {
    u32x4_t wf[TPW][NC];
    float zv[TPW][4];
    float gn[SAMPLE ? TPW : 1][4];
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
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (vok && bok[i]) ? zrow[i] + static_cast<uint32_t>(v * 4) : kOOB;
        zv[u][i] = bload_f32(rz, off);
        if constexpr (SAMPLE) {
          // entry v of row b0 + 4 grp + i: word v % 4 of its quad's Philox call
          gn[u][i] = 0.f;
          if (vok && bok[i]) {
            const u32x4_t x = philox4x32_10(
                u32x4_t{static_cast<uint32_t>(v) >> 2, static_cast<uint32_t>(b0 + 4 * grp + i),
                        static_cast<uint32_t>(pos), kStreamDraft},
                g.seed_lo, g.seed_hi);
            const int w = static_cast<int>(v & 3);
            gn[u][i] = gumbel_of(bits_to_uniform(w == 0 ? x[0] : w == 1 ? x[1] : w == 2 ? x[2] : x[3]));
          }
        }
      }
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
        float key = s;
        if constexpr (SAMPLE) {
          key = s * g.inv_t + gn[u][i];
          xstore_f32(s, rx, (v < g.V && xok[i]) ? zrow[i] + static_cast<uint32_t>(v * 4) : kOOB);
        }
        if (v < g.V && bok[i] && key > bv[i]) {
          bv[i] = key;
          bi[i] = static_cast<uint32_t>(v);
        }
      }
    }
  }
  publish_rows(g, b0, pos, wave, r16, grp, bv, bi, sk);
}

// last position's tokens; then the keys go back to zero (the per-position
// launches never wait on one another: the status is the error word as it stands)
static __global__ __launch_bounds__(256) void markov_finalize_kernel(MarkovArgs g) {
  if (g.status && threadIdx.x == 0) {
    g.status[0] = static_cast<int32_t>(fetch_u32(g.err));
    __hip_atomic_store(g.err, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int64_t b = threadIdx.x; b < g.B; b += blockDim.x)
    g.draft[b * g.k + (g.k - 1)] = key_index(final_key(g, g.k - 1, b));
  __syncthreads();
  const int64_t nkeys = static_cast<int64_t>(g.k) * kArriveGroups * g.B;
  for (int64_t i = threadIdx.x; i < nkeys; i += blockDim.x) g.keys[i] = 0ull;
}

constexpr size_t kChainLdsMax = 150 * 1024;

template <typename S, int RKS, int MAXT, bool SAMPLE, bool ONE, bool W4 = false>
static hipError_t launch_chain_r(const MarkovArgs& g, unsigned G, size_t lds, hipStream_t st) {
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&markov_chain_kernel<S, RKS, MAXT, SAMPLE, ONE, W4>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kChainLdsMax));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((markov_chain_kernel<S, RKS, MAXT, SAMPLE, ONE, W4>), dim3(G),
                     dim3(64 * chain_waves<W4>()), lds, st, g);
  return hipSuccess;
}

template <typename S, int RKS, int MAXT, bool SAMPLE>
static hipError_t launch_chain_t(const MarkovArgs& g, unsigned G, size_t lds, hipStream_t st) {
  if (g.B == 1) return launch_chain_r<S, RKS, MAXT, SAMPLE, true>(g, G, lds, st);
  if constexpr (!SAMPLE && RKS <= 2 && MAXT <= 10) {
    if (g.B >= kChainW4MinB) return launch_chain_r<S, RKS, MAXT, false, false, true>(g, G, lds, st);
  }
  return launch_chain_r<S, RKS, MAXT, SAMPLE, false>(g, G, lds, st);
}

// MAXT: 16-entry vocabulary tiles per wave (the workgroup's tiles / 4, rounded up)
template <typename S, int RKS, bool SAMPLE>
static hipError_t launch_chain(const MarkovArgs& g, unsigned G, size_t lds, int64_t tiles_per_wg,
                               hipStream_t st) {
  const int64_t per_wave = (tiles_per_wg + 3) / 4;
  if (per_wave <= 2) return launch_chain_t<S, RKS, 2, SAMPLE>(g, G, lds, st);
  if (per_wave <= 4) return launch_chain_t<S, RKS, 4, SAMPLE>(g, G, lds, st);
  if (per_wave <= 8) return launch_chain_t<S, RKS, 8, SAMPLE>(g, G, lds, st);
  if (per_wave <= 10) return launch_chain_t<S, RKS, 10, SAMPLE>(g, G, lds, st);
  if (per_wave <= 12) return launch_chain_t<S, RKS, 12, SAMPLE>(g, G, lds, st);
  return launch_chain_t<S, RKS, 16, SAMPLE>(g, G, lds, st);
}

template <typename S, int RKS, bool SAMPLE>
static void launch_passes(const MarkovArgs& g, hipStream_t st) {
  constexpr int TPW = RKS <= 2 ? 8 : (RKS <= 4 ? 4 : 2);
  const int64_t wgs = std::min<int64_t>((g.vtiles + 4 * TPW - 1) / (4 * TPW), 1024);
  const dim3 grid(static_cast<unsigned>(wgs), static_cast<unsigned>((g.B + 15) / 16));
  for (int pos = 0; pos < g.k; ++pos)
    hipLaunchKernelGGL((markov_pass_kernel<S, RKS, TPW, SAMPLE>), grid, dim3(256), 0, st, g, pos);
  hipLaunchKernelGGL(markov_finalize_kernel, dim3(1), dim3(256), 0, st, g);
}

template <typename S, bool SAMPLE>
static hipError_t launch_typed(const MarkovArgs& g, int rks, int n_cu, hipStream_t st) {
  const unsigned G = static_cast<unsigned>(
      std::min<int64_t>(std::min(std::max(n_cu, 1), kChainSlots), g.vtiles));
  const int64_t tiles = (g.vtiles + G - 1) / G;
  const size_t lds = static_cast<size_t>(tiles) * rks * 64 * 16;
  if (lds <= kChainLdsMax && tiles <= 64 && g.B <= kChainMaxB) {
    switch (rks) {
      case 0: return launch_chain<S, 0, SAMPLE>(g, G, lds, tiles, st);
      case 1: return launch_chain<S, 1, SAMPLE>(g, G, lds, tiles, st);
      case 2: return launch_chain<S, 2, SAMPLE>(g, G, lds, tiles, st);
      case 3: return launch_chain<S, 3, SAMPLE>(g, G, lds, tiles, st);
      case 4: return launch_chain<S, 4, SAMPLE>(g, G, lds, tiles, st);
      default: break;  // larger fp32 ranks: per-position launches
    }
  }
  switch (rks) {
    case 0: launch_passes<S, 0, SAMPLE>(g, st); break;
    case 1: launch_passes<S, 1, SAMPLE>(g, st); break;
    case 2: launch_passes<S, 2, SAMPLE>(g, st); break;
    case 3: launch_passes<S, 3, SAMPLE>(g, st); break;
    case 4: launch_passes<S, 4, SAMPLE>(g, st); break;
    case 5: launch_passes<S, 5, SAMPLE>(g, st); break;
    case 6: launch_passes<S, 6, SAMPLE>(g, st); break;
    case 7: launch_passes<S, 7, SAMPLE>(g, st); break;
    default: launch_passes<S, 8, SAMPLE>(g, st); break;
  }
  return hipSuccess;
}

// MarkovArgs over a workspace of markov_workspace(B, k) bytes (sampling fields unset).
MarkovArgs markov_args(const float* logits, int64_t B, int k, int64_t V, const void* w1,
                       const void* w2, int rank, const int32_t* prev, int32_t* draft,
                       int32_t* status, void* workspace);

// Launch the schedule that fits (g.r already 0 when no Markov weights are given).
template <bool SAMPLE>
hipError_t markov_dispatch(const MarkovArgs& g, bdr_dtype wdt, int n_cu, hipStream_t stream) {
  const int ks = wdt == BDR_BF16 ? Elem<uint16_t>::KSTEP : Elem<float>::KSTEP;
  const int rks = (g.r + ks - 1) / ks;
  hipError_t e = wdt == BDR_BF16 ? launch_typed<uint16_t, SAMPLE>(g, rks, n_cu, stream)
                                 : launch_typed<float, SAMPLE>(g, rks, n_cu, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace bdr
