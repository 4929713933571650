// Device-side helpers shared by the gfx950 kernels of libbdr.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Storage element traits.  Every lane moves 16 bytes per load; KSTEP is the
// reduction depth one 16-byte load per lane covers across the four 16-lane
// groups of a wave (the K extent of the MFMA work issued for it).
template <typename S> struct Elem;
template <> struct Elem<uint16_t> {  // bfloat16 bit patterns
  static constexpr int PER16 = 8;
  static constexpr int KSTEP = 32;
  static constexpr int MFMA_PER16 = 1;   // MFMA instructions per 16-byte operand chunk
};
template <> struct Elem<float> {
  static constexpr int PER16 = 4;
  static constexpr int KSTEP = 16;
  static constexpr int MFMA_PER16 = 4;
};

// ----------------------------------------------------------------------------
// Raw buffer loads.  A buffer resource carries a base address and a byte size;
// a 16-byte load whose offset lies at or beyond the size returns zeros without
// touching memory, which pads ragged tiles with no branches.
// ----------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw-buffer data format word
constexpr uint32_t kOOB = 0x80000000u;   // an offset beyond every resource used here

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kRsrcWord3);
}

__device__ __forceinline__ u32x4_t bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// the same with the non-temporal hint (data streamed once)
__device__ __forceinline__ u32x4_t bload16_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

__device__ __forceinline__ float bload_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Buffer stores: a store whose offset lies at or beyond the size is dropped.
__device__ __forceinline__ void bstore16(f32x4_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, 0);
}

__device__ __forceinline__ void bstore_f32(float v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left unconstrained), and keep the
// scheduler from moving anything across.  Needed after buffer-to-LDS loads,
// which the compiler's own wait insertion does not track.
#define BDR_WAIT_VM(n)                                                                        \
  do {                                                                                        \
    __builtin_amdgcn_s_waitcnt(((n)&0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 3) << 14)); \
    __builtin_amdgcn_sched_barrier(0);                                                        \
  } while (0)

// Cross-workgroup hand-off without cache maintenance: data published for other
// workgroups is stored and loaded with agent-scope atomic accesses (coherent
// across the chip's L2 slices), and a wave orders its publications before an
// arrival counter by waiting for its own outstanding memory operations.
// (A full __threadfence() writes back and invalidates the whole L2 slice.)
__device__ __forceinline__ void publish_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long fetch_u64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned fetch_u32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#define BDR_WAIT_ALL_MEM()                    \
  do {                                        \
    __builtin_amdgcn_s_waitcnt(0);            \
    __builtin_amdgcn_sched_barrier(0);        \
  } while (0)

// Two-level arrival counting.  Same-address device-scope atomics serialise,
// so G workgroups arrive on group counters (workgroup w in group w % 16, each
// counter on its own 128-byte line) and only each group's last arriver
// touches the top counter.  Called by one thread per workgroup.
constexpr int kArriveGroups = 16;
constexpr int kLineWords = 32;   // 128-byte stride between counters (uint32 units)

__device__ __forceinline__ unsigned arrive_groups(unsigned G) {
  return G < kArriveGroups ? G : kArriveGroups;
}

// true for the last workgroup of w's group to arrive
__device__ __forceinline__ bool arrive_group(unsigned* grp_cnt, unsigned w, unsigned G) {
  const unsigned gi = w % kArriveGroups;
  const unsigned gsz = G < kArriveGroups ? 1u : G / kArriveGroups + (gi < G % kArriveGroups ? 1u : 0u);
  return atomicAdd(&grp_cnt[gi * kLineWords], 1u) + 1 == gsz;
}

// true for the last group to arrive
__device__ __forceinline__ bool arrive_top(unsigned* top_cnt, unsigned G) {
  return atomicAdd(top_cnt, 1u) + 1 == arrive_groups(G);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ u32x4_t load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// D(16x16, fp32) += A(16 x KSTEP) * B(KSTEP x 16) for one 16-byte operand chunk
// per lane.  Lane l supplies row/column (l & 15) and reduction group (l >> 4) of
// both operands with the same element order, so the reduction index is paired
// identically on both sides whatever the hardware's slot order within a group.
__device__ __forceinline__ f32x4_t mma16(u32x4_t a, u32x4_t b, f32x4_t c, uint16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma16(u32x4_t a, u32x4_t b, f32x4_t c, float) {
  // four K=4 fp32 MFMAs; element e of lane group g is reduction index 4g + e
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename S> __device__ __forceinline__ float to_f32(S x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

// ---------------------------------------------------------------------------
// Argmax keys.  A (value, index) pair packs into a uint64 whose unsigned order
// is: larger value first, then lower index.  -0.0 is folded into +0.0 so the
// two tie.  Key 0 is below every real key and serves as "empty".
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long pack_key(float v, uint32_t idx) {
  return (static_cast<unsigned long long>(ordered_bits(v)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ int32_t key_index(unsigned long long key) {
  return static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

// The k <= N int32 / fp32 values of a block row, all loaded before any is
// used (one memory round trip rather than one per element); entries past k
// read as `fill`.
template <typename T, int N>
__device__ __forceinline__ void load_block_row(const T* row, int k, T fill, T (&out)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = i < k ? row[i] : fill;
}

// Block length by confidence (k <= N positions): the first position whose
// confidence is strictly below th, else k (a NaN confidence never truncates).
template <int N>
__device__ __forceinline__ int truncated_length(const float* conf_row, float th, int k) {
  float c[N];
  load_block_row(conf_row, k, 0.f, c);
  int L = k;
#pragma unroll
  for (int i = N - 1; i >= 0; --i)
    if (i < k && c[i] < th) L = i;
  return L;
}

// acc[i] += v with a device atomic that returns nothing (no round trip waited on)
__device__ __forceinline__ void add_count(int64_t* acc, int v) {
  if (v != 0)
    atomicAdd(reinterpret_cast<unsigned long long*>(acc), static_cast<unsigned long long>(static_cast<int64_t>(v)));
}

// Data-parallel-primitive (DPP) moves inside rows of 16 lanes, 64 bits as two
// 32-bit moves: quad_perm [1,0,3,2] and [2,3,0,1] (lane xor 1, xor 2),
// row_half_mirror (lane i of each 8 <- 7 - i) and row_mirror (lane i of each
// 16 <- 15 - i).  No LDS traffic, unlike a general lane shuffle.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long k) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(static_cast<uint32_t>(k)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(static_cast<uint32_t>(k >> 32)), CTRL, 0xF, 0xF, false));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// max over the 16 lanes of a row group (lanes with equal l >> 4), in every
// lane of the group: quads, then halves, then the row.  Called by whole waves.
__device__ __forceinline__ unsigned long long rowgroup_max16(unsigned long long k) {
  k = umax64(k, dpp_u64<kDppQuadXor1>(k));
  k = umax64(k, dpp_u64<kDppQuadXor2>(k));
  k = umax64(k, dpp_u64<kDppRowHalfMirror>(k));
  k = umax64(k, dpp_u64<kDppRowMirror>(k));
  return k;
}

// max over a whole 64-lane wave, in every lane: the row maxima, then the four
// rows' values read from lanes 0, 16, 32 and 48.  Called by whole waves.
__device__ __forceinline__ unsigned long long wave_max64(unsigned long long k) {
  k = rowgroup_max16(k);
  const uint32_t lo = static_cast<uint32_t>(k);
  const uint32_t hi = static_cast<uint32_t>(k >> 32);
  unsigned long long m = 0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t l = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), 16 * r));
    const uint32_t h = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), 16 * r));
    m = umax64(m, (static_cast<unsigned long long>(h) << 32) | l);
  }
  return m;
}

// ---------------------------------------------------------------------------
// Counter-based random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011).  A round multiplies
// words 0 and 2 by the two round constants, swaps the word pairs and mixes the
// high halves of the products with the other words and the key; the key grows
// by the two Weyl constants between rounds.
// ---------------------------------------------------------------------------
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

// Streams of the sampling path (counter word 3).
constexpr uint32_t kStreamDraft = 0;      // Gumbel noise of the draft draws
constexpr uint32_t kStreamAccept = 1;     // acceptance uniform of (row, position)
constexpr uint32_t kStreamResample = 2;   // Gumbel noise of the residual / bonus draw

__device__ __forceinline__ u32x4_t philox4x32_10(u32x4_t c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(kPhiloxM0, c.x);
    const uint32_t lo0 = kPhiloxM0 * c.x;
    const uint32_t hi1 = __umulhi(kPhiloxM1, c.z);
    const uint32_t lo1 = kPhiloxM1 * c.z;
    c = u32x4_t{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return c;
}

// (2m + 1) * 2^-24 with m the top 23 bits: strictly inside (0, 1), exact in fp32.
__device__ __forceinline__ float bits_to_uniform(uint32_t x) {
  return static_cast<float>(x >> 9) * 0x1p-23f + 0x1p-24f;
}

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Standard Gumbel variate -log(-log(u)) from the hardware base-2 logarithm
// (v_log_f32): -ln u = -log2(u) ln 2, then -ln of that.  The log2 result keeps
// its relative accuracy next to u = 1, where -ln u is small; over every
// uniform of the 23-bit grid the variate is within 1.7e-6 of the exact value.
__device__ __forceinline__ float gumbel_of(float u) {
  const float t = -__builtin_amdgcn_logf(u) * kLn2;
  return -__builtin_amdgcn_logf(t) * kLn2;
}

}  // namespace bdr
