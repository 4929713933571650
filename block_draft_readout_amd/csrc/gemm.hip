// Weight-streaming MFMA GEMM for gfx950: C[M, N] = A[M, K] * W[N, K]^T.
//
// Serves the drafter fc (A = the tapped hidden states, concatenated along K
// segment by segment; W = fc.weight [H, T*H]) and the LM head (A = the block's
// hidden states; W = [V, H]).  Both are dense contractions with few rows
// (M = 4..144) against a large weight read exactly once, so every variant is
// organised around streaming W from HBM:
//   * ws_gemm_stream_kernel (M <= 16): one-wave workgroups, each streaming a
//     balanced range of W rows through LDS with buffer-to-LDS loads while
//     holding A in registers (this file);
//   * ws_gemm_ns_kernel (16 < M <= 160, bf16 or fp8 weights): four-wave
//     workgroups, each wave streaming its own W rows, the A slice staged once
//     per workgroup and K block (gemm_ns.h, instantiated in gemm_ns_*.hip);
//   * gemm_tile_kernel (bf16, M > 160): LDS-tiled MFMA GEMM (gemm_tile.hip);
//   * ws_gemm_kernel: a register-only fallback for the shapes the others do
//     not take (fp32 with M > 16, tap segments not a multiple of 128 elements);
//   * when N alone gives too few workgroups (the fc: N = H), K is split too;
//     partials are summed in a fixed order by splitk_reduce_kernel, so the
//     result is deterministic.
// Loads are raw buffer loads: a lane whose row or K index falls outside an
// operand reads zeros from the hardware range check, so ragged M, N and K need
// no branches.  Inputs are bf16 (v_mfma_f32_16x16x32_bf16) or fp32
// (v_mfma_f32_16x16x4_f32); accumulation is fp32.

#include <atomic>
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "gemm_kernels.h"

namespace bdr {


template <typename S, int MT, int JN, int PF>
__global__ __launch_bounds__(64) void ws_gemm_kernel(const GemmArgs g) {
  constexpr int E = Elem<S>::PER16;
  constexpr int KS = Elem<S>::KSTEP;
  constexpr int ES = static_cast<int>(sizeof(S));
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (16 * JN);
  const int64_t m0 = static_cast<int64_t>(blockIdx.z) * (MT * 16);
  const int64_t total_steps = (g.K + KS - 1) / KS;
  const int64_t s_lo = static_cast<int64_t>(blockIdx.y) * g.steps_per_split;
  const int64_t s_hi = min(total_steps, s_lo + g.steps_per_split);

  // W rows [n0, n0 + 16*JN) as one resource; rows past N read zeros
  const int64_t nrows = min<int64_t>(16 * JN, g.N - n0);
  const rsrc_t rw = make_rsrc(static_cast<const S*>(g.w) + n0 * g.K,
                              static_cast<uint32_t>(nrows * g.K * ES));
  uint32_t offw[JN];
#pragma unroll
  for (int j = 0; j < JN; ++j)
    offw[j] = static_cast<uint32_t>(((16 * j + r16) * g.K + grp * E) * ES);
  // A rows past M lie beyond the segment resource and read zeros
  const uint32_t abytes = static_cast<uint32_t>(g.M * g.seg * ES);
  uint32_t offa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    offa[mt] = static_cast<uint32_t>(((m0 + 16 * mt + r16) * g.seg + grp * E) * ES);

  f32x4_t acc[MT][JN];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < JN; ++j) acc[mt][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // next step to issue, with its A segment and offset inside the segment
  int64_t si = s_lo;
  int ti = static_cast<int>((s_lo * KS) / g.seg);
  int64_t hi = s_lo * KS - static_cast<int64_t>(ti) * g.seg;

  auto issue = [&](u32x4_t(&b)[JN], u32x4_t(&a)[MT]) {
    const int64_t kb = si * KS;
    const bool kok = si < s_hi && kb + grp * E < g.K;
    const uint32_t kw = kok ? static_cast<uint32_t>(kb * ES) : kOOB;
#pragma unroll
    for (int j = 0; j < JN; ++j) b[j] = bload16(rw, offw[j] + kw);
    const rsrc_t ra = make_rsrc(seg_base(g, ti), abytes);
    const uint32_t ka = kok ? static_cast<uint32_t>(hi * ES) : kOOB;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = bload16(ra, offa[mt] + ka);
    ++si;
    hi += KS;
    if (hi >= g.seg) {
      hi -= g.seg;
      ++ti;
    }
  };

  u32x4_t bb[PF][JN];
  u32x4_t aa[PF][MT];
#pragma unroll
  for (int d = 0; d < PF; ++d) issue(bb[d], aa[d]);

  for (int64_t sc = s_lo; sc < s_hi; sc += PF) {
#pragma unroll
    for (int d = 0; d < PF; ++d) {
      if (sc + d < s_hi) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < JN; ++j) acc[mt][j] = mma16(aa[d][mt], bb[d][j], acc[mt][j], S());
        issue(bb[d], aa[d]);
      }
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 16 * mt + 4 * grp + i;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int64_t n = n0 + 16 * j + r16;
        if (n >= g.N) continue;
        const float v = acc[mt][j][i];
        if (g.partial) {
          static_cast<float*>(g.out)[(static_cast<int64_t>(blockIdx.y) * g.M + m) * g.N + n] = v;
        } else if (g.out_kind == OUT_BF16) {
          static_cast<uint16_t*>(g.out)[m * g.N + n] = f32_to_bf16(v);
        } else {
          static_cast<float*>(g.out)[m * g.N + n] = v;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Streaming variant for M <= 16 (one 16-row tile of A).
//
// Each one-wave workgroup owns a balanced contiguous range of W rows and a
// range of K blocks of KBB bytes per row.  The loop runs K blocks outside and
// 16-row tiles of its range inside ("visits"); every visit copies 16 rows x
// KBB contiguous bytes of W straight into LDS with buffer-to-LDS loads (one
// row per instruction, 1 KB contiguous, non-temporal), double-buffered, and
// the MFMAs read it back in operand layout from padded rows (no bank
// conflicts).  The accumulators of every tile of the range live in registers,
// and the A slice of a K block is loaded once into registers and reused by all
// tiles of the range, so A costs ~M/(16*tiles) of the W traffic.  The loads to
// LDS are not tracked by the compiler's wait insertion, so the waits on them
// are explicit: the only memory operations issued after a visit's loads are
// the next visit's 16, hence "vmcnt <= 16" before reading a visit.
// ----------------------------------------------------------------------------
constexpr int kKBB = 1024;            // bytes of each W row per visit
// LDS row stride: 1056 bytes put the 32 lanes of one 16-byte read phase (rows
// r16, chunks grp and grp + 1) on 32 disjoint groups of 4 of the 128 banks; a
// 1040-byte stride measured ~4 conflict cycles per LDS read
constexpr int kPadRow = kKBB + 32;
constexpr int kStreamTiles = 16;      // max 16-row tiles per workgroup
constexpr int kStreamTilesFp8 = 12;   // the same for fp8 weights (register budget)



// NT: 16-row tiles per workgroup (compile time; the last ones may be empty)
template <typename S, int NT>
__global__ __launch_bounds__(64) void ws_gemm_stream_kernel(const StreamArgs sa) {
  constexpr int STEPS = kKBB / 64;      // 16-byte-per-lane MFMA operand steps per visit
  constexpr int ES = static_cast<int>(sizeof(S));
  const GemmArgs& g = sa.g;
  __shared__ __attribute__((aligned(16))) char lds[2][16 * kPadRow];
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const int64_t n_lo = static_cast<int64_t>(blockIdx.x) * g.N / sa.n_waves;
  const int64_t n_hi = static_cast<int64_t>(blockIdx.x + 1) * g.N / sa.n_waves;
  const int ntiles = static_cast<int>((n_hi - n_lo + 15) / 16);
  const uint32_t kb_lo = static_cast<uint32_t>(blockIdx.y * sa.kb_per_split);
  const uint32_t kb_hi = static_cast<uint32_t>(min<int64_t>(sa.kblocks, kb_lo + sa.kb_per_split));
  if (ntiles <= 0 || kb_lo >= kb_hi) return;
  const OutRef out(g, blockIdx.y);
  const uint32_t kbytes = static_cast<uint32_t>(g.K * ES);
  const uint32_t segbytes = static_cast<uint32_t>(g.seg * ES);

  const rsrc_t rw = make_rsrc(static_cast<const S*>(g.w) + n_lo * g.K,
                              static_cast<uint32_t>(n_hi - n_lo) * kbytes);
  const uint32_t abytes = static_cast<uint32_t>(g.M) * segbytes;
  const uint32_t lane16 = static_cast<uint32_t>(lane) * 16;
  const uint32_t a_lane = static_cast<uint32_t>(r16) * segbytes + static_cast<uint32_t>(grp) * 16;
  const uint32_t lds_rd = static_cast<uint32_t>(r16 * kPadRow + grp * 16);

  f32x4_t acc[NT];
  static_for<NT>([&](auto t) { acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f}; });
  u32x4_t a0[STEPS], a1[STEPS];

  // 16 rows of tile t, K block kb -> LDS buffer b (rows past the range and
  // bytes past a row read zeros)
  auto dma = [&](uint32_t kb, int t, int b) {
    const uint32_t k0 = kb * kKBB;
    const uint32_t lo = k0 + lane16 < kbytes ? lane16 : kOOB;
    const uint32_t base = static_cast<uint32_t>(16 * t) * kbytes + k0;
    char* dst = &lds[b][0];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(dst + r * kPadRow), 16,
          lo + base + static_cast<uint32_t>(r) * kbytes, 0, 0, 2);
  };
  // A slice of K block kb in operand layout (rows >= M read zeros); blocks
  // never straddle A segments
  auto load_a = [&](uint32_t kb, u32x4_t(&a)[STEPS]) {
    const uint32_t k0 = kb * kKBB;
    const uint32_t ts = k0 / segbytes;
    const rsrc_t ra = make_rsrc(seg_base(g, static_cast<int>(ts)), abytes);
    const uint32_t off = a_lane + (k0 - ts * segbytes);
    static_for<STEPS>([&](auto st) { a[st] = bload16(ra, off + st * 64); });
  };
  auto compute = [&](auto t, int b, const u32x4_t(&a)[STEPS], int nsteps) {
    const char* src = &lds[b][0] + lds_rd;
    if (nsteps == STEPS) {
      static_for<STEPS>([&](auto st) {
        const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(src + st * 64);
        acc[t] = mma16(a[st], bv, acc[t], S());
      });
    } else {
      static_for<STEPS>([&](auto st) {
        if (st < nsteps) {
          const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(src + st * 64);
          acc[t] = mma16(a[st], bv, acc[t], S());
        }
      });
    }
  };

  int buf = 0;
  // one K block: visit every tile; prefetch the next visit (and the next
  // block's A slice) before waiting on the current one
  auto block = [&](uint32_t kb, const u32x4_t(&acur)[STEPS], u32x4_t(&anext)[STEPS]) {
    const int nsteps = static_cast<int>(min<uint32_t>(STEPS, (kbytes - kb * kKBB) / 64));
    static_for<NT>([&](auto t) {
      if (t < ntiles) {
        if (t + 1 < ntiles) {
          dma(kb, t + 1, buf ^ 1);
          BDR_WAIT_VM(16);
        } else if (kb + 1 < kb_hi) {
          load_a(kb + 1, anext);
          dma(kb + 1, 0, buf ^ 1);
          BDR_WAIT_VM(16);
        } else {
          BDR_WAIT_VM(0);
        }
        compute(t, buf, acur, nsteps);
        buf ^= 1;
      }
    });
  };

  load_a(kb_lo, a0);
  dma(kb_lo, 0, 0);
  for (uint32_t kb = kb_lo; kb < kb_hi; kb += 2) {
    block(kb, a0, a1);
    if (kb + 1 < kb_hi) block(kb + 1, a1, a0);
  }

  static_for<NT>([&](auto t) {
    const int64_t n = n_lo + 16 * t + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = 4 * grp + i;
      if (t < ntiles && m < out.M && n < n_hi) out.put(m, n, acc[t][i]);
    }
  });

}


// out[i] = sum_p part[p][i] in order p = 0, 1, ...; one output per thread (the
// partials are a few MB at most: a wide grid keeps enough loads in flight),
// the loads of up to 16 splits issued before their ordered sums.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int ksplit, int64_t mn, void* out,
                                                            int out_kind) {
  constexpr int PMAX = 16;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= mn) return;
  float sum = 0.f;
  for (int p0 = 0; p0 < ksplit; p0 += PMAX) {
    float v[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) v[p] = p0 + p < ksplit ? part[(p0 + p) * mn + i] : 0.f;
#pragma unroll
    for (int p = 0; p < PMAX; ++p)
      if (p0 + p < ksplit) sum += v[p];
  }
  if (out_kind == OUT_BF16)
    static_cast<uint16_t*>(out)[i] = f32_to_bf16(sum);
  else
    static_cast<float*>(out)[i] = sum;
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

// Column tiles per wave and prefetch depth by the number of 16-row tiles of A.
static int pick_jn(int mt) { return mt <= 2 ? 4 : 2; }

// Streaming plan: balanced row ranges (at most kStreamTiles tiles each) and a
// K split chosen to minimise per-wave cost = W bytes + a quarter of the A bytes
// it re-reads from L2 (+ the partial-sum round trip and a second launch).
// fp8 weights (esize 1): visits of 1 KB of codes, A segments in multiples of 64
// elements (the fp8 kernel loads A step by step from the segment of each step).
static bool plan_stream(int64_t M, int64_t N, int64_t K, int esize, bool allow_split, int n_seg,
                        GemmPlan* p) {
  const int64_t kbytes = K * esize;
  const int64_t segbytes = kbytes / n_seg;
  if (M > 16 || kbytes % 64 != 0) return false;
  if (n_seg > 1 && segbytes % (esize == 1 ? 64 : kKBB) != 0) return false;
  const int64_t max_tiles = esize == 1 ? kStreamTilesFp8 : kStreamTiles;
  // bf16 split-K plans (the fc) use two one-wave workgroups per compute unit
  // rather than four: alone the fc barely slows (48 -> 49 us on the 27B shape),
  // and it leaves LDS for the Markov chain that runs beside it on another
  // stream (block-step 308.5 -> 303.3 us).  One per CU made the fc itself too
  // slow, and the fp8 fc (half the K blocks) loses more than the chain gains.
  const int64_t waves = (allow_split && esize == 2 ? 2 : 4) * static_cast<int64_t>(kNumCU);
  const int64_t kblocks = (kbytes + kKBB - 1) / kKBB;
  double best = 1e300;
  for (int64_t ks = 1; ks <= (allow_split ? std::min<int64_t>(64, kblocks) : 1); ++ks) {
    int64_t nw = std::max<int64_t>(1, waves / ks);
    nw = std::max<int64_t>(nw, (N + 16 * max_tiles - 1) / (16 * max_tiles));
    nw = std::min<int64_t>(nw, N);
    const int64_t kbps = (kblocks + ks - 1) / ks;
    const int64_t ks_eff = (kblocks + kbps - 1) / kbps;
    const int64_t rows = (N + nw - 1) / nw;
    const int64_t rounds = (nw * ks_eff + waves - 1) / waves;
    double cost = static_cast<double>(rounds) * kbps * kKBB * (rows + 0.25 * M);
    if (ks_eff > 1) cost += 34e3 + static_cast<double>(ks_eff) * M * N * 8 / waves;
    if (cost < best) {
      best = cost;
      p->n_waves = nw;
      p->kb_per_split = kbps;
      p->ksplit = static_cast<int>(ks_eff);
    }
  }
  p->stream = true;
  p->kblocks = kblocks;
  p->mt = 1;
  p->m_groups = 1;
  p->n_wg = p->n_waves;
  p->workspace = p->ksplit > 1 ? align256(static_cast<size_t>(p->ksplit) * M * N * 4) : 0;
  return true;
}

// Row-split workgroup plan (gemm_ns.h; bf16 or fp8 weights, bf16 A, 16 < M <=
// 160): K blocks of 128 elements that never straddle a tap segment; one
// workgroup per compute unit and K split, its rows split over four waves, each
// walking its tiles in passes.  The K split minimises the per-compute-unit
// cost W bytes + a quarter of the A bytes staged per pass (+ the partial-sum
// round trip).
//
// Passes are groups of `ring` slots (gemm_ns.h, ns_lean_body): with t
// tiles a wave walks npass passes of ng groups; the ring depth is the one of
// kNsLeanRings that leaves the fewest slots (empty ones still cost their
// MFMAs and issue), the deepest among equals.
// reg: the register ring (packed weights), whose passes hold one group of
// `ring` tiles
static int64_t ns_lean_passes(int mt, int ring, int64_t tiles, bool reg = false) {
  const int64_t ntw = reg ? ring : kNsLeanNtwMax[mt] / ring * ring;
  return std::max<int64_t>(1, (tiles + ntw - 1) / ntw);
}

static int64_t ns_lean_slots(int mt, int ring, int64_t tiles, bool reg = false) {
  const int64_t npass = ns_lean_passes(mt, ring, tiles, reg);
  const int64_t ng = reg ? 1 : std::max<int64_t>(1, (tiles + npass * ring - 1) / (npass * ring));
  return npass * ng * ring;
}

// pass `rings` to restrict the choice (the two-problem launch builds fewer)
static int ns_pick_ring(int mt, int64_t tiles, const int* rings = nullptr, bool reg = false) {
  if (rings == nullptr) rings = kNsLeanRings[mt];
  int best = 0;
  int64_t best_slots = 0;
  for (int i = 0; i < 3; ++i) {
    const int r = rings[i];
    if (r == 0) continue;
    const int64_t s = ns_lean_slots(mt, r, tiles, reg);
    if (best == 0 || s < best_slots) {
      best = r;
      best_slots = s;
    }
  }
  return best;
}

// largest tile count of one wave when N rows are split over nwg workgroups
static int64_t ns_wave_tiles(int64_t N, int64_t nwg) {
  const int64_t n_t = (N + 15) / 16;
  return ((n_t + nwg - 1) / nwg + 3) / 4;
}

// passes of a wave with the ring it would take (kNsLeanRings)
static int64_t ns_passes(int mt, int64_t tiles, int* ring, bool reg = false) {
  const int r = ns_pick_ring(mt, tiles, nullptr, reg);
  if (ring) *ring = r;
  return ns_lean_passes(mt, r, tiles, reg);
}

static std::atomic<int> g_ns_ring{0};
static std::atomic<int64_t> g_ns_wg{0};
static std::atomic<int> g_ns_ks{0};

void set_row_split_override(int ring, int64_t workgroups, int ksplit) {
  g_ns_ring.store(std::max(ring, 0));
  g_ns_wg.store(std::max<int64_t>(workgroups, 0));
  g_ns_ks.store(std::max(ksplit, 0));
}

static bool ns_overridden() {
  return g_ns_ring.load() != 0 || g_ns_wg.load() != 0 || g_ns_ks.load() != 0;
}

// packed: bf16 weights in the packed layout, any M in 1..160 (at least two A
// row tiles; rows past M read as zero), by the register ring from
// kNsRegMinMt row tiles on.  The row ranges and K splits are chosen as for the
// row-major layout (so the two give the same sums bit for bit); only the ring
// depth follows the register ring.
static bool plan_ns(int64_t M, int64_t N, int64_t K, int esize, bool allow_split, int n_seg,
                    GemmPlan* p, bool packed = false) {
  constexpr int KE = 128;
  const int64_t mtiles = packed ? std::max<int64_t>(2, (M + 15) / 16) : (M + 15) / 16;
  if (esize > 2 || (M <= 16 && !packed) || M < 1 || mtiles > 10 ||
      K % (esize == 1 ? 16 : 8) != 0)
    return false;
  if (packed && (esize != 2 || packed_weight_bytes(N, K) == 0)) return false;
  if (n_seg > 1 && (K / n_seg) % KE != 0) return false;
  const int64_t kblocks = (K + KE - 1) / KE;
  double best = 1e300;
  for (int64_t ks = 1; ks <= (allow_split ? std::min<int64_t>(64, kblocks) : 1); ++ks) {
    const int64_t kbps = (kblocks + ks - 1) / ks;
    const int64_t ks_eff = (kblocks + kbps - 1) / kbps;
    if (ks_eff > kNumCU) continue;
    int64_t nwg = std::max<int64_t>(1, kNumCU / ks_eff);
    nwg = std::min<int64_t>(nwg, (N + 63) / 64);
    const int64_t rows = (N + nwg - 1) / nwg;
    const int64_t npass = ns_passes(static_cast<int>(mtiles), ns_wave_tiles(N, nwg), nullptr);
    double cost = static_cast<double>(kbps) * KE * (esize * rows + 0.5 * M * npass);
    if (ks_eff > 1) cost += 34e3 + static_cast<double>(ks_eff) * M * N * 8 / kNumCU;
    if (cost < best) {
      best = cost;
      p->n_waves = nwg;
      p->kb_per_split = kbps;
      p->ksplit = static_cast<int>(ks_eff);
    }
  }
  if (const int64_t ks_o = std::min<int64_t>(g_ns_ks.load(), kblocks); ks_o > 0 && allow_split) {
    p->kb_per_split = (kblocks + ks_o - 1) / ks_o;
    p->ksplit = static_cast<int>((kblocks + p->kb_per_split - 1) / p->kb_per_split);
  }
  if (const int64_t wg_o = g_ns_wg.load(); wg_o > 0)
    p->n_waves = std::min<int64_t>(wg_o, (N + 15) / 16);
  // the output (or one K split's partials) is addressed with 32-bit offsets
  if (M * N * 4 >= (int64_t(1) << 32)) return false;
  // a wave's rows x row bytes are addressed with 32-bit offsets (with room for
  // the empty slots of its last pass); packed weights: the whole copy is under
  // 2^31 bytes
  const int64_t rows_w = ((N + p->n_waves - 1) / p->n_waves + 3) / 4;
  if (!packed && (rows_w + 256) * K * esize >= (int64_t(1) << 31)) return false;
  p->stream = true;
  p->ns = true;
  p->mt = static_cast<int>(mtiles);
  // (fp8 codes: only K-split plans, the fc: straight operand loads of row-major
  // codes slowed the fp8 LM head 205 -> 237 us, while the fc, bound by its
  // widening and MFMAs rather than its stream, fits beside the chain with them)
  p->reg = p->mt >= kNsRegMinMt && (packed || (esize == 1 && p->ksplit > 1));
  ns_passes(p->mt, ns_wave_tiles(N, p->n_waves), &p->ring, p->reg);
  if (g_ns_ring.load() > 0) p->ring = g_ns_ring.load();   // (the launch checks it is built)
  p->kblocks = kblocks;
  p->m_groups = 1;
  p->n_wg = p->n_waves;
  p->workspace = p->ksplit > 1 ? align256(static_cast<size_t>(p->ksplit) * M * N * 4) : 0;
  return true;
}

// Pair plan: the compute units are shared in proportion to each problem's
// cost (weight bytes + a quarter of the A bytes staged per pass + split-K
// partials), the split of problem 1 chosen so that its slowest workgroup and
// problem 0's finish together.  Problem 1 (the fc: two or three tiles a wave)
// takes ring 3.
static double ns_wg_cost(int64_t M, int64_t rows, int64_t kbps, int64_t npass, int64_t ks,
                         int64_t N) {
  double c = static_cast<double>(kbps) * 128 * (2.0 * rows + 0.5 * M * npass);
  if (ks > 1) c += static_cast<double>(ks) * M * N * 8 / kNumCU;
  return c;
}

// rings of problem 0 built for the two-problem launch (gemm_ns_pair_*.hip;
// seven row tiles with ring 3 spills beside the fc and is left out)
static constexpr int kPairRings[11][3] = {{0, 0, 0}, {0, 0, 0}, {8, 5, 3}, {7, 5, 3}, {6, 5, 3},
                                          {6, 5, 3}, {6, 5, 3}, {5, 0, 0}, {5, 3, 0}, {4, 3, 0},
                                          {0, 0, 0}};

PairPlan plan_gemm_pair(int64_t M0, int64_t N0, int64_t K0, int64_t M1, int64_t N1, int64_t K1,
                        int n_seg1, bool packed) {
  PairPlan pp;
  GemmPlan q0, q1;
  if (ns_overridden()) return pp;
  if (!plan_ns(M0, N0, K0, 2, false, 1, &q0) || !plan_ns(M1, N1, K1, 2, true, n_seg1, &q1))
    return pp;
  if ((q1.mt != q0.mt && q1.mt != q0.mt + 1) || q1.mt > 9) return pp;
  const int64_t kb0 = q0.kblocks, kb1 = q1.kblocks;
  // passes of problem 0's waves on its own (one workgroup per compute unit):
  // sharing the chip must not add a pass (each restages the whole A matrix)
  auto passes0 = [&](int64_t nwg) {
    const int64_t t = ns_wave_tiles(N0, nwg);
    return ns_lean_passes(q0.mt, ns_pick_ring(q0.mt, t, kPairRings[q0.mt]), t);
  };
  auto passes1 = [&](int64_t nwg) { return ns_lean_passes(q1.mt, 3, ns_wave_tiles(N1, nwg)); };
  const int64_t alone = passes0(q0.n_waves);
  double best = 1e300, best_c0 = 0, best_c1 = 0;
  for (int64_t ks = 1; ks <= std::min<int64_t>(8, kb1); ++ks) {
    const int64_t kbps = (kb1 + ks - 1) / ks;
    const int64_t ks_eff = (kb1 + kbps - 1) / kbps;
    for (int64_t nx = 1; nx * ks_eff <= kNumCU / 2 && nx <= (N1 + 63) / 64; ++nx) {
      const int64_t n1 = nx * ks_eff, n0 = kNumCU - n1;
      if (n0 > (N0 + 63) / 64 || passes0(n0) > alone) continue;
      const double c0 = ns_wg_cost(M0, (N0 + n0 - 1) / n0, kb0, passes0(n0), 1, N0);
      const double c1 = ns_wg_cost(M1, (N1 + nx - 1) / nx, kbps, passes1(nx), ks_eff, N1);
      const double c = std::max(c0, c1);
      if (c < best) {
        best = c;
        best_c0 = c0;
        best_c1 = c1;
        pp.n0 = static_cast<unsigned>(n0);
        pp.n1 = static_cast<unsigned>(n1);
        q1.n_waves = nx;
        q1.ksplit = static_cast<int>(ks_eff);
        q1.kb_per_split = kbps;
      }
    }
  }
  if (pp.n0 == 0) return pp;
  // one launch only when problem 1's workgroups finish with problem 0's: when
  // the pass rule leaves too few compute units for problem 1, two launches one
  // after the other are faster
  if (best_c1 > 1.15 * best_c0) {
    pp.n0 = pp.n1 = 0;
    return pp;
  }
  q0.n_waves = pp.n0;
  q0.ksplit = 1;
  q0.kb_per_split = kb0;
  q0.workspace = 0;
  // (the register ring, packed weights from kNsRegMinMt row tiles on, is
  // built for every ring of kNsLeanRings; the fc beside it takes it too)
  const bool reg = packed && q0.mt >= kNsRegMinMt;
  q0.ring = ns_pick_ring(q0.mt, ns_wave_tiles(N0, pp.n0),
                         reg ? kNsLeanRings[q0.mt] : kPairRings[q0.mt], reg);
  q1.ring = 3;
  q0.reg = q1.reg = reg;
  q1.workspace = q1.ksplit > 1 ? align256(static_cast<size_t>(q1.ksplit) * M1 * N1 * 4) : 0;
  // the row ranges must keep their 32-bit offsets with the fewer workgroups
  const int64_t rows_w0 = ((N0 + pp.n0 - 1) / pp.n0 + 3) / 4;
  const int64_t rows_w1 = ((N1 + q1.n_waves - 1) / q1.n_waves + 3) / 4;
  if ((rows_w0 + 256) * K0 * 2 >= (int64_t(1) << 31) || (rows_w1 + 256) * K1 * 2 >= (int64_t(1) << 31))
    return pp;
  pp.p0 = q0;
  pp.p1 = q1;
  pp.workspace = q1.workspace;
  pp.M0 = M0, pp.N0 = N0, pp.K0 = K0, pp.M1 = M1, pp.N1 = N1, pp.K1 = K1;
  pp.ok = true;
  return pp;
}

// bounds keeping the tiled variant's tile count and indices in 32 bits
constexpr int64_t kMaxTileRows = int64_t(1) << 22;
constexpr int64_t kMaxTileCols = int64_t(1) << 22;

// Tiled variant (gemm_tile.hip) for bf16 with more rows than the streaming
// kernels take: 256 x 160 or 256 x 320 tiles, K steps of 64 that never
// straddle a segment, output columns in whole groups of four.  Split K only
// when the tiles alone leave compute units idle, each split keeping >= 16
// steps.
static bool plan_tile(int64_t M, int64_t N, int64_t K, int esize, bool allow_split, int n_seg,
                      GemmPlan* out) {
  const int64_t seg = K / std::max(n_seg, 1);
  if (esize != 2 || M <= 160 || seg % 64 != 0 || N % 4 != 0) return false;
  if (N > kMaxTileCols || M > kMaxTileRows) return false;
  // Shape 1 (256 x 320, eight waves) reached ~0.49 of the MFMA peak on the
  // 4096-row fc, shape 0 (256 x 160, four waves) ~0.35; pick the shape (and a
  // K split that fills the compute units) with the lower estimated time,
  // counting rounds of workgroups and the fp32 partials' round trip.
  const double eff[2] = {0.35, 0.49};
  const double cu_flops = 2.5e15 / kNumCU;
  const double bw = 5e12;
  const int64_t kblocks = K / 64;
  const int64_t tiles_m = (M + 255) / 256;
  double best = 1e30;
  GemmPlan p;
  for (int shape = 0; shape < 2; ++shape) {
    const int64_t cols = tile_cols(shape);
    const int64_t tiles = tiles_m * ((N + cols - 1) / cols);
    int64_t split = 1;
    if (allow_split && tiles < kNumCU)
      split = std::max<int64_t>(1, std::min<int64_t>({kNumCU / tiles, kblocks / 16, 16}));
    const int64_t kps = (kblocks + split - 1) / split;
    split = (kblocks + kps - 1) / kps;
    const double rounds = std::ceil(static_cast<double>(tiles * split) / kNumCU);
    double t = rounds * 2.0 * 256 * cols * 64.0 * kps / (eff[shape] * cu_flops);
    if (split > 1) t += (static_cast<double>(split) * M * N * 8 + static_cast<double>(M) * N * 2) / bw;
    if (t < best) {
      best = t;
      p = GemmPlan{};
      p.tile = true;
      p.tile_shape = shape;
      p.tiles_m = static_cast<int>(tiles_m);
      p.tiles_n = static_cast<int>((N + cols - 1) / cols);
      p.kblocks = kblocks;
      p.kb_per_split = kps;
      p.ksplit = static_cast<int>(split);
      p.workspace = split > 1 ? align256(static_cast<size_t>(split) * M * N * 4) : 0;
    }
  }
  *out = p;
  return true;
}

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bdr_dtype dt, bool allow_split, int n_seg) {
  GemmPlan p;
  if (dt == BDR_BF16_PACKED) {
    // the row-split kernel over slabs of at most kPackedSlabRows rows, each
    // planned as the largest (the last may be shorter); p.ns stays false when
    // the shape does not fit it
    const int64_t slab = std::min<int64_t>(M, kPackedSlabRows);
    plan_ns(slab, N, K, 2, allow_split, n_seg, &p, true);
    p.packed = true;
    p.slab = M > slab ? slab : 0;
    return p;
  }
  const int ks = dt == BDR_BF16 ? Elem<uint16_t>::KSTEP : Elem<float>::KSTEP;
  const int esize = dt == BDR_BF16 ? 2 : 4;
  if (plan_stream(M, N, K, esize, allow_split, n_seg, &p)) return p;
  {
    GemmPlan q;
    if (plan_ns(M, N, K, esize, allow_split, n_seg, &q)) return q;
    if (plan_tile(M, N, K, esize, allow_split, n_seg, &q)) return q;
  }
  const int64_t mtiles = std::max<int64_t>(1, (M + 15) / 16);
  if (mtiles <= 9) {
    p.mt = static_cast<int>(mtiles);
    p.m_groups = 1;
  } else {
    p.mt = 8;
    p.m_groups = static_cast<int>((mtiles + 7) / 8);
  }
  p.jn = pick_jn(p.mt);
  const int64_t cols = 16 * p.jn;
  p.n_wg = (N + cols - 1) / cols;
  const int64_t steps = (K + ks - 1) / ks;
  int64_t split = 1;
  if (allow_split) {
    // about ten resident waves per compute unit
    const int64_t target_wgs = 2560;
    const int64_t base = p.n_wg * p.m_groups;
    split = (target_wgs + base - 1) / base;
    split = std::min<int64_t>(split, std::max<int64_t>(1, steps / 16));
    // keep partial-sum traffic (write + read, fp32) under ~8% of the weight bytes
    const int64_t cap = std::max<int64_t>(
        1, static_cast<int64_t>(0.08 * static_cast<double>(K) * esize / (8.0 * std::max<int64_t>(M, 1))));
    split = std::max<int64_t>(1, std::min<int64_t>({split, cap, 64}));
  }
  p.steps_per_split = (steps + split - 1) / split;
  p.ksplit = static_cast<int>((steps + p.steps_per_split - 1) / p.steps_per_split);
  p.workspace = p.ksplit > 1 ? align256(static_cast<size_t>(p.ksplit) * M * N * 4) : 0;
  return p;
}

// fp8 plans cover one slab of at most 16 rows; launch_gemm_fp8 runs the
// slabs of a taller A one after another on the stream (sharing the workspace).
GemmPlan plan_gemm_fp8(int64_t M, int64_t N, int64_t K, bool allow_split, int n_seg) {
  GemmPlan p;
  if (M > 16) {
    GemmPlan q;
    if (plan_ns(M, N, K, 1, allow_split, n_seg, &q)) return q;
  }
  if (!plan_stream(std::min<int64_t>(M, 16), N, K, 1, allow_split, n_seg, &p)) p.stream = false;
  return p;
}

template <typename S, int MT>
static void launch_mt(const GemmPlan& p, const GemmArgs& g, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.n_wg), static_cast<unsigned>(p.ksplit),
                  static_cast<unsigned>(p.m_groups));
  // tile shapes per MT as chosen by pick_jn()
  if constexpr (MT <= 2)
    hipLaunchKernelGGL((ws_gemm_kernel<S, MT, 4, 4>), grid, dim3(64), 0, st, g);
  else if constexpr (MT <= 4)
    hipLaunchKernelGGL((ws_gemm_kernel<S, MT, 2, 4>), grid, dim3(64), 0, st, g);
  else
    hipLaunchKernelGGL((ws_gemm_kernel<S, MT, 2, 2>), grid, dim3(64), 0, st, g);
}

template <typename S>
static void launch_typed(const GemmPlan& p, const GemmArgs& g, hipStream_t st) {
  switch (p.mt) {
    case 1: launch_mt<S, 1>(p, g, st); break;
    case 2: launch_mt<S, 2>(p, g, st); break;
    case 3: launch_mt<S, 3>(p, g, st); break;
    case 4: launch_mt<S, 4>(p, g, st); break;
    case 5: launch_mt<S, 5>(p, g, st); break;
    case 6: launch_mt<S, 6>(p, g, st); break;
    case 7: launch_mt<S, 7>(p, g, st); break;
    case 8: launch_mt<S, 8>(p, g, st); break;
    default: launch_mt<S, 9>(p, g, st); break;
  }
}

template <typename S>
static void launch_stream(const GemmPlan& p, const GemmArgs& g, hipStream_t st) {
  const StreamArgs sa{g, p.n_waves, p.kblocks, p.kb_per_split};
  const dim3 grid(static_cast<unsigned>(p.n_waves), static_cast<unsigned>(p.ksplit));
  const int64_t tiles = ((g.N + p.n_waves - 1) / p.n_waves + 15) / 16;
  if (tiles <= 1) hipLaunchKernelGGL((ws_gemm_stream_kernel<S, 1>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 2) hipLaunchKernelGGL((ws_gemm_stream_kernel<S, 2>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 4) hipLaunchKernelGGL((ws_gemm_stream_kernel<S, 4>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 8) hipLaunchKernelGGL((ws_gemm_stream_kernel<S, 8>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 10) hipLaunchKernelGGL((ws_gemm_stream_kernel<S, 10>), grid, dim3(64), 0, st, sa);
  else if (tiles <= 12) hipLaunchKernelGGL((ws_gemm_stream_kernel<S, 12>), grid, dim3(64), 0, st, sa);
  else hipLaunchKernelGGL((ws_gemm_stream_kernel<S, 16>), grid, dim3(64), 0, st, sa);
}

// out = ordered sum of the ksplit fp32 partials in the workspace
static hipError_t launch_splitk_reduce(const GemmPlan& p, int64_t M, int64_t N, void* out,
                                       OutKind out_kind, void* workspace, hipStream_t stream) {
  const int64_t mn = M * N;
  const int64_t blocks = (mn + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const float*>(workspace), p.ksplit, mn, out,
                     static_cast<int>(out_kind));
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan& p, bdr_dtype dt, const void* const* a, int n_seg,
                       int64_t seg, int64_t M, int64_t N, const void* w, void* out,
                       OutKind out_kind, void* workspace, hipStream_t stream) {
  GemmArgs g{};
  for (int t = 0; t < n_seg; ++t) g.a[t] = a[t];
  g.seg = seg;
  g.M = M;
  g.N = N;
  g.K = seg * n_seg;
  g.w = w;
  g.out_kind = out_kind;
  g.steps_per_split = p.steps_per_split;
  const bool split = p.ksplit > 1;
  g.partial = split ? 1 : 0;
  g.out = split ? workspace : out;
  if (p.packed) {
    // slab by slab (sharing the workspace, in stream order)
    if (!p.ns) return hipErrorInvalidValue;
    g.w_packed = 1;
    const int64_t slab = p.slab > 0 ? p.slab : M;
    const int64_t out_es = out_kind == OUT_BF16 ? 2 : 4;
    for (int64_t m0 = 0; m0 < M; m0 += slab) {
      GemmArgs gs = g;
      gs.M = std::min<int64_t>(slab, M - m0);
      for (int t = 0; t < n_seg; ++t) gs.a[t] = static_cast<const char*>(a[t]) + m0 * seg * 2;
      void* o = static_cast<char*>(out) + m0 * N * out_es;
      gs.out = split ? workspace : o;
      const StreamArgs sa{gs, p.n_waves, p.kblocks, p.kb_per_split};
      hipError_t e = p.reg ? launch_ns_bf16_packed(p, sa, stream) : launch_ns_bf16(p, sa, stream);
      if (e == hipSuccess) e = hipGetLastError();
      if (e == hipSuccess && split) e = launch_splitk_reduce(p, gs.M, N, o, out_kind, workspace, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (p.tile) {
    const hipError_t le = launch_gemm_tile(p, g, stream);
    if (le != hipSuccess) return le;
  } else if (p.ns) {
    const StreamArgs sa{g, p.n_waves, p.kblocks, p.kb_per_split};
    const hipError_t le = launch_ns_bf16(p, sa, stream);
    if (le != hipSuccess) return le;
  } else if (p.stream) {
    if (dt == BDR_BF16)
      launch_stream<uint16_t>(p, g, stream);
    else
      launch_stream<float>(p, g, stream);
  } else if (dt == BDR_BF16) {
    launch_typed<uint16_t>(p, g, stream);
  } else {
    launch_typed<float>(p, g, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  return launch_splitk_reduce(p, M, N, out, out_kind, workspace, stream);
}

hipError_t launch_gemm_pair(const PairPlan& pp, const void* a0, const void* w0, float* out0,
                            const void* const* a1, int n_seg1, int64_t seg1, const void* w1,
                            void* out1, void* workspace, bool packed, hipStream_t stream) {
  if (!pp.ok) return hipErrorInvalidValue;
  GemmArgs g0{};
  g0.a[0] = a0;
  g0.seg = pp.K0;
  g0.M = pp.M0;
  g0.N = pp.N0;
  g0.K = pp.K0;
  g0.w = w0;
  g0.out = out0;
  g0.out_kind = OUT_F32;
  g0.partial = 0;
  g0.w_packed = packed ? 1 : 0;
  GemmArgs g1{};
  for (int t = 0; t < n_seg1; ++t) g1.a[t] = a1[t];
  g1.seg = seg1;
  g1.M = pp.M1;
  g1.N = pp.N1;
  g1.K = pp.K1;
  g1.w = w1;
  g1.w_packed = packed ? 1 : 0;
  g1.out_kind = OUT_BF16;
  const bool split = pp.p1.ksplit > 1;
  g1.partial = split ? 1 : 0;
  g1.out = split ? workspace : out1;
  const StreamArgs s0{g0, pp.p0.n_waves, pp.p0.kblocks, pp.p0.kb_per_split};
  const StreamArgs s1{g1, pp.p1.n_waves, pp.p1.kblocks, pp.p1.kb_per_split};
  const int m0 = pp.p0.mt, r0 = pp.p0.ring, m1 = pp.p1.mt;
  const unsigned n0 = pp.n0, n1 = pp.n1;
  hipError_t e = pp.p0.reg ? launch_ns_pair_bf16_packed(m0, r0, m1, s0, s1, n0, n1, stream)
                 : m0 <= 4 ? launch_ns_pair_bf16_a(m0, r0, m1, s0, s1, n0, n1, stream)
                           : launch_ns_pair_bf16_b(m0, r0, m1, s0, s1, n0, n1, stream);
  if (e != hipSuccess || !split) return e;
  return launch_splitk_reduce(pp.p1, pp.M1, pp.N1, out1, OUT_BF16, workspace, stream);
}

hipError_t launch_gemm_fp8(const GemmPlan& p, const void* const* a, int n_seg, int64_t seg,
                           int64_t M, int64_t N, const uint8_t* w_q, const float* w_scale,
                           void* out, OutKind out_kind, void* workspace, hipStream_t stream) {
  if (!p.stream) return hipErrorInvalidValue;
  if (p.ns) {     // all rows in one launch of the row-split kernel
    GemmArgs g{};
    for (int t = 0; t < n_seg; ++t) g.a[t] = a[t];
    g.seg = seg;
    g.M = M;
    g.N = N;
    g.K = seg * n_seg;
    g.w = w_q;
    g.w_scale = w_scale;
    g.out_kind = out_kind;
    const bool split = p.ksplit > 1;
    g.partial = split ? 1 : 0;
    g.out = split ? workspace : out;
    const StreamArgs sa{g, p.n_waves, p.kblocks, p.kb_per_split};
    hipError_t e = launch_ns_fp8(p, sa, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess && split) e = launch_splitk_reduce(p, M, N, out, out_kind, workspace, stream);
    return e;
  }
  const int64_t out_es = out_kind == OUT_BF16 ? 2 : 4;
  for (int64_t m0 = 0; m0 < M; m0 += 16) {
    const int64_t ms = std::min<int64_t>(16, M - m0);
    GemmArgs g{};
    for (int t = 0; t < n_seg; ++t) g.a[t] = static_cast<const uint16_t*>(a[t]) + m0 * seg;
    g.seg = seg;
    g.M = ms;
    g.N = N;
    g.K = seg * n_seg;
    g.w = w_q;
    g.w_scale = w_scale;
    g.out_kind = out_kind;
    const bool split = p.ksplit > 1;
    void* out_s = static_cast<char*>(out) + m0 * N * out_es;
    g.partial = split ? 1 : 0;
    g.out = split ? workspace : out_s;
    hipError_t e = launch_stream_fp8(p, g, stream);
    if (e == hipSuccess && split) e = launch_splitk_reduce(p, ms, N, out_s, out_kind, workspace, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bdr
