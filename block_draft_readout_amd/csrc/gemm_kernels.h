// Weight-streaming GEMM kernels shared by the gemm translation units (gfx950).
// C[M, N] = A[M, K] * W[N, K]^T with A given as segments laid side by side
// along K; see gemm.hip for the plans that choose between them.
#pragma once

#include <algorithm>
#include <type_traits>
#include <utility>

#include "bdr_device.h"
#include "bdr_internal.h"

namespace bdr {

struct GemmArgs {
  const void* a[BDR_MAX_TAPS];  // A segments, each [M, seg]
  int64_t seg;
  int64_t M, N, K;              // K = n_seg * seg
  const void* w;                // [N, K]
  void* out;                    // final [M, N] or fp32 partials [ksplit, M, N]
  int out_kind;                 // OutKind of a final output
  int partial;                  // 1: write fp32 partials indexed by blockIdx.y
  int64_t steps_per_split;      // K steps handled by one workgroup along K
  const float* w_scale;         // fp8 weights: one scale per W row [N]; else unused
};

// Segment base pointer chosen with scalar selects (t is uniform), so the
// pointer array is never indexed dynamically.
__device__ __forceinline__ const void* seg_base(const GemmArgs& g, int t) {
  const void* p = g.a[0];
#pragma unroll
  for (int c = 1; c < BDR_MAX_TAPS; ++c)
    if (t == c) p = g.a[c];
  return p;
}

struct StreamArgs {
  GemmArgs g;
  int64_t n_waves;      // workgroups along N (balanced row ranges)
  int64_t kblocks;      // K blocks per row (the last may be partial)
  int64_t kb_per_split; // K blocks per workgroup along K
};

// Output of one workgroup, read out of the kernel arguments once: fp32
// partials of K split `split` ([ksplit, M, N]), or the final fp32 / bf16 C.
struct OutRef {
  float* f32;
  uint16_t* bf16;   // non-null: final bf16 output
  int64_t M, N;
  __device__ __forceinline__ OutRef(const GemmArgs& g, unsigned split) : M(g.M), N(g.N) {
    if (g.partial) {
      f32 = static_cast<float*>(g.out) + static_cast<int64_t>(split) * g.M * g.N;
      bf16 = nullptr;
    } else if (g.out_kind == OUT_BF16) {
      f32 = nullptr;
      bf16 = static_cast<uint16_t*>(g.out);
    } else {
      f32 = static_cast<float*>(g.out);
      bf16 = nullptr;
    }
  }
  __device__ __forceinline__ void put(int64_t m, int64_t n, float v) const {
    if (bf16)
      bf16[m * N + n] = f32_to_bf16(v);
    else
      f32[m * N + n] = v;
  }
};

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, every index a compile-time constant
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ----------------------------------------------------------------------------
// Shared-visit streaming variant for 16 < M <= 160 with fp32 operands (bf16
// and fp8 weights take the row-split kernel of gemm_ns.h).
//
// A workgroup of four waves owns a balanced contiguous range of W rows, walked
// in passes of at most NT 16-row tiles (the accumulators of one pass live in
// registers), and a range of K blocks (KBB bytes of every row).  The waves share every visit
// (VT tiles of 16 W rows x one K block): each wave copies a quarter of its
// rows into a ring of R LDS slots with buffer-to-LDS loads, kAhead = R - 2
// visits ahead of the one being multiplied, and a workgroup barrier per visit
// publishes the slot.  Wave w multiplies the visit against A row tiles w, w+4, w+8.  Their
// slice of the next K block is copied the same way into a per-tile LDS area
// while the current block runs, and moved into registers once per block, so
// A costs one read per workgroup and K block whatever the rows it owns.
//
// Visits run pass by pass, K block by K block, and the loads stream on across
// block and pass boundaries.
//
// Slot reuse: visit v goes to slot v % R and is loaded while visit v - kAhead
// is multiplied; the slot last held visit v - 2, which every wave finished
// reading before arriving at the barrier of visit v - 1.
//
// Loads to LDS are not tracked by the compiler, so every wait on them is
// explicit and counts what this wave issued afterwards (vmcnt retires loads in
// issue order):
//  * before multiplying visit v: its loads are followed by those of visits
//    v+1 .. v+kAhead and, if v is within kAhead visits of its block's first,
//    by the next block's A slice;
//  * before moving a block's A slice into registers: it is followed by the
//    loads of at least min(tiles, kAhead) visits.
// Past the last visit to load, waits drain everything.
// ----------------------------------------------------------------------------
constexpr int kWgWaves = 4;
constexpr int kWgKBB = 512;                   // W bytes per row per visit
constexpr int kWgMaxTiles = 10;               // A row tiles (M <= 160)

template <int KBB>
struct VisitShape {
  static constexpr int RPI = 1024 / KBB;             // rows per 1 KB buffer-to-LDS load
  static constexpr int GROUP = 1024 + 16 * RPI;      // LDS bytes per load (padded: no bank aliasing)
  static constexpr int SLOT = (16 / RPI) * GROUP;    // one 16-row x KBB tile
  static constexpr int NI = 16 / RPI / kWgWaves;     // loads per wave per W visit
  static constexpr int NIA = 16 / RPI;               // loads per A tile
  static constexpr int STEPS = KBB / 64;             // 16-byte operand steps per row
};

// Explicit waits on buffer-to-LDS loads (gfx9 encoding: vmcnt <= n, lgkmcnt
// <= l, expcnt free).  The empty assembly statement with a memory clobber and
// the scheduling barrier keep loads and stores from moving across.
#define BDR_WAIT_VM_LGKM(n, l)                                                          \
  do {                                                                                  \
    __builtin_amdgcn_s_waitcnt(((n)&0xF) | (0x7 << 4) | (((l)&0xF) << 8) |               \
                               ((((n) >> 4) & 3) << 14));                               \
    asm volatile("" ::: "memory");                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                  \
  } while (0)
#define BDR_WG_BARRIER()                 \
  do {                                   \
    asm volatile("s_barrier" ::: "memory"); \
    __builtin_amdgcn_sched_barrier(0);   \
  } while (0)

// wait until at most NI * c loads are outstanding, c = min(tiles, kAhead) in 1..kAhead
template <int NI, int C>
__device__ __forceinline__ void wait_vm_tiles(int c) {
  if constexpr (C > 1) {
    if (c < C) {
      wait_vm_tiles<NI, C - 1>(c);
      return;
    }
  }
  BDR_WAIT_VM_LGKM(NI * C, 15);
}

// wait until at most BASE + PER * n loads are outstanding, n in 0..N
template <int BASE, int PER, int N>
__device__ __forceinline__ void wait_vm_visit(int n) {
  if constexpr (N > 0) {
    if (n < N) {
      wait_vm_visit<BASE, PER, N - 1>(n);
      return;
    }
  }
  BDR_WAIT_VM_LGKM(BASE + PER * N, 0);
}

// fp8 weights (row-split kernel): S = uint8_t means E4M3 codes with one fp32
// scale per W row against bf16 A
template <typename S> constexpr bool kIsFp8 = std::is_same_v<S, uint8_t>;

// LDS bytes of the workgroup kernel: R visits of VT tiles + one staging tile per A tile
inline size_t wg_lds_bytes(int ring, int vt, int mtiles) {
  return static_cast<size_t>(ring * vt + mtiles) * VisitShape<kWgKBB>::SLOT;
}

// 16 E4M3 codes (little-endian bytes of q) -> bf16 operands of elements 0..7 (lo)
// and 8..15 (hi); exact, every E4M3 value being a bf16 value
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4_t q, u32x4_t& lo, u32x4_t& hi) {
  lo.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false));
  lo.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true));
  lo.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false));
  lo.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true));
  hi.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.z, 1.0f, false));
  hi.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.z, 1.0f, true));
  hi.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.w, 1.0f, false));
  hi.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.w, 1.0f, true));
}

template <typename S, int MTW, int NT, int VT, int R>
__global__ __launch_bounds__(256) void ws_gemm_stream_wg_kernel(const StreamArgs sa) {
  constexpr int KBB = kWgKBB;            // bytes per row per visit (W and A)
  using VS = VisitShape<KBB>;            // W visit geometry
  using VA = VS;                         // A staging geometry
  constexpr int STEPS = VA::STEPS;       // 16-byte A operands per row and block
  constexpr int NI = VT * VS::NI;        // W loads per wave per visit
  constexpr int NA = MTW * VA::NIA;      // A loads per wave per K block
  constexpr int NV = NT / VT;            // visits per K block and pass (compile-time bound)
  constexpr int kAhead = R - 2;
  static_assert(NT % VT == 0, "tiles per pass must be whole visits");
  static_assert(NI * kAhead + NA <= 63, "vmcnt range");
  const GemmArgs& g = sa.g;
  extern __shared__ __attribute__((aligned(16))) char lds[];   // [R * VT + mtiles][SLOT]
  // wave index in a scalar register, so per-wave choices are uniform branches
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const int64_t n_lo = static_cast<int64_t>(blockIdx.x) * g.N / sa.n_waves;
  const int64_t n_hi = static_cast<int64_t>(blockIdx.x + 1) * g.N / sa.n_waves;
  const int ntiles = static_cast<int>((n_hi - n_lo + 15) / 16);
  const uint32_t kb_lo = static_cast<uint32_t>(blockIdx.y * sa.kb_per_split);
  const uint32_t kb_hi = static_cast<uint32_t>(min<int64_t>(sa.kblocks, kb_lo + sa.kb_per_split));
  if (ntiles <= 0 || kb_lo >= kb_hi) return;   // whole workgroup
  // the range's tiles in npass balanced passes of at most NT tiles
  const int npass = (ntiles + NT - 1) / NT;
  auto pass_lo = [&](int p) { return p * ntiles / npass; };
  auto pass_visits = [&](int p) { return (pass_lo(p + 1) - pass_lo(p) + VT - 1) / VT; };
  const int nkb = static_cast<int>(kb_hi - kb_lo);
  const OutRef out(g, blockIdx.y);
  const uint32_t kbytes = static_cast<uint32_t>(g.K * static_cast<int64_t>(sizeof(S)));
  const uint32_t akbytes = kbytes;                                      // A row bytes
  const uint32_t segbytes = static_cast<uint32_t>(g.seg * static_cast<int64_t>(sizeof(S)));
  const int mtiles = static_cast<int>((g.M + 15) / 16);

  // rows past the range (also those of a last visit's missing tile) read zeros
  const rsrc_t rw = make_rsrc(static_cast<const S*>(g.w) + n_lo * g.K,
                              static_cast<uint32_t>(n_hi - n_lo) * kbytes);
  const uint32_t abytes = static_cast<uint32_t>(g.M) * segbytes;
  // buffer-to-LDS lane mapping: row (lane % RPI) of the load, 16-byte chunk lane / RPI
  const uint32_t dma_chunk = static_cast<uint32_t>(lane / VS::RPI) * 16;
  const uint32_t dma_row = static_cast<uint32_t>(lane % VS::RPI);
  const uint32_t dma_chunk_a = static_cast<uint32_t>(lane / VA::RPI) * 16;
  const uint32_t dma_row_a = static_cast<uint32_t>(lane % VA::RPI);
  // operand read of row r16, chunk grp + 4 * step inside a W tile
  const uint32_t rd = static_cast<uint32_t>((r16 / VS::RPI) * VS::GROUP +
                                            (grp * VS::RPI + r16 % VS::RPI) * 16);
  // chunk c of row r16 inside an A staging tile: rd_a + c * 16 * VA::RPI
  const uint32_t rd_a = static_cast<uint32_t>((r16 / VA::RPI) * VA::GROUP + (r16 % VA::RPI) * 16);
  constexpr int VSLOT = VT * VS::SLOT;        // one visit
  char* const stage = lds + R * VSLOT;        // A staging, one VA::SLOT per A tile

  f32x4_t acc[NT][MTW];
  auto zero_acc = [&]() {
    static_for<NT>([&](auto t) {
      static_for<MTW>([&](auto mw) { acc[t][mw] = f32x4_t{0.f, 0.f, 0.f, 0.f}; });
    });
  };
  zero_acc();
  // A operands; tiles past M stay zero (their products are never stored, and
  // the wave holding the most valid tiles sets the pace either way)
  u32x4_t a[MTW][STEPS];
  static_for<MTW>([&](auto mw) {
    static_for<STEPS>([&](auto st) { a[mw][st] = u32x4_t{0u, 0u, 0u, 0u}; });
  });

  // this wave's rows of the W visit starting at tile tile0 of the range, K block kb -> ring slot
  auto dma_w = [&](uint32_t kb, int tile0, int slot) {
    const uint32_t k0 = kb * KBB;
    const uint32_t lo = k0 + dma_chunk < kbytes ? dma_chunk : kOOB;
    char* dst = lds + slot * VSLOT;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int gi = wave * NI + j;           // load index inside the visit
      const uint32_t row = static_cast<uint32_t>(16 * tile0 + gi * VS::RPI) + dma_row;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(dst + gi * VS::GROUP), 16,
          lo + row * kbytes + k0, 0, 0, 2);
    }
  };
  // this wave's A tiles of K block kb -> staging (rows >= M and bytes past K
  // read zeros; K blocks never straddle A segments); tiles_w * NIA loads
  auto dma_a = [&](uint32_t kb) {
    const uint32_t k0 = kb * kWgKBB;          // A bytes
    const uint32_t ts = k0 / segbytes;
    const rsrc_t ra = make_rsrc(seg_base(g, static_cast<int>(ts)), abytes);
    const uint32_t lo = k0 + dma_chunk_a < akbytes ? (k0 - ts * segbytes) + dma_chunk_a : kOOB;
    static_for<MTW>([&](auto mw) {
      const int mt = wave + kWgWaves * mw;
      if (mt < mtiles) {
        char* dst = stage + mt * VA::SLOT;
#pragma unroll
        for (int j = 0; j < VA::NIA; ++j) {
          const uint32_t row = static_cast<uint32_t>(16 * mt + j * VA::RPI) + dma_row_a;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              ra, (__attribute__((address_space(3))) void*)(dst + j * VA::GROUP), 16,
              lo + row * segbytes, 0, 0, 0);
        }
      }
    });
  };
  // A operand i of row r16: chunk 4i + grp (elements of MFMA step i)
  auto stage_to_regs = [&]() {
    static_for<MTW>([&](auto mw) {
      const int mt = wave + kWgWaves * mw;
      if (mt < mtiles) {
        const char* src = stage + mt * VA::SLOT + rd_a;
        static_for<STEPS>([&](auto st) {
          a[mw][st] = *reinterpret_cast<const u32x4_t*>(src + (4 * st + grp) * 16 * VA::RPI);
        });
      }
    });
  };
  // all VT tiles of visit vt (compile-time) of the current pass, from a ring slot
  auto compute = [&](auto vt, int slot) {
    const char* src = lds + slot * VSLOT + rd;
    {
      u32x4_t bv[VT][STEPS];
      static_for<VT>([&](auto u) {
        static_for<STEPS>([&](auto st) {
          bv[u][st] = *reinterpret_cast<const u32x4_t*>(src + u * VS::SLOT + st * 64 * VS::RPI);
        });
      });
      static_for<VT>([&](auto u) {
        constexpr int t = VT * decltype(vt)::value + decltype(u)::value;
        static_for<STEPS>([&](auto st) {
          static_for<MTW>([&](auto mw) {
            acc[t][mw] = mma16(a[mw][st], bv[u][st], acc[t][mw], S());
          });
        });
      });
      // issue all of the visit's LDS reads before its MFMAs (one latency per visit)
      __builtin_amdgcn_sched_group_barrier(0x100, VT * STEPS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, VT * STEPS * MTW * Elem<S>::MFMA_PER16, 0);
    }
  };

  int nvis = 0;
  for (int p = 0; p < npass; ++p) nvis += pass_visits(p) * nkb;
  // fewest visits of a K block in any pass (every pass has floor or ceil of ntiles / npass tiles)
  const int cwait = min((ntiles / npass + VT - 1) / VT, kAhead);
  // A tiles this wave holds (its A loads per block: tiles_w * NIA)
  const int tiles_w = mtiles > wave ? min(MTW, (mtiles - wave + kWgWaves - 1) / kWgWaves) : 0;
  // load cursor: visit iv = (pass ip, block ikb, visit ivt of ivn)
  int iv = 0, ip = 0, ivt = 0, ivn = pass_visits(0), itile = pass_lo(0);
  uint32_t ikb = kb_lo;
  auto issue_next = [&]() {
    dma_w(ikb, itile + VT * ivt, iv % R);
    ++iv;
    if (++ivt == ivn) {
      ivt = 0;
      if (++ikb == kb_hi && ip + 1 < npass) {
        ikb = kb_lo;
        ++ip;
        ivn = pass_visits(ip);
        itile = pass_lo(ip);
      }
    }
  };

  dma_a(kb_lo);
  for (int d = 0; d < kAhead && iv < nvis; ++d) issue_next();
  int v = 0;                // visit multiplied next
  int p = 0;                // pass of the block multiplied next
  int tp_lo = 0, ntp = pass_lo(1), nvtp = pass_visits(0);
  uint32_t kb = kb_lo;
  for (int blk = 0; blk < npass * nkb; ++blk) {
    const bool last_kb = kb + 1 == kb_hi;
    // the next block's A slice: this pass's next K block, or the next pass's first
    const bool more = !last_kb || p + 1 < npass;
    const uint32_t kb_next = last_kb ? kb_lo : kb + 1;
    static_for<NV>([&](auto vt) {
      if (vt < nvtp) {
        const bool full = v + kAhead < nvis;
        if (full) issue_next();
        if constexpr (vt == 0) {
          // this block's A slice: followed by >= min(visits, kAhead) visits' loads
          if (full)
            wait_vm_tiles<NI, kAhead>(cwait);
          else
            BDR_WAIT_VM_LGKM(0, 15);
          stage_to_regs();
          BDR_WAIT_VM_LGKM(63, 0);    // staging read out before it is refilled
          if (more) dma_a(kb_next);
        }
        if (full) {
          if (vt <= kAhead && more)
            wait_vm_visit<NI * kAhead, VA::NIA, MTW>(tiles_w);
          else
            BDR_WAIT_VM_LGKM(NI * kAhead, 0);
        } else {
          BDR_WAIT_VM_LGKM(0, 0);
        }
        BDR_WG_BARRIER();
        compute(vt, v % R);
        ++v;
      }
    });
    if (!last_kb) {
      ++kb;
      continue;
    }
    // pass p complete.  The stores join the memory queue behind loads still in
    // flight; the waits above count loads only, so a store can only make them
    // stricter.  The row base is made opaque here so that no part of the
    // addresses is kept live across the loop.
    int64_t nbase = n_lo + 16 * tp_lo + r16;
    asm volatile("" : "+v"(nbase));
    static_for<NT>([&](auto t) {
      const int64_t n = nbase + 16 * t;
      static_for<MTW>([&](auto mw) {
        const int mt = wave + kWgWaves * mw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = 16 * mt + 4 * grp + i;
          if (t < ntp && m < out.M && n < n_hi) out.put(m, n, acc[t][mw][i]);
        }
      });
    });
    zero_acc();
    ++p;
    kb = kb_lo;
    tp_lo = pass_lo(p);
    ntp = pass_lo(p + 1) - tp_lo;
    nvtp = pass_visits(p);
  }
}

// Visit width and ring depth by A tiles per wave.  Two tiles per visit halve
// the barriers per byte and give each wave twice the independent accumulator
// chains per visit (4-5 % faster on a bf16 LM head than one-tile visits when
// this kernel served bf16).  With three A tiles per wave the A staging leaves
// room for too shallow a ring of two-tile visits, so visits keep one tile
// there.  The ring is as deep as LDS holds next to the staging of 4 * MTW tiles.
template <int MTW> struct WgShape {
  static constexpr int VT = MTW < 3 ? 2 : 1;
  static constexpr int R = MTW == 1 ? 6 : MTW == 2 ? 5 : 9;
};

// Launch one instantiation with its dynamic LDS (ring + staging for mt tiles).
template <typename S, int MTW, int NT>
hipError_t launch_wg_one(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
  constexpr int VT = WgShape<MTW>::VT;
  constexpr int R = WgShape<MTW>::R;
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&ws_gemm_stream_wg_kernel<S, MTW, NT, VT, R>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(wg_lds_bytes(R, VT, std::min(kWgWaves * MTW, kWgMaxTiles))));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid(static_cast<unsigned>(p.n_waves), static_cast<unsigned>(p.ksplit));
  hipLaunchKernelGGL((ws_gemm_stream_wg_kernel<S, MTW, NT, VT, R>), grid, dim3(64 * kWgWaves),
                     wg_lds_bytes(R, VT, p.mt), st, sa);
  return hipSuccess;
}

// Launchers of the workgroup streaming kernel, one translation unit per number
// of A tiles a wave holds (p.mtw), so the instantiations compile in parallel;
// each returns hipErrorInvalidValue for a tile count it does not instantiate.
hipError_t launch_gemm_tile(const GemmPlan& p, const GemmArgs& g, hipStream_t stream);
int tile_cols(int shape);   // output columns of a tiled-variant workgroup tile
hipError_t launch_wg_mtw1(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
hipError_t launch_wg_mtw2(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
hipError_t launch_wg_mtw3(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
// fp8 (E4M3) weights with per-row scales, bf16 A: one-wave streaming kernel
// (gemm_fp8.hip)
hipError_t launch_stream_fp8(const GemmPlan& p, const GemmArgs& g, hipStream_t st);
// row-split workgroup kernel (gemm_ns.h): bf16 and fp8 weights, bf16 A
hipError_t launch_ns_bf16(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
hipError_t launch_ns_fp8(const GemmPlan& p, const StreamArgs& sa, hipStream_t st);
hipError_t launch_ns_pair_bf16(int mt0, int mt1, const StreamArgs& a0, const StreamArgs& a1,
                               unsigned n0, unsigned n1, hipStream_t st);

}  // namespace bdr
