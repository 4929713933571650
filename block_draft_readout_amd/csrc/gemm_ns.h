// Row-split workgroup GEMM for 16 < M <= 160 (gfx950): C[M, N] = A[M, K] * W[N, K]^T,
// W in bf16, or in fp8 (E4M3 codes, one fp32 scale per row) against bf16 A.
//
// Four waves per workgroup; the workgroup owns a balanced range of W rows (in
// whole 16-row tiles) and each wave a quarter of it.  Every wave streams its
// own rows through a private LDS ring with buffer-to-LDS loads (no workgroup
// barrier per visit, and each fp8 code is widened once), while the A slice of
// the current K block is shared: staged once per workgroup into LDS (double-
// buffered, one barrier per K block) and held in every wave's registers for
// all the A row tiles, so one W visit (16 rows x 128 reduction elements)
// feeds MT independent accumulator chains.
//
//   K block   128 reduction elements: W visit rows of 256 bytes (bf16) or 128
//             bytes (fp8), A slice rows of 256 bytes (never straddling a tap
//             segment: segments are multiples of 128 elements);
//   passes    a wave walks its tiles in passes (accumulator budget NTW * MT *
//             4 registers); every wave of a workgroup runs the same number of
//             passes and K blocks, so the barriers match;
//   order     visits run pass by pass, K block by K block, tile by tile, and
//             each wave's loads stream on across block and pass boundaries,
//             R visits ahead (a ring slot is refilled as soon as this wave's
//             LDS reads of the visit it held are done, before that visit's
//             MFMAs, so R visits are in flight while they run);
//   A stage   the slice of the next block is copied (each wave a quarter of
//             the loads) right after the barrier of the current one; the
//             buffer it overwrites was last read before that barrier.
//
// The schedule is fixed at compile time, so the loop carries almost no
// bookkeeping (a loop that tracked its visits at run time spent about as
// many scalar instructions as MFMAs and kept the MFMA pipe ~28 % busy):
//   * a pass holds ng groups of R tile slots (ng <= NG, chosen per workgroup
//     from its range so that few slots stay empty); tile t of a pass lives in
//     ring slot t % R in every K block;
//   * the visit loaded at step t is the one R ahead, into the slot step t has
//     just read: tile t + R of this block, or tile t + R - ng R of the next
//     block (or of the next pass's first) -- the slot is known at compile
//     time, only the tile's offset is selected at run time;
//   * a slot past the wave's tiles (at most a few in its last pass) reads
//     nothing (out-of-range loads) and is not stored;
//   * loads to LDS are not tracked by the compiler, so the waits are explicit
//     and count what this wave issued after the data it needs (vmcnt retires
//     in issue order).  Every block issues its MT A-staging loads (out of
//     range past the last block or row), so each wait counts a compile-time
//     number of loads: before step t NI * (R - 1), + MT while the visit
//     predates the block's A loads (t < R); before a block's barrier NI * R
//     (at least R visits followed its A loads).
// R is a template argument: deep rings for long ranges (the LM head), shallow
// ones where a wave has two or three tiles (a K-split fc), so that the ring is
// not filled with empty slots.
//
// Weights in the packed layout (bf16) come in visits stored in MFMA operand
// order (1 KB part i holds, for lane l = 16 g + r, elements 32 i + 8 g .. + 7
// of the visit's row r).  The LDS ring copies each part to one load group and
// reads it back linearly; with REG = true (five or more A row tiles) they skip
// LDS: four contiguous 1 KB loads put a visit straight into the registers the
// MFMAs read, and the ring is R visits of registers (a pass is one group of R
// tiles, the register budget).  Its slot is refilled once the visit's MFMAs
// are issued; the waits count the same loads as above.  fp8 codes (the fc's
// K-split plans) take the register ring from the row-major matrix: load p of
// a visit gives lane l = 16 g + r the 16 codes of row r at 64 p + 16 g, the
// operand order of the LDS path's reads, with no LDS ring beside the chain.
#pragma once

#include "gemm_kernels.h"

namespace bdr {

constexpr int kNsWaves = 4;
constexpr int kNsKE = 128;             // reduction elements per K block

template <typename S>
struct NsShape {
  static constexpr bool F8 = kIsFp8<S>;
  static constexpr int WROW = F8 ? 128 : 256;       // W bytes per row per visit
  static constexpr int RPI = 1024 / WROW;           // rows per 1 KB load
  static constexpr int GROUP = 1024 + 16 * RPI;     // padded LDS bytes per load
  static constexpr int NI = 16 / RPI;               // loads per visit
  static constexpr int SLOT = NI * GROUP;           // one visit
  static constexpr int ASLOT = 4 * (1024 + 64);     // one A tile: 16 rows x 256 B, 4 rows per load
  static constexpr int WSTEPS = F8 ? 2 : 4;         // 16-byte W reads per row per visit
  // LDS position of 16-byte chunk c of a row = c ^ wx(row in load, load of the
  // visit) for W, c ^ ax(row in load) for A.  Chosen so that the 16 rows one
  // operand read touches spread over the banks with no conflict, with 128
  // banks served 32 lanes at a time (the fp8 reads of the bf16 permutation
  // measured about one conflict cycle per LDS instruction).
  static constexpr int wx(int ril, int load) { return F8 ? (ril >> 1) ^ (load ? 4 : 0) : ril; }
  static constexpr int ax(int ril) { return F8 ? ril ^ (ril >> 1) : ril; }
};

template <int MT> constexpr int ns_lean_ntw_max() { return kNsLeanNtwMax[MT]; }

template <int MT, int R, bool REG = false>
struct NsLean {
  // groups of R slots per pass, at most (the register ring: one)
  static constexpr int NG = REG ? 1 : ns_lean_ntw_max<MT>() / R;
  static constexpr int NTW = NG * R;
};

template <typename S, int MT, int R, bool REG = false>
constexpr size_t ns_lean_lds_bytes() {
  using SH = NsShape<S>;
  return (REG ? size_t(0) : static_cast<size_t>(kNsWaves * R * SH::SLOT)) +
         static_cast<size_t>(2 * MT) * SH::ASLOT;
}

template <int N>
__device__ __forceinline__ void ns_wait_vm() {
  constexpr int n = N > 63 ? 63 : N;   // (a stricter wait is always safe)
  BDR_WAIT_VM_LGKM(n, 15);
}

template <typename S, int MT, int R, bool REG = false>
__device__ __forceinline__ void ns_lean_body(const StreamArgs& sa, unsigned bx, unsigned by,
                                             char* lds) {
  using SH = NsShape<S>;
  constexpr bool F8 = SH::F8;
  constexpr int NG = NsLean<MT, R, REG>::NG;
  constexpr int NTW = NsLean<MT, R, REG>::NTW;
  static_assert(NG >= 1 && R >= 2, "ring shape");
  static_assert(ns_lean_lds_bytes<S, MT, R, REG>() <= 160 * 1024, "LDS budget");
  constexpr int NI = SH::NI;        // loads per visit
  constexpr int NA = MT;            // A loads per wave per block
  static_assert(NI * (R - 1) + NA <= 63, "vmcnt range");
  const GemmArgs& g = sa.g;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  // the workgroup's 16-row tiles, then this wave's quarter of them: ranges
  // start on a tile boundary, so each 16-column piece of an output row is one
  // aligned 64-byte store (a range starting mid-tile made every piece straddle
  // two 64-byte blocks: 1.8x the logits' bytes written).  Row indices fit 31
  // bits; readfirstlane keeps everything derived from the wave index in
  // scalar registers, so the load descriptors stay uniform.
  const int64_t n_t = (g.N + 15) / 16;
  const int64_t t_lo = static_cast<int64_t>(bx) * n_t / sa.n_waves;
  const int64_t t_hi = static_cast<int64_t>(bx + 1) * n_t / sa.n_waves;
  const int n_lo = __builtin_amdgcn_readfirstlane(
      static_cast<int>(16 * (t_lo + (t_hi - t_lo) * wave / kNsWaves)));
  const int n_hi = __builtin_amdgcn_readfirstlane(static_cast<int>(
      min<int64_t>(g.N, 16 * (t_lo + (t_hi - t_lo) * (wave + 1) / kNsWaves))));
  // passes and groups: the same on every wave (from the largest quarter)
  const int max_tiles = static_cast<int>((t_hi - t_lo + kNsWaves - 1) / kNsWaves);
  const int npass = max(1, (max_tiles + NTW - 1) / NTW);
  const int ng = __builtin_amdgcn_readfirstlane(
      max(1, (max_tiles + npass * R - 1) / (npass * R)));
  const uint32_t kb_lo = static_cast<uint32_t>(by * sa.kb_per_split);
  const uint32_t kb_hi = static_cast<uint32_t>(min<int64_t>(sa.kblocks, kb_lo + sa.kb_per_split));
  if (t_hi <= t_lo || kb_lo >= kb_hi) return;   // whole workgroup
  // output: fp32 partials of K split `by`, or the final fp32 / bf16 C (the
  // plan keeps M * N * 4 below 2^32)
  const bool o_bf16 = !g.partial && g.out_kind == OUT_BF16;
  const uint32_t o_es = o_bf16 ? 2 : 4;
  const uint32_t o_row = static_cast<uint32_t>(g.N) * o_es;      // bytes per output row
  const rsrc_t ro = make_rsrc(
      static_cast<char*>(g.out) + (g.partial ? static_cast<int64_t>(by) * g.M * g.N * 4 : 0),
      static_cast<uint32_t>(g.M) * o_row);
  const uint32_t o_lane = static_cast<uint32_t>(4 * grp) * o_row;  // this lane's first row
  const uint32_t kbytes = static_cast<uint32_t>(g.K * static_cast<int64_t>(sizeof(S)));
  const uint32_t akbytes = static_cast<uint32_t>(g.K * 2);
  const uint32_t segbytes = static_cast<uint32_t>(g.seg * 2);
  const uint32_t abytes = static_cast<uint32_t>(g.M) * segbytes;
  // W layout.  Rows: [N, K].  Packed (bf16 only; always with the register
  // ring): the visits themselves, K block by K block and tile by tile
  // ([kblocks][ceil(N / 16)][4096 bytes], zero-padded, each in operand order),
  // so a visit is one contiguous 4 KB and the visits of one K block are
  // adjacent.  A visit's bytes sit at block * kb_str + tile * tile_bytes (rows
  // row_str apart in the row-major layout).
  const bool packed = !F8 && (REG || g.w_packed != 0);
  const uint32_t row_str = packed ? static_cast<uint32_t>(SH::WROW) : kbytes;
  const uint32_t kb_str = packed ? static_cast<uint32_t>(n_t * 16 * SH::WROW)
                                 : static_cast<uint32_t>(SH::WROW);
  const uint32_t wrows = static_cast<uint32_t>(n_hi > n_lo ? n_hi - n_lo : 0);
  const rsrc_t rw =
      packed ? make_rsrc(static_cast<const char*>(g.w) + static_cast<int64_t>(n_lo) * SH::WROW,
                         static_cast<uint32_t>((sa.kblocks * n_t * 16 - n_lo) * SH::WROW))
             : make_rsrc(static_cast<const S*>(g.w) + static_cast<int64_t>(n_lo) * g.K,
                         wrows * kbytes);
  char* const ring = lds + wave * (R * SH::SLOT);                // (LDS ring)
  char* const stage = lds + (REG ? 0 : kNsWaves * R * SH::SLOT);  // [2][MT][ASLOT]
  // Load lane mapping: consecutive lanes read one row's bytes (row lane / CPR
  // of the load, CPR = 16-byte chunks per row), so every quad of lanes reads
  // 64 contiguous bytes.  Each row is stored in LDS with its chunks permuted
  // (NsShape::wx / ax): lane l of load j fetches the chunk that belongs at
  // position l % CPR, and operand reads undo the permutation.
  constexpr int CPR = SH::WROW / 16;
  constexpr int NPERM = F8 ? NI : 1;   // distinct permutations among a visit's loads
  // (packed: load j of a visit is its part j, lane l's 16 bytes at 16 l,
  // stored as they come and read back linearly)
  const uint32_t lane16 = static_cast<uint32_t>(lane) * 16;
  uint32_t w_chunk[NPERM], lane_off[NPERM];
#pragma unroll
  for (int j = 0; j < NPERM; ++j) {
    w_chunk[j] = static_cast<uint32_t>((lane % CPR) ^ SH::wx(lane / CPR, j)) * 16;
    lane_off[j] = packed ? lane16 : static_cast<uint32_t>(lane / CPR) * row_str + w_chunk[j];
    if constexpr (!REG) asm volatile("" : "+v"(lane_off[j]));
  }
  const uint32_t jstride = packed ? 1024u : static_cast<uint32_t>(SH::RPI) * row_str;
  // (fp8, register ring) the column of load q of a visit's row and the lane's
  // offset within the visit
  uint32_t f8_col[2], f8_lane[2];
  static_for<2>([&](auto q) {
    f8_col[q] = static_cast<uint32_t>(64 * q + 16 * grp);
    f8_lane[q] = static_cast<uint32_t>(r16) * row_str + f8_col[q];
  });
  const uint32_t a_row = static_cast<uint32_t>(lane / 16);
  const uint32_t a_chunk = static_cast<uint32_t>((lane % 16) ^ SH::ax(lane / 16)) * 16;
  const uint32_t rd = static_cast<uint32_t>((r16 / SH::RPI) * SH::GROUP + (r16 % SH::RPI) * SH::WROW);
  const int rs = SH::wx(r16 % SH::RPI, r16 / SH::RPI);
  uint32_t w_rd[SH::WSTEPS];   // LDS offset of each 16-byte W operand read within a slot
  static_for<SH::WSTEPS>([&](auto q) {
    w_rd[q] = packed ? static_cast<uint32_t>(q * SH::GROUP) + lane16
                     : rd + static_cast<uint32_t>(((4 * q + grp) ^ rs) * 16);
  });
  const uint32_t rd_a = static_cast<uint32_t>((r16 / 4) * (1024 + 64) + (r16 % 4) * 256);
  const int rs_a = SH::ax(r16 % 4);
  const uint32_t tile_bytes = 16 * row_str;
  const uint32_t pass_bytes = static_cast<uint32_t>(ng * R) * tile_bytes;
  // the last K block may be partial: its row pieces end at tail_bytes
  const uint32_t tail_bytes = kbytes - (static_cast<uint32_t>(sa.kblocks) - 1) * SH::WROW;
  const uint32_t kb_last = static_cast<uint32_t>(sa.kblocks) - 1;

  f32x4_t acc[NTW][MT];
  auto zero_acc = [&]() {
    static_for<NTW>([&](auto t) {
      static_for<MT>([&](auto m) { acc[t][m] = f32x4_t{0.f, 0.f, 0.f, 0.f}; });
    });
  };
  zero_acc();
  u32x4_t a[MT][4];
  u32x4_t wr[REG ? R : 1][SH::WSTEPS];   // the register ring

  // visit -> ring slot: sb = the visit's byte offset within this wave's rows
  // (pass base + K block + tile), kOOB for a visit past the last pass; ti = its
  // tile within the wave's range, a tile past the range (an empty slot) reads
  // nothing (in the packed layout the descriptor reaches past the range).  The
  // slot is a compile-time constant.
  const int wtiles = __builtin_amdgcn_readfirstlane((n_hi - n_lo + 15) / 16);
  auto dma_w = [&](uint32_t sb, int ti, uint32_t kb, auto slot) {
    const bool none = sb == kOOB || ti >= wtiles;
    if constexpr (REG && F8) {
      // row-major codes straight into operand layout: load p gives lane
      // (grp, r16) the 16 codes of the visit's row r16 at 64 p + 16 grp (rows
      // past the wave's range lie beyond the descriptor; codes past a partial
      // last block are cut)
      const uint32_t s_off = __builtin_amdgcn_readfirstlane(none ? kOOB : sb);
      static_for<2>([&](auto q) {
        const bool cut = kb == kb_last && f8_col[q] >= tail_bytes;
        wr[slot][q] = bload16_nt(rw, cut ? kOOB : s_off + f8_lane[q]);
      });
    } else if constexpr (REG) {
      // part i (1 KB) -> wr[slot][i]; a partial last block reads the copy's zeros
      const uint32_t s_off = __builtin_amdgcn_readfirstlane(none ? kOOB : sb);
      static_for<4>([&](auto i) {
        wr[slot][i] = bload16_nt(rw, s_off + static_cast<uint32_t>(i * 1024) + lane16);
      });
    } else {
      char* dst = ring + slot * SH::SLOT;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int jp = NPERM > 1 ? j : 0;
        // past a partial block's end (the packed copy holds zeros there)
        const bool cut = !packed && kb == kb_last && w_chunk[jp] >= tail_bytes;
        const uint32_t s_off = __builtin_amdgcn_readfirstlane(
            none ? kOOB : sb + static_cast<uint32_t>(j) * jstride);
        const uint32_t off = cut ? kOOB : lane_off[jp] + s_off;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (__attribute__((address_space(3))) void*)(dst + j * SH::GROUP), 16, off, 0, 0, 2);
      }
    }
  };
  // this wave's share of the A slice of block kb -> staging buffer b (all MT
  // loads issued, out of range when !valid or past M)
  auto dma_a = [&](uint32_t kb, int b, bool valid) {
    const uint32_t k0 = kb * (kNsKE * 2);
    const uint32_t ts = k0 / segbytes;
    const rsrc_t ra = make_rsrc(seg_base(g, static_cast<int>(ts)), abytes);
    const uint32_t lo = (valid && k0 + a_chunk < akbytes) ? (k0 - ts * segbytes) + a_chunk : kOOB;
    char* dst = stage + b * (MT * SH::ASLOT);
    static_for<MT>([&](auto i) {
      const int j = wave + kNsWaves * i;
      const int mt = j / 4;
      const uint32_t row = static_cast<uint32_t>(16 * mt + 4 * (j % 4)) + a_row;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(dst + mt * SH::ASLOT + (j % 4) * (1024 + 64)),
          16, lo == kOOB ? kOOB : lo + row * segbytes, 0, 0, 0);
    });
  };
  // Operands of one visit.  A: bf16 W -> chunk 4i + grp of each A row
  // (elements 32i + 8grp ..); fp8 W -> chunk 8(i/2) + 2grp + i%2 (elements
  // 64(i/2) + 16grp + 8(i%2) .., the order of the 16 codes a lane reads).  W
  // part i (i = 0..3) of the visit: bf16 its read q[i]; fp8 the low (i even)
  // or high (i odd) eight codes of read q[i/2], widened.  Each accumulator
  // takes parts 0, 1, 2, 3 in that order.
  auto read_a = [&](int b, auto i) {
    const char* src = stage + b * (MT * SH::ASLOT) + rd_a;
    const int c = F8 ? 8 * (i / 2) + 2 * grp + i % 2 : 4 * i + grp;
    static_for<MT>([&](auto m) {
      a[m][i] = *reinterpret_cast<const u32x4_t*>(src + m * SH::ASLOT + ((c ^ rs_a) * 16));
    });
  };
  auto read_w = [&](int slot, u32x4_t (&q)[SH::WSTEPS]) {
    const char* src = ring + slot * SH::SLOT;
    static_for<SH::WSTEPS>([&](auto s) { q[s] = *reinterpret_cast<const u32x4_t*>(src + w_rd[s]); });
  };
  auto mma_part = [&](auto t, auto i, const u32x4_t (&q)[SH::WSTEPS], u32x4_t& lo, u32x4_t& hi) {
    if constexpr (F8) {
      if constexpr (i % 2 == 0) e4m3x16_to_bf16(q[i / 2], lo, hi);
      static_for<MT>([&](auto m) {
        acc[t][m] = mma16(a[m][i], i % 2 == 0 ? lo : hi, acc[t][m], uint16_t());
      });
    } else {
      static_for<MT>([&](auto m) { acc[t][m] = mma16(a[m][i], q[i], acc[t][m], uint16_t()); });
    }
  };
  // a visit with the A operands in registers: its LDS reads; once they are
  // done the slot is refilled (`refill`: the visit R ahead), so those loads are
  // in flight during this visit's MFMAs.  The register ring refills the slot
  // after its MFMAs are issued (their order left to the compiler: scheduling
  // groups as below made it wait for every A read before each MFMA of a
  // block's first visit).
  auto compute = [&](auto t, auto slot, auto&& refill) {
    u32x4_t lo, hi;
    if constexpr (REG) {
      static_for<4>([&](auto i) { mma_part(t, i, wr[slot], lo, hi); });
      refill();
    } else {
      u32x4_t q[SH::WSTEPS];
      read_w(slot, q);
      BDR_WAIT_VM_LGKM(63, 0);
      refill();
      __builtin_amdgcn_sched_barrier(0);
      static_for<4>([&](auto i) { mma_part(t, i, q, lo, hi); });
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * MT, 0);
    }
  };
  // the first visit of a block, which also brings the block's A slice (staging
  // buffer b) into registers: the weight reads and part 0's A reads, the
  // refill, then part i's MFMAs with part i + 1's A reads in flight (at most 15
  // LDS reads can be outstanding)
  auto compute_first = [&](auto t, auto slot, int b, auto&& refill) {
    u32x4_t lo, hi;
    if constexpr (REG) {
      static_for<4>([&](auto i) {
        read_a(b, i);
        mma_part(t, i, wr[slot], lo, hi);
      });
      refill();
    } else {
      u32x4_t q[SH::WSTEPS];
      read_w(slot, q);
      read_a(b, std::integral_constant<int, 0>{});
      BDR_WAIT_VM_LGKM(63, 0);
      refill();
      static_for<4>([&](auto i) {
        if constexpr (i > 0) read_a(b, i);
        mma_part(t, i, q, lo, hi);
        if constexpr (i > 0) __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
      });
    }
  };

  // prologue: A of the first block, then tiles 0 .. R - 1 of pass 0 (ng >= 1)
  dma_a(kb_lo, 0, true);
  static_for<R>([&](auto t) { dma_w(kb_lo * kb_str + t * tile_bytes, t, kb_lo, t); });
  int blk = 0;
  const int nblk = npass * static_cast<int>(kb_hi - kb_lo);
  const int pass_tiles = ng * R;
  uint32_t base = 0;
  int pt = 0;   // first tile of the pass
  for (int p = 0; p < npass; ++p, base += pass_bytes, pt += pass_tiles) {
    for (uint32_t kb = kb_lo; kb < kb_hi; ++kb, ++blk) {
      // this block's A slice has landed once at most R visits are outstanding
      // (R or more followed its loads)
      ns_wait_vm<NI * R>();
      BDR_WG_BARRIER();
      // the next block's A slice first: its segment pointer may come from a
      // scalar load, whose wait would otherwise also wait for this block's A
      // reads
      const bool last_blk = kb + 1 == kb_hi;
      const uint32_t nkb = last_blk ? kb_lo : kb + 1;
      const uint32_t nbase = last_blk ? (p + 1 < npass ? base + pass_bytes : kOOB) : base;
      const int npt = last_blk ? pt + pass_tiles : pt;
      dma_a(nkb, (blk + 1) & 1, blk + 1 < nblk);
      const uint32_t here = base + kb * kb_str;
      const uint32_t next = nbase == kOOB ? kOOB : nbase + nkb * kb_str;
      static_for<NG>([&](auto gc) {
        constexpr int G = decltype(gc)::value;
        if (G < ng) {
          const bool last_g = G + 1 >= ng;
          static_for<R>([&](auto jc) {
            constexpr int J = decltype(jc)::value;
            constexpr int T = G * R + J;
            __builtin_amdgcn_sched_barrier(0);
            // visit T (slot J) has landed: issued R steps back, R - 1 visits
            // followed it, and this block's A loads too while T < R
            ns_wait_vm<NI * (R - 1) + (T < R ? NA : 0)>();
            // The refill writes the slot this step reads: visit T + R, tile
            // (G + 1) R + J of this block or tile J of the next block.  The
            // compiler does not see the buffer-to-LDS write as touching those
            // addresses; it is issued after a wait for this step's LDS reads
            // (an out-of-range load, for an empty slot, lands within a few
            // cycles and would zero the slot under reads still in flight).
            const uint32_t in_blk = here + ((G + 1) * R + J) * tile_bytes;
            const uint32_t nx_blk = next == kOOB ? kOOB : next + J * tile_bytes;
            auto refill = [&]() {
              dma_w(last_g ? nx_blk : in_blk, last_g ? npt + J : pt + (G + 1) * R + J,
                    last_g ? nkb : kb, jc);
            };
            if constexpr (T == 0)
              compute_first(std::integral_constant<int, T>{}, jc, blk & 1, refill);
            else
              compute(std::integral_constant<int, T>{}, jc, refill);
          });
        }
      });
    }
    // pass p complete: store the tiles in this wave's range, then clear.  The
    // stores go through a descriptor over this output (or K split), one 32-bit
    // byte offset per store: rows past M fall beyond its size and are dropped.
    const int nb = n_lo + 16 * ng * R * p + r16;
    static_for<NTW>([&](auto t) {
      const int n = nb + 16 * t;
      if (t < ng * R && n < n_hi) {
        float sc = 1.f;
        if constexpr (F8) sc = g.w_scale[n];
        uint32_t off = o_lane + static_cast<uint32_t>(n) * o_es;
        asm volatile("" : "+v"(off));
        static_for<MT>([&](auto m) {
          static_for<4>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const float v = F8 ? acc[t][m][i] * sc : acc[t][m][i];
            const uint32_t o = off + static_cast<uint32_t>(16 * m + i) * o_row;
            if (o_bf16)
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), ro, o, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ro, o, 0, 0);
          });
        });
      }
    });
    zero_acc();
  }
  BDR_WAIT_VM_LGKM(0, 15);
}


// K splits of one problem: ceil(kblocks / kb_per_split)
__device__ __forceinline__ unsigned ns_splits(const StreamArgs& sa) {
  return static_cast<unsigned>((sa.kblocks + sa.kb_per_split - 1) / sa.kb_per_split);
}

// One-dimensional grid of n_waves x splits workgroups.  Workgroup i takes K
// split i % splits of row range i / splits: consecutive workgroups, which the
// dispatcher spreads over the eight XCDs in turn, take different splits, so
// with eight splits every XCD holds one split's workgroups and the A slice
// they all read stays in that XCD's L2.
template <typename S, int MT, int R, bool REG = false>
__global__ __launch_bounds__(256) void ws_gemm_ns_kernel(const StreamArgs sa) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const unsigned ks = ns_splits(sa);
  ns_lean_body<S, MT, R, REG>(sa, blockIdx.x / ks, blockIdx.x % ks, lds);
}

// Two GEMMs in one launch (the drafter fc beside the LM head): the first n0
// workgroups take problem 0 (row ranges of a0, no K split); the others take
// problem 1, workgroup n0 + i being K split i % splits of row range i / splits.
template <typename S, int MT0, int R0, int MT1, int R1, bool REG = false>
__global__ __launch_bounds__(256) void ws_gemm_ns_pair_kernel(const StreamArgs a0,
                                                              const StreamArgs a1, unsigned n0) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  if (blockIdx.x < n0) {
    ns_lean_body<S, MT0, R0, REG>(a0, blockIdx.x, 0, lds);
  } else {
    const unsigned i = blockIdx.x - n0;
    const unsigned ks = ns_splits(a1);
    ns_lean_body<S, MT1, R1, REG>(a1, i / ks, i % ks, lds);
  }
}

// REG: the register ring (bf16 weights: the packed layout only; fp8 codes:
// row-major)
template <typename S, int MT, int R, bool REG = false>
hipError_t launch_ns_one(const GemmPlan& p, const StreamArgs& sa, hipStream_t st) {
  if (REG && !kIsFp8<S> && sa.g.w_packed == 0) return hipErrorInvalidValue;
  constexpr size_t lds = ns_lean_lds_bytes<S, MT, R, REG>();
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&ws_gemm_ns_kernel<S, MT, R, REG>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid(static_cast<unsigned>(p.n_waves * p.ksplit));
  hipLaunchKernelGGL((ws_gemm_ns_kernel<S, MT, R, REG>), grid, dim3(64 * kNsWaves), lds, st, sa);
  return hipGetLastError();
}

template <typename S, int MT0, int R0, int MT1, int R1, bool REG = false>
hipError_t launch_ns_pair_one(const StreamArgs& a0, const StreamArgs& a1, unsigned n0,
                              unsigned n1, hipStream_t st) {
  if (REG && !kIsFp8<S> && (a0.g.w_packed == 0 || a1.g.w_packed == 0)) return hipErrorInvalidValue;
  constexpr size_t l0 = ns_lean_lds_bytes<S, MT0, R0, REG>();
  constexpr size_t l1 = ns_lean_lds_bytes<S, MT1, R1, REG>();
  constexpr size_t lds = l0 > l1 ? l0 : l1;
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&ws_gemm_ns_pair_kernel<S, MT0, R0, MT1, R1, REG>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((ws_gemm_ns_pair_kernel<S, MT0, R0, MT1, R1, REG>), dim3(n0 + n1),
                     dim3(64 * kNsWaves), lds, st, a0, a1, n0);
  return hipGetLastError();
}

}  // namespace bdr
