// Grouped GEMM tile body for gfx950 (bf16 and MX-scaled fp8 MFMA) and the host-side
// choices of tile shape, K-start rotation and cache policy.  Included by gemm.hip (the
// grouped-GEMM kernels) and fused.hip (the single-launch forward), which run the same
// body per workgroup tile.
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {

// ============================================================ bf16 / MX MFMA GEMM
// Workgroup tile BM x BN, K staged in KB-byte row slices (KB = 128: 64 bf16 or
// 128 fp8; KB = 64: 32 bf16) through an S-stage LDS ring.  WM x WN waves (4, 8 or
// 16); each wave owns FM x FN 32x32 fragments.
//
// SWIGLU: the B tile stacks BN/2 rows of W_gate over the same BN/2 rows of
// W_up, and every wave holds matching gate and up fragments, so the epilogue
// forms h = silu(a) * u in registers.
//
// LDS serves a 128-bit read 16 lanes (256 bytes) at a time; a fragment read has
// lanes 0..15 on 16 consecutive rows at the same logical 16-byte chunk.  The
// chunks of a row are XOR-swizzled so that those 16 reads hit 16 distinct 16-byte
// bank groups of the 256-byte bank line: by ((row >> 1) & 7) for 128-byte rows
// (two rows per bank line), by ((row >> 2) & 3) for 64-byte rows (four rows per
// bank line).  The bank-conflict counter reads zero for both.
template <int KB>
__device__ __forceinline__ int swz(int r, int c) {
  static_assert(KB == 128 || KB == 64, "row slice");
  if constexpr (KB == 128) return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
  else return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}

struct GemmArgs {
  const uint8_t* A;        // ring rows [C, K] (bf16 or E4M3)
  const uint8_t* A_scale;  // MX: [C, K/32]
  const uint8_t* B0;       // [E, N, K]: W_gate (SWIGLU) or W_down
  const uint8_t* B1;       // SWIGLU: W_up [E, N, K]
  const uint8_t* B0_scale; // MX: [E, N, K/32]
  const uint8_t* B1_scale;
  int K;                   // reduction length (elements)
  int N;                   // SWIGLU: f (per half); else output width
  const int32_t* offset;
  const int32_t* tiles;
  const int32_t* ntiles;
  int64_t head, C;
  uint8_t* out;            // SWIGLU: H (bf16 [C, f], or MX codes [C, f]); else ring_y bf16 [C, N]
  uint8_t* out_scale;      // SWIGLU + MX: H scales [C, f/32]
  uint16_t* saved_au;      // SWIGLU + bf16: [C, 2f] or null
  int rotate;              // 1: tile L starts its K loop at step L mod (K steps), see kstart_rotates
  int64_t a_rows, b_rows;  // MX: rows of the A scale tensor (C) and of each B scale tensor (E N);
                           // scale layout [K / 128][rows][4 bytes]
};

// Tile order.  The grid is 1-D; workgroup b runs on XCD b % 8 (round-robin
// dispatch).  Logical tile L = (row tile, column tile), column tiles fastest,
// is given to XCD x as one contiguous range of ceil(V / 8) tiles, V the number
// of live tiles read on the device: all column tiles of one expert's row tile
// then share the token rows through one XCD's L2.
__device__ __forceinline__ bool xcd_tile(int b, int nt_cols, int ntiles, int& mt, int& ct) {
  const int V = ntiles * nt_cols;
  const int per = (V + 7) / 8;
  const int li = b >> 3, x = b & 7;
  if (li >= per) return false;
  const int L = x * per + li;
  if (L >= V) return false;
  mt = L / nt_cols;
  ct = L - mt * nt_cols;
  return true;
}

// Global -> LDS copies of 16 (or 4) bytes per lane, issued from asm so that the
// compiler does not wait for them: the kernel places its own vmcnt waits.  The
// wave's 64 lanes write one contiguous run of LDS at m0 (+ lane * size).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
// The same copy with the non-temporal cache policy (see gemm_policy).
__device__ __forceinline__ void dma16nt(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Stage layout in LDS: A tile [BM][KB] | B tile [BN][KB] | MX: A scale dwords [BM] |
// B scale dwords [BN] | padding.  The scale dwords arrive in whole-wave copies of 64 rows
// each (BM / 64 for A, then BN / 64 for B); the count is padded to a multiple of the
// wave count with clamped duplicates written past the B dwords, so that every wave
// issues the same copies.  S stages form a ring.
template <int BM, int BN, int KB, bool MX, int NW>
struct StageLayout {
  static constexpr int NSC = MX ? (BM / 64 + BN / 64 + NW - 1) / NW : 0;   // scale copies per wave
  static constexpr int A = 0;
  static constexpr int B = BM * KB;
  static constexpr int ASC = B + BN * KB;
  static constexpr int BSC = ASC + (MX ? BM * 4 : 0);
  static constexpr int SIZE = ASC + NSC * NW * 256;
};

// Epilogue staging in LDS: the output tile row-major, OUTC columns of OEB bytes,
// rows padded by 16 bytes (the two row groups a fragment store touches then fall on
// different banks).  CPR 16-byte pieces per row.
template <int BM, int BN, bool SWIGLU, bool MX>
struct EpiLayout {
  static constexpr int OUTC = SWIGLU ? BN / 2 : BN;
  static constexpr int OEB = (SWIGLU && MX) ? 1 : 2;
  static constexpr int RS = OUTC * OEB + 16;
  static constexpr int CPR = OUTC * OEB / 16;
  static constexpr int SIZE = BM * RS;
};

// POL: bit 0 = weight (B) copies with the non-temporal policy, bit 1 = output rows
// stored with the non-temporal policy (see gemm_policy).
//
// The body of one workgroup's tile: vb is the workgroup's place in the 1-D grid (its
// XCD is vb % 8), lds the dynamic LDS of the stage ring.  The kernel below runs it once
// per workgroup; the single-launch forward runs it for a sequence of vb per workgroup.
// F32OUT (not SWIGLU): the output rows are fp32 [C, N], stored from the accumulators.
// MXSAVE (SWIGLU + MX): also write the saved A|U planes (bf16 takes them whenever
// p.saved_au is set; the MX tiles have no registers to spare for that choice at run time:
// the accumulators would stay live across the extra planes and spill).
template <int BM, int BN, int WM, int WN, int KB, bool SWIGLU, bool MX, int S, int POL,
          bool F32OUT = false, bool MXSAVE = false>
__device__ __forceinline__ void gg_mfma_body(const GemmArgs p, int vb, uint8_t* lds) {
  constexpr int EB = MX ? 1 : 2;                 // element bytes
  constexpr int WTM = BM / WM, WTN = BN / WN;    // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CH = KB / 16;                    // 16-byte chunks per row slice
  constexpr int RPC = 64 / CH;                   // rows per 1 KB copy
  constexpr int NW = WM * WN, NT = NW * 64;      // waves, threads
  using SL = StageLayout<BM, BN, KB, MX, NW>;
  constexpr int NA = BM * KB / (NW * 1024), NB = BN * KB / (NW * 1024);   // 1 KB copies per wave
  // MX scale copies: copy k of the tile (wave k mod NW) brings 64 rows' dwords, A rows
  // for k < SCA, then B rows.  Per stage that is BM / 64 + BN / 64 whole-wave copies
  // (one per wave in both tile shapes) where a copy of A and of B rows per wave took
  // twice as many: 2,048-token MX gate/up | down 1.486 | 0.746 ms with them, 1.425 |
  // 0.703 ms with no scale copies at all (a timing probe).
  constexpr int SCA = MX ? BM / 64 : 0, SCB = MX ? BN / 64 : 0;
  constexpr int NSC = SL::NSC;
  constexpr int L = NA + NB + NSC;               // copies per wave per stage
  static_assert(BM * KB % (NW * 1024) == 0 && BN * KB % (NW * 1024) == 0, "tile / wave mismatch");
  static_assert(!MX || KB == 128, "MX stages hold whole 128-element scale groups");
  static_assert(NW == 4 || NW == 8 || (NW == 16 && !MX), "four or eight waves, sixteen without scales");
  static_assert(!MX || (BM % 64 == 0 && BN % 64 == 0), "scale copies of 64 rows");
  static_assert(!SWIGLU || (FN % 2 == 0), "gate/up fragments come in pairs");
  static_assert(S >= 2 && S <= 4, "stages");

  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

  const int nt_cols = SWIGLU ? (p.N + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  int mt, ct;
  // The tile's coordinates are uniform over the workgroup.  Where the kernel itself wrote
  // the tile list and offsets before (the single-launch forward) they arrive through
  // vector loads; readfirstlane keeps them, and every address derived from them, in
  // scalar registers (the copies below take their base address from one).
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  if (!xcd_tile(uni(vb), nt_cols, uni(*p.ntiles), mt, ct)) return;
  const int e = uni(p.tiles[2 * mt]);
  const int row0 = uni(p.tiles[2 * mt + 1]);
  const int32_t seg = uni(p.offset[e]);
  const int rows = min(BM, uni(p.offset[e + 1]) - seg - row0);
  const int n0 = ct * (SWIGLU ? BN / 2 : BN);   // first output column

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t Kb = (uint32_t)p.K * EB;                 // row bytes


  // Copy i of this wave fills 16-byte chunks j = (NW i + wave) * 64 + lane of a tile:
  // row j / CH, slot j % CH, which holds the global chunk whose swizzled slot it is
  // (the swizzle is an involution on the chunk index: swz(r, c) - r * KB = 16 * slot).
  uint32_t a_off[NA], b_off[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int j = (NW * i + wave) * 64 + lane, r = j / CH;
    const int c = (swz<KB>(r, j % CH) - r * KB) >> 4;
    const int64_t sl = ring_slot(p.head, seg, row0 + min(r, rows - 1), p.C);
    a_off[i] = (uint32_t)sl * Kb + c * 16;
  }
  // B rows: SWIGLU stacks BN/2 rows of W_gate over BN/2 rows of W_up; a copy covers
  // RPC rows, so each copy reads from a single matrix (decided by its first row).
  const uint8_t* b_base[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int j = (NW * i + wave) * 64 + lane, r = j / CH;
    const int c = (swz<KB>(r, j % CH) - r * KB) >> 4;
    const bool up = SWIGLU && (NW * i + wave) * RPC >= BN / 2;
    const int rr = up ? r - BN / 2 : r;
    b_base[i] = (up ? p.B1 : p.B0) + (int64_t)e * p.N * Kb;
    b_off[i] = (uint32_t)min(n0 + rr, p.N - 1) * Kb + c * 16;
  }
  uint32_t sc_off[NSC > 0 ? NSC : 1];
  const uint8_t* sc_base[NSC > 0 ? NSC : 1];
  int64_t sc_rows[NSC > 0 ? NSC : 1];           // rows of the [K/128][rows][4] scale array
  if (MX) {
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
      const int k = NW * i + wave;              // the tile's scale copy k (wave-uniform)
      if (k < SCA) {
        const int r = 64 * k + lane;
        sc_base[i] = p.A_scale;
        sc_rows[i] = p.a_rows;
        sc_off[i] = (uint32_t)ring_slot(p.head, seg, row0 + min(r, rows - 1), p.C) * 4;
      } else {
        const int kb = k < SCA + SCB ? k - SCA : 0;   // padding copies repeat B copy 0
        const int r = 64 * kb + lane;
        const bool up = SWIGLU && 64 * kb >= BN / 2;
        const int rr = up ? r - BN / 2 : r;
        sc_base[i] = (up ? p.B1_scale : p.B0_scale) + (int64_t)e * p.N * 4;
        sc_rows[i] = p.b_rows;
        sc_off[i] = (uint32_t)min(n0 + rr, p.N - 1) * 4;
      }
    }
  }
  // K steps are taken in the order s0, s0 + 1, ..., KT - 1, 0, ..., s0 - 1: with
  // rotation, tiles that run at the same time read different K slices of their
  // weight rows (a fixed order per tile, so results stay deterministic).
  const int KT = (int)(Kb / KB);
  const int s0 = p.rotate ? (int)(((int64_t)mt * nt_cols + ct) % KT) : 0;
  // Copy c (0 <= c < L) of this wave for the i-th K step of the loop, into ring
  // buffer i % S.
  auto issue_one = [&](int i_, int c) __attribute__((always_inline)) {
    const uint32_t st = lds0 + (uint32_t)(i_ % S) * SL::SIZE;
    const int kt = i_ + s0 >= KT ? i_ + s0 - KT : i_ + s0;
    if (c < NA) {
      dma16(p.A + (size_t)kt * KB, a_off[c], __builtin_amdgcn_readfirstlane(st + SL::A + (NW * c + wave) * 1024));
    } else if (c < NA + NB) {
      const int i = c - NA;
      if (POL & 1) dma16nt(b_base[i] + (size_t)kt * KB, b_off[i], __builtin_amdgcn_readfirstlane(st + SL::B + (NW * i + wave) * 1024));
      else dma16(b_base[i] + (size_t)kt * KB, b_off[i], __builtin_amdgcn_readfirstlane(st + SL::B + (NW * i + wave) * 1024));
    } else {
      const int i = c - NA - NB;
      dma4(sc_base[i] + (size_t)kt * sc_rows[i] * 4, sc_off[i],
           __builtin_amdgcn_readfirstlane(st + SL::ASC + (NW * i + wave) * 256));
    }
  };
  auto issue = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < L; ++c) issue_one(kt, c);
  };
  // wait until this wave's copies of the stage issued `later` stages before the
  // newest one have landed
  auto wait_stage = [&](int later) __attribute__((always_inline)) {
    if (later <= 0) wait_vm<0>();
    else if (later == 1) wait_vm<L>();
    else if (later == 2) wait_vm<2 * L>();
    else wait_vm<3 * L>();
  };

  // B fragment row (inside the B tile) of fragment fn
  auto brow = [&](int fn) {
    if (SWIGLU) {
      constexpr int HALF = FN / 2;
      const int j = fn % HALF;
      return (fn < HALF ? 0 : BN / 2) + wn * (WTN / 2) + j * 32;
    }
    return wn * WTN + fn * 32;
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lr = lane & 31, lg = lane >> 5;
  // One stage: KK sub-steps of FM x FN MFMAs.  The schedule is fixed by hand (the
  // compiler would otherwise group all memory instructions at the start): the
  // fragments of sub-step kk + 1 are read between the MFMAs of sub-step kk, and the
  // L copies of the stage `next` (the one that will be computed S - 1 stages later;
  // negative for none) are spread evenly over all MFMAs of the stage.  A wave
  // issues in order, so a copy placed after an MFMA is handed to the memory
  // pipeline while the MFMA executes instead of before all of them.
  constexpr int KK = MX ? KB / 128 * 2 : KB / 32;   // sub-steps per stage
  constexpr int NMF = KK * FM * FN;                  // MFMAs per stage
  // Fragments of sub-step kk + 1 are read into the second register set during the
  // MFMAs of sub-step kk, except for MX waves of 64 x 128 (eight waves in 256 x 256),
  // whose two register sets would not fit beside the accumulators: there each sub-step
  // reads its own fragments first and the SIMD's other wave covers the LDS latency.
  constexpr bool PF = !(MX && NW == 8 && FM * FN >= 8);
  using Frag = std::conditional_t<MX, i32x8, bf16x8>;
  Frag af[2][FM], bfr[2][FN];
  int sa[2][FM], sb[2][FN];
  auto stage_ptrs = [&](int buf, const uint8_t*& as, const uint8_t*& bs, const uint32_t*& asc,
                        const uint32_t*& bsc) __attribute__((always_inline)) {
    as = lds + buf * SL::SIZE + SL::A;
    bs = lds + buf * SL::SIZE + SL::B;
    asc = (const uint32_t*)(lds + buf * SL::SIZE + SL::ASC);
    bsc = (const uint32_t*)(lds + buf * SL::SIZE + SL::BSC);
  };
  // fragment q of sub-step kk of ring buffer buf into register set `set`: q < FM is
  // A fragment q, else B fragment q - FM
  auto read = [&](int buf, int kk, int q, int set, auto nl) __attribute__((always_inline)) {
    constexpr int NL = decltype(nl)::value;
    if (q < FM ? q >= NL : NL == 0) return;   // a fragment of rows past the tile's end
    const uint8_t *as, *bs;
    const uint32_t *asc, *bsc;
    stage_ptrs(buf, as, bs, asc, bsc);
    const bool isa = q < FM;
    const int r = isa ? wm * WTM + q * 32 + lr : brow(q - FM) + lr;
    const uint8_t* base = isa ? as : bs;
    if constexpr (!MX) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, *(const u32x4*)(base + swz<KB>(r, kk * 2 + lg)));
      if (isa) af[set][q] = v; else bfr[set][q - FM] = v;
    } else {
      // Operand layout of the 32x32x64 E4M3 MFMA: of a lane's 32 bytes, bytes
      // 0-15 belong to the first 32-element scale block of the 64-wide K step and
      // bytes 16-31 to the second; lane group g (= lane / 32) holds elements
      // [16g, 16g + 16) of each block and supplies the scale of block g.
      const int ca = kk * 4 + lg, cb = kk * 4 + 2 + lg;
      const int blk = kk * 2 + lg;             // its scale byte inside the row's dword
      const u32x4 lo = *(const u32x4*)(base + swz<KB>(r, ca));
      const u32x4 hi = *(const u32x4*)(base + swz<KB>(r, cb));
      const i32x8 v = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      const int ri = r;                          // row r's dword (A rows and B rows alike)
      const int sc = (int)(((isa ? asc : bsc)[ri] >> (8 * blk)) & 0xffu);
      if (isa) { af[set][q] = v; sa[set][q] = sc; }
      else { bfr[set][q - FM] = v; sb[set][q - FM] = sc; }
    }
  };
  // The FM x FN MFMAs of one sub-step on register set `set`, with interleaved work:
  // the FM + FN fragment reads of (rbuf, rkk) into set ^ 1 (rbuf < 0: none), and the
  // copies [c0, c1) of K step `next` (next < 0: none) spread evenly.
  auto substep = [&](int set, int rbuf, int rkk, int next, int c0, int c1, auto nl)
      __attribute__((always_inline)) {
    constexpr int NL = decltype(nl)::value;
#pragma unroll
    for (int m = 0; m < FM * FN; ++m) {
      const int i = m / FN, j = m % FN;
      if (i < NL) {
        if constexpr (!MX)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[set][i], bfr[set][j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[set][i], bfr[set][j], acc[i][j], 0, 0, 0, sa[set][i], 0, sb[set][j]);
      }
      if (rbuf >= 0 && m < FM + FN) read(rbuf, rkk, m, set ^ 1, nl);
#pragma unroll
      for (int c = c0; c < c1; ++c)   // copy c goes after MFMA number floor((c - c0) * FM * FN / (c1 - c0))
        if ((c - c0) * FM * FN / (c1 - c0) == m && next >= 0) issue_one(next, c);
      __builtin_amdgcn_sched_barrier(0);
    }
    // fewer MFMAs than fragments (a 32-row wave tile): read the rest after them
#pragma unroll
    for (int q = FM * FN; q < FM + FN; ++q)
      if (rbuf >= 0) read(rbuf, rkk, q, set ^ 1, nl);
  };

  // Without prefetch (MX, eight waves): fragment rows start at multiples of 32, so the
  // swizzled offset of row rowc + lr, 16-byte chunk 4 kk + 2 h + lg is
  // rowc * 128 + (l0 ^ ((4 kk + 2 h) << 4)) with the per-lane
  // l0 = lr * 128 + ((lg ^ ((lr >> 1) & 7)) << 4), and a row's scale dword sits at a
  // wave-uniform offset + 4 lr.  Both per-lane values pass through an empty asm once
  // per stage, so the compiler cannot hoist one address per fragment out of the K loop
  // (those addresses spilled, and each reload waited for every copy in flight).
  auto read_np = [&](int buf, int kk, int q, uint32_t l0, uint32_t l4, auto nl)
      __attribute__((always_inline)) {
    static_assert(PF || KB == 128, "fragment addressing");
    constexpr int NL = decltype(nl)::value;
    if (q < FM ? q >= NL : NL == 0) return;
    const uint8_t* st = lds + buf * SL::SIZE;
    const bool isa = q < FM;
    const int rowc = isa ? wm * WTM + q * 32 : brow(q - FM);
    const uint8_t* base = st + (isa ? SL::A : SL::B) + rowc * KB;
    if constexpr (MX) {
      const u32x4 lo = *(const u32x4*)(base + (l0 ^ ((kk * 4) << 4)));
      const u32x4 hi = *(const u32x4*)(base + (l0 ^ ((kk * 4 + 2) << 4)));
      const i32x8 v = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      const uint32_t w = *(const uint32_t*)(st + (isa ? SL::ASC : SL::BSC) + rowc * 4 + l4);
      const int sc = (int)((w >> (8 * (kk * 2 + lg))) & 0xffu);
      if (isa) { af[0][q] = v; sa[0][q] = sc; }
      else { bfr[0][q - FM] = v; sb[0][q - FM] = sc; }
    } else {
      read(buf, kk, q, 0, nl);
    }
  };
  const uint32_t l0_lane = (uint32_t)(lr * KB + ((lg ^ ((lr >> 1) & 7)) << 4)), l4_lane = (uint32_t)lr * 4;
  // Without prefetch: the FM A fragments of sub-step kk, then per B fragment j its read
  // followed by its FM MFMAs (one B fragment live at a time); copies spread as above.
  auto substep_np = [&](int buf, int kk, int next, int c0, int c1, uint32_t l0, uint32_t l4,
                        auto nl) __attribute__((always_inline)) {
    constexpr int NL = decltype(nl)::value;
#pragma unroll
    for (int q = 0; q < FM; ++q) read_np(buf, kk, q, l0, l4, nl);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      read_np(buf, kk, FM + j, l0, l4, nl);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = j * FM + i;
        if (i < NL) {
          if constexpr (!MX)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0][i], bfr[0][j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[0][i], bfr[0][j], acc[i][j], 0, 0, 0, sa[0][i], 0, sb[0][j]);
        }
#pragma unroll
        for (int c = c0; c < c1; ++c)
          if ((c - c0) * FM * FN / (c1 - c0) == m && next >= 0) issue_one(next, c);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // S-stage ring: stages kt+1 .. kt+S-1 stream in while stage kt is computed.
  // One barrier per stage: it publishes stage kt (every wave waited for its own
  // copies) and retires the buffer of stage kt-1, which the copies of stage kt+S-1
  // then overwrite.
  // The wave's A fragments wholly past the tile's last row (a segment's ragged last
  // tile) take no MFMAs and no fragment reads; the wave still makes its share of the
  // copies and meets every barrier.  Rows below `rows` get the same MFMAs in the same
  // order either way.  Measured in one process pair on one GPU, forward per call:
  // 2,048 tokens bf16 3.873 -> 3.719 ms, MXFP8 2.395 -> 2.306 ms, skewed 8,192 tokens
  // 4.05 -> 3.94 ms.
  const int nlive = min(FM, max(0, (rows - wm * WTM + 31) / 32));
  auto kloop = [&](auto nl) __attribute__((always_inline)) {
  if constexpr (S < 4) {
    // Barrier at the start of each stage; the stage's copies (K step kt + S - 1)
    // spread over all its MFMAs.
    for (int kt = 0; kt < KT; ++kt) {
      wait_stage(min(S - 2, KT - 1 - kt));
      __syncthreads();
      const int buf = kt % S, next = kt + S - 1 < KT ? kt + S - 1 : -1;
      if constexpr (PF) {
#pragma unroll
        for (int q = 0; q < FM + FN; ++q) read(buf, 0, q, 0, nl);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          substep(kk & 1, kk + 1 < KK ? buf : -1, kk + 1, next, kk * L / KK, (kk + 1) * L / KK, nl);
      } else {
        uint32_t l0 = l0_lane, l4 = l4_lane;
        asm volatile("" : "+v"(l0), "+v"(l4));
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          substep_np(buf, kk, next, kk * L / KK, (kk + 1) * L / KK, l0, l4, nl);
      }
    }
  } else {
    // Barrier before the last sub-step of each stage: the next stage is waited for
    // and published there, so its first fragments are read while the last MFMAs of
    // this stage run (no exposed LDS latency at stage starts), and the buffer it
    // frees (stage kt - 1, finished by every wave) takes the copies of K step
    // kt + S - 1 during that last sub-step.
    static_assert(KK % 2 == 0, "sub-step 0 of every stage uses register set 0");
    wait_stage(min(S - 2, KT - 1));
    __syncthreads();
#pragma unroll
    for (int q = 0; q < FM + FN; ++q) read(0, 0, q, 0, nl);
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt % S;
#pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk) substep(kk & 1, buf, kk + 1, -1, 0, 0, nl);
      const bool more = kt + 1 < KT;
      if (more) {
        wait_stage(min(kt + S - 2, KT - 1) - (kt + 1));
        __syncthreads();
      }
      substep((KK - 1) & 1, more ? (kt + 1) % S : -1, 0, kt + S - 1 < KT ? kt + S - 1 : -1, 0, L,
              nl);
    }
  }
  };
  for (int s = 0; s < S - 1 && s < KT; ++s) issue(s);
  static_assert(FM == 2, "three loop forms: 2, 1 or 0 live A fragments");
  if (nlive == FM) kloop(std::integral_constant<int, FM>{});
  else if (nlive == 1) kloop(std::integral_constant<int, 1>{});
  else kloop(std::integral_constant<int, 0>{});
  __syncthreads();

  // ---------------------------------------------------------------- epilogue
  // acc register r of a 32x32 fragment: row 8*(r/4) + 4*(lane/32) + r%4, column lane%32.
  // The output tile is staged row-major in LDS (the ring is idle now: every copy has
  // landed and the barrier below retires the last reads) and written out as whole
  // 16-byte pieces of rows, instead of 2-byte stores scattered over rows.
  using EL = EpiLayout<BM, BN, SWIGLU, MX>;
  uint8_t* stg = lds;
  __syncthreads();
  // Copy the staged plane to dst (row pitch `pitch` bytes, tile columns from byte
  // col0b); rows beyond the segment and columns beyond N are not written.
  // RS, CPR: the staged row stride and 16-byte pieces per row (the layout of EL, or of
  // bf16 planes beside an MX epilogue)
  auto flush_as = [&](uint8_t* dst, int64_t pitch, int col0b, int rowb, int RS, int CPR)
      __attribute__((always_inline)) {
    __syncthreads();
#pragma unroll 4
    for (int q = tid; q < BM * CPR; q += NT) {
      const int m = q / CPR, cb = (q % CPR) * 16;
      if (m < rows && col0b + cb < rowb) {
        const int64_t sl = ring_slot(p.head, seg, row0 + m, p.C);
        const u32x4 v = *(const u32x4*)(stg + m * RS + cb);
        if (POL & 2) __builtin_nontemporal_store(v, (u32x4*)(dst + sl * pitch + col0b + cb));
        else *(u32x4*)(dst + sl * pitch + col0b + cb) = v;
      }
    }
    __syncthreads();
  };
  auto flush = [&](uint8_t* dst, int64_t pitch, int col0b, int rowb) __attribute__((always_inline)) {
    flush_as(dst, pitch, col0b, rowb, EL::RS, EL::CPR);
  };
  if constexpr (SWIGLU) {
    constexpr int HALF = FN / 2;
    // plane 0: h = silu(a) * u (bf16, or E4M3 codes with per-32 scales); with saved
    // A|U, planes 1 and 2 hold a and u in bf16 (also beside MX codes: the MXFP8 backward
    // reads them like the bf16 one), staged with a bf16 row stride
    constexpr int RS16 = (BN / 2) * 2 + 16, CPR16 = (BN / 2) * 2 / 16;
    static_assert(!SWIGLU || BM * RS16 <= S * SL::SIZE, "bf16 planes fit the stage ring");
    // MX h plane: the 16 block exponents of each (fragment pair, half-wave), handed from
    // the lanes that computed them to every lane of the half-wave through LDS past the
    // staged planes
    constexpr int XOFF = ((EL::SIZE > BM * RS16 ? EL::SIZE : BM * RS16) + 255) / 256 * 256;
    static_assert(!MX || XOFF + NW * FM * HALF * 2 * 16 <= S * SL::SIZE, "exponent bytes fit the ring");
    auto stage_plane = [&](auto plane_tag) __attribute__((always_inline)) {
      constexpr int plane = decltype(plane_tag)::value;
      // beside MX codes the lane's row and column are re-derived per plane, so that no
      // plane's addresses stay live across the others
      int plr = lr, plg = lg;
      if constexpr (MX && MXSAVE) asm volatile("" : "+v"(plr), "+v"(plg));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
          const int cl = wn * (WTN / 2) + j * 32 + plr;   // column inside the tile
          if constexpr (MX && plane == 0) {
            // The 32 columns of a row's block sit in the 32 lanes of a half-wave, and a
            // lane holds 16 rows (r).  Halving exchanges give each lane the block maximum
            // of one row: with partners lane ^ 16 (permlane16 swap), ^ 15 (row mirror),
            // ^ 7 (half-row mirror), ^ 2 and ^ 1 (quad permutations), each step keeps
            // half of the rows still held and takes the partner's values of the same rows;
            // lane l ends with row rr = 8 b4 + 4 b3 + 2 b2 + b1 (bits of l mod 32).  That
            // is 8 + 4 + 2 + 1 + 1 cross-lane moves for the 16 rows instead of 5 per row,
            // one block exponent per row instead of one per value, and one store
            // instruction for 16 rows' scale bytes.  Maxima are exact in any order: the
            // same codes and scales as a per-row reduction.
            float hv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) hv[r] = silu(acc[i][j][r]) * acc[i][j + HALF][r];
            auto dpp = [](float v, auto ctrl) __attribute__((always_inline)) {
              return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
            };
            float t8[8], t4[4], t2[2];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_int(fabsf(hv[q])),
                                                               __float_as_int(fabsf(hv[q + 8])), false, false);
              t8[q] = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
            }
            const bool b3 = plr & 8, b2 = plr & 4, b1 = plr & 2;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              t4[q] = fmaxf(b3 ? t8[q + 4] : t8[q], dpp(b3 ? t8[q] : t8[q + 4], std::integral_constant<int, 0x140>{}));
#pragma unroll
            for (int q = 0; q < 2; ++q)
              t2[q] = fmaxf(b2 ? t4[q + 2] : t4[q], dpp(b2 ? t4[q] : t4[q + 2], std::integral_constant<int, 0x141>{}));
            float t1 = fmaxf(b1 ? t2[1] : t2[0], dpp(b1 ? t2[0] : t2[1], std::integral_constant<int, 0x4E>{}));
            t1 = fmaxf(t1, dpp(t1, std::integral_constant<int, 0xB1>{}));
            const int X = mx_block_exp(t1);
            const int rr = ((plr >> 4) & 1) * 8 + ((plr >> 3) & 1) * 4 + ((plr >> 2) & 1) * 2 + ((plr >> 1) & 1);
            uint8_t* xb = lds + XOFF + (((wave * FM + i) * HALF + j) * 2 + plg) * 16;
            if ((plr & 1) == 0) {
              xb[rr] = (uint8_t)(X + 127);
              const int m = wm * WTM + i * 32 + 8 * (rr / 4) + 4 * plg + (rr % 4);
              const int col = n0 + wn * (WTN / 2) + j * 32;   // the block's first column
              if (m < rows && col < p.N)
                p.out_scale[((int64_t)(col / 128) * p.C + ring_slot(p.head, seg, row0 + m, p.C)) * 4 +
                            (col / 32) % 4] = (uint8_t)(X + 127);
            }
            const u32x4 xw = *(const u32x4*)xb;   // the half-wave's 16 exponents (one wave: in order)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = wm * WTM + i * 32 + 8 * (r / 4) + 4 * plg + (r % 4);
              const int Xr = (int)((xw[r / 4] >> (8 * (r % 4))) & 0xffu) - 127;
              stg[m * EL::RS + cl] = (uint8_t)e4m3_encode(hv[r], Xr);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = wm * WTM + i * 32 + 8 * (r / 4) + 4 * plg + (r % 4);
              const float a = acc[i][j][r], u = acc[i][j + HALF][r];
              const float v = plane == 0 ? silu(a) * u : plane == 1 ? a : u;
              *(uint16_t*)(stg + m * (MX ? RS16 : EL::RS) + cl * 2) = f2bf(v);
            }
          }
        }
      if constexpr (plane == 0) flush(p.out, (int64_t)p.N * EL::OEB, n0 * EL::OEB, p.N * EL::OEB);
      else flush_as((uint8_t*)p.saved_au + (plane == 2 ? (int64_t)p.N * 2 : 0), (int64_t)p.N * 4,
                    n0 * 2, p.N * 2, MX ? RS16 : EL::RS, MX ? CPR16 : EL::CPR);
    };
    if constexpr (MX) {
      // the h plane last: it is the accumulators' final use, so its block reductions run
      // as the accumulators die
      if constexpr (MXSAVE) {
        stage_plane(std::integral_constant<int, 1>{});
        stage_plane(std::integral_constant<int, 2>{});
      }
      stage_plane(std::integral_constant<int, 0>{});
    } else {
      stage_plane(std::integral_constant<int, 0>{});
      if (p.saved_au) {
        stage_plane(std::integral_constant<int, 1>{});
        stage_plane(std::integral_constant<int, 2>{});
      }
    }
  } else if constexpr (F32OUT) {
    // 32 lanes store 32 consecutive columns of one row: 128-byte pieces
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * WTM + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        if (m < rows) {
          float* orow = (float*)p.out + ring_slot(p.head, seg, row0 + m, p.C) * p.N;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WTN + j * 32 + lr;
            if (col < p.N) orow[col] = acc[i][j][r];
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cl = wn * WTN + j * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * WTM + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
          *(uint16_t*)(stg + m * EL::RS + cl * 2) = f2bf(acc[i][j][r]);
        }
      }
    flush(p.out, (int64_t)p.N * 2, n0 * 2, p.N * 2);
  }
}

// Two MFMA tile shapes (bf16 and MX alike).
//  * 128 x 256, 128-byte K slices, 3 stages, eight waves of 64 x 64: one row tile
//    holds every row of an expert with up to 128 rows, so each weight is read from
//    HBM once; the 2,048-token layer (64 rows per expert on average) is bound by that
//    stream.  Eight waves (two per SIMD) instead of four of 64 x 128: while one wave
//    waits at a stage barrier or on its copies the other's MFMAs run (2,048 tokens,
//    gate/up | down in ms: bf16 2.547 | 1.309 -> 2.532 | 1.257, MX 1.652 | 0.800 ->
//    1.491 | 0.755; skewed 8,192 tokens bf16 2.153 | 1.446 -> 2.111 | 1.320).
//  * 256 x 256, 128-byte K slices, 2 stages (128 KB), sixteen waves of 64 x 64 for
//    bf16 (four per SIMD, so that one wave's MFMAs run while the others wait; eight
//    waves of 64 x 128 measured 1.534 ms against 1.514 at the per-GPU share; in the
//    128 x 256 tile sixteen waves of 32 x 64 were slower: down GEMM 1.277 -> 1.353 ms
//    at 2,048 tokens), eight
//    waves of 64 x 128 for MX: with many rows per expert every row tile re-reads the
//    weights and the kernel is bound inside the CU, by the rate at which L2 serves
//    the stages.  Whole 128-byte
//    lines per copy and one barrier per 64 K measured ~2 % faster than 64-byte
//    slices in 4 stages.  Per 64-wide K stage a SIMD runs 64 MFMAs (2048 clocks)
//    while LDS serves 192 KB of fragment reads and 64 KB of copies (1024 clocks at
//    256 B/clock).
// MX takes the same two shapes, with 128 K elements per stage.  In the 256 x 256 tile
// its operand fragments (twice the bf16 size) are not prefetched into a second register
// set; the fragments of a sub-step are read just before its MFMAs.  Per-GPU share
// (4 experts, 16,384 rows), MXFP8 gate/up | down in ms, 128 x 256 -> 256 x 256:
// 0.827 -> 0.585 | 0.391 -> 0.290.
constexpr int MFMA_BM = 128, MFMA_BM_BIG = 256;
constexpr int BIG_ROWS_MIN = 256;   // mean rows per expert from which the 256-row tile is used

inline bool use_big(int dtype, int64_t n, int E) {
  return (dtype == 1 || dtype == 2) && n >= (int64_t)BIG_ROWS_MIN * E;
}

// Rotation of the K loop's starting step per tile (measured on gfx950, gate/up | down
// GEMM in ms without -> with):
//  * many row tiles per expert (the per-GPU share shapes, where every weight panel is
//    re-read by each row tile and the stage rate through L2 bounds the kernel): tiles
//    that run together read different K slices, bf16 1.042 -> 1.007 | 0.503 -> 0.503,
//    MX 0.923 -> 0.873 | 0.435 -> 0.423;
//  * the bf16 down GEMM with one row tile per expert: a tile's copies of one K step
//    read 128 bytes from each of 256 weight rows 4 KB (2 KB) apart, all at the same
//    offset inside a 4 KB page, which crowds them onto a subset of the HBM channels;
//    rotation spreads them: 2,048 tokens 1.504 -> 1.421, skewed 8,192 tokens 1.517 ->
//    1.484 (a bare copy of that pattern: 5.4 -> 6.1 TB/s);
//  * the gate/up GEMM with one row tile per expert loses (2.582 -> 2.605 at 2,048 tokens,
//    2.218 -> 2.298 skewed): the column tiles of a row tile then no longer read the same
//    token-row slices at the same time, so those rows are held in L2 longer; the MX
//    down GEMM there is unchanged within noise (0.907 -> 0.918), so it is not rotated.
// Re-measured with the eight-wave 128 x 256 tile (2,048 tokens, without -> with): bf16
// down 1.472 -> 1.279, gate/up 2.307 -> 2.336; MX down 0.733 -> 0.756; the rules stand.
inline int kstart_rotates(bool swiglu, int dtype, int64_t n, int E, int BM) {
  if (n >= 2 * (int64_t)BM * E) return 1;
  return (!swiglu && dtype == 1) ? 1 : 0;
}

// Cache policy of the copies and stores (measured on gfx950, in one process, ms for
// default | non-temporal stores | non-temporal stores and weight copies):
//  * output rows (H, saved A|U, ring_y) are written once and read once by a later
//    kernel: non-temporal stores never lost and sometimes won (share MX down GEMM
//    0.422 | 0.399; 2,048-token bf16 down GEMM 1.434 | 1.415), whole forward included;
//  * non-temporal weight copies pay only where every weight panel is read once, i.e.
//    one row tile per expert, and then only in the down GEMM (2,048 tokens bf16 1.434 |
//    1.415 | 1.292, MX 0.907 | 0.876 | 0.859); the gate/up GEMM loses there (2.583 |
//    2.578 | 2.728) and so does every GEMM whose panels several row tiles share (skewed
//    gate/up 2.273 | 2.252 | 2.628, share bf16 1.006 | 0.992 | 1.165).
// A bare copy of the gate/up pattern with a per-tile store behaves the same way: 2.54 ms
// with default stores whichever the load policy, 2.29 ms with both non-temporal.
// Whole 2,048-token bf16 forward: 4.205 -> 4.093 ms.  These figures are for the tile of
// four waves.  With eight waves the bf16 gate/up GEMM with one row tile per expert
// gains from non-temporal weight copies too (2.550 | 2.340 ms at 2,048 tokens, whole
// forward 4.019 -> 3.837 ms); the MX gate/up GEMM still loses (1.485 | 1.553), and so
// does a gate/up GEMM whose panels several row tiles share (skewed 2.166 | 2.431).
inline int gemm_policy(bool swiglu, int dtype, int64_t n, int E, int BM) {
  if (n > (int64_t)BM * E) return 2;   // weight panels shared by several row tiles
  return (!swiglu || dtype == 1) ? 3 : 2;
}

inline int max_tiles_for(int64_t n, int E, int BM) { return (int)((n + BM - 1) / BM) + E; }


}  // namespace moe
