// Backward of the MoE layer, L = sum_t <dy_t, y_t>, routing held fixed.
//
// The pages' ring buffer is walked in reverse in the backward pass to cut
// activation replay (dzen.guru page, ring-buffer paragraph of "Три решения…").
// Here the weight gradients schedule experts E-1 -> 0 and every output tile
// consumes its expert's ring rows from the last slot to the first; everything
// else reads the forward's ring-ordered state (ring_x, saved [A|U]) in place.
//
// Per copy (t, j) of expert e with gate g, a = W_g x, u = W_u x, s = sigmoid(a):
//   dh = W_d^T dy_t;  dg = <dh, h>;  da = g dh u s (1 + a (1 - s));  du = g dh a s
//   dx_t += W_g^T da + W_u^T du;  dW_d += g dy_t h^T;  dW_g += da x^T;  dW_u += du x^T
//   dl_j = g_j (dg_j - sum_i g_i dg_i);  dW_r[e_j] += dl_j x_t;  dx_t += dl_j W_r[e_j]
//
// Kernels:
//   dgrad_kernel<DOWN>  ring rows of dy x W_down[e] (K = d rows), epilogue:
//                       SwiGLU backward -> dA|dU (bf16), g*h (bf16), row partials of dg
//   dgrad_kernel<UP>    [dA|dU] x [W_gate[e]; W_up[e]] (K = 2f rows) -> dX per copy (bf16)
//   token_kernel        dg, dl per token; dx = sum_j dX[copy] + dl_j W_r[e_j] (bf16)
//   router_wgrad_*      dW_r[e] = sum over the segment (last slot first) of dl x  (fp32),
//                       per 128-row tile, then over the expert's tiles (last first)
//   gather_to_ring      dy rows copied into ring order, one per copy (t, j)
//   wgrad_kernel        dW_down[e] = dY_e^T (g H)_e;  [dW_gate;dW_up][e] = [dA|dU]_e^T X_e
// The dgrad tiles are 128 x 256 (eight waves; 128 x 128 with four when the output
// width is not a multiple of 256) with K in 32-element stages filled by global -> LDS
// copies; the weights, whose K index is their row index, are staged row-major and
// read as MFMA fragments with transposing LDS reads, as are both operands of the
// weight gradients.  No floating-point atomics: every sum has one fixed order.
// The 256-column tiles copy each 128-row tile of copy rows once per 256 output columns
// instead of once per 128 (skewed 8,192-token backward, same-GPU A/B: 9.85 ms with
// 128 x 128 tiles, 9.37 with the gate/up dgrad widened, 9.04 with both).
#include "common.h"
#include "gemm_body.h"
#include "kernels.h"

namespace moe {

constexpr int BT = 128;            // dgrad tile rows and columns
// Output tiles are staged row-major in LDS (BT rows of BT bf16, rows padded by 16
// bytes) and written as whole 16-byte pieces of rows instead of 2-byte stores
// scattered over rows.
template <int W>   // staged tile width in columns
struct Staging {
  static constexpr int SRS = W * 2 + 16;    // staged row stride in bytes
  static constexpr int BYTES = BT * SRS;    // 34,816 for 128 columns
};

template <int W = BT>
__device__ __forceinline__ void stage_put(uint8_t* stg, int m, int n, float v) {
  *(uint16_t*)(stg + m * Staging<W>::SRS + n * 2) = f2bf(v);
}

// Write the staged tile: row m < rows goes to dst_row(m) (a pointer to the tile's first
// column in that row), 16 bytes per thread and step, NT threads, with the non-temporal
// policy (as the weight-gradient stores: skewed backward 8.84 -> 8.71 ms with both, same-GPU
// A/B).  Barriers before and after.
template <int W = BT, int NT = 256, typename RowF>
__device__ __forceinline__ void stage_flush(const uint8_t* stg, int rows, RowF dst_row) {
  __syncthreads();
  constexpr int CPR = W * 2 / 16;
#pragma unroll 4
  for (int q = threadIdx.x; q < BT * CPR; q += NT) {
    const int m = q / CPR, c = q % CPR;
    if (m < rows)
      __builtin_nontemporal_store(*(const u32x4*)(stg + m * Staging<W>::SRS + c * 16), (u32x4*)((uint8_t*)dst_row(m) + c * 16));
  }
  __syncthreads();
}

template <typename T>
__device__ __forceinline__ T bld_meta(const T* q) {   // scalar load of data written by earlier kernels
  return *(const __attribute__((address_space(4))) T*)q;
}

// ----------------------------------------------------------------------------- dgrad
struct DgradArgs {
  const bf16_t* A;          // ring-ordered rows: DOWN dy [C, d] (gathered into ring order); UP dAU [C, 2f]
  const bf16_t* B0;         // DOWN: W_down [E, d, f]; UP: W_gate [E, f, d]
  const bf16_t* B1;         // UP: W_up [E, f, d]
  int K, N;                 // DOWN: K = d, N = f; UP: K = 2f, N = d
  int f;                    // expert intermediate width
  const int32_t* offset;
  const int32_t* tiles;
  const int32_t* ntiles;
  const int32_t* slot_copy;
  const float* gate;        // [T*k] by copy id
  int k;
  int64_t head, C;
  const bf16_t* saved_au;   // DOWN: [C, 2f]
  bf16_t* dau;              // DOWN out: [C, 2f]
  bf16_t* gh;               // DOWN out: [C, f]
  float* dgpart;            // DOWN out: [C, f / (tile columns)]
  bf16_t* dxc;              // UP out: [C, d]
};

// Global -> LDS copy of 16 bytes per lane from a per-lane address (the wave's 64
// lanes fill 1 KB of LDS at m0 + lane * 16), and a wait for this wave's copies.
__device__ __forceinline__ void dma16_at(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(addr), "s"(lds) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void bwait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ int wsw(int r, int c) { return c ^ ((r & 3) << 2); }
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i16_t ds_tr16(const uint8_t* lds_ptr) {
  typedef __attribute__((address_space(3))) v4i16_t lds_v4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4*)((__attribute__((address_space(3))) uint8_t*)lds_ptr));
}

// dgrad stages: DK = 32 K elements.  A: BT ring rows x 64 bytes, 16-byte chunks
// XOR-swizzled by (row >> 2) & 3 (a 128-bit fragment read is served 16 lanes = 16 rows
// at a time, which then hit 16 distinct chunk positions of the 256-byte bank line).
// B: DK weight rows (K) x BT columns (256 bytes), chunks swizzled by (row & 3) << 2,
// read as MFMA fragments with transposing reads: lane l receives column l % 32 at K
// rows 8 (l / 32) .. 8 (l / 32) + 7 of a 16-row sub-step, in two reads of 4 rows.
// Both tiles are filled by global -> LDS copies (no register staging) through a ring
// of DWS stages, DWS - 1 of them in flight while one is multiplied.  Three stages
// (48 KB), so three workgroups share a CU: skewed 8,192-token backward 9.92 -> 9.79 ms
// against four stages and two workgroups; five stages and two workgroups 10.9 ms, two
// stages and four workgroups 9.76 ms.
constexpr int DK = 32, DWS = 3;
// Tile shape: 128 rows x 64 NWN columns, waves in 2 x NWN of 64 x 64.
template <int NWN>
struct DgShape {
  static constexpr int NW = 2 * NWN, NT = 64 * NW;     // waves, threads
  static constexpr int BN = 64 * NWN;                  // tile columns
  static constexpr int A_BYTES = BT * DK * 2, B_BYTES = DK * BN * 2, STAGE = A_BYTES + B_BYTES;
  // the stage ring; the epilogue staging reuses it
  static constexpr int LDS = DWS * STAGE > Staging<BN>::BYTES ? DWS * STAGE : Staging<BN>::BYTES;
  static constexpr int NA = A_BYTES / (1024 * NW), NB = B_BYTES / (1024 * NW);   // 1 KB copies per wave
  static constexpr int L = NA + NB;
  static constexpr int RPK = 1024 / (BN * 2), CPRB = BN * 2 / 16;   // B rows per KB, 16-byte chunks per B row
  static constexpr int OCC = NWN == 2 ? 3 : 2;         // workgroups per CU (the LDS of each)
};

__device__ __forceinline__ int aswz(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// Row tiles per group in the dgrad tile order (below): the down dgrad's copy rows are
// d wide (1 MB per 128-row tile at d = 4096) and its 8 column tiles all run at once;
// the gate/up dgrad's are 2f wide (512 KB) against 32 column tiles.
constexpr int DG_GROUP_DOWN = 8, DG_GROUP_UP = 4;

// Logical tile L of an expert-major list of (row tile, column tile) pairs, nct column
// tiles per row tile, row tiles in groups of G per expert with the column tile slower
// than the row tile inside a group.  The expert of L is that of row tile L / nct (the
// expert's range of L is the same in row-major order); tiles[2 i + 1] / BT is row tile
// i's index inside its expert.
__device__ __forceinline__ void grouped_tile(int L, int nct, int G, const int32_t* tiles,
                                             const int32_t* offset, int& mt, int& ct) {
  const int mr = L / nct;
  const int e = tiles[2 * mr];
  const int t0 = mr - tiles[2 * mr + 1] / BT;                       // the expert's first row tile
  const int R = (offset[e + 1] - offset[e] + BT - 1) / BT;          // its row tiles
  const int local = L - t0 * nct;
  const int g = local / (G * nct);
  const int rg = min(G, R - g * G);                                 // row tiles in group g
  const int rem = local - g * G * nct;
  ct = rem / rg;
  mt = t0 + g * G + rem % rg;
}

// NWN = 2: 128 x 128 tiles, four waves (both dgrads); NWN = 4: 128 x 256, eight waves (the
// gate/up dgrad: each 128-row tile of [dA|dU] is copied once per 256 output columns
// instead of once per 128).
template <bool DOWN, int NWN>
__global__ __launch_bounds__(DgShape<NWN>::NT, DgShape<NWN>::OCC) void dgrad_kernel(DgradArgs p) {
  using Sh = DgShape<NWN>;
  constexpr int DA_BYTES = Sh::A_BYTES, NW = Sh::NW, BN = Sh::BN, DL = Sh::L;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  __shared__ float red[NWN][BT];   // DOWN: per wave column, each row's partial of dg
  // Tile order: workgroup b runs on XCD b % 8, and XCD x takes the logical tiles
  // [x per, (x + 1) per), per = ceil(V / 8) of the V live tiles.  Logical tiles are
  // expert-major; an expert's row tiles form groups of G, and inside a group the column
  // tile is slower than the row tile: the group's row tiles read each weight panel
  // together, through one L2, and the group's copy rows stay there for all its column
  // tiles.  Fetched at 8,192 skewed tokens (FETCH_SIZE, copy-calibrated), down | gate/up
  // dgrad: column tile as blockIdx.x (every XCD fetched every row tile's copy rows) 10.8 |
  // 12.5 GB; row-major contiguous ranges (the gate/up weights re-fetched per row tile)
  // 7.6 | 15.6 GB; this order 7.0 | 10.8 GB, against 5.3 | 8.9 GB algorithmic.  The
  // kernel times did not change (1.79 | 2.91 ms): these kernels are bound by their
  // copy-to-MFMA pipeline, not by HBM traffic.
  const int nct = p.N / BN;
  const int V = *p.ntiles * nct, per = (V + 7) / 8;
  const int li = (int)(blockIdx.x >> 3), L = (int)(blockIdx.x & 7) * per + li;
  if (li >= per || L >= V) return;
  int mt, ct;
  grouped_tile(L, nct, DOWN ? DG_GROUP_DOWN : DG_GROUP_UP, p.tiles, p.offset, mt, ct);
  const int e = p.tiles[2 * mt], row0 = p.tiles[2 * mt + 1];
  const int32_t seg = p.offset[e];
  const int rows = min(BT, p.offset[e + 1] - seg - row0);
  const int n0 = ct * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN, lr = lane & 31, lg = lane >> 5;

  // Copy i of this wave fills LDS kilobyte wave + NW i of the A tile, rows
  // 16 (wave + NW i) .. + 15, or of the B tile, K rows RPK (wave + NW i) .. + RPK - 1.
  const uint8_t* a_addr[Sh::NA];
  int b_row[Sh::NB], b_col[Sh::NB];
#pragma unroll
  for (int i = 0; i < Sh::NA; ++i) {
    const int j = wave + NW * i;
    const int r = j * 16 + (lane >> 2), slot = lane & 3, c = slot ^ ((r >> 2) & 3);
    const int64_t sl = ring_slot(p.head, seg, row0 + min(r, rows - 1), p.C);
    a_addr[i] = (const uint8_t*)p.A + (sl * p.K) * 2 + c * 16;
  }
#pragma unroll
  for (int i = 0; i < Sh::NB; ++i) {
    const int j = wave + NW * i;
    const int rb = j * Sh::RPK + lane / Sh::CPRB, sb = lane % Sh::CPRB;
    b_row[i] = rb;
    b_col[i] = (n0 + wsw(rb, sb) * 8) * 2;
  }
  auto brow_ptr = [&](int kk) -> const uint8_t* {   // K row kk of the stacked B
    if (DOWN) return (const uint8_t*)(p.B0 + ((int64_t)e * p.K + kk) * p.N);
    return (const uint8_t*)(kk < p.f ? p.B0 + ((int64_t)e * p.f + kk) * p.N
                                     : p.B1 + ((int64_t)e * p.f + (kk - p.f)) * p.N);
  };
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const uint32_t st = lds0 + (uint32_t)(kt % DWS) * Sh::STAGE;
#pragma unroll
    for (int i = 0; i < Sh::NA; ++i)
      dma16_at(a_addr[i] + kt * (DK * 2), __builtin_amdgcn_readfirstlane(st + (wave + NW * i) * 1024));
#pragma unroll
    for (int i = 0; i < Sh::NB; ++i)
      dma16_at(brow_ptr(kt * DK + b_row[i]) + b_col[i],
               __builtin_amdgcn_readfirstlane(st + DA_BYTES + (wave + NW * i) * 1024));
  };
  auto wait_stage = [&](int later) __attribute__((always_inline)) {
    if (later <= 0) bwait_vm<0>();
    else if (later == 1) bwait_vm<DL>();
    else bwait_vm<2 * DL>();
  };
  // this lane's first transposing read of B fragment j (tile columns wn*64 + 32j ..)
  int boff[2];
  {
    const int g = lane >> 4, gi = lane & 15, qq = gi >> 2, ss = gi & 3;
    const int r0 = 8 * (g >> 1) + qq;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int col = wn * 64 + jj * 32 + 16 * (g & 1) + 4 * ss;
      boff[jj] = DA_BYTES + r0 * (BN * 2) + wsw(r0, col >> 3) * 16 + (col & 7) * 2;
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = p.K / DK;
  for (int s = 0; s < DWS - 1 && s < KT; ++s) issue(s);
  for (int kt = 0; kt < KT; ++kt) {
    wait_stage(min(DWS - 2, KT - 1 - kt));
    __syncthreads();   // stage kt published; the buffer of stage kt - 1 is free
    if (kt + DWS - 1 < KT) issue(kt + DWS - 1);
    const uint8_t* sb = smem + (kt % DWS) * Sh::STAGE;
#pragma unroll
    for (int kk = 0; kk < DK / 16; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sb + aswz(wm * 64 + i * 32 + lr, kk * 2 + lg)));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint8_t* b = sb + boff[j] + kk * 16 * (BN * 2);
        const v4i16_t lo = ds_tr16(b), hi = ds_tr16(b + 4 * (BN * 2));
        bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();   // every wave is done with the stages: the epilogue reuses them

  // the loop ended with a barrier: the operand tiles are free for staging
  uint8_t* stg = smem;
  if (DOWN) {
    // dA, dU and g*h are written directly (three outputs per element)
    const int f = p.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        const bool live = m < rows;
        const int64_t s = ring_slot(p.head, seg, row0 + min(m, rows - 1), p.C);
        const float g = p.gate[p.slot_copy[s]];
        float dgp = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 64 + j * 32 + lr;
          const float a = bf2f(p.saved_au[s * 2 * f + n]);
          const float u = bf2f(p.saved_au[s * 2 * f + f + n]);
          const float sg = sigm(a);
          const float h = a * sg * u;
          const float dhr = acc[i][j][r];
          dgp = fmaf(dhr, h, dgp);
          const float dh = g * dhr;
          if (live) {
            p.dau[s * 2 * f + n] = f2bf(dh * u * sg * (1.f + a * (1.f - sg)));
            p.dau[s * 2 * f + f + n] = f2bf(dh * a * sg);
            p.gh[s * f + n] = f2bf(g * h);
          }
        }
        // sum over this wave's 64 columns of the row: 32 lanes x 2 fragments
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) dgp += __shfl_xor(dgp, o, 64);
        if (lr == 0) red[wn][m] = dgp;
      }
    __syncthreads();
    if (tid < rows) {
      const int64_t s = ring_slot(p.head, seg, row0 + tid, p.C);
      float dgt = red[0][tid];
#pragma unroll
      for (int w = 1; w < NWN; ++w) dgt += red[w][tid];   // wave columns in order
      p.dgpart[s * (f / BN) + n0 / BN] = dgt;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nl = wn * 64 + j * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * 64 + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
          stage_put<BN>(stg, m, nl, acc[i][j][r]);
        }
      }
    stage_flush<BN, Sh::NT>(stg, rows, [&](int m) -> void* {
      return p.dxc + ring_slot(p.head, seg, row0 + m, p.C) * p.N + n0;
    });
  }
}

// ----------------------------------------------------------------------------- per token
// dg of each copy (fixed-order sum of the column-tile partials), dl, and
// dx[t] = sum_j (dX[copy_slot[t, j]] + dl_j W_r[e_j]) in ascending expert order.
__global__ __launch_bounds__(256) void token_kernel(const int32_t* __restrict__ copy_slot,
                                                    const int32_t* __restrict__ topk_idx,
                                                    const float* __restrict__ gate,
                                                    const float* __restrict__ dgpart, int nt,
                                                    const bf16_t* __restrict__ dxc,
                                                    const float* __restrict__ w_r, int d, int k,
                                                    float* __restrict__ dl_slot,
                                                    bf16_t* __restrict__ dx) {
  __shared__ int64_t slot[64];
  __shared__ int32_t ex[64];
  __shared__ float dl[64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 64) {   // one wavefront: lanes j < k
    float dg = 0.f, g = 0.f;
    int64_t s = 0;
    if (tid < k) {
      s = copy_slot[t * k + tid];
      g = gate[t * k + tid];
      for (int q = 0; q < nt; ++q) dg += dgpart[s * nt + q];
      slot[tid] = s;
      ex[tid] = topk_idx[t * k + tid];
    }
    const float S = wave_sum(g * dg);
    if (tid < k) {
      const float v = g * (dg - S);
      dl[tid] = v;
      dl_slot[s] = v;
    }
  }
  __syncthreads();
  for (int v = tid; v < d / 8; v += 256) {
    float acc[8] = {};
    for (int j = 0; j < k; ++j) {
      const u32x4 w = ((const u32x4*)(dxc + slot[j] * d))[v];
      const f32x4 r0 = *(const f32x4*)(w_r + (int64_t)ex[j] * d + v * 8);
      const f32x4 r1 = *(const f32x4*)(w_r + (int64_t)ex[j] * d + v * 8 + 4);
      const float l = dl[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += lo_bf(w[q]);
        acc[2 * q + 1] += hi_bf(w[q]);
      }
      acc[0] = fmaf(l, r0[0], acc[0]); acc[1] = fmaf(l, r0[1], acc[1]);
      acc[2] = fmaf(l, r0[2], acc[2]); acc[3] = fmaf(l, r0[3], acc[3]);
      acc[4] = fmaf(l, r1[0], acc[4]); acc[5] = fmaf(l, r1[1], acc[5]);
      acc[6] = fmaf(l, r1[2], acc[6]); acc[7] = fmaf(l, r1[3], acc[7]);
    }
    ((u32x4*)(dx + t * d))[v] = u32x4{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]),
                                      pack_bf2(acc[4], acc[5]), pack_bf2(acc[6], acc[7])};
  }
}

// dW_r[e] = sum over the expert's rows, last slot first, of dl x.  Step 1: every
// 128-row tile of the tile list (expert-major, rows ascending) sums its rows, last
// first, into an fp32 partial; the expert's first tile records its index.  Step 2
// sums each expert's partials, last tile first.  A hot expert's rows are thus spread
// over many workgroups, in a fixed order.
__global__ __launch_bounds__(128) void router_wgrad_part_kernel(
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    const int32_t* __restrict__ offset, int64_t head, int64_t C,
    const bf16_t* __restrict__ ring_x, const float* __restrict__ dl_slot, int d,
    float* __restrict__ part, int32_t* __restrict__ first_tile, const int32_t* __restrict__ x_map,
    int kdiv) {
  // x_map set: ring_x is token-major x [T, d] and ring slot s takes row x_map[s] / kdiv
  const int mt = blockIdx.x;
  if (mt >= *ntiles) return;
  const int e = tiles[2 * mt], row0 = tiles[2 * mt + 1];
  const int v = blockIdx.y * 128 + threadIdx.x;   // 8 columns per thread
  if (row0 == 0 && blockIdx.y == 0 && threadIdx.x == 0) first_tile[e] = mt;
  if (v * 8 >= d) return;
  const int32_t seg = offset[e];
  const int rows = min(BT, offset[e + 1] - seg - row0);
  float acc[8] = {};
  auto add = [&](float l, const u32x4& w) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(l, lo_bf(w[q]), acc[2 * q]);
      acc[2 * q + 1] = fmaf(l, hi_bf(w[q]), acc[2 * q + 1]);
    }
  };
  // the loads of RB rows are issued together, then added in the same order
  constexpr int RB = 16;
  int i = rows - 1;
  for (; i >= RB - 1; i -= RB) {
    float l[RB];
    u32x4 w[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int64_t s = ring_slot(head, seg, row0 + i - u, C);
      const int64_t xr = x_map ? (int64_t)(bld_meta(x_map + s) / kdiv) : s;
      l[u] = dl_slot[s];
      w[u] = ((const u32x4*)(ring_x + xr * d))[v];
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) add(l[u], w[u]);
  }
  for (; i >= 0; --i) {
    const int64_t s = ring_slot(head, seg, row0 + i, C);
    const int64_t xr = x_map ? (int64_t)(bld_meta(x_map + s) / kdiv) : s;
    add(dl_slot[s], ((const u32x4*)(ring_x + xr * d))[v]);
  }
  f32x4* dst = (f32x4*)(part + (int64_t)mt * d + v * 8);
  dst[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  dst[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

__global__ __launch_bounds__(256) void router_wgrad_sum_kernel(
    const int32_t* __restrict__ offset, const int32_t* __restrict__ first_tile,
    const float* __restrict__ part, int d, float* __restrict__ dw_r) {
  const int e = blockIdx.x;
  const int v = blockIdx.y * 256 + threadIdx.x;   // 4 columns per thread
  if (v * 4 >= d) return;
  const int n = offset[e + 1] - offset[e];
  const int nt = (n + BT - 1) / BT;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (nt > 0) {
    const int t0 = first_tile[e];
    for (int c = nt - 1; c >= 0; --c) acc += *(const f32x4*)(part + (int64_t)(t0 + c) * d + v * 4);
  }
  *(f32x4*)(dw_r + (int64_t)e * d + v * 4) = acc;
}

// ----------------------------------------------------------------------------- wgrad
// dW[e] = A_e^T B_e over expert e's ring rows.  Both operands are row-major with the
// reduction index (the ring row) as the row, so a stage holds WK rows of each in
// their natural layout, copied global -> LDS by DMA, and the MFMA fragments (8
// consecutive K of one column) are read with ds_read_b64_tr_b16: within each
// 16-lane group, lane 4q + s addresses row k0 + q, columns c0 + 4s .. 4s + 3, and
// lane i receives column c0 + i at rows k0 .. k0 + 3 (measured on gfx950).  Two
// such reads give a lane its 8 K values.
//
// The experts hold few rows each (K is short) while dW is large, so the kernel is
// bound by writing dW.  Each workgroup computes one WM x WN tile in 4 waves of
// 64 x WN/2 with WS stages of WK = 32 rows; small tiles and LDS used for the stages
// only let several workgroups share a CU, so that one's loads, MFMAs and stores
// overlap another's.  Stage kt holds the segment rows [n - WK (kt + 1), n - WK kt):
// the expert's rows are consumed last slot first, and rows before the segment
// start are read from a zero row (they add nothing).  The 16-byte chunks of a
// staged row are XOR-swizzled by ((row & 3) << 2): a transposing read is served 32
// lanes (4 rows x 64 bytes) at a time, and the four rows then fall on distinct banks.
//
// The MFMA is given the B fragment first, so it accumulates the transposed tile:
// a lane holds one output row and, per group of 4 accumulators, 4 consecutive
// columns.  Lanes l and l + 32 hold the two halves of 8 columns; one
// v_permlane32_swap per packed word pair gives each lane 8 consecutive bf16 of one
// row, which it writes straight from registers as one 16-byte piece.
constexpr int WK_ = 32;

// WGM x WGN waves, each 64 rows x 32 NJ columns of the dW tile.
template <int WGM, int WGN, int NJ>
struct WgShape {
  static constexpr int NW = WGM * WGN, NT = 64 * NW;
  static constexpr int WM = 64 * WGM, WN = 32 * NJ * WGN;   // tile rows (of dW) and columns
  static constexpr int ARB = WM * 2, BRB = WN * 2;          // staged row bytes of A and B
  static constexpr int STAGE = WK_ * (ARB + BRB);
  static constexpr int LA = WK_ * ARB / (1024 * NW), LB = WK_ * BRB / (1024 * NW);   // 1 KB copies per wave
  static constexpr int L = LA + LB;
  static_assert(WK_ * ARB % (1024 * NW) == 0 && WK_ * BRB % (1024 * NW) == 0, "copies split evenly");
};



struct WgradArgs {
  const bf16_t* A;          // ring-ordered rows: DOWN dy gathered into ring order [C, d]; UP dAU [C, 2f]
  const bf16_t* B;          // ring-ordered rows: DOWN gH [C, f]; UP ring_x [C, d]
  int M, N;                 // DOWN: M = d, N = f; UP: M = 2f, N = d
  int msplit;               // rows m < msplit go to out0, the rest to out1
  int lda, ldb;             // row lengths (elements)
  const int32_t* offset;
  int E;
  int64_t head, C;
  const bf16_t* zero;       // >= 1024 zero bytes
  bf16_t* out0;             // [E, msplit, N]
  bf16_t* out1;             // [E, M - msplit, N]
};

template <int WGM, int WGN, int NJ, int WS, int OCC>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void wgrad_kernel(WgradArgs p) {
  using S = WgShape<WGM, WGN, NJ>;
  constexpr int WM_ = S::WM, NW = S::NW;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const int mtiles = (p.M + WM_ - 1) / WM_, ntiles = (p.N + S::WN - 1) / S::WN;
  const int P = mtiles * ntiles;   // tiles per expert
  // Workgroup b runs on XCD b % 8.  XCD x takes whole experts, those with e % 8 == x,
  // from the largest id down (experts E-1 -> 0 overall), all P tiles of each: both
  // operand panels of an expert are then fetched once, into one XCD's L2.  Interleaved
  // ids spread the hottest experts over the eight XCDs.  Dealing every expert's tiles
  // over all eight XCDs fetched each panel once per XCD: 2.03 + 3.39 GB (down, gate/up)
  // against 0.84 + 1.0 GB algorithmic in the skewed 8,192-token backward; this order
  // fetches 0.93 + 1.80 GB in the same time (1.67 + 3.06 ms: the dW stores bound it).
  const int x = blockIdx.x & 7, li = blockIdx.x >> 3;
  if (x >= p.E) return;
  const int etop = p.E - 1 - ((p.E - 1 - x) & 7);   // the largest expert id = x (mod 8)
  const int e = etop - 8 * (li / P), jt = li % P;
  if (e < 0) return;
  const bool nmajor = p.M < p.N;
  const int m0 = (nmajor ? jt % mtiles : jt / ntiles) * WM_;
  const int n0 = (nmajor ? jt / mtiles : jt % ntiles) * S::WN;
  const int32_t seg = bld_meta(p.offset + e);
  const int nrows = bld_meta(p.offset + e + 1) - seg;
  const int KT = max(1, (nrows + WK_ - 1) / WK_);
  const int64_t hs = p.head + seg;   // ring slot of segment row i: hs + i, less C once past the end

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN, lr = lane & 31, lg = lane >> 5;

  // Per copy c of this wave (fixed for the tile): the staged row this lane fills and
  // the byte offset of its 16-byte piece inside a source row.
  int crow[S::L], ccol[S::L];
#pragma unroll
  for (int c = 0; c < S::L; ++c) {
    const bool isa = c < S::LA;
    const int j = NW * (isa ? c : c - S::LA) + wave;
    const int rb = isa ? S::ARB : S::BRB;
    const int q = lane / (rb / 16), r = j * (1024 / rb) + q, lc = wsw(r, lane % (rb / 16));
    crow[c] = r;
    ccol[c] = 2 * (isa ? min(m0 + lc * 8, p.M - 8) : min(n0 + lc * 8, p.N - 8));
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const uint32_t st = lds0 + (uint32_t)(kt % WS) * S::STAGE;
    const int rbase = nrows - WK_ * (kt + 1);   // segment row of staged row 0
#pragma unroll
    for (int c = 0; c < S::L; ++c) {
      const bool isa = c < S::LA;
      const int j = NW * (isa ? c : c - S::LA) + wave;
      const int i = rbase + crow[c];
      int64_t sl = hs + i;
      sl = sl >= p.C ? sl - p.C : sl;
      const int64_t rowbytes = (int64_t)(isa ? p.lda : p.ldb) * 2;
      const uint8_t* src = i >= 0 ? (const uint8_t*)(isa ? p.A : p.B) + sl * rowbytes + ccol[c]
                                  : (const uint8_t*)p.zero + lane * 16;
      dma16_at(src, __builtin_amdgcn_readfirstlane(st + (isa ? 0 : WK_ * S::ARB) + j * 1024));
    }
  };
  auto wait_stage = [&](int later) __attribute__((always_inline)) {
    if (later <= 0) bwait_vm<0>();
    else if (later == 1) bwait_vm<S::L>();
    else bwait_vm<2 * S::L>();
  };

  f32x16 acc[NJ][2];
#pragma unroll
  for (int jn = 0; jn < NJ; ++jn)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[jn][i][r] = 0.f;

  // Fragment q of sub-step 0: q < 2 is A fragment q (tile columns wm*64 + 32q), else B
  // fragment q - 2 (columns wn*32*NJ + 32(q-2)).  Offset inside a stage of this lane's
  // first transposing read (4 K rows); the second is 4 rows further (same swizzle,
  // since it depends on row & 3), and sub-step kk is 16 rows further.
  int foff[2 + NJ];
  {
    const int g = lane >> 4, gi = lane & 15, qq = gi >> 2, ss = gi & 3;
    const int r0 = 8 * (g >> 1) + qq;
#pragma unroll
    for (int q = 0; q < 2 + NJ; ++q) {
      const bool isa = q < 2;
      const int col = (isa ? wm * 64 + q * 32 : wn * 32 * NJ + (q - 2) * 32) + 16 * (g & 1) + 4 * ss;
      foff[q] = (isa ? 0 : WK_ * S::ARB) + r0 * (isa ? S::ARB : S::BRB) + wsw(r0, col >> 3) * 16 +
                (col & 7) * 2;
    }
  }
  auto frag = [&](const uint8_t* sb, int kk, int q) __attribute__((always_inline)) -> bf16x8 {
    const int rowb = q < 2 ? S::ARB : S::BRB;
    const uint8_t* a = sb + foff[q] + kk * 16 * rowb;
    const v4i16_t lo = ds_tr16(a), hi = ds_tr16(a + 4 * rowb);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  for (int s = 0; s < WS - 1 && s < KT; ++s) issue(s);
  for (int kt = 0; kt < KT; ++kt) {
    wait_stage(min(WS - 2, KT - 1 - kt));
    __syncthreads();
    if (kt + WS - 1 < KT) issue(kt + WS - 1);
    const uint8_t* sb = lds + (kt % WS) * S::STAGE;
    bf16x8 fa[2][2], fb[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[0][i] = frag(sb, 0, i);
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) fb[0][jn] = frag(sb, 0, 2 + jn);
#pragma unroll
    for (int kk = 0; kk < WK_ / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < WK_ / 16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[cur ^ 1][i] = frag(sb, kk + 1, i);
#pragma unroll
        for (int jn = 0; jn < NJ; ++jn) fb[cur ^ 1][jn] = frag(sb, kk + 1, 2 + jn);
      }
#pragma unroll
      for (int jn = 0; jn < NJ; ++jn)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[jn][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][jn], fa[cur][i], acc[jn][i], 0, 0, 0);
    }
  }

  // acc[jn][i][r]: output row m0 + wm*64 + 32i + lr, column
  // n0 + wn*32*NJ + 32jn + 8(r/4) + 4lg + r%4.  Each half i (32 rows x 32 NJ columns) is
  // staged in a wave-private LDS area and written back as whole row pieces: 64 lanes store
  // four rows' 256 contiguous bytes, 8 full cache lines per instruction, where storing
  // from the accumulator layout would put 32 bytes into each of 32 rows.
  static_assert(NJ == 4, "the staging swizzle assumes 256-byte rows (16 chunks)");
  static_assert(NW * 32 * 64 * NJ <= WS * S::STAGE, "the staging areas fit in the stage ring");
  __syncthreads();   // every wave is done with the stages
  uint8_t* wl = lds + wave * (32 * 64 * NJ);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x16& a = acc[jn][i];
        // x: columns 16h + 4lg + 0..3, y: columns 16h + 8 + 4lg + 0..3.  The swap hands
        // x of lanes 32..63 to lanes 0..31 and y of lanes 0..31 to lanes 32..63.
        const uint32_t x0 = pack_bf2(a[8 * h + 0], a[8 * h + 1]), x1 = pack_bf2(a[8 * h + 2], a[8 * h + 3]);
        const uint32_t y0 = pack_bf2(a[8 * h + 4], a[8 * h + 5]), y1 = pack_bf2(a[8 * h + 6], a[8 * h + 7]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
        // chunk 4jn + 2h + lg of row lr; chunks XOR-swizzled by the row so the 16 rows
        // of a 16-lane group land on distinct 16-byte groups of the bank line
        *(u32x4*)(wl + lr * 256 + (((4 * jn + 2 * h + lg) ^ (lr & 15)) << 4)) = v;
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const int r = 4 * s2 + (lane >> 4), c = lane & 15;
      const u32x4 v = *(const u32x4*)(wl + r * 256 + ((c ^ (r & 15)) << 4));
      const int m = m0 + wm * 64 + 32 * i + r, n = n0 + wn * 32 * NJ + 8 * c;
      bf16_t* row = m < p.msplit ? p.out0 + ((int64_t)e * p.msplit + m) * p.N
                                 : p.out1 + ((int64_t)e * (p.M - p.msplit) + (m - p.msplit)) * p.N;
      if (m < p.M && n < p.N) __builtin_nontemporal_store(v, (u32x4*)(row + n));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// dy rows into ring order: rdy[copy_slot[t, j]] = dy[t] (the layout of the ring).
__global__ __launch_bounds__(256) void gather_to_ring_kernel(const bf16_t* __restrict__ dy,
                                                             const int32_t* __restrict__ copy_slot,
                                                             int k, int d, bf16_t* __restrict__ rdy) {
  const int64_t t = blockIdx.x;
  const u32x4* src = (const u32x4*)(dy + t * d);
  for (int v = threadIdx.x; v < d / 8; v += 256) {
    const u32x4 val = src[v];
    for (int j = 0; j < k; ++j) ((u32x4*)(rdy + (int64_t)copy_slot[t * k + j] * d))[v] = val;
  }
}

// ----------------------------------------------------------------------------- launcher
static int bwd_max_tiles(int64_t n, int E) { return (int)((n + BT - 1) / BT) + E; }

struct BwdLayout {
  size_t tiles, dau, gh, dgpart, dxc, dl, zero, rdy, rpart, rfirst, total;
};

static BwdLayout bwd_layout(int64_t T, int64_t C, int d, int E, int k, int f) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  BwdLayout L;
  size_t o = 0;
  L.tiles = o; o += al((size_t)(2 * bwd_max_tiles(T * k, E) + 64) * 4);
  L.dau = o;   o += al((size_t)C * 2 * f * 2);
  L.gh = o;    o += al((size_t)C * f * 2);
  L.dgpart = o; o += al((size_t)C * (f / BT) * 4);
  L.dxc = o;   o += al((size_t)C * d * 2);
  L.dl = o;    o += al((size_t)C * 4);
  L.rpart = o; o += al((size_t)bwd_max_tiles(T * k, E) * d * 4);   // router-gradient tile partials
  L.rfirst = o; o += al((size_t)E * 4);
  L.zero = o;  o += 1024;   // a zero row for the weight-gradient stages
  L.rdy = o;   o += al((size_t)C * d * 2);   // dy in ring order
  L.total = o;
  return L;
}

size_t backward_workspace_bytes(int64_t T, int64_t C, int d, int E, int k, int f) {
  return bwd_layout(T, C, d, E, k, f).total;
}

__global__ void zero_fill_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// 128 x 256 tiles (2 x 2 waves of 64 x 128), 2 stages, 3 workgroups per CU (measured best of
// 128 x 128 / 128 x 256, 2 / 3 stages, 2 to 4 workgroups per CU).  Skewed 8,192-token bf16
// backward, same-GPU A/B: this shape 9.0 ms; 256 x 256 in 4 x 4 waves of 64 x 64, one
// workgroup per CU, 2 / 3 / 4 stages 9.8-10.0 / 9.2-9.3 / 9.1-9.2 ms; 128 x 256 in 2 x 4
// waves of 64 x 64, two per CU, 9.6 ms (a third fewer copied bytes per dW element does not
// pay for fewer independent workgroups per CU).
constexpr int WG_M = 2, WG_N = 2, WG_NJ = 4, WG_WS = 2, WG_OCC = 3;

static hipError_t run_wgrad(const WgradArgs& a, hipStream_t st) {
  using S = WgShape<WG_M, WG_N, WG_NJ>;
  auto kern = wgrad_kernel<WG_M, WG_N, WG_NJ, WG_WS, WG_OCC>;
  constexpr int lds = WG_WS * S::STAGE;
  if (lds > 65536) {   // opt in to more than 64 KB of LDS (a host-side call, on every launch)
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
  }
  const int64_t P = (int64_t)((a.M + S::WM - 1) / S::WM) * ((a.N + S::WN - 1) / S::WN);
  kern<<<(unsigned)(8 * P * ((a.E + 7) / 8)), S::NT, lds, st>>>(a);   // 8 XCDs x P x the longest expert list
  return hipGetLastError();
}

hipError_t launch_backward(const void* dy, const void* x, const float* w_r,
                           const int32_t* topk_idx, const float* topk_gate, const void* ring_x,
                           const int32_t* expert_offset, const int32_t* copy_slot,
                           const int32_t* slot_copy, int64_t head, int64_t C, const void* saved_au,
                           const void* w_gate, const void* w_up, const void* w_down, int64_t T,
                           int d, int E, int k, int f, void* dx, void* dw_gate, void* dw_up,
                           void* dw_down, float* dw_r, void* ws, hipStream_t st) {
  (void)x;
  if (d % BT || f % BT) return hipErrorInvalidValue;
  const BwdLayout L = bwd_layout(T, C, d, E, k, f);
  uint8_t* w = (uint8_t*)ws;
  int32_t* ntiles = (int32_t*)(w + L.tiles);
  int32_t* tiles = ntiles + 64;
  bf16_t* dau = (bf16_t*)(w + L.dau);
  bf16_t* gh = (bf16_t*)(w + L.gh);
  float* dgpart = (float*)(w + L.dgpart);
  bf16_t* dxc = (bf16_t*)(w + L.dxc);
  float* dl = (float*)(w + L.dl);
  const int n = (int)(T * k);
  const int max_tiles = bwd_max_tiles(n, E);

  hipError_t err = launch_build_tiles(expert_offset, E, BT, tiles, ntiles, st);
  if (err != hipSuccess) return err;
  zero_fill_kernel<<<1, 256, 0, st>>>((uint32_t*)(w + L.zero), 256);
  bf16_t* rdy = (bf16_t*)(w + L.rdy);
  gather_to_ring_kernel<<<(unsigned)T, 256, 0, st>>>((const bf16_t*)dy, copy_slot, k, d, rdy);
  // dynamic LDS of the dgrad kernels: the stage ring (or the epilogue staging), asked for
  // on every call (a host-side attribute, no state kept here)
  // 256-column tiles where the output width allows (the copy rows are then copied once
  // per 256 output columns instead of once per 128)
  const bool wide = d % DgShape<4>::BN == 0, wide_down = f % DgShape<4>::BN == 0;
  const int dg_cols = wide_down ? DgShape<4>::BN : BT;   // column tile of the down dgrad (dg partials)
  if ((err = hipFuncSetAttribute(wide_down ? (const void*)dgrad_kernel<true, 4> : (const void*)dgrad_kernel<true, 2>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                 wide_down ? DgShape<4>::LDS : DgShape<2>::LDS)) != hipSuccess ||
      (err = hipFuncSetAttribute(wide ? (const void*)dgrad_kernel<false, 4> : (const void*)dgrad_kernel<false, 2>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                 wide ? DgShape<4>::LDS : DgShape<2>::LDS)) != hipSuccess)
    return err;
  DgradArgs a{};
  a.A = rdy;
  a.B0 = (const bf16_t*)w_down;
  a.K = d;
  a.N = f;
  a.f = f;
  a.offset = expert_offset;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.slot_copy = slot_copy;
  a.gate = topk_gate;
  a.k = k;
  a.head = head;
  a.C = C;
  a.saved_au = (const bf16_t*)saved_au;
  a.dau = dau;
  a.gh = gh;
  a.dgpart = dgpart;
  // 1-D grids over the bound max_tiles x column tiles (XCD-contiguous tile order inside)
  if (wide_down)
    dgrad_kernel<true, 4><<<(unsigned)(8 * (((int64_t)max_tiles * (f / DgShape<4>::BN) + 7) / 8)),
                            DgShape<4>::NT, DgShape<4>::LDS, st>>>(a);
  else
    dgrad_kernel<true, 2><<<(unsigned)(8 * (((int64_t)max_tiles * (f / BT) + 7) / 8)), DgShape<2>::NT,
                            DgShape<2>::LDS, st>>>(a);
  DgradArgs b = a;
  b.A = dau;
  b.B0 = (const bf16_t*)w_gate;
  b.B1 = (const bf16_t*)w_up;
  b.K = 2 * f;
  b.N = d;
  b.dxc = dxc;
  if (wide)
    dgrad_kernel<false, 4><<<(unsigned)(8 * (((int64_t)max_tiles * (d / DgShape<4>::BN) + 7) / 8)),
                             DgShape<4>::NT, DgShape<4>::LDS, st>>>(b);
  else
    dgrad_kernel<false, 2><<<(unsigned)(8 * (((int64_t)max_tiles * (d / BT) + 7) / 8)), DgShape<2>::NT,
                             DgShape<2>::LDS, st>>>(b);
  token_kernel<<<(unsigned)T, 256, 0, st>>>(copy_slot, topk_idx, topk_gate, dgpart, f / dg_cols, dxc,
                                            w_r, d, k, dl, (bf16_t*)dx);
  float* rpart = (float*)(w + L.rpart);
  int32_t* rfirst = (int32_t*)(w + L.rfirst);
  router_wgrad_part_kernel<<<dim3(max_tiles, (d / 8 + 127) / 128), 128, 0, st>>>(
      tiles, ntiles, expert_offset, head, C, (const bf16_t*)ring_x, dl, d, rpart, rfirst, nullptr, 1);
  router_wgrad_sum_kernel<<<dim3(E, (d / 4 + 255) / 256), 256, 0, st>>>(expert_offset, rfirst,
                                                                        rpart, d, dw_r);
  WgradArgs wd{};
  wd.A = rdy;
  wd.B = gh;
  wd.M = d;
  wd.N = f;
  wd.msplit = d;
  wd.lda = d;
  wd.ldb = f;
  wd.offset = expert_offset;
  wd.E = E;
  wd.head = head;
  wd.C = C;
  wd.zero = (const bf16_t*)(w + L.zero);
  wd.out0 = (bf16_t*)dw_down;
  wd.out1 = (bf16_t*)dw_down;
  if ((err = run_wgrad(wd, st)) != hipSuccess) return err;
  WgradArgs wu = wd;
  wu.A = dau;
  wu.B = (const bf16_t*)ring_x;
  wu.M = 2 * f;
  wu.N = d;
  wu.msplit = f;
  wu.lda = 2 * f;
  wu.ldb = d;
  wu.out0 = (bf16_t*)dw_gate;
  wu.out1 = (bf16_t*)dw_up;
  if ((err = run_wgrad(wu, st)) != hipSuccess) return err;
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- MXFP8 backward
// The MXFP8 layer's backward: every GEMM takes its two operands MX-quantised (E4M3, one
// E8M0 scale per 32) along its own reduction dimension, with fp32 accumulation; the
// SwiGLU backward and the router part are the bf16 backward's.
//   down dgrad     dH_raw = Q_d(dY) Q_d(W_down)     the MX grouped GEMM (gemm.hip) on dY
//                  quantised along d into ring order and W_down^T quantised along d
//                  (moe_quantize_mx_t); dH_raw in fp32
//   SwiGLU bwd     per copy: dg (one fixed-order sum over f), dA, dU, g H in fp32, and dA|dU
//                  quantised along f for the next GEMM
//   gate/up dgrad  dX_c = [Q_f(dA) | Q_f(dU)] [Q_f(W_gate) ; Q_f(W_up)]: the same GEMM
//                  with K = 2f over [W_gate^T | W_up^T] quantised along f
//   wgrad          dW = Q_t(.)^T Q_t(.): each expert's ring rows quantised along the token
//                  axis in blocks of 32 aligned to the segment's end (its last slot, where
//                  the weight gradients start), decoded to bf16 (every MX value is a bf16
//                  value), then the bf16 weight-gradient kernel above.  The products
//                  are those of the MX operands; the token axis is these operands' row
//                  axis, which the scaled MFMA (K along a lane's registers) cannot stream
//                  without a transposed copy, and the kernel is bound by writing dW.

// dy[t] MX-quantised along d (blocks of 32, 4 lanes each) into the k ring slots of its
// copies: codes [C, d], scales [d/128][C][4].
__global__ __launch_bounds__(256) void gather_mx_kernel(const bf16_t* __restrict__ src,
                                                        const int32_t* __restrict__ copy_slot,
                                                        int k, int d, int64_t C,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  const int64_t t = blockIdx.x;
  __shared__ int64_t slots[64];
  if (threadIdx.x < k) slots[threadIdx.x] = copy_slot[t * k + threadIdx.x];
  __syncthreads();
  const int nv = d / 8;
  const int iters = (nv + 255) / 256;   // uniform trip count: all lanes join the shuffles
  for (int it = 0; it < iters; ++it) {
    const int v = it * 256 + threadIdx.x;
    const bool ok = v < nv;
    const u32x4 w = ok ? ((const u32x4*)(src + t * d))[v] : u32x4{0, 0, 0, 0};
    float fv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) { fv[2 * q] = lo_bf(w[q]); fv[2 * q + 1] = hi_bf(w[q]); }
    float am = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) am = fmaxf(am, fabsf(fv[q]));
    am = group_max<4>(am);
    const int X = mx_block_exp(am);
    const uint32_t lo = e4m3_encode4(fv[0], fv[1], fv[2], fv[3], X);
    const uint32_t hi = e4m3_encode4(fv[4], fv[5], fv[6], fv[7], X);
    if (ok)
      for (int j = 0; j < k; ++j) {
        *(u32x2*)(codes + slots[j] * d + (int64_t)v * 8) = u32x2{lo, hi};
        if ((v & 3) == 0)
          scales[((int64_t)(v / 16) * C + slots[j]) * 4 + ((v / 4) & 3)] = (uint8_t)(X + 127);
      }
  }
}

// Two values through their E4M3 codes and back, packed as bf16 (a in the low half): each
// value times 2^-X, clamped to +-448, converted to E4M3 with round to nearest even (the
// codes of e4m3_encode), the pair decoded by the hardware fp8 -> fp32 conversion (exact:
// every E4M3 value is an fp32 value) and scaled back by 2^X, where decoding the codes bit by
// bit took a few dozen instructions per value.
typedef float f32x2_rt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3_round_trip2(float a, float b, int Xa, int Xb) {
  const float ca = __builtin_amdgcn_fmed3f(ldexpf(a, -Xa), -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(ldexpf(b, -Xb), -448.0f, 448.0f);
  const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
  const f32x2_rt v = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
  return pack_bf2(ldexpf(v[0], Xa), ldexpf(v[1], Xb));
}
// Every expert's ring rows of a bf16 src MX round-tripped along the token axis into dst
// [C, cols] bf16: blocks of 32 rows aligned to the segment's end.  src is ring-ordered
// [C, cols] (dst may be src itself), or with src_map token-major [T, cols], ring slot s taking
// row src_map[s] / kdiv.  blocks: the tile list of 32-row tiles; tile (e, 32 q) is taken as
// the q-th block from the end, rows [n_e - 32 (q + 1), n_e - 32 q) of the segment (the first
// block is the partial one).  One thread per 8 consecutive columns: the block's rows are
// read once into registers (16-byte pieces, all in flight together) and written in 16-byte
// pieces; a thread owns its columns in every row of the block, so the round trip may be in
// place.  (One thread per column with 2-byte accesses: 735 us per launch at 8,192 skewed
// tokens; two passes over the rows with a bit-level decode: 352 us; now ~290 us.)  The
// decoded values are bf16 values (3 significant bits and a power-of-two scale).
__global__ __launch_bounds__(256) void token_quant_kernel(
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ nblocks,
    const int32_t* __restrict__ offset, int64_t head, int64_t C, int cols,
    const bf16_t* src, bf16_t* dst, const int32_t* __restrict__ src_map, int kdiv) {
  const int bi = blockIdx.x;
  if (bi >= *nblocks) return;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  // the block's coordinates are uniform over the workgroup: kept in scalar registers
  const int e = __builtin_amdgcn_readfirstlane(blocks[2 * bi]);
  const int q = __builtin_amdgcn_readfirstlane(blocks[2 * bi + 1]) / 32;
  const int32_t seg = __builtin_amdgcn_readfirstlane(offset[e]);
  const int n = __builtin_amdgcn_readfirstlane(offset[e + 1]) - seg;
  const int hi = n - 32 * q, lo = max(0, hi - 32);
  // lane i of each wavefront holds the source row of block row lo + i (one vector load of
  // the map, read back per row by readlane: 32 scalar loads held too many registers); every
  // lane takes part, before the lanes past the last column leave
  int srow;
  {
    const int64_t sl = ring_slot(head, seg, min(lo + (int)(threadIdx.x & 31), hi - 1), C);
    srow = src_map ? src_map[sl] / kdiv : (int)sl;
  }
  if (c >= cols) return;
  // the block's (at most 32) row pieces are held in registers, read once
  u32x4 w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (lo + i < hi) {
      const int64_t sr = __builtin_amdgcn_readlane(srow, i);
      w[i] = *(const u32x4*)(src + sr * cols + c);
    }
  float am[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) am[j] = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (lo + i < hi)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        am[2 * k] = fmaxf(am[2 * k], fabsf(lo_bf(w[i][k])));
        am[2 * k + 1] = fmaxf(am[2 * k + 1], fabsf(hi_bf(w[i][k])));
      }
  int X[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) X[j] = mx_block_exp(am[j]);
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (lo + i < hi) {
      u32x4 out;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        out[k] = e4m3_round_trip2(lo_bf(w[i][k]), hi_bf(w[i][k]), X[2 * k], X[2 * k + 1]);
      *(u32x4*)(dst + ring_slot(head, seg, lo + i, C) * cols + c) = out;
    }
}

// The SwiGLU backward of the MXFP8 backward with both of its quantisations, per 32-row token
// block (the blocks of token_quant_kernel).  Per copy, from dH_raw (fp32 [C, f]) and the
// saved A|U: dg = sum_i dH_raw_i h_i (lane partials in column order, then the wavefront's
// fixed butterfly), dA|dU quantised along f (codes [C, 2f], scales [2f/128][C][4], as the
// gate/up dgrad reads them), and dA|dU and g·h round-tripped along the token axis into dau16
// and gh16 (bf16 [C, 2f] and [C, f], the weight gradients' operands).  The block's column
// maxima are gathered in LDS and the values recomputed from the same inputs for the round
// trip (read again; at 8,192 skewed tokens the second read mostly misses L2: 1.37 GB
// fetched for 0.67 GB of inputs), instead of being stored in fp32 and read back by a
// separate round-trip pass: skewed MXFP8 backward 8.35 -> 7.74 ms (same GPU, gradients
// bitwise equal).  Four wavefronts, each the block rows lo + wave + 4 j, one at a time.
__global__ __launch_bounds__(256) void swiglu_bwd_mx_tq_kernel(
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ nblocks,
    const int32_t* __restrict__ offset, int64_t head, int64_t C, int f,
    const float* __restrict__ dhr, const bf16_t* __restrict__ saved_au,
    const int32_t* __restrict__ slot_copy, const float* __restrict__ gate,
    uint8_t* __restrict__ dau_q, uint8_t* __restrict__ dau_s, bf16_t* __restrict__ dau16,
    bf16_t* __restrict__ gh16, float* __restrict__ dg_out) {
  extern __shared__ uint32_t colmax[];   // [3][f]: |dA|, |dU|, |g h| maxima over the block's rows
  const int bi = blockIdx.x;
  if (bi >= *nblocks) return;
  const int e = __builtin_amdgcn_readfirstlane(blocks[2 * bi]);
  const int q = __builtin_amdgcn_readfirstlane(blocks[2 * bi + 1]) / 32;
  const int32_t seg = __builtin_amdgcn_readfirstlane(offset[e]);
  const int n = __builtin_amdgcn_readfirstlane(offset[e + 1]) - seg;
  const int hi = n - 32 * q, lo = max(0, hi - 32);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nv = f / 8, iters = (nv + 63) / 64;
  for (int i = threadIdx.x; i < 3 * f; i += 256) colmax[i] = 0u;
  __syncthreads();
  // one row's values at the 8 columns 8 v .. 8 v + 7 (ok: v inside the row)
  auto row_values = [&](int64_t s, float g, int v, bool ok, float (&da)[8], float (&du)[8],
                        float (&hh)[8], float& dgp) __attribute__((always_inline)) {
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const f32x4 wd0 = ok ? ((const f32x4*)(dhr + s * f))[2 * v] : z4;
    const f32x4 wd1 = ok ? ((const f32x4*)(dhr + s * f))[2 * v + 1] : z4;
    const u32x4 wa = ok ? ((const u32x4*)(saved_au + s * 2 * f))[v] : u32x4{0, 0, 0, 0};
    const u32x4 wu = ok ? ((const u32x4*)(saved_au + s * 2 * f + f))[v] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float dh_raw = k < 4 ? wd0[k] : wd1[k - 4];
      const float a = k & 1 ? hi_bf(wa[k / 2]) : lo_bf(wa[k / 2]);
      const float u = k & 1 ? hi_bf(wu[k / 2]) : lo_bf(wu[k / 2]);
      const float sg = sigm(a);
      const float h = a * sg * u;
      dgp = fmaf(dh_raw, h, dgp);
      const float dh = g * dh_raw;
      da[k] = dh * u * sg * (1.f + a * (1.f - sg));
      du[k] = dh * a * sg;
      hh[k] = g * h;
    }
  };
  // pass 1: f-axis codes, dg, the block's column maxima
  for (int r = lo + wave; r < hi; r += 4) {
    const int64_t s = ring_slot(head, seg, r, C);
    const float g = gate[slot_copy[s]];
    float dgp = 0.f;
    for (int it = 0; it < iters; ++it) {
      const int v = it * 64 + lane;
      const bool ok = v < nv;
      float da[8], du[8], hh[8];
      row_values(s, g, v, ok, da, du, hh, dgp);
      float ama = 0.f, amu = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) { ama = fmaxf(ama, fabsf(da[k])); amu = fmaxf(amu, fabsf(du[k])); }
      ama = group_max<4>(ama);
      amu = group_max<4>(amu);
      const int Xa = mx_block_exp(ama), Xu = mx_block_exp(amu);
      if (ok) {
        const uint32_t ca0 = e4m3_encode4(da[0], da[1], da[2], da[3], Xa);
        const uint32_t ca1 = e4m3_encode4(da[4], da[5], da[6], da[7], Xa);
        const uint32_t cu0 = e4m3_encode4(du[0], du[1], du[2], du[3], Xu);
        const uint32_t cu1 = e4m3_encode4(du[4], du[5], du[6], du[7], Xu);
        *(u32x2*)(dau_q + s * 2 * f + (int64_t)v * 8) = u32x2{ca0, ca1};
        *(u32x2*)(dau_q + s * 2 * f + f + (int64_t)v * 8) = u32x2{cu0, cu1};
        if ((v & 3) == 0) {
          const int ba = v / 4, bu = f / 32 + v / 4;   // block indices along the 2f row
          dau_s[((int64_t)(ba / 4) * C + s) * 4 + (ba & 3)] = (uint8_t)(Xa + 127);
          dau_s[((int64_t)(bu / 4) * C + s) * 4 + (bu & 3)] = (uint8_t)(Xu + 127);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {   // non-negative floats order as their bits
          atomicMax(&colmax[8 * v + k], __float_as_uint(fabsf(da[k])));
          atomicMax(&colmax[f + 8 * v + k], __float_as_uint(fabsf(du[k])));
          atomicMax(&colmax[2 * f + 8 * v + k], __float_as_uint(fabsf(hh[k])));
        }
      }
    }
    const float dg = wave_sum(dgp);
    if (lane == 0) dg_out[s] = dg;
  }
  __syncthreads();
  // pass 2: the token-axis round trip of the recomputed values
  for (int it = 0; it < iters; ++it) {
    const int v = it * 64 + lane;
    const bool ok = v < nv;
    if (!ok) continue;
    int Xa[8], Xu[8], Xh[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      Xa[k] = mx_block_exp(__uint_as_float(colmax[8 * v + k]));
      Xu[k] = mx_block_exp(__uint_as_float(colmax[f + 8 * v + k]));
      Xh[k] = mx_block_exp(__uint_as_float(colmax[2 * f + 8 * v + k]));
    }
    for (int r = lo + wave; r < hi; r += 4) {
      const int64_t s = ring_slot(head, seg, r, C);
      const float g = gate[slot_copy[s]];
      float da[8], du[8], hh[8], dgp = 0.f;
      row_values(s, g, v, true, da, du, hh, dgp);
      u32x4 oa, ou, oh;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        oa[k] = e4m3_round_trip2(da[2 * k], da[2 * k + 1], Xa[2 * k], Xa[2 * k + 1]);
        ou[k] = e4m3_round_trip2(du[2 * k], du[2 * k + 1], Xu[2 * k], Xu[2 * k + 1]);
        oh[k] = e4m3_round_trip2(hh[2 * k], hh[2 * k + 1], Xh[2 * k], Xh[2 * k + 1]);
      }
      ((u32x4*)(dau16 + s * 2 * f))[v] = oa;
      ((u32x4*)(dau16 + s * 2 * f + f))[v] = ou;
      ((u32x4*)(gh16 + s * f))[v] = oh;
    }
  }
}

struct BwdMxLayout {
  size_t tiles, blocks, rdy, rq, rqs, dhr, dauq, daus, dau16, gh16, dg, dxc, dl, xr,
      rpart, rfirst, zero, total;
};

static BwdMxLayout bwd_mx_layout(int64_t T, int64_t C, int d, int E, int k, int f) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const int64_t n = T * k;
  BwdMxLayout L;
  size_t o = 0;
  L.tiles = o;  o += al((size_t)(2 * bwd_max_tiles(n, E) + 64) * 4);
  L.blocks = o; o += al((size_t)(2 * ((n + 31) / 32 + E) + 64) * 4);
  L.rdy = o;    o += al((size_t)C * d * 2);
  L.rq = o;     o += al((size_t)C * d);
  L.rqs = o;    o += al((size_t)C * (d / 32));
  L.dhr = o;    o += al((size_t)C * f * 4);
  L.dauq = o;   o += al((size_t)C * 2 * f);
  L.daus = o;   o += al((size_t)C * (2 * f / 32));
  L.dau16 = o;  o += al((size_t)C * 2 * f * 2);
  L.gh16 = o;   o += al((size_t)C * f * 2);
  L.dg = o;     o += al((size_t)C * 4);
  L.dxc = o;    o += al((size_t)C * d * 2);
  L.dl = o;     o += al((size_t)C * 4);
  L.xr = o;     o += al((size_t)C * d * 2);
  L.rpart = o;  o += al((size_t)bwd_max_tiles(n, E) * d * 4);
  L.rfirst = o; o += al((size_t)E * 4);
  L.zero = o;   o += 1024;
  L.total = o;
  return L;
}

size_t backward_mx_workspace_bytes(int64_t T, int64_t C, int d, int E, int k, int f) {
  return bwd_mx_layout(T, C, d, E, k, f).total;
}

hipError_t launch_backward_mx(const void* dy, const void* x, const float* w_r,
                              const int32_t* topk_idx, const float* topk_gate,
                              const int32_t* expert_offset, const int32_t* copy_slot,
                              const int32_t* slot_copy, int64_t head, int64_t C,
                              const void* saved_au, const uint8_t* w_gu_t,
                              const uint8_t* w_gu_t_scale, const uint8_t* w_down_t,
                              const uint8_t* w_down_t_scale, int64_t T, int d, int E, int k,
                              int f, void* dx, void* dw_gate, void* dw_up, void* dw_down,
                              float* dw_r, void* ws, hipStream_t st) {
  if (d % BT || f % BT || 3 * f * 4 > 160 * 1024) return hipErrorInvalidValue;
  const BwdMxLayout L = bwd_mx_layout(T, C, d, E, k, f);
  uint8_t* w = (uint8_t*)ws;
  int32_t* ntiles = (int32_t*)(w + L.tiles);
  int32_t* tiles = ntiles + 64;
  int32_t* nblocks = (int32_t*)(w + L.blocks);
  int32_t* blocks = nblocks + 64;
  bf16_t* rdy = (bf16_t*)(w + L.rdy);
  float* dhr = (float*)(w + L.dhr);
  bf16_t* dau16 = (bf16_t*)(w + L.dau16);
  bf16_t* gh16 = (bf16_t*)(w + L.gh16);
  float* dg = (float*)(w + L.dg);
  bf16_t* dxc = (bf16_t*)(w + L.dxc);
  float* dl = (float*)(w + L.dl);
  bf16_t* xr = (bf16_t*)(w + L.xr);
  const int64_t n = T * k;
  const int max_tiles = bwd_max_tiles(n, E);
  const int max_blocks = (int)((n + 31) / 32) + E;

  hipError_t err = launch_build_tiles(expert_offset, E, BT, tiles, ntiles, st);
  if (err == hipSuccess) err = launch_build_tiles(expert_offset, E, 32, blocks, nblocks, st);
  if (err != hipSuccess) return err;
  zero_fill_kernel<<<1, 256, 0, st>>>((uint32_t*)(w + L.zero), 256);
  gather_mx_kernel<<<(unsigned)T, 256, 0, st>>>((const bf16_t*)dy, copy_slot, k, d, C,
                                                w + L.rq, w + L.rqs);
  // down dgrad: dH_raw = Q_d(dY) Q_d(W_down)
  GemmArgs g{};
  g.A = w + L.rq;
  g.A_scale = w + L.rqs;
  g.B0 = w_down_t;
  g.B0_scale = w_down_t_scale;
  g.K = d;
  g.N = f;
  g.offset = expert_offset;
  g.tiles = tiles;
  g.ntiles = ntiles;
  g.head = head;
  g.C = C;
  g.out = (uint8_t*)dhr;
  g.a_rows = C;
  g.b_rows = (int64_t)E * f;
  if ((err = launch_mx_plain_gemm128(g, n, E, true, st)) != hipSuccess) return err;
  // the block's column maxima: 3 f words of dynamic LDS
  if ((err = hipFuncSetAttribute((const void*)swiglu_bwd_mx_tq_kernel,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 3 * f * 4)) != hipSuccess)
    return err;
  swiglu_bwd_mx_tq_kernel<<<(unsigned)max_blocks, 256, (size_t)3 * f * 4, st>>>(
      blocks, nblocks, expert_offset, head, C, f, dhr, (const bf16_t*)saved_au, slot_copy,
      topk_gate, w + L.dauq, w + L.daus, dau16, gh16, dg);
  // gate/up dgrad: dX_c = [Q_f(dA) | Q_f(dU)] [Q_f(W_gate); Q_f(W_up)]
  GemmArgs g2 = g;
  g2.A = w + L.dauq;
  g2.A_scale = w + L.daus;
  g2.B0 = w_gu_t;
  g2.B0_scale = w_gu_t_scale;
  g2.K = 2 * f;
  g2.N = d;
  g2.out = (uint8_t*)dxc;
  g2.b_rows = (int64_t)E * d;
  if ((err = launch_mx_plain_gemm128(g2, n, E, false, st)) != hipSuccess) return err;
  token_kernel<<<(unsigned)T, 256, 0, st>>>(copy_slot, topk_idx, topk_gate, dg, 1, dxc, w_r, d,
                                            k, dl, (bf16_t*)dx);
  float* rpart = (float*)(w + L.rpart);
  int32_t* rfirst = (int32_t*)(w + L.rfirst);
  router_wgrad_part_kernel<<<dim3(max_tiles, (d / 8 + 127) / 128), 128, 0, st>>>(
      tiles, ntiles, expert_offset, head, C, (const bf16_t*)x, dl, d, rpart, rfirst, slot_copy, k);
  router_wgrad_sum_kernel<<<dim3(E, (d / 4 + 255) / 256), 256, 0, st>>>(expert_offset, rfirst,
                                                                        rpart, d, dw_r);
  // weight gradients on the operands quantised along the token axis; dy and x are read in
  // place, each ring slot's token row through slot_copy (no copy into ring order first)
  token_quant_kernel<<<dim3(max_blocks, (d + 2047) / 2048), 256, 0, st>>>(
      blocks, nblocks, expert_offset, head, C, d, (const bf16_t*)dy, rdy, slot_copy, k);
  token_quant_kernel<<<dim3(max_blocks, (d + 2047) / 2048), 256, 0, st>>>(
      blocks, nblocks, expert_offset, head, C, d, (const bf16_t*)x, xr, slot_copy, k);
  WgradArgs wd{};
  wd.A = rdy;
  wd.B = gh16;
  wd.M = d;
  wd.N = f;
  wd.msplit = d;
  wd.lda = d;
  wd.ldb = f;
  wd.offset = expert_offset;
  wd.E = E;
  wd.head = head;
  wd.C = C;
  wd.zero = (const bf16_t*)(w + L.zero);
  wd.out0 = (bf16_t*)dw_down;
  wd.out1 = (bf16_t*)dw_down;
  if ((err = run_wgrad(wd, st)) != hipSuccess) return err;
  WgradArgs wu = wd;
  wu.A = dau16;
  wu.B = xr;
  wu.M = 2 * f;
  wu.N = d;
  wu.msplit = f;
  wu.lda = 2 * f;
  wu.ldb = d;
  wu.out0 = (bf16_t*)dw_gate;
  wu.out1 = (bf16_t*)dw_up;
  if ((err = run_wgrad(wu, st)) != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace moe
