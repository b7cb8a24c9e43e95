// Expert FFN as grouped GEMMs over the ring segments.
//
// Every expert e owns the ring rows (head + offset[e] + i) mod C, i < count_e
// (the expert-centric scheme; toolnavs.com warp-decode page, "Cursor a réécrit
// le décodage de MoE").  Per expert:
//   GEMM-1   [A|U] = X_e [W_gate[e]; W_up[e]]^T, epilogue H = silu(A) * U
//   GEMM-2   Y_e   = H W_down[e]^T
// Both are "NT" products (operands K-contiguous), so one kernel shape serves
// both.  Output tiles are computed by exactly one workgroup with a fixed K
// order: the result does not depend on scheduling (deterministic, as the
// megakernel paragraph of the dzen.guru page requires).
//
// Tile lists are built on the device from expert_offset (no host sync); the
// grid is sized from the host-known bound sum_e ceil(n_e / BM) <= n / BM + E.
//
// Paths: bf16 MFMA (v_mfma_f32_32x32x16_bf16), MX fp8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 operands, one E8M0 scale per 32 K),
// and an fp32 VALU path for fp32 layers.
#include "common.h"
#include "kernels.h"

namespace moe {

// ============================================================ tile list
// tiles[2*i] = expert, tiles[2*i+1] = first row of the tile inside the segment;
// *ntiles = number of valid entries.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offset,
                                                           int E, int BM,
                                                           int32_t* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles) {
  __shared__ int32_t sc[1024];
  const int e = threadIdx.x;
  const int32_t cnt = e < E ? offset[e + 1] - offset[e] : 0;
  const int32_t nt = (cnt + BM - 1) / BM;
  sc[e] = nt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t v = e >= o ? sc[e - o] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  const int32_t start = sc[e] - nt;
  for (int32_t i = 0; i < nt; ++i) {
    tiles[2 * (start + i)] = e;
    tiles[2 * (start + i) + 1] = i * BM;
  }
  if (e == 1023) *ntiles = sc[1023];
}

hipError_t launch_build_tiles(const int32_t* expert_offset, int E, int BM, int32_t* tiles,
                              int32_t* ntiles, hipStream_t st) {
  build_tiles_kernel<<<1, 1024, 0, st>>>(expert_offset, E, BM, tiles, ntiles);
  return hipGetLastError();
}

// ============================================================ bf16 / MX MFMA GEMM
// Workgroup tile BM x BN, K staged in 128-byte row slices (64 bf16 or 128 fp8)
// through double-buffered LDS.  16-byte chunks of a row are XOR-swizzled by
// (row & 7) so that the fragment reads of 8 consecutive rows hit distinct
// banks.  4 waves in a WM x WN grid; each wave owns FM x FN 32x32 fragments.
//
// SWIGLU: the B tile stacks BN/2 rows of W_gate over the same BN/2 rows of
// W_up, and every wave holds matching gate and up fragments, so the epilogue
// forms h = silu(a) * u in registers.
constexpr int KBYTES = 128;            // bytes of K per row per stage
constexpr int CHUNKS = KBYTES / 16;    // 16-byte chunks per row slice

__device__ __forceinline__ int swz(int r, int c) { return r * KBYTES + ((c ^ (r & 7)) << 4); }

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
};

template <int BM, int BN, int WM, int WN, bool SWIGLU, bool MX>
__global__ __launch_bounds__(256) void gg_mfma_kernel(GemmArgs p) {
  constexpr int EB = MX ? 1 : 2;                 // element bytes
  constexpr int WTM = BM / WM, WTN = BN / WN;    // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_LD = BM * CHUNKS / 256, B_LD = BN * CHUNKS / 256;   // 16B loads per thread
  static_assert(BM * CHUNKS % 256 == 0 && BN * CHUNKS % 256 == 0, "tile / thread mismatch");
  static_assert(!SWIGLU || (FN % 2 == 0), "gate/up fragments come in pairs");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* As = lds;                               // [2][BM * KBYTES]
  uint8_t* Bs = lds + 2 * BM * KBYTES;             // [2][BN * KBYTES]
  uint32_t* Asc = (uint32_t*)(Bs + 2 * BN * KBYTES);   // MX: [2][BM]
  uint32_t* Bsc = Asc + 2 * BM;                        // MX: [2][BN]

  const int mt = blockIdx.y;
  if (mt >= *p.ntiles) return;
  const int e = p.tiles[2 * mt];
  const int row0 = p.tiles[2 * mt + 1];
  const int32_t seg = p.offset[e];
  const int rows = min(BM, p.offset[e + 1] - seg - row0);
  const int n0 = blockIdx.x * (SWIGLU ? BN / 2 : BN);   // first output column

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t Kb = (int64_t)p.K * EB;                 // row bytes

  // per-thread global row pointers (rows past the segment reuse its last row)
  const uint8_t* a_src[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = (tid + 256 * i) / CHUNKS;
    const int64_t s = ring_slot(p.head, seg, row0 + min(r, rows - 1), p.C);
    a_src[i] = p.A + s * Kb + ((tid + 256 * i) % CHUNKS) * 16;
  }
  const uint8_t* b_src[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = (tid + 256 * i) / CHUNKS;
    int64_t wrow;
    const uint8_t* base;
    if (SWIGLU) {
      const bool up = r >= BN / 2;
      wrow = (int64_t)e * p.N + min(n0 + (up ? r - BN / 2 : r), p.N - 1);
      base = up ? p.B1 : p.B0;
    } else {
      wrow = (int64_t)e * p.N + min(n0 + r, p.N - 1);
      base = p.B0;
    }
    b_src[i] = base + wrow * Kb + ((tid + 256 * i) % CHUNKS) * 16;
  }

  u32x4 ra[A_LD], rb[B_LD];
  uint32_t rsa = 0, rsb[2] = {0, 0};
  auto gload = [&](int kt) {
    const int64_t kb = (int64_t)kt * KBYTES;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *(const u32x4*)(a_src[i] + kb);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *(const u32x4*)(b_src[i] + kb);
    if (MX) {
      // one scale dword (4 blocks of 32) per row: threads 0..BM-1 take A rows,
      // threads 0..BN-1 take B rows
      if (tid < BM) {
        const int64_t s = ring_slot(p.head, seg, row0 + min(tid, rows - 1), p.C);
        rsa = *(const uint32_t*)(p.A_scale + s * (p.K / 32) + kt * 4);
      }
#pragma unroll
      for (int h = 0; h < (BN + 255) / 256; ++h) {
        const int r = tid + 256 * h;
        if (r < BN) {
          int64_t wrow;
          const uint8_t* sbase;
          if (SWIGLU) {
            const bool up = r >= BN / 2;
            wrow = (int64_t)e * p.N + min(n0 + (up ? r - BN / 2 : r), p.N - 1);
            sbase = up ? p.B1_scale : p.B0_scale;
          } else {
            wrow = (int64_t)e * p.N + min(n0 + r, p.N - 1);
            sbase = p.B0_scale;
          }
          rsb[h] = *(const uint32_t*)(sbase + wrow * (p.K / 32) + kt * 4);
        }
      }
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* as = As + buf * BM * KBYTES;
    uint8_t* bs = Bs + buf * BN * KBYTES;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + 256 * i;
      *(u32x4*)(as + swz(q / CHUNKS, q % CHUNKS)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int q = tid + 256 * i;
      *(u32x4*)(bs + swz(q / CHUNKS, q % CHUNKS)) = rb[i];
    }
    if (MX) {
      if (tid < BM) Asc[buf * BM + tid] = rsa;
#pragma unroll
      for (int h = 0; h < (BN + 255) / 256; ++h)
        if (tid + 256 * h < BN) Bsc[buf * BN + tid + 256 * h] = rsb[h];
    }
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

  const int KT = (int)(Kb / KBYTES);
  gload(0);
  sstore(0);
  __syncthreads();
  const int lr = lane & 31, lg = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t* as = As + cur * BM * KBYTES;
    const uint8_t* bs = Bs + cur * BN * KBYTES;
    if constexpr (!MX) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {           // 4 x 16 K per stage
        const int c = kk * 2 + lg;
        bf16x8 af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * WTM + i * 32 + lr;
          af[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(as + swz(r, c)));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = brow(j) + lr;
          bfr[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(bs + swz(r, c)));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
      const uint32_t* asc = Asc + cur * BM;
      const uint32_t* bsc = Bsc + cur * BN;
      // Operand layout of the 32x32x64 E4M3 MFMA: of a lane's 32 bytes, bytes
      // 0-15 belong to the first 32-element scale block of the 64-wide K step and
      // bytes 16-31 to the second; lane group g (= lane / 32) holds elements
      // [16g, 16g + 16) of each block and supplies the scale of block g.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {           // 2 x 64 K per stage
        const int ca = kk * 4 + lg, cb = kk * 4 + 2 + lg;   // 16-byte chunks of this lane
        const int blk = kk * 2 + lg;             // its scale byte inside the row's dword
        i32x8 af[FM], bfr[FN];
        int sa[FM], sb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * WTM + i * 32 + lr;
          const u32x4 lo = *(const u32x4*)(as + swz(r, ca));
          const u32x4 hi = *(const u32x4*)(as + swz(r, cb));
          af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          sa[i] = (int)((asc[r] >> (8 * blk)) & 0xffu);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = brow(j) + lr;
          const u32x4 lo = *(const u32x4*)(bs + swz(r, ca));
          const u32x4 hi = *(const u32x4*)(bs + swz(r, cb));
          bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          sb[j] = (int)((bsc[r] >> (8 * blk)) & 0xffu);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bfr[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
      }
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // acc register r of a 32x32 fragment: row 8*(r/4) + 4*(lane/32) + r%4, column lane%32.
  if (SWIGLU) {
    constexpr int HALF = FN / 2;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const int col = n0 + wn * (WTN / 2) + j * 32 + lr;   // f index
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * WTM + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
          const float a = acc[i][j][r], u = acc[i][j + HALF][r];
          const float h = silu(a) * u;
          const bool live = m < rows && col < p.N;
          const int64_t s = ring_slot(p.head, seg, row0 + min(m, rows - 1), p.C);
          if (MX) {
            // the 32 columns of one row's block sit in the 32 lanes of a half-wave
            const float am = group_max<32>(fabsf(h));
            const int X = mx_block_exp(am);
            if (live) {
              p.out[s * p.N + col] = (uint8_t)e4m3_encode(h, X);
              if (lr == 0) p.out_scale[s * (p.N / 32) + col / 32] = (uint8_t)(X + 127);
            }
          } else if (live) {
            ((uint16_t*)p.out)[s * p.N + col] = f2bf(h);
            if (p.saved_au) {
              p.saved_au[s * 2 * p.N + col] = f2bf(a);
              p.saved_au[s * 2 * p.N + p.N + col] = f2bf(u);
            }
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WTN + j * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * WTM + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
          if (m < rows && col < p.N) {
            const int64_t s = ring_slot(p.head, seg, row0 + m, p.C);
            ((uint16_t*)p.out)[s * p.N + col] = f2bf(acc[i][j][r]);
          }
        }
      }
  }
}

template <int BM, int BN, int WM, int WN, bool SWIGLU, bool MX>
static hipError_t run_mfma(const GemmArgs& a, int max_tiles, hipStream_t st) {
  const int nt = SWIGLU ? (a.N + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  const size_t lds = 2 * (BM + BN) * KBYTES + (MX ? 2 * (BM + BN) * 4 : 0);
  auto kern = gg_mfma_kernel<BM, BN, WM, WN, SWIGLU, MX>;
  static bool attr_set = false;   // opt in to more than 64 KB of LDS once per process
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  kern<<<dim3(nt, max_tiles), 256, lds, st>>>(a);
  return hipGetLastError();
}

// ============================================================ fp32 VALU path
// 64 rows x 64 columns per workgroup, 256 threads with 4x4 outputs each, K in
// steps of 16 through LDS.  SWIGLU keeps a gate and an up accumulator.
constexpr int FT_M = 64, FT_N = 64, FT_K = 16;

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gg_f32_kernel(const float* __restrict__ A,
                                                     const float* __restrict__ B0,
                                                     const float* __restrict__ B1, int K, int N,
                                                     const int32_t* __restrict__ offset,
                                                     const int32_t* __restrict__ tiles,
                                                     const int32_t* __restrict__ ntiles,
                                                     int64_t head, int64_t C,
                                                     float* __restrict__ out) {
  __shared__ float as[FT_K][FT_M + 4];
  __shared__ float bs0[FT_K][FT_N + 4];
  __shared__ float bs1[SWIGLU ? FT_K : 1][FT_N + 4];
  const int mt = blockIdx.y;
  if (mt >= *ntiles) return;
  const int e = tiles[2 * mt], row0 = tiles[2 * mt + 1];
  const int32_t seg = offset[e];
  const int rows = min(FT_M, offset[e + 1] - seg - row0);
  const int n0 = blockIdx.x * FT_N;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float ag[4][4] = {}, au[4][4] = {};
  const int r = tid >> 2, kq = (tid & 3) * 4;   // staging: row r, k offsets kq..kq+3
  const int64_t srow = ring_slot(head, seg, row0 + min(r, rows - 1), C);
  const int64_t wrow = (int64_t)e * N + min(n0 + r, N - 1);
  for (int k0 = 0; k0 < K; k0 += FT_K) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = k0 + kq + q;
      as[kq + q][r] = kk < K ? A[srow * K + kk] : 0.f;
      bs0[kq + q][r] = kk < K ? B0[wrow * K + kk] : 0.f;
      if (SWIGLU) bs1[kq + q][r] = kk < K ? B1[wrow * K + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FT_K; ++kk) {
      float a[4], b[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = bs0[kk][tx * 4 + j];
        if (SWIGLU) u[j] = bs1[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ag[i][j] = fmaf(a[i], b[j], ag[i][j]);
          if (SWIGLU) au[i][j] = fmaf(a[i], u[j], au[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty * 4 + i;
    if (m >= rows) continue;
    const int64_t s = ring_slot(head, seg, row0 + m, C);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col < N) out[s * N + col] = SWIGLU ? silu(ag[i][j]) * au[i][j] : ag[i][j];
    }
  }
}

// ============================================================ launcher
// Row-tile height of the MFMA paths and the fp32 path.
constexpr int MFMA_BM = 128;

static int max_tiles_for(int64_t n, int E, int BM) { return (int)((n + BM - 1) / BM) + E; }

size_t ffn_workspace_bytes(int64_t n, int64_t C, int d, int E, int f, int dtype) {
  const int BM = dtype == 0 ? FT_M : MFMA_BM;
  size_t b = (size_t)(2 * max_tiles_for(n, E, BM) + 64) * sizeof(int32_t);
  b = (b + 255) & ~(size_t)255;
  if (dtype == 0) b += (size_t)C * f * 4;                       // H fp32
  else if (dtype == 1) b += (size_t)C * f * 2;                  // H bf16
  else b += (size_t)C * f + (size_t)C * (f / 32) + 256;         // H MX codes + scales
  return b;
}

hipError_t launch_ffn(int dtype, const void* ring_x, const uint8_t* ring_x_scale,
                      const int32_t* expert_offset, int64_t head, int64_t C, int64_t n, int d,
                      int E, int f, const void* w_gate, const void* w_up, const void* w_down,
                      const uint8_t* wg_scale, const uint8_t* wu_scale, const uint8_t* wd_scale,
                      void* ring_y, void* saved_au, void* ws, hipEvent_t* events,
                      hipStream_t st) {
  const int BM = dtype == 0 ? FT_M : MFMA_BM;
  const int max_tiles = max_tiles_for(n, E, BM);
  int32_t* ntiles = (int32_t*)ws;
  int32_t* tiles = ntiles + 64;
  size_t hoff = (size_t)(2 * max_tiles + 64) * sizeof(int32_t);
  hoff = (hoff + 255) & ~(size_t)255;
  uint8_t* H = (uint8_t*)ws + hoff;
  build_tiles_kernel<<<1, 1024, 0, st>>>(expert_offset, E, BM, tiles, ntiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  auto mark = [&](int i) { return events ? hipEventRecord(events[i], st) : hipSuccess; };
  if ((err = mark(0)) != hipSuccess) return err;

  if (dtype == 0) {
    gg_f32_kernel<true><<<dim3((f + FT_N - 1) / FT_N, max_tiles), 256, 0, st>>>(
        (const float*)ring_x, (const float*)w_gate, (const float*)w_up, d, f, expert_offset,
        tiles, ntiles, head, C, (float*)H);
    if ((err = mark(1)) != hipSuccess) return err;
    gg_f32_kernel<false><<<dim3((d + FT_N - 1) / FT_N, max_tiles), 256, 0, st>>>(
        (const float*)H, (const float*)w_down, nullptr, f, d, expert_offset, tiles, ntiles, head,
        C, (float*)ring_y);
    if ((err = mark(2)) != hipSuccess) return err;
    return hipGetLastError();
  }
  GemmArgs g1{};
  g1.A = (const uint8_t*)ring_x;
  g1.A_scale = ring_x_scale;
  g1.B0 = (const uint8_t*)w_gate;
  g1.B1 = (const uint8_t*)w_up;
  g1.B0_scale = wg_scale;
  g1.B1_scale = wu_scale;
  g1.K = d;
  g1.N = f;
  g1.offset = expert_offset;
  g1.tiles = tiles;
  g1.ntiles = ntiles;
  g1.head = head;
  g1.C = C;
  g1.out = H;
  g1.out_scale = dtype == 2 ? H + (size_t)C * f : nullptr;
  g1.saved_au = (uint16_t*)saved_au;
  GemmArgs g2 = g1;
  g2.A = H;
  g2.A_scale = g1.out_scale;
  g2.B0 = (const uint8_t*)w_down;
  g2.B1 = nullptr;
  g2.B0_scale = wd_scale;
  g2.B1_scale = nullptr;
  g2.K = f;
  g2.N = d;
  g2.out = (uint8_t*)ring_y;
  g2.out_scale = nullptr;
  g2.saved_au = nullptr;
  if (dtype == 1) err = run_mfma<MFMA_BM, 256, 2, 2, true, false>(g1, max_tiles, st);
  else err = run_mfma<MFMA_BM, 256, 2, 2, true, true>(g1, max_tiles, st);
  if (err != hipSuccess || (err = mark(1)) != hipSuccess) return err;
  if (dtype == 1) err = run_mfma<MFMA_BM, 256, 2, 2, false, false>(g2, max_tiles, st);
  else err = run_mfma<MFMA_BM, 256, 2, 2, false, true>(g2, max_tiles, st);
  if (err != hipSuccess) return err;
  return mark(2);
}

}  // namespace moe
