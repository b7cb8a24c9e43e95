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
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm_body.h"
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

template <int BM, int BN, int WM, int WN, int KB, bool SWIGLU, bool MX, int S, int POL,
          bool F32OUT = false, bool MXSAVE = false>
__global__ __launch_bounds__(WM * WN * 64) void gg_mfma_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  gg_mfma_body<BM, BN, WM, WN, KB, SWIGLU, MX, S, POL, F32OUT, MXSAVE>(p, (int)blockIdx.x, lds);
}

template <int BM, int BN, int WM, int WN, int KB, bool SWIGLU, bool MX, int S, int POL,
          bool F32OUT = false, bool MXSAVE = false>
static hipError_t run_mfma(const GemmArgs& a, int max_tiles, hipStream_t st) {
  const int nt = SWIGLU ? (a.N + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  const size_t lds = std::max<size_t>((size_t)S * StageLayout<BM, BN, KB, MX, WM * WN>::SIZE,
                                      EpiLayout<BM, BN, SWIGLU, MX>::SIZE);
  auto kern = gg_mfma_kernel<BM, BN, WM, WN, KB, SWIGLU, MX, S, POL, F32OUT, MXSAVE>;
  // opt in to more than 64 KB of LDS: a host-side attribute, set on every launch so that
  // nothing is kept between calls
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  const int64_t vmax = (int64_t)max_tiles * nt;          // bound on live tiles
  const int64_t grid = 8 * ((vmax + 7) / 8);
  kern<<<(unsigned)grid, WM * WN * 64, lds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_mx_plain_gemm128(GemmArgs& g, int64_t n, int E, bool f32_out, hipStream_t st) {
  g.rotate = kstart_rotates(false, 2, n, E, MFMA_BM);
  const int max_tiles = max_tiles_for(n, E, MFMA_BM);
  const bool nt = gemm_policy(false, 2, n, E, MFMA_BM) == 3;
  if (f32_out)
    return nt ? run_mfma<MFMA_BM, 256, 2, 4, 128, false, true, 3, 3, true>(g, max_tiles, st)
              : run_mfma<MFMA_BM, 256, 2, 4, 128, false, true, 3, 2, true>(g, max_tiles, st);
  return nt ? run_mfma<MFMA_BM, 256, 2, 4, 128, false, true, 3, 3>(g, max_tiles, st)
            : run_mfma<MFMA_BM, 256, 2, 4, 128, false, true, 3, 2>(g, max_tiles, st);
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
size_t ffn_workspace_bytes(int64_t n, int64_t C, int d, int E, int f, int dtype) {
  const int BM = dtype == 0 ? FT_M : MFMA_BM;   // the larger count of the two MFMA shapes
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
  const bool big = use_big(dtype, n, E);
  const int BM = dtype == 0 ? FT_M : big ? MFMA_BM_BIG : MFMA_BM;
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
  g1.a_rows = C;
  g1.b_rows = (int64_t)E * f;
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
  g2.b_rows = (int64_t)E * d;
  g1.rotate = kstart_rotates(true, dtype, n, E, BM);
  g2.rotate = kstart_rotates(false, dtype, n, E, BM);
  const int pol1 = gemm_policy(true, dtype, n, E, BM), pol2 = gemm_policy(false, dtype, n, E, BM);
#define RUN_POL(P, G, ...)                                                 \
  err = (P) == 3 ? run_mfma<__VA_ARGS__, 3>(G, max_tiles, st)              \
                 : run_mfma<__VA_ARGS__, 2>(G, max_tiles, st);
#define RUN_POL_MXSAVE(P, G, ...)                                              \
  err = (P) == 3 ? run_mfma<__VA_ARGS__, 3, false, true>(G, max_tiles, st)     \
                 : run_mfma<__VA_ARGS__, 2, false, true>(G, max_tiles, st);
  const bool mxsave = dtype == 2 && saved_au != nullptr;
  if (big && mxsave) { RUN_POL_MXSAVE(pol1, g1, MFMA_BM_BIG, 256, 4, 2, 128, true, true, 2) }
  else if (big && dtype == 2) { RUN_POL(pol1, g1, MFMA_BM_BIG, 256, 4, 2, 128, true, true, 2) }
  else if (big) { RUN_POL(pol1, g1, MFMA_BM_BIG, 256, 4, 4, 128, true, false, 2) }
  else if (dtype == 1) { RUN_POL(pol1, g1, MFMA_BM, 256, 2, 4, 128, true, false, 3) }
  else if (mxsave) { RUN_POL_MXSAVE(pol1, g1, MFMA_BM, 256, 2, 4, 128, true, true, 3) }
  else { RUN_POL(pol1, g1, MFMA_BM, 256, 2, 4, 128, true, true, 3) }
#undef RUN_POL_MXSAVE
  if (err != hipSuccess || (err = mark(1)) != hipSuccess) return err;
  if (big && dtype == 2) { RUN_POL(pol2, g2, MFMA_BM_BIG, 256, 4, 2, 128, false, true, 2) }
  else if (big) { RUN_POL(pol2, g2, MFMA_BM_BIG, 256, 4, 4, 128, false, false, 2) }
  else if (dtype == 1) { RUN_POL(pol2, g2, MFMA_BM, 256, 2, 4, 128, false, false, 3) }
  else { RUN_POL(pol2, g2, MFMA_BM, 256, 2, 4, 128, false, true, 3) }
#undef RUN_POL
  if (err != hipSuccess) return err;
  return mark(2);
}

}  // namespace moe
