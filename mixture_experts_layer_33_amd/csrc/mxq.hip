// MX quantisation of a bf16 matrix along its rows (the weight helper): per
// block of 32 elements X = floor(log2 amax) - 8 (clamped, -127 for a zero
// block), codes = RNE E4M3 of v / 2^X saturated to +-448, scale byte X + 127.
// The MXFP8 format is the one the pages name for the expert kernels (khabar-ai
// page, @rohanpaul_ai tweet; dzen.guru page, megakernel paragraph); the bits
// follow the OCP MX v1.0 rule.  4 lanes hold one block (8 bf16 each).
//
// Scale layout (every MX scale tensor of the library): [cols / 128][rows][4] bytes, i.e.
// for each group of 128 columns one dword per row holding its 4 block scales.  A
// grouped-GEMM stage (128 columns of K) then finds the scales of consecutive rows in
// consecutive dwords; with the row layout [rows][cols / 32] they sat 4 bytes per row
// cols / 32 bytes apart, one cache line per row (MX gate/up GEMM 1.83 -> 1.62 ms).
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void quantize_mx_kernel(const bf16_t* __restrict__ src,
                                                          int64_t nvec, int64_t rows, int64_t vpr,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  // nvec = rows * cols / 8 vectors of 8 bf16; blocks never straddle rows (cols % 32 == 0)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t rounds = (nvec + stride - 1) / stride;
  for (int64_t it = 0; it < rounds; ++it) {
    const int64_t v = it * stride + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool ok = v < nvec;
    const u32x4 w = ok ? ((const u32x4*)src)[v] : u32x4{0, 0, 0, 0};
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) { f[2 * q] = lo_bf(w[q]); f[2 * q + 1] = hi_bf(w[q]); }
    float am = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) am = fmaxf(am, fabsf(f[q]));
    am = group_max<4>(am);
    const int X = mx_block_exp(am);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) lo |= e4m3_encode(f[q], X) << (8 * q);
#pragma unroll
    for (int q = 0; q < 4; ++q) hi |= e4m3_encode(f[4 + q], X) << (8 * q);
    if (ok) {
      ((u32x2*)codes)[v] = u32x2{lo, hi};
      if ((v & 3) == 0) {   // block cb of row r: vpr = cols / 8 vectors per row
        const int64_t r = v / vpr, cb = (v - r * vpr) / 4;
        scales[((cb / 4) * rows + r) * 4 + (cb & 3)] = (uint8_t)(X + 127);
      }
    }
  }
}

// The transposed helper for the MXFP8 backward, whose GEMMs reduce over the other axis of
// the weights: src [batch, R, Cc] bf16; every source column c of batch item b becomes the
// destination row b Cc + c, its R values the destination columns col0 .. col0 + R - 1 of a
// row of ld bytes, MX-quantised in blocks of 32 consecutive source rows; the scales go to
// the destination matrix's layout [ld / 128][batch Cc][4].  One thread per (item, block,
// column), columns fastest (consecutive threads read consecutive source columns).
__global__ __launch_bounds__(256) void quantize_mx_t_kernel(const bf16_t* __restrict__ src,
                                                            int64_t batch, int64_t R, int64_t Cc,
                                                            uint8_t* __restrict__ codes,
                                                            int64_t ld, int64_t col0,
                                                            uint8_t* __restrict__ scales) {
  const int64_t nq = R / 32;
  const int64_t n = batch * nq * Cc;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = i % Cc, bq = i / Cc, q = bq % nq, b = bq / nq;
    const bf16_t* s = src + (b * R + q * 32) * Cc + c;
    float v[32];
    float am = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      v[r] = bf2f(s[(int64_t)r * Cc]);
      am = fmaxf(am, fabsf(v[r]));
    }
    const int X = mx_block_exp(am);
    uint32_t w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      w[u] = 0;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) w[u] |= e4m3_encode(v[4 * u + q4], X) << (8 * q4);
    }
    const int64_t row = b * Cc + c, col = col0 + q * 32;
    u32x4* dst = (u32x4*)(codes + row * ld + col);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    const int64_t blk = col / 32;
    scales[((blk / 4) * (batch * Cc) + row) * 4 + (blk & 3)] = (uint8_t)(X + 127);
  }
}

hipError_t launch_quantize_mx_t(const void* src, int64_t batch, int64_t R, int64_t Cc,
                                uint8_t* codes, int64_t ld, int64_t col0, uint8_t* scales,
                                hipStream_t st) {
  const int64_t n = batch * (R / 32) * Cc;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  quantize_mx_t_kernel<<<(unsigned)blocks, 256, 0, st>>>((const bf16_t*)src, batch, R, Cc, codes,
                                                          ld, col0, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const void* src, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t st) {
  const int64_t nvec = rows * cols / 8;
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  quantize_mx_kernel<<<(unsigned)blocks, 256, 0, st>>>((const bf16_t*)src, nvec, rows, cols / 8,
                                                        codes, scales);
  return hipGetLastError();
}

}  // namespace moe
