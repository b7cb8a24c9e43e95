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
    const uint32_t lo = e4m3_encode4(f[0], f[1], f[2], f[3], X);
    const uint32_t hi = e4m3_encode4(f[4], f[5], f[6], f[7], X);
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
      w[u] = e4m3_encode4(v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3], X);
    }
    const int64_t row = b * Cc + c, col = col0 + q * 32;
    u32x4* dst = (u32x4*)(codes + row * ld + col);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    const int64_t blk = col / 32;
    scales[((blk / 4) * (batch * Cc) + row) * 4 + (blk & 3)] = (uint8_t)(X + 127);
  }
}

// Both layouts in one pass, for an MXFP8 training step that re-quantises every weight for the
// forward (blocks of 32 along its rows, as quantize_mx_kernel) and for the backward (blocks of
// 32 along its columns, transposed, as quantize_mx_t_kernel): each bf16 weight is read once
// instead of twice.  A workgroup stages a 128 x 128 tile of src[b] in LDS; each of its rows
// holds four whole row blocks and each of its columns four whole column blocks.  The codes
// and scales are those of the two kernels bit for bit (the same block rule on the same
// values).  The transposed codes are assembled in the same LDS space (after the tile is
// read) so that both outputs leave as whole 128-byte pieces of their rows.
constexpr int QB_T = 128;                 // tile rows and columns
constexpr int QB_RS = QB_T * 2 + 16;      // staged bf16 row stride in bytes (34,816 in all)
constexpr int QB_TS = QB_T + 16;          // staged transposed code row stride in bytes

__global__ __launch_bounds__(256) void quantize_mx_both_kernel(
    const bf16_t* __restrict__ src, int64_t batch, int64_t R, int64_t Cc,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
    int64_t ld, int64_t col0, uint8_t* __restrict__ scales_t) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[QB_T * QB_RS];
  __shared__ __attribute__((aligned(4))) uint8_t tscb[QB_T * 4];   // transposed scale bytes per dest row
  static_assert(QB_T * QB_TS <= QB_T * QB_RS, "the transposed codes fit the tile's space");
  const int t = threadIdx.x;
  const int64_t rt = R / QB_T, ct = Cc / QB_T, ntiles = batch * rt * ct;
  for (int64_t ti = blockIdx.x; ti < ntiles; ti += gridDim.x) {
    const int64_t b = ti / (rt * ct), rem = ti % (rt * ct);
    const int64_t r0 = (rem / ct) * QB_T, c0 = (rem % ct) * QB_T;
    const bf16_t* s = src + (b * R + r0) * Cc + c0;
    // 128 rows of 256 bytes: thread t copies 16-byte chunk t % 16 of rows t / 16 + 16 i
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = t / 16 + 16 * i, ch = t % 16;
      *(u32x4*)(tile + r * QB_RS + ch * 16) =
          __builtin_nontemporal_load((const u32x4*)(s + (int64_t)r * Cc + ch * 8));
    }
    __syncthreads();
    // forward layout: thread t takes row t / 2, columns 64 (t % 2) .. + 63 (two blocks)
    {
      const int r = t >> 1, h = t & 1;
      const uint8_t* row = tile + r * QB_RS + h * 128;
      u32x4 out[4];
      uint32_t sc = 0;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        float v[32];
        float am = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 w = *(const u32x4*)(row + blk * 64 + q * 16);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[8 * q + 2 * k] = lo_bf(w[k]);
            v[8 * q + 2 * k + 1] = hi_bf(w[k]);
          }
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
        const int X = mx_block_exp(am);
        uint32_t w32[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          w32[u] = e4m3_encode4(v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3], X);
        }
        out[2 * blk] = u32x4{w32[0], w32[1], w32[2], w32[3]};
        out[2 * blk + 1] = u32x4{w32[4], w32[5], w32[6], w32[7]};
        sc |= (uint32_t)(X + 127) << (8 * (2 * h + blk));
      }
      const int64_t grow = b * R + r0 + r;   // row of the [batch R, Cc] matrix
      u32x4* dst = (u32x4*)(codes + grow * Cc + c0 + h * 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = out[q];
      const uint32_t other = __shfl_xor(sc, 1, 64);
      if (h == 0) ((uint32_t*)scales)[(c0 / 128) * (batch * R) + grow] = sc | other;
    }
    // transposed layout: thread t takes source columns 2p, 2p + 1 (p = t % 64), rows
    // 32 q .. 32 q + 31 (q = t / 64): one block per column
    float v0[32], v1[32];
    float a0 = 0.f, a1 = 0.f;
    const int p = t & 63, q = t >> 6;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t w = *(const uint32_t*)(tile + (32 * q + k) * QB_RS + p * 4);
      v0[k] = lo_bf(w);
      v1[k] = hi_bf(w);
      a0 = fmaxf(a0, fabsf(v0[k]));
      a1 = fmaxf(a1, fabsf(v1[k]));
    }
    __syncthreads();   // the tile is read: its space takes the transposed codes
    {
      const int X0 = mx_block_exp(a0), X1 = mx_block_exp(a1);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t w0 = e4m3_encode4(v0[4 * u], v0[4 * u + 1], v0[4 * u + 2], v0[4 * u + 3], X0);
        const uint32_t w1 = e4m3_encode4(v1[4 * u], v1[4 * u + 1], v1[4 * u + 2], v1[4 * u + 3], X1);
        *(uint32_t*)(tile + (2 * p) * QB_TS + 32 * q + 4 * u) = w0;
        *(uint32_t*)(tile + (2 * p + 1) * QB_TS + 32 * q + 4 * u) = w1;
      }
      tscb[(2 * p) * 4 + q] = (uint8_t)(X0 + 127);
      tscb[(2 * p + 1) * 4 + q] = (uint8_t)(X1 + 127);
    }
    __syncthreads();
    // destination rows c0 + c of item b, bytes col0 + r0 .. + 127: per store instruction a
    // wave writes 8 whole rows (consecutive lanes take consecutive 16-byte pieces); two
    // lanes per row, a quarter row per instruction, took 5.400 ms against 5.354 for the
    // skewed training weights
    {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int id = k * 256 + t, c = id >> 3, ch = id & 7;
        *(u32x4*)(codes_t + (b * Cc + c0 + c) * ld + col0 + r0 + ch * 16) = *(const u32x4*)(tile + c * QB_TS + ch * 16);
      }
      if (t < QB_T) ((uint32_t*)scales_t)[((col0 + r0) / 128) * (batch * Cc) + b * Cc + c0 + t] = ((const uint32_t*)tscb)[t];
    }
    __syncthreads();   // before the next tile overwrites the LDS
  }
}

hipError_t launch_quantize_mx_both(const void* src, int64_t batch, int64_t R, int64_t Cc,
                                   uint8_t* codes, uint8_t* scales, uint8_t* codes_t, int64_t ld,
                                   int64_t col0, uint8_t* scales_t, hipStream_t st) {
  const int64_t ntiles = batch * (R / QB_T) * (Cc / QB_T);
  if (ntiles == 0) return hipSuccess;
  const int64_t blocks = ntiles < 32768 ? ntiles : 32768;
  quantize_mx_both_kernel<<<(unsigned)blocks, 256, 0, st>>>((const bf16_t*)src, batch, R, Cc, codes,
                                                             scales, codes_t, ld, col0, scales_t);
  return hipGetLastError();
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
