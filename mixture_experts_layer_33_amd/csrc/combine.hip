// Combine: y[t] = sum_j g[t, j] ring_y[copy_slot[t, j]], j in ascending expert
// order, fp32 accumulation and one final rounding.  A fixed gather order makes
// the layer's result reproducible (dzen.guru page, megakernel paragraph of
// "Три решения…": one deterministic result).  One workgroup per token; each
// thread owns 8 consecutive columns (16-byte bf16 loads, 32-byte fp32 loads).
// bf16 rows are read once each: the rows of up to 8 copies are requested before any
// is added (the sum keeps its order), with the non-temporal cache policy.  Measured
// with the last-level cache evicted first, 2,048 tokens: 98.4 us with one copy's row
// at a time, 96.3 us batched, 54.5 us batched and non-temporal (8,192 tokens, k = 10:
// 197 -> 144 us).
#include "common.h"
#include "kernels.h"

namespace moe {

template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ ring_y,
                                                      const int32_t* __restrict__ copy_slot,
                                                      const float* __restrict__ gate, int d, int k,
                                                      void* __restrict__ y) {
  const int64_t t = blockIdx.x;
  __shared__ int64_t slot[64];
  __shared__ float g[64];
  if (threadIdx.x < k) {
    slot[threadIdx.x] = copy_slot[t * k + threadIdx.x];
    g[threadIdx.x] = gate[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int v = threadIdx.x; v < d / 8; v += blockDim.x) {
    float acc[8] = {};
    if (!F32) {
      for (int j0 = 0; j0 < k; j0 += 8) {
        u32x4 w[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {   // copies past k reload the last row, unused
          const int j = min(j0 + jj, k - 1);
          w[jj] = __builtin_nontemporal_load((const u32x4*)((const bf16_t*)ring_y + slot[j] * d) + v);
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          if (j0 + jj >= k) break;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = fmaf(g[j0 + jj], lo_bf(w[jj][q]), acc[2 * q]);
            acc[2 * q + 1] = fmaf(g[j0 + jj], hi_bf(w[jj][q]), acc[2 * q + 1]);
          }
        }
      }
    } else {
      for (int j = 0; j < k; ++j) {
        const f32x4* src = (const f32x4*)((const float*)ring_y + slot[j] * d) + 2 * v;
        const f32x4 a = src[0], b = src[1];
        const float r[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(g[j], r[q], acc[q]);
      }
    }
    if (F32) {
      f32x4* dst = (f32x4*)((float*)y + t * d) + 2 * v;
      dst[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      dst[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      ((u32x4*)((bf16_t*)y + t * d))[v] =
          u32x4{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]), pack_bf2(acc[4], acc[5]),
                pack_bf2(acc[6], acc[7])};
    }
  }
}

hipError_t launch_combine(bool f32, const void* ring_y, const int32_t* copy_slot,
                          const float* gate, int64_t T, int d, int k, void* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (f32) combine_kernel<true><<<(unsigned)T, 256, 0, st>>>(ring_y, copy_slot, gate, d, k, y);
  else combine_kernel<false><<<(unsigned)T, 256, 0, st>>>(ring_y, copy_slot, gate, d, k, y);
  return hipGetLastError();
}

}  // namespace moe
