// Combine body shared by combine.hip (the combine kernel) and fused.hip (the
// single-launch forward).
#pragma once

#include "common.h"

namespace moe {

// Token t's output row; slot and g: LDS of 64 slot numbers and 64 gates.  Any block size.
template <bool F32>
__device__ __forceinline__ void combine_token(const void* __restrict__ ring_y,
                                              const int32_t* __restrict__ copy_slot,
                                              const float* __restrict__ gate, int d, int k,
                                              void* __restrict__ y, int64_t t, int64_t* slot,
                                              float* g) {
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

}  // namespace moe
