// Dispatch: a deterministic counting sort of the T*k token copies into the
// fixed-capacity ring buffer, expert-contiguous, tokens ascending inside each
// expert's segment.  The pages' token ring buffer has a fixed size, drops no
// token and needs no size computed on the CPU (dzen.guru page, ring-buffer
// paragraph of "Три решения, которые дали результат"); every count and offset
// here stays on the device.
//
//   1. per chunk of 64 tokens (one wavefront): for every expert a 64-bit mask
//      of the chunk's tokens that chose it (LDS atomicOr), and its popcount;
//   2. one workgroup scans the chunk counts per expert and the expert totals:
//      base[chunk][e] = rank of the chunk's first copy of expert e;
//   3. one workgroup per token: rank = base + popcount(mask below the token),
//      slot = (head + rank) mod C; the row is read once and written to its k
//      slots (MX: quantised once, codes and scales written k times).
#include "common.h"
#include "dispatch_body.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(64) void dispatch_hist_kernel(const int32_t* __restrict__ idx,
                                                           int64_t T, int k, int E,
                                                           unsigned long long* __restrict__ masks,
                                                           int32_t* __restrict__ hist) {
  extern __shared__ unsigned long long m[];
  dispatch_hist_chunk(idx, T, k, E, masks, hist, blockIdx.x, m);
}

// One workgroup of 1024 threads, one expert per thread (E <= 1024).  A thread walks
// its expert's column of chunk counts twice (totals, then bases), issuing the loads of
// 16 chunks at a time so that one memory latency covers 16 chunks.
constexpr int SCAN_BATCH = 16;
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ hist, int nch,
                                                             int E,
                                                             int32_t* __restrict__ expert_offset) {
  __shared__ int32_t sc[1024];
  const int e = threadIdx.x;
  int32_t run = 0;
  if (e < E)
    for (int c0 = 0; c0 < nch; c0 += SCAN_BATCH) {
      int32_t h[SCAN_BATCH];
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i) h[i] = c0 + i < nch ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i) run += h[i];
    }
  sc[e] = e < E ? run : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over the expert totals
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t v = e >= o ? sc[e - o] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  const int32_t off = sc[e] - run;  // exclusive
  if (e < E) {
    expert_offset[e] = off;
    // base[c][e] = off + copies of expert e in chunks before c
    int32_t acc = off;
    for (int c0 = 0; c0 < nch; c0 += SCAN_BATCH) {
      int32_t h[SCAN_BATCH];
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i) h[i] = c0 + i < nch ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i)
        if (c0 + i < nch) {
          hist[(int64_t)(c0 + i) * E + e] = acc;
          acc += h[i];
        }
    }
  }
  if (e == E - 1) expert_offset[E] = sc[e];
}

// Plain copy of one token row (row_bytes a multiple of 16) into its k slots, read and
// written with the non-temporal cache policy (every byte moves once; whole forward at
// 2,048 tokens 4.081 -> 4.050 ms, skewed 8,192 tokens 4.242 -> 4.184 ms).
__global__ __launch_bounds__(256) void dispatch_copy_kernel(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ idx,
    const unsigned long long* __restrict__ masks, const int32_t* __restrict__ base, int k, int E,
    int64_t head, int64_t C, int64_t row_bytes, uint8_t* __restrict__ ring,
    int32_t* __restrict__ copy_slot, int32_t* __restrict__ slot_copy) {
  __shared__ int64_t slots[64];
  dispatch_copy_token(x, idx, masks, base, k, E, head, C, row_bytes, ring, copy_slot, slot_copy,
                      blockIdx.x, slots);
}

// MX: each 32-element block is held by 4 consecutive lanes (8 bf16 each).
__global__ __launch_bounds__(256) void dispatch_mx_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ idx,
    const unsigned long long* __restrict__ masks, const int32_t* __restrict__ base, int k, int E,
    int64_t head, int64_t C, int d, uint8_t* __restrict__ ring, uint8_t* __restrict__ ring_scale,
    int32_t* __restrict__ copy_slot, int32_t* __restrict__ slot_copy) {
  __shared__ int64_t slots[64];
  const int64_t t = blockIdx.x;
  copy_slots(idx, masks, base, t, k, E, head, C, copy_slot, slot_copy, slots);
  const int nv = d / 8;
  const int iters = (nv + 255) / 256;  // uniform trip count: all lanes join the shuffles
  for (int it = 0; it < iters; ++it) {
    const int v = it * 256 + threadIdx.x;
    const bool ok = v < nv;
    u32x4 w = ok ? ((const u32x4*)(x + t * d))[v] : u32x4{0, 0, 0, 0};
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
    if (ok)
      for (int j = 0; j < k; ++j) {
        *(u32x2*)(ring + slots[j] * d + (int64_t)v * 8) = u32x2{lo, hi};
        if ((v & 3) == 0)   // scale layout [d / 128][C][4]: block v / 4 of ring row slots[j]
          ring_scale[((int64_t)(v / 16) * C + slots[j]) * 4 + ((v / 4) & 3)] = (uint8_t)(X + 127);
      }
  }
}

size_t dispatch_workspace_bytes(int64_t T, int E) {
  const int64_t nch = (T + DCH - 1) / DCH;
  return (size_t)nch * E * (sizeof(unsigned long long) + sizeof(int32_t));
}

hipError_t launch_dispatch(const void* x, int elem_bytes, bool mx, const int32_t* topk_idx,
                           int64_t T, int d, int E, int k, int64_t head, int64_t C, void* ring_x,
                           uint8_t* ring_scale, int32_t* expert_offset, int32_t* copy_slot,
                           int32_t* slot_copy, void* ws, hipStream_t st) {
  const int64_t nch = (T + DCH - 1) / DCH;
  unsigned long long* masks = (unsigned long long*)ws;
  int32_t* base = (int32_t*)(masks + nch * E);
  dispatch_hist_kernel<<<(unsigned)nch, 64, E * sizeof(unsigned long long), st>>>(
      topk_idx, T, k, E, masks, base);
  dispatch_scan_kernel<<<1, 1024, 0, st>>>(base, (int)nch, E, expert_offset);
  if (mx)
    dispatch_mx_kernel<<<(unsigned)T, 256, 0, st>>>((const bf16_t*)x, topk_idx, masks, base, k, E,
                                                    head, C, d, (uint8_t*)ring_x, ring_scale,
                                                    copy_slot, slot_copy);
  else
    dispatch_copy_kernel<<<(unsigned)T, 256, 0, st>>>((const uint8_t*)x, topk_idx, masks, base, k,
                                                      E, head, C, (int64_t)d * elem_bytes,
                                                      (uint8_t*)ring_x, copy_slot, slot_copy);
  return hipGetLastError();
}

}  // namespace moe
