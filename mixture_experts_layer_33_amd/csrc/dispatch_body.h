// Dispatch bodies shared by dispatch.hip (the dispatch kernels) and fused.hip (the
// single-launch forward): one chunk's expert masks and counts, a token's ring slots, and
// the plain copy of one token row into its k slots.
#pragma once

#include "common.h"

namespace moe {

constexpr int DCH = 64;  // tokens per chunk = wavefront width

// Chunk `chunk` (tokens 64 chunk .. + 63): for every expert the mask of the chunk's tokens
// that chose it and its popcount.  Threads 0..63 take one token each; m is LDS of E words.
// Any block size >= 64; every thread of the block must call it.
__device__ __forceinline__ void dispatch_hist_chunk(const int32_t* __restrict__ idx, int64_t T,
                                                    int k, int E,
                                                    unsigned long long* __restrict__ masks,
                                                    int32_t* __restrict__ hist, int64_t chunk,
                                                    unsigned long long* m) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e < E; e += nt) m[e] = 0ull;
  __syncthreads();
  const int64_t t = chunk * DCH + tid;
  if (tid < DCH && t < T)
    for (int j = 0; j < k; ++j) atomicOr(&m[idx[t * k + j]], 1ull << tid);
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    masks[chunk * E + e] = m[e];
    hist[chunk * E + e] = __popcll(m[e]);
  }
}

__device__ __forceinline__ void copy_slots(const int32_t* __restrict__ idx,
                                           const unsigned long long* __restrict__ masks,
                                           const int32_t* __restrict__ base, int64_t t, int k,
                                           int E, int64_t head, int64_t C,
                                           int32_t* __restrict__ copy_slot,
                                           int32_t* __restrict__ slot_copy, int64_t* slots) {
  const int j = threadIdx.x;
  if (j < k) {
    const int64_t chunk = t / DCH;
    const int lc = (int)(t % DCH);
    const int e = idx[t * k + j];
    const unsigned long long mk = masks[chunk * E + e];
    const int64_t rank = base[chunk * E + e] + __popcll(mk & ((1ull << lc) - 1ull));
    int64_t s = head + rank;
    if (s >= C) s -= C;
    slots[j] = s;
    copy_slot[t * k + j] = (int32_t)s;
    slot_copy[s] = (int32_t)(t * k + j);
  }
  __syncthreads();
}

// Token t's row (row_bytes a multiple of 16) into its k slots, read and written with the
// non-temporal cache policy.  slots: LDS of 64 slot numbers.
__device__ __forceinline__ void dispatch_copy_token(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ idx,
    const unsigned long long* __restrict__ masks, const int32_t* __restrict__ base, int k, int E,
    int64_t head, int64_t C, int64_t row_bytes, uint8_t* __restrict__ ring,
    int32_t* __restrict__ copy_slot, int32_t* __restrict__ slot_copy, int64_t t, int64_t* slots) {
  copy_slots(idx, masks, base, t, k, E, head, C, copy_slot, slot_copy, slots);
  const int64_t nv = row_bytes / 16;
  const u32x4* src = (const u32x4*)(x + t * row_bytes);
  for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
    const u32x4 val = __builtin_nontemporal_load(src + v);
    for (int j = 0; j < k; ++j) __builtin_nontemporal_store(val, (u32x4*)(ring + slots[j] * row_bytes) + v);
  }
}

}  // namespace moe
