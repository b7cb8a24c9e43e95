// Router bodies shared by route.hip (the router kernels) and fused.hip (the
// single-launch forward): the exact three-plane split of W_r, one MFMA logit tile, one
// token's top-k, and the host-side choices of tile and K split.
#pragma once

#include <algorithm>

#include "common.h"

namespace moe {

// Eight consecutive fp32 weights into the three bf16 planes w = hi + mid + lo (hi = bf16(w),
// mid = bf16(w - hi), lo = bf16(w - hi - mid), round to nearest even; the differences are
// exact in fp32, and 3 x 8 significand bits cover fp32's 24), as packed 16-byte pieces.
__device__ __forceinline__ void router_split8(const f32x4 (&w)[2], u32x4& hi, u32x4& mid, u32x4& lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float v0 = w[j / 2][2 * (j % 2)], v1 = w[j / 2][2 * (j % 2) + 1];
    hi[j] = pack_bf2(v0, v1);
    const float r0 = v0 - lo_bf(hi[j]), r1 = v1 - hi_bf(hi[j]);
    mid[j] = pack_bf2(r0, r1);
    lo[j] = pack_bf2(r0 - lo_bf(mid[j]), r1 - hi_bf(mid[j]));
  }
}

// BM tokens x 64 experts per workgroup; waves (BM/32) x 2, each a 32 x 32 tile
// with one accumulator per plane; K in 64-element slices through double-buffered,
// XOR-swizzled LDS.  The K range is split over gridDim.z workgroups: split z sums
// slices [z KT / KS, (z + 1) KT / KS) and writes partial plane z of the logits,
// (acc_hi + acc_mid) + acc_lo; the top-k kernel adds the planes in order z = 0, 1, ...
// and then the bias.  Two K slices are in flight while one is multiplied: slice
// kt + 1 (requested during the previous slice) and kt + 2, in two register sets.
constexpr int RM_K = 128;   // bytes of K per row per stage

__device__ __forceinline__ int rswz(int r, int c) { return r * RM_K + ((c ^ (r & 7)) << 4); }

// One workgroup's tile: expert tile bx (64 experts), token tile by (BM tokens), K split z
// of KS; As / Bs: two LDS buffers of BM x RM_K and 192 x RM_K bytes each.
// W_r is read in fp32 and split into its planes in registers (router_split8): 4 bytes per
// weight instead of the planes' 6, and no separate split pass.
template <int BM>
__device__ __forceinline__ void router_mfma_body(
    const bf16_t* __restrict__ x, const float* __restrict__ w_r, float* __restrict__ logits,
    int64_t T, int d, int E, int bx, int by, int z, int KS, uint8_t* As0, uint8_t* Bs0) {
  constexpr int NT = BM * 4;                     // threads; B rows = 3 planes x 64 experts
  constexpr int A_LD = BM * 8 / NT, BG = 64 * 8 / NT;   // 8-weight groups per thread and slice
  static_assert(64 * 8 % NT == 0, "whole 8-weight groups per thread");
  auto As = [&](int buf) { return As0 + buf * (BM * RM_K); };
  auto Bs = [&](int buf) { return Bs0 + buf * (192 * RM_K); };
  const int64_t t0 = (int64_t)by * BM;
  const int e0 = bx * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lg = lane >> 5;
  const int KA = d / 64;
  const int kb = (int)((int64_t)KA * z / KS);
  const int KT = (int)((int64_t)KA * (z + 1) / KS) - kb;
  const bf16_t* a_src[A_LD];
  const float* b_src[BG];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = tid + NT * i;
    const int64_t t = min(t0 + q / 8, T - 1);
    a_src[i] = x + t * d + (int64_t)kb * 64 + (q % 8) * 8;
  }
#pragma unroll
  for (int g = 0; g < BG; ++g) {   // group q: expert row q / 8, weights 8 (q % 8) .. + 7
    const int q = tid + NT * g;
    b_src[g] = w_r + (int64_t)min(e0 + q / 8, E - 1) * d + (int64_t)kb * 64 + (q % 8) * 8;
  }
  u32x4 ra0[A_LD], ra1[A_LD];
  f32x4 rb0[BG][2], rb1[BG][2];
#define R_LOAD(kt, RA, RB)                                                                   \
  {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) RA[i] = *(const u32x4*)(a_src[i] + (kt) * 64); \
    _Pragma("unroll") for (int g = 0; g < BG; ++g) {                                        \
      RB[g][0] = *(const f32x4*)(b_src[g] + (kt) * 64);                                      \
      RB[g][1] = *(const f32x4*)(b_src[g] + (kt) * 64 + 4);                                  \
    }                                                                                        \
  }
#define R_STORE(buf, RA, RB)                                                                 \
  {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) {                                      \
      const int q = tid + NT * i;                                                            \
      *(u32x4*)(As(buf) + rswz(q / 8, q % 8)) = RA[i];                                       \
    }                                                                                        \
    _Pragma("unroll") for (int g = 0; g < BG; ++g) {                                        \
      const int q = tid + NT * g;                                                            \
      u32x4 ph, pm, pl;                                                                      \
      router_split8(RB[g], ph, pm, pl);                                                      \
      *(u32x4*)(Bs(buf) + rswz(q / 8, q % 8)) = ph;                                          \
      *(u32x4*)(Bs(buf) + rswz(64 + q / 8, q % 8)) = pm;                                     \
      *(u32x4*)(Bs(buf) + rswz(128 + q / 8, q % 8)) = pl;                                    \
    }                                                                                        \
  }
  f32x16 acc[3];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[p][r] = 0.f;
  auto compute = [&](int cur) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + lg;
      const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(As(cur) + rswz(wm * 32 + lr, c)));
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8 b =
            __builtin_bit_cast(bf16x8, *(const u32x4*)(Bs(cur) + rswz(p * 64 + wn * 32 + lr, c)));
        acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[p], 0, 0, 0);
      }
    }
  };
  R_LOAD(0, ra0, rb0);
  if (KT > 1) R_LOAD(1, ra1, rb1);
  R_STORE(0, ra0, rb0);
  __syncthreads();
  // LDS buffer 0 holds even slices, buffer 1 odd ones; each buffer is rewritten only
  // after the barrier that follows its last read.
  for (int kt = 0; kt < KT; kt += 2) {
    if (kt + 2 < KT) R_LOAD(kt + 2, ra0, rb0);
    compute(0);
    if (kt + 1 >= KT) break;
    R_STORE(1, ra1, rb1);
    __syncthreads();
    if (kt + 3 < KT) R_LOAD(kt + 3, ra1, rb1);
    compute(1);
    if (kt + 2 >= KT) break;
    R_STORE(0, ra0, rb0);
    __syncthreads();
  }
#undef R_LOAD
#undef R_STORE
  const int e = e0 + wn * 32 + lr;
  if (e >= E) return;
  float* out = logits + (int64_t)z * T * E;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t t = t0 + wm * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
    if (t < T) out[t * E + e] = (acc[0][r] + acc[1][r]) + acc[2][r];
  }
}

// With 128 or more experts the 128 x 128 tile is taken: its expert tiles are mostly full,
// and it halves the L2 traffic per logit (60 -> 55 us for 2,048 tokens, d 7168, 256
// experts; 219 -> 175 us for 8,192 tokens, d 4096, 512 experts).
inline bool router_big(int E) { return E >= 128; }

constexpr int RT_MAX_KS = 8;   // most K splits of the bf16 router (partial logit planes)

// Number of K splits of the bf16 router: enough workgroups to give every CU two 64 x 64
// tiles or one 128 x 128 tile, keeping at least 8 K slices per split.
inline int router_ksplit(int64_t T, int E, int d) {
  const bool big = router_big(E);
  const int64_t tiles = big ? ((T + 127) / 128) * ((E + 127) / 128) : ((T + 63) / 64) * ((E + 63) / 64);
  const int64_t target = big ? 256 : 512;
  int ks = (int)std::min<int64_t>(RT_MAX_KS, std::max<int64_t>(1, target / std::max<int64_t>(tiles, 1)));
  while (ks > 1 && d / 64 / ks < 8) --ks;
  return ks;
}

// ----------------------------------------------------------------------------
// One wavefront per token: softmax statistics, top-k (ties to the lower id),
// ascending-id output order, renormalised gates.
template <int VPL, bool SPLIT>
__device__ __forceinline__ void route_token(
    const float* __restrict__ logits, int KS, const float* __restrict__ bias, int64_t T, int E,
    int k, int64_t t, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  const int lane = threadIdx.x & 63;
  // logit = ((plane 0 + plane 1) + ...) + bias, every lane for its experts lane + 64 i.
  // With K split (SPLIT, KS <= RT_MAX_KS planes), all planes' loads are issued before
  // the first addition: a loop over the runtime plane count waited for each load in turn
  // (2,048 tokens, 8 planes: 20.4 -> 17.1 us).  A separate instantiation, so that the
  // single-plane launches keep their few registers and their occupancy.
  float lv[VPL];
  if constexpr (!SPLIT) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = min(lane + 64 * i, E - 1);
      lv[i] = logits[t * E + e] + (bias ? bias[e] : 0.f);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = min(lane + 64 * i, E - 1);
      float part[RT_MAX_KS];
#pragma unroll
      for (int zz = 0; zz < RT_MAX_KS; ++zz)
        part[zz] = zz < KS ? logits[((int64_t)zz * T + t) * E + e] : 0.f;
      float v = part[0];
#pragma unroll
      for (int zz = 1; zz < RT_MAX_KS; ++zz)
        if (zz < KS) v += part[zz];
      lv[i] = v + (bias ? bias[e] : 0.f);
    }
  }
  int choice, rank;
  float gate;
  wave_route_row_f<VPL>([&](int e) { return lv[(e - lane) >> 6]; }, E, k, choice, rank, gate);
  if (lane < k) {
    topk_idx[t * k + rank] = choice;
    topk_gate[t * k + rank] = gate;
  }
}

// workspace: KS partial planes of the logits [KS, T, E] f32, then the three bf16
// planes of W_r [3, E, d] (bf16 tokens)
inline size_t logits_bytes(int64_t T, int E, int d) {
  return ((size_t)router_ksplit(T, E, d) * T * E * sizeof(float) + 255) & ~(size_t)255;
}
}  // namespace moe
