// Shared device helpers for the gfx950 MoE kernels: bf16 bits, ring addressing,
// wave64 reductions and the MX (E4M3 + E8M0 per 32) encoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bit pattern

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN), by gfx950's v_cvt_pk_bf16_f32:
// one instruction for two values where the bit-level rounding took about six per value.
// The GEMM epilogues convert 64 accumulators per lane per tile; in the bf16 down GEMM
// staging them took ~2.6 us of a ~44 us tile.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_hw){lo, hi}, bf16x2_hw));
}

// Low / high bf16 of a packed 32-bit word, widened exactly.
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Ring slot of row i of a segment that starts `off` rows after the head.
__device__ __forceinline__ int64_t ring_slot(int64_t head, int64_t off, int64_t i, int64_t C) {
  int64_t s = head + off + i;
  return s >= C ? s - C : s;
}

// SiLU and the logistic function on the hardware exp and reciprocal (about 2 ulp each) instead of
// the full-precision expf and an IEEE division: in the GEMM epilogue that is 32 evaluations per
// lane per tile.  Same-GPU A/B in alternating processes, forward per call: 2,048 tokens bf16
// 3.720 -> 3.710 ms, MXFP8 2.258 -> 2.236 ms, skewed 8,192 tokens 4.04 -> 3.995 ms bf16,
// 2.71 -> 2.65 ms MXFP8.  For a -> -inf, exp(-a) overflows to inf and the result is -0 (or 0).
__device__ __forceinline__ float sigm(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ __forceinline__ float silu(float a) { return a * sigm(a); }

// Butterfly sum over the 64 lanes of a wavefront (fixed order: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Maximum over aligned groups of `G` lanes (G a power of two <= 64), in VALU cross-lane
// moves instead of LDS permutes: DPP quad permutations (lanes 1 and 2 apart), the half-row
// and row mirrors (4 and 8 apart), and gfx950's permlane swaps of 16- and 32-lane halves
// (given the same value twice, a swap hands each lane its partner's value in one of its
// two results).  Checked on the GPU against the ds_bpermute butterfly for G = 4 .. 64
// (bitwise equal).  The butterfly left a wave waiting ~100 cycles per step: the MX
// gate/up epilogue's 32 block maxima per wave took ~10 us of its tile's time.
template <int G>
__device__ __forceinline__ float group_max(float v) {
  static_assert(G >= 2 && G <= 64 && (G & (G - 1)) == 0, "groups of 2 .. 64 lanes");
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false)));  // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false)));  // [2,3,0,1]
  if constexpr (G >= 8) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));  // row_half_mirror
  if constexpr (G >= 16) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));  // row_mirror
  if constexpr (G >= 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = fmaxf(__int_as_float(s[0]), __int_as_float(s[1]));
  }
  if constexpr (G >= 64) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = fmaxf(__int_as_float(s[0]), __int_as_float(s[1]));
  }
  return v;
}

// Minimum over aligned groups of `G` lanes, by the same cross-lane moves as group_max.
template <int G>
__device__ __forceinline__ int group_min_i(int v) {
  static_assert(G >= 2 && G <= 64 && (G & (G - 1)) == 0, "groups of 2 .. 64 lanes");
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false));
  if constexpr (G >= 4) v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false));
  if constexpr (G >= 8) v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false));
  if constexpr (G >= 16) v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false));
  if constexpr (G >= 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = min((int)s[0], (int)s[1]);
  }
  if constexpr (G >= 64) {
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = min((int)s[0], (int)s[1]);
  }
  return v;
}

// ---------------------------------------------------------------- router row
// Softmax statistics and top-k of one row of E <= 64*VPL logits held by a
// wavefront (lane owns entries lane + 64 i).  k rounds of a wave-wide argmax,
// ties to the lower expert id.  On return lane r < k holds the r-th selected
// expert (`choice`), its rank in ascending expert order (`rank`) and its
// renormalised gate p / sum_S p with p = exp(l - max) / sum_e exp(l - max).
// Each round's wave-wide argmax is a maximum (group_max) and then the lowest expert id
// among the lanes holding it (group_min_i), both exact, so the selection is that of a
// pairwise butterfly; with ds_bpermute shuffles (two per step, six steps, eight rounds)
// the decode's routing wavefront took ~13 us beside the weight stream.
template <int VPL, typename LogitF>
__device__ __forceinline__ void wave_route_row_f(LogitF logit, int E, int k, int& choice, int& rank,
                                                 float& gate) {
  const int lane = threadIdx.x & 63;
  float v[VPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? logit(e) : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  m = group_max<64>(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) s += (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
  s = wave_sum(s);
  uint32_t taken = 0;
  choice = 0;
  float my_logit = 0.f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      if (64 * i >= E) break;   // uniform: no lane holds entries from here on
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
    const float mv = group_max<64>(bv);
    bi = group_min_i<64>(bv == mv ? bi : 0x7fffffff);
    bv = mv;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) { choice = bi; my_logit = bv; }
  }
  const float p = lane < k ? expf(my_logit - m) / s : 0.f;
  const float ps = wave_sum(p);
  rank = 0;
  for (int i = 0; i < k; ++i) rank += (__builtin_amdgcn_readlane(choice, i) < choice) ? 1 : 0;
  gate = p / ps;
}


// ---------------------------------------------------------------- MX / E4M3
// Block exponent of the OCP MX rule: X = floor(log2 amax) - 8, clamped to
// [-127, 127]; a zero (or fp32-subnormal) amax gives -127.  amax >= 0.
__device__ __forceinline__ int mx_block_exp(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  if (ef == 0) return -127;
  int X = ef - 127 - 8;
  return X < -127 ? -127 : X;
}

// E4M3 code of v * 2^-X: saturate to +-448, round to nearest even.  The sign
// is kept also when the magnitude rounds to zero.  v * 2^-X is exact in fp32 (a power
// of two; block values stay below 2^9), the clamp is a med3, and gfx950's fp32 -> OCP
// E4M3 conversion rounds to nearest even: compared on every bf16 value, every midpoint
// between adjacent E4M3 magnitudes with its fp32 neighbours, the saturation edges and a
// million random fp32 values, it gave the codes of the exact rule (sign, subnormal steps
// of 2^-9, carry into the next binade) without one difference, at a few instructions
// instead of a few dozen.
__device__ __forceinline__ uint32_t e4m3_encode(float v, int X) {
  const float c = __builtin_amdgcn_fmed3f(ldexpf(v, -X), -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
}
// Four codes of one block, a in the low byte: the conversion takes two values and writes
// them into the half word its last argument selects, so a dword of codes costs two
// conversions (each value converted as by e4m3_encode) instead of four plus the masks and
// shifts of packing single bytes.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d, int X) {
  auto clamp = [X](float v) { return __builtin_amdgcn_fmed3f(ldexpf(v, -X), -448.0f, 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(a), clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp(c), clamp(d), lo, true);
}

}  // namespace moe
