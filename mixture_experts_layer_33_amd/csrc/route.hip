// Router: fp32 logits, softmax over all experts, top-k, renormalised gates, counts.
//
// Routing of every token to a few experts is the first step of each MoE layer
// (dzen.guru page, "Что именно тормозило обучение MoE-моделей?").  The rule
// (softmax over E, top-k, renormalise the k gates to sum 1) is the layer's
// workload definition.  Everything here is fp32; bf16 tokens are widened exactly.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "route_body.h"

namespace moe {

// ----------------------------------------------------------------------------
// logits[t, e] = sum_i x[t, i] W_r[e, i] (the bias is added by the top-k kernel).  64x64 output tile per
// workgroup, 256 threads, 4x4 outputs per thread, K staged through LDS in
// steps of 32.  The K order is fixed, so the result is bitwise reproducible.
constexpr int RT_M = 64, RT_N = 64, RT_K = 32;

template <bool X_F32>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void* __restrict__ xv, const float* __restrict__ w, float* __restrict__ logits,
    int64_t T, int d, int E) {
  __shared__ float xs[RT_K][RT_M + 4];
  __shared__ float ws[RT_K][RT_N + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t t0 = (int64_t)blockIdx.y * RT_M;
  const int e0 = blockIdx.x * RT_N;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += RT_K) {
    // each thread stages 8 x values and 8 W values (rows r, k-offsets kk..kk+7)
    const int r = tid >> 2, kk = (tid & 3) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int kq = k0 + kk + q;
      const int64_t t = t0 + r;
      float xv_ = 0.f;
      if (t < T && kq < d) {
        if (X_F32) xv_ = ((const float*)xv)[t * d + kq];
        else xv_ = bf2f(((const bf16_t*)xv)[t * d + kq]);
      }
      xs[kk + q][r] = xv_;
      const int e = e0 + r;
      ws[kk + q][r] = (e < E && kq < d) ? w[(int64_t)e * d + kq] : 0.f;
    }
    __syncthreads();
    // two-level sum: a partial over this K slice, then the running total, so the
    // rounding error grows with d/32 + 32 terms rather than d
    float part[4][4] = {};
#pragma unroll 8
    for (int kq = 0; kq < RT_K; ++kq) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kq][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kq][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = fmaf(a[i], b[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += part[i][j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[t * E + e] = acc[i][j];
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 tokens: the same fp32 logits on MFMA.  W_r is split exactly into three
// bf16 planes, w = hi + mid + lo (hi = bf16(w), mid = bf16(w - hi),
// lo = w - hi - mid; 3 x 8 significand bits cover fp32's 24), so every product
// x * w_plane of a bf16 x is exact in fp32 and the MFMA accumulates in fp32.
// The split is done in registers as each K slice of W_r is staged (router_split8).

template <int BM>
__global__ __launch_bounds__(BM * 4) void router_mfma_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ w_r, float* __restrict__ logits,
    int64_t T, int d, int E) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * BM * RM_K];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2 * 192 * RM_K];
  router_mfma_body<BM>(x, w_r, logits, T, d, E, (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z,
                       (int)gridDim.z, As, Bs);
}

// The same logits with 128 tokens x 128 experts per workgroup: sixteen waves in 4 x 4, each
// 32 tokens x 32 experts x 3 planes.  Per K slice a workgroup stages 16 KB of tokens and 48 KB of
// weights for four times the MFMA work of the 64 x 64 tile, halving the L2 traffic per
// logit; the double buffer (128 KB) is dynamic LDS, one workgroup per CU.  One slice is in
// flight in registers while the other is multiplied: a second register set would spill.
constexpr int R2_BM = 128, R2_BN = 128, R2_NT = 1024;
constexpr int R2_LDS = 2 * (R2_BM + 3 * R2_BN) * RM_K;
//
// W_r is read in fp32 and split into its three planes in registers (router_split8): thread q
// takes 8 consecutive weights of expert row q / 8 per 64-wide K slice.
__global__ __launch_bounds__(R2_NT) void router_mfma2_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ w_r, float* __restrict__ logits,
    int64_t T, int d, int E) {
  constexpr int BM = R2_BM, BNE = R2_BN, BNR = 3 * BNE, NT = R2_NT;
  constexpr int A_LD = BM * 8 / NT;
  static_assert(BNE * 8 == NT, "one 8-weight group of one expert row per thread and slice");
  extern __shared__ __attribute__((aligned(16))) uint8_t r2lds[];
#define AS2(buf) (r2lds + (buf) * (BM * RM_K))
#define BS2(buf) (r2lds + 2 * BM * RM_K + (buf) * (BNR * RM_K))
  const int64_t t0 = (int64_t)blockIdx.y * BM;
  const int e0 = blockIdx.x * BNE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, lr = lane & 31, lg = lane >> 5;
  const int KS = gridDim.z, z = blockIdx.z, KA = d / 64;
  const int kb = (int)((int64_t)KA * z / KS);
  const int KT = (int)((int64_t)KA * (z + 1) / KS) - kb;
  const bf16_t* a_src[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = tid + NT * i;
    const int64_t t = min(t0 + q / 8, T - 1);
    a_src[i] = x + t * d + (int64_t)kb * 64 + (q % 8) * 8;
  }
  const int br = tid / 8, bc = tid % 8;   // this thread's expert row and 8-weight group
  const float* b_src = w_r + (int64_t)min(e0 + br, E - 1) * d + (int64_t)kb * 64 + bc * 8;
  u32x4 ra0[A_LD];
  f32x4 rb0[2];
#define R_LOAD(kt, RA, RB)                                                                   \
  {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) RA[i] = *(const u32x4*)(a_src[i] + (kt) * 64); \
    RB[0] = *(const f32x4*)(b_src + (kt) * 64);                                              \
    RB[1] = *(const f32x4*)(b_src + (kt) * 64 + 4);                                          \
  }
#define R_STORE(buf, RA, RB)                                                                 \
  {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) {                                      \
      const int q = tid + NT * i;                                                            \
      *(u32x4*)(AS2(buf) + rswz(q / 8, q % 8)) = RA[i];                                      \
    }                                                                                        \
    u32x4 ph, pm, pl;                                                                        \
    router_split8(RB, ph, pm, pl);                                                           \
    *(u32x4*)(BS2(buf) + rswz(br, bc)) = ph;                                                 \
    *(u32x4*)(BS2(buf) + rswz(BNE + br, bc)) = pm;                                           \
    *(u32x4*)(BS2(buf) + rswz(2 * BNE + br, bc)) = pl;                                       \
  }
  f32x16 acc[3];
#pragma unroll
  for (int pl = 0; pl < 3; ++pl)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[pl][r] = 0.f;
  auto compute = [&](int cur) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + lg;
      const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(AS2(cur) + rswz(wm * 32 + lr, c)));
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const bf16x8 b = __builtin_bit_cast(
            bf16x8, *(const u32x4*)(BS2(cur) + rswz(pl * BNE + wn * 32 + lr, c)));
        acc[pl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[pl], 0, 0, 0);
      }
    }
  };
  R_LOAD(0, ra0, rb0);
  R_STORE(0, ra0, rb0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) R_LOAD(kt + 1, ra0, rb0);
    compute(cur);
    if (kt + 1 >= KT) break;
    R_STORE(cur ^ 1, ra0, rb0);
    __syncthreads();
  }
#undef R_LOAD
#undef R_STORE
#undef AS2
#undef BS2
  float* out = logits + (int64_t)z * T * E;
  const int e = e0 + wn * 32 + lr;
  if (e >= E) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t t = t0 + wm * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
    if (t < T) out[t * E + e] = (acc[0][r] + acc[1][r]) + acc[2][r];
  }
}

template <int VPL, bool SPLIT>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ logits, int KS, const float* __restrict__ bias, int64_t T, int E,
    int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<VPL, SPLIT>(logits, KS, bias, T, E, k, t, topk_idx, topk_gate);
}

// ----------------------------------------------------------------------------
// expert_count[e] = number of copies routed to e: one workgroup, LDS histogram
// with integer atomics (exact, order-free).
__global__ __launch_bounds__(1024) void expert_count_kernel(const int32_t* __restrict__ idx,
                                                            int64_t n, int E,
                                                            int32_t* __restrict__ count) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  // eight independent loads per thread before their atomics: one latency per 8 copies
  for (int64_t c0 = threadIdx.x; c0 < n; c0 += 8 * (int64_t)blockDim.x) {
    int32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t c = c0 + (int64_t)i * blockDim.x;
      v[i] = c < n ? idx[c] : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (v[i] >= 0) atomicAdd(&hist[v[i]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) count[e] = hist[e];
}

size_t route_workspace_bytes(int64_t T, int E, int d) {
  return logits_bytes(T, E, d);
}

hipError_t launch_route(const void* x, bool x_f32, const float* w_r, const float* b_r, int64_t T,
                        int d, int E, int k, float* logits, int32_t* topk_idx, float* topk_gate,
                        int32_t* expert_count, hipStream_t st) {
  int ks = 1;
  if (x_f32) {
    dim3 g1((E + RT_N - 1) / RT_N, (unsigned)((T + RT_M - 1) / RT_M));
    router_logits_kernel<true><<<g1, 256, 0, st>>>(x, w_r, logits, T, d, E);
  } else {
    // d % 64 == 0 for bf16 layers
    ks = router_ksplit(T, E, d);
    if (router_big(E)) {
      hipError_t e = hipFuncSetAttribute((const void*)router_mfma2_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, R2_LDS);
      if (e != hipSuccess) return e;
      router_mfma2_kernel<<<dim3((unsigned)((E + 127) / 128), (unsigned)((T + 127) / 128), (unsigned)ks),
                            R2_NT, R2_LDS, st>>>((const bf16_t*)x, w_r, logits, T, d, E);
    } else {
      router_mfma_kernel<64><<<dim3((unsigned)((E + 63) / 64), (unsigned)((T + 63) / 64), (unsigned)ks),
                               256, 0, st>>>((const bf16_t*)x, w_r, logits, T, d, E);
    }
  }
  const unsigned g2 = (unsigned)((T + 3) / 4);
  const int vpl = (E + 63) / 64;
#define TOPK(V)                                                                                   \
  {                                                                                               \
    if (ks > 1) router_topk_kernel<V, true><<<g2, 256, 0, st>>>(logits, ks, b_r, T, E, k, topk_idx, topk_gate); \
    else router_topk_kernel<V, false><<<g2, 256, 0, st>>>(logits, ks, b_r, T, E, k, topk_idx, topk_gate);      \
  }
  if (vpl <= 1) TOPK(1)
  else if (vpl <= 2) TOPK(2)
  else if (vpl <= 4) TOPK(4)
  else if (vpl <= 8) TOPK(8)
  else TOPK(16)
#undef TOPK
  expert_count_kernel<<<1, 1024, E * sizeof(int32_t), st>>>(topk_idx, T * k, E, expert_count);
  return hipGetLastError();
}

}  // namespace moe
