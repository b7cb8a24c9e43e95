// Router: fp32 logits, softmax over all experts, top-k, renormalised gates, counts.
//
// Routing of every token to a few experts is the first step of each MoE layer
// (dzen.guru page, "Что именно тормозило обучение MoE-моделей?").  The rule
// (softmax over E, top-k, renormalise the k gates to sum 1) is the layer's
// workload definition.  Everything here is fp32; bf16 tokens are widened exactly.
#include "common.h"
#include "kernels.h"

namespace moe {

// ----------------------------------------------------------------------------
// logits[t, e] = sum_i x[t, i] W_r[e, i] (+ b[e]).  64x64 output tile per
// workgroup, 256 threads, 4x4 outputs per thread, K staged through LDS in
// steps of 32.  The K order is fixed, so the result is bitwise reproducible.
constexpr int RT_M = 64, RT_N = 64, RT_K = 32;

template <bool X_F32>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void* __restrict__ xv, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ logits, int64_t T, int d, int E) {
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
      if (e < E) logits[t * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 tokens: the same fp32 logits on MFMA.  W_r is split exactly into three
// bf16 planes, w = hi + mid + lo (hi = bf16(w), mid = bf16(w - hi),
// lo = w - hi - mid; 3 x 8 significand bits cover fp32's 24), so every product
// x * w_plane of a bf16 x is exact in fp32 and the MFMA accumulates in fp32.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w,
                                                           int64_t n, bf16_t* __restrict__ w3) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float v = w[i];
    const bf16_t hi = f2bf(v);
    const float r1 = v - bf2f(hi);
    const bf16_t mid = f2bf(r1);
    const bf16_t lo = f2bf(r1 - bf2f(mid));
    w3[i] = hi;
    w3[n + i] = mid;
    w3[2 * n + i] = lo;
  }
}

// BM tokens x 64 experts per workgroup; waves (BM/32) x 2, each a 32 x 32 tile
// with one accumulator per plane; K in 64-element slices through double-buffered,
// XOR-swizzled LDS.  logit = (acc_hi + acc_mid) + acc_lo (+ b).
constexpr int RM_K = 128;   // bytes of K per row per stage

__device__ __forceinline__ int rswz(int r, int c) { return r * RM_K + ((c ^ (r & 7)) << 4); }

template <int BM>
__global__ __launch_bounds__(BM * 4) void router_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w3, const float* __restrict__ bias,
    float* __restrict__ logits, int64_t T, int d, int E) {
  constexpr int NT = BM * 4, BNR = 192;          // threads; B rows = 3 planes x 64 experts
  constexpr int A_LD = BM * 8 / NT, B_LD = BNR * 8 / NT;
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * RM_K];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BNR * RM_K];
  const int64_t t0 = (int64_t)blockIdx.y * BM;
  const int e0 = blockIdx.x * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lg = lane >> 5;
  const int64_t n = (int64_t)E * d;
  const bf16_t* a_src[A_LD];
  const bf16_t* b_src[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = tid + NT * i;
    const int64_t t = min(t0 + q / 8, T - 1);
    a_src[i] = x + t * d + (q % 8) * 8;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int q = tid + NT * i, r = q / 8;
    const int e = min(e0 + r % 64, E - 1);
    b_src[i] = w3 + (r / 64) * n + (int64_t)e * d + (q % 8) * 8;
  }
  u32x4 ra[A_LD], rb[B_LD];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *(const u32x4*)(a_src[i] + kt * 64);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *(const u32x4*)(b_src[i] + kt * 64);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + NT * i;
      *(u32x4*)(As[buf] + rswz(q / 8, q % 8)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int q = tid + NT * i;
      *(u32x4*)(Bs[buf] + rswz(q / 8, q % 8)) = rb[i];
    }
  };
  f32x16 acc[3];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[p][r] = 0.f;
  const int KT = d / 64;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + lg;
      const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(As[cur] + rswz(wm * 32 + lr, c)));
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8 b =
            __builtin_bit_cast(bf16x8, *(const u32x4*)(Bs[cur] + rswz(p * 64 + wn * 32 + lr, c)));
        acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[p], 0, 0, 0);
      }
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }
  const int e = e0 + wn * 32 + lr;
  if (e >= E) return;
  const float be = bias ? bias[e] : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t t = t0 + wm * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
    if (t < T) logits[t * E + e] = (acc[0][r] + acc[1][r]) + acc[2][r] + be;
  }
}

// ----------------------------------------------------------------------------
// One wavefront per token: softmax statistics, top-k (ties to the lower id),
// ascending-id output order, renormalised gates.
template <int VPL>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int choice, rank;
  float gate;
  wave_route_row<VPL>(logits + t * E, E, k, choice, rank, gate);
  if (lane < k) {
    topk_idx[t * k + rank] = choice;
    topk_gate[t * k + rank] = gate;
  }
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
  for (int64_t c = threadIdx.x; c < n; c += blockDim.x) atomicAdd(&hist[idx[c]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) count[e] = hist[e];
}

// workspace: logits [T, E] f32, then the three bf16 planes of W_r [3, E, d] (bf16 tokens)
size_t route_workspace_bytes(int64_t T, int E, int d) {
  return (((size_t)T * E * sizeof(float) + 255) & ~(size_t)255) + (size_t)3 * E * d * 2;
}

hipError_t launch_route(const void* x, bool x_f32, const float* w_r, const float* b_r, int64_t T,
                        int d, int E, int k, float* logits, int32_t* topk_idx, float* topk_gate,
                        int32_t* expert_count, hipStream_t st) {
  if (x_f32) {
    dim3 g1((E + RT_N - 1) / RT_N, (unsigned)((T + RT_M - 1) / RT_M));
    router_logits_kernel<true><<<g1, 256, 0, st>>>(x, w_r, b_r, logits, T, d, E);
  } else {
    // d % 64 == 0 for bf16 layers
    bf16_t* w3 = (bf16_t*)((uint8_t*)logits + (((size_t)T * E * sizeof(float) + 255) & ~(size_t)255));
    const int64_t n = (int64_t)E * d;
    router_split_kernel<<<(unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096), 256, 0, st>>>(w_r, n, w3);
    const unsigned ge = (unsigned)((E + 63) / 64);
    // 64-token tiles when that still gives every CU a workgroup, else 32-token tiles
    if (((T + 63) / 64) * ge >= 256)
      router_mfma_kernel<64><<<dim3(ge, (unsigned)((T + 63) / 64)), 256, 0, st>>>(
          (const bf16_t*)x, w3, b_r, logits, T, d, E);
    else
      router_mfma_kernel<32><<<dim3(ge, (unsigned)((T + 31) / 32)), 128, 0, st>>>(
          (const bf16_t*)x, w3, b_r, logits, T, d, E);
  }
  const unsigned g2 = (unsigned)((T + 3) / 4);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1) router_topk_kernel<1><<<g2, 256, 0, st>>>(logits, T, E, k, topk_idx, topk_gate);
  else if (vpl <= 2) router_topk_kernel<2><<<g2, 256, 0, st>>>(logits, T, E, k, topk_idx, topk_gate);
  else if (vpl <= 4) router_topk_kernel<4><<<g2, 256, 0, st>>>(logits, T, E, k, topk_idx, topk_gate);
  else if (vpl <= 8) router_topk_kernel<8><<<g2, 256, 0, st>>>(logits, T, E, k, topk_idx, topk_gate);
  else router_topk_kernel<16><<<g2, 256, 0, st>>>(logits, T, E, k, topk_idx, topk_gate);
  expert_count_kernel<<<1, 1024, E * sizeof(int32_t), st>>>(topk_idx, T * k, E, expert_count);
  return hipGetLastError();
}

}  // namespace moe
