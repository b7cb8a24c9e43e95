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

size_t route_workspace_bytes(int64_t T, int E) { return (size_t)T * E * sizeof(float); }

hipError_t launch_route(const void* x, bool x_f32, const float* w_r, const float* b_r, int64_t T,
                        int d, int E, int k, float* logits, int32_t* topk_idx, float* topk_gate,
                        int32_t* expert_count, hipStream_t st) {
  dim3 g1((E + RT_N - 1) / RT_N, (unsigned)((T + RT_M - 1) / RT_M));
  if (x_f32)
    router_logits_kernel<true><<<g1, 256, 0, st>>>(x, w_r, b_r, logits, T, d, E);
  else
    router_logits_kernel<false><<<g1, 256, 0, st>>>(x, w_r, b_r, logits, T, d, E);
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
