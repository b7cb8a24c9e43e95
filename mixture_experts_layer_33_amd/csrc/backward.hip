// Backward of the MoE layer, L = sum_t <dy_t, y_t>, routing held fixed.
//
// The pages' ring buffer is walked in reverse in the backward pass to cut
// activation replay (dzen.guru page, ring-buffer paragraph of "Три решения…").
// Here the weight gradients schedule experts E-1 -> 0 and every output tile
// consumes its expert's ring rows from the last slot to the first; everything
// else reads the forward's ring-ordered state (ring_x, saved [A|U]) in place.
//
// Per copy (t, j) of expert e with gate g, a = W_g x, u = W_u x, s = sigmoid(a):
//   dh = W_d^T dy_t;  dg = <dh, h>;  da = g dh u s (1 + a (1 - s));  du = g dh a s
//   dx_t += W_g^T da + W_u^T du;  dW_d += g dy_t h^T;  dW_g += da x^T;  dW_u += du x^T
//   dl_j = g_j (dg_j - sum_i g_i dg_i);  dW_r[e_j] += dl_j x_t;  dx_t += dl_j W_r[e_j]
//
// Kernels:
//   dgrad_kernel<DOWN>  ring rows of dy (gathered) x W_down[e] (K = d rows), epilogue:
//                       SwiGLU backward -> dA|dU (bf16), g*h (bf16), row partials of dg
//   dgrad_kernel<UP>    [dA|dU] x [W_gate[e]; W_up[e]] (K = 2f rows) -> dX per copy (bf16)
//   token_kernel        dg, dl per token; dx = sum_j dX[copy] + dl_j W_r[e_j] (bf16)
//   router_wgrad        dW_r[e] = sum over the segment (last slot first) of dl x  (fp32)
//   wgrad_kernel<DOWN>  dW_down[e] = dY_e^T (g H)_e;  <UP>  [dW_gate;dW_up][e] = [dA|dU]_e^T X_e
// GEMM tiles are 128 x 128 with K in 64-element slices; operands whose K index is
// the row index are transposed 8 x 8 in registers on the way into LDS.  No
// floating-point atomics: every sum has one fixed order.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int BT = 128;            // tile rows and columns
constexpr int BKB = 128;           // K bytes per stage (64 bf16)
constexpr int BCH = BKB / 16;      // 16-byte chunks per row slice

__device__ __forceinline__ int bswz(int r, int c) { return r * BKB + ((c ^ (r & 7)) << 4); }

// 8 rows (K) x 8 bf16 (M or N) in, 8 vectors of 8 bf16 along K out.
__device__ __forceinline__ void transpose8x8(const u32x4 (&r)[8], u32x4 (&o)[8]) {
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = r[2 * q][m >> 1], hi = r[2 * q + 1][m >> 1];
      o[m][q] = (m & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
}

__device__ __forceinline__ int64_t tok_of_slot(const int32_t* slot_copy, int64_t s, int k) {
  return slot_copy[s] / k;
}

// ----------------------------------------------------------------------------- dgrad
struct DgradArgs {
  const bf16_t* A;          // DOWN: dy [T, d] (gathered through slot_copy); UP: dAU [C, 2f]
  const bf16_t* B0;         // DOWN: W_down [E, d, f]; UP: W_gate [E, f, d]
  const bf16_t* B1;         // UP: W_up [E, f, d]
  int K, N;                 // DOWN: K = d, N = f; UP: K = 2f, N = d
  int f;                    // expert intermediate width
  const int32_t* offset;
  const int32_t* tiles;
  const int32_t* ntiles;
  const int32_t* slot_copy;
  const float* gate;        // [T*k] by copy id
  int k;
  int64_t head, C;
  const bf16_t* saved_au;   // DOWN: [C, 2f]
  bf16_t* dau;              // DOWN out: [C, 2f]
  bf16_t* gh;               // DOWN out: [C, f]
  float* dgpart;            // DOWN out: [C, f / BT]
  bf16_t* dxc;              // UP out: [C, d]
};

template <bool DOWN>
__global__ __launch_bounds__(256) void dgrad_kernel(DgradArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BT * BKB];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BT * BKB];
  __shared__ float red[2][BT];
  const int mt = blockIdx.y;
  if (mt >= *p.ntiles) return;
  const int e = p.tiles[2 * mt], row0 = p.tiles[2 * mt + 1];
  const int32_t seg = p.offset[e];
  const int rows = min(BT, p.offset[e + 1] - seg - row0);
  const int n0 = blockIdx.x * BT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lg = lane >> 5;
  const int lda = DOWN ? p.K : p.K;   // row length of A in elements

  // A: 4 chunks per thread, rows (tid + 256 i) / 8
  const bf16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, r = q / BCH;
    const int64_t s = ring_slot(p.head, seg, row0 + min(r, rows - 1), p.C);
    const int64_t arow = DOWN ? tok_of_slot(p.slot_copy, s, p.k) : s;
    a_src[i] = p.A + arow * lda + (q % BCH) * 8;
  }
  // B: threads 0..127 load one 8 (K) x 8 (N) block each: K rows kb*8.., columns nb*8..
  const int kb = (tid & 127) >> 4, nb = tid & 15;
  const bool bload = tid < 128;
  auto brow_ptr = [&](int kk) -> const bf16_t* {   // K row kk of the stacked B
    if (DOWN) return p.B0 + ((int64_t)e * p.K + kk) * p.N;
    return kk < p.f ? p.B0 + ((int64_t)e * p.f + kk) * p.N
                    : p.B1 + ((int64_t)e * p.f + (kk - p.f)) * p.N;
  };

  u32x4 ra[4], rb[8];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *(const u32x4*)(a_src[i] + kt * 64);
    if (bload) {
      const int col = min(n0 + nb * 8, p.N - 8);
#pragma unroll
      for (int q = 0; q < 8; ++q) rb[q] = *(const u32x4*)(brow_ptr(kt * 64 + kb * 8 + q) + col);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      *(u32x4*)(As[buf] + bswz(q / BCH, q % BCH)) = ra[i];
    }
    if (bload) {
      u32x4 o[8];
      transpose8x8(rb, o);
#pragma unroll
      for (int m = 0; m < 8; ++m) *(u32x4*)(Bs[buf] + bswz(nb * 8 + m, kb)) = o[m];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = p.K / 64;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + lg;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(As[cur] + bswz(wm * 64 + i * 32 + lr, c)));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Bs[cur] + bswz(wn * 64 + j * 32 + lr, c)));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  if (DOWN) {
    const int f = p.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        const bool live = m < rows;
        const int64_t s = ring_slot(p.head, seg, row0 + min(m, rows - 1), p.C);
        const float g = p.gate[p.slot_copy[s]];
        float dgp = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 64 + j * 32 + lr;
          const float a = bf2f(p.saved_au[s * 2 * f + n]);
          const float u = bf2f(p.saved_au[s * 2 * f + f + n]);
          const float sg = sigm(a);
          const float h = a * sg * u;
          const float dhr = acc[i][j][r];
          dgp = fmaf(dhr, h, dgp);
          const float dh = g * dhr;
          if (live) {
            p.dau[s * 2 * f + n] = f2bf(dh * u * sg * (1.f + a * (1.f - sg)));
            p.dau[s * 2 * f + f + n] = f2bf(dh * a * sg);
            p.gh[s * f + n] = f2bf(g * h);
          }
        }
        // sum over this wave's 64 columns of the row: 32 lanes x 2 fragments
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) dgp += __shfl_xor(dgp, o, 64);
        if (lr == 0) red[wn][m] = dgp;
      }
    __syncthreads();
    if (tid < rows) {
      const int64_t s = ring_slot(p.head, seg, row0 + tid, p.C);
      p.dgpart[s * (f / BT) + blockIdx.x] = red[0][tid] + red[1][tid];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * 64 + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
          if (m < rows) {
            const int64_t s = ring_slot(p.head, seg, row0 + m, p.C);
            p.dxc[s * p.N + n] = f2bf(acc[i][j][r]);
          }
        }
      }
  }
}

// ----------------------------------------------------------------------------- per token
// dg of each copy (fixed-order sum of the column-tile partials), dl, and
// dx[t] = sum_j (dX[copy_slot[t, j]] + dl_j W_r[e_j]) in ascending expert order.
__global__ __launch_bounds__(256) void token_kernel(const int32_t* __restrict__ copy_slot,
                                                    const int32_t* __restrict__ topk_idx,
                                                    const float* __restrict__ gate,
                                                    const float* __restrict__ dgpart, int nt,
                                                    const bf16_t* __restrict__ dxc,
                                                    const float* __restrict__ w_r, int d, int k,
                                                    float* __restrict__ dl_slot,
                                                    bf16_t* __restrict__ dx) {
  __shared__ int64_t slot[64];
  __shared__ int32_t ex[64];
  __shared__ float dl[64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 64) {   // one wavefront: lanes j < k
    float dg = 0.f, g = 0.f;
    int64_t s = 0;
    if (tid < k) {
      s = copy_slot[t * k + tid];
      g = gate[t * k + tid];
      for (int q = 0; q < nt; ++q) dg += dgpart[s * nt + q];
      slot[tid] = s;
      ex[tid] = topk_idx[t * k + tid];
    }
    const float S = wave_sum(g * dg);
    if (tid < k) {
      const float v = g * (dg - S);
      dl[tid] = v;
      dl_slot[s] = v;
    }
  }
  __syncthreads();
  for (int v = tid; v < d / 8; v += 256) {
    float acc[8] = {};
    for (int j = 0; j < k; ++j) {
      const u32x4 w = ((const u32x4*)(dxc + slot[j] * d))[v];
      const f32x4 r0 = *(const f32x4*)(w_r + (int64_t)ex[j] * d + v * 8);
      const f32x4 r1 = *(const f32x4*)(w_r + (int64_t)ex[j] * d + v * 8 + 4);
      const float l = dl[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += lo_bf(w[q]);
        acc[2 * q + 1] += hi_bf(w[q]);
      }
      acc[0] = fmaf(l, r0[0], acc[0]); acc[1] = fmaf(l, r0[1], acc[1]);
      acc[2] = fmaf(l, r0[2], acc[2]); acc[3] = fmaf(l, r0[3], acc[3]);
      acc[4] = fmaf(l, r1[0], acc[4]); acc[5] = fmaf(l, r1[1], acc[5]);
      acc[6] = fmaf(l, r1[2], acc[6]); acc[7] = fmaf(l, r1[3], acc[7]);
    }
    ((u32x4*)(dx + t * d))[v] = u32x4{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]),
                                      pack_bf2(acc[4], acc[5]), pack_bf2(acc[6], acc[7])};
  }
}

// dW_r[e][c] = sum over the segment's rows, last slot first, of dl * x  (fp32).
__global__ __launch_bounds__(128) void router_wgrad_kernel(const int32_t* __restrict__ offset,
                                                           int64_t head, int64_t C,
                                                           const bf16_t* __restrict__ ring_x,
                                                           const float* __restrict__ dl_slot,
                                                           int d, float* __restrict__ dw_r) {
  const int e = blockIdx.x;
  const int v = blockIdx.y * 128 + threadIdx.x;   // 8 columns per thread
  if (v * 8 >= d) return;
  const int32_t seg = offset[e], n = offset[e + 1] - seg;
  float acc[8] = {};
  for (int i = n - 1; i >= 0; --i) {
    const int64_t s = ring_slot(head, seg, i, C);
    const float l = dl_slot[s];
    const u32x4 w = ((const u32x4*)(ring_x + s * d))[v];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(l, lo_bf(w[q]), acc[2 * q]);
      acc[2 * q + 1] = fmaf(l, hi_bf(w[q]), acc[2 * q + 1]);
    }
  }
  f32x4* dst = (f32x4*)(dw_r + (int64_t)e * d + v * 8);
  dst[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  dst[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// ----------------------------------------------------------------------------- wgrad
struct WgradArgs {
  const bf16_t* A;          // DOWN: dy [T, d] (gathered); UP: dAU [C, 2f]
  const bf16_t* B;          // DOWN: gH [C, f]; UP: ring_x [C, d]
  int M, N;                 // DOWN: M = d, N = f; UP: M = 2f, N = d
  int msplit;               // UP: rows m < msplit go to out0, the rest to out1
  int lda, ldb;
  const int32_t* offset;
  const int32_t* slot_copy;
  int k, E;
  int64_t head, C;
  bf16_t* out0;             // [E, msplit or M, N]
  bf16_t* out1;
};

template <bool GATHER_A>
__global__ __launch_bounds__(256) void wgrad_kernel(WgradArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BT * BKB];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BT * BKB];
  const int e = p.E - 1 - (int)blockIdx.z;        // experts E-1 -> 0
  const int m0 = blockIdx.y * BT, n0 = blockIdx.x * BT;
  const int32_t seg = p.offset[e], nrows = p.offset[e + 1] - seg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lg = lane >> 5;
  // threads 0..127 stage A (8 K-rows x 8 M), threads 128..255 stage B (8 K-rows x 8 N)
  const bool isA = tid < 128;
  const int kb = (tid & 127) >> 4, cb = tid & 15;
  const int KT = (nrows + 63) / 64;

  u32x4 rr[8];
  auto gload = [&](int kt) {
    // stage kt holds segment rows [nrows - 64 (kt + 1), nrows - 64 kt): the last rows first
    const int base = nrows - 64 * (kt + 1) + kb * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = base + q;
      if (i < 0) {
        rr[q] = u32x4{0, 0, 0, 0};
        continue;
      }
      const int64_t s = ring_slot(p.head, seg, i, p.C);
      if (isA) {
        const int64_t row = GATHER_A ? tok_of_slot(p.slot_copy, s, p.k) : s;
        rr[q] = *(const u32x4*)(p.A + row * p.lda + m0 + cb * 8);
      } else {
        rr[q] = *(const u32x4*)(p.B + s * p.ldb + n0 + cb * 8);
      }
    }
  };
  auto sstore = [&](int buf) {
    u32x4 o[8];
    transpose8x8(rr, o);
    uint8_t* dst = isA ? As[buf] : Bs[buf];
#pragma unroll
    for (int m = 0; m < 8; ++m) *(u32x4*)(dst + bswz(cb * 8 + m, kb)) = o[m];
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (KT > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + lg;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(As[cur] + bswz(wm * 64 + i * 32 + lr, c)));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Bs[cur] + bswz(wn * 64 + j * 32 + lr, c)));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        bf16_t* dst = m < p.msplit ? p.out0 + ((int64_t)e * p.msplit + m) * p.N
                                   : p.out1 + ((int64_t)e * (p.M - p.msplit) + (m - p.msplit)) * p.N;
        dst[n] = f2bf(acc[i][j][r]);
      }
    }
}

// ----------------------------------------------------------------------------- launcher
static int bwd_max_tiles(int64_t n, int E) { return (int)((n + BT - 1) / BT) + E; }

struct BwdLayout {
  size_t tiles, dau, gh, dgpart, dxc, dl, total;
};

static BwdLayout bwd_layout(int64_t T, int64_t C, int d, int E, int k, int f) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  BwdLayout L;
  size_t o = 0;
  L.tiles = o; o += al((size_t)(2 * bwd_max_tiles(T * k, E) + 64) * 4);
  L.dau = o;   o += al((size_t)C * 2 * f * 2);
  L.gh = o;    o += al((size_t)C * f * 2);
  L.dgpart = o; o += al((size_t)C * (f / BT) * 4);
  L.dxc = o;   o += al((size_t)C * d * 2);
  L.dl = o;    o += al((size_t)C * 4);
  L.total = o;
  return L;
}

size_t backward_workspace_bytes(int64_t T, int64_t C, int d, int E, int k, int f) {
  return bwd_layout(T, C, d, E, k, f).total;
}

hipError_t launch_backward(const void* dy, const void* x, const float* w_r,
                           const int32_t* topk_idx, const float* topk_gate, const void* ring_x,
                           const int32_t* expert_offset, const int32_t* copy_slot,
                           const int32_t* slot_copy, int64_t head, int64_t C, const void* saved_au,
                           const void* w_gate, const void* w_up, const void* w_down, int64_t T,
                           int d, int E, int k, int f, void* dx, void* dw_gate, void* dw_up,
                           void* dw_down, float* dw_r, void* ws, hipStream_t st) {
  (void)x;
  if (d % BT || f % BT) return hipErrorInvalidValue;
  const BwdLayout L = bwd_layout(T, C, d, E, k, f);
  uint8_t* w = (uint8_t*)ws;
  int32_t* ntiles = (int32_t*)(w + L.tiles);
  int32_t* tiles = ntiles + 64;
  bf16_t* dau = (bf16_t*)(w + L.dau);
  bf16_t* gh = (bf16_t*)(w + L.gh);
  float* dgpart = (float*)(w + L.dgpart);
  bf16_t* dxc = (bf16_t*)(w + L.dxc);
  float* dl = (float*)(w + L.dl);
  const int n = (int)(T * k);
  const int max_tiles = bwd_max_tiles(n, E);

  hipError_t err = launch_build_tiles(expert_offset, E, BT, tiles, ntiles, st);
  if (err != hipSuccess) return err;
  DgradArgs a{};
  a.A = (const bf16_t*)dy;
  a.B0 = (const bf16_t*)w_down;
  a.K = d;
  a.N = f;
  a.f = f;
  a.offset = expert_offset;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.slot_copy = slot_copy;
  a.gate = topk_gate;
  a.k = k;
  a.head = head;
  a.C = C;
  a.saved_au = (const bf16_t*)saved_au;
  a.dau = dau;
  a.gh = gh;
  a.dgpart = dgpart;
  dgrad_kernel<true><<<dim3(f / BT, max_tiles), 256, 0, st>>>(a);
  DgradArgs b = a;
  b.A = dau;
  b.B0 = (const bf16_t*)w_gate;
  b.B1 = (const bf16_t*)w_up;
  b.K = 2 * f;
  b.N = d;
  b.dxc = dxc;
  dgrad_kernel<false><<<dim3(d / BT, max_tiles), 256, 0, st>>>(b);
  token_kernel<<<(unsigned)T, 256, 0, st>>>(copy_slot, topk_idx, topk_gate, dgpart, f / BT, dxc,
                                            w_r, d, k, dl, (bf16_t*)dx);
  router_wgrad_kernel<<<dim3(E, (d / 8 + 127) / 128), 128, 0, st>>>(
      expert_offset, head, C, (const bf16_t*)ring_x, dl, d, dw_r);
  WgradArgs wd{};
  wd.A = (const bf16_t*)dy;
  wd.B = gh;
  wd.M = d;
  wd.N = f;
  wd.msplit = d;
  wd.lda = d;
  wd.ldb = f;
  wd.offset = expert_offset;
  wd.slot_copy = slot_copy;
  wd.k = k;
  wd.E = E;
  wd.head = head;
  wd.C = C;
  wd.out0 = (bf16_t*)dw_down;
  wd.out1 = (bf16_t*)dw_down;
  wgrad_kernel<true><<<dim3(f / BT, d / BT, E), 256, 0, st>>>(wd);
  WgradArgs wu = wd;
  wu.A = dau;
  wu.B = (const bf16_t*)ring_x;
  wu.M = 2 * f;
  wu.N = d;
  wu.msplit = f;
  wu.lda = 2 * f;
  wu.ldb = d;
  wu.out0 = (bf16_t*)dw_gate;
  wu.out1 = (bf16_t*)dw_up;
  wgrad_kernel<false><<<dim3(d / BT, 2 * f / BT, E), 256, 0, st>>>(wu);
  return hipGetLastError();
}

}  // namespace moe
