// Small-batch decode in two kernels, parallel over outputs, with no permuted
// token buffer.  The warp-decode page (toolnavs.com, sections "Cursor a réécrit
// le décodage de MoE" and "1.84x plus de vitesse…") turns the parallel axis from
// experts to outputs: each unit of work owns output values, the layer runs in
// two kernels, and the staging buffers of the expert-centric scheme disappear.
// On gfx950 the unit is a 64-lane wavefront owning a group of output elements.
//
// Kernel 1 (cooperative, persistent):
//   A. router logits (one wavefront per expert row of W_r, all B tokens) and
//      the shared expert's gate/up rows: hs[b][i] = silu(a) u, fp32;
//   B. grid barrier;
//   C. every workgroup rebuilds top-k and gates from the logits, and the list of
//      experts the batch selected; one wavefront per (expert, row i) streams the
//      W_gate and W_up rows once and writes h[b][j][i] = silu(a) u (fp32,
//      token-major) for every token b that chose that expert as its j-th.
// Kernel 2: one wavefront per group of DEC_R output rows o streams W_down[e][o,:]
//   of every selected expert and W_s_down[o,:], and writes
//   y[b][o] = sum_j g[b][j] (W_down[e_bj][o,:] . h[b][j]) + W_s_down[o,:] . hs[b]
//   in bf16 (fp32 partials per lane, one fixed-order wave reduction).
//
// h stays fp32 end to end (the page reports decode output closer to the fp32
// reference).  Weight rows are read with 16-byte loads, one contiguous KB per
// wavefront instruction.
#include <hip/hip_cooperative_groups.h>

#include "common.h"
#include "kernels.h"

namespace cg = cooperative_groups;

namespace moe {

constexpr int DEC_BMAX = 8;      // largest batch
constexpr int DEC_KMAX = 16;     // largest top-k
constexpr int DEC_THREADS = 512;
constexpr int DEC_R = 8;         // output rows per wavefront in kernel 2

struct DecodeArgs {
  const bf16_t* x;
  const float* w_r;
  const float* b_r;
  const bf16_t* w_gate;
  const bf16_t* w_up;
  const bf16_t* w_down;
  const bf16_t* ws_gate;
  const bf16_t* ws_up;
  const bf16_t* ws_down;
  int B, d, E, k, f, fs;
  float* logits;   // [B][E]
  float* hs;       // [B][fs]
  float* h;        // [B][k][f]
  int32_t* uniq;   // [DEC_BMAX*DEC_KMAX + 1]: selected experts ascending, then their count
  int32_t* topk_idx;
  float* topk_gate;
  bf16_t* y;
};

// dot of a bf16 weight row with the B tokens held in LDS (bf16), per-lane partials.
// Lane handles elements q*512 + lane*8 + [0, 8).
__device__ __forceinline__ void row_dots_bf16(const bf16_t* __restrict__ wrow,
                                              const bf16_t* __restrict__ xs, int B, int d,
                                              float* part) {
  const int lane = threadIdx.x & 63;
  for (int b = 0; b < DEC_BMAX; ++b) part[b] = 0.f;
  for (int q = lane * 8; q < d; q += 512) {
    const u32x4 w = *(const u32x4*)(wrow + q);
    float wf[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) { wf[2 * r] = lo_bf(w[r]); wf[2 * r + 1] = hi_bf(w[r]); }
#pragma unroll
    for (int b = 0; b < DEC_BMAX; ++b) {
      if (b >= B) break;
      const u32x4 xv = *(const u32x4*)(xs + b * d + q);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        part[b] = fmaf(wf[2 * r], lo_bf(xv[r]), part[b]);
        part[b] = fmaf(wf[2 * r + 1], hi_bf(xv[r]), part[b]);
      }
    }
  }
}

__global__ __launch_bounds__(DEC_THREADS) void decode_k1(DecodeArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  bf16_t* xs = (bf16_t*)lds;                                   // [B][d]
  int32_t* sel = (int32_t*)(lds + (size_t)p.B * p.d * 2);      // [B][k]
  int32_t* uniq = sel + DEC_BMAX * DEC_KMAX;                   // [<= B*k]
  int32_t* nuniq = uniq + DEC_BMAX * DEC_KMAX;
  uint32_t* bits = (uint32_t*)(nuniq + 1);                     // [E/32]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6, nwave = DEC_THREADS / 64;
  const int gw = blockIdx.x * nwave + wave, W = gridDim.x * nwave;
  const int B = p.B, d = p.d, E = p.E, k = p.k, f = p.f, fs = p.fs;

  for (int v = tid; v < B * d / 8; v += DEC_THREADS) ((u32x4*)xs)[v] = ((const u32x4*)p.x)[v];
  __syncthreads();

  // ---- A: router rows and shared gate/up rows
  for (int item = gw; item < E + fs; item += W) {
    float part[DEC_BMAX];
    if (item < E) {
      const float* wr = p.w_r + (int64_t)item * d;
      for (int b = 0; b < DEC_BMAX; ++b) part[b] = 0.f;
      for (int q = lane * 8; q < d; q += 512) {
        const f32x4 w0 = *(const f32x4*)(wr + q), w1 = *(const f32x4*)(wr + q + 4);
#pragma unroll
        for (int b = 0; b < DEC_BMAX; ++b) {
          if (b >= B) break;
          const u32x4 xv = *(const u32x4*)(xs + b * d + q);
          part[b] = fmaf(w0[0], lo_bf(xv[0]), part[b]);
          part[b] = fmaf(w0[1], hi_bf(xv[0]), part[b]);
          part[b] = fmaf(w0[2], lo_bf(xv[1]), part[b]);
          part[b] = fmaf(w0[3], hi_bf(xv[1]), part[b]);
          part[b] = fmaf(w1[0], lo_bf(xv[2]), part[b]);
          part[b] = fmaf(w1[1], hi_bf(xv[2]), part[b]);
          part[b] = fmaf(w1[2], lo_bf(xv[3]), part[b]);
          part[b] = fmaf(w1[3], hi_bf(xv[3]), part[b]);
        }
      }
      for (int b = 0; b < B; ++b) {
        const float l = wave_sum(part[b]);
        if (lane == 0) p.logits[b * E + item] = l + (p.b_r ? p.b_r[item] : 0.f);
      }
    } else {
      const int i = item - E;
      float pu[DEC_BMAX];
      row_dots_bf16(p.ws_gate + (int64_t)i * d, xs, B, d, part);
      row_dots_bf16(p.ws_up + (int64_t)i * d, xs, B, d, pu);
      for (int b = 0; b < B; ++b) {
        const float a = wave_sum(part[b]);
        const float u = wave_sum(pu[b]);
        if (lane == 0) p.hs[b * fs + i] = silu(a) * u;
      }
    }
  }

  // ---- B: every workgroup waits for all logits
  cg::this_grid().sync();

  // ---- C: routing in LDS (one wavefront per token), then the selected experts' rows
  for (int b = wave; b < B; b += nwave) {
    int choice, rank;
    float gate;
    wave_route_row<16>(p.logits + b * E, E, k, choice, rank, gate);
    if (lane < k) {
      sel[b * DEC_KMAX + rank] = choice;             // ascending expert id
      if (blockIdx.x == 0) {
        p.topk_idx[b * k + rank] = choice;
        p.topk_gate[b * k + rank] = gate;
      }
    }
  }
  for (int w = tid; w < (E + 31) / 32; w += DEC_THREADS) bits[w] = 0u;
  __syncthreads();
  for (int q = tid; q < B * k; q += DEC_THREADS)
    atomicOr(&bits[sel[(q / k) * DEC_KMAX + q % k] >> 5], 1u << (sel[(q / k) * DEC_KMAX + q % k] & 31));
  __syncthreads();
  if (tid == 0) {
    int u = 0;
    for (int e = 0; e < E; ++e)
      if ((bits[e >> 5] >> (e & 31)) & 1u) uniq[u++] = e;
    *nuniq = u;
    if (blockIdx.x == 0) {       // the list kernel 2 reads
      for (int q = 0; q < u; ++q) p.uniq[q] = uniq[q];
      p.uniq[DEC_BMAX * DEC_KMAX] = u;
    }
  }
  __syncthreads();
  const int U = *nuniq;
  for (int item = gw; item < U * f; item += W) {
    const int e = uniq[item / f], i = item % f;
    float pa[DEC_BMAX], pu[DEC_BMAX];
    row_dots_bf16(p.w_gate + ((int64_t)e * f + i) * d, xs, B, d, pa);
    row_dots_bf16(p.w_up + ((int64_t)e * f + i) * d, xs, B, d, pu);
    for (int b = 0; b < B; ++b) {
      int j = -1;
      for (int q = 0; q < k; ++q) j = sel[b * DEC_KMAX + q] == e ? q : j;
      if (j < 0) continue;                 // uniform across the wave
      const float a = wave_sum(pa[b]);
      const float u = wave_sum(pu[b]);
      if (lane == 0) p.h[((int64_t)b * k + j) * f + i] = silu(a) * u;
    }
  }
}

__global__ __launch_bounds__(256) void decode_k2(DecodeArgs p) {
  __shared__ int32_t sel[DEC_BMAX * DEC_KMAX];
  __shared__ float gate[DEC_BMAX * DEC_KMAX];
  __shared__ int32_t uniq[DEC_BMAX * DEC_KMAX];
  __shared__ int32_t nuniq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = p.B, d = p.d, k = p.k, f = p.f, fs = p.fs;
  for (int q = tid; q < B * k; q += 256) {
    sel[q] = p.topk_idx[q];
    gate[q] = p.topk_gate[q];
    uniq[q] = p.uniq[q];
  }
  if (tid == 0) nuniq = p.uniq[DEC_BMAX * DEC_KMAX];
  __syncthreads();
  const int o0 = (blockIdx.x * 4 + (tid >> 6)) * DEC_R;
  if (o0 >= d) return;
  float acc[DEC_R][DEC_BMAX];
#pragma unroll
  for (int r = 0; r < DEC_R; ++r)
#pragma unroll
    for (int b = 0; b < DEC_BMAX; ++b) acc[r][b] = 0.f;

  const int U = nuniq;
  for (int ui = 0; ui <= U; ++ui) {
    const bool shared = ui == U;
    if (shared && fs == 0) break;
    const int e = shared ? -1 : uniq[ui];
    const int ff = shared ? fs : f;
    const bf16_t* wbase = shared ? p.ws_down : p.w_down + (int64_t)e * d * f;
    for (int q0 = 0; q0 < ff; q0 += 512) {
      const int q = q0 + lane * 8;
      const bool ok = q < ff;
      float w[DEC_R][8];
#pragma unroll
      for (int r = 0; r < DEC_R; ++r) {
        const int o = min(o0 + r, d - 1);
        const u32x4 v = ok ? *(const u32x4*)(wbase + (int64_t)o * ff + q) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c) { w[r][2 * c] = lo_bf(v[c]); w[r][2 * c + 1] = hi_bf(v[c]); }
      }
#pragma unroll
      for (int b = 0; b < DEC_BMAX; ++b) {
        if (b >= B) break;
        int j = -1;
        float g = 1.f;
        if (!shared) {
          for (int qq = 0; qq < k; ++qq)
            if (sel[b * k + qq] == e) { j = qq; g = gate[b * k + qq]; }
          if (j < 0) continue;
        }
        const float* hv = shared ? p.hs + (int64_t)b * fs : p.h + ((int64_t)b * k + j) * f;
        float hh[8];
        if (ok) {
          const f32x4 h0 = *(const f32x4*)(hv + q), h1 = *(const f32x4*)(hv + q + 4);
          hh[0] = h0[0]; hh[1] = h0[1]; hh[2] = h0[2]; hh[3] = h0[3];
          hh[4] = h1[0]; hh[5] = h1[1]; hh[6] = h1[2]; hh[7] = h1[3];
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) hh[c] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < DEC_R; ++r) {
          float s = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) s = fmaf(w[r][c], hh[c], s);
          acc[r][b] = fmaf(g, s, acc[r][b]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < DEC_R; ++r)
#pragma unroll
    for (int b = 0; b < DEC_BMAX; ++b) {
      if (b >= B) break;
      const float v = wave_sum(acc[r][b]);
      if (lane == 0 && o0 + r < d) p.y[(int64_t)b * d + o0 + r] = f2bf(v);
    }
}

size_t decode_workspace_bytes(int B, int E, int k, int f, int fs) {
  return ((size_t)B * E + (size_t)B * (fs > 0 ? fs : 1) + (size_t)B * k * f) * sizeof(float) +
         (DEC_BMAX * DEC_KMAX + 1) * sizeof(int32_t);
}

hipError_t launch_decode(const void* x, const float* w_r, const float* b_r, const void* w_gate,
                         const void* w_up, const void* w_down, const void* ws_gate,
                         const void* ws_up, const void* ws_down, int B, int d, int E, int k,
                         int f, int fs, void* y, int32_t* topk_idx, float* topk_gate, void* ws,
                         hipStream_t st) {
  if (B > DEC_BMAX || k > DEC_KMAX || d % 512 != 0 || f % 512 != 0 || (fs && fs % 512 != 0))
    return hipErrorInvalidValue;
  DecodeArgs a;
  a.x = (const bf16_t*)x;
  a.w_r = w_r;
  a.b_r = b_r;
  a.w_gate = (const bf16_t*)w_gate;
  a.w_up = (const bf16_t*)w_up;
  a.w_down = (const bf16_t*)w_down;
  a.ws_gate = (const bf16_t*)ws_gate;
  a.ws_up = (const bf16_t*)ws_up;
  a.ws_down = (const bf16_t*)ws_down;
  a.B = B; a.d = d; a.E = E; a.k = k; a.f = f; a.fs = fs;
  a.logits = (float*)ws;
  a.hs = a.logits + (size_t)B * E;
  a.h = a.hs + (size_t)B * (fs > 0 ? fs : 1);
  a.uniq = (int32_t*)(a.h + (size_t)B * k * f);
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.y = (bf16_t*)y;

  const size_t lds = (size_t)B * d * 2 + (2 * DEC_BMAX * DEC_KMAX + 1) * 4 + ((E + 31) / 32) * 4;
  int dev = 0, ncu = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  err = hipFuncSetAttribute((const void*)decode_k1, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
  if (err != hipSuccess) return err;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_k1, DEC_THREADS, lds);
  if (err != hipSuccess) return err;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const int grid = ncu * per_cu;   // every workgroup resident: the grid barrier cannot stall
  void* kargs[] = {&a};
  err = hipLaunchCooperativeKernel((const void*)decode_k1, dim3(grid), dim3(DEC_THREADS), kargs,
                                   (unsigned)lds, st);
  if (err != hipSuccess) return err;
  const int waves = (d + DEC_R - 1) / DEC_R;
  decode_k2<<<(waves + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
