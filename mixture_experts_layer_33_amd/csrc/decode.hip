// Small-batch decode: the router, then two kernels parallel over outputs, with no permuted
// token buffer.  The warp-decode page (toolnavs.com, sections "Cursor a réécrit
// le décodage de MoE" and "1.84x plus de vitesse…") turns the parallel axis from
// experts to outputs: each unit of work owns output values, the layer runs in
// two kernels, and the staging buffers of the expert-centric scheme disappear.
// On gfx950 the unit is a 64-lane wavefront owning a group of output elements.
//
// Kernel 0: the router logits, quarter rows of W_r (fp32) per wavefront, all B
//   tokens each, the four partial sums kept apart (no cross-workgroup sync: the
//   next launch consumes them).
// Kernel 1: every workgroup rebuilds top-k and gates from the logits
//   (((p0 + p1) + p2) + p3 + bias) and the list of experts the batch selected; then
//   its wavefronts claim rows one at a time: the shared expert's gate/up rows,
//   hs[b][i] = silu(a) u, and the selected experts' rows (expert, row i): the
//   W_gate and W_up rows are read once and h[b][j][i] = silu(a) u (fp32,
//   token-major) is written for every token b that chose that expert as its j-th.
// Kernel 2: one wavefront per group of DEC_R output rows o streams W_down[e][o,:]
//   of every selected expert and W_s_down[o,:], and writes
//   y[b][o] = sum_j g[b][j] (W_down[e_bj][o,:] . h[b][j]) + W_s_down[o,:] . hs[b]
//   in bf16 (fp32 partials per lane, one fixed-order wave reduction).
//
// h stays fp32 end to end (the page reports decode output closer to the fp32
// reference).  Weight rows are read with 16-byte loads, one contiguous KB per
// wavefront instruction, with the non-temporal cache policy: every weight byte is
// used once per call, and on gfx950 such streaming loads reach a higher HBM rate
// (a bare 16-byte-per-lane read: about 6.9 against 6.2 TB/s; at B = 1 the call went
// from 154.6 to 138-141 us) while W_r, x and h keep the default policy.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int DEC_BMAX = 8;      // largest batch
constexpr int DEC_KMAX = 16;     // largest top-k
constexpr int DEC_THREADS = 512; // kernel 1: 8 wavefronts share the token rows in LDS
constexpr int DEC_RP = 4;        // router row parts (kernel 0)
constexpr int DQ = 16;           // largest row, in groups of 512 elements (d <= 8192)
constexpr int DEC_R = 4;         // output rows per wavefront in kernel 2
constexpr int DEC_NF = 8;        // largest f (and fs) in groups of 512 in kernel 2
// Kernel 2's workgroups hold ceil(ceil(d / DEC_R) / CUs) wavefronts (at most this many), so
// every CU gets one workgroup and an equal share of the output rows: with four-wavefront
// workgroups (448 at d = 7168) three quarters of the CUs ran two of them and finished last.
// Rows of more than 5 x 512 elements keep four-wavefront workgroups: at two wavefronts per
// SIMD their two register sets would spill.
constexpr int DEC_K2_MAXW = 8;
__host__ __device__ constexpr int dec_k2_maxw(int nf) { return nf <= 5 ? DEC_K2_MAXW : 4; }

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
  float* logits;   // [DEC_RP][B][E]: the partial logits of the quarters of each W_r row
  float* hs;       // [B][fs]
  float* h;        // [B][k][f]
  int32_t* uniq;   // [DEC_BMAX*DEC_KMAX + 1]: selected experts ascending, then their count
  int32_t* topk_idx;
  float* topk_gate;
  bf16_t* y;
};

// Lane `lane` owns elements c*512 + lane*8 + [0, 8) of a row, c < nq.  All loads
// of a row are issued before any is used, so a wavefront keeps the whole row
// (up to 16 KB) in flight.
template <int NQ>
__device__ __forceinline__ void load_row(const bf16_t* __restrict__ row, u32x4 (&w)[NQ]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < NQ; ++c)
    w[c] = __builtin_nontemporal_load((const u32x4*)(row + c * 512 + lane * 8));
}

// per-lane partial of <row, x_b> with x_b (bf16) in LDS
template <int NQ>
__device__ __forceinline__ float part_dot(const u32x4 (&w)[NQ], const bf16_t* __restrict__ xb) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    const u32x4 xv = *(const u32x4*)(xb + c * 512 + lane * 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s = fmaf(lo_bf(w[c][r]), lo_bf(xv[r]), s);
      s = fmaf(hi_bf(w[c][r]), hi_bf(xv[r]), s);
    }
  }
  return s;
}

// per-lane partials of <gate row, x_b> and <up row, x_b>, each chunk of x_b read once
template <int NQ>
__device__ __forceinline__ void part_dot2(const u32x4 (&wg)[NQ], const u32x4 (&wu)[NQ],
                                          const bf16_t* __restrict__ xb, float& sa, float& su) {
  const int lane = threadIdx.x & 63;
  sa = 0.f;
  su = 0.f;
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    const u32x4 xv = *(const u32x4*)(xb + c * 512 + lane * 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x0 = lo_bf(xv[r]), x1 = hi_bf(xv[r]);
      sa = fmaf(lo_bf(wg[c][r]), x0, sa);
      sa = fmaf(hi_bf(wg[c][r]), x1, sa);
      su = fmaf(lo_bf(wu[c][r]), x0, su);
      su = fmaf(hi_bf(wu[c][r]), x1, su);
    }
  }
}

// 64-bit masks of the (token, slot) pairs q = b*k + j whose expert is e (B*k <= 128)
__device__ __forceinline__ void pairs_of(const int32_t* sel, int B, int k, int e,
                                         unsigned long long& m0, unsigned long long& m1) {
  const int lane = threadIdx.x & 63;
  const int q0 = lane, q1 = lane + 64;
  m0 = __ballot(q0 < B * k && sel[(q0 / k) * DEC_KMAX + q0 % k] == e);
  m1 = __ballot(q1 < B * k && sel[(q1 / k) * DEC_KMAX + q1 % k] == e);
}

// Kernel 0: wavefront w computes part w % DEC_RP of W_r row w / DEC_RP: chunks
// [p QC, min(NQ, (p + 1) QC)) (loads past the end repeat the last chunk and are not
// used; an empty part contributes 0).  x is read through the cache (B d bf16).
template <int NQ>   // d = NQ * 512
__global__ __launch_bounds__(256) void decode_router(DecodeArgs p) {
  constexpr int d = NQ * 512;
  constexpr int QC = (NQ + DEC_RP - 1) / DEC_RP;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int B = p.B, E = p.E;
  if (item >= DEC_RP * E) return;
  const int e = item / DEC_RP, part = item % DEC_RP;
  const int c0 = part * QC, nc = min(NQ - c0, QC);
  const float* wr = p.w_r + (int64_t)e * d;
  f32x4 w0[QC], w1[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    const int cc = min(c0 + c, NQ - 1);
    w0[c] = *(const f32x4*)(wr + cc * 512 + lane * 8);
    w1[c] = *(const f32x4*)(wr + cc * 512 + lane * 8 + 4);
  }
  for (int b = 0; b < B; ++b) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      if (c >= nc) break;
      const u32x4 xv = *(const u32x4*)(p.x + (int64_t)b * d + (c0 + c) * 512 + lane * 8);
      s = fmaf(w0[c][0], lo_bf(xv[0]), s);
      s = fmaf(w0[c][1], hi_bf(xv[0]), s);
      s = fmaf(w0[c][2], lo_bf(xv[1]), s);
      s = fmaf(w0[c][3], hi_bf(xv[1]), s);
      s = fmaf(w1[c][0], lo_bf(xv[2]), s);
      s = fmaf(w1[c][1], hi_bf(xv[2]), s);
      s = fmaf(w1[c][2], lo_bf(xv[3]), s);
      s = fmaf(w1[c][3], hi_bf(xv[3]), s);
    }
    const float l = wave_sum(s);
    if (lane == 0) p.logits[((int64_t)part * B + b) * E + e] = l;
  }
}

// Kernel 1's rows: the shared expert's fs rows, then the (distinct expert, row) items
// of the U selected experts, numbered g = 0 .. fs + U f - 1.  Workgroup b owns the rows g
// with (g / 8) mod G = b (groups of 8 consecutive rows dealt round-robin, so the rows in
// flight across the chip are neighbours), and its wavefronts claim them in order from a
// counter in LDS: the c-th claim is row 8b + c mod 8 + (c / 8) 8G.  Every row is computed
// whole by one wavefront with the same code, so the results do not depend on who takes it.
//
// Timestamps of a B = 1 call (wall clock, per wavefront) showed where the time went when
// the routing sat between barriers: the weight stream ran at ~6.9 TB/s once every
// workgroup had its expert list, but that took ~20 us from the kernel's start, because
// the routing wave's logit loads queued behind the shared expert's rows already in
// flight.  Now the routing waves issue their logit loads before any weight row is
// requested, and after one barrier (x in LDS, logits arrived) nothing waits for the
// routing: the other wavefronts stream the shared expert's rows at once, and a wavefront
// that claims a routed row before the expert list is ready waits on an LDS flag that the
// last routing wavefront raises (a bounded wait: were it ever exceeded, the wavefront would
// stop claiming rather than hang).
constexpr int DEC_SPIN_MAX = 1 << 20;   // ~64 cycles each: ~30 ms, far beyond any routing

template <int NQ>   // d = NQ * 512
__global__ __launch_bounds__(DEC_THREADS) void decode_k1(DecodeArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int claims, routed, ready;
  bf16_t* xs = (bf16_t*)lds;                                   // [B][d]
  int32_t* sel = (int32_t*)(lds + (size_t)p.B * p.d * 2);      // [B][DEC_KMAX]
  int32_t* uniq = sel + DEC_BMAX * DEC_KMAX;                   // [<= B*k]
  int32_t* nuniq = uniq + DEC_BMAX * DEC_KMAX;
  uint32_t* bits = (uint32_t*)(nuniq + 1);                     // [E/32]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nwave = DEC_THREADS / 64;
  const int W = gridDim.x * nwave;
  const int B = p.B, E = p.E, k = p.k, f = p.f, fs = p.fs;
  constexpr int d = NQ * 512;
  const bool routes = wave < B;   // wavefronts 0..B-1 route one token each

  // The logits (four partial planes + bias) of all of the lane's experts, loaded
  // unconditionally (indices clamped, values past E masked afterwards) so the loads go
  // out together, and before any weight row is requested.
  float lv[16];
  if (routes) {
    const float* l0 = p.logits + (int64_t)wave * E;
    const int64_t ps = (int64_t)B * E;   // stride between the partial-logit planes
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = min(lane + 64 * i, E - 1);
      lv[i] = (((l0[e] + l0[ps + e]) + l0[2 * ps + e]) + l0[3 * ps + e]) + (p.b_r ? p.b_r[e] : 0.f);
    }
  }
  for (int v = tid; v < B * d / 8; v += DEC_THREADS) ((u32x4*)xs)[v] = ((const u32x4*)p.x)[v];
  for (int w = tid; w < (E + 31) / 32; w += DEC_THREADS) bits[w] = 0u;
  if (tid == 0) {
    claims = 0;
    routed = 0;
    ready = 0;
  }
  __syncthreads();

  if (routes) {
    int choice, rank;
    float gate;
    wave_route_row_f<16>([&](int e) { return lv[(e - lane) >> 6]; }, E, k, choice, rank, gate);
    if (lane < k) {
      sel[wave * DEC_KMAX + rank] = choice;          // ascending expert id
      if (blockIdx.x == 0) {
        p.topk_idx[wave * k + rank] = choice;
        p.topk_gate[wave * k + rank] = gate;
      }
    }
    int done = 0;
    if (lane == 0) done = __hip_atomic_fetch_add(&routed, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(done) == B - 1) {
      // the last routing wavefront: the distinct experts, ascending
      for (int q = lane; q < B * k; q += 64) {
        const int e = sel[(q / k) * DEC_KMAX + q % k];
        atomicOr(&bits[e >> 5], 1u << (e & 31));
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");   // every lane's bits before lane 0 reads them
      if (lane == 0) {
        int u = 0;
        for (int w = 0; w < (E + 31) / 32; ++w)
          for (uint32_t m = bits[w]; m; m &= m - 1) uniq[u++] = w * 32 + __builtin_ctz(m);
        *nuniq = u;
        if (blockIdx.x == 0) {     // the list kernel 2 reads
          for (int q = 0; q < u; ++q) p.uniq[q] = uniq[q];
          p.uniq[DEC_BMAX * DEC_KMAX] = u;
        }
        __hip_atomic_store(&ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }

  // The next row of this wavefront, or -1 once the workgroup's rows are all claimed (or
  // the expert list never came).  Once the list is ready, lane l keeps the experts of the
  // (token, slot) pairs l and l + 64 (16 bits each, 0xffff for none: E <= 1024), so a
  // row's pairs are two ballots.
  bool listed = false;
  uint32_t pe = 0xffffffffu;
  auto next = [&]() __attribute__((always_inline)) -> int {
    int c = 0;
    if (lane == 0) c = __hip_atomic_fetch_add(&claims, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    c = __builtin_amdgcn_readfirstlane(c);
    const int g = blockIdx.x * nwave + c % nwave + (c / nwave) * W;
    if (g < fs) return g;
    if (!listed) {
      for (int n = 0; n < DEC_SPIN_MAX && !listed; ++n) {
        listed = __hip_atomic_load(&ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
        if (!listed) __builtin_amdgcn_s_sleep(1);
      }
      if (!listed) return -1;
      const int q0 = lane, q1 = lane + 64;
      const uint32_t e0 = q0 < B * k ? (uint32_t)sel[(q0 / k) * DEC_KMAX + q0 % k] : 0xffffu;
      const uint32_t e1 = q1 < B * k ? (uint32_t)sel[(q1 / k) * DEC_KMAX + q1 % k] : 0xffffu;
      pe = e0 | e1 << 16;
    }
    return g < fs + *nuniq * f ? g : -1;
  };
  // the W_gate and W_up rows of row g (routed rows only once the expert list is ready)
  auto load = [&](int g, u32x4(&wg)[NQ], u32x4(&wu)[NQ]) __attribute__((always_inline)) {
    const bf16_t *rg, *ru;
    if (g < fs) {
      rg = p.ws_gate + (int64_t)g * d;
      ru = p.ws_up + (int64_t)g * d;
    } else {
      const int it = g - fs, e = uniq[it / f], i = it % f;
      rg = p.w_gate + ((int64_t)e * f + i) * d;
      ru = p.w_up + ((int64_t)e * f + i) * d;
    }
    load_row<NQ>(rg, wg);
    load_row<NQ>(ru, wu);
  };
  // hs[b][g] = silu(a) u for every token (shared row), or h[b][j][i] for every token b
  // that chose the row's expert as its j-th
  auto consume = [&](int g, const u32x4(&wg)[NQ], const u32x4(&wu)[NQ]) __attribute__((always_inline)) {
    if (g < fs) {
      for (int b = 0; b < B; ++b) {
        float sa, su;
        part_dot2<NQ>(wg, wu, xs + b * d, sa, su);
        const float a = wave_sum(sa), u = wave_sum(su);
        if (lane == 0) p.hs[b * fs + g] = silu(a) * u;
      }
      return;
    }
    const int it = g - fs, e = uniq[it / f], i = it % f;
    const unsigned long long m0 = __ballot((pe & 0xffffu) == (uint32_t)e), m1 = __ballot(pe >> 16 == (uint32_t)e);
    for (int half = 0; half < 2; ++half)
      for (unsigned long long m = half ? m1 : m0; m; m &= m - 1) {
        const int q = half * 64 + __builtin_ctzll(m), b = q / k, j = q % k;
        float sa, su;
        part_dot2<NQ>(wg, wu, xs + b * d, sa, su);
        const float a = wave_sum(sa), u = wave_sum(su);
        if (lane == 0) p.h[((int64_t)b * k + j) * f + i] = silu(a) * u;
      }
  };

  // One row in flight per wavefront: a second register set (the next row's loads issued
  // before this row is consumed) measured slower at B = 1 / 4 / 8 (132.6 / 451 / 838 us
  // against 130.7 / 449 / 831): 2,048 wavefronts already keep ~57 MB in flight.
  u32x4 wg[NQ], wu[NQ];
  for (int row = next(); row >= 0; row = next()) {
    load(row, wg, wu);
    consume(row, wg, wu);
  }
}

// Kernel 2: a wavefront owns DEC_R output rows.  For every selected expert (then
// the shared one) it issues the loads of its DEC_R W_down rows at once, and adds
// g * <row, h> for each token that chose the expert into per-lane partials;
// one fixed-order wave reduction per (row, token) at the end.
template <int NF>   // f = fs (when present) = NF * 512
__global__ __launch_bounds__(64 * dec_k2_maxw(NF)) void decode_k2(DecodeArgs p) {
  __shared__ int32_t sel[DEC_BMAX * DEC_KMAX];
  __shared__ float gate[DEC_BMAX * DEC_KMAX];
  __shared__ int32_t uniq[DEC_BMAX * DEC_KMAX];
  __shared__ int32_t nuniq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = p.B, d = p.d, k = p.k, f = p.f, fs = p.fs;
  (void)f;
  for (int q = tid; q < DEC_BMAX * DEC_KMAX; q += blockDim.x) {
    sel[q] = -1;
    gate[q] = 0.f;
    uniq[q] = p.uniq[q];
  }
  if (tid == 0) nuniq = p.uniq[DEC_BMAX * DEC_KMAX];
  __syncthreads();
  for (int q = tid; q < B * k; q += blockDim.x) {   // b < B <= 8, j < k <= 16: index < 128
    sel[(q / k) * DEC_KMAX + q % k] = p.topk_idx[q];
    gate[(q / k) * DEC_KMAX + q % k] = p.topk_gate[q];
  }
  __syncthreads();
  const int o0 = (int)(blockIdx.x * (blockDim.x >> 6) + (tid >> 6)) * DEC_R;
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
    constexpr int ff = NF * 512;
    const bf16_t* wbase = shared ? p.ws_down : p.w_down + (int64_t)e * d * ff;
    u32x4 w[DEC_R][NF];
#pragma unroll
    for (int r = 0; r < DEC_R; ++r) {
      const int o = min(o0 + r, d - 1);
#pragma unroll
      for (int c = 0; c < NF; ++c)
        w[r][c] = __builtin_nontemporal_load((const u32x4*)(wbase + (int64_t)o * ff + c * 512 + lane * 8));
    }
    unsigned long long m0 = 0, m1 = 0;
    if (shared) m0 = B >= 64 ? ~0ull : ((1ull << B) - 1);   // bit b: token b, weight 1
    else pairs_of(sel, B, k, e, m0, m1);
    for (int half = 0; half < 2; ++half)
      for (unsigned long long m = half ? m1 : m0; m; m &= m - 1) {
        const int q = half * 64 + __builtin_ctzll(m);
        const int b = shared ? q : q / k, j = shared ? 0 : q % k;
        const float g = shared ? 1.f : gate[b * DEC_KMAX + j];
        const float* hv = shared ? p.hs + (int64_t)b * fs : p.h + ((int64_t)b * k + j) * f;
        float s[DEC_R] = {};
#pragma unroll
        for (int c = 0; c < NF; ++c) {
          const f32x4 h0 = *(const f32x4*)(hv + c * 512 + lane * 8);
          const f32x4 h1 = *(const f32x4*)(hv + c * 512 + lane * 8 + 4);
#pragma unroll
          for (int r = 0; r < DEC_R; ++r) {
            s[r] = fmaf(lo_bf(w[r][c][0]), h0[0], s[r]);
            s[r] = fmaf(hi_bf(w[r][c][0]), h0[1], s[r]);
            s[r] = fmaf(lo_bf(w[r][c][1]), h0[2], s[r]);
            s[r] = fmaf(hi_bf(w[r][c][1]), h0[3], s[r]);
            s[r] = fmaf(lo_bf(w[r][c][2]), h1[0], s[r]);
            s[r] = fmaf(hi_bf(w[r][c][2]), h1[1], s[r]);
            s[r] = fmaf(lo_bf(w[r][c][3]), h1[2], s[r]);
            s[r] = fmaf(hi_bf(w[r][c][3]), h1[3], s[r]);
          }
        }
        // add into the accumulator of token b (static index for the registers)
#pragma unroll
        for (int bb = 0; bb < DEC_BMAX; ++bb)
          if (bb == b)
#pragma unroll
            for (int r = 0; r < DEC_R; ++r) acc[r][bb] = fmaf(g, s[r], acc[r][bb]);
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

// Kernel 2 for one token (B = 1).  Its k experts are distinct and topk_idx lists them
// ascending, so expert u of the sequence (u < k, then the shared expert) has exactly one
// h row, h[u] (hs for the shared one), and the gate topk_gate[u].  A wavefront keeps two
// experts in flight: the W_down rows and the h row of expert u + 1 are requested before
// expert u is consumed, so waiting for expert u never waits for anything issued after it
// (vector memory operations complete in issue order; decode_k2, whose h rows are read as
// each expert is consumed, cannot prefetch that way).  The products and sums are those of
// decode_k2 in the same order: bitwise the same y.
template <int NF>   // f = fs (when present) = NF * 512
__global__ __launch_bounds__(64 * DEC_K2_MAXW) void decode_k2_one(DecodeArgs p) {
  __shared__ int32_t ex[DEC_KMAX];
  __shared__ float gt[DEC_KMAX];
  const int tid = threadIdx.x, lane = tid & 63;
  const int d = p.d, k = p.k, fs = p.fs;
  constexpr int ff = NF * 512;
  if (tid < k) {
    ex[tid] = p.topk_idx[tid];
    gt[tid] = p.topk_gate[tid];
  }
  __syncthreads();
  const int o0 = (int)(blockIdx.x * (blockDim.x >> 6) + (tid >> 6)) * DEC_R;
  if (o0 >= d) return;
  const int U = k + (fs > 0 ? 1 : 0);
  auto fetch = [&](int u, u32x4(&w)[DEC_R][NF], f32x4(&h)[NF][2]) __attribute__((always_inline)) {
    const bool shared = u == k;
    const bf16_t* wbase = shared ? p.ws_down : p.w_down + (int64_t)ex[u] * d * ff;
#pragma unroll
    for (int r = 0; r < DEC_R; ++r) {
      const int o = min(o0 + r, d - 1);
#pragma unroll
      for (int c = 0; c < NF; ++c)
        w[r][c] = __builtin_nontemporal_load((const u32x4*)(wbase + (int64_t)o * ff + c * 512 + lane * 8));
    }
    const float* hv = shared ? p.hs : p.h + (int64_t)u * ff;
#pragma unroll
    for (int c = 0; c < NF; ++c) {
      h[c][0] = *(const f32x4*)(hv + c * 512 + lane * 8);
      h[c][1] = *(const f32x4*)(hv + c * 512 + lane * 8 + 4);
    }
  };
  float acc[DEC_R] = {};
  auto consume = [&](int u, const u32x4(&w)[DEC_R][NF], const f32x4(&h)[NF][2]) __attribute__((always_inline)) {
    const float g = u == k ? 1.f : gt[u];
    float s[DEC_R] = {};
#pragma unroll
    for (int c = 0; c < NF; ++c) {
      const f32x4 h0 = h[c][0], h1 = h[c][1];
#pragma unroll
      for (int r = 0; r < DEC_R; ++r) {
        s[r] = fmaf(lo_bf(w[r][c][0]), h0[0], s[r]);
        s[r] = fmaf(hi_bf(w[r][c][0]), h0[1], s[r]);
        s[r] = fmaf(lo_bf(w[r][c][1]), h0[2], s[r]);
        s[r] = fmaf(hi_bf(w[r][c][1]), h0[3], s[r]);
        s[r] = fmaf(lo_bf(w[r][c][2]), h1[0], s[r]);
        s[r] = fmaf(hi_bf(w[r][c][2]), h1[1], s[r]);
        s[r] = fmaf(lo_bf(w[r][c][3]), h1[2], s[r]);
        s[r] = fmaf(hi_bf(w[r][c][3]), h1[3], s[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < DEC_R; ++r) acc[r] = fmaf(g, s[r], acc[r]);
  };
  u32x4 wa[DEC_R][NF], wb[DEC_R][NF];
  f32x4 ha[NF][2], hb[NF][2];
  fetch(0, wa, ha);
  for (int u = 0; u < U; u += 2) {
    if (u + 1 < U) fetch(u + 1, wb, hb);
    consume(u, wa, ha);
    if (u + 1 >= U) break;
    if (u + 2 < U) fetch(u + 2, wa, ha);
    consume(u + 1, wb, hb);
  }
#pragma unroll
  for (int r = 0; r < DEC_R; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0 && o0 + r < d) p.y[o0 + r] = f2bf(v);
  }
}

// Workspace: partial logits [DEC_RP,B,E] f32 | shared h [B,max(fs,1)] f32 |
// h [B,k,f] f32 | unique-expert list [DEC_BMAX*DEC_KMAX + 1] i32.
size_t decode_workspace_bytes(int B, int E, int k, int f, int fs) {
  return ((size_t)DEC_RP * B * E + (size_t)B * (fs > 0 ? fs : 1) + (size_t)B * k * f) * sizeof(float) +
         (DEC_BMAX * DEC_KMAX + 1) * sizeof(int32_t);
}

// Scratch for callers that cannot allocate (moe_decode_noalloc): the decode workspace of
// the largest shape that variant accepts, in a file-scope device array.  Each GPU the
// library runs on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol): the
// address used is the one hipGetSymbolAddress returns on each device, taken once per
// device with that device current.
static __device__ __align__(256) uint8_t scratch[DECODE_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
static std::once_flag scratch_once[SCRATCH_MAX_DEVICES];
static void* scratch_ptr[SCRATCH_MAX_DEVICES];
static hipError_t scratch_err[SCRATCH_MAX_DEVICES];

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = scratch_ptr[dev];
  return scratch_err[dev];
}

hipError_t launch_decode(const void* x, const float* w_r, const float* b_r, const void* w_gate,
                         const void* w_up, const void* w_down, const void* ws_gate,
                         const void* ws_up, const void* ws_down, int B, int d, int E, int k,
                         int f, int fs, void* y, int32_t* topk_idx, float* topk_gate, void* ws,
                         hipStream_t st) {
  if (B > DEC_BMAX || k > DEC_KMAX || d % 512 != 0 || f % 512 != 0 || (fs && fs != f) ||
      d > DQ * 512 || f > DEC_NF * 512)
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
  a.hs = a.logits + (size_t)DEC_RP * B * E;
  a.h = a.hs + (size_t)B * (fs > 0 ? fs : 1);
  a.uniq = (int32_t*)(a.h + (size_t)B * k * f);
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.y = (bf16_t*)y;

  const void* k1 = nullptr;
  switch (d / 512) {
#define K1_CASE(n) case n: k1 = (const void*)decode_k1<n>; break;
    K1_CASE(1) K1_CASE(2) K1_CASE(3) K1_CASE(4) K1_CASE(5) K1_CASE(6) K1_CASE(7) K1_CASE(8)
    K1_CASE(9) K1_CASE(10) K1_CASE(11) K1_CASE(12) K1_CASE(13) K1_CASE(14) K1_CASE(15) K1_CASE(16)
#undef K1_CASE
    default: return hipErrorInvalidValue;
  }
  const size_t lds = (size_t)B * d * 2 + (2 * DEC_BMAX * DEC_KMAX + 1) * 4 + ((E + 31) / 32) * 4;
  int dev = 0, ncu = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  // the largest LDS any call of this d may need, asked for on every call (host side only)
  err = hipFuncSetAttribute(k1, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)((size_t)DEC_BMAX * d * 2 + (2 * DEC_BMAX * DEC_KMAX + 1) * 4 +
                                  (1024 / 32) * 4));
  if (err != hipSuccess) return err;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k1, DEC_THREADS, lds);
  if (err != hipSuccess) return err;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  // at most 2 workgroups per CU: enough wavefronts to keep every row's loads in flight
  const int grid = ncu * (per_cu < 2 ? per_cu : 2);
  const unsigned g0 = (unsigned)((DEC_RP * E + 3) / 4);
  switch (d / 512) {
#define K1_LAUNCH(n) \
  case n:                                                  \
    decode_router<n><<<g0, 256, 0, st>>>(a);               \
    decode_k1<n><<<grid, DEC_THREADS, lds, st>>>(a);       \
    break;
    K1_LAUNCH(1) K1_LAUNCH(2) K1_LAUNCH(3) K1_LAUNCH(4) K1_LAUNCH(5) K1_LAUNCH(6) K1_LAUNCH(7)
    K1_LAUNCH(8) K1_LAUNCH(9) K1_LAUNCH(10) K1_LAUNCH(11) K1_LAUNCH(12) K1_LAUNCH(13)
    K1_LAUNCH(14) K1_LAUNCH(15) K1_LAUNCH(16)
#undef K1_LAUNCH
    default: return hipErrorInvalidValue;
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int waves2 = (d + DEC_R - 1) / DEC_R;
  const int nw2 = std::min(dec_k2_maxw(f / 512), std::max(1, (waves2 + ncu - 1) / ncu));
  const unsigned g2 = (unsigned)((waves2 + nw2 - 1) / nw2), t2 = (unsigned)(64 * nw2);
  if (B == 1 && f / 512 <= 4) {   // two experts in flight per wavefront (registers allow up to f = 2048)
    switch (f / 512) {
      case 1: decode_k2_one<1><<<g2, t2, 0, st>>>(a); break;
      case 2: decode_k2_one<2><<<g2, t2, 0, st>>>(a); break;
      case 3: decode_k2_one<3><<<g2, t2, 0, st>>>(a); break;
      default: decode_k2_one<4><<<g2, t2, 0, st>>>(a); break;
    }
    return hipGetLastError();
  }
  switch (f / 512) {
    case 1: decode_k2<1><<<g2, t2, 0, st>>>(a); break;
    case 2: decode_k2<2><<<g2, t2, 0, st>>>(a); break;
    case 3: decode_k2<3><<<g2, t2, 0, st>>>(a); break;
    case 4: decode_k2<4><<<g2, t2, 0, st>>>(a); break;
    case 5: decode_k2<5><<<g2, t2, 0, st>>>(a); break;
    case 6: decode_k2<6><<<g2, t2, 0, st>>>(a); break;
    case 7: decode_k2<7><<<g2, t2, 0, st>>>(a); break;
    case 8: decode_k2<8><<<g2, t2, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
