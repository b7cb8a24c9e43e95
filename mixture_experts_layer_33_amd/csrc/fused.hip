// The whole forward in one launch: route -> dispatch -> gate/up GEMM + SwiGLU -> down
// GEMM -> combine, in one persistent, cooperative kernel.  The dzen.guru page ("Три
// решения, которые дали результат", megakernel paragraph) has one GPU call do the layer
// with one deterministic result; the @cursor_ai tweet on the khabar-ai page calls it a
// single, fully deterministic kernel.
//
// One workgroup of 512 threads (eight waves, the GEMM tile's) per CU; every workgroup
// runs the phases in order and waits at a grid barrier between them:
//   P1 router logit tiles (MFMA, W_r split into     P5 every token row copied to its k slots
//      its bf16 planes as it is staged)            P6 gate/up GEMM tiles, SwiGLU epilogue
//   P2 top-k and gates, one wavefront per token    P7 down GEMM tiles
//   P3 per-chunk expert masks                      P8 gate-weighted combine per token
//   P4 (workgroup 0) offsets, counts, tile list
// Each phase runs the same device code as the separate kernels (route_body.h,
// dispatch_body.h, gemm_body.h, combine_body.h) with the same K splits, tile order and
// cache policies, so every output is bitwise the one of the multi-launch path (the
// 128 x 256 GEMM tile; shapes where the separate kernels take the 256-row tile get the
// same results up to fp32 rounding order).  Nothing is accumulated across workgroups:
// the result does not depend on the schedule.
//
// Measured (2,048 tokens, d 7168, 256 experts, one MI355X): 4.03 ms per call (HIP events
// around back-to-back calls) against 3.89 ms for the separate kernels.  Per-phase
// timestamps of every workgroup (an instrumented copy, 4.16 ms per call) show the GEMM
// phases taking the time of the separate GEMMs (2.29 | 1.34 ms per workgroup); each grid
// barrier costs about 15 us from the last arrival to the release (the arriving
// workgroup's L2 write-back, which cross-XCD visibility needs, is on the critical path),
// eight of them about 0.12 ms.  (W_r's bf16 planes were then a phase of their own; made
// while the logit tiles stage W_r, they save that phase and its barrier: 3.935 -> 3.910 ms.)  Earlier forms: an acquire load in the polling loop
// invalidated the caches at every poll (about 30 us per barrier); a fixed assignment of
// GEMM tiles to workgroups ended each GEMM phase 0.2 ms after its median workgroup; one
// token per workgroup in the copy and combine phases was latency-bound (2x slower).
//
// Grid barrier: a 64-bit ticket counter in the workspace, never reset.  A workgroup takes
// ticket i = old value of the counter and waits until the counter reaches
// (i / G + 1) G (G workgroups), so the counter only grows and is consistent from call to
// call.  Each wait gives up after spin_limit polls: the workgroup sets bit 0 of the status
// word and ends, and so, one barrier later at most, does every other (none passes a
// barrier the one that gave up has not reached), so no phase runs on another phase's
// unfinished output.  A call that finds the bit set does nothing: the counter may then be
// out of step, and the caller clears the status word and the counter.  The launch is
// cooperative: the runtime refuses it unless all G workgroups are resident at once.
#include <hip/hip_runtime.h>

#include "combine_body.h"
#include "common.h"
#include "dispatch_body.h"
#include "gemm_body.h"
#include "kernels.h"
#include "route_body.h"

namespace moe {

constexpr int FU_NT = 512;   // threads per workgroup: the eight waves of the GEMM tile
constexpr int FU_BM = MFMA_BM;

struct FusedArgs {
  const bf16_t* x;
  const float* w_r;
  const float* b_r;
  int64_t T;
  int d, E, k, f;
  int64_t head, C;
  // router
  float* logits;         // [ks, T, E]
  int ks;
  // dispatch
  unsigned long long* masks;   // [nch, E]
  int32_t* base;               // [nch, E]
  int64_t nch;
  // outputs
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* expert_count;
  uint8_t* ring_x;
  int32_t* expert_offset;
  int32_t* copy_slot;
  int32_t* slot_copy;
  bf16_t* y;
  // the two grouped GEMMs (tile list, H, ring_y and saved A|U inside)
  GemmArgs g1, g2;
  int grid1, grid2;      // workgroup counts the separate GEMM launches would use
  // grid barrier and the GEMM phases' per-XCD tile counters [2][8]
  uint32_t* queue;
  unsigned long long* ticket;
  uint32_t* status;
  uint32_t spin_limit;
};

// Returns false (in every thread of the workgroup) when the wait gave up.  Every wave's
// stores reach L2 before the workgroup arrives; thread 0's release (an L2 write-back)
// then publishes them device-wide, and its acquire after the wait (an invalidation of
// this CU's L1 and the XCD's L2 lines) covers every wave of the workgroup, which all
// run on this CU.  The wait polls with relaxed loads: an acquire in the loop would
// invalidate the caches at every poll (about 30 us per barrier, and slower workgroups
// still computing lose their cached lines).
__device__ __forceinline__ bool grid_sync(const FusedArgs a, volatile int* ok) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long G = gridDim.x;
    const unsigned long long i =
        __hip_atomic_fetch_add(a.ticket, 1ull, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long target = (i / G + 1) * G;
    uint32_t polls = 0;
    int passed = 1;
    while (__hip_atomic_load(a.ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++polls > a.spin_limit) {
        __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        passed = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *ok = passed;
  }
  __syncthreads();
  return *ok != 0;
}

// The next place of XCD x (workgroup places x, x + 8, x + 16, ... run there) in a GEMM
// phase, from the XCD's own counter: tiles go to whichever of the XCD's workgroups is
// free, in the order the hardware dispatcher hands a separate launch's workgroups to that
// XCD, so a phase ends when the last tile does rather than when the workgroup with the
// most work does.  Each tile is still computed by exactly one workgroup with its fixed K
// order: the results do not depend on the order of claims.
__device__ __forceinline__ int claim_place(uint32_t* queue, int x, volatile int* slot) {
  if (threadIdx.x == 0)
    *slot = (int)__hip_atomic_fetch_add(queue + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int li = *slot;
  __syncthreads();
  return li * 8 + x;
}

// P5 for one token per wavefront: the copy_slots and row copy of dispatch_copy_token with
// the k slots held by lanes j < k (shuffled to every lane), the same stores.
__device__ __forceinline__ void fused_copy_token(const FusedArgs a, int64_t t) {
  const int lane = threadIdx.x & 63, k = a.k, E = a.E;
  int64_t s = 0;
  if (lane < k) {
    const int64_t chunk = t / DCH;
    const int lc = (int)(t % DCH);
    const int e = a.topk_idx[t * k + lane];
    const unsigned long long mk = a.masks[chunk * E + e];
    const int64_t rank = a.base[chunk * E + e] + __popcll(mk & ((1ull << lc) - 1ull));
    s = a.head + rank;
    if (s >= a.C) s -= a.C;
    a.copy_slot[t * k + lane] = (int32_t)s;
    a.slot_copy[s] = (int32_t)(t * k + lane);
  }
  const int64_t row_bytes = (int64_t)a.d * 2, nv = row_bytes / 16;
  const u32x4* src = (const u32x4*)((const uint8_t*)a.x + t * row_bytes);
  for (int64_t v = lane; v < nv; v += 64) {
    const u32x4 val = __builtin_nontemporal_load(src + v);
    for (int j = 0; j < k; ++j) {
      const int64_t sj = __shfl(s, j, 64);
      __builtin_nontemporal_store(val, (u32x4*)(a.ring_x + sj * row_bytes) + v);
    }
  }
}

// P8 for one token per wavefront: combine_token's sum, element by element the same
// operations in the same order (gates and slots of lanes j < k shuffled to every lane).
__device__ __forceinline__ void fused_combine_token(const FusedArgs a, int64_t t) {
  const int lane = threadIdx.x & 63, k = a.k, d = a.d;
  int64_t sl = 0;
  float gl = 0.f;
  if (lane < k) {
    sl = a.copy_slot[t * k + lane];
    gl = a.topk_gate[t * k + lane];
  }
  const bf16_t* ring_y = (const bf16_t*)a.g2.out;
  for (int v = lane; v < d / 8; v += 64) {
    float acc[8] = {};
    for (int j0 = 0; j0 < k; j0 += 8) {
      u32x4 w[8];
      float g[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {   // copies past k reload the last row, unused
        const int j = min(j0 + jj, k - 1);
        const int64_t s = __shfl(sl, j, 64);
        g[jj] = __shfl(gl, j, 64);
        w[jj] = __builtin_nontemporal_load((const u32x4*)(ring_y + s * d) + v);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= k) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(g[jj], lo_bf(w[jj][q]), acc[2 * q]);
          acc[2 * q + 1] = fmaf(g[jj], hi_bf(w[jj][q]), acc[2 * q + 1]);
        }
      }
    }
    ((u32x4*)(a.y + t * d))[v] =
        u32x4{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]), pack_bf2(acc[4], acc[5]),
              pack_bf2(acc[6], acc[7])};
  }
}

// P4, workgroup 0 alone: per-expert totals (expert_count), exclusive offsets, the chunk
// bases base[c][e] = offset[e] + copies of e in chunks before c (in place over the chunk
// counts), and the GEMM tile list (expert, first row) of 128-row tiles.  Integer sums
// only: the results equal those of the separate scan, count and tile-list kernels.
__device__ __forceinline__ void fused_scan_tiles(const FusedArgs a, uint8_t* lds) {
  int32_t* sc = (int32_t*)lds;   // [1024]
  const int tid = threadIdx.x, E = a.E;
  constexpr int PER = 1024 / FU_NT;
  int32_t run[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + FU_NT * i;
    run[i] = 0;
    if (e < E) {
      for (int64_t c0 = 0; c0 < a.nch; c0 += 16) {
        int32_t h[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) h[u] = c0 + u < a.nch ? a.base[(c0 + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) run[i] += h[u];
      }
    }
    sc[e] = run[i];
  }
  __syncthreads();
  auto scan1024 = [&]() {   // inclusive scan of sc[0 .. 1024)
    for (int o = 1; o < 1024; o <<= 1) {
      int32_t v[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = tid + FU_NT * i;
        v[i] = e >= o ? sc[e - o] : 0;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < PER; ++i) sc[tid + FU_NT * i] += v[i];
      __syncthreads();
    }
  };
  scan1024();
  int32_t off[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + FU_NT * i;
    off[i] = sc[e] - run[i];
    if (e < E) {
      a.expert_offset[e] = off[i];
      a.expert_count[e] = run[i];
      int32_t acc = off[i];
      for (int64_t c0 = 0; c0 < a.nch; c0 += 16) {
        int32_t h[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) h[u] = c0 + u < a.nch ? a.base[(c0 + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (c0 + u < a.nch) {
            a.base[(c0 + u) * E + e] = acc;
            acc += h[u];
          }
      }
    }
    if (e == E - 1) a.expert_offset[E] = sc[e];
  }
  __syncthreads();
  // tile list: row tiles per expert, inclusive scan, then each expert's entries
  int32_t nt[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + FU_NT * i;
    nt[i] = e < E ? (run[i] + FU_BM - 1) / FU_BM : 0;
    sc[e] = nt[i];
  }
  __syncthreads();
  scan1024();
  int32_t* tiles = const_cast<int32_t*>(a.g1.tiles);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + FU_NT * i;
    const int32_t start = sc[e] - nt[i];
    for (int32_t q = 0; q < nt[i]; ++q) {
      tiles[2 * (start + q)] = e;
      tiles[2 * (start + q) + 1] = q * FU_BM;
    }
    if (e == 1023) *const_cast<int32_t*>(a.g1.ntiles) = sc[1023];
  }
  if (tid < 16) a.queue[tid] = 0u;   // the GEMM phases' tile counters, 8 XCDs each
}

template <bool SPLIT>
__device__ __forceinline__ void fused_route_token(const FusedArgs a, int64_t t) {
  const int vpl = (a.E + 63) / 64;
  if (vpl <= 1) route_token<1, SPLIT>(a.logits, a.ks, a.b_r, a.T, a.E, a.k, t, a.topk_idx, a.topk_gate);
  else if (vpl <= 2) route_token<2, SPLIT>(a.logits, a.ks, a.b_r, a.T, a.E, a.k, t, a.topk_idx, a.topk_gate);
  else if (vpl <= 4) route_token<4, SPLIT>(a.logits, a.ks, a.b_r, a.T, a.E, a.k, t, a.topk_idx, a.topk_gate);
  else if (vpl <= 8) route_token<8, SPLIT>(a.logits, a.ks, a.b_r, a.T, a.E, a.k, t, a.topk_idx, a.topk_gate);
  else route_token<16, SPLIT>(a.logits, a.ks, a.b_r, a.T, a.E, a.k, t, a.topk_idx, a.topk_gate);
}

// POL: the cache policy of both GEMMs (equal for bf16: see gemm_policy).
template <int POL>
__global__ __launch_bounds__(FU_NT) void fused_forward_kernel(FusedArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  __shared__ int ok[1];
  const int G = gridDim.x, b = blockIdx.x, tid = threadIdx.x;
  // a barrier of an earlier call gave up: its state may be out of step, do nothing
  if (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u) return;

  // P1: router logits, 128 tokens x 64 experts x K split z per tile
  {
    const int nbx = (a.E + 63) / 64, nby = (int)((a.T + 127) / 128);
    const int ntile = nbx * nby * a.ks;
    for (int v = b; v < ntile; v += G) {
      const int bx = v % nbx, by = (v / nbx) % nby, z = v / (nbx * nby);
      router_mfma_body<128>(a.x, a.w_r, a.logits, a.T, a.d, a.E, bx, by, z, a.ks, lds,
                            lds + 2 * 128 * RM_K);
      __syncthreads();
    }
  }
  if (!grid_sync(a, ok)) return;

  // P2: top-k and gates, one wavefront per token
  {
    const int nw = FU_NT / 64;
    for (int64_t t = (int64_t)b * nw + (tid >> 6); t < a.T; t += (int64_t)G * nw) {
      if (a.ks > 1) fused_route_token<true>(a, t);
      else fused_route_token<false>(a, t);
    }
  }
  if (!grid_sync(a, ok)) return;

  // P3: expert masks and counts per chunk of 64 tokens
  for (int64_t c = b; c < a.nch; c += G) {
    dispatch_hist_chunk(a.topk_idx, a.T, a.k, a.E, a.masks, a.base, c, (unsigned long long*)lds);
    __syncthreads();
  }
  if (!grid_sync(a, ok)) return;

  // P4: offsets, counts and the tile list
  if (b == 0) fused_scan_tiles(a, lds);
  if (!grid_sync(a, ok)) return;

  // P5: token rows into their ring slots, one token per wavefront
  {
    const int nw = FU_NT / 64;
    for (int64_t t = (int64_t)b * nw + (tid >> 6); t < a.T; t += (int64_t)G * nw) fused_copy_token(a, t);
  }
  if (!grid_sync(a, ok)) return;

  // P6, P7: the grouped GEMMs; workgroup b (on XCD b % 8, G being a multiple of 8) takes
  // its XCD's next place of the separate launch's grid until they run out
  __shared__ int place[1];
  for (int vb = claim_place(a.queue, b & 7, place); vb < a.grid1; vb = claim_place(a.queue, b & 7, place)) {
    gg_mfma_body<FU_BM, 256, 2, 4, 128, true, false, 3, POL>(a.g1, vb, lds);
    __syncthreads();
  }
  if (!grid_sync(a, ok)) return;
  for (int vb = claim_place(a.queue + 8, b & 7, place); vb < a.grid2;
       vb = claim_place(a.queue + 8, b & 7, place)) {
    gg_mfma_body<FU_BM, 256, 2, 4, 128, false, false, 3, POL>(a.g2, vb, lds);
    __syncthreads();
  }
  if (!grid_sync(a, ok)) return;

  // P8: y[t] = sum_j g[t, j] ring_y[copy_slot[t, j]], ascending expert order, one token
  // per wavefront
  {
    const int nw = FU_NT / 64;
    for (int64_t t = (int64_t)b * nw + (tid >> 6); t < a.T; t += (int64_t)G * nw) fused_combine_token(a, t);
  }
}

// Workspace: [0, 256) ticket counter (8 bytes), status word (at byte 8), the GEMM phases'
// tile counters (16 words at byte 64, reset inside every call) | logit planes | chunk masks | chunk counts/bases | tile list | H.
struct FusedLayout {
  size_t logits, masks, base, tiles, H, total;
};

static FusedLayout fused_layout(int64_t T, int64_t C, int d, int E, int f) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const int64_t nch = (T + DCH - 1) / DCH;
  const int ks = router_ksplit(T, E, d);
  const int64_t n_max_tiles = max_tiles_for(C, E, FU_BM);   // C >= n copies
  FusedLayout L;
  size_t o = 256;
  L.logits = o; o += al((size_t)ks * T * E * 4);
  L.masks = o;  o += al((size_t)nch * E * 8);
  L.base = o;   o += al((size_t)nch * E * 4);
  L.tiles = o;  o += al((size_t)(2 * n_max_tiles + 64) * 4);
  L.H = o;      o += al((size_t)C * f * 2);
  L.total = o;
  return L;
}

size_t fused_workspace_bytes(int64_t T, int64_t C, int d, int E, int f) {
  return fused_layout(T, C, d, E, f).total;
}

hipError_t launch_forward_fused(const void* x, const float* w_r, const float* b_r,
                                const void* w_gate, const void* w_up, const void* w_down,
                                int64_t T, int d, int E, int k, int f, int64_t C, int64_t head,
                                int32_t* topk_idx, float* topk_gate, int32_t* expert_count,
                                void* ring_x, int32_t* expert_offset, int32_t* copy_slot,
                                int32_t* slot_copy, void* ring_y, void* saved_au, void* y,
                                uint32_t spin_limit, void* ws, hipStream_t st) {
  const FusedLayout L = fused_layout(T, C, d, E, f);
  uint8_t* w = (uint8_t*)ws;
  const int64_t n = T * k;
  FusedArgs a{};
  a.x = (const bf16_t*)x;
  a.w_r = w_r;
  a.b_r = b_r;
  a.T = T; a.d = d; a.E = E; a.k = k; a.f = f;
  a.head = head; a.C = C;
  a.logits = (float*)(w + L.logits);
  a.ks = router_ksplit(T, E, d);
  a.masks = (unsigned long long*)(w + L.masks);
  a.base = (int32_t*)(w + L.base);
  a.nch = (T + DCH - 1) / DCH;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.expert_count = expert_count;
  a.ring_x = (uint8_t*)ring_x;
  a.expert_offset = expert_offset;
  a.copy_slot = copy_slot;
  a.slot_copy = slot_copy;
  a.y = (bf16_t*)y;
  int32_t* ntiles = (int32_t*)(w + L.tiles);
  const int max_tiles = max_tiles_for(n, E, FU_BM);
  GemmArgs g1{};
  g1.A = (const uint8_t*)ring_x;
  g1.B0 = (const uint8_t*)w_gate;
  g1.B1 = (const uint8_t*)w_up;
  g1.K = d;
  g1.N = f;
  g1.offset = expert_offset;
  g1.tiles = ntiles + 64;
  g1.ntiles = ntiles;
  g1.head = head;
  g1.C = C;
  g1.out = w + L.H;
  g1.saved_au = (uint16_t*)saved_au;
  g1.a_rows = C;
  g1.b_rows = (int64_t)E * f;
  GemmArgs g2 = g1;
  g2.A = w + L.H;
  g2.B0 = (const uint8_t*)w_down;
  g2.B1 = nullptr;
  g2.K = f;
  g2.N = d;
  g2.out = (uint8_t*)ring_y;
  g2.saved_au = nullptr;
  g2.b_rows = (int64_t)E * d;
  g1.rotate = kstart_rotates(true, 1, n, E, FU_BM);
  g2.rotate = kstart_rotates(false, 1, n, E, FU_BM);
  a.g1 = g1;
  a.g2 = g2;
  const int nt1 = (f + 127) / 128, nt2 = (d + 255) / 256;
  a.grid1 = (int)(8 * (((int64_t)max_tiles * nt1 + 7) / 8));
  a.grid2 = (int)(8 * (((int64_t)max_tiles * nt2 + 7) / 8));
  a.ticket = (unsigned long long*)w;
  a.queue = (uint32_t*)(w + 64);
  a.status = (uint32_t*)(w + 8);
  a.spin_limit = spin_limit ? spin_limit : (1u << 22);

  const int pol = gemm_policy(true, 1, n, E, FU_BM);   // equals the down GEMM's for bf16
  const void* kern = pol == 3 ? (const void*)fused_forward_kernel<3> : (const void*)fused_forward_kernel<2>;
  const size_t lds = std::max<size_t>((size_t)3 * StageLayout<FU_BM, 256, 128, false, 8>::SIZE,
                                      EpiLayout<FU_BM, 256, true, false>::SIZE);
  hipError_t err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  int dev = 0, ncu = 0, per_cu = 0;
  if ((err = hipGetDevice(&dev)) != hipSuccess) return err;
  if ((err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return err;
  if ((err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, FU_NT, lds)) != hipSuccess)
    return err;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const int G = ncu - ncu % 8;   // one workgroup per CU, a multiple of the 8 XCDs
  if (G < 8) return hipErrorInvalidConfiguration;
  void* args[] = {&a};
  return hipLaunchCooperativeKernel(kern, dim3(G), dim3(FU_NT), args, (unsigned)lds, st);
}

}  // namespace moe
