// Host side of the C ABI declared in include/moe.h: argument validation from
// the shape alone (before any HIP call), workspace sizing, and launches on the
// caller's stream.  No allocation, no host synchronisation, no exception
// crosses the boundary.
#include "moe.h"

#include <exception>

#include "kernels.h"

namespace {

constexpr int MAX_E = 1024;   // expert ids fit one workgroup scan
constexpr int MAX_K = 32;

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// A per-token array (x, dy, y, dx, topk_idx, topk_gate, copy_slot) may be NULL when
// the call has no tokens, like any zero-length array.
bool missing_tok(const void* p, int64_t T) { return p == nullptr && T > 0; }

// Zero `words` 32-bit words (a fill kernel rather than hipMemsetAsync, so that a call
// stays safe to capture in a graph).  Used for the outputs of calls with no tokens.
__global__ void zero_words_kernel(uint32_t* __restrict__ p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
hipError_t zero_words(void* p, size_t words, hipStream_t st) {
  if (words == 0) return hipSuccess;
  const size_t blocks = (words + 255) / 256;
  zero_words_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, st>>>((uint32_t*)p, words);
  return hipGetLastError();
}

bool bad_dtype(int dt) { return dt != MOE_F32 && dt != MOE_BF16 && dt != MOE_MXFP8; }

// Shape checks common to the forward calls.  K-dimension multiples follow the
// kernels' 128-byte K slices: bf16 needs d, f % 64; MX needs d, f % 128.
int check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_NULL;
  if (bad_dtype(s->dtype)) return MOE_ERR_DTYPE;
  if (s->tokens < 0 || s->hidden <= 0 || s->experts <= 0 || s->ffn <= 0 || s->shared_ffn < 0)
    return MOE_ERR_SHAPE;
  if (s->experts > MAX_E || s->top_k < 1 || s->top_k > s->experts || s->top_k > MAX_K)
    return MOE_ERR_SHAPE;
  if (s->tokens > (int64_t)1 << 30) return MOE_ERR_SHAPE;
  const int q = s->dtype == MOE_MXFP8 ? 128 : s->dtype == MOE_BF16 ? 64 : 8;
  if (s->hidden % q || s->ffn % q) return MOE_ERR_SHAPE;
  if (s->capacity < s->tokens * s->top_k) return MOE_ERR_CAPACITY;
  if (s->capacity > ((int64_t)1 << 31) - 1) return MOE_ERR_SHAPE;
  // The MFMA grouped GEMM addresses its ring-ordered operand rows (ring_x [C, d] in
  // GEMM-1, H [C, f] in GEMM-2) with 32-bit byte offsets from the array's start:
  // each of those arrays must stay below 4 GiB.
  if (s->dtype != MOE_F32) {
    const int64_t eb = s->dtype == MOE_BF16 ? 2 : 1;
    const int64_t row = (s->hidden > s->ffn ? s->hidden : s->ffn) * eb;
    if (s->capacity * row >= ((int64_t)1 << 32)) return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* s, int op) {
  if (!s || check_shape(s) != MOE_OK) return 0;
  const int64_t T = s->tokens, n = s->tokens * s->top_k, C = s->capacity;
  switch (op) {
    case MOE_OP_ROUTE: return align256(moe::route_workspace_bytes(T, s->experts, s->hidden));
    case MOE_OP_DISPATCH: return align256(moe::dispatch_workspace_bytes(T, s->experts));
    case MOE_OP_EXPERT_FFN:
      return align256(moe::ffn_workspace_bytes(n, C, s->hidden, s->experts, s->ffn, s->dtype));
    case MOE_OP_COMBINE: return 0;
    case MOE_OP_DECODE:
      return align256(moe::decode_workspace_bytes((int)T, s->experts, s->top_k, s->ffn,
                                                  s->shared_ffn));
    case MOE_OP_FORWARD:
      return s->dtype == MOE_BF16
                 ? align256(moe::fused_workspace_bytes(T, C, s->hidden, s->experts, s->ffn))
                 : 0;
    case MOE_OP_BACKWARD:
      if (s->dtype == MOE_MXFP8)
        return align256(moe::backward_mx_workspace_bytes(T, C, s->hidden, s->experts, s->top_k,
                                                         s->ffn));
      return align256(moe::backward_workspace_bytes(T, C, s->hidden, s->experts, s->top_k,
                                                    s->ffn));
    default: return 0;
  }
}

int moe_check_shape(const moe_shape* s) { return check_shape(s); }

const char* moe_status_string(int st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid shape";
    case MOE_ERR_CAPACITY: return "ring capacity below tokens * top_k (tokens would be dropped)";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_DTYPE: return "unknown or unsupported dtype";
    case MOE_ERR_SCRATCH:
      return "shape needs more scratch than the library's static buffer holds (moe_decode_noalloc)";
    default: return "unknown status";
  }
}

int moe_route(const moe_shape* s, const void* x, const float* w_router, const float* b_router,
              int32_t* topk_idx, float* topk_gate, int32_t* expert_count, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  try {
    int st = check_shape(s);
    if (st) return st;
    const int64_t T = s->tokens;
    if (missing_tok(x, T) || !w_router || missing_tok(topk_idx, T) || missing_tok(topk_gate, T) ||
        !expert_count || !workspace)
      return MOE_ERR_NULL;
    if (workspace_bytes < moe_workspace_bytes(s, MOE_OP_ROUTE)) return MOE_ERR_WORKSPACE;
    if (s->tokens == 0) return hip_status(zero_words(expert_count, (size_t)s->experts, stream));
    return hip_status(moe::launch_route(x, s->dtype == MOE_F32, w_router, b_router, s->tokens,
                                        s->hidden, s->experts, s->top_k, (float*)workspace,
                                        topk_idx, topk_gate, expert_count, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx, int64_t ring_head,
                 void* ring_x, uint8_t* ring_x_scale, int32_t* expert_offset, int32_t* copy_slot,
                 int32_t* slot_copy, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    int st = check_shape(s);
    if (st) return st;
    const int64_t T = s->tokens;
    if (missing_tok(x, T) || missing_tok(topk_idx, T) || !ring_x || !expert_offset ||
        missing_tok(copy_slot, T) || !slot_copy || !workspace)
      return MOE_ERR_NULL;
    if (s->dtype == MOE_MXFP8 && !ring_x_scale) return MOE_ERR_NULL;
    if (ring_head < 0 || ring_head >= s->capacity) return MOE_ERR_SHAPE;
    if (workspace_bytes < moe_workspace_bytes(s, MOE_OP_DISPATCH)) return MOE_ERR_WORKSPACE;
    if (s->tokens == 0)   // no copies: every expert's segment is empty
      return hip_status(zero_words(expert_offset, (size_t)s->experts + 1, stream));
    return hip_status(moe::launch_dispatch(
        x, s->dtype == MOE_F32 ? 4 : 2, s->dtype == MOE_MXFP8, topk_idx, s->tokens, s->hidden,
        s->experts, s->top_k, ring_head, s->capacity, ring_x, ring_x_scale, expert_offset,
        copy_slot, slot_copy, workspace, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_expert_ffn_timed(const moe_shape* s, const void* ring_x, const uint8_t* ring_x_scale,
                   const int32_t* expert_offset, int64_t ring_head, const void* w_gate,
                   const void* w_up, const void* w_down, const uint8_t* w_gate_scale,
                   const uint8_t* w_up_scale, const uint8_t* w_down_scale, void* ring_y,
                   void* saved_au, void* workspace, size_t workspace_bytes,
                         hipEvent_t* events, hipStream_t stream) {
  try {
    int st = check_shape(s);
    if (st) return st;
    if (!ring_x || !expert_offset || !w_gate || !w_up || !w_down || !ring_y || !workspace)
      return MOE_ERR_NULL;
    const bool mx = s->dtype == MOE_MXFP8;
    if (mx && (!ring_x_scale || !w_gate_scale || !w_up_scale || !w_down_scale))
      return MOE_ERR_NULL;
    if (saved_au && s->dtype == MOE_F32) return MOE_ERR_DTYPE;
    if (ring_head < 0 || ring_head >= s->capacity) return MOE_ERR_SHAPE;
    if (workspace_bytes < moe_workspace_bytes(s, MOE_OP_EXPERT_FFN)) return MOE_ERR_WORKSPACE;
    if (s->tokens == 0) return MOE_OK;
    return hip_status(moe::launch_ffn(s->dtype, ring_x, ring_x_scale, expert_offset, ring_head,
                                      s->capacity, s->tokens * s->top_k, s->hidden, s->experts,
                                      s->ffn, w_gate, w_up, w_down, w_gate_scale, w_up_scale,
                                      w_down_scale, ring_y, saved_au, workspace, events, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_expert_ffn(const moe_shape* s, const void* ring_x, const uint8_t* ring_x_scale,
                   const int32_t* expert_offset, int64_t ring_head, const void* w_gate,
                   const void* w_up, const void* w_down, const uint8_t* w_gate_scale,
                   const uint8_t* w_up_scale, const uint8_t* w_down_scale, void* ring_y,
                   void* saved_au, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return moe_expert_ffn_timed(s, ring_x, ring_x_scale, expert_offset, ring_head, w_gate, w_up,
                              w_down, w_gate_scale, w_up_scale, w_down_scale, ring_y, saved_au,
                              workspace, workspace_bytes, nullptr, stream);
}

int moe_combine(const moe_shape* s, const void* ring_y, const int32_t* copy_slot,
                const float* topk_gate, void* y, hipStream_t stream) {
  try {
    int st = check_shape(s);
    if (st) return st;
    const int64_t T = s->tokens;
    if (!ring_y || missing_tok(copy_slot, T) || missing_tok(topk_gate, T) || missing_tok(y, T))
      return MOE_ERR_NULL;
    return hip_status(moe::launch_combine(s->dtype == MOE_F32, ring_y, copy_slot, topk_gate,
                                          s->tokens, s->hidden, s->top_k, y, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_forward(const moe_shape* s, const void* x, const float* w_router, const float* b_router,
                const void* w_gate, const void* w_up, const void* w_down, int64_t ring_head,
                int32_t* topk_idx, float* topk_gate, int32_t* expert_count, void* ring_x,
                int32_t* expert_offset, int32_t* copy_slot, int32_t* slot_copy, void* ring_y,
                void* saved_au, void* y, uint32_t spin_limit, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  try {
    int st = check_shape(s);
    if (st) return st;
    if (s->dtype != MOE_BF16) return MOE_ERR_DTYPE;
    const int64_t T = s->tokens;
    if (missing_tok(x, T) || !w_router || !w_gate || !w_up || !w_down ||
        missing_tok(topk_idx, T) || missing_tok(topk_gate, T) || !expert_count || !ring_x ||
        !expert_offset || missing_tok(copy_slot, T) || !slot_copy || !ring_y ||
        missing_tok(y, T) || !workspace)
      return MOE_ERR_NULL;
    if (ring_head < 0 || ring_head >= s->capacity) return MOE_ERR_SHAPE;
    if (workspace_bytes < moe_workspace_bytes(s, MOE_OP_FORWARD)) return MOE_ERR_WORKSPACE;
    if (T == 0) {   // no copies: every count and segment offset is zero
      hipError_t err = zero_words(expert_count, (size_t)s->experts, stream);
      if (err == hipSuccess) err = zero_words(expert_offset, (size_t)s->experts + 1, stream);
      return hip_status(err);
    }
    return hip_status(moe::launch_forward_fused(
        x, w_router, b_router, w_gate, w_up, w_down, T, s->hidden, s->experts, s->top_k, s->ffn,
        s->capacity, ring_head, topk_idx, topk_gate, expert_count, ring_x, expert_offset,
        copy_slot, slot_copy, ring_y, saved_au, y, spin_limit, workspace, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

namespace {
// Checks of moe_decode and moe_decode_noalloc apart from the workspace.
int decode_checks(const moe_shape* s, const void* x, const float* w_router, const void* w_gate,
                  const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                  const void* ws_down, const void* y, const int32_t* topk_idx,
                  const float* topk_gate) {
  int st = check_shape(s);
  if (st) return st;
  if (s->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (s->tokens < 1 || s->tokens > 8 || s->top_k > 16) return MOE_ERR_SHAPE;
  if (s->hidden % 512 || s->ffn % 512 || s->hidden > 8192 || s->ffn > 4096) return MOE_ERR_SHAPE;
  if (s->shared_ffn != 0 && s->shared_ffn != s->ffn) return MOE_ERR_SHAPE;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y || !topk_idx || !topk_gate)
    return MOE_ERR_NULL;
  if (s->shared_ffn > 0 && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_NULL;
  return MOE_OK;
}
}  // namespace

int moe_decode(const moe_shape* s, const void* x, const float* w_router, const float* b_router,
               const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
               const void* ws_up, const void* ws_down, void* y, int32_t* topk_idx,
               float* topk_gate, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    int st = decode_checks(s, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                           topk_idx, topk_gate);
    if (st) return st;
    if (!workspace) return MOE_ERR_NULL;
    if (workspace_bytes < moe_workspace_bytes(s, MOE_OP_DECODE)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_decode(x, w_router, b_router, w_gate, w_up, w_down, ws_gate,
                                         ws_up, ws_down, (int)s->tokens, s->hidden, s->experts,
                                         s->top_k, s->ffn, s->shared_ffn, y, topk_idx, topk_gate,
                                         workspace, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_decode_noalloc(const moe_shape* s, const void* x, const float* w_router,
                       const float* b_router, const void* w_gate, const void* w_up,
                       const void* w_down, const void* ws_gate, const void* ws_up,
                       const void* ws_down, void* y, int32_t* topk_idx, float* topk_gate,
                       hipStream_t stream) {
  try {
    int st = decode_checks(s, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                           topk_idx, topk_gate);
    if (st) return st;
    if (moe_workspace_bytes(s, MOE_OP_DECODE) > moe::DECODE_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    void* scratch = nullptr;
    hipError_t err = moe::decode_scratch(&scratch);
    if (err != hipSuccess || !scratch) return MOE_ERR_HIP;
    return hip_status(moe::launch_decode(x, w_router, b_router, w_gate, w_up, w_down, ws_gate,
                                         ws_up, ws_down, (int)s->tokens, s->hidden, s->experts,
                                         s->top_k, s->ffn, s->shared_ffn, y, topk_idx, topk_gate,
                                         scratch, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_backward(const moe_shape* s, const void* dy, const void* x, const float* w_router,
                 const int32_t* topk_idx, const float* topk_gate, const void* ring_x,
                 const int32_t* expert_offset, const int32_t* copy_slot,
                 const int32_t* slot_copy, int64_t ring_head, const void* saved_au,
                 const void* w_gate, const void* w_up, const void* w_down, void* dx,
                 void* dw_gate, void* dw_up, void* dw_down, float* dw_router, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  try {
    int st = check_shape(s);
    if (st) return st;
    if (s->dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (s->hidden % 128 || s->ffn % 128) return MOE_ERR_SHAPE;   // 128 x 128 gradient tiles
    const int64_t T = s->tokens;
    if (missing_tok(dy, T) || missing_tok(x, T) || !w_router || missing_tok(topk_idx, T) ||
        missing_tok(topk_gate, T) || !ring_x || !expert_offset ||
        missing_tok(copy_slot, T) || !slot_copy || !saved_au || !w_gate || !w_up || !w_down ||
        missing_tok(dx, T) || !dw_gate ||
        !dw_up || !dw_down || !dw_router || !workspace)
      return MOE_ERR_NULL;
    if (ring_head < 0 || ring_head >= s->capacity) return MOE_ERR_SHAPE;
    if (workspace_bytes < moe_workspace_bytes(s, MOE_OP_BACKWARD)) return MOE_ERR_WORKSPACE;
    if (s->tokens == 0) {   // no tokens: every weight gradient is zero (dx is empty)
      const size_t wbytes = (size_t)s->experts * s->ffn * s->hidden * 2;   // bf16, even count
      hipError_t err = zero_words(dw_gate, wbytes / 4, stream);
      if (err == hipSuccess) err = zero_words(dw_up, wbytes / 4, stream);
      if (err == hipSuccess) err = zero_words(dw_down, wbytes / 4, stream);
      if (err == hipSuccess) err = zero_words(dw_router, (size_t)s->experts * s->hidden, stream);
      return hip_status(err);
    }
    return hip_status(moe::launch_backward(
        dy, x, w_router, topk_idx, topk_gate, ring_x, expert_offset, copy_slot, slot_copy,
        ring_head, s->capacity, saved_au, w_gate, w_up, w_down, s->tokens, s->hidden, s->experts,
        s->top_k, s->ffn, dx, dw_gate, dw_up, dw_down, dw_router, workspace, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_backward_mx(const moe_shape* s, const void* dy, const void* x, const float* w_router,
                    const int32_t* topk_idx, const float* topk_gate,
                    const int32_t* expert_offset, const int32_t* copy_slot,
                    const int32_t* slot_copy, int64_t ring_head, const void* saved_au,
                    const uint8_t* w_gu_t, const uint8_t* w_gu_t_scale, const uint8_t* w_down_t,
                    const uint8_t* w_down_t_scale, void* dx, void* dw_gate, void* dw_up,
                    void* dw_down, float* dw_router, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  try {
    int st = check_shape(s);
    if (st) return st;
    if (s->dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
    // f: the SwiGLU backward keeps 3 f words of column maxima in a workgroup's 160 KB of LDS
    if (s->hidden % 128 || s->ffn % 128 || s->ffn > 13568) return MOE_ERR_SHAPE;
    const int64_t T = s->tokens;
    if (missing_tok(dy, T) || missing_tok(x, T) || !w_router || missing_tok(topk_idx, T) ||
        missing_tok(topk_gate, T) || !expert_offset || missing_tok(copy_slot, T) || !slot_copy ||
        !saved_au || !w_gu_t || !w_gu_t_scale || !w_down_t || !w_down_t_scale ||
        missing_tok(dx, T) || !dw_gate || !dw_up || !dw_down || !dw_router || !workspace)
      return MOE_ERR_NULL;
    if (ring_head < 0 || ring_head >= s->capacity) return MOE_ERR_SHAPE;
    if (workspace_bytes < moe_workspace_bytes(s, MOE_OP_BACKWARD)) return MOE_ERR_WORKSPACE;
    if (T == 0) {
      const size_t wbytes = (size_t)s->experts * s->ffn * s->hidden * 2;
      hipError_t err = zero_words(dw_gate, wbytes / 4, stream);
      if (err == hipSuccess) err = zero_words(dw_up, wbytes / 4, stream);
      if (err == hipSuccess) err = zero_words(dw_down, wbytes / 4, stream);
      if (err == hipSuccess) err = zero_words(dw_router, (size_t)s->experts * s->hidden, stream);
      return hip_status(err);
    }
    return hip_status(moe::launch_backward_mx(
        dy, x, w_router, topk_idx, topk_gate, expert_offset, copy_slot, slot_copy, ring_head,
        s->capacity, saved_au, w_gu_t, w_gu_t_scale, w_down_t, w_down_t_scale, T, s->hidden,
        s->experts, s->top_k, s->ffn, dx, dw_gate, dw_up, dw_down, dw_router, workspace, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_quantize_mx_t(const void* src_bf16, int64_t batch, int64_t rows, int64_t cols,
                      uint8_t* codes, int64_t ld, int64_t col0, uint8_t* scales,
                      hipStream_t stream) {
  try {
    if (!src_bf16 || !codes || !scales) return MOE_ERR_NULL;
    if (batch < 0 || rows <= 0 || cols <= 0 || rows % 32 || ld % 128 || col0 < 0 || col0 % 32 ||
        col0 + rows > ld)
      return MOE_ERR_SHAPE;
    return hip_status(moe::launch_quantize_mx_t(src_bf16, batch, rows, cols, codes, ld, col0,
                                                scales, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_quantize_mx_both(const void* src_bf16, int64_t batch, int64_t rows, int64_t cols,
                         uint8_t* codes, uint8_t* scales, uint8_t* codes_t, int64_t ld,
                         int64_t col0, uint8_t* scales_t, hipStream_t stream) {
  try {
    if (!src_bf16 || !codes || !scales || !codes_t || !scales_t) return MOE_ERR_NULL;
    if (batch < 0 || rows <= 0 || cols <= 0 || rows % 128 || cols % 128 || ld % 128 || col0 < 0 ||
        col0 % 128 || col0 + rows > ld)
      return MOE_ERR_SHAPE;
    return hip_status(moe::launch_quantize_mx_both(src_bf16, batch, rows, cols, codes, scales,
                                                   codes_t, ld, col0, scales_t, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

int moe_quantize_mx(const void* src_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                    uint8_t* scales, hipStream_t stream) {
  try {
    if (!src_bf16 || !codes || !scales) return MOE_ERR_NULL;
    if (rows < 0 || cols <= 0 || cols % 128) return MOE_ERR_SHAPE;   // scale groups of 128 columns
    return hip_status(moe::launch_quantize_mx(src_bf16, rows, cols, codes, scales, stream));
  } catch (...) {
    return MOE_ERR_HIP;
  }
}

}  // extern "C"
