/*
 * moe.h: C ABI of a single Mixture-of-Experts layer on one MI355X (gfx950) GPU.
 *
 * The layer computes y = sum_k g_k E_k(x): an fp32 router picks k experts per
 * token and renormalised gates g; token copies are dispatched into an
 * expert-contiguous ring buffer; every expert applies a SwiGLU FFN
 * E(x) = W_down (silu(W_gate x) * (W_up x)); the results are combined with the
 * gates in a fixed order.  Sources of each step:
 *
 *   routing of tokens to experts ........ dzen.guru page, section "Что именно тормозило
 *                                          обучение MoE-моделей?"
 *   fixed ring buffer, no dropped tokens,
 *   reverse traversal in the backward ... dzen.guru page, ring-buffer paragraph of
 *                                          "Три решения, которые дали результат"
 *   one deterministic result; BF16 and
 *   MXFP8 ................................ dzen.guru page, megakernel paragraph of the same
 *                                          section; @cursor_ai tweet on the khabar-ai page
 *   no CPU in the loop .................. @rohanpaul_ai tweet on the khabar-ai page
 *   output-parallel two-kernel decode ... toolnavs.com warp-decode page, sections "Cursor a
 *                                          réécrit le décodage de MoE" and "1.84x plus de
 *                                          vitesse…"
 * The pages give no formulas; the router (softmax over all experts, top-k,
 * renormalise), the SwiGLU expert and the MXFP8 encoding (E4M3 elements, one
 * E8M0 scale per 32 elements along the reduction dimension, RNE) are those of
 * the layer's workload definition.
 *
 * Conventions for every call
 *   - Every tensor pointer is a DEVICE pointer; `shape` is a HOST pointer.
 *   - Row-major, nn.Linear layout: W_gate, W_up [E, f, d]; W_down [E, d, f];
 *     W_r [E, d] fp32; b_r [E] fp32 (may be NULL).
 *   - "act" tensors are fp32 when shape->dtype == MOE_F32, otherwise bf16
 *     (raw 16-bit patterns).  With MOE_MXFP8 the router and the tokens x stay
 *     bf16; ring_x, H and the expert weights are E4M3 codes (uint8) with one
 *     E8M0 scale byte per 32 elements along the reduction dimension.  Every MX
 *     scale tensor of a matrix [rows, cols] is laid out [cols/128][rows][4]: for each
 *     group of 128 columns one 32-bit word per row holding that row's 4 block scales
 *     in column order (cols % 128 == 0), so that the scales a GEMM stage needs for
 *     consecutive rows are consecutive words.
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     pointer after return, and only enqueues work on `stream`: there is no
 *     host synchronisation and no device-to-host copy inside any call.
 *   - Outputs are fully overwritten; read-only inputs are never written.  With
 *     tokens = 0 the per-expert outputs are zeros (expert_count, expert_offset,
 *     every weight gradient) and per-token outputs are empty; per-token arrays
 *     (x, dy, y, dx, topk_idx, topk_gate, copy_slot) may then be NULL.
 *   - Results are bitwise reproducible run to run (fixed reduction orders,
 *     no floating-point atomics).
 *   - Errors: arguments are validated on the host from `shape` before any
 *     launch.  A launch failure returns MOE_ERR_HIP.  No exception crosses
 *     the ABI.  Calls that share a workspace must not overlap in time.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,       /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,      /* non-positive size, k > E, a length outside the kernels'
                             domain (see each call), a ring array of 4 GiB or more, ... */
  MOE_ERR_CAPACITY = 3,   /* ring capacity below tokens * top_k: tokens would be dropped */
  MOE_ERR_WORKSPACE = 4,  /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 5,        /* a HIP launch or runtime call failed */
  MOE_ERR_DTYPE = 6,      /* unknown dtype, or a dtype the call does not support */
  MOE_ERR_SCRATCH = 7     /* shape needs more than the static scratch of moe_decode_noalloc */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2 };

enum moe_op {
  MOE_OP_ROUTE = 0, MOE_OP_DISPATCH = 1, MOE_OP_EXPERT_FFN = 2,
  MOE_OP_COMBINE = 3, MOE_OP_DECODE = 4, MOE_OP_BACKWARD = 5, MOE_OP_FORWARD = 6
};

/* Shape of one layer call (host struct). */
typedef struct moe_shape {
  int64_t tokens;      /* T: tokens of this call (decode: batch B) */
  int64_t capacity;    /* C: ring rows; must be >= tokens * top_k */
  int32_t hidden;      /* d */
  int32_t experts;     /* E */
  int32_t top_k;       /* k, 1 <= k <= E */
  int32_t ffn;         /* f: expert intermediate size */
  int32_t shared_ffn;  /* fs: always-on shared expert width (decode only), 0 = none */
  int32_t dtype;       /* enum moe_dtype */
} moe_shape;

/*
 * moe_route: the router (dzen.guru, "Что именно тормозило…": each layer routes
 * tokens to experts).  In fp32, with x widened exactly from bf16:
 *   l[t,e] = sum_i x[t,i] W_r[e,i] (+ b_r[e]);  p = softmax_e(l);
 *   S_t = the k largest l (ties to the lower id);  g[t,j] = p[S_tj] / sum_S p.
 * In:  x [T,d] act (bf16 for MOE_MXFP8), w_router [E,d] f32, b_router [E] f32 or NULL.
 * Out: topk_idx [T,k] int32, ascending expert id per token; topk_gate [T,k] f32;
 *      expert_count [E] int32 = copies routed to each expert.
 * workspace: moe_workspace_bytes(shape, MOE_OP_ROUTE) bytes (router logits).
 */
int moe_route(const moe_shape* shape, const void* x, const float* w_router,
              const float* b_router, int32_t* topk_idx, float* topk_gate,
              int32_t* expert_count, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/*
 * moe_dispatch: deterministic counting sort of the T*k token copies into the
 * fixed ring buffer (dzen.guru, ring-buffer paragraph: fixed size, nothing
 * dropped, no size computed on the CPU).  Copy c = t*k + j goes to
 *   slot = (ring_head + rank(c)) mod C,
 * where rank orders copies by (expert, token): segments are expert-contiguous
 * and hold their tokens in ascending order.
 * In:  x [T,d] act (bf16 for MOE_MXFP8), topk_idx [T,k], ring_head in [0, C).
 * Out: ring_x [C,d] act (MOE_MXFP8: E4M3 codes, each row MX-quantised along d)
 *        — only the T*k used slots are written;
 *      ring_x_scale [d/128][C][4] E8M0 bytes (MOE_MXFP8 only, else NULL);
 *      expert_offset [E+1] int32, segment starts relative to the head (offset[E] = T*k);
 *      copy_slot [T,k] int32 absolute slot of each copy;
 *      slot_copy [C] int32 copy id t*k+j held by each used slot (other slots untouched).
 * workspace: moe_workspace_bytes(shape, MOE_OP_DISPATCH) bytes.
 */
int moe_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                 int64_t ring_head, void* ring_x, uint8_t* ring_x_scale,
                 int32_t* expert_offset, int32_t* copy_slot, int32_t* slot_copy,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expert_ffn: every expert's SwiGLU FFN over its own ring segment, as two
 * grouped GEMMs (the expert-centric scheme the warp-decode page contrasts with;
 * MXFP8 expert kernels per the @rohanpaul_ai tweet on the khabar-ai page):
 *   [A|U] = X_e [W_gate[e]; W_up[e]]^T,  H = silu(A) * U,  Y_e = H W_down[e]^T.
 * H is bf16 (fp32 for MOE_F32; MX along f for MOE_MXFP8) and lives in the workspace.
 * In:  ring_x (+ ring_x_scale), expert_offset, ring_head; w_gate, w_up [E,f,d] and
 *      w_down [E,d,f] act, or E4M3 codes with w_gate_scale/w_up_scale [d/128][E*f][4]
 *      and w_down_scale [f/128][E*d][4] for MOE_MXFP8 (NULL otherwise), as
 *      moe_quantize_mx writes them for the [E*f, d] and [E*d, f] matrices.
 * Out: ring_y [C,d] (bf16; fp32 for MOE_F32) at the segment slots;
 *      saved_au [C,2f] bf16 (A then U per slot) when not NULL — the backward's input
 *      (MOE_BF16 and MOE_MXFP8: the gate/up fp32 accumulations rounded to bf16; NULL for
 *      MOE_F32).
 * workspace: moe_workspace_bytes(shape, MOE_OP_EXPERT_FFN) bytes.
 */
int moe_expert_ffn(const moe_shape* shape, const void* ring_x, const uint8_t* ring_x_scale,
                   const int32_t* expert_offset, int64_t ring_head,
                   const void* w_gate, const void* w_up, const void* w_down,
                   const uint8_t* w_gate_scale, const uint8_t* w_up_scale,
                   const uint8_t* w_down_scale, void* ring_y, void* saved_au,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_timed: moe_expert_ffn for measurement.  When `events` is not
 * NULL, events[0] is recorded on `stream` before GEMM-1, events[1] between GEMM-1
 * and GEMM-2, events[2] after GEMM-2 (caller-created hipEvent_t handles).  No
 * host synchronisation; results identical to moe_expert_ffn.
 */
int moe_expert_ffn_timed(const moe_shape* shape, const void* ring_x, const uint8_t* ring_x_scale,
                         const int32_t* expert_offset, int64_t ring_head,
                         const void* w_gate, const void* w_up, const void* w_down,
                         const uint8_t* w_gate_scale, const uint8_t* w_up_scale,
                         const uint8_t* w_down_scale, void* ring_y, void* saved_au,
                         void* workspace, size_t workspace_bytes, hipEvent_t* events,
                         hipStream_t stream);

/*
 * moe_combine: y[t] = sum_j g[t,j] ring_y[copy_slot[t,j]], j in ascending expert
 * order, fp32 accumulation, one final rounding (deterministic gather; dzen.guru,
 * megakernel paragraph).
 * In: ring_y [C,d], copy_slot [T,k], topk_gate [T,k].  Out: y [T,d] (bf16; f32 for MOE_F32).
 */
int moe_combine(const moe_shape* shape, const void* ring_y, const int32_t* copy_slot,
                const float* topk_gate, void* y, hipStream_t stream);

/*
 * moe_forward: the whole forward (moe_route, moe_dispatch, moe_expert_ffn, moe_combine)
 * in ONE kernel launch, persistent and deterministic (dzen.guru page, megakernel
 * paragraph of "Три решения…": one GPU call moves and computes, with one deterministic
 * result; @cursor_ai tweet on the khabar-ai page: a single, fully deterministic kernel).
 * Same arguments and outputs as the four calls chained (the router's workspace, the
 * dispatch's and the FFN's live inside this call's workspace); every output is bitwise
 * the chained calls' where those run the 128-row GEMM tile (fewer than 256 copies per
 * expert on average), and equal up to fp32 rounding order otherwise.
 * In:  x [T,d] bf16, w_router [E,d] f32, b_router [E] f32 or NULL, w_gate/w_up [E,f,d] and
 *      w_down [E,d,f] bf16, ring_head in [0, C).
 * Out: topk_idx, topk_gate, expert_count (as moe_route); ring_x, expert_offset, copy_slot,
 *      slot_copy (as moe_dispatch); ring_y [C,d] bf16 and saved_au [C,2f] bf16 or NULL
 *      (as moe_expert_ffn); y [T,d] bf16 (as moe_combine).
 * The kernel is launched cooperatively, one workgroup per CU (a multiple of 8), and its
 * phases meet at grid barriers kept in the first 256 bytes of the workspace: those bytes
 * must be zero before the first call on a workspace and are kept consistent by every
 * call (the rest of the workspace needs no initial contents).  A barrier wait gives up
 * after spin_limit polls (0: 4,194,304, far beyond any normal wait) and then sets bit 0
 * of the 32-bit status word at byte offset 8 of the workspace; the results of that call
 * are then undefined, the bit stays set until the caller clears it, and the first 256
 * bytes must be zeroed before the next call.  Calls sharing a workspace must not overlap.
 * workspace: moe_workspace_bytes(shape, MOE_OP_FORWARD) bytes.  MOE_BF16 only.
 */
int moe_forward(const moe_shape* shape, const void* x, const float* w_router,
                const float* b_router, const void* w_gate, const void* w_up, const void* w_down,
                int64_t ring_head, int32_t* topk_idx, float* topk_gate, int32_t* expert_count,
                void* ring_x, int32_t* expert_offset, int32_t* copy_slot, int32_t* slot_copy,
                void* ring_y, void* saved_au, void* y, uint32_t spin_limit, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * moe_decode: small-batch decode parallelised over outputs, in two kernels and
 * with no permuted buffer (toolnavs.com warp-decode page, "1.84x plus de vitesse…"),
 * after a router kernel that writes the fp32 logits.  Kernel 1: the routing (rebuilt
 * in every workgroup), then each wavefront streams rows of W_gate/W_up of the shared
 * expert and of the experts the batch selected and
 * writes h = silu(a) * u in fp32, token-major.  Kernel 2: each wavefront owns a
 * group of output rows, streams W_down rows of every selected expert and of the
 * shared expert, and writes y = sum_j g_j (W_down h_j) + W_s_down h_s in bf16.
 * In:  x [B,d] bf16 (B = shape->tokens, 1..8; top_k <= 16), w_router, b_router (or NULL),
 *      w_gate/w_up/w_down bf16, shared ws_gate/ws_up [fs,d], ws_down [d,fs] bf16
 *      or NULL when shape->shared_ffn == 0.
 * Out: y [B,d] bf16, topk_idx [B,k], topk_gate [B,k].
 * workspace: moe_workspace_bytes(shape, MOE_OP_DECODE) bytes (no initial contents needed).
 * MOE_BF16 only; d a multiple of 512 up to 8192, f a multiple of 512 up to 4096,
 * shared_ffn 0 or equal to f (MOE_ERR_SHAPE otherwise).
 */
int moe_decode(const moe_shape* shape, const void* x, const float* w_router,
               const float* b_router, const void* w_gate, const void* w_up,
               const void* w_down, const void* ws_gate, const void* ws_up,
               const void* ws_down, void* y, int32_t* topk_idx, float* topk_gate,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_decode_noalloc: moe_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, bitwise, but the workspace is the library's own static
 * device array of 1 MiB (one per GPU, held until the process ends), so the caller passes
 * inputs and outputs only.  Shapes whose decode workspace
 * (moe_workspace_bytes(shape, MOE_OP_DECODE)) exceeds 1 MiB return MOE_ERR_SCRATCH
 * before any launch: B = 8, k = 8, f = fs = 2048, E = 256 needs 0.6 MiB, while
 * B = 8, k = 16, f = 4096 (2.3 MiB) is rejected.
 * No allocation of any kind happens inside the call.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (two streams, or two threads) race
 * and must not be issued.  The array needs no initial contents (every word a call reads
 * it first writes in the same call).
 */
int moe_decode_noalloc(const moe_shape* shape, const void* x, const float* w_router,
                       const float* b_router, const void* w_gate, const void* w_up,
                       const void* w_down, const void* ws_gate, const void* ws_up,
                       const void* ws_down, void* y, int32_t* topk_idx, float* topk_gate,
                       hipStream_t stream);

/*
 * moe_backward: gradients of L = sum_t <dy_t, y_t> with the routing S held
 * fixed; the ring is traversed in reverse (dzen.guru, ring-buffer paragraph):
 * experts E-1 -> 0, and every weight gradient sums its segment's rows from the
 * last slot to the first.  Per copy (t,j) of expert e with gate g:
 *   dh = W_down[e]^T dy_t,  dg = <dh, h>,  da = g dh u s (1 + a (1 - s)),
 *   du = g dh a s  (s = sigmoid(a)),   dx_t += W_gate[e]^T da + W_up[e]^T du,
 *   dW_down[e] += g dy_t h^T,  dW_gate[e] += da x_t^T,  dW_up[e] += du x_t^T;
 *   router: dl_j = g_j (dg_j - sum_i g_i dg_i),  dW_r[e_j] += dl_j x_t,  dx_t += dl_j W_r[e_j].
 * In:  dy [T,d] bf16; x [T,d] bf16; w_router [E,d]; topk_idx, topk_gate; ring_x,
 *      expert_offset, copy_slot, slot_copy, ring_head from moe_dispatch; saved_au from
 *      moe_expert_ffn; w_gate, w_up, w_down bf16.
 * Out: dx [T,d] bf16; dw_gate, dw_up [E,f,d] bf16; dw_down [E,d,f] bf16 (zero for
 *      experts with no rows); dw_router [E,d] f32.
 * workspace: moe_workspace_bytes(shape, MOE_OP_BACKWARD) bytes.  MOE_BF16 only (the MXFP8
 * layer's backward is moe_backward_mx); d and f must be multiples of 128 (MOE_ERR_SHAPE
 * otherwise).
 */
int moe_backward(const moe_shape* shape, const void* dy, const void* x,
                 const float* w_router, const int32_t* topk_idx, const float* topk_gate,
                 const void* ring_x, const int32_t* expert_offset, const int32_t* copy_slot,
                 const int32_t* slot_copy, int64_t ring_head, const void* saved_au,
                 const void* w_gate, const void* w_up, const void* w_down,
                 void* dx, void* dw_gate, void* dw_up, void* dw_down, float* dw_router,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Validation of `shape` alone, as every call performs it first (MOE_OK or the status
 * a call would return; includes: every ring array the MFMA GEMMs address, C * d and
 * C * f elements of bf16 or E4M3, must stay below 4 GiB).  Host only, no GPU call. */
int moe_check_shape(const moe_shape* shape);

/*
 * moe_backward_mx: the MXFP8 layer's backward (the MXFP8 backward of the dzen.guru page,
 * "Что показали замеры?").  The gradients of moe_backward, with every backward GEMM's two
 * operands MX-quantised (E4M3, one E8M0 scale per 32) along that GEMM's reduction
 * dimension and fp32 accumulation; the forward's quantisation counts as the identity:
 *   dh = Q_d(W_down)^T Q_d(dy_t)        (W_down quantised along d, i.e. transposed)
 *   dx_t += Q_f(W_gate)^T Q_f(da) + Q_f(W_up)^T Q_f(du)   (weights along f)
 *   dW_down[e] = Q_t(dY_e)^T Q_t(g H_e),  dW_gate[e] = Q_t(dA_e)^T Q_t(X_e),
 *   dW_up[e] = Q_t(dU_e)^T Q_t(X_e)
 * Q_t: along the token axis, each expert's copies in ring-segment order in blocks of 32
 * aligned to the segment's last slot (the first block partial).  dg, da, du, the router
 * gradient and dx's router term as in moe_backward; saved_au from the MXFP8 forward's
 * moe_expert_ffn.
 * In:  dy, x [T,d] bf16; w_router; topk_idx, topk_gate; expert_offset, copy_slot,
 *      slot_copy, ring_head from moe_dispatch; saved_au [C,2f] bf16;
 *      w_gu_t [E,d,2f] E4M3 = [W_gate^T | W_up^T] of every expert quantised along f, scales
 *      w_gu_t_scale [2f/128][E*d][4]; w_down_t [E,f,d] = W_down^T quantised along d,
 *      scales w_down_t_scale [d/128][E*f][4] (both as moe_quantize_mx_t writes them).
 * Out: dx [T,d] bf16; dw_gate, dw_up [E,f,d] and dw_down [E,d,f] bf16; dw_router [E,d] f32.
 * workspace: moe_workspace_bytes(shape with dtype MOE_MXFP8, MOE_OP_BACKWARD) bytes.
 * MOE_MXFP8 only; d and f multiples of 128, f at most 13568 (the SwiGLU backward keeps
 * three f-wide rows of column maxima in LDS); MOE_ERR_SHAPE otherwise.
 */
int moe_backward_mx(const moe_shape* shape, const void* dy, const void* x,
                    const float* w_router, const int32_t* topk_idx, const float* topk_gate,
                    const int32_t* expert_offset, const int32_t* copy_slot,
                    const int32_t* slot_copy, int64_t ring_head, const void* saved_au,
                    const uint8_t* w_gu_t, const uint8_t* w_gu_t_scale, const uint8_t* w_down_t,
                    const uint8_t* w_down_t_scale, void* dx, void* dw_gate, void* dw_up,
                    void* dw_down, float* dw_router, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Bytes of workspace `op` needs for `shape` (0 if none).  Host only, no GPU call. */
size_t moe_workspace_bytes(const moe_shape* shape, int op);

/* Static description of a status code. */
const char* moe_status_string(int status);

/*
 * moe_quantize_mx: MX-quantise a bf16 matrix [rows, cols] along cols (cols % 128 == 0):
 * per block of 32, X = floor(log2 amax) - 8 clamped to [-127, 127] (-127 for a zero
 * block), code = RNE_E4M3(clamp(v / 2^X, +-448)), scale = X + 127.
 * Out: codes [rows, cols] uint8, scales [cols/128][rows][4] uint8 (the MX scale
 * layout above).  Used for the weights.
 */
int moe_quantize_mx(const void* src_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                    uint8_t* scales, hipStream_t stream);

/*
 * moe_quantize_mx_t: MX-quantise `batch` bf16 matrices [rows, cols] (src [batch, rows, cols])
 * along their rows and write them transposed: source column c of matrix b becomes row
 * b*cols + c of a code matrix with rows of ld bytes, its values in columns col0 .. col0 +
 * rows - 1; scales in that code matrix's layout [ld/128][batch*cols][4].  The MXFP8
 * backward's weights: W_down [E,d,f] -> (E, d, f, ld = d, col0 = 0); W_gate and W_up [E,f,d]
 * -> (E, f, d, ld = 2f, col0 = 0 and f).  rows % 32 == 0, ld % 128 == 0, col0 % 32 == 0.
 */
int moe_quantize_mx_t(const void* src_bf16, int64_t batch, int64_t rows, int64_t cols,
                      uint8_t* codes, int64_t ld, int64_t col0, uint8_t* scales,
                      hipStream_t stream);

/*
 * moe_quantize_mx_both: both MX layouts of `batch` bf16 matrices in one pass, for an MXFP8
 * training step that re-quantises its weights for the forward and for moe_backward_mx.
 * Writes exactly what moe_quantize_mx(src, batch*rows, cols, codes, scales) and
 * moe_quantize_mx_t(src, batch, rows, cols, codes_t, ld, col0, scales_t) write, bit for
 * bit, reading each bf16 value once.  rows, cols, ld and col0 multiples of 128, col0 +
 * rows <= ld (MOE_ERR_SHAPE otherwise); NULL pointers: MOE_ERR_NULL.  Both code matrices
 * and scale arrays are the caller's, as for the two calls it replaces.
 */
int moe_quantize_mx_both(const void* src_bf16, int64_t batch, int64_t rows, int64_t cols,
                         uint8_t* codes, uint8_t* scales, uint8_t* codes_t, int64_t ld,
                         int64_t col0, uint8_t* scales_t, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
