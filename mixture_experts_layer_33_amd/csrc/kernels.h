// Host-side launchers of the gfx950 kernels (called by api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// router
size_t route_workspace_bytes(int64_t T, int E, int d);
hipError_t launch_route(const void* x, bool x_f32, const float* w_r, const float* b_r, int64_t T,
                        int d, int E, int k, float* logits, int32_t* topk_idx, float* topk_gate,
                        int32_t* expert_count, hipStream_t st);

// dispatch (elem_bytes: 4 f32, 2 bf16; mx: quantise bf16 rows to E4M3 + E8M0)
size_t dispatch_workspace_bytes(int64_t T, int E);
hipError_t launch_dispatch(const void* x, int elem_bytes, bool mx, const int32_t* topk_idx,
                           int64_t T, int d, int E, int k, int64_t head, int64_t C, void* ring_x,
                           uint8_t* ring_scale, int32_t* expert_offset, int32_t* copy_slot,
                           int32_t* slot_copy, void* ws, hipStream_t st);

// expert FFN (grouped GEMMs)
// tiles[2i] = expert, tiles[2i+1] = first segment row of row-tile i (height BM); *ntiles = count
hipError_t launch_build_tiles(const int32_t* expert_offset, int E, int BM, int32_t* tiles,
                              int32_t* ntiles, hipStream_t st);
size_t ffn_workspace_bytes(int64_t n, int64_t C, int d, int E, int f, int dtype);
hipError_t launch_ffn(int dtype, const void* ring_x, const uint8_t* ring_x_scale,
                      const int32_t* expert_offset, int64_t head, int64_t C, int64_t n, int d,
                      int E, int f, const void* w_gate, const void* w_up, const void* w_down,
                      const uint8_t* wg_scale, const uint8_t* wu_scale, const uint8_t* wd_scale,
                      void* ring_y, void* saved_au, void* ws, hipEvent_t* events,
                      hipStream_t st);

// combine
hipError_t launch_combine(bool f32, const void* ring_y, const int32_t* copy_slot,
                          const float* gate, int64_t T, int d, int k, void* y, hipStream_t st);

// decode
size_t decode_workspace_bytes(int B, int E, int k, int f, int fs);
hipError_t launch_decode(const void* x, const float* w_r, const float* b_r, const void* w_gate,
                         const void* w_up, const void* w_down, const void* ws_gate,
                         const void* ws_up, const void* ws_down, int B, int d, int E, int k,
                         int f, int fs, void* y, int32_t* topk_idx, float* topk_gate, void* ws,
                         hipStream_t st);

// the whole forward in one cooperative launch (bf16)
size_t fused_workspace_bytes(int64_t T, int64_t C, int d, int E, int f);
hipError_t launch_forward_fused(const void* x, const float* w_r, const float* b_r,
                                const void* w_gate, const void* w_up, const void* w_down,
                                int64_t T, int d, int E, int k, int f, int64_t C, int64_t head,
                                int32_t* topk_idx, float* topk_gate, int32_t* expert_count,
                                void* ring_x, int32_t* expert_offset, int32_t* copy_slot,
                                int32_t* slot_copy, void* ring_y, void* saved_au, void* y,
                                uint32_t spin_limit, void* ws, hipStream_t st);

// decode without a caller workspace: the device address of the library's static scratch
// array on the current device (DECODE_SCRATCH_BYTES), looked up once per device
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)1 << 20;   // 1 MiB
hipError_t decode_scratch(void** ptr);

// backward
size_t backward_workspace_bytes(int64_t T, int64_t C, int d, int E, int k, int f);
hipError_t launch_backward(const void* dy, const void* x, const float* w_r,
                           const int32_t* topk_idx, const float* topk_gate, const void* ring_x,
                           const int32_t* expert_offset, const int32_t* copy_slot,
                           const int32_t* slot_copy, int64_t head, int64_t C, const void* saved_au,
                           const void* w_gate, const void* w_up, const void* w_down, int64_t T,
                           int d, int E, int k, int f, void* dx, void* dw_gate, void* dw_up,
                           void* dw_down, float* dw_r, void* ws, hipStream_t st);

// MX quantisation of a bf16 matrix along its rows
hipError_t launch_quantize_mx(const void* src, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t st);
// ... and of the columns of each of `batch` matrices [R, Cc], written transposed
hipError_t launch_quantize_mx_both(const void* src, int64_t batch, int64_t R, int64_t Cc,
                                   uint8_t* codes, uint8_t* scales, uint8_t* codes_t, int64_t ld,
                                   int64_t col0, uint8_t* scales_t, hipStream_t st);
hipError_t launch_quantize_mx_t(const void* src, int64_t batch, int64_t R, int64_t Cc,
                                uint8_t* codes, int64_t ld, int64_t col0, uint8_t* scales,
                                hipStream_t st);

// a plain MX grouped GEMM with 128-row tiles over a prebuilt tile list (the MXFP8 backward's
// dgrad GEMMs): out[slot] = A[slot] B[e]^T in bf16, or in fp32
struct GemmArgs;
hipError_t launch_mx_plain_gemm128(GemmArgs& g, int64_t n, int E, bool f32_out, hipStream_t st);

// MXFP8 backward
size_t backward_mx_workspace_bytes(int64_t T, int64_t C, int d, int E, int k, int f);
hipError_t launch_backward_mx(const void* dy, const void* x, const float* w_r,
                              const int32_t* topk_idx, const float* topk_gate,
                              const int32_t* expert_offset, const int32_t* copy_slot,
                              const int32_t* slot_copy, int64_t head, int64_t C,
                              const void* saved_au, const uint8_t* w_gu_t,
                              const uint8_t* w_gu_t_scale, const uint8_t* w_down_t,
                              const uint8_t* w_down_t_scale, int64_t T, int d, int E, int k,
                              int f, void* dx, void* dw_gate, void* dw_up, void* dw_down,
                              float* dw_r, void* ws, hipStream_t st);

}  // namespace moe
