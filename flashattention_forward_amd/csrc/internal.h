// Host-side launchers of the gfx950 kernels, called by the C ABI in api.hip
// after it has validated every argument.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Tiled prefill forward (any Nq >= 1), bf16/fp16, d in {64, 128}.
hipError_t launch_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int H, int Nq, int Nk, int d, float scale, bool causal, bool bf16,
                          hipStream_t stream);

// Split-KV decode (Nq == 1): partial kernel + merge kernel.
size_t decode_workspace_bytes(int B, int H, int d, int splits);
int decode_default_splits(int B, int H, int Nk, int d);
hipError_t launch_decode(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int H, int Nk, int d, float scale, bool bf16, int splits,
                         void* workspace, hipStream_t stream);

// Backward pass: preprocess (log-sum-exp in base 2, rowsum(dO * O)) into a
// float2 [B, H, Nq] workspace, then the dK/dV and dQ kernels.
size_t bwd_workspace_bytes(int B, int H, int Nq);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d, float scale, bool causal,
                      bool bf16, void* workspace, hipStream_t stream);

// Quantisation kernels and the quantised forward.
hipError_t launch_quantize_rows_i8(const void* x, int8_t* x8, float* scales, long rows, int d,
                                   hipStream_t stream);
size_t quantize_e4m3_workspace_bytes(long n);
hipError_t launch_quantize_tensor_e4m3(const void* x, uint8_t* x8, float* scale_out, long n,
                                       void* workspace, hipStream_t stream);
hipError_t launch_prefill_q8(const int8_t* q8, const int8_t* k8, const uint8_t* v8,
                             const float* q_scale, const float* k_scale, const float* v_scale,
                             void* out, float* lse, int B, int H, int Nq, int Nk, int d,
                             float scale, bool causal, hipStream_t stream);
hipError_t launch_debug_qk_i32(const int8_t* q8, const int8_t* k8, int32_t* s, int Nq, int Nk, int d,
                               hipStream_t stream);
hipError_t launch_debug_cvt_e4m3(const float* x, uint8_t* y, long n, hipStream_t stream);

}  // namespace attn
