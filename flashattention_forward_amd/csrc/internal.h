// Host-side launchers of the gfx950 kernels, called by the C ABI in api.cpp
// after it has validated every argument, and the host-side sizing rules
// (workspace sizes, split counts) in plan.cpp.  Host-only declarations: the
// validation layer builds against this header without any device code.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "seq_shape.h"

namespace attn {

// Largest byte span one buffer resource may cover.  The kernels address a
// head of Q, K, V or O (and the backward's per-row statistics) through
// buffer resources with 32-bit offsets, and form offsets up to one tile
// (16 KiB; 64 KiB allowed here) past the end of a span when they prefetch a
// tile that is then never used.  Spans of at most 2^31 - 2^16 bytes keep
// every such offset below 2^31, so no offset wraps around and its signed
// and unsigned readings agree.  The C ABI rejects larger heads
// (ATTN_E_INVALID); the decode path takes its vector-ALU kernel, which
// addresses memory through 64-bit pointers, for longer key ranges.
constexpr long long kMaxSpanBytes = (1LL << 31) - (1LL << 16);
inline bool span_ok(long long bytes) { return bytes >= 0 && bytes <= kMaxSpanBytes; }

// Partial maxima of the two-pass per-tensor reduction over n elements.
int e4m3_partials(long n);

// Tiled prefill forward, bf16/fp16, d in {64, 128}, over nseq sequences of
// at most max_nq queries each (see SeqShape for the layouts).
hipError_t launch_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                          const SeqShape& sh, int nseq, int max_nq, int d, float scale, bool causal, bool bf16,
                          hipStream_t stream);

// Split-KV decode (Nq == 1): partial kernel + merge kernel; query head h
// reads K/V head h / (H / Hkv).
size_t decode_workspace_bytes(int B, int H, int d, int splits);
int decode_heads_per_workgroup(int H, int Hkv);  // query heads one decode workgroup serves
int decode_default_splits(int B, int H, int Hkv, int Nk, int d);
hipError_t launch_decode(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int H, int Hkv, int Nk, int d, float scale, bool bf16, int splits,
                         void* workspace, hipStream_t stream);
// The same decode with its split partials in the library's static device
// scratch (no workspace argument, no allocation); needs
// decode_workspace_bytes(B, H, d, splits) <= kDecodeStaticScratchBytes.
constexpr size_t kDecodeStaticScratchBytes = (size_t)8 << 20;
hipError_t launch_decode_static(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int H, int Nk, int d, float scale, bool bf16, int splits,
                                hipStream_t stream);

// Backward pass: preprocess (log-sum-exp in base 2, rowsum(dO * O)) into a
// float2 workspace with one entry per query row (q_rows of them: B*H*Nq dense,
// H*total_q packed), then the dK/dV and dQ kernels, over nseq sequences of at
// most max_nq queries and max_nk keys (see SeqShape for the layouts).
size_t bwd_workspace_bytes(long q_rows);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, const SeqShape& sh, int nseq, int max_nq, int max_nk, long q_rows,
                      int d, float scale, bool causal, bool bf16, void* workspace, hipStream_t stream);

// Quantisation kernels and the quantised forward.
hipError_t launch_quantize_rows_i8(const void* x, int8_t* x8, float* scales, long rows, int d,
                                   hipStream_t stream);
size_t quantize_e4m3_workspace_bytes(long n);
hipError_t launch_quantize_tensor_e4m3(const void* x, uint8_t* x8, float* scale_out, long n,
                                       void* workspace, hipStream_t stream);
// The quantised forwards share one kernel: kInt8Scores has int8 Q8/K8 and
// E4M3 V8 and P (int8 scores, fp8 P . V); kAllInt8 has int8 V8 and P
// (both products on the int8 MFMA); kFp8 has E4M3 Q8/K8, V8 and P (both
// products on the fp8 MFMA); kFp8P4 is kFp8 with P in MXFP4 (E2M1 codes,
// one power-of-two scale per 32 keys of a query; P . V on the mixed
// fp8 x fp4 MFMA).
enum class QVariant : int { kInt8Scores = 0, kAllInt8 = 1, kFp8 = 2, kFp8P4 = 3 };
hipError_t launch_prefill_q8(const void* q8, const void* k8, const void* v8,
                             const float* q_scale, const float* k_scale, const float* v_scale,
                             void* out, float* lse, int B, int H, int Nq, int Nk, int d,
                             float scale, bool causal, QVariant variant, hipStream_t stream);
// Block E4M3 quantisation of x [BH, N, d] bf16, optionally after the
// random-sign Hadamard rotation (signs != nullptr): per-row scales [BH, N].
hipError_t launch_rotate_quantize_e4m3(const void* x, const float* signs, uint8_t* x8, float* scales, int BH,
                                       int N, int d, int block_rows, hipStream_t stream);
hipError_t launch_quantize_tensor_i8(const void* x, int8_t* x8, float* scale_out, long n, void* workspace,
                                     hipStream_t stream);
// s: int32 scores of int8 codes, or fp32 scores of E4M3 codes (fp8)
hipError_t launch_debug_qk(const void* q8, const void* k8, void* s, int Nq, int Nk, int d, bool fp8,
                           hipStream_t stream);
hipError_t launch_debug_cvt_e4m3(const float* x, uint8_t* y, long n, hipStream_t stream);
hipError_t launch_debug_cvt_e2m1(const float* x, uint8_t* y, long n, hipStream_t stream);
// the d = 128 prefill with poly_per_8 (2 or 4) of every 8 softmax exponentials
// on the FMA-pipe polynomial; its evaluation hook
hipError_t launch_prefill_exp2_split(const void* q, const void* k, const void* v, void* out, float* lse,
                                     const SeqShape& sh, int nseq, int max_nq, int d, float scale, bool causal, bool bf16,
                                     int poly_per_8, hipStream_t stream);
hipError_t launch_debug_exp2_poly(const float* x, float* y, long n, hipStream_t stream);

}  // namespace attn
