// C ABI of libattn_mi355x.so: argument validation and kernel dispatch.
// Every check runs on the host before anything is launched; a validation
// error means no work was enqueued.  See include/attn_mi355x.h for the
// contract.  Host-only C++: it calls the launchers declared in internal.h
// and nothing else of HIP, so it also builds for the CPU against stub
// launchers (the sanitizer build of the validation layer used by the tests).
#include <cmath>
#include <algorithm>
#include <climits>
#include <cstdint>

#include "attn_mi355x.h"
#include "internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }
int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_E_HIP; }

// the prefill grid has at most ceil(Nq / 128) * B * H workgroups; it must fit an int
bool prefill_grid_ok(int B, int H, int Nq) {
  const long long g = ((long long)Nq + 127) / 128 * (long long)B * (long long)H;
  return g <= INT_MAX;
}

// the bf16/fp16 prefill and the backward address one head of Q, K, V, O
// through buffer resources: each head spans at most kMaxSpanBytes
bool prefill_head_ok(int Nq, int Nk, int d) {
  return attn::span_ok((long long)Nq * d * 2) && attn::span_ok((long long)Nk * d * 2);
}

int check_common(const void* q, const void* k, const void* v, const void* out, const float* lse, int B, int H, int Nq,
                 int Nk, float scale, int causal) {
  if (!q || !k || !v || !out) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_E_INVALID;
  if (lse && !aligned4(lse)) return ATTN_E_INVALID;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_E_INVALID;
  if (!good_scale(scale)) return ATTN_E_INVALID;
  if (causal && Nq > Nk) return ATTN_E_INVALID;
  if (!prefill_grid_ok(B, H, Nq)) return ATTN_E_INVALID;
  return ATTN_OK;
}

bool decode_sizes_ok(int B, int H, int splits) { return (long long)B * H * splits <= INT_MAX; }

int decode_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv, int Nk,
                int d, float scale, int dtype, int num_splits, void* workspace, size_t workspace_bytes,
                void* stream) {
  int rc = check_common(q, k, v, out, lse, B, H, 1, Nk, scale, 0);
  if (rc != ATTN_OK) return rc;
  if (Hkv < 1 || H % Hkv != 0) return ATTN_E_INVALID;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_E_UNSUPPORTED;
  if (num_splits < 1 || num_splits > 256 || num_splits > Nk) return ATTN_E_INVALID;
  if (!decode_sizes_ok(B, H, num_splits)) return ATTN_E_INVALID;
  const size_t need = attn::decode_workspace_bytes(B, H, d, num_splits);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return ATTN_E_WORKSPACE;
  return hip_status(attn::launch_decode(q, k, v, out, lse, B, H, Hkv, Nk, d, scale, dtype == ATTN_BF16, num_splits,
                                        workspace, static_cast<hipStream_t>(stream)));
}

int fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv, int Nq, int Nk,
             int d, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(q, k, v, out, lse, B, H, Nq, Nk, scale, causal);
  if (rc != ATTN_OK) return rc;
  if (Hkv < 1 || H % Hkv != 0) return ATTN_E_INVALID;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_E_UNSUPPORTED;
  if (Nq == 1) {
    const int splits = attn::decode_default_splits(B, H, Hkv, Nk, d);
    return decode_impl(q, k, v, out, lse, B, H, Hkv, Nk, d, scale, dtype, splits, workspace, workspace_bytes, stream);
  }
  if (!prefill_head_ok(Nq, Nk, d)) return ATTN_E_INVALID;
  const attn::SeqShape sh{nullptr, nullptr, H, H / Hkv, Nq, Nk};
  return hip_status(attn::launch_prefill(q, k, v, out, lse, sh, B, Nq, d, scale, causal != 0, dtype == ATTN_BF16,
                                         static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

size_t attn_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 1 || H < 1 || (d != 64 && d != 128) || num_splits < 1 || num_splits > 256) return 0;
  return attn::decode_workspace_bytes(B, H, d, num_splits);
}

int attn_fwd_decode_splits(int B, int H, int Nk, int d) {
  if (B < 1 || H < 1 || Nk < 1) return 0;
  return attn::decode_default_splits(B, H, H, Nk, d);
}

size_t attn_fwd_gqa_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d, int dtype) {
  if (Hkv < 1 || H < 1 || H % Hkv != 0) return 0;
  if (B < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128) || (dtype != ATTN_BF16 && dtype != ATTN_FP16)) return 0;
  if (Nq != 1) return 0;
  return attn::decode_workspace_bytes(B, H, d, attn::decode_default_splits(B, H, Hkv, Nk, d));
}

size_t attn_fwd_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128) || (dtype != ATTN_BF16 && dtype != ATTN_FP16))
    return 0;
  if (Nq != 1) return 0;
  return attn::decode_workspace_bytes(B, H, d, attn::decode_default_splits(B, H, H, Nk, d));
}

int attn_fwd_decode(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nk, int d,
                    float scale, int dtype, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k, v, out, lse, B, H, H, Nk, d, scale, dtype, num_splits, workspace, workspace_bytes, stream);
}

int attn_fwd_decode_static(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nk,
                           int d, float scale, int dtype, int num_splits, void* stream) {
  int rc = check_common(q, k, v, out, lse, B, H, 1, Nk, scale, 0);
  if (rc != ATTN_OK) return rc;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_E_UNSUPPORTED;
  if (num_splits < 1 || num_splits > 256 || num_splits > Nk) return ATTN_E_INVALID;
  if (!decode_sizes_ok(B, H, num_splits)) return ATTN_E_INVALID;
  if (attn::decode_workspace_bytes(B, H, d, num_splits) > attn::kDecodeStaticScratchBytes) return ATTN_E_WORKSPACE;
  return hip_status(attn::launch_decode_static(q, k, v, out, lse, B, H, Nk, d, scale, dtype == ATTN_BF16,
                                               num_splits, static_cast<hipStream_t>(stream)));
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nq, int Nk, int d,
             float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, out, lse, B, H, H, Nq, Nk, d, scale, causal, dtype, workspace, workspace_bytes, stream);
}

int attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv, int Nq,
                 int Nk, int d, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return fwd_impl(q, k, v, out, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, workspace, workspace_bytes, stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int nseq, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                    int H, int Hkv, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_k) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_E_INVALID;
  if ((lse && !aligned4(lse)) || !aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k)) return ATTN_E_INVALID;
  if (nseq < 1 || H < 1 || Hkv < 1 || H % Hkv != 0) return ATTN_E_INVALID;
  if (max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0) return ATTN_E_INVALID;
  if (!good_scale(scale)) return ATTN_E_INVALID;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_E_UNSUPPORTED;
  if (!prefill_head_ok(max_seqlen_q, max_seqlen_k, d) || !prefill_grid_ok(nseq, H, max_seqlen_q))
    return ATTN_E_INVALID;
  if (max_seqlen_q == 0 || total_q == 0) return ATTN_OK;  // no query: nothing to write
  const attn::SeqShape sh{cu_seqlens_q, cu_seqlens_k, H, H / Hkv, total_q, total_k};
  return hip_status(attn::launch_prefill(q, k, v, out, lse, sh, nseq, max_seqlen_q, d, scale, causal != 0,
                                         dtype == ATTN_BF16, static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype) {
  (void)Nk;
  (void)d;
  (void)dtype;
  if (B < 1 || H < 1 || Nq < 1) return 0;
  return attn::bwd_workspace_bytes((long)B * H * Nq);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
             void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_gqa(q, k, v, out, dout, lse, dq, dk, dv, B, H, H, Nq, Nk, d, scale, causal, dtype, workspace,
                      workspace_bytes, stream);
}

int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(q, k, v, out, lse, B, H, Nq, Nk, scale, causal);
  if (rc != ATTN_OK) return rc;
  if (Hkv < 1 || H % Hkv != 0) return ATTN_E_INVALID;
  if (!dout || !lse || !dq || !dk || !dv) return ATTN_E_INVALID;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return ATTN_E_INVALID;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_E_UNSUPPORTED;
  if (!prefill_head_ok(Nq, Nk, d) || !prefill_grid_ok(B, H, Nk)) return ATTN_E_INVALID;
  if (!attn::span_ok((long long)Nq * 8)) return ATTN_E_INVALID;  // per-row (lse, D) pairs
  const long rows = (long)B * H * Nq;
  if (!workspace || workspace_bytes < attn::bwd_workspace_bytes(rows) || !aligned16(workspace))
    return ATTN_E_WORKSPACE;
  const attn::SeqShape sh{nullptr, nullptr, H, H / Hkv, Nq, Nk};
  return hip_status(attn::launch_bwd(q, k, v, out, dout, lse, dq, dk, dv, sh, B, Nq, Nk, rows, d, scale,
                                     causal != 0, dtype == ATTN_BF16, workspace, static_cast<hipStream_t>(stream)));
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                    int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int H, int Hkv, int d, float scale,
                    int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k)
    return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned4(lse) || !aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k))
    return ATTN_E_INVALID;
  if (nseq < 1 || H < 1 || Hkv < 1 || H % Hkv != 0) return ATTN_E_INVALID;
  if (max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0) return ATTN_E_INVALID;
  if (!good_scale(scale)) return ATTN_E_INVALID;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_E_UNSUPPORTED;
  if (!prefill_head_ok(max_seqlen_q, max_seqlen_k, d) || !prefill_grid_ok(nseq, H, max_seqlen_q) ||
      !prefill_grid_ok(nseq, H, max_seqlen_k) || !attn::span_ok((long long)max_seqlen_q * 8))
    return ATTN_E_INVALID;
  const long rows = (long)H * total_q;
  if (!workspace || workspace_bytes < attn::bwd_workspace_bytes(rows) || !aligned16(workspace))
    return ATTN_E_WORKSPACE;
  if (total_q == 0 && total_k == 0) return ATTN_OK;  // nothing to differentiate
  const attn::SeqShape sh{cu_seqlens_q, cu_seqlens_k, H, H / Hkv, total_q, total_k};
  return hip_status(attn::launch_bwd(q, k, v, out, dout, lse, dq, dk, dv, sh, nseq, max_seqlen_q, max_seqlen_k,
                                     rows, d, scale, causal != 0, dtype == ATTN_BF16, workspace,
                                     static_cast<hipStream_t>(stream)));
}

int attn_quantize_rows_i8(const void* x, int8_t* x8, float* scales, long rows, int d, void* stream) {
  if (!x || !x8 || !scales || rows < 1) return ATTN_E_INVALID;
  if (!aligned16(x) || !aligned16(x8) || !aligned4(scales)) return ATTN_E_INVALID;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if ((rows + 15) / 16 > INT_MAX) return ATTN_E_INVALID;
  return hip_status(attn::launch_quantize_rows_i8(x, x8, scales, rows, d, static_cast<hipStream_t>(stream)));
}

size_t attn_quantize_e4m3_workspace_bytes(long n) {
  if (n < 8 || n % 8) return 0;
  return attn::quantize_e4m3_workspace_bytes(n);
}

int attn_quantize_tensor_e4m3(const void* x, uint8_t* x8, float* scale_out, long n, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!x || !x8 || !scale_out || n < 8 || n % 8) return ATTN_E_INVALID;
  if (!aligned16(x) || !aligned16(x8) || !aligned4(scale_out)) return ATTN_E_INVALID;
  if (!workspace || workspace_bytes < attn::quantize_e4m3_workspace_bytes(n) || !aligned4(workspace))
    return ATTN_E_WORKSPACE;
  return hip_status(
      attn::launch_quantize_tensor_e4m3(x, x8, scale_out, n, workspace, static_cast<hipStream_t>(stream)));
}

int attn_fwd_q8(const int8_t* q8, const int8_t* k8, const uint8_t* v8, const float* q_scale, const float* k_scale,
                const float* v_scale, void* out, float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                int causal, void* stream) {
  int rc = check_common(q8, k8, v8, out, lse, B, H, Nq, Nk, scale, causal);
  if (rc != ATTN_OK) return rc;
  if (!q_scale || !k_scale || !v_scale || !aligned4(q_scale) || !aligned4(k_scale) || !aligned4(v_scale))
    return ATTN_E_INVALID;
  if (d != 128) return ATTN_E_UNSUPPORTED;
  return hip_status(attn::launch_prefill_q8(q8, k8, v8, q_scale, k_scale, v_scale, out, lse, B, H, Nq, Nk, d, scale,
                                            causal != 0, attn::QVariant::kInt8Scores,
                                            static_cast<hipStream_t>(stream)));
}

int attn_fwd_i8(const int8_t* q8, const int8_t* k8, const int8_t* v8, const float* q_scale, const float* k_scale,
                const float* v_scale, void* out, float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                int causal, void* stream) {
  int rc = check_common(q8, k8, v8, out, lse, B, H, Nq, Nk, scale, causal);
  if (rc != ATTN_OK) return rc;
  if (!q_scale || !k_scale || !v_scale || !aligned4(q_scale) || !aligned4(k_scale) || !aligned4(v_scale))
    return ATTN_E_INVALID;
  if (d != 128) return ATTN_E_UNSUPPORTED;
  return hip_status(attn::launch_prefill_q8(q8, k8, reinterpret_cast<const uint8_t*>(v8), q_scale, k_scale, v_scale,
                                            out, lse, B, H, Nq, Nk, d, scale, causal != 0, attn::QVariant::kAllInt8,
                                            static_cast<hipStream_t>(stream)));
}

int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale, const float* k_scale,
                 const float* v_scale, void* out, float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                 int causal, void* stream) {
  int rc = check_common(q8, k8, v8, out, lse, B, H, Nq, Nk, scale, causal);
  if (rc != ATTN_OK) return rc;
  if (!q_scale || !k_scale || !v_scale || !aligned4(q_scale) || !aligned4(k_scale) || !aligned4(v_scale))
    return ATTN_E_INVALID;
  if (d != 128) return ATTN_E_UNSUPPORTED;
  return hip_status(attn::launch_prefill_q8(q8, k8, v8, q_scale, k_scale, v_scale, out, lse, B, H, Nq, Nk, d, scale,
                                            causal != 0, attn::QVariant::kFp8, static_cast<hipStream_t>(stream)));
}

int attn_fwd_fp4p(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale, const float* k_scale,
                  const float* v_scale, void* out, float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                  int causal, void* stream) {
  int rc = check_common(q8, k8, v8, out, lse, B, H, Nq, Nk, scale, causal);
  if (rc != ATTN_OK) return rc;
  if (!q_scale || !k_scale || !v_scale || !aligned4(q_scale) || !aligned4(k_scale) || !aligned4(v_scale))
    return ATTN_E_INVALID;
  if (d != 128) return ATTN_E_UNSUPPORTED;
  return hip_status(attn::launch_prefill_q8(q8, k8, v8, q_scale, k_scale, v_scale, out, lse, B, H, Nq, Nk, d, scale,
                                            causal != 0, attn::QVariant::kFp8P4, static_cast<hipStream_t>(stream)));
}

int attn_rotate_quantize_e4m3(const void* x, const float* signs, uint8_t* x8, float* scales, int BH, int N, int d,
                              int block_rows, void* stream) {
  if (!x || !x8 || !scales || BH < 1 || N < 1 || block_rows < 1) return ATTN_E_INVALID;
  if (!aligned16(x) || !aligned16(x8) || !aligned4(scales) || (signs && !aligned4(signs))) return ATTN_E_INVALID;
  if (d != 128) return ATTN_E_UNSUPPORTED;
  const long nblk = (N + (long)std::min(block_rows, N) - 1) / std::min(block_rows, N);
  if ((long)BH * nblk > 0x7fffffffL) return ATTN_E_INVALID;
  return hip_status(attn::launch_rotate_quantize_e4m3(x, signs, x8, scales, BH, N, d, block_rows,
                                                      static_cast<hipStream_t>(stream)));
}

int attn_quantize_tensor_i8(const void* x, int8_t* x8, float* scale_out, long n, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!x || !x8 || !scale_out || n < 8 || n % 8 != 0) return ATTN_E_INVALID;
  if (!aligned16(x) || !aligned16(x8) || !aligned4(scale_out)) return ATTN_E_INVALID;
  if (!workspace || workspace_bytes < attn::quantize_e4m3_workspace_bytes(n) || !aligned4(workspace))
    return ATTN_E_WORKSPACE;
  return hip_status(attn::launch_quantize_tensor_i8(x, x8, scale_out, n, workspace, static_cast<hipStream_t>(stream)));
}

int attn_debug_qk_i32(const int8_t* q8, const int8_t* k8, int32_t* s, int Nq, int Nk, int d, void* stream) {
  if (!q8 || !k8 || !s || Nq < 1 || Nk < 1) return ATTN_E_INVALID;
  if (!aligned16(q8) || !aligned16(k8) || !aligned4(s)) return ATTN_E_INVALID;
  if (d != 128) return ATTN_E_UNSUPPORTED;
  return hip_status(attn::launch_debug_qk(q8, k8, s, Nq, Nk, d, false, static_cast<hipStream_t>(stream)));
}

int attn_debug_qk_f8(const uint8_t* q8, const uint8_t* k8, float* s, int Nq, int Nk, int d, void* stream) {
  if (!q8 || !k8 || !s || Nq < 1 || Nk < 1) return ATTN_E_INVALID;
  if (!aligned16(q8) || !aligned16(k8) || !aligned4(s)) return ATTN_E_INVALID;
  if (d != 128) return ATTN_E_UNSUPPORTED;
  return hip_status(attn::launch_debug_qk(q8, k8, s, Nq, Nk, d, true, static_cast<hipStream_t>(stream)));
}

int attn_debug_cvt_e2m1(const float* x, uint8_t* y, long n, void* stream) {
  if (!x || !y || n < 8 || n % 8) return ATTN_E_INVALID;
  if (!aligned4(x)) return ATTN_E_INVALID;
  if ((n / 8 + 255) / 256 > INT_MAX) return ATTN_E_INVALID;
  return hip_status(attn::launch_debug_cvt_e2m1(x, y, n, static_cast<hipStream_t>(stream)));
}

int attn_fwd_exp2_split(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nq,
                        int Nk, int d, float scale, int causal, int dtype, int poly_per_8, void* stream) {
  const int rc = check_common(q, k, v, out, lse, B, H, Nq, Nk, scale, causal);
  if (rc != ATTN_OK) return rc;
  if (poly_per_8 != 0 && poly_per_8 != 2 && poly_per_8 != 4) return ATTN_E_INVALID;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_E_UNSUPPORTED;
  if (poly_per_8 != 0 && d != 128) return ATTN_E_UNSUPPORTED;
  if (!prefill_head_ok(Nq, Nk, d)) return ATTN_E_INVALID;
  const attn::SeqShape sh{nullptr, nullptr, H, 1, Nq, Nk};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (poly_per_8 == 0)
    return hip_status(attn::launch_prefill(q, k, v, out, lse, sh, B, Nq, d, scale, causal != 0, dtype == ATTN_BF16, st));
  return hip_status(attn::launch_prefill_exp2_split(q, k, v, out, lse, sh, B, Nq, d, scale, causal != 0,
                                                    dtype == ATTN_BF16, poly_per_8, st));
}

int attn_debug_exp2_poly(const float* x, float* y, long n, void* stream) {
  if (!x || !y || n < 1) return ATTN_E_INVALID;
  if (!aligned4(x) || !aligned4(y)) return ATTN_E_INVALID;
  if ((n + 255) / 256 > INT_MAX) return ATTN_E_INVALID;
  return hip_status(attn::launch_debug_exp2_poly(x, y, n, static_cast<hipStream_t>(stream)));
}

int attn_debug_cvt_e4m3(const float* x, uint8_t* y, long n, void* stream) {
  if (!x || !y || n < 2 || n % 2) return ATTN_E_INVALID;
  if (!aligned4(x)) return ATTN_E_INVALID;
  if ((n / 2 + 255) / 256 > INT_MAX) return ATTN_E_INVALID;
  return hip_status(attn::launch_debug_cvt_e4m3(x, y, n, static_cast<hipStream_t>(stream)));
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_INVALID: return "invalid argument (null/misaligned pointer, bad or too large size, bad scale, causal with Nq > Nk)";
    case ATTN_E_UNSUPPORTED: return "unsupported head size or dtype";
    case ATTN_E_WORKSPACE:
      return "workspace missing or too small (attn_fwd_decode_static: partials larger than its static scratch)";
    case ATTN_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* attn_build_info(void) {
  return "libattn_mi355x: gfx950; prefill bf16/fp16 d=128 BM=256 (8 waves, 2 groups ping-ponging MFMA and "
         "softmax phases, 32 rows/wave), BN=64, causal blocks paired on large grids; d=64 BM=128 BN=64 (4 waves, "
         "3 workgroups/CU interleaving MFMA and softmax freely); direct-to-LDS double-buffered K/V tiles, 32x32x16 "
         "MFMA, S^T=KQ^T, V^T via ds_read_b64_tr_b16, running max raised only when a lane's tile P sums past 2^14; "
         "decode split-KV 256 threads, 8 rows in flight/lane + LSE merge (static 8 MiB scratch variant); "
         "q8 prefill d=128 BM=128 BN=64 (3 workgroups/CU, double-buffered direct-to-LDS K8/V8 tiles), int8 32x32x32 + "
         "fp8 32x32x64 MFMA, V^T via ds_read_b64_tr_b8; "
         "backward: (lse, D) preprocess, dK/dV kernel (128 keys/WG; d=128 dense non-causal: P/dV and dS/dK wave "
         "groups ping-ponging MFMA and vector phases over 64-query steps, else 32-query steps with K and V rows "
         "resident), "
         "dQ kernel (128 queries/WG, 32-key steps), no atomics";
}

}  // extern "C"
