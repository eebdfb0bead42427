/*
 * attn_mi355x.h -- C ABI of the MI355X (gfx950) FlashAttention library
 * (libattn_mi355x.so): the forward pass (prefill, split-KV decode, quantised)
 * and its backward pass.
 *
 * What the library computes.  For every batch b and head h, exact attention
 *     O = softmax(Q K^T * scale) V
 * ("Why attention is bound to memory" in the marketmaker.cc post "Can a full
 * trading day of context beat one minute? Flash attention and the
 * sequence-length question"; "Introduction" of the linux-konsole.com post
 * "FlashAttention 4: fast, memory-efficient attention for LLMs"), computed
 * tile by tile with the online-softmax recurrence of that post's sections
 * "The Flash Attention algorithm" and "The online softmax recurrence", so the
 * Nq x Nk score matrix never reaches device memory.  Next to O the library
 * writes the per-row log-sum-exp
 *     LSE[b,h,i] = ln sum_{j visible} exp(scale * q_i . k_j)
 * (natural log; the stored softmax statistics (m, l) of "Backward: recompute
 * instead of store", folded as m + ln l), which attn_bwd takes back to
 * rebuild the probabilities for the gradients.
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, row-major [B, H, N, d] (batch, heads, sequence,
 *     head_dim), the layout of "Integration in eight lines"; LSE is [B, H, Nq]
 *     float32.  Every pointer is DEVICE memory owned by the caller and must
 *     be 16-byte aligned.  Inputs are only read; outputs are fully
 *     overwritten (every element, including tail rows); nothing needs to be
 *     zeroed first.
 *   - causal != 0 masks future keys ("Causal masking" section) with
 *     bottom-right alignment: query i sees key j iff j <= i + (Nk - Nq).
 *     For Nq == Nk this is the usual lower-triangular mask.  causal with
 *     Nq > Nk is rejected.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising.  The library never
 *     allocates or frees device memory and, apart from the static split
 *     array of attn_fwd_decode_static (below), keeps no mutable global
 *     state: the other calls are reentrant and thread-safe.  Asynchronous
 *     GPU faults surface at the caller's next synchronisation.
 *   - Every argument is validated before anything is launched: a return of
 *     ATTN_E_INVALID, ATTN_E_UNSUPPORTED or ATTN_E_WORKSPACE means nothing
 *     was launched.  ATTN_E_HIP reports a launch error; the entry points
 *     that run several kernels stop at the first such error, but kernels
 *     enqueued before it in the same call may still run.  There is no silent fallback
 *     to another algorithm: an unsupported head size or dtype is an error
 *     (the silent math-path fallback criticised in "Integration in eight
 *     lines" is exactly what this library refuses to do).
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = -1,     /* null/misaligned pointer, non-positive or too large size, bad scale,
                              causal with Nq > Nk */
  ATTN_E_UNSUPPORTED = -2, /* head size or dtype outside what is built */
  ATTN_E_WORKSPACE = -3,   /* workspace missing or smaller than *_workspace_bytes() */
  ATTN_E_HIP = -4          /* a HIP launch error was reported */
};

/* Storage types of Q, K, V and O. */
enum { ATTN_BF16 = 0, ATTN_FP16 = 1 };

/*
 * Bytes of device workspace attn_fwd() needs for these sizes.  Prefill
 * (Nq > 1) needs none (returns 0).  Decode (Nq == 1) runs split-KV and
 * needs room for the per-split partial results: B*H*splits*(d+1) floats,
 * with `splits` chosen by the library (see attn_fwd_decode_splits()).
 * Returns 0 for invalid sizes as well; attn_fwd() reports those.
 */
size_t attn_fwd_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype);

/*
 * Attention forward, bf16 or fp16 storage, fp32 accumulation.
 *   q   [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,d]   (dtype)
 *   out [B,H,Nq,d] (dtype), rounded to nearest even from fp32
 *   lse [B,H,Nq] float32, natural log; may be NULL (not written)
 *   d in {64, 128}; B, H, Nq, Nk >= 1; scale finite and > 0
 *   (use 1/sqrt(d) for the usual softmax(Q K^T / sqrt(d)) V).
 *   workspace: device buffer of at least attn_fwd_workspace_bytes() bytes
 *   (may be NULL when that is 0).  The workspace is scratch: its contents
 *   after the call are unspecified.
 * Nq == 1 dispatches to the split-KV decode kernels (partials over key
 * ranges, then a log-sum-exp merge); every other Nq runs the tiled prefill
 * kernel, which addresses one head of Q, K or V through 32-bit buffer
 * offsets: Nq*d*2 and Nk*d*2 must be at most 2^31 - 2^16 bytes (the headroom
 * keeps the offset of the tile requested past Nk below 2^31), else
 * ATTN_E_INVALID.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped-query attention (GQA; MQA with Hkv = 1), one of the features the
 * linux-konsole.com post "FlashAttention 4: fast, memory-efficient attention
 * for LLMs" lists as missing from FA4: H query heads share Hkv key/value
 * heads, and query head h attends with K/V head h / (H / Hkv) (consecutive
 * query heads share one K/V head).  H must be a multiple of Hkv.
 *   q, out [B,H,Nq,d]; k, v [B,Hkv,Nk,d]; lse [B,H,Nq].
 * Everything else (dtype, d, causal, errors) is as for attn_fwd, which is
 * this call with Hkv = H.  Nq == 1 needs a workspace of
 * attn_fwd_gqa_workspace_bytes() bytes.  The decode kernels serve up to 8
 * query heads of a group per workgroup, reading each K/V row once for all
 * of them.
 */
size_t attn_fwd_gqa_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d, int dtype);
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed variable-length batch ("varlen" in the same post's list): nseq
 * sequences of different lengths stored back to back along the token axis,
 * head-major:
 *   q, out [H, total_q, d]; k, v [Hkv, total_k, d]; lse [H, total_q] (may be NULL)
 *   cu_seqlens_q, cu_seqlens_k: DEVICE int32 arrays of nseq + 1 offsets,
 *   0 = cu[0] <= cu[1] <= ... <= cu[nseq] = total; sequence s owns query
 *   tokens cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and key tokens
 *   cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1.
 *   max_seqlen_q, max_seqlen_k: upper bounds of the per-sequence lengths
 *   (the grid covers max_seqlen_q queries per sequence; rows past it in a
 *   longer sequence are not written).
 * Each sequence is plain attention of its queries over its keys (GQA head
 * mapping as in attn_fwd_gqa); causal masks are bottom-right aligned within
 * each sequence.  A query row that sees no key (an empty key range, or
 * causal with more queries than keys in its sequence) gets out = 0 and
 * lse = -inf.  The offsets live in device memory and cannot be checked on
 * the host: the kernel clamps them into [0, total] so malformed offsets
 * address only rows of the right head.  No workspace.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq, int max_seqlen_q,
                    int max_seqlen_k, int total_q, int total_k, int H, int Hkv, int d, float scale,
                    int causal, int dtype, void* stream);

/* Split count attn_fwd() uses for a decode problem (Nq == 1). */
int attn_fwd_decode_splits(int B, int H, int Nk, int d);

/*
 * Split-KV decode with an explicit split count (1 <= num_splits <= 256,
 * num_splits <= Nk).  Query length is 1: q and out are [B,H,1,d].  Keys are
 * cut into num_splits contiguous ranges; each range produces a normalised
 * partial output and its log-sum-exp in `workspace`
 * (>= attn_decode_workspace_bytes() bytes), and a second kernel merges the
 * partials: LSE = M + ln sum_s exp(LSE_s - M), O = sum_s exp(LSE_s - LSE) O_s,
 * which is one application of the running-statistics update of "The Flash
 * Attention algorithm" to states computed over disjoint key ranges.
 * causal is accepted and has no effect (the single query is the newest and
 * sees every key).  dtype: ATTN_BF16 or ATTN_FP16; d in {64, 128}.
 */
size_t attn_decode_workspace_bytes(int B, int H, int d, int num_splits);
int attn_fwd_decode(const void* q, const void* k, const void* v, void* out, float* lse,
                    int B, int H, int Nk, int d, float scale, int dtype, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same split-KV decode with the same arguments minus the workspace.  The
 * split partials (B*H*num_splits*(d+1) floats, attn_decode_workspace_bytes())
 * go to a static device array of ATTN_DECODE_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; this call
 * allocates and frees nothing.  Larger partials are refused with
 * ATTN_E_WORKSPACE before anything is launched.  Every call on one GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller; calls in order
 * on one stream are safe, and nothing in the array needs clearing between
 * them.  The first call on a device looks the array's address up once.
 */
#define ATTN_DECODE_STATIC_SCRATCH_BYTES (8u << 20)
int attn_fwd_decode_static(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int H, int Nk, int d, float scale, int dtype, int num_splits,
                           void* stream);

/*
 * Attention backward: the gradients of sum(dout * out) with respect to q, k
 * and v, for out = attention(q, k, v) as computed by attn_fwd (same scale and
 * causal flag).  The probability tiles are rebuilt from q, k and the
 * forward's log-sum-exp instead of being stored ("Backward: recompute
 * instead of store" in the marketmaker.cc post "Can a full trading day of
 * context beat one minute?"): with P = softmax(scale q k^T) (future keys
 * masked when causal), dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with
 * D_i = sum_c dO_ic O_ic, dQ = scale dS K, dK = scale dS^T Q.
 *   q, k, v, out, dout as in attn_fwd ([B,H,N,d], dtype); lse [B,H,Nq]
 *   float32 (natural log) from attn_fwd, required.
 *   dq [B,H,Nq,d], dk, dv [B,H,Nk,d] (dtype), fully overwritten; fp32
 *   accumulation, rounded to nearest even.
 *   workspace: device buffer of at least attn_bwd_workspace_bytes() bytes
 *   (B*H*Nq float pairs: lse in base 2 and D), 16-byte aligned; its contents
 *   after the call are unspecified.
 *   d in {64, 128}; B, H, Nq, Nk >= 1; causal needs Nq <= Nk; one head of
 *   q, k, v spans at most 2^31 - 2^16 bytes, as for attn_fwd (ATTN_E_INVALID
 *   otherwise).
 * Three kernels run on `stream`: the (lse, D) preprocess, a key-block kernel
 * for dK and dV and a query-block kernel for dQ.  No atomics: the result does
 * not depend on scheduling.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype);
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d,
             float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of attn_fwd_gqa: q, out, dout, dq [B,H,Nq,d]; k, v, dk, dv
 * [B,Hkv,Nk,d]; lse [B,H,Nq].  dK and dV of a shared K/V head are the sums of
 * the contributions of all H/Hkv query heads that read it (computed inside
 * one workgroup per key block, no atomics).  Workspace as attn_bwd
 * (attn_bwd_workspace_bytes with the query head count H).
 */
int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk,
                 int d, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Backward of attn_fwd_varlen (same packed layouts and offsets; dq like q,
 * dk and dv like k and v; lse [H, total_q] as attn_fwd_varlen wrote it, so a
 * row that saw no key carries -inf and gets dq = 0).  Every token row inside
 * a sequence is written (a sequence with no keys gets dq = 0, one with no
 * queries dk = dv = 0).  workspace: at least H * total_q * 8 bytes
 * (attn_bwd_workspace_bytes(1, H, total_q, ...)), 16-byte aligned.
 */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int nseq, int max_seqlen_q, int max_seqlen_k, int total_q,
                    int total_k, int H, int Hkv, int d, float scale, int causal, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Quantisation of bf16 inputs for the quantised forward (token-level INT8
 * post-training quantisation of Q and K as in the hoodcat.net post
 * "INT-FlashAttention: an INT8 quantisation architecture compatible with
 * FlashAttention"; V in OCP FP8 E4M3 with one scale for the whole tensor).
 *
 * attn_quantize_rows_i8: x [rows, d] bf16 -> x8 [rows, d] int8 and
 *   scales [rows] float32 with s = max|row| / 127 and
 *   x8 = clamp(rint(x / s), -127, 127) (IEEE fp32 division, round half to
 *   even); an all-zero row gives s = 0 and x8 = 0.  d in {64, 128}.
 * attn_quantize_e4m3_workspace_bytes / attn_quantize_tensor_e4m3:
 *   x [n] bf16 -> x8 [n] E4M3FN codes and *scale_out (DEVICE float) with
 *   s = max|x| / 448 and x8 = E4M3(x / s), round to nearest even,
 *   saturating at 448.  n >= 1 and a multiple of 8.  The workspace holds
 *   the partial maxima of the two-pass reduction.
 */
int attn_quantize_rows_i8(const void* x, int8_t* x8, float* scales, long rows, int d, void* stream);
size_t attn_quantize_e4m3_workspace_bytes(long n);
int attn_quantize_tensor_e4m3(const void* x, uint8_t* x8, float* scale_out, long n,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Quantised attention forward:
 *   S_ij = (sum_t q8[i,t] k8[j,t]) * q_scale[i] * k_scale[j] * scale,
 * with the integer dot products accumulated exactly in int32 by int8 MFMA;
 * P = exp(S - running max) is cast to E4M3 before the P.V product on fp8
 * MFMA; the row sum l uses the fp32 P; O = (P~ V8) * v_scale / l.
 *   q8 [B,H,Nq,d] int8, k8 [B,H,Nk,d] int8, v8 [B,H,Nk,d] E4M3 codes,
 *   q_scale [B,H,Nq], k_scale [B,H,Nk] float32, v_scale DEVICE pointer to
 *   one float32; out [B,H,Nq,d] bf16; lse [B,H,Nq] float32 or NULL.
 *   d == 128; causal as above; Nq, Nk >= 1.
 */
int attn_fwd_q8(const int8_t* q8, const int8_t* k8, const uint8_t* v8,
                const float* q_scale, const float* k_scale, const float* v_scale,
                void* out, float* lse, int B, int H, int Nq, int Nk, int d,
                float scale, int causal, void* stream);

/*
 * All-INT8 quantised forward: both products of the attention as INT8 GEMMs,
 * the INT-FlashAttention scheme of the hoodcat.net post "INT-FlashAttention:
 * an INT8 quantisation architecture compatible with FlashAttention".  Scores
 * as in attn_fwd_q8; V in int8 with one per-tensor scale
 * (attn_quantize_tensor_i8); P = exp(S - running max), kept <= 1 by raising
 * the running max on every increase, is quantised as rint(127 P) and P.V is
 * accumulated exactly in int32 per 64-key tile on int8 MFMA;
 * O = (sum of tiles) * v_scale / (127 l) with l the sum of the fp32 P.
 *   q8, k8 as attn_fwd_q8; v8 [B,H,Nk,d] int8; v_scale DEVICE pointer to
 *   one float32; out, lse, d, causal and errors as attn_fwd_q8.
 */
int attn_fwd_i8(const int8_t* q8, const int8_t* k8, const int8_t* v8,
                const float* q_scale, const float* k_scale, const float* v_scale,
                void* out, float* lse, int B, int H, int Nq, int Nk, int d,
                float scale, int causal, void* stream);

/*
 * Per-tensor int8 for attn_fwd_i8's V: x [n] bf16 -> x8 [n] int8 and
 * *scale_out (DEVICE float) with s = max|x| / 127 and
 * x8 = clamp(rint(x / s), -127, 127) (IEEE fp32 division, round half to
 * even); an all-zero tensor gives s = 0 and x8 = 0.  n >= 8, a multiple of
 * 8; workspace as attn_quantize_tensor_e4m3 (the partial maxima).
 */
int attn_quantize_tensor_i8(const void* x, int8_t* x8, float* scale_out, long n,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 forward with rotated, block-quantised Q and K: the incoherent processing
 * of FlashAttention-3 as the marketmaker.cc post "Can a full trading day of
 * context beat one minute? Flash attention and the sequence-length question"
 * describes it (section "FA3: Hopper mechanisms", FP8 with incoherent
 * processing).  Scores S = decode(q8) decode(k8)^T * q_scale[i] * k_scale[j]
 * * scale on the fp8 MFMA (exact products, fp32 sums); P cast to E4M3 and
 * P.V on the fp8 MFMA with V per-tensor E4M3, as attn_fwd_q8.
 *   q8 [B,H,Nq,d], k8, v8 [B,H,Nk,d] E4M3 codes (uint8); q_scale [B,H,Nq],
 *   k_scale [B,H,Nk] per-row fp32 scales (attn_rotate_quantize_e4m3 gives
 *   them block-constant); v_scale DEVICE pointer to one float32
 *   (attn_quantize_tensor_e4m3); out, lse, d, causal and errors as
 *   attn_fwd_q8.  Q8 and K8 rotated by the same R give the attention of the
 *   unrotated Q and K, since R is orthogonal.
 */
int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                 const float* q_scale, const float* k_scale, const float* v_scale,
                 void* out, float* lse, int B, int H, int Nq, int Nk, int d,
                 float scale, int causal, void* stream);

/*
 * attn_fwd_fp8 with the probabilities in four-bit floating point: the FP4
 * attention of the gist.science summary of "Hardware-Aware FP4
 * FlashAttention-4" (summary and explainer).  P = exp(S - running max) is
 * encoded as OCP E2M1 (0, 0.5, 1, 1.5, 2, 3, 4, 6; round to nearest even,
 * clamped at 6) with one power-of-two scale 2^e per 32 consecutive keys of a
 * query (OCP MX: e = floor(log2 max P of the block) - 2); P.V runs on the
 * mixed fp8 x fp4 MFMA with the scales applied by the matrix cores; l sums
 * the unquantised P.  Arguments and errors as attn_fwd_fp8.
 */
int attn_fwd_fp4p(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                  const float* q_scale, const float* k_scale, const float* v_scale,
                  void* out, float* lse, int B, int H, int Nq, int Nk, int d,
                  float scale, int causal, void* stream);

/*
 * Rotation and block E4M3 quantisation of Q or K for attn_fwd_fp8 (same
 * source as attn_fwd_fp8).  x [BH, N, d] bf16, d = 128.  With signs (DEVICE,
 * d float32 values, each +1 or -1; the caller draws them once and uses the
 * same signs for Q and K) each row becomes y = (x * signs) H_d, H_d the
 * Sylvester Hadamard matrix, evaluated in fp32 by butterflies at strides 1,
 * 2, ..., d/2; signs == NULL leaves rows unrotated (y = x).  Rows are grouped
 * per head into blocks of block_rows (the last block of a head may be
 * shorter); a block's s = max|y| / 448 (IEEE fp32), its codes
 * E4M3(y / s) (round to nearest even, saturating), and every row of the block
 * gets scales[row] = s / sqrt(d) rounded to fp32 when rotated (the
 * orthogonal rotation's normalisation), s when not; an all-zero block gives
 * scale 0 and codes 0.  x8 [BH, N, d] uint8; scales [BH, N] float32.
 * Errors: ATTN_E_INVALID for a NULL or misaligned pointer (x, x8 16-byte;
 * scales, signs 4-byte) or BH, N, block_rows < 1; ATTN_E_UNSUPPORTED for
 * d != 128.  Sign values other than +-1 are not checked.
 */
int attn_rotate_quantize_e4m3(const void* x, const float* signs, uint8_t* x8, float* scales,
                              int BH, int N, int d, int block_rows, void* stream);

/*
 * Test hooks that expose the quantised kernel's own device code:
 * attn_debug_qk_i32: s[i,j] = sum_t q8[i,t] k8[j,t] for one head
 *   (q8 [Nq,d], k8 [Nk,d] int8, s [Nq,Nk] int32), through the same int8
 *   MFMA tile routine as attn_fwd_q8; d == 128.
 * attn_debug_qk_f8: s[i,j] = sum_t E4M3(q8[i,t]) E4M3(k8[j,t]) for one
 *   head (uint8 codes, s fp32), through the same fp8 MFMA tile routine as
 *   attn_fwd_fp8; d == 128.
 * attn_debug_cvt_e4m3: y[i] = E4M3(x[i]) through the same conversion
 *   routine attn_quantize_tensor_e4m3 uses (saturating); n even.
 * attn_debug_cvt_e2m1: y[i] = E2M1 code (0 .. 15) of x[i] through the same
 *   conversion routine attn_fwd_fp4p uses for P (clamped at 6), eight values
 *   packed per 32-bit word as the P operand is; n a multiple of 8.
 */
int attn_debug_qk_i32(const int8_t* q8, const int8_t* k8, int32_t* s, int Nq, int Nk, int d, void* stream);
int attn_debug_qk_f8(const uint8_t* q8, const uint8_t* k8, float* s, int Nq, int Nk, int d, void* stream);
int attn_debug_cvt_e4m3(const float* x, uint8_t* y, long n, void* stream);
int attn_debug_cvt_e2m1(const float* x, uint8_t* y, long n, void* stream);

/*
 * Software-exp2 split ("Software exp2" in the linux-konsole.com post
 * "FlashAttention 4: fast, memory-efficient attention for LLMs": part of the
 * softmax's exponentials computed by a polynomial on the FMA units instead of
 * the transcendental unit).  attn_fwd_exp2_split is the dense prefill of
 * attn_fwd (Hkv = H, any Nq >= 1, the same layouts, scale, causal rule and
 * errors) with poly_per_8 of every 8 exponentials on the polynomial:
 *   poly_per_8 in {0, 2, 4}; 0 is attn_fwd's prefill kernel itself;
 *   2 and 4 need d == 128 (ATTN_E_UNSUPPORTED otherwise).
 * The polynomial is 2^x = 2^floor(x) * c(x - floor(x)) with a cubic c fitted
 * for relative error (at most 7.5e-5); arguments below -125 give 0.  On
 * gfx950 v_exp_f32 costs about two FMAs, so the split is slower than the
 * default; it is kept to measure that.
 * attn_debug_exp2_poly: y[i] = that polynomial at x[i] (fp32 device arrays,
 *   n >= 1), the routine the split softmax calls.
 */
int attn_fwd_exp2_split(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nq,
                        int Nk, int d, float scale, int causal, int dtype, int poly_per_8, void* stream);
int attn_debug_exp2_poly(const float* x, float* y, long n, void* stream);

/* Static text for a return code. */
const char* attn_status_str(int status);

/* Static text describing the build: target, kernels, tile sizes. */
const char* attn_build_info(void);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_MI355X_H */
