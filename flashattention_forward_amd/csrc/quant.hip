// Quantised attention forward for gfx950: int8 scores, fp8 (OCP E4M3) P.V.
//
// Follows the token-level INT8 scheme of the hoodcat.net post
// "INT-FlashAttention: an INT8 quantisation architecture compatible with
// FlashAttention" (integer GEMM for Q K^T with one fp32 scale per token of Q
// and of K), with V in E4M3 under one per-tensor scale and P cast to E4M3
// before the P.V product.  The tiled online softmax is the same as in the
// 16-bit prefill kernel (see prefill.hip); what changes:
//   * S^T = K8 Q8^T on v_mfma_i32_32x32x32_i8 with exact int32 accumulation
//     (|S| <= 127^2 d < 2^24, so the conversion to fp32 is exact too);
//     scores are acc * k_scale[key] * (q_scale[q] * scale * log2 e);
//   * P^T is converted to E4M3 in registers (v_cvt_pk_fp8_f32, round to
//     nearest even) and fed to v_mfma_f32_32x32x64_f8f6f4 as the B operand:
//     a lane's 32 values of a 64-key tile are exactly one k-step;
//   * K8 (with its key scales) and V8 tiles go from global memory straight
//     into double-buffered LDS, rows permuted so that the 32 keys each
//     half-wave holds in the S^T accumulator are 32 consecutive LDS rows;
//     four transposing 8-bit LDS reads (ds_read_b64_tr_b8) then give every
//     lane its 32 V values in the same key order;
//   * the softmax is vector-ALU bound (its exponentials, conversions and
//     scales outweigh the 8-bit MFMAs), so each wave runs its tile's matrix
//     and vector work in turn and three workgroups per CU (three waves per
//     SIMD) interleave them;
//   * l sums the fp32 P (only the MFMA operand is quantised) and the epilogue
//     applies v_scale / l.
// The quantisation kernels (per-token int8, per-tensor E4M3) and two test
// hooks that run this file's own tile routines live here as well.
#include <cfloat>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace attn {

namespace {

template <int CTRL>
__device__ __forceinline__ float dppq(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// max over aligned groups of G lanes (8 or 16), every lane gets it
template <int G>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dppq<0xB1>(x));
  x = fmaxf(x, dppq<0x4E>(x));
  if (G == 16) {
    x = fmaxf(x, dppq<0x124>(x));
    x = fmaxf(x, dppq<0x128>(x));
  } else {
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x101F)));
  }
  return x;
}

__device__ __forceinline__ float block_max_256(float x, float* red) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// E4M3 (OCP FN) codes of four floats, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3x4_sat(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}
// Same without the clamp, for values known to be within [0, 448] (P).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ void bf16x8_to_f32(u32x4 u, float* f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __builtin_bit_cast(float, u[j] << 16);
    f[2 * j + 1] = __builtin_bit_cast(float, u[j] & 0xFFFF0000u);
  }
}

// ------------------------------------------------------------ per-token int8
template <int D>
__global__ __launch_bounds__(256) void quantize_rows_i8_kernel(const uint16_t* __restrict__ X, int8_t* __restrict__ X8,
                                                               float* __restrict__ S, long rows) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int ch = threadIdx.x % LPR;
  const bool valid = row < rows;
  float f[8];
  u32x4 u = {0u, 0u, 0u, 0u};
  if (valid) u = reinterpret_cast<const u32x4*>(X + row * D)[ch];
  bf16x8_to_f32(u, f);
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
  amax = group_max<LPR>(amax);
  const float s = amax / 127.0f;  // IEEE division
  uint32_t lo = 0, hi = 0;
  if (s > 0.f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q = fminf(fmaxf(__builtin_rintf(f[j] / s), -127.f), 127.f);
      const uint32_t b = (uint32_t)((int)q) & 0xFFu;
      if (j < 4) lo |= b << (8 * j);
      else hi |= b << (8 * (j - 4));
    }
  }
  if (valid) {
    u32x2 o;
    o[0] = lo;
    o[1] = hi;
    reinterpret_cast<u32x2*>(X8 + row * D)[ch] = o;
    if (ch == 0) S[row] = s;
  }
}

// ------------------------------------------------------------ per-tensor E4M3
// (the number of partial maxima, e4m3_partials(), is a host rule in plan.cpp)

__global__ __launch_bounds__(256) void amax_partial_kernel(const uint16_t* __restrict__ X, long chunks,
                                                           float* __restrict__ partial) {
  __shared__ float red[4];
  float m = 0.f;
  for (long c = (long)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (long)gridDim.x * 256) {
    float f[8];
    bf16x8_to_f32(reinterpret_cast<const u32x4*>(X)[c], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
  }
  m = block_max_256(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const uint16_t* __restrict__ X, long chunks,
                                                            const float* __restrict__ partial, int npart,
                                                            uint8_t* __restrict__ X8, float* __restrict__ scale_out) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < npart; i += 256) m = fmaxf(m, partial[i]);
  m = block_max_256(m, red);
  const float s = m / 448.0f;  // IEEE division
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  for (long c = (long)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (long)gridDim.x * 256) {
    u32x2 o = {0u, 0u};
    if (s > 0.f) {
      float f[8];
      bf16x8_to_f32(reinterpret_cast<const u32x4*>(X)[c], f);
      o[0] = e4m3x4_sat(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
      o[1] = e4m3x4_sat(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
    }
    reinterpret_cast<u32x2*>(X8)[c] = o;
  }
}

// per-tensor symmetric int8 (the all-INT8 variant's V): s = max|x| / 127,
// codes clamp(rint(x / s), -127, 127), IEEE fp32 division
__global__ __launch_bounds__(256) void quantize_i8_tensor_kernel(const uint16_t* __restrict__ X, long chunks,
                                                                 const float* __restrict__ partial, int npart,
                                                                 int8_t* __restrict__ X8, float* __restrict__ scale_out) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < npart; i += 256) m = fmaxf(m, partial[i]);
  m = block_max_256(m, red);
  const float s = m / 127.0f;  // IEEE division
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  for (long c = (long)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (long)gridDim.x * 256) {
    u32x2 o = {0u, 0u};
    if (s > 0.f) {
      float f[8];
      bf16x8_to_f32(reinterpret_cast<const u32x4*>(X)[c], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float q = fminf(fmaxf(__builtin_rintf(f[j] / s), -127.f), 127.f);
        o[j >> 2] |= ((uint32_t)((int)q) & 0xFFu) << (8 * (j & 3));
      }
    }
    reinterpret_cast<u32x2*>(X8)[c] = o;
  }
}

// E2M1 (OCP FP4) codes of two non-negative floats in one byte (first value in
// the low nibble), through the hardware conversion (scale 1); values above
// the largest code's 6 are clamped to it first.
__device__ __forceinline__ uint32_t e2m1x2_into(uint32_t word, float a, float b, int byte) {
  a = fminf(a, 6.f);
  b = fminf(b, 6.f);
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, 3);
  }
}

// eight values per thread packed into one dword through bytes 0 .. 3 in
// turn, as the P operand is packed, then unpacked one code per byte
__global__ __launch_bounds__(256) void debug_cvt_e2m1_kernel(const float* __restrict__ x, uint8_t* __restrict__ y,
                                                             long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (8 * i + 7 < n) {
    const float* xi = x + 8 * i;
    uint32_t w = e2m1x2_into(0u, xi[0], xi[1], 0);
    w = e2m1x2_into(w, xi[2], xi[3], 1);
    w = e2m1x2_into(w, xi[4], xi[5], 2);
    w = e2m1x2_into(w, xi[6], xi[7], 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) y[8 * i + j] = (w >> (4 * j)) & 0xFu;
  }
}

__global__ __launch_bounds__(256) void debug_cvt_e4m3_kernel(const float* __restrict__ x, uint8_t* __restrict__ y, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (2 * i + 1 < n) {
    const uint32_t r = e4m3x4_sat(x[2 * i], x[2 * i + 1], 0.f, 0.f);
    y[2 * i] = r & 0xFFu;
    y[2 * i + 1] = (r >> 8) & 0xFFu;
  }
}

// ------------------------------------------------ rotated block quantisation
// One row (d = 128) of the unnormalised Walsh-Hadamard transform of x * sigma
// in fp32, held by 16 lanes: lane j of the group holds elements 8j .. 8j+7.
// Butterflies (lo, hi) -> (lo + hi, lo - hi) at element strides 1, 2, 4
// (inside the lane), then 8, 16, 32, 64 (lane strides 1, 2, 4, 8: DPP quad
// permutes, a 32-lane swizzle and a 16-lane rotation by 8), in that order.
// Without rotation the row is returned as read.
template <int CTRL>
__device__ __forceinline__ void butterfly_x(float* y, bool hi) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float p;
    if constexpr (CTRL < 0)
      p = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, y[e]), -CTRL));
    else
      p = dppq<CTRL>(y[e]);
    const float lo = y[e] + p, hv = p - y[e];
    y[e] = hi ? hv : lo;
  }
}

__device__ __forceinline__ void fwht_row128_x16(u32x4 u, const float* sg, bool rot, int j, float* y) {
  bf16x8_to_f32(u, y);
  if (!rot) return;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] *= sg[e];  // exact: the signs are +-1
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!(e & h)) {
        const float lo = y[e], hi = y[e + h];
        y[e] = lo + hi;
        y[e + h] = lo - hi;
      }
  butterfly_x<0xB1>(y, (j & 1) != 0);      // lane xor 1 (quad_perm 1,0,3,2)
  butterfly_x<0x4E>(y, (j & 2) != 0);      // lane xor 2 (quad_perm 2,3,0,1)
  butterfly_x<-0x101F>(y, (j & 4) != 0);   // lane xor 4 (swizzle, bit mode)
  butterfly_x<0x128>(y, (j & 8) != 0);     // lane xor 8 (row rotate by 8)
}

// Workgroup = one block of up to R consecutive rows of one head, four rows
// per wave at a time; pass 1 finds the block's max |y|, pass 2 recomputes the
// (deterministic) transform and writes E4M3(y / s), s = max / 448 (IEEE fp32
// division); every row of the block stores s * post (post = 1 / sqrt(d) when
// rotating, else 1).
__global__ __launch_bounds__(256) void rotate_quantize_e4m3_kernel(const uint16_t* __restrict__ X,
                                                                   const float* __restrict__ signs,
                                                                   uint8_t* __restrict__ X8, float* __restrict__ S,
                                                                   int N, int R, int nblk, float post) {
  __shared__ float red[4];
  const int bh = blockIdx.x / nblk, blk = blockIdx.x - bh * nblk;
  const int r0 = blk * R, r1 = min(N, r0 + R);
  const int tid = threadIdx.x, j = tid & 15, rg = tid >> 4;  // 16 row slots per pass
  const bool rot = signs != nullptr;
  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = rot ? signs[8 * j + e] : 1.f;
  const uint16_t* Xh = X + (size_t)bh * N * 128;
  float amax = 0.f;
  // every lane runs the same trip count (the cross-lane steps need the whole
  // row group); rows past the block read as zero and are not stored
  const int npass = (r1 - r0 + 15) / 16;
  for (int it = 0; it < npass; ++it) {
    const int r = r0 + 16 * it + rg;
    const u32x4 u = r < r1 ? reinterpret_cast<const u32x4*>(Xh + (size_t)r * 128)[j] : u32x4{0u, 0u, 0u, 0u};
    float y[8];
    fwht_row128_x16(u, sg, rot, j, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
  }
  amax = block_max_256(amax, red);
  const float sc = amax / 448.0f;
  const float stored = rot ? sc * post : sc;
  for (int r = r0 + tid; r < r1; r += 256) S[(size_t)bh * N + r] = stored;
  uint8_t* X8h = X8 + (size_t)bh * N * 128;
  for (int it = 0; it < npass; ++it) {
    const int r = r0 + 16 * it + rg;
    const u32x4 u = r < r1 ? reinterpret_cast<const u32x4*>(Xh + (size_t)r * 128)[j] : u32x4{0u, 0u, 0u, 0u};
    float y[8];
    fwht_row128_x16(u, sg, rot, j, y);
    u32x2 c = {0u, 0u};
    if (sc > 0.f) {
      c[0] = e4m3x4_sat(y[0] / sc, y[1] / sc, y[2] / sc, y[3] / sc);
      c[1] = e4m3x4_sat(y[4] / sc, y[5] / sc, y[6] / sc, y[7] / sc);
    }
    if (r < r1) reinterpret_cast<u32x2*>(X8h + (size_t)r * 128)[j] = c;
  }
}

// ------------------------------------------------------------ quantised tiles
struct Q8Cfg {
  static constexpr int D = 128, BM = 128, BN = 64, NT = 256;  // 4 waves of 32 query rows
  static constexpr int ROWB = D;                 // bytes per K8 / V8 row
  static constexpr int SPR = ROWB / 16;          // 16-byte slots per row
  static constexpr int TILEB = BN * ROWB;        // bytes per K8 or V8 tile
  static constexpr int KBUF = TILEB + BN * 4;    // K8 tile followed by its 64 key scales
  static constexpr int RPI = 1024 / ROWB;        // rows per 1 KB wave load
  static constexpr int LPW = TILEB / 1024 / 4;   // 1 KB loads per K8 or V8 tile for each wave
  static constexpr int KSTEPS = D / 32;          // int8 k-steps per 32-key block
  static constexpr int MB_O = D / 32;            // 32-row blocks of O^T
};

// Key order of a score tile.  The K8 tile is staged so that row 8g + 4h + r
// of score block nb holds tile key 32h + 16nb + 4g + r: score s[nb][i] of a
// lane in half h is then key 32h + 16nb + i, i.e. each lane half holds the 32
// consecutive keys 32h .. 32h+31 (one scale block of the fp4 P operand).  P^T
// byte (or nibble) j of lane half h is key 32h + j, which is the V row the
// transposing V^T read of that half returns at position j, so V rows are
// staged in key order.
// The mixed fp8 x fp4 MFMA pairs its operands by K index, and the two
// formats lay K out differently: fp4 element j of lane half h is K = 32h + j
// (the P nibbles, key 32h + j as above), fp8 element j of lane half h is
// K = 16h + j for j < 16 and 32 + 16h + (j - 16) for j >= 16.  For P in fp4
// the V row of tile key kt is therefore staged at the LDS row whose
// transposed read lands on the fp8 element with K index kt.
__device__ __forceinline__ int score_key(int nb, int i, int h) { return 32 * h + 16 * nb + i; }

// tile key held by LDS row R of a K8 tile: row 8g + 4h + r of score block nb
// holds key 32h + 16nb + 4g + r
__device__ __forceinline__ int k8_row_key(int R) {
  return 32 * ((R >> 2) & 1) + 16 * (R >> 5) + 4 * ((R >> 3) & 3) + (R & 3);
}
// tile key held by LDS row R of a V8 tile: R itself, or for FP4 P the key
// whose fp8 K index the transposed read of row R lands on
template <bool P4>
__device__ __forceinline__ int v8_row_key(int R) {
  if (!P4) return R;
  return ((R >> 4) & 1) ? 32 + 16 * (R >> 5) + (R & 15) : 16 * (R >> 5) + (R & 15);
}
// slot swizzles: the K operand reads (16 lanes read one slot of 16 consecutive
// rows) and the transposing V reads (16 lanes read 16 bytes of 8 consecutive
// rows) then hit distinct banks
__device__ __forceinline__ int k8_swz(int R) { return (R >> 1) & 7; }
__device__ __forceinline__ int v8_swz(int R) { return (R >> 1) & 3; }

// direct global -> LDS loads: lane i's BYTES bytes at voff land at dst + BYTES i
__device__ __forceinline__ void q8_load_lds16(const __amdgpu_buffer_rsrc_t& r, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void q8_load_lds4(const __amdgpu_buffer_rsrc_t& r, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)dst, 4, voff, 0, 0, 0);
}

// S^T of one 64-key K8 tile held in LDS against the lane's query: acc[nb][i]
// is the score of tile key score_key(nb, i, h), exact int32 (F8 false; |S| <=
// 127^2 d < 2^24) or fp32 from E4M3 codes (F8 true: each fp8 step contracts
// 64 of d, its operands two int8-form 32-wide chunks side by side, A and B
// paired byte for byte).  ka_off[kk]: the lane's byte offset of int8 k-step kk
// in key block 0; qop[kk]: Q8[qrow][32kk + 16h .. +15].
template <bool F8>
__device__ __forceinline__ void qk_tile(const char* lk, const i32x4* qop, const uint32_t* ka_off,
                                        typename std::conditional<F8, f32x16, i32x16>::type* acc) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    acc[nb] = {};
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < Q8Cfg::KSTEPS / 2; ++j) {
        const i32x4 a0 = lds_load<i32x4>(lk, ka_off[2 * j] + nb * 32 * Q8Cfg::ROWB);
        const i32x4 a1 = lds_load<i32x4>(lk, ka_off[2 * j + 1] + nb * 32 * Q8Cfg::ROWB);
        const i32x4 b0 = qop[2 * j], b1 = qop[2 * j + 1];
        const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[nb], 0, 0, 0, 127, 0, 127);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < Q8Cfg::KSTEPS; ++kk) {
        const i32x4 a = lds_load<i32x4>(lk, ka_off[kk] + nb * 32 * Q8Cfg::ROWB);
        acc[nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qop[kk], acc[nb], 0, 0, 0);
      }
    }
  }
}

// rint(127 p) of four probabilities p in [0, 1] as bytes (P's scale is the
// constant 1/127 in the all-INT8 variant)
__device__ __forceinline__ uint32_t p_u8x4(float a, float b, float c, float d) {
  const uint32_t x0 = (uint32_t)__builtin_rintf(127.f * a), x1 = (uint32_t)__builtin_rintf(127.f * b);
  const uint32_t x2 = (uint32_t)__builtin_rintf(127.f * c), x3 = (uint32_t)__builtin_rintf(127.f * d);
  return x0 | (x1 << 8) | (x2 << 16) | (x3 << 24);
}

// VAR (QVariant): kInt8Scores -- int8 scores, E4M3 P . V; kAllInt8 -- I8V
// below; kFp8 -- E4M3 Q8/K8 and the scores on the fp8 MFMA, P . V as in
// kInt8Scores; kFp8P4 -- kFp8 with P in MXFP4.
// Every variant raises the running max on every increase (no lazy
// threshold), so P = exp2(s - m_running) <= 1 when it is quantised and the
// row's largest probability is cast as exactly 1; a lazy threshold would cast
// P * 2^delta for a fractional delta and put up to half an E4M3 step of error
// on the dominant key of a peaked row.
// I8V: the all-INT8 variant -- V8 holds per-tensor int8 codes and P . V runs
// on the int8 MFMA: P is quantised as rint(127 P) (P <= 1 as above); each
// 64-key tile is two 32-key int8 steps whose operands are the two halves of
// the E4M3 form's (same key order), and the exact int32 tile product is
// added into the fp32 accumulator (a float rescale of an int32 running sum
// would not be exact).
// The forward: 4 waves of 32 query rows per workgroup, three workgroups per
// CU.  Tile t+1 (K8 rows and scales, V8 rows) is requested at the start of
// tile t into the other LDS buffer, one barrier per tile.  Each wave runs
// S(t), the softmax and O += P(t) V(t) in turn; the workgroups' waves on a
// SIMD interleave their matrix and vector work.
template <bool CAUSAL, int VAR>
__global__ __launch_bounds__(256, 3) void prefill_q8_kernel(
    const int8_t* __restrict__ Q8, const int8_t* __restrict__ K8, const uint8_t* __restrict__ V8,
    const float* __restrict__ QS, const float* __restrict__ KS, const float* __restrict__ VS,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Nq, int Nk, float c, int nqb, int total) {
  using C = Q8Cfg;
  constexpr int BM = C::BM, LPW = C::LPW;
  constexpr bool I8V = VAR == (int)QVariant::kAllInt8;
  constexpr bool P4 = VAR == (int)QVariant::kFp8P4;
  constexpr bool F8QK = VAR == (int)QVariant::kFp8 || P4;
  using SAcc = typename std::conditional<F8QK, f32x16, i32x16>::type;
  __shared__ __attribute__((aligned(1024))) char k0s[C::KBUF];
  __shared__ __attribute__((aligned(1024))) char k1s[C::KBUF];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILEB];

  const int logical = xcd_remap(blockIdx.x, total);
  const int bh = logical / nqb;
  int qb = logical - bh * nqb;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest blocks first
  const int q0 = qb * BM;
  const int off = Nk - Nq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const size_t qbase = (size_t)bh * Nq, kbase = (size_t)bh * Nk;
  const auto rk = make_rsrc(K8 + kbase * C::D, (uint32_t)Nk * C::D);
  const auto rv = make_rsrc(V8 + kbase * C::D, (uint32_t)Nk * C::D);
  const auto rs = make_rsrc(KS + kbase, (uint32_t)Nk * 4);

  // wave w fills 1 KB blocks LPW w .. LPW w + LPW-1 of each tile: lane i lands
  // at LDS row R = block RPI + i / SPR, slot i % SPR, so it fetches the row's
  // key and the chunk that slot holds under the swizzle
  uint32_t gk_off[LPW], gv_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int R = (LPW * w + i) * C::RPI + lane / C::SPR, slot = lane % C::SPR;
    gk_off[i] = (uint32_t)k8_row_key(R) * C::ROWB + 16 * (slot ^ k8_swz(R));
    gv_off[i] = (uint32_t)v8_row_key<P4>(R) * C::ROWB + 16 * (slot ^ v8_swz(R));
  }
  // tile t: K8 rows and scales into ldk, V8 rows into ldv (keys past Nk read as 0)
  auto issue_tile = [&](int t, char* ldk, char* ldv) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      q8_load_lds16(rk, ldk + 1024 * (LPW * w + i), (uint32_t)t * C::TILEB + gk_off[i]);
      q8_load_lds16(rv, ldv + 1024 * (LPW * w + i), (uint32_t)t * C::TILEB + gv_off[i]);
    }
    if (w == 0) q8_load_lds4(rs, ldk + C::TILEB, (uint32_t)(t * C::BN + lane) * 4);
  };
  // K operand: row l32 (+32 per key block), logical slot 2kk + h
  uint32_t ka_off[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) ka_off[kk] = l32 * C::ROWB + 16 * ((2 * kk + h) ^ k8_swz(l32));
  // V^T operand of d block mb: read r (0..3) covers rows 32h + 8r + r16/2,
  // bytes 32mb + 16g1 + 8(r16&1) .. +7 of the unswizzled row
  const int r16 = lane & 15, g1 = (lane >> 4) & 1;
  auto vt_load = [&](const char* lv, int mb) {
    i32x8 a;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int R = 32 * h + 8 * r + (r16 >> 1);
      const uint32_t addr = R * C::ROWB + 16 * ((2 * mb + g1) ^ v8_swz(R)) + 8 * (r16 & 1);
      const i32x2 x = lds_read_tr8(lv, addr);
      a[2 * r] = x[0];
      a[2 * r + 1] = x[1];
    }
    return a;
  };

  const int qmin_w = q0 + 32 * w;
  const int qrow = qmin_w + l32;
  i32x4 qop[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    i32x4 x = {0, 0, 0, 0};
    if (qrow < Nq) x = reinterpret_cast<const i32x4*>(Q8 + (qbase + qrow) * C::D)[2 * kk + h];
    qop[kk] = x;
  }
  // query scale x softmax scale x log2 e, applied in the exponent's FMA; kept
  // positive (a zero query row has zero scores) so masked -inf scores stay -inf
  const float cq = fmaxf((qrow < Nq ? QS[qbase + qrow] : 0.f) * c, FLT_MIN);

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + BM, Nq) - 1 + off + 1);
  const int T = max(0, (kv_end + C::BN - 1) / C::BN);

  f32x16 o[C::MB_O];
#pragma unroll
  for (int mb = 0; mb < C::MB_O; ++mb) o[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto tile = [&](int t, const char* lk, const char* lv, char* ldk, char* ldv) {
    if (t + 1 < T) issue_tile(t + 1, ldk, ldv);
    const int kv0 = t * C::BN;
    if (CAUSAL && kv0 > qmin_w + 31 + off) return;  // no key of the tile is visible to this wave
    // S(t), scaled per key: s[nb][i] belongs to tile key 32h + 16nb + i
    f32x16 s[2];
    {
      SAcc acc[2];
      qk_tile<F8QK>(lk, qop, ka_off, acc);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 ks4 = lds_load<f32x4>(lk, C::TILEB + (32 * h + 16 * nb + 4 * g) * 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) s[nb][4 * g + j] = (float)acc[nb][4 * g + j] * ks4[j];
        }
    }
    if ((kv0 + C::BN > Nk) || (CAUSAL && kv0 + C::BN - 1 > qmin_w + off)) {
      // keys past Nk or past the causal diagonal: -inf, as a bit blend (see prefill.hip)
      const int lim = min(Nk - 1, CAUSAL ? qrow + off : Nk - 1) - (kv0 + 32 * h);
      constexpr uint32_t kNegInf = 0xFF800000u;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t hide = (uint32_t)((lim - (16 * nb + i)) >> 31);
          const float v = s[nb][i];
          const uint32_t bits = __builtin_bit_cast(uint32_t, v);
          s[nb][i] = __builtin_bit_cast(float, (bits & ~hide) | (kNegInf & hide));
        }
    }
    float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mt = fmaxf(mt, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[1][i]);
    const float mloc = mt;  // max over this lane's 32 keys (one MX block)
    mt = pair_max(mt) * cq;
    if (__any(mt > m_run)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
      for (int mb = 0; mb < C::MB_O; ++mb) o[mb] *= alpha;
      l_run *= alpha;
      m_run = mn;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    // MXFP4: the lane's 32 keys share 2^e, e = floor(max log2 P) - 2, so the
    // largest P / 2^e lies in [4, 8) (E8M0 byte e + 127 for the MFMA).  The
    // block max is the same rounded product the running max came from, with
    // contraction off (a fused multiply-add's residual just below 0 would take
    // e one binade too low)
    int e_mx = -127;
    float inv_mx = 0.f;
    if constexpr (P4) {
      float tmax;
      {
#pragma clang fp contract(off)
        tmax = mloc * cq - m_use;
      }
      if (tmax != -INFINITY) e_mx = max(-127, (int)floorf(tmax) - 2);
      inv_mx = __builtin_bit_cast(float, (uint32_t)(127 - e_mx) << 23);
    }
    i32x8 pb;
    float lsum = 0.f;
#pragma unroll
    for (int jw = 0; jw < 8; ++jw) {
      const int nb = jw >> 2, i0 = 4 * (jw & 3);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[nb][i0 + 0], cq, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[nb][i0 + 1], cq, -m_use));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(s[nb][i0 + 2], cq, -m_use));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(s[nb][i0 + 3], cq, -m_use));
      lsum += (p0 + p1) + (p2 + p3);
      if constexpr (P4) {
        // nibbles 4jw .. 4jw+3: dword jw / 2, bytes 2 (jw % 2) and 2 (jw % 2) + 1
        const uint32_t prev = (jw & 1) ? (uint32_t)pb[jw >> 1] : 0u;
        uint32_t wd = e2m1x2_into(prev, p0 * inv_mx, p1 * inv_mx, 2 * (jw & 1));
        wd = e2m1x2_into(wd, p2 * inv_mx, p3 * inv_mx, 2 * (jw & 1) + 1);
        pb[jw >> 1] = (int)wd;
      } else {
        pb[jw] = I8V ? (int)p_u8x4(p0, p1, p2, p3) : (int)e4m3x4(p0, p1, p2, p3);
      }
    }
    if constexpr (P4) {
#pragma unroll
      for (int k = 4; k < 8; ++k) pb[k] = 0;
    }
    l_run += lsum;
#pragma unroll
    for (int mb = 0; mb < C::MB_O; ++mb) {
      const i32x8 a = vt_load(lv, mb);
      if constexpr (I8V) {
        i32x16 acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{a[0], a[1], a[2], a[3]},
                                                           i32x4{pb[0], pb[1], pb[2], pb[3]}, i32x16{}, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{a[4], a[5], a[6], a[7]},
                                                    i32x4{pb[4], pb[5], pb[6], pb[7]}, acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 16; ++j) o[mb][j] += (float)acc[j];  // |acc| < 64 * 127^2 < 2^24: exact
      } else if constexpr (P4) {
        o[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o[mb], 0, 4, 0, 127, 0, e_mx + 127);
      } else {
        o[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o[mb], 0, 0, 0, 127, 0, 127);
      }
    }
  };

  if (T > 0) issue_tile(0, k0s, v0s);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < T; t += 2) {
    tile(t, k0s, v0s, k1s, v1s);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < T) {
      tile(t + 1, k1s, v1s, k0s, v0s);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  const float l_tot = pair_sum(l_run);
  const float f = l_tot > 0.f ? (I8V ? *VS / (127.f * l_tot) : *VS / l_tot) : 0.f;
  if (qrow < Nq) {
    uint16_t* dst = O + (qbase + qrow) * C::D;
#pragma unroll
    for (int mb = 0; mb < C::MB_O; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2 x0 = Mfma<true>::pack2(o[mb][4 * g + 0] * f, o[mb][4 * g + 1] * f);
        const bf16x2 x1 = Mfma<true>::pack2(o[mb][4 * g + 2] * f, o[mb][4 * g + 3] * f);
        u32x2 u;
        u[0] = __builtin_bit_cast(uint32_t, x0);
        u[1] = __builtin_bit_cast(uint32_t, x1);
        *reinterpret_cast<u32x2*>(dst + 32 * mb + 8 * g + 4 * h) = u;
      }
    if (LSE != nullptr && h == 0) LSE[qbase + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// Test hooks: the scores of one head through the forward's own tile routine
// and LDS layout, exact int32 (F8 false) or fp32 from E4M3 codes (F8
// true).  One workgroup of 4 waves per (128 queries, 64 keys).
template <bool F8>
__global__ __launch_bounds__(256) void debug_qk_kernel(const int8_t* __restrict__ Q8, const int8_t* __restrict__ K8,
                                                       void* __restrict__ Sv, int Nq, int Nk) {
  using C = Q8Cfg;
  __shared__ __attribute__((aligned(1024))) char lk[C::KBUF];
  const int q0 = blockIdx.x * C::BM, kv0 = blockIdx.y * C::BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int qrow = q0 + 32 * w + l32;
  const auto rk = make_rsrc(K8, (uint32_t)Nk * C::D);
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 8 KB tile: 2 loads of 1 KB per wave
    const int R = (2 * w + i) * C::RPI + lane / C::SPR, slot = lane % C::SPR;
    q8_load_lds16(rk, lk + 1024 * (2 * w + i),
                  (uint32_t)(kv0 + k8_row_key(R)) * C::ROWB + 16 * (slot ^ k8_swz(R)));
  }
  i32x4 qop[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    i32x4 x = {0, 0, 0, 0};
    if (qrow < Nq) x = reinterpret_cast<const i32x4*>(Q8 + (size_t)qrow * C::D)[2 * kk + h];
    qop[kk] = x;
  }
  uint32_t ka_off[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) ka_off[kk] = l32 * C::ROWB + 16 * ((2 * kk + h) ^ k8_swz(l32));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  using Acc = typename std::conditional<F8, f32x16, i32x16>::type;
  using Out = typename std::conditional<F8, float, int32_t>::type;
  Acc acc[2];
  qk_tile<F8>(lk, qop, ka_off, acc);
  Out* S = static_cast<Out*>(Sv);
  if (qrow < Nq) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kv0 + score_key(nb, i, h);
        if (key < Nk) S[(size_t)qrow * Nk + key] = acc[nb][i];
      }
  }
}

}  // namespace

hipError_t launch_quantize_rows_i8(const void* x, int8_t* x8, float* scales, long rows, int d, hipStream_t stream) {
  if (d == 128) {
    const long grid = (rows + 15) / 16;
    hipLaunchKernelGGL(quantize_rows_i8_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), x8, scales, rows);
  } else if (d == 64) {
    const long grid = (rows + 31) / 32;
    hipLaunchKernelGGL(quantize_rows_i8_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), x8, scales, rows);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_tensor_e4m3(const void* x, uint8_t* x8, float* scale_out, long n, void* workspace,
                                       hipStream_t stream) {
  const long chunks = n / 8;
  const int g = e4m3_partials(n);
  float* partial = static_cast<float*>(workspace);
  hipLaunchKernelGGL(amax_partial_kernel, dim3(g), dim3(256), 0, stream, static_cast<const uint16_t*>(x), chunks,
                     partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3(g), dim3(256), 0, stream, static_cast<const uint16_t*>(x), chunks,
                     partial, g, x8, scale_out);
  return hipGetLastError();
}

hipError_t launch_prefill_q8(const void* q8v, const void* k8v, const void* v8v, const float* q_scale,
                             const float* k_scale, const float* v_scale, void* out, float* lse, int B, int H, int Nq,
                             int Nk, int d, float scale, bool causal, QVariant variant, hipStream_t stream) {
  if (d != Q8Cfg::D) return hipErrorInvalidValue;
  const int nqb = (Nq + Q8Cfg::BM - 1) / Q8Cfg::BM;
  const int total = nqb * B * H;
  const int8_t* q8 = static_cast<const int8_t*>(q8v);
  const int8_t* k8 = static_cast<const int8_t*>(k8v);
  const uint8_t* v8 = static_cast<const uint8_t*>(v8v);
  const int var = (int)variant;
#define ATTN_Q8(CA_, VAR_)                                                                                     \
  if (causal == CA_ && var == VAR_)                                                                            \
    hipLaunchKernelGGL((prefill_q8_kernel<CA_, VAR_>), dim3(total), dim3(Q8Cfg::NT), 0, stream, q8, k8, v8,     \
                       q_scale, k_scale, v_scale, static_cast<uint16_t*>(out), lse, Nq, Nk, scale * kLog2e, nqb,   \
                       total);
  ATTN_Q8(true, 0)
  ATTN_Q8(false, 0)
  ATTN_Q8(true, 1)
  ATTN_Q8(false, 1)
  ATTN_Q8(true, 2)
  ATTN_Q8(false, 2)
  ATTN_Q8(true, 3)
  ATTN_Q8(false, 3)
#undef ATTN_Q8
  return hipGetLastError();
}

hipError_t launch_rotate_quantize_e4m3(const void* x, const float* signs, uint8_t* x8, float* scales, int BH, int N,
                                       int d, int block_rows, hipStream_t stream) {
  if (d != 128 || BH < 1 || N < 1 || block_rows < 1) return hipErrorInvalidValue;
  const int R = min(block_rows, N);
  const int nblk = (N + R - 1) / R;
  if ((long)BH * nblk > 0x7fffffffL) return hipErrorInvalidValue;
  const float post = (float)(1.0 / std::sqrt((double)d));
  hipLaunchKernelGGL(rotate_quantize_e4m3_kernel, dim3(BH * nblk), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), signs, x8, scales, N, R, nblk, post);
  return hipGetLastError();
}

hipError_t launch_quantize_tensor_i8(const void* x, int8_t* x8, float* scale_out, long n, void* workspace,
                                     hipStream_t stream) {
  const long chunks = n / 8;
  const int g = e4m3_partials(n);
  float* partial = static_cast<float*>(workspace);
  hipLaunchKernelGGL(amax_partial_kernel, dim3(g), dim3(256), 0, stream, static_cast<const uint16_t*>(x), chunks,
                     partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quantize_i8_tensor_kernel, dim3(g), dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                     chunks, partial, g, x8, scale_out);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const void* q8, const void* k8, void* s, int Nq, int Nk, int d, bool fp8,
                           hipStream_t stream) {
  if (d != Q8Cfg::D) return hipErrorInvalidValue;
  dim3 grid((Nq + Q8Cfg::BM - 1) / Q8Cfg::BM, (Nk + Q8Cfg::BN - 1) / Q8Cfg::BN);
  const int8_t* a = static_cast<const int8_t*>(q8);
  const int8_t* b = static_cast<const int8_t*>(k8);
  if (fp8)
    hipLaunchKernelGGL(debug_qk_kernel<true>, grid, dim3(256), 0, stream, a, b, s, Nq, Nk);
  else
    hipLaunchKernelGGL(debug_qk_kernel<false>, grid, dim3(256), 0, stream, a, b, s, Nq, Nk);
  return hipGetLastError();
}

hipError_t launch_debug_cvt_e2m1(const float* x, uint8_t* y, long n, hipStream_t stream) {
  const long groups = n / 8;
  hipLaunchKernelGGL(debug_cvt_e2m1_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

hipError_t launch_debug_cvt_e4m3(const float* x, uint8_t* y, long n, hipStream_t stream) {
  const long pairs = n / 2;
  hipLaunchKernelGGL(debug_cvt_e4m3_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

}  // namespace attn
