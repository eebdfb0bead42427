// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, MFMA wrappers, LDS address helpers, the XCD-aware workgroup
// order and wave-level reductions.  gfx950 (CDNA4) only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "seq_shape.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- MFMA
// Lane layouts (verified on gfx950), with l = lane, h = l / 32:
//   32x32x16 (bf16/f16): A lane holds A[m = l%32][k = 8h .. 8h+7],
//                        B lane holds B[k = 8h .. 8h+7][n = l%32],
//                        D element i holds D[8(i/4) + 4h + i%4][l%32].
// The int8 32x32x32 and fp8 32x32x64 forms use the same m/n/D layout and
// the same k-order for A and B.

template <bool BF16> struct Mfma;
template <> struct Mfma<true> {
  typedef bf16x8 op8;
  typedef bf16x2 op2;
  static __device__ __forceinline__ f32x16 mma(op8 a, op8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ op2 pack2(float x, float y) {
    op2 r; r[0] = (__bf16)x; r[1] = (__bf16)y; return r;   // v_cvt_pk_bf16_f32, RNE
  }
  static __device__ __forceinline__ float dot2(op2 a, op2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};
template <> struct Mfma<false> {
  typedef f16x8 op8;
  typedef f16x2 op2;
  static __device__ __forceinline__ f32x16 mma(op8 a, op8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ op2 pack2(float x, float y) {
    op2 r; r[0] = (_Float16)x; r[1] = (_Float16)y; return r;  // v_cvt_pk_f16_f32, RNE
  }
  static __device__ __forceinline__ float dot2(op2 a, op2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
};

// ---------------------------------------------------------------- LDS
template <class T>
__device__ __forceinline__ T lds_load(const char* base, uint32_t byte_off) {
  return *(const ATTN_LDS T*)((const ATTN_LDS char*)(base) + byte_off);
}
template <class T>
__device__ __forceinline__ void lds_store(char* base, uint32_t byte_off, T v) {
  *(ATTN_LDS T*)((ATTN_LDS char*)(base) + byte_off) = v;
}
// Transposing 64-bit LDS read (gfx950 ds_read_b64_tr_b16).  In each group of
// 16 lanes, lane r supplies the address of 4 consecutive 16-bit elements; the
// result of lane i is element (i % 4) of the chunks supplied by lanes
// i/4, 4 + i/4, 8 + i/4, 12 + i/4.  Pointing lane r at row (r/4), columns
// 4(r%4)..4(r%4)+3 of a 4 x 16 block therefore hands lane i column i, rows
// 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const char* base, uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS s16x4*)((ATTN_LDS char*)(base) + byte_off));
}

// ---------------------------------------------------------------- waves
// Transposing 64-bit LDS read of 8-bit elements (ds_read_b64_tr_b8): in each
// group of 16 lanes, pointing lane r at row (r/2), columns 8(r%2)..8(r%2)+7
// of an 8 x 16 block hands lane i column i, rows 0..7.
__device__ __forceinline__ i32x2 lds_read_tr8(const char* base, uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS i32x2*)((ATTN_LDS char*)(base) + byte_off));
}

// Reductions over the lane pair (l, l ^ 32) with v_permlane32_swap: the two
// results of the swap are the lane's own value and its partner's (in some
// order), so a symmetric operation on them is the pair reduction.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)s[0]), __builtin_bit_cast(float, (unsigned)s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)s[0]) + __builtin_bit_cast(float, (unsigned)s[1]);
}

// ---------------------------------------------------------------- buffers
// Raw buffer resource over `bytes` bytes at `base`: loads at offsets at or
// beyond `bytes` return zero (hardware range check), which is how the
// kernels read tail rows without branches.  Offsets are 32-bit, so one
// resource covers less than 2 GiB (checked on the host).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// scheduling-group masks for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedValu = 0x002, kSchedDsRead = 0x100, kSchedDsWrite = 0x200,
              kSchedVmemRead = 0x020;

// ---------------------------------------------------------------- sequences
// The rows of one (sequence, head) in the dense or packed layout (SeqShape).
struct SeqSpan {
  size_t q_row0, k_row0;  // first Q/O/LSE row and first K/V row of the (sequence, head)
  int nq, nk;             // its query and key counts
};
__device__ __forceinline__ SeqSpan seq_span(const SeqShape& a, int s, int h) {
  SeqSpan r;
  const int hk = h / a.group;
  if (a.cu_q != nullptr) {
    // offsets clamped into [0, total] and made non-decreasing, so malformed
    // offsets can only select wrong rows of this head, never memory outside it
    const int qa = min(max(a.cu_q[s], 0), a.Nq), ka = min(max(a.cu_k[s], 0), a.Nk);
    r.nq = min(max(a.cu_q[s + 1], qa), a.Nq) - qa;
    r.nk = min(max(a.cu_k[s + 1], ka), a.Nk) - ka;
    r.q_row0 = (size_t)h * a.Nq + qa;
    r.k_row0 = (size_t)hk * a.Nk + ka;
  } else {
    r.nq = a.Nq;
    r.nk = a.Nk;
    r.q_row0 = ((size_t)s * a.H + h) * a.Nq;
    r.k_row0 = ((size_t)s * (a.H / a.group) + hk) * a.Nk;
  }
  return r;
}

// ---------------------------------------------------------------- grid order
// Workgroups are handed to the 8 XCDs round robin (id % 8).  Renumber them so
// each XCD receives one contiguous range of logical work items; neighbouring
// items share K/V in that XCD's L2.  Bijective for any total.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

}  // namespace attn
