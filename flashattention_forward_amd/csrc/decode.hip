// Split-KV decode forward for gfx950 (one query per (batch, head)).
//
// With a single query the work is one pass over K and V (about one FLOP per
// byte), so the kernel is built for HBM streaming, not for MFMA: the keys of
// each (batch, head) are cut into `splits` contiguous ranges, one workgroup
// per range, and every lane streams 16-byte pieces of K and V rows
// (d/8 lanes cover one row, so each wave load is fully coalesced).
//
// Inside a workgroup every group of d/8 lanes keeps its own online-softmax
// state (running max m, running sum l, an fp32 accumulator for its 8 columns
// of O) over the rows it reads -- the recurrence of "The Flash Attention
// algorithm" (marketmaker.cc post "Can a full trading day of context beat one
// minute? Flash attention and the sequence-length question") applied to a
// single query row.  Dot products are reduced across the d/8 lanes with DPP
// and swizzle steps (no LDS).  At the end the states of the workgroup are
// merged through LDS and the range's normalised partial output O_s and its
// log-sum-exp LSE_s are written to the workspace.
//
// A second kernel merges the ranges: LSE = M + ln sum_s exp(LSE_s - M),
// O = sum_s exp(LSE_s - LSE) O_s -- the same running-statistics update
// applied to states over disjoint key ranges.
#include "common.h"
#include "internal.h"

namespace attn {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 8;  // row loads in flight per lane per step (x2 for K and V)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 8 or 16); every lane gets the sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  if (G == 16) {
    x += dpp<0x124>(x);  // row_ror:4
    x += dpp<0x128>(x);  // row_ror:8
  } else {
    // xor 4 within 32-lane halves (bitmask swizzle: and 0x1F, xor 4)
    x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x101F));
  }
  return x;
}

__device__ __forceinline__ void widen8(u32x4 u, bool bf16, float* f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = u[j];
    if (bf16) {
      f[2 * j] = __builtin_bit_cast(float, w << 16);
      f[2 * j + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
    } else {
      const f16x2 hv = __builtin_bit_cast(f16x2, w);
      f[2 * j] = (float)hv[0];
      f[2 * j + 1] = (float)hv[1];
    }
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ Opart, float* __restrict__ Lpart, int Nk, float c, int splits, int H, int group) {
  constexpr int LPR = D / 8;            // lanes per K/V row
  constexpr int RPW = 64 / LPR;         // rows per wave load
  constexpr int NW = kDecThreads / 64;  // waves
  constexpr int NS = NW * RPW;          // partial states per workgroup
  constexpr int KCW = RPW * kDecUnroll; // keys per wave step
  __shared__ float st_m[NS], st_l[NS];
  __shared__ float st_o[NS][D];

  const int bh = blockIdx.x / splits, split = blockIdx.x - bh * splits;
  const int s0 = (int)(((long)split * Nk) / splits), s1 = (int)(((long)(split + 1) * Nk) / splits);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = lane / LPR, ch = lane % LPR;
  // query head bh % H of batch bh / H reads K/V head (bh % H) / group
  const size_t kbase = ((size_t)(bh / H) * (H / group) + (bh % H) / group) * Nk * D;

  float q[8];
  widen8(reinterpret_cast<const u32x4*>(Q + (size_t)bh * D)[ch], BF16, q);

  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  for (int base = s0 + w * KCW; base < s1; base += NW * KCW) {
    u32x4 kr[kDecUnroll], vr[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int key = base + u * RPW + row;
      kr[u] = u32x4{0u, 0u, 0u, 0u};
      vr[u] = u32x4{0u, 0u, 0u, 0u};
      if (key < s1) {
        kr[u] = reinterpret_cast<const u32x4*>(K + kbase + (size_t)key * D)[ch];
        vr[u] = reinterpret_cast<const u32x4*>(V + kbase + (size_t)key * D)[ch];
      }
    }
    float s[kDecUnroll];
    float mc = -INFINITY;
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float kf[8];
      widen8(kr[u], BF16, kf);
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) d = fmaf(q[j], kf[j], d);
      d = group_sum<LPR>(d);
      const int key = base + u * RPW + row;
      s[u] = key < s1 ? d * c : -INFINITY;
      mc = fmaxf(mc, s[u]);
    }
    const float mn = fmaxf(m, mc);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mref);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    m = mn;
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const float p = __builtin_amdgcn_exp2f(s[u] - mref);
      l += p;
      float vf[8];
      widen8(vr[u], BF16, vf);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(p, vf[j], acc[j]);
    }
  }

  // merge the NS states of this workgroup
  const int g = w * RPW + row;
  if (ch == 0) {
    st_m[g] = m;
    st_l[g] = l;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) st_o[g][8 * ch + j] = acc[j];
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
    for (int i = 0; i < NS; ++i) M = fmaxf(M, st_m[i]);
    float L = 0.f, o = 0.f;
    for (int i = 0; i < NS; ++i) {
      const float wgt = st_m[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st_m[i] - M);
      L = fmaf(st_l[i], wgt, L);
      o = fmaf(st_o[i][tid], wgt, o);
    }
    const size_t ps = (size_t)bh * splits + split;
    Opart[ps * D + tid] = o / L;
    if (tid == 0) Lpart[ps] = (M + __log2f(L)) * kLn2;
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ Opart,
                                                         const float* __restrict__ Lpart,
                                                         uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                         int splits) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* lp = Lpart + (size_t)bh * splits;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, lp[s]);
  float tot = 0.f;
  for (int s = 0; s < splits; ++s) tot += __expf(lp[s] - M);
  const float lse = M + __logf(tot);
  float o = 0.f;
  const float* op = Opart + (size_t)bh * splits * D + d;
  for (int s = 0; s < splits; ++s) o = fmaf(__expf(lp[s] - lse), op[(size_t)s * D], o);
  uint16_t bits;
  if (BF16) bits = __builtin_bit_cast(uint16_t, (__bf16)o);
  else bits = __builtin_bit_cast(uint16_t, (_Float16)o);
  O[(size_t)bh * D + d] = bits;
  if (LSE != nullptr && d == 0) LSE[bh] = lse;
}

template <int D, bool BF16>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                           int Hkv, int Nk, float scale, int splits, void* workspace, hipStream_t stream) {
  float* opart = static_cast<float*>(workspace);
  float* lpart = opart + (size_t)B * H * splits * D;
  hipLaunchKernelGGL((decode_partial_kernel<D, BF16>), dim3(B * H * splits), dim3(kDecThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), opart, lpart, Nk, scale * kLog2e, splits, H, H / Hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, BF16>), dim3(B * H), dim3(D), 0, stream, opart, lpart,
                     static_cast<uint16_t*>(out), lse, splits);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int d, int splits) {
  return (size_t)B * H * splits * (d + 1) * sizeof(float);
}

int decode_default_splits(int B, int H, int Nk, int d) {
  (void)d;
  // aim for about 8192 workgroups (32 per CU) with at least 128 keys each
  long bh = (long)B * H;
  int s = 1;
  while (bh * s < 8192 && s < 256 && (long)(s * 2) * 128 <= Nk) s *= 2;
  return s;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv,
                         int Nk, int d, float scale, bool bf16, int splits, void* workspace, hipStream_t stream) {
  if (d == 128 && bf16)
    return launch_decode_t<128, true>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  if (d == 128 && !bf16)
    return launch_decode_t<128, false>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  if (d == 64 && bf16)
    return launch_decode_t<64, true>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  if (d == 64 && !bf16)
    return launch_decode_t<64, false>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
