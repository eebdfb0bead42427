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

// HG query heads that share one K/V head are served by one workgroup: every
// K and V row is read and widened once and used for all HG queries, each with
// its own online-softmax state (grouped-query attention raises the work per
// byte read by HG).  HG = 1 is plain multi-head attention.
template <int D, bool BF16, int HG>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ Opart, float* __restrict__ Lpart, int Nk, float c, int splits, int H, int group) {
  constexpr int LPR = D / 8;            // lanes per K/V row
  constexpr int RPW = 64 / LPR;         // rows per wave load
  constexpr int NW = kDecThreads / 64;  // waves
  constexpr int NS = NW * RPW;          // partial states per workgroup and head
  constexpr int UNR = HG >= 4 ? kDecUnroll / 2 : kDecUnroll;  // row loads in flight (registers)
  constexpr int KCW = RPW * UNR;        // keys per wave step
  __shared__ float st_m[NS], st_l[NS];
  __shared__ float st_o[NS][D];

  const int wgi = blockIdx.x / splits, split = blockIdx.x - wgi * splits;
  const int s0 = (int)(((long)split * Nk) / splits), s1 = (int)(((long)(split + 1) * Nk) / splits);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = lane / LPR, ch = lane % LPR;
  // query heads bh0 .. bh0 + HG-1 (one batch b, heads h0 ..) all read K/V head h0 / group
  const int bh0 = wgi * HG;
  const int b = bh0 / H, h0 = bh0 - b * H;
  const size_t kbase = ((size_t)b * (H / group) + h0 / group) * Nk * D;

  float q[HG][8];
#pragma unroll
  for (int g = 0; g < HG; ++g) widen8(reinterpret_cast<const u32x4*>(Q + (size_t)(bh0 + g) * D)[ch], BF16, q[g]);

  float m[HG], l[HG], acc[HG][8];
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
  }

  for (int base = s0 + w * KCW; base < s1; base += NW * KCW) {
    u32x4 kr[UNR], vr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int key = base + u * RPW + row;
      kr[u] = u32x4{0u, 0u, 0u, 0u};
      vr[u] = u32x4{0u, 0u, 0u, 0u};
      if (key < s1) {
        kr[u] = reinterpret_cast<const u32x4*>(K + kbase + (size_t)key * D)[ch];
        vr[u] = reinterpret_cast<const u32x4*>(V + kbase + (size_t)key * D)[ch];
      }
    }
    float s[HG][UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float kf[8];
      widen8(kr[u], BF16, kf);
      const bool live = base + u * RPW + row < s1;
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) d = fmaf(q[g][j], kf[j], d);
        d = group_sum<LPR>(d);
        s[g][u] = live ? d * c : -INFINITY;
      }
    }
    float mref[HG];
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      float mc = s[g][0];
#pragma unroll
      for (int u = 1; u < UNR; ++u) mc = fmaxf(mc, s[g][u]);
      const float mn = fmaxf(m[g], mc);
      mref[g] = mn == -INFINITY ? 0.f : mn;
      const float alpha = m[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[g] - mref[g]);
      l[g] *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[g][j] *= alpha;
      m[g] = mn;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float vf[8];
      widen8(vr[u], BF16, vf);
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        const float p = __builtin_amdgcn_exp2f(s[g][u] - mref[g]);
        l[g] += p;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[g][j] = fmaf(p, vf[j], acc[g][j]);
      }
    }
  }

  // merge the NS states of this workgroup, one head at a time through LDS
  const int st = w * RPW + row;
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    if (ch == 0) {
      st_m[st] = m[g];
      st_l[st] = l[g];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) st_o[st][8 * ch + j] = acc[g][j];
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
      const size_t ps = (size_t)(bh0 + g) * splits + split;
      Opart[ps * D + tid] = o / L;
      if (tid == 0) Lpart[ps] = (M + __log2f(L)) * kLn2;
    }
    if (g + 1 < HG) __syncthreads();  // the LDS states are rewritten for the next head
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

template <int D, bool BF16, int HG>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                           int Hkv, int Nk, float scale, int splits, void* workspace, hipStream_t stream) {
  float* opart = static_cast<float*>(workspace);
  float* lpart = opart + (size_t)B * H * splits * D;
  hipLaunchKernelGGL((decode_partial_kernel<D, BF16, HG>), dim3(B * H / HG * splits), dim3(kDecThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), opart, lpart, Nk, scale * kLog2e, splits, H, H / Hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, BF16>), dim3(B * H), dim3(D), 0, stream, opart, lpart,
                     static_cast<uint16_t*>(out), lse, splits);
  return hipGetLastError();
}

// heads per workgroup: the largest of 8, 4, 2 that divides the group size
template <int D, bool BF16>
hipError_t launch_decode_g(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                           int Hkv, int Nk, float scale, int splits, void* workspace, hipStream_t stream) {
  switch (decode_heads_per_workgroup(H, Hkv)) {
    case 8: return launch_decode_t<D, BF16, 8>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
    case 4: return launch_decode_t<D, BF16, 4>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
    case 2: return launch_decode_t<D, BF16, 2>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
    default: return launch_decode_t<D, BF16, 1>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  }
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int d, int splits) {
  return (size_t)B * H * splits * (d + 1) * sizeof(float);
}

int decode_heads_per_workgroup(int H, int Hkv) {
  const int group = H / Hkv;
  return group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}

int decode_default_splits(int B, int H, int Hkv, int Nk, int d) {
  (void)d;
  // aim for about 8192 (query head, key range) streams with at least 128 keys
  // each.  A grouped workgroup serves several heads of a range at once; counting
  // streams per query head still measured best for it (splitting its key range
  // further only added partial states to write and merge)
  (void)Hkv;
  long bh = (long)B * H;
  int s = 1;
  while (bh * s < 8192 && s < 256 && (long)(s * 2) * 128 <= Nk) s *= 2;
  return s;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv,
                         int Nk, int d, float scale, bool bf16, int splits, void* workspace, hipStream_t stream) {
  if (d == 128 && bf16)
    return launch_decode_g<128, true>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  if (d == 128 && !bf16)
    return launch_decode_g<128, false>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  if (d == 64 && bf16)
    return launch_decode_g<64, true>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  if (d == 64 && !bf16)
    return launch_decode_g<64, false>(q, k, v, out, lse, B, H, Hkv, Nk, scale, splits, workspace, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
