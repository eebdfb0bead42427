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
#include <mutex>
#include <type_traits>

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
        // every K/V byte is read exactly once: the loads carry the
        // nontemporal hint (12 % faster on the decode workload)
        kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(K + kbase + (size_t)key * D) + ch);
        vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(V + kbase + (size_t)key * D) + ch);
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

// ---------------------------------------------------------- grouped, on MFMA
// With HG = 4 or 8 query heads per K/V head the vector-ALU kernel above does
// HG dot products and HG cross-lane reductions per row and becomes bound by
// the vector ALU, not by HBM.  This kernel moves both products to the matrix
// cores, in the operand layouts of the prefill kernel with the HG heads as
// its query columns: each wave streams 32-key tiles of the workgroup's key
// range, S^T = K Q^T with the K tile as the A operand loaded from HBM straight
// into registers and the HG queries as B columns (columns past HG read 0),
// the online softmax on the 16 scores a lane holds for its head, then
// O^T += V^T P^T with the V tile read transposed from wave-private LDS.  The
// next tile's K and V loads are in flight while the current tile is used.
// The matrix cores run 32 - HG empty columns; they have the throughput to
// spare, and the vector ALU does about a tenth of the other kernel's work.

// cache policy of the V tile loads: nontemporal (each V row is read once, in
// whole 1 KB pieces; measured 12 % faster).  The K operand loads keep the
// default policy: a wave reads each K row in 16-byte pieces over its k-steps,
// and with the hint on them the kernel measured 16 % slower.
constexpr int kNtPolicy = 2;
__device__ __forceinline__ void dec_lds_load(const __amdgpu_buffer_rsrc_t& r, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, kNtPolicy);
}
// V tile swizzle (16-byte slot XOR a function of the row): the transposing
// reads of 16-lane groups (4 consecutive rows, 32 bytes each) hit distinct banks
template <int D>
__device__ __forceinline__ int dec_v_swz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

constexpr float kDecRescaleThreshold = 8.0f;  // log2 units, as the prefill kernel

template <int D, bool BF16, int HG>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ Opart, float* __restrict__ Lpart, int Nk, float c, int splits, int H, int group) {
  using M = Mfma<BF16>;
  typedef typename M::op8 op8;
  typedef typename M::op2 op2;
  constexpr int BN = 32, ROWB = D * 2, SPR = ROWB / 16, RPI = 1024 / ROWB;
  constexpr int KSTEPS = D / 16, MB_O = D / 32, TILEB = BN * ROWB, LPW = TILEB / 1024;
  static_assert(4 * HG * D * 4 <= 4 * 2 * TILEB, "the merge area fits in the V buffers");
  __shared__ __attribute__((aligned(1024))) char vbuf[4][2][TILEB];
  __shared__ float mst[4][HG], lst[4][HG];

  const int wgi = blockIdx.x / splits, split = blockIdx.x - wgi * splits;
  const int s0 = (int)(((long)split * Nk) / splits), s1 = (int)(((long)(split + 1) * Nk) / splits);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int bh0 = wgi * HG;
  const int b = bh0 / H, h0 = bh0 - b * H;
  const size_t kbase = ((size_t)b * (H / group) + h0 / group) * Nk * D;
  const auto rk = make_rsrc(K + kbase, (uint32_t)Nk * ROWB);
  const auto rv = make_rsrc(V + kbase, (uint32_t)Nk * ROWB);
  const auto rq = make_rsrc(Q + (size_t)bh0 * D, (uint32_t)HG * ROWB);

  // B operand: head l32 (its row of Q), d = 16kk + 8h .. +7; columns >= HG read 0
  op8 qop[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
    qop[kk] = __builtin_bit_cast(op8, buf_load16(rq, (uint32_t)l32 * ROWB + (2 * kk + h) * 16));

  // V^T operand offsets in a V tile (rows = keys), as the prefill reads them
  const int r16 = lane & 15, g1 = (lane >> 4) & 1;
  const int vrow = (r16 >> 2) + 4 * h;
  uint32_t va_off[MB_O];
#pragma unroll
  for (int mb = 0; mb < MB_O; ++mb) {
    const int col = 32 * mb + 16 * g1 + 4 * (r16 & 3);
    va_off[mb] = vrow * ROWB + 16 * ((col >> 3) ^ dec_v_swz<D>(vrow)) + 2 * (col & 7);
  }

  const int ntile = (s1 - s0 + BN - 1) / BN;  // wave w takes tiles w, w + 4, ...
  f32x16 o[MB_O];
#pragma unroll
  for (int mb = 0; mb < MB_O; ++mb) o[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  op8 kr[2][KSTEPS];

  // K rows key0 + l32 into registers (A operand: chunk 2kk + h), the V tile
  // into this wave's LDS buffer; rows past Nk read 0, keys past s1 are masked
  auto load_tile = [&](auto bc, int t) {
    constexpr int BUF = decltype(bc)::value;
    const int key0 = s0 + t * BN;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      kr[BUF][kk] = __builtin_bit_cast(op8, buf_load16(rk, (uint32_t)(key0 + l32) * ROWB + (2 * kk + h) * 16));
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row = i * RPI + lane / SPR, slot = lane % SPR;
      dec_lds_load(rv, vbuf[w][BUF] + 1024 * i, (uint32_t)(key0 + row) * ROWB + 16 * (slot ^ dec_v_swz<D>(row)));
    }
  };
  // loads complete in order: with the next tile's KSTEPS + LPW loads issued
  // after this tile's, waiting for at most that many outstanding is enough
  constexpr int VM = KSTEPS + LPW;
  constexpr int kWaitNext = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8);
  auto step = [&](auto bc, int t) {
    constexpr int BUF = decltype(bc)::value;
    const bool more = t + 4 < ntile;
    if (more) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS reads done before the other buffer is refilled
      load_tile(std::integral_constant<int, BUF ^ 1>{}, t + 4);
      __builtin_amdgcn_s_waitcnt(kWaitNext);
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) s = M::mma(kr[BUF][kk], qop[kk], s);
    const int key0 = s0 + t * BN;
    if (key0 + BN > s1) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + 8 * (i >> 2) + 4 * h + (i & 3) >= s1) s[i] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    const float mt = pair_max(mx) * c;
    if (__any(mt > m_run + kDecRescaleThreshold)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
      for (int mb = 0; mb < MB_O; ++mb) o[mb] *= alpha;
      l_run *= alpha;
      m_run = mn;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    op8 pb[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      op2 pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * tt + 2 * j], c, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * tt + 2 * j + 1], c, -m_use));
        pr[j] = M::pack2(p0, p1);
        l_run += p0 + p1;
      }
      pb[tt] = __builtin_shufflevector(__builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3),
                                       __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const char* lv = vbuf[w][BUF];
#pragma unroll
    for (int j = 0; j < 2 * MB_O; ++j) {
      const uint32_t a0 = va_off[j % MB_O] + 16 * (j / MB_O) * ROWB;
      const s16x4 lo = lds_read_tr16(lv, a0);
      const s16x4 hi = lds_read_tr16(lv, a0 + 8 * ROWB);
      const op8 va = __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[j % MB_O] = M::mma(va, pb[j / MB_O], o[j % MB_O]);
    }
  };
  if (w < ntile) load_tile(std::integral_constant<int, 0>{}, w);
  for (int t = w; t < ntile; t += 8) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 4 < ntile) step(std::integral_constant<int, 1>{}, t + 4);
  }

  // merge the 4 waves' states per head through LDS (the V buffers are free now)
  const float l_tot = pair_sum(l_run);
  __syncthreads();
  float* so = reinterpret_cast<float*>(&vbuf[0][0][0]);  // [wave][head][d]
  if (l32 < HG) {
#pragma unroll
    for (int mb = 0; mb < MB_O; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) so[(w * HG + l32) * D + 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3)] = o[mb][i];
    if (h == 0) {
      mst[w][l32] = m_run;
      lst[w][l32] = l_tot;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < HG * D; idx += 256) {
    const int g = idx / D, d = idx - g * D;
    float Mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) Mx = fmaxf(Mx, mst[v][g]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float wgt = mst[v][g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mst[v][g] - Mx);
      L = fmaf(lst[v][g], wgt, L);
      acc = fmaf(so[(v * HG + g) * D + d], wgt, acc);
    }
    const size_t ps = (size_t)(bh0 + g) * splits + split;
    Opart[ps * D + d] = acc / L;
    if (d == 0) Lpart[ps] = (Mx + __log2f(L)) * kLn2;
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
  // 4 or 8 heads per K/V head go to the matrix cores, which address one
  // head's K/V through buffer resources (at most kMaxSpanBytes)
  if constexpr (HG >= 4) {
    if (span_ok((long long)Nk * D * 2))
      hipLaunchKernelGGL((decode_mfma_kernel<D, BF16, HG>), dim3(B * H / HG * splits), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), opart, lpart, Nk, scale * kLog2e, splits, H, H / Hkv);
    else
      hipLaunchKernelGGL((decode_partial_kernel<D, BF16, HG>), dim3(B * H / HG * splits), dim3(kDecThreads), 0,
                         stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), opart, lpart, Nk, scale * kLog2e, splits, H, H / Hkv);
  } else {
    hipLaunchKernelGGL((decode_partial_kernel<D, BF16, HG>), dim3(B * H / HG * splits), dim3(kDecThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), opart, lpart, Nk, scale * kLog2e, splits, H, H / Hkv);
  }
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

// ------------------------------------------------- decode without allocation
// Split partials of attn_fwd_decode_static, for callers that cannot allocate
// device memory (code under graph capture, serving loops, harnesses that
// forbid allocation): a file-scope device array that every GPU the library
// runs on holds from module load to process end.  Host code must not pass
// the array's own name to a kernel (on the host it is only a stand-in, not a
// device address): its device address is looked up once per device with
// hipGetSymbolAddress and used from then on.  The partial kernels write every
// (head, split) slot that the merge kernel reads, so nothing in it has to be
// cleared between calls; two calls that overlap on one GPU share it and race.
static __device__ __align__(256) unsigned char scratch[kDecodeStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device id
}  // namespace

hipError_t decode_static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_static(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                                int Nk, int d, float scale, bool bf16, int splits, hipStream_t stream) {
  if (decode_workspace_bytes(B, H, d, splits) > kDecodeStaticScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = decode_static_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_decode(q, k, v, out, lse, B, H, H, Nk, d, scale, bf16, splits, ws, stream);
}

}  // namespace attn
