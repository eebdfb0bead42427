// Backward pass of attention for gfx950 (bf16/fp16, d in {64, 128}): the
// gradients dQ, dK, dV of sum(dO * O), recomputing the probability tiles from
// Q, K and the forward's log-sum-exp instead of storing them ("Backward:
// recompute instead of store" in the marketmaker.cc post "Can a full trading
// day of context beat one minute? Flash attention and the sequence-length
// question").  With P = softmax(scale Q K^T) (future keys masked when causal):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = rowsum(dO_i * O_i),
//   dQ = scale dS K,  dK = scale dS^T Q.
// D_i equals rowsum(P_i * dP_i) (both are dO_i . O_i); it is computed once per
// row from the stored O.
//
// Three kernels, no atomics:
//   bwd_pre: per query row, (LSE log2 e, D) into a float2 workspace;
//   bwd_kv:  a workgroup owns 128 keys (32 per wave, K and V held in registers
//            as MFMA operands) and streams the queries in steps of 32 through
//            LDS (Q and dO tiles, and the step's 32 LSE values followed by
//            its 32 D values, double-buffered, loaded straight into LDS, so
//            a lane reads the four it needs at a time in one 16-byte read).
//            Per step and wave: S = Q K^T and
//            dP = dO V^T come out with one key per lane, which is exactly the
//            A-operand layout of P^T and dS^T, so dV += P^T dO and
//            dK += dS^T Q follow with dO and Q read transposed from LDS.
//            At d = 128 on dense non-causal grids bwd_kv_pp takes its place:
//            the same products split between a P/dV and a dS/dK group of
//            waves on the forward's ping-pong schedule;
//   bwd_dq:  a workgroup owns 128 queries (Q and dO in registers) and streams
//            K and V tiles; S^T = K Q^T and dP^T = V dO^T come out with one
//            query per lane, the A-operand layout of dS, and dQ += dS K reads
//            K transposed from LDS.
// S and dP are thus computed twice (7 matrix products instead of 5) in
// exchange for no cross-workgroup reduction.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace attn {

namespace {

template <int D>
struct BwdCfg {
  static constexpr int ROWB = 2 * D;               // bytes per row
  static constexpr int SPR = ROWB / 16;            // 16-byte slots per row
  static constexpr int RPI = 1024 / ROWB;          // rows per 1 KB wave load
  static constexpr int NW = 4;                     // waves per workgroup
  static constexpr int BO = 32 * NW;               // rows owned by a workgroup (32 per wave)
  static constexpr int BS = 32;                    // rows streamed per step
  static constexpr int TILEB = BS * ROWB;          // bytes per streamed tile
  static constexpr int LPW = TILEB / 1024 / NW;    // 1 KB loads per wave per tile
  static constexpr int KSTEPS = D / 16;            // MFMA k-steps over d
  static constexpr int NBD = D / 32;               // 32-column blocks of d
};

// XOR swizzle of the 16-byte slots of a streamed tile row.  Conflict-free for
// both access patterns of these tiles: row reads (ds_read_b128, 16 consecutive
// rows at one logical slot) and transposing reads (ds_read_b64_tr_b16, 4
// consecutive rows x 64 bytes).  It depends on the row's low 4 bits only, so
// rows 16 apart share it.
template <int D>
__device__ __forceinline__ int bswz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

__device__ __forceinline__ void bwd_load_lds16(const __amdgpu_buffer_rsrc_t& r, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void bwd_load_lds4(const __amdgpu_buffer_rsrc_t& r, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)dst, 4, voff, 0, 0, 0);
}

template <class M>
__device__ __forceinline__ typename M::op8 pack8(const f32x16& x, int base) {
  typedef typename M::op2 op2;
  const op2 a = M::pack2(x[base + 0], x[base + 1]), b = M::pack2(x[base + 2], x[base + 3]);
  const op2 e = M::pack2(x[base + 4], x[base + 5]), f = M::pack2(x[base + 6], x[base + 7]);
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3), __builtin_shufflevector(e, f, 0, 1, 2, 3),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// element j of a packed 16-bit operand, widened to fp32 (exact): bf16 by
// moving its bits into the high half of the word, fp16 by conversion
template <class M>
__device__ __forceinline__ float op8_elem(typename M::op8 v, int j) {
  const uint32_t dw = __builtin_bit_cast(u32x4, v)[j >> 1];
  if constexpr (std::is_same<typename M::op8, bf16x8>::value)
    return __builtin_bit_cast(float, (j & 1) ? (dw & 0xffff0000u) : (dw << 16));
  else
    return (float)__builtin_bit_cast(typename M::op2, dw)[j & 1];
}

template <bool BF16>
__device__ __forceinline__ uint16_t to_half_bits(float x) {
  typedef typename Mfma<BF16>::op2 op2;
  const op2 p = Mfma<BF16>::pack2(x, 0.f);
  return __builtin_bit_cast(uint32_t, p) & 0xffffu;
}

// Causal grids: the blocks of one head differ in work (a key block near the
// start is seen by many queries, a query block near the end sees many keys).
// Items are taken in chunks of `chunk` heads, block-major inside a chunk (rank
// 0, the most work, of every head of the chunk first), and chunks stay
// contiguous, so each XCD's contiguous range of items (xcd_remap) still covers
// whole heads while the dispatcher starts the longest items first.
__device__ __forceinline__ void heavy_first(int logical, int nblk, int nheads, int chunk, int& head, int& rank) {
  const int c = logical / (nblk * chunk);
  const int c0 = c * chunk;
  const int ch = min(chunk, nheads - c0);
  const int i = logical - c * nblk * chunk;
  rank = i / ch;
  head = c0 + (i - rank * ch);
}

// ---------------------------------------------------------------- bwd_pre
// One row per D/8 lanes (16 bytes each): D_i = sum_c dO_ic O_ic in fp32 and
// the log-sum-exp in base 2.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ LSE, float2* __restrict__ LD,
                                                      long rows) {
  constexpr int TPR = D / 8;
  const long row = (long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(O + row * D + part * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + row * D + part * 8);
    const f16x8 oh = __builtin_bit_cast(f16x8, o), gh = __builtin_bit_cast(f16x8, g);
    // widen each 16-bit pair exactly to fp32 (the products are exact in fp32)
    // and keep the two halves of each pair in separate sums: a single chain
    // over both halves is fused by the compiler into a packed dot product
    // that, on this target, reads the first 32-bit word of the row chunk
    // four times
    float acc1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float o0, o1, g0, g1;
      if (BF16) {
        o0 = __builtin_bit_cast(float, o[j] << 16);
        o1 = __builtin_bit_cast(float, o[j] & 0xffff0000u);
        g0 = __builtin_bit_cast(float, g[j] << 16);
        g1 = __builtin_bit_cast(float, g[j] & 0xffff0000u);
      } else {
        o0 = (float)oh[2 * j];
        o1 = (float)oh[2 * j + 1];
        g0 = (float)gh[2 * j];
        g1 = (float)gh[2 * j + 1];
      }
      acc = fmaf(o0, g0, acc);
      acc1 = fmaf(o1, g1, acc1);
    }
    acc += acc1;
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  // a row that saw no key (LSE = -inf, packed batches) gets +inf, so every
  // probability rebuilt for it is exp2(-inf) = 0 and it adds no gradient
  if (row < rows && part == 0) {
    const float lse = LSE[row];
    LD[row] = make_float2(lse == -INFINITY ? INFINITY : lse * kLog2e, acc);
  }
}

// ---------------------------------------------------------------- bwd_kv
template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_kv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float2* __restrict__ LD, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, SeqShape sh, float c, float scale, int nkb, int total, int chunk) {
  using C = BwdCfg<D>;
  using M = Mfma<BF16>;
  typedef typename M::op8 op8;
  __shared__ __attribute__((aligned(1024))) char q0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char q1s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char d0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char d1s[C::TILEB];
  __shared__ __attribute__((aligned(256))) char l0s[C::BS * 8];
  __shared__ __attribute__((aligned(256))) char l1s[C::BS * 8];
  // at d = 128 each wave's V rows live in LDS (same swizzled row layout as the
  // streamed tiles) instead of 32 more registers
  constexpr bool VLDS = D == 128;
  __shared__ __attribute__((aligned(1024))) char vws[VLDS ? C::NW * 32 * C::ROWB : 16];

  // work item: 128 keys of one (sequence, K/V head); the group's query heads
  // all read them, so dK and dV sum over the group's queries
  // packed batches: plain dispatch order and one chunk of all heads, so the
  // longest blocks of every sequence start first on every XCD
  const bool packed = sh.cu_q != nullptr;
  const int logical = packed ? (int)blockIdx.x : xcd_remap(blockIdx.x, total);
  const int Hkv = sh.H / sh.group;
  int sk, kb;
  if (CAUSAL || packed) {
    heavy_first(logical, nkb, total / nkb, chunk, sk, kb);  // key block 0 has the most queries
  } else {
    sk = logical / nkb;
    kb = logical - sk * nkb;
  }
  const int k0 = kb * C::BO;
  const int sq = sk / Hkv, hk = sk - sq * Hkv;
  const SeqSpan sp = seq_span(sh, sq, hk * sh.group);  // the group's first query head
  const int Nq = sp.nq, Nk = sp.nk;
  if (k0 >= Nk) return;  // past a short packed sequence (uniform over the workgroup)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int off = Nk - Nq;  // bottom-right causal alignment
  const size_t kbase = sp.k_row0 * D;
  // query head gi of the group starts qstride rows after head gi-1
  const size_t qstride = sh.cu_q != nullptr ? (size_t)sh.Nq : (size_t)Nq;
  const auto rk = make_rsrc(K + kbase, (uint32_t)Nk * D * 2);
  const auto rv = make_rsrc(V + kbase, (uint32_t)Nk * D * 2);

  // this wave's keys: K and V rows as B operands (n = key, k = d)
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;
  op8 kop[C::KSTEPS], vop[VLDS ? 1 : C::KSTEPS];
  char* const vw = vws + (VLDS ? w * 32 * C::ROWB : 0);
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    kop[kk] = __builtin_bit_cast(op8, buf_load16(rk, (uint32_t)key * C::ROWB + (16 * kk + 8 * h) * 2));
    const u32x4 x = buf_load16(rv, (uint32_t)key * C::ROWB + (16 * kk + 8 * h) * 2);
    if (VLDS)
      lds_store<u32x4>(vw, l32 * C::ROWB + 16 * ((2 * kk + h) ^ bswz<D>(l32)), x);
    else
      vop[kk < (VLDS ? 1 : C::KSTEPS) ? kk : 0] = __builtin_bit_cast(op8, x);
  }
  __builtin_amdgcn_sched_barrier(0);

  // tile loads: wave w fills 1 KB blocks LPW w .. LPW w + LPW-1 of a Q and a dO tile
  uint32_t goff[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int row = (C::LPW * w + i) * C::RPI + lane / C::SPR, ps = lane % C::SPR;
    goff[i] = (uint32_t)row * C::ROWB + 16 * (ps ^ bswz<D>(row));
  }
  // Q, dO and (LSE, D) rows of query step st of the group's query head gi
  auto issue = [&](int gi, int st, char* qt, char* dt, char* lt) __attribute__((always_inline)) {
    const size_t qrow0 = sp.q_row0 + (size_t)gi * qstride;
    const auto rq = make_rsrc(Q + qrow0 * D, (uint32_t)Nq * D * 2);
    const auto rdo = make_rsrc(dO + qrow0 * D, (uint32_t)Nq * D * 2);
    const auto rld = make_rsrc(LD + qrow0, (uint32_t)Nq * 8);
    const uint32_t base = (uint32_t)(st * C::BS) * C::ROWB;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      bwd_load_lds16(rq, qt + 1024 * (C::LPW * w + i), base + goff[i]);
      bwd_load_lds16(rdo, dt + 1024 * (C::LPW * w + i), base + goff[i]);
    }
    // lane i < 32 fetches row i's LSE, lane 32 + i its D: the tile holds 32
    // LSE values, then 32 D values
    if (w == 0) bwd_load_lds4(rld, lt, (uint32_t)(st * C::BS + (lane & 31)) * 8 + 4 * (lane >> 5));
  };
  // row reads (A operand: m = query l32, k = d 16 kk + 8h .. +7): byte offset
  // l32 ROWB + ((32 kk + 16 h) ^ 16 swz(l32)), one XOR-add per read
  const uint32_t ra_base = l32 * C::ROWB, ra_x = 16 * (h ^ bswz<D>(l32));
  // transposing reads (B operand: k = queries {4h..4h+3, 8+4h..8+4h+3} (+16 t), n = d 32 nb + l32)
  // lane r16 of each 16 points at row (r16/4) + 4h (+ 8 for the upper half,
  // + 16 ti), columns 32 nb + 16 g1 + 4 (r16%4) .. +3: byte offset
  // tr_base[hi] + ((64 nb) ^ tr_x[hi]) + 32 ti ROWB, with the swizzle folded into tr_x
  uint32_t tr_base[2], tr_x[2];
  {
    const int r16 = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = (r16 >> 2) + 4 * h + 8 * hi;
      tr_base[hi] = row * C::ROWB + 8 * (r16 & 1);
      tr_x[hi] = 16 * ((2 * g1 + ((r16 & 3) >> 1)) ^ bswz<D>(row));
    }
  }
  auto tr_load = [&](const char* t, int nb, int ti) __attribute__((always_inline)) {
    const s16x4 lo = lds_read_tr16(t, tr_base[0] + ((64u * nb) ^ tr_x[0]) + 16 * ti * C::ROWB);
    const s16x4 hi = lds_read_tr16(t, tr_base[1] + ((64u * nb) ^ tr_x[1]) + 16 * ti * C::ROWB);
    return __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 dv[C::NBD], dk[C::NBD];
#pragma unroll
  for (int nb = 0; nb < C::NBD; ++nb) {
    dv[nb] = f32x16{};
    dk[nb] = f32x16{};
  }

  // acc += A B over the KSTEPS k-steps: A = rows of tile t (two k-steps ahead),
  // B = bop (registers) or, with BL, this wave's LDS rows, which share the A
  // rows' offsets
  auto row_gemm = [&](auto BL, const char* t, const op8* bop, const char* bl, f32x16 acc)
                      __attribute__((always_inline)) {
    constexpr bool FROM_LDS = decltype(BL)::value;
    op8 ar[2], br[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      ar[kk] = lds_load<op8>(t, ra_base + ((32u * kk) ^ ra_x));
      if (FROM_LDS) br[kk] = lds_load<op8>(bl, ra_base + ((32u * kk) ^ ra_x));
    }
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const op8 x = ar[kk & 1];
      const op8 y = FROM_LDS ? br[kk & 1] : bop[FROM_LDS ? 0 : kk];
      if (kk + 2 < C::KSTEPS) {
        ar[kk & 1] = lds_load<op8>(t, ra_base + ((32u * (kk + 2)) ^ ra_x));
        if (FROM_LDS) br[kk & 1] = lds_load<op8>(bl, ra_base + ((32u * (kk + 2)) ^ ra_x));
      }
      acc = M::mma(x, y, acc);
    }
    constexpr int NR = FROM_LDS ? 2 : 1;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * NR, 0);
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (kk + 2 < C::KSTEPS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NR, 0);
    }
    return acc;
  };
  // acc[nb] += A[ti] * (tile t read transposed), B operands two ahead
  auto tr_gemm = [&](const char* t, const op8* am, f32x16* acc) __attribute__((always_inline)) {
    constexpr int NT = 2 * C::NBD;
    op8 br[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) br[u] = tr_load(t, u % C::NBD, u / C::NBD);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const op8 x = br[u & 1];
      if (u + 2 < NT) br[u & 1] = tr_load(t, (u + 2) % C::NBD, (u + 2) / C::NBD);
      acc[u % C::NBD] = M::mma(am[u / C::NBD], x, acc[u % C::NBD]);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (u + 2 < NT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
  };

  // step: queries q0 .. q0+31 from tiles qt, dt, lt.  Element i of S, dP:
  // query q0 + 8 (i/4) + 4h + i%4 of this lane's key.
  auto step = [&](int st, const char* qt, const char* dt, const char* lt) __attribute__((always_inline)) {
    const int q0 = st * C::BS;
    const bool edge = (q0 + C::BS > Nq) || (CAUSAL && kw0 + 31 > q0 + off);
    // P = exp2(S c - LSE log2 e), masked; kept only as the 16-bit MFMA operand
    op8 pa[2];
    {
      f32x16 sv = row_gemm(std::false_type{}, qt, kop, nullptr, f32x16{});
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 Lr = lds_load<f32x4>(lt, (8 * a + 4 * h) * 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * a + b;
          sv[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], c, -Lr[b]));
        }
      }
      // masked pairs (query past Nq, or key after the query on causal tiles)
      // only on edge steps: a uniform branch, so other steps carry no selects
      if (edge) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = q0 + 8 * (i >> 2) + 4 * h + (i & 3);
          const uint32_t hide = (qi >= Nq || (CAUSAL && key > qi + off)) ? 0xFFFFFFFFu : 0u;
          const float v = sv[i];  // copied out first (a bit cast of a vector element in place misreads)
          sv[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & ~hide);
        }
      }
      pa[0] = pack8<M>(sv, 0);
      pa[1] = pack8<M>(sv, 8);
    }
    // the phases stay in order: overlapping them only raises the register peak
    __builtin_amdgcn_sched_barrier(0);
    // dV += P^T dO
    tr_gemm(dt, pa, dv);
    __builtin_amdgcn_sched_barrier(0);
    // dS = P (dP - D), from the 16-bit P; dK += dS^T Q
    op8 da[2];
    {
      f32x16 dpv = row_gemm(std::integral_constant<bool, VLDS>{}, dt, vop, vw, f32x16{});
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 Dr = lds_load<f32x4>(lt, 4 * C::BS + (8 * a + 4 * h) * 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * a + b;
          const float p = op8_elem<M>(pa[i >> 3], i & 7);
          dpv[i] = p * (dpv[i] - Dr[b]);
        }
      }
      da[0] = pack8<M>(dpv, 0);
      da[1] = pack8<M>(dpv, 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    tr_gemm(qt, da, dk);
    __builtin_amdgcn_sched_barrier(0);
  };

  // query steps that see at least one of this workgroup's keys, for every
  // query head of the group in turn: step u is step s0 + u % nper of head u / nper
  int s0 = 0;
  if (CAUSAL) s0 = max(0, k0 - off) / C::BS;
  const int ns = (Nq + C::BS - 1) / C::BS;
  const int nper = max(0, ns - s0);
  const int nu = sh.group * nper;
  if (nu > 0) issue(0, s0, q0s, d0s, l0s);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int u = 0; u < nu; ++u) {
    const bool odd = u & 1;
    if (u + 1 < nu) {
      const int gn = (u + 1) / nper;
      issue(gn, s0 + (u + 1 - gn * nper), odd ? q0s : q1s, odd ? d0s : d1s, odd ? l0s : l1s);
    }
    step(s0 + u % nper, odd ? q1s : q0s, odd ? d1s : d0s, odd ? l1s : l0s);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // element i of block nb: key kw0 + 8 (i/4) + 4h + i%4, column 32 nb + l32
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kr = kw0 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (kr < Nk) {
      uint16_t* pv = dV + kbase + (size_t)kr * D + l32;
      uint16_t* pk = dK + kbase + (size_t)kr * D + l32;
#pragma unroll
      for (int nb = 0; nb < C::NBD; ++nb) {
        pv[32 * nb] = to_half_bits<BF16>(dv[nb][i]);
        pk[32 * nb] = to_half_bits<BF16>(dk[nb][i] * scale);
      }
    }
  }
}

// ---------------------------------------------------------------- bwd_kv, d = 128
// At d = 128 the dK/dV work of a key block is split between two groups of 4
// waves that run the forward's ping-pong schedule.  The workgroup owns 128
// keys; wave w & 3 of either group takes 32 of them.  Group 0 forms P and
// accumulates dV, group 1 forms dS and accumulates dK, so each wave holds one
// 128-register accumulator set and one of K, V as its B operand (holding both
// accumulator sets and K, as the kernel above does, leaves no room for the
// schedule).  Per query step u (64 queries) a wave has an MFMA phase G_u and
// a vector phase X_u:
//   group 0  G_u: dV += P(u-1)^T dO(u-1), then S(u) = Q(u) K^T
//            X_u: P(u) = exp2(S c - LSE log2 e), masked, packed; P(u) to LDS
//   group 1  G_u: dK += dS(u-1)^T Q(u-1), then dP(u) = dO(u) V^T
//            X_u: dS(u) = P(u) (dP(u) - D), with P(u) read back from LDS
// Group 1 runs its sequence one phase behind group 0, so on every SIMD (one
// wave of each group) one wave feeds the matrix cores while the other feeds
// the vector ALU; a workgroup barrier ends every step (every other phase).
// Step u's Q, dO, (LSE, D) and P tiles are read from phase 2u to phase 2u+3,
// so three tile sets rotate; group 0 requests step u+1 during its S products
// in phase 2u, and the barrier that ends phase 2u+1 waits for it.  Dense
// non-causal grids only (every workgroup walks every query step of its heads).
template <bool BF16>
__global__ __launch_bounds__(512, 1) void bwd_kv_pp_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float2* __restrict__ LD, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, SeqShape sh, float c, float scale, int nkb, int total) {
  constexpr int D = 128;
  using C = BwdCfg<D>;
  using M = Mfma<BF16>;
  typedef typename M::op8 op8;
  constexpr int SQ = 64;                    // queries per step: two 32-query halves
  constexpr int TB = SQ * C::ROWB;          // bytes per Q or dO tile
  constexpr int PWB = 2 * 2 * 64 * 16;      // P of one wave and step: 2 halves x 2 packed operands x 64 lanes x 16 B
  static_assert(C::BO == 128, "128 keys per workgroup");
  // three tile sets (step u in set u % 3): Q, dO, (LSE, D) of each half, P
  __shared__ __attribute__((aligned(1024))) char q0s[TB];
  __shared__ __attribute__((aligned(1024))) char q1s[TB];
  __shared__ __attribute__((aligned(1024))) char q2s[TB];
  __shared__ __attribute__((aligned(1024))) char d0s[TB];
  __shared__ __attribute__((aligned(1024))) char d1s[TB];
  __shared__ __attribute__((aligned(1024))) char d2s[TB];
  __shared__ __attribute__((aligned(256))) char l0s[SQ * 8];
  __shared__ __attribute__((aligned(256))) char l1s[SQ * 8];
  __shared__ __attribute__((aligned(256))) char l2s[SQ * 8];
  __shared__ __attribute__((aligned(1024))) char p0s[4 * PWB];
  __shared__ __attribute__((aligned(1024))) char p1s[4 * PWB];
  __shared__ __attribute__((aligned(1024))) char p2s[4 * PWB];

  // work item as in the kernel above: 128 keys of one (batch, K/V head),
  // each XCD taking a contiguous range of them
  const int logical = xcd_remap(blockIdx.x, total);
  const int Hkv = sh.H / sh.group;
  const int sk = logical / nkb, kb = logical - sk * nkb;
  const int k0 = kb * C::BO;
  const int sq = sk / Hkv, hk = sk - sq * Hkv;
  const SeqSpan sp = seq_span(sh, sq, hk * sh.group);
  const int Nq = sp.nq, Nk = sp.nk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wg = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const size_t kbase = sp.k_row0 * D;

  // this wave's keys; group 0 holds their K rows, group 1 their V rows, as B
  // operands (n = key, k = d)
  const int kw0 = k0 + 32 * wg;
  const int key = kw0 + l32;
  op8 bop[C::KSTEPS];
  {
    const auto rb = make_rsrc((grp == 0 ? K : V) + kbase, (uint32_t)Nk * D * 2);
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk)
      bop[kk] = __builtin_bit_cast(op8, buf_load16(rb, (uint32_t)key * C::ROWB + (16 * kk + 8 * h) * 2));
  }
  __builtin_amdgcn_sched_barrier(0);

  // the query steps of every query head of the group in turn: step u is step
  // u % nper of head u / nper
  const int nper = (Nq + SQ - 1) / SQ;
  const int nu = sh.group * nper;

  // tile loads of step u, issued by the 4 waves of group 0: wave wg fills 1 KB
  // blocks LPG wg .. LPG wg + LPG-1 of the Q and of the dO tile, and waves 0
  // and 1 fetch the LSE and D of half 0 and half 1 (lane i < 32: row i's LSE,
  // lane 32 + i: its D, so a half's 32 LSE values are followed by its 32 D values)
  constexpr int LPG = TB / 1024 / 4;
  uint32_t goff[LPG];
#pragma unroll
  for (int i = 0; i < LPG; ++i) {
    const int row = (LPG * wg + i) * C::RPI + lane / C::SPR, ps = lane % C::SPR;
    goff[i] = (uint32_t)row * C::ROWB + 16 * (ps ^ bswz<D>(row));
  }
  typedef __amdgpu_buffer_rsrc_t Rsrc;
  struct StepSrc {
    Rsrc rq, rdo, rld;
    uint32_t row0;  // the step's first query row
  };
  auto step_src = [&](int u) __attribute__((always_inline)) {
    const int gi = u / nper;
    const size_t qrow0 = sp.q_row0 + (size_t)gi * Nq;
    StepSrc r;
    r.rq = make_rsrc(Q + qrow0 * D, (uint32_t)Nq * D * 2);
    r.rdo = make_rsrc(dO + qrow0 * D, (uint32_t)Nq * D * 2);
    r.rld = make_rsrc(LD + qrow0, (uint32_t)Nq * 8);
    r.row0 = (uint32_t)((u - gi * nper) * SQ);
    return r;
  };
  // load i of this wave (i < LPG: a Q block, else a dO block)
  auto load_one = [&](const StepSrc& r, int i, char* qt, char* dt) __attribute__((always_inline)) {
    if (i < LPG)
      bwd_load_lds16(r.rq, qt + 1024 * (LPG * wg + i), r.row0 * C::ROWB + goff[i]);
    else
      bwd_load_lds16(r.rdo, dt + 1024 * (LPG * wg + i - LPG), r.row0 * C::ROWB + goff[i - LPG]);
  };
  auto load_ld = [&](const StepSrc& r, char* lt) __attribute__((always_inline)) {
    if (w < 2) bwd_load_lds4(r.rld, lt + 256 * w, (r.row0 + 32 * w + (lane & 31)) * 8 + 4 * (lane >> 5));
  };
  // row reads and transposing reads of a 32-row half, as in the kernel above
  const uint32_t ra_base = l32 * C::ROWB, ra_x = 16 * (h ^ bswz<D>(l32));
  uint32_t tr_base[2], tr_x[2];
  {
    const int r16 = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = (r16 >> 2) + 4 * h + 8 * hi;
      tr_base[hi] = row * C::ROWB + 8 * (r16 & 1);
      tr_x[hi] = 16 * ((2 * g1 + ((r16 & 3) >> 1)) ^ bswz<D>(row));
    }
  }
  auto tr_load = [&](const char* t, int nb, int ti) __attribute__((always_inline)) {
    const s16x4 lo = lds_read_tr16(t, tr_base[0] + ((64u * nb) ^ tr_x[0]) + 16 * ti * C::ROWB);
    const s16x4 hi = lds_read_tr16(t, tr_base[1] + ((64u * nb) ^ tr_x[1]) + 16 * ti * C::ROWB);
    return __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // rows of half t times bop over d, operand reads two ahead; with LDS_ (group
  // 0, when a next step exists) also loads LPG of that step's tile blocks,
  // lq .. lq + LPG-1, one every other MFMA, so the address unit sees a steady
  // trickle instead of every wave's loads at once
  auto row_gemm = [&](const char* t, auto LDS_, const StepSrc& nx, int lq, char* qn, char* dn)
                      __attribute__((always_inline)) {
    constexpr bool L = decltype(LDS_)::value;
    f32x16 acc = f32x16{};
    op8 ar[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ar[kk] = lds_load<op8>(t, ra_base + ((32u * kk) ^ ra_x));
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const op8 x = ar[kk & 1];
      if (kk + 2 < C::KSTEPS) ar[kk & 1] = lds_load<op8>(t, ra_base + ((32u * (kk + 2)) ^ ra_x));
      acc = M::mma(x, bop[kk], acc);
      if (L && (kk & 1)) load_one(nx, lq + kk / 2, qn, dn);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (kk + 2 < C::KSTEPS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if (L && (kk & 1)) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
    return acc;
  };
  static_assert(2 * (C::KSTEPS / 2) == 2 * LPG, "the S products of a step carry its 2 LPG tile loads");
  f32x16 acc[C::NBD];  // group 0: dV, group 1: dK (before the scale)
#pragma unroll
  for (int nb = 0; nb < C::NBD; ++nb) acc[nb] = f32x16{};
  // acc[nb] += am[ti] * (half t read transposed), B operands two ahead
  auto tr_gemm = [&](const char* t, const op8* am) __attribute__((always_inline)) {
    constexpr int NT = 2 * C::NBD;
    op8 br[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) br[u] = tr_load(t, u % C::NBD, u / C::NBD);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const op8 x = br[u & 1];
      if (u + 2 < NT) br[u & 1] = tr_load(t, (u + 2) % C::NBD, (u + 2) / C::NBD);
      acc[u % C::NBD] = M::mma(am[u / C::NBD], x, acc[u % C::NBD]);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (u + 2 < NT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
  };

  // S(u) or dP(u) between the MFMA and vector phases, and P(u) or dS(u),
  // packed, between the vector phase and the next MFMA phase; element i of
  // half j: query 32 j + 8 (i/4) + 4h + i%4 of the step, key of this lane
  f32x16 sx[2];
  op8 px[2][2];
  // G_u of this wave's group: (qc, dc) hold step u, (qp, dp) step u-1; group
  // 0 also loads step u+1 into (qn, dn, ln)
  auto gphase = [&](int u, const char* qc, const char* dc, const char* qp, const char* dp, char* qn, char* dn,
                    char* ln) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (u >= 1) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (grp == 0)
          tr_gemm(dp + 32 * j * C::ROWB, px[j]);  // dV += P^T dO
        else
          tr_gemm(qp + 32 * j * C::ROWB, px[j]);  // dK += dS^T Q
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (u < nu) {
      if (grp == 0 && u + 1 < nu) {
        const StepSrc nx = step_src(u + 1);
        load_ld(nx, ln);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          sx[j] = row_gemm(qc + 32 * j * C::ROWB, std::true_type{}, nx, LPG * j, qn, dn);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        const StepSrc none{};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          sx[j] = row_gemm((grp == 0 ? qc : dc) + 32 * j * C::ROWB, std::false_type{}, none, 0, nullptr, nullptr);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // X_u: lt holds step u's (LSE, D), pt its P
  auto xphase = [&](int u, const char* lt, char* pt) __attribute__((always_inline)) {
    if (u < 0 || u >= nu) return;
    const int q0 = (u % nper) * SQ;
    char* const pw = pt + wg * PWB;  // this key block's P, written by group 0, read by group 1
    if (grp == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int qj = q0 + 32 * j;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 Lr = lds_load<f32x4>(lt, 256 * j + (8 * a + 4 * h) * 4);
#pragma unroll
          for (int b = 0; b < 4; ++b) sx[j][4 * a + b] = __builtin_amdgcn_exp2f(fmaf(sx[j][4 * a + b], c, -Lr[b]));
        }
        // queries past Nq are masked, on the last half only
        if (qj + 32 > Nq) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = qj + 8 * (i >> 2) + 4 * h + (i & 3);
            const uint32_t hide = qi >= Nq ? 0xFFFFFFFFu : 0u;
            const float v = sx[j][i];  // copied out first (a bit cast of a vector element in place misreads)
            sx[j][i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & ~hide);
          }
        }
        px[j][0] = pack8<M>(sx[j], 0);
        px[j][1] = pack8<M>(sx[j], 8);
        lds_store<u32x4>(pw, (2 * j) * 1024 + 16 * lane, __builtin_bit_cast(u32x4, px[j][0]));
        lds_store<u32x4>(pw, (2 * j + 1) * 1024 + 16 * lane, __builtin_bit_cast(u32x4, px[j][1]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const op8 pa[2] = {__builtin_bit_cast(op8, lds_load<u32x4>(pw, (2 * j) * 1024 + 16 * lane)),
                           __builtin_bit_cast(op8, lds_load<u32x4>(pw, (2 * j + 1) * 1024 + 16 * lane))};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 Dr = lds_load<f32x4>(lt, 256 * j + 128 + (8 * a + 4 * h) * 4);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int i = 4 * a + b;
            sx[j][i] = op8_elem<M>(pa[i >> 3], i & 7) * (sx[j][i] - Dr[b]);
          }
        }
        px[j][0] = pack8<M>(sx[j], 0);
        px[j][1] = pack8<M>(sx[j], 8);
      }
    }
  };
  // phases 2u (group 0: G_u, group 1: X_{u-1}) and 2u+1 (group 0: X_u,
  // group 1: G_u); set c holds step u, set p step u-1, and step u+1 is
  // loaded into set n
  auto pair = [&](int u, const char* qc, const char* dc, const char* lc, char* pc, const char* qp, const char* dp,
                  const char* lp, char* pp, char* qn, char* dn, char* ln) __attribute__((always_inline)) {
    if (grp == 0)
      gphase(u, qc, dc, qp, dp, qn, dn, ln);
    else
      xphase(u - 1, lp, pp);
    if (grp == 0)
      xphase(u, lc, pc);
    else
      gphase(u, qc, dc, qp, dp, qn, dn, ln);
    // the loads of step u+1 have landed, P(u) is written, and every wave is
    // done with step u-1's set, which step u+2 overwrites next
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  if (nu > 0 && grp == 0) {
    const StepSrc s0src = step_src(0);
    load_ld(s0src, l0s);
#pragma unroll
    for (int i = 0; i < 2 * LPG; ++i) load_one(s0src, i, q0s, d0s);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int u = 0; u <= nu; u += 3) {
    pair(u, q0s, d0s, l0s, p0s, q2s, d2s, l2s, p2s, q1s, d1s, l1s);
    if (u + 1 <= nu) pair(u + 1, q1s, d1s, l1s, p1s, q0s, d0s, l0s, p0s, q2s, d2s, l2s);
    if (u + 2 <= nu) pair(u + 2, q2s, d2s, l2s, p2s, q1s, d1s, l1s, p1s, q0s, d0s, l0s);
  }

  // element i of block nb: key kw0 + 8 (i/4) + 4h + i%4, column 32 nb + l32
  uint16_t* const out = grp == 0 ? dV : dK;
  const float osc = grp == 0 ? 1.f : scale;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kr = kw0 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (kr < Nk) {
      uint16_t* po = out + kbase + (size_t)kr * D + l32;
#pragma unroll
      for (int nb = 0; nb < C::NBD; ++nb) po[32 * nb] = to_half_bits<BF16>(acc[nb][i] * osc);
    }
  }
}

// ---------------------------------------------------------------- bwd_dq
template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float2* __restrict__ LD, uint16_t* __restrict__ dQ, SeqShape sh,
    float c, float scale, int nqb, int total, int chunk) {
  using C = BwdCfg<D>;
  using M = Mfma<BF16>;
  typedef typename M::op8 op8;
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILEB];

  const bool packed = sh.cu_q != nullptr;
  const int logical = packed ? (int)blockIdx.x : xcd_remap(blockIdx.x, total);
  int bh, qb;
  if (CAUSAL || packed) {
    int rank;
    heavy_first(logical, nqb, total / nqb, chunk, bh, rank);
    qb = nqb - 1 - rank;  // the last query block sees the most keys
  } else {
    bh = logical / nqb;
    qb = logical - bh * nqb;
  }
  const int q0 = qb * C::BO;
  // this (sequence, query head)'s rows; its K/V head is head / group
  const SeqSpan sp = seq_span(sh, bh / sh.H, bh % sh.H);
  const int Nq = sp.nq, Nk = sp.nk;
  if (q0 >= Nq) return;  // past a short packed sequence (uniform over the workgroup)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int off = Nk - Nq;
  const size_t qbase = sp.q_row0 * D, kbase = sp.k_row0 * D;
  const auto rq = make_rsrc(Q + qbase, (uint32_t)Nq * D * 2);
  const auto rdo = make_rsrc(dO + qbase, (uint32_t)Nq * D * 2);
  const auto rk = make_rsrc(K + kbase, (uint32_t)Nk * D * 2);
  const auto rv = make_rsrc(V + kbase, (uint32_t)Nk * D * 2);

  // this wave's queries: Q and dO rows as B operands (n = query, k = d)
  const int qw0 = q0 + 32 * w;
  const int query = qw0 + l32;
  op8 qop[C::KSTEPS], dop[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    qop[kk] = __builtin_bit_cast(op8, buf_load16(rq, (uint32_t)query * C::ROWB + (16 * kk + 8 * h) * 2));
    dop[kk] = __builtin_bit_cast(op8, buf_load16(rdo, (uint32_t)query * C::ROWB + (16 * kk + 8 * h) * 2));
  }
  float Lq = 0.f, Dq = 0.f;
  if (query < Nq) {
    const float2 x = LD[sp.q_row0 + query];
    Lq = x.x;
    Dq = x.y;
  }
  __builtin_amdgcn_sched_barrier(0);

  uint32_t goff[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int row = (C::LPW * w + i) * C::RPI + lane / C::SPR, ps = lane % C::SPR;
    goff[i] = (uint32_t)row * C::ROWB + 16 * (ps ^ bswz<D>(row));
  }
  auto issue = [&](int st, char* kt, char* vt) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(st * C::BS) * C::ROWB;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      bwd_load_lds16(rk, kt + 1024 * (C::LPW * w + i), base + goff[i]);
      bwd_load_lds16(rv, vt + 1024 * (C::LPW * w + i), base + goff[i]);
    }
  };
  uint32_t ra[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) ra[kk] = l32 * C::ROWB + 16 * ((2 * kk + h) ^ bswz<D>(l32));
  // lane r16 of each 16 points at row (r16/4) + 4h (+ 8 for the upper half,
  // + 16 ti), columns 32 nb + 16 g1 + 4 (r16%4) .. +3: byte offset
  // tr_base[hi] + ((64 nb) ^ tr_x[hi]) + 32 ti ROWB, with the swizzle folded into tr_x
  uint32_t tr_base[2], tr_x[2];
  {
    const int r16 = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = (r16 >> 2) + 4 * h + 8 * hi;
      tr_base[hi] = row * C::ROWB + 8 * (r16 & 1);
      tr_x[hi] = 16 * ((2 * g1 + ((r16 & 3) >> 1)) ^ bswz<D>(row));
    }
  }
  auto tr_load = [&](const char* t, int nb, int ti) __attribute__((always_inline)) {
    const s16x4 lo = lds_read_tr16(t, tr_base[0] + ((64u * nb) ^ tr_x[0]) + 16 * ti * C::ROWB);
    const s16x4 hi = lds_read_tr16(t, tr_base[1] + ((64u * nb) ^ tr_x[1]) + 16 * ti * C::ROWB);
    return __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 dq[C::NBD];
#pragma unroll
  for (int nb = 0; nb < C::NBD; ++nb) dq[nb] = f32x16{};

  // step: keys j0 .. j0+31 from tiles kt, vt
  auto step = [&](int st, const char* kt, const char* vt) __attribute__((always_inline)) {
    const int j0 = st * C::BS;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      s = M::mma(lds_load<op8>(kt, ra[kk]), qop[kk], s);
      dp = M::mma(lds_load<op8>(vt, ra[kk]), dop[kk], dp);
    }
    // element i: key j0 + 8 (i/4) + 4h + i%4 of this lane's query
    const bool edge = (j0 + C::BS > Nk) || (CAUSAL && j0 + 31 > qw0 + off);
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -Lq));
    // masked pairs only on edge steps (a uniform branch, as in bwd_kv)
    if (edge) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = j0 + 8 * (i >> 2) + 4 * h + (i & 3);
        const uint32_t hide = (kj >= Nk || (CAUSAL && kj > query + off)) ? 0xFFFFFFFFu : 0u;
        const float v = s[i];
        s[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & ~hide);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = s[i] * (dp[i] - Dq);
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const op8 da = pack8<M>(dp, 8 * ti);
#pragma unroll
      for (int nb = 0; nb < C::NBD; ++nb) dq[nb] = M::mma(da, tr_load(kt, nb, ti), dq[nb]);
    }
  };

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + C::BO, Nq) - 1 + off + 1);
  const int ns = (kv_end + C::BS - 1) / C::BS;
  issue(0, k0s, v0s);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < ns; st += 2) {
    if (st + 1 < ns) issue(st + 1, k1s, v1s);
    step(st, k0s, v0s);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (st + 1 < ns) {
      if (st + 2 < ns) issue(st + 2, k0s, v0s);
      step(st + 1, k1s, v1s);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // element i of block nb: query qw0 + 8 (i/4) + 4h + i%4, column 32 nb + l32
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int qr = qw0 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (qr < Nq) {
      uint16_t* pq = dQ + qbase + (size_t)qr * D + l32;
#pragma unroll
      for (int nb = 0; nb < C::NBD; ++nb) pq[32 * nb] = to_half_bits<BF16>(dq[nb][i] * scale);
    }
  }
}

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, const SeqShape& sh, int nseq, int max_nq,
                        int max_nk, long q_rows, float scale, void* workspace, hipStream_t stream) {
  using C = BwdCfg<D>;
  float2* ld = static_cast<float2*>(workspace);
  constexpr int RPB = 256 / (D / 8);  // rows per bwd_pre block
  // a packed batch may have no query rows at all (its keys still get dK = dV = 0);
  // a grid of zero blocks is a launch error, so the preprocess is skipped then
  if (q_rows > 0) {
    hipLaunchKernelGGL((bwd_pre_kernel<D, BF16>), dim3((unsigned)((q_rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), lse, ld, q_rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const float c = scale * kLog2e;
  const int nkb = (max_nk + C::BO - 1) / C::BO;
  const int totk = nkb * nseq * (sh.H / sh.group);
  if (totk > 0) {
    const int chunk = sh.cu_q != nullptr ? totk / nkb : max(1, totk / nkb / 8);
    // the split kernel at d = 128 on dense non-causal grids, where every
    // workgroup walks all query steps; causal and packed grids have short key
    // blocks whose fixed costs the two workgroups per CU of the other kernel
    // overlap better than the split kernel's one
    bool split = false;
    if constexpr (D == 128 && !CAUSAL) split = sh.cu_q == nullptr;
    if (split) {
      if constexpr (D == 128 && !CAUSAL)
        hipLaunchKernelGGL((bwd_kv_pp_kernel<BF16>), dim3(totk), dim3(512), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), ld,
                           static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), sh, c, scale, nkb, totk);
    } else {
      hipLaunchKernelGGL((bwd_kv_kernel<D, BF16, CAUSAL>), dim3(totk), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), ld,
                         static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), sh, c, scale, nkb, totk, chunk);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nqb = (max_nq + C::BO - 1) / C::BO;
  const int totq = nqb * nseq * sh.H;
  if (totq > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, CAUSAL>), dim3(totq), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), ld,
                       static_cast<uint16_t*>(dq), sh, c, scale, nqb, totq,
                       sh.cu_q != nullptr ? totq / nqb : max(1, totq / nqb / 8));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, const SeqShape& sh, int nseq, int max_nq, int max_nk, long q_rows,
                      int d, float scale, bool causal, bool bf16, void* workspace, hipStream_t stream) {
#define ATTN_BWD(D_, BF_, CA_)                                                                                \
  if (d == D_ && bf16 == BF_ && causal == CA_)                                                                \
    return launch_bwd_t<D_, BF_, CA_>(q, k, v, out, dout, lse, dq, dk, dv, sh, nseq, max_nq, max_nk, q_rows,  \
                                      scale, workspace, stream);
  ATTN_BWD(128, true, false)
  ATTN_BWD(128, true, true)
  ATTN_BWD(128, false, false)
  ATTN_BWD(128, false, true)
  ATTN_BWD(64, true, false)
  ATTN_BWD(64, true, true)
  ATTN_BWD(64, false, false)
  ATTN_BWD(64, false, true)
#undef ATTN_BWD
  return hipErrorInvalidValue;
}

}  // namespace attn
