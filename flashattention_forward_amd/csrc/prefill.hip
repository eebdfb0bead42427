// Tiled FlashAttention forward (prefill) for gfx950, bf16/fp16, d in {64, 128}.
//
// The method is the tiled online softmax of "The Flash Attention algorithm"
// and "The online softmax recurrence" (marketmaker.cc post "Can a full
// trading day of context beat one minute? Flash attention and the
// sequence-length question"): Q is cut into row blocks, K/V into column
// blocks, and per query row a running max m, running sum l and an fp32
// output accumulator are carried across the key blocks, so the score matrix
// never leaves the chip.  Schedule choices follow that post's "FA2" section:
// the grid spans query blocks as well as (batch, head), each wave owns its
// own 32 query rows (no cross-wave reductions), and the division by l is
// deferred to the end.  Causal blocks stop at the diagonal ("Causal
// masking": tiles holding only future keys are never loaded).
//
// gfx950 mapping (one workgroup = 4 waves = 128 query rows, key tiles of 64):
//   * S^T = K Q^T on 32x32x16 MFMA: the K tile (LDS) is the A operand and the
//     wave's Q rows (VGPRs, loaded once) the B operand.  Working on S^T puts
//     one query per lane (16 keys in each of lanes l and l^32), so the row
//     max is 31 in-lane max ops and one exchange between the two half-waves.
//   * O^T += V^T P^T on 32x32x16 MFMA: P^T is the S^T accumulator converted
//     in registers (no LDS round trip: the accumulator layout of S^T is the
//     B-operand layout once the keys of each 16-key step are taken in the
//     order the accumulator holds them); V^T comes from the row-major V tile
//     through the gfx950 transposing LDS read, with the same key order.
//   * Softmax in the exp2 domain: p = exp2(s * scale * log2(e) - m), one FMA
//     and one v_exp_f32 per score; the row sum l adds the fp32 P (rounding P
//     to bf16 first would cost up to 2^-8 of l on rows with few keys).
//   * The running max is only raised when a tile's max exceeds it by more
//     than 2^8 (the adaptive rescaling of "Smarter online softmax rescaling"
//     in the linux-konsole.com post "FlashAttention 4: fast, memory-efficient
//     attention for LLMs"): P then stays below 2^8, and O and l are rescaled
//     only on those rare tiles.  The result is exact after the final 1/l.
//   * K/V tiles are staged through registers: the global loads of tile t+1
//     are issued before the MFMAs of tile t and written to LDS after it.
//   * LDS rows are padded (K: +16 B, V: +64 B per row) so the 16-byte K reads
//     and the transposing V reads of one wave fall on distinct banks.
//   * Workgroups are renumbered so each XCD walks a contiguous range of
//     (head, query block) items (K/V of a head stay in that XCD's L2);
//     causal grids start with the longest (bottom) query blocks.
#include "common.h"
#include "internal.h"

namespace attn {

template <int D>
struct PrefillCfg {
  static constexpr int BM = 128;              // query rows per workgroup
  static constexpr int BN = 64;               // keys per tile
  static constexpr int NT = 256;              // threads (4 waves)
  static constexpr int KSTRIDE = D * 2 + 16;  // LDS bytes per K row
  static constexpr int VSTRIDE = D * 2 + 64;  // LDS bytes per V row
  static constexpr int KBYTES = BN * KSTRIDE;
  static constexpr int VBYTES = BN * VSTRIDE;
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int RPP = NT / CPR;        // rows per staging pass
  static constexpr int PASSES = BN / RPP;
  static constexpr int KSTEPS = D / 16;       // k-steps of S^T = K Q^T
  static constexpr int MB_O = D / 32;         // 32-row blocks of O^T
};

// Raise the running max only when a tile exceeds it by more than this
// (log2 units): P = exp2(s - m) then stays below 2^8.
constexpr float kRescaleThreshold = 8.0f;

typedef short s16x8 __attribute__((ext_vector_type(8)));

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void prefill_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Nq, int Nk, float c, int nqb, int total) {
  using C = PrefillCfg<D>;
  using M = Mfma<BF16>;
  typedef typename M::op8 op8;
  typedef typename M::op2 op2;
  __shared__ __attribute__((aligned(16))) char smem[C::KBYTES + C::VBYTES];
  char* lk = smem;
  char* lv = smem + C::KBYTES;

  const int logical = xcd_remap(blockIdx.x, total);
  const int bh = logical / nqb;
  int qb = logical - bh * nqb;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest query blocks first
  const int q0 = qb * C::BM;
  const int off = Nk - Nq;        // bottom-right causal alignment

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const size_t qbase = (size_t)bh * Nq * D;
  const size_t kbase = (size_t)bh * Nk * D;

  // B operand of S^T = K Q^T: lane holds Q[qrow][16kk + 8h .. +7].
  const int qrow = q0 + 32 * w + l32;
  op8 qop[C::KSTEPS];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(Q + qbase + (size_t)qrow * D);
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < Nq) x = src[2 * kk + h];
      qop[kk] = __builtin_bit_cast(op8, x);
    }
  }

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + C::BM, Nq) - 1 + off + 1);
  const int ntiles = (kv_end + C::BN - 1) / C::BN;

  // register staging of one K/V tile
  u32x4 kreg[C::PASSES], vreg[C::PASSES];
  auto gload = [&](int t) {
    const int kv0 = t * C::BN;
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int row = p * C::RPP + tid / C::CPR, ch = tid % C::CPR;
      const int key = kv0 + row;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < Nk) {
        a = reinterpret_cast<const u32x4*>(K + kbase + (size_t)key * D)[ch];
        b = reinterpret_cast<const u32x4*>(V + kbase + (size_t)key * D)[ch];
      }
      kreg[p] = a;
      vreg[p] = b;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int row = p * C::RPP + tid / C::CPR, ch = tid % C::CPR;
      lds_store<u32x4>(lk, row * C::KSTRIDE + ch * 16, kreg[p]);
      lds_store<u32x4>(lv, row * C::VSTRIDE + ch * 16, vreg[p]);
    }
  };

  f32x16 o[C::MB_O];
#pragma unroll
  for (int mb = 0; mb < C::MB_O; ++mb) o[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int qmin_w = q0 + 32 * w;  // smallest query row of this wave

  gload(0);
  lstore();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) gload(t + 1);
    const int kv0 = t * C::BN;
    // whole tile in this wave's future: nothing to add
    const bool skip = CAUSAL && (kv0 > qmin_w + 31 + off);
    if (!skip) {
      // ---- S^T = K Q^T  (two 32-key blocks)
      f32x16 s[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        s[nb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk) {
          const op8 a = lds_load<op8>(lk, (32 * nb + l32) * C::KSTRIDE + (16 * kk + 8 * h) * 2);
          s[nb] = M::mma(a, qop[kk], s[nb]);
        }
      }
      // ---- masks: key tail, causal diagonal
      const bool need_mask = (kv0 + C::BN > Nk) || (CAUSAL && kv0 + C::BN - 1 > qmin_w + off);
      if (need_mask) {
        const int qlim = CAUSAL ? (qrow + off) : 0x7fffffff;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + 32 * nb + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key >= Nk || key > qlim) s[nb][i] = -INFINITY;
          }
      }
      // ---- row max over the tile (this lane's 32 keys, then the other half-wave)
      float mx = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mt = mx * c;
      if (__any(mt > m_run + kRescaleThreshold)) {
        const float mn = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
        for (int mb = 0; mb < C::MB_O; ++mb) o[mb] *= alpha;
        l_run *= alpha;
        m_run = mn;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      // ---- P = exp2(s*c - m), packed to 16-bit B operands; l sums the fp32 P
      op8 pb[2][2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          op2 pr[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[nb][8 * tt + 2 * j], c, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[nb][8 * tt + 2 * j + 1], c, -m_use));
            pr[j] = M::pack2(p0, p1);
            l_run += p0 + p1;
          }
          pb[nb][tt] = __builtin_shufflevector(__builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3),
                                               __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
        }
      // ---- O^T += V^T P^T
      const int r16 = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
      for (int mb = 0; mb < C::MB_O; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int key0 = 32 * nb + 16 * tt + 4 * h;
            const uint32_t a0 = (key0 + (r16 >> 2)) * C::VSTRIDE + (32 * mb + 16 * g1 + 4 * (r16 & 3)) * 2;
            const s16x4 lo = lds_read_tr16(lv, a0);
            const s16x4 hi = lds_read_tr16(lv, a0 + 8 * C::VSTRIDE);
            const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[mb] = M::mma(__builtin_bit_cast(op8, a), pb[nb][tt], o[mb]);
          }
    }
    __syncthreads();
    if (t + 1 < ntiles) {
      lstore();
      __syncthreads();
    }
  }

  // ---- epilogue: combine the half-wave row sums, normalise, write O and LSE
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = 1.f / l_tot;
  if (qrow < Nq) {
    uint16_t* dst = O + qbase + (size_t)qrow * D;
#pragma unroll
    for (int mb = 0; mb < C::MB_O; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const op2 x0 = M::pack2(o[mb][4 * g + 0] * inv, o[mb][4 * g + 1] * inv);
        const op2 x1 = M::pack2(o[mb][4 * g + 2] * inv, o[mb][4 * g + 3] * inv);
        u32x2 u;
        u[0] = __builtin_bit_cast(uint32_t, x0);
        u[1] = __builtin_bit_cast(uint32_t, x1);
        *reinterpret_cast<u32x2*>(dst + 32 * mb + 8 * g + 4 * h) = u;
      }
    if (LSE != nullptr && h == 0) LSE[(size_t)bh * Nq + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool BF16, bool CAUSAL>
static hipError_t launch_t(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                           int Nq, int Nk, float scale, hipStream_t stream) {
  using C = PrefillCfg<D>;
  const int nqb = (Nq + C::BM - 1) / C::BM;
  const int total = nqb * B * H;
  hipLaunchKernelGGL((prefill_kernel<D, BF16, CAUSAL>), dim3(total), dim3(C::NT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse, Nq, Nk,
                     scale * kLog2e, nqb, total);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                          int Nq, int Nk, int d, float scale, bool causal, bool bf16, hipStream_t stream) {
#define ATTN_DISPATCH(D_, BF_, CA_) \
  if (d == D_ && bf16 == BF_ && causal == CA_) return launch_t<D_, BF_, CA_>(q, k, v, out, lse, B, H, Nq, Nk, scale, stream);
  ATTN_DISPATCH(128, true, false)
  ATTN_DISPATCH(128, true, true)
  ATTN_DISPATCH(128, false, false)
  ATTN_DISPATCH(128, false, true)
  ATTN_DISPATCH(64, true, false)
  ATTN_DISPATCH(64, true, true)
  ATTN_DISPATCH(64, false, false)
  ATTN_DISPATCH(64, false, true)
#undef ATTN_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace attn
