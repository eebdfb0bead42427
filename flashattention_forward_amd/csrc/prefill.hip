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
// gfx950 mapping, d = 128 (one workgroup = 8 waves = 256 query rows, key tiles
// of 64; d = 64 runs the interleaved kernel further below):
//   * S^T = K Q^T on 32x32x16 MFMA: the K tile (LDS) is the A operand and the
//     wave's Q rows (VGPRs, loaded once) the B operand.  Working on S^T puts
//     one query per lane (16 keys in each of lanes l and l^32), so the row
//     max is in-lane max ops and one exchange between the two half-waves.
//   * O^T += V^T P^T on 32x32x16 MFMA: P^T is the S^T accumulator converted
//     in registers (no LDS round trip: the accumulator layout of S^T is the
//     B-operand layout once the keys of each 16-key step are taken in the
//     order the accumulator holds them); V^T comes from the row-major V tile
//     through the gfx950 transposing LDS read, with the same key order.
//   * Softmax in the exp2 domain: p = exp2(s * scale * log2(e) - m), one FMA
//     and one v_exp_f32 per score; the row sum l adds the fp32 P (rounding P
//     to bf16 first would cost up to 2^-8 of l on rows with few keys).
//   * The running max is raised only when P would otherwise grow too large
//     (the adaptive rescaling of "Smarter online softmax rescaling" in the
//     linux-konsole.com post "FlashAttention 4: fast, memory-efficient
//     attention for LLMs"): P(t) is formed against the running max as it
//     stands, and only on a row's first tile, or when a lane's P over the
//     tile sums past 2^14, is the max raised, O and l rescaled and P(t)
//     formed again.  P stays at or below 2^14 (inside fp16), no tile max is
//     formed on the common path, and the result after the final 1/l does
//     not depend on where m stands.
//   * Two groups of 4 waves alternate: while one group runs the MFMAs of its
//     tile (S(t) and O += P(t-1) V(t-1), the two streams interleaved), the
//     other runs the softmax of its previous tile, so the matrix cores and
//     the vector ALUs of a SIMD (which holds one wave of each group) work at
//     the same time; a workgroup barrier ends every tile (every other phase).
//   * K/V tiles go from global memory straight into LDS (buffer loads with
//     the LDS-destination form, 1 KB per wave instruction), double-buffered;
//     only the waves in their MFMA phase issue them, one every other MFMA
//     step, and the buffer range check turns keys past Nk into zeros.  The
//     16-byte slots of each LDS row are XOR-swizzled on the load side so the
//     K operand reads and the transposing V reads hit distinct banks.
//   * The epilogue writes O through LDS, so that every global store covers
//     whole 128-byte pieces of rows, and on dense grids it first requests the
//     workgroup's next item's Q rows and first K tile, which then arrive
//     while O is written instead of after it.
//   * Workgroups are renumbered so each XCD walks a contiguous range of
//     (head, query block) items (K/V of a head stay in that XCD's L2).  A
//     causal grid with many heads gives each workgroup two query blocks, the
//     j-th longest and the j-th shortest, so all workgroups do equal work;
//     with few heads it takes single blocks, longest first.
#include "common.h"
#include "internal.h"

namespace attn {

template <int D>
struct PrefillCfg {
  static constexpr int BM = 256;             // query rows per workgroup: 2 groups x 4 waves x 32
  static constexpr int BN = D == 128 ? 64 : 128;  // keys per tile (multiple of 32)
  static constexpr int NB = BN / 32;         // 32-key blocks of S^T per tile
  static constexpr int NG = BN / 16;         // 16-key groups (k-steps of O^T) per tile
  static constexpr int NT = 512;             // threads (8 waves, 2 per SIMD)
  static constexpr int ROWB = D * 2;         // bytes per K/V row
  static constexpr int SPR = ROWB / 16;      // 16-byte slots per row
  static constexpr int TILEB = BN * ROWB;    // bytes per K or V tile in LDS
  static constexpr int RPI = 1024 / ROWB;    // rows per 1 KB direct-to-LDS wave load
  static constexpr int LPG = TILEB / 1024 / 4;  // such loads per tile for each of the 4 loading waves
  static constexpr int NLD = 2 * LPG;        // loads a wave issues per G phase (K tile, then V tile)
  static constexpr int KSTEPS = D / 16;      // k-steps of S^T = K Q^T
  static constexpr int MB_O = D / 32;        // 32-row blocks of O^T
  static constexpr int NA = NB * KSTEPS;     // MFMAs of S^T per tile
  static constexpr int NC = NG * MB_O;       // MFMAs of O^T per tile
  static_assert(NA == NC, "S and PV MFMA streams are interleaved one to one");
  static_assert(NA % NLD == 0, "loads are spread evenly over the MFMA steps");
};

// LDS swizzles (16-byte slot index XOR a function of the row), chosen so the
// MFMA operand reads of a wave hit distinct banks.  K: 16 lanes read one slot
// of 16 consecutive rows; V: 16-lane groups read 32 bytes of 4 consecutive
// rows for the transposing read.
template <int D>
__device__ __forceinline__ int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// exp2 on the FMA pipe, for the software-exp2 split of "Software exp2" in the
// linux-konsole.com post "FlashAttention 4: fast, memory-efficient attention
// for LLMs" (a share of the exponentials computed by a polynomial instead of
// the transcendental unit).  Range reduction 2^x = 2^n 2^f with n = floor(x),
// f = x - n in [0, 1) (exact in fp32), a cubic for 2^f, and 2^n added to the
// exponent field.  The cubic is our relative-error minimax fit of 2^f on
// [0, 1] (Remez exchange; flashattention_forward_amd/exp2_poly_fit.py
// reproduces these fp32 coefficients); its relative error is at most 7.5e-5,
// and arguments below -125 (masked keys, -inf) give 0; from -125 up to 128
// every result is a normal fp32 number, so adding n to the exponent field is
// exact; arguments from 128 up give +inf (the softmax's overflow check sees it).
constexpr float kExp2C0 = 0.9999251961708069f, kExp2C1 = 0.6958335638046265f, kExp2C2 = 0.22606715559959412f,
                kExp2C3 = 0.07802452147006989f;
__device__ __forceinline__ float exp2_poly(float x) {
  const float xc = fmaxf(x, -125.f);
  const float n = floorf(xc);
  const float f = xc - n;
  const float p = fmaf(fmaf(fmaf(kExp2C3, f, kExp2C2), f, kExp2C1), f, kExp2C0);
  const float r = __builtin_bit_cast(float, __builtin_bit_cast(int, p) + ((int)n << 23));
  return x < -125.f ? 0.f : (x >= 128.f ? INFINITY : r);
}

// Largest sum of one lane's probabilities in a tile, P = exp2(s c - m), before
// the running max m is raised: every P then stays at or below 2^14, inside the
// range of the fp16 P operand (largest finite 65504) and far inside that of
// bf16 and of the fp32 O and l accumulators; the result after the final
// division by l does not depend on m.
constexpr float kMaxTileSum = 16384.0f;

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Ping-pong schedule.  The two groups of 4 waves share the SIMDs pairwise and
// run the same tile sequence half a step apart.  Per tile t a wave has a GEMM
// phase G_t (S(t) = K(t) Q^T and O += P(t-1) V(t-1): MFMA only) and a softmax
// phase X_t (mask, running max, exp, row sum of S(t): VALU only).  Group 0
// runs G_t while group 1 runs X_{t-1}, then group 0 runs X_t while group 1
// runs G_t, with a workgroup barrier at the end of each tile, so on every SIMD
// one wave feeds the matrix cores while the other feeds the vector ALU.
// one 1 KB direct global -> LDS load: lane i's 16 bytes at voff land at dst + 16 i
// (a free function: the same builtin called from a lambda in the kernel made
// the host compilation pass drop the kernel's launch stub)
__device__ __forceinline__ void tile_load_lds(const __amdgpu_buffer_rsrc_t& r, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)dst, 16, voff, 0, 0, 0);
}

// SWX: how many of every 8 exponentials of the softmax take exp2_poly (the
// rest take v_exp_f32); 0 in the default forward
template <int D, bool BF16, bool CAUSAL, int SWX>
__global__ __launch_bounds__(512, 1) void prefill_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, SeqShape sh, float c, int nqb, int total, int paired,
    int persist) {
  using C = PrefillCfg<D>;
  using M = Mfma<BF16>;
  typedef typename M::op8 op8;
  typedef typename M::op2 op2;
  // two K and two V tile buffers: K(t), V(t-1) are read in phases 2t, 2t+1;
  // K(t+1) and V(t) arrive during them.  Four separate objects, each access
  // naming its buffer statically, so the compiler can tell the tile loads in
  // flight from the operand reads (one shared array would make every operand
  // read wait for the loads issued just before it).
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILEB];

  // work item: one 256-row query block of one (batch, head).  A paired causal
  // grid puts block nqb-1-j and block j in one workgroup (heavy one first), so
  // every workgroup walks the same number of key tiles; otherwise causal blocks
  // of a head are taken longest first.  Dense batches give each XCD a
  // contiguous range of heads (their K/V stay in its L2).  Packed batches, whose
  // sequences differ in length, instead take block rank j slowest over all
  // (sequence, head) pairs in plain dispatch order: the longest blocks of every
  // sequence start first and spread over all XCDs.
  // persist > 0: a grid of one workgroup per CU walks virtual blocks
  // blockIdx.x, blockIdx.x + gridDim.x, ... (gridDim.x a multiple of 8, so each
  // virtual block stays on its workgroup's XCD); otherwise one block each
  // the next item's Q operand and first K tile are requested during this item's
  // epilogue (dense grids): `pre` says they are in flight
  op8 qop[C::KSTEPS];
  bool pre = false;
  for (int vb = blockIdx.x; vb < total; vb += persist ? (int)gridDim.x : total) {
    const bool packed = sh.cu_q != nullptr;
    const int logical = packed ? vb : xcd_remap(vb, total);
    const int per_head = paired ? (nqb + 1) / 2 : nqb;
    int bh, j_item;
    if (packed) {
      const int nh = total / per_head;
      j_item = logical / nh;
      bh = logical - j_item * nh;
    } else {
      bh = logical / per_head;
      j_item = logical - bh * per_head;
    }
    const int nitems = (paired && nqb - 1 - j_item != j_item) ? 2 : 1;
    // this (sequence, head)'s rows; Nq and Nk are its own lengths from here on
    const SeqSpan sp = seq_span(sh, bh / sh.H, bh % sh.H);
    const int Nq = sp.nq, Nk = sp.nk;
    const int off = Nk - Nq;        // bottom-right causal alignment

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int grp = w >> 2, wg = w & 3;
    const int h = lane >> 5, l32 = lane & 31;
    const size_t qbase = sp.q_row0 * D;
    const size_t kbase = sp.k_row0 * D;
    const auto rq = make_rsrc(Q + qbase, (uint32_t)Nq * D * 2);
    const auto rk = make_rsrc(K + kbase, (uint32_t)Nk * D * 2);
    const auto rv = make_rsrc(V + kbase, (uint32_t)Nk * D * 2);

    // direct global -> LDS loads of one tile, issued by the 4 waves of group 0
    // only: wave wg fills 1 KB blocks LPG*wg .. LPG*wg + LPG-1; lane i lands at
    // byte 16 i of its block (row i/SPR, slot i%SPR) and therefore fetches
    // global chunk slot ^ swizzle(row).  Keys past Nk read as 0 (buffer range check).
    uint32_t gk_off[C::LPG], gv_off[C::LPG];
#pragma unroll
    for (int i = 0; i < C::LPG; ++i) {
      const int blk = C::LPG * wg + i;
      const int row = blk * C::RPI + lane / C::SPR, slot = lane % C::SPR;
      gk_off[i] = (uint32_t)row * C::ROWB + 16 * (slot ^ k_swz<D>(row));
      gv_off[i] = (uint32_t)row * C::ROWB + 16 * (slot ^ v_swz<D>(row));
    }
    // load q of the NLD a wave issues per G phase: K(tk) blocks first, then V(tv)
    typedef __amdgpu_buffer_rsrc_t Rsrc;
    auto issue_load = [&](const Rsrc& rk_, const Rsrc& rv_, int q, char* ldk, char* ldv, int tk, int tv) {
      if (q < C::LPG)
        tile_load_lds(rk_, ldk + 1024 * (C::LPG * wg + q), (uint32_t)tk * C::TILEB + gk_off[q]);
      else
        tile_load_lds(rv_, ldv + 1024 * (C::LPG * wg + q - C::LPG), (uint32_t)tv * C::TILEB + gv_off[q - C::LPG]);
    };
    // per-lane LDS operand offsets (constant across tiles)
    uint32_t ka_off[C::KSTEPS];  // K operand, row l32 (+32 per key block), logical slot 2kk+h
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) ka_off[kk] = l32 * C::ROWB + 16 * ((2 * kk + h) ^ k_swz<D>(l32));
    const int r16 = lane & 15, g1 = (lane >> 4) & 1;
    const int vrow = (r16 >> 2) + 4 * h;  // + 16 per key group, + 8 for the second read
    uint32_t va_off[C::MB_O];            // V^T operand: columns 32mb + 16g1 + 4(r16&3)
#pragma unroll
    for (int mb = 0; mb < C::MB_O; ++mb) {
      const int col = 32 * mb + 16 * g1 + 4 * (r16 & 3);
      va_off[mb] = vrow * C::ROWB + 16 * ((col >> 3) ^ v_swz<D>(vrow)) + 2 * (col & 7);
    }
    auto ka_load = [&](const char* lk, int i) {  // K operand of S^T step i: key block i/KSTEPS, k-step i%KSTEPS
      return lds_load<op8>(lk, ka_off[i % C::KSTEPS] + (i / C::KSTEPS) * 32 * C::ROWB);
    };
    auto va_load = [&](const char* lv, int j) {  // V^T operand of O^T step j: 16-key group j/MB_O, d block j%MB_O
      const uint32_t a0 = va_off[j % C::MB_O] + 16 * (j / C::MB_O) * C::ROWB;
      const s16x4 lo = lds_read_tr16(lv, a0);
      const s16x4 hi = lds_read_tr16(lv, a0 + 8 * C::ROWB);
      return __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    for (int item = 0; item < nitems; ++item) {
      const int qb = paired ? (item == 0 ? nqb - 1 - j_item : j_item) : (CAUSAL ? nqb - 1 - j_item : j_item);
      const int q0 = qb * C::BM;
      if (q0 >= Nq) continue;  // past a short packed sequence (uniform over the workgroup)
      // B operand of S^T = K Q^T: lane holds Q[qrow][16kk + 8h .. +7]; rows past Nq read as 0
      const int qmin_w = q0 + 128 * grp + 32 * wg;  // smallest query row of this wave
      const int qrow = qmin_w + l32;
      if (!pre) {
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk)
          qop[kk] = __builtin_bit_cast(op8, buf_load16(rq, (uint32_t)qrow * C::ROWB + (16 * kk + 8 * h) * 2));
      }
      // keep the Q loads ahead of the first tile's: the in-order load counter then
      // retires them before the first tile is read, and no wait on them lands in the loop
      __builtin_amdgcn_sched_barrier(0);

      int kv_end = Nk;
      if (CAUSAL) kv_end = min(Nk, min(q0 + C::BM, Nq) - 1 + off + 1);
      const int T = max(0, (kv_end + C::BN - 1) / C::BN);  // 0: no key visible to the block
      // tiles this wave group's rows can see: on a causal block the first group
      // (the block's first 128 rows) stops up to two tiles before the second
      int Tg = T;
      if (CAUSAL) Tg = min(T, max(0, (min(Nk, min(q0 + 128 * grp + 128, Nq) + off) + C::BN - 1) / C::BN));

      f32x16 o[C::MB_O];
#pragma unroll
      for (int mb = 0; mb < C::MB_O; ++mb) o[mb] = f32x16{};
      f32x16 s[C::NB];  // S(t) between its GEMM and softmax phases
      op8 pb[C::NG];    // P(t) between its softmax phase and the next GEMM phase
      float m_run = -INFINITY, l_run = 0.f;

      // P of one half of the key blocks of S(t) against the reference m_ref: half 0
      // is S blocks [0, NB/2) -> P groups [0, NG/2), half 1 the rest.  Writes those
      // P groups and returns this lane's sum of the P it formed.
      auto exps_half = [&](int half, float m_ref) {
        float lsum[4];
#pragma unroll
        for (int gg = 0; gg < C::NG / 2; ++gg) {
          const int g = half * (C::NG / 2) + gg;
          const int nb = g >> 1, tt = g & 1;
          op2 pr[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = fmaf(s[nb][8 * tt + 2 * j], c, -m_ref);
            const float x1 = fmaf(s[nb][8 * tt + 2 * j + 1], c, -m_ref);
            const float p0 = 2 * j < SWX ? exp2_poly(x0) : __builtin_amdgcn_exp2f(x0);
            const float p1 = 2 * j + 1 < SWX ? exp2_poly(x1) : __builtin_amdgcn_exp2f(x1);
            pr[j] = M::pack2(p0, p1);
            lsum[j] = gg == 0 ? p0 + p1 : lsum[j] + (p0 + p1);
          }
          pb[g] = __builtin_shufflevector(__builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3),
                                          __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
        }
        return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
      };
      // tile t holds keys a row of this wave must not see (causal diagonal, or keys
      // past Nk): wave-uniform
      auto edge_tile = [&](int t) {
        const int kv0 = t * C::BN;
        return (kv0 + C::BN > Nk) || (CAUSAL && kv0 + C::BN - 1 > qmin_w + off);
      };

      // ---- G_t: S(t) (t < T) and O += P(t-1) V(t-1) (t >= 1), MFMA streams interleaved;
      // lk holds K(t), lv holds V(t-1).  With LD (group 0) it also issues the loads
      // of K(t+1) into ldk and V(t) into ldv, one every STEP MFMA steps, so that the
      // address unit sees a steady trickle rather than every wave's loads at once.
      // K(t+1) is loaded even when t+1 = T: those rows read as 0 or are never used.
      auto gemm_phase = [&](const Rsrc& rk_, const Rsrc& rv_, bool LD, int t, const char* lk, const char* lv,
                            char* ldk, char* ldv) {
        constexpr int STEP = C::NA / C::NLD;
        const bool do_s = t < (CAUSAL ? Tg : T), do_pv = t >= 1 && (!CAUSAL || t <= Tg);
        if (do_s && do_pv) {
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) s[nb] = f32x16{};
          constexpr int PF = 4;  // operand reads in flight per stream
          op8 ka[PF], va[PF];
#pragma unroll
          for (int i = 0; i < PF; ++i) {
            ka[i] = ka_load(lk, i);
            va[i] = va_load(lv, i);
          }
#pragma unroll
          for (int i = 0; i < C::NA; ++i) {
            const op8 a = ka[i % PF], b = va[i % PF];
            if (i + PF < C::NA) {
              ka[i % PF] = ka_load(lk, i + PF);
              va[i % PF] = va_load(lv, i + PF);
            }
            s[i / C::KSTEPS] = M::mma(a, qop[i % C::KSTEPS], s[i / C::KSTEPS]);
            o[i % C::MB_O] = M::mma(b, pb[i / C::MB_O], o[i % C::MB_O]);
            if (LD && i % STEP == STEP - 1) issue_load(rk_, rv_, i / STEP, ldk, ldv, t + 1, t);
          }
          // issue order: the first PF steps' operand reads, then per step its two
          // MFMAs each followed by the reads of the step PF ahead, then its load
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 3 * PF, 0);
#pragma unroll
          for (int i = 0; i < C::NA; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (i + PF < C::NA) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (i + PF < C::NA) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            if (LD && i % STEP == STEP - 1) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
          }
        } else if (do_s) {
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) s[nb] = f32x16{};
          op8 ka[2];
          ka[0] = ka_load(lk, 0);
          ka[1] = ka_load(lk, 1);
#pragma unroll
          for (int i = 0; i < C::NA; ++i) {
            const op8 a = ka[i & 1];
            if (i + 2 < C::NA) ka[i & 1] = ka_load(lk, i + 2);
            s[i / C::KSTEPS] = M::mma(a, qop[i % C::KSTEPS], s[i / C::KSTEPS]);
            if (LD && i % STEP == STEP - 1) issue_load(rk_, rv_, i / STEP, ldk, ldv, t + 1, t);
          }
        } else {
          // past this group's last tile the loading group still fetches the
          // other group's tiles
          if (CAUSAL && LD && t < T) {
#pragma unroll
            for (int q = 0; q < C::NLD; ++q) issue_load(rk_, rv_, q, ldk, ldv, t + 1, t);
          }
          if (do_pv) {
            op8 va[2];
            va[0] = va_load(lv, 0);
            va[1] = va_load(lv, 1);
#pragma unroll
            for (int i = 0; i < C::NC; ++i) {
              const op8 b = va[i & 1];
              if (i + 2 < C::NC) va[i & 1] = va_load(lv, i + 2);
              o[i % C::MB_O] = M::mma(b, pb[i / C::MB_O], o[i % C::MB_O]);
            }
          }
        }
      };

      // ---- X_t: mask, running max, rescale, P(t) = exp2(S c - m), row sum
      auto softmax_phase = [&](int t) {
        if (CAUSAL && t >= Tg) return;
        const int kv0 = t * C::BN;
        const bool edge = edge_tile(t);
        if (edge) {
          // element i of block nb holds key kv0 + 4h + e with e = 32 nb + 8 (i/4) + i%4;
          // it is visible iff e <= lim.  The select is a bit blend with the all-ones
          // or all-zeros word (lim - e) >> 31, so no per-element compare results
          // have to be held in scalar registers.
          const int lim = min(Nk - 1, CAUSAL ? qrow + off : Nk - 1) - (kv0 + 4 * h);
          constexpr uint32_t kNegInf = 0xFF800000u;
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int e = 32 * nb + 8 * (i >> 2) + (i & 3);
              const uint32_t hide = (uint32_t)((lim - e) >> 31);
              // the element is copied out first: a bit cast applied to a vector
              // element lvalue in place read element 0 of the vector here
              const float v = s[nb][i];
              const uint32_t bits = __builtin_bit_cast(uint32_t, v);
              s[nb][i] = __builtin_bit_cast(float, (bits & ~hide) | (kNegInf & hide));
            }
        }
        // P(t) against the running max as it stands.  The tile's own row max is
        // only formed when that fails: on a row's first tile (no max yet), or when
        // a lane's probabilities would sum past kMaxTileSum.  Then the running max
        // is raised to the row max, O and l are rescaled, and P(t) is formed again.
        const bool first = __any(m_run == -INFINITY);
        float tot = 0.f;
        bool raise = first;
        if (!first) {
          tot = exps_half(0, m_run) + exps_half(1, m_run);
          // not (tot <= bound) also catches an overflow to inf
          raise = __any(!(tot <= kMaxTileSum));
        }
        // the row max is formed only here, on the rare raising tiles (a loop around
        // both paths let the compiler hoist it onto every tile)
        if (raise) {
          float mx[C::NB];
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) {
            mx[nb] = fmaxf(s[nb][0], s[nb][1]);
#pragma unroll
            for (int i = 2; i < 16; ++i) mx[nb] = fmaxf(mx[nb], s[nb][i]);
          }
#pragma unroll
          for (int nb = 1; nb < C::NB; ++nb) mx[0] = fmaxf(mx[0], mx[nb]);
          const float m_new = fmaxf(m_run, pair_max(mx[0]) * c);
          const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
          for (int mb = 0; mb < C::MB_O; ++mb) o[mb] *= alpha;
          l_run *= alpha;
          m_run = m_new;
          // a row that has seen no visible key keeps m = -inf: exponent base 0, P = 0
          const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
          tot = exps_half(0, m_use) + exps_half(1, m_use);
        }
        l_run += tot;
      };

      // prologue: K(0) into LDS, unless the previous item's epilogue requested it
      // together with Q; then only the previous item's 8 O stores per wave, issued
      // after those loads, may still be in flight (vmcnt 8, lgkmcnt 0)
      if (!pre) {
        if (grp == 0) {
#pragma unroll
          for (int q = 0; q < C::LPG; ++q) issue_load(rk, rv, q, k0s, nullptr, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);
      } else {
        // s_waitcnt immediate 0x0078: vmcnt 8 (bits 3:0, 15:14), expcnt 7 = no
        // wait (bits 6:4), lgkmcnt 0 (bits 11:8)
        __builtin_amdgcn_s_waitcnt(0x0078);
      }
      __syncthreads();

      // phase p: group 0 runs phase p of its own sequence G_0 X_0 G_1 X_1 ... G_T,
      // group 1 runs phase p-1.  K(s+1) and V(s) are loaded by group 0 during its
      // G_s in phase 2s (into buffers last read in phases 2s-2 and 2s-1) and
      // waited for at the end of phase 2s+1.  K(t) lives in buffer t%2, V(t) in
      // buffer t%2, so the buffer roles repeat every 4 phases.
      auto phase = [&](const Rsrc& rk_, const Rsrc& rv_, bool EVEN, int p, const char* gk, const char* gv, char* ldk,
                       char* ldv) {
        const int mp = p - grp;
        if (mp >= 0 && mp <= 2 * T) {
          if ((mp & 1) == 0) {
            __builtin_amdgcn_s_setprio(1);
            gemm_phase(rk_, rv_, EVEN, mp >> 1, gk, gv, ldk, ldv);
            __builtin_amdgcn_s_setprio(0);
          } else {
            softmax_phase(mp >> 1);
          }
        }
        if (!EVEN) {
          // once per tile: the tile loads issued in phase p-1 have landed in every
          // wave's part of LDS, and every wave is done with the buffers they replace
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
        }
        // no barrier after even phases: nothing read in phase p+1 was written in
        // phase p, and letting the groups drift within a tile measured faster
        // than holding them in step
      };
      const int nphase = 2 * T + 2;  // even
      for (int p = 0; p < nphase; p += 4) {
        phase(rk, rv, true, p, k0s, v1s, k1s, v0s);  // G of even t: K(t) in k0, V(t-1) in v1; loads K(t+1)->k1, V(t)->v0
        phase(rk, rv, false, p + 1, k0s, v1s, k1s, v0s);
        if (p + 2 < nphase) {
          phase(rk, rv, true, p + 2, k1s, v0s, k0s, v1s);  // G of odd t
          phase(rk, rv, false, p + 3, k1s, v0s, k0s, v1s);
        }
      }

      // ---- epilogue: combine the half-wave row sums, normalise, write O and LSE
      // a row that saw no key (packed batches only) has l = 0: O = 0, LSE = -inf
      const float l_tot = pair_sum(l_run);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      static_assert(D % 64 == 0, "O is staged 64 columns at a time");
      if (qrow < Nq && LSE != nullptr && h == 0) LSE[sp.q_row0 + qrow] = (m_run + __log2f(l_tot)) * kLn2;
      // the next item of this workgroup (dense grids): the second block of a
      // causal pair (same head), else the first block of the next virtual
      // block.  Its Q rows go straight into qop (dead since this item's last S)
      // and group 0 loads its K(0) into k0s (no wave reads K after the item's
      // last barrier); both land while this item's O is written.
      pre = false;
      if (!packed) {
        int nbh = bh, nqblk = -1;
        if (item + 1 < nitems) {
          nqblk = j_item;
        } else if (persist && vb + (int)gridDim.x < total) {
          const int lg = xcd_remap(vb + (int)gridDim.x, total);
          nbh = lg / per_head;
          const int nj = lg - nbh * per_head;
          nqblk = (CAUSAL || paired) ? nqb - 1 - nj : nj;
        }
        if (nqblk >= 0) {
          const SeqSpan sn = seq_span(sh, nbh / sh.H, nbh % sh.H);
          const auto rqn = make_rsrc(Q + sn.q_row0 * D, (uint32_t)sn.nq * D * 2);
          const auto rkn = make_rsrc(K + sn.k_row0 * D, (uint32_t)sn.nk * D * 2);
          const int qrn = nqblk * C::BM + 128 * grp + 32 * wg + l32;
#pragma unroll
          for (int kk = 0; kk < C::KSTEPS; ++kk)
            qop[kk] = __builtin_bit_cast(op8, buf_load16(rqn, (uint32_t)qrn * C::ROWB + (16 * kk + 8 * h) * 2));
          if (grp == 0) {
#pragma unroll
            for (int q = 0; q < C::LPG; ++q) issue_load(rkn, rkn, q, k0s, nullptr, 0, 0);
          }
          pre = true;
        }
      }
      // the 8 O stores below must follow those loads (the next item waits for
      // the loads with vmcnt 8)
      __builtin_amdgcn_sched_barrier(0);
      // O leaves through LDS, so that every global store writes whole 128-byte
      // pieces of rows (the accumulator layout gives a lane 8-byte pieces of one
      // row, 16 bytes apart).  Each wave stages its 32 rows 64 columns at a time
      // in a private 4 KB region of the V tile buffers, which no wave reads or
      // loads into between the item's last barrier and the next item's first;
      // 16-byte chunks are XOR-swizzled by row.
      char* const stg = (w < 4 ? v0s : v1s) + (w & 3) * 4096;
      // O stores through a buffer resource over this head's rows: rows past Nq
      // fall outside it and are dropped, so every wave issues exactly 8 stores
      const auto ro = make_rsrc(O + qbase, (uint32_t)Nq * D * 2);
      // lane index made opaque here, so that the staging addresses (the same for
      // every item) are formed in the epilogue instead of being kept in registers
      // across the tile loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int sr = ln & 31, sh_ = ln >> 5;
#pragma unroll
      for (int pass = 0; pass < D / 64; ++pass) {
#pragma unroll
        for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int mb = 2 * pass + mb2, chunk = 4 * mb2 + g;
            const op2 x0 = M::pack2(o[mb][4 * g + 0] * inv, o[mb][4 * g + 1] * inv);
            const op2 x1 = M::pack2(o[mb][4 * g + 2] * inv, o[mb][4 * g + 3] * inv);
            u32x2 u;
            u[0] = __builtin_bit_cast(uint32_t, x0);
            u[1] = __builtin_bit_cast(uint32_t, x1);
            lds_store<u32x2>(stg, sr * 128 + 16 * (chunk ^ (sr & 7)) + 8 * sh_, u);
          }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 8 * j + (ln >> 3), c = ln & 7;
          const u32x4 x = lds_load<u32x4>(stg, r * 128 + 16 * (c ^ (r & 7)));
          __builtin_amdgcn_raw_buffer_store_b128(x, ro, (uint32_t)(qmin_w + r) * C::ROWB + 128 * pass + 16 * c, 0, 0);
        }
      }
    }  // work items
  }  // virtual blocks
}

// compute units of the current device (asked on every call: no cached state)
static int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

template <int D, bool BF16, bool CAUSAL, int SWX = 0>
static hipError_t launch_t(const void* q, const void* k, const void* v, void* out, float* lse, const SeqShape& sh,
                           int nseq, int max_nq, float scale, hipStream_t stream) {
  using C = PrefillCfg<D>;
  const int nqb = (max_nq + C::BM - 1) / C::BM;
  // pair causal blocks when the paired grid still fills every CU several times
  // over (otherwise the last round of workgroups would run on few CUs); packed
  // batches have blocks of unequal length and are never paired
  const long pairs = (long)((nqb + 1) / 2) * nseq * sh.H;
  const int paired = (CAUSAL && sh.cu_q == nullptr && pairs >= 4L * device_cu_count()) ? 1 : 0;
  const int total = (paired ? (nqb + 1) / 2 : nqb) * nseq * sh.H;
  if (total == 0) return hipSuccess;
  // items of equal work (dense non-causal, or paired causal) run on a
  // persistent grid of one workgroup per CU: no workgroup launch between
  // items; packed and unpaired causal grids keep the hardware's dynamic order
  const int cus = device_cu_count() & ~7;
  const int persist = (sh.cu_q == nullptr && (!CAUSAL || paired) && cus >= 8 && total > cus) ? 1 : 0;
  const int grid = persist ? cus : total;
  hipLaunchKernelGGL((prefill_kernel<D, BF16, CAUSAL, SWX>), dim3(grid), dim3(C::NT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse, sh, scale * kLog2e, nqb,
                     total, paired, persist);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Interleaved schedule for d = 64, where the softmax (two vector instructions
// or more per score, exponentials at a quarter of the rate) outweighs the
// matrix work.  A workgroup is 4 waves of 32 query rows; each wave runs S(t),
// the softmax and O += P(t) V(t) in turn, and three workgroups share a CU
// (three waves per SIMD), so the waves of a SIMD interleave their matrix and
// vector work freely.  K/V tiles of 64 keys go from global memory straight
// into double-buffered LDS (layouts and swizzles as in the ping-pong kernel);
// tile t+1 is requested at the start of tile t, one barrier per tile.
template <int D>
struct FiCfg {
  static constexpr int BM = 128;             // query rows per workgroup: 4 waves x 32
  static constexpr int BN = 64;              // keys per tile
  static constexpr int NT = 256;
  static constexpr int NB = BN / 32;         // 32-key blocks of S^T per tile
  static constexpr int NG = BN / 16;         // 16-key groups (k-steps of O^T) per tile
  static constexpr int ROWB = D * 2;
  static constexpr int SPR = ROWB / 16;
  static constexpr int TILEB = BN * ROWB;
  static constexpr int RPI = 1024 / ROWB;
  static constexpr int LPW = TILEB / 1024 / 4;  // 1 KB loads per K or V tile for each wave
  static constexpr int KSTEPS = D / 16;
  static constexpr int MB_O = D / 32;
  static constexpr int NA = NB * KSTEPS;     // MFMAs of S^T per tile
  static constexpr int NC = NG * MB_O;       // MFMAs of O^T per tile
};

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256, 3) void prefill_fi_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, SeqShape sh, float c, int nqb, int total) {
  using C = FiCfg<D>;
  using M = Mfma<BF16>;
  typedef typename M::op8 op8;
  typedef typename M::op2 op2;
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILEB];

  // work item: one 128-row query block of one (sequence, head), longest first
  // when causal; dense batches give each XCD a contiguous range of heads,
  // packed batches take block rank j slowest over all (sequence, head) pairs
  const bool packed = sh.cu_q != nullptr;
  const int logical = packed ? (int)blockIdx.x : xcd_remap(blockIdx.x, total);
  int bh, j_item;
  if (packed) {
    const int nh = total / nqb;
    j_item = logical / nh;
    bh = logical - j_item * nh;
  } else {
    bh = logical / nqb;
    j_item = logical - bh * nqb;
  }
  const int qb = CAUSAL ? nqb - 1 - j_item : j_item;
  const SeqSpan sp = seq_span(sh, bh / sh.H, bh % sh.H);
  const int Nq = sp.nq, Nk = sp.nk;
  const int off = Nk - Nq;
  const int q0 = qb * C::BM;
  if (q0 >= Nq) return;  // past a short packed sequence (uniform over the workgroup)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const size_t qbase = sp.q_row0 * D;
  const size_t kbase = sp.k_row0 * D;
  const auto rq = make_rsrc(Q + qbase, (uint32_t)Nq * D * 2);
  const auto rk = make_rsrc(K + kbase, (uint32_t)Nk * D * 2);
  const auto rv = make_rsrc(V + kbase, (uint32_t)Nk * D * 2);

  uint32_t gk_off[C::LPW], gv_off[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int row = (C::LPW * w + i) * C::RPI + lane / C::SPR, slot = lane % C::SPR;
    gk_off[i] = (uint32_t)row * C::ROWB + 16 * (slot ^ k_swz<D>(row));
    gv_off[i] = (uint32_t)row * C::ROWB + 16 * (slot ^ v_swz<D>(row));
  }
  auto issue_tile = [&](int t, char* ldk, char* ldv) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      tile_load_lds(rk, ldk + 1024 * (C::LPW * w + i), (uint32_t)t * C::TILEB + gk_off[i]);
      tile_load_lds(rv, ldv + 1024 * (C::LPW * w + i), (uint32_t)t * C::TILEB + gv_off[i]);
    }
  };
  uint32_t ka_off[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) ka_off[kk] = l32 * C::ROWB + 16 * ((2 * kk + h) ^ k_swz<D>(l32));
  const int r16 = lane & 15, g1 = (lane >> 4) & 1;
  const int vrow = (r16 >> 2) + 4 * h;
  uint32_t va_off[C::MB_O];
#pragma unroll
  for (int mb = 0; mb < C::MB_O; ++mb) {
    const int col = 32 * mb + 16 * g1 + 4 * (r16 & 3);
    va_off[mb] = vrow * C::ROWB + 16 * ((col >> 3) ^ v_swz<D>(vrow)) + 2 * (col & 7);
  }
  auto ka_load = [&](const char* lk, int i) {  // K operand of S^T step i: key block i/KSTEPS, k-step i%KSTEPS
    return lds_load<op8>(lk, ka_off[i % C::KSTEPS] + (i / C::KSTEPS) * 32 * C::ROWB);
  };
  auto va_load = [&](const char* lv, int j) {  // V^T operand of O^T step j: 16-key group j/MB_O, d block j%MB_O
    const uint32_t a0 = va_off[j % C::MB_O] + 16 * (j / C::MB_O) * C::ROWB;
    const s16x4 lo = lds_read_tr16(lv, a0);
    const s16x4 hi = lds_read_tr16(lv, a0 + 8 * C::ROWB);
    return __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  const int qmin_w = q0 + 32 * w;
  const int qrow = qmin_w + l32;
  op8 qop[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk)
    qop[kk] = __builtin_bit_cast(op8, buf_load16(rq, (uint32_t)qrow * C::ROWB + (16 * kk + 8 * h) * 2));

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + C::BM, Nq) - 1 + off + 1);
  const int T = max(0, (kv_end + C::BN - 1) / C::BN);

  f32x16 o[C::MB_O];
#pragma unroll
  for (int mb = 0; mb < C::MB_O; ++mb) o[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto tile = [&](int t, const char* lk, const char* lv, char* ldk, char* ldv) {
    if (t + 1 < T) issue_tile(t + 1, ldk, ldv);
    const int kv0 = t * C::BN;
    if (CAUSAL && kv0 > qmin_w + 31 + off) return;  // no key of the tile is visible to this wave
    f32x16 s[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) s[nb] = f32x16{};
    // the S MFMAs at raised wave priority: a wave holding the matrix core is
    // not made to wait behind the other waves' softmax (about 1 % on the long
    // sequence; the same on the P.V MFMAs measured no gain)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < C::NA; ++i) s[i / C::KSTEPS] = M::mma(ka_load(lk, i), qop[i % C::KSTEPS], s[i / C::KSTEPS]);
    __builtin_amdgcn_s_setprio(0);
    const bool edge = (kv0 + C::BN > Nk) || (CAUSAL && kv0 + C::BN - 1 > qmin_w + off);
    if (edge) {
      // element i of block nb holds key kv0 + 4h + 32 nb + 8 (i/4) + i%4 (bit blend as in prefill_kernel)
      const int lim = min(Nk - 1, CAUSAL ? qrow + off : Nk - 1) - (kv0 + 4 * h);
      constexpr uint32_t kNegInf = 0xFF800000u;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = 32 * nb + 8 * (i >> 2) + (i & 3);
          const uint32_t hide = (uint32_t)((lim - e) >> 31);
          const float v = s[nb][i];
          const uint32_t bits = __builtin_bit_cast(uint32_t, v);
          s[nb][i] = __builtin_bit_cast(float, (bits & ~hide) | (kNegInf & hide));
        }
    }
    op8 pb[C::NG];
    // P(t) against m_ref into pb; this lane's sum of it
    auto exps = [&](float m_ref) {
      float lsum[4];
#pragma unroll
      for (int g = 0; g < C::NG; ++g) {
        const int nb = g >> 1, tt = g & 1;
        op2 pr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[nb][8 * tt + 2 * j], c, -m_ref));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[nb][8 * tt + 2 * j + 1], c, -m_ref));
          pr[j] = M::pack2(p0, p1);
          lsum[j] = g == 0 ? p0 + p1 : lsum[j] + (p0 + p1);
        }
        pb[g] = __builtin_shufflevector(__builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3),
                                        __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      }
      return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };
    // the running max is raised only on a row's first tile or when a lane's P
    // would sum past kMaxTileSum, as in prefill_kernel
    const bool first = __any(m_run == -INFINITY);
    float tot = 0.f;
    bool raise = first;
    if (!first) {
      tot = exps(m_run);
      raise = __any(!(tot <= kMaxTileSum));
    }
    if (raise) {
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int i = nb == 0 ? 2 : 0; i < 16; ++i) mx = fmaxf(mx, s[nb][i]);
      const float m_new = fmaxf(m_run, pair_max(mx) * c);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int mb = 0; mb < C::MB_O; ++mb) o[mb] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      tot = exps((m_run == -INFINITY) ? 0.f : m_run);
    }
    l_run += tot;
#pragma unroll
    for (int j = 0; j < C::NC; ++j) o[j % C::MB_O] = M::mma(va_load(lv, j), pb[j / C::MB_O], o[j % C::MB_O]);
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
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
    if (LSE != nullptr && h == 0) LSE[sp.q_row0 + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool BF16, bool CAUSAL>
static hipError_t launch_fi(const void* q, const void* k, const void* v, void* out, float* lse, const SeqShape& sh,
                            int nseq, int max_nq, float scale, hipStream_t stream) {
  using C = FiCfg<D>;
  const int nqb = (max_nq + C::BM - 1) / C::BM;
  const int total = nqb * nseq * sh.H;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_fi_kernel<D, BF16, CAUSAL>), dim3(total), dim3(C::NT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse, sh, scale * kLog2e, nqb,
                     total);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, void* out, float* lse, const SeqShape& sh,
                          int nseq, int max_nq, int d, float scale, bool causal, bool bf16, hipStream_t stream) {
#define ATTN_DISPATCH(D_, BF_, CA_)          \
  if (d == D_ && bf16 == BF_ && causal == CA_) \
    return launch_t<D_, BF_, CA_>(q, k, v, out, lse, sh, nseq, max_nq, scale, stream);
  ATTN_DISPATCH(128, true, false)
  ATTN_DISPATCH(128, true, true)
  ATTN_DISPATCH(128, false, false)
  ATTN_DISPATCH(128, false, true)
  if (d == 64 && bf16 == true && causal == false) return launch_fi<64, true, false>(q, k, v, out, lse, sh, nseq, max_nq, scale, stream);
  if (d == 64 && bf16 == true && causal == true) return launch_fi<64, true, true>(q, k, v, out, lse, sh, nseq, max_nq, scale, stream);
  if (d == 64 && bf16 == false && causal == false) return launch_fi<64, false, false>(q, k, v, out, lse, sh, nseq, max_nq, scale, stream);
  if (d == 64 && bf16 == false && causal == true) return launch_fi<64, false, true>(q, k, v, out, lse, sh, nseq, max_nq, scale, stream);
#undef ATTN_DISPATCH
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_exp2_split(const void* q, const void* k, const void* v, void* out, float* lse,
                                     const SeqShape& sh, int nseq, int max_nq, int d, float scale, bool causal, bool bf16,
                                     int poly_per_8, hipStream_t stream) {
#define ATTN_DISPATCH(BF_, CA_, SW_)                                      \
  if (d == 128 && bf16 == BF_ && causal == CA_ && poly_per_8 == SW_) \
    return launch_t<128, BF_, CA_, SW_>(q, k, v, out, lse, sh, nseq, max_nq, scale, stream);
  ATTN_DISPATCH(true, false, 2)
  ATTN_DISPATCH(true, true, 2)
  ATTN_DISPATCH(false, false, 2)
  ATTN_DISPATCH(false, true, 2)
  ATTN_DISPATCH(true, false, 4)
  ATTN_DISPATCH(true, true, 4)
  ATTN_DISPATCH(false, false, 4)
  ATTN_DISPATCH(false, true, 4)
#undef ATTN_DISPATCH
  return hipErrorInvalidValue;
}

// y[i] = exp2_poly(x[i]): the polynomial exactly as the split softmax uses it
__global__ void debug_exp2_poly_kernel(const float* __restrict__ x, float* __restrict__ y, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = exp2_poly(x[i]);
}

hipError_t launch_debug_exp2_poly(const float* x, float* y, long n, hipStream_t stream) {
  hipLaunchKernelGGL(debug_exp2_poly_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

}  // namespace attn
