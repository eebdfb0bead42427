// The dense and packed batch layouts shared by the kernels and their
// launchers: which rows of Q, K, V, O and LSE one (sequence, head) owns.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Where the rows of one (sequence, query head) live.  Dense batches
// (cu_q == nullptr): sequence s of Nq queries and Nk keys, Q/O laid out
// [nseq, H, Nq, d], K/V [nseq, H/group, Nk, d], LSE [nseq, H, Nq].  Packed
// batches: sequence s owns query tokens cu_q[s] .. cu_q[s+1]-1 and key tokens
// cu_k[s] .. cu_k[s+1]-1 of head-major Q/O [H, Nq, d], K/V [H/group, Nk, d],
// LSE [H, Nq], where Nq and Nk are the token totals.  Query head h reads K/V
// head h / group (grouped-query attention; group = H for one shared head).
struct SeqShape {
  const int* cu_q;
  const int* cu_k;
  int H, group;
  int Nq, Nk;
};
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

}  // namespace attn
