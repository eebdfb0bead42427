// The dense and packed batch layouts shared by the kernels, their launchers
// and the host-side validation: which rows of Q, K, V, O and LSE one
// (sequence, head) owns.  Plain C++ (no device code), so host-only builds of
// the validation layer can include it.
#pragma once
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

}  // namespace attn
