// Host-side sizing rules of the kernels: workspace sizes, the decode's split
// count and head grouping, the per-tensor reduction's partial count.  Plain
// C++ with no device code, shared by the library and by the host-only build
// of the validation layer (which needs the same sizes to check workspaces).
#include "internal.h"

namespace attn {

size_t decode_workspace_bytes(int B, int H, int d, int splits) {
  return (size_t)B * H * splits * (d + 1) * sizeof(float);
}

int decode_heads_per_workgroup(int H, int Hkv) {
  const int group = H / Hkv;
  return group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}

int decode_default_splits(int B, int H, int Hkv, int Nk, int d) {
  (void)d;
  // aim for about 4096 (query head, key range) streams with at least 128 keys
  // each.  A grouped workgroup serves several heads of a range at once; counting
  // streams per query head still measured best for it (splitting its key range
  // further only added partial states to write and merge)
  (void)Hkv;
  long bh = (long)B * H;
  int s = 1;
  while (bh * s < 4096 && s < 256 && (long)(s * 2) * 128 <= Nk) s *= 2;
  return s;
}

// one (lse, D) float pair per query row
size_t bwd_workspace_bytes(long q_rows) { return (size_t)q_rows * 2 * sizeof(float); }

// one partial maximum per 256 chunks of 8 elements, at most 1024 partials
int e4m3_partials(long n) {
  constexpr long kMaxPartials = 1024;
  const long chunks = n / 8;
  long g = (chunks + 255) / 256;
  if (g > kMaxPartials) g = kMaxPartials;
  if (g < 1) g = 1;
  return (int)g;
}

size_t quantize_e4m3_workspace_bytes(long n) { return (size_t)e4m3_partials(n) * sizeof(float); }

}  // namespace attn
