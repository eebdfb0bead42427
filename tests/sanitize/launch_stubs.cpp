// Stand-ins for the kernel launchers of libattn_mi355x.so, for the host-only
// sanitizer build of its validation layer (api.cpp + plan.cpp).  Each stub
// records that a launch was asked for and returns success, so the C ABI's
// argument checks can run on the CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer, including the calls that pass every check.
// Test infrastructure: never part of the library.
#include <atomic>

#include "internal.h"

namespace {
std::atomic<int> g_launches{0};
hipError_t launched() {
  g_launches.fetch_add(1);
  return hipSuccess;
}
}  // namespace

extern "C" int attn_stub_launches(void) { return g_launches.load(); }

namespace attn {

hipError_t launch_prefill(const void*, const void*, const void*, void*, float*, const SeqShape&, int, int, int, float,
                          bool, bool, hipStream_t) {
  return launched();
}
hipError_t launch_decode(const void*, const void*, const void*, void*, float*, int, int, int, int, int, float, bool,
                         int, void*, hipStream_t) {
  return launched();
}
hipError_t launch_decode_static(const void*, const void*, const void*, void*, float*, int, int, int, int, float, bool,
                                int, hipStream_t) {
  return launched();
}
hipError_t launch_bwd(const void*, const void*, const void*, const void*, const void*, const float*, void*, void*,
                      void*, const SeqShape&, int, int, int, long, int, float, bool, bool, void*, hipStream_t) {
  return launched();
}
hipError_t launch_quantize_rows_i8(const void*, int8_t*, float*, long, int, hipStream_t) { return launched(); }
hipError_t launch_quantize_tensor_e4m3(const void*, uint8_t*, float*, long, void*, hipStream_t) { return launched(); }
hipError_t launch_prefill_q8(const void*, const void*, const void*, const float*, const float*, const float*, void*,
                             float*, int, int, int, int, int, float, bool, QVariant, hipStream_t) {
  return launched();
}
hipError_t launch_rotate_quantize_e4m3(const void*, const float*, uint8_t*, float*, int, int, int, int, hipStream_t) {
  return launched();
}
hipError_t launch_quantize_tensor_i8(const void*, int8_t*, float*, long, void*, hipStream_t) { return launched(); }
hipError_t launch_debug_qk(const void*, const void*, void*, int, int, int, bool, hipStream_t) { return launched(); }
hipError_t launch_debug_cvt_e4m3(const float*, uint8_t*, long, hipStream_t) { return launched(); }
hipError_t launch_debug_cvt_e2m1(const float*, uint8_t*, long, hipStream_t) { return launched(); }
hipError_t launch_prefill_exp2_split(const void*, const void*, const void*, void*, float*, const SeqShape&, int, int,
                                     int, float, bool, bool, int, hipStream_t) {
  return launched();
}
hipError_t launch_debug_exp2_poly(const float*, float*, long, hipStream_t) { return launched(); }

}  // namespace attn

// Reads element `index` of a fresh heap array of n ints: the sanitizer test
// calls it once in bounds and once one past the end, to show that
// AddressSanitizer is active in the process that runs the ABI cases (the
// size is a run-time value, so only the heap check can see the overrun).
extern "C" int attn_stub_heap_read(int n, int index) {
  int* a = new int[n];
  for (int i = 0; i < n; ++i) a[i] = i + 1;
  const int v = a[index];
  delete[] a;
  return v;
}
