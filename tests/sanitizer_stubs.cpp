// Host-only stand-ins for the kernel launchers of libsparse_attn.so, so that the C ABI's argument
// checks (csrc/capi.cpp) can be built and exercised under AddressSanitizer and UBSan on a machine
// without a GPU. The size queries return what the real library returns; a launch "succeeds"
// without doing anything (the host-ABI tests only pass pointers that the checks must reject).
#include <stddef.h>
#include <stdint.h>

extern "C" {
int sa_internal_launch_sparse(const void*, const void*, const float*, const int32_t*, void*, int64_t, int64_t, int64_t,
                              int64_t, int64_t, int64_t, float, int, void*, int, int, void*) {
  return 0;
}
int sa_internal_head_blocks(int64_t H) {
  const int hb = (int)((H + 15) / 16);
  return hb <= 2 ? hb : (hb <= 4 ? 4 : 8);
}
size_t sa_internal_sparse_ws_bytes(int64_t ntok, int64_t H, int64_t D, int nsplit) {
  if (nsplit <= 1) return 0;
  auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t pairs = (size_t)ntok * nsplit, hp = (size_t)sa_internal_head_blocks(H) * 16;
  return r256(pairs * hp * D * 2) + r256(pairs * hp * 8);
}
size_t sa_internal_scratch_bytes(void) { return (size_t)40 << 20; }
int sa_internal_scratch_ptr(void** out) {
  *out = nullptr;
  return 1;
}
int sa_internal_launch_bitmask(const int32_t*, const int32_t*, const int32_t*, uint32_t*, int64_t, int64_t, int64_t,
                               int64_t, int64_t, int64_t, void*) {
  return 0;
}
int64_t sa_internal_bitmask_max_words(void) { return 32768; }
int sa_internal_launch_masked(const void*, const void*, const void*, const uint32_t*, void*, float*, int64_t, int64_t,
                              int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, float, int, int, void*) {
  return 0;
}
int sa_internal_candidate_gcols(int64_t rows, int64_t width) {
  const int64_t tiles = (width + 1023) / 1024;  // 1024-column tiles
  int64_t g = rows > 0 ? 4096 / rows : 1;
  if (g < 1) g = 1;
  if (g > tiles) g = tiles;
  return (int)(g < 1 ? 1 : g);
}
int sa_internal_launch_candidate_mask(float*, const int32_t*, const int32_t*, const uint8_t*, int64_t, int64_t,
                                      int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, void*) {
  return 0;
}
}
