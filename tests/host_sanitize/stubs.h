// Call record of the launcher stubs (see stubs.cpp).
#ifndef MX_TEST_STUBS_H
#define MX_TEST_STUBS_H
#include <stdint.h>

struct StubCall {
  const char *name = nullptr;
  int64_t nitems = -1;
  int bf16 = -1, mode = -1;
  const void *p[6] = {};
  int64_t space = -1;  // partial-sum space (doubles) handed to an error launch
};
// the address the scratch-address stub hands out for device d
inline const void *stub_scratch(int d) {
  return reinterpret_cast<const void *>(static_cast<uintptr_t>(0x5C000000u) + 0x1000u * d);
}
constexpr int64_t kFailItems = 4 * 1024 * 1024 + 16;  // rows * k / 8 that makes a stub fail
extern thread_local StubCall g_last;
extern thread_local int g_calls;
#endif
