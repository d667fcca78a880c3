// The call log of the stand-in launchers (stub_launchers.cpp).
#pragma once

#include "ssd_launch.h"

namespace stub {
struct Call {
  const char* name;
  bool has_shape;
  ssd::Shape shape;
  const void* p[3];
  bool flag[2];
};
constexpr int kMaxCalls = 16;
extern Call calls[kMaxCalls];
extern int ncalls;
extern int fail_with;   // status every launcher returns (0 = success)
void reset();
}  // namespace stub
