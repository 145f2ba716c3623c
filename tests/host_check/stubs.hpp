// Shared between the launcher stand-ins and the host-check driver.
#pragma once

#include "kernels.hpp"

namespace stub {
struct Record {
  const char* what = "";
  int B = 0, D = 0;
  int ints[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  void* ptrs[2] = {nullptr, nullptr};
  ca::AttnParams p{};
  ca::SeqInfo seq{};
};
extern Record last;
}  // namespace stub
