// What the test-only launchers (launch_stubs.cpp) record.
#pragma once

#include "common.h"

namespace stubs {
extern hipError_t result;   // returned by every launcher
extern int launches;
extern yoco::ComposeParams compose;
extern yoco::ComposeBackwardParams backward;
extern float* backward_partial;
extern yoco::DecodeParams decode;
extern bool decode_bf16;
extern yoco::PrefillParams prefill;
struct Merge {
  const float* part_o;
  const float* part_lse;
  int B, Hq, D, S;
  float* out;
  float* lse;
};
extern struct Merge merge;
extern char scratch_bytes[1 << 12];
}  // namespace stubs
