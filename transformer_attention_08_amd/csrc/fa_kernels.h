// Launch entry points shared between the host front end (fa_api.cpp) and the
// HIP kernels (fa_fwd.hip). Internal to the library; the public interface is
// include/fa.h.
#pragma once

#include <hip/hip_runtime_api.h>

namespace fa {

enum class Elt { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;      // may be null
  int bh;          // batch * heads
  int n;           // queries = keys per (batch, head)
  int d;           // 64 or 128
  bool causal;
  float c;         // scale (times both fp8 descales) times log2(e)
  float o_mult;    // multiplier applied to O in the epilogue (v descale; 1 otherwise)
  Elt elt;
};

// Enqueue the forward kernel for validated arguments. Returns the HIP status
// of the launch.
hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);

}  // namespace fa
