// step.h -- device-side view of one ssd_step call (the decode step) and its
// launcher. Not part of the public ABI.
#pragma once

#include "ssd_internal.h"

namespace ssd {

// Dense batch, one token per sequence; the state is updated in place.
struct StepArgs {
  const void *x;        // (batch, H, P)  dtype
  const void *dt;       // (batch, H)     dtype
  const float *A;       // (H)
  const void *B;        // (batch, G, N)  dtype
  const void *C;        // (batch, G, N)  dtype
  const float *D;       // (H) or null
  float *state;         // (batch, H, P, N), read and written in place
  void *y;              // (batch, H, P)  dtype
  int64_t rows;         // batch * H * P state rows
  int32_t H, N, G, heads_per_group;
  int32_t p_shift;      // log2(P); P is a power of two
};

int64_t step_blocks(const StepArgs &a);
hipError_t launch_step(const StepArgs &a, bool bf16_io, hipStream_t s);

}  // namespace ssd
