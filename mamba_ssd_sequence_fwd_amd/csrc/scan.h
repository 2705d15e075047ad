// scan.h -- device-side view of one ssd_selective_scan call (the Mamba-1
// selective scan) and its launcher. Not part of the public ABI.
#pragma once

#include "ssd_internal.h"

namespace ssd {

struct ScanArgs {
  const void *x;        // (batch, L, dim)  dtype
  const void *delta;    // (batch, L, dim)  dtype, the step (already positive)
  const float *A;       // (dim, N)
  const void *B;        // (batch, L, N)    dtype
  const void *C;        // (batch, L, N)    dtype
  const float *D;       // (dim) or null
  const float *h0;      // (batch, dim, N) or null
  void *y;              // (batch, L, dim)  dtype
  float *hT;            // (batch, dim, N) or null
  int32_t batch, L, dim, N;
};

int scan_channels_per_block(int N);
hipError_t launch_selective_scan(const ScanArgs &a, bool bf16_io, hipStream_t s);

}  // namespace ssd
