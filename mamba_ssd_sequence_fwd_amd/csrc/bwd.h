// bwd.h -- device-side view of one ssd_backward call (the gradients of the
// SSD layer) and its launchers. Not part of the public ABI.
#pragma once

#include "ssd_internal.h"

namespace ssd {

struct BwdArgs {
  Args f;               // the forward problem; f.states holds the state entering
                        // every chunk and f.hT each sequence's final state, both
                        // recomputed into the workspace
  const void *dy;       // (T, H, P) dtype: dL/dy
  const float *dhT;     // (S, H, P, N) or null: dL/d(final state)
  float *gst;           // (chunks, H, P, N): per-chunk dstate, then dL/d(state
                        // leaving the chunk)
  void *dx;             // (T, H, P) dtype
  void *ddt;            // (T, H) dtype
  void *dB;             // (T, G, N) dtype
  void *dC;             // (T, G, N) dtype
  float *dh0;           // (S, H, P, N) or null
  float *dA_part;       // (chunks, H)
  float *dD_part;       // (chunks, H)
  float *dA;            // (H)
  float *dD;            // (H) or null
  bf16 *hinT;           // (chunks, H, N, P): h_in as bf16, transposed (written by
                        // the dx kernel for the dB / dC kernel)
  bf16 *gT;             // (chunks, H, N, P): g_c likewise
};

// Row block of the dB / dC kernel (tokens per workgroup).
constexpr int kBwdRows = 32;

bool bwd_supports(const Args &a);
hipError_t launch_chunk_dstate_mfma(const Args &a, hipStream_t s);
hipError_t launch_state_passing_bwd(const BwdArgs &b, hipStream_t s);
hipError_t launch_bwd_cbt(const BwdArgs &b, hipStream_t s);
hipError_t launch_bwd_dx(const BwdArgs &b, hipStream_t s);
hipError_t launch_bwd_dbc(const BwdArgs &b, hipStream_t s);
hipError_t launch_bwd_reduce(const BwdArgs &b, hipStream_t s);

}  // namespace ssd
