// conv.h -- device-side view of one ssd_conv1d_silu call (the convolution
// front that produces x, B and C) and its launcher. Not part of the public ABI.
#pragma once

#include "ssd_internal.h"

namespace ssd {

struct ConvArgs {
  const void *xbc;       // (T, in_stride) dtype; the channels are [0, ch) of each row
  const float *w;        // (ch, K) taps, tap K-1 on the current token
  const float *bias;     // (ch) or null
  const void *hist_in;   // (nseq, K-1, ch) dtype or null (zeros)
  const int32_t *cu;     // (nseq + 1) packed offsets, or null (dense rows of seqlen)
  void *x;               // (T, x_dim) dtype
  void *B;               // (T, bc_dim) dtype
  void *C;               // (T, bc_dim) dtype
  void *hist_out;        // (nseq, K-1, ch) dtype or null
  int32_t T;             // tokens
  int32_t seqlen;        // dense: tokens per sequence
  int32_t nseq;          // sequences (dense: batch rows)
  int32_t ch, x_dim, bc_dim;
  int32_t in_stride;     // elements between token rows of xbc
  int32_t groups;        // ch / 8: channel groups, one per lane
  int32_t tiles;         // token tiles of kConvTile tokens
};

constexpr int kConvTile = 16;      // tokens per lane
constexpr int kConvThreads = 256;  // threads per workgroup

hipError_t launch_conv(const ConvArgs &a, int width, bool bf16_io, hipStream_t s);

}  // namespace ssd
