// k_cumsum.hip -- per-chunk prefix of the log-decay dt*A (row a2 of the path).
//
// The discretised decay of one step is exp(dt_t * A_h) (tj-hxxt.cn long read
// of the Mamba-1 paper, part III item 3, the paragraph on A). Inside a chunk
// the decay between tokens s <= l is the product of the per-step decays, i.e.
// 2^(cs[l] - cs[s]) with cs the inclusive prefix of dt*A*log2(e). Only these
// differences (never 2^(-cs)) are used downstream, so no exponent can overflow.
//
// Layout: one workgroup per (chunk, block of 16 heads). The chunk's dt rows
// (contiguous across heads in HBM) are read coalesced into LDS, then each of
// the four waves scans one head at a time with the DPP wavefront prefix
// (Q/64 tokens per lane, sequential inside the lane).
#include "ssd_internal.h"

namespace ssd {

constexpr int kCsHeads = 16;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__global__ __launch_bounds__(256) void k_chunk_cumsum(Args a) {
  __shared__ float s_da[kCsHeads][256 + 1];
  Chunk k;
  const int c = blockIdx.x;
  if (!chunk_of(a, c, k)) return;
  const int h0 = blockIdx.y * kCsHeads;
  const int nh = min(kCsHeads, a.H - h0);
  const int tid = threadIdx.x;
  {
    // One token row per thread: its (up to) 16 head values are independent
    // loads, all issued before the LDS writes.
    const int l = tid, lc = min(l, k.len - 1);
    float v[kCsHeads];
#pragma unroll
    for (int j = 0; j < kCsHeads; ++j)  // unconditional loads (clamped), then select
      v[j] = dt_of(a, ld<T>(a.dt, (size_t)(k.start + lc) * a.H + h0 + min(j, nh - 1)),
                   h0 + min(j, nh - 1));
#pragma unroll
    for (int j = 0; j < kCsHeads; ++j) v[j] = (l < k.len) ? v[j] : 0.f;
#pragma unroll
    for (int j = 0; j < kCsHeads; ++j)
      if (j < nh) s_da[j][l] = v[j] * a.A[h0 + j] * kLog2e;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int per = a.Q >> 6;  // 1, 2 or 4 tokens per lane
  for (int j = wave; j < nh; j += 4) {
    float v[4];
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < per) {
        const int l = lane * per + i;
        run += (l < k.len) ? s_da[j][l] : 0.f;
        v[i] = run;
      }
    }
    const float incl = wave_inclusive_sum(run);
    float excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.f;
    float *out = a.cs + ((size_t)c * a.H + h0 + j) * a.Q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int l = lane * per + i;
      if (i < per && l < k.len) out[l] = v[i] + excl;
    }
  }
}

hipError_t launch_chunk_cumsum(const Args &a, bool bf16_io, hipStream_t st) {
  dim3 grid(a.nc_max, (a.H + kCsHeads - 1) / kCsHeads);
  if (bf16_io)
    hipLaunchKernelGGL(k_chunk_cumsum<bf16>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_chunk_cumsum<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd
