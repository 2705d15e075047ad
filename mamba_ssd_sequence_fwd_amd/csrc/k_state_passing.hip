// k_state_passing.hip -- the recurrence between chunks (row a4 of the path).
//
// With S_c the state a chunk produces from a zero start and 2^(cs_last) its
// total decay, the state entering chunk c+1 is 2^(cs_last[c]) * h_c + S_c,
// starting from the sequence's initial state (zeros if none) and restarting
// at every sequence start (tj-hxxt.cn long read of the Mamba-1 paper, part
// III item 2.3, "Boundary Resetting"). The pass is serial over chunks and
// parallel over (sequence, head, P*N): each thread owns four consecutive fp32
// elements of one head's state, so every chunk step reads and writes whole
// 16-byte vectors, coalesced across the wave. S_c is replaced in place by the
// state entering chunk c, which is what the output kernel consumes. Loads of
// the next chunks are issued ahead of the dependent update (a small register
// ring) so HBM latency overlaps the serial chain.
#include "ssd_internal.h"

namespace ssd {

constexpr int kSpThreads = 256;
constexpr int kSpDepth = 4;  // chunks in flight per thread

__global__ __launch_bounds__(kSpThreads) void k_state_passing(Args a) {
  const int PN = a.P * a.N;
  const int nb = (PN / 4 + kSpThreads - 1) / kSpThreads;  // blocks per head
  const int s = blockIdx.x / (a.H * nb);
  const int rem = blockIdx.x - s * (a.H * nb);
  const int h = rem / nb;
  const int e = ((rem - h * nb) * kSpThreads + threadIdx.x) * 4;
  if (e >= PN) return;
  int c0, c1;
  chunks_of_seq(a, s, c0, c1);
  float4 st = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.h0) st = *reinterpret_cast<const float4 *>(a.h0 + ((size_t)s * a.H + h) * PN + e);

  float4 ring[kSpDepth];
  float dec[kSpDepth];
#pragma unroll
  for (int i = 0; i < kSpDepth; ++i) {
    const int c = c0 + i;
    if (c < c1) {
      ring[i] = *reinterpret_cast<const float4 *>(a.states + ((size_t)c * a.H + h) * PN + e);
      const int len = a.varlen ? a.plan[a.rec_off + 4 * c + 2] : min(a.Q, a.L - (c - c0) * a.Q);
      dec[i] = exp2_fast(a.cs[((size_t)c * a.H + h) * a.Q + len - 1]);
    }
  }
  for (int cb = c0; cb < c1; cb += kSpDepth) {
#pragma unroll
    for (int i = 0; i < kSpDepth; ++i) {
      const int c = cb + i;
      if (c < c1) {
        const float4 S = ring[i];
        const float d = dec[i];
        // Refill this slot with chunk c + depth before the dependent math.
        const int cn = c + kSpDepth;
        if (cn < c1) {
          ring[i] = *reinterpret_cast<const float4 *>(a.states + ((size_t)cn * a.H + h) * PN + e);
          const int len = a.varlen ? a.plan[a.rec_off + 4 * cn + 2] : min(a.Q, a.L - (cn - c0) * a.Q);
          dec[i] = exp2_fast(a.cs[((size_t)cn * a.H + h) * a.Q + len - 1]);
        }
        *reinterpret_cast<float4 *>(a.states + ((size_t)c * a.H + h) * PN + e) = st;
        st.x = d * st.x + S.x;
        st.y = d * st.y + S.y;
        st.z = d * st.z + S.z;
        st.w = d * st.w + S.w;
      }
    }
  }
  if (a.hT) *reinterpret_cast<float4 *>(a.hT + ((size_t)s * a.H + h) * PN + e) = st;
}

hipError_t launch_state_passing(const Args &a, hipStream_t st) {
  const int PN = a.P * a.N;
  const int nb = (PN / 4 + kSpThreads - 1) / kSpThreads;
  dim3 grid(nb * a.H * a.nseq);
  hipLaunchKernelGGL(k_state_passing, grid, dim3(kSpThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd
