// k_step.hip -- one decode step: the recurrence advanced by one token per
// sequence, with the fp32 state updated in place.
//
// Generating one token at a time needs only the state of each (sequence,
// head): the discretised SSM runs as a recurrence (tj-hxxt.cn long read of the
// Mamba-1 paper, part II (一), "from continuous systems to discrete
// modelling"), and this state cache is what makes generation linear in the
// sequence length (same page, part IV (五), the inference-speed item). Per
// sequence b, head h, group g = h / (H/G):
//
//   state[b,h] <- exp(dt A_h) state[b,h] + dt x[b,h] B[b,g]^T      (P x N)
//   y[b,h,p]    = sum_n C[b,g,n] state[b,h,p,n] + D_h x[b,h,p]
//
// Every state element is read and written once (8 bytes) for about 4 flops,
// so the step is bound by HBM bandwidth. A state row (b, h, p) is N
// contiguous floats. Each lane owns 4 consecutive columns of one row (one
// 16-byte load and one 16-byte store); R lanes (N/4 rounded up to a power of
// two) cover a row, a wave covers 64/R consecutive rows per pass, and it makes
// kStepPasses passes with every load issued before the first use. The state
// is streamed with nontemporal loads and stores (nothing reuses it within the
// step). Measured on a 671 MB state: two passes with nontemporal accesses
// move 6.2 TB/s, one or four passes and plain accesses 5.5-6.1 TB/s. The row
// sum for y is a butterfly over the row's R lanes.
#include "step.h"

namespace ssd {

constexpr int kStepPasses = 2;
constexpr int kStepWaves = 4;

template <typename T> struct Vec4Of;
template <> struct Vec4Of<float> {
  static __device__ __forceinline__ void load(const void *p, size_t i, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  }
};
template <> struct Vec4Of<bf16> {
  // Four bf16 (8 bytes) widened exactly: a bf16 is the top half of an fp32.
  static __device__ __forceinline__ void load(const void *p, size_t i, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2 *>(static_cast<const bf16 *>(p) + i);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
};

typedef float f32x4_nt __attribute__((ext_vector_type(4)));

template <int R, typename T>
__global__ __launch_bounds__(kStepWaves * 64) void k_ssd_step(StepArgs a) {
  constexpr int kRowsPerPass = 64 / R;
  constexpr float kLog2e = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 =
      ((int64_t)blockIdx.x * kStepWaves + wave) * (kRowsPerPass * kStepPasses) + lane / R;
  const int n0 = 4 * (lane % R);
  const bool col_ok = n0 < a.N;

  float4 st[kStepPasses];
  float bv[kStepPasses][4], cv[kStepPasses][4];
  float xv[kStepPasses], dtv[kStepPasses], av[kStepPasses], dv[kStepPasses];
  bool ok[kStepPasses];
#pragma unroll
  for (int it = 0; it < kStepPasses; ++it) {
    const int64_t row = row0 + it * kRowsPerPass;
    ok[it] = row < a.rows;
    st[it] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 4; ++k) bv[it][k] = cv[it][k] = 0.f;
    xv[it] = dtv[it] = av[it] = dv[it] = 0.f;
    if (ok[it]) {
      // row = (b * H + h) * P + p; batch * H fits 32 bits (checked on the host)
      const uint32_t bh = (uint32_t)(row >> a.p_shift);
      const uint32_t b = bh / (uint32_t)a.H;
      const uint32_t h = bh - b * (uint32_t)a.H;
      const uint32_t g = h / (uint32_t)a.heads_per_group;
      xv[it] = ld<T>(a.x, (size_t)row);
      dtv[it] = ld<T>(a.dt, (size_t)bh);
      av[it] = a.A[h];
      dv[it] = a.D ? a.D[h] : 0.f;
      if (col_ok) {
        const size_t bc = ((size_t)b * a.G + g) * a.N + n0;
        const f32x4_nt q = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_nt *>(a.state + (size_t)row * a.N + n0));
        st[it] = make_float4(q[0], q[1], q[2], q[3]);
        Vec4Of<T>::load(a.B, bc, bv[it]);
        Vec4Of<T>::load(a.C, bc, cv[it]);
      }
    }
  }
#pragma unroll
  for (int it = 0; it < kStepPasses; ++it) {
    const float decay = exp2_fast(dtv[it] * av[it] * kLog2e);
    const float u = dtv[it] * xv[it];
    float4 s = st[it];
    s.x = decay * s.x + u * bv[it][0];
    s.y = decay * s.y + u * bv[it][1];
    s.z = decay * s.z + u * bv[it][2];
    s.w = decay * s.w + u * bv[it][3];
    float part = cv[it][0] * s.x + cv[it][1] * s.y + cv[it][2] * s.z + cv[it][3] * s.w;
#pragma unroll
    for (int off = R / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    const int64_t row = row0 + it * kRowsPerPass;
    if (ok[it]) {
      if (col_ok) {
        const f32x4_nt q = {s.x, s.y, s.z, s.w};
        __builtin_nontemporal_store(q, reinterpret_cast<f32x4_nt *>(a.state + (size_t)row * a.N + n0));
      }
      if (n0 == 0) static_cast<T *>(a.y)[row] = from_f32<T>(part + dv[it] * xv[it]);
    }
  }
}

int step_lanes_per_row(int N) {
  int r = 4;
  while (r < 64 && 4 * r < N) r *= 2;
  return r;
}

int64_t step_blocks(const StepArgs &a) {
  const int64_t rows_per_block = (int64_t)kStepWaves * (64 / step_lanes_per_row(a.N)) * kStepPasses;
  return (a.rows + rows_per_block - 1) / rows_per_block;
}

template <typename T>
hipError_t launch_step_t(const StepArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)step_blocks(a)), block(kStepWaves * 64);
  switch (step_lanes_per_row(a.N)) {
    case 4: hipLaunchKernelGGL((k_ssd_step<4, T>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_ssd_step<8, T>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_ssd_step<16, T>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_ssd_step<32, T>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_ssd_step<64, T>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, bool bf16_io, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  return bf16_io ? launch_step_t<bf16>(a, s) : launch_step_t<float>(a, s);
}

}  // namespace ssd
