// k_generic.hip -- plain fp32-FMA versions of the two chunk kernels.
//
// They serve fp32 inputs (where fp32 accuracy is asked for) and any shape
// the MFMA kernels do not cover. Same algebra as the MFMA kernels:
//
//   chunk_state (row a3): S_c[p, n] = sum_{s in c} 2^(cs_last - cs_s) dt_s x_s[p] B_s[n]
//   chunk_scan  (row a5): y_l = 2^(cs_l) C_l . h_prev  +  sum_{s <= l} (C_l . B_s)
//                               2^(cs_l - cs_s) dt_s x_s  +  D x_l
//
// i.e. the block decomposition of the semiseparable matrix: the diagonal
// block is the masked-attention product, off-diagonal blocks go through the
// state (QbitAI "Mamba-2" article, srwj168 repost, sections "Unifying SSM and
// attention" and "Mamba-2: stronger learning, faster training and inference").
#include "ssd_internal.h"

namespace ssd {

// ---- chunk_state ------------------------------------------------------------
// One workgroup per (chunk, head, 256 outputs); one output (p, n) per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_chunk_state_generic(Args a) {
  __shared__ float s_w[256];
  __shared__ float s_x[32][128 + 1];
  __shared__ float s_b[32][256 + 1];
  Chunk k;
  const int c = blockIdx.x;
  if (!chunk_of(a, c, k)) return;
  const int h = blockIdx.y, g = h / a.heads_per_group;
  const int P = a.P, N = a.N, tid = threadIdx.x;
  const int o = blockIdx.z * 256 + tid;
  const bool valid = o < P * N;
  const int p = o / N, n = o - (o / N) * N;
  const float *cs = a.cs + ((size_t)c * a.H + h) * a.Q;
  const float last = cs[k.len - 1];
  for (int l = tid; l < k.len; l += 256)
    s_w[l] = exp2_fast(last - cs[l]) * dt_of(a, ld<T>(a.dt, (size_t)(k.start + l) * a.H + h), h);
  __syncthreads();
  float acc = 0.f;
  for (int l0 = 0; l0 < k.len; l0 += 32) {
    const int nl = min(32, k.len - l0);
    for (int e = tid; e < nl * P; e += 256) {
      const int j = e / P, q = e - j * P;
      s_x[j][q] = ld<T>(a.x, ((size_t)(k.start + l0 + j) * a.H + h) * P + q) * s_w[l0 + j];
    }
    for (int e = tid; e < nl * N; e += 256) {
      const int j = e / N, q = e - j * N;
      s_b[j][q] = ld<T>(a.B, ((size_t)(k.start + l0 + j) * a.G + g) * N + q);
    }
    __syncthreads();
    if (valid)
      for (int j = 0; j < nl; ++j) acc += s_x[j][p] * s_b[j][n];
    __syncthreads();
  }
  if (valid) a.states[((size_t)c * a.H + h) * P * N + o] = acc;
}

hipError_t launch_chunk_state_generic(const Args &a, bool bf16_io, hipStream_t st) {
  dim3 grid(a.nc_max, a.H, (a.P * a.N + 255) / 256);
  if (bf16_io)
    hipLaunchKernelGGL(k_chunk_state_generic<bf16>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_chunk_state_generic<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---- chunk_scan ---------------------------------------------------------------
// One workgroup per (chunk, head, 16 rows). Thread (r, q) owns row l0 + r and
// columns p = q, q + 16, ... (P / 16 of them).
constexpr int kScanRows = 16;

template <typename T>
__global__ __launch_bounds__(256) void k_chunk_scan_generic(Args a) {
  __shared__ float s_cs[256];
  __shared__ float s_dt[256];
  __shared__ float s_c[kScanRows][256 + 1];
  __shared__ float s_g[kScanRows][256 + 1];
  __shared__ float s_t[128 * 33];  // staging: h_prev [P][32+1] or x [32][P+1]
  Chunk k;
  const int c = blockIdx.x;
  if (!chunk_of(a, c, k)) return;
  const int l0 = blockIdx.z * kScanRows;
  if (l0 >= k.len) return;
  const int h = blockIdx.y, g = h / a.heads_per_group;
  const int P = a.P, N = a.N, tid = threadIdx.x;
  const int r = tid >> 4, q = tid & 15, np = P >> 4;
  const int l = l0 + r;
  const bool row_ok = l < k.len;
  const float *cs = a.cs + ((size_t)c * a.H + h) * a.Q;
  for (int i = tid; i < k.len; i += 256) {
    s_cs[i] = cs[i];
    s_dt[i] = dt_of(a, ld<T>(a.dt, (size_t)(k.start + i) * a.H + h), h);
  }
  for (int e = tid; e < kScanRows * N; e += 256) {
    const int rr = e / N, n = e - rr * N;
    s_c[rr][n] = (l0 + rr < k.len)
                     ? ld<T>(a.C, ((size_t)(k.start + l0 + rr) * a.G + g) * N + n)
                     : 0.f;
  }
  __syncthreads();

  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  // 1. Contribution of the state entering the chunk.
  const float *hp = a.states + ((size_t)c * a.H + h) * P * N;
  for (int n0 = 0; n0 < N; n0 += 32) {
    const int nn = min(32, N - n0);  // N is a multiple of 16, not of 32
    for (int e = tid; e < P * 32; e += 256) {
      const int pp = e >> 5, j = e & 31;
      s_t[pp * 33 + j] = j < nn ? hp[(size_t)pp * N + n0 + j] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < nn; ++j) {
      const float cv = s_c[r][n0 + j];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < np) acc[u] += cv * s_t[(q + 16 * u) * 33 + j];
    }
    __syncthreads();
  }
  const float row_decay = row_ok ? exp2_fast(s_cs[l]) : 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] *= row_decay;

  // 2. Masked scores (C_l . B_s) 2^(cs_l - cs_s) dt_s for s <= l.
  const int smax = min(l0 + kScanRows, k.len);
  for (int s = q; s < smax; s += 16) {
    float dot = 0.f;
    const size_t boff = ((size_t)(k.start + s) * a.G + g) * N;
    for (int n = 0; n < N; ++n) dot += s_c[r][n] * ld<T>(a.B, boff + n);
    const bool causal = row_ok && s <= l;
    s_g[r][s] = causal ? dot * exp2_fast(s_cs[l] - s_cs[s]) * s_dt[s] : 0.f;
  }
  __syncthreads();

  // 3. y += scores . x
  for (int s0 = 0; s0 < smax; s0 += 32) {
    const int ns = min(32, smax - s0);
    for (int e = tid; e < ns * P; e += 256) {
      const int j = e / P, pp = e - j * P;
      s_t[j * 129 + pp] = ld<T>(a.x, ((size_t)(k.start + s0 + j) * a.H + h) * P + pp);
    }
    __syncthreads();
    for (int j = 0; j < ns; ++j) {
      const float m = s_g[r][s0 + j];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < np) acc[u] += m * s_t[j * 129 + q + 16 * u];
    }
    __syncthreads();
  }

  // 4. Skip term and store.
  if (row_ok) {
    const float dsk = a.D ? a.D[h] : 0.f;
    const size_t yo = ((size_t)(k.start + l) * a.H + h) * P;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < np) {
        const int pp = q + 16 * u;
        const float v = acc[u] + dsk * ld<T>(a.x, yo + pp);
        static_cast<T *>(a.y)[yo + pp] = from_f32<T>(v);
      }
    }
  }
}

hipError_t launch_chunk_scan_generic(const Args &a, bool bf16_io, hipStream_t st) {
  dim3 grid(a.nc_max, a.H, a.Q / kScanRows);
  if (bf16_io)
    hipLaunchKernelGGL(k_chunk_scan_generic<bf16>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_chunk_scan_generic<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd
