// k_conv.hip -- the convolution front: a causal depthwise 1-D convolution over
// the packed (x, B, C) channels of each token, then SiLU, written straight
// into the x, B and C arrays the SSD forward pass reads.
//
// In the Mamba-2 model part of the input projection passes through a 1-D
// convolution that captures local dependencies along the sequence without
// looking ahead (CSDN csdn_xmj page, related-article snippet on implementing
// the Mamba-2 model), and the block applies an activation where H3 had a gate
// (tj-hxxt.cn long read of the Mamba-1 paper, part III, the closing paragraph
// on the selection mechanism). Per channel c of a sequence, with the K - 1
// inputs before its first token taken from a history (or zeros):
//
//   pre[t, c] = bias[c] + sum_k w[c, k] u[t - (K - 1) + k, c]
//   out[t, c] = pre / (1 + exp(-pre))
//
// Every input is read once and every output written once, for 2K + 4 flops,
// so the kernel is bound by HBM bandwidth. Each lane owns 8 consecutive
// channels (16 bytes of bf16) and walks kConvTile tokens (16: measured faster
// than 32 or 64, the extra K - 1 halo rows per tile mostly hit in L2), keeping
// the last K - 1 inputs in registers; a wave reads 64 x 8 channels of one token row, 1
// KB contiguous, per load. Token rows are loaded kConvBatch at a time, the
// next batch issued before the current one is used. Sequence starts reset the
// window from the history, and a sequence's last token writes its final
// history (the last K - 1 inputs, oldest first).
#include "conv.h"

namespace ssd {

constexpr int kConvBatch = 8;
static_assert(kConvTile % kConvBatch == 0, "tile must hold whole batches");

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Eight consecutive elements of one row, widened exactly to fp32, and back.
// Rows are stored with nontemporal stores: nothing in the call reads them
// again, and keeping them out of the caches was measured 20-25% faster on the
// 2.7B-shaped front (nontemporal loads as well were slower).
template <typename T> struct Row8;
template <> struct Row8<bf16> {
  uint4 q;
  __device__ __forceinline__ void load(const void *p, size_t i) {
    q = *reinterpret_cast<const uint4 *>(static_cast<const bf16 *>(p) + i);
  }
  __device__ __forceinline__ void widen(float (&v)[8]) const {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(void *p, size_t i, const float (&v)[8]) {
    u32x4_t q;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16 lo = (bf16)v[2 * k], hi = (bf16)v[2 * k + 1];
      q[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    __builtin_nontemporal_store(q, reinterpret_cast<u32x4_t *>(static_cast<bf16 *>(p) + i));
  }
};
template <> struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const void *p, size_t i) {
    const float4 *s = reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
    a = s[0];
    b = s[1];
  }
  __device__ __forceinline__ void widen(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(void *p, size_t i, const float (&v)[8]) {
    f32x4_t *d = reinterpret_cast<f32x4_t *>(static_cast<float *>(p) + i);
    const f32x4_t lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(lo, d);
    __builtin_nontemporal_store(hi, d + 1);
  }
};

// v * sigmoid(v) on the hardware exp and reciprocal units: for very negative
// v the exponential overflows to +inf and the result is -0, for very
// positive v it is v.
__device__ __forceinline__ float silu(float v) {
  constexpr float kLog2e = 1.4426950408889634f;
  return v * __builtin_amdgcn_rcpf(1.f + exp2_fast(-v * kLog2e));
}

// The K - 1 history rows of sequence s for this lane's channels (zeros when
// there is no history).
template <int K, typename T>
__device__ __forceinline__ void load_history(const ConvArgs &a, int s, int c0,
                                             float (&win)[K - 1][8]) {
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    if (a.hist_in) {
      Row8<T> r;
      r.load(a.hist_in, ((size_t)s * (K - 1) + j) * a.ch + c0);
      r.widen(win[j]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) win[j][c] = 0.f;
    }
  }
}

// One token of this lane's 8 channels: out = silu(bias + taps . window) with
// the current input last, then the window slides by one.
template <int K>
__device__ __forceinline__ void conv_token(const float (&w)[8][K], const float (&bias)[8],
                                           float (&win)[K - 1][8], const float (&cur)[8],
                                           float (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float acc = bias[c] + w[c][K - 1] * cur[c];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) acc += w[c][j] * win[j][c];
    out[c] = silu(acc);
  }
#pragma unroll
  for (int j = 0; j + 1 < K - 1; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) win[j][c] = win[j + 1][c];
#pragma unroll
  for (int c = 0; c < 8; ++c) win[K - 2][c] = cur[c];
}

// A full tile inside one sequence whose K - 1 predecessors are in the same
// sequence: no boundary, every load and store unconditional, so the waits
// for each batch of loads are exact. Leaves the last K - 1 inputs in win.
template <int K, typename T>
__device__ __forceinline__ void conv_tile_interior(const ConvArgs &a, int t0, int c0,
                                                   const float (&w)[8][K],
                                                   const float (&bias)[8], void *dst,
                                                   int dcol, int dstride,
                                                   float (&win)[K - 1][8]) {
  Row8<T> head[K - 1], rows[kConvBatch], next[kConvBatch];
#pragma unroll
  for (int j = 0; j < K - 1; ++j)
    head[j].load(a.xbc, (size_t)(t0 - (K - 1) + j) * a.in_stride + c0);
#pragma unroll
  for (int u = 0; u < kConvBatch; ++u)
    rows[u].load(a.xbc, (size_t)(t0 + u) * a.in_stride + c0);
#pragma unroll
  for (int j = 0; j < K - 1; ++j) head[j].widen(win[j]);
#pragma unroll
  for (int tb = 0; tb < kConvTile; tb += kConvBatch) {
    if (tb + kConvBatch < kConvTile) {
#pragma unroll
      for (int u = 0; u < kConvBatch; ++u)
        next[u].load(a.xbc, (size_t)(t0 + tb + kConvBatch + u) * a.in_stride + c0);
    }
#pragma unroll
    for (int u = 0; u < kConvBatch; ++u) {
      float cur[8], out[8];
      rows[u].widen(cur);
      conv_token<K>(w, bias, win, cur, out);
      Row8<T>::store(dst, (size_t)(t0 + tb + u) * dstride + dcol, out);
    }
#pragma unroll
    for (int u = 0; u < kConvBatch; ++u) rows[u] = next[u];
  }
}

template <int K, typename T>
__global__ __launch_bounds__(kConvThreads) void k_conv_silu(ConvArgs a) {
  // Workgroups are dealt to the 8 XCDs in turn; renumber them so that each
  // XCD runs one contiguous range, keeping neighbouring token tiles (which
  // share K - 1 rows) in one L2.
  const int nb = gridDim.x, bid = blockIdx.x;
  const int q = nb >> 3, r = nb & 7, xcd = bid & 7;
  const int lb = xcd * q + min(xcd, r) + (bid >> 3);
  const int64_t gid = (int64_t)lb * kConvThreads + threadIdx.x;
  const int tile = (int)(gid / a.groups);
  if (tile >= a.tiles) return;
  const int c0 = (int)(gid - (int64_t)tile * a.groups) * 8;
  const int t0 = tile * kConvTile, t1 = min(t0 + kConvTile, a.T);

  // The sequence holding t0: [ss, se).
  int s, ss, se;
  if (a.cu) {
    int lo = 0, hi = a.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    s = lo;
    ss = a.cu[s];
    se = a.cu[s + 1];
  } else {
    s = t0 / a.seqlen;
    ss = s * a.seqlen;
    se = ss + a.seqlen;
  }

  // Output array and column of this lane's channels (uniform per lane).
  void *dst;
  int dcol, dstride;
  if (c0 < a.x_dim) {
    dst = a.x; dcol = c0; dstride = a.x_dim;
  } else if (c0 < a.x_dim + a.bc_dim) {
    dst = a.B; dcol = c0 - a.x_dim; dstride = a.bc_dim;
  } else {
    dst = a.C; dcol = c0 - a.x_dim - a.bc_dim; dstride = a.bc_dim;
  }

  float w[8][K], bias[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int k = 0; k < K; ++k) w[c][k] = a.w[(size_t)(c0 + c) * K + k];
    bias[c] = a.bias ? a.bias[c0 + c] : 0.f;
  }

  // The window: the K - 1 inputs before t0, oldest first.
  float win[K - 1][8];
  if (t1 - t0 == kConvTile && t0 >= K - 1 && t0 - (K - 1) >= ss && t1 <= se) {
    conv_tile_interior<K, T>(a, t0, c0, w, bias, dst, dcol, dstride, win);
    if (t1 == se && a.hist_out) {
#pragma unroll
      for (int j = 0; j < K - 1; ++j)
        Row8<T>::store(a.hist_out, ((size_t)s * (K - 1) + j) * a.ch + c0, win[j]);
    }
    return;
  }

  // General tiles: a sequence starts inside the tile or within its first
  // K - 1 tokens, or the tile is the ragged last one.
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int tok = t0 - (K - 1) + j;
    if (tok >= ss && tok >= 0) {
      Row8<T> row;
      row.load(a.xbc, (size_t)tok * a.in_stride + c0);
      row.widen(win[j]);
    } else {
      const int hj = (K - 1) - (ss - tok);
      const bool have = a.hist_in && hj >= 0 && hj < K - 1;
      Row8<T> row;
      if (have) row.load(a.hist_in, ((size_t)s * (K - 1) + hj) * a.ch + c0);
#pragma unroll
      for (int c = 0; c < 8; ++c) win[j][c] = 0.f;
      if (have) row.widen(win[j]);
    }
  }

  Row8<T> rows[kConvBatch], next[kConvBatch];
#pragma unroll
  for (int u = 0; u < kConvBatch; ++u)
    if (t0 + u < t1) rows[u].load(a.xbc, (size_t)(t0 + u) * a.in_stride + c0);

#pragma unroll
  for (int tb = 0; tb < kConvTile; tb += kConvBatch) {
    const int tn = t0 + tb + kConvBatch;
    if (tb + kConvBatch < kConvTile) {
#pragma unroll
      for (int u = 0; u < kConvBatch; ++u)
        if (tn + u < t1) next[u].load(a.xbc, (size_t)(tn + u) * a.in_stride + c0);
    }
#pragma unroll
    for (int u = 0; u < kConvBatch; ++u) {
      const int t = t0 + tb + u;
      if (t < t1) {
        if (t == se) {  // the next non-empty sequence starts here
          if (a.cu) {
            // (clamped: offsets that are not a valid partition must not
            // send s past the last sequence)
            s = min(s + 1, a.nseq - 1);
            while (s + 1 < a.nseq && a.cu[s + 1] <= t) ++s;
            se = a.cu[s + 1];
          } else {
            ++s;
            se = t + a.seqlen;
          }
          ss = t;
          load_history<K, T>(a, s, c0, win);
        }
        float cur[8], out[8];
        rows[u].widen(cur);
        conv_token<K>(w, bias, win, cur, out);
        Row8<T>::store(dst, (size_t)t * dstride + dcol, out);
        if (t == se - 1 && a.hist_out) {
#pragma unroll
          for (int j = 0; j < K - 1; ++j)
            Row8<T>::store(a.hist_out, ((size_t)s * (K - 1) + j) * a.ch + c0, win[j]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kConvBatch; ++u) rows[u] = next[u];
  }
}

// The final history of every sequence without tokens: its initial history,
// or zeros. One lane per (sequence, channel group).
template <int K, typename T>
__global__ __launch_bounds__(kConvThreads) void k_conv_history_of_empty(ConvArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
  const int s = (int)(gid / a.groups);
  if (s >= a.nseq) return;
  const int c0 = (int)(gid - (int64_t)s * a.groups) * 8;
  const int len = a.cu ? a.cu[s + 1] - a.cu[s] : a.seqlen;
  if (len != 0) return;
  float win[K - 1][8];
  load_history<K, T>(a, s, c0, win);
#pragma unroll
  for (int j = 0; j < K - 1; ++j)
    Row8<T>::store(a.hist_out, ((size_t)s * (K - 1) + j) * a.ch + c0, win[j]);
}

template <int K, typename T>
static hipError_t launch_width(const ConvArgs &a, hipStream_t st) {
  if (a.T > 0) {
    const int64_t threads = (int64_t)a.tiles * a.groups;
    const unsigned blocks = (unsigned)((threads + kConvThreads - 1) / kConvThreads);
    hipLaunchKernelGGL((k_conv_silu<K, T>), dim3(blocks), dim3(kConvThreads), 0, st, a);
  }
  // Empty sequences exist only when packed (a zero length) or when the dense
  // rows have no tokens.
  if (a.hist_out && (a.cu || a.seqlen == 0)) {
    const int64_t threads = (int64_t)a.nseq * a.groups;
    const unsigned blocks = (unsigned)((threads + kConvThreads - 1) / kConvThreads);
    hipLaunchKernelGGL((k_conv_history_of_empty<K, T>), dim3(blocks), dim3(kConvThreads), 0,
                       st, a);
  }
  return hipGetLastError();
}

hipError_t launch_conv(const ConvArgs &a, int width, bool bf16_io, hipStream_t st) {
  switch (width) {
    case 2: return bf16_io ? launch_width<2, bf16>(a, st) : launch_width<2, float>(a, st);
    case 3: return bf16_io ? launch_width<3, bf16>(a, st) : launch_width<3, float>(a, st);
    case 4: return bf16_io ? launch_width<4, bf16>(a, st) : launch_width<4, float>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
