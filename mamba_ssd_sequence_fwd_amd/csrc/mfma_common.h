// mfma_common.h -- bf16 MFMA building blocks shared by the chunk kernels and
// the fused kernel (gfx950): operand types, the 16x16x32 MFMA, swizzled LDS
// addressing, clamped 16-byte loads and transposed LDS staging.
#pragma once

#include "ssd_internal.h"

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kP = 64;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
  return z;
}

// Element offset of (row, col) in a swizzled [rows][W] bf16 LDS tile.
template <int W>
__device__ __forceinline__ int swz(int row, int col) {
  return row * W + ((((col >> 3) ^ (row & 7))) << 3) + (col & 7);
}

__device__ __forceinline__ bf16x8 ldg8(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// 16 bytes of token row r of a token-major matrix, or zeros when r >= len.
// The load itself is unconditional (row clamped into the chunk) so that the
// compiler keeps a batch of such loads in flight instead of branching and
// waiting on each one.
__device__ __forceinline__ bf16x8 ldg8_row(const bf16 *base, size_t ld, int r, int len,
                                          int col) {
  const bf16x8 v = ldg8(base + (size_t)min(r, len - 1) * ld + col);
  return r < len ? v : zero8();
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16 a = (bf16)lo, b = (bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Transposed staging of a token-major bf16 matrix (row stride `ld` elements,
// W columns) into a swizzled LDS tile dst[col][s - s0] of row width WT, for
// tokens [s0, s0 + 2*NPAIRS), rows >= len read as zero, token s scaled by
// scale[s]. Each work item moves 2 tokens x 8 columns (two 16-byte loads,
// eight 32-bit LDS stores with the token pair packed). Split in two phases
// so every global load of a thread is in flight before the first store:
// stage_load() fills registers, stage_store() writes LDS.
template <int W, int NPAIRS, int NTHR>
struct Stager {
  static constexpr int kItems = NPAIRS * (W / 8);
  static constexpr int kPer = (kItems + NTHR - 1) / NTHR;
  bf16x8 v0[kPer], v1[kPer];

  __device__ __forceinline__ void load(const bf16 *src, size_t ld, int s0, int len) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int it = threadIdx.x + k * NTHR;
      const int sp = it % NPAIRS, cg = it / NPAIRS;
      const int s = s0 + 2 * sp;
      static_assert(kItems % NTHR == 0, "staging work must divide evenly");
      v0[k] = ldg8_row(src, ld, s, len, 8 * cg);
      v1[k] = ldg8_row(src, ld, s + 1, len, 8 * cg);
    }
  }

  template <int WT>
  __device__ __forceinline__ void store(bf16 *dst, int s0, const float *scale) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int it = threadIdx.x + k * NTHR;
      const int sp = it % NPAIRS, cg = it / NPAIRS;
      const int s = s0 + 2 * sp;
      const float w0 = scale ? scale[s] : 1.f, w1 = scale ? scale[s + 1] : 1.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t pr = pack2((float)v0[k][e] * w0, (float)v1[k][e] * w1);
        *reinterpret_cast<uint32_t *>(dst + swz<WT>(8 * cg + e, 2 * sp)) = pr;
      }
    }
  }
};

// Outputs of the 32-row tile i of one chunk and one head (rows 32i..32i+31):
//   y_l = 2^(cs_l) C_l h_in^T + sum_{s<=l} CB[l,s] 2^(cs_l - cs_s) dt_s x_s + D x_l
// One wave. Inputs: sX = x^T [p][s] (row width Q), sH = h_in bf16 [p][n]
// (row width N), sCs/sDt = chunk log2-decay prefix and dt (zero dt past the
// chunk end), C = the chunk's first C row of this group (row stride ldc),
// cbase = this (chunk, group)'s C B^T tiles already offset by lane*8, y = the
// chunk's first output row of this head (row stride ystride).
// The mask M[l,s] = CB[l,s] 2^(cs_l - cs_s) dt_s is built in registers: for
// off-diagonal tiles (j < i) the decay is split at the tile's first row r0,
// 2^(cs_l - cs_r0) 2^(cs_r0 - cs_s), both factors <= 1, so nothing can
// overflow; diagonal tiles take the exact masked exponent. The CB tile of
// the next step is always in flight while the current one is used.
template <int N, int Q>
__device__ __forceinline__ void chunk_rows_out(int i, const bf16 *sX, const bf16 *sH,
                                               const float *sCs, const float *sDt,
                                               const bf16 *C, size_t ldc, const bf16 *cbase,
                                               int len, bf16 *y, size_t ystride, float dsk) {
  constexpr int KS = N / 32;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int pair0 = i * (i + 1) / 2;
  // First CB tile of this row tile: in flight during the state term.
  bf16x8 mnext[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) mnext[u] = ldg8(cbase + (size_t)(pair0 * 2 + u) * 512);
  bf16x8 ac[2][KS];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 32 * i + 16 * u + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ac[u][ks] = ldg8_row(C, ldc, row, len, 32 * ks + 8 * lg);
  }

  f32x4 Y[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[u][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // (a) state entering the chunk: C h_in^T, then 2^(cs_l) per row.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x8 bh =
          *reinterpret_cast<const bf16x8 *>(sH + swz<N>(16 * pt + lr, 32 * ks + 8 * lg));
#pragma unroll
      for (int u = 0; u < 2; ++u) Y[u][pt] = mfma(ac[u][ks], bh, Y[u][pt]);
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float f = exp2_fast(sCs[32 * i + 16 * u + 4 * lg + r]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) Y[u][pt][r] *= f;
    }

  // (b) intra-chunk tiles j <= i.
  const float cs_r0 = sCs[32 * i];
  float cs_row[2], rdec[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    cs_row[u] = sCs[32 * i + 16 * u + lr];
    rdec[u] = exp2_fast(cs_row[u] - cs_r0);
  }
#pragma unroll 1
  for (int j = 0; j <= i; ++j) {
    bf16x8 m[2] = {mnext[0], mnext[1]};
    if (j < i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) mnext[u] = ldg8(cbase + (size_t)((pair0 + j + 1) * 2 + u) * 512);
      float q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int s = 32 * j + 16 * (e >> 2) + 4 * lg + (e & 3);
        q[e] = exp2_fast(cs_r0 - sCs[s]) * sDt[s];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) m[u][e] = (bf16)((float)m[u][e] * (rdec[u] * q[e]));
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int l = 32 * i + 16 * u + lr;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = 32 * j + 16 * (e >> 2) + 4 * lg + (e & 3);
          const float v = (float)m[u][e] * exp2_fast(cs_row[u] - sCs[s]) * sDt[s];
          m[u][e] = (bf16)(s <= l ? v : 0.f);
        }
      }
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int p = 16 * pt + lr;
      const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(sX + swz<Q>(p, 32 * j + 4 * lg));
      const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(sX + swz<Q>(p, 32 * j + 16 + 4 * lg));
      bf16x8 xv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[e] = lo[e];
        xv[4 + e] = hi[e];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) Y[u][pt] = mfma(m[u], xv, Y[u][pt]);
    }
  }

  // (c) skip term (x from LDS), round to bf16, store. Lane holds column p
  // and rows 4*lg .. 4*lg+3 of each 16-row half.
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int l0 = 32 * i + 16 * u + 4 * lg;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int p = 16 * pt + lr;
      const bf16x4 xs = *reinterpret_cast<const bf16x4 *>(sX + swz<Q>(p, l0));
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (l0 + r < len) y[(size_t)(l0 + r) * ystride + p] = (bf16)(Y[u][pt][r] + dsk * (float)xs[r]);
    }
  }
}

}  // namespace ssd
