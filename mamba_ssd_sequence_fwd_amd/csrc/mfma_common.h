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
  // one vector conversion (v_cvt_pk_bf16_f32 takes both halves at once)
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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

// ---- row-major staging + LDS transpose reads ------------------------------
// Token-major tiles live in LDS as [token][W] bf16 rows with 16-byte chunks
// XOR-swizzled by (token & 7): element (s, c) at s*W + (((c>>3) ^ (s&7))<<3) + (c&7).
// Operands that need the token index inside a lane's K slots are read with
// ds_read_b64_tr_b16, which transposes inside each 16-lane block: a lane
// receives element (d % 4) of the 8-byte segments addressed by lanes d/4,
// d/4 + 4, d/4 + 8, d/4 + 12 of its block (d = lane % 16).
template <int W>
__device__ __forceinline__ int rswz(int s, int c) {
  return s * W + ((((c >> 3) ^ (s & 7))) << 3) + (c & 7);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 4 bf16 of a transposed read; `elem` = this lane's 8-byte segment.
__device__ __forceinline__ bf16x4 ds_tr4(const bf16 *lds_base, int elem) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(lds_base + elem));
  return __builtin_bit_cast(bf16x4, v);
}

// K = 8 consecutive tokens s0 + 8*lg .. +7 for column c0 + lane%16 of a
// row-major [token][W] tile: the MFMA operand whose rows are columns of the
// tile and whose K is the token index (natural K order).
template <int W>
__device__ __forceinline__ bf16x8 tr_operand(const bf16 *t, int s0, int c0) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int row = s0 + 8 * lg + (lr >> 2), col = c0 + 4 * (lr & 3);
  const bf16x4 a = ds_tr4(t, rswz<W>(row, col));
  const bf16x4 b = ds_tr4(t, rswz<W>(row + 4, col));
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Same, in the K order of the C B^T tiles: slot e <-> token
// s0 + 16 (e / 4) + 4 lg + (e % 4).
template <int W>
__device__ __forceinline__ bf16x8 tr_operand_cb(const bf16 *t, int s0, int c0) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int row = s0 + 4 * lg + (lr >> 2), col = c0 + 4 * (lr & 3);
  const bf16x4 a = ds_tr4(t, rswz<W>(row, col));
  const bf16x4 b = ds_tr4(t, rswz<W>(row + 16, col));
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Row-major staging of NTOK tokens x W columns of a token-major bf16 matrix
// (row stride ld, rows >= len read as zero). Work item = 16 bytes; the
// column chunk varies fastest so a wave's loads cover whole rows. Loads go to
// registers first (load()), LDS later (store()), so they can be issued early.
template <int W, int NTOK, int NTHR>
struct RowStager {
  static constexpr int kItems = NTOK * (W / 8);
  static constexpr int kPer = kItems / NTHR;
  static_assert(kItems % NTHR == 0, "staging work must divide evenly");
  bf16x8 v[kPer];

  __device__ __forceinline__ void load(const bf16 *src, size_t ld, int s0, int len) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int it = threadIdx.x + k * NTHR;
      const int c = it % (W / 8), s = it / (W / 8);
      v[k] = ldg8_row(src, ld, s0 + s, len, 8 * c);
    }
  }
  // Plain copy into dst[(s) * W ...] (rows relative to s0).
  __device__ __forceinline__ void store(bf16 *dst) const {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int it = threadIdx.x + k * NTHR;
      const int c = it % (W / 8), s = it / (W / 8);
      *reinterpret_cast<bf16x8 *>(dst + rswz<W>(s, 8 * c)) = v[k];
    }
  }
  // Copy with every token row s scaled by scale[s0 + s] (rounded to bf16).
  __device__ __forceinline__ void store_scaled(bf16 *dst, const float *scale, int s0) const {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int it = threadIdx.x + k * NTHR;
      const int c = it % (W / 8), s = it / (W / 8);
      const float w = scale[s0 + s];
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[k][e] * w);
      *reinterpret_cast<bf16x8 *>(dst + rswz<W>(s, 8 * c)) = o;
    }
  }
};

// Per-chunk decay tables, one token per thread (t < Q):
//   sU[t] = 2^(cs_e - cs_t) dt_t, e = last token of t's 32-token tile
// used by the off-diagonal output tiles.
template <int Q>
__device__ __forceinline__ void fill_tile_decay(float *sU, const float *sCs, const float *sDt,
                                                int t) {
  if (t < Q) sU[t] = exp2_fast(sCs[(t | 31)] - sCs[t]) * sDt[t];
}

// Outputs of the 32-row tile i of one chunk and one head (rows 32i..32i+31),
// computed transposed (y^T = p x l) so each lane ends with one row l and four
// consecutive p:
//   y_l = 2^(cs_l) C_l h_in^T + sum_{s<=l} CB[l,s] 2^(cs_l - cs_s) dt_s x_s + D x_l
// One wave. sX = x [token][P] row-major (swizzled), sH = h_in bf16 [p][n]
// (row width N), sCs/sDt/sU = log2-decay prefix, dt (zero past the chunk
// end) and the tile decay table; C = the chunk's first C row of this group
// (row stride ldc); cbase = this (chunk, group)'s C B^T tiles already offset
// by lane*8; y = the chunk's first output row of this head (stride ystride).
// Off-diagonal tiles (j < i): the decay 2^(cs_l - cs_s) is the product of
// 2^(cs_l - cs_r0) (r0 = first row of tile i), 2^(cs_r0 - cs_e) (e = last
// token of tile j) and 2^(cs_e - cs_s): three factors <= 1, so nothing can
// overflow. The diagonal tile takes the exact masked exponent and carries the
// skip term D on its diagonal. The next C B^T tile is always in flight.
template <int N, int Q>
__device__ __forceinline__ void chunk_rows_out(int i, const bf16 *sX, const bf16 *sH,
                                               const float *sCs, const float *sDt,
                                               const float *sU, const bf16 *C, size_t ldc,
                                               const bf16 *cbase, int len, bf16 *y,
                                               size_t ystride, float dsk) {
  constexpr int KS = N / 32;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int pair0 = i * (i + 1) / 2;
  bf16x8 mnext[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) mnext[u] = ldg8(cbase + (size_t)(pair0 * 2 + u) * 512);

  f32x4 Y[2][4];  // Y[u][pt]: column l = 32i + 16u + lr, rows p = 16pt + 4lg + r
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[u][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // (a) state entering the chunk: h C^T, then 2^(cs_l) per column l.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 ac[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) ac[u] = ldg8_row(C, ldc, 32 * i + 16 * u + lr, len, 32 * ks + 8 * lg);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x8 bh =
          *reinterpret_cast<const bf16x8 *>(sH + swz<N>(16 * pt + lr, 32 * ks + 8 * lg));
#pragma unroll
      for (int u = 0; u < 2; ++u) Y[u][pt] = mfma(bh, ac[u], Y[u][pt]);
    }
  }
  float cs_l[2], rdec[2];
  const float cs_r0 = sCs[32 * i];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    cs_l[u] = sCs[32 * i + 16 * u + lr];
    rdec[u] = exp2_fast(cs_l[u] - cs_r0);
    const float f = exp2_fast(cs_l[u]);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[u][pt] *= f;
  }

  // (b) intra-chunk tiles j <= i.
#pragma unroll 1
  for (int j = 0; j <= i; ++j) {
    bf16x8 m[2] = {mnext[0], mnext[1]};
    if (j < i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) mnext[u] = ldg8(cbase + (size_t)((pair0 + j + 1) * 2 + u) * 512);
      const float alpha = exp2_fast(cs_r0 - sCs[32 * j + 31]);
      const float4 ua = *reinterpret_cast<const float4 *>(sU + 32 * j + 4 * lg);
      const float4 ub = *reinterpret_cast<const float4 *>(sU + 32 * j + 16 + 4 * lg);
      const float uu[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float fa = rdec[u] * alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) m[u][e] = (bf16)((float)m[u][e] * (fa * uu[e]));
      }
    } else {
      const float4 ca = *reinterpret_cast<const float4 *>(sCs + 32 * j + 4 * lg);
      const float4 cb4 = *reinterpret_cast<const float4 *>(sCs + 32 * j + 16 + 4 * lg);
      const float4 da = *reinterpret_cast<const float4 *>(sDt + 32 * j + 4 * lg);
      const float4 db = *reinterpret_cast<const float4 *>(sDt + 32 * j + 16 + 4 * lg);
      const float cc[8] = {ca.x, ca.y, ca.z, ca.w, cb4.x, cb4.y, cb4.z, cb4.w};
      const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int l = 32 * i + 16 * u + lr;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = 32 * j + 16 * (e >> 2) + 4 * lg + (e & 3);
          const float v = (float)m[u][e] * exp2_fast(cs_l[u] - cc[e]) * dd[e] + (s == l ? dsk : 0.f);
          m[u][e] = (bf16)(s <= l ? v : 0.f);
        }
      }
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x8 xv = tr_operand_cb<kP>(sX, 32 * j, 16 * pt);
#pragma unroll
      for (int u = 0; u < 2; ++u) Y[u][pt] = mfma(xv, m[u], Y[u][pt]);
    }
  }

  // (c) round to bf16 and store: lane holds row l, columns 16pt+4lg .. +3.
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int l = 32 * i + 16 * u + lr;
    if (l < len) {
      bf16 *yr = y + (size_t)l * ystride + 4 * lg;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        uint2 o;
        o.x = pack2(Y[u][pt][0], Y[u][pt][1]);
        o.y = pack2(Y[u][pt][2], Y[u][pt][3]);
        *reinterpret_cast<uint2 *>(yr + 16 * pt) = o;
      }
    }
  }
}

// Lane-constant part of the address of a transposed read of a row-major
// [token][W] tile (see tr_operand): row r0 + 8*lg + (lr >> 2) (+4 for the
// second half), column c0 + 4*(lr & 3). Only the token base differs between
// calls, and it is a multiple of 8, so the swizzle (row & 7) is lane-constant.
template <int W>
__device__ __forceinline__ int tr_lane_off(int c0, int row_in_8) {
  const int lane = threadIdx.x & 63, lr = lane & 15;
  const int c = c0 + 4 * (lr & 3);
  return ((((c >> 3) ^ row_in_8)) << 3) + (c & 7);
}

// Loads of one 16-row half tile that can be issued early (before the
// barriers of a chunk step): its C rows and its first two C B^T tiles.
template <int N>
struct HalfTileLoads {
  bf16x8 ac[N / 32];
  bf16x8 m0, m1;

  __device__ __forceinline__ void issue(int i, int u, const bf16 *C, size_t ldc, int len,
                                        const bf16 *cbase) {
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const int l = 32 * i + 16 * u + lr;
    const bf16 *crow = C + (size_t)min(l, len - 1) * ldc + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) ac[ks] = ldg8(crow + 32 * ks);
    const int pair0 = i * (i + 1) / 2;
    m0 = ldg8(cbase + (size_t)(pair0 * 2 + u) * 512);
    m1 = ldg8(cbase + (size_t)((pair0 + min(1, i)) * 2 + u) * 512);
  }
};

// Outputs of rows 32i + 16u .. +15 of one chunk and one head (one wave), in
// the same way as chunk_rows_out but for a 16-row half tile; see there.
// `ld` holds the early loads of this half tile; C B^T tiles stream two ahead.
template <int N, int Q>
__device__ __forceinline__ void chunk_rows_out16(int i, int u, HalfTileLoads<N> &ld,
                                                 const bf16 *sX, const bf16 *sH,
                                                 const float *sCs, const float *sDt,
                                                 const float *sU, const bf16 *cbase, int len,
                                                 bf16 *y, size_t ystride, float dsk) {
  constexpr int KS = N / 32;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int pair0 = i * (i + 1) / 2;
  const int l = 32 * i + 16 * u + lr;

  f32x4 Y[4];  // column l, rows p = 16pt + 4lg + r
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) Y[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // (a) state entering the chunk: h C^T, then 2^(cs_l).
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 acv = l < len ? ld.ac[ks] : zero8();
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x8 bh =
          *reinterpret_cast<const bf16x8 *>(sH + swz<N>(16 * pt + lr, 32 * ks + 8 * lg));
      Y[pt] = mfma(bh, acv, Y[pt]);
    }
  }
  const float cs_l = sCs[l];
  const float cs_r0 = sCs[32 * i];
  const float rdec = exp2_fast(cs_l - cs_r0);
  {
    const float f = exp2_fast(cs_l);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[pt] *= f;
  }

  // Transposed-read addresses of the x operand (K order of the C B^T tiles):
  // rows 32j + 4lg + (lr>>2) and +16, columns 16pt + 4(lr&3).
  const int xrow = 4 * lg + (lr >> 2);
  int xoff[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) xoff[pt] = xrow * kP + tr_lane_off<kP>(16 * pt, xrow & 7);

  // (b) intra-chunk tiles j <= i.
  bf16x8 mq0 = ld.m0, mq1 = ld.m1;
#pragma unroll 1
  for (int j = 0; j <= i; ++j) {
    bf16x8 m = mq0;
    mq0 = mq1;
    mq1 = ldg8(cbase + (size_t)((pair0 + min(j + 2, i)) * 2 + u) * 512);
    if (j < i) {
      const float fa = rdec * exp2_fast(cs_r0 - sCs[32 * j + 31]);
      const float4 ua = *reinterpret_cast<const float4 *>(sU + 32 * j + 4 * lg);
      const float4 ub = *reinterpret_cast<const float4 *>(sU + 32 * j + 16 + 4 * lg);
      const float uu[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = (bf16)((float)m[e] * (fa * uu[e]));
    } else {
      // Diagonal tile: local offsets decide the causal mask (lane-constant).
      const float4 ca = *reinterpret_cast<const float4 *>(sCs + 32 * j + 4 * lg);
      const float4 cb4 = *reinterpret_cast<const float4 *>(sCs + 32 * j + 16 + 4 * lg);
      const float4 da = *reinterpret_cast<const float4 *>(sDt + 32 * j + 4 * lg);
      const float4 db = *reinterpret_cast<const float4 *>(sDt + 32 * j + 16 + 4 * lg);
      const float cc[8] = {ca.x, ca.y, ca.z, ca.w, cb4.x, cb4.y, cb4.z, cb4.w};
      const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
      const int lloc = 16 * u + lr;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sloc = 16 * (e >> 2) + 4 * lg + (e & 3);
        const float v = (float)m[e] * exp2_fast(cs_l - cc[e]) * dd[e];
        const float w = sloc == lloc ? v + dsk : v;
        m[e] = (bf16)(sloc <= lloc ? w : 0.f);
      }
    }
    const int jb = 32 * j * kP;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x4 lo = ds_tr4(sX, jb + xoff[pt]);
      const bf16x4 hi = ds_tr4(sX, jb + xoff[pt] + 16 * kP);
      const bf16x8 xv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      Y[pt] = mfma(xv, m, Y[pt]);
    }
  }

  // (c) round to bf16 and store: lane holds row l, columns 16pt+4lg .. +3.
  if (l < len) {
    bf16 *yr = y + (size_t)l * ystride + 4 * lg;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      uint2 o;
      o.x = pack2(Y[pt][0], Y[pt][1]);
      o.y = pack2(Y[pt][2], Y[pt][3]);
      *reinterpret_cast<uint2 *>(yr + 16 * pt) = o;
    }
  }
}

// ---- direct global -> LDS staging (gfx950 global_load_lds, 16 B per lane) --
typedef __attribute__((address_space(3))) void lds_void;

// Asynchronously copy ROWS token rows (row stride ld, W bf16 columns) into
// the row-major swizzled LDS tile `tile` (layout of rswz<W>). Lane L of a
// wave instruction fills LDS slot L, so each lane fetches the source chunk
// that the swizzle maps to its slot; rows >= len are read from `zeros`.
// All waves of a 512-thread workgroup share the work. The data is only
// visible after s_waitcnt vmcnt(0) and a barrier.
template <int W, int ROWS>
__device__ __forceinline__ void async_tile(bf16 *tile, const bf16 *src, size_t ld, int len,
                                           const bf16 *zeros) {
  constexpr int R = 512 / W;   // rows per 1 KB wave instruction
  constexpr int NI = ROWS / R; // wave instructions for the tile
  static_assert(NI % 8 == 0, "tile must split over 8 waves");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / (W / 8), pc = lane % (W / 8);
#pragma unroll
  for (int k = 0; k < NI / 8; ++k) {
    const int m = wave + 8 * k;
    const int s = m * R + rl;
    const int c = (pc & ~7) | ((pc & 7) ^ (s & 7));
    const bf16 *g = s < len ? src + (size_t)s * ld + 8 * c : zeros;
    __builtin_amdgcn_global_load_lds(g, (lds_void *)(tile + m * 512), 16, 0, 0);
  }
}

// Same copy with rows >= len read from row len - 1 instead (finite data the
// caller multiplies by zero), by a workgroup of NW waves. Every lane
// addresses `src` (a workgroup-uniform base) plus a 32-bit byte offset, so no
// per-lane 64-bit addresses stay alive between copies. Needs len >= 1 and
// ROWS * ld * 2 < 2^31.
template <int W, int ROWS, int NW>
__device__ __forceinline__ void async_rows(bf16 *tile, const bf16 *src, size_t ld, int len,
                                           int lane) {
  constexpr int R = 512 / W;   // rows per 1 KB wave instruction
  constexpr int NI = ROWS / R; // wave instructions for the tile
  static_assert(NI % NW == 0, "tile must split evenly over the waves");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane / (W / 8), pc = lane % (W / 8);
  const char *base = reinterpret_cast<const char *>(src);
#pragma unroll
  for (int k = 0; k < NI / NW; ++k) {
    const int m = wave + NW * k;
    const int s = m * R + rl;
    const int c = (pc & ~7) | ((pc & 7) ^ (s & 7));
    const uint32_t off = (uint32_t)min(s, len - 1) * (uint32_t)(ld * 2) + 16u * (uint32_t)c;
    __builtin_amdgcn_global_load_lds(base + off, (lds_void *)(tile + m * 512), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Entry idx of a register-resident tile array (idx wave-uniform): a chain of
// selects, so the array stays in registers.
template <int NE>
__device__ __forceinline__ bf16x8 pick(const bf16x8 (&t)[NE], int idx) {
  bf16x8 r = t[0];
#pragma unroll
  for (int e = 1; e < NE; ++e)
    if (idx == e) r = t[e];
  return r;
}

// Outputs of rows 32i + 16u .. +15 of one chunk and one head (one wave), with
// every global operand already in registers: ac = the half tile's C rows
// (zeros past the chunk end are applied here), cbt = its C B^T tiles, tile j
// at entry j (rev = false) or NE-1-j (rev = true). Same arithmetic as
// chunk_rows_out; this variant issues no global load, so it never waits on
// loads issued after the caller's prefetch point.
template <int N, int Q, int NE>
__device__ __forceinline__ void half_tile_out(int i, int u, bool rev, const bf16x8 (&cbt)[NE],
                                              const bf16x8 (&ac)[N / 32], const bf16 *sX,
                                              const bf16 *sH, const float *sCs,
                                              const float *sDt, const float *sU, int len,
                                              bf16 *y, size_t ystride, float dsk) {
  constexpr int KS = N / 32, T = Q / 32;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int l = 32 * i + 16 * u + lr;

  f32x4 Y[4];  // column l, rows p = 16pt + 4lg + r
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) Y[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // State entering the chunk: h C^T, then 2^(cs_l).
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 acv = l < len ? ac[ks] : zero8();
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x8 bh =
          *reinterpret_cast<const bf16x8 *>(sH + swz<N>(16 * pt + lr, 32 * ks + 8 * lg));
      Y[pt] = mfma(bh, acv, Y[pt]);
    }
  }
  const float cs_l = sCs[l];
  const float cs_r0 = sCs[32 * i];
  const float rdec = exp2_fast(cs_l - cs_r0);
  {
    const float f = exp2_fast(cs_l);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[pt] *= f;
  }

  const int xrow = 4 * lg + (lr >> 2);
  int xoff[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) xoff[pt] = xrow * kP + tr_lane_off<kP>(16 * pt, xrow & 7);

  // Off-diagonal tiles j < i.
#pragma unroll
  for (int j = 0; j < T - 1; ++j) {
    if (j < i) {
      bf16x8 m = rev ? cbt[NE - 1 - j] : cbt[j];
      const float fa = rdec * exp2_fast(cs_r0 - sCs[32 * j + 31]);
      const float4 ua = *reinterpret_cast<const float4 *>(sU + 32 * j + 4 * lg);
      const float4 ub = *reinterpret_cast<const float4 *>(sU + 32 * j + 16 + 4 * lg);
      const float uu[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = (bf16)((float)m[e] * (fa * uu[e]));
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const bf16x4 lo = ds_tr4(sX, 32 * j * kP + xoff[pt]);
        const bf16x4 hi = ds_tr4(sX, (32 * j + 16) * kP + xoff[pt]);
        const bf16x8 xv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        Y[pt] = mfma(xv, m, Y[pt]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // Diagonal tile j = i: exact masked exponent, skip term D on its diagonal.
  {
    bf16x8 m = pick(cbt, rev ? NE - 1 - i : i);
    const float4 ca = *reinterpret_cast<const float4 *>(sCs + 32 * i + 4 * lg);
    const float4 cb4 = *reinterpret_cast<const float4 *>(sCs + 32 * i + 16 + 4 * lg);
    const float4 da = *reinterpret_cast<const float4 *>(sDt + 32 * i + 4 * lg);
    const float4 db = *reinterpret_cast<const float4 *>(sDt + 32 * i + 16 + 4 * lg);
    const float cc[8] = {ca.x, ca.y, ca.z, ca.w, cb4.x, cb4.y, cb4.z, cb4.w};
    const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
    const int lloc = 16 * u + lr;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sloc = 16 * (e >> 2) + 4 * lg + (e & 3);
      const float v = (float)m[e] * exp2_fast(cs_l - cc[e]) * dd[e];
      const float w = sloc == lloc ? v + dsk : v;
      m[e] = (bf16)(sloc <= lloc ? w : 0.f);
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x4 lo = ds_tr4(sX, 32 * i * kP + xoff[pt]);
      const bf16x4 hi = ds_tr4(sX, (32 * i + 16) * kP + xoff[pt]);
      const bf16x8 xv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      Y[pt] = mfma(xv, m, Y[pt]);
    }
  }

  // Round to bf16 and store: lane holds row l, columns 16pt+4lg .. +3.
  if (l < len) {
    bf16 *yr = y + (size_t)l * ystride + 4 * lg;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      uint2 o;
      o.x = pack2(Y[pt][0], Y[pt][1]);
      o.y = pack2(Y[pt][2], Y[pt][3]);
      *reinterpret_cast<uint2 *>(yr + 16 * pt) = o;
    }
  }
}

}  // namespace ssd
