// k_scan.hip -- the Mamba-1 selective scan (a diagonal A per channel), the
// comparator of the SSD forward pass.
//
// The selective SSM discretises with exp(step * A), with the step, B and C
// functions of the input (tj-hxxt.cn long read of the Mamba-1 paper, part III
// (二) and item 3); A is a diagonal N x D matrix broadcast over the expanded
// state of every channel (kuaisou snippet on selective SSMs as linear
// attention). Its efficient form keeps the (batch, L, D, N) state on chip:
// load the step, A, B and C, discretise and scan in fast memory, write only
// the (batch, L, D) output (same long read, part III (三)). Mamba-2 restricts
// A to one scalar per head, which the pages credit with a 2-8x speed-up over
// this scan. Per sequence b, channel d, state index n:
//
//   h[d,n] <- exp(step[t,d] A[d,n]) h[d,n] + step[t,d] B[t,n] x[t,d]
//   y[t,d]  = sum_n C[t,n] h[d,n] + D[d] x[t,d]
//
// Every (t, d, n) costs one exp and two fused multiply-adds, so the scan is
// bound by vector-ALU issue (the exp runs at a quarter of the rate of the
// others), not by HBM. Layout: one lane holds 4 consecutive states of one
// channel (R = N/4 lanes per channel, 64/R channels per wave), a 4-wave
// workgroup covers CPB = 256/R consecutive channels of one sequence, and the
// time axis is walked in tiles of kScanTile tokens. Each tile's x and step
// (interleaved per channel), B and C (interleaved per state) sit in LDS,
// widened to fp32 once when the tile is stored (rather than at every read);
// the next tile is loaded into registers while the current one is scanned;
// y goes through an LDS tile so that it is written as whole rows. The sum
// over a channel's lanes uses DPP lane moves inside 16-lane rows. Measured at
// N = 16 on 5120 channels x 2048 tokens x 8: 602 us with shuffles through
// LDS for the sum and bf16 tiles, 520 us with DPP, 440 us with fp32 tiles.
#include "scan.h"

namespace ssd {

constexpr int kScanTile = 32;
constexpr float kLog2eScan = 1.4426950408889634f;

// Sum over the R lanes of one channel (R a power of two, lanes aligned).
template <int Ctrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Ctrl, 0xf, 0xf, false));
}
template <int R>
__device__ __forceinline__ float channel_sum(float v) {
  // within a row of 16 lanes: quad swaps (xor 1, xor 2), then the half-row
  // and row mirrors pair quads and half rows; wider sums cross rows
  if (R >= 2) v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if (R >= 4) v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if (R >= 8) v += dpp_move<0x141>(v);  // row_half_mirror
  if (R >= 16) v += dpp_move<0x140>(v); // row_mirror
#pragma unroll
  for (int off = 16; off < R; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

template <int R, typename T>
__global__ __launch_bounds__(256) void k_selective_scan(ScanArgs a) {
  constexpr int N = 4 * R, CPW = 64 / R, CPB = 4 * CPW;
  constexpr int ES = sizeof(T);
  // A tile row of x (or step) is CPB * ES bytes, of B (or C) N * ES bytes;
  // both move in chunks of up to 16 bytes.
  constexpr int RX = CPB * ES, CHX = RX >= 16 ? 16 : RX, XPR = RX / CHX;
  constexpr int RB = N * ES, CHB = RB >= 16 ? 16 : RB, BPR = RB / CHB;
  constexpr int XN = kScanTile * XPR, BN = kScanTile * BPR;
  constexpr int XPER = (XN + 255) / 256, BPER = (BN + 255) / 256;
  __shared__ __attribute__((aligned(16))) float sXD[kScanTile][CPB][2];  // (x, step), fp32
  __shared__ __attribute__((aligned(16))) float sBC[kScanTile][N][2];    // (B, C), fp32
  __shared__ __attribute__((aligned(16))) T sY[kScanTile][CPB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y, d0 = blockIdx.x * CPB;
  const int c = wave * CPW + lane / R, n0 = 4 * (lane % R), d = d0 + c;
  const int64_t L = a.L, Dm = a.dim;
  const T *xg = static_cast<const T *>(a.x) + (size_t)b * L * Dm + d0;
  const T *dg = static_cast<const T *>(a.delta) + (size_t)b * L * Dm + d0;
  const T *Bg = static_cast<const T *>(a.B) + (size_t)b * L * N;
  const T *Cg = static_cast<const T *>(a.C) + (size_t)b * L * N;
  T *yg = static_cast<T *>(a.y) + (size_t)b * L * Dm + d0;

  // This lane's decay rates (base 2), skip weight and initial state.
  const float4 av = *reinterpret_cast<const float4 *>(a.A + (size_t)d * N + n0);
  const float a2[4] = {av.x * kLog2eScan, av.y * kLog2eScan, av.z * kLog2eScan,
                       av.w * kLog2eScan};
  const float dskip = a.D ? a.D[d] : 0.f;
  float h[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.h0) {
    const float4 v = *reinterpret_cast<const float4 *>(a.h0 + ((size_t)b * Dm + d) * N + n0);
    h[0] = v.x;
    h[1] = v.y;
    h[2] = v.z;
    h[3] = v.w;
  }

  // Registers of the next tile: item i of this thread is chunk tid + 256 i.
  // Token rows past the sequence end read the last token (finite values);
  // their step is set to zero when the tile is stored, so they change nothing.
  typedef __attribute__((ext_vector_type(CHX / 4))) uint32_t XChunk;
  typedef __attribute__((ext_vector_type(CHB / 4))) uint32_t BChunk;
  XChunk xr[XPER], dr[XPER];
  BChunk br[BPER], cr[BPER];
  auto load_tile = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < XPER; ++i) {
      const int q = tid + 256 * i;
      if (XN % 256 == 0 || q < XN) {
        const int r = q / XPR, k = q % XPR;
        const int64_t t = min(t0 + r, L - 1);
        xr[i] = *reinterpret_cast<const XChunk *>(reinterpret_cast<const char *>(xg + t * Dm) + k * CHX);
        dr[i] = *reinterpret_cast<const XChunk *>(reinterpret_cast<const char *>(dg + t * Dm) + k * CHX);
      }
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int q = tid + 256 * i;
      if (BN % 256 == 0 || q < BN) {
        const int r = q / BPR, k = q % BPR;
        const int64_t t = min(t0 + r, L - 1);
        br[i] = *reinterpret_cast<const BChunk *>(reinterpret_cast<const char *>(Bg + t * N) + k * CHB);
        cr[i] = *reinterpret_cast<const BChunk *>(reinterpret_cast<const char *>(Cg + t * N) + k * CHB);
      }
    }
  };
  auto store_tile = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < XPER; ++i) {
      const int q = tid + 256 * i;
      if (XN % 256 == 0 || q < XN) {
        constexpr int EPC = CHX / ES;
        const int r = q / XPR, k = q % XPR;
        const bool live = t0 + r < L;
        const XChunk vx = xr[i], vd = dr[i];
        const T *ex = reinterpret_cast<const T *>(&vx);
        const T *ed = reinterpret_cast<const T *>(&vd);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          sXD[r][k * EPC + e][0] = to_f32(ex[e]);
          sXD[r][k * EPC + e][1] = live ? to_f32(ed[e]) : 0.f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int q = tid + 256 * i;
      if (BN % 256 == 0 || q < BN) {
        constexpr int EPC = CHB / ES;
        const int r = q / BPR, k = q % BPR;
        const BChunk vb = br[i], vc = cr[i];
        const T *eb = reinterpret_cast<const T *>(&vb);
        const T *ec = reinterpret_cast<const T *>(&vc);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          sBC[r][k * EPC + e][0] = to_f32(eb[e]);
          sBC[r][k * EPC + e][1] = to_f32(ec[e]);
        }
      }
    }
  };

  const int64_t ntiles = (L + kScanTile - 1) / kScanTile;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int64_t tt = 0; tt < ntiles; ++tt) {
    const int64_t t0 = tt * kScanTile;
    if (tt + 1 < ntiles) load_tile(t0 + kScanTile);  // in flight during the scan
#pragma unroll 4
    for (int t = 0; t < kScanTile; ++t) {
      const float2 xs = *reinterpret_cast<const float2 *>(&sXD[t][c][0]);
      const float xv = xs.x, stp = xs.y;
      const float4 p01 = *reinterpret_cast<const float4 *>(&sBC[t][n0][0]);
      const float4 p23 = *reinterpret_cast<const float4 *>(&sBC[t][n0 + 2][0]);
      const float bv[4] = {p01.x, p01.z, p23.x, p23.z}, cv[4] = {p01.y, p01.w, p23.y, p23.w};
      const float u = stp * xv;
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[k] = exp2_fast(stp * a2[k]) * h[k] + u * bv[k];
        part += cv[k] * h[k];
      }
      part = channel_sum<R>(part);
      if (lane % R == 0) sY[t][c] = from_f32<T>(part + dskip * xv);
    }
    __syncthreads();  // the tile's LDS reads and sY writes are done
    {
      // y rows of the tile (CPB * ES bytes per token), in x's chunking
      for (int q = tid; q < XN; q += 256) {
        const int r = q / XPR, k = q % XPR;
        if (t0 + r < L)
          *reinterpret_cast<XChunk *>(reinterpret_cast<char *>(yg + (t0 + r) * Dm) + k * CHX) =
              *reinterpret_cast<const XChunk *>(reinterpret_cast<const char *>(&sY[r][0]) + k * CHX);
      }
    }
    if (tt + 1 < ntiles) store_tile(t0 + kScanTile);
    __syncthreads();
  }
  if (a.hT)
    *reinterpret_cast<float4 *>(a.hT + ((size_t)b * Dm + d) * N + n0) =
        make_float4(h[0], h[1], h[2], h[3]);
}

int scan_channels_per_block(int N) { return 4 * (64 / (N / 4)); }

template <typename T>
static hipError_t launch_scan_t(const ScanArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.dim / scan_channels_per_block(a.N)), (unsigned)a.batch);
  switch (a.N) {
    case 16: hipLaunchKernelGGL((k_selective_scan<4, T>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_selective_scan<8, T>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_selective_scan<16, T>), grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((k_selective_scan<32, T>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_selective_scan<64, T>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_selective_scan(const ScanArgs &a, bool bf16_io, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  return bf16_io ? launch_scan_t<bf16>(a, s) : launch_scan_t<float>(a, s);
}

}  // namespace ssd
