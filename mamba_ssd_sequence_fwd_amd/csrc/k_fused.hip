// k_fused.hip -- the whole chunked SSD forward pass of one (sequence, head)
// in one workgroup (bf16 inputs, MFMA, fp32 state).
//
// The SSD layer evaluates the semiseparable matrix by blocks: inside a chunk
// a masked-attention product, across chunks a linear recurrence on one state
// per chunk (QbitAI "Mamba-2" article, srwj168 repost, sections "Unifying SSM
// and attention" and "Mamba-2: stronger learning, faster training and
// inference"). Here the recurrence is carried by the workgroup itself: it
// walks the chunks of its sequence in order and keeps the running state
// h (P x N, fp32) in MFMA accumulators, so no per-chunk state ever goes to
// HBM. Per chunk c, with cs the log2-decay prefix of dt*A inside the chunk:
//
//   1. cs, dt and x^T of chunk c into LDS (x prefetched during chunk c-1);
//      cs by a wavefront prefix (the chunk_cumsum step).
//   2. outputs: y = 2^(cs_l) C h_in^T + (C B^T o decay mask) (dt o x) + D x,
//      with C B^T tiles precomputed once per (chunk, group) (chunk_scan step).
//   3. state: h <- 2^(cs_last) h + ((w o B)^T x), w_s = 2^(cs_last - cs_s) dt_s
//      (the chunk_state and state_passing steps, fused into one MFMA
//      accumulation whose accumulator input is the decayed state).
//   4. h (bf16) into LDS as the next chunk's h_in; after the last chunk,
//      h (fp32) is the sequence's final state.
//
// HBM traffic is x and y once, B/C/dt once per head through L2, and the
// initial/final states: the fused minimum of the method, up to the C B^T
// tiles. Four waves: in step 2 wave w owns row tiles {w, T-1-w}; in step 3
// wave w owns state rows n in [w*N/4, (w+1)*N/4) (state held as h^T, n x p).
#include "mfma_common.h"

namespace ssd {

constexpr float kLog2eFused = 1.4426950408889634f;

template <int N, int Q>
__global__ __launch_bounds__(256) void k_ssd_fused(Args a, const bf16 *cb, int xcd_remap) {
  constexpr int T = Q / 32, PAIRS = T * (T + 1) / 2;
  constexpr int QB = N <= 128 ? 128 : 64;  // tokens per (w o B)^T slice in LDS
  constexpr int NSL = Q / QB;
  constexpr int NTW = N / 64;  // 16-row n tiles per wave in step 3
  static_assert(Q == 128 || Q == 256, "fused kernel: chunk 128 or 256");
  __shared__ __attribute__((aligned(16))) bf16 sX[kP * Q];
  __shared__ __attribute__((aligned(16))) bf16 sB[N * QB];
  __shared__ __attribute__((aligned(16))) bf16 sH[kP * N];
  __shared__ float sCs[Q];
  __shared__ float sDt[Q];
  __shared__ float sW[Q];
  __shared__ float sTot[4];

  // Block -> (sequence, head). With xcd_remap the blocks a chiplet (XCD)
  // receives under round-robin dispatch cover consecutive (sequence, head)
  // pairs, so one sequence's B, C and C B^T tiles are shared in one L2.
  int bid = blockIdx.x;
  if (xcd_remap) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int s = bid / a.H, h = bid - s * a.H, g = h / a.heads_per_group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  int c0, c1;
  chunks_of_seq(a, s, c0, c1);
  const float ah = a.A[h] * kLog2eFused;
  const float dsk = a.D ? a.D[h] : 0.f;
  const size_t PN = (size_t)kP * N;
  const size_t ldx = (size_t)a.H * kP, ldb = (size_t)a.G * N;
  const bf16 *xg = static_cast<const bf16 *>(a.x) + (size_t)h * kP;
  const bf16 *dtg = static_cast<const bf16 *>(a.dt) + h;
  const bf16 *bg = static_cast<const bf16 *>(a.B) + (size_t)g * N;
  const bf16 *cg = static_cast<const bf16 *>(a.C) + (size_t)g * N;
  bf16 *yg = static_cast<bf16 *>(a.y) + (size_t)h * kP;

  // Running state, h^T tiles: rows n = 16 (wave*NTW + nt) + 4 lg + r, column
  // p = 16 pt + lr.
  f32x4 hs[NTW][4];
  const float *h0 = a.h0 ? a.h0 + ((size_t)s * a.H + h) * PN : nullptr;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int n = 16 * (wave * NTW + nt) + 4 * lg, p = 16 * pt + lr;
      if (h0) {
        const float4 v = *reinterpret_cast<const float4 *>(h0 + (size_t)p * N + n);
        hs[nt][pt] = f32x4{v.x, v.y, v.z, v.w};
      } else {
        hs[nt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

  // Prologue: first chunk's x and dt in flight.
  Stager<kP, Q / 2, 256> sx;
  Stager<N, QB / 2, 256> sb;
  Chunk k{0, 0, 1, 0};
  float dtv = 0.f;
  if (c0 < c1) {
    chunk_of(a, c0, k);
    sx.load(xg + (size_t)k.start * ldx, ldx, 0, k.len);
    const int t = min(tid, k.len - 1);
    const float d = (float)dtg[(size_t)(k.start + t) * a.H];
    dtv = tid < k.len ? d : 0.f;
  }

  // h_in of the first chunk, bf16, into sH[p][n].
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int n = 16 * (wave * NTW + nt) + 4 * lg, p = 16 * pt + lr;
      uint2 v;
      v.x = pack2(hs[nt][pt][0], hs[nt][pt][1]);
      v.y = pack2(hs[nt][pt][2], hs[nt][pt][3]);
      *reinterpret_cast<uint2 *>(sH + swz<N>(p, n)) = v;
    }

#pragma unroll 1
  for (int c = c0; c < c1; ++c) {
    const Chunk kc = k;
    __syncthreads();  // previous chunk done with sX, sB, sCs, sW; sH written

    // ---- 1. x^T, dt, cs of chunk c ---------------------------------------
    sx.template store<Q>(sX, 0, nullptr);
    const float v = dtv * ah;  // zero past the chunk end
    const float incl = wave_inclusive_sum(v);
    if (lane == 63) sTot[wave] = incl;
    const float my_dt = dtv;
    // Prefetch chunk c+1 (x and dt) and the first B slice of chunk c.
    if (c + 1 < c1) {
      chunk_of(a, c + 1, k);
      sx.load(xg + (size_t)k.start * ldx, ldx, 0, k.len);
      const int t = min(tid, k.len - 1);
      const float d = (float)dtg[(size_t)(k.start + t) * a.H];
      dtv = tid < k.len ? d : 0.f;
    }
    const bf16 *bsrc = bg + (size_t)kc.start * ldb;
    sb.load(bsrc, ldb, 0, kc.len);
    __syncthreads();
    float pre = 0.f, cs_last = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float t = sTot[w];
      pre += w < wave ? t : 0.f;
      cs_last += t;
    }
    const float cst = incl + pre;
    if (tid < Q) {
      sCs[tid] = cst;
      sDt[tid] = my_dt;
      sW[tid] = exp2_fast(cs_last - cst) * my_dt;
    }
    __syncthreads();

    // ---- 2. outputs of chunk c ---------------------------------------------
    {
      const bf16 *Cc = cg + (size_t)kc.start * ldb;
      const bf16 *cbase = cb + ((size_t)c * a.G + g) * PAIRS * 2 * 512 + lane * 8;
      bf16 *yc = yg + (size_t)kc.start * ldx;
#pragma unroll 1
      for (int ti = 0; ti < (T >= 8 ? 2 : 1); ++ti)
        chunk_rows_out<N, Q>(ti == 0 ? wave : T - 1 - wave, sX, sH, sCs, sDt, Cc, ldb, cbase,
                             kc.len, yc, ldx, dsk);
    }

    // ---- 3. state: h <- 2^(cs_last) h + (w o B)^T x --------------------------
    const float dec = exp2_fast(cs_last);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) hs[nt][pt] *= dec;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      if (sl > 0) {
        __syncthreads();  // previous slice consumed
        sb.load(bsrc, ldb, sl * QB, kc.len);
      }
      sb.template store<QB>(sB, sl * QB, sW);
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < QB / 32; ++ks) {
        bf16x8 av[NTW], xv[4];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          av[nt] = *reinterpret_cast<const bf16x8 *>(
              sB + swz<QB>(16 * (wave * NTW + nt) + lr, 32 * ks + 8 * lg));
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          xv[pt] = *reinterpret_cast<const bf16x8 *>(
              sX + swz<Q>(16 * pt + lr, sl * QB + 32 * ks + 8 * lg));
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) hs[nt][pt] = mfma(av[nt], xv[pt], hs[nt][pt]);
      }
    }

    // ---- 4. h (bf16) -> sH for chunk c+1 -------------------------------------
    __syncthreads();  // every wave done reading sH (step 2) and sB (step 3)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int n = 16 * (wave * NTW + nt) + 4 * lg, p = 16 * pt + lr;
        uint2 u;
        u.x = pack2(hs[nt][pt][0], hs[nt][pt][1]);
        u.y = pack2(hs[nt][pt][2], hs[nt][pt][3]);
        *reinterpret_cast<uint2 *>(sH + swz<N>(p, n)) = u;
      }
  }

  if (a.hT) {
    float *out = a.hT + ((size_t)s * a.H + h) * PN;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int n = 16 * (wave * NTW + nt) + 4 * lg, p = 16 * pt + lr;
        *reinterpret_cast<float4 *>(out + (size_t)p * N + n) =
            make_float4(hs[nt][pt][0], hs[nt][pt][1], hs[nt][pt][2], hs[nt][pt][3]);
      }
  }
}

bool fused_path_supports(const Args &a) {
  return mfma_path_supports(a) && (a.Q == 128 || a.Q == 256);
}

template <int N, int Q>
static hipError_t launch_fused_nq(const Args &a, const void *cb, hipStream_t st) {
  const int blocks = a.nseq * a.H;
  const int remap = (!a.varlen && blocks % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((k_ssd_fused<N, Q>), dim3(blocks), dim3(256), 0, st, a,
                     static_cast<const bf16 *>(cb), remap);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_fused_n(const Args &a, const void *cb, hipStream_t st) {
  return a.Q == 128 ? launch_fused_nq<N, 128>(a, cb, st) : launch_fused_nq<N, 256>(a, cb, st);
}

hipError_t launch_fused(const Args &a, const void *cb, hipStream_t st) {
  switch (a.N) {
    case 64: return launch_fused_n<64>(a, cb, st);
    case 128: return launch_fused_n<128>(a, cb, st);
    default: return launch_fused_n<256>(a, cb, st);
  }
}

}  // namespace ssd
