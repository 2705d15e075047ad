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
//   1. cs, dt and x of chunk c into LDS (x prefetched during chunk c-1);
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
// tiles. Eight waves: in step 2 wave w owns the 16-row half tiles (w, upper)
// and (T-1-w, lower) (equal work per wave); in step 3 wave w owns state rows
// n in [w*N/8, (w+1)*N/8) (state held as h^T, n x p).
#include "mfma_common.h"

namespace ssd {

constexpr float kLog2eFused = 1.4426950408889634f;

template <int N, int Q>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ssd_fused(
    Args a, const bf16 *cb, const bf16 *zeros, int xcd_remap) {
  constexpr int T = Q / 32, PAIRS = T * (T + 1) / 2, KS = N / 32;
  constexpr int BW = N >= 128 ? 8 : N / 16;     // waves that own state rows
  constexpr int NTW = N >= 128 ? N / 128 : 1;   // 16-row n tiles per such wave
  constexpr int NE = T == 8 ? 9 : 4;            // C B^T tiles a wave holds per chunk
  static_assert(Q == 128 || Q == 256, "fused kernel: chunk 128 or 256");
  static_assert(N <= 128, "fused kernel: N <= 128");
  __shared__ __attribute__((aligned(16))) bf16 sX[2][Q * kP];  // x, [token][p], double buffered
  __shared__ __attribute__((aligned(16))) bf16 sB[Q * N];      // B, [token][n]
  __shared__ __attribute__((aligned(16))) bf16 sH[kP * N];     // h_in, [p][n]
  __shared__ __attribute__((aligned(16))) float sCs[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];
  __shared__ __attribute__((aligned(16))) float sU[Q];
  __shared__ __attribute__((aligned(16))) float sW[Q];
  __shared__ float sTot[4];

  // Block -> (sequence, head). With xcd_remap the blocks a chiplet (XCD)
  // receives under round-robin dispatch cover consecutive (sequence, head)
  // pairs, so one sequence's B, C and C B^T tiles are shared in one L2.
  int bid = blockIdx.x;
  if (xcd_remap) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int s = bid / a.H, h = bid - s * a.H, g = h / a.heads_per_group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const bool owns_state = wave < BW;
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

  // Running state (state-owning waves), h^T tiles: rows
  // n = 16 (wave*NTW + nt) + 4 lg + r, column p = 16 pt + lr.
  f32x4 hs[NTW][4];
  const float *h0 = a.h0 ? a.h0 + ((size_t)s * a.H + h) * PN : nullptr;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int n = 16 * (wave * NTW + nt) + 4 * lg, p = 16 * pt + lr;
      hs[nt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (h0 && owns_state) {
        const float4 v = *reinterpret_cast<const float4 *>(h0 + (size_t)p * N + n);
        hs[nt][pt] = f32x4{v.x, v.y, v.z, v.w};
      }
    }
  if (owns_state) {
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
  }

  // Lane-constant parts of the transposed reads of the state product (K =
  // token, natural order): rows 8lg + (lr>>2) and +4, which differ in swizzle.
  const int trow = 8 * lg + (lr >> 2);
  int boff[NTW][2], xoff[4][2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = trow + 4 * q;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      boff[nt][q] = r * N + tr_lane_off<N>(16 * (wave * NTW + nt), r & 7);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) xoff[pt][q] = r * kP + tr_lane_off<kP>(16 * pt, r & 7);
  }
  // Output half tiles of this wave: (iA, uA) and, with 8 row tiles, (iB, 1).
  const int iA = T == 8 ? wave : wave >> 1, uA = T == 8 ? 0 : wave & 1, iB = T - 1 - wave;

  // Prologue: chunk c0's dt in registers, x and B on their way into LDS.
  Chunk k{0, 0, 1, 0};
  float dtv = 0.f;
  if (c0 < c1) {
    chunk_of(a, c0, k);
    const int t = min(tid, k.len - 1);
    const float d = dt_of(a, (float)dtg[(size_t)(k.start + t) * a.H], h);
    dtv = tid < k.len ? d : 0.f;
    async_tile<N, Q>(sB, bg + (size_t)k.start * ldb, ldb, k.len, zeros);
    async_tile<kP, Q>(sX[0], xg + (size_t)k.start * ldx, ldx, k.len, zeros);
  }

#pragma unroll 1
  for (int c = c0; c < c1; ++c) {
    const int cur = (c - c0) & 1;
    const Chunk kc = k;
    wait_vmem_all();
    __syncthreads();  // x, B, dt of chunk c have landed; sH holds h_in of chunk c

    // ---- 1. decay tables of chunk c (wavefront prefix of dt*A) -------------
    const float incl = wave_inclusive_sum(dtv * ah);  // zero past the chunk end
    if (lane == 63 && wave < 4) sTot[wave] = incl;
    const float my_dt = dtv;
    __syncthreads();
    float pre = 0.f, cs_last = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float t = sTot[w];
      pre += w < wave ? t : 0.f;
      cs_last += t;
    }
    const float cst = incl + pre;
    const float cs_tile_end = __shfl(cst, lane | 31);  // cs at the end of this 32-token tile
    if (tid < Q) {
      sCs[tid] = cst;
      sDt[tid] = my_dt;
      sW[tid] = exp2_fast(cs_last - cst) * my_dt;
      sU[tid] = exp2_fast(cs_tile_end - cst) * my_dt;
    }
    __syncthreads();

    // ---- 2. state: h <- 2^(cs_last) h + (w o B)^T x ----------------------------
    if (owns_state) {
      const float dec = exp2_fast(cs_last);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) hs[nt][pt] *= dec;
#pragma unroll
      for (int ks = 0; ks < Q / 32; ++ks) {
        const float4 wa = *reinterpret_cast<const float4 *>(sW + 32 * ks + 8 * lg);
        const float4 wb = *reinterpret_cast<const float4 *>(sW + 32 * ks + 8 * lg + 4);
        const float ww[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        bf16x8 av[NTW], xv[4];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const bf16x4 lo = ds_tr4(sB, 32 * ks * N + boff[nt][0]);
          const bf16x4 hi = ds_tr4(sB, 32 * ks * N + boff[nt][1]);
          const bf16 raw[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e) av[nt][e] = (bf16)((float)raw[e] * ww[e]);
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const bf16x4 lo = ds_tr4(sX[cur], 32 * ks * kP + xoff[pt][0]);
          const bf16x4 hi = ds_tr4(sX[cur], 32 * ks * kP + xoff[pt][1]);
          xv[pt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) hs[nt][pt] = mfma(av[nt], xv[pt], hs[nt][pt]);
        // Keep each k-step's operand reads next to its MFMAs (bounds register use).
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // every wave done reading sB

    // Register operands of the outputs (C rows, C B^T tiles) go out before
    // the next chunk's prefetch, so no wait of step 3 depends on it.
    const bf16 *Cc = cg + (size_t)kc.start * ldb;
    const bf16 *cbase = cb + ((size_t)c * a.G + g) * PAIRS * 2 * 512 + lane * 8;
    bf16x8 acA[KS], acB[KS], cbt[NE];
    {
      const bf16 *ra = Cc + (size_t)min(32 * iA + 16 * uA + lr, kc.len - 1) * ldb + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acA[ks] = ldg8(ra + 32 * ks);
      if (T == 8) {
        const bf16 *rb = Cc + (size_t)min(32 * iB + 16 + lr, kc.len - 1) * ldb + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acB[ks] = ldg8(rb + 32 * ks);
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        int pair, u;
        if (T == 8) {
          const bool first = e <= iA;  // tiles of (iA, 0) then, reversed, of (iB, 1)
          pair = first ? iA * (iA + 1) / 2 + e : iB * (iB + 1) / 2 + (NE - 1 - e);
          u = first ? 0 : 1;
        } else {
          pair = iA * (iA + 1) / 2 + min(e, iA);
          u = uA;
        }
        cbt[e] = ldg8(cbase + (size_t)(pair * 2 + u) * 512);
      }
    }

    // ---- next chunk's dt, B and x on their way (overlap step 3) ---------------
    if (c + 1 < c1) {
      chunk_of(a, c + 1, k);
      const int t = min(tid, k.len - 1);
      const float d = dt_of(a, (float)dtg[(size_t)(k.start + t) * a.H], h);
      dtv = tid < k.len ? d : 0.f;
      async_tile<N, Q>(sB, bg + (size_t)k.start * ldb, ldb, k.len, zeros);
      async_tile<kP, Q>(sX[cur ^ 1], xg + (size_t)k.start * ldx, ldx, k.len, zeros);
    }

    // ---- 3. outputs of chunk c -----------------------------------------------
    {
      bf16 *yc = yg + (size_t)kc.start * ldx;
      half_tile_out<N, Q, NE>(iA, uA, false, cbt, acA, sX[cur], sH, sCs, sDt, sU, kc.len, yc,
                              ldx, dsk);
      if (T == 8)
        half_tile_out<N, Q, NE>(iB, 1, true, cbt, acB, sX[cur], sH, sCs, sDt, sU, kc.len, yc,
                                ldx, dsk);
    }

    // ---- 4. h (bf16) -> sH for chunk c+1 -------------------------------------
    __syncthreads();  // every wave done reading sH
    if (owns_state) {
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
  }

  if (a.hT && owns_state) {
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
  return mfma_path_supports(a) && (a.Q == 128 || a.Q == 256) && a.N <= 128;
}

template <int N, int Q>
static hipError_t launch_fused_nq(const Args &a, const void *cb, const void *zeros,
                                  hipStream_t st) {
  const int blocks = a.nseq * a.H;
  const int remap = (!a.varlen && blocks % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((k_ssd_fused<N, Q>), dim3(blocks), dim3(512), 0, st, a,
                     static_cast<const bf16 *>(cb), static_cast<const bf16 *>(zeros), remap);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_fused_n(const Args &a, const void *cb, const void *zeros,
                                 hipStream_t st) {
  return a.Q == 128 ? launch_fused_nq<N, 128>(a, cb, zeros, st)
                    : launch_fused_nq<N, 256>(a, cb, zeros, st);
}

hipError_t launch_fused(const Args &a, const void *cb, const void *zeros, hipStream_t st) {
  return a.N == 64 ? launch_fused_n<64>(a, cb, zeros, st) : launch_fused_n<128>(a, cb, zeros, st);
}

}  // namespace ssd
