// k_f32seq.hip -- the whole chunked SSD forward pass of one (sequence, head)
// in one workgroup, for fp32 inputs, on fp32 MFMA (v_mfma_f32_16x16x4_f32).
//
// Same block decomposition as the bf16 kernels (QbitAI "Mamba-2" article,
// srwj168 repost, sections "Unifying SSM and attention" and "Mamba-2:
// stronger learning, faster training and inference"): inside a chunk of 64
// tokens a masked-attention product, across chunks a linear recurrence on the
// state. The workgroup walks its sequence's chunks in order and keeps the
// running state h (N x P, fp32) in MFMA accumulators, so one launch does the
// whole pass and no per-chunk intermediate leaves the chip. Every product is
// an fp32 MFMA (fp32 operands, fp32 accumulation), so the result carries no
// rounding beyond fp32. Per chunk, with cs the log2-decay prefix of dt*A:
//
//   1. x, B, C, dt of the chunk into LDS (loaded into registers during the
//      previous chunk); cs by a wavefront prefix (the chunk_cumsum step).
//   2. M = (C B^T) o 2^(cs_l - cs_s) dt_s for s <= l, causal 16 x 16 tiles
//      into LDS; the state-owning waves write h_in to LDS.
//   3. outputs y^T = h_in^T C^T 2^(cs_l) + x^T M^T + D x^T (the chunk_scan
//      step); meanwhile h <- 2^(cs_last) h + (w o B)^T x with
//      w_s = 2^(cs_last - cs_s) dt_s, one MFMA accumulation whose accumulator
//      input is the decayed state (the chunk_state and state_passing steps).
//
// fp32 problems are small here (one launch instead of one per step matters
// more than bandwidth): chunk 64, P and N in {16, 32, 64}.
#include "ssd_internal.h"

namespace ssd {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kQ32 = 64;        // tokens per chunk
constexpr int kF32Threads = 256;
constexpr float kLog2eF32 = 1.4426950408889634f;

__device__ __forceinline__ f32x4v mfma4(float a, float b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operand layout of v_mfma_f32_16x16x4_f32, lane l: A[row l % 16][k l / 16],
// B[k l / 16][col l % 16]; result D[row 4 (l / 16) + i][col l % 16], i < 4.

template <int P, int N>
__global__ __launch_bounds__(kF32Threads) void k_ssd_f32seq(Args a) {
  constexpr int Q = kQ32, LT = Q / 16;
  constexpr int XS = P + 1, BS = N + 1, MS = Q + 1, HS = P + 1;  // padded row strides
  constexpr int NST = (N / 16) * (P / 16);  // 16 x 16 state tiles
  constexpr int SPW = (NST + 3) / 4;        // state tiles per wave (at most)
  constexpr int NYT = (P / 16) * LT;        // 16 x 16 output tiles (p, l)
  constexpr int XV = Q * P / 4 / kF32Threads, BV = Q * N / 4 / kF32Threads;
  static_assert(XV >= 1 && BV >= 1, "f32 kernel: P, N >= 16");
  __shared__ float sX[Q * XS], sB[Q * BS], sC[Q * BS], sM[Q * MS], sH[N * HS];
  __shared__ float sCs[Q], sDt[Q], sW[Q];
  __shared__ float sTot;

  const int s = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
  const int g = h / a.heads_per_group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  int c0, c1;
  chunks_of_seq(a, s, c0, c1);
  const float ah = a.A[h] * kLog2eF32;
  const float dsk = a.D ? a.D[h] : 0.f;
  const size_t PN = (size_t)P * N;
  const size_t ldx = (size_t)a.H * P, ldb = (size_t)a.G * N;

  // Running state tiles of this wave: tile t = wave + 4 j, (nt, pt) = (t / (P/16),
  // t % (P/16)); lane holds h[n = 16 nt + 4 lq + i][p = 16 pt + lr].
  f32x4v hs[SPW];
  const float *h0 = a.h0 ? a.h0 + ((size_t)s * a.H + h) * PN : nullptr;
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int t = wave + 4 * j;
    hs[j] = f32x4v{0.f, 0.f, 0.f, 0.f};
    if (t < NST && h0) {
      const int nt = t / (P / 16), pt = t - nt * (P / 16);
      const float4 v = *reinterpret_cast<const float4 *>(h0 + (size_t)(16 * pt + lr) * N +
                                                         16 * nt + 4 * lq);
      hs[j] = f32x4v{v.x, v.y, v.z, v.w};
    }
  }

  // Loads of one chunk into registers (rows past the chunk end read as zero).
  float4 rx[XV], rb[BV], rc[BV];
  float rdt = 0.f;
  auto load_chunk = [&](int c) {
    Chunk k;
    chunk_of(a, c, k);
    const float *xg = static_cast<const float *>(a.x) + (size_t)k.start * ldx + (size_t)h * P;
    const float *bg = static_cast<const float *>(a.B) + (size_t)k.start * ldb + (size_t)g * N;
    const float *cg = static_cast<const float *>(a.C) + (size_t)k.start * ldb + (size_t)g * N;
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + kF32Threads * v, r = i / (P / 4), q = i - r * (P / 4);
      const float4 val = *reinterpret_cast<const float4 *>(xg + (size_t)min(r, k.len - 1) * ldx + 4 * q);
      rx[v] = r < k.len ? val : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + kF32Threads * v, r = i / (N / 4), q = i - r * (N / 4);
      const size_t off = (size_t)min(r, k.len - 1) * ldb + 4 * q;
      const float4 vb = *reinterpret_cast<const float4 *>(bg + off);
      const float4 vc = *reinterpret_cast<const float4 *>(cg + off);
      rb[v] = r < k.len ? vb : make_float4(0.f, 0.f, 0.f, 0.f);
      rc[v] = r < k.len ? vc : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < Q) {
      const float d = dt_of(a, static_cast<const float *>(a.dt)[(size_t)(k.start + min(tid, k.len - 1)) * a.H + h], h);
      rdt = tid < k.len ? d : 0.f;
    }
  };
  if (c0 < c1) load_chunk(c0);

  for (int c = c0; c < c1; ++c) {
    Chunk k;
    chunk_of(a, c, k);
    __syncthreads();  // the previous chunk is done with LDS
    // ---- 1. the chunk into LDS; cs prefix ------------------------------------
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + kF32Threads * v, r = i / (P / 4), q = i - r * (P / 4);
      float *d = sX + r * XS + 4 * q;
      d[0] = rx[v].x; d[1] = rx[v].y; d[2] = rx[v].z; d[3] = rx[v].w;
    }
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + kF32Threads * v, r = i / (N / 4), q = i - r * (N / 4);
      float *db = sB + r * BS + 4 * q, *dc = sC + r * BS + 4 * q;
      db[0] = rb[v].x; db[1] = rb[v].y; db[2] = rb[v].z; db[3] = rb[v].w;
      dc[0] = rc[v].x; dc[1] = rc[v].y; dc[2] = rc[v].z; dc[3] = rc[v].w;
    }
    if (wave == 0) {
      const float cst = wave_inclusive_sum(rdt * ah);
      sCs[lane] = cst;
      sDt[lane] = rdt;
      if (lane == 63) sTot = cst;
    }
    if (c + 1 < c1) load_chunk(c + 1);  // in flight during this chunk's products
    __syncthreads();
    const float cs_last = sTot;
    if (tid < Q) sW[tid] = exp2_fast(cs_last - sCs[tid]) * sDt[tid];

    // ---- 2. M = (C B^T) o decay o dt, causal tiles; h_in into LDS ----------
    for (int t = wave; t < LT * (LT + 1) / 2; t += 4) {
      int lt = 0;
      while ((lt + 1) * (lt + 2) / 2 <= t) ++lt;
      const int st = t - lt * (lt + 1) / 2;
      f32x4v gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < N / 4; ++kk)
        gacc = mfma4(sC[(16 * lt + lr) * BS + 4 * kk + lq], sB[(16 * st + lr) * BS + 4 * kk + lq], gacc);
      const int sc = 16 * st + lr;
      const float css = sCs[sc], dts = sDt[sc];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int l = 16 * lt + 4 * lq + i;
        sM[l * MS + sc] = sc <= l ? gacc[i] * exp2_fast(sCs[l] - css) * dts : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int t = wave + 4 * j;
      if (t < NST) {
        const int nt = t / (P / 16), pt = t - nt * (P / 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) sH[(16 * nt + 4 * lq + i) * HS + 16 * pt + lr] = hs[j][i];
      }
    }
    __syncthreads();

    // ---- 3. outputs (y^T tiles) and the state update ---------------------------
    float *yg = static_cast<float *>(a.y) + (size_t)k.start * ldx + (size_t)h * P;
    for (int t = wave; t < NYT; t += 4) {
      // odd p tiles walk the l tiles backwards, so that the waves' shares of
      // the causal triangle even out
      const int pt = t / LT, lt = (pt & 1) ? LT - 1 - (t - pt * LT) : t - pt * LT;
      const int l = 16 * lt + lr;
      f32x4v st = {0.f, 0.f, 0.f, 0.f}, in = {0.f, 0.f, 0.f, 0.f};
      // state part: sum_n h_in[n][p] C[l][n]
#pragma unroll
      for (int kk = 0; kk < N / 4; ++kk)
        st = mfma4(sH[(4 * kk + lq) * HS + 16 * pt + lr], sC[l * BS + 4 * kk + lq], st);
      // intra-chunk part: sum_{s <= l} x[s][p] M[l][s], one 16-token s tile
      // at a time: its eight operand reads issued together, then four
      // independent accumulations (no chain of dependent MFMAs)
      f32x4v in4[4] = {in, in, in, in};
      for (int stile = 0; stile <= lt; ++stile) {
        float xa[4], ma[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int sr = 16 * stile + 4 * q + lq;
          xa[q] = sX[sr * XS + 16 * pt + lr];
          ma[q] = sM[l * MS + sr];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) in4[q] = mfma4(xa[q], ma[q], in4[q]);
      }
      in = (in4[0] + in4[1]) + (in4[2] + in4[3]);
      const float el = exp2_fast(sCs[l]);
      float4 o;
      float ov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = 16 * pt + 4 * lq + i;
        ov[i] = el * st[i] + in[i] + dsk * sX[l * XS + p];
      }
      o = make_float4(ov[0], ov[1], ov[2], ov[3]);
      if (l < k.len) *reinterpret_cast<float4 *>(yg + (size_t)l * ldx + 16 * pt + 4 * lq) = o;
    }
    const float dec = exp2_fast(cs_last);
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int t = wave + 4 * j;
      if (t < NST) {
        const int nt = t / (P / 16), pt = t - nt * (P / 16);
        // four independent accumulations over the chunk's 64 tokens, the
        // decayed state entering the first
        f32x4v acc[4] = {dec * hs[j], f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f},
                         f32x4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < Q / 4; ++kk) {
          const int sr = 4 * kk + lq;
          acc[kk % 4] = mfma4(sW[sr] * sB[sr * BS + 16 * nt + lr], sX[sr * XS + 16 * pt + lr],
                              acc[kk % 4]);
        }
        hs[j] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      }
    }
  }
  // final state (or the initial state / zeros for a sequence without tokens)
  if (a.hT) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int t = wave + 4 * j;
      if (t < NST) {
        const int nt = t / (P / 16), pt = t - nt * (P / 16);
        *reinterpret_cast<float4 *>(a.hT + ((size_t)s * a.H + h) * PN + (size_t)(16 * pt + lr) * N +
                                    16 * nt + 4 * lq) = make_float4(hs[j][0], hs[j][1], hs[j][2], hs[j][3]);
      }
    }
  }
}

template <int P>
hipError_t launch_p(const Args &a, unsigned blocks, hipStream_t st) {
  if (a.N == 16) hipLaunchKernelGGL((k_ssd_f32seq<P, 16>), dim3(blocks), dim3(kF32Threads), 0, st, a);
  else if (a.N == 32) hipLaunchKernelGGL((k_ssd_f32seq<P, 32>), dim3(blocks), dim3(kF32Threads), 0, st, a);
  else hipLaunchKernelGGL((k_ssd_f32seq<P, 64>), dim3(blocks), dim3(kF32Threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool f32seq_path_supports(const Args &a) {
  return a.Q == kQ32 && (a.P == 16 || a.P == 32 || a.P == 64) &&
         (a.N == 16 || a.N == 32 || a.N == 64);
}

hipError_t launch_f32seq(const Args &a, hipStream_t st) {
  const int64_t blocks = (int64_t)a.nseq * a.H;
  if (blocks == 0) return hipSuccess;
  if (a.P == 16) return launch_p<16>(a, (unsigned)blocks, st);
  if (a.P == 32) return launch_p<32>(a, (unsigned)blocks, st);
  return launch_p<64>(a, (unsigned)blocks, st);
}

}  // namespace ssd
