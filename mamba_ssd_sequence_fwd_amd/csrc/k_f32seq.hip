// k_f32seq.hip -- the whole chunked SSD forward pass of one (sequence, head)
// in one workgroup, for fp32 inputs, on fp32 MFMA (v_mfma_f32_16x16x4_f32).
//
// The block decomposition of the semiseparable matrix (QbitAI "Mamba-2"
// article, srwj168 repost, sections "Unifying SSM and attention" and
// "Mamba-2: stronger learning, faster training and inference"): inside a
// chunk of 64 tokens a masked-attention product, across chunks a linear
// recurrence on the state. One workgroup per (sequence, head) takes its
// chunks CC at a time (CC = as many as its LDS holds, up to 4), one group of
// four waves per chunk, so the chunk-local work of CC chunks runs side by
// side and only the short recurrence between them is serial:
//
//   A. x, B, C, dt of every chunk of the group into LDS; the log2-decay
//      prefix cs of each chunk by a wavefront prefix (the chunk_cumsum step).
//   B. per chunk: M = (C B^T) o 2^(cs_l - cs_s) dt_s for s <= l (causal 16 x 16
//      tiles), and the chunk's own state S = (w o B)^T x from zero, with
//      w_s = 2^(cs_last - cs_s) dt_s (the chunk_state step).
//   C. the recurrence over the group's chunks, element by element of the
//      state: h_in(k) recorded for chunk k, then h <- 2^(cs_last(k)) h + S_k
//      (the state_passing step); h stays in registers across groups.
//   D. per chunk: y^T = 2^(cs_l) h_in^T C^T + x^T M^T + D x^T (the chunk_scan
//      step).
//
// Every product is an fp32 MFMA (fp32 operands and accumulation), so the
// result carries no rounding beyond fp32. Chunk 64, P and N in {16, 32, 64}.
#include "ssd_internal.h"

namespace ssd {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kQ32 = 64;  // tokens per chunk
constexpr float kLog2eF32 = 1.4426950408889634f;

__device__ __forceinline__ f32x4v mfma4(float a, float b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operand layout of v_mfma_f32_16x16x4_f32, lane l: A[row l % 16][k l / 16],
// B[k l / 16][col l % 16]; result D[row 4 (l / 16) + i][col l % 16], i < 4.

// LDS floats per chunk: x [Q][P+1], B and C [Q][N+1], M [Q][Q+1], h_in and
// S [N][P+1] (padded rows), cs, dt, w [Q].
template <int P, int N>
struct F32Lds {
  static constexpr int XS = P + 1, BS = N + 1, MS = kQ32 + 1, HS = P + 1;
  static constexpr int X = 0, B = X + kQ32 * XS, C = B + kQ32 * BS, M = C + kQ32 * BS,
                       H = M + kQ32 * MS, S = H + N * HS, CS = S + N * HS, DT = CS + kQ32,
                       W = DT + kQ32, PER = W + kQ32;
  static constexpr int CC = (150 * 1024) / (PER * 4) >= 4 ? 4 : (150 * 1024) / (PER * 4);
  static_assert(CC >= 1, "f32 kernel: one chunk must fit LDS");
};

template <int P, int N>
__global__ __launch_bounds__((256 * F32Lds<P, N>::CC)) void k_ssd_f32seq(Args a) {
  using L = F32Lds<P, N>;
  constexpr int Q = kQ32, LT = Q / 16, CC = L::CC, NT = 256 * CC;
  constexpr int XS = L::XS, BS = L::BS, MS = L::MS, HS = L::HS;
  constexpr int NST = (N / 16) * (P / 16);  // 16 x 16 state tiles of a chunk
  constexpr int NYT = (P / 16) * LT;        // 16 x 16 output tiles of a chunk
  constexpr int EPT = (P * N + NT - 1) / NT;  // state elements per thread
  __shared__ float smem[CC * L::PER];
  __shared__ float sDec[CC];

  const int s = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
  const int g = h / a.heads_per_group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kc = wave >> 2, wq = wave & 3;  // chunk of the group, wave within it
  const int tq = tid & 255;                 // thread within the chunk's waves
  const int lr = lane & 15, lq = lane >> 4;
  float *R = smem + kc * L::PER;            // this chunk's LDS region
  int c0, c1;
  chunks_of_seq(a, s, c0, c1);
  const float ah = a.A[h] * kLog2eF32;
  const float dsk = a.D ? a.D[h] : 0.f;
  const size_t PN = (size_t)P * N;
  const size_t ldx = (size_t)a.H * P, ldb = (size_t)a.G * N;

  // Running state, element e = p N + n (the memory order of the states).
  float hreg[EPT];
  const float *h0 = a.h0 ? a.h0 + ((size_t)s * a.H + h) * PN : nullptr;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + NT * j;
    hreg[j] = (h0 && e < P * N) ? h0[e] : 0.f;
  }

  for (int cg = c0; cg < c1; cg += CC) {
    const int c = cg + kc;
    const bool active = c < c1;
    Chunk k;
    if (active) chunk_of(a, c, k);
    else k.start = k.len = k.seq = k.idx = 0;
    __syncthreads();  // the previous group is done with LDS
    // ---- A. the chunk into LDS (rows past its end read as zero); cs ----------
    if (active) {
      const float *xg = static_cast<const float *>(a.x) + (size_t)k.start * ldx + (size_t)h * P;
      const float *bg = static_cast<const float *>(a.B) + (size_t)k.start * ldb + (size_t)g * N;
      const float *cgp = static_cast<const float *>(a.C) + (size_t)k.start * ldb + (size_t)g * N;
      constexpr int XV = Q * P / 4 / 256, BV = Q * N / 4 / 256;
      float4 rx[XV], rb[BV], rc[BV];
#pragma unroll
      for (int v = 0; v < XV; ++v) {
        const int i = tq + 256 * v, r = i / (P / 4), q = i - r * (P / 4);
        const float4 val = *reinterpret_cast<const float4 *>(xg + (size_t)min(r, k.len - 1) * ldx + 4 * q);
        rx[v] = r < k.len ? val : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int v = 0; v < BV; ++v) {
        const int i = tq + 256 * v, r = i / (N / 4), q = i - r * (N / 4);
        const size_t off = (size_t)min(r, k.len - 1) * ldb + 4 * q;
        const float4 vb = *reinterpret_cast<const float4 *>(bg + off);
        const float4 vc = *reinterpret_cast<const float4 *>(cgp + off);
        rb[v] = r < k.len ? vb : make_float4(0.f, 0.f, 0.f, 0.f);
        rc[v] = r < k.len ? vc : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float rdt = 0.f;
      if (tq < Q) {
        const float d = dt_of(a, static_cast<const float *>(a.dt)[(size_t)(k.start + min(tq, k.len - 1)) * a.H + h], h);
        rdt = tq < k.len ? d : 0.f;
      }
#pragma unroll
      for (int v = 0; v < XV; ++v) {
        const int i = tq + 256 * v, r = i / (P / 4), q = i - r * (P / 4);
        float *d = R + L::X + r * XS + 4 * q;
        d[0] = rx[v].x; d[1] = rx[v].y; d[2] = rx[v].z; d[3] = rx[v].w;
      }
#pragma unroll
      for (int v = 0; v < BV; ++v) {
        const int i = tq + 256 * v, r = i / (N / 4), q = i - r * (N / 4);
        float *db = R + L::B + r * BS + 4 * q, *dc = R + L::C + r * BS + 4 * q;
        db[0] = rb[v].x; db[1] = rb[v].y; db[2] = rb[v].z; db[3] = rb[v].w;
        dc[0] = rc[v].x; dc[1] = rc[v].y; dc[2] = rc[v].z; dc[3] = rc[v].w;
      }
      if (wq == 0) {
        const float cst = wave_inclusive_sum(rdt * ah);
        const float cs_last = __shfl(cst, 63);
        R[L::CS + lane] = cst;
        R[L::DT + lane] = rdt;
        R[L::W + lane] = exp2_fast(cs_last - cst) * rdt;
        if (lane == 0) sDec[kc] = exp2_fast(cs_last);
      }
    }
    __syncthreads();

    // ---- B. M tiles and the chunk's own state S ---------------------------------
    if (active) {
      for (int t = wq; t < LT * (LT + 1) / 2; t += 4) {
        int lt = 0;
        while ((lt + 1) * (lt + 2) / 2 <= t) ++lt;
        const int st = t - lt * (lt + 1) / 2;
        float ca[N / 4], cb[N / 4];
#pragma unroll
        for (int kk = 0; kk < N / 4; ++kk) {
          ca[kk] = R[L::C + (16 * lt + lr) * BS + 4 * kk + lq];
          cb[kk] = R[L::B + (16 * st + lr) * BS + 4 * kk + lq];
        }
        f32x4v gacc[2] = {f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < N / 4; ++kk) gacc[kk & 1] = mfma4(ca[kk], cb[kk], gacc[kk & 1]);
        const f32x4v gv = gacc[0] + gacc[1];
        const int sc = 16 * st + lr;
        const float css = R[L::CS + sc], dts = R[L::DT + sc];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int l = 16 * lt + 4 * lq + i;
          R[L::M + l * MS + sc] = sc <= l ? gv[i] * exp2_fast(R[L::CS + l] - css) * dts : 0.f;
        }
      }
      for (int t = wq; t < NST; t += 4) {
        const int nt = t / (P / 16), pt = t - nt * (P / 16);
        f32x4v acc[4] = {f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f},
                         f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < Q / 4; ++kk) {
          const int sr = 4 * kk + lq;
          acc[kk % 4] = mfma4(R[L::W + sr] * R[L::B + sr * BS + 16 * nt + lr],
                              R[L::X + sr * XS + 16 * pt + lr], acc[kk % 4]);
        }
        const f32x4v sv = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) R[L::S + (16 * nt + 4 * lq + i) * HS + 16 * pt + lr] = sv[i];
      }
    }
    __syncthreads();

    // ---- C. the recurrence across the group's chunks, per state element --------
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + NT * j;
      if (e < P * N) {
        const int p = e / N, n = e - (e / N) * N;
        float hv = hreg[j];
#pragma unroll
        for (int q = 0; q < CC; ++q) {
          if (cg + q < c1) {
            float *Rq = smem + q * L::PER;
            Rq[L::H + n * HS + p] = hv;
            hv = sDec[q] * hv + Rq[L::S + n * HS + p];
          }
        }
        hreg[j] = hv;
      }
    }
    __syncthreads();

    // ---- D. outputs (y^T tiles) --------------------------------------------------
    if (active) {
      float *yg = static_cast<float *>(a.y) + (size_t)k.start * ldx + (size_t)h * P;
      for (int t = wq; t < NYT; t += 4) {
        // odd p tiles walk the l tiles backwards, so that the waves' shares of
        // the causal triangle even out
        const int pt = t / LT, lt = (pt & 1) ? LT - 1 - (t - pt * LT) : t - pt * LT;
        const int l = 16 * lt + lr;
        // state part: sum_n h_in[n][p] C[l][n]
        float ha[N / 4], cl[N / 4];
#pragma unroll
        for (int kk = 0; kk < N / 4; ++kk) {
          ha[kk] = R[L::H + (4 * kk + lq) * HS + 16 * pt + lr];
          cl[kk] = R[L::C + l * BS + 4 * kk + lq];
        }
        f32x4v st2[2] = {f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < N / 4; ++kk) st2[kk & 1] = mfma4(ha[kk], cl[kk], st2[kk & 1]);
        const f32x4v st = st2[0] + st2[1];
        // intra-chunk part: sum_{s <= l} x[s][p] M[l][s], one 16-token s tile
        // at a time (eight operand reads, then four independent MFMAs)
        f32x4v in4[4] = {f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f},
                         f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f}};
        for (int stile = 0; stile <= lt; ++stile) {
          float xa[4], ma[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int sr = 16 * stile + 4 * q + lq;
            xa[q] = R[L::X + sr * XS + 16 * pt + lr];
            ma[q] = R[L::M + l * MS + sr];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) in4[q] = mfma4(xa[q], ma[q], in4[q]);
        }
        const f32x4v in = (in4[0] + in4[1]) + (in4[2] + in4[3]);
        const float el = exp2_fast(R[L::CS + l]);
        float ov[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = 16 * pt + 4 * lq + i;
          ov[i] = el * st[i] + in[i] + dsk * R[L::X + l * XS + p];
        }
        if (l < k.len)
          *reinterpret_cast<float4 *>(yg + (size_t)l * ldx + 16 * pt + 4 * lq) =
              make_float4(ov[0], ov[1], ov[2], ov[3]);
      }
    }
  }
  // final state (or the initial state / zeros for a sequence without tokens)
  if (a.hT) {
    float *hT = a.hT + ((size_t)s * a.H + h) * PN;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + NT * j;
      if (e < P * N) hT[e] = hreg[j];
    }
  }
}

template <int P>
hipError_t launch_p(const Args &a, unsigned blocks, hipStream_t st) {
  if (a.N == 16)
    hipLaunchKernelGGL((k_ssd_f32seq<P, 16>), dim3(blocks), dim3(256 * F32Lds<P, 16>::CC), 0, st, a);
  else if (a.N == 32)
    hipLaunchKernelGGL((k_ssd_f32seq<P, 32>), dim3(blocks), dim3(256 * F32Lds<P, 32>::CC), 0, st, a);
  else
    hipLaunchKernelGGL((k_ssd_f32seq<P, 64>), dim3(blocks), dim3(256 * F32Lds<P, 64>::CC), 0, st, a);
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
