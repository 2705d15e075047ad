// k_bwd.hip -- the backward pass of the SSD layer: gradients of a loss with
// respect to x, dt, A, B, C, D and the initial state, given dL/dy and
// dL/d(final state).
//
// Training recomputes the states in the backward pass instead of storing them
// (tj-hxxt.cn long read of the Mamba-1 paper, part III (三), the efficient
// implementation). Here the forward's per-step kernels recompute the log2
// decay prefix cs of every chunk, the state h_in entering every chunk and the
// final states; then, per chunk c of a sequence and head h (decays 2^cs, P x N
// states, g_c = dL/d(state leaving chunk c)):
//
//   G_c    = sum_l 2^(cs_l) dy_l C_l^T                     (chunk dstate, MFMA)
//   g_c    = dL/dh_in(c + 1);  dh_in(c) = 2^(cs_last) g_c + G_c
//            (a reverse recurrence over chunks, from dL/d(final state);
//             dh_in of the first chunk is dL/dh0)
//   dxd_s  = sum_{l >= s} M[l, s] dy_l + 2^(cs_last - cs_s) g_c B_s,
//            M[l, s] = (C_l . B_s) 2^(cs_l - cs_s)
//   dx_s   = D dy_s + dt_s dxd_s
//   dL_t   = dy_t . (y_t - D x_t) - dt_t (x_t . dxd_t) + [t last] <g_c, h_out(c)>
//            (the gradient of the natural-log decay prefix at token t; taken
//             from the pair terms of the chunk, see k_bwd_dx)
//   ddt_t  = x_t . dxd_t + A sum_{u >= t} dL_u
//   dA    += sum_t dL_t sum_{v <= t} dt_v;   dD += sum_t dy_t . x_t
//   dC_l   = sum_h [ sum_{s <= l} Z_h[l, s] B_s + 2^(cs_l) dy_l h_in ]
//   dB_s   = sum_h [ sum_{l >= s} Z_h[l, s] C_l + dt_s 2^(cs_last - cs_s) x_s g_c ]
//            with Z_h[l, s] = 2^(cs_l - cs_s) dt_s (dy_l . x_s), l >= s
//
// All products run on bf16 MFMA with fp32 accumulation; the sums over the
// heads that share B and C run inside one workgroup.
#include "bwd.h"
#include "mfma_common.h"

namespace ssd {

// dB / dC kernel: 16 waves per workgroup at N = 128 (128 VGPRs each, one
// workgroup per CU), 8 at N = 64.
template <int N> constexpr int dbc_threads() { return N == 128 ? 1024 : 512; }

bool bwd_supports(const Args &a) {
  return a.P == kP && (a.N == 64 || a.N == 128) && (a.Q == 128 || a.Q == 256);
}

// ---------------------------------------------------------------------------
// Reverse state passing: serial over the chunks of a sequence, from its last
// to its first, parallel over (sequence, head, 4 state elements). gst[c]
// holds G_c on entry and g_c on exit; dh0 gets dL/d(initial state).
// ---------------------------------------------------------------------------
constexpr int kSpbThreads = 256;

__global__ __launch_bounds__(kSpbThreads) void k_state_passing_bwd(BwdArgs b) {
  const Args &a = b.f;
  const int PN = a.P * a.N;
  const int nb = (PN / 4 + kSpbThreads - 1) / kSpbThreads;
  const int s = blockIdx.x / (a.H * nb);
  const int rem = blockIdx.x - s * (a.H * nb);
  const int h = rem / nb;
  const int e = ((rem - h * nb) * kSpbThreads + threadIdx.x) * 4;
  if (e >= PN) return;
  int c0, c1;
  chunks_of_seq(a, s, c0, c1);
  float4 carry = make_float4(0.f, 0.f, 0.f, 0.f);
  if (b.dhT) carry = *reinterpret_cast<const float4 *>(b.dhT + ((size_t)s * a.H + h) * PN + e);
  float4 nextG = make_float4(0.f, 0.f, 0.f, 0.f);
  float nextD = 1.f;
  auto fetch = [&](int c, float4 &G, float &d) {
    G = *reinterpret_cast<const float4 *>(b.gst + ((size_t)c * a.H + h) * PN + e);
    const int len = a.varlen ? a.plan[a.rec_off + 4 * c + 2] : min(a.Q, a.L - (c - c0) * a.Q);
    d = exp2_fast(a.cs[((size_t)c * a.H + h) * a.Q + len - 1]);
  };
  if (c1 > c0) fetch(c1 - 1, nextG, nextD);
  for (int c = c1 - 1; c >= c0; --c) {
    const float4 G = nextG;
    const float d = nextD;
    if (c - 1 >= c0) fetch(c - 1, nextG, nextD);
    *reinterpret_cast<float4 *>(b.gst + ((size_t)c * a.H + h) * PN + e) = carry;
    carry.x = d * carry.x + G.x;
    carry.y = d * carry.y + G.y;
    carry.z = d * carry.z + G.z;
    carry.w = d * carry.w + G.w;
  }
  if (b.dh0) *reinterpret_cast<float4 *>(b.dh0 + ((size_t)s * a.H + h) * PN + e) = carry;
}

// ---------------------------------------------------------------------------
// Block-wide helpers (256 threads).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Sum over the block; every thread gets the result. red: 4 floats of LDS.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// In-place inclusive prefix sums of v[0..Q) by wave 0 (reverse: suffix sums).
template <int Q, bool kReverse>
__device__ __forceinline__ void wave0_scan(float *v) {
  constexpr int E = Q / 64;
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  float loc[E];
  float run = 0.f;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int i = kReverse ? Q - 1 - (lane * E + k) : lane * E + k;
    run += v[i];
    loc[k] = run;
  }
  float incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const float excl = incl - run;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int i = kReverse ? Q - 1 - (lane * E + k) : lane * E + k;
    v[i] = excl + loc[k];
  }
}

// 4 consecutive bf16 of a row (8 bytes), widened.
__device__ __forceinline__ void ld4(const bf16 *p, float (&v)[4]) {
  const uint2 q = *reinterpret_cast<const uint2 *>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ __forceinline__ void st4(bf16 *p, const float (&v)[4]) {
  *reinterpret_cast<uint2 *>(p) = make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
}

// ---------------------------------------------------------------------------
// C B^T of every causal 32 x 32 tile pair of a (chunk, group), once for all
// the heads of the group, stored transposed for the dx kernel: for tile pair
// (i, j), i >= j (l in tile i, s in tile j) and half u (s = 32 j + 16 u ..),
// lane L holds s = 32 j + 16 u + L % 16 and eight l = 32 i + 16 (e / 4)
// + 4 (L / 16) + (e % 4), e = 0..7: the column operand of the M^T dy product
// in the token order of the transposed dy reads. One wave per tile pair.
// ---------------------------------------------------------------------------
template <int N, int Q>
__global__ __launch_bounds__(64) void k_bwd_cbt(Args a) {
  constexpr int KS = N / 32;
  constexpr int T = Q / 32;
  Chunk k;
  const int c = blockIdx.x, g = blockIdx.y, pr = blockIdx.z;
  if (!chunk_of(a, c, k)) return;
  int i = 0;
  while ((i + 1) * (i + 2) / 2 <= pr) ++i;
  const int j = pr - i * (i + 1) / 2;
  const int len = k.len;
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const size_t ldb = (size_t)a.G * N;
  const bf16 *Bs = static_cast<const bf16 *>(a.B) + ((size_t)k.start * a.G + g) * N;
  const bf16 *Cs = static_cast<const bf16 *>(a.C) + ((size_t)k.start * a.G + g) * N;
  bf16x8 cop[2][KS], bop[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      cop[t][ks] = ldg8_row(Cs, ldb, 32 * i + 16 * t + lr, len, 32 * ks + 8 * lg);
      bop[t][ks] = ldg8_row(Bs, ldb, 32 * j + 16 * t + lr, len, 32 * ks + 8 * lg);
    }
  bf16 *dst = static_cast<bf16 *>(a.cb) +
              ((((size_t)c * a.G + g) * (T * (T + 1) / 2) + pr) * 2) * 512;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    f32x4 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc[t] = mfma(cop[t][ks], bop[u][ks], acc[t]);
    }
    bf16x8 v;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * t + r] = (bf16)acc[t][r];
    *reinterpret_cast<bf16x8 *>(dst + (size_t)u * 512 + lane * 8) = v;
  }
}

// ---------------------------------------------------------------------------
// dx, ddt and the per-chunk partials of dA and dD: one workgroup (4 waves) per
// (chunk, head). The transposed output dxd^T (p x s) is built per 16-column
// tile of tokens s: the column operand M^T is a precomputed C B^T tile (once
// per group, k_bwd_cbt) masked and decayed in registers, the row operand is
// dy^T read transposed from LDS;
// the state term adds g_c (bf16 in LDS) times B_s scaled by 2^(cs_last - cs_s).
//
// The decay gradient dL_t is a difference of large terms of both signs
// (their sum over a chunk is thousands of times the result at fast decay), so
// every piece of it comes from one set of fp32 values: the pair terms
// W[l, s] = (C_l . B_s) 2^(cs_l - cs_s) dt_s (dy_l . x_s), l >= s, each taken
// once from two MFMA tiles in the same register layout, give
//   dL_t = sum_{s <= t} W[t, s] - sum_{l >= t} W[l, t] + V_t - E_t + [t last] K
// with V_t = 2^(cs_t) dy_t . (h_in C_t) (the entering state's share of y_t),
// E_t = dt_t 2^(cs_last - cs_t) x_t . (g_c B_t) and
// K = 2^(cs_last) <g_c, h_in> + sum_u E_u (= <g_c, h_out>), so the sums that
// cancel do so in the same arithmetic.
// ---------------------------------------------------------------------------
template <int N, int Q>
__global__ __launch_bounds__(256) void k_bwd_dx(BwdArgs b) {
  const Args &a = b.f;
  constexpr int KS = N / 32;   // 32-wide n steps
  constexpr int TS = Q / 16;   // 16-token column tiles
  __shared__ __attribute__((aligned(16))) bf16 sDY[Q * kP];
  __shared__ __attribute__((aligned(16))) bf16 sG[kP * N];
  __shared__ __attribute__((aligned(16))) bf16 sHin[kP * N];
  __shared__ float sCs[Q], sDt[Q], sCum[Q], sDd[Q], sRow[Q], sCol[Q], sE[Q], sV[Q], sDyx[Q];
  // row sums of W, one partial per wave (each wave adds its column tiles in a
  // fixed order; the four partials are then added in wave order), so that
  // dx, ddt and dA do not depend on the order the waves run in
  __shared__ float sRowW[4][Q];
  __shared__ float sRed[4];
  Chunk k;
  const int c = blockIdx.x;
  if (!chunk_of(a, c, k)) return;
  const int h = blockIdx.y, g = h / a.heads_per_group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lr = lane & 15, lg = lane >> 4;
  const int len = k.len;
  const size_t ldx = (size_t)a.H * kP, ldb = (size_t)a.G * N;
  const bf16 *dy = static_cast<const bf16 *>(b.dy) + ((size_t)k.start * a.H + h) * kP;
  const bf16 *xs = static_cast<const bf16 *>(a.x) + ((size_t)k.start * a.H + h) * kP;
  const bf16 *Bs = static_cast<const bf16 *>(a.B) + ((size_t)k.start * a.G + g) * N;
  const bf16 *Cs = static_cast<const bf16 *>(a.C) + ((size_t)k.start * a.G + g) * N;
  const float *gc = b.gst + ((size_t)c * a.H + h) * kP * N;
  const float *hin = a.states + ((size_t)c * a.H + h) * kP * N;
  const bf16 *cbt = static_cast<const bf16 *>(a.cb) +
                    ((size_t)c * a.G + g) * ((Q / 32) * (Q / 32 + 1) / 2) * 2 * 512;
  const float Dh = a.D ? a.D[h] : 0.f;

  // dy rows into LDS (rows past the chunk end read as zero).
  {
    RowStager<kP, Q, 256> st;
    st.load(dy, ldx, 0, len);
    st.store(sDY);
  }
  // g_c and h_in as bf16 [p][n]; <g_c, h_in> in fp32 on the way.
  float ghin = 0.f;
  constexpr int GI = kP * N / 8 / 256;  // 8-element pieces per thread
  float4 gu[GI][2], hv[GI][2];
#pragma unroll
  for (int q = 0; q < GI; ++q) {       // every load in flight before the first use
    const int i = tid + 256 * q;
    const int p = i / (N / 8), n0 = (i - p * (N / 8)) * 8;
    gu[q][0] = *reinterpret_cast<const float4 *>(gc + (size_t)p * N + n0);
    gu[q][1] = *reinterpret_cast<const float4 *>(gc + (size_t)p * N + n0 + 4);
    hv[q][0] = *reinterpret_cast<const float4 *>(hin + (size_t)p * N + n0);
    hv[q][1] = *reinterpret_cast<const float4 *>(hin + (size_t)p * N + n0 + 4);
  }
#pragma unroll
  for (int q = 0; q < GI; ++q) {
    const int i = tid + 256 * q;
    const int p = i / (N / 8), n0 = (i - p * (N / 8)) * 8;
    const float4 u0 = gu[q][0], u1 = gu[q][1], v0 = hv[q][0], v1 = hv[q][1];
    ghin += u0.x * v0.x + u0.y * v0.y + u0.z * v0.z + u0.w * v0.w + u1.x * v1.x + u1.y * v1.y +
            u1.z * v1.z + u1.w * v1.w;
    *reinterpret_cast<bf16x8 *>(sG + swz<N>(p, n0)) =
        bf16x8{(bf16)u0.x, (bf16)u0.y, (bf16)u0.z, (bf16)u0.w, (bf16)u1.x, (bf16)u1.y,
               (bf16)u1.z, (bf16)u1.w};
    *reinterpret_cast<bf16x8 *>(sHin + swz<N>(p, n0)) =
        bf16x8{(bf16)v0.x, (bf16)v0.y, (bf16)v0.z, (bf16)v0.w, (bf16)v1.x, (bf16)v1.y,
               (bf16)v1.z, (bf16)v1.w};
  }
  const float *cs = a.cs + ((size_t)c * a.H + h) * Q;
  for (int t = tid; t < Q; t += 256) {
    sCs[t] = cs[min(t, len - 1)];
    const float d = t < len ? (float)static_cast<const bf16 *>(a.dt)[(size_t)(k.start + t) * a.H + h]
                            : 0.f;
    sDt[t] = d;
    sCum[t] = d;
#pragma unroll
    for (int w = 0; w < 4; ++w) sRowW[w][t] = 0.f;
    sDyx[t] = 0.f;  // tokens past the chunk end; the column tiles fill the rest
  }
  __syncthreads();
  wave0_scan<Q, false>(sCum);  // prefix sums of dt inside the chunk
  // h_in and g_c transposed ([n][p], bf16) for the dB / dC kernel: a
  // transposed LDS read gives each lane 8 consecutive p of one n.
  {
    bf16 *hT = b.hinT + ((size_t)c * a.H + h) * N * kP;
    bf16 *gT = b.gT + ((size_t)c * a.H + h) * N * kP;
    for (int u = wave; u < (N / 16) * (kP / 32); u += 4) {
      const int n0 = 16 * (u % (N / 16)), p0 = 32 * (u / (N / 16));
      const size_t off = (size_t)(n0 + lr) * kP + p0 + 8 * lg;
      *reinterpret_cast<bf16x8 *>(hT + off) = tr_operand<N>(sHin, p0, n0);
      *reinterpret_cast<bf16x8 *>(gT + off) = tr_operand<N>(sG, p0, n0);
    }
  }

  __syncthreads();

  const float cs_last = sCs[len - 1];
  for (int jt = wave; jt < TS; jt += 4) {
    // Column tiles in the order w, 7 - w, 8 + w, ... balance the triangle.
    const int j = (jt / 4) % 2 == 0 ? jt : (jt / 4) * 4 + 3 - (jt % 4);
    const int s0 = 16 * j;
    if (s0 >= len) continue;
    const int s = s0 + lr;
    const bool sv = s < len;
    bf16x8 bB[KS], bBs[KS], bC[KS], bX[kP / 32];
    const float cs_s = sv ? sCs[s] : 0.f;
    const float dts = sv ? sDt[s] : 0.f;
    const float es = sv ? exp2_fast(cs_last - cs_s) : 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bB[ks] = ldg8_row(Bs, ldb, s, len, 32 * ks + 8 * lg);
      bC[ks] = ldg8_row(Cs, ldb, s, len, 32 * ks + 8 * lg);
#pragma unroll
      for (int e = 0; e < 8; ++e) bBs[ks][e] = (bf16)((float)bB[ks][e] * es);
    }
#pragma unroll
    for (int kp = 0; kp < kP / 32; ++kp) bX[kp] = ldg8_row(xs, ldx, s, len, 32 * kp + 8 * lg);
    // dy_s . x_s (for dD) from the same x row: each lane has 16 of the 64 p,
    // the four lanes of column s together all of them. x is read from HBM
    // only here and in the epilogue just after, while the row is in cache.
    {
      float dyx = 0.f;
#pragma unroll
      for (int kp = 0; kp < kP / 32; ++kp) {
        const bf16x8 d8 = *reinterpret_cast<const bf16x8 *>(sDY + rswz<kP>(s, 32 * kp + 8 * lg));
#pragma unroll
        for (int e = 0; e < 8; ++e) dyx += (float)d8[e] * (float)bX[kp][e];
      }
      dyx += __shfl_xor(dyx, 16);
      dyx += __shfl_xor(dyx, 32);
      if (lg == 0 && sv) sDyx[s] = dyx;
    }
    f32x4 acc1[4], acc2[4], acc3[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
      acc1[pt] = acc2[pt] = acc3[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // state terms: g_c B_s (scaled) and h_in C_s
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int off = swz<N>(16 * pt + lr, 32 * ks + 8 * lg);
        acc2[pt] = mfma(*reinterpret_cast<const bf16x8 *>(sG + off), bBs[ks], acc2[pt]);
        acc3[pt] = mfma(*reinterpret_cast<const bf16x8 *>(sHin + off), bC[ks], acc3[pt]);
      }
    // intra-chunk terms over 32-token blocks l0 >= the block holding s0
    float colp = 0.f;
    const int nl = (len + 31) / 32;
    // C_l . B_s for a block's 32 l (the precomputed transposed tiles), the
    // next block's always in flight
    auto cbt_tile = [&](int ib) {
      return *reinterpret_cast<const bf16x8 *>(
          cbt + ((size_t)(ib * (ib + 1) / 2 + j / 2) * 2 + (j % 2)) * 512 + lane * 8);
    };
    bf16x8 mdn = cbt_tile(s0 / 32);
    for (int ib = s0 / 32; ib < nl; ++ib) {
      const int l0 = 32 * ib;
      const bf16x8 md = mdn;
      mdn = cbt_tile(min(ib + 1, nl - 1));  // unconditional, so it stays in flight
      f32x4 dyx[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        dyx[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < kP / 32; ++kp)
          dyx[t] = mfma(*reinterpret_cast<const bf16x8 *>(sDY + rswz<kP>(l0 + 16 * t + lr, 32 * kp + 8 * lg)),
                        bX[kp], dyx[t]);
      }
      // the decay prefix of this lane's 8 row tokens: two 16-byte LDS reads,
      // no per-element branch (sCs past the chunk end repeats its last value;
      // masked entries are dropped by a select, never multiplied)
      const float4 c0 = *reinterpret_cast<const float4 *>(sCs + l0 + 4 * lg);
      const float4 c1 = *reinterpret_cast<const float4 *>(sCs + l0 + 16 + 4 * lg);
      const float csl[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      bf16x8 bm;
      float wv[8];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * t + r, l = l0 + 16 * t + 4 * lg + r;
          const bool in = sv && l >= s && l < len;
          const float mv = (float)md[e] * exp2_fast(csl[e] - cs_s);
          bm[e] = (bf16)(in ? mv : 0.f);
          wv[e] = in ? mv * dts * dyx[t][r] : 0.f;
          colp += wv[e];
        }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        acc1[pt] = mfma(tr_operand_cb<kP>(sDY, l0, 16 * pt), bm, acc1[pt]);
      // row sums of W over this tile's 16 columns: a transposing butterfly
      // over the 16 lanes of a row group (each step keeps half the values and
      // adds the partner's other half), leaving lanes 2e, 2e + 1 with row e
      {
        float v4[4], v2[2], v1;
        const bool b0 = lr & 1, b1 = (lr >> 1) & 1, b2 = (lr >> 2) & 1;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float keep = b0 ? wv[m + 4] : wv[m], give = b0 ? wv[m] : wv[m + 4];
          v4[m] = keep + __shfl_xor(give, 1);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float keep = b1 ? v4[m + 2] : v4[m], give = b1 ? v4[m] : v4[m + 2];
          v2[m] = keep + __shfl_xor(give, 2);
        }
        {
          const float keep = b2 ? v2[1] : v2[0], give = b2 ? v2[0] : v2[1];
          v1 = keep + __shfl_xor(give, 4);
        }
        v1 += __shfl_xor(v1, 8);
        // lane bits (b0, b1, b2) select value index 4 b0 + 2 b1 + b2
        const int e = 4 * b0 + 2 * b1 + b2;
        const int l = l0 + 16 * (e / 4) + 4 * lg + (e % 4);
        if ((lr >> 3) == 0 && l < len) sRowW[wave][l] += v1;
      }
    }
    colp += __shfl_xor(colp, 16);
    colp += __shfl_xor(colp, 32);
    // epilogue: lane holds dxd[s][16 pt + 4 lg + r] = acc1 + acc2
    float direct = 0.f, ev = 0.f, vv = 0.f;
    bf16 *dxr = static_cast<bf16 *>(b.dx) + ((size_t)(k.start + min(s, len - 1)) * a.H + h) * kP;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int p = 16 * pt + 4 * lg;
      float dv[4], xv[4], o[4];
      ld4(sDY + rswz<kP>(s, p), dv);
      ld4(xs + (size_t)min(s, len - 1) * ldx + p, xv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float dxd = acc1[pt][r] + acc2[pt][r];
        direct += xv[r] * dxd;
        ev += xv[r] * acc2[pt][r];
        vv += dv[r] * acc3[pt][r];
        o[r] = Dh * dv[r] + dts * dxd;
      }
      if (sv) st4(dxr + p, o);
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      direct += __shfl_xor(direct, off);
      ev += __shfl_xor(ev, off);
      vv += __shfl_xor(vv, off);
    }
    if (lg == 0 && sv) {
      sDd[s] = direct;
      sCol[s] = colp;
      sE[s] = dts * ev;
      sV[s] = exp2_fast(cs_s) * vv;
    }
  }
  __syncthreads();

  // K = <g_c, h_out> = 2^(cs_last) <g_c, h_in> + sum_u E_u
  float esum = 0.f;
  for (int t = tid; t < len; t += 256) esum += sE[t];
  const float K = exp2_fast(cs_last) * block_sum(ghin, sRed) + block_sum(esum, sRed);

  // dL_t into sRow, and a copy for the suffix sums (in sCol)
  for (int t = tid; t < Q; t += 256) {
    const float row = ((sRowW[0][t] + sRowW[1][t]) + sRowW[2][t]) + sRowW[3][t];
    const float d = t < len ? row - sCol[t] + sV[t] - sE[t] + (t == len - 1 ? K : 0.f) : 0.f;
    sRow[t] = d;
    sCol[t] = d;
  }
  __syncthreads();
  wave0_scan<Q, true>(sCol);  // suffix sums of dL
  __syncthreads();
  const float Ah = a.A[h];
  float pa = 0.f, pd = 0.f;
  for (int t = tid; t < Q; t += 256) {
    if (t < len) {
      const float v = sDd[t] + Ah * sCol[t];
      if (b.ddt) static_cast<bf16 *>(b.ddt)[(size_t)(k.start + t) * a.H + h] = (bf16)v;
      pa += sRow[t] * sCum[t];
      pd += sDyx[t];
    }
  }
  pa = block_sum(pa, sRed);
  pd = block_sum(pd, sRed);
  if (tid == 0) {
    b.dA_part[(size_t)c * a.H + h] = pa;
    b.dD_part[(size_t)c * a.H + h] = pd;
  }
}

// ---------------------------------------------------------------------------
// dB and dC: one workgroup per (chunk, group, block of kBwdRows tokens
// r0 .. r0 + 31), summing over the heads of the group. Per head it adds,
// into fp32 accumulators:
//   ZR[s][l] = Z_h[l, s] for l in the block and s <= l       (feeds dC rows l)
//   ZC[l][s] = Z_h[l, s] for s in the block and l >= s       (feeds dB rows s)
//   DC[n][l] += sum_p h_in[p][n] 2^(cs_l) dy[l][p]           (dC state term)
//   DB[n][s] += sum_p g_c[p][n] dt_s 2^(cs_last - cs_s) x[s][p]  (dB state term)
// (h_in and g_c read as the transposed bf16 copies the dx kernel wrote)
// each Z tile computed as x . dy^T or dy . x^T over p. Z's 16 x 16 tiles are
// taken in pairs (a 32-token K step of the final products); the 2 + 2 Q/32
// pairs, and the (n tile, half) tiles of DC and DB, are dealt round-robin to
// the waves. The decay factor of an off-diagonal Z element is a column
// factor times a row factor (split at the block's ends, both <= 1); the
// state terms are scaled after each head's product. The head's operands go
// through two LDS buffers (head j + 1 is written while head j is read, one
// barrier per head). After the last head the pairs go to LDS as bf16 column
// operands in the token order of the transposed B / C reads, and DC +=
// B^T-ZR, DB += C^T-ZC finish the sums. Workgroups of one chunk run on one
// XCD so the per-head operands they all read share an L2.
// ---------------------------------------------------------------------------
template <int N, int Q>
__global__ __launch_bounds__(dbc_threads<N>()) void k_bwd_dbc(BwdArgs b) {
  const Args &a = b.f;
  constexpr int kDbcThreads = dbc_threads<N>();
  constexpr int NW = kDbcThreads / 64;  // waves
  constexpr int R = kBwdRows;
  constexpr int NB = Q / R;
  constexpr int NPAIR = 2 + 2 * NB;
  constexpr int PPW = (NPAIR + NW - 1) / NW;
  constexpr int UPW = (N / 16) * 2 / NW;  // (n tile, half) units of DC and DB per wave
  constexpr int XROWS = Q + R;            // x rows [0, r0 + R) then dy rows [r0, Q)
  constexpr int BROWS = 128;              // B / C rows staged at a time in the final phase
  // One LDS area: the per-head operands during the head loop, then the B / C
  // rows and the Z operands (small enough for two workgroups per CU).
  constexpr int kLoop = XROWS * kP + 2 * N * kP, kFinal = BROWS * N + NPAIR * 512;
  __shared__ __attribute__((aligned(16))) bf16 sMem[2 * kLoop > kFinal ? 2 * kLoop : kFinal];
  bf16 *const sBC = sMem, *const sZ = sMem + BROWS * N;
  __shared__ __attribute__((aligned(16))) float sTab[2][3][Q];

  const int nb = gridDim.x, bid = blockIdx.x;
  const int q8 = nb >> 3, r8 = nb & 7, xcd = bid & 7;
  const int lbk = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const int rb = lbk % NB, cg = lbk / NB;
  const int g = cg % a.G, c = cg / a.G;
  Chunk k;
  if (c >= a.nc_max || !chunk_of(a, c, k)) return;
  const int len = k.len, r0 = R * rb;
  if (r0 >= len) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lr = lane & 15, lg = lane >> 4;
  const size_t ldx = (size_t)a.H * kP, ldb = (size_t)a.G * N;
  const int nxr = r0 + R;              // x rows staged

  f32x4 zacc[PPW][2], dcacc[UPW], dbacc[UPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) zacc[i][0] = zacc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < UPW; ++i) dcacc[i] = dbacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-head operands staged through registers: the next head's loads are
  // issued before the current head's products, so their latency overlaps.
  // Every load is unconditional (indices clamped; only the LDS stores are
  // guarded), and nothing converts or selects a loaded value before the
  // store, so the compiler has no reason to wait for them early. Rows past
  // the chunk end hold copies of its last row: every product that reads
  // them is masked (l < len) or scaled by zero.
  // Each load instruction is issued only by the waves that need it (the
  // vector memory pipe, not the bandwidth, bounds the head walk): XF full
  // rounds of 16-byte x / dy pieces, a last partial round of XR pieces by the
  // last XR threads, the bf16 states (one piece per thread), and the decays
  // and steps of the chunk by the Q threads before those (the last waves,
  // whose Z pairs are the fewer).
  constexpr int XU = XROWS * (kP / 8), XF = XU / kDbcThreads, XR = XU % kDbcThreads;
  static_assert(XR % 64 == 0 && XR + Q <= kDbcThreads, "wave-uniform load split");
  static_assert(N * (kP / 8) == kDbcThreads, "one state piece per thread");
  bf16x8 vx[XF + 1], vh, vg;
  float vcs, vref[3];
  bf16 vdt;
  auto fetch = [&](int h) {
    const bf16 *xs = static_cast<const bf16 *>(a.x) + ((size_t)k.start * a.H + h) * kP;
    const bf16 *dys = static_cast<const bf16 *>(b.dy) + ((size_t)k.start * a.H + h) * kP;
    const bf16 *hinT = b.hinT + ((size_t)c * a.H + h) * N * kP;
    const bf16 *gT = b.gT + ((size_t)c * a.H + h) * N * kP;
#pragma unroll
    for (int i = 0; i <= XF; ++i) {
      if (i == XF && tid < kDbcThreads - XR) break;  // wave-uniform
      const int it = i == XF ? tid - (kDbcThreads - XR) + i * kDbcThreads : tid + i * kDbcThreads;
      const int row = it / (kP / 8), col = (it % (kP / 8)) * 8;
      const bf16 *src = row < nxr ? xs + (size_t)min(row, len - 1) * ldx
                                  : dys + (size_t)min(row - R, len - 1) * ldx;
      vx[i] = ldg8(src + col);
    }
    vh = ldg8(hinT + (size_t)(tid / (kP / 8)) * kP + (tid % (kP / 8)) * 8);
    vg = ldg8(gT + (size_t)(tid / (kP / 8)) * kP + (tid % (kP / 8)) * 8);
    const float *cs = a.cs + ((size_t)c * a.H + h) * Q;
    if (tid >= kDbcThreads - XR - Q && tid < kDbcThreads - XR) {  // wave-uniform
      const int t = min(tid - (kDbcThreads - XR - Q), len - 1);
      vcs = cs[t];
      vdt = static_cast<const bf16 *>(a.dt)[(size_t)(k.start + t) * a.H + h];
    }
    vref[0] = cs[r0];                      // the block's first token
    vref[1] = cs[min(r0 + R, len) - 1];    // its last (inside the chunk)
    vref[2] = cs[len - 1];                 // the chunk's last
  };
  // writes the fetched head into LDS buffer `buf`
  auto stage = [&](int buf) {
    bf16 *const sXD = sMem + buf * kLoop, *const sHt = sXD + XROWS * kP, *const sGt = sHt + N * kP;
    float *const sCs = sTab[buf][0], *const sDt = sTab[buf][1], *const sW = sTab[buf][2];
#pragma unroll
    for (int i = 0; i <= XF; ++i) {
      if (i == XF && tid < kDbcThreads - XR) break;
      const int it = i == XF ? tid - (kDbcThreads - XR) + i * kDbcThreads : tid + i * kDbcThreads;
      *reinterpret_cast<bf16x8 *>(sXD + rswz<kP>(it / (kP / 8), (it % (kP / 8)) * 8)) = vx[i];
    }
    *reinterpret_cast<bf16x8 *>(sHt + rswz<kP>(tid / (kP / 8), (tid % (kP / 8)) * 8)) = vh;
    *reinterpret_cast<bf16x8 *>(sGt + rswz<kP>(tid / (kP / 8), (tid % (kP / 8)) * 8)) = vg;
    // Decay factors of the head, split at the block's ends so that no factor
    // exceeds 1: W[t] = dt_t 2^(cs_r0 - cs_t) before the block, 2^(cs_t -
    // cs_e) after it (e its last token), 0 inside it and past the chunk end.
    const float cs_r0 = vref[0], cs_e = vref[1];
    if (tid >= kDbcThreads - XR - Q && tid < kDbcThreads - XR) {
      const int t = tid - (kDbcThreads - XR - Q);
      const float dtv = t < len ? (float)vdt : 0.f;
      sCs[t] = vcs;
      sDt[t] = dtv;
      sW[t] = t < r0 ? dtv * exp2_fast(cs_r0 - vcs)
                     : (t >= r0 + R && t < len ? exp2_fast(vcs - cs_e) : 0.f);
    }
  };
  // Two LDS buffers: head j is read from buffer j % 2 while head j + 1,
  // loaded into registers meanwhile, is written into the other; one barrier
  // per head.
  fetch(g * a.heads_per_group);
  stage(0);
  __syncthreads();
  for (int hj = 0; hj < a.heads_per_group; ++hj) {
    const int buf = hj & 1;
    const bf16 *const sXD = sMem + buf * kLoop, *const sHt = sXD + XROWS * kP, *const sGt = sHt + N * kP;
    const float *const sCs = sTab[buf][0], *const sDt = sTab[buf][1], *const sW = sTab[buf][2];
    const float cs_r0 = vref[0], cs_e = vref[1], cs_last = vref[2];
    // The next head's loads and staging are unconditional (the last head
    // fetches itself again, into the unused buffer): a skipped fetch on the
    // last head would make the compiler assume loads pending at the loop top
    // and wait for this head's first loads there.
    fetch(g * a.heads_per_group + min(hj + 1, a.heads_per_group - 1));

    // Z pairs of this wave
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int q = wave + NW * i;
      if (q >= NPAIR) break;
      const bool zr = q < 2 * (rb + 1);
      const int kb = zr ? q / 2 : rb + (q - 2 * (rb + 1)) / 2;
      const int half = zr ? q % 2 : (q - 2 * (rb + 1)) % 2;
      // the column token of this pair's tiles (l for ZR, s for ZC)
      const int coltok = r0 + 16 * half + lr;
      const float cs_c = sCs[coltok], dt_c = sDt[coltok];
      // the column's share of the off-diagonal factor (zr: 2^(cs_l - cs_r0);
      // zc: dt_s 2^(cs_e - cs_s))
      const float colf = kb == rb ? 0.f : zr ? exp2_fast(cs_c - cs_r0) : dt_c * exp2_fast(cs_e - cs_c);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int t16 = 2 * kb + ti;   // the 16-token tile along K of the final product
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
        // zr: D[s][l], s = 16 t16 + .., l = r0 + 16 half + lr (x . dy^T)
        // zc: D[l][s], l = 16 t16 + .., s = r0 + 16 half + lr (dy . x^T)
        const int arow = zr ? 16 * t16 + lr : R + 16 * t16 + lr;
        const int brow = zr ? R + r0 + 16 * half + lr : r0 + 16 * half + lr;
#pragma unroll
        for (int kp = 0; kp < kP / 32; ++kp) {
          const bf16x8 av = *reinterpret_cast<const bf16x8 *>(sXD + rswz<kP>(arow, 32 * kp + 8 * lg));
          const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(sXD + rswz<kP>(brow, 32 * kp + 8 * lg));
          d = mfma(av, bv, d);
        }
        if (kb != rb) {
          // off the block's diagonal: the factor is the column's times W of the row
          const float4 w4 = *reinterpret_cast<const float4 *>(sW + 16 * t16 + 4 * lg);
          const float wr[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) zacc[i][ti][r] += d[r] * (colf * wr[r]);
        } else {
          // the decay and step of this lane's four row tokens in two 16-byte reads
          const float4 cs4 = *reinterpret_cast<const float4 *>(sCs + 16 * t16 + 4 * lg);
          const float4 dt4 = *reinterpret_cast<const float4 *>(sDt + 16 * t16 + 4 * lg);
          const float csr[4] = {cs4.x, cs4.y, cs4.z, cs4.w}, dtr[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rowtok = 16 * t16 + 4 * lg + r;
            const int s = zr ? rowtok : coltok, l = zr ? coltok : rowtok;
            const bool in = s <= l && l < len;
            // Z[l, s] = 2^(cs_l - cs_s) dt_s (dy_l . x_s)
            const float f = zr ? exp2_fast(cs_c - csr[r]) * dtr[r] : exp2_fast(csr[r] - cs_c) * dt_c;
            zacc[i][ti][r] += in ? d[r] * f : 0.f;
          }
        }
      }
    }
    // state terms of this wave's units (n tile, half): DC[n][l], l = r0 + 16 half + lr,
    // and DB[n][s], s = r0 + 16 half + lr; the column scale is applied to the
    // head's product (one scalar per lane)
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
      const int u = wave + NW * ui, nt = u >> 1, half = u & 1;
      const int tok = r0 + 16 * half + lr;
      const int n = 16 * nt + lr;
      f32x4 tc = f32x4{0.f, 0.f, 0.f, 0.f}, tb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kp = 0; kp < kP / 32; ++kp) {
        const bf16x8 dyv = *reinterpret_cast<const bf16x8 *>(sXD + rswz<kP>(R + tok, 32 * kp + 8 * lg));
        const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(sXD + rswz<kP>(tok, 32 * kp + 8 * lg));
        tc = mfma(*reinterpret_cast<const bf16x8 *>(sHt + rswz<kP>(n, 32 * kp + 8 * lg)), dyv, tc);
        tb = mfma(*reinterpret_cast<const bf16x8 *>(sGt + rswz<kP>(n, 32 * kp + 8 * lg)), xv, tb);
      }
      const float cs_t = sCs[tok];
      const float el = tok < len ? exp2_fast(cs_t) : 0.f, es = sDt[tok] * exp2_fast(cs_last - cs_t);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dcacc[ui][r] += el * tc[r];
        dbacc[ui][r] += es * tb[r];
      }
    }
    stage(buf ^ 1);
    __syncthreads();  // head j + 1 is in LDS, and every wave is done with head j
  }

  // Z pairs to LDS as column operands (the head loop's operands are dead).
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int q = wave + NW * i;
    if (q >= NPAIR) break;
    bf16x8 v;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * ti + r] = (bf16)zacc[i][ti][r];
    *reinterpret_cast<bf16x8 *>(sZ + q * 512 + lane * 8) = v;
  }
  const bf16 *Bs = static_cast<const bf16 *>(a.B) + ((size_t)k.start * a.G + g) * N;
  const bf16 *Cs = static_cast<const bf16 *>(a.C) + ((size_t)k.start * a.G + g) * N;
  // dC rows: B rows [0, r0 + R), BROWS at a time
  for (int b0 = 0; b0 < nxr; b0 += BROWS) {
    __syncthreads();
    const int nr = min(BROWS, nxr - b0);
    for (int it = tid; it < nr * (N / 8); it += kDbcThreads) {
      const int row = it / (N / 8), col = (it % (N / 8)) * 8;
      *reinterpret_cast<bf16x8 *>(sBC + rswz<N>(row, col)) = ldg8_row(Bs, ldb, b0 + row, len, col);
    }
    __syncthreads();
    for (int kb = b0 / 32; kb < (b0 + nr) / 32; ++kb)
#pragma unroll
      for (int ui = 0; ui < UPW; ++ui) {
        const int u = wave + NW * ui, nt = u >> 1, t = u & 1;
        const bf16x8 zv = *reinterpret_cast<const bf16x8 *>(sZ + (2 * kb + t) * 512 + lane * 8);
        dcacc[ui] = mfma(tr_operand_cb<N>(sBC, 32 * kb - b0, 16 * nt), zv, dcacc[ui]);
      }
  }
#pragma unroll
  for (int ui = 0; ui < UPW; ++ui) {
    const int u = wave + NW * ui, nt = u >> 1, t = u & 1;
    const int l = r0 + 16 * t + lr;
    if (l < len) {
      bf16 *dst = static_cast<bf16 *>(b.dC) + ((size_t)(k.start + l) * a.G + g) * N;
      float o[4] = {dcacc[ui][0], dcacc[ui][1], dcacc[ui][2], dcacc[ui][3]};
      st4(dst + 16 * nt + 4 * lg, o);
    }
  }
  // dB rows: C rows [r0, Q), BROWS at a time
  for (int b0 = r0; b0 < Q; b0 += BROWS) {
    __syncthreads();
    const int nr = min(BROWS, Q - b0);
    for (int it = tid; it < nr * (N / 8); it += kDbcThreads) {
      const int row = it / (N / 8), col = (it % (N / 8)) * 8;
      *reinterpret_cast<bf16x8 *>(sBC + rswz<N>(row, col)) = ldg8_row(Cs, ldb, b0 + row, len, col);
    }
    __syncthreads();
    for (int kb = b0 / 32; kb < (b0 + nr) / 32; ++kb)
#pragma unroll
      for (int ui = 0; ui < UPW; ++ui) {
        const int u = wave + NW * ui, nt = u >> 1, half = u & 1;
        const int q = 2 * (rb + 1) + 2 * (kb - rb) + half;
        const bf16x8 zv = *reinterpret_cast<const bf16x8 *>(sZ + q * 512 + lane * 8);
        dbacc[ui] = mfma(tr_operand_cb<N>(sBC, 32 * kb - b0, 16 * nt), zv, dbacc[ui]);
      }
  }
#pragma unroll
  for (int ui = 0; ui < UPW; ++ui) {
    const int u = wave + NW * ui, nt = u >> 1, half = u & 1;
    const int s = r0 + 16 * half + lr;
    if (s < len) {
      bf16 *dst = static_cast<bf16 *>(b.dB) + ((size_t)(k.start + s) * a.G + g) * N;
      float o[4] = {dbacc[ui][0], dbacc[ui][1], dbacc[ui][2], dbacc[ui][3]};
      st4(dst + 16 * nt + 4 * lg, o);
    }
  }
}

// ---------------------------------------------------------------------------
// dA and dD: sums of the per-chunk partials, one workgroup per head, in a
// fixed order (deterministic).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_reduce(BwdArgs b) {
  __shared__ float red[4];
  const Args &a = b.f;
  const int h = blockIdx.x;
  const int nch = a.varlen ? a.plan[0] : a.batch * a.nc_per;
  float sa = 0.f, sd = 0.f;
  for (int c = threadIdx.x; c < nch; c += 256) {
    sa += b.dA_part[(size_t)c * a.H + h];
    sd += b.dD_part[(size_t)c * a.H + h];
  }
  sa = block_sum(sa, red);
  sd = block_sum(sd, red);
  if (threadIdx.x == 0) {
    b.dA[h] = sa;
    if (b.dD) b.dD[h] = sd;
  }
}

hipError_t launch_state_passing_bwd(const BwdArgs &b, hipStream_t st) {
  const int PN = b.f.P * b.f.N;
  const int nb = (PN / 4 + kSpbThreads - 1) / kSpbThreads;
  hipLaunchKernelGGL(k_state_passing_bwd, dim3(nb * b.f.H * b.f.nseq), dim3(kSpbThreads), 0, st,
                     b);
  return hipGetLastError();
}

template <int N, int Q>
static hipError_t launch_cbt_nq(const BwdArgs &b, hipStream_t st) {
  constexpr int T = Q / 32;
  hipLaunchKernelGGL((k_bwd_cbt<N, Q>), dim3(b.f.nc_max, b.f.G, T * (T + 1) / 2), dim3(64), 0,
                     st, b.f);
  return hipGetLastError();
}

hipError_t launch_bwd_cbt(const BwdArgs &b, hipStream_t st) {
  if (b.f.N == 64) return b.f.Q == 128 ? launch_cbt_nq<64, 128>(b, st) : launch_cbt_nq<64, 256>(b, st);
  return b.f.Q == 128 ? launch_cbt_nq<128, 128>(b, st) : launch_cbt_nq<128, 256>(b, st);
}

template <int N, int Q>
static hipError_t launch_dx_nq(const BwdArgs &b, hipStream_t st) {
  hipLaunchKernelGGL((k_bwd_dx<N, Q>), dim3(b.f.nc_max, b.f.H), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdArgs &b, hipStream_t st) {
  if (b.f.N == 64) return b.f.Q == 128 ? launch_dx_nq<64, 128>(b, st) : launch_dx_nq<64, 256>(b, st);
  return b.f.Q == 128 ? launch_dx_nq<128, 128>(b, st) : launch_dx_nq<128, 256>(b, st);
}

template <int N, int Q>
static hipError_t launch_dbc_nq(const BwdArgs &b, hipStream_t st) {
  const int64_t blocks = (int64_t)b.f.nc_max * b.f.G * (Q / kBwdRows);
  hipLaunchKernelGGL((k_bwd_dbc<N, Q>), dim3((unsigned)blocks), dim3(dbc_threads<N>()), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_bwd_dbc(const BwdArgs &b, hipStream_t st) {
  if (b.f.N == 64) return b.f.Q == 128 ? launch_dbc_nq<64, 128>(b, st) : launch_dbc_nq<64, 256>(b, st);
  return b.f.Q == 128 ? launch_dbc_nq<128, 128>(b, st) : launch_dbc_nq<128, 256>(b, st);
}

hipError_t launch_bwd_reduce(const BwdArgs &b, hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_reduce, dim3(b.f.H), dim3(256), 0, st, b);
  return hipGetLastError();
}

}  // namespace ssd
