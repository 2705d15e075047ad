// k_mfma.hip -- bf16 MFMA kernels of the chunked SSD forward pass (gfx950).
//
// The SSD layer multiplies the sequence by a semiseparable matrix; cut into
// chunks of Q tokens, the diagonal blocks are masked-attention products
// (C B^T, masked by the decay matrix, times x) and the off-diagonal blocks
// factor through one state per chunk (QbitAI "Mamba-2" article, srwj168
// repost, sections "Unifying SSM and attention" and "Mamba-2: stronger
// learning, faster training and inference"; C, B, x play query, key, value:
// kuaisou "mamba model explained" snippets). Three kernels here:
//
//   k_chunk_state_mfma (row a3): S_c = (w o X_c)^T B_c, w_s = 2^(cs_last-cs_s) dt_s.
//   k_chunk_cb         (row a5, part 1): C_c B_c^T once per (chunk, group),
//                      lower-triangular 32x32 tiles only, stored in bf16 in the
//                      exact register layout chunk_scan feeds to the MFMA.
//   k_chunk_scan_mfma  (row a5, part 2): y = 2^(cs_l) C h_prev^T
//                      + (CB o decay mask) (dt o X) + D x.
//
// MFMA used: v_mfma_f32_16x16x32_bf16 (D 16x16 fp32 += A 16x32 * B 32x16).
// Lane L holds A row (L % 16), B column (L % 16), K elements
// 8*(L/16) .. 8*(L/16)+7 of both; D column (L % 16), rows 4*(L/16) .. +3.
// Any fixed permutation of the K slots works as long as A and B use the same
// one; chunk_scan uses the permutation that the C B^T accumulators produce.
//
// Shapes: P = 64, N in {64, 128, 256}, Q in {64, 128, 256}.
// LDS tiles are [row][col] bf16 with 16-byte chunks XOR-swizzled by (row & 7)
// so that the 16 rows an MFMA operand read touches fall in distinct banks.
#include "ssd_internal.h"
#include "mfma_common.h"
#include "bwd.h"

namespace ssd {

// ============================================================================
// chunk_state: S_c[p, n] = sum_s w_s x_s[p] B_s[n]
// One workgroup (4 waves) per (chunk, head); wave w owns n in
// [w*N/4, (w+1)*N/4) and all 64 p. Tokens go through LDS 128 at a time.
// ============================================================================
// Three workgroups per CU fit the LDS for N <= 128; the occupancy request keeps
// the register allocation within that (156 VGPRs for N = 128, Q = 256, where
// the compiler otherwise takes 176 and runs two waves per SIMD).
// kDstate: the backward pass's per-chunk dstate G_c = sum_l 2^(cs_l) dy_l C_l^T,
// the same product with x -> dy, B -> C and token weights 2^(cs_l) (the decay
// from the chunk's entering state to token l); the caller points a.x at dy,
// a.B at C and a.states at the output.
template <int N, int Q, bool kDstate = false>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(N == 256 ? 2 : 3))) void k_chunk_state_mfma(Args a) {
  constexpr int QH = Q < 128 ? Q : 128;
  constexpr int NT = N / 64;  // 16-wide n tiles per wave
  __shared__ __attribute__((aligned(16))) bf16 sX[kP * QH];
  __shared__ __attribute__((aligned(16))) bf16 sB[N * QH];
  __shared__ float sW[Q];
  Chunk k;
  const int c = blockIdx.x;
  if (!chunk_of(a, c, k)) return;
  const int h = blockIdx.y, g = h / a.heads_per_group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const bf16 *xsrc = static_cast<const bf16 *>(a.x) + ((size_t)k.start * a.H + h) * kP;
  const bf16 *bsrc = static_cast<const bf16 *>(a.B) + ((size_t)k.start * a.G + g) * N;
  Stager<kP, QH / 2, 256> sx;
  Stager<N, QH / 2, 256> sb;
  sx.load(xsrc, (size_t)a.H * kP, 0, k.len);
  sb.load(bsrc, (size_t)a.G * N, 0, k.len);

  const float *cs = a.cs + ((size_t)c * a.H + h) * Q;
  const float last = cs[k.len - 1];
#pragma unroll
  for (int q = 0; q < (Q + 255) / 256; ++q) {
    const int l = tid + 256 * q;
    if (Q >= 256 || l < Q) {
      const int lc = min(l, k.len - 1);
      const float w = kDstate ? exp2_fast(cs[lc])
                              : exp2_fast(last - cs[lc]) *
                                    dt_of(a, (float)static_cast<const bf16 *>(a.dt)[(size_t)(k.start + lc) * a.H + h], h);
      sW[l] = l < k.len ? w : 0.f;
    }
  }

  f32x4 acc[4][NT];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[pt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s0 = 0; s0 < Q; s0 += QH) {
    __syncthreads();  // previous half consumed; sW visible
    sx.template store<QH>(sX, s0, sW);
    sb.template store<QH>(sB, s0, nullptr);
    if (s0 + QH < Q) {  // next half's loads overlap this half's MFMAs
      sx.load(xsrc, (size_t)a.H * kP, s0 + QH, k.len);
      sb.load(bsrc, (size_t)a.G * N, s0 + QH, k.len);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < QH / 32; ++ks) {
      const int col = 32 * ks + 8 * lg;
      bf16x8 av[4], bv[NT];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        av[pt] = *reinterpret_cast<const bf16x8 *>(sX + swz<QH>(16 * pt + lr, col));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bv[nt] = *reinterpret_cast<const bf16x8 *>(
            sB + swz<QH>(16 * (wave * NT + nt) + lr, col));
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[pt][nt] = mfma(av[pt], bv[nt], acc[pt][nt]);
    }
  }
  float *out = a.states + ((size_t)c * a.H + h) * kP * N;
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(16 * pt + 4 * lg + r) * N + 16 * (wave * NT + nt) + lr] = acc[pt][nt][r];
}

// ============================================================================
// chunk_cb: CB[l, s] = C_l . B_s for the lower-triangular 32x32 tiles (i >= j)
// of each (chunk, group). Computed as CB^T = B C^T so that each lane ends up
// with one row l and eight s values -- the A-operand layout of the product
// with x in chunk_scan. Slot e of lane L holds s = 32 j + 16 (e / 4)
// + 4 (L / 16) + (e % 4). Storage: [chunk][group][tile pair][half u][lane][8]
// bf16, tile pair = i (i + 1) / 2 + j, half u = rows 16u..16u+15 of tile i.
// Two launch shapes, one wave per block:
//   PAIRWISE: one wave per (chunk, group, tile pair), every load issued at
//     once, and on the chain path one wave per (chunk, group, B^T step) --
//     for small problems, where the grid would otherwise not fill the GPU;
//   otherwise: one wave per (chunk, group, {i, T-1-i}), T+1 tile pairs each,
//     C rows loaded once per row tile.
// On the chain path the same kernel writes B^T in the A-operand layout of the
// chunk-state product (tile (nt, ks), lane L: n = 16 nt + L%16, tokens
// 32 ks + 8 (L/16) .. +7, zeros past the chunk end), transposing through LDS.
// ============================================================================
// Product of one tile pair from its operands: bop = B rows 32j + 16t + lr,
// cop = C rows 32i + 16u + lr (both: columns 32ks + 8 (L/16) .. +7).
template <int N>
__device__ __forceinline__ void cb_pair_ops(const bf16x8 (&bop)[2][N / 32],
                                            const bf16x8 (&cop)[2][N / 32], bf16 *dst) {
  constexpr int KS = N / 32;
  const int lane = threadIdx.x & 63;
  f32x4 acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u][t] = mfma(bop[t][ks], cop[u][ks], acc[u][t]);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    bf16x8 v;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * t + r] = (bf16)acc[u][t][r];
    *reinterpret_cast<bf16x8 *>(dst + (size_t)u * 512 + lane * 8) = v;
  }
}


template <int N>
__device__ __forceinline__ void cb_pair(const bf16 *B, size_t ldr, int len, int j,
                                        const bf16x8 (&cop)[2][N / 32], bf16 *dst) {
  constexpr int KS = N / 32;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  bf16x8 bop[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bop[t][ks] = ldg8_row(B, ldr, 32 * j + 16 * t + lr, len, 32 * ks + 8 * lg);
  cb_pair_ops<N>(bop, cop, dst);
}

template <int N>
__device__ __forceinline__ void bt_step(const bf16 *B, size_t ldr, int len, int ks, int nks,
                                        bf16 *btb, bf16 *sBt) {
  const int lane = threadIdx.x & 63;
  RowStager<N, 32, 64> st;
  st.load(B, ldr, 32 * ks, len);
  __syncthreads();  // a previous step's transposed reads are done
  st.store(sBt);
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt)
    *reinterpret_cast<bf16x8 *>(btb + ((size_t)nt * nks + ks) * 512 + lane * 8) =
        tr_operand<N>(sBt, 0, 16 * nt);
}

template <int N, int Q, bool PAIRWISE>
__global__ __launch_bounds__(64) void k_chunk_cb(Args a, bf16 *cb) {
  constexpr int T = Q / 32, KS = N / 32, PAIRS = T * (T + 1) / 2;
  __shared__ __attribute__((aligned(16))) bf16 sBt[32 * N];
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < 16)
    reinterpret_cast<uint4 *>(a.zeros)[threadIdx.x] = make_uint4(0, 0, 0, 0);
  {
    // Chain path: clear the ticket, error word and published-chunk counters
    // for the kernel that follows on the stream.
    const int nb = gridDim.x * gridDim.y * gridDim.z;
    const int b = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    for (int i = b * 64 + threadIdx.x; i < a.nsync; i += nb * 64) a.sync[i] = 0;
  }
  Chunk k;
  const int c = blockIdx.x;
  if (!chunk_of(a, c, k)) return;
  const int g = blockIdx.y;
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const bf16 *C = static_cast<const bf16 *>(a.C) + ((size_t)k.start * a.G + g) * N;
  const bf16 *B = static_cast<const bf16 *>(a.B) + ((size_t)k.start * a.G + g) * N;
  const size_t ldr = (size_t)a.G * N;
  bf16 *base = cb + ((size_t)c * a.G + g) * PAIRS * 2 * 512;
  bf16 *btb =
      a.bt ? static_cast<bf16 *>(a.bt) + ((size_t)c * a.G + g) * (N / 16) * T * 512 : nullptr;
  if (PAIRWISE) {
    if ((int)blockIdx.z >= PAIRS) {  // chain path: one wave per B^T step
      bt_step<N>(B, ldr, k.len, (int)blockIdx.z - PAIRS, T, btb, sBt);
      return;
    }
    const int pair = blockIdx.z;
    int i = 0;
    while ((i + 1) * (i + 2) / 2 <= pair) ++i;
    const int j = pair - i * (i + 1) / 2;
    bf16x8 cop[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        cop[u][ks] = ldg8_row(C, ldr, 32 * i + 16 * u + lr, k.len, 32 * ks + 8 * lg);
    cb_pair<N>(B, ldr, k.len, j, cop, base + (size_t)pair * 2 * 512);
  } else {
    const int w = blockIdx.z;
#pragma unroll 1
    for (int ti = 0; ti < 2; ++ti) {
      const int i = ti == 0 ? w : T - 1 - w;
      bf16x8 cop[2][KS];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          cop[u][ks] = ldg8_row(C, ldr, 32 * i + 16 * u + lr, k.len, 32 * ks + 8 * lg);
#pragma unroll 1
      for (int j = 0; j <= i; ++j)
        cb_pair<N>(B, ldr, k.len, j, cop, base + (size_t)(i * (i + 1) / 2 + j) * 2 * 512);
    }
    if (btb) {
#pragma unroll 1
      for (int q = 0; q < 2; ++q) bt_step<N>(B, ldr, k.len, 2 * w + q, T, btb, sBt);
    }
  }
}

// Large problems: one 4-wave workgroup per (chunk, group). The chunk's B
// rows are copied into LDS once (row-major, swizzled; rows past the chunk end
// are zero); wave w computes the tile pairs of its row tiles (w and T-1-w at
// chunk 256, w at chunk 128) from C rows in registers and B tiles read from
// LDS, and writes its share of the B^T operand tiles by transposed reads of
// the same copy. B and C are each read once per (chunk, group).
template <int N, int Q>
__global__ __launch_bounds__(256) void k_chunk_cb_staged(Args a, bf16 *cb) {
  constexpr int T = Q / 32, KS = N / 32, PAIRS = T * (T + 1) / 2, NRT = T / 4;
  static_assert(T == 4 || T == 8, "staged C B^T: chunk 128 or 256");
  __shared__ __attribute__((aligned(16))) bf16 sB[Q * N];
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 16)
    reinterpret_cast<uint4 *>(a.zeros)[threadIdx.x] = make_uint4(0, 0, 0, 0);
  {
    // Chain path: clear the ticket, error word and published-chunk counters
    // for the kernel that follows on the stream.
    const int nb = gridDim.x * gridDim.y;
    const int b = blockIdx.x + gridDim.x * blockIdx.y;
    for (int i = b * 256 + threadIdx.x; i < a.nsync; i += nb * 256) a.sync[i] = 0;
  }
  Chunk k;
  const int c = blockIdx.x;
  if (!chunk_of(a, c, k)) return;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bf16 *C = static_cast<const bf16 *>(a.C) + ((size_t)k.start * a.G + g) * N;
  const bf16 *B = static_cast<const bf16 *>(a.B) + ((size_t)k.start * a.G + g) * N;
  const size_t ldr = (size_t)a.G * N;
  bf16 *base = cb + ((size_t)c * a.G + g) * PAIRS * 2 * 512;
  {
    RowStager<N, Q, 256> st;
    st.load(B, ldr, 0, k.len);
    st.store(sB);
  }
  __syncthreads();
#pragma unroll 1
  for (int ti = 0; ti < NRT; ++ti) {
    const int i = ti == 0 ? wave : T - 1 - wave;
    bf16x8 cop[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        cop[u][ks] = ldg8_row(C, ldr, 32 * i + 16 * u + lr, k.len, 32 * ks + 8 * lg);
#pragma unroll 1
    for (int j = 0; j <= i; ++j) {
      bf16x8 bop[2][KS];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          bop[t][ks] = *reinterpret_cast<const bf16x8 *>(
              sB + rswz<N>(32 * j + 16 * t + lr, 32 * ks + 8 * lg));
      cb_pair_ops<N>(bop, cop, base + (size_t)(i * (i + 1) / 2 + j) * 2 * 512);
    }
  }
  if (a.bt) {
    // B^T operand tiles (nt, ks): this wave's n tiles, every 32-token step.
    bf16 *btb = static_cast<bf16 *>(a.bt) + ((size_t)c * a.G + g) * (N / 16) * T * 512;
    constexpr int NTW = N / 64;
#pragma unroll 1
    for (int q = 0; q < NTW; ++q) {
      const int nt = wave * NTW + q;
#pragma unroll
      for (int ks = 0; ks < T; ++ks)
        *reinterpret_cast<bf16x8 *>(btb + ((size_t)nt * T + ks) * 512 + lane * 8) =
            tr_operand<N>(sB, 32 * ks, 16 * nt);
    }
  }
}

// ============================================================================
// chunk_scan: y_l = 2^(cs_l) C_l h_prev^T + sum_{s<=l} CB[l,s] 2^(cs_l - cs_s)
//             dt_s x_s + D x_l.
// One workgroup per (chunk, head) with Q/64 waves; wave w owns the 32-row
// tiles w and T-1-w (equal work per wave). x^T and h_prev (bf16) sit in LDS;
// C rows and the precomputed CB tiles are read straight into registers, the
// CB tile of the next step always in flight while the current one is used.
// The mask M[l,s] = CB[l,s] 2^(cs_l - cs_s) dt_s is built in registers: for
// off-diagonal tiles (j < i) the decay is split at the tile's first row r0,
// 2^(cs_l - cs_r0) 2^(cs_r0 - cs_s), both factors <= 1, so nothing can
// overflow; diagonal tiles take the exact masked exponent.
// ============================================================================
template <int N, int Q>
__global__ __launch_bounds__(Q) void k_chunk_scan_mfma(Args a, const bf16 *cb) {
  constexpr int T = Q / 32, NTHR = Q, PAIRS = T * (T + 1) / 2;
  constexpr int HITEMS = kP * N / 8, HPER = HITEMS / NTHR;
  static_assert(HITEMS % NTHR == 0, "state staging must divide evenly");
  __shared__ __attribute__((aligned(16))) bf16 sX[Q * kP];
  __shared__ __attribute__((aligned(16))) bf16 sH[kP * N];
  __shared__ __attribute__((aligned(16))) float sCs[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];
  __shared__ __attribute__((aligned(16))) float sU[Q];
  Chunk k;
  const int c = blockIdx.x;
  if (!chunk_of(a, c, k)) return;
  const int h = blockIdx.y, g = h / a.heads_per_group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Issue every global load of the staging phase first.
  const bf16 *xsrc = static_cast<const bf16 *>(a.x) + ((size_t)k.start * a.H + h) * kP;
  RowStager<kP, Q, NTHR> sx;
  sx.load(xsrc, (size_t)a.H * kP, 0, k.len);
  const float *hp = a.states + ((size_t)c * a.H + h) * kP * N;
  float4 hv[HPER][2];
#pragma unroll
  for (int q = 0; q < HPER; ++q) {
    const int it = tid + q * NTHR;
    const int p = it / (N / 8), n8 = it - p * (N / 8);
    hv[q][0] = *reinterpret_cast<const float4 *>(hp + p * N + 8 * n8);
    hv[q][1] = *reinterpret_cast<const float4 *>(hp + p * N + 8 * n8 + 4);
  }
  const float *cs = a.cs + ((size_t)c * a.H + h) * Q;
  const int lc = min(tid, k.len - 1);  // one token per thread (NTHR == Q)
  const float cst = cs[lc];
  const float cse = cs[min(tid | 31, k.len - 1)];
  const float d = dt_of(a, (float)static_cast<const bf16 *>(a.dt)[(size_t)(k.start + lc) * a.H + h], h);
  const float dtv = tid < k.len ? d : 0.f;
  sCs[tid] = cst;
  sDt[tid] = dtv;
  sU[tid] = exp2_fast(cse - cst) * dtv;
  sx.store(sX);
#pragma unroll
  for (int q = 0; q < HPER; ++q) {
    const int it = tid + q * NTHR;
    const int p = it / (N / 8), n8 = it - p * (N / 8);
    uint4 v;
    v.x = pack2(hv[q][0].x, hv[q][0].y);
    v.y = pack2(hv[q][0].z, hv[q][0].w);
    v.z = pack2(hv[q][1].x, hv[q][1].y);
    v.w = pack2(hv[q][1].z, hv[q][1].w);
    *reinterpret_cast<uint4 *>(sH + swz<N>(p, 8 * n8)) = v;
  }
  __syncthreads();

  const bf16 *C = static_cast<const bf16 *>(a.C) + ((size_t)k.start * a.G + g) * N;
  const size_t ldc = (size_t)a.G * N;
  const bf16 *cbase = cb + ((size_t)c * a.G + g) * PAIRS * 2 * 512 + lane * 8;
  const float dsk = a.D ? a.D[h] : 0.f;
  bf16 *yg = static_cast<bf16 *>(a.y);
#pragma unroll 1
  for (int ti = 0; ti < 2; ++ti)
    chunk_rows_out<N, Q>(ti == 0 ? wave : T - 1 - wave, sX, sH, sCs, sDt, sU, C, ldc, cbase,
                         k.len, yg + ((size_t)k.start * a.H + h) * kP, (size_t)a.H * kP, dsk);
}

// ---- launchers ----------------------------------------------------------------
bool mfma_path_supports(const Args &a) {
  return a.P == kP && (a.N == 64 || a.N == 128 || a.N == 256) &&
         (a.Q == 64 || a.Q == 128 || a.Q == 256);
}

size_t cb_bytes(const Args &a) {
  const int T = a.Q / 32;
  return (size_t)a.nc_max * a.G * (T * (T + 1) / 2) * 2 * 1024;
}

template <int N, int Q>
static hipError_t launch_nq(const Args &a, bf16 *cb, hipStream_t st, int which) {
  if (which == 0) {
    hipLaunchKernelGGL((k_chunk_state_mfma<N, Q>), dim3(a.nc_max, a.H), dim3(256), 0, st, a);
  } else if (which == 3) {
    hipLaunchKernelGGL((k_chunk_state_mfma<N, Q, true>), dim3(a.nc_max, a.H), dim3(256), 0, st,
                       a);
  } else if (which == 1) {
    // Small problems: one wave per tile pair, and on the chain path one more
    // per B^T step, so the grid fills the GPU and no wave does both.
    constexpr int T = Q / 32;
    if ((int64_t)a.nc_max * a.G <= 256)
      hipLaunchKernelGGL((k_chunk_cb<N, Q, true>),
                         dim3(a.nc_max, a.G, T * (T + 1) / 2 + (a.bt ? T : 0)), dim3(64), 0,
                         st, a, cb);
    else if (Q >= 128)
      hipLaunchKernelGGL((k_chunk_cb_staged<N, (Q >= 128 ? Q : 128)>), dim3(a.nc_max, a.G),
                         dim3(256), 0, st, a, cb);
    else
      hipLaunchKernelGGL((k_chunk_cb<N, Q, false>), dim3(a.nc_max, a.G, Q / 64), dim3(64), 0, st,
                         a, cb);
  } else {
    hipLaunchKernelGGL((k_chunk_scan_mfma<N, Q>), dim3(a.nc_max, a.H), dim3(Q), 0, st, a,
                       (const bf16 *)cb);
  }
  return hipGetLastError();
}

template <int N>
static hipError_t launch_n(const Args &a, bf16 *cb, hipStream_t st, int which) {
  switch (a.Q) {
    case 64: return launch_nq<N, 64>(a, cb, st, which);
    case 128: return launch_nq<N, 128>(a, cb, st, which);
    default: return launch_nq<N, 256>(a, cb, st, which);
  }
}

static hipError_t launch_mfma(const Args &a, void *cb, hipStream_t st, int which) {
  bf16 *p = static_cast<bf16 *>(cb);
  switch (a.N) {
    case 64: return launch_n<64>(a, p, st, which);
    case 128: return launch_n<128>(a, p, st, which);
    default: return launch_n<256>(a, p, st, which);
  }
}

hipError_t launch_chunk_state_mfma(const Args &a, hipStream_t st) {
  return launch_mfma(a, nullptr, st, 0);
}
hipError_t launch_chunk_dstate_mfma(const Args &a, hipStream_t st) {
  return launch_mfma(a, nullptr, st, 3);
}
hipError_t launch_chunk_cb(const Args &a, void *cb, hipStream_t st) {
  return launch_mfma(a, cb, st, 1);
}
hipError_t launch_chunk_scan_mfma(const Args &a, const void *cb, hipStream_t st) {
  return launch_mfma(a, const_cast<void *>(cb), st, 2);
}

}  // namespace ssd
