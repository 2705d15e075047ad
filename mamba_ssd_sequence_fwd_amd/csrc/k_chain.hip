// k_chain.hip -- the chunked SSD forward pass with one workgroup per
// (chunk, head), the inter-chunk recurrence carried by a chain of
// workgroups (bf16 inputs, MFMA, fp32 state).
//
// The SSD layer evaluates the semiseparable matrix by blocks: inside a chunk
// a masked-attention product, across chunks a linear recurrence on one state
// per chunk (QbitAI "Mamba-2" article, srwj168 repost, sections "Unifying SSM
// and attention" and "Mamba-2: stronger learning, faster training and
// inference"). Every (chunk, head) is an independent workgroup; only the
// recurrence h_out = 2^(cs_last) h_in + S_c links the chunks of one
// (sequence, head), and it is handed from the workgroup of chunk j to that
// of chunk j+1 through a two-slot fp32 ring in device memory plus a
// published-chunk counter. Per workgroup (four waves), with cs the log2-decay
// prefix of dt*A inside the chunk:
//
//   1. ticket -> (chunk, head); dt, the chunk's first B^T operand tiles and
//      x into registers (loads complete in issue order, so x is waited for
//      step by step); the decay tables (cs, w, u) by a wavefront prefix; the
//      first half of x into LDS (the second half halfway through step 2).
//   2. S_c = (w o B)^T x (w_s = 2^(cs_last - cs_s) dt_s): the chunk's own
//      state from a zero start (the chunk_state step).
//   3. h_in from the previous chunk's workgroup (loaded while step 2 runs when
//      it is already published), or the initial state / zero at a sequence
//      start; h_out = 2^(cs_last) h_in + S_c goes to the ring (or to the final
//      state after the sequence's last chunk) and is published (the
//      state_passing step).
//   4. outputs, per 32-row tile: (C B^T o decay mask)(dt o x) + D x with the
//      C B^T tiles precomputed once per (chunk, group), plus 2^(cs_l) C_l h_in^T
//      (the chunk_scan step); y.
//
// Tickets from an atomic counter order the work units by chunk index inside
// the sequence, then sequence, then head, so the predecessor of a unit took
// its ticket a whole chunk-index level earlier and has normally published by
// the time step 3 asks. A workgroup only ever waits on a smaller ticket, i.e.
// on one that is already running, so the chain cannot deadlock whatever order
// the hardware dispatches in. Every wait is bounded by a wall-clock limit; a
// wait that runs out sets an error word instead of hanging (the outputs are
// then wrong).
//
// LDS holds only x (the operand both products read transposed) and h_in
// (bf16), 52 KB at chunk 256, so three workgroups share a CU. Each wave owns
// whole 32-row output tiles, so the two 16-row halves of a tile share every
// x and h_in read. x is staged through registers rather than copied
// global->LDS directly: while such a copy is pending, every wait on a
// register load drains all outstanding loads, which would serialise the
// prefetches. Within each 32-token step, the small LDS reads go first and the
// x operand reads right after, so their latency hides behind the scaling
// arithmetic (LDS returns in order).
//
// HBM traffic: x, y once; B, C, dt and the C B^T tiles once per head
// through L2; 32 KB of fp32 state written and read per (chunk, head).
#include "mfma_common.h"

namespace ssd {

constexpr float kLog2eChain = 1.4426950408889634f;
constexpr int kChainWaves = 4;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Intra-chunk outputs of the 32-row tile i (rows 32i .. 32i+31), both 16-row
// halves u, added into Y[u] (transposed: lane holds column l = 32i + 16u +
// lane%16 and rows p = 16pt + 4(lane/16) + r). Off-diagonal 32-token tiles
// j < i use the split decay 2^(cs_l - cs_r0) 2^(cs_r0 - cs_e) 2^(cs_e - cs_s)
// (three factors <= 1, e = last token of tile j, r0 = first row of tile i,
// the last one folded into sU); the diagonal tile takes the exact masked
// exponent and carries D on its diagonal. C B^T tiles stream from L2 two
// ahead; each x operand read serves both halves.
template <int Q>
__device__ __forceinline__ void intra_tile(int i, f32x4 (&Y)[2][4], const bf16 *sX,
                                           const float *sCs, const float *sDt, const float *sU,
                                           const bf16 *cbase, float dsk, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int pair0 = i * (i + 1) / 2;
  const float cs_r0 = sCs[32 * i];
  float cs_l[2], rdec[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    cs_l[u] = sCs[32 * i + 16 * u + lr];
    rdec[u] = exp2_fast(cs_l[u] - cs_r0);
  }
  const int xrow = 4 * lg + (lr >> 2);
  int xoff[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) xoff[pt] = xrow * kP + tr_lane_off<kP>(16 * pt, xrow & 7);

  bf16x8 m0[2], m1[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    m0[u] = ldg8(cbase + (size_t)(pair0 * 2 + u) * 512);
    m1[u] = ldg8(cbase + (size_t)((pair0 + min(1, i)) * 2 + u) * 512);
  }
#pragma unroll 1
  for (int j = 0; j < i; ++j) {
    bf16x8 m[2] = {m0[0], m0[1]};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      m0[u] = m1[u];
      m1[u] = ldg8(cbase + (size_t)((pair0 + min(j + 2, i)) * 2 + u) * 512);
    }
    // LDS reads first (they return in order): the decay inputs, then every
    // x operand of the step, whose latency the scaling below then hides.
    const float cs_e = sCs[32 * j + 31];
    const float4 ua = *reinterpret_cast<const float4 *>(sU + 32 * j + 4 * lg);
    const float4 ub = *reinterpret_cast<const float4 *>(sU + 32 * j + 16 + 4 * lg);
    bf16x8 xv[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x4 lo = ds_tr4(sX, 32 * j * kP + xoff[pt]);
      const bf16x4 hi = ds_tr4(sX, (32 * j + 16) * kP + xoff[pt]);
      xv[pt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    const float e_r0 = exp2_fast(cs_r0 - cs_e);
    const float uu[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float fa = rdec[u] * e_r0;
#pragma unroll
      for (int e = 0; e < 8; ++e) m[u][e] = (bf16)((float)m[u][e] * (fa * uu[e]));
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int u = 0; u < 2; ++u) Y[u][pt] = mfma(xv[pt], m[u], Y[u][pt]);
  }
  // Diagonal tile j = i (m0 holds it: the stream clamps at i).
  {
    const float4 ca = *reinterpret_cast<const float4 *>(sCs + 32 * i + 4 * lg);
    const float4 cb4 = *reinterpret_cast<const float4 *>(sCs + 32 * i + 16 + 4 * lg);
    const float4 da = *reinterpret_cast<const float4 *>(sDt + 32 * i + 4 * lg);
    const float4 db = *reinterpret_cast<const float4 *>(sDt + 32 * i + 16 + 4 * lg);
    const float cc[8] = {ca.x, ca.y, ca.z, ca.w, cb4.x, cb4.y, cb4.z, cb4.w};
    const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
    bf16x8 m[2] = {m0[0], m0[1]};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int lloc = 16 * u + lr;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sloc = 16 * (e >> 2) + 4 * lg + (e & 3);
        const float v = (float)m[u][e] * exp2_fast(cs_l[u] - cc[e]) * dd[e];
        const float w = sloc == lloc ? v + dsk : v;
        m[u][e] = (bf16)(sloc <= lloc ? w : 0.f);
      }
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x4 lo = ds_tr4(sX, 32 * i * kP + xoff[pt]);
      const bf16x4 hi = ds_tr4(sX, (32 * i + 16) * kP + xoff[pt]);
      const bf16x8 xv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int u = 0; u < 2; ++u) Y[u][pt] = mfma(xv, m[u], Y[u][pt]);
    }
  }
}

// C rows of the 32-row tile i, both halves: row 32i + 16u + lane%16 (clamped
// into the chunk), n = 32ks + 8(lane/16) .. +7.
template <int N>
__device__ __forceinline__ void load_c_tile(bf16x8 (&ac)[2][N / 32], const bf16 *cc, size_t ldb,
                                            int i, int len, int lane) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const bf16 *row = cc + (size_t)min(32 * i + 16 * u + (lane & 15), len - 1) * ldb +
                      8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) ac[u][ks] = ldg8(row + 32 * ks);
  }
}

// State part of tile i, computed first: Y[u] = 2^(cs_l) C_l h_in^T (the
// intra-chunk part then accumulates on top). sH = h_in bf16 [p][n] (swizzled
// rows of N); each h_in read serves both halves; C rows past len are zero.
template <int N>
__device__ __forceinline__ void state_tile(int i, f32x4 (&Y)[2][4], const bf16 *sH,
                                           const float *sCs, const bf16x8 (&ac)[2][N / 32],
                                           int len, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  int hbase = 0;
  asm volatile("" : "+v"(hbase));
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[u][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < N / 32; ++ks) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(
          sH + hbase + swz<N>(16 * pt + lr, 32 * ks + 8 * lg));
#pragma unroll
      for (int u = 0; u < 2; ++u) Y[u][pt] = mfma(bh, ac[u][ks], Y[u][pt]);
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float f = exp2_fast(sCs[32 * i + 16 * u + lr]);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[u][pt] *= f;
  }
}

__device__ __forceinline__ void store_tile(int i, const f32x4 (&Y)[2][4], int len, bf16 *y,
                                           size_t ystride, int lane) {
  // Lanes 16 apart (same row l) exchange one p tile's worth of packed values
  // so that each lane holds 8 consecutive p: 16-byte stores, 64 contiguous
  // bytes per row and instruction. v_permlane16_swap swaps the odd 16-lane
  // rows of its first operand with the even rows of its second, so after
  // swapping (p tile 2m, p tile 2m+1) every lane holds its output in order.
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int l = 32 * i + 16 * u + lr;
    uint32_t pk[4][2];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      pk[pt][0] = pack2(Y[u][pt][0], Y[u][pt][1]);
      pk[pt][1] = pack2(Y[u][pt][2], Y[u][pt][3]);
    }
    bf16 *yr = y + (size_t)l * ystride + 8 * (lg >> 1) + 16 * (lg & 1);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const auto sx = __builtin_amdgcn_permlane16_swap(pk[2 * m][0], pk[2 * m + 1][0], false, false);
      const auto sy = __builtin_amdgcn_permlane16_swap(pk[2 * m][1], pk[2 * m + 1][1], false, false);
      const uint4 o = make_uint4(sx[0], sy[0], sx[1], sy[1]);
      // y is written once and read by nothing in this pass: nontemporal
      // stores (measured 5-8% faster on the 2.7B-shaped workload, 2%
      // slower on the long varlen one)
      if (l < len) {
        const u32x4_t ov = {o.x, o.y, o.z, o.w};
        __builtin_nontemporal_store(ov, reinterpret_cast<u32x4_t *>(yr + 32 * m));
      }
    }
  }
}

// The state hand-off between workgroups that may sit on different XCDs
// (each with its own L2). Ring entries are written and read by 16-byte buffer
// accesses with the sc1 cache policy (device scope, the same bits a relaxed
// device-scope atomic access carries), which are coherent across the whole
// GPU without flushing or invalidating any cache: a producer's ring stores
// are complete once its s_waitcnt vmcnt(0) returns, it then bumps the
// counter, and a consumer issues its ring loads only after it has seen the
// counter. The counter alone orders the hand-off, so the entries need no
// atomicity of their own.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCachePolicyDevice = 16;  // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ring_rsrc(const float *slot, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(slot), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void ring_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kCachePolicyDevice);
}
__device__ __forceinline__ f32x4 ring_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyDevice));
}

// Bounded wait until the published-chunk counter reaches `want`. Returns
// false if the wall-clock limit ran out first.
__device__ __forceinline__ bool wait_published(const int32_t *ctr, int want) {
  constexpr uint64_t kLimitTicks = 100000000ull;  // 1 s of the 100 MHz constant clock
  if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) return true;
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
    __builtin_amdgcn_s_sleep(2);
    if (wall_clock64() - t0 > kLimitTicks) return false;
  }
  return true;
}

// Incoming state of head h, chunk k, in the state-tile layout of this wave
// (tile (j, pt): rows n = 16 (nt0 + j) + 4(lane/16) + r, column p = 16 pt +
// lane%16): the ring slot of the previous chunk, or at a sequence start the
// initial state (or zeros). Ring slot layout: [wave][j][pt][lane][r], one
// 16-byte access per lane and 1 KB contiguous per wave access.
template <int N, int NTW>
__device__ __forceinline__ void load_h_in(f32x4 (&hin)[NTW][4], const Args &a, const Chunk &k,
                                          int h, int wave, int nt0, int lane) {
  const size_t PN = (size_t)kP * N;
  const int lr = lane & 15, lg = lane >> 4;
  if (k.idx > 0) {
    const __amdgpu_buffer_rsrc_t rin = ring_rsrc(
        a.ring + ((size_t)(k.seq * a.H + h) * 2 + ((k.idx + 1) & 1)) * PN, (int)(PN * 4));
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        hin[j][pt] = ring_load4(rin, (uint32_t)((((wave * NTW + j) * 4 + pt) * 64 + lane) * 16));
  } else if (a.h0) {
    const float *h0 = a.h0 + (size_t)(k.seq * a.H + h) * PN;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int n = 16 * (nt0 + j) + 4 * lg, p = 16 * pt + lr;
        const float4 v = *reinterpret_cast<const float4 *>(h0 + (size_t)p * N + n);
        hin[j][pt] = f32x4{v.x, v.y, v.z, v.w};
      }
  } else {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) hin[j][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// kDeep: every B^T tile of step 2 is loaded up front instead of four steps
// ahead, at two workgroups per CU instead of three (more registers). When a
// problem has no more work units than the chip holds at once, each
// workgroup's own latency is the whole time and this wins (config-1 shapes:
// 66 -> 56 us); with many units per slot the third workgroup per CU hides
// that latency better (the 2.7B shapes: equal; long packed input: 13%
// slower), so the launcher picks it by grid size.
template <int N, int Q, bool kDeep>
__global__ __launch_bounds__(64 * kChainWaves)
__attribute__((amdgpu_waves_per_eu(N == 256 || kDeep ? 2 : 3, N == 256 || kDeep ? 2 : 3)))
void k_ssd_chain(Args a, const bf16 *cb, const bf16 *bt) {
  constexpr int T = Q / 32, PAIRS = T * (T + 1) / 2, NKS = Q / 32;
  constexpr int NTW = N / 64;                 // 16-row n tiles of the state per wave
  constexpr int NTILE = T == 8 ? 2 : 1;       // 32-row output tiles per wave
  static_assert(Q == 128 || Q == 256, "chain kernel: chunk 128 or 256");
  static_assert(N == 64 || N == 128 || N == 256, "chain kernel: N 64, 128 or 256");
  __shared__ __attribute__((aligned(16))) bf16 sX[Q * kP];  // x, [token][p]
  __shared__ __attribute__((aligned(16))) bf16 sH[kP * N];  // h_in (bf16), [p][n]
  __shared__ __attribute__((aligned(16))) float sCs[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];
  __shared__ __attribute__((aligned(16))) float sU[Q];
  __shared__ __attribute__((aligned(16))) float sW[Q];
  __shared__ float sTot[4];
  __shared__ int sTicket, sReady;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  int32_t *ticket = a.sync, *err = a.sync + 1, *pub = a.sync + kSyncHeader;

  // ---- 1. work unit, loads, decay tables -----------------------------------
  if (tid == 0) sTicket = atomicAdd(ticket, 1);
  __syncthreads();
  const int tk = sTicket;
  int c, h;
  if (!a.varlen) {
    const int per = a.nseq * a.H;
    const int j = tk / per, r = tk - j * per, s = r / a.H;
    h = r - s * a.H;
    c = s * a.nc_per + j;
  } else {  // chunk order of the plan (by index inside the sequence)
    const int kk = tk / a.H;
    h = tk - kk * a.H;
    if (kk >= a.plan[0]) return;  // unused chunk slot: uniform per workgroup
    c = a.plan[a.order_off + kk];
  }
  Chunk k;
  if (!chunk_of(a, c, k)) return;
  const int g = h / a.heads_per_group;
  const size_t ldx = (size_t)a.H * kP, ldb = (size_t)a.G * N, PN = (size_t)kP * N;
  const bf16 *xc = static_cast<const bf16 *>(a.x) + (size_t)k.start * ldx + (size_t)h * kP;
  const bf16 *cc = static_cast<const bf16 *>(a.C) + (size_t)k.start * ldb + (size_t)g * N;
  // Loads in the order they are needed (vector memory loads complete in
  // issue order): dt, the predecessor poll, the first B^T tiles, then x into
  // registers, one instruction per 32-token step (instruction k of wave w:
  // rows 32k + 8w + lane/8, 16 bytes each). x reaches LDS step by step, so
  // S_c starts once the first half has arrived.
  float dtv;
  {
    const int t = min(tid, k.len - 1);
    const float d = dt_of(a, (float)static_cast<const bf16 *>(a.dt)[(size_t)(k.start + t) * a.H + h], h);
    dtv = tid < k.len ? d : 0.f;  // zero past the chunk end (and for tid >= Q)
  }
  const int pair = k.seq * a.H + h;
  const bool first = k.idx == 0;
  int early = 0;  // published count of the predecessor, read early
  if (!first && tid == 0)
    early = __hip_atomic_load(pub + pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float ah = a.A[h] * kLog2eChain;
  const float dsk = a.D ? a.D[h] : 0.f;
  const int nt0 = wave * NTW;
  // This wave's B^T operand tiles (n tiles nt0..), streamed KPF 32-token
  // steps ahead of their use; the first KPF steps now.
  constexpr int KPF = kDeep ? NKS : (NKS < 4 ? NKS : 4);
  const bf16 *btc = bt + (((size_t)c * a.G + g) * (N / 16) + nt0) * NKS * 512 + lane * 8;
  bf16x8 bts[NTW][KPF];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int ks = 0; ks < KPF; ++ks) bts[j][ks] = ldg8(btc + (size_t)(j * NKS + ks) * 512);
  const int xrl = lane >> 3, xcol = lane & 7;
  bf16x8 xr[NKS];
  {
    const char *xb = reinterpret_cast<const char *>(xc);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int r = 32 * ks + 8 * wave + xrl;
      xr[ks] = *reinterpret_cast<const bf16x8 *>(
          xb + (uint32_t)min(r, k.len - 1) * (uint32_t)(ldx * 2) + 16u * (uint32_t)xcol);
    }
  }
  // x rows of step ks into the swizzled LDS tile (rows past len hold copies
  // of the last row: finite values that are multiplied by zero weights).
  auto put_x = [&](int ks) {
    const int r = 32 * ks + 8 * wave + xrl;
    *reinterpret_cast<bf16x8 *>(sX + r * kP + ((xcol ^ (r & 7)) << 3)) = xr[ks];
  };
  const float incl = wave_inclusive_sum(dtv * ah);
  if (lane == 63 && wave < Q / 64) sTot[wave] = incl;
  if (tid == 0) sReady = (first || early >= k.idx) ? 1 : 0;
  __syncthreads();
  float pre = 0.f, cs_last = 0.f;
#pragma unroll
  for (int w = 0; w < Q / 64; ++w) {
    const float t = sTot[w];
    pre += w < wave ? t : 0.f;
    cs_last += t;
  }
  const bool ready = sReady != 0;
  const float cst = incl + pre;
  const float cs_tile_end = __shfl(cst, lane | 31);
  if (tid < Q) {
    sCs[tid] = cst;
    sDt[tid] = dtv;
    sW[tid] = exp2_fast(cs_last - cst) * dtv;
    sU[tid] = exp2_fast(cs_tile_end - cst) * dtv;
  }
  constexpr int XH = NKS / 2;  // x steps in LDS before S_c starts
#pragma unroll
  for (int ks = 0; ks < XH; ++ks) put_x(ks);
  __syncthreads();

  // ---- 2. S_c = (w o B)^T x; h_in loads in flight when already published ------
  f32x4 hin[NTW][4];
  if (ready) load_h_in<N, NTW>(hin, a, k, h, wave, nt0, lane);
  f32x4 hs[NTW][4];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) hs[j][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int trow = 8 * lg + (lr >> 2);
  int xoff[4][2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = trow + 4 * q;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) xoff[pt][q] = r * kP + tr_lane_off<kP>(16 * pt, r & 7);
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (ks == XH) {  // second half of x
#pragma unroll
      for (int k2 = XH; k2 < NKS; ++k2) put_x(k2);
      __syncthreads();
    }
    const int s0 = 32 * ks;
    // LDS reads first (in-order return): the weights, then the x operands.
    const float4 wa = *reinterpret_cast<const float4 *>(sW + s0 + 8 * lg);
    const float4 wb = *reinterpret_cast<const float4 *>(sW + s0 + 8 * lg + 4);
    bf16x8 xv[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x4 xl = ds_tr4(sX, s0 * kP + xoff[pt][0]);
      const bf16x4 xh = ds_tr4(sX, s0 * kP + xoff[pt][1]);
      xv[pt] = bf16x8{xl[0], xl[1], xl[2], xl[3], xh[0], xh[1], xh[2], xh[3]};
    }
    const float ww[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
    bf16x8 av[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) av[j][e] = (bf16)((float)bts[j][ks % KPF][e] * ww[e]);
      if (ks + KPF < NKS) bts[j][ks % KPF] = ldg8(btc + (size_t)(j * NKS + ks + KPF) * 512);
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int j = 0; j < NTW; ++j) hs[j][pt] = mfma(av[j], xv[pt], hs[j][pt]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- 3. h_in; h_out = 2^(cs_last) h_in + S_c to the ring; publish ------------
  const int iA = T == 8 ? wave : wave, iB = T - 1 - wave;
  bf16x8 acA[2][N / 32];
  load_c_tile<N>(acA, cc, ldb, iA, k.len, lane);  // used after the hand-off
  if (!ready) {
    if (tid == 0 && !wait_published(pub + pair, k.idx))
      __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    load_h_in<N, NTW>(hin, a, k, h, wave, nt0, lane);
  }
  int cs0, cs1;
  chunks_of_seq(a, k.seq, cs0, cs1);
  const bool last = c + 1 >= cs1;
  const float dec = exp2_fast(cs_last);
  const __amdgpu_buffer_rsrc_t rout = ring_rsrc(a.ring + ((size_t)pair * 2 + (k.idx & 1)) * PN, (int)(PN * 4));
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int n = 16 * (nt0 + j) + 4 * lg, p = 16 * pt + lr;
      const f32x4 hout = dec * hin[j][pt] + hs[j][pt];
      if (!last) {
        ring_store4(rout, (uint32_t)((((wave * NTW + j) * 4 + pt) * 64 + lane) * 16), hout);
      } else if (a.hT) {
        *reinterpret_cast<float4 *>(a.hT + (size_t)pair * PN + (size_t)p * N + n) =
            make_float4(hout[0], hout[1], hout[2], hout[3]);
      }
      uint2 hb;
      hb.x = pack2(hin[j][pt][0], hin[j][pt][1]);
      hb.y = pack2(hin[j][pt][2], hin[j][pt][3]);
      *reinterpret_cast<uint2 *>(sH + swz<N>(p, n)) = hb;
    }
  wait_vmem_all();  // this wave's ring stores have completed (device-coherent)
  __syncthreads();  // ... and every other wave's; sH complete
  if (!last && tid == 0)
    __hip_atomic_store(pub + pair, k.idx + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- 4. outputs, one 32-row tile at a time ------------------------------------
  const bf16 *cbase = cb + ((size_t)c * a.G + g) * PAIRS * 2 * 512 + lane * 8;
  bf16 *yc = static_cast<bf16 *>(a.y) + (size_t)k.start * ldx + (size_t)h * kP;
  bf16x8 acB[2][N / 32];
  {
    f32x4 Y[2][4];
    state_tile<N>(iA, Y, sH, sCs, acA, k.len, lane);
    intra_tile<Q>(iA, Y, sX, sCs, sDt, sU, cbase, dsk, lane);
    if (NTILE == 2) load_c_tile<N>(acB, cc, ldb, iB, k.len, lane);  // in flight during the stores
    store_tile(iA, Y, k.len, yc, ldx, lane);
  }
  if (NTILE == 2) {
    f32x4 Y[2][4];
    state_tile<N>(iB, Y, sH, sCs, acB, k.len, lane);
    intra_tile<Q>(iB, Y, sX, sCs, sDt, sU, cbase, dsk, lane);
    store_tile(iB, Y, k.len, yc, ldx, lane);
  }
}

// Final state of every (sequence, head) whose sequence has no tokens (no
// chunk workgroup exists for it): the initial state, or zeros.
__global__ __launch_bounds__(256) void k_final_of_empty(Args a) {
  const int s = blockIdx.x / a.H, h = blockIdx.x - s * a.H;
  int c0, c1;
  chunks_of_seq(a, s, c0, c1);
  if (c0 != c1) return;
  const size_t PN4 = (size_t)a.P * a.N / 4;
  const size_t off = ((size_t)s * a.H + h) * PN4;
  float4 *out = reinterpret_cast<float4 *>(a.hT) + off;
  const float4 *in = a.h0 ? reinterpret_cast<const float4 *>(a.h0) + off : nullptr;
  for (size_t i = threadIdx.x; i < PN4; i += 256)
    out[i] = in ? in[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_final_of_empty(const Args &a, hipStream_t st) {
  hipLaunchKernelGGL(k_final_of_empty, dim3((unsigned)(a.nseq * a.H)), dim3(256), 0, st, a);
  return hipGetLastError();
}

bool chain_path_supports(const Args &a) {
  return mfma_path_supports(a) && (a.Q == 128 || a.Q == 256) &&
         (a.N == 64 || a.N == 128 || a.N == 256);
}

// Work units up to which the deep-prefetch kernel is used: what 256 CUs hold
// at three workgroups each.
constexpr int64_t kDeepMaxUnits = 3 * 256;

template <int N, int Q>
static hipError_t launch_chain_nq(const Args &a, const void *cb, const void *bt,
                                  hipStream_t st) {
  const int64_t blocks = (int64_t)a.nc_max * a.H;
  if (blocks == 0) return hipSuccess;
  const bf16 *cbp = static_cast<const bf16 *>(cb), *btp = static_cast<const bf16 *>(bt);
  if constexpr (N != 256) {  // at N = 256 the deep variant does not fit the registers
    if (blocks <= kDeepMaxUnits) {
      hipLaunchKernelGGL((k_ssd_chain<N, Q, true>), dim3((unsigned)blocks),
                         dim3(64 * kChainWaves), 0, st, a, cbp, btp);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_ssd_chain<N, Q, false>), dim3((unsigned)blocks), dim3(64 * kChainWaves),
                     0, st, a, cbp, btp);
  return hipGetLastError();
}

hipError_t launch_chain(const Args &a, const void *cb, const void *bt, hipStream_t st) {
  if (a.N == 64)
    return a.Q == 128 ? launch_chain_nq<64, 128>(a, cb, bt, st)
                      : launch_chain_nq<64, 256>(a, cb, bt, st);
  if (a.N == 256)
    return a.Q == 128 ? launch_chain_nq<256, 128>(a, cb, bt, st)
                      : launch_chain_nq<256, 256>(a, cb, bt, st);
  return a.Q == 128 ? launch_chain_nq<128, 128>(a, cb, bt, st)
                    : launch_chain_nq<128, 256>(a, cb, bt, st);
}

}  // namespace ssd
