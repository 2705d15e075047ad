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
// published-chunk counter. Per workgroup, with cs the log2-decay prefix of
// dt*A inside the chunk:
//
//   1. ticket -> (chunk, head); dt, the decay tables (cs, w, u) by a
//      wavefront prefix; x and B of the chunk into LDS (direct global->LDS).
//   2. S_c = (w o B)^T x (w_s = 2^(cs_last - cs_s) dt_s): the chunk's own
//      state from a zero start (the chunk_state step).
//   3. intra-chunk outputs: (C B^T o decay mask) (dt o x) + D x, with C B^T
//      tiles precomputed once per (chunk, group).
//   4. h_in from the previous chunk's workgroup (or the initial state / zero
//      at a sequence start); h_out = 2^(cs_last) h_in + S_c goes to the ring
//      (or to the final state after the sequence's last chunk) and is
//      published (the state_passing step).
//   5. outputs += 2^(cs_l) C_l h_in^T (the rest of the chunk_scan step); y.
//
// Steps 2-3 need nothing from other workgroups. Tickets from an atomic
// counter order the work units by chunk index inside the sequence, then
// sequence, then head, so the predecessor of a unit took its ticket a whole
// chunk-index level earlier and has normally published by the time step 4
// asks. A workgroup only ever waits on a smaller ticket, i.e. on one that is
// already running, so the chain cannot deadlock whatever order the hardware
// dispatches in. Every wait is bounded by a wall-clock limit; a wait that
// runs out sets an error word instead of hanging (the outputs are then
// wrong).
//
// HBM traffic: x, y once; B, C, dt and the C B^T tiles once per head
// through L2; 32 KB of fp32 state written and read per (chunk, head).
#include "mfma_common.h"

namespace ssd {

constexpr float kLog2eChain = 1.4426950408889634f;

// Intra-chunk outputs of the 16-row half tile (i, u), rows 32i+16u .. +15,
// added into Y (transposed: lane holds column l = 32i + 16u + lane%16 and
// rows p = 16pt + 4(lane/16) + r). Off-diagonal 32-token tiles j < i use the
// split decay 2^(cs_l - cs_r0) 2^(cs_r0 - cs_e) 2^(cs_e - cs_s) (three
// factors <= 1, e = last token of tile j, r0 = first row of tile i, the last
// one folded into sU); the diagonal tile takes the exact masked exponent and
// carries D on its diagonal. C B^T tiles stream from L2 two ahead.
template <int Q>
__device__ __forceinline__ void intra_half(int i, int u, f32x4 (&Y)[4], const bf16 *sX,
                                           const float *sCs, const float *sDt, const float *sU,
                                           const bf16 *cbase, float dsk) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int pair0 = i * (i + 1) / 2;
  const int lloc = 16 * u + lr;
  const float cs_l = sCs[32 * i + lloc];
  const float cs_r0 = sCs[32 * i];
  const float rdec = exp2_fast(cs_l - cs_r0);

  const int xrow = 4 * lg + (lr >> 2);
  int xoff[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) xoff[pt] = xrow * kP + tr_lane_off<kP>(16 * pt, xrow & 7);

  bf16x8 m0 = ldg8(cbase + (size_t)(pair0 * 2 + u) * 512);
  bf16x8 m1 = ldg8(cbase + (size_t)((pair0 + min(1, i)) * 2 + u) * 512);
#pragma unroll 1
  for (int j = 0; j < i; ++j) {
    bf16x8 m = m0;
    m0 = m1;
    m1 = ldg8(cbase + (size_t)((pair0 + min(j + 2, i)) * 2 + u) * 512);
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
      Y[pt] = mfma(bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, m, Y[pt]);
    }
  }
  // Diagonal tile j = i (m0 holds it: the stream clamps at i).
  {
    bf16x8 m = m0;
    const float4 ca = *reinterpret_cast<const float4 *>(sCs + 32 * i + 4 * lg);
    const float4 cb4 = *reinterpret_cast<const float4 *>(sCs + 32 * i + 16 + 4 * lg);
    const float4 da = *reinterpret_cast<const float4 *>(sDt + 32 * i + 4 * lg);
    const float4 db = *reinterpret_cast<const float4 *>(sDt + 32 * i + 16 + 4 * lg);
    const float cc[8] = {ca.x, ca.y, ca.z, ca.w, cb4.x, cb4.y, cb4.z, cb4.w};
    const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
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
      Y[pt] = mfma(bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, m, Y[pt]);
    }
  }
}

// State part of half tile (i, u): Y += 2^(cs_l) C_l h_in^T, then y (bf16).
// sH = h_in bf16 [p][n] (swizzled rows of N); ac = C row l of this group
// (load_c_rows of the row clamped into the chunk, offset by 8*(lane/16));
// rows l >= len are neither used nor stored.
template <int N>
__device__ __forceinline__ void load_c_rows(bf16x8 (&ac)[N / 32], const bf16 *crow) {
#pragma unroll
  for (int ks = 0; ks < N / 32; ++ks) ac[ks] = ldg8(crow + 32 * ks);
}

template <int N>
__device__ __forceinline__ void state_half_store(int i, int u, f32x4 (&Y)[4], const bf16 *sH,
                                                 const float *sCs, const bf16x8 (&ac)[N / 32],
                                                 int len, bf16 *y, size_t ystride) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int l = 32 * i + 16 * u + lr;
  const bool valid = l < len;
  f32x4 S[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) S[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < N / 32; ++ks) {
    const bf16x8 acv = valid ? ac[ks] : zero8();
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const bf16x8 bh =
          *reinterpret_cast<const bf16x8 *>(sH + swz<N>(16 * pt + lr, 32 * ks + 8 * lg));
      S[pt] = mfma(bh, acv, S[pt]);
    }
  }
  const float f = exp2_fast(sCs[l]);
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) Y[pt] += f * S[pt];
  if (valid) {
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

// The state hand-off between workgroups that may sit on different XCDs
// (each with its own L2). Ring entries are written and read with
// device-scope atomic accesses, which are coherent across the whole GPU
// without flushing or invalidating any cache: a producer's ring stores are
// complete once its s_waitcnt vmcnt(0) returns, it then bumps the counter,
// and a consumer issues its ring loads only after it has seen the counter.
__device__ __forceinline__ void ring_store(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ring_load(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

template <int N, int Q>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_ssd_chain(
    Args a, const bf16 *cb, const bf16 *zeros) {
  constexpr int T = Q / 32, PAIRS = T * (T + 1) / 2;
  constexpr int QB = Q * N <= 16384 ? Q : 16384 / N;  // tokens per B slice (32 KB of LDS)
  constexpr int NSL = Q / QB;
  constexpr int NT16 = N / 16;        // 16-row n tiles of the state
  constexpr int TPW = N / 32;         // state tiles per wave (8 waves, 4 p tiles)
  constexpr int SBH = QB * N > kP * N ? QB * N : kP * N;
  static_assert(Q == 128 || Q == 256, "chain kernel: chunk 128 or 256");
  static_assert(N == 64 || N == 128, "chain kernel: N 64 or 128");
  static_assert(NSL <= 2, "at most two B slices");
  __shared__ __attribute__((aligned(16))) bf16 sX[Q * kP];  // x, [token][p]
  __shared__ __attribute__((aligned(16))) bf16 sBH[SBH];    // B slice [token][n], then h_in [p][n]
  __shared__ __attribute__((aligned(16))) float sCs[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];
  __shared__ __attribute__((aligned(16))) float sU[Q];
  __shared__ __attribute__((aligned(16))) float sW[Q];
  __shared__ float sTot[4];
  __shared__ int sTicket;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  int32_t *ticket = a.sync, *err = a.sync + 1, *pub = a.sync + kSyncHeader;

  // ---- 1. work unit, decay tables, x and B into LDS ---------------------------
  if (tid == 0) sTicket = atomicAdd(ticket, 1);
  __syncthreads();
  const int tk = sTicket;
  // Ticket order: chunk index by chunk index across all sequences (all first
  // chunks, then all second chunks, ...), so a chunk's predecessor is many
  // tickets back and has usually finished by then.
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
  const size_t ldx = (size_t)a.H * kP, ldb = (size_t)a.G * N;
  const bf16 *xc = static_cast<const bf16 *>(a.x) + (size_t)k.start * ldx + (size_t)h * kP;
  const bf16 *bc = static_cast<const bf16 *>(a.B) + (size_t)k.start * ldb + (size_t)g * N;
  const bf16 *cc = static_cast<const bf16 *>(a.C) + (size_t)k.start * ldb + (size_t)g * N;
  async_tile<kP, Q>(sX, xc, ldx, k.len, zeros);
  async_tile<N, QB>(sBH, bc, ldb, k.len, zeros);
  // C rows of this wave's output half tiles (used last; loaded first).
  constexpr int NH = T == 8 ? 2 : 1;  // half tiles per wave
  const int iA = T == 8 ? wave : wave >> 1, uA = T == 8 ? 0 : wave & 1;
  const int iB = T - 1 - wave;
  bf16x8 acA[N / 32], acB[N / 32];
  load_c_rows<N>(acA, cc + (size_t)min(32 * iA + 16 * uA + lr, k.len - 1) * ldb + 8 * lg);
  if (NH == 2) load_c_rows<N>(acB, cc + (size_t)min(32 * iB + 16 + lr, k.len - 1) * ldb + 8 * lg);
  // Published count of the predecessor, read early: usually it is already
  // there and step 4 need not poll.
  const int pair = k.seq * a.H + h;
  const bool first = k.idx == 0;
  int early = 0;
  if (!first && tid == 0)
    early = __hip_atomic_load(pub + pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float dtv = 0.f;
  {
    const int t = min(tid, k.len - 1);
    const float d = (float)static_cast<const bf16 *>(a.dt)[(size_t)(k.start + t) * a.H + h];
    dtv = tid < k.len ? d : 0.f;  // zero past the chunk end (and for tid >= Q)
  }
  const float ah = a.A[h] * kLog2eChain;
  const float dsk = a.D ? a.D[h] : 0.f;
  const float incl = wave_inclusive_sum(dtv * ah);
  if (lane == 63 && wave < Q / 64) sTot[wave] = incl;
  __syncthreads();
  float pre = 0.f, cs_last = 0.f;
#pragma unroll
  for (int w = 0; w < Q / 64; ++w) {
    const float t = sTot[w];
    pre += w < wave ? t : 0.f;
    cs_last += t;
  }
  const float cst = incl + pre;
  const float cs_tile_end = __shfl(cst, lane | 31);
  if (tid < Q) {
    sCs[tid] = cst;
    sDt[tid] = dtv;
    sW[tid] = exp2_fast(cs_last - cst) * dtv;
    sU[tid] = exp2_fast(cs_tile_end - cst) * dtv;
  }
  wait_vmem_all();
  __syncthreads();

  // ---- 2. S_c = (w o B)^T x, state tiles (n tile nt, p tile pt0 + q) -------------
  const int nt = wave % NT16, pt0 = (wave / NT16) * TPW;
  const int trow = 8 * lg + (lr >> 2);
  int boff[2], xoff[TPW][2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = trow + 4 * q;
    boff[q] = r * N + tr_lane_off<N>(16 * nt, r & 7);
#pragma unroll
    for (int t = 0; t < TPW; ++t) xoff[t][q] = r * kP + tr_lane_off<kP>(16 * (pt0 + t), r & 7);
  }
  f32x4 hs[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) hs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto state_slice = [&](int sl) {
#pragma unroll
    for (int ks = 0; ks < QB / 32; ++ks) {
      const int s0 = sl * QB + 32 * ks;
      const float4 wa = *reinterpret_cast<const float4 *>(sW + s0 + 8 * lg);
      const float4 wb = *reinterpret_cast<const float4 *>(sW + s0 + 8 * lg + 4);
      const float ww[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
      const bf16x4 lo = ds_tr4(sBH, 32 * ks * N + boff[0]);
      const bf16x4 hi = ds_tr4(sBH, 32 * ks * N + boff[1]);
      const bf16 raw[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      bf16x8 av;
#pragma unroll
      for (int e = 0; e < 8; ++e) av[e] = (bf16)((float)raw[e] * ww[e]);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const bf16x4 xl = ds_tr4(sX, s0 * kP + xoff[t][0]);
        const bf16x4 xh = ds_tr4(sX, s0 * kP + xoff[t][1]);
        hs[t] = mfma(av, bf16x8{xl[0], xl[1], xl[2], xl[3], xh[0], xh[1], xh[2], xh[3]}, hs[t]);
      }
    }
  };
  state_slice(0);
  if (NSL == 2) {
    __syncthreads();  // every wave done with the first B slice
    async_tile<N, QB>(sBH, bc + (size_t)QB * ldb, ldb, k.len - QB, zeros);
  }

  // ---- 3. intra-chunk outputs (the second B slice lands meanwhile) -----------------
  const bf16 *cbase = cb + ((size_t)c * a.G + g) * PAIRS * 2 * 512 + lane * 8;
  f32x4 Y[NH][4];
#pragma unroll
  for (int t = 0; t < NH; ++t)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[t][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
  intra_half<Q>(iA, uA, Y[0], sX, sCs, sDt, sU, cbase, dsk);
  if (NH == 2) intra_half<Q>(iB, 1, Y[NH - 1], sX, sCs, sDt, sU, cbase, dsk);

  if (NSL == 2) {
    wait_vmem_all();
    __syncthreads();
    state_slice(1);
  }

  // ---- 4. h_in from the chain; h_out = 2^(cs_last) h_in + S_c ----------------------
  int cs0, cs1;
  chunks_of_seq(a, k.seq, cs0, cs1);
  const bool last = c + 1 >= cs1;
  if (!first && tid == 0 && early < k.idx && !wait_published(pub + pair, k.idx))
    __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();  // h_in published; every wave done reading the B slice

  const size_t PN = (size_t)kP * N;
  float *ring = a.ring + (size_t)pair * 2 * PN;
  const float *rin = ring + (size_t)((k.idx + 1) & 1) * PN;  // slot of chunk idx-1
  float *rout = ring + (size_t)(k.idx & 1) * PN;
  const float *h0 = a.h0 ? a.h0 + ((size_t)k.seq * a.H + h) * PN : nullptr;
  const float dec = exp2_fast(cs_last);
  bf16 *sH = sBH;
  // ring slot layout: [wave][tile][r][lane], 256 contiguous bytes per
  // access; every load is issued before the first store.
  f32x4 hin[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int n = 16 * nt + 4 * lg, p = 16 * (pt0 + t) + lr;
    hin[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!first) {
      const float *src = rin + (size_t)(wave * TPW + t) * 256 + lane;
#pragma unroll
      for (int r = 0; r < 4; ++r) hin[t][r] = ring_load(src + 64 * r);
    } else if (h0) {
      const float4 v = *reinterpret_cast<const float4 *>(h0 + (size_t)p * N + n);
      hin[t] = f32x4{v.x, v.y, v.z, v.w};
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int n = 16 * nt + 4 * lg, p = 16 * (pt0 + t) + lr;
    const f32x4 hout = dec * hin[t] + hs[t];
    if (!last) {
      float *dst = rout + (size_t)(wave * TPW + t) * 256 + lane;
#pragma unroll
      for (int r = 0; r < 4; ++r) ring_store(dst + 64 * r, hout[r]);
    } else if (a.hT) {
      *reinterpret_cast<float4 *>(a.hT + ((size_t)k.seq * a.H + h) * PN + (size_t)p * N + n) =
          make_float4(hout[0], hout[1], hout[2], hout[3]);
    }
    uint2 hb;
    hb.x = pack2(hin[t][0], hin[t][1]);
    hb.y = pack2(hin[t][2], hin[t][3]);
    *reinterpret_cast<uint2 *>(sH + swz<N>(p, n)) = hb;
  }
  wait_vmem_all();  // this wave's ring stores have completed (device-coherent)
  __syncthreads();  // ... and every other wave's; sH complete
  if (!last && tid == 0)
    __hip_atomic_store(pub + pair, k.idx + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- 5. outputs += 2^(cs_l) C_l h_in^T; y ------------------------------------------
  bf16 *yc = static_cast<bf16 *>(a.y) + (size_t)k.start * ldx + (size_t)h * kP;
  state_half_store<N>(iA, uA, Y[0], sH, sCs, acA, k.len, yc, ldx);
  if (NH == 2) state_half_store<N>(iB, 1, Y[NH - 1], sH, sCs, acB, k.len, yc, ldx);
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
  return mfma_path_supports(a) && (a.Q == 128 || a.Q == 256) && (a.N == 64 || a.N == 128);
}

template <int N, int Q>
static hipError_t launch_chain_nq(const Args &a, const void *cb, const void *zeros,
                                  hipStream_t st) {
  const int64_t blocks = (int64_t)a.nc_max * a.H;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((k_ssd_chain<N, Q>), dim3((unsigned)blocks), dim3(512), 0, st, a,
                     static_cast<const bf16 *>(cb), static_cast<const bf16 *>(zeros));
  return hipGetLastError();
}

hipError_t launch_chain(const Args &a, const void *cb, const void *zeros, hipStream_t st) {
  if (a.N == 64)
    return a.Q == 128 ? launch_chain_nq<64, 128>(a, cb, zeros, st)
                      : launch_chain_nq<64, 256>(a, cb, zeros, st);
  return a.Q == 128 ? launch_chain_nq<128, 128>(a, cb, zeros, st)
                    : launch_chain_nq<128, 256>(a, cb, zeros, st);
}

}  // namespace ssd
