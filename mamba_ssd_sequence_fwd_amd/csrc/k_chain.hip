// k_chain.hip -- the chunked SSD forward pass with one workgroup per
// (chunk, head) or per run of consecutive chunks, the inter-chunk
// recurrence carried between workgroups (bf16 inputs, MFMA, fp32 state).
//
// The SSD layer evaluates the semiseparable matrix by blocks: inside a chunk
// a masked-attention product, across chunks a linear recurrence on one state
// per chunk (QbitAI "Mamba-2" article, srwj168 repost, sections "Unifying SSM
// and attention" and "Mamba-2: stronger learning, faster training and
// inference"). Only the recurrence h_out = 2^(cs_last) h_in + S_c links the
// chunks of one (sequence, head); the workgroup of a chunk publishes the
// state leaving it in device memory and sets the chunk's status word, and
// the workgroup of the next chunk reads it. Per chunk (four waves), with cs
// the log2-decay prefix of dt*A inside the chunk:
//
//   1. ticket -> work unit; dt, the chunk's first B^T operand tiles and x
//      into registers (every load issued before any is waited for; loads
//      complete in issue order, so x is waited for step by step); the decay
//      tables (cs, w, u) by a wavefront prefix; the first half of x into LDS
//      (the second half halfway through step 2).
//   2. S_c = (w o B)^T x (w_s = 2^(cs_last - cs_s) dt_s): the chunk's own
//      state from a zero start (the chunk_state step).
//   3. h_in: the previous chunk's published state (loaded while step 2 runs
//      when it is already there), the state carried in registers inside a
//      run, or the initial state / zero at a sequence start; h_out =
//      2^(cs_last) h_in + S_c is published (or kept for the run's next
//      chunk, or written as the final state) (the state_passing step).
//   4. outputs, per 32-row tile: (C B^T o decay mask)(dt o x) + D x with the
//      C B^T tiles precomputed once per (chunk, group), plus 2^(cs_l) C_l h_in^T
//      (the chunk_scan step); y.
//
// Work units, chosen by the launcher from the grid size:
//   - problems of up to about twice what the chip holds at once (kDeep):
//     one chunk each; a unit whose predecessor's state is late publishes its
//     own aggregate (S_c and its decay) and rebuilds h_in from the nearest
//     published state and the aggregates after it (the chunk maps compose
//     associatively), so no unit waits for its predecessor's own wait (a
//     sequence's second chunk, whose predecessor never waits, waits plainly);
//   - problems with more units than that and many (sequence, head) pairs
//     (kSeg): runs of consecutive chunks of one pair with the state carried
//     in registers: dense input with at least one pair per resident
//     workgroup in one balanced range of the (sequence, head, chunk) order
//     per workgroup; packed input with at least two pairs per resident
//     workgroup in segments of up to twelve chunks. Only range or segment
//     boundaries go through memory;
//   - everything else (N = 256, fewer pairs): one chunk each.
// One-chunk units and ranges come from one queue per XCD (one-chunk units:
// over a contiguous eighth of the heads, whole groups where they split
// evenly), segments from one counter.
//
// Tickets from these counters, each taken in order, order the work units so
// that a unit's predecessors took smaller tickets of the same queue. A
// workgroup only ever waits on a smaller ticket, i.e. on one that is
// already running, and every unit publishes without waiting on a larger
// one, so the chain cannot deadlock whatever order the hardware dispatches
// in. Every wait is bounded by a
// wall-clock limit; a wait that runs out sets an error word instead of
// hanging (the outputs are then wrong).
//
// LDS holds only x (the operand both products read transposed) and h_in
// (bf16), 52 KB at chunk 256 and N = 128, so three one-chunk workgroups
// share a CU (two of the deep, segment and N = 256 kernels, by registers). Each wave owns
// whole 32-row output tiles, so the two 16-row halves of a tile share every
// x and h_in read. x is staged through registers rather than copied
// global->LDS directly: while such a copy is pending, every wait on a
// register load drains all outstanding loads, which would serialise the
// prefetches. Within each 32-token step, the small LDS reads go first and the
// x operand reads right after, so their latency hides behind the scaling
// arithmetic (LDS returns in order).
//
// HBM traffic: x, y once; B, C, dt and the C B^T tiles once per head
// through L2; 32 KB of fp32 state written and read per hand-off (N = 128),
// plus 32 KB per published aggregate.
#include "mfma_common.h"

namespace ssd {

constexpr float kLog2eChain = 1.4426950408889634f;
constexpr int kChainWaves = 4;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The C B^T tiles of one 32-row output tile i, streamed from L2 two steps
// ahead in two register buffers: a holds the even steps j and b the odd ones
// (step i, the diagonal tile, is the last; loads past it repeat it). Each
// buffer is refilled right after its step's products, never copied, so a
// load is waited for only when its own step comes (copying a buffer whose
// load is in flight would wait for it at once).
struct CbStream {
  bf16x8 a[2], b[2];
};
__device__ __forceinline__ void cb_load(bf16x8 (&m)[2], const bf16 *cbase, int pair) {
#pragma unroll
  for (int u = 0; u < 2; ++u) m[u] = ldg8(cbase + (size_t)(pair * 2 + u) * 512);
}
// The stream's first two steps, issued by the caller ahead of time (before
// its y stores: a load issued after a store can only be waited for together
// with it).
__device__ __forceinline__ void cb_begin(int i, CbStream &st, const bf16 *cbase) {
  const int pair0 = i * (i + 1) / 2;
  cb_load(st.a, cbase, pair0);
  cb_load(st.b, cbase, pair0 + min(1, i));
}

// Intra-chunk outputs of the 32-row tile i (rows 32i .. 32i+31), both 16-row
// halves u, added into Y[u] (transposed: lane holds column l = 32i + 16u +
// lane%16 and rows p = 16pt + 4(lane/16) + r). Off-diagonal 32-token tiles
// j < i use the split decay 2^(cs_l - cs_r0) 2^(cs_r0 - cs_e) 2^(cs_e - cs_s)
// (three factors <= 1, e = last token of tile j, r0 = first row of tile i,
// the last one folded into sU); the diagonal tile takes the exact masked
// exponent and carries D on its diagonal. Each x operand read serves both
// halves.
template <int Q>
__device__ __forceinline__ void intra_tile(int i, f32x4 (&Y)[2][4], CbStream &st, const bf16 *sX,
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

  // One off-diagonal step j with its tiles in m (scaled in place, then
  // refilled by the caller).
  auto step = [&](int j, bf16x8 (&m)[2]) {
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
    bf16x8 ms[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float fa = rdec[u] * e_r0;
#pragma unroll
      for (int e = 0; e < 8; ++e) ms[u][e] = (bf16)((float)m[u][e] * (fa * uu[e]));
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int u = 0; u < 2; ++u) Y[u][pt] = mfma(xv[pt], ms[u], Y[u][pt]);
  };
  // Unrolled over the at most Q/32 - 1 steps, every step refilling its
  // buffer (clamped at the diagonal), so that the only way into a step is
  // through the one before it and each wait counts exactly the loads it
  // needs (a join of paths that issued different loads, or a loop's back
  // edge, merges the counts conservatively: the step would also wait for the
  // other buffer's tiles, issued one step ago).
#pragma unroll
  for (int j = 0; j < Q / 32 - 1; ++j) {
    if (j >= i) break;
    if (j & 1) {
      step(j, st.b);
      cb_load(st.b, cbase, pair0 + min(j + 2, i));
    } else {
      step(j, st.a);
      cb_load(st.a, cbase, pair0 + min(j + 2, i));
    }
  }
  // Diagonal tile j = i: b holds it for odd i (loaded one step earlier than
  // a's copy), a for even i.
  auto diag = [&](const bf16x8 (&md)[2]) {
    const float4 ca = *reinterpret_cast<const float4 *>(sCs + 32 * i + 4 * lg);
    const float4 cb4 = *reinterpret_cast<const float4 *>(sCs + 32 * i + 16 + 4 * lg);
    const float4 da = *reinterpret_cast<const float4 *>(sDt + 32 * i + 4 * lg);
    const float4 db = *reinterpret_cast<const float4 *>(sDt + 32 * i + 16 + 4 * lg);
    const float cc[8] = {ca.x, ca.y, ca.z, ca.w, cb4.x, cb4.y, cb4.z, cb4.w};
    const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
    bf16x8 m[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int lloc = 16 * u + lr;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sloc = 16 * (e >> 2) + 4 * lg + (e & 3);
        const float v = (float)md[u][e] * exp2_fast(cs_l[u] - cc[e]) * dd[e];
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
  };
  if (i & 1)
    diag(st.b);
  else
    diag(st.a);
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

__device__ __forceinline__ uint32_t swap_adjacent(uint32_t v) {
  // lanes 2k and 2k + 1 exchange v (DPP quad_perm [1, 0, 3, 2])
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);
}

// y rows of the 32-row tile i, both halves. A lane holds, for its row l, four
// p tiles of packed values; lanes 16 apart (same row l) exchange one p tile's
// worth so that each lane holds 8 consecutive p, a 16-byte piece (v_permlane16
// _swap swaps the odd 16-lane rows of its first operand with the even rows of
// its second, so after swapping (p tile 2m, p tile 2m+1) every lane holds its
// output in order). The four lanes of a row then hold its two 64-byte halves
// m = 0, 1; adjacent lanes (rows 2k, 2k + 1) swap one half more, so that in
// each of two stores lane 2k + m writes half m of row 2k, then of row 2k + 1:
// every store instruction writes eight whole 128-byte rows.
__device__ __forceinline__ void store_tile(int i, const f32x4 (&Y)[2][4], int len, bf16 *y,
                                           size_t ystride, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int odd = lr & 1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    uint32_t pk[4][2];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      pk[pt][0] = pack2(Y[u][pt][0], Y[u][pt][1]);
      pk[pt][1] = pack2(Y[u][pt][2], Y[u][pt][3]);
    }
    uint32_t o[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const auto sx = __builtin_amdgcn_permlane16_swap(pk[2 * m][0], pk[2 * m + 1][0], false, false);
      const auto sy = __builtin_amdgcn_permlane16_swap(pk[2 * m][1], pk[2 * m + 1][1], false, false);
      o[m][0] = sx[0];
      o[m][1] = sy[0];
      o[m][2] = sx[1];
      o[m][3] = sy[1];
    }
    uint32_t fa[4], fb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t recv = swap_adjacent(odd ? o[0][e] : o[1][e]);
      fa[e] = odd ? recv : o[0][e];
      fb[e] = odd ? o[1][e] : recv;
    }
    // y is written once and read by nothing in this pass: nontemporal stores
    // of whole rows (order-balanced A/B against 64-byte half rows: the
    // 2.7B-shaped workload 176 -> 164 us per pass, the long packed one
    // 1691 -> 1586 us)
    const int ra = 32 * i + 16 * u + (lr & ~1);
    bf16 *ya = y + (size_t)ra * ystride + 8 * (lg >> 1) + 16 * (lg & 1) + 32 * odd;
    if (ra < len) {
      const u32x4_t va = {fa[0], fa[1], fa[2], fa[3]};
      __builtin_nontemporal_store(va, reinterpret_cast<u32x4_t *>(ya));
    }
    if (ra + 1 < len) {
      const u32x4_t vb = {fb[0], fb[1], fb[2], fb[3]};
      __builtin_nontemporal_store(vb, reinterpret_cast<u32x4_t *>(ya + ystride));
    }
  }
}

// The state hand-off between workgroups that may sit on different XCDs
// (each with its own L2). State slots are written and read by 16-byte buffer
// accesses with the sc1 cache policy (device scope, the same bits a relaxed
// device-scope atomic access carries), which are coherent across the whole
// GPU without flushing or invalidating any cache: a producer's slot stores
// are complete once its s_waitcnt vmcnt(0) returns, it then sets the chunk's
// status word, and a consumer issues its slot loads only after it has seen
// the status. The status alone orders the hand-off, so the slots need no
// atomicity of their own.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCachePolicyDevice = 16;  // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const float *slot, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(slot), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void slot_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kCachePolicyDevice);
}
__device__ __forceinline__ f32x4 slot_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyDevice));
}

// Work units (= workgroups) of a one-chunk-unit launch: every (chunk, head)
// of a dense batch, or every chunk slot of packed input times the heads.
__host__ __device__ inline int64_t chain_grid(const Args &a) {
  return (int64_t)(a.varlen ? a.nc_max : a.nseq * a.nc_per) * a.H;
}

// First head of XCD queue q (of kRangeQueues) over H heads: contiguous
// ranges whose sizes differ by at most one.
__host__ __device__ inline int head_lo(int H, int q) { return (int)((int64_t)H * q / kRangeQueues); }

// Per-(chunk, head) state slots in the workspace (the state leaving a chunk,
// and a chunk's aggregate), in the state-tile layout of the waves (tile (j,
// pt) of wave w: rows n = 16 (w NTW + j) + 4(lane/16) + r, column p = 16 pt
// + lane%16), stored [wave][j][pt][lane][r]: one 16-byte access per lane and
// 1 KB contiguous per wave access.
__device__ __forceinline__ uint32_t slot_off(int wave, int ntw, int j, int pt, int lane) {
  return (uint32_t)((((wave * ntw + j) * 4 + pt) * 64 + lane) * 16);
}
template <int N, int NTW>
__device__ __forceinline__ void load_slot(f32x4 (&v)[NTW][4], const float *slot, int wave,
                                          int lane) {
  const __amdgpu_buffer_rsrc_t r = slot_rsrc(slot, kP * N * 4);
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) v[j][pt] = slot_load4(r, slot_off(wave, NTW, j, pt, lane));
}

// The initial state of head h of sequence s (or zeros), this wave's tiles.
template <int N, int NTW>
__device__ __forceinline__ void load_h0(f32x4 (&v)[NTW][4], const Args &a, int s, int h,
                                        int nt0, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  if (a.h0) {
    const float *h0 = a.h0 + (size_t)(s * a.H + h) * kP * N;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int n = 16 * (nt0 + j) + 4 * lg, p = 16 * pt + lr;
        const float4 q = *reinterpret_cast<const float4 *>(h0 + (size_t)p * N + n);
        v[j][pt] = f32x4{q.x, q.y, q.z, q.w};
      }
  } else {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) v[j][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// The slot of the state leaving chunk number idx (global index c) of
// sequence s, head h. With aggregates (kLook): one slot per (chunk, head),
// never reused (a successor rebuilding its input may read it late).
// Otherwise two per (sequence, head), by chunk parity: the state leaving
// chunk i is read only by the unit of chunk i + 1, and the slot is next
// written with the state leaving chunk i + 2, which needs that unit's result
// first.
template <int N, bool kLook>
__device__ __forceinline__ float *inc_slot(const Args &a, int c, int idx, int s, int h) {
  const size_t PN = (size_t)kP * N;
  return kLook ? a.inc + ((size_t)c * a.H + h) * PN
               : a.inc + ((size_t)(s * a.H + h) * 2 + (idx & 1)) * PN;
}

// Incoming state of chunk k (global index c), head h: the published state
// leaving chunk c - 1, or at a sequence start the initial state.
template <int N, int NTW, bool kLook>
__device__ __forceinline__ void load_h_in(f32x4 (&hin)[NTW][4], const Args &a, const Chunk &k,
                                          int c, int h, int wave, int nt0, int lane) {
  if (k.idx > 0)
    load_slot<N, NTW>(hin, inc_slot<N, kLook>(a, c - 1, k.idx - 1, k.seq, h), wave, lane);
  else
    load_h0<N, NTW>(hin, a, k.seq, h, nt0, lane);
}

// d h + S, one rounding per element: the state recurrence across a chunk
// boundary, written out so that every place that evaluates it (the chunk's
// own unit, a successor rebuilding it from the chunk's aggregate) gets the
// same bits.
__device__ __forceinline__ f32x4 step_state(float d, const f32x4 &h, const f32x4 &S) {
  return f32x4{__builtin_fmaf(d, h[0], S[0]), __builtin_fmaf(d, h[1], S[1]),
               __builtin_fmaf(d, h[2], S[2]), __builtin_fmaf(d, h[3], S[3])};
}

// Bounded wait until a status word is nonzero; its value, or 0 if the
// wall-clock limit ran out first.
__device__ __forceinline__ int wait_status(const int32_t *st) {
  constexpr uint64_t kLimitTicks = 100000000ull;  // 1 s of the 100 MHz constant clock
  int v = __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v != 0) return v;
  const uint64_t t0 = wall_clock64();
  while ((v = __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
    __builtin_amdgcn_s_sleep(2);
    if (wall_clock64() - t0 > kLimitTicks) return 0;
  }
  return v;
}

// kDeep: every B^T tile of step 2 is loaded up front instead of four steps
// ahead, at two workgroups per CU instead of three (more registers), and
// units publish aggregates (one state slot per chunk). When a problem has
// about as many work units as the chip holds at once, each workgroup's own
// latency is most of the time and this wins (4 sequences x 24 heads x 8
// chunks, 768 units: 66 -> 56 us, then 57.0 -> 51.2 us with aggregates; the
// same aggregates with three workgroups per CU and four-step prefetch: 56.3
// us; up to twice as many units it still wins, kDeepMaxUnits); with many
// units per slot the third workgroup per CU hides that latency better (the
// 2.7B shapes: equal; long packed input: 13% slower), and aggregates there
// cost more than they save (N = 256 long sequences: 592 -> 662 us), so the
// layout picks it by grid size.
//
// kSeg: a work unit is a segment of up to a.seg consecutive chunks of one
// (sequence, head), walked in order by the same workgroup. Inside a segment
// the state passes from chunk to chunk in registers (it is carried through
// the output phase of the chunk before), so only the segment's last chunk
// publishes its state and only its first reads one: a segment of k chunks moves
// 1/k of the hand-off bytes of k one-chunk units. The carried state costs 32
// registers (N = 128), so segments run two workgroups per CU.
//
// kSeg with a.nrange > 0 (dense input with at least as many (sequence, head)
// pairs as the chip holds workgroups): instead of equal segments, each
// workgroup takes one of a.nrange balanced ranges of the chunk order
// (sequence, head, chunk index), so that every workgroup walks the same
// number of chunks and none is left for a partial last wave. The ranges come
// from one queue per XCD, each over an eighth of the pairs, so that the
// workgroups of one L2 read the same B, C and C B^T tiles. A range holds at
// least one pair's worth of chunks, so it is a run of whole pairs with at
// most a partial pair at each end: one that continues the previous range of
// its queue and one that the next range continues. The workgroup walks its
// last part first (it starts at a pair's first chunk and waits on nothing),
// then the whole pairs, then the first part, whose predecessor the workgroup
// of the previous range (taken earlier from the same queue) walked first.
// kStreamX (segments of packed input): x is loaded with the nontemporal
// hint, so that the rows every unit reads once do not push the B, C and
// C B^T tiles that all heads share out of the L2 (there every XCD walks
// every sequence's chunks). Dense grids keep plain loads, which wait less.
template <int N, int Q, bool kDeep, bool kSeg, bool kStreamX = false>
__global__ __launch_bounds__(64 * kChainWaves)
__attribute__((amdgpu_waves_per_eu(N == 256 || kDeep || kSeg ? 2 : 3,
                                   N == 256 || kDeep || kSeg ? 2 : 3)))
void k_ssd_chain(Args a, const bf16 *cb, const bf16 *bt) {
  constexpr int T = Q / 32, PAIRS = T * (T + 1) / 2, NKS = Q / 32;
  constexpr int NTW = N / 64;                 // 16-row n tiles of the state per wave
  constexpr int NTILE = T == 8 ? 2 : 1;       // 32-row output tiles per wave
  static_assert(Q == 128 || Q == 256, "chain kernel: chunk 128 or 256");
  static_assert(N == 64 || N == 128 || N == 256, "chain kernel: N 64, 128 or 256");
  static_assert(!kSeg || N != 256, "chain kernel: no segments at N = 256 (registers)");
  __shared__ __attribute__((aligned(16))) bf16 sX[Q * kP];  // x, [token][p]
  __shared__ __attribute__((aligned(16))) bf16 sH[kP * N];  // h_in (bf16), [p][n]
  __shared__ __attribute__((aligned(16))) float sCs[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];
  __shared__ __attribute__((aligned(16))) float sU[Q];
  __shared__ __attribute__((aligned(16))) float sW[Q];
  __shared__ float sTot[4];
  __shared__ int sTicket, sQueue, sReady, sNb;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int32_t *ticket = a.sync, *err = a.sync + 1, *stat = a.sync + kSyncHeader;
  int32_t *decw = stat + (size_t)a.nc_max * a.H;  // log2 decay of each published aggregate

  // ---- work unit: (first chunk, head, chunks in the segment) -----------------
  if (tid == 0) {
    if (kSeg && a.nrange > 0) {
      // range mode: a queue of ranges per XCD, over a contiguous block of
      // (sequence, head) pairs, so that the workgroups sharing an L2 read
      // the same B, C and C B^T tiles; an XCD whose queue is used up takes
      // from the next ones. Each queue is taken in order, and a range waits
      // only on the one before it in its queue.
      unsigned x;
      asm volatile("s_getreg_b32 %0, hwreg(20, 0, 4)" : "=s"(x));  // XCC_ID
      const int per = a.nrange / kRangeQueues;
      int got = -1;
      for (int d = 0; d < kRangeQueues && got < 0; ++d) {
        const int q = (int)((x + d) % kRangeQueues);
        const int t = atomicAdd(a.sync + kRangeQueueWord + q * kQueueStride, 1);
        if (t < per) got = q * per + t;
      }
      sTicket = got;
    } else if (!kSeg && a.gqueue) {
      // one queue per XCD over a contiguous eighth of the heads (whole groups
      // when they split evenly), taken in chunk order: the workgroups sharing
      // an L2 read the same groups' B^T and C B^T tiles, eight counters take
      // the atomics one counter took, and a unit's predecessor (same head)
      // comes earlier from the same queue. An XCD whose queue is used up
      // takes from the next ones.
      unsigned x;
      asm volatile("s_getreg_b32 %0, hwreg(20, 0, 4)" : "=s"(x));  // XCC_ID
      const int64_t per_head = chain_grid(a) / a.H;  // units of one head
      int got = -1, gq = 0;
      for (int d = 0; d < kRangeQueues && got < 0; ++d) {
        const int q = (int)((x + d) % kRangeQueues);
        const int64_t cap = per_head * (head_lo(a.H, q + 1) - head_lo(a.H, q));
        if (cap == 0) continue;
        const int t = atomicAdd(a.sync + kRangeQueueWord + q * kQueueStride, 1);
        if (t < cap) got = t, gq = q;
      }
      sTicket = got;
      sQueue = gq;
    } else {
      sTicket = atomicAdd(ticket, 1);
    }
  }
  __syncthreads();
  const int tk = sTicket;
  int c0 = 0, h = 0, nk = 1;
  int64_t rlo = 0, rhi = 0;  // range mode: [rlo, rhi) of the (sequence, head, chunk) order
  if (kSeg && a.nrange > 0) {
    if (tk < 0) return;  // (every workgroup finds a range: as many ranges as workgroups)
    const int per = a.nrange / kRangeQueues, q = tk / per, t = tk - q * per;
    const int64_t pairs = (int64_t)a.nseq * a.H;
    const int64_t p0 = q * pairs / kRangeQueues, p1 = (q + 1) * pairs / kRangeQueues;
    const int64_t u0 = p0 * a.nc_per, units = (p1 - p0) * a.nc_per;
    rlo = u0 + t * units / per;
    rhi = u0 + (t + 1) * units / per;
  } else if (!kSeg && a.gqueue) {
    if (tk < 0) return;  // (every workgroup finds a unit: as many units as workgroups)
    const int q = sQueue, hl = head_lo(a.H, q), hq = head_lo(a.H, q + 1) - hl, t = tk;
    if (!a.varlen) {
      const int j = t / (a.nseq * hq), r = t - j * (a.nseq * hq), s = r / hq;
      h = hl + (r - s * hq);
      c0 = s * a.nc_per + j;
    } else {
      const int kk = t / hq;
      h = hl + (t - kk * hq);
      if (kk >= a.plan[0]) return;  // unused slot: uniform per workgroup
      c0 = a.plan[a.order_off + kk];
    }
  } else if (!a.varlen) {
    const int per = a.nseq * a.H;
    const int j = tk / per, r = tk - j * per, s = r / a.H;
    h = r - s * a.H;
    const int i0 = kSeg ? j * a.seg : j;
    c0 = s * a.nc_per + i0;
    if (kSeg) nk = min(a.seg, a.nc_per - i0);
  } else {  // segment order of the plan (by segment index inside the sequence)
    const int kk = tk / a.H;
    h = tk - kk * a.H;
    if (kk >= a.plan[kSeg ? a.nseg_off : 0]) return;  // unused slot: uniform per workgroup
    c0 = a.plan[a.order_off + kk];
  }
  if (kSeg && a.varlen) {
    Chunk k0;
    if (!chunk_of(a, c0, k0)) return;
    int q0, q1;
    chunks_of_seq(a, k0.seq, q0, q1);
    nk = min(a.seg, q1 - c0);
  }
  const size_t ldx = (size_t)a.H * kP, ldb = (size_t)a.G * N, PN = (size_t)kP * N;
  // per-head constants, read once per run of chunks of one head
  float ah, dsk, dtb;
  auto set_head = [&]() {
    ah = a.A[h] * kLog2eChain;
    dsk = a.D ? a.D[h] : 0.f;
    dtb = a.dt_softplus && a.dt_bias ? a.dt_bias[h] : 0.f;
  };
  f32x4 hcarry[NTW][4];  // kSeg: the state leaving the previous chunk of the segment
  // x rows of one chunk into registers, one instruction per 32-token step
  // (instruction k of wave w: rows 32k + 8w + lane/8, 16 bytes each; rows
  // past len repeat the last row)
  auto load_x = [&](const bf16 *xc, int len, int lane, bf16x8 (&dst)[NKS]) {
    const char *xb = reinterpret_cast<const char *>(xc);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int r = 32 * ks + 8 * wave + (lane >> 3);
      const bf16x8 *src = reinterpret_cast<const bf16x8 *>(
          xb + (uint32_t)min(r, len - 1) * (uint32_t)(ldx * 2) + 16u * (uint32_t)(lane & 7));
      if constexpr (kStreamX)
        dst[ks] = __builtin_nontemporal_load(src);
      else
        dst[ks] = *src;
    }
  };

  // One chunk of the work unit; `tid` is passed in so that a segment's loop
  // recomputes the lane-derived offsets per chunk instead of keeping them
  // live (in registers) across the whole walk.
  // `after` = some chunk of this workgroup came before (whose outputs must
  // have read LDS before it is refilled).
  auto chunk_body = [&](const int ci, const int tid, const bool after) -> bool {
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int g = h / a.heads_per_group;
  const int c = c0 + ci;
  Chunk k;
  if (!chunk_of(a, c, k)) return false;
  if (kSeg && after) __syncthreads();
  const bool head = !kSeg || ci == 0;   // first chunk of the work unit
  const bool tail = !kSeg || ci == nk - 1;  // last chunk of the work unit
  const bf16 *xc = static_cast<const bf16 *>(a.x) + (size_t)k.start * ldx + (size_t)h * kP;
  const bf16 *cc = static_cast<const bf16 *>(a.C) + (size_t)k.start * ldb + (size_t)g * N;
  // ---- 1. loads, decay tables ------------------------------------------------
  // Every load is issued before any result is used, in the order they are
  // needed (vector memory loads complete in issue order): dt, the predecessor
  // poll, the first B^T tiles, then x into registers, one instruction per
  // 32-token step (instruction k of wave w: rows 32k + 8w + lane/8, 16 bytes
  // each). x reaches LDS step by step, so S_c starts once the first half has
  // arrived.
  const bf16 dtraw = static_cast<const bf16 *>(a.dt)[(size_t)(k.start + min(tid, k.len - 1)) * a.H + h];
  const int pair = k.seq * a.H + h;
  const bool first = k.idx == 0;
  int early = 0;  // the predecessor's status, read early
  if (head && !first && tid == 0)
    early = __hip_atomic_load(stat + (size_t)(c - 1) * a.H + h, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
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
  load_x(xc, k.len, lane, xr);
  float dtv = (float)dtraw;
  if (a.dt_softplus) dtv = softplus_f32(dtv + dtb);
  dtv = tid < k.len ? dtv : 0.f;  // zero past the chunk end (and for tid >= Q)
  // x rows of step ks into the swizzled LDS tile (rows past len hold copies
  // of the last row: finite values that are multiplied by zero weights).
  auto put_x = [&](int ks) {
    const int r = 32 * ks + 8 * wave + xrl;
    *reinterpret_cast<bf16x8 *>(sX + r * kP + ((xcol ^ (r & 7)) << 3)) = xr[ks];
  };
  const float incl = wave_inclusive_sum(dtv * ah);
  if (lane == 63 && wave < Q / 64) sTot[wave] = incl;
  if (head && tid == 0) sReady = (first || early == kIncReady) ? 1 : 0;
  __syncthreads();
  float pre = 0.f, cs_last = 0.f;
#pragma unroll
  for (int w = 0; w < Q / 64; ++w) {
    const float t = sTot[w];
    pre += w < wave ? t : 0.f;
    cs_last += t;
  }
  const bool ready = !head || sReady != 0;
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
  if (!head) {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) hin[j][pt] = hcarry[j][pt];
  } else if (ready) {
    load_h_in<N, NTW, kDeep>(hin, a, k, c, h, wave, nt0, lane);
  }
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

  // ---- 3. h_in; h_out = 2^(cs_last) h_in + S_c published; ----------------------
  const int iA = wave, iB = T - 1 - wave;
  if (!ready && (!kDeep || k.idx == 1)) {
    // The state leaving the previous chunk was not published before S_c:
    // wait for it (these units publish nothing else). Under kDeep this is
    // the second chunk of a sequence, whose predecessor (the first chunk)
    // never waits: it publishes soon, and an aggregate would only delay this
    // unit.
    if (tid == 0 && wait_status(stat + (size_t)(c - 1) * a.H + h) != kIncReady)
      __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    load_h_in<N, NTW, kDeep>(hin, a, k, c, h, wave, nt0, lane);
  } else if (!ready) {
    // kDeep (every unit resident at once): rather than wait for the
    // predecessor's own wait, publish this chunk's aggregate (S_c and its
    // decay) if that state is still missing, then rebuild h_in from the
    // nearest predecessor whose leaving state is published (or the sequence
    // start) and the aggregates of the chunks after it: h = 2^(d_m) h + S_m,
    // chunk by chunk, the very evaluation each of those units performs, so
    // h_in has the bits the plain chain would give it.
    if (tid == 0)  // (every wave read sReady before S_c)
      sReady = __hip_atomic_load(stat + (size_t)(c - 1) * a.H + h, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (sReady != kIncReady) {
      const __amdgpu_buffer_rsrc_t r = slot_rsrc(a.agg + ((size_t)c * a.H + h) * PN, (int)(PN * 4));
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) slot_store4(r, slot_off(wave, NTW, j, pt, lane), hs[j][pt]);
      if (tid == 0)
        __hip_atomic_store(decw + (size_t)c * a.H + h, __float_as_int(cs_last), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      wait_vmem_all();  // this wave's stores have completed (device-coherent)
      __syncthreads();  // ... and every other wave's
      if (tid == 0)
        __hip_atomic_store(stat + (size_t)c * a.H + h, kAggReady, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // Wave 0 reads the status of up to 64 predecessors at once (lane i:
    // chunk c - 1 - i) until the nearest published leaving state (or the
    // sequence start, when within reach) has only published aggregates after
    // it; sNb = how many chunks to rebuild from aggregates.
    if (wave == 0) {
      constexpr uint64_t kLimitTicks = 100000000ull;  // 1 s of the 100 MHz constant clock
      const int m = min(64, k.idx);
      const uint64_t t0 = wall_clock64();
      int nb = 0;
      for (;;) {
        const int v = lane < m ? __hip_atomic_load(stat + (size_t)(c - 1 - lane) * a.H + h,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : 0;
        const uint64_t incm = __ballot(lane < m && v == kIncReady);
        const uint64_t aggm = __ballot(lane < m && v != 0);
        // the base: the nearest published leaving state, else the start
        const int b = incm ? __builtin_ctzll(incm) : (k.idx <= 64 ? m : -1);
        const uint64_t need = b >= 64 ? ~0ull : ((1ull << b) - 1);
        if (b >= 0 && (aggm & need) == need) {
          nb = b;
          break;
        }
        if (wall_clock64() - t0 > kLimitTicks) {  // flagged; the outputs are then wrong
          if (lane == 0) __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          nb = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (lane == 0) sNb = nb;
    }
    __syncthreads();
    const int nb = sNb;
    if (nb < k.idx) {
      load_slot<N, NTW>(hin, inc_slot<N, true>(a, c - 1 - nb, k.idx - 1 - nb, k.seq, h), wave, lane);
    } else {
      load_h0<N, NTW>(hin, a, k.seq, h, nt0, lane);
    }
#pragma unroll 1
    for (int q = c - nb; q < c; ++q) {
      f32x4 t[NTW][4];
      load_slot<N, NTW>(t, a.agg + ((size_t)q * a.H + h) * PN, wave, lane);
      const float d = exp2_fast(__int_as_float(
          __hip_atomic_load(decw + (size_t)q * a.H + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) hin[j][pt] = step_state(d, hin[j][pt], t[j][pt]);
    }
  }
  const bool last = k.last;
  const float dec = exp2_fast(cs_last);
  // The C rows of the first output tile: issued now only when no state store
  // follows (the wait for the stores would wait for them too), else after
  // the publish.
  bf16x8 acA[2][N / 32];
  if (!tail) load_c_tile<N>(acA, cc, ldb, iA, k.len, lane);
  if (!tail) {  // the next chunk of the segment starts from h_out
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) hcarry[j][pt] = step_state(dec, hin[j][pt], hs[j][pt]);
  } else if (!last) {
    const __amdgpu_buffer_rsrc_t rout =
        slot_rsrc(inc_slot<N, kDeep>(a, c, k.idx, k.seq, h), (int)(PN * 4));
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        slot_store4(rout, slot_off(wave, NTW, j, pt, lane), step_state(dec, hin[j][pt], hs[j][pt]));
  } else if (a.hT) {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int n = 16 * (nt0 + j) + 4 * lg, p = 16 * pt + lr;
        const f32x4 hout = step_state(dec, hin[j][pt], hs[j][pt]);
        *reinterpret_cast<float4 *>(a.hT + (size_t)pair * PN + (size_t)p * N + n) =
            make_float4(hout[0], hout[1], hout[2], hout[3]);
      }
  }
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int n = 16 * (nt0 + j) + 4 * lg, p = 16 * pt + lr;
      uint2 hb;
      hb.x = pack2(hin[j][pt][0], hin[j][pt][1]);
      hb.y = pack2(hin[j][pt][2], hin[j][pt][3]);
      *reinterpret_cast<uint2 *>(sH + swz<N>(p, n)) = hb;
    }
  if (tail) wait_vmem_all();  // this wave's state stores have completed (device-coherent)
  __syncthreads();  // ... and every other wave's; sH complete
  if (tail && !last && tid == 0)
    __hip_atomic_store(stat + (size_t)c * a.H + h, kIncReady, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (tail) load_c_tile<N>(acA, cc, ldb, iA, k.len, lane);

  // ---- 4. outputs, one 32-row tile at a time ------------------------------------
  const bf16 *cbase = cb + ((size_t)c * a.G + g) * PAIRS * 2 * 512 + lane * 8;
  bf16 *yc = static_cast<bf16 *>(a.y) + (size_t)k.start * ldx + (size_t)h * kP;
  bf16x8 acB[2][N / 32];
  CbStream sA, sB;
  {
    f32x4 Y[2][4];
    cb_begin(iA, sA, cbase);  // in flight during the state product
    state_tile<N>(iA, Y, sH, sCs, acA, k.len, lane);
    intra_tile<Q>(iA, Y, sA, sX, sCs, sDt, sU, cbase, dsk, lane);
    if (NTILE == 2) {  // the second tile's first loads, in flight during the stores
      load_c_tile<N>(acB, cc, ldb, iB, k.len, lane);
      cb_begin(iB, sB, cbase);
    }
    store_tile(iA, Y, k.len, yc, ldx, lane);
  }
  if (NTILE == 2) {
    f32x4 Y[2][4];
    state_tile<N>(iB, Y, sH, sCs, acB, k.len, lane);
    intra_tile<Q>(iB, Y, sB, sX, sCs, sDt, sU, cbase, dsk, lane);
    store_tile(iB, Y, k.len, yc, ldx, lane);
  }
  return true;
  };  // chunk_body

  if constexpr (kSeg) {
    if (a.nrange > 0) {
      // parts of the range from the last back to the first
      bool after = false;
#pragma unroll 1
      for (int64_t e = rhi; e > rlo;) {
        const int64_t pair = (e - 1) / a.nc_per;
        const int64_t b = max(rlo, pair * a.nc_per);
        const int s = (int)(pair / a.H);
        h = (int)(pair - (int64_t)s * a.H);
        c0 = s * a.nc_per + (int)(b - pair * a.nc_per);
        nk = (int)(e - b);
        set_head();
#pragma unroll 1
        for (int ci = 0; ci < nk; ++ci) {
          int t = tid;
          asm volatile("" : "+v"(t));
          chunk_body(ci, t, after);
          after = true;
        }
        e = b;
      }
    } else {
      set_head();
#pragma unroll 1
      for (int ci = 0; ci < nk; ++ci) {
        int t = tid;
        asm volatile("" : "+v"(t));
        if (!chunk_body(ci, t, ci > 0)) break;
      }
    }
  } else {
    set_head();
    chunk_body(0, tid, false);
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

// Work units that 256 CUs hold at once, three workgroups each.
constexpr int64_t kResidentUnits = 3 * 256;

// One-chunk units up to which the look-back kernel (deep prefetch, two
// workgroups per CU) runs when the layout gives it its per-chunk slots.
// Order-balanced A/B on one box against the plain-wait kernel, outputs
// bit-identical: 1,024 units (2 x 8 chunks x 64 heads) 62.2 -> 58.4 us per
// pass; 1,152 (36 pairs x 32 chunks) 98.8 -> 79.9; 1,280 (80 pairs x 16)
// 75.6 -> 71.5; 1,536 even. Above that the plain wait is faster (4,096 to
// 8,192 units).
constexpr int64_t kDeepMaxUnits = 6 * 256;

// Chunks per work unit for dense problems with more units than the chip holds
// at once and at least as many (sequence, head) pairs as it holds segment
// workgroups (2 per CU on 256 CUs; these take balanced ranges when they have
// two or more chunks per sequence). Order-balanced A/B on one box, with
// whole-row y stores, the 2.7B-shaped workload: units of 1, 2, 3 and 4 chunks
// within 3% of each other (163-170 us per pass over two rounds), so the
// longest is taken: it moves the fewest hand-off bytes (42 MB per launch
// against 294 MB for one-chunk units). With fewer pairs a segment's chunks
// run one after another inside a workgroup and the sequences' chains
// lengthen: segments of 4 against one-chunk units, order-balanced, 160 pairs
// of 32 chunks: 292.8 -> 183.5 us per pass; 64 pairs of 128 chunks: 1000.3
// -> 413.8 us; 384 pairs of 8 chunks: 141.1 -> 115.4 us (bit-identical).
constexpr int kChainSeg = 4;
constexpr int64_t kSegDenseMinPairs = 2 * 256;

// Packed input: segments of up to 12 chunks when there are at least twice as
// many (sequence, head) pairs as the chip holds segment workgroups (2 per CU
// on 256 CUs), so that one pair's walk, chunk after chunk inside a workgroup,
// is at most half of a workgroup's share of the work. Order-balanced A/B on
// one box, 64 packed sequences of 0 to 16 chunks, 80 heads (5,120 pairs):
// one-chunk units 1509 us per pass, segments of 2: 1518, 4: 1417, 8: 1380,
// 12: 1365, 16: 1420 (the same with slow decay: 1384, -, 1288, 1271, 1239,
// 1271), outputs bit-identical. Fewer pairs keep one-chunk units, whose
// chain of hand-offs overlaps the chunks of a sequence across workgroups.
constexpr int kChainSegPacked = 12;
constexpr int64_t kSegPackedMinPairs = 2 * 2 * 256;

int chain_segment(const Args &a) {
  if (a.N == 256) return 1;
  // one-chunk units when they all fit the chip at once: there each unit's
  // latency is the whole time, and a longer chain of dependent links within a
  // workgroup would only lengthen it
  if ((int64_t)a.nc_max * a.H <= kResidentUnits) return 1;
  if (a.varlen) return (int64_t)a.nseq * a.H >= kSegPackedMinPairs ? kChainSegPacked : 1;
  return (int64_t)a.nseq * a.H >= kSegDenseMinPairs ? kChainSeg : 1;
}

// Workgroups of the segment kernel that one CU holds (its registers).
constexpr int kSegWorkgroupsPerCu = 2;

// Balanced ranges (one per workgroup, all resident at once) when a dense
// problem has at least as many (sequence, head) pairs as the chip holds
// segment workgroups and more than one chunk per sequence; 0 otherwise.
// Order-balanced A/B on one box, the 2.7B-shaped workload (640 pairs of 8
// chunks: 512 workgroups of 10 chunks against 1280 segments of 4, whose last
// 256 ran as a half-full wave): 165.4 -> 158.9 us per pass, outputs
// bit-identical.
int chain_ranges(const Args &a, int compute_units) {
  if (a.varlen || a.N == 256 || a.seg <= 1 || a.nc_per < 2) return 0;
  // a whole number of ranges per queue
  const int64_t slots = (int64_t)compute_units * kSegWorkgroupsPerCu / kRangeQueues * kRangeQueues;
  if (slots <= 0 || (int64_t)a.nseq * a.H < slots) return 0;
  return (int)slots;
}

int64_t chain_units(const Args &a) {
  if (a.nrange > 0) return a.nrange;
  const int s = a.seg;
  if (!a.varlen) return (int64_t)a.nseq * ((a.nc_per + s - 1) / s) * a.H;
  // sum over sequences of ceil(chunks / s) <= (chunks + sequences (s - 1)) / s
  return (((int64_t)a.nc_max + (int64_t)a.nseq * (s - 1)) / s) * a.H;
}

// One-chunk units take their units from one queue per XCD, each over a
// contiguous eighth of the heads (whole groups when there are at least 8 and
// they split evenly), where one ticket counter served grids with fewer
// groups. The ticket is the first thing every workgroup waits for: a
// timing-only copy that took the grid's block order as the ticket ran 4 x 8
// chunks x 24 heads (look-back kernel) at 45.8 us per pass against 50.1, and
// one that took the ticket but used the block order at 50.0. Order-balanced
// A/B on one box, outputs bit-identical, per pass: eight queues against the
// one counter, their counters packed in one line: 51.5 against 50.5, 2 x 8
// x 64 heads 56.5 against 55.9, 2 x 32 x 64 heads (plain wait) 156.9 against
// 161.9; with the counters 256 bytes apart (kQueueStride): 51.0 -> 47.7,
// 56.9 -> 53.0, 152.4 -> 148.1.
bool chain_group_queues(const Args &a) { return a.seg <= 1; }

// Whether a problem's layout gives the chained kernel per-chunk state and
// aggregate slots (Args::agg non-null), with which the launch takes the kDeep
// kernel: its units publish aggregates and the state leaving every chunk.
bool chain_lookback(const Args &a) {
  return a.N != 256 && a.seg <= 1 && chain_units(a) <= kDeepMaxUnits;
}

template <int N, int Q>
static hipError_t launch_chain_nq(const Args &a, const void *cb, const void *bt,
                                  hipStream_t st) {
  const int64_t blocks = chain_units(a);
  if (blocks == 0) return hipSuccess;
  const bf16 *cbp = static_cast<const bf16 *>(cb), *btp = static_cast<const bf16 *>(bt);
  if constexpr (N != 256) {  // at N = 256 neither variant fits the registers
    if (a.seg > 1) {
      if (a.varlen)
        hipLaunchKernelGGL((k_ssd_chain<N, Q, false, true, true>), dim3((unsigned)blocks),
                           dim3(64 * kChainWaves), 0, st, a, cbp, btp);
      else
        hipLaunchKernelGGL((k_ssd_chain<N, Q, false, true>), dim3((unsigned)blocks),
                           dim3(64 * kChainWaves), 0, st, a, cbp, btp);
      return hipGetLastError();
    }
    if (a.agg) {  // per-chunk slots (at most kDeepMaxUnits one-chunk units)
      hipLaunchKernelGGL((k_ssd_chain<N, Q, true, false>), dim3((unsigned)blocks),
                         dim3(64 * kChainWaves), 0, st, a, cbp, btp);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_ssd_chain<N, Q, false, false>), dim3((unsigned)blocks),
                     dim3(64 * kChainWaves), 0, st, a, cbp, btp);
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
