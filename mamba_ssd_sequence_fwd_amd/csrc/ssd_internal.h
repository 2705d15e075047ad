// ssd_internal.h -- shared definitions of the SSD forward kernels (gfx950).
//
// Device-side view of one ssd_forward call, chunk geometry, bf16 helpers and
// wavefront primitives. Included by every kernel source and by the host
// dispatcher; nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Everything a kernel needs, passed by value as the kernel argument.
struct Args {
  const void *x;        // (T, H, P)  dtype
  const void *dt;       // (T, H)     dtype
  const float *A;       // (H)
  const void *B;        // (T, G, N)  dtype
  const void *C;        // (T, G, N)  dtype
  const float *D;       // (H) or null
  const float *h0;      // (S, H, P, N) or null
  void *y;              // (T, H, P)  dtype
  float *hT;            // (S, H, P, N) or null
  const int32_t *cu;    // (S + 1) device, varlen only
  int32_t *plan;        // chunk table (varlen)
  float *cs;            // (chunks, H, Q): log2 decay prefix inside the chunk
  float *states;        // (chunks, H, P, N)
  void *cb;             // bf16 C B^T tiles (MFMA path only)
  void *zeros;          // 256 zero bytes (written by the C B^T kernel)
  void *bt;             // chain path: bf16 B^T operand tiles per (chunk, group), or null
  int32_t *sync;        // chain path: [0] ticket, [1] error word, [kSyncHeader + c*H + h]
                        // status of chunk c, head h (kAggReady / kIncReady), then the
                        // chunk's log2 decay as float bits at [kSyncHeader + nc_max*H +
                        // c*H + h]; the first kSyncHeader + nc_max*H ints are zeroed by
                        // the C B^T kernel
  float *inc;           // chain path: (chunks, H, P, N) fp32 state leaving each chunk
  float *agg;           // chain path, one-chunk units: (chunks, H, P, N) fp32 state each
                        // chunk builds from a zero start, published when its
                        // predecessor's was late (null otherwise)
  int32_t nsync;        // ints of `sync` to zero (0 off the chain path)
  int32_t batch, L, H, P, N, G, Q;
  int32_t nseq;         // sequences: batch (dense) or num_seqs (varlen)
  int32_t varlen;       // 0 / 1
  int32_t nc_per;       // dense: chunks per batch row
  int32_t nc_max;       // chunk slots in the workspace
  int32_t heads_per_group;
  int32_t rec_off;      // int offset of the chunk records inside plan
  int32_t order_off;    // int offset of the chunk order (by index in sequence) inside plan
  const float *dt_bias; // (H) or null: per-head offset of the step pre-activation
  int32_t dt_softplus;  // 0: dt is the step; 1: dt is its pre-activation
  int32_t seg;          // chain path: consecutive chunks per work unit (1 = one chunk)
  int32_t nseg_off;     // int offset inside plan of the number of segments (varlen)
  int32_t nrange;       // chain path, dense input: > 0 when each workgroup takes one of
                        // nrange balanced ranges of the (sequence, head, chunk) order
  int32_t gqueue;       // chain path, one-chunk units: 1 when the units come from one
                        // queue per XCD, each over a contiguous eighth of the heads
};

// The chained kernel's XCD queues (of ranges, or of one-chunk units): one
// per XCD, whose counters are Args::sync[kRangeQueueWord + q kQueueStride],
// each in a 256-byte block of its own. The workgroups of a launch all take
// their ticket at the start; packed into one line, the counters' atomics
// queued behind each other (4 sequences x 8 chunks x 24 heads: 51.0 ->
// 47.7 us per pass with the counters apart).
constexpr int kRangeQueues = 8, kQueueStride = 64, kRangeQueueWord = 64;
// Ints ahead of the per-(chunk, head) status words in Args::sync ([0] the
// ticket of launches without queues, [1] the error word, then the queue
// counters), and the status values: the chunk's aggregate (its own state
// from a zero start and its decay) is published, or the state leaving it is.
constexpr int kSyncHeader = kRangeQueueWord + kRangeQueues * kQueueStride;
constexpr int kAggReady = 1, kIncReady = 2;

// Packed sequences up to which the plan orders the chained kernel's work
// units by their index inside the sequence (above it: sequence by sequence,
// one chunk per unit).
constexpr int kOrderMaxSeqs = 4096;

// Checks of packed-sequence offsets, shared by the device plan kernel (which
// must never index out of bounds whatever the device cu_seqlens hold) and
// the host validation of cu_seqlens:
// chunks of sequence [lo, hi) of a stream of L tokens, or -1 if malformed,
__host__ __device__ inline int seq_chunk_count(int lo, int hi, int L, int Q) {
  return (hi < lo || lo < 0 || hi > L) ? -1 : (hi - lo + Q - 1) / Q;
}
// and whether the offsets start at 0 and end at the stream's length.
__host__ __device__ inline bool stream_ends_ok(int first, int last, int L) {
  return first == 0 && last == L;
}

// Chunk c's place in the token stream.
struct Chunk {
  int32_t seq;    // sequence (batch row) it belongs to
  int32_t start;  // first token (flat index)
  int32_t len;    // tokens in the chunk, 1..Q
  int32_t idx;    // chunk number inside its sequence
  bool last;      // the last chunk of its sequence
};

// Flag on the index field of a packed-input chunk record: the chunk is the
// last of its sequence (so that no reader needs the sequence's offsets).
constexpr int32_t kLastChunkFlag = 1 << 30;

// Returns false if chunk slot c is unused (past the last chunk).
__device__ __forceinline__ bool chunk_of(const Args &a, int c, Chunk &k) {
  int seq, start, len, idx;
  bool ok, last;
  if (!a.varlen) {
    ok = c < a.batch * a.nc_per;
    seq = c / max(a.nc_per, 1);
    idx = c - seq * a.nc_per;
    start = seq * a.L + idx * a.Q;
    len = min(a.Q, a.L - idx * a.Q);
    last = idx == a.nc_per - 1;
  } else {
    ok = c < a.plan[0];
    const int4 r = ok ? reinterpret_cast<const int4 *>(a.plan + a.rec_off)[c]
                      : make_int4(0, 0, 1, 0);
    seq = r.x;
    start = r.y;
    len = r.z;
    idx = r.w & ~kLastChunkFlag;
    last = (r.w & kLastChunkFlag) != 0;
  }
  k.seq = seq;
  k.start = start;
  k.len = len;
  k.idx = idx;
  k.last = last;
  return ok;
}

// First chunk of sequence s and one past its last.
__device__ __forceinline__ void chunks_of_seq(const Args &a, int s, int &c0,
                                              int &c1) {
  if (!a.varlen) {
    c0 = s * a.nc_per;
    c1 = c0 + a.nc_per;
  } else if (a.plan[1] != 0) {  // malformed cu_seqlens: no chunks at all
    c0 = c1 = 0;
  } else {
    c0 = a.plan[2 + s];
    c1 = a.plan[3 + s];
  }
}

// ---- element types --------------------------------------------------------
typedef __bf16 bf16;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

template <typename T>
__device__ __forceinline__ float ld(const void *p, size_t i) {
  return to_f32(static_cast<const T *>(p)[i]);
}

// 2^x on the hardware exp unit (v_exp_f32); exact 0 for very negative x.
__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// The step of token t, head h, as the recurrence uses it: dt as given, or,
// when dt holds the step's pre-activation, softplus(dt + dt_bias[h]) (the
// selection mechanism's step activation). softplus(v) = log(1 + e^v), taken
// as v itself above 20 (the difference is below fp32 resolution).
__device__ __forceinline__ float softplus_f32(float v) {
  return v > 20.f ? v : log1pf(__expf(v));
}
__device__ __forceinline__ float dt_of(const Args &a, float raw, int h) {
  if (!a.dt_softplus) return raw;
  return softplus_f32(raw + (a.dt_bias ? a.dt_bias[h] : 0.f));
}

// ---- wavefront (64-lane) primitives ---------------------------------------
// DPP control codes (GFX9 encoding).
enum : int {
  kDppRowShr1 = 0x111,
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143,
};

template <int Ctrl, int RowMask>
__device__ __forceinline__ int dpp_or_zero(int v) {
  return __builtin_amdgcn_update_dpp(0, v, Ctrl, RowMask, 0xf, true);
}
template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(dpp_or_zero<Ctrl, RowMask>(__float_as_int(v)));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts inside each row
// of 16 lanes, then the row totals are carried with the GFX9 row broadcasts
// (lane 15 -> rows 1 and 3, lane 31 -> rows 2 and 3).
template <typename V>
__device__ __forceinline__ V wave_inclusive_sum(V v) {
  v += dpp_or_zero<kDppRowShr1, 0xf>(v);
  v += dpp_or_zero<kDppRowShr2, 0xf>(v);
  v += dpp_or_zero<kDppRowShr4, 0xf>(v);
  v += dpp_or_zero<kDppRowShr8, 0xf>(v);
  v += dpp_or_zero<kDppRowBcast15, 0xa>(v);
  v += dpp_or_zero<kDppRowBcast31, 0xc>(v);
  return v;
}

// ---- launchers (defined next to their kernels) ------------------------------
hipError_t launch_plan(const Args &a, hipStream_t s);
hipError_t launch_chunk_cumsum(const Args &a, bool bf16_io, hipStream_t s);
hipError_t launch_chunk_state_generic(const Args &a, bool bf16_io, hipStream_t s);
hipError_t launch_state_passing(const Args &a, hipStream_t s);
hipError_t launch_chunk_scan_generic(const Args &a, bool bf16_io, hipStream_t s);
bool mfma_path_supports(const Args &a);
size_t cb_bytes(const Args &a);
hipError_t launch_chunk_state_mfma(const Args &a, hipStream_t s);
hipError_t launch_chunk_cb(const Args &a, void *cb, hipStream_t s);
hipError_t launch_chunk_scan_mfma(const Args &a, const void *cb, hipStream_t s);
bool fused_path_supports(const Args &a);
hipError_t launch_fused(const Args &a, const void *cb, const void *zeros, hipStream_t s);
bool chain_path_supports(const Args &a);
hipError_t launch_chain(const Args &a, const void *cb, const void *bt, hipStream_t s);
int chain_segment(const Args &a);
int chain_ranges(const Args &a, int compute_units);
bool chain_group_queues(const Args &a);
bool chain_lookback(const Args &a);
bool f32seq_path_supports(const Args &a);
hipError_t launch_f32seq(const Args &a, hipStream_t s);
hipError_t launch_final_of_empty(const Args &a, hipStream_t s);

}  // namespace ssd
