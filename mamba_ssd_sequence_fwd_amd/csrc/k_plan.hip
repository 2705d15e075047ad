// k_plan.hip -- chunk table of a packed varlen batch, built on the device.
//
// Packed sequences are independent (the state restarts at every sequence
// start: tj-hxxt.cn long read of the Mamba-1 paper, part III item 2.3,
// "Boundary Resetting"). Each sequence is cut into ceil(len/Q) chunks of its
// own, so no chunk straddles a boundary and the state passing between chunks
// never crosses sequences. One workgroup scans the per-sequence chunk counts
// and writes one (sequence, first token, length, index) record per chunk, the
// index flagged on the sequence's last chunk.
// Malformed cu_seqlens (cu[0] != 0, decreasing, cu[S] != total) set the error
// word and leave zero chunks, so every later kernel does nothing.
#include "ssd_internal.h"

namespace ssd {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void k_plan(Args a) {
  __shared__ int s_wave_tot[kPlanThreads / 64];
  __shared__ int s_bad;
  __shared__ int s_first[kOrderMaxSeqs];
  __shared__ int s_nch[kOrderMaxSeqs];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.nseq, Q = a.Q;
  int *first = a.plan + 2;  // first chunk of each sequence, then the total
  int4 *rec = reinterpret_cast<int4 *>(a.plan + a.rec_off);
  if (tid == 0) s_bad = stream_ends_ok(a.cu[0], a.cu[S], a.L) ? 0 : 1;
  __syncthreads();

  int carry = 0;  // chunks of all earlier tiles
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int cnt = 0;
    if (s < S) {
      const int n = seq_chunk_count(a.cu[s], a.cu[s + 1], a.L, Q);
      if (n < 0) s_bad = 1;  // benign race: all write 1
      else cnt = n;
    }
    // Block-wide exclusive scan of cnt: wave scan, then scan of wave totals.
    const int incl = wave_inclusive_sum(cnt);
    if (lane == 63) s_wave_tot[wave] = incl;
    __syncthreads();
    int before = 0, tile_tot = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      const int t = s_wave_tot[w];
      before += (w < wave) ? t : 0;
      tile_tot += t;
    }
    if (s < S) first[s] = carry + before + incl - cnt;
    carry += tile_tot;
    __syncthreads();
  }
  __syncthreads();
  const bool bad = s_bad != 0 || carry > a.nc_max;
  if (tid == 0) {
    a.plan[0] = bad ? 0 : carry;
    a.plan[1] = bad ? 1 : 0;
    first[S] = bad ? 0 : carry;
    if (bad) a.plan[a.nseg_off] = 0;  // no chained work units either
  }
  if (bad) return;
  for (int s = tid; s < S; s += kPlanThreads) {
    const int lo = a.cu[s], len = a.cu[s + 1] - lo, c0 = first[s];
    for (int i = 0, off = 0; off < len; ++i, off += Q)
      rec[c0 + i] = make_int4(s, lo + off, min(Q, len - off), i | (off + Q >= len ? kLastChunkFlag : 0));
  }
  // Work-unit order for the chained kernel. A unit is a segment of up to
  // a.seg consecutive chunks of one sequence (a.seg = 1: one chunk), and the
  // list holds each segment's first chunk: by segment index inside the
  // sequence, then by sequence (all first segments, then all second ones,
  // ...), so that a segment comes long after its predecessor. Segment j of
  // sequence s goes to position sum_s' min(segs(s'), j) + #{s' < s : segs(s')
  // > j}. With more than kOrderMaxSeqs sequences (the host then uses one-chunk
  // units) the sequence-major chunk order is kept.
  int *order = a.plan + a.order_off;
  const int nc = carry;
  const int seg = max(a.seg, 1);
  if (S > kOrderMaxSeqs) {
    for (int c = tid; c < nc; c += kPlanThreads) order[c] = c;
    if (tid == 0) a.plan[a.nseg_off] = nc;
    return;
  }
  int nseg_part = 0;
  for (int s = tid; s < S; s += kPlanThreads) {
    s_first[s] = first[s];
    s_nch[s] = (a.cu[s + 1] - a.cu[s] + Q - 1) / Q;
    nseg_part += (s_nch[s] + seg - 1) / seg;
  }
  // total number of segments: wave sums, then one thread adds the waves
  nseg_part = wave_inclusive_sum(nseg_part);
  if (lane == 63) s_wave_tot[wave] = nseg_part;
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) tot += s_wave_tot[w];
    a.plan[a.nseg_off] = tot;
  }
  for (int c = tid; c < nc; c += kPlanThreads) {
    int lo = 0, hi = S - 1;  // last sequence whose first chunk is <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_first[mid] <= c) lo = mid;
      else hi = mid - 1;
    }
    const int i = c - s_first[lo];
    if (i % seg != 0) continue;  // not the first chunk of a segment
    const int j = i / seg;
    int pos = 0;
    for (int s2 = 0; s2 < S; ++s2) {
      const int n2 = (s_nch[s2] + seg - 1) / seg;
      pos += min(n2, j) + ((s2 < lo && n2 > j) ? 1 : 0);
    }
    order[pos] = c;
  }
}

hipError_t launch_plan(const Args &a, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd
