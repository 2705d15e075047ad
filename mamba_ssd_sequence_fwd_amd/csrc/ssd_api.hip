// ssd_api.hip -- the C ABI (include/ssd.h): validation, workspace layout and
// the launch sequence of one SSD forward pass.
//
// Launch order on the caller's stream (one pass over the hot path):
//   [varlen] k_plan            chunk table from cu_seqlens (device side)
// then, by default for bf16 (chunk 128/256, P 64, N 64/128/256):
//   k_chunk_cb                 C B^T once per (chunk, group); clears the
//                              chain counters
//   k_ssd_chain                one workgroup per (chunk, head); the state
//                              recurrence handed from chunk to chunk
// or, with SSD_FLAG_PER_SEQUENCE,
//   k_chunk_cb, k_ssd_fused    one workgroup per (sequence, head) walks its
//                              chunks with the state in registers
// otherwise (fp32, other shapes, or SSD_FLAG_UNFUSED), one kernel per step:
//   k_chunk_cumsum             log2-decay prefix inside each chunk
//   k_chunk_state_{mfma,generic}  per-chunk states from a zero start
//   k_state_passing            serial recurrence across chunks (in place)
//   [bf16] k_chunk_cb          C B^T once per (chunk, group)
//   k_chunk_scan_{mfma,generic}   outputs
// Nothing is allocated, synchronised or read back; host work is O(1).
#include <stdarg.h>
#include <stdio.h>

#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "ssd.h"
#include "ssd_internal.h"
#include "step.h"
#include "scan.h"
#include "conv.h"
#include "bwd.h"

namespace {

thread_local std::string g_detail;

ssd_status fail(ssd_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return st;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Which kernels a problem runs on.
enum Path {
  kF32Seq,       // fp32: one workgroup per (sequence, head) on fp32 MFMA, one launch
  kGeneric,      // plain FMA chunk kernels (fp32, and shapes MFMA does not cover)
  kMfmaUnfused,  // one MFMA kernel per step of the method
  kMfmaFused,    // C B^T per (chunk, group) + one fused kernel per (sequence, head)
  kMfmaChain     // C B^T per (chunk, group) + one workgroup per (chunk, head), chained
};

struct Layout {
  int64_t nc_max;
  int64_t rec_off;  // int32 offset of the chunk records in the plan area
  size_t plan, cs, states, cb, bt, zeros, sync, inc, agg, total;
  int64_t nsync;     // int32 words of the chained kernel's sync area
  int64_t nzero;     // ... of which the C B^T kernel zeroes the first nzero
  int seg;           // chained kernel: chunks per work unit
  Path path;
  bool mfma;
};

Path path_of(const ssd_problem &p) {
  ssd::Args a{};
  a.P = p.headdim;
  a.N = p.dstate;
  a.Q = p.chunk_size;
  if (p.dtype == SSD_DTYPE_F32 && !(p.flags & (SSD_FLAG_GENERIC_KERNELS | SSD_FLAG_UNFUSED)) &&
      ssd::f32seq_path_supports(a))
    return kF32Seq;
  if (p.dtype != SSD_DTYPE_BF16 || (p.flags & SSD_FLAG_GENERIC_KERNELS)) return kGeneric;
  if (!ssd::mfma_path_supports(a)) return kGeneric;
  if (p.flags & SSD_FLAG_UNFUSED) return kMfmaUnfused;
  if (p.flags & SSD_FLAG_PER_SEQUENCE)
    return ssd::fused_path_supports(a) ? kMfmaFused : kMfmaUnfused;
  return ssd::chain_path_supports(a) ? kMfmaChain : kMfmaUnfused;
}

// allow_look false: the chained kernel's compact layout (two state slots per
// (sequence, head), plain waits) even where per-chunk look-back slots would
// be chosen, for a workspace of fixed size.
Layout make_layout(const ssd_problem &p, bool allow_look = true) {
  Layout L{};
  const int64_t Q = p.chunk_size;
  L.nc_max = p.num_seqs > 0 ? p.seqlen / Q + p.num_seqs
                            : (int64_t)p.batch * ((p.seqlen + Q - 1) / Q);
  L.rec_off = p.num_seqs > 0 ? (int64_t)round_up(4 + (size_t)p.num_seqs, 4) : 0;
  // varlen: header, first chunk per sequence and the total, the number of
  // chained work units, 4-int records, work-unit order
  const size_t plan_ints = p.num_seqs > 0 ? (size_t)(L.rec_off + 5 * L.nc_max) : 4;
  L.path = path_of(p);
  L.mfma = L.path != kGeneric && L.path != kF32Seq;
  const bool unfused = L.path == kGeneric || L.path == kMfmaUnfused;  // per-chunk intermediates
  size_t off = 0;
  L.plan = off;
  off = round_up(off + plan_ints * sizeof(int32_t), kAlign);
  L.cs = off;
  if (unfused) off = round_up(off + (size_t)L.nc_max * p.nheads * Q * sizeof(float), kAlign);
  L.states = off;
  if (unfused)
    off = round_up(off + (size_t)L.nc_max * p.nheads * p.headdim * p.dstate * sizeof(float),
                   kAlign);
  L.cb = off;
  if (L.mfma) {
    const int64_t T = Q / 32;
    off = round_up(off + (size_t)L.nc_max * p.ngroups * (T * (T + 1) / 2) * 2 * 1024, kAlign);
  }
  L.bt = off;  // chain path: B^T operand tiles, (chunks, G, N/16, Q/32) x 1 KB
  if (L.path == kMfmaChain)
    off = round_up(off + (size_t)L.nc_max * p.ngroups * (p.dstate / 16) * (Q / 32) * 1024, kAlign);
  L.zeros = off;
  if (L.mfma) off += kAlign;
  const int64_t nseq = p.num_seqs > 0 ? p.num_seqs : p.batch;
  // chained kernel: a status word and a decay per (chunk, head), the state
  // leaving every chunk, and (one-chunk units) every chunk's aggregate
  const bool chain = L.path == kMfmaChain && L.nc_max > 0;
  L.seg = 1;
  bool look = false;  // units publish aggregates (one state slot per chunk)
  if (chain) {
    ssd::Args a{};
    a.N = p.dstate;
    a.H = p.nheads;
    a.varlen = p.num_seqs > 0 ? 1 : 0;
    a.nseq = (int32_t)nseq;
    a.nc_per = a.varlen ? 0 : (p.seqlen + p.chunk_size - 1) / p.chunk_size;
    a.nc_max = (int32_t)L.nc_max;
    L.seg = a.seg = ssd::chain_segment(a);
    look = allow_look && ssd::chain_lookback(a);
  }
  const size_t state_bytes = (size_t)p.headdim * p.dstate * sizeof(float);
  const size_t per_chunk = (size_t)L.nc_max * p.nheads * state_bytes;
  L.sync = off;
  L.nzero = chain ? ssd::kSyncHeader + L.nc_max * p.nheads : 0;
  L.nsync = chain ? L.nzero + L.nc_max * p.nheads : 0;
  off = round_up(off + (size_t)L.nsync * sizeof(int32_t), kAlign);
  // the state leaving a chunk: two slots per (sequence, head), or with
  // aggregates one per (chunk, head), then the aggregates
  L.inc = off;
  if (chain)
    off = round_up(off + (look ? per_chunk : (size_t)nseq * p.nheads * 2 * state_bytes), kAlign);
  L.agg = off;
  if (look) off = round_up(off + per_chunk, kAlign);
  L.total = off;
  return L;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

ssd_status check_args(const ssd_problem *p, const void *x, const void *dt, const float *A,
                      const void *B, const void *C, const int32_t *cu_seqlens, const void *y,
                      const float *initial_state, const float *final_state,
                      const void *workspace, size_t workspace_bytes,
                      bool allow_look = true) {
  ssd_status st = ssd_validate(p);
  if (st != SSD_OK) return st;
  const bool varlen = p->num_seqs > 0;
  const int64_t tokens = (int64_t)p->batch * p->seqlen;
  if (tokens > 0 && (!x || !dt || !B || !C || !y))
    return fail(SSD_ERR_INVALID_ARG, "x, dt, B, C and y must be non-NULL");
  if (!A) return fail(SSD_ERR_INVALID_ARG, "A must be non-NULL");
  if (varlen && !cu_seqlens) return fail(SSD_ERR_INVALID_ARG, "varlen needs cu_seqlens");
  if (!varlen && cu_seqlens)
    return fail(SSD_ERR_INVALID_ARG, "cu_seqlens given but num_seqs is 0");
  if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) ||
      !aligned16(initial_state) || !aligned16(final_state))
    return fail(SSD_ERR_INVALID_ARG, "x, B, C, y and the states must be 16-byte aligned");
  const Layout L = make_layout(*p, allow_look);
  if (!workspace || ((uintptr_t)workspace % kAlign) != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                L.total);
  return SSD_OK;
}

// Compute units of the current device, cached per device; 256 (MI355X) when
// no device answers, as for a layout query on a machine without a GPU.
int device_compute_units() {
  static int cached[64] = {};
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  cached[dev] = n;
  return n;
}

ssd::Args make_args(const ssd_problem *p, const Layout &L, const void *x, const void *dt,
                    const float *A, const void *B, const void *C, const float *D,
                    const float *initial_state, const int32_t *cu_seqlens, void *y,
                    float *final_state, void *workspace) {
  const bool varlen = p->num_seqs > 0;
  char *ws = static_cast<char *>(workspace);
  ssd::Args a{};
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.h0 = initial_state;
  a.y = y;
  a.hT = final_state;
  a.cu = cu_seqlens;
  a.plan = reinterpret_cast<int32_t *>(ws + L.plan);
  a.cs = reinterpret_cast<float *>(ws + L.cs);
  a.states = reinterpret_cast<float *>(ws + L.states);
  a.cb = ws + L.cb;
  a.zeros = ws + L.zeros;
  a.bt = L.path == kMfmaChain ? ws + L.bt : nullptr;
  a.sync = reinterpret_cast<int32_t *>(ws + L.sync);
  a.inc = reinterpret_cast<float *>(ws + L.inc);
  a.agg = L.agg < L.total ? reinterpret_cast<float *>(ws + L.agg) : nullptr;
  a.nsync = (int32_t)L.nzero;
  a.batch = p->batch;
  a.L = p->seqlen;
  a.H = p->nheads;
  a.P = p->headdim;
  a.N = p->dstate;
  a.G = p->ngroups;
  a.Q = p->chunk_size;
  a.nseq = varlen ? p->num_seqs : p->batch;
  a.varlen = varlen ? 1 : 0;
  a.nc_per = varlen ? 0 : (p->seqlen + p->chunk_size - 1) / p->chunk_size;
  a.nc_max = (int32_t)L.nc_max;
  a.heads_per_group = p->nheads / p->ngroups;
  a.rec_off = (int32_t)L.rec_off;
  a.order_off = (int32_t)(L.rec_off + 4 * L.nc_max);
  a.nseg_off = varlen ? 3 + p->num_seqs : 0;
  a.seg = L.path == kMfmaChain ? L.seg : 1;
  a.nrange = L.path == kMfmaChain ? ssd::chain_ranges(a, device_compute_units()) : 0;
  a.gqueue = L.path == kMfmaChain && ssd::chain_group_queues(a) ? 1 : 0;
  return a;
}

// Sequences without tokens get no chunk workgroup on the chain path; their
// final states (initial state or zeros) come from a separate small pass.
// Only varlen problems and empty dense batches can have such sequences.
bool chain_needs_empty_pass(const ssd::Args &a) {
  return a.hT != nullptr && (a.varlen || a.L == 0);
}

struct StageNames {
  int count;
  const char *name[SSD_MAX_STAGES];
};

StageNames stage_names(const ssd::Args &a, const Layout &L, bool) {
  StageNames n{};
  if (a.varlen) n.name[n.count++] = "plan";
  if (L.path == kF32Seq) {
    n.name[n.count++] = "ssd_f32seq";
    return n;
  }
  if (L.path == kMfmaFused) {
    if (a.nc_max > 0) n.name[n.count++] = "chunk_cb";
    n.name[n.count++] = "ssd_fused";
    return n;
  }
  if (L.path == kMfmaChain) {
    if (a.nc_max > 0) {
      n.name[n.count++] = "chunk_cb";
      n.name[n.count++] = "ssd_chain";
    }
    if (chain_needs_empty_pass(a)) n.name[n.count++] = "final_of_empty";
    return n;
  }
  if (a.nc_max > 0) {
    n.name[n.count++] = "chunk_cumsum";
    n.name[n.count++] = "chunk_state";
  }
  n.name[n.count++] = "state_passing";
  if (a.nc_max > 0) {
    if (L.mfma) n.name[n.count++] = "chunk_cb";
    n.name[n.count++] = "chunk_scan";
  }
  return n;
}

// Enqueue the whole pass; with `ev` non-null, record ev[0] before the first
// kernel and ev[k+1] after stage k (for per-kernel timing).
ssd_status enqueue(const ssd::Args &a, const Layout &L, bool bf, hipStream_t s,
                   hipEvent_t *ev) {
  int k = 0;
  auto mark = [&]() -> bool {
    return ev == nullptr || hipEventRecord(ev[k++], s) == hipSuccess;
  };
#define SSD_LAUNCH(call, name)                                                       \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess)                                                            \
      return fail(SSD_ERR_HIP, "%s launch failed: %s", name, hipGetErrorString(e_)); \
    if (!mark()) return fail(SSD_ERR_HIP, "hipEventRecord failed after %s", name);   \
  } while (0)
  if (!mark()) return fail(SSD_ERR_HIP, "hipEventRecord failed");
  if (a.varlen) SSD_LAUNCH(ssd::launch_plan(a, s), "plan");
  if (L.path == kF32Seq) {
    SSD_LAUNCH(ssd::launch_f32seq(a, s), "ssd_f32seq");
    return SSD_OK;
  }
  if (L.path == kMfmaFused) {
    if (a.nc_max > 0) SSD_LAUNCH(ssd::launch_chunk_cb(a, a.cb, s), "chunk_cb");
    SSD_LAUNCH(ssd::launch_fused(a, a.cb, a.zeros, s), "ssd_fused");
    return SSD_OK;
  }
  if (L.path == kMfmaChain) {
    if (a.nc_max > 0) {
      SSD_LAUNCH(ssd::launch_chunk_cb(a, a.cb, s), "chunk_cb");
      SSD_LAUNCH(ssd::launch_chain(a, a.cb, a.bt, s), "ssd_chain");
    }
    if (chain_needs_empty_pass(a))
      SSD_LAUNCH(ssd::launch_final_of_empty(a, s), "final_of_empty");
    return SSD_OK;
  }
  if (a.nc_max > 0) {
    SSD_LAUNCH(ssd::launch_chunk_cumsum(a, bf, s), "chunk_cumsum");
    if (L.mfma)
      SSD_LAUNCH(ssd::launch_chunk_state_mfma(a, s), "chunk_state");
    else
      SSD_LAUNCH(ssd::launch_chunk_state_generic(a, bf, s), "chunk_state");
  }
  SSD_LAUNCH(ssd::launch_state_passing(a, s), "state_passing");
  if (a.nc_max > 0) {
    if (L.mfma) {
      SSD_LAUNCH(ssd::launch_chunk_cb(a, a.cb, s), "chunk_cb");
      SSD_LAUNCH(ssd::launch_chunk_scan_mfma(a, a.cb, s), "chunk_scan");
    } else {
      SSD_LAUNCH(ssd::launch_chunk_scan_generic(a, bf, s), "chunk_scan");
    }
  }
#undef SSD_LAUNCH
  return SSD_OK;
}

// ---- backward pass -----------------------------------------------------------
// Workspace: the per-step forward layout (plan, cs, per-chunk states), then
// the recomputed final states, the per-chunk gradient states, the per-chunk
// partials of dA and dD, and bf16 transposed copies of the entering and
// gradient states.
struct BwdLayout {
  ssd_problem fp;   // the problem with the per-step flag: whose layout comes first
  Layout F;
  size_t final_states, gst, dA_part, dD_part, hinT, gT, total;
};

BwdLayout make_bwd_layout(const ssd_problem &p) {
  BwdLayout B{};
  B.fp = p;
  B.fp.flags = SSD_FLAG_UNFUSED;
  B.F = make_layout(B.fp);
  const int64_t nseq = p.num_seqs > 0 ? p.num_seqs : p.batch;
  const size_t PN = (size_t)p.headdim * p.dstate;
  size_t off = B.F.total;
  B.final_states = off;
  off = round_up(off + (size_t)nseq * p.nheads * PN * sizeof(float), kAlign);
  B.gst = off;
  off = round_up(off + (size_t)B.F.nc_max * p.nheads * PN * sizeof(float), kAlign);
  B.dA_part = off;
  off = round_up(off + (size_t)B.F.nc_max * p.nheads * sizeof(float), kAlign);
  B.dD_part = off;
  off = round_up(off + (size_t)B.F.nc_max * p.nheads * sizeof(float), kAlign);
  B.hinT = off;
  off = round_up(off + (size_t)B.F.nc_max * p.nheads * PN * 2, kAlign);
  B.gT = off;
  off = round_up(off + (size_t)B.F.nc_max * p.nheads * PN * 2, kAlign);
  B.total = off;
  return B;
}

ssd_status check_bwd_problem(const ssd_problem *p) {
  ssd_status st = ssd_validate(p);
  if (st != SSD_OK) return st;
  if (p->flags != 0)
    return fail(SSD_ERR_INVALID_ARG, "the backward pass takes no flags (0x%x)", p->flags);
  if (p->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "the backward pass runs bf16 problems only");
  ssd::Args a{};
  a.P = p->headdim;
  a.N = p->dstate;
  a.Q = p->chunk_size;
  if (!ssd::bwd_supports(a))
    return fail(SSD_ERR_UNSUPPORTED,
                "the backward pass needs headdim 64, dstate 64 or 128 and chunk_size 128 or "
                "256 (got %d, %d, %d)", p->headdim, p->dstate, p->chunk_size);
  if ((int64_t)make_bwd_layout(*p).F.nc_max * p->ngroups * (p->chunk_size / ssd::kBwdRows) >
      INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "problem too large for one launch");
  return SSD_OK;
}

const char *const kBwdStages[] = {"plan", "chunk_cumsum", "chunk_state", "state_passing",
                                  "chunk_dstate", "state_passing_bwd", "bwd_cbt", "bwd_dx",
                                  "bwd_dbc", "bwd_reduce"};

// Enqueue the backward pass; with `ev` non-null, record ev[0] first and one
// event after each stage that runs (names appended to `names`).
ssd_status enqueue_bwd(const ssd::BwdArgs &b, hipStream_t s, hipEvent_t *ev,
                       const char **names, int *count) {
  int k = 0, n = 0;
  auto mark = [&](const char *name) -> bool {
    if (names) names[n] = name;
    ++n;
    return ev == nullptr || hipEventRecord(ev[k++], s) == hipSuccess;
  };
  if (ev && hipEventRecord(ev[k++], s) != hipSuccess)
    return fail(SSD_ERR_HIP, "hipEventRecord failed");
#define SSD_BLAUNCH(call, name)                                                      \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess)                                                            \
      return fail(SSD_ERR_HIP, "%s launch failed: %s", name, hipGetErrorString(e_)); \
    if (!mark(name)) return fail(SSD_ERR_HIP, "hipEventRecord failed after %s", name); \
  } while (0)
  const ssd::Args &a = b.f;
  if (a.varlen) SSD_BLAUNCH(ssd::launch_plan(a, s), kBwdStages[0]);
  if (a.nc_max > 0) {
    SSD_BLAUNCH(ssd::launch_chunk_cumsum(a, true, s), kBwdStages[1]);
    SSD_BLAUNCH(ssd::launch_chunk_state_mfma(a, s), kBwdStages[2]);
  }
  SSD_BLAUNCH(ssd::launch_state_passing(a, s), kBwdStages[3]);
  if (a.nc_max > 0) {
    ssd::Args d = a;  // dstate: x -> dy, B -> C, output -> gst
    d.x = b.dy;
    d.B = a.C;
    d.states = b.gst;
    SSD_BLAUNCH(ssd::launch_chunk_dstate_mfma(d, s), kBwdStages[4]);
  }
  SSD_BLAUNCH(ssd::launch_state_passing_bwd(b, s), kBwdStages[5]);
  if (a.nc_max > 0) {
    SSD_BLAUNCH(ssd::launch_bwd_cbt(b, s), kBwdStages[6]);
    SSD_BLAUNCH(ssd::launch_bwd_dx(b, s), kBwdStages[7]);
    SSD_BLAUNCH(ssd::launch_bwd_dbc(b, s), kBwdStages[8]);
  }
  SSD_BLAUNCH(ssd::launch_bwd_reduce(b, s), kBwdStages[9]);
#undef SSD_BLAUNCH
  if (count) *count = n;
  return SSD_OK;
}

ssd_status prepare_bwd(const ssd_problem *p, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D,
                       const float *initial_state, const int32_t *cu_seqlens,
                       const void *dy, const float *dfinal_state, void *dx, void *ddt,
                       float *dA, void *dB, void *dC, float *dD, float *dinitial_state,
                       void *workspace, size_t workspace_bytes, ssd::BwdArgs *out) {
  g_detail.clear();
  ssd_status st = check_bwd_problem(p);
  if (st != SSD_OK) return st;
  const bool varlen = p->num_seqs > 0;
  const int64_t tokens = (int64_t)p->batch * p->seqlen;
  if (!A || !dA) return fail(SSD_ERR_INVALID_ARG, "A and dA must be non-NULL");
  if (tokens > 0 && (!x || !dt || !B || !C || !dy || !dx || !dB || !dC))
    return fail(SSD_ERR_INVALID_ARG, "x, dt, B, C, dy, dx, dB and dC must be non-NULL");
  if (varlen && !cu_seqlens) return fail(SSD_ERR_INVALID_ARG, "varlen needs cu_seqlens");
  if (!varlen && cu_seqlens)
    return fail(SSD_ERR_INVALID_ARG, "cu_seqlens given but num_seqs is 0");
  if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(dy) || !aligned16(dx) ||
      !aligned16(dB) || !aligned16(dC) || !aligned16(initial_state) ||
      !aligned16(dfinal_state) || !aligned16(dinitial_state))
    return fail(SSD_ERR_INVALID_ARG, "x, B, C, dy, dx, dB, dC and the states must be "
                "16-byte aligned");
  const BwdLayout L = make_bwd_layout(*p);
  if (!workspace || ((uintptr_t)workspace % kAlign) != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                L.total);
  char *ws = static_cast<char *>(workspace);
  ssd::BwdArgs b{};
  b.f = make_args(&L.fp, L.F, x, dt, A, B, C, D, initial_state, cu_seqlens, nullptr,
                  reinterpret_cast<float *>(ws + L.final_states), workspace);
  b.dy = dy;
  b.dhT = dfinal_state;
  b.gst = reinterpret_cast<float *>(ws + L.gst);
  b.dx = dx;
  b.ddt = ddt;
  b.dB = dB;
  b.dC = dC;
  b.dh0 = dinitial_state;
  b.dA_part = reinterpret_cast<float *>(ws + L.dA_part);
  b.dD_part = reinterpret_cast<float *>(ws + L.dD_part);
  b.dA = dA;
  b.dD = dD;
  b.hinT = reinterpret_cast<ssd::bf16 *>(ws + L.hinT);
  b.gT = reinterpret_cast<ssd::bf16 *>(ws + L.gT);
  *out = b;
  return SSD_OK;
}

// ---- allocation-free entry point ------------------------------------------------
// The workspace of ssd_forward_noalloc: a file-scope device array (one copy on
// every GPU the library runs on, held until the process ends). In host code
// `scratch` names a host-side stand-in, not device memory, so kernels are
// given the device address looked up once per device below.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's `scratch`, looked up on the first call on
// the device (with that device current) and kept; nullptr on failure.
void *scratch_for_current_device(int *dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(SSD_ERR_HIP, "hipGetDevice failed or device index %d above %d", dev, kMaxDevices - 1);
    return nullptr;
  }
  *dev_out = dev;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void *q = nullptr;
  const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
  if (e != hipSuccess || q == nullptr) {
    fail(SSD_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
         hipGetErrorString(e));
    return nullptr;
  }
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" {

const char *ssd_status_string(ssd_status s) {
  switch (s) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported problem";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *ssd_last_error_detail(void) { return g_detail.c_str(); }

ssd_status ssd_validate(const ssd_problem *p) {
  g_detail.clear();
  if (!p) return fail(SSD_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1 || p->seqlen < 0 || p->nheads < 1 || p->headdim < 1 ||
      p->dstate < 1 || p->ngroups < 1 || p->chunk_size < 1 || p->num_seqs < 0)
    return fail(SSD_ERR_INVALID_ARG,
                "sizes must be positive (batch %d seqlen %d nheads %d headdim %d "
                "dstate %d ngroups %d chunk_size %d num_seqs %d)",
                p->batch, p->seqlen, p->nheads, p->headdim, p->dstate, p->ngroups,
                p->chunk_size, p->num_seqs);
  if (p->nheads % p->ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "nheads %d not divisible by ngroups %d",
                p->nheads, p->ngroups);
  if (p->num_seqs > 0 && p->batch != 1)
    return fail(SSD_ERR_INVALID_ARG, "varlen (num_seqs %d) needs batch == 1, got %d",
                p->num_seqs, p->batch);
  if (p->flags & ~(SSD_FLAG_GENERIC_KERNELS | SSD_FLAG_UNFUSED | SSD_FLAG_PER_SEQUENCE))
    return fail(SSD_ERR_INVALID_ARG, "unknown flags 0x%x", p->flags);
  if (p->dtype != SSD_DTYPE_F32 && p->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "dtype %d not supported", p->dtype);
  if (p->headdim != 16 && p->headdim != 32 && p->headdim != 64 && p->headdim != 128)
    return fail(SSD_ERR_UNSUPPORTED, "headdim %d not in {16, 32, 64, 128}", p->headdim);
  if (p->dstate % 16 != 0 || p->dstate > 256)
    return fail(SSD_ERR_UNSUPPORTED, "dstate %d not a multiple of 16 in [16, 256]", p->dstate);
  if (p->chunk_size != 64 && p->chunk_size != 128 && p->chunk_size != 256)
    return fail(SSD_ERR_UNSUPPORTED, "chunk_size %d not in {64, 128, 256}", p->chunk_size);
  if (p->nheads > 65535)
    return fail(SSD_ERR_UNSUPPORTED, "nheads %d above 65535", p->nheads);
  const int64_t tokens = (int64_t)p->batch * p->seqlen;
  if (tokens > INT32_MAX / 2)
    return fail(SSD_ERR_UNSUPPORTED, "%lld tokens exceed the int32 token index",
                (long long)tokens);
  const int64_t nseq = p->num_seqs > 0 ? p->num_seqs : p->batch;
  const int64_t sp_blocks = (int64_t)((p->headdim * p->dstate / 4 + 255) / 256) * p->nheads * nseq;
  const Layout L = make_layout(*p);
  if (sp_blocks > INT32_MAX || L.nc_max * 5 + L.rec_off > INT32_MAX ||
      L.nc_max * p->nheads > INT32_MAX || L.nsync > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "problem too large for 32-bit grid indexing");
  return SSD_OK;
}

ssd_status ssd_validate_cu_seqlens(const ssd_problem *p, const int32_t *cu) {
  ssd_status st = ssd_validate(p);
  if (st != SSD_OK) return st;
  if (p->num_seqs <= 0) return fail(SSD_ERR_INVALID_ARG, "problem is not varlen (num_seqs 0)");
  if (!cu) return fail(SSD_ERR_INVALID_ARG, "cu_seqlens is NULL");
  // the same checks the device plan kernel applies (ssd::seq_chunk_count,
  // ssd::stream_ends_ok), with a message naming the first offending entry
  if (cu[0] != 0) return fail(SSD_ERR_INVALID_ARG, "cu_seqlens[0] = %d, must be 0", cu[0]);
  int64_t chunks = 0;
  for (int s = 0; s < p->num_seqs; ++s) {
    const int n = ssd::seq_chunk_count(cu[s], cu[s + 1], p->seqlen, p->chunk_size);
    if (n < 0)
      return fail(SSD_ERR_INVALID_ARG,
                  "cu_seqlens[%d..%d] = (%d, %d) is not a sequence of the %d tokens", s, s + 1,
                  cu[s], cu[s + 1], p->seqlen);
    chunks += n;
  }
  if (!ssd::stream_ends_ok(cu[0], cu[p->num_seqs], p->seqlen))
    return fail(SSD_ERR_INVALID_ARG, "cu_seqlens[%d] = %d, must equal seqlen %d",
                p->num_seqs, cu[p->num_seqs], p->seqlen);
  if (chunks > make_layout(*p).nc_max)  // cannot happen once the checks above pass
    return fail(SSD_ERR_INVALID_ARG, "cu_seqlens give %lld chunks, more than the layout's %lld",
                (long long)chunks, (long long)make_layout(*p).nc_max);
  return SSD_OK;
}

ssd_status ssd_workspace_size(const ssd_problem *p, size_t *bytes) {
  ssd_status st = ssd_validate(p);
  if (st != SSD_OK) return st;
  if (!bytes) return fail(SSD_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_layout(*p).total;
  return SSD_OK;
}

ssd_status ssd_get_workspace_layout(const ssd_problem *p, ssd_workspace_layout *out) {
  ssd_status st = ssd_validate(p);
  if (st != SSD_OK) return st;
  if (!out) return fail(SSD_ERR_INVALID_ARG, "layout is NULL");
  const Layout L = make_layout(*p);
  out->chunk_cumsum = L.cs;
  out->chunk_states = L.states;
  out->chunk_table = L.plan;
  out->chunk_records = L.rec_off;
  out->max_chunks = L.nc_max;
  out->chain_sync = L.nsync ? L.sync : 0;
  out->chain_sync_words = L.nsync;
  out->chain_chunks_per_unit = 0;
  out->chain_ranges = 0;
  if (L.nsync) {
    ssd::Args a{};
    a.N = p->dstate;
    a.H = p->nheads;
    a.varlen = p->num_seqs > 0 ? 1 : 0;
    a.nseq = a.varlen ? p->num_seqs : p->batch;
    a.nc_per = a.varlen ? 0 : (p->seqlen + p->chunk_size - 1) / p->chunk_size;
    a.nc_max = (int32_t)L.nc_max;
    a.seg = ssd::chain_segment(a);
    // balanced ranges walk whole sequences of chunks
    out->chain_ranges = ssd::chain_ranges(a, device_compute_units());
    out->chain_chunks_per_unit = out->chain_ranges > 0 ? a.nc_per : a.seg;
  }
  return SSD_OK;
}

ssd_status ssd_forward(const ssd_problem *p, const void *x, const void *dt,
                       const float *A, const void *B, const void *C, const float *D,
                       const float *initial_state, const int32_t *cu_seqlens, void *y,
                       float *final_state, void *workspace, size_t workspace_bytes,
                       void *stream) {
  ssd_status st = check_args(p, x, dt, A, B, C, cu_seqlens, y, initial_state, final_state,
                             workspace, workspace_bytes);
  if (st != SSD_OK) return st;
  const Layout L = make_layout(*p);
  const ssd::Args a = make_args(p, L, x, dt, A, B, C, D, initial_state, cu_seqlens, y,
                                final_state, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return enqueue(a, L, p->dtype == SSD_DTYPE_BF16, s, nullptr);
}

ssd_status ssd_forward_noalloc(const ssd_problem *p, const void *x, const void *dt,
                               const float *A, const void *B, const void *C, const float *D,
                               const float *initial_state, const int32_t *cu_seqlens, void *y,
                               float *final_state, void *stream) {
  g_detail.clear();
  ssd_status st = ssd_validate(p);
  if (st != SSD_OK) return st;
  // the compact chained layout when the look-back slots would not fit
  Layout L = make_layout(*p);
  const bool look = L.total <= kScratchBytes;
  if (!look) L = make_layout(*p, false);
  if (L.total > kScratchBytes)
    return fail(SSD_ERR_WORKSPACE,
                "the problem needs %zu bytes of workspace; the allocation-free entry point has "
                "a fixed %zu-byte scratch area (call ssd_forward with a workspace instead)",
                L.total, kScratchBytes);
  int dev = -1;
  void *ws = scratch_for_current_device(&dev);
  if (!ws) return SSD_ERR_HIP;
  st = check_args(p, x, dt, A, B, C, cu_seqlens, y, initial_state, final_state, ws,
                  kScratchBytes, look);
  if (st != SSD_OK) return st;
  const ssd::Args a = make_args(p, L, x, dt, A, B, C, D, initial_state, cu_seqlens, y,
                                final_state, ws);
  return enqueue(a, L, p->dtype == SSD_DTYPE_BF16, static_cast<hipStream_t>(stream), nullptr);
}

ssd_status ssd_forward_dt_softplus(const ssd_problem *p, const void *x, const void *dt_raw,
                                   const float *dt_bias, const float *A, const void *B,
                                   const void *C, const float *D, const float *initial_state,
                                   const int32_t *cu_seqlens, void *y, float *final_state,
                                   void *workspace, size_t workspace_bytes, void *stream) {
  ssd_status st = check_args(p, x, dt_raw, A, B, C, cu_seqlens, y, initial_state, final_state,
                             workspace, workspace_bytes);
  if (st != SSD_OK) return st;
  const Layout L = make_layout(*p);
  ssd::Args a = make_args(p, L, x, dt_raw, A, B, C, D, initial_state, cu_seqlens, y,
                          final_state, workspace);
  a.dt_softplus = 1;
  a.dt_bias = dt_bias;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return enqueue(a, L, p->dtype == SSD_DTYPE_BF16, s, nullptr);
}

ssd_status ssd_forward_timed(const ssd_problem *p, const void *x, const void *dt,
                             const float *A, const void *B, const void *C, const float *D,
                             const float *initial_state, const int32_t *cu_seqlens,
                             void *y, float *final_state, void *workspace,
                             size_t workspace_bytes, void *stream, int32_t iterations,
                             ssd_stage_times *times) {
  if (iterations < 1 || !times)
    return fail(SSD_ERR_INVALID_ARG, "iterations must be >= 1 and times non-NULL");
  // Validate by a dry run of the argument checks of ssd_forward.
  ssd_status st = check_args(p, x, dt, A, B, C, cu_seqlens, y, initial_state, final_state,
                             workspace, workspace_bytes);
  if (st != SSD_OK) return st;
  const Layout L = make_layout(*p);
  ssd::Args a = make_args(p, L, x, dt, A, B, C, D, initial_state, cu_seqlens, y, final_state,
                          workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = p->dtype == SSD_DTYPE_BF16;
  StageNames names = stage_names(a, L, bf);
  const int ns = names.count;
  std::vector<hipEvent_t> ev((size_t)iterations * (ns + 1));
  for (auto &e : ev)
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto &f : ev) if (f) (void)hipEventDestroy(f);
      return fail(SSD_ERR_HIP, "hipEventCreate failed");
    }
  ssd_status rc = SSD_OK;
  for (int it = 0; it < iterations && rc == SSD_OK; ++it)
    rc = enqueue(a, L, bf, s, &ev[(size_t)it * (ns + 1)]);
  if (rc == SSD_OK && hipStreamSynchronize(s) != hipSuccess)
    rc = fail(SSD_ERR_HIP, "stream synchronisation failed");
  if (rc == SSD_OK) {
    memset(times, 0, sizeof(*times));
    times->num_stages = ns;
    for (int k = 0; k < ns; ++k) snprintf(times->names[k], sizeof(times->names[k]), "%s", names.name[k]);
    for (int it = 0; it < iterations; ++it) {
      hipEvent_t *e = &ev[(size_t)it * (ns + 1)];
      for (int k = 0; k < ns; ++k) {
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, e[k], e[k + 1]);
        times->ms[k] += ms;
      }
    }
    float tot = 0.f;
    (void)hipEventElapsedTime(&tot, ev[0], ev[ev.size() - 1]);
    times->total_ms = tot;
    times->iterations = iterations;
  }
  for (auto &e : ev) (void)hipEventDestroy(e);
  return rc;
}

ssd_status ssd_step(const ssd_problem *p, const void *x, const void *dt, const float *A,
                    const void *B, const void *C, const float *D, float *state, void *y,
                    void *stream) {
  g_detail.clear();
  if (!p) return fail(SSD_ERR_INVALID_ARG, "problem is NULL");
  if (p->seqlen != 1)
    return fail(SSD_ERR_INVALID_ARG, "a step advances one token: seqlen must be 1, got %d",
                p->seqlen);
  if (p->num_seqs != 0)
    return fail(SSD_ERR_INVALID_ARG, "a step takes a dense batch: num_seqs must be 0, got %d",
                p->num_seqs);
  if (p->batch < 0 || p->nheads < 1 || p->headdim < 1 || p->dstate < 1 || p->ngroups < 1)
    return fail(SSD_ERR_INVALID_ARG,
                "sizes must be positive (batch %d >= 0, nheads %d headdim %d dstate %d "
                "ngroups %d)", p->batch, p->nheads, p->headdim, p->dstate, p->ngroups);
  if (p->nheads % p->ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "nheads %d not divisible by ngroups %d", p->nheads,
                p->ngroups);
  if (p->flags != 0) return fail(SSD_ERR_INVALID_ARG, "a step takes no flags (0x%x)", p->flags);
  if (p->dtype != SSD_DTYPE_F32 && p->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "dtype %d not supported", p->dtype);
  if (p->headdim != 16 && p->headdim != 32 && p->headdim != 64 && p->headdim != 128)
    return fail(SSD_ERR_UNSUPPORTED, "headdim %d not in {16, 32, 64, 128}", p->headdim);
  if (p->dstate % 16 != 0 || p->dstate > 256)
    return fail(SSD_ERR_UNSUPPORTED, "dstate %d not a multiple of 16 in [16, 256]", p->dstate);
  ssd::StepArgs a{};
  a.rows = (int64_t)p->batch * p->nheads * p->headdim;
  a.H = p->nheads;
  a.N = p->dstate;
  a.G = p->ngroups;
  a.heads_per_group = p->nheads / p->ngroups;
  a.p_shift = __builtin_ctz((unsigned)p->headdim);
  if ((int64_t)p->batch * p->nheads > INT32_MAX || ssd::step_blocks(a) > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "batch %d too large for one launch", p->batch);
  if (p->batch == 0) return SSD_OK;
  if (!x || !dt || !A || !B || !C || !state || !y)
    return fail(SSD_ERR_INVALID_ARG, "x, dt, A, B, C, state and y must be non-NULL");
  if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) || !aligned16(state))
    return fail(SSD_ERR_INVALID_ARG, "x, B, C, y and state must be 16-byte aligned");
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.state = state;
  a.y = y;
  if (ssd::launch_step(a, p->dtype == SSD_DTYPE_BF16, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return fail(SSD_ERR_HIP, "step kernel launch failed");
  return SSD_OK;
}

ssd_status ssd_selective_scan(const ssd_scan_problem *p, const void *x, const void *delta,
                              const float *A, const void *B, const void *C, const float *D,
                              const float *initial_state, void *y, float *final_state,
                              void *stream) {
  g_detail.clear();
  if (!p) return fail(SSD_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 0 || p->seqlen < 0 || p->dim < 1)
    return fail(SSD_ERR_INVALID_ARG, "sizes must be valid (batch %d >= 0, seqlen %d >= 0, dim %d >= 1)",
                p->batch, p->seqlen, p->dim);
  if (p->flags != 0) return fail(SSD_ERR_INVALID_ARG, "the scan takes no flags (0x%x)", p->flags);
  if (p->dtype != SSD_DTYPE_F32 && p->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "dtype %d not supported", p->dtype);
  if (p->dstate != 16 && p->dstate != 32 && p->dstate != 64 && p->dstate != 128 &&
      p->dstate != 256)
    return fail(SSD_ERR_UNSUPPORTED, "dstate %d not in {16, 32, 64, 128, 256}", p->dstate);
  if (p->dim % 64 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "dim %d is not a multiple of 64", p->dim);
  if (p->batch > 65535) return fail(SSD_ERR_UNSUPPORTED, "batch %d above 65535", p->batch);
  if (p->batch == 0) return SSD_OK;
  const bool tokens = p->seqlen > 0;
  if (!A || (tokens && (!x || !delta || !B || !C || !y)))
    return fail(SSD_ERR_INVALID_ARG, "A, and with tokens x, delta, B, C and y, must be non-NULL");
  if (!aligned16(x) || !aligned16(delta) || !aligned16(B) || !aligned16(C) || !aligned16(y) ||
      !aligned16(A) || !aligned16(initial_state) || !aligned16(final_state))
    return fail(SSD_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  ssd::ScanArgs a{};
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.h0 = initial_state;
  a.y = y;
  a.hT = final_state;
  a.batch = p->batch;
  a.L = p->seqlen;
  a.dim = p->dim;
  a.N = p->dstate;
  if (ssd::launch_selective_scan(a, p->dtype == SSD_DTYPE_BF16, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return fail(SSD_ERR_HIP, "selective scan kernel launch failed");
  return SSD_OK;
}

ssd_status ssd_backward_workspace_size(const ssd_problem *p, size_t *bytes) {
  g_detail.clear();
  ssd_status st = check_bwd_problem(p);
  if (st != SSD_OK) return st;
  if (!bytes) return fail(SSD_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_bwd_layout(*p).total;
  return SSD_OK;
}

ssd_status ssd_backward(const ssd_problem *p, const void *x, const void *dt, const float *A,
                        const void *B, const void *C, const float *D,
                        const float *initial_state, const int32_t *cu_seqlens,
                        const void *dy, const float *dfinal_state, void *dx, void *ddt,
                        float *dA, void *dB, void *dC, float *dD, float *dinitial_state,
                        void *workspace, size_t workspace_bytes, void *stream) {
  ssd::BwdArgs b;
  ssd_status st = prepare_bwd(p, x, dt, A, B, C, D, initial_state, cu_seqlens, dy,
                              dfinal_state, dx, ddt, dA, dB, dC, dD, dinitial_state, workspace,
                              workspace_bytes, &b);
  if (st != SSD_OK) return st;
  return enqueue_bwd(b, static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr);
}

ssd_status ssd_backward_timed(const ssd_problem *p, const void *x, const void *dt,
                              const float *A, const void *B, const void *C, const float *D,
                              const float *initial_state, const int32_t *cu_seqlens,
                              const void *dy, const float *dfinal_state, void *dx, void *ddt,
                              float *dA, void *dB, void *dC, float *dD, float *dinitial_state,
                              void *workspace, size_t workspace_bytes, void *stream,
                              int32_t iterations, ssd_stage_times *times) {
  if (iterations < 1 || !times)
    return fail(SSD_ERR_INVALID_ARG, "iterations must be >= 1 and times non-NULL");
  ssd::BwdArgs b;
  ssd_status st = prepare_bwd(p, x, dt, A, B, C, D, initial_state, cu_seqlens, dy,
                              dfinal_state, dx, ddt, dA, dB, dC, dD, dinitial_state, workspace,
                              workspace_bytes, &b);
  if (st != SSD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  constexpr int kMax = (int)(sizeof(kBwdStages) / sizeof(kBwdStages[0]));  // stages of enqueue_bwd
  static_assert(kMax <= SSD_MAX_STAGES, "ssd_stage_times holds every backward stage");
  std::vector<hipEvent_t> ev((size_t)iterations * (kMax + 1), nullptr);
  for (auto &e : ev)
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto &f : ev) if (f) (void)hipEventDestroy(f);
      return fail(SSD_ERR_HIP, "hipEventCreate failed");
    }
  const char *names[kMax] = {};
  int ns = 0;
  ssd_status rc = SSD_OK;
  for (int it = 0; it < iterations && rc == SSD_OK; ++it)
    rc = enqueue_bwd(b, s, &ev[(size_t)it * (kMax + 1)], names, &ns);
  if (rc == SSD_OK && hipStreamSynchronize(s) != hipSuccess)
    rc = fail(SSD_ERR_HIP, "stream synchronisation failed");
  if (rc == SSD_OK) {
    memset(times, 0, sizeof(*times));
    times->num_stages = ns < SSD_MAX_STAGES ? ns : SSD_MAX_STAGES;
    for (int k = 0; k < times->num_stages; ++k)
      snprintf(times->names[k], sizeof(times->names[k]), "%s", names[k]);
    float tot = 0.f;
    for (int it = 0; it < iterations; ++it) {
      hipEvent_t *e = &ev[(size_t)it * (kMax + 1)];
      for (int k = 0; k < times->num_stages; ++k) {
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, e[k], e[k + 1]);
        times->ms[k] += ms;
      }
      float t = 0.f;
      (void)hipEventElapsedTime(&t, e[0], e[ns]);
      tot += t;
    }
    times->total_ms = tot;
    times->iterations = iterations;
  }
  for (auto &e : ev) (void)hipEventDestroy(e);
  return rc;
}

ssd_status ssd_conv1d_silu(const ssd_conv_problem *p, const void *xbc, const float *weight,
                           const float *bias, const void *history_in,
                           const int32_t *cu_seqlens, void *x, void *B, void *C,
                           void *history_out, void *stream) {
  g_detail.clear();
  if (!p) return fail(SSD_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 0 || p->seqlen < 0 || p->num_seqs < 0 || p->x_dim < 0 || p->bc_dim < 0)
    return fail(SSD_ERR_INVALID_ARG,
                "sizes must be non-negative (batch %d, seqlen %d, num_seqs %d, x_dim %d, "
                "bc_dim %d)", p->batch, p->seqlen, p->num_seqs, p->x_dim, p->bc_dim);
  if (p->flags != 0)
    return fail(SSD_ERR_INVALID_ARG, "the convolution takes no flags (0x%x)", p->flags);
  if (p->dtype != SSD_DTYPE_F32 && p->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "dtype %d not supported", p->dtype);
  if (p->width < 2 || p->width > 4)
    return fail(SSD_ERR_UNSUPPORTED, "width %d not in {2, 3, 4}", p->width);
  if (p->x_dim % 8 != 0 || p->bc_dim % 8 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "x_dim %d and bc_dim %d must be multiples of 8", p->x_dim,
                p->bc_dim);
  const int64_t ch = (int64_t)p->x_dim + 2 * (int64_t)p->bc_dim;
  if (ch < 8 || ch > INT32_MAX / 8)
    return fail(SSD_ERR_INVALID_ARG, "channel count %lld out of range",
                (long long)ch);
  const size_t esz = p->dtype == SSD_DTYPE_BF16 ? 2 : 4;
  if (p->in_stride < ch || ((size_t)p->in_stride * esz) % 16 != 0)
    return fail(SSD_ERR_INVALID_ARG,
                "in_stride %d must be >= the channel count %lld and a multiple of 16 bytes",
                p->in_stride, (long long)ch);
  const bool varlen = p->num_seqs > 0;
  if (varlen && p->batch != 1)
    return fail(SSD_ERR_INVALID_ARG, "packed sequences take batch 1, got %d", p->batch);
  if (varlen && !cu_seqlens)
    return fail(SSD_ERR_INVALID_ARG, "num_seqs > 0 needs cu_seqlens");
  const int64_t T = (int64_t)p->batch * p->seqlen;
  const int64_t nseq = varlen ? p->num_seqs : p->batch;
  const int64_t tiles = (T + ssd::kConvTile - 1) / ssd::kConvTile;
  if (T > INT32_MAX - ssd::kConvTile ||
      (tiles * (ch / 8) + ssd::kConvThreads - 1) / ssd::kConvThreads > INT32_MAX ||
      (nseq * (ch / 8) + ssd::kConvThreads - 1) / ssd::kConvThreads > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "%lld tokens x %lld channels too large for one launch",
                (long long)T, (long long)ch);
  if (nseq == 0 || (T == 0 && !history_out)) return SSD_OK;
  if (!weight) return fail(SSD_ERR_INVALID_ARG, "weight must be non-NULL");
  if (T > 0 && (!xbc || (p->x_dim > 0 && !x) || (p->bc_dim > 0 && (!B || !C))))
    return fail(SSD_ERR_INVALID_ARG, "xbc, and x, B, C for non-empty parts, must be non-NULL");
  if (!aligned16(xbc) || !aligned16(x) || !aligned16(B) || !aligned16(C) ||
      !aligned16(history_in) || !aligned16(history_out))
    return fail(SSD_ERR_INVALID_ARG, "xbc, x, B, C and the histories must be 16-byte aligned");
  ssd::ConvArgs a{};
  a.xbc = xbc;
  a.w = weight;
  a.bias = bias;
  a.hist_in = history_in;
  a.cu = varlen ? cu_seqlens : nullptr;
  a.x = x;
  a.B = B;
  a.C = C;
  a.hist_out = history_out;
  a.T = (int32_t)T;
  a.seqlen = p->seqlen;
  a.nseq = (int32_t)nseq;
  a.ch = (int32_t)ch;
  a.x_dim = p->x_dim;
  a.bc_dim = p->bc_dim;
  a.in_stride = p->in_stride;
  a.groups = (int32_t)(ch / 8);
  a.tiles = (int32_t)tiles;
  if (ssd::launch_conv(a, p->width, p->dtype == SSD_DTYPE_BF16,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(SSD_ERR_HIP, "convolution kernel launch failed");
  return SSD_OK;
}

}  // extern "C"
