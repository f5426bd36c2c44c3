// kda_api.cpp -- the C ABI of libkda.so (see include/kda.h).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_dev.h"
#include "kda_launch.h"

using namespace kda;

namespace {

thread_local std::string g_hip_msg;

struct Region {
  size_t off, size;
};

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Everything derived from a kda_problem after validation.
struct Plan {
  Shape s;
  int64_t NC = 0;
  size_t es = 0;  // bytes per act element
  // workspace regions
  Region chunks, seq_off, order, qn, kn, rq, rk, groups, grp_off, Tm, PT, eGT, INV, MqkT, dstates, dAl,
      ddt, Pg, Qg, bnd, hsaved;
  Region fWn, fKrT, fUvT, fQd, fMq, fEgt;  // production forward (from fwd_bytes on)
  Region fgroups, fgrp_off, fPg, fQg, fbnd;
  Region rWn, rKrT, rUvT, rQd, rMq;        // the same operands for the in-stream recompute
  size_t fwdp_bytes = 0;
  int64_t rows = 0;  // tokens * heads
  bool l2 = false;   // q, k L2-normalised inside the method
  size_t fwd_bytes = 0, bwd_bytes = 0;
};

int count_chunks(const kda_problem* p, int64_t* nc) {
  int64_t total = 0;
  if (p->cu_seqlens_host) {
    for (int n = 0; n < p->num_seqs; ++n) {
      int64_t len = (int64_t)p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n];
      total += (len + CH - 1) / CH;
    }
  } else {
    total = (int64_t)p->B * ((p->T + CH - 1) / CH);
  }
  *nc = total;
  return KDA_OK;
}

int64_t seq_chunks(const kda_problem* p, int n) {
  const int64_t len = p->cu_seqlens_host
                          ? (int64_t)p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n]
                          : (int64_t)p->T;
  return (len + CH - 1) / CH;
}

// Chunks per group of the state scans (backward and forward).  With few (sequence, head)
// units the serial chain over a sequence's chunks leaves most CUs idle, so sequences are
// split into groups (three passes: group maps side by side, the boundaries, the groups
// again): the smallest power-of-two group size, at least 4 chunks, that keeps the
// group-map pass within about 512 workgroups (two per CU).  Measured with one GPU on the
// single-sequence workload (16 units of 32 chunks: scan 0.122 ms unsplit, 0.069 with groups
// of 4, 0.080 with 8) and the long-context one (16 units of 2048 chunks: 2.20, 1.86, 1.66,
// 1.54 and 2.10 ms with groups of 16 to 256).  With many units the GPU is full without
// splitting; sequences of more than 128 chunks are then still cut into groups of 64.
// KDA_SCAN_GROUP=<chunks> overrides (0: never split).
int scan_group_size(const kda_problem* p, int N) {
  if (const char* env = std::getenv("KDA_SCAN_GROUP")) {
    const int v = std::atoi(env);
    if (v >= 0) return v;
  }
  int64_t mx = 0;
  for (int n = 0; n < N; ++n) mx = std::max(mx, seq_chunks(p, n));
  const int64_t units = (int64_t)N * p->H;
  if (units >= 256) return mx > 128 ? 64 : 0;
  for (int64_t gs = 4; gs < mx; gs *= 2) {
    int64_t ng = 0;
    for (int n = 0; n < N; ++n) ng += (seq_chunks(p, n) + gs - 1) / gs;
    if (ng * p->H * 2 <= 512) return (int)gs;
  }
  return 0;
}

// Whether prep runs the state scans itself (one workgroup per (sequence, head) unit at a
// time, walking its chunks).  The units, sorted by chunk count (longest first), are dealt
// to the resident workgroups in a snake; that is used when every sequence has at least
// one chunk, there are at least as many units as workgroups, and the busiest workgroup's
// chunk count stays within 10% of the mean (the train workload: 256 units of 64 chunks on
// 256 workgroups, exactly the mean; the varlen workload: 137 against 129).  Otherwise the
// separate per-chunk pass and scan kernels, which spread single chunks over the GPU, are
// better balanced.  KDA_PREPSCAN=0 / 1 forces the separate kernels / the fused ones (when
// every sequence has a chunk).
bool use_prepscan(const kda_problem* p, const Shape& s) {
  if (s.N < 1 || s.N > kMaxOrderSeqs) return false;
  std::vector<int> nck(s.N);
  for (int n = 0; n < s.N; ++n) {
    nck[n] = (int)seq_chunks(p, n);
    if (nck[n] < 1) return false;
  }
  if (const char* env = std::getenv("KDA_PREPSCAN")) {
    if (env[0] == '0') return false;
    if (env[0] == '1') return true;
  }
  int grid = 0;
  if (prepscan_grid(s, &grid) != hipSuccess || grid <= 0) return false;
  const int64_t units = (int64_t)s.N * s.H;
  if (units < grid) return false;
  std::vector<int> order(s.N);
  for (int n = 0; n < s.N; ++n) order[n] = n;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return nck[a] > nck[b]; });
  std::vector<int64_t> load(grid, 0);
  int64_t total = 0;
  for (int64_t pos = 0; pos < units; ++pos) {
    const int64_t k = pos / grid, r = pos % grid;
    const int64_t g = (k & 1) ? grid - 1 - r : r;
    load[g] += nck[order[pos / s.H]];
    total += nck[order[pos / s.H]];
  }
  const int64_t mx = *std::max_element(load.begin(), load.end());
  return (double)mx <= 1.1 * (double)total / grid;
}

int validate_problem(const kda_problem* p) {
  if (!p) return KDA_ERR_INVALID_ARGUMENT;
  if (p->B < 1 || p->T < 0 || p->H < 1 || p->K < 1 || p->V < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (p->chunk != 64) return KDA_ERR_UNSUPPORTED;
  if (p->gate_units != KDA_GATE_LN && p->gate_units != KDA_GATE_LOG2) return KDA_ERR_INVALID_ARGUMENT;
  if (p->qk_l2norm != 0 && p->qk_l2norm != 1) return KDA_ERR_INVALID_ARGUMENT;
  if (p->act_dtype != KDA_DTYPE_F32 && p->act_dtype != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
  if (p->K != p->V) return KDA_ERR_UNSUPPORTED;
  if (p->act_dtype == KDA_DTYPE_BF16 && p->K != 64 && p->K != 128) return KDA_ERR_UNSUPPORTED;
  if (p->act_dtype == KDA_DTYPE_F32 && p->K != 64) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)p->B * p->T >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
  // per-lane row offsets are formed on the 24-bit multiplier: a token row of fp32
  // (H * K * 4 bytes) must stay below 2^24 bytes
  if ((int64_t)p->H * p->K * 4 >= ((int64_t)1 << 24)) return KDA_ERR_UNSUPPORTED;
  const bool hv = p->cu_seqlens_host != nullptr, dv = p->cu_seqlens_dev != nullptr;
  if (hv != dv) return KDA_ERR_INVALID_ARGUMENT;
  if (hv) {
    if (p->B != 1 || p->num_seqs < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (p->cu_seqlens_host[0] != 0) return KDA_ERR_INVALID_ARGUMENT;
    for (int n = 0; n < p->num_seqs; ++n)
      if (p->cu_seqlens_host[n + 1] < p->cu_seqlens_host[n]) return KDA_ERR_INVALID_ARGUMENT;
    if (p->cu_seqlens_host[p->num_seqs] != p->T) return KDA_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)p->cu_seqlens_dev & 3) != 0) return KDA_ERR_INVALID_ARGUMENT;
  }
  // the kernels index (chunk, head) work items and (token, head) rows in 32 bits
  int64_t nc = 0;
  count_chunks(p, &nc);
  if (nc * p->H >= ((int64_t)1 << 31) || (int64_t)p->B * p->T * p->H >= ((int64_t)1 << 31))
    return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

int make_plan(const kda_problem* p, Plan* pl) {
  int st = validate_problem(p);
  if (st != KDA_OK) return st;
  Shape& s = pl->s;
  s.N = p->cu_seqlens_host ? p->num_seqs : p->B;
  s.H = p->H;
  s.D = p->K;
  s.T = p->T;
  s.bf16 = p->act_dtype == KDA_DTYPE_BF16;
  s.cu = p->cu_seqlens_dev;
  s.gu = p->gate_units == KDA_GATE_LOG2 ? 0.69314718055994531f : 1.f;
  s.qn = p->qk_l2norm == 1;
  count_chunks(p, &pl->NC);
  s.NC = pl->NC;
  s.gs = scan_group_size(p, s.N);
  s.NG = 0;
  for (int n = 0; n < s.N; ++n) {
    const int64_t nck = seq_chunks(p, n);
    s.NG += s.gs > 0 ? std::max<int64_t>(1, (nck + s.gs - 1) / s.gs) : 1;
  }
  pl->es = s.bf16 ? 2 : 4;
  const size_t NCH = (size_t)pl->NC * s.H;
  const size_t NGH = (size_t)s.NG * s.H;
  const size_t D = s.D;
  size_t off = 0;
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.size = bytes;
    off = align_up(off + bytes);
  };
  take(pl->chunks, (size_t)pl->NC * sizeof(ChunkInfo));
  take(pl->seq_off, ((size_t)s.N + 1) * sizeof(int));
  take(pl->order, (size_t)s.N * sizeof(int));  // sequences by chunk count (scans in prep)
  const size_t common = off;
  // the reference forward normalises q, k (qk_l2norm) into copies; kda_bwd and kda_fwd
  // normalise inside their kernels and do not use these regions
  pl->rows = (int64_t)p->B * p->T * p->H;
  pl->l2 = p->qk_l2norm == 1;
  const size_t l2 = pl->l2 ? 1 : 0;
  take(pl->qn, l2 * (size_t)pl->rows * D * pl->es);
  take(pl->kn, l2 * (size_t)pl->rows * D * pl->es);
  take(pl->rq, l2 * (size_t)pl->rows * 4);
  take(pl->rk, l2 * (size_t)pl->rows * 4);
  pl->fwd_bytes = off;
  off = common;
  take(pl->groups, (size_t)s.NG * sizeof(GroupInfo));
  take(pl->grp_off, ((size_t)s.N + 1) * sizeof(int));
  take(pl->Tm, NCH * D * D * pl->es);
  take(pl->PT, NCH * D * 64 * pl->es);
  take(pl->eGT, NCH * D * 4);
  take(pl->INV, NCH * 64 * 64 * pl->es);
  take(pl->MqkT, NCH * 64 * 64 * pl->es);
  take(pl->dstates, NCH * D * D * pl->es);
  take(pl->dAl, NCH * 4);
  take(pl->ddt, NCH * D * 4);
  const size_t split = s.gs > 0 ? 1 : 0;
  take(pl->Pg, split * NGH * D * D * pl->es);
  take(pl->Qg, split * NGH * D * D * 4);
  take(pl->bnd, split * NGH * D * D * 4);
  take(pl->hsaved, NCH * D * D * pl->es);
  // the forward's per-chunk operands for the state recompute (only without h_saved; the
  // recompute regions are the last ones)
  take(pl->rWn, NCH * 64 * D * pl->es);
  take(pl->rKrT, NCH * D * 64 * pl->es);
  take(pl->rUvT, NCH * D * 64 * pl->es);
  take(pl->rQd, NCH * 64 * D * pl->es);
  take(pl->rMq, NCH * 64 * 64 * pl->es);
  pl->bwd_bytes = off;
  // the production forward's per-chunk operands
  off = common;
  take(pl->fgroups, (size_t)s.NG * sizeof(GroupInfo));
  take(pl->fgrp_off, ((size_t)s.N + 1) * sizeof(int));
  take(pl->fPg, split * NGH * D * D * pl->es);
  take(pl->fQg, split * NGH * D * D * 4);
  take(pl->fbnd, split * NGH * D * D * 4);
  take(pl->fWn, NCH * 64 * D * pl->es);
  take(pl->fKrT, NCH * D * 64 * pl->es);
  take(pl->fUvT, NCH * D * 64 * pl->es);
  take(pl->fQd, NCH * 64 * D * pl->es);
  take(pl->fMq, NCH * 64 * 64 * pl->es);
  take(pl->fEgt, NCH * D * 4);
  pl->fwdp_bytes = std::max(off, pl->fwd_bytes);  // also enough for kda_fwd_ref
  return KDA_OK;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

// A device byte range [p, p + n); null or empty ranges never overlap anything.
struct Span {
  const void* p;
  size_t n;
};
bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}
// Outputs must not overlap inputs, each other or the workspace, and the workspace must
// not overlap inputs: the kernels read inputs while other workgroups write outputs.
bool aliased(const Span* in, int nin, const Span* out, int nout, const Span& ws) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(out[o], in[i])) return true;
    for (int j = o + 1; j < nout; ++j)
      if (overlap(out[o], out[j])) return true;
    if (overlap(out[o], ws)) return true;
  }
  for (int i = 0; i < nin; ++i)
    if (overlap(in[i], ws)) return true;
  return false;
}

// Byte sizes of the tensors of one call (kda.h gives the shapes).
struct Sizes {
  size_t act_k, act_v, f32_k, rowsf, heads, hk, state_n, state_c;
};
Sizes sizes_of(const kda_problem* p, const Plan& pl) {
  const size_t rows = (size_t)p->B * p->T * p->H;
  const size_t N = pl.s.N, KV = (size_t)p->K * p->V;
  Sizes z;
  z.act_k = rows * p->K * pl.es;
  z.act_v = rows * p->V * pl.es;
  z.f32_k = rows * p->K * 4;
  z.rowsf = rows * 4;
  z.heads = (size_t)p->H * 4;
  z.hk = (size_t)p->H * p->K * 4;
  z.state_n = N * p->H * KV * 4;
  z.state_c = (size_t)pl.NC * p->H * KV * pl.es;
  return z;
}

bool fwd_aliased(const kda_problem* p, const Plan& pl, const kda_fwd_io* io, const void* ws,
                 size_t ws_n) {
  const Sizes z = sizes_of(p, pl);
  const Span in[] = {{io->q, z.act_k}, {io->k, z.act_k}, {io->v, z.act_v}, {io->g_raw, z.f32_k},
                     {io->beta, z.rowsf}, {io->A_log, z.heads}, {io->h0, z.state_n},
                     {io->dt_bias, z.hk}};
  const Span out[] = {{io->o, z.act_v}, {io->ht, z.state_n}, {io->h_saved, z.state_c}};
  return aliased(in, 8, out, 3, Span{ws, ws_n});
}

bool bwd_aliased(const kda_problem* p, const Plan& pl, const kda_bwd_io* io, const void* ws,
                 size_t ws_n) {
  const Sizes z = sizes_of(p, pl);
  const Span in[] = {{io->q, z.act_k},      {io->k, z.act_k},       {io->v, z.act_v},
                     {io->g_raw, z.f32_k},  {io->beta, z.rowsf},    {io->A_log, z.heads},
                     {io->h0, z.state_n},   {io->dO, z.act_v},      {io->dht, z.state_n},
                     {io->h_saved, z.state_c}, {io->dt_bias, z.hk}};
  const Span out[] = {{io->dq, z.act_k},    {io->dk, z.act_k},      {io->dv, z.act_v},
                      {io->dg_raw, z.f32_k}, {io->dbeta, z.rowsf},  {io->dA_log, z.heads},
                      {io->dh0, z.state_n}, {io->dstates, z.state_c}, {io->ddt_bias, z.hk}};
  return aliased(in, 11, out, 9, Span{ws, ws_n});
}

// ---- optional per-stage timing
struct TimedLaunch {
  int stage;
  hipEvent_t a, b;
};
bool g_timing = false;
std::vector<TimedLaunch> g_events;
constexpr int kStages = 7;

template <typename F>
hipError_t timed(int stage, hipStream_t st, F&& launch) {
  if (!g_timing) return launch();
  TimedLaunch t{stage, nullptr, nullptr};
  auto drop = [&] {
    if (t.a) (void)hipEventDestroy(t.a);
    if (t.b) (void)hipEventDestroy(t.b);
  };
  // no system-scope release at the event: the launches it separates are on one stream and
  // the host reads the times only after hipEventSynchronize
  hipError_t e = hipEventCreateWithFlags(&t.a, hipEventDisableSystemFence);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&t.b, hipEventDisableSystemFence);
  if (e == hipSuccess) e = hipEventRecord(t.a, st);
  if (e != hipSuccess) {  // the launch is not made: the caller reports the error
    drop();
    return e;
  }
  e = launch();
  const hipError_t r = hipEventRecord(t.b, st);
  if (e == hipSuccess && r == hipSuccess) {
    g_events.push_back(t);
    return hipSuccess;
  }
  drop();
  return e != hipSuccess ? e : r;
}

int hip_fail(hipError_t e) {
  g_hip_msg = std::string("HIP error: ") + hipGetErrorName(e) + ": " + hipGetErrorString(e);
  return KDA_ERR_HIP;
}

}  // namespace

namespace kda {

hipError_t resident_blocks(const void* kernel, int threads, int* out) {
  struct Entry {
    int dev;
    const void* fn;
    int threads, blocks;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  // KDA_GRID_CAP=<n> caps the result (tests: a few workgroups walk many items)
  int cap = 0;
  if (const char* env = std::getenv("KDA_GRID_CAP")) cap = std::atoi(env);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int blocks = 0;
  {
    std::lock_guard<std::mutex> lk(mu);
    for (const Entry& x : cache)
      if (x.dev == dev && x.fn == kernel && x.threads == threads) blocks = x.blocks;
  }
  if (blocks == 0) {
    int ncu = 0, per = 0;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0);
    if (e != hipSuccess) return e;
    blocks = std::max(1, ncu * per);
    std::lock_guard<std::mutex> lk(mu);
    cache.push_back({dev, kernel, threads, blocks});
  }
  *out = cap > 0 && cap < blocks ? cap : blocks;
  return hipSuccess;
}

int bwd_workspace_need(const kda_problem* p, bool has_h_saved, size_t* bytes) {
  Plan pl;
  const int st = make_plan(p, &pl);
  if (st != KDA_OK) return st;
  *bytes = has_h_saved ? pl.hsaved.off : pl.bwd_bytes;
  return KDA_OK;
}

}  // namespace kda

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KDA_ERR_HIP: return g_hip_msg.empty() ? "HIP error" : g_hip_msg.c_str();
    case KDA_ERR_SCRATCH_TOO_SMALL:
      return "problem needs more scratch than kda_bwd_noalloc holds (KDA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int kda_num_chunks(const kda_problem* p, int64_t* nchunks) {
  if (!nchunks) return KDA_ERR_INVALID_ARGUMENT;
  int st = validate_problem(p);
  if (st != KDA_OK) return st;
  return count_chunks(p, nchunks);
}

int kda_workspace_size(const kda_problem* p, int which, size_t* bytes) {
  if (!bytes || (which != KDA_WS_BWD && which != KDA_WS_FWD && which != KDA_WS_FWD_REF))
    return KDA_ERR_INVALID_ARGUMENT;
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != KDA_OK) return st;
  *bytes = which == KDA_WS_BWD ? pl.bwd_bytes : which == KDA_WS_FWD ? pl.fwdp_bytes : pl.fwd_bytes;
  return KDA_OK;
}

int kda_fwd_ref(const kda_problem* p, const kda_fwd_io* io, void* workspace, size_t ws_bytes,
                void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != KDA_OK) return st;
  // per-token tensors may be NULL when there are no tokens (nothing reads them then)
  const bool tok = (int64_t)p->B * p->T > 0;
  if (!io || (tok && (!io->q || !io->k || !io->v || !io->g_raw || !io->beta)) || !io->A_log)
    return KDA_ERR_INVALID_ARGUMENT;
  if (!aligned16(io->q) || !aligned16(io->k) || !aligned16(io->v) || !aligned16(io->h_saved) ||
      !aligned16(io->dt_bias))
    return KDA_ERR_INVALID_ARGUMENT;
  if (ws_bytes < pl.fwd_bytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
  if (pl.fwd_bytes > 0 && !workspace) return KDA_ERR_INVALID_ARGUMENT;
  if (fwd_aliased(p, pl, io, workspace, pl.fwd_bytes)) return KDA_ERR_INVALID_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  ChunkInfo* tab = (ChunkInfo*)(ws + pl.chunks.off);
  int* seq_off = (int*)(ws + pl.seq_off.off);
  hipError_t e = launch_chunk_table(pl.s, tab, seq_off, nullptr, nullptr, s);
  if (e != hipSuccess) return hip_fail(e);
  const void *q = io->q, *k = io->k;
  if (pl.l2) {
    q = ws + pl.qn.off;
    k = ws + pl.kn.off;
    e = launch_l2norm(pl.s, pl.rows, io->q, (void*)q, (float*)(ws + pl.rq.off), s);
    if (e == hipSuccess)
      e = launch_l2norm(pl.s, pl.rows, io->k, (void*)k, (float*)(ws + pl.rk.off), s);
    if (e != hipSuccess) return hip_fail(e);
  }
  e = launch_fwd_ref(pl.s, seq_off, q, k, io->v, io->g_raw, io->beta, io->A_log,
                     io->dt_bias, io->h0, io->o, io->ht, io->h_saved, s);
  if (e != hipSuccess) return hip_fail(e);
  return KDA_OK;
}

int kda_fwd(const kda_problem* p, const kda_fwd_io* io, void* workspace, size_t ws_bytes,
            void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != KDA_OK) return st;
  const bool tok = (int64_t)p->B * p->T > 0;  // per-token tensors may be NULL without tokens
  if (!io || (tok && (!io->q || !io->k || !io->v || !io->g_raw || !io->beta)) || !io->A_log)
    return KDA_ERR_INVALID_ARGUMENT;
  const void* al[] = {io->q, io->k, io->v, io->g_raw, io->h_saved, io->o, io->dt_bias};
  for (const void* x : al)
    if (!aligned16(x)) return KDA_ERR_INVALID_ARGUMENT;
  if (ws_bytes < pl.fwdp_bytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
  if (pl.fwdp_bytes > 0 && !workspace) return KDA_ERR_INVALID_ARGUMENT;
  if (fwd_aliased(p, pl, io, workspace, pl.fwdp_bytes)) return KDA_ERR_INVALID_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  FwdPtrs f;
  f.chunks = (const ChunkInfo*)(ws + pl.chunks.off);
  f.seq_off = (const int*)(ws + pl.seq_off.off);
  f.groups = (const GroupInfo*)(ws + pl.fgroups.off);
  f.grp_off = (const int*)(ws + pl.fgrp_off.off);
  f.Pg = ws + pl.fPg.off;
  f.Qg = (float*)(ws + pl.fQg.off);
  f.bnd = (float*)(ws + pl.fbnd.off);
  const bool fused = use_prepscan(p, pl.s);
  int* order = fused ? (int*)(ws + pl.order.off) : nullptr;
  hipError_t e = launch_chunk_table(pl.s, (ChunkInfo*)f.chunks, (int*)f.seq_off,
                                    (GroupInfo*)f.groups, (int*)f.grp_off, s, order);
  if (e != hipSuccess) return hip_fail(e);
  f.q = io->q;  // raw: with qk_l2norm the per-chunk pass normalises the rows itself
  f.k = io->k;
  f.v = io->v;
  f.g_raw = io->g_raw; f.beta = io->beta; f.A_log = io->A_log; f.h0 = io->h0;
  f.dt_bias = io->dt_bias ? io->dt_bias : io->g_raw;
  f.has_db = io->dt_bias != nullptr;
  f.Wn = ws + pl.fWn.off; f.KrT = ws + pl.fKrT.off; f.UvT = ws + pl.fUvT.off;
  f.Qd = ws + pl.fQd.off; f.Mq = ws + pl.fMq.off; f.eGT = (float*)(ws + pl.fEgt.off);
  f.o = io->o; f.ht = io->ht; f.h_saved = io->h_saved;
  if (fused) {  // the state scan inside prep
    e = launch_fprepscan(pl.s, f, order, s);
    if (e != hipSuccess) return hip_fail(e);
    return KDA_OK;
  }
  e = launch_fprep(pl.s, f, s);
  if (e != hipSuccess) return hip_fail(e);
  e = launch_fscan(pl.s, f, s);
  if (e != hipSuccess) return hip_fail(e);
  return KDA_OK;
}

int kda_bwd(const kda_problem* p, const kda_bwd_io* io, void* workspace, size_t ws_bytes,
            void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != KDA_OK) return st;
  if (!io) return KDA_ERR_INVALID_ARGUMENT;
  // per-token tensors (inputs and gradients) may be NULL when there are no tokens
  const bool tok = (int64_t)p->B * p->T > 0;
  if ((tok && (!io->q || !io->k || !io->v || !io->g_raw || !io->beta || !io->dO || !io->dq ||
               !io->dk || !io->dv || !io->dg_raw || !io->dbeta)) ||
      !io->A_log || !io->dA_log)
    return KDA_ERR_INVALID_ARGUMENT;
  const void* al[] = {io->q, io->k, io->v, io->dO, io->g_raw, io->h_saved, io->h0, io->dht,
                      io->dq, io->dk, io->dv, io->dg_raw, io->dh0, io->dstates, io->dt_bias};
  for (const void* x : al)
    if (!aligned16(x)) return KDA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)io->ddt_bias & 3) != 0) return KDA_ERR_INVALID_ARGUMENT;
  const size_t need = io->h_saved ? pl.hsaved.off : pl.bwd_bytes;  // recompute region last
  if (ws_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && !workspace) return KDA_ERR_INVALID_ARGUMENT;
  if (bwd_aliased(p, pl, io, workspace, need)) return KDA_ERR_INVALID_ARGUMENT;

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  BwdPtrs b;
  b.q = io->q;  // raw: with qk_l2norm prep and the gradient pass normalise the rows
  b.k = io->k;
  b.v = io->v; b.dO = io->dO;
  b.g_raw = io->g_raw; b.beta = io->beta; b.A_log = io->A_log; b.h0 = io->h0; b.dht = io->dht;
  b.dt_bias = io->dt_bias ? io->dt_bias : io->g_raw;
  b.has_db = io->dt_bias != nullptr;
  b.ddt_bias = io->ddt_bias;
  b.dq = io->dq; b.dk = io->dk; b.dv = io->dv;
  b.dg_raw = io->dg_raw; b.dbeta = io->dbeta; b.dA_log = io->dA_log; b.dh0 = io->dh0;
  b.chunks = (const ChunkInfo*)(ws + pl.chunks.off);
  b.seq_off = (const int*)(ws + pl.seq_off.off);
  b.Tm = ws + pl.Tm.off;
  b.PT = ws + pl.PT.off;
  b.eGT = (float*)(ws + pl.eGT.off);
  b.INV = ws + pl.INV.off;
  b.MqkT = ws + pl.MqkT.off;
  b.dstates = io->dstates ? io->dstates : (void*)(ws + pl.dstates.off);
  b.dAl_part = (float*)(ws + pl.dAl.off);
  b.ddt_part = (float*)(ws + pl.ddt.off);
  b.h_saved = io->h_saved ? io->h_saved : (const void*)(ws + pl.hsaved.off);
  b.groups = (const GroupInfo*)(ws + pl.groups.off);
  b.grp_off = (const int*)(ws + pl.grp_off.off);
  b.Pg = ws + pl.Pg.off;
  b.Qg = (float*)(ws + pl.Qg.off);
  b.bnd = (float*)(ws + pl.bnd.off);
  const Shape& sh = pl.s;
  hipError_t e;
  const bool fused = use_prepscan(p, pl.s);
  int* order = fused ? (int*)(ws + pl.order.off) : nullptr;
  // with the scan inside prep, prep hands dU to the gradient pass in the Tm region (Tm and
  // PT are not formed in that mode; the region holds NC*H*K*K >= NC*H*64*V elements)
  b.dU = fused ? b.Tm : nullptr;
  e = timed(0, s, [&] {
    return launch_chunk_table(sh, (ChunkInfo*)b.chunks, (int*)b.seq_off, (GroupInfo*)b.groups,
                              (int*)b.grp_off, s, order);
  });
  if (e != hipSuccess) return hip_fail(e);
  if (!io->h_saved) {  // the chunk-start states by the production forward
    FwdPtrs f;
    f.q = b.q; f.k = b.k; f.v = io->v;
    f.g_raw = io->g_raw; f.beta = io->beta; f.A_log = io->A_log; f.h0 = io->h0;
    f.dt_bias = b.dt_bias; f.has_db = b.has_db;
    f.chunks = b.chunks; f.seq_off = b.seq_off;
    f.groups = b.groups; f.grp_off = b.grp_off;  // the split-scan regions, free until the scan
    f.Pg = b.Pg; f.Qg = b.Qg; f.bnd = b.bnd;
    f.Wn = ws + pl.rWn.off; f.KrT = ws + pl.rKrT.off; f.UvT = ws + pl.rUvT.off;
    f.Qd = ws + pl.rQd.off; f.Mq = ws + pl.rMq.off;
    f.eGT = b.eGT;  // prep writes the same values again
    f.o = nullptr; f.ht = nullptr; f.h_saved = (void*)b.h_saved;
    e = timed(5, s, [&] {
      if (fused) return launch_fprepscan(sh, f, order, s);
      hipError_t x = launch_fprep(sh, f, s);
      return x == hipSuccess ? launch_fscan(sh, f, s) : x;
    });
    if (e != hipSuccess) return hip_fail(e);
  }
  if (fused) {  // prep with the scan inside
    e = timed(1, s, [&] { return launch_prepscan(sh, b, order, s); });
    if (e != hipSuccess) return hip_fail(e);
  } else {
    e = timed(1, s, [&] { return launch_prep(sh, b, s); });
    if (e != hipSuccess) return hip_fail(e);
    e = timed(2, s, [&] { return launch_scan(sh, b, s); });
    if (e != hipSuccess) return hip_fail(e);
  }
  e = timed(3, s, [&] { return launch_gradf(sh, b, s); });
  if (e != hipSuccess) return hip_fail(e);
  e = timed(4, s, [&] { return launch_dalog(sh, b, s); });
  if (e != hipSuccess) return hip_fail(e);
  if (io->ddt_bias) {
    e = timed(4, s, [&] { return launch_ddt(sh, b, s); });
    if (e != hipSuccess) return hip_fail(e);
  }
  return KDA_OK;
}

int kda_timing_enable(int on) {
  g_timing = on != 0;
  return KDA_OK;
}

int kda_timing_read(double* ms, int* launches, int n) {
  std::vector<double> tot(kStages, 0.0);
  std::vector<int> cnt(kStages, 0);
  for (auto& t : g_events) {
    float x = 0.f;
    if (hipEventSynchronize(t.b) == hipSuccess && hipEventElapsedTime(&x, t.a, t.b) == hipSuccess) {
      tot[t.stage] += x;
      cnt[t.stage] += 1;
    }
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  g_events.clear();
  for (int i = 0; i < n && i < kStages; ++i) {
    if (ms) ms[i] = tot[i];
    if (launches) launches[i] = cnt[i];
  }
  return kStages;
}

}  // extern "C"
