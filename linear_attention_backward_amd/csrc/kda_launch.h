// kda_launch.h -- host-side launchers of the KDA kernels (internal to libkda.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

struct ChunkInfo;
struct GroupInfo;

// Pointers of one backward call, as the kernels see them (device memory).
struct BwdPtrs {
  const void *q, *k, *v, *dO;
  const float *g_raw, *beta, *A_log, *h0, *dht;
  // per-channel gate bias [H,K]: always a readable address of at least H*K floats
  // (g_raw when there is no bias); has_db = 0 makes the kernels use zero instead
  const float* dt_bias;
  int has_db;
  const void* h_saved;
  void *dq, *dk, *dv;
  float *dg_raw, *dbeta, *dA_log, *dh0;
  float* ddt_bias;         // [H,K] or nullptr
  // workspace
  const ChunkInfo* chunks;
  const int* seq_off;      // [N+1] first chunk of every sequence
  // Tm, PT, exp(G_T): formed by prep for the separate scan kernels only
  void* Tm;                // [NC,H,K,K] act dtype : -W^T Kr (low-rank part of the chunk transition)
  void* PT;                // [NC,H,K,64] act dtype: (Qd - Mqk W)^T
  float* eGT;              // [NC,H,K]  exp(G_T)
  void* INV;               // [NC,H,64,64] act dtype: (I + diag(beta) A)^{-1}
  void* MqkT;              // [NC,H,64,64] act dtype: Mqk transposed (separate kernels only)
  void* dstates;           // [NC,H,K,V] act dtype: dL/dS at the end of every chunk
  // [NC,H,64,V] act dtype: dU = Mqk^T dO + Kr dS_out of every chunk, written by prep when
  // the state scan runs inside it (then over Tm, which that mode does not use) and read
  // by the gradient pass; nullptr: the gradient pass forms dU itself
  void* dU;
  float* dAl_part;         // [NC,H] per chunk-head partial sums for dA_log
  float* ddt_part;         // [NC,H,K] per chunk-head column sums of dg_raw (for ddt_bias)
  const GroupInfo* groups; // [NG] chunk groups of the state-gradient scan
  const int* grp_off;      // [N+1] first group of every sequence
  void* Pg;                // [NG,H,K,K] act dtype: transition of every group (split scan only)
  float* Qg;               // [NG,H,K,V] offset of every group (split scan only)
  float* bnd;              // [NG,H,K,V] state gradient at the end of every group (split scan only)
};

// Pointers of one production-forward call.
struct FwdPtrs {
  const void *q, *k, *v;
  const float *g_raw, *beta, *A_log, *h0;
  const float* dt_bias;  // always readable (g_raw without a bias); has_db selects it
  int has_db;
  const ChunkInfo* chunks;
  const int* seq_off;
  const GroupInfo* groups;  // chunk groups of the state scan (one per sequence unless split)
  const int* grp_off;
  void* Pg;                 // [NG,H,K,K] act dtype: group transitions (split scan only)
  float* Qg;                // [NG,H,K,V] group offsets (split scan only)
  float* bnd;               // [NG,H,K,V] state at the start of every group (split scan only)
  // per chunk-head operands (workspace), act dtype unless noted
  void* Wn;    // [NC,H,64,K]  -W, W = INV diag(beta) K e^G
  void* KrT;   // [NC,H,K,64]  (K e^{G_T - G})^T
  void* UvT;   // [NC,H,V,64]  (INV diag(beta) V)^T
  void* Qd;    // [NC,H,64,K]  Q e^G
  void* Mq;    // [NC,H,64,64] Mqk
  float* eGT;  // [NC,H,K]     e^{G_T}
  // outputs
  void* o;       // [B,T,H,V] or nullptr
  float* ht;     // [N,H,K,V] or nullptr
  void* h_saved; // [NC,H,K,V] or nullptr
};

struct Shape {
  int N, H, D, T;  // sequences, heads, K = V, tokens per row when not packed
  int64_t NC;      // total chunks
  int bf16;        // act dtype is bf16
  const int32_t* cu;  // device cu_seqlens or nullptr (uniform rows of T tokens)
  int gs;          // chunks per scan group; 0: one group per sequence
  int64_t NG;      // groups
  float gu;        // natural-log decay per unit of the gate: 1, or ln 2 for log2 units
  int qn;          // q and k L2-normalised inside the kernels (prep, gradient pass)
};

// order (optional, N ints): the sequences sorted by chunk count, longest first, for the
// scans inside prep (at most kMaxOrderSeqs sequences)
constexpr int kMaxOrderSeqs = 4096;
hipError_t launch_chunk_table(const Shape& s, ChunkInfo* tab, int* seq_off, GroupInfo* groups,
                              int* grp_off, hipStream_t st, int* order = nullptr);
hipError_t launch_fwd_ref(const Shape& s, const int* seq_off, const void* q, const void* k,
                          const void* v, const float* g_raw, const float* beta,
                          const float* A_log, const float* dt_bias, const float* h0, void* o,
                          float* ht, void* h_saved, hipStream_t st);
// Workgroups of `kernel` (block of `threads`) that the current device holds at
// once: CU count times the per-CU occupancy; cached per device and kernel.  The
// environment variable KDA_GRID_CAP, when set to n > 0, caps it at n.
hipError_t resident_blocks(const void* kernel, int threads, int* out);

// Workspace bytes kda_bwd needs for this problem, with or without a caller's h_saved.
int bwd_workspace_need(const struct ::kda_problem* p, bool has_h_saved, size_t* bytes);

hipError_t launch_prep(const Shape& s, const BwdPtrs& p, hipStream_t st);
hipError_t launch_fprep(const Shape& s, const FwdPtrs& p, hipStream_t st);
hipError_t launch_fscan(const Shape& s, const FwdPtrs& p, hipStream_t st);
hipError_t launch_scan(const Shape& s, const BwdPtrs& p, hipStream_t st);
// prep with the reverse state-gradient scan inside (every sequence has at least one chunk;
// workgroups take (sequence, head) units from the chunk-count order `order` in a snake):
// writes INV, dstates, dU (into p.dU) and dh0 instead of Tm, PT, exp(G_T) and Mqk^T
hipError_t launch_prepscan(const Shape& s, const BwdPtrs& p, const int* order, hipStream_t st);
// the production forward with the state scan inside prep's forward mode (same conditions):
// o, h_saved and ht without the per-chunk operands in memory
hipError_t launch_fprepscan(const Shape& s, const FwdPtrs& p, const int* order, hipStream_t st);
// workgroups of the backward one the current device holds at once (the forward one's is
// the same: same LDS)
hipError_t prepscan_grid(const Shape& s, int* grid);
hipError_t launch_gradf(const Shape& s, const BwdPtrs& p, hipStream_t st);
hipError_t launch_dalog(const Shape& s, const BwdPtrs& p, hipStream_t st);
hipError_t launch_ddt(const Shape& s, const BwdPtrs& p, hipStream_t st);
// rows = tokens * heads of a [.., H, D] act-dtype tensor: xn = x / |x|, r = 1 / |x|
hipError_t launch_l2norm(const Shape& s, int64_t rows, const void* x, void* xn, float* r,
                         hipStream_t st);

}  // namespace kda
