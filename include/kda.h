/*
 * kda.h -- C ABI of libkda.so: the chunkwise backward pass of KDA-style gated
 * delta-rule linear attention on AMD Instinct MI355X (gfx950).
 *
 * Method.  Per (sequence n, head h), with S in R^{K x V}:
 *   g_t = -exp(A_log[h]) * softplus(g_raw_t + dt_bias[h])      (per key channel)
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t,            S_{-1} = h0[n,h] (zero if absent)
 * dt_bias [H,K] is optional (zero if absent).  With gate_units = KDA_GATE_LOG2 the
 * gate is in log2 units: Diag(2^g_t) replaces Diag(exp g_t) (bwd-kernelB-beginner-
 * guide-full, R1, applies the gate with exp2; its K1 reduces ddt_bias).  kda_bwd
 * returns the gradients of  L = sum(dO . o) + sum(dht . S_T)  with respect to q, k, v,
 * g_raw, A_log, beta, h0 and dt_bias.  With qk_l2norm = 1, q and k are first
 * L2-normalised per (token, head), x / sqrt(sum x^2 + 1e-6) (R1 of the same guide;
 * its K1 holds the norm's backward), and dq, dk are with respect to the raw q, k.
 * It is computed chunkwise (64 tokens):
 * a serial reverse scan carries the state gradient dS back across chunks
 * ("Kernel A", bwd-ncu-and-optimization-playbook, section 3.5 on split-V), then a
 * data-parallel pass per chunk produces the per-token gradients, the gate
 * gradient with its in-chunk reverse cumulative sum and the per-head dA_log sum
 * ("Kernel B", bwd-kernelB-beginner-guide-full, part 2, B1/B2/B3).
 *
 * Layouts (all row-major, contiguous, no padding):
 *   per-token tensors  [B, T, H, D]  (token stride H*D); with cu_seqlens, B = 1
 *                      and the T tokens are the packed sequences back to back.
 *   states             [.., H, K, V]  (V contiguous).
 *   chunk-indexed      [NC, H, K, V]  where chunk c of sequence n has global index
 *                      sum_{m<n} ceil(len_m / 64) + c  (kda_num_chunks gives NC).
 *
 * Dtypes: act_dtype (KDA_DTYPE_F32 or KDA_DTYPE_BF16) applies to q, k, v, dO, o,
 * dq, dk, dv, h_saved and dstates.  g_raw, beta, A_log, h0, dht, ht, dg_raw, dbeta,
 * dA_log and dh0 are always fp32.  All accumulation is fp32.
 *
 * Supported shapes: chunk = 64; K == V; K in {64, 128} for bf16,
 * K == 64 for fp32; B*T*H < 2^31 (token-head rows and chunk-head items are indexed in
 * 32 bits); H*K < 2^22 (a token row of fp32, H*K*4 bytes, stays below 2^24 bytes, so
 * row offsets fit the 24-bit multiplier).  Anything else returns KDA_ERR_UNSUPPORTED.
 *
 * Ownership and synchronisation.  The caller owns every buffer (device memory)
 * and the stream.  The library allocates no device memory and keeps no pointer
 * after a call returns; scratch lives in the caller's workspace, sized by
 * kda_workspace_size.  Calls are asynchronous on `stream` (a hipStream_t; NULL =
 * the default stream) and enqueue work only after every argument has been
 * validated: a non-OK return means nothing was launched.  Concurrent calls need
 * distinct workspaces.  Outputs are overwritten, never accumulated.  No output may
 * overlap an input, another output or the workspace, and the workspace may not overlap
 * an input (KDA_ERR_INVALID_ARGUMENT otherwise; inputs may overlap one another).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

#if defined(__GNUC__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

/* Status codes.  0 = success; negative = error.  Validation errors (-1, -2, -3, -5) are
 * returned before anything is enqueued; with KDA_ERR_HIP the launches before the failing
 * one may already be on the stream, and the outputs are then undefined. */
#define KDA_OK 0
#define KDA_ERR_INVALID_ARGUMENT (-1) /* NULL required pointer, bad size, misaligned
                                         pointer, non-monotone cu_seqlens, sum != T */
#define KDA_ERR_UNSUPPORTED (-2)      /* shape or dtype not supported */
#define KDA_ERR_WORKSPACE_TOO_SMALL (-3)
#define KDA_ERR_HIP (-4)              /* a HIP launch failed; kda_status_string(-4)
                                         then names the HIP error of this thread */
#define KDA_ERR_SCRATCH_TOO_SMALL (-5) /* kda_bwd_noalloc: the problem needs more than
                                          KDA_NOALLOC_SCRATCH_BYTES of workspace */

#define KDA_DTYPE_F32 0
#define KDA_DTYPE_BF16 1

/* Units of the gate g (kda_problem.gate_units). */
#define KDA_GATE_LN 0   /* decay exp(g) per step */
#define KDA_GATE_LOG2 1 /* decay 2^g per step */

/* Problem description.  Host memory; read during the call only. */
typedef struct kda_problem {
  int B, T, H, K, V;  /* batch, tokens per batch row, heads, key dim, value dim */
  int chunk;          /* must be 64 */
  int act_dtype;      /* KDA_DTYPE_F32 or KDA_DTYPE_BF16 */
  int num_seqs;       /* with cu_seqlens: number of sequences N; else ignored (N = B) */
  /* Optional variable-length packing: int32 [N+1], cu[0] = 0, non-decreasing,
   * cu[N] = T, B must be 1.  Give both the host copy (sizes the grids; no device
   * synchronisation is needed) and the device copy (indexed by the kernels), or
   * neither. */
  const int32_t* cu_seqlens_host;
  const int32_t* cu_seqlens_dev;
  int gate_units;     /* KDA_GATE_LN or KDA_GATE_LOG2 (anything else: invalid) */
  int qk_l2norm;      /* 0, or 1: L2-normalise q and k inside the method (see above) */
} kda_problem;

/* Device pointers for kda_bwd.  16-byte aligned.  With no tokens at all (B*T == 0) the
 * per-token tensors ([B,T,...]) may be NULL: then dh0 = dht, dA_log = 0 and ddt_bias = 0
 * (kda_fwd_ref and kda_fwd likewise give ht = h0). */
typedef struct kda_bwd_io {
  /* inputs */
  const void* q;        /* [B,T,H,K] act_dtype */
  const void* k;        /* [B,T,H,K] act_dtype */
  const void* v;        /* [B,T,H,V] act_dtype */
  const float* g_raw;   /* [B,T,H,K] */
  const float* beta;    /* [B,T,H]   (after the sigmoid) */
  const float* A_log;   /* [H] */
  const float* h0;      /* [N,H,K,V] or NULL (zero initial state) */
  const void* dO;       /* [B,T,H,V] act_dtype */
  const float* dht;     /* [N,H,K,V] or NULL (zero) */
  const void* h_saved;  /* [NC,H,K,V] act_dtype: state at the start of every chunk,
                           as kda_fwd_ref writes it; NULL = recomputed in-stream */
  /* outputs (overwritten) */
  void* dq;             /* [B,T,H,K] act_dtype */
  void* dk;             /* [B,T,H,K] act_dtype */
  void* dv;             /* [B,T,H,V] act_dtype */
  float* dg_raw;        /* [B,T,H,K] */
  float* dbeta;         /* [B,T,H] */
  float* dA_log;        /* [H] */
  float* dh0;           /* [N,H,K,V] or NULL (not produced) */
  void* dstates;        /* [NC,H,K,V] act_dtype or NULL: if given, receives dL/dS at
                           the end of every chunk (uses by later tokens only) */
  const float* dt_bias; /* [H,K] or NULL (zero bias) -- input */
  float* ddt_bias;      /* [H,K] or NULL (not produced) -- output: the sum of dg_raw over
                           all tokens of every sequence */
} kda_bwd_io;

/* Device pointers for kda_fwd_ref (reference-quality forward that produces the
 * chunk states the backward consumes). */
typedef struct kda_fwd_io {
  const void* q;
  const void* k;
  const void* v;
  const float* g_raw;
  const float* beta;
  const float* A_log;
  const float* h0;      /* [N,H,K,V] or NULL */
  void* o;              /* [B,T,H,V] act_dtype, or NULL */
  float* ht;            /* [N,H,K,V] or NULL */
  void* h_saved;        /* [NC,H,K,V] act_dtype, or NULL */
  const float* dt_bias; /* [H,K] or NULL (zero bias) */
} kda_fwd_io;

#define KDA_WS_BWD 0
#define KDA_WS_FWD 1     /* kda_fwd (also enough for kda_fwd_ref) */
#define KDA_WS_FWD_REF 2 /* kda_fwd_ref */

/* Bytes of workspace kda_bwd (which = KDA_WS_BWD), kda_fwd (KDA_WS_FWD) or
 * kda_fwd_ref (KDA_WS_FWD_REF) needs for this problem.  Needs the host cu_seqlens
 * when packed.  The bwd size with h_saved == NULL is the one returned (it is the
 * larger). */
KDA_API int kda_workspace_size(const kda_problem* p, int which, size_t* bytes);

/* Total number of 64-token chunks NC over all sequences. */
KDA_API int kda_num_chunks(const kda_problem* p, int64_t* nchunks);

/* The backward pass (see the method above).  kda_bwd, kda_fwd_ref and kda_fwd only
 * enqueue kernels on `stream` (no allocation, memory set, copy or host
 * synchronisation), so a call may be captured into a HIP graph and replayed while its
 * pointers, workspace and problem stay valid; kernels are deterministic, so replays
 * reproduce the call bit for bit. */
KDA_API int kda_bwd(const kda_problem* p, const kda_bwd_io* io, void* workspace, size_t ws_bytes,
            void* stream);

/* Reference forward: o, ht and the per-chunk start states h_saved, by the per-token
 * recurrence of the method above taken token by token (one work-item per (sequence,
 * head, 64 value columns)).  The backward consumes the state saved at the start of
 * every chunk (bwd-kernelB-beginner-guide-full, part 2, B0 and B2: the chunk-start
 * state S_in that the state-side products and the p = rowsum(S_in . dS) term read).
 * o, ht and h_saved may each be NULL.  Workspace: kda_workspace_size(KDA_WS_FWD_REF);
 * errors as for kda_bwd. */
KDA_API int kda_fwd_ref(const kda_problem* p, const kda_fwd_io* io, void* workspace, size_t ws_bytes,
                void* stream);

/* Production forward, same arguments and results as kda_fwd_ref, in chunk form
 * (bwd-kernelB-beginner-guide-full, part 2: the UT/WY quantities A, INV, W and
 * Mqk): a data-parallel pass per chunk forms W = INV diag(beta) K e^G,
 * Uv = INV diag(beta) V, Qd, Mqk, Kr and e^{G_T}; then one workgroup per (sequence,
 * head) carries the state over its chunks, U = Uv - W S, O = Qd S + Mqk U,
 * S <- e^{G_T} . S + Kr^T U.  o, ht and h_saved may each be NULL. */
KDA_API int kda_fwd(const kda_problem* p, const kda_fwd_io* io, void* workspace, size_t ws_bytes,
            void* stream);

/* The backward pass for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): kda_bwd with its
 * workspace taken from a static device array of KDA_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends, instead of a caller
 * workspace.  The caller still passes every input and output.  Problems whose workspace
 * (kda_workspace_size, or less when h_saved is given) exceeds that size return
 * KDA_ERR_SCRATCH_TOO_SMALL without launching; other errors as for kda_bwd.  Allocates
 * nothing.  The first call on a device looks the array's device address up once (not
 * allowed under stream capture: make one call on each device before capturing).  Every
 * call on one GPU shares that GPU's array, so calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
KDA_API int kda_bwd_noalloc(const kda_problem* p, const kda_bwd_io* io, void* stream);

/* Text for a status code (for KDA_ERR_HIP: the last HIP error of this thread). */
KDA_API const char* kda_status_string(int status);

KDA_API int kda_abi_version(void);

/* Optional per-stage timing for measurement.  While enabled, kda_bwd brackets
 * each kernel launch with HIP events on the call's stream.  kda_timing_read
 * waits for the recorded events, writes per-stage totals (milliseconds) and
 * launch counts for up to n stages, clears them, and returns the number of
 * stages.  Stages: 0 chunk table, 1 prep, 2 state-gradient scan, 3 gradient
 * pass, 4 dA_log and dt_bias reductions, 5 state recompute (h_saved == NULL),
 * 6 q/k L2 normalisation and its backward (qk_l2norm).
 * Not thread-safe; meant for benchmarks. */
KDA_API int kda_timing_enable(int on);
KDA_API int kda_timing_read(double* ms, int* launches, int n);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
