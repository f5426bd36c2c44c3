/*
 * kda_oracle.c -- fp64 CPU oracle for the KDA (gated delta rule) backward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *   [KB] "bwd-kernelB-beginner-guide-full" (yuyanqi.com, 2026-07-20): the Kernel-B
 *        guide.  Part 2, B1/B2/B3, lists the chunk-level backward quantities
 *        (dU, dvcorr, dv, dkr, dqd, dkd, kdS, the dbeta terms, the gate-gradient
 *        combination and its reverse cumsum, the dA_log reduction).
 *   [PB] "bwd-ncu-and-optimization-playbook" (yuyanqi.com, 2026-07-22): Kernel A
 *        is the serial reverse scan of the state gradient over chunks.
 *
 * The pages never write the forward recurrence out; the method they differentiate
 * is the KDA gated delta rule, taken here in its plain per-token form:
 *
 *   g_t   = -exp(A_log[h]) * softplus(g_raw_t)              (per key channel, <= 0)
 *   S_t   = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *
 * Optionally q and k are L2-normalised per token first ([KB] R1 / K1: the norm
 * forward and its backward); the recurrence then runs on the normalised vectors.
 *
 * Gate variants ([KB] part 2, the gate epilogue K1 and its dt_bias reduction): a
 * per-channel bias inside the softplus, and a gate given in log2 units (decay 2^g);
 * both live in the gate map and its chain rule below.
 *   o_t   = S_t^T q_t
 *
 * with S in R^{K x V}, S_{-1} = h0 (or 0), one recurrence per (sequence, head).
 * A loss L = sum(dO . o) + sum(dht . S_T) defines the gradients.
 *
 * Three pieces, each plain loops in fp64:
 *   1. kda_oracle_forward          -- the per-token recurrence above.
 *   2. kda_oracle_forward_chunked  -- an independent chunk form (pairwise decays,
 *                                     (I + diag(beta) A)^{-1} by forward
 *                                     substitution); must agree with piece 1.
 *   3. kda_oracle_backward         -- hand-derived reverse mode of piece 1,
 *                                     replaying the forward from checkpoints.
 * plus the gate map and its chain rule (dg -> dg_raw, dA_log).
 *
 * Layout of every per-token array: packed tokens, [TT][H][D] with D the feature
 * dimension; sequence n owns tokens cu[n] .. cu[n+1]-1.  States are [.][H][K][V].
 * Chunk c of sequence n (chunk size C) has global index  sum_{m<n} ceil(len_m/C) + c.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX3(t, h, d, H, D) ((((int64_t)(t)) * (H) + (h)) * (int64_t)(D) + (d))

static double softplus(double x) { return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x))); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static int64_t nchunks_of(int64_t len, int C) { return (len + C - 1) / C; }

static void chunk_offsets(int N, const int64_t* cu, int C, int64_t* off /* N+1 */) {
  off[0] = 0;
  for (int n = 0; n < N; ++n) off[n + 1] = off[n] + nchunks_of(cu[n + 1] - cu[n], C);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int kda_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Gate map.  The gate of token t, head h, key channel i is
 *   g' = -exp(A_log[h]) * softplus(g_raw + dt_bias[h][i]),   dt_bias absent = 0,
 * softplus(x) = max(x,0) + log1p(exp(-|x|)).  The per-step decay is exp(g') for a
 * gate in natural-log units (unit = 1) and 2^{g'} = exp(g' ln 2) for a gate in log2
 * units (unit = ln 2).  Returned: g = unit * g', the natural-log exponent the
 * recurrence applies. */
void kda_oracle_gate(int64_t TT, int H, int K, const double* g_raw, const double* A_log,
                     const double* dt_bias, double unit, double* g) {
  for (int64_t t = 0; t < TT; ++t)
    for (int h = 0; h < H; ++h) {
      double a = exp(A_log[h]);
      for (int i = 0; i < K; ++i) {
        double x = g_raw[IDX3(t, h, i, H, K)] + (dt_bias ? dt_bias[(int64_t)h * K + i] : 0.0);
        g[IDX3(t, h, i, H, K)] = unit * (-a * softplus(x));
      }
    }
}

/* Chain rule through the gate map, from dg = dL/dg (g as returned above):
 *   dg_raw = dg * unit * (-exp(A_log) * sigmoid(g_raw + dt_bias)),
 *   dA_log[h] = sum over tokens and key channels of dg * g   (dg/dA_log = g),
 *   ddt_bias[h][i] = sum over tokens of dg_raw                (NULL = not wanted). */
void kda_oracle_gate_backward(int64_t TT, int H, int K, const double* g_raw, const double* A_log,
                              const double* dt_bias, double unit, const double* g,
                              const double* dg, double* dg_raw, double* dA_log,
                              double* ddt_bias) {
  for (int h = 0; h < H; ++h) {
    double a = exp(A_log[h]);
    double acc = 0.0;
    if (ddt_bias)
      for (int i = 0; i < K; ++i) ddt_bias[(int64_t)h * K + i] = 0.0;
    for (int64_t t = 0; t < TT; ++t)
      for (int i = 0; i < K; ++i) {
        int64_t x = IDX3(t, h, i, H, K);
        double xr = g_raw[x] + (dt_bias ? dt_bias[(int64_t)h * K + i] : 0.0);
        dg_raw[x] = dg[x] * unit * (-a * sigmoid(xr));
        acc += dg[x] * g[x];
        if (ddt_bias) ddt_bias[(int64_t)h * K + i] += dg_raw[x];
      }
    dA_log[h] = acc;
  }
}

/* L2 normalisation of q or k per (token, head), over the D features:
 *   xn = x * r,  r = 1 / sqrt(sum_i x_i^2 + eps),
 * the reciprocal r kept for the backward ([KB] R1 computes it per row, K1 reuses
 * it).  Its chain rule, from dxn = dL/dxn:
 *   dx = r * (dxn - xn * (xn . dxn)). */
void kda_oracle_l2norm(int64_t TT, int H, int D, const double* x, double eps, double* xn,
                       double* r) {
  for (int64_t t = 0; t < TT; ++t)
    for (int h = 0; h < H; ++h) {
      const double* a = x + IDX3(t, h, 0, H, D);
      double ss = 0.0;
      for (int i = 0; i < D; ++i) ss += a[i] * a[i];
      double rr = 1.0 / sqrt(ss + eps);
      r[(int64_t)t * H + h] = rr;
      for (int i = 0; i < D; ++i) xn[IDX3(t, h, i, H, D)] = a[i] * rr;
    }
}

void kda_oracle_l2norm_backward(int64_t TT, int H, int D, const double* xn, const double* r,
                                const double* dxn, double* dx) {
  for (int64_t t = 0; t < TT; ++t)
    for (int h = 0; h < H; ++h) {
      const double* a = xn + IDX3(t, h, 0, H, D);
      const double* g = dxn + IDX3(t, h, 0, H, D);
      double dot = 0.0;
      for (int i = 0; i < D; ++i) dot += a[i] * g[i];
      double rr = r[(int64_t)t * H + h];
      for (int i = 0; i < D; ++i) dx[IDX3(t, h, i, H, D)] = rr * (g[i] - a[i] * dot);
    }
}

/* One forward token step on a K x V state (row-major, V contiguous):
 *   S <- Diag(a) S ;  u = S^T k ;  S <- S + beta k (v - u)^T ;  o = S^T q.
 * Diag(a) S is the decayed state; (I - beta k k^T) applied to it equals the
 * rank-one correction above. */
static void token_step(int K, int V, double* S, const double* q, const double* k,
                       const double* v, const double* g, double beta, double* o,
                       double* u /* scratch V */) {
  for (int i = 0; i < K; ++i) {
    double a = exp(g[i]);
    double* Si = S + (int64_t)i * V;
    for (int j = 0; j < V; ++j) Si[j] *= a;
  }
  for (int j = 0; j < V; ++j) u[j] = 0.0;
  for (int i = 0; i < K; ++i) {
    const double* Si = S + (int64_t)i * V;
    double ki = k[i];
    for (int j = 0; j < V; ++j) u[j] += Si[j] * ki;
  }
  for (int j = 0; j < V; ++j) u[j] = beta * (v[j] - u[j]);
  for (int i = 0; i < K; ++i) {
    double* Si = S + (int64_t)i * V;
    double ki = k[i];
    for (int j = 0; j < V; ++j) Si[j] += ki * u[j];
  }
  if (o) {
    for (int j = 0; j < V; ++j) o[j] = 0.0;
    for (int i = 0; i < K; ++i) {
      const double* Si = S + (int64_t)i * V;
      double qi = q[i];
      for (int j = 0; j < V; ++j) o[j] += Si[j] * qi;
    }
  }
}

/* Gather the per-token vectors of head h at token t. */
#define ROW(ptr, t, h, D) ((ptr) + IDX3((t), (h), 0, H, (D)))

/* ---------------------------------------------------------------------------
 * Piece 1: per-token forward.
 *   o      [TT][H][V]
 *   ht     [N][H][K][V]          (nullable) final state of each sequence
 *   states [NC][H][K][V]         (nullable) state at the START of each chunk of
 *                                size C (S_{-1} = h0 for the first chunk)
 * Returns 0, or -1 on bad arguments.
 * ------------------------------------------------------------------------- */
int kda_oracle_forward(int N, const int64_t* cu, int H, int K, int V, const double* q,
                       const double* k, const double* v, const double* g, const double* beta,
                       const double* h0, int C, double* o, double* ht, double* states,
                       int nthreads) {
  if (N <= 0 || H <= 0 || K <= 0 || V <= 0 || C <= 0) return -1;
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (N + 1));
  chunk_offsets(N, cu, C, off);
  set_threads(nthreads);
  int64_t KV = (int64_t)K * V;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < (int64_t)N * H; ++unit) {
    int n = (int)(unit / H), h = (int)(unit % H);
    double* S = (double*)malloc(sizeof(double) * KV);
    double* u = (double*)malloc(sizeof(double) * V);
    if (h0)
      memcpy(S, h0 + ((int64_t)n * H + h) * KV, sizeof(double) * KV);
    else
      memset(S, 0, sizeof(double) * KV);
    int64_t t0 = cu[n], t1 = cu[n + 1];
    for (int64_t t = t0; t < t1; ++t) {
      int64_t local = t - t0;
      if (states && local % C == 0)
        memcpy(states + ((off[n] + local / C) * H + h) * KV, S, sizeof(double) * KV);
      token_step(K, V, S, ROW(q, t, h, K), ROW(k, t, h, K), ROW(v, t, h, V), ROW(g, t, h, K),
                 beta[(int64_t)t * H + h], o ? (double*)ROW(o, t, h, V) : NULL, u);
    }
    if (ht) memcpy(ht + ((int64_t)n * H + h) * KV, S, sizeof(double) * KV);
    free(S);
    free(u);
  }
  free(off);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Piece 2: chunk form of the same forward, written from the chunk quantities the
 * pages name ([KB] part 2, B1/B2: U, INV, Mqk, kdS), independent of piece 1.
 * For a chunk of L rows with in-chunk cumulative gate G_r = sum_{s<=r} g_s:
 *   A_rs   = sum_i k_ri k_si exp(G_ri - G_si)           (s <  r)
 *   Mqk_rs = sum_i q_ri k_si exp(G_ri - G_si)           (s <= r)
 *   INV    = (I + diag(beta) A)^{-1}                    (forward substitution)
 *   Y      = V - (K . exp G) S_in ,   U = INV diag(beta) Y
 *   O      = (Q . exp G) S_in + Mqk U
 *   S_out  = Diag(exp G_T) S_in + (K . exp(G_T - G))^T U,  G_T = G_{L-1}.
 * Every exponent used is a non-positive difference, so nothing overflows.
 * ------------------------------------------------------------------------- */
int kda_oracle_forward_chunked(int N, const int64_t* cu, int H, int K, int V, const double* q,
                               const double* k, const double* v, const double* g,
                               const double* beta, const double* h0, int C, double* o,
                               double* ht, double* states, int nthreads) {
  if (N <= 0 || H <= 0 || K <= 0 || V <= 0 || C <= 0) return -1;
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (N + 1));
  chunk_offsets(N, cu, C, off);
  set_threads(nthreads);
  int64_t KV = (int64_t)K * V;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < (int64_t)N * H; ++unit) {
    int n = (int)(unit / H), h = (int)(unit % H);
    double* S = (double*)malloc(sizeof(double) * KV);
    double* Snew = (double*)malloc(sizeof(double) * KV);
    double* G = (double*)malloc(sizeof(double) * (size_t)C * K);
    double* A = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* M = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* INV = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* Y = (double*)malloc(sizeof(double) * (size_t)C * V);
    double* U = (double*)malloc(sizeof(double) * (size_t)C * V);
    if (h0)
      memcpy(S, h0 + ((int64_t)n * H + h) * KV, sizeof(double) * KV);
    else
      memset(S, 0, sizeof(double) * KV);
    int64_t t0 = cu[n], t1 = cu[n + 1];
    for (int64_t c0 = t0, ci = 0; c0 < t1; c0 += C, ++ci) {
      int L = (int)((t1 - c0) < C ? (t1 - c0) : C);
      if (states) memcpy(states + ((off[n] + ci) * H + h) * KV, S, sizeof(double) * KV);
      /* in-chunk cumulative gate */
      for (int i = 0; i < K; ++i) {
        double acc = 0.0;
        for (int r = 0; r < L; ++r) {
          acc += g[IDX3(c0 + r, h, i, H, K)];
          G[r * K + i] = acc;
        }
      }
      /* A (strictly lower) and Mqk (lower incl. diagonal) with pairwise decays */
      for (int r = 0; r < L; ++r)
        for (int s = 0; s < L; ++s) {
          double a = 0.0, m = 0.0;
          if (s <= r) {
            for (int i = 0; i < K; ++i) {
              double dec = exp(G[r * K + i] - G[s * K + i]);
              double ks = k[IDX3(c0 + s, h, i, H, K)];
              a += k[IDX3(c0 + r, h, i, H, K)] * ks * dec;
              m += q[IDX3(c0 + r, h, i, H, K)] * ks * dec;
            }
          }
          A[r * C + s] = (s < r) ? a : 0.0;
          M[r * C + s] = (s <= r) ? m : 0.0;
        }
      /* INV = (I + diag(beta) A)^{-1}: column by column forward substitution */
      for (int col = 0; col < L; ++col)
        for (int r = 0; r < L; ++r) {
          double x = (r == col) ? 1.0 : 0.0;
          double br = beta[(c0 + r) * H + h];
          for (int s = 0; s < r; ++s) x -= br * A[r * C + s] * INV[s * C + col];
          INV[r * C + col] = x;
        }
      /* Y = V - Kd S_in */
      for (int r = 0; r < L; ++r)
        for (int j = 0; j < V; ++j) {
          double acc = v[IDX3(c0 + r, h, j, H, V)];
          for (int i = 0; i < K; ++i)
            acc -= k[IDX3(c0 + r, h, i, H, K)] * exp(G[r * K + i]) * S[(int64_t)i * V + j];
          Y[r * V + j] = acc;
        }
      /* U = INV diag(beta) Y */
      for (int r = 0; r < L; ++r)
        for (int j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int s = 0; s <= r; ++s) acc += INV[r * C + s] * beta[(c0 + s) * H + h] * Y[s * V + j];
          U[r * V + j] = acc;
        }
      /* O = Qd S_in + Mqk U */
      if (o)
        for (int r = 0; r < L; ++r)
          for (int j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int i = 0; i < K; ++i)
              acc += q[IDX3(c0 + r, h, i, H, K)] * exp(G[r * K + i]) * S[(int64_t)i * V + j];
            for (int s = 0; s <= r; ++s) acc += M[r * C + s] * U[s * V + j];
            o[IDX3(c0 + r, h, j, H, V)] = acc;
          }
      /* S_out = Diag(exp G_T) S_in + Kr^T U */
      for (int i = 0; i < K; ++i) {
        double GT = G[(L - 1) * K + i];
        for (int j = 0; j < V; ++j) {
          double acc = exp(GT) * S[(int64_t)i * V + j];
          for (int r = 0; r < L; ++r)
            acc += k[IDX3(c0 + r, h, i, H, K)] * exp(GT - G[r * K + i]) * U[r * V + j];
          Snew[(int64_t)i * V + j] = acc;
        }
      }
      memcpy(S, Snew, sizeof(double) * KV);
    }
    if (ht) memcpy(ht + ((int64_t)n * H + h) * KV, S, sizeof(double) * KV);
    free(S); free(Snew); free(G); free(A); free(M); free(INV); free(Y); free(U);
  }
  free(off);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Piece 3: reverse-mode backward of piece 1, derived by hand per token.
 * For token t with a = exp(g_t), S~ = Diag(a) S_{t-1}, u = S~^T k, e = v - u,
 * S_t = S~ + beta k e^T, o = S_t^T q, and dS = dL/dS_t from later tokens:
 *   dS  += q dO^T
 *   dq   = S_t dO
 *   de   = beta dS^T k           (= dv)
 *   dbeta= k^T dS e
 *   dk   = beta dS e - S~ de
 *   dS~  = dS - k de^T
 *   da_i = sum_j dS~_ij S_{t-1,ij} ,  dg = a . da
 *   dS   = Diag(a) dS~            (gradient w.r.t. S_{t-1})
 * The state is replayed forward from checkpoints taken every C tokens (C is also
 * the chunk size used for the boundary exports).
 *
 * Inputs may have dht == NULL (zero) and h0 == NULL (zero).
 * Outputs: dq, dk [TT][H][K]; dv [TT][H][V]; dg [TT][H][K] (w.r.t. the gate g);
 *          dbeta [TT][H]; dh0 [N][H][K][V] (nullable);
 *          dstates [NC][H][K][V] (nullable): dL/dS at the END of each chunk,
 *          counting only its uses by later tokens (dht for the last chunk).
 * ------------------------------------------------------------------------- */
int kda_oracle_backward(int N, const int64_t* cu, int H, int K, int V, const double* q,
                        const double* k, const double* v, const double* g, const double* beta,
                        const double* h0, const double* dO, const double* dht, int C,
                        double* dq, double* dk, double* dv, double* dg, double* dbeta,
                        double* dh0, double* dstates, int nthreads) {
  if (N <= 0 || H <= 0 || K <= 0 || V <= 0 || C <= 0) return -1;
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (N + 1));
  chunk_offsets(N, cu, C, off);
  set_threads(nthreads);
  int64_t KV = (int64_t)K * V;
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < (int64_t)N * H; ++unit) {
    int n = (int)(unit / H), h = (int)(unit % H);
    int64_t t0 = cu[n], t1 = cu[n + 1], len = t1 - t0;
    int64_t nck = nchunks_of(len, C);
    /* checkpoints: state before token t0 + c*C, c = 0..nck-1 */
    double* ck = (double*)malloc(sizeof(double) * KV * (nck > 0 ? nck : 1));
    /* per-token states inside one segment: seg[0] = state before the segment,
     * seg[j+1] = state after its j-th token */
    double* seg = (double*)malloc(sizeof(double) * KV * (C + 1));
    double* dS = (double*)malloc(sizeof(double) * KV);
    double* u = (double*)malloc(sizeof(double) * V);
    double* e = (double*)malloc(sizeof(double) * V);
    double* de = (double*)malloc(sizeof(double) * V);
    if (!ck || !seg || !dS || !u || !e || !de) {
      fail = 1;
    } else {
      /* forward to collect checkpoints */
      double* S = seg; /* reuse as running state */
      if (h0)
        memcpy(S, h0 + ((int64_t)n * H + h) * KV, sizeof(double) * KV);
      else
        memset(S, 0, sizeof(double) * KV);
      for (int64_t t = t0; t < t1; ++t) {
        int64_t local = t - t0;
        if (local % C == 0) memcpy(ck + (local / C) * KV, S, sizeof(double) * KV);
        token_step(K, V, S, NULL, ROW(k, t, h, K), ROW(v, t, h, V), ROW(g, t, h, K),
                   beta[t * H + h], NULL, u);
      }
      if (dht)
        memcpy(dS, dht + ((int64_t)n * H + h) * KV, sizeof(double) * KV);
      else
        memset(dS, 0, sizeof(double) * KV);
      for (int64_t c = nck - 1; c >= 0; --c) {
        int64_t s0 = t0 + c * C;
        int L = (int)((t1 - s0) < C ? (t1 - s0) : C);
        if (dstates) memcpy(dstates + ((off[n] + c) * H + h) * KV, dS, sizeof(double) * KV);
        /* replay the segment */
        memcpy(seg, ck + c * KV, sizeof(double) * KV);
        for (int j = 0; j < L; ++j) {
          memcpy(seg + (j + 1) * KV, seg + j * KV, sizeof(double) * KV);
          token_step(K, V, seg + (j + 1) * KV, NULL, ROW(k, s0 + j, h, K), ROW(v, s0 + j, h, V),
                     ROW(g, s0 + j, h, K), beta[(s0 + j) * H + h], NULL, u);
        }
        for (int j = L - 1; j >= 0; --j) {
          int64_t t = s0 + j;
          const double* Sp = seg + j * KV;        /* S_{t-1} */
          const double* St = seg + (j + 1) * KV;  /* S_t */
          const double* qt = ROW(q, t, h, K);
          const double* kt = ROW(k, t, h, K);
          const double* vt = ROW(v, t, h, V);
          const double* gt = ROW(g, t, h, K);
          const double* dOt = ROW(dO, t, h, V);
          double bt = beta[t * H + h];
          /* dS += q dO^T ; dq = S_t dO */
          for (int i = 0; i < K; ++i) {
            double* dSi = dS + (int64_t)i * V;
            const double* Sti = St + (int64_t)i * V;
            double qi = qt[i], acc = 0.0;
            for (int jj = 0; jj < V; ++jj) {
              dSi[jj] += qi * dOt[jj];
              acc += Sti[jj] * dOt[jj];
            }
            dq[IDX3(t, h, i, H, K)] = acc;
          }
          /* e = v - S~^T k  (S~ = Diag(a) S_{t-1}) */
          for (int jj = 0; jj < V; ++jj) u[jj] = 0.0;
          for (int i = 0; i < K; ++i) {
            double ai = exp(gt[i]);
            const double* Spi = Sp + (int64_t)i * V;
            double w = ai * kt[i];
            for (int jj = 0; jj < V; ++jj) u[jj] += Spi[jj] * w;
          }
          for (int jj = 0; jj < V; ++jj) e[jj] = vt[jj] - u[jj];
          /* de = beta dS^T k ; dbeta = k^T dS e */
          for (int jj = 0; jj < V; ++jj) de[jj] = 0.0;
          double db = 0.0;
          for (int i = 0; i < K; ++i) {
            const double* dSi = dS + (int64_t)i * V;
            double ki = kt[i], rowdot = 0.0;
            for (int jj = 0; jj < V; ++jj) {
              de[jj] += dSi[jj] * ki;
              rowdot += dSi[jj] * e[jj];
            }
            db += ki * rowdot;
            /* dk first term: beta (dS e)_i */
            dk[IDX3(t, h, i, H, K)] = bt * rowdot;
          }
          for (int jj = 0; jj < V; ++jj) de[jj] *= bt;
          dbeta[t * H + h] = db;
          for (int jj = 0; jj < V; ++jj) dv[IDX3(t, h, jj, H, V)] = de[jj];
          /* dk -= S~ de ; dS~ = dS - k de^T ; da = rowsum(dS~ . S_{t-1}) ; dS = a dS~ */
          for (int i = 0; i < K; ++i) {
            double ai = exp(gt[i]);
            const double* Spi = Sp + (int64_t)i * V;
            double* dSi = dS + (int64_t)i * V;
            double ki = kt[i], sde = 0.0, da = 0.0;
            for (int jj = 0; jj < V; ++jj) {
              sde += ai * Spi[jj] * de[jj];
              double dst = dSi[jj] - ki * de[jj];
              da += dst * Spi[jj];
              dSi[jj] = ai * dst;
            }
            dk[IDX3(t, h, i, H, K)] -= sde;
            dg[IDX3(t, h, i, H, K)] = ai * da;
          }
        }
      }
      if (dh0) memcpy(dh0 + ((int64_t)n * H + h) * KV, dS, sizeof(double) * KV);
    }
    free(ck); free(seg); free(dS); free(u); free(e); free(de);
  }
  free(off);
  return fail ? -2 : 0;
}
