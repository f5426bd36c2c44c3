// kda_fwd.hip -- chunk table, reference forward (chunk start states), the optional
// q/k L2 normalisation and its backward, and the per-head dA_log and per-channel
// dt_bias reductions.
#include "kda_dev.h"
#include "kda_launch.h"

namespace kda {

// ---------------------------------------------------------------------------
// Chunk table: one entry per 64-token chunk of every sequence, sequences back to
// back (chunk c of sequence n at index seq_off[n] + c).  With a group table
// requested, also the chunk groups of the state-gradient scan: runs of gs chunks
// of one sequence (gs = 0: the whole sequence), at least one per sequence, with
// grp_off[n] the first group of sequence n.  One workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_chunk_table(const int32_t* __restrict__ cu, int N, int T,
                                                     int gs, ChunkInfo* __restrict__ tab,
                                                     int* __restrict__ seq_off,
                                                     GroupInfo* __restrict__ groups,
                                                     int* __restrict__ grp_off,
                                                     int* __restrict__ order) {
  __shared__ int part[256], gpart[256];
  __shared__ int snck[kMaxOrderSeqs];
  const int tid = threadIdx.x;
  const int per = (N + 255) / 256;
  const int n0 = min(N, tid * per), n1 = min(N, n0 + per);
  auto nchunks = [&](int n) {
    const int len = cu ? cu[n + 1] - cu[n] : T;
    return (len + CH - 1) / CH;
  };
  auto ngroups = [&](int nck) { return gs > 0 ? max(1, (nck + gs - 1) / gs) : 1; };
  int cnt = 0, gcnt = 0;
  for (int n = n0; n < n1; ++n) {
    const int nck = nchunks(n);
    cnt += nck;
    gcnt += ngroups(nck);
  }
  // exclusive prefix sums over the 256 threads (inclusive scan by doubling, then shift)
  int x = cnt, y = gcnt;
  for (int d = 1; d < 256; d <<= 1) {
    part[tid] = x;
    gpart[tid] = y;
    __syncthreads();
    if (tid >= d) {
      x += part[tid - d];
      y += gpart[tid - d];
    }
    __syncthreads();
  }
  int off = x - cnt, goff = y - gcnt;
  for (int n = n0; n < n1; ++n) {
    const int len = cu ? cu[n + 1] - cu[n] : T;
    const int nck = (len + CH - 1) / CH;
    seq_off[n] = off;
    if (groups) {
      const int ng = ngroups(nck);
      grp_off[n] = goff;
      for (int gi = 0; gi < ng; ++gi) {
        GroupInfo gr;
        gr.c0 = off + (gs > 0 ? gi * gs : 0);
        gr.cnt = gs > 0 ? min(gs, nck - gi * gs) : nck;
        gr.seq = n;
        gr.flags = (gi == 0 ? GRP_FIRST : 0) | (gi == ng - 1 ? GRP_LAST : 0);
        groups[goff + gi] = gr;
      }
      goff += ng;
    }
    off += nck;
  }
  if (n0 < N && n1 == N) {
    seq_off[N] = off;
    if (groups) grp_off[N] = goff;
  }
  if (N == 0 && tid == 0) {
    seq_off[0] = 0;
    if (groups) grp_off[0] = 0;
  }
  // the chunk entries, all threads over all chunks (a long sequence has thousands): the
  // sequence of chunk i is the last n with seq_off[n] <= i (seq_off is visible to the
  // whole block after the barrier)
  __syncthreads();
  const int total = N > 0 ? seq_off[N] : 0;
  for (int i = tid; i < total; i += 256) {
    int lo = 0, hi = N - 1;  // seq_off[lo] <= i < seq_off[hi + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seq_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int n = lo, c = i - seq_off[n];
    const int start = cu ? cu[n] : n * T;
    const int len = cu ? cu[n + 1] - cu[n] : T;
    ChunkInfo e;
    e.t0 = start + c * CH;
    e.len = min(CH, len - c * CH);
    e.seq = n;
    e.cidx = c;
    tab[i] = e;
  }
  if (order && N <= kMaxOrderSeqs) {
    // the sequences sorted by chunk count, longest first (ties by index): order[rank] = n
    for (int n = tid; n < N; n += 256) snck[n] = nchunks(n);
    __syncthreads();
    for (int n = tid; n < N; n += 256) {
      const int a = snck[n];
      int rank = 0;
      for (int m = 0; m < N; ++m) rank += snck[m] > a || (snck[m] == a && m < n);
      order[rank] = n;
    }
  }
}

__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
}

// ---------------------------------------------------------------------------
// Reference forward, token by token.  One wave per (sequence, head, 64-column
// slice of V); lane j keeps column j of the K x 64 state slice in registers, so
// the rank-one update and both projections are per-lane loops over K with no
// cross-lane reduction.  Writes the state at the start of every chunk (h_saved),
// the outputs o and the final state.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void k_fwd_ref(const int* __restrict__ seq_off,
                                                const int32_t* __restrict__ cu, int H,
                                                int Tn, const T* __restrict__ q,
                                                const T* __restrict__ k,
                                                const T* __restrict__ v,
                                                const float* __restrict__ g_raw,
                                                const float* __restrict__ beta,
                                                const float* __restrict__ A_log,
                                                const float* __restrict__ dt_bias, float gu,
                                                const float* __restrict__ h0, T* __restrict__ o,
                                                float* __restrict__ ht, T* __restrict__ h_saved) {
  constexpr int NVS = D / 64;
  constexpr int TB = 16;  // tokens staged per round
  __shared__ float sk[TB][D], sq[TB][D], sa[TB][D], sb[TB];
  const int b = blockIdx.x;
  const int vs = b % NVS, u = b / NVS;
  const int n = u / H, h = u % H;
  const int j = threadIdx.x, d = vs * 64 + j;
  const int start = cu ? cu[n] : n * Tn;
  const int len = cu ? cu[n + 1] - cu[n] : Tn;
  const size_t KV = (size_t)D * D;
  float S[D];
  if (h0) {
    const float* src = h0 + ((size_t)n * H + h) * KV + d;
#pragma unroll
    for (int i = 0; i < D; ++i) S[i] = src[(size_t)i * D];
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) S[i] = 0.f;
  }
  // decay per token and key channel: exp(gu * g), g = -e^{A_log} softplus(g_raw + dt_bias)
  const float aA = __expf(A_log[h]) * gu;
  const int c0 = seq_off[n];
  for (int tb = 0; tb < len; tb += TB) {
    const int nt = min(TB, len - tb);
    __syncthreads();
    for (int idx = j; idx < TB * D; idx += 64) {
      int r = idx / D, i = idx % D;
      if (r < nt) {
        size_t off = ((size_t)(start + tb + r) * H + h) * D + i;
        sk[r][i] = to_f(k[off]);
        sq[r][i] = to_f(q[off]);
        sa[r][i] = __expf(-aA * softplus_f(g_raw[off] + (dt_bias ? dt_bias[h * D + i] : 0.f)));
      }
    }
    if (j < nt) sb[j] = beta[(size_t)(start + tb + j) * H + h];
    __syncthreads();
    for (int r = 0; r < nt; ++r) {
      const int local = tb + r;
      const size_t t = (size_t)(start + local);
      if (h_saved && (local % CH) == 0) {
        T* dst = h_saved + ((size_t)(c0 + local / CH) * H + h) * KV + d;
#pragma unroll
        for (int i = 0; i < D; ++i) dst[(size_t)i * D] = from_f<T>(S[i]);
      }
      const float vv = to_f(v[(t * H + h) * D + d]);
      float uu = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        S[i] *= sa[r][i];
        uu += S[i] * sk[r][i];
      }
      const float e = sb[r] * (vv - uu);
      float oo = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        S[i] += sk[r][i] * e;
        oo += S[i] * sq[r][i];
      }
      if (o) o[(t * H + h) * D + d] = from_f<T>(oo);
    }
  }
  if (ht) {
    float* dst = ht + ((size_t)n * H + h) * KV + d;
#pragma unroll
    for (int i = 0; i < D; ++i) dst[(size_t)i * D] = S[i];
  }
}

// ---------------------------------------------------------------------------
// dA_log[h] = sum over chunks of the per chunk-head partials (fixed order, so
// the result is deterministic).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dalog(const float* __restrict__ part, int64_t NC, int H,
                                               float* __restrict__ out) {
  __shared__ float red[4];
  const int h = blockIdx.x, tid = threadIdx.x;
  float acc = 0.f;
  for (int64_t c = tid; c < NC; c += 256) acc += part[c * H + h];
  acc = sum64(acc);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) out[h] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------------------
// L2 normalisation of q and k per (token, head) for the reference forward:
//   xn = x r,  r = 1 / sqrt(sum_i x_i^2 + eps)
// (the backward and the production forward normalise inside their own kernels with the
// same helpers).  A row of D elements is LPR lanes holding one 16-byte piece each; every
// lane of a block works (rows past the end are clamped and not stored), so the DPP sums
// over a lane group never see an idle lane.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_l2norm(const T* __restrict__ x, int64_t rows,
                                                T* __restrict__ xn, float* __restrict__ r) {
  constexpr int EPV = 16 / (int)sizeof(T), LPR = D / EPV, RPB = 256 / LPR;
  static_assert(LPR == 8 || LPR == 16, "row split");
  const int sub = threadIdx.x % LPR;
  const int64_t row0 = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int64_t row = row0 < rows ? row0 : rows - 1;
  const size_t o = (size_t)row * D + sub * EPV;
  u32x4 piece = *(const u32x4*)(x + o);
  const float rr = l2n_piece<T, LPR>(piece);
  if (row0 < rows) {
    *(u32x4*)(xn + o) = piece;
    if (sub == 0) r[row] = rr;
  }
}

template <typename T, int D>
static hipError_t l2norm_t(int64_t rows, const void* x, void* xn, float* r, hipStream_t st) {
  constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  hipLaunchKernelGGL((k_l2norm<T, D>), grid, dim3(256), 0, st, (const T*)x, rows, (T*)xn, r);
  return hipGetLastError();
}

hipError_t launch_l2norm(const Shape& s, int64_t rows, const void* x, void* xn, float* r,
                         hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (s.bf16)
    return s.D == 128 ? l2norm_t<bf16, 128>(rows, x, xn, r, st)
                      : l2norm_t<bf16, 64>(rows, x, xn, r, st);
  return l2norm_t<float, 64>(rows, x, xn, r, st);
}

// ddt_bias[h][i] = sum over chunks of the per chunk-head column sums of dg_raw, in a
// fixed order (deterministic).  Block (h, 16-channel group); lane i + 16 l of the
// block's 256 threads takes channel i and chunks l, l + 16, ... with four running
// sums (chunk index mod 64), which are then added in a fixed order.
__global__ __launch_bounds__(256) void k_ddt(const float* __restrict__ part, int64_t NC, int H,
                                             int D, float* __restrict__ out) {
  __shared__ float red[16][17];
  const int h = blockIdx.x, ch = 16 * blockIdx.y + (threadIdx.x & 15), l = threadIdx.x >> 4;
  const float* src = part + (size_t)h * D + ch;
  const size_t step = (size_t)H * D;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int64_t c = l;
  for (; c + 48 < NC; c += 64) {
    a0 += src[c * step];
    a1 += src[(c + 16) * step];
    a2 += src[(c + 32) * step];
    a3 += src[(c + 48) * step];
  }
  if (c < NC) a0 += src[c * step];
  if (c + 16 < NC) a1 += src[(c + 16) * step];
  if (c + 32 < NC) a2 += src[(c + 32) * step];
  red[l][threadIdx.x & 15] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (l == 0) {
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) acc += red[x][threadIdx.x & 15];
    out[h * D + ch] = acc;
  }
}

hipError_t launch_chunk_table(const Shape& s, ChunkInfo* tab, int* seq_off, GroupInfo* groups,
                              int* grp_off, hipStream_t st, int* order) {
  hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(256), 0, st, s.cu, s.N, s.T, s.gs, tab, seq_off,
                     groups, grp_off, order);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t fwd_ref_t(const Shape& s, const int* seq_off, const void* q, const void* k,
                            const void* v, const float* g_raw, const float* beta,
                            const float* A_log, const float* dt_bias, const float* h0, void* o,
                            float* ht, void* h_saved, hipStream_t st) {
  dim3 grid((unsigned)(s.N * s.H * (D / 64)));
  hipLaunchKernelGGL((k_fwd_ref<T, D>), grid, dim3(64), 0, st, seq_off, s.cu, s.H, s.T,
                     (const T*)q, (const T*)k, (const T*)v, g_raw, beta, A_log, dt_bias, s.gu, h0,
                     (T*)o, ht, (T*)h_saved);
  return hipGetLastError();
}

hipError_t launch_fwd_ref(const Shape& s, const int* seq_off, const void* q, const void* k,
                          const void* v, const float* g_raw, const float* beta,
                          const float* A_log, const float* dt_bias, const float* h0, void* o,
                          float* ht, void* h_saved, hipStream_t st) {
  if (s.N * s.H == 0) return hipSuccess;
  if (s.bf16) {
    if (s.D == 128)
      return fwd_ref_t<bf16, 128>(s, seq_off, q, k, v, g_raw, beta, A_log, dt_bias, h0, o, ht,
                                  h_saved, st);
    return fwd_ref_t<bf16, 64>(s, seq_off, q, k, v, g_raw, beta, A_log, dt_bias, h0, o, ht,
                               h_saved, st);
  }
  return fwd_ref_t<float, 64>(s, seq_off, q, k, v, g_raw, beta, A_log, dt_bias, h0, o, ht,
                              h_saved, st);
}

hipError_t launch_dalog(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  hipLaunchKernelGGL(k_dalog, dim3(s.H), dim3(256), 0, st, p.dAl_part, s.NC, s.H, p.dA_log);
  return hipGetLastError();
}

hipError_t launch_ddt(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  hipLaunchKernelGGL(k_ddt, dim3(s.H, s.D / 16), dim3(256), 0, st, p.ddt_part, s.NC, s.H, s.D,
                     p.ddt_bias);
  return hipGetLastError();
}

}  // namespace kda
