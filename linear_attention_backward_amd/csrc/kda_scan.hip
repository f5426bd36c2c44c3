// kda_scan.hip -- reverse scan of the state gradient across chunks.
//
// For the chunks of one sequence, last to first ([PB] section 3: Kernel A is
// the serial dstate scan; section 3.5 splits its V axis over workgroups):
//   dS_out(c) = dS                       (stored for the gradient pass)
//   dS       <- exp(G_T) . dS + Tm_c dS + PT_c dO_c
// and dh0 = dS after the first chunk.  The recurrence is separable in the V
// columns of dS, so each workgroup owns one (sequence, head, V-slice) and the
// slices never communicate.  dS is carried in fp32 MFMA accumulators; the
// operands Tm_c, PT_c (act dtype, from the prep pass) are read straight from
// global memory into MFMA A-fragments and prefetched one chunk ahead.
#include "kda_dev.h"
#include "kda_launch.h"

namespace kda {

template <typename T, int D, int VS>
__global__ __launch_bounds__(256) void k_scan(const ChunkInfo* __restrict__ chunks,
                                              const int* __restrict__ seq_off, int H, int nunits,
                                              const T* __restrict__ Tm, const T* __restrict__ PT,
                                              const float* __restrict__ eGT,
                                              const T* __restrict__ dO,
                                              const float* __restrict__ dht,
                                              T* __restrict__ dstates, float* __restrict__ dh0) {
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int KS = MM::KS, KPL = MM::KPL;
  constexpr int VW = D / VS;       // value columns of this workgroup
  constexpr int NCT = VW / 16;     // column tiles
  constexpr int RT = D / 64;       // row tiles per wave (rows = key channels)
  constexpr int PD = D + 16 / (int)sizeof(T);   // dS^T pitch  ([VW][D])
  constexpr int PO = Pitch<T, D>::TT;           // dO^T pitch ([VW][64])
  constexpr int EPV = 16 / (int)sizeof(T);      // elements per 16-byte vector
  constexpr int VPR = VW / EPV;                 // vectors per dO row slice
  constexpr int NLD = (64 * VPR + NTHR - 1) / NTHR;
  __shared__ __attribute__((aligned(16))) T sdST[VW * PD];
  __shared__ __attribute__((aligned(16))) T sdOT[2][VW * PO];

  // Block -> (unit, slice): the VS slices of a unit get block ids congruent mod 8,
  // so they are dispatched to the same XCD and share its L2 for Tm / PT.
  const int b = blockIdx.x;
  const int xcd = b & 7, y = b >> 3;
  const int vs = y % VS, u = (y / VS) * 8 + xcd;
  if (u >= nunits) return;
  const int n = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cbeg = seq_off[n], nck = seq_off[n + 1] - cbeg;
  const int col0 = vs * VW;
  const size_t DD = (size_t)D * D;

  f4 acc[RT][NCT];
  {
    const float* src = dht ? dht + ((size_t)n * H + h) * DD : nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int i = (w * RT + rt) * 16 + (lane >> 4) * 4;
        const int d = col0 + ct * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rt][ct][j] = src ? src[(size_t)(i + j) * D + d] : 0.f;
      }
  }

  Frag ta[RT][D / KS], pa[RT][64 / KS];
  f4 eg[RT];
  uint4 dov[NLD];
  auto load_ops = [&](int cg, Frag (&A)[RT][D / KS], Frag (&P)[RT][64 / KS], f4 (&E)[RT]) {
    const size_t ch = (size_t)cg * H + h;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int i = (w * RT + rt) * 16 + (lane & 15);
#pragma unroll
      for (int kk = 0; kk < D / KS; ++kk)
        A[rt][kk] = MM::load(Tm + ch * DD + (size_t)i * D + kk * KS + (lane >> 4) * KPL);
#pragma unroll
      for (int kk = 0; kk < 64 / KS; ++kk)
        P[rt][kk] = MM::load(PT + ch * D * 64 + (size_t)i * 64 + kk * KS + (lane >> 4) * KPL);
      E[rt] = *(const f4*)(eGT + ch * D + (w * RT + rt) * 16 + (lane >> 4) * 4);
    }
  };
  auto load_do = [&](int cg, uint4 (&R)[NLD]) {
    const ChunkInfo ci = chunks[cg];
#pragma unroll
    for (int l = 0; l < NLD; ++l) {
      const int idx = tid + l * NTHR;
      const int r = idx / VPR, sv = idx % VPR;
      uint4 x = {0u, 0u, 0u, 0u};
      if (idx < 64 * VPR && r < ci.len)
        x = *(const uint4*)(dO + ((size_t)(ci.t0 + r) * H + h) * D + col0 + sv * EPV);
      R[l] = x;
    }
  };
  auto store_do = [&](const uint4 (&R)[NLD], T* dst) {
#pragma unroll
    for (int l = 0; l < NLD; ++l) {
      const int idx = tid + l * NTHR;
      if (idx < 64 * VPR) {
        const int r = idx / VPR, sv = idx % VPR;
        const T* e = (const T*)&R[l];
#pragma unroll
        for (int q = 0; q < EPV; ++q) dst[(sv * EPV + q) * PO + r] = e[q];
      }
    }
  };

  if (nck > 0) {
    load_ops(cbeg + nck - 1, ta, pa, eg);
    load_do(cbeg + nck - 1, dov);
    store_do(dov, sdOT[0]);
  }
  int buf = 0;
  for (int cc = nck - 1; cc >= 0; --cc) {
    const int cg = cbeg + cc;
    // dS_out of this chunk
    {
      T* dst = dstates + ((size_t)cg * H + h) * DD;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          store_c<T>(dst, D, (w * RT + rt) * 16, col0 + ct * 16, acc[rt][ct], lane);
          store_ct<T>(sdST, PD, (w * RT + rt) * 16, ct * 16, acc[rt][ct], lane);
        }
    }
    __syncthreads();
    Frag tn[RT][D / KS], pn[RT][64 / KS];
    f4 en[RT];
    if (cc > 0) {
      load_ops(cg - 1, tn, pn, en);
      load_do(cg - 1, dov);
    }
    // dS <- exp(G_T) . dS + Tm dS + PT dO
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rt][ct][j] *= eg[rt][j];
#pragma unroll
    for (int kk = 0; kk < D / KS; ++kk) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const Frag bfr = MM::load(sdST + (ct * 16 + (lane & 15)) * PD + kk * KS + (lane >> 4) * KPL);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][ct] = MM::mma(ta[rt][kk], bfr, acc[rt][ct]);
      }
    }
    const T* sO = sdOT[buf];
#pragma unroll
    for (int kk = 0; kk < 64 / KS; ++kk) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const Frag bfr = MM::load(sO + (ct * 16 + (lane & 15)) * PO + kk * KS + (lane >> 4) * KPL);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][ct] = MM::mma(pa[rt][kk], bfr, acc[rt][ct]);
      }
    }
    if (cc > 0) {
      store_do(dov, sdOT[buf ^ 1]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int kk = 0; kk < D / KS; ++kk) ta[rt][kk] = tn[rt][kk];
#pragma unroll
        for (int kk = 0; kk < 64 / KS; ++kk) pa[rt][kk] = pn[rt][kk];
        eg[rt] = en[rt];
      }
    }
    buf ^= 1;
    __syncthreads();
  }
  if (dh0) {
    float* dst = dh0 + ((size_t)n * H + h) * DD;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        store_c<float>(dst, D, (w * RT + rt) * 16, col0 + ct * 16, acc[rt][ct], lane);
  }
}

template <typename T, int D, int VS>
static hipError_t scan_t(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  const int nunits = s.N * s.H;
  const int groups = (nunits + 7) / 8;
  dim3 grid((unsigned)(groups * 8 * VS));
  hipLaunchKernelGGL((k_scan<T, D, VS>), grid, dim3(NTHR), 0, st, p.chunks, p.seq_off, s.H, nunits,
                     (const T*)p.Tm, (const T*)p.PT, p.eGT, (const T*)p.dO, p.dht,
                     (T*)p.dstates, p.dh0);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t scan_d(const Shape& s, const BwdPtrs& p, int vs, hipStream_t st) {
  switch (vs) {
    case 1: return scan_t<T, D, 1>(s, p, st);
    case 2: return scan_t<T, D, 2>(s, p, st);
    case 4: return scan_t<T, D, 4>(s, p, st);
    default: break;
  }
  if constexpr (D >= 128) return scan_t<T, D, 8>(s, p, st);
  return scan_t<T, D, 4>(s, p, st);
}

hipError_t launch_scan(const Shape& s, const BwdPtrs& p, int vsplit, hipStream_t st) {
  if (s.N * s.H == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? scan_d<bf16, 128>(s, p, vsplit, st) : scan_d<bf16, 64>(s, p, vsplit, st);
  return scan_d<float, 64>(s, p, vsplit, st);
}

}  // namespace kda
