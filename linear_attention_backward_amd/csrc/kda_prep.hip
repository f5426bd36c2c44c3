// kda_prep.hip -- per chunk-head recompute of the intra-chunk UT/WY quantities.
//
// For a 64-token chunk with in-chunk cumulative gate G (G_r = sum_{s<=r} g_s):
//   A_rs   = sum_i k_ri k_si exp(G_ri - G_si)  (s <  r)        [KB part 2, B1: Mqk, INV]
//   Mqk_rs = sum_i q_ri k_si exp(G_ri - G_si)  (s <= r)
//   INV    = (I + diag(beta) A)^{-1}
//   W      = INV diag(beta) Kd,  Kd = K exp(G),  Kr = K exp(G_T - G),  Qd = Q exp(G)
// and the two pieces of the chunk's state-gradient transition used by the
// reverse scan ([PB] section 3: Kernel A is the serial dstate scan):
//   dS_in = exp(G_T) . dS_out + Tm dS_out + PT dO,  Tm = -W^T Kr,  PT = (Qd - Mqk W)^T.
// exp(-G) overflows fp32 under strong decay, so the pairwise decays are never
// formed from exp(+-G) directly: 16-row blocks of A/Mqk below the diagonal use an
// anchor row a between the two blocks (both exp(G_r - G_a) and exp(G_a - G_s) are
// <= 1) and run on MFMA; the 16x16 diagonal blocks take exp(G_r - G_s) per pair.
// The gate is kept in log2 units so that v_exp_f32 (2^x) applies directly.
#include "kda_dev.h"
#include "kda_launch.h"

namespace kda {

__device__ __forceinline__ float softplus_p(float x) {
  return fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)));
}

template <typename T, int D> struct PrepLds {
  using P = Pitch<T, D>;
  static constexpr int G_SZ = 64 * P::NF * 4;
  static constexpr int QK_SZ = 64 * P::N * (int)sizeof(T);
  static constexpr int CC_SZ = 64 * P::CC * 4;
  static constexpr int TT_SZ = D * P::TT * (int)sizeof(T);
  static constexpr int U_SZ = CC_SZ > TT_SZ ? CC_SZ : TT_SZ;
  static constexpr int G_OFF = 0;
  static constexpr int Q_OFF = G_OFF + G_SZ;
  static constexpr int K_OFF = Q_OFF + QK_SZ;
  static constexpr int M_OFF = K_OFF + QK_SZ;
  static constexpr int INV_OFF = M_OFF + CC_SZ;  // later: W^T
  static constexpr int A_OFF = INV_OFF + U_SZ;   // later: (beta Kd)^T
  static constexpr int KRT_OFF = A_OFF + U_SZ;
  static constexpr int BETA_OFF = KRT_OFF + TT_SZ;
  static constexpr int SCR_OFF = BETA_OFF + 256;
  static constexpr int TOTAL = SCR_OFF + 4 * 16 * 17 * 4;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void k_prep(const ChunkInfo* __restrict__ chunks, int H,
                                              const T* __restrict__ q, const T* __restrict__ k,
                                              const float* __restrict__ g_raw,
                                              const float* __restrict__ beta,
                                              const float* __restrict__ A_log,
                                              T* __restrict__ Tm, T* __restrict__ PT,
                                              float* __restrict__ eGT, T* __restrict__ INVo,
                                              T* __restrict__ INVTo, T* __restrict__ MqkTo) {
  using L = PrepLds<T, D>;
  using P = Pitch<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int KS = MM::KS, KPL = MM::KPL;
  constexpr int NF = P::NF, PN = P::N, CC = P::CC, TT = P::TT;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  float* sG = (float*)(smem + L::G_OFF);
  T* sQ = (T*)(smem + L::Q_OFF);
  T* sK = (T*)(smem + L::K_OFF);
  float* sM = (float*)(smem + L::M_OFF);
  float* sINV = (float*)(smem + L::INV_OFF);
  T* sWT = (T*)(smem + L::INV_OFF);
  float* sA = (float*)(smem + L::A_OFF);
  T* sKdT = (T*)(smem + L::A_OFF);
  T* sKrT = (T*)(smem + L::KRT_OFF);
  float* sBeta = (float*)(smem + L::BETA_OFF);
  float* sScr = (float*)(smem + L::SCR_OFF);

  const int c = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const ChunkInfo ci = chunks[c];
  const int t0 = ci.t0, Lr = ci.len;
  const size_t ch = (size_t)c * H + h;

  // ---- load q, k (rows beyond the chunk are zero), beta, gate.  Every global
  // load is issued before any of them is used.
  constexpr int VPR = D * (int)sizeof(T) / 16;
  constexpr int NLT = 64 * VPR / NTHR;
  constexpr int PARTS = NTHR / D;
  constexpr int RPP = 64 / PARTS;
  const size_t rs = (size_t)H * D;
  uint4 rq[NLT], rk[NLT];
  float rg[RPP];
  {
    const T* qh = q + (size_t)t0 * rs + (size_t)h * D;
    const T* kh = k + (size_t)t0 * rs + (size_t)h * D;
#pragma unroll
    for (int l = 0; l < NLT; ++l) {
      const int idx = tid + l * NTHR, r = idx / VPR, vv = idx % VPR;
      uint4 xq = {0u, 0u, 0u, 0u}, xk = {0u, 0u, 0u, 0u};
      if (r < Lr) {
        xq = ((const uint4*)(qh + r * rs))[vv];
        xk = ((const uint4*)(kh + r * rs))[vv];
      }
      rq[l] = xq;
      rk[l] = xk;
    }
    const float* gh = g_raw + (size_t)t0 * rs + (size_t)h * D + tid % D;
    const int part = tid / D;
#pragma unroll
    for (int rr = 0; rr < RPP; ++rr) {
      const int r = part * RPP + rr;
      rg[rr] = r < Lr ? gh[r * rs] : 0.f;
    }
  }
  if (tid < 64) sBeta[tid] = tid < Lr ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
  const float aA = __expf(A_log[h]);
#pragma unroll
  for (int l = 0; l < NLT; ++l) {
    const int idx = tid + l * NTHR, r = idx / VPR, vv = idx % VPR;
    *(uint4*)((char*)(sQ + r * PN) + vv * 16) = rq[l];
    *(uint4*)((char*)(sK + r * PN) + vv * 16) = rk[l];
  }
  {
    const int i = tid % D, part = tid / D;
    float run = 0.f;
#pragma unroll
    for (int rr = 0; rr < RPP; ++rr) {
      const int r = part * RPP + rr;
      const float g = r < Lr ? -aA * softplus_p(rg[rr]) : 0.f;
      run += g * LOG2E;
      sG[r * NF + i] = run;
    }
  }
  __syncthreads();
  {
    const int i = tid % D, part = tid / D;
    float add = 0.f;
    for (int pp = 0; pp < part; ++pp) add += sG[(pp * RPP + RPP - 1) * NF + i];
    __syncthreads();
    if (part > 0)
      for (int rr = 0; rr < RPP; ++rr) sG[(part * RPP + rr) * NF + i] += add;
  }
  __syncthreads();

  // ---- A and Mqk.  Wave w owns row block R = w.
  {
    const int R = w;
    const int arow = 16 * R;  // anchor: first row of the block
    f4 accA[3], accM[3];
#pragma unroll
    for (int S = 0; S < 3; ++S) accA[S] = accM[S] = zero4();
    if (R > 0) {
      const int rrow = 16 * R + (lane & 15);
      for (int kk = 0; kk < D; kk += KS) {
        const int i0 = kk + (lane >> 4) * KPL;
        float kf[KPL], qf[KPL], ga[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          ga[j] = sG[arow * NF + i0 + j];
          const float e = ex2(sG[rrow * NF + i0 + j] - ga[j]);
          kf[j] = to_f(sK[rrow * PN + i0 + j]) * e;
          qf[j] = to_f(sQ[rrow * PN + i0 + j]) * e;
        }
        const Frag KF = MM::from_vals(kf), QF = MM::from_vals(qf);
#pragma unroll
        for (int S = 0; S < 3; ++S) {
          if (S < R) {
            const int srow = 16 * S + (lane & 15);
            float kb[KPL];
#pragma unroll
            for (int j = 0; j < KPL; ++j)
              kb[j] = to_f(sK[srow * PN + i0 + j]) * ex2(ga[j] - sG[srow * NF + i0 + j]);
            const Frag KB = MM::from_vals(kb);
            accA[S] = MM::mma(KF, KB, accA[S]);
            accM[S] = MM::mma(QF, KB, accM[S]);
          }
        }
      }
    }
#pragma unroll
    for (int S = 0; S < 4; ++S) {
      if (S < R) {
        store_c<float>(sA, CC, 16 * R, 16 * S, accA[S < 3 ? S : 0], lane);
        store_c<float>(sM, CC, 16 * R, 16 * S, accM[S < 3 ? S : 0], lane);
      } else if (S > R) {
        store_c<float>(sA, CC, 16 * R, 16 * S, zero4(), lane);
        store_c<float>(sM, CC, 16 * R, 16 * S, zero4(), lane);
      }
    }
    // diagonal block (R, R), by 4-row sub-blocks:
    //  (i) rows r of sub-block rho against s in earlier sub-blocks of the block,
    //      anchored at a = 16R + 4 rho (between them): one MFMA pass per rho with
    //      the A rows outside rho and the B columns at or after a set to zero;
    //  (ii) pairs inside a 4x4 diagonal sub-block: pairwise decays on VALU, one
    //      (sub-block, channel group) per lane, summed over the 16 groups.
    {
      const int r0 = 16 * R;
      const int cl = lane & 15;
      const int rA = r0 + cl;                  // A row of this lane
      const int rho_l = cl >> 2;               // its sub-block
      const int anc = r0 + 4 * rho_l;          // its anchor
      f4 dA = zero4(), dM = zero4();
      float zv[KPL];
#pragma unroll
      for (int j = 0; j < KPL; ++j) zv[j] = 0.f;
      const Frag ZF = MM::from_vals(zv);
      for (int kk = 0; kk < D; kk += KS) {
        const int i0 = kk + (lane >> 4) * KPL;
        float kf[KPL], qf[KPL], ks[KPL], gs[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const float e = ex2(sG[rA * NF + i0 + j] - sG[anc * NF + i0 + j]);
          kf[j] = to_f(sK[rA * PN + i0 + j]) * e;
          qf[j] = to_f(sQ[rA * PN + i0 + j]) * e;
          ks[j] = to_f(sK[rA * PN + i0 + j]);  // B column s = r0 + cl: same row data
          gs[j] = sG[rA * NF + i0 + j];
        }
        const Frag KF = MM::from_vals(kf), QF = MM::from_vals(qf);
#pragma unroll
        for (int rho = 1; rho < 4; ++rho) {
          const int a = r0 + 4 * rho;
          const bool colok = cl < 4 * rho;
          float kb[KPL];
#pragma unroll
          for (int j = 0; j < KPL; ++j)
            kb[j] = colok ? ks[j] * ex2(sG[a * NF + i0 + j] - gs[j]) : 0.f;
          const Frag KB = MM::from_vals(kb);
          const bool rowok = rho_l == rho;
          dA = MM::mma(rowok ? KF : ZF, KB, dA);
          dM = MM::mma(rowok ? QF : ZF, KB, dM);
        }
      }
      {
        constexpr int CPG = D / 16;
        const int sb = lane >> 4, cg = lane & 15;
        float pa[10], pm[10];
#pragma unroll
        for (int p = 0; p < 10; ++p) pa[p] = pm[p] = 0.f;
        for (int c8 = 0; c8 < CPG; ++c8) {
          const int i = cg * CPG + c8;
          float kk4[4], qq4[4], gg4[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = r0 + 4 * sb + t;
            kk4[t] = to_f(sK[r * PN + i]);
            qq4[t] = to_f(sQ[r * PN + i]);
            gg4[t] = sG[r * NF + i];
          }
#pragma unroll
          for (int a_ = 0; a_ < 4; ++a_)
#pragma unroll
            for (int b_ = 0; b_ <= a_; ++b_) {
              const int p = a_ * (a_ + 1) / 2 + b_;
              const float kb = kk4[b_] * ex2(gg4[a_] - gg4[b_]);
              pa[p] += kk4[a_] * kb;
              pm[p] += qq4[a_] * kb;
            }
        }
#pragma unroll
        for (int p = 0; p < 10; ++p) {
          pa[p] = sum16(pa[p]);
          pm[p] = sum16(pm[p]);
        }
        // C layout: lane holds rows 4 sb + j, column cl; the diagonal sub-block of
        // those rows has columns 4 sb .. 4 sb + 3.
        if ((cl >> 2) == sb) {
          const int b_ = cl & 3;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (b_ <= j) {
              const int p = j * (j + 1) / 2 + b_;
              if (b_ < j) dA[j] += pa[p];
              dM[j] += pm[p];
            }
          }
        }
      }
      store_c<float>(sA, CC, r0, r0, dA, lane);
      store_c<float>(sM, CC, r0, r0, dM, lane);
    }
  }
  __syncthreads();

  // ---- INV = (I + L)^{-1}, L = diag(beta) A (strictly lower), blocked by 16.
  // Step 1: wave R inverts its unit lower-triangular diagonal block.
  {
    const int R = w;
    if (lane < 16) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == lane) ? 1.f : 0.f;
        const float br = sBeta[16 * R + r];
#pragma unroll
        for (int s = 0; s < r; ++s) acc -= br * sA[(16 * R + r) * CC + 16 * R + s] * x[s];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sINV[(16 * R + r) * CC + 16 * R + lane] = x[r];
    }
    for (int e = lane; e < 16 * 64; e += 64) {
      const int r = e >> 6, col = e & 63;
      if (col >= 16 * (R + 1)) sINV[(16 * R + r) * CC + col] = 0.f;
    }
  }
  __syncthreads();
  // Step 2: wave S fills column block S below the diagonal, top to bottom:
  //   INV_{R,S} = -D_R * sum_{J=S}^{R-1} L_{R,J} INV_{J,S}.
  {
    const int S = w;
    float* scr = sScr + w * 16 * 17;
    for (int R = S + 1; R < 4; ++R) {
      f4 X = zero4();
      for (int J = S; J < R; ++J) {
#pragma unroll
        for (int kk = 0; kk < 16; kk += 4) {
          const int row = lane & 15, kx = kk + (lane >> 4);
          const float a = sBeta[16 * R + row] * sA[(16 * R + row) * CC + 16 * J + kx];
          const float b = sINV[(16 * J + kx) * CC + 16 * S + row];
          X = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, X, 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) scr[((lane >> 4) * 4 + j) * 17 + (lane & 15)] = X[j];
      __builtin_amdgcn_wave_barrier();
      f4 Y = zero4();
#pragma unroll
      for (int kk = 0; kk < 16; kk += 4) {
        const int row = lane & 15, kx = kk + (lane >> 4);
        const float a = sINV[(16 * R + row) * CC + 16 * R + kx];
        const float b = scr[kx * 17 + row];
        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, Y, 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sINV[(16 * R + (lane >> 4) * 4 + j) * CC + 16 * S + (lane & 15)] = -Y[j];
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  // ---- write INV, INV^T, Mqk^T (act dtype) for the gradient pass
  {
    T* o1 = INVo + ch * 64 * 64;
    T* o2 = INVTo + ch * 64 * 64;
    T* o3 = MqkTo + ch * 64 * 64;
    for (int e = tid; e < 64 * 64; e += NTHR) {
      const int r = e >> 6, s = e & 63;
      o1[e] = from_f<T>(sINV[r * CC + s]);
      o2[e] = from_f<T>(sINV[s * CC + r]);
      o3[e] = from_f<T>(sM[s * CC + r]);
    }
  }
  __syncthreads();  // sA (aliased by KdT) is dead from here on

  // ---- (beta Kd)^T and Kr^T, [D][64]
  for (int idx = tid; idx < 64 * D; idx += NTHR) {
    const int s = idx / D, i = idx % D;
    const float kv = to_f(sK[s * PN + i]);
    const float G = sG[s * NF + i], GT = sG[63 * NF + i];
    sKdT[i * TT + s] = from_f<T>(sBeta[s] * kv * ex2(G));
    sKrT[i * TT + s] = from_f<T>(kv * ex2(GT - G));
  }
  __syncthreads();

  // ---- W = INV (beta Kd): wave R -> rows of block R, all D columns
  {
    const int R = w;
    f4 acc[D / 16];
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) acc[nt] = zero4();
    for (int kk = 0; kk < 64; kk += KS) {
      const Frag a = MM::from_f32(sINV + (16 * R + (lane & 15)) * CC + kk + (lane >> 4) * KPL);
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        const Frag b = MM::load(sKdT + (nt * 16 + (lane & 15)) * TT + kk + (lane >> 4) * KPL);
        acc[nt] = MM::mma(a, b, acc[nt]);
      }
    }
    __syncthreads();  // every wave is done reading INV before W^T overwrites it
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) store_ct<T>(sWT, TT, 16 * R, nt * 16, acc[nt], lane);
  }
  __syncthreads();

  constexpr int RT = D / 64;  // row tiles per wave for D-row outputs
  // ---- Tm = -W^T Kr  [D x D]
  {
    f4 acc[RT][D / 16];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) acc[rt][nt] = zero4();
    for (int kk = 0; kk < 64; kk += KS) {
      Frag a[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        a[rt] = MM::load(sWT + ((w * RT + rt) * 16 + (lane & 15)) * TT + kk + (lane >> 4) * KPL);
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        const Frag b = MM::load(sKrT + (nt * 16 + (lane & 15)) * TT + kk + (lane >> 4) * KPL);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = MM::mma(a[rt], b, acc[rt][nt]);
      }
    }
    T* dst = Tm + ch * D * D;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt)
        store_c<T>(dst, D, (w * RT + rt) * 16, nt * 16, -acc[rt][nt], lane);
  }
  // ---- PT = Qd^T - W^T Mqk^T  [D x 64]
  {
    f4 acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[rt][nt] = zero4();
    for (int kk = 0; kk < 64; kk += KS) {
      Frag a[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        a[rt] = MM::load(sWT + ((w * RT + rt) * 16 + (lane & 15)) * TT + kk + (lane >> 4) * KPL);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const Frag b = MM::from_f32(sM + (nt * 16 + (lane & 15)) * CC + kk + (lane >> 4) * KPL);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = MM::mma(a[rt], b, acc[rt][nt]);
      }
    }
    T* dst = PT + ch * D * 64;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int r = nt * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = (w * RT + rt) * 16 + (lane >> 4) * 4 + j;
          const float qd = to_f(sQ[r * PN + i]) * ex2(sG[r * NF + i]);
          dst[i * 64 + r] = from_f<T>(qd - acc[rt][nt][j]);
        }
      }
  }
  if (tid < D) eGT[ch * D + tid] = ex2(sG[63 * NF + tid]);
}

template <typename T, int D>
static hipError_t prep_t(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  dim3 grid((unsigned)s.NC, (unsigned)s.H);
  hipLaunchKernelGGL((k_prep<T, D>), grid, dim3(NTHR), 0, st, p.chunks, s.H, (const T*)p.q,
                     (const T*)p.k, p.g_raw, p.beta, p.A_log, (T*)p.Tm, (T*)p.PT, p.eGT,
                     (T*)p.INV, (T*)p.INVT, (T*)p.MqkT);
  return hipGetLastError();
}

hipError_t launch_prep(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  if (s.NC == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? prep_t<bf16, 128>(s, p, st) : prep_t<bf16, 64>(s, p, st);
  return prep_t<float, 64>(s, p, st);
}

}  // namespace kda
