// kda_grad.hip -- the data-parallel gradient pass, one workgroup per chunk-head.
//
// Chunk quantities (G: in-chunk cumulative gate, Kd = K e^G, Kr = K e^{G_T-G},
// Qd = Q e^G; INV, Mqk from the prep pass; S_in the chunk's start state; dS_out
// the state gradient at its end, from the scan):
//   grad1 ([KB] part 2, B1 and the kdS / dbeta part of B2):
//     Y = V - Kd S_in,  U = INV diag(beta) Y,
//     dU = Mqk^T dO + Kr dS_out,  dvcorr = INV^T dU,  dv = beta . dvcorr,
//     dbeta_r  = sum_d dvcorr_rd Y_rd                      (first part)
//   grad2 ([KB] part 2, B2 and B3 with the inlined gate epilogue K1):
//     dKr = U dS_out^T,  dQd0 = dO S_in^T,  dKd0 = dvcorr S_in^T,
//     p_i = sum_d S_in[i,d] dS_out[i,d],
//     dMqk = tril(dO U^T),  dL = -stril(dvcorr U^T),
//     dq   = e^G dQd0 + sum_{s<=r} dMqk_rs k_s e^{G_r-G_s}
//     dk_d = beta_r (-e^G dKd0 + sum_{s<r} dL_rs k_s e^{G_r-G_s})
//     dk_i = sum_{r>=s} (dMqk_rs q_r + beta_r dL_rs k_r) e^{G_r-G_s}
//     dk_r = e^{G_T-G} dKr,  dk = dk_d + dk_i + dk_r
//     dbeta_r += sum_s dL_rs A_rs  (= sum_i k_ri (dk_d/beta_r + e^G dKd0)_ri)
//     dG = q.dq + k.(dk_d - dk_i - dk_r);  dG_last += sum_r k.dk_r + e^{G_T}.p
//     dg = reverse cumsum of dG over the chunk;  dg_raw = dg . (-e^{A_log} sigmoid(g_raw))
//     dA_log partial = sum dg . g
// The gate epilogue stays in fp32 ([KB] part 2, B3: the signed combination
// dk_d - dk_i - dk_r cancels strongly).  Pairwise decays e^{G_r-G_s} are formed
// without exp(-G): across 16-row blocks through an anchor row between them (MFMA),
// inside a 16-row diagonal block by running products of per-token decays (VALU).
#include "kda_dev.h"
#include "kda_launch.h"

namespace kda {

__device__ __forceinline__ float softplus_g(float x) {
  return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
}

// Cooperative load of the chunk gate: sG[r][i] = log2(e) * G_r[i] (rows past the
// chunk end repeat the last value, i.e. g = 0 there).
template <int D, int NF>
__device__ __forceinline__ void load_gate(float* sG, const float* __restrict__ g_raw, size_t t0,
                                          int Lr, int H, int h, float aA, int tid) {
  constexpr int PARTS = NTHR / D;
  constexpr int RPP = 64 / PARTS;
  const int i = tid % D, part = tid / D;
  float run = 0.f;
  for (int rr = 0; rr < RPP; ++rr) {
    const int r = part * RPP + rr;
    float g = 0.f;
    if (r < Lr) g = -aA * softplus_g(g_raw[((t0 + r) * H + h) * D + i]);
    run += g * LOG2E;
    sG[r * NF + i] = run;
  }
  __syncthreads();
  float add = 0.f;
  for (int pp = 0; pp < part; ++pp) add += sG[(pp * RPP + RPP - 1) * NF + i];
  __syncthreads();
  if (part > 0)
    for (int rr = 0; rr < RPP; ++rr) sG[(part * RPP + rr) * NF + i] += add;
  __syncthreads();
}

// ===========================================================================
// grad1: wave w owns the 16 rows of block w, all V columns.
// ===========================================================================
template <typename T, int D> struct G1Lds {
  using P = Pitch<T, D>;
  static constexpr int PD = D + 16 / (int)sizeof(T);  // [D][D] transposed state pitch
  static constexpr int G_OFF = 0;
  static constexpr int G_SZ = 64 * P::NF * 4;
  static constexpr int ST_OFF = G_OFF + G_SZ;          // S_in^T, later dS_out^T: [V][K]
  static constexpr int ST_SZ = D * PD * (int)sizeof(T);
  static constexpr int YT_OFF = ST_OFF + ST_SZ;        // (beta Y)^T, later dU^T: [V][64]
  static constexpr int TT_SZ = D * P::TT * (int)sizeof(T);
  static constexpr int OT_OFF = YT_OFF + TT_SZ;        // dO^T: [V][64]
  static constexpr int B_OFF = OT_OFF + TT_SZ;
  static constexpr int TOTAL = B_OFF + 256;
};

template <typename T, int D>
__device__ __forceinline__ void load_state_t(T* dst, const T* __restrict__ src, int tid) {
  // dst[d * PD + i] = src[i * D + d]
  constexpr int PD = D + 16 / (int)sizeof(T);
  constexpr int EPV = 16 / (int)sizeof(T);
  constexpr int VPR = D / EPV;
  for (int idx = tid; idx < D * VPR; idx += NTHR) {
    const int i = idx / VPR, sv = idx % VPR;
    const uint4 x = *(const uint4*)(src + (size_t)i * D + sv * EPV);
    const T* e = (const T*)&x;
#pragma unroll
    for (int q = 0; q < EPV; ++q) dst[(sv * EPV + q) * PD + i] = e[q];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_grad1(const ChunkInfo* __restrict__ chunks, int H,
                                               const T* __restrict__ k, const T* __restrict__ v,
                                               const T* __restrict__ dO,
                                               const float* __restrict__ g_raw,
                                               const float* __restrict__ beta,
                                               const float* __restrict__ A_log,
                                               const T* __restrict__ h_saved,
                                               const T* __restrict__ dstates,
                                               const T* __restrict__ INV, const T* __restrict__ INVT,
                                               const T* __restrict__ MqkT, T* __restrict__ dv,
                                               T* __restrict__ Uo, T* __restrict__ dvco,
                                               float* __restrict__ dbeta) {
  using L = G1Lds<T, D>;
  using P = Pitch<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int KS = MM::KS, KPL = MM::KPL;
  constexpr int NF = P::NF, TT = P::TT, PD = L::PD;
  constexpr int NT = D / 16;   // column tiles over V
  constexpr int NK = D / KS;   // k-steps over K
  constexpr int NS = 64 / KS;  // k-steps over the chunk
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  float* sG = (float*)(smem + L::G_OFF);
  T* sST = (T*)(smem + L::ST_OFF);
  T* sYT = (T*)(smem + L::YT_OFF);
  T* sOT = (T*)(smem + L::OT_OFF);
  float* sBeta = (float*)(smem + L::B_OFF);

  const int c = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const ChunkInfo ci = chunks[c];
  const size_t t0 = ci.t0;
  const int Lr = ci.len;
  const size_t ch = (size_t)c * H + h;
  const size_t DD = (size_t)D * D;

  if (tid < 64) sBeta[tid] = tid < Lr ? beta[(t0 + tid) * H + h] : 0.f;
  load_state_t<T, D>(sST, h_saved + ch * DD, tid);
  {  // dO^T
    constexpr int EPV = 16 / (int)sizeof(T);
    constexpr int VPR = D / EPV;
    for (int idx = tid; idx < 64 * VPR; idx += NTHR) {
      const int r = idx / VPR, sv = idx % VPR;
      uint4 x = {0u, 0u, 0u, 0u};
      if (r < Lr) x = *(const uint4*)(dO + ((t0 + r) * H + h) * D + sv * EPV);
      const T* e = (const T*)&x;
#pragma unroll
      for (int q = 0; q < EPV; ++q) sOT[(sv * EPV + q) * TT + r] = e[q];
    }
  }
  load_gate<D, NF>(sG, g_raw, t0, Lr, H, h, __expf(A_log[h]), tid);

  const int R = w;
  const int arow = 16 * R + (lane & 15);  // A-operand row of this lane
  // raw k fragments of this lane's row
  float kraw[NK][KPL];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    if (arow < Lr)
      load_f<T, KPL>(k + ((t0 + arow) * H + h) * D + kk * KS + (lane >> 4) * KPL, kraw[kk]);
    else
#pragma unroll
      for (int j = 0; j < KPL; ++j) kraw[kk][j] = 0.f;
  }
  // ---- Y = V - Kd S_in
  f4 Y[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) Y[nt] = zero4();
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    float kd[KPL];
    const int i0 = kk * KS + (lane >> 4) * KPL;
#pragma unroll
    for (int j = 0; j < KPL; ++j) kd[j] = kraw[kk][j] * ex2(sG[arow * NF + i0 + j]);
    const Frag a = MM::from_vals(kd);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const Frag b = MM::load(sST + (nt * 16 + (lane & 15)) * PD + i0);
      Y[nt] = MM::mma(a, b, Y[nt]);
    }
  }
  const int crow = 16 * R + (lane >> 4) * 4;  // first C row of this lane
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int d = nt * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = crow + j;
      const float vv = r < Lr ? to_f(v[((t0 + r) * H + h) * D + d]) : 0.f;
      Y[nt][j] = vv - Y[nt][j];
    }
    f4 by;
#pragma unroll
    for (int j = 0; j < 4; ++j) by[j] = sBeta[crow + j] * Y[nt][j];
    store_ct<T>(sYT, TT, 16 * R, nt * 16, by, lane);
  }
  __syncthreads();
  // S_in^T is dead: bring in dS_out^T
  load_state_t<T, D>(sST, dstates + ch * DD, tid);
  // ---- U = INV (beta Y)
  {
    f4 U[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) U[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
      const Frag a = MM::load(INV + ch * 4096 + arow * 64 + ks * KS + (lane >> 4) * KPL);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const Frag b = MM::load(sYT + (nt * 16 + (lane & 15)) * TT + ks * KS + (lane >> 4) * KPL);
        U[nt] = MM::mma(a, b, U[nt]);
      }
    }
    T* dst = Uo + ch * 64 * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) store_c<T>(dst, D, 16 * R, nt * 16, U[nt], lane);
  }
  __syncthreads();  // dS_out^T is in; (beta Y)^T is dead
  // ---- dU = Mqk^T dO + Kr dS_out
  f4 dU[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) dU[nt] = zero4();
#pragma unroll
  for (int ks = 0; ks < NS; ++ks) {
    const Frag a = MM::load(MqkT + ch * 4096 + arow * 64 + ks * KS + (lane >> 4) * KPL);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const Frag b = MM::load(sOT + (nt * 16 + (lane & 15)) * TT + ks * KS + (lane >> 4) * KPL);
      dU[nt] = MM::mma(a, b, dU[nt]);
    }
  }
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    float kr[KPL];
    const int i0 = kk * KS + (lane >> 4) * KPL;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      kr[j] = kraw[kk][j] * ex2(sG[63 * NF + i0 + j] - sG[arow * NF + i0 + j]);
    const Frag a = MM::from_vals(kr);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const Frag b = MM::load(sST + (nt * 16 + (lane & 15)) * PD + i0);
      dU[nt] = MM::mma(a, b, dU[nt]);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) store_ct<T>(sYT, TT, 16 * R, nt * 16, dU[nt], lane);
  __syncthreads();
  // ---- dvcorr = INV^T dU;  dv = beta . dvcorr;  dbeta part 1
  {
    f4 dvc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dvc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
      const Frag a = MM::load(INVT + ch * 4096 + arow * 64 + ks * KS + (lane >> 4) * KPL);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const Frag b = MM::load(sYT + (nt * 16 + (lane & 15)) * TT + ks * KS + (lane >> 4) * KPL);
        dvc[nt] = MM::mma(a, b, dvc[nt]);
      }
    }
    T* dst = dvco + ch * 64 * D;
    float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      store_c<T>(dst, D, 16 * R, nt * 16, dvc[nt], lane);
      const int d = nt * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = crow + j;
        db[j] += dvc[nt][j] * Y[nt][j];
        if (r < Lr) dv[((t0 + r) * H + h) * D + d] = from_f<T>(sBeta[r] * dvc[nt][j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float s = sum16(db[j]);
      const int r = crow + j;
      if ((lane & 15) == 0 && r < Lr) dbeta[(t0 + r) * H + h] = s;
    }
  }
}

// ===========================================================================
// grad2: wave w owns key channels [w*D/4, (w+1)*D/4), all 64 rows.
// ===========================================================================
template <typename T, int D> struct G2Lds {
  using P = Pitch<T, D>;
  static constexpr int G_OFF = 0;
  static constexpr int G_SZ = 64 * P::NF * 4;
  static constexpr int Q_OFF = G_OFF + G_SZ;
  static constexpr int QK_SZ = 64 * P::N * (int)sizeof(T);
  static constexpr int K_OFF = Q_OFF + QK_SZ;
  static constexpr int DM_OFF = K_OFF + QK_SZ;       // dMqk fp32 [64][CC]
  static constexpr int CC_SZ = 64 * P::CC * 4;
  static constexpr int DL_OFF = DM_OFF + CC_SZ;      // dL fp32 [64][CC]
  static constexpr int DG_OFF = DL_OFF + CC_SZ;      // per-wave diagonal-block outputs
  static constexpr int DGW = 3 * 64 * 17;            // floats per wave
  static constexpr int B_OFF = DG_OFF + 4 * DGW * 4;
  static constexpr int DB_OFF = B_OFF + 256;         // [4][64] dbeta partials
  static constexpr int RED_OFF = DB_OFF + 4 * 64 * 4;
  static constexpr int TOTAL = RED_OFF + 64;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void k_grad2(const ChunkInfo* __restrict__ chunks, int H,
                                               const T* __restrict__ q, const T* __restrict__ k,
                                               const T* __restrict__ dO,
                                               const float* __restrict__ g_raw,
                                               const float* __restrict__ beta,
                                               const float* __restrict__ A_log,
                                               const T* __restrict__ h_saved,
                                               const T* __restrict__ dstates,
                                               const T* __restrict__ U, const T* __restrict__ dvc,
                                               T* __restrict__ dq, T* __restrict__ dk,
                                               float* __restrict__ dg_raw,
                                               float* __restrict__ dbeta,
                                               float* __restrict__ dAl_part) {
  using L = G2Lds<T, D>;
  using P = Pitch<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int KS = MM::KS, KPL = MM::KPL;
  constexpr int NF = P::NF, PN = P::N, CC = P::CC;
  constexpr int NK = D / KS;   // k-steps over V
  constexpr int NKT = D / 64;  // key-channel tiles per wave
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  float* sG = (float*)(smem + L::G_OFF);
  T* sQ = (T*)(smem + L::Q_OFF);
  T* sK = (T*)(smem + L::K_OFF);
  float* sDM = (float*)(smem + L::DM_OFF);
  float* sDL = (float*)(smem + L::DL_OFF);
  float* sDG = (float*)(smem + L::DG_OFF);
  float* sBeta = (float*)(smem + L::B_OFF);
  float* sDB = (float*)(smem + L::DB_OFF);
  float* sRed = (float*)(smem + L::RED_OFF);

  const int c = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const ChunkInfo ci = chunks[c];
  const size_t t0 = ci.t0;
  const int Lr = ci.len;
  const size_t ch = (size_t)c * H + h;
  const size_t DD = (size_t)D * D;
  const float aA = __expf(A_log[h]);

  {
    constexpr int VPR = D * (int)sizeof(T) / 16;
    for (int idx = tid; idx < 64 * VPR; idx += NTHR) {
      const int r = idx / VPR, vv = idx % VPR;
      uint4 xq = {0u, 0u, 0u, 0u}, xk = {0u, 0u, 0u, 0u};
      if (r < Lr) {
        const size_t off = ((t0 + r) * H + h) * D;
        xq = ((const uint4*)(q + off))[vv];
        xk = ((const uint4*)(k + off))[vv];
      }
      *(uint4*)((char*)(sQ + r * PN) + vv * 16) = xq;
      *(uint4*)((char*)(sK + r * PN) + vv * 16) = xk;
    }
  }
  if (tid < 64) sBeta[tid] = tid < Lr ? beta[(t0 + tid) * H + h] : 0.f;
  load_gate<D, NF>(sG, g_raw, t0, Lr, H, h, aA, tid);

  const T* Uc = U + ch * 64 * D;
  const T* Vc = dvc + ch * 64 * D;
  // ---- dMqk = tril(dO U^T), dL = -stril(dvcorr U^T); wave w -> rows of block w
  {
    const int r = 16 * w + cl;
    f4 am[4], al[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) am[st] = al[st] = zero4();
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int d0 = kk * KS + g4 * KPL;
      Frag ao, av;
      if (r < Lr)
        ao = MM::load(dO + ((t0 + r) * H + h) * D + d0);
      else {
        float z[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) z[j] = 0.f;
        ao = MM::from_vals(z);
      }
      av = MM::load(Vc + r * D + d0);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const Frag b = MM::load(Uc + (st * 16 + cl) * D + d0);
        am[st] = MM::mma(ao, b, am[st]);
        al[st] = MM::mma(av, b, al[st]);
      }
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int s = st * 16 + cl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 16 * w + g4 * 4 + j;
        sDM[rr * CC + s] = (s <= rr) ? am[st][j] : 0.f;
        sDL[rr * CC + s] = (s < rr) ? -al[st][j] : 0.f;
      }
    }
  }
  __syncthreads();

  float dal = 0.f;   // dA_log partial of this lane
  float dbp[4][4];   // dbeta partials: [row tile][j]
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) dbp[rt][j] = 0.f;
  float* myDG = sDG + w * L::DGW;  // [3][64][17]

#pragma unroll 1
  for (int it = 0; it < NKT; ++it) {
    const int i0 = (w * NKT + it) * 16;
    const int ic = i0 + cl;  // this lane's key channel (C/B column)
    // ---- 16x16 diagonal blocks (VALU, running products of per-token decays).
    // lane -> (block R = g4, channel ic); writes [3][64][17] into this wave's area.
    {
      const int R = g4, r0 = 16 * R;
      float kk_[16], ff[16], dki[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        kk_[s] = to_f(sK[(r0 + s) * PN + ic]);
        dki[s] = 0.f;
        ff[s] = 1.f;
      }
      float gprev = sG[r0 * NF + ic];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float gr = sG[(r0 + r) * NF + ic];
        if (r > 0) {
          const float ar = ex2(gr - gprev);
#pragma unroll
          for (int s = 0; s < r; ++s) ff[s] *= ar;
        }
        gprev = gr;
        const float qr = to_f(sQ[(r0 + r) * PN + ic]);
        const float br = sBeta[r0 + r];
        float x1 = 0.f, x2 = 0.f;
#pragma unroll
        for (int s = 0; s <= r; ++s) {
          const float m = sDM[(r0 + r) * CC + r0 + s];
          const float l = sDL[(r0 + r) * CC + r0 + s];
          const float kf = kk_[s] * ff[s];
          x1 += m * kf;
          x2 += l * kf;
          dki[s] += (m * qr + br * l * kk_[r]) * ff[s];
        }
        myDG[(0 * 64 + r0 + r) * 17 + cl] = x1;
        myDG[(1 * 64 + r0 + r) * 17 + cl] = x2;
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) myDG[(2 * 64 + r0 + s) * 17 + cl] = dki[s];
    }
    __builtin_amdgcn_wave_barrier();

    // ---- across 16-row blocks (anchored MFMA at fp32 accuracy), added into the same buffer
    //   X1 = sum_{s<a} dMqk_rs k_s e^{G_a-G_s},  X2 = sum_{s<a} dL_rs k_s e^{G_a-G_s}  (a = 16R)
    //   Z  = sum_{r>=b} (dMqk_rs q_r + beta_r dL_rs k_r) e^{G_r-G_b}                (b = 16(S+1))
#pragma unroll 1
    for (int R = 1; R < 4; ++R) {
      const int a = 16 * R;
      const float ga = sG[a * NF + ic];
      f4 X1 = zero4(), X2 = zero4();
      for (int kk = 0; kk < a; kk += KS) {
        float bv[KPL], am[KPL], al[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int s = kk + g4 * KPL + j;
          const bool ok = s < a;
          bv[j] = ok ? to_f(sK[s * PN + ic]) * ex2(ga - sG[s * NF + ic]) : 0.f;
          const int rr = 16 * R + cl;
          am[j] = ok ? sDM[rr * CC + s] : 0.f;
          al[j] = ok ? sDL[rr * CC + s] : 0.f;
        }
        X1 = MM::mma3(am, bv, X1);
        X2 = MM::mma3(al, bv, X2);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * R + g4 * 4 + j;
        const float sc = ex2(sG[r * NF + ic] - ga);
        myDG[(0 * 64 + r) * 17 + cl] += X1[j] * sc;
        myDG[(1 * 64 + r) * 17 + cl] += X2[j] * sc;
      }
    }
#pragma unroll 1
    for (int S = 0; S < 3; ++S) {
      const int bb = 16 * (S + 1);
      const float gb = sG[bb * NF + ic];
      f4 Z = zero4();
      for (int kk = (bb / KS) * KS; kk < 64; kk += KS) {
        float bq[KPL], bk[KPL], a1[KPL], a2[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int r = kk + g4 * KPL + j;
          const bool ok = r >= bb;
          const float e = ok ? ex2(sG[r * NF + ic] - gb) : 0.f;
          bq[j] = to_f(sQ[r * PN + ic]) * e;
          bk[j] = to_f(sK[r * PN + ic]) * e;
          const int ss = 16 * S + cl;
          a1[j] = ok ? sDM[r * CC + ss] : 0.f;
          a2[j] = ok ? sBeta[r] * sDL[r * CC + ss] : 0.f;
        }
        Z = MM::mma3(a1, bq, Z);
        Z = MM::mma3(a2, bk, Z);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 16 * S + g4 * 4 + j;
        myDG[(2 * 64 + s) * 17 + cl] += Z[j] * ex2(gb - sG[s * NF + ic]);
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- dKr = U dS_out^T, dQd0 = dO S_in^T, dKd0 = dvcorr S_in^T, p
    f4 aKr[4], aQd[4], aKd[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) aKr[rt] = aQd[rt] = aKd[rt] = zero4();
    float pp = 0.f;
    const T* Sin = h_saved + ch * DD + (size_t)ic * D;
    const T* dSo = dstates + ch * DD + (size_t)ic * D;
#pragma unroll 1
    for (int kk = 0; kk < NK; ++kk) {
      const int d0 = kk * KS + g4 * KPL;
      const Frag bS = MM::load(Sin + d0);
      const Frag bD = MM::load(dSo + d0);
      pp += MM::dot(bS, bD);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = rt * 16 + cl;
        const Frag aU = MM::load(Uc + r * D + d0);
        const Frag aV = MM::load(Vc + r * D + d0);
        Frag aO;
        if (r < Lr)
          aO = MM::load(dO + ((t0 + r) * H + h) * D + d0);
        else {
          float z[KPL];
#pragma unroll
          for (int j = 0; j < KPL; ++j) z[j] = 0.f;
          aO = MM::from_vals(z);
        }
        aKr[rt] = MM::mma(aU, bD, aKr[rt]);
        aQd[rt] = MM::mma(aO, bS, aQd[rt]);
        aKd[rt] = MM::mma(aV, bS, aKd[rt]);
      }
    }
    pp += __shfl_xor(pp, 16);
    pp += __shfl_xor(pp, 32);  // p[ic] on every lane of column cl


    // ---- combine, gate gradient, reverse cumsum, stores
    const float gT = sG[63 * NF + ic];
    float dG[4][4], dkr_col = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = rt * 16 + g4 * 4 + j;
        const float Gr = sG[r * NF + ic];
        const float eG = ex2(Gr);
        const float qv = to_f(sQ[r * PN + ic]);
        const float kv = to_f(sK[r * PN + ic]);
        const float br = sBeta[r];
        const float x1 = myDG[(0 * 64 + r) * 17 + cl];
        const float x2 = myDG[(1 * 64 + r) * 17 + cl];
        const float dki = myDG[(2 * 64 + r) * 17 + cl];
        const float dqv = eG * aQd[rt][j] + x1;
        const float dkd_base = -eG * aKd[rt][j] + x2;
        const float dkd = br * dkd_base;
        const float dkr = ex2(gT - Gr) * aKr[rt][j];
        const float dkv = dkd + dki + dkr;
        dG[rt][j] = qv * dqv + kv * (dkd - dki - dkr);
        dkr_col += kv * dkr;
        dbp[rt][j] += kv * x2;
        if (r < Lr) {
          const size_t o = ((t0 + r) * H + h) * D + ic;
          dq[o] = from_f<T>(dqv);
          dk[o] = from_f<T>(dkv);
        }
      }
    }
    // column sums over all 64 rows: lanes cl, cl+16, cl+32, cl+48
    dkr_col += __shfl_xor(dkr_col, 16);
    dkr_col += __shfl_xor(dkr_col, 32);
    const float extra = dkr_col + ex2(gT) * pp;
    if (g4 == 3) dG[3][3] += extra;  // row 63
    // reverse cumsum over r = 16 rt + 4 g4 + j
    float carry = 0.f;
#pragma unroll
    for (int rt = 3; rt >= 0; --rt) {
      const float tot = dG[rt][0] + dG[rt][1] + dG[rt][2] + dG[rt][3];
      const float t1 = __shfl(tot, cl + 16), t2 = __shfl(tot, cl + 32), t3 = __shfl(tot, cl + 48);
      const float t0v = __shfl(tot, cl);
      float after = carry;  // rows of later groups in this tile and of later tiles
      if (g4 < 3) after += t3;
      if (g4 < 2) after += t2;
      if (g4 < 1) after += t1;
      carry += t0v + t1 + t2 + t3;
      float run = after;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        run += dG[rt][j];
        const int r = rt * 16 + g4 * 4 + j;
        if (r < Lr) {
          const size_t o = ((t0 + r) * H + h) * D + ic;
          const float x = g_raw[o];
          const float sg = 1.f / (1.f + __expf(-x));
          dg_raw[o] = run * (-aA * sg);
          dal += run * (-aA * softplus_g(x));
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- dbeta second part: sum_s dL_rs A_rs = sum_i k_ri x2_ri, reduced over waves
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float s = sum16(dbp[rt][j]);
      if (cl == 0) sDB[w * 64 + rt * 16 + g4 * 4 + j] = s;
    }
  dal = sum64(dal);
  if (lane == 0) sRed[w] = dal;
  __syncthreads();
  if (tid < 64 && tid < Lr) {
    const size_t o = (t0 + tid) * H + h;
    dbeta[o] = dbeta[o] + ((sDB[tid] + sDB[64 + tid]) + (sDB[128 + tid] + sDB[192 + tid]));
  }
  if (tid == 0) dAl_part[ch] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
}

template <typename T, int D>
static hipError_t grad1_t(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  dim3 grid((unsigned)s.NC, (unsigned)s.H);
  hipLaunchKernelGGL((k_grad1<T, D>), grid, dim3(NTHR), 0, st, p.chunks, s.H, (const T*)p.k,
                     (const T*)p.v, (const T*)p.dO, p.g_raw, p.beta, p.A_log,
                     (const T*)p.h_saved, (const T*)p.dstates, (const T*)p.INV,
                     (const T*)p.INVT, (const T*)p.MqkT, (T*)p.dv, (T*)p.U, (T*)p.dvc, p.dbeta);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t grad2_t(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  dim3 grid((unsigned)s.NC, (unsigned)s.H);
  hipLaunchKernelGGL((k_grad2<T, D>), grid, dim3(NTHR), 0, st, p.chunks, s.H, (const T*)p.q,
                     (const T*)p.k, (const T*)p.dO, p.g_raw, p.beta, p.A_log,
                     (const T*)p.h_saved, (const T*)p.dstates, (const T*)p.U, (const T*)p.dvc,
                     (T*)p.dq, (T*)p.dk, p.dg_raw, p.dbeta, p.dAl_part);
  return hipGetLastError();
}

hipError_t launch_grad1(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  if (s.NC == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? grad1_t<bf16, 128>(s, p, st) : grad1_t<bf16, 64>(s, p, st);
  return grad1_t<float, 64>(s, p, st);
}

hipError_t launch_grad2(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  if (s.NC == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? grad2_t<bf16, 128>(s, p, st) : grad2_t<bf16, 64>(s, p, st);
  return grad2_t<float, 64>(s, p, st);
}

}  // namespace kda
