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

template <typename T, int D> struct PL {
  static constexpr int NW = D / 16;               // waves
  static constexpr int NT = NW * 64;
  static constexpr int ES = (int)sizeof(T);
  static constexpr int HALVES = NW / 4;           // column halves of W per row block
  static constexpr int PGN = D + 4;               // sG [64][PGN] fp32, natural
  static constexpr int PN = D + 16 / ES;          // [64][PN] tiles of T, natural
  static constexpr int PC = 68;                   // [64][PC] fp32
  static constexpr int PTM = D + 16 / ES;         // Tm staging [D][PTM] of T
  static constexpr int PPT = 64 + 16 / ES;        // PT staging [D][PPT] of T
  static constexpr int G_SZ = 64 * PGN * 4;
  static constexpr int N_SZ = 64 * PN * ES;
  static constexpr int C_SZ = 64 * PC * 4;
  static constexpr int G_OFF = 0;
  static constexpr int Q_OFF = G_OFF + G_SZ;
  static constexpr int K_OFF = Q_OFF + N_SZ;    // k, later W
  static constexpr int M_OFF = K_OFF + N_SZ;    // Mqk
  static constexpr int KR_OFF = M_OFF + C_SZ;   // Kr
  static constexpr int A_OFF = KR_OFF + N_SZ;   // L = diag(beta) A
  static constexpr int INV_OFF = A_OFF + C_SZ;  // INV
  static constexpr int KD_OFF = INV_OFF + C_SZ; // beta Kd
  static constexpr int SCR_OFF = KD_OFF + N_SZ; // INV block-substitution scratch
  static constexpr int SCR_SZ = 4 * 16 * 17 * 4;
  static constexpr int B_OFF = SCR_OFF + SCR_SZ;
  static constexpr int TOT_OFF = B_OFF + 256;     // gate totals of the 4 row parts [4][D]
  static constexpr int TOTAL = TOT_OFF + 4 * D * 4;
  // Tm and PT staging, over A, INV, Kd and the scratch once W is formed
  static constexpr int TMS_OFF = A_OFF;
  static constexpr int PTS_OFF = TMS_OFF + D * PTM * ES;
  static_assert(PTS_OFF + D * PPT * ES <= B_OFF, "staging fits the dead region");
  // SCAN (backward): the state tile [D][PSS] and the chunk's dO tile [64][PSS] (act dtype)
  // over the A, INV, Kd and scratch tiles, dead once W is formed and INV stored; the tile
  // X = -(Kr dS + Mqk^T dO) [64][PSX] over the gate tile, dead once Qd and e^{G_T} are
  // formed.  32-byte row pads: the transposing operand reads of 8 consecutive rows hit 64
  // distinct banks (fp32 X: 16-byte pads, to fit the gate tile).
  static constexpr int PSS = D + 32 / ES;
  static constexpr int PSX = ES == 2 ? PSS : D + 4;
  static constexpr int SS_OFF = A_OFF;
  static constexpr int SO_OFF = SS_OFF + D * PSS * ES;
  static constexpr int SX_OFF = G_OFF;
  static_assert(SO_OFF + 64 * PSS * ES <= B_OFF, "state and dO tiles fit the dead region");
  static_assert(64 * PSX * ES <= G_SZ, "X fits the gate tile");
  // SCAN in forward mode: the state tile [D][PSS] and the X tile [64][PSS] over the beta v,
  // INV, Kd and scratch tiles, dead once W and Uv are formed
  static constexpr int FS_OFF = A_OFF;
  static constexpr int FX_OFF = FS_OFF + D * PSS * ES;
  static_assert(FX_OFF + 64 * PSS * ES <= B_OFF, "forward scan tiles fit");
};

// GV: gate bias present (or its gradient asked for); without it the bias is not read.
// FWD: the forward's per-chunk operands instead of the backward's (see the end of the
// item loop).  QN: q and k are L2-normalised per row as they enter LDS (every quantity
// below is then formed from the normalised rows).
// SCAN (every sequence has at least one chunk): the state scan runs inside this kernel
// instead of a separate one.  A workgroup owns whole (sequence, head) units and walks
// each unit's chunks, carrying the K x V state in fp32 MFMA accumulators.  The units,
// sorted by chunk count (longest first: `order` holds the sequences in that order, heads
// fastest), are dealt to the workgroups in a snake: unit k of workgroup g is position
// k G + g for even k and k G + G - 1 - g for odd k, which pairs long units with short ones.  Backward: chunks last to
// first, the state gradient dS from dht: once a chunk's W is formed it stores dS_out of the
// chunk and applies dS <- exp(G_T) . dS + Tm dS + PT dO in the factored form
// exp(G_T) . dS + Qd^T dO - W^T (Kr dS + Mqk^T dO), so Tm and PT are never formed and
// nothing of the scan goes to memory but dS_out; dh0 after a unit's first chunk.  Forward: chunks first
// to last, the state S from h0: with W and Uv = INV diag(beta) V formed (Uv kept in
// registers) it stores h_saved, forms X = Uv - W S, O = Qd S + Mqk X and
// S <- exp(G_T) . S + Kr^T X, and stores O; ht after a unit's last chunk.  In forward
// mode the scan arguments are reused: dht = h0, dstates = h_saved, dh0 = ht.
template <typename T, int D, bool GV, bool FWD, bool QN, bool SCAN>
__global__ __launch_bounds__(4 * D) void k_prep(const ChunkInfo* __restrict__ chunks, int NC, int H,
                                                const T* __restrict__ q, const T* __restrict__ k,
                                                const float* __restrict__ g_raw,
                                                const float* __restrict__ beta,
                                                const float* __restrict__ A_log,
                                                const float* __restrict__ dt_bias, int has_db,
                                                float gu,
                                                T* __restrict__ Tm, T* __restrict__ PT,
                                                float* __restrict__ eGT, T* __restrict__ INVo,
                                                T* __restrict__ MqkTo, const T* __restrict__ v,
                                                T* __restrict__ Wn, T* __restrict__ KrT,
                                                T* __restrict__ UvT, T* __restrict__ Qd,
                                                T* __restrict__ Mq, const T* __restrict__ dO,
                                                const float* __restrict__ dht,
                                                T* __restrict__ dstates,
                                                float* __restrict__ dh0,
                                                const int* __restrict__ seq_off,
                                                const int* __restrict__ order, int NS,
                                                T* __restrict__ o, T* __restrict__ dUo) {
  using L = PL<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int NW = L::NW, NT = L::NT, HALVES = L::HALVES;
  constexpr int KS = MM::KS, KPL = MM::KPL;
  constexpr int PGN = L::PGN, PN = L::PN, PC = L::PC, PTM = L::PTM, PPT = L::PPT;
  constexpr int NKC = 64 / KS;
  // scan mode with eight waves: Qd is formed by the waves INV step 1 leaves idle
  constexpr bool QD_EARLY = SCAN && NW == 8;
  constexpr int DH = D / HALVES;           // columns of W per wave
  constexpr int EPV = 16 / L::ES;          // elements per 16-byte vector
  constexpr int VPR = D / EPV;             // vectors per D-long row
  constexpr int NLT = 64 * VPR / NT;       // vectors per thread, 64 x D tile
  static_assert(64 * VPR % NT == 0 && NT == 4 * D, "tile split");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  float* sG = (float*)(smem + L::G_OFF);
  T* sQ = (T*)(smem + L::Q_OFF);
  T* sK = (T*)(smem + L::K_OFF);
  T* sW = sK;
  float* sM = (float*)(smem + L::M_OFF);
  T* sKr = (T*)(smem + L::KR_OFF);
  float* sA = (float*)(smem + L::A_OFF);
  float* sINV = (float*)(smem + L::INV_OFF);
  T* sKd = (T*)(smem + L::KD_OFF);
  float* sScr = (float*)(smem + L::SCR_OFF);
  float* sBeta = (float*)(smem + L::B_OFF);
  T* sTm = (T*)(smem + L::TMS_OFF);
  T* sPT = (T*)(smem + L::PTS_OFF);

  const size_t rs = (size_t)H * D;
  const int items = NC * H;
  const int tid0 = threadIdx.x;

  // Persistent: one workgroup fills a CU's LDS, so each workgroup walks the
  // (chunk, head) items with stride gridDim.x (chunk fastest: item = head * NC + chunk;
  // head-fastest order measured slower here) and holds the next item's g_raw,
  // beta, q and k in registers while it works on the current one. Rows beyond
  // the chunk are zero (q, k) or masked at the cumsum (g_raw).
  float rg[16], rbeta, rdb;
  u32x4 rq[NLT], rk[NLT];
  // parts: 1 = g_raw rows 0-7 of the thread's 16 and beta, 2 = g_raw rows 8-15,
  // 4 = q, 8 = k.  A CU keeps a bounded number of cache lines in flight and a wave
  // stalls at issue once that is reached, so the loads go out in two portions,
  // at the start and at the end of the A/Mqk phase, not in one burst.
  auto issue_loads = [&](int it, int t, const ChunkInfo ci, const int parts) {
    const int h = it / NC;
    const size_t hD = (size_t)h * D;
    // 4 parts of 16 rows; a part is one (D = 64) or two (D = 128) whole waves, so
    // the row addresses are uniform and the 16 loads share one lane offset
    const int part = __builtin_amdgcn_readfirstlane(t / D);
    const float* gh = g_raw + (size_t)ci.t0 * rs + hD;
    const unsigned lo = (unsigned)(t % D);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      if (!(parts & (rr < 8 ? 1 : 2))) continue;
      const int r = part * 16 + rr;
      const float* rowp = gh + (unsigned)((r < ci.len ? r : ci.len - 1) * (int)rs);
      rg[rr] = rowp[lo];
    }
    if (parts & 1) {
      rbeta = beta[(size_t)(ci.t0 + ((t & 63) < ci.len ? (t & 63) : ci.len - 1)) * H + h];
      if constexpr (GV) rdb = dt_bias[hD + lo];  // always a readable address
    }
    const T* qh = q + (size_t)ci.t0 * rs + hD;
    const T* kh = k + (size_t)ci.t0 * rs + hD;
#pragma unroll
    for (int l = 0; l < NLT; ++l) {  // rows past the chunk: zeroed when stored
      const int idx = t + l * NT, r = idx / VPR, vv = idx % VPR;
      const unsigned o = (unsigned)(r < ci.len ? r : ci.len - 1) * (unsigned)rs + vv * EPV;
      if (parts & 4) rq[l] = *(const u32x4*)(qh + o);
      if (parts & 8) rk[l] = *(const u32x4*)(kh + o);
    }
  };
  auto settle_loads = [&]() {
    settle(rg);
    settle(rbeta);
    if constexpr (GV) settle(rdb);
    settle(rq);
    settle(rk);
  };
  // Items (item = head * NC + chunk) in this workgroup's order.  Without SCAN: items
  // blockIdx.x, + gridDim.x, ...  With SCAN: a cursor over its units (k) and the chunk
  // (cl, local to the sequence; first to last forward, last to first backward).
  struct Cursor {
    int it, k, n, hh, cl, nck;
  };
  auto unit_at = [&](Cursor& cu, int k) -> bool {  // unit k of this workgroup, if any
    const int G = (int)gridDim.x, g = (int)blockIdx.x;
    for (;; ++k) {
      const int p = k * G + ((k & 1) ? G - 1 - g : g);
      if (p >= NS * H) return false;
      const int n = order[p / H];
      const int nck = seq_off[n + 1] - seq_off[n];
      if (nck == 0) continue;
      cu.k = k;
      cu.n = n;
      cu.hh = p % H;
      cu.nck = nck;
      cu.cl = FWD ? 0 : nck - 1;
      cu.it = cu.hh * NC + seq_off[n] + cu.cl;
      return true;
    }
  };
  auto first_item = [&](Cursor& cu) -> void {
    if constexpr (SCAN) {
      if (!unit_at(cu, 0)) cu.it = -1;
    } else {
      cu.it = (int)blockIdx.x < items ? (int)blockIdx.x : -1;
    }
  };
  auto next_item = [&](Cursor cu) -> Cursor {
    if constexpr (SCAN) {
      if (FWD ? cu.cl + 1 < cu.nck : cu.cl > 0) {
        cu.cl += FWD ? 1 : -1;
        cu.it = cu.hh * NC + seq_off[cu.n] + cu.cl;
      } else if (!unit_at(cu, cu.k + 1)) {
        cu.it = -1;
      }
    } else {
      cu.it = cu.it + (int)gridDim.x < items ? cu.it + (int)gridDim.x : -1;
    }
    return cu;
  };
  // SCAN: wave w owns the state rows of row group w % 4 and the columns of group w / 4
  constexpr int SCW = NW / 4, SRT = D / 64, SCT = D / 16 / SCW;
  constexpr int NLO = 64 * VPR / NT;  // dO vectors per thread
  f4 sacc[SCAN ? SRT : 1][SCAN ? SCT : 1];
  const int srg = (tid0 >> 6) & 3, scg = (tid0 >> 6) >> 2;
  Cursor cur;
  first_item(cur);
  if (cur.it >= 0) issue_loads(cur.it, tid0, chunks[cur.it % NC], 15);
  settle_loads();
  for (; cur.it >= 0;) {
  const int it = cur.it;
  const Cursor ncur = next_item(cur);
  const int nxt = ncur.it;
  // thread indices re-derived per item so that the lane-dependent LDS addresses
  // below stay inside the loop instead of being held in registers across it
  int tid = tid0;
  asm volatile("" : "+v"(tid));
  tid &= NT - 1;  // its range, for the compiler (24-bit multiplies in the addresses below)
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, cl = lane & 15;
  const int c = it % NC, h = it / NC;
  const int Lr = chunks[c].len;
  const ChunkInfo cnx = chunks[(nxt >= 0 ? nxt : it) % NC];  // early: scalar-load latency
  const size_t ch = (size_t)c * H + h;
  const float aA = __expf(A_log[h]) * gu;  // gu: natural-log decay per unit of the gate
  float db = 0.f;
  if constexpr (GV) db = has_db ? rdb : 0.f;
  if (tid < 64) sBeta[tid] = tid < Lr ? rbeta : 0.f;
  u32x4 rdo[SCAN ? NLO : 1];  // SCAN: this chunk's dO rows (zero past the chunk)
  if constexpr (SCAN) {
    const int n = chunks[c].seq;
    // a unit's first chunk in walking order (backward: its last, dS = dht; forward: its
    // first, S = h0)
    if (chunks[c].cidx == (FWD ? 0 : cur.nck - 1)) {
      const float* src = dht ? dht + ((size_t)n * H + h) * D * D : nullptr;
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < SCT; ++ct) {
          const int i0 = (srg * SRT + rt) * 16 + 4 * g4, col = (scg * SCT + ct) * 16 + cl;
#pragma unroll
          for (int j = 0; j < 4; ++j) sacc[rt][ct][j] = src ? src[(size_t)(i0 + j) * D + col] : 0.f;
        }
    }
    if constexpr (!FWD) {
      const T* oh = dO + (size_t)chunks[c].t0 * rs + (size_t)h * D;
#pragma unroll
      for (int l = 0; l < NLO; ++l) {
        const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (r < Lr) x = *(const u32x4*)(oh + (size_t)r * rs + vv * EPV);
        rdo[l] = x;
      }
    }
  }
  // in-chunk cumulative gate (log2 units), natural: sG[r][i].  Thread (part, i) sums
  // channel i over rows 16 part .. + 15 in registers and publishes the part's total;
  // after the barrier it adds the totals of the earlier parts and writes its rows.
  float* sTot = (float*)(smem + L::TOT_OFF);
  float gx[16];
  {
    const int i = tid % D, part = tid / D;
    float run = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int r = part * 16 + rr;
      const float gv = gate_log2(rg[rr] + db, aA);
      run += r < Lr ? gv : 0.f;
      gx[rr] = run;
    }
    sTot[part * D + i] = run;
  }
#pragma unroll
  for (int l = 0; l < NLT; ++l) {
    const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
    const unsigned m = r < Lr ? ~0u : 0u;
    u32x4 qv = rq[l], kv = rk[l];
    if constexpr (QN) {  // a row is VPR consecutive lanes: one DPP (half) row
      l2n_piece<T, VPR>(qv);
      l2n_piece<T, VPR>(kv);
    }
    *(u32x4*)(sQ + r * PN + vv * EPV) = qv & m;
    *(u32x4*)(sK + r * PN + vv * EPV) = kv & m;
  }
  __syncthreads();
  {
    const int i = tid % D, part = tid / D;
    float add = 0.f;
    for (int pp = 0; pp < part; ++pp) add += sTot[pp * D + i];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sG[(part * 16 + rr) * PGN + i] = gx[rr] + add;
  }
  __syncthreads();
  if (nxt >= 0) issue_loads(nxt, tid, cnx, 1 | 4);  // g_raw rows 0-7, beta, q

  // Kr = K exp(G_T - G), beta Kd = beta K exp(G): natural tiles of T
  auto kr_kd = [&](int t, int n) {
    for (int e = t; e < 64 * VPR; e += n) {
      const int r = e / VPR, i0 = (e % VPR) * EPV;
      float kv[EPV], gv[EPV], gt[EPV];
      load_f<T, EPV>(sK + r * PN + i0, kv);
#pragma unroll
      for (int j = 0; j < EPV; ++j) {
        gv[j] = sG[r * PGN + i0 + j];
        gt[j] = sG[63 * PGN + i0 + j];
      }
      const float br = sBeta[r];
      T kr[EPV], kd[EPV];
#pragma unroll
      for (int j = 0; j < EPV; ++j) {
        kr[j] = from_f<T>(kv[j] * ex2(gt[j] - gv[j]));
        kd[j] = from_f<T>(br * kv[j] * ex2(gv[j]));
      }
      *(uint4*)(sKr + r * PN + i0) = *(const uint4*)kr;
      *(uint4*)(sKd + r * PN + i0) = *(const uint4*)kd;
    }
  };
  // ---- A and Mqk, by 16-row blocks.  A goes to its tile with the rows scaled by
  //   beta (L = diag(beta) A), the only form INV reads.
  //   offdiag(R, S0, S1): blocks (R, S), S0 <= S < S1 < R, anchored at the first row
  //   of block R; diag(R): block (R, R) and the zero blocks right of it.
  auto offdiag = [&](const int R, const int S0, const int S1) {
    const int r0 = 16 * R;
    const int rrow = r0 + cl;
    f4 accA[3], accM[3];
#pragma unroll
    for (int S = 0; S < 3; ++S) accA[S] = accM[S] = zero4();
    //   rows of block R against the earlier blocks: anchor r0 (first row of R)
    {
      for (int kk = 0; kk < D; kk += KS) {
        const int i0 = kk + g4 * KPL;
        float kf[KPL], qf[KPL], ga[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          ga[j] = sG[r0 * PGN + i0 + j];
          const float e = ex2(sG[rrow * PGN + i0 + j] - ga[j]);
          kf[j] = to_f(sK[rrow * PN + i0 + j]) * e;
          qf[j] = to_f(sQ[rrow * PN + i0 + j]) * e;
        }
        const Frag KF = MM::from_vals(kf), QF = MM::from_vals(qf);
#pragma unroll
        for (int S = 0; S < 3; ++S) {
          if (S >= S0 && S < S1) {
            const int srow = 16 * S + cl;
            float kb[KPL];
#pragma unroll
            for (int j = 0; j < KPL; ++j)
              kb[j] = to_f(sK[srow * PN + i0 + j]) * ex2(ga[j] - sG[srow * PGN + i0 + j]);
            const Frag KB = MM::from_vals(kb);
            accA[S] = MM::mma(KF, KB, accA[S]);
            accM[S] = MM::mma(QF, KB, accM[S]);
          }
        }
      }
    }
    const f4 bt = *(const f4*)(sBeta + r0 + 4 * g4);  // beta of this lane's C rows
#pragma unroll
    for (int S = 0; S < 3; ++S)
      if (S >= S0 && S < S1) {
        store_c<float>(sA, PC, r0, 16 * S, accA[S] * bt, lane);
        store_c<float>(sM, PC, r0, 16 * S, accM[S], lane);
      }
  };
  auto diag = [&](const int R) {
    const int r0 = 16 * R;
    const int rrow = r0 + cl;
    // diagonal block (R, R), by 4-row sub-blocks:
    //  (i) rows r of sub-block rho against s in earlier sub-blocks of the block,
    //      anchored at a = r0 + 4 rho (between them): one MFMA pass per rho with
    //      the A rows outside rho and the B columns at or after a set to zero;
    //  (ii) pairs inside a 4x4 diagonal sub-block: pairwise decays on VALU, one
    //      (sub-block, channel group) per lane, summed over the 16 groups.
    f4 dA = zero4(), dM = zero4();
    {
      const int rho_l = cl >> 2;               // sub-block of this lane's A row
      const int anc = r0 + 4 * rho_l;          // its anchor
      float zv[KPL];
#pragma unroll
      for (int j = 0; j < KPL; ++j) zv[j] = 0.f;
      const Frag ZF = MM::from_vals(zv);
      for (int kk = 0; kk < D; kk += KS) {
        const int i0 = kk + g4 * KPL;
        float kf[KPL], qf[KPL], ks[KPL], gs[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const float e = ex2(sG[rrow * PGN + i0 + j] - sG[anc * PGN + i0 + j]);
          ks[j] = to_f(sK[rrow * PN + i0 + j]);  // B column s = r0 + cl: same row data
          kf[j] = ks[j] * e;
          qf[j] = to_f(sQ[rrow * PN + i0 + j]) * e;
          gs[j] = sG[rrow * PGN + i0 + j];
        }
        const Frag KF = MM::from_vals(kf), QF = MM::from_vals(qf);
#pragma unroll
        for (int rho = 1; rho < 4; ++rho) {
          const int a = r0 + 4 * rho;
          const bool colok = cl < 4 * rho;
          float kb[KPL];
#pragma unroll
          for (int j = 0; j < KPL; ++j)
            kb[j] = (colok ? ks[j] : 0.f) * ex2(fminf(sG[a * PGN + i0 + j] - gs[j], 0.f));
          const Frag KB = MM::from_vals(kb);
          const bool rowok = rho_l == rho;
          dA = MM::mma(rowok ? KF : ZF, KB, dA);
          dM = MM::mma(rowok ? QF : ZF, KB, dM);
        }
      }
      {
        constexpr int CPG = D / 16;
        const int sb = g4, cg = cl;
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
            gg4[t] = sG[r * PGN + i];
          }
          // pairwise decays inside the sub-block from the per-token factors
          const float a1 = ex2(gg4[1] - gg4[0]), a2 = ex2(gg4[2] - gg4[1]), a3 = ex2(gg4[3] - gg4[2]);
          float dec[4][4];
          dec[0][0] = dec[1][1] = dec[2][2] = dec[3][3] = 1.f;
          dec[1][0] = a1;
          dec[2][1] = a2;
          dec[2][0] = a1 * a2;
          dec[3][2] = a3;
          dec[3][1] = a2 * a3;
          dec[3][0] = dec[2][0] * a3;
#pragma unroll
          for (int a_ = 0; a_ < 4; ++a_)
#pragma unroll
            for (int b_ = 0; b_ <= a_; ++b_) {
              const int p = a_ * (a_ + 1) / 2 + b_;
              const float kb = kk4[b_] * dec[a_][b_];
              pa[p] += kk4[a_] * kb;
              pm[p] += qq4[a_] * kb;
            }
        }
        sum16_n(pa);
        sum16_n(pm);
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
    }
    const f4 bt = *(const f4*)(sBeta + r0 + 4 * g4);
#pragma unroll
    for (int S = 0; S < 4; ++S) {
      if (S < R) continue;
      const f4 a = S == R ? dA * bt : zero4();
      const f4 m = S == R ? dM : zero4();
      store_c<float>(sA, PC, r0, 16 * S, a, lane);
      store_c<float>(sM, PC, r0, 16 * S, m, lane);
    }
  };
  if constexpr (NW == 8) {
    // waves 0-3: the diagonal blocks; waves 4-7: the six blocks below them, in
    // shares of about equal cost (one anchored row-block operand per block row)
    if (w < 4) {
      diag(w);
    } else if (w == 4) {
      offdiag(3, 0, 2);
    } else if (w == 5) {
      offdiag(3, 2, 3);
    } else if (w == 6) {
      offdiag(2, 0, 2);
    } else {
      offdiag(1, 0, 1);
    }
  } else {
    if (w < 4) {
      if (w > 0) offdiag(w, 0, w);
      diag(w);
    }
  }
  if constexpr (NW == 4) kr_kd(tid, NT);
  __syncthreads();
  if (nxt >= 0) issue_loads(nxt, tid, cnx, 2 | 8);  // g_raw rows 8-15, k
  u32x4 rv[NLT];  // forward: this item's v, put into the A tile as beta v once INV is formed
  if constexpr (FWD) {
    const T* vh = v + (size_t)chunks[c].t0 * rs + (size_t)h * D;
#pragma unroll
    for (int l = 0; l < NLT; ++l) {  // rows past the chunk: scaled by beta = 0 when stored
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      rv[l] = *(const u32x4*)(vh + (unsigned)(r < Lr ? r : Lr - 1) * (unsigned)rs + vv * EPV);
    }
  }

  // ---- INV = (I + L)^{-1}, L = diag(beta) A (strictly lower), blocked by 16.
  // Step 1: wave R < 4 inverts its unit lower-triangular diagonal block (forward
  // substitution, one column per lane).
  if (w < 4) {
    const int R = w;
    if (lane < 16) {
      // right-looking: once x_s is final it is taken off every later row, so the
      // dependent chain is one FMA per row; each row still sums its terms in the
      // order s = 0, 1, ...
      float acc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = (r == lane) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const float xs = acc[s];
#pragma unroll
        for (int r = s + 1; r < 16; ++r)
          acc[r] -= sA[(16 * R + r) * PC + 16 * R + s] * xs;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sINV[(16 * R + r) * PC + 16 * R + lane] = acc[r];
    }
    for (int e = lane; e < 16 * 64; e += 64) {
      const int r = e >> 6, col = e & 63;
      if (col >= 16 * (R + 1)) sINV[(16 * R + r) * PC + col] = 0.f;
    }
  } else if constexpr (QD_EARLY) {
    // waves 4-7, idle in this step: Qd = Q e^G in place over q for the scan step (Qd^T dO
    // backward, Qd S forward; with the scan inside, nothing else reads q once A and Mqk
    // are formed)
#pragma unroll
    for (int e = tid - NT / 2; e < 64 * VPR; e += NT / 2) {
      const int r = e / VPR, vv = e % VPR;
      const u32x4 qv = *(const u32x4*)(sQ + r * PN + vv * EPV);
      const T* qe = (const T*)&qv;
      T qd[EPV];
#pragma unroll
      for (int j = 0; j < EPV; ++j)
        qd[j] = from_f<T>(to_f(qe[j]) * ex2(sG[r * PGN + vv * EPV + j]));
      *(u32x4*)(sQ + r * PN + vv * EPV) = *(const u32x4*)qd;
    }
  }
  __syncthreads();
  // Step 2: wave S < 3 fills column block S below the diagonal, top to bottom:
  //   INV_{R,S} = -D_R * sum_{J=S}^{R-1} L_{R,J} INV_{J,S};
  // with eight waves, waves 3-7 form Kr and Kd meanwhile (first read by W and Tm).
  if constexpr (NW == 8) {
    if (w >= 3) kr_kd(tid - 192, NT - 192);
  }
  if (w < 3) {
    const int S = w;
    float* scr = sScr + w * 16 * 17;
    for (int R = S + 1; R < 4; ++R) {
      f4 X = zero4();
      for (int J = S; J < R; ++J) {
#pragma unroll
        for (int kk = 0; kk < 16; kk += 4) {
          const int row = cl, kx = kk + g4;
          const float a = sA[(16 * R + row) * PC + 16 * J + kx];
          const float b = sINV[(16 * J + kx) * PC + 16 * S + row];
          X = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, X, 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) scr[(g4 * 4 + j) * 17 + cl] = X[j];
      __builtin_amdgcn_wave_barrier();
      f4 Y = zero4();
#pragma unroll
      for (int kk = 0; kk < 16; kk += 4) {
        const int row = cl, kx = kk + g4;
        const float a = sINV[(16 * R + row) * PC + 16 * R + kx];
        const float b = scr[kx * 17 + row];
        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, Y, 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j) sINV[(16 * R + g4 * 4 + j) * PC + 16 * S + cl] = -Y[j];
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  settle_loads();  // the next item's inputs, before this item's first stores
  if constexpr (FWD) {  // beta v into the A tile (dead once INV is formed)
    T* sVb = (T*)(smem + L::A_OFF);
#pragma unroll
    for (int l = 0; l < NLT; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      const T* e = (const T*)&rv[l];
      const float br = sBeta[r];
      T out[EPV];
#pragma unroll
      for (int j = 0; j < EPV; ++j) out[j] = from_f<T>(br * to_f(e[j]));
      *(u32x4*)(sVb + r * PN + vv * EPV) = *(const u32x4*)out;
    }
  }

  // ---- W = INV (beta Kd): wave w -> rows of block w % 4, columns [c0, c0 + DH)
  {
    const int R = w & 3, c0 = (w >> 2) * DH;
    constexpr int NTW = DH / 16;
    f4 acc[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      const Frag a = MM::ld_perm_f32(sINV + (16 * R + cl) * PC, ks * KS, lane);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
        acc[nt] = MM::mma(a, MM::ld_tr(sKd, PN, ks * KS, c0 + nt * 16, lane), acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) store_c<T>(sW, PN, 16 * R, c0 + nt * 16, acc[nt], lane);
  }
  if constexpr (FWD) {
    __syncthreads();  // W formed; beta v in the A tile
    // Uv = INV (beta V), rows of block w % 4, columns [c0, c0 + DH); written as Uv^T
    // straight from the C tiles (a lane holds 4 consecutive rows of one column)
    const int R = w & 3, c0 = (w >> 2) * DH;
    constexpr int NTW = DH / 16;
    f4 acc[NTW];  // Uv: rows 16 R + 4 g4 + j, columns c0 + 16 nt + cl
    {
      const T* sVb = (const T*)(smem + L::A_OFF);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) acc[nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks) {
        const Frag a = MM::ld_perm_f32(sINV + (16 * R + cl) * PC, ks * KS, lane);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          acc[nt] = MM::mma(a, MM::ld_tr(sVb, PN, ks * KS, c0 + nt * 16, lane), acc[nt]);
      }
    }
    if constexpr (SCAN) {
      // exp(G_T) of this lane's state rows
      f4 eg[SRT];
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          eg[rt][j] = ex2(sG[63 * PGN + (srg * SRT + rt) * 16 + 4 * g4 + j]);
      // Qd = Q e^G in place over q (each thread its own pieces; with eight waves already
      // formed during INV step 1)
#pragma unroll
      for (int l = 0; l < (QD_EARLY ? 0 : NLT); ++l) {
        const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
        const u32x4 qv = *(const u32x4*)(sQ + r * PN + vv * EPV);
        const T* qe = (const T*)&qv;
        T qd[EPV];
#pragma unroll
        for (int j = 0; j < EPV; ++j) qd[j] = from_f<T>(to_f(qe[j]) * ex2(sG[r * PGN + vv * EPV + j]));
        *(u32x4*)(sQ + r * PN + vv * EPV) = *(const u32x4*)qd;
      }
      T* sS = (T*)(smem + L::FS_OFF);
      T* sX = (T*)(smem + L::FX_OFF);
      constexpr int PSS = L::PSS;
      __syncthreads();  // Uv formed: beta v, INV and Kd dead; Qd in place
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < SCT; ++ct)
          store_c<T>(sS, PSS, (srg * SRT + rt) * 16, (scg * SCT + ct) * 16, sacc[rt][ct], lane);
      __syncthreads();
      if (dstates) {  // h_saved: the state at the start of this chunk, 16-byte rows
        T* dst = dstates + ch * D * D;
#pragma unroll
        for (int l = 0; l < D * VPR / NT; ++l) {
          const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
          *(u32x4*)(dst + (size_t)r * D + vv * EPV) = *(const u32x4*)(sS + r * PSS + vv * EPV);
        }
      }
      // P = W S and the first part of O, Qd S (same B fragments); X = Uv - P
      f4 P[NTW], Oa[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) P[nt] = Oa[nt] = zero4();
#pragma unroll
      for (int kk = 0; kk < D / KS; ++kk) {
        const Frag aw = MM::load(sW + (16 * R + cl) * PN + kk * KS + g4 * KPL);
        const Frag aq = MM::load(sQ + (16 * R + cl) * PN + kk * KS + g4 * KPL);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const Frag b = MM::ld_tr_nat(sS, PSS, kk * KS, c0 + nt * 16, lane);
          P[nt] = MM::mma(aw, b, P[nt]);
          Oa[nt] = MM::mma(aq, b, Oa[nt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) store_c<T>(sX, PSS, 16 * R, c0 + nt * 16, acc[nt] - P[nt], lane);
      __syncthreads();  // X complete; the state tile is dead
      // O += Mqk X;  S <- exp(G_T) . S + Kr^T X
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) {
        const Frag am = MM::from_f32(sM + (16 * R + cl) * PC + kk * KS + g4 * KPL);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          Oa[nt] = MM::mma(am, MM::ld_tr_nat(sX, PSS, kk * KS, c0 + nt * 16, lane), Oa[nt]);
      }
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) sacc[rt][ct][j] *= eg[rt][j];
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) {
        Frag ak[SRT];
#pragma unroll
        for (int rt = 0; rt < SRT; ++rt) ak[rt] = MM::ld_tr_nat(sKr, PN, kk * KS, (srg * SRT + rt) * 16, lane);
#pragma unroll
        for (int ct = 0; ct < SCT; ++ct) {
          const Frag b = MM::ld_tr_nat(sX, PSS, kk * KS, (scg * SCT + ct) * 16, lane);
#pragma unroll
          for (int rt = 0; rt < SRT; ++rt) sacc[rt][ct] = MM::mma(ak[rt], b, sacc[rt][ct]);
        }
      }
      // O staged over the state tile (dead since X was formed), then out
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) store_c<T>(sS, PSS, 16 * R, c0 + nt * 16, Oa[nt], lane);
      __syncthreads();
      if (o) {  // rows past the chunk store row Lr - 1 again (the same bytes as the lane that
                // owns it), so that every lane issues the same stores
        T* oh = o + (size_t)chunks[c].t0 * rs + (size_t)h * D;
#pragma unroll
        for (int l = 0; l < NLT; ++l) {
          const int idx = tid + l * NT, r0 = idx / VPR, vv = idx % VPR;
          const int r = r0 < Lr ? r0 : Lr - 1;
          *at((u32x4*)oh, row_off(r, (unsigned)rs * L::ES) + vv * 16) =
              *(const u32x4*)(sS + r * PSS + vv * EPV);
        }
      }
      if (chunks[c].cidx == cur.nck - 1 && dh0) {  // ht after the sequence's last chunk
        float* d0 = dh0 + ((size_t)chunks[c].seq * H + h) * D * D;
#pragma unroll
        for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
          for (int ct = 0; ct < SCT; ++ct)
            store_c<float>(d0, D, (srg * SRT + rt) * 16, (scg * SCT + ct) * 16, sacc[rt][ct],
                           lane);
      }
      // the O staging is read out before the next item's A/Mqk phase writes over it (two
      // barriers later); the gate, q and k tiles have no reader left
    } else {
    {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        T u4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) u4[j] = from_f<T>(acc[nt][j]);
        T* dst = UvT + ch * D * 64 + (size_t)(c0 + nt * 16 + cl) * 64 + 16 * R + 4 * g4;
        if constexpr (L::ES == 2) *(uint2*)dst = *(const uint2*)u4;
        else *(uint4*)dst = *(const uint4*)u4;
      }
    }
    // -W and Qd = Q e^G (natural rows)
#pragma unroll
    for (int l = 0; l < NLT; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      const u32x4 wv = *(const u32x4*)(sW + r * PN + vv * EPV);
      const u32x4 qv = *(const u32x4*)(sQ + r * PN + vv * EPV);
      const T* we = (const T*)&wv;
      const T* qe = (const T*)&qv;
      T wn[EPV], qd[EPV];
#pragma unroll
      for (int j = 0; j < EPV; ++j) {
        wn[j] = from_f<T>(-to_f(we[j]));
        qd[j] = from_f<T>(to_f(qe[j]) * ex2(sG[r * PGN + vv * EPV + j]));
      }
      const size_t off = ch * 64 * D + (size_t)r * D + vv * EPV;
      *(u32x4*)(Wn + off) = *(const u32x4*)wn;
      *(u32x4*)(Qd + off) = *(const u32x4*)qd;
    }
    // Mqk (natural rows) and Kr^T, 8 elements per piece
    for (int e = tid; e < 64 * 8; e += NT) {
      const int r = e >> 3, c8 = (e & 7) * 8;
      T tm[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tm[j] = from_f<T>(sM[r * PC + c8 + j]);
#pragma unroll
      for (int x = 0; x < 8 * L::ES / 16; ++x)
        ((uint4*)(Mq + ch * 64 * 64 + r * 64 + c8))[x] = ((const uint4*)tm)[x];
    }
    for (int e = tid; e < D * 8; e += NT) {
      const int i = e >> 3, r8 = (e & 7) * 8;
      T kt[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) kt[j] = sKr[(r8 + j) * PN + i];
#pragma unroll
      for (int x = 0; x < 8 * L::ES / 16; ++x)
        ((uint4*)(KrT + ch * D * 64 + (size_t)i * 64 + r8))[x] = ((const uint4*)kt)[x];
    }
    if (tid < D) eGT[ch * D + tid] = ex2(sG[63 * PGN + tid]);
    __syncthreads();  // the next item overwrites sG, sQ and sK (here read as W)
    }
  } else {
  // ---- INV and Mqk^T (act dtype, natural rows) for the gradient pass (which reads
  // INV^T out of its copy of INV).  With the scan inside, Mqk^T is not stored: its only
  // use there is dU, which this kernel forms and hands over.
  for (int e = tid; e < 64 * 8; e += NT) {
    const int r = e >> 3, c8 = (e & 7) * 8;
    float a[8], m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = sINV[r * PC + c8 + j];
      if constexpr (!SCAN) m[j] = sM[(c8 + j) * PC + r];
    }
    T ta[8], tm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ta[j] = from_f<T>(a[j]);
      if constexpr (!SCAN) tm[j] = from_f<T>(m[j]);
    }
    const size_t o = ch * 64 * 64 + r * 64 + c8;
#pragma unroll
    for (int v = 0; v < 8 * L::ES / 16; ++v) {
      ((uint4*)(INVo + o))[v] = ((const uint4*)ta)[v];
      if constexpr (!SCAN) ((uint4*)(MqkTo + o))[v] = ((const uint4*)tm)[v];
    }
  }
  __syncthreads();

  if constexpr (SCAN) {
    // dS_in = e^{G_T} . dS_out + Tm dS_out + PT dO with Tm = -W^T Kr, PT = Qd^T - W^T Mqk^T,
    // applied factored: dS <- e^{G_T} . dS + Qd^T dO + W^T X, X = -(Kr dS + Mqk^T dO).
    // Tm and PT are never formed (about 22% fewer MFMA operations than forming them).
    T* sS = (T*)(smem + L::SS_OFF);
    T* sO = (T*)(smem + L::SO_OFF);
    T* sX = (T*)(smem + L::SX_OFF);
    constexpr int PSS = L::PSS, PSX = L::PSX;
    // e^{G_T} of this lane's state rows; Qd = Q e^G in place over q (each thread its own
    // pieces; with eight waves already formed during INV step 1); the state and dO tiles
    // over the dead A, INV, Kd and scratch tiles
    f4 eg[SRT];
#pragma unroll
    for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        eg[rt][j] = ex2(sG[63 * PGN + (srg * SRT + rt) * 16 + 4 * g4 + j]);
#pragma unroll
    for (int l = 0; l < (QD_EARLY ? 0 : NLT); ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      const u32x4 qv = *(const u32x4*)(sQ + r * PN + vv * EPV);
      const T* qe = (const T*)&qv;
      T qd[EPV];
#pragma unroll
      for (int j = 0; j < EPV; ++j)
        qd[j] = from_f<T>(to_f(qe[j]) * ex2(sG[r * PGN + vv * EPV + j]));
      *(u32x4*)(sQ + r * PN + vv * EPV) = *(const u32x4*)qd;
    }
#pragma unroll
    for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < SCT; ++ct)
        store_c<T>(sS, PSS, (srg * SRT + rt) * 16, (scg * SCT + ct) * 16, sacc[rt][ct], lane);
#pragma unroll
    for (int l = 0; l < NLO; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      *(u32x4*)(sO + r * PSS + vv * EPV) = rdo[l];
    }
    __syncthreads();  // Qd in place, state and dO tiles staged; the gate tile is dead
    {  // dS_out of this chunk (the state gradient at its end), 16-byte rows
      T* dst = dstates + ch * D * D;
#pragma unroll
      for (int l = 0; l < D * VPR / NT; ++l) {
        const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
        *(u32x4*)(dst + (size_t)r * D + vv * EPV) = *(const u32x4*)(sS + r * PSS + vv * EPV);
      }
    }
    {  // X = -(Kr dS + Mqk^T dO): wave w -> rows of block w % 4, columns [c0, c0 + DH)
      const int R = w & 3, c0 = (w >> 2) * DH, ar = 16 * R + cl;
      constexpr int NTW = DH / 16;
      f4 acc[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) acc[nt] = zero4();
#pragma unroll
      for (int kk = 0; kk < D / KS; ++kk) {
        const Frag a = MM::ld_perm(sKr + ar * PN, kk * KS, lane);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          acc[nt] = MM::mma(a, MM::ld_tr(sS, PSS, kk * KS, c0 + nt * 16, lane), acc[nt]);
      }
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks) {
        float mv[KPL];  // Mqk^T row ar = column ar of the fp32 Mqk tile, permuted order
#pragma unroll
        for (int j = 0; j < KPL; ++j) mv[j] = sM[(ks * KS + MM::kperm(g4, j)) * PC + ar];
        const Frag a = MM::from_vals(mv);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          acc[nt] = MM::mma(a, MM::ld_tr(sO, PSS, ks * KS, c0 + nt * 16, lane), acc[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) store_c<T>(sX, PSX, 16 * R, c0 + nt * 16, -acc[nt], lane);
    }
    __syncthreads();  // X complete
    if (dUo) {  // dU = -X for the gradient pass, natural [64][D] rows (sign bits flipped)
      constexpr unsigned SGN = L::ES == 2 ? 0x80008000u : 0x80000000u;
      T* dst = dUo + ch * 64 * D;
#pragma unroll
      for (int l = 0; l < NLT; ++l) {
        const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
        *(u32x4*)(dst + r * D + vv * EPV) = *(const u32x4*)(sX + r * PSX + vv * EPV) ^ SGN;
      }
    }
    // dS <- e^{G_T} . dS + Qd^T dO + W^T X  (A: Qd^T / W^T rows, read across the q / W
    // tiles; B: the dO / X tiles read across their rows, in the same order)
#pragma unroll
    for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[rt][ct][j] *= eg[rt][j];
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      Frag aq[SRT], aw[SRT];
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt) {
        aq[rt] = MM::ld_tr(sQ, PN, ks * KS, (srg * SRT + rt) * 16, lane);
        aw[rt] = MM::ld_tr(sW, PN, ks * KS, (srg * SRT + rt) * 16, lane);
      }
#pragma unroll
      for (int ct = 0; ct < SCT; ++ct) {
        const Frag bo = MM::ld_tr(sO, PSS, ks * KS, (scg * SCT + ct) * 16, lane);
        const Frag bx = MM::ld_tr(sX, PSX, ks * KS, (scg * SCT + ct) * 16, lane);
#pragma unroll
        for (int rt = 0; rt < SRT; ++rt) {
          sacc[rt][ct] = MM::mma(aq[rt], bo, sacc[rt][ct]);
          sacc[rt][ct] = MM::mma(aw[rt], bx, sacc[rt][ct]);
        }
      }
    }
    if (chunks[c].cidx == 0 && dh0) {  // the sequence's first chunk: dh0 = dS
      float* d0 = dh0 + ((size_t)chunks[c].seq * H + h) * D * D;
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < SCT; ++ct)
          store_c<float>(d0, D, (srg * SRT + rt) * 16, (scg * SCT + ct) * 16, sacc[rt][ct],
                         lane);
    }
    __syncthreads();  // the next item's gate, q and k tiles overwrite X, Qd and W
  } else {
  // ---- Tm = -W^T Kr [D x D] and PT = Qd^T - W^T Mqk^T [D x 64], computed as their
  // transposes (C tiles over rows j / r, columns i) so that a lane holds 4
  // consecutive entries of one row; wave w -> key channels i in [16 w, 16 w + 16).
  {
    Frag bw[NKC];  // W[s][16 w + cl], s in the permuted order of k-step ks
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) bw[ks] = MM::ld_tr(sW, PN, ks * KS, 16 * w, lane);
#pragma unroll
    for (int mt = 0; mt < NW; ++mt) {
      f4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
        acc = MM::mma(MM::ld_tr(sKr, PN, ks * KS, 16 * mt, lane), bw[ks], acc);
      store_ct<T>(sTm, PTM, 16 * mt, 16 * w, -acc, lane);  // sTm[i][j] = Tm[i][j]
    }
    const int i = 16 * w + cl;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
        acc = MM::mma(MM::ld_perm_f32(sM + (16 * mt + cl) * PC, ks * KS, lane), bw[ks], acc);
      f4 pt;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * mt + 4 * g4 + j;
        pt[j] = to_f(sQ[r * PN + i]) * ex2(sG[r * PGN + i]) - acc[j];
      }
      store_ct<T>(sPT, PPT, 16 * mt, 16 * w, pt, lane);  // sPT[i][r] = PT[i][r]
    }
  }
  if (tid < D) eGT[ch * D + tid] = ex2(sG[63 * PGN + tid]);
  __syncthreads();
  {
    T* dst = Tm + ch * D * D;
#pragma unroll
    for (int l = 0; l < D * VPR / NT; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      *(uint4*)(dst + r * D + vv * EPV) = *(const uint4*)(sTm + r * PTM + vv * EPV);
    }
    constexpr int VP = 64 / EPV;  // vectors per 64-long row
    T* dp = PT + ch * D * 64;
#pragma unroll
    for (int l = 0; l < D * VP / NT; ++l) {
      const int idx = tid + l * NT, r = idx / VP, vv = idx % VP;
      *(uint4*)(dp + r * 64 + vv * EPV) = *(const uint4*)(sPT + r * PPT + vv * EPV);
    }
  }
  }
  }
  // the next item writes sG, sQ, sK and sBeta only: no reader of those is left
  cur = ncur;
  }
}

template <typename T, int D, bool GV, bool QN>
static hipError_t prep_v(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  const int items = s.NC * s.H;
  int resident = 0;
  hipError_t e =
      resident_blocks((const void*)k_prep<T, D, GV, false, QN, false>, PL<T, D>::NT, &resident);
  if (e != hipSuccess) return e;
  const int grid = items < resident ? items : resident;
  hipLaunchKernelGGL((k_prep<T, D, GV, false, QN, false>), dim3(grid), dim3(PL<T, D>::NT), 0, st,
                     p.chunks, s.NC, s.H, (const T*)p.q, (const T*)p.k, p.g_raw, p.beta,
                     p.A_log, p.dt_bias, p.has_db, s.gu, (T*)p.Tm, (T*)p.PT, p.eGT,
                     (T*)p.INV, (T*)p.MqkT, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr);
  return hipGetLastError();
}

// prep with the state-gradient scan inside (every sequence has ncs chunks)
template <typename T, int D, bool GV, bool QN>
static hipError_t prepscan_v(const Shape& s, const BwdPtrs& p, const int* order,
                             hipStream_t st) {
  const int units = s.N * s.H;
  int resident = 0;
  hipError_t e =
      resident_blocks((const void*)k_prep<T, D, GV, false, QN, true>, PL<T, D>::NT, &resident);
  if (e != hipSuccess) return e;
  const int grid = units < resident ? units : resident;
  hipLaunchKernelGGL((k_prep<T, D, GV, false, QN, true>), dim3(grid), dim3(PL<T, D>::NT), 0, st,
                     p.chunks, s.NC, s.H, (const T*)p.q, (const T*)p.k, p.g_raw, p.beta,
                     p.A_log, p.dt_bias, p.has_db, s.gu, nullptr, nullptr, nullptr,
                     (T*)p.INV, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     (const T*)p.dO, p.dht, (T*)p.dstates, p.dh0, p.seq_off, order, s.N,
                     nullptr, (T*)p.dU);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t prepscan_t(const Shape& s, const BwdPtrs& p, const int* order,
                             hipStream_t st) {
  const bool gv = p.has_db || p.ddt_bias;
  if (s.qn)
    return gv ? prepscan_v<T, D, true, true>(s, p, order, st)
              : prepscan_v<T, D, false, true>(s, p, order, st);
  return gv ? prepscan_v<T, D, true, false>(s, p, order, st)
            : prepscan_v<T, D, false, false>(s, p, order, st);
}

hipError_t launch_prepscan(const Shape& s, const BwdPtrs& p, const int* order, hipStream_t st) {
  if (s.NC == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? prepscan_t<bf16, 128>(s, p, order, st)
                                : prepscan_t<bf16, 64>(s, p, order, st);
  return prepscan_t<float, 64>(s, p, order, st);
}

// the production forward in one kernel: prep in forward mode with the state scan inside
template <typename T, int D, bool GV, bool QN>
static hipError_t fprepscan_v(const Shape& s, const FwdPtrs& p, const int* order,
                              hipStream_t st) {
  const int units = s.N * s.H;
  int resident = 0;
  hipError_t e =
      resident_blocks((const void*)k_prep<T, D, GV, true, QN, true>, PL<T, D>::NT, &resident);
  if (e != hipSuccess) return e;
  const int grid = units < resident ? units : resident;
  hipLaunchKernelGGL((k_prep<T, D, GV, true, QN, true>), dim3(grid), dim3(PL<T, D>::NT), 0, st,
                     p.chunks, s.NC, s.H, (const T*)p.q, (const T*)p.k, p.g_raw, p.beta,
                     p.A_log, p.dt_bias, p.has_db, s.gu, nullptr, nullptr, nullptr, nullptr,
                     nullptr, (const T*)p.v, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, p.h0, (T*)p.h_saved, p.ht, p.seq_off, order, s.N, (T*)p.o,
                     nullptr);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t fprepscan_t(const Shape& s, const FwdPtrs& p, const int* order,
                              hipStream_t st) {
  if (s.qn)
    return p.has_db ? fprepscan_v<T, D, true, true>(s, p, order, st)
                    : fprepscan_v<T, D, false, true>(s, p, order, st);
  return p.has_db ? fprepscan_v<T, D, true, false>(s, p, order, st)
                  : fprepscan_v<T, D, false, false>(s, p, order, st);
}

hipError_t launch_fprepscan(const Shape& s, const FwdPtrs& p, const int* order, hipStream_t st) {
  if (s.NC == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? fprepscan_t<bf16, 128>(s, p, order, st)
                                : fprepscan_t<bf16, 64>(s, p, order, st);
  return fprepscan_t<float, 64>(s, p, order, st);
}

hipError_t prepscan_grid(const Shape& s, int* grid) {
  const void* k = s.bf16 ? (s.D == 128 ? (const void*)k_prep<bf16, 128, false, false, false, true>
                                       : (const void*)k_prep<bf16, 64, false, false, false, true>)
                         : (const void*)k_prep<float, 64, false, false, false, true>;
  const int nt = s.bf16 ? (s.D == 128 ? PL<bf16, 128>::NT : PL<bf16, 64>::NT) : PL<float, 64>::NT;
  return resident_blocks(k, nt, grid);
}

template <typename T, int D, bool GV, bool QN>
static hipError_t fprep_v(const Shape& s, const FwdPtrs& p, hipStream_t st) {
  const int items = s.NC * s.H;
  int resident = 0;
  hipError_t e =
      resident_blocks((const void*)k_prep<T, D, GV, true, QN, false>, PL<T, D>::NT, &resident);
  if (e != hipSuccess) return e;
  const int grid = items < resident ? items : resident;
  hipLaunchKernelGGL((k_prep<T, D, GV, true, QN, false>), dim3(grid), dim3(PL<T, D>::NT), 0, st,
                     p.chunks, s.NC, s.H, (const T*)p.q, (const T*)p.k, p.g_raw, p.beta,
                     p.A_log, p.dt_bias, p.has_db, s.gu, nullptr, nullptr, p.eGT, nullptr,
                     nullptr, (const T*)p.v, (T*)p.Wn, (T*)p.KrT, (T*)p.UvT, (T*)p.Qd,
                     (T*)p.Mq, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr,
                     nullptr);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t prep_t(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  const bool gv = p.has_db || p.ddt_bias;
  if (s.qn) return gv ? prep_v<T, D, true, true>(s, p, st) : prep_v<T, D, false, true>(s, p, st);
  return gv ? prep_v<T, D, true, false>(s, p, st) : prep_v<T, D, false, false>(s, p, st);
}

template <typename T, int D>
static hipError_t fprep_t(const Shape& s, const FwdPtrs& p, hipStream_t st) {
  if (s.qn)
    return p.has_db ? fprep_v<T, D, true, true>(s, p, st) : fprep_v<T, D, false, true>(s, p, st);
  return p.has_db ? fprep_v<T, D, true, false>(s, p, st) : fprep_v<T, D, false, false>(s, p, st);
}

hipError_t launch_fprep(const Shape& s, const FwdPtrs& p, hipStream_t st) {
  if (s.NC == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? fprep_t<bf16, 128>(s, p, st) : fprep_t<bf16, 64>(s, p, st);
  return fprep_t<float, 64>(s, p, st);
}

hipError_t launch_prep(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  if (s.NC == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? prep_t<bf16, 128>(s, p, st) : prep_t<bf16, 64>(s, p, st);
  return prep_t<float, 64>(s, p, st);
}

}  // namespace kda
