// kda_gradf.hip -- fused gradient pass: workgroups of D/16 waves, each walking a share of
// the chunk-heads (persistent; the next one's tiles are fetched during the current one).
//
// Quantities per chunk (G: in-chunk cumulative gate; Kd = K e^G, Kr = K e^{G_T-G},
// Qd = Q e^G; INV and Mqk from the prep pass; S_in the chunk start state; dS_out
// the state gradient at the chunk end from the scan).  [KB] = the Kernel-B guide
// ("bwd-kernelB-beginner-guide-full"), part 2.
//   state side ([KB] B1, and the kdS / dbeta part of B2):
//     Y = V - Kd S_in,  U = INV diag(beta) Y,
//     dU = Mqk^T dO + Kr dS_out,  dvcorr = INV^T dU,  dv = beta . dvcorr,
//     dbeta_r  = sum_d dvcorr_rd Y_rd
//   key side ([KB] B2, B3 and the inlined gate epilogue K1):
//     dKr = U dS_out^T,  dQd0 = dO S_in^T,  dKd0 = dvcorr S_in^T,
//     p_i = sum_d S_in[i,d] dS_out[i,d]                       ([KB] B0, folded into B2)
//     dMqk = tril(dO U^T),  dL = -stril(dvcorr U^T)
//     dq   = e^G dQd0 + sum_{s<=r} dMqk_rs k_s e^{G_r-G_s}
//     dk_d = beta_r (-e^G dKd0 + x2),  x2_r = sum_{s<r} dL_rs k_s e^{G_r-G_s}
//     dk_i = sum_{r>=s} (dMqk_rs q_r + beta_r dL_rs k_r) e^{G_r-G_s}
//     dk_r = e^{G_T-G} dKr,  dk = dk_d + dk_i + dk_r
//     dbeta_r += sum_s dL_rs A_rs = sum_i k_ri x2_ri
//     dG = q.dq + k.(dk_d - dk_i - dk_r);  dG_last += sum_r k.dk_r + e^{G_T}.p
//     dg = reverse cumsum of dG (rows);  dg_raw = dg . gu (-e^{A_log} sigmoid(g_raw + dt_bias))
//     (gu = 1, or ln 2 for a gate in log2 units);  ddt_bias = column sums of dg_raw
//     dA_log partial = sum dg . g
// The epilogue stays fp32 ([KB] B3: dk_d - dk_i - dk_r cancels strongly).  The
// pairwise decays e^{G_r-G_s} never come from exp(-G) (it overflows): across 16-row
// blocks they factor through an anchor row between r and s (both factors <= 1) and
// run on MFMA with the decayed operand carried at fp32 accuracy (hi + lo bf16); inside
// a 16-row diagonal block they are running products of per-token decays, summed
// exactly in fp32 on VALU.
#include "kda_dev.h"
#include "kda_launch.h"

namespace kda {

template <typename T, int D> struct GF {
  static constexpr int NW = D / 16;  // waves
  static constexpr int NT = NW * 64;
  static constexpr int WPR = NW / 4;  // waves per 16-row block in the state side
  static constexpr int ES = (int)sizeof(T);
  // Row pitches.  gfx950 LDS has 64 banks of 4 bytes; 16- to 64-bit accesses are served
  // 32 lanes per cycle and 128-bit ones 16 lanes per cycle (lanes 0-31 or 32-63, split by
  // the parity of lane bits 2..4).  A bf16 row pitch of 32 (mod 256) bytes lets both the
  // MFMA operand reads (16 rows x 16 bytes at one column) and the transposing reads
  // (8 rows x 32 bytes per 32 lanes) hit 64 distinct banks; 16 bytes of padding leaves
  // both 2-way conflicted (measured with rocprofv3 SQ_LDS_BANK_CONFLICT on probe kernels).
  static constexpr int PG = 68;                 // sG  [D][PG] fp32 (channel-major G)
  static constexpr int NPAD = ES == 2 ? 2 : 1;  // 16-byte pad granules per natural row
  static constexpr int PN = D + NPAD * 16 / ES; // natural [rows][D] tiles of T
  static constexpr int PT = ES == 2 ? 80 : 68;  // [D][64] token-minor tiles of T
  static constexpr int PC = ES == 2 ? 80 : 68;  // [64][64] tiles of T
  static constexpr int CPAD = (PC - 64) * ES / 16;  // pad granules of a [64][PC] tile
  static constexpr int PDG = 20;                // fp32 diagonal-block tables [16][PDG]
  static constexpr int PR = D + 4;              // dg_raw staging [64][PR] fp32
  static constexpr int G_OFF = 0;
  static constexpr int G_SZ = D * PG * 4;
  static constexpr int N_SZ = 64 * PN * ES;
  static constexpr int S_SZ = D * PN * ES;
  static constexpr int YT_SZ = D * PT * ES;
  static constexpr int PCT = 64 * PC * ES;  // one [64][PC] tile
  // fp32 copies of the four diagonal 16x16 blocks of dMqk and dL (bf16 tiles only)
  static constexpr int DGBS = 16 * PDG + 4;     // block stride of those tables
  static constexpr int DG_SZ = ES == 2 ? 2 * 4 * DGBS * 4 : 0;
  // Regions by phase (state side / intra-chunk phase):
  //   O : dO                  / q, then dq staged in place
  //   YT: (beta Y)^T, dU^T    / k, then dk staged in place; past it dMqk, dL and
  //                             the diagonal tables
  //   K0: k, then dvcorr      / (under dMqk, dL; refilled once the intra phase is done)
  //   S : S_in, dS_out, dv    / -
  //   V : v, then U           / -
  // S and V lie above every intra-phase tile, so the next chunk-head's S_in and v
  // stream in during the whole intra phase.
  static constexpr int O_OFF = G_OFF + G_SZ;
  static constexpr int YT_OFF = O_OFF + N_SZ;
  static constexpr int Q_OFF = O_OFF;
  static constexpr int K_OFF = YT_OFF;
  static constexpr int DM_OFF = K_OFF + N_SZ;
  static constexpr int DL_OFF = DM_OFF + PCT;
  static constexpr int DG_OFF = DL_OFF + PCT;
  static constexpr int I_END = DG_OFF + DG_SZ;
  static constexpr int K0_OFF = YT_OFF + (N_SZ > YT_SZ ? N_SZ : YT_SZ);
  static constexpr int S_OFF = K0_OFF + N_SZ > I_END ? K0_OFF + N_SZ : I_END;
  static constexpr int V_OFF = S_OFF + S_SZ;
  static constexpr int C_END = V_OFF + N_SZ;
  // INV [64][PC] (act dtype; INV^T is read out of it with transposing reads): over the
  // diagonal tables for bf16 (they are dead from the intra tile loop until the key
  // side writes them, after INV's last use), past the state tiles for fp32
  static constexpr int IV_SZ = PCT;
  static constexpr int IV_OFF = ES == 2 ? DG_OFF : C_END;
  static constexpr int L_END = ES == 2 ? C_END : C_END + IV_SZ;
  static_assert(ES != 2 || IV_SZ <= DG_SZ, "INV fits the diagonal-table region");
  // k (then dvcorr) and INV are both live through the state side
  static_assert(K0_OFF + N_SZ <= IV_OFF || IV_OFF + IV_SZ <= K0_OFF, "k tile clear of INV");
  static constexpr int B_OFF = (L_END + 15) / 16 * 16;     // beta [64]
  static constexpr int DB1_OFF = B_OFF + 256;             // [WPR][64]
  static constexpr int DB2_OFF = DB1_OFF + WPR * 256;     // [NW][64]
  static constexpr int RED_OFF = DB2_OFF + NW * 256;      // [NW]
  static constexpr int RQ_OFF = RED_OFF + NW * 4;         // q/k reciprocal norms [2][64]
  static constexpr int MD_OFF = RQ_OFF + 2 * 64 * 4;      // diagonal of dMqk [64] fp32
  static constexpr int TOTAL = MD_OFF + 64 * 4;
  static_assert(S_OFF >= I_END && K0_OFF >= DM_OFF, "prefetch tiles clear the intra phase");
  static_assert(TOTAL <= 160 * 1024, "LDS");
  static_assert(64 * PR * 4 <= G_SZ, "dg_raw staging fits the gate region");
  static_assert(N_SZ <= D * PN * ES, "dv staging fits the state tile");
};

// GV: gate bias present or its gradient asked for; without it the bias is not read and
// no column sums of dg_raw are formed.  QN: q and k are L2-normalised per row inside the
// pass (k in its LDS tile at the start of an item, q in registers on its way to LDS) and
// dq, dk are projected back to the raw rows as they are written out, with the cached
// reciprocal norms: dx = r (dxn - xn (xn . dxn)).  DU: dU = Mqk^T dO + Kr dS_out comes
// from memory (prep forms it when the state scan runs inside prep) instead of being
// formed here, which also drops the Kr fragments and the Mqk^T loads.
template <typename T, int D, bool GV, bool QN, bool DU>
__global__ __launch_bounds__(4 * D) void k_gradf(
    const ChunkInfo* __restrict__ chunks, int NC, int H, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dO,
    const float* __restrict__ g_raw, const float* __restrict__ beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, int has_db, float gu,
    const T* __restrict__ h_saved,
    const T* __restrict__ dstates, const T* __restrict__ INV,
    const T* __restrict__ MqkT, const T* __restrict__ dUin, T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv,
    float* __restrict__ dg_raw, float* __restrict__ dbeta, float* __restrict__ dAl_part,
    float* __restrict__ ddt_part) {
  using L = GF<T, D>;
  using MM = Mma<T>;
  using MS = M16<T>;
  typedef typename MM::Frag Frag;
  constexpr int NW = L::NW, NT = L::NT, WPR = L::WPR;
  constexpr int KS = MM::KS, KPL = MM::KPL;
  constexpr int PG = L::PG, PN = L::PN, PT = L::PT, PC = L::PC, PR = L::PR;
  constexpr int NKD = D / KS;  // k-steps over a D-long contraction
  constexpr int NKC = 64 / KS; // k-steps over the chunk
  constexpr int EPV = 16 / L::ES;
  constexpr int VPR = D / EPV;              // 16-byte vectors per D-long row
  constexpr int NLS = D * VPR / NT;         // vectors per thread for a D x D state
  constexpr int NLT = 64 * VPR / NT;        // vectors per thread for a 64 x D tile
  constexpr int NLR = 64 * D / 4 / NT;      // 16-byte vectors per thread, 64 x D fp32
  static_assert(D * VPR % NT == 0 && 64 * VPR % NT == 0 && 16 * D % NT == 0, "tile split");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  float* sG = (float*)(smem + L::G_OFF);
  float* sR = sG;  // dg_raw staging at the end
  T* sO = (T*)(smem + L::O_OFF);
  T* sV = (T*)(smem + L::V_OFF);
  T* sU = sV;
  T* sK0 = (T*)(smem + L::K0_OFF);  // k for the intra-chunk phase, then dvcorr
  T* sDVC = sK0;
  T* sS = (T*)(smem + L::S_OFF);
  T* sDV = sS;
  T* sYT = (T*)(smem + L::YT_OFF);
  T* sQ = (T*)(smem + L::Q_OFF);
  T* sK = (T*)(smem + L::K_OFF);
  T* sIV = (T*)(smem + L::IV_OFF);
  T* sDM = (T*)(smem + L::DM_OFF);
  T* sDL = (T*)(smem + L::DL_OFF);
  T* sDQ = sQ;  // dq, dk staged in place of q, k: each lane overwrites only the
  T* sDK = sK;  // entries (row, own channel) it has just read
  float* sBeta = (float*)(smem + L::B_OFF);
  float* sDB1 = (float*)(smem + L::DB1_OFF);
  float* sDB2 = (float*)(smem + L::DB2_OFF);
  float* sRed = (float*)(smem + L::RED_OFF);
  float* sRq = (float*)(smem + L::RQ_OFF);  // reciprocal norms of q, k rows (QN)
  float* sRk = sRq + 64;
  float* sMd = (float*)(smem + L::MD_OFF);  // dMqk_rr of every row
  // diagonal 16x16 blocks of dMqk and dL in fp32, natural: block R, row rr, col cc at
  // dg*[R * DGB + rr * DGP + cc]
  float* dgM;
  float* dgL;
  int DGP, DGB;
  if constexpr (L::ES == 2) {
    float* base = (float*)(smem + L::DG_OFF);
    dgM = base;
    dgL = base + 4 * L::DGBS;
    DGP = L::PDG;
    DGB = L::DGBS;
  } else {
    dgM = (float*)sDM;
    dgL = (float*)sDL;
    DGP = PC;
    DGB = 16 * PC + 16;
  }

  const size_t DD = (size_t)D * D;
  const size_t rs = (size_t)H * D;  // token stride of per-token tensors
  const int items = NC * H;
  const int tid0 = threadIdx.x;
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_void*)smem;  // LDS byte address of smem

  // ------------------------------------------------------------------ loads
  // Persistent: one workgroup fills a CU's LDS, so each workgroup walks the
  // (chunk, head) items with stride gridDim.x, head fastest (item = chunk * H + head:
  // the workgroups in flight together read whole token rows of q, k, v, dO and g_raw,
  // all heads of the same chunks, and write whole rows of the gradients; about 2%
  // faster here than chunk-fastest order, which prep keeps: there it is the faster
  // one), and copies the next item's tiles
  // straight into LDS as soon as their regions are dead: S_in and v when the key
  // side is done (they then land during the intra phase), k, g_raw and beta once
  // the intra phase is done, dO once the dq staging over its tile is read out.
  // g_raw of wave w's 16 channels in 16-byte quads: lane l holds rows 16 t + (l >> 2),
  // channels 16 w + 4 (l & 3) .. + 3, t = 0..3 (rows past the chunk: masked later)
  f4 rg[4], rdb;  // rdb: the gate bias of the same four channels
  float rbeta;
  // (t: this thread's index, passed in so that the address arithmetic is redone per
  // item rather than held across the loop)
  // (part: 0 = all of S_in, v and INV; 1..3 = the pieces that the intra phase spreads over its
  // row tiles, so that the copies do not queue up ahead of the epilogue's loads and stores)
  auto issue_early = [&](int it, int t, int part) {
    const int c = it / H, h = it % H;
    const ChunkInfo ci = chunks[c];
    const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const T* sin = h_saved + ((size_t)c * H + h) * DD;
    if (part == 0 || part == 1)
      g2l_tile<T, D, D, NW, 0, 2, L::NPAD>(lds0 + L::S_OFF, sS, sin, D, D, w, lane);
    if (part == 0 || part == 2)
      g2l_tile<T, D, D, NW, 2, 1 << 20, L::NPAD>(lds0 + L::S_OFF, sS, sin, D, D, w, lane);
    if (part == 0 || part == 3) {
      g2l_tile<T, D, 64, NW, 0, 1 << 20, L::NPAD>(lds0 + L::V_OFF, sV,
                                                  v + (size_t)ci.t0 * rs + (size_t)h * D,
                                                  (unsigned)rs, ci.len, w, lane);
      g2l_tile<T, 64, 64, NW, 0, 1 << 20, L::CPAD>(lds0 + L::IV_OFF, sIV,
                                                   INV + ((size_t)c * H + h) * 4096, 64, 64, w,
                                                   lane);
    }
  };
  auto issue_front = [&](int it, int t) {
    const int c = it / H, h = it % H;
    const ChunkInfo ci = chunks[c];
    const size_t base = (size_t)ci.t0 * rs + (size_t)h * D;
    const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    g2l_tile<T, D, 64, NW, 0, 1 << 20, L::NPAD>(lds0 + L::K0_OFF, sK0, k + base, (unsigned)rs,
                                                ci.len, w, lane);
    const unsigned gcol = (16 * w + 4 * (lane & 3)) * 4;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int r = 16 * t4 + (lane >> 2);
      rg[t4] = *at((const f4*)(g_raw + base),
                   row_off(r < ci.len ? r : ci.len - 1, (unsigned)rs * 4) + gcol);
    }
    rbeta = *at(beta + (size_t)ci.t0 * H + h, row_off(lane < ci.len ? lane : ci.len - 1, H * 4));
    if constexpr (GV) rdb = *(const f4*)(dt_bias + (size_t)h * D + 16 * w + 4 * (lane & 3));
  };
  auto issue_late = [&](int it, int t) {
    const int c = it / H, h = it % H;
    const ChunkInfo ci = chunks[c];
    g2l_tile<T, D, 64, NW, 0, 1 << 20, L::NPAD>(lds0 + L::O_OFF, sO,
                                                dO + (size_t)ci.t0 * rs + (size_t)h * D,
                                                (unsigned)rs, ci.len,
                                                __builtin_amdgcn_readfirstlane(t >> 6),
                                                t & 63);
  };
  if ((int)blockIdx.x < items) {
    issue_early(blockIdx.x, tid0, 0);
    issue_front(blockIdx.x, tid0);
    issue_late(blockIdx.x, tid0);
  }
  settle(rg);  // waits for all of the first item's copies as well
  if constexpr (QN) __syncthreads();  // the first k tile is normalised in place below
  settle(rbeta);
  if constexpr (GV) settle(rdb);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
  // thread indices re-derived per item so that the lane-dependent LDS addresses
  // below stay inside the loop instead of being held in registers across it
  int tid = tid0;
  asm volatile("" : "+v"(tid));
  tid &= NT - 1;  // its range, for the compiler (24-bit multiplies in the addresses below)
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, cl = lane & 15;
  const int c = it / H, h = it % H;
  const int nxt = it + (int)gridDim.x;
  const ChunkInfo ci = chunks[c];
  const size_t t0 = ci.t0;
  const int Lr = ci.len;
  const size_t ch = (size_t)c * H + h;
  const size_t hD = (size_t)h * D;
  const T* qh = q + t0 * rs + hD;
  const unsigned rsb = (unsigned)rs * L::ES;  // token row stride in bytes
  const T* dSo = dstates + ch * DD;
  const float aA = __expf(A_log[h]) * gu;  // gu: natural-log decay per unit of the gate
  const int gch = 16 * w + cl;
  // state side: wave w owns the rows of block R1, value columns [64 half, +64)
  const int R1 = w / WPR, half = w % WPR;
  const int arow = 16 * R1 + cl;            // A-operand row of this lane
  const int crow = 16 * R1 + g4 * 4;        // first C row of this lane
  // dS_out into registers now (the gate, Kd / Kr and Y hide the load); it goes to LDS
  // over S_in once Y is done
  u32x4 rD[NLS];
#pragma unroll
  for (int l = 0; l < NLS; ++l) {
    const int idx = tid + l * NT, r = idx / VPR, sv = idx % VPR;
    rD[l] = *at((const u32x4*)dSo, (unsigned)(r * D + sv * EPV) * L::ES);
  }
  u32x4 rU[DU ? NLT : 1];  // DU: this chunk's dU rows
  if constexpr (DU) {
#pragma unroll
    for (int l = 0; l < NLT; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, sv = idx % VPR;
      rU[l] = *at((const u32x4*)(dUin + ch * 64 * D), (unsigned)(r * D + sv * EPV) * L::ES);
    }
  }
  if (tid < 64) sBeta[tid] = tid < Lr ? rbeta : 0.f;
  if constexpr (QN) {  // k rows normalised in place (rows past the chunk are zero)
#pragma unroll
    for (int l = 0; l < NLT; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, sv = idx % VPR;
      u32x4 kv = *(const u32x4*)(sK0 + r * PN + sv * EPV);
      const float rr = l2n_piece<T, VPR>(kv);
      *(u32x4*)(sK0 + r * PN + sv * EPV) = kv;
      if (sv == 0) sRk[r] = rr;
    }
  }
  {  // in-chunk cumulative gate (log2 units), channel-major: sG[i][r].  The per-token
     // gates go into this wave's 16 channel rows of the tile (written and read back by
     // this wave only), then lane (g4, cl) sums channel 16 w + cl over rows 16 g4 .. + 15
     // and the sums of the earlier row parts come from the lanes that hold them
    f4 db = f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (GV) db = has_db ? rdb : db;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int r = 16 * t4 + (lane >> 2);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sG[(16 * w + 4 * (lane & 3) + e) * PG + r] =
            r < Lr ? gate_log2(rg[t4][e] + db[e], aA) : 0.f;
    }
    float x[16];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const f4 t = *(const f4*)(sG + gch * PG + g4 * 16 + 4 * qq);
      x[4 * qq] = t[0]; x[4 * qq + 1] = t[1]; x[4 * qq + 2] = t[2]; x[4 * qq + 3] = t[3];
    }
    float run = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      run += x[rr];
      x[rr] = run;
    }
    float tp[4];
    rows_gather(run, tp);
    const float add = (g4 > 0 ? tp[0] : 0.f) + (g4 > 1 ? tp[1] : 0.f) + (g4 > 2 ? tp[2] : 0.f);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      *(f4*)(sG + gch * PG + g4 * 16 + 4 * qq) =
          f4{x[4 * qq] + add, x[4 * qq + 1] + add, x[4 * qq + 2] + add, x[4 * qq + 3] + add};
  }
  // S_in, v, INV and k have landed: they were issued before g_raw and beta, which the
  // previous item waited for (dO and dS_out may still be in flight; the dS_out stores to
  // LDS wait for both, in issue order)
  __syncthreads();
  Frag kf[NKD];                              // raw k of row arow (permuted k order)
#pragma unroll
  for (int kk = 0; kk < NKD; ++kk) kf[kk] = MM::ld_perm(sK0 + arow * PN, kk * KS, lane);
  Frag fI[NKC], fIT[NKC], fMT[DU ? 1 : NKC];  // rows arow of INV, INV^T, Mqk^T
#pragma unroll
  for (int ks = 0; ks < NKC; ++ks) {
    fI[ks] = MM::load(sIV + arow * PC + ks * KS + g4 * KPL);
    if constexpr (DU) {  // row arow of INV^T, permuted order (dU is read across its rows)
      fIT[ks] = MM::ld_tr(sIV, PC, ks * KS, 16 * R1, lane);
    } else {
      fMT[ks] = MM::ld_perm(MqkT + ch * 4096 + arow * 64, ks * KS, lane);
      fIT[ks] = MM::ld_tr_nat(sIV, PC, ks * KS, 16 * R1, lane);
    }
  }

  // ------------------------------------------------------------- state side
  // decayed key rows of this lane: Kd = K e^G (for Y), Kr = K e^{G_T - G} (for dU)
  Frag akd[NKD], akr[DU ? 1 : NKD];
#pragma unroll
  for (int kk = 0; kk < NKD; ++kk) {
    float kd[KPL], kr[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int i = kk * KS + MM::kperm(g4, j);
      const float gg = sG[i * PG + arow];
      const float kv = MM::elem(kf[kk], j);
      kd[j] = kv * ex2(gg);
      if constexpr (!DU) kr[j] = kv * ex2(sG[i * PG + 63] - gg);
    }
    akd[kk] = MM::from_vals(kd);
    if constexpr (!DU) akr[kk] = MM::from_vals(kr);
  }
  // Y = V - Kd S_in
  f4 Y[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) Y[nt] = zero4();
#pragma unroll
  for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      Y[nt] = MM::mma(akd[kk], MM::ld_tr(sS, PN, kk * KS, 64 * half + nt * 16, lane), Y[nt]);
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int d = 64 * half + nt * 16 + cl;
    f4 by;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Y[nt][j] = to_f(sV[(crow + j) * PN + d]) - Y[nt][j];
      by[j] = sBeta[crow + j] * Y[nt][j];
    }
    store_ct<T>(sYT, PT, 16 * R1, 64 * half + nt * 16, by, lane);
  }
  // key-side operands: S_in row of this lane's key channel
  const int ic = 16 * w + cl;
  Frag bS[NKD];
#pragma unroll
  for (int kk = 0; kk < NKD; ++kk) bS[kk] = MM::load(sS + ic * PN + kk * KS + g4 * KPL);
  __syncthreads();  // (beta Y)^T complete; S_in and v are dead
#pragma unroll
  for (int l = 0; l < NLS; ++l) {  // dS_out over S_in, natural
    const int idx = tid + l * NT, r = idx / VPR, sv = idx % VPR;
    *(u32x4*)(sS + r * PN + sv * EPV) = rD[l];
  }
  {  // U = INV (beta Y)
    f4 U[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) U[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      const Frag a = fI[ks];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const Frag b = MM::load(sYT + (64 * half + nt * 16 + cl) * PT + ks * KS + g4 * KPL);
        U[nt] = MM::mma(a, b, U[nt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) store_c<T>(sU, PN, 16 * R1, 64 * half + nt * 16, U[nt], lane);
  }
  wait_vmem();      // (dO: already waited for by the dS_out stores, which follow it)
  __syncthreads();  // dS_out in place; U complete; (beta Y)^T dead
  if constexpr (DU) {  // dU from memory, natural rows, over the dead (beta Y)^T
#pragma unroll
    for (int l = 0; l < NLT; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, sv = idx % VPR;
      *(u32x4*)(sYT + r * PN + sv * EPV) = rU[l];
    }
  } else {  // dU = Mqk^T dO + Kr dS_out  ->  dU^T
    f4 dU[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) dU[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        dU[nt] = MM::mma(fMT[ks], MM::ld_tr(sO, PN, ks * KS, 64 * half + nt * 16, lane), dU[nt]);
    }
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        dU[nt] = MM::mma(akr[kk], MM::ld_tr(sS, PN, kk * KS, 64 * half + nt * 16, lane), dU[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) store_ct<T>(sYT, PT, 16 * R1, 64 * half + nt * 16, dU[nt], lane);
  }
  u32x4 rK[NLT];  // k for the intra-chunk phase, before the dvcorr tile is overwritten
#pragma unroll
  for (int l = 0; l < NLT; ++l) {
    const int idx = tid + l * NT, r = idx / VPR, sv = idx % VPR;
    rK[l] = *(const u32x4*)(sK0 + r * PN + sv * EPV);
  }
  Frag bD[NKD];  // dS_out row of this lane's key channel
#pragma unroll
  for (int kk = 0; kk < NKD; ++kk) bD[kk] = MM::load(sS + ic * PN + kk * KS + g4 * KPL);
  __syncthreads();  // dU^T complete; dS_out is dead
  {  // dvcorr = INV^T dU;  dv = beta . dvcorr (staged);  dbeta (first part)
    f4 dvc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) dvc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      const Frag a = fIT[ks];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const Frag b = DU ? MM::ld_tr(sYT, PN, ks * KS, 64 * half + nt * 16, lane)
                          : MM::load(sYT + (64 * half + nt * 16 + cl) * PT + ks * KS + g4 * KPL);
        dvc[nt] = MM::mma(a, b, dvc[nt]);
      }
    }
    float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      store_c<T>(sDVC, PN, 16 * R1, 64 * half + nt * 16, dvc[nt], lane);
      f4 dvv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        db[j] += dvc[nt][j] * Y[nt][j];
        dvv[j] = sBeta[crow + j] * dvc[nt][j];
      }
      store_c<T>(sDV, PN, 16 * R1, 64 * half + nt * 16, dvv, lane);
    }
    sum16_n(db);
    if (cl == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sDB1[half * 64 + crow + j] = db[j];
    }
  }
  // q for the intra-chunk phase (registers now, LDS once its tile is free); rows
  // past the chunk read the last row and are zeroed when stored
  u32x4 rQ[NLT];
#pragma unroll
  for (int l = 0; l < NLT; ++l) {
    const int idx = tid + l * NT, r = idx / VPR, sv = idx % VPR;
    rQ[l] = *at((const u32x4*)qh, row_off(r < Lr ? r : Lr - 1, rsb) + sv * 16);
  }
  __syncthreads();  // dvcorr and dv staged
  // Output copies: rows past the chunk store row Lr - 1 again (the same bytes as
  // the lane that owns it), so that every lane issues the same stores.
#pragma unroll
  for (int l = 0; l < NLT; ++l) {  // dv out, 16-byte vectors
    const int idx = tid + l * NT, r0 = idx / VPR, sv = idx % VPR;
    const int r = r0 < Lr ? r0 : Lr - 1;
    *at((u32x4*)(dv + t0 * rs + hD), row_off(r, rsb) + sv * 16) =
        *(const u32x4*)(sDV + r * PN + sv * EPV);
  }

  // --------------------------------------------------------------- key side
  // dKr = U dS_out^T, dQd0 = dO S_in^T, dKd0 = dvcorr S_in^T for key channels
  // [16w, 16w+16) and all 64 rows; p for the same channels.
  f4 aKr[4], aQd[4], aKd[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) aKr[rt] = aQd[rt] = aKd[rt] = zero4();
  float pp = 0.f;
#pragma unroll
  for (int kk = 0; kk < NKD; ++kk) {
    const int d0 = kk * KS + g4 * KPL;
    pp += MM::dot(bS[kk], bD[kk]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int r = rt * 16 + cl;
      aKr[rt] = MM::mma(MM::load(sU + r * PN + d0), bD[kk], aKr[rt]);
      aQd[rt] = MM::mma(MM::load(sO + r * PN + d0), bS[kk], aQd[rt]);
      aKd[rt] = MM::mma(MM::load(sDVC + r * PN + d0), bS[kk], aKd[rt]);
    }
  }
  pp = sum_rows(pp);
  // dMqk = tril(dO U^T), dL = -stril(dvcorr U^T): wave -> rows of block R1,
  // column tiles [4/WPR * half, ...)
  constexpr int CTW = 4 / WPR;
  f4 am[CTW], al[CTW];
#pragma unroll
  for (int st = 0; st < CTW; ++st) am[st] = al[st] = zero4();
#pragma unroll
  for (int kk = 0; kk < NKD; ++kk) {
    const int d0 = kk * KS + g4 * KPL;
    const Frag ao = MM::load(sO + arow * PN + d0);
    const Frag av = MM::load(sDVC + arow * PN + d0);
#pragma unroll
    for (int st = 0; st < CTW; ++st) {
      const Frag b = MM::load(sU + ((CTW * half + st) * 16 + cl) * PN + d0);
      am[st] = MM::mma(ao, b, am[st]);
      al[st] = MM::mma(av, b, al[st]);
    }
  }
  __syncthreads();  // dO, U, dvcorr and the dv staging are dead
  // dMqk, dL (masked, natural) as act-dtype tiles; fp32 copies of the diagonal blocks
#pragma unroll
  for (int st = 0; st < CTW; ++st) {
    const int s = (CTW * half + st) * 16 + cl;
    f4 m, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = crow + j;
      m[j] = s <= r ? am[st][j] : 0.f;
      l[j] = s < r ? -al[st][j] : 0.f;
      if (s == r) sMd[r] = m[j];
    }
    store_c<T>(sDM, PC, 16 * R1, (CTW * half + st) * 16, m, lane);
    store_c<T>(sDL, PC, 16 * R1, (CTW * half + st) * 16, l, lane);
    if constexpr (L::ES == 2) {
      if (CTW * half + st == R1) {
        float* b0 = dgM + R1 * DGB;
        float* b1 = dgL + R1 * DGB;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b0[(g4 * 4 + j) * DGP + cl] = m[j];
          b1[(g4 * 4 + j) * DGP + cl] = l[j];
        }
      }
    }
  }
#pragma unroll
  for (int l = 0; l < NLT; ++l) {  // q, k natural
    const int idx = tid + l * NT, r = idx / VPR, sv = idx % VPR;
    u32x4 qv = rQ[l];
    if constexpr (QN) {
      const float rr = l2n_piece<T, VPR>(qv);
      if (sv == 0) sRq[r] = rr;
    }
    *(u32x4*)(sQ + r * PN + sv * EPV) = qv & (r < Lr ? ~0u : 0u);
    *(u32x4*)(sK + r * PN + sv * EPV) = rK[l];
  }
  __syncthreads();

  // ------------------------------------------------ intra-chunk decay terms
  // Lane: key channel ic.  Pairs (r, s) inside one 16-row block are summed exactly
  // in fp32 on VALU, one (channel, block) per lane, with the pairwise decays built
  // as running products of per-token factors 2^{G_t - G_{t-1}} <= 1.  Pairs across
  // blocks run on MFMA with anchored operands (formed once per block, reused for
  // every row tile).
  const float* Gi = sG + ic * PG;  // G of channel ic, by row
  const int n0 = 16 * w;           // first key channel of this wave
  const float gT = Gi[63];
  // (1) diagonal blocks: lane -> block g4 of channel ic (dec[s] = e^{G_r - G_s}).  x1_r =
  //     sum_{s<r} dMqk_rs k_s e^{G_r-G_s}, x2_r = the same with dL, z_s = sum_{r>s}
  //     (dMqk_rs q_r + beta_r dL_rs k_r) e^{G_r-G_s}; all rows and columns inside the
  //     block, the pairs r = s left out: their terms, dMqk_rr k_r in dq and dMqk_rr q_r
  //     in dk, carry no decay and cancel exactly in the gate gradient, so they are added
  //     to dq and dk alone (the gate gradient is formed without them, and is exactly 0
  //     where every decay between two tokens underflows).
  float x1d[4][4], x2d[4][4], zd[4][4];  // C layout: rows 16 rt + 4 g4 + j
  {
    const int rb = 16 * g4;
    float Gb[16], kb[16], dec[16], x1[16], x2[16], z[16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f4 t = *(const f4*)(Gi + rb + 4 * m);
      Gb[4 * m] = t[0]; Gb[4 * m + 1] = t[1]; Gb[4 * m + 2] = t[2]; Gb[4 * m + 3] = t[3];
    }
    // k and q of column ic, rows rb .. rb + 15: transposing reads of four rows each
    // for bf16 (lane (g4, cl) receives rows rb + 4 m + e of column 16 w + cl)
    if constexpr (L::ES == 2) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x4 t4 = ld_tr4(sK, PN, rb + 4 * m, 16 * w, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) kb[4 * m + e] = (float)t4[e];
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) kb[t] = to_f(sK[(rb + t) * PN + ic]);
    }
    const float* mb = dgM + g4 * DGB;
    const float* lb = dgL + g4 * DGB;
    bf16x4 q4;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float qr;
      if constexpr (L::ES == 2) {
        if (r % 4 == 0) q4 = ld_tr4(sQ, PN, rb + r, 16 * w, lane);
        qr = (float)q4[r % 4];
      } else {
        qr = to_f(sQ[(rb + r) * PN + ic]);
      }
      const float bkr = sBeta[rb + r] * kb[r];
      if (r > 0) {
        const float al = ex2(Gb[r] - Gb[r - 1]);
#pragma unroll
        for (int s = 0; s < r; ++s) dec[s] *= al;
      }
      dec[r] = 1.f;
      z[r] = 0.f;
      float mv[16], lv[16];
#pragma unroll
      for (int m = 0; m <= r / 4; ++m) {
        const f4 a = *(const f4*)(mb + r * DGP + 4 * m);
        const f4 b = *(const f4*)(lb + r * DGP + 4 * m);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mv[4 * m + e] = a[e];
          lv[4 * m + e] = b[e];
        }
      }
      float a1 = 0.f, a2 = 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) {
        const float kd = kb[s] * dec[s];
        a1 = fmaf(mv[s], kd, a1);
        a2 = fmaf(lv[s], kd, a2);
        z[s] = fmaf(fmaf(mv[s], qr, lv[s] * bkr), dec[s], z[s]);
      }
      x1[r] = a1;
      x2[r] = a2;
    }
    // to the C layout: lane (g4, cl) holds rows 16 g4 + t and wants rows
    // 16 rt + 4 g4 + j, i.e. a transpose of 4-row chunks across the four 16-lane rows
    // of the wave: one 32-lane swap stage and one 16-lane swap stage per element.
    // (swap32 / swap16: the lane swaps of the device helpers)
    auto exch = [&](const float (&src)[16], float (&dst)[4][4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = src[e], x1 = src[4 + e], x2 = src[8 + e], x3 = src[12 + e];
        swap32(x0, x2);
        swap32(x1, x3);
        swap16(x0, x1);
        swap16(x2, x3);
        dst[0][e] = x0;
        dst[1][e] = x1;
        dst[2][e] = x2;
        dst[3][e] = x3;
      }
    };
    exch(x1, x1d);
    exch(x2, x2d);
    exch(z, zd);
  }
  // (2) operands of the cross-block products, anchored once per block:
  //   X side (rows r of block R, s in block S < R):  k_s e^{G_e - G_s}, e = 16 S + 16;
  //   Z side (rows s of block S, r in block R > S):  (q_r, beta_r k_r) e^{G_r - G_a},
  //   a = 16 R.  The remaining factors e^{G_r - G_e} (X) and e^{G_a - G_s} (Z) are
  //   split into a per-channel factor between anchors and a per-row factor.
  typename MS::Op BX[3], BZq[4], BZk[4];
#pragma unroll
  for (int S = 0; S < 3; ++S) {
    float kv[4], gv[4], b[4];
    MS::ld_tr(sK, PN, 16 * S, n0, lane, kv);
    MS::ldf(Gi + 16 * S, g4, gv);
    const float ge = Gi[16 * S + 16];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = kv[j] * ex2(ge - gv[j]);
    BX[S] = MS::split(b);
  }
#pragma unroll
  for (int R = 1; R < 4; ++R) {
    float qv[4], kv[4], gv[4], bq[4], bk[4];
    MS::ld_tr(sQ, PN, 16 * R, n0, lane, qv);
    MS::ld_tr(sK, PN, 16 * R, n0, lane, kv);
    MS::ldf(Gi + 16 * R, g4, gv);
    const float ga = Gi[16 * R];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = ex2(gv[j] - ga);
      bq[j] = qv[j] * e;
      bk[j] = sBeta[16 * R + MS::kidx(g4, j)] * kv[j] * e;
    }
    BZq[R] = MS::split(bq);
    BZk[R] = MS::split(bk);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the operand set-up out of the tile loop
  float dG[4][4];
  float dkr_col = 0.f, dal = 0.f;
  float dbp[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int r0 = 16 * rt;
    const int ar = r0 + cl;  // A-operand row of this lane inside the tile
    float Gr[4];
    {
      const f4 t = *(const f4*)(Gi + r0 + 4 * g4);
      Gr[0] = t[0]; Gr[1] = t[1]; Gr[2] = t[2]; Gr[3] = t[3];
    }
    f4 X1a = zero4(), X2a = zero4(), Za = zero4();
    // e^{G_r} and e^{G_T - G_r} of this lane's rows, taken from the anchored row factors
    // below where a tile has them (a product of two factors <= 1: no overflow)
    float eGr[4], eTr[4];
    if (rt > 0) {
      const float ga = Gi[r0];
#pragma unroll
      for (int S = 0; S < rt; ++S) {
        const typename MS::Op a1 = MS::ld_op(sDM + ar * PC + 16 * S, g4);
        const typename MS::Op a2 = MS::ld_op(sDL + ar * PC + 16 * S, g4);
        if (S == rt - 1) {
          X1a = MS::op_sb(a1, BX[S], X1a);
          X2a = MS::op_sb(a2, BX[S], X2a);
        } else {
          const f4 p1 = MS::op_sb(a1, BX[S], zero4());
          const f4 p2 = MS::op_sb(a2, BX[S], zero4());
          const float m = ex2(ga - Gi[16 * S + 16]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            X1a[j] = fmaf(m, p1[j], X1a[j]);
            X2a[j] = fmaf(m, p2[j], X2a[j]);
          }
        }
      }
      const float eGa = ex2(ga);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = ex2(Gr[j] - ga);
        X1a[j] *= sc;
        X2a[j] *= sc;
        eGr[j] = sc * eGa;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) eGr[j] = ex2(Gr[j]);
    }
    if (rt < 3) {
      const float gb = Gi[r0 + 16];
#pragma unroll
      for (int R = rt + 1; R < 4; ++R) {
        const typename MS::Op a1 = MS::ld_tr_op(sDM, PC, 16 * R, r0, lane);
        const typename MS::Op a2 = MS::ld_tr_op(sDL, PC, 16 * R, r0, lane);
        if (R == rt + 1) {
          Za = MS::op_sb(a1, BZq[R], Za);
          Za = MS::op_sb(a2, BZk[R], Za);
        } else {
          f4 p = MS::op_sb(a1, BZq[R], zero4());
          p = MS::op_sb(a2, BZk[R], p);
          const float m = ex2(Gi[16 * R] - gb);
#pragma unroll
          for (int j = 0; j < 4; ++j) Za[j] = fmaf(m, p[j], Za[j]);
        }
      }
      const float eTb = ex2(gT - gb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = ex2(gb - Gr[j]);
        Za[j] *= sc;
        eTr[j] = sc * eTb;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) eTr[j] = ex2(gT - Gr[j]);
    }
    // combine and form the gate gradient of this tile
    const int rb = r0 + 4 * g4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rb + j;
      const float kr = to_f(sK[r * PN + ic]);
      const float qr = to_f(sQ[r * PN + ic]);
      const float br = sBeta[r];
      const float eG = eGr[j];
      const float x1 = X1a[j] + x1d[rt][j];
      const float x2 = X2a[j] + x2d[rt][j];
      const float dki = Za[j] + zd[rt][j];
      const float dqv = eG * aQd[rt][j] + x1;
      const float dkd = br * (-eG * aKd[rt][j] + x2);
      const float dkr = eTr[j] * aKr[rt][j];
      const float mrr = sMd[r];  // the pair r = s
      // the last row's own e^{G_T - G_r} carries no decay either: its two terms in the
      // gate gradient (-k dk_r here, +k dk_r in the last row's sum) are left out together
      const float dkg = r == 63 ? 0.f : dkr;
      dG[rt][j] = qr * dqv + kr * (dkd - dki - dkg);
      dkr_col += kr * dkg;
      dbp[rt][j] = kr * x2;
      sDQ[r * PN + ic] = from_f<T>(fmaf(mrr, kr, dqv));
      sDK[r * PN + ic] = from_f<T>(dkd + fmaf(mrr, qr, dki) + dkr);
    }
    // the next item's S_in and v, in pieces (their tiles are clear of the intra phase)
    if (rt < 3 && nxt < items) issue_early(nxt, tid, rt + 1);
  }
  // (QN) the raw q, k pieces that the output copies project with, issued now so that the
  // reductions below hide their latency
  u32x4 rawq[QN ? NLT : 1], rawk[QN ? NLT : 1];
  if constexpr (QN) {
#pragma unroll
    for (int l = 0; l < NLT; ++l) {
      const int idx = tid + l * NT, r0 = idx / VPR, sv = idx % VPR;
      const unsigned o = row_off(r0 < Lr ? r0 : Lr - 1, rsb) + sv * 16;
      rawq[l] = *at((const u32x4*)qh, o);
      rawk[l] = *at((const u32x4*)(k + t0 * rs + hD), o);
    }
  }
  // last row: sum_r k.dk_r + e^{G_T} p
  dkr_col = sum_rows(dkr_col);
  if (g4 == 3) dG[3][3] += dkr_col + ex2(gT) * pp;
  // reverse cumsum over r = 16 rt + 4 g4 + j; dG becomes dg_raw.  The gate's own
  // derivative comes from the cumulative gate: with aA = gu e^{A_log}, x = g_raw + dt_bias
  // and d = G_r - G_{r-1} = -aA softplus(x) log2(e), softplus(x) = -d ln 2 / aA and
  // sigmoid(x) = 1 - e^{-softplus(x)} = 1 - 2^{d / aA}, so dg_raw = dg . aA (2^{d / aA} - 1)
  // and the dA_log term is dg . d ln 2 (dg here is the gradient of the natural-log decay).
  // With no decay (A_log -> -inf, or e^{A_log} below 1e-30) d is 0 and 1/aA would overflow:
  // the factor is taken as 0 there, so dg_raw is 0 (its true size is below 1e-30 |dg|).
  const float inv_aA = aA > 1e-30f ? 1.f / aA : 0.f;
  float carry = 0.f;
#pragma unroll
  for (int rt = 3; rt >= 0; --rt) {
    const float tot = dG[rt][0] + dG[rt][1] + dG[rt][2] + dG[rt][3];
    float tr[4];
    rows_gather(tot, tr);
    const float t0v = tr[0], t1 = tr[1], t2 = tr[2], t3 = tr[3];
    float run = carry;
    if (g4 < 3) run += t3;
    if (g4 < 2) run += t2;
    if (g4 < 1) run += t1;
    carry += t0v + t1 + t2 + t3;
    float gq[5];  // G at rows rb - 1 .. rb + 3 of this lane (rb = 16 rt + 4 g4)
    {
      const int rb = rt * 16 + g4 * 4;
      const f4 t = *(const f4*)(Gi + rb);
      gq[0] = rb > 0 ? Gi[rb - 1] : 0.f;
      gq[1] = t[0]; gq[2] = t[1]; gq[3] = t[2]; gq[4] = t[3];
    }
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      run += dG[rt][j];
      const int r = rt * 16 + g4 * 4 + j;
      const float d = gq[j + 1] - gq[j];
      dG[rt][j] = run * (aA * (ex2(d * inv_aA) - 1.f));
      if (r < Lr) dal += run * (d * 0.69314718055994531f);
    }
  }
  if constexpr (GV) {  // this item's column sum of dg_raw (channel ic), for ddt_bias; every lane stores
    float sdt = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sdt += dG[rt][j];
    sdt = sum_rows(sdt);
    ddt_part[ch * D + ic] = sdt;
  }
  // dbeta second part, reduced over this wave's channels
  {
    float db2[16];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) db2[rt * 4 + j] = dbp[rt][j];
    sum16_n(db2);
    if (cl == 0) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) sDB2[w * 64 + rt * 16 + g4 * 4 + j] = db2[rt * 4 + j];
    }
  }
  dal = sum64(dal);
  if (lane == 0) sRed[w] = dal;
  __syncthreads();  // dq, dk staged; the gate tile is dead
  if (nxt < items) issue_front(nxt, tid);  // k over dMqk / dL, dead since the intra phase
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) sR[(rt * 16 + g4 * 4 + j) * PR + ic] = dG[rt][j];
#pragma unroll
  for (int l = 0; l < NLT; ++l) {  // dq, dk out, 16-byte vectors
    const int idx = tid + l * NT, r0 = idx / VPR, sv = idx % VPR;
    const int r = r0 < Lr ? r0 : Lr - 1;
    const unsigned o = row_off(r, rsb) + sv * 16;
    u32x4 vq = *(const u32x4*)(sDQ + r * PN + sv * EPV);
    u32x4 vk = *(const u32x4*)(sDK + r * PN + sv * EPV);
    if constexpr (QN) {  // back to the raw rows: dx = r (dxn - xn (xn . dxn)); the row's
                         // VPR pieces are VPR consecutive lanes (one DPP row)
      const float rrq = sRq[r], rrk = sRk[r];
      const u32x4 qn = l2n_apply<T>(rawq[l], rrq);
      const u32x4 kn = l2n_apply<T>(rawk[l], rrk);
      vq = l2n_project<T>(qn, vq, rrq, sum_group<VPR>(dot_piece<T>(qn, vq)));
      vk = l2n_project<T>(kn, vk, rrk, sum_group<VPR>(dot_piece<T>(kn, vk)));
    }
    *at((u32x4*)(dq + t0 * rs + hD), o) = vq;
    *at((u32x4*)(dk + t0 * rs + hD), o) = vk;
  }
  if (tid < 64 && tid < Lr) {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < WPR; ++x) s += sDB1[x * 64 + tid];
#pragma unroll
    for (int x = 0; x < NW; ++x) s += sDB2[x * 64 + tid];
    *at(dbeta + t0 * H + h, row_off(tid, H * 4)) = s;
  }
  if (tid == 0) {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) s += sRed[x];
    dAl_part[ch] = s;
  }
  __syncthreads();  // dg_raw staged
#pragma unroll
  for (int l = 0; l < NLR; ++l) {  // dg_raw out, 16-byte vectors
    const int idx = tid + l * NT, r0 = idx / (D / 4), sv = idx % (D / 4);
    const int r = r0 < Lr ? r0 : Lr - 1;
    *at((f4*)(dg_raw + t0 * rs + hD), row_off(r, (unsigned)rs * 4) + sv * 16) =
        *(const f4*)(sR + r * PR + sv * 4);
  }
  // The next item's g_raw and beta (and so, in issue order, its k, S_in, v and INV)
  // are waited for here, before the dO copy: the compiler does not see that copy, so a
  // wait at their first use would also cover this item's dq and dk stores.
  settle(rg);
  settle(rbeta);
  if constexpr (GV) settle(rdb);
  // dO over the dq staging, which is read out; issued after this item's last stores
  // so that the next item's first waits skip it
  if (nxt < items) issue_late(nxt, tid);
  __syncthreads();  // the gate tile (dg_raw staging) is read out before the next gate
  }
}

template <typename T, int D, bool GV, bool QN, bool DU>
static hipError_t gradf_v(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  const int items = s.NC * s.H;
  int resident = 0;
  hipError_t e = resident_blocks((const void*)k_gradf<T, D, GV, QN, DU>, GF<T, D>::NT, &resident);
  if (e != hipSuccess) return e;
  const int grid = items < resident ? items : resident;
  hipLaunchKernelGGL((k_gradf<T, D, GV, QN, DU>), dim3(grid), dim3(GF<T, D>::NT), 0, st, p.chunks,
                     s.NC, s.H, (const T*)p.q, (const T*)p.k, (const T*)p.v, (const T*)p.dO,
                     p.g_raw, p.beta, p.A_log, p.dt_bias, p.has_db, s.gu, (const T*)p.h_saved,
                     (const T*)p.dstates, (const T*)p.INV, (const T*)p.MqkT, (const T*)p.dU,
                     (T*)p.dq, (T*)p.dk, (T*)p.dv, p.dg_raw, p.dbeta, p.dAl_part, p.ddt_part);
  return hipGetLastError();
}

template <typename T, int D, bool DU>
static hipError_t gradf_d(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  const bool gv = p.has_db || p.ddt_bias;
  if (s.qn)
    return gv ? gradf_v<T, D, true, true, DU>(s, p, st) : gradf_v<T, D, false, true, DU>(s, p, st);
  return gv ? gradf_v<T, D, true, false, DU>(s, p, st) : gradf_v<T, D, false, false, DU>(s, p, st);
}

template <typename T, int D>
static hipError_t gradf_t(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  return p.dU ? gradf_d<T, D, true>(s, p, st) : gradf_d<T, D, false>(s, p, st);
}

hipError_t launch_gradf(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  if (s.NC == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? gradf_t<bf16, 128>(s, p, st) : gradf_t<bf16, 64>(s, p, st);
  return gradf_t<float, 64>(s, p, st);
}

}  // namespace kda
