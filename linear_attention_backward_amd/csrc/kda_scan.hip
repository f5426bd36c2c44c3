// kda_scan.hip -- reverse scan of the state gradient across chunks.
//
// For the chunks of one sequence, last to first ([PB] section 3: Kernel A is the
// serial dstate scan):
//   dS_out(c) = dS                       (stored for the gradient pass)
//   dS       <- exp(G_T) . dS + Tm_c dS + PT_c dO_c
// and dh0 = dS after the first chunk.  The map is affine in dS with a K x K linear
// part M_c = Diag(exp(G_T)) + Tm_c acting from the left, so every column of dS
// evolves on its own and a run of chunks composes into one affine map.
//
// One workgroup carries the whole K x V state of a (chunk group, head) in fp32
// MFMA accumulators and reads each chunk's Tm, PT, exp(G_T) and dO once.  The
// state goes through LDS as a natural bf16 tile, read back transposed as the B
// operand; Tm and PT rows are A fragments in the natural contraction order (one
// 16-byte load per lane), read straight from global memory one chunk ahead.
//
// Long sequences are split into groups of gs chunks and scanned in three passes
// (the pages name context parallelism as the lever for long contexts; here the
// groups run side by side on one GPU):
//   1. every group from the boundary I (transition workgroups: P_g, no dO terms)
//      and from 0 (offset workgroups: Q_g, with the dO terms), so that the state
//      before the group is P_g B_g + Q_g for the state B_g at its end;
//   2. per (sequence, head), the group boundaries B_g from the last group back;
//   3. every group again from its true boundary, storing dS_out of every chunk.
#include <cstdlib>

#include "kda_dev.h"
#include "kda_launch.h"

namespace kda {

// Tiling of a scan workgroup: the K x V right-hand side, wave w owning row tiles of
// row group w % 4 and column tiles of column group w / 4.
template <typename T, int D> struct SL {
  static constexpr int NW = D / 16;
  static constexpr int NT = NW * 64;
  static constexpr int ES = (int)sizeof(T);
  static constexpr int CW = NW / 4;           // column groups
  static constexpr int RTW = D / 64;          // row tiles per wave
  static constexpr int CTW = D / 16 / CW;     // column tiles per wave
  static constexpr int PS = D + 16 / ES;      // state tile pitch, natural [D][D]
  static constexpr int PO = D + 16 / ES;      // dO tile pitch, natural [64][D]
  static constexpr int S_SZ = D * PS * ES;
  static constexpr int O_SZ = 64 * PO * ES;
  static constexpr int TOTAL = 2 * S_SZ + 2 * O_SZ;
};

// PQ = false: scan a group from its boundary (dht for the last group of a
// sequence, else bnd), store dS_out of every chunk and, for the first group, dh0.
// PQ = true: blockIdx.z = 0 scans a group from I without the dO terms and stores
// P_g (act dtype); blockIdx.z = 1 scans it from 0 and stores Q_g (fp32).
template <typename T, int D, bool PQ>
__global__ __launch_bounds__(4 * D) void k_scanw(
    const ChunkInfo* __restrict__ chunks, const GroupInfo* __restrict__ groups, int H,
    const T* __restrict__ Tm, const T* __restrict__ PT, const float* __restrict__ eGT,
    const T* __restrict__ dO, const float* __restrict__ dht, const float* __restrict__ bnd,
    T* __restrict__ dstates, float* __restrict__ dh0, T* __restrict__ Pg,
    float* __restrict__ Qg) {
  using L = SL<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int NT = L::NT, RTW = L::RTW, CTW = L::CTW, PS = L::PS, PO = L::PO;
  constexpr int KS = MM::KS;
  constexpr int NKD = D / KS, NKC = 64 / KS;
  constexpr int EPV = 16 / L::ES;
  constexpr int VPR = D / EPV;                 // 16-byte vectors per D-long row
  constexpr int NLO = 64 * VPR / NT;           // dO vectors per thread
  constexpr int NLS = D * VPR / NT;            // state vectors per thread
  static_assert(64 * VPR % NT == 0 && D * VPR % NT == 0, "tile split");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  T* sS0 = (T*)smem;
  T* sO0 = (T*)(smem + 2 * L::S_SZ);

  const int g = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int rgp = w & 3, cgp = w >> 2;
  const GroupInfo gi = groups[g];
  const size_t DD = (size_t)D * D;
  const size_t uh = (size_t)gi.seq * H + h;  // (sequence, head)
  const size_t gh = (size_t)g * H + h;       // (group, head)
  const bool trans = PQ && blockIdx.z == 0;  // transition columns: identity start, no dO

  f4 acc[RTW][CTW];
  {
    const float* src = nullptr;
    if constexpr (!PQ) src = (gi.flags & GRP_LAST) ? (dht ? dht + uh * DD : nullptr) : bnd + gh * DD;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const int i0 = (rgp * RTW + rt) * 16 + 4 * g4;
        const int col = (cgp * CTW + ct) * 16 + cl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (PQ)
            acc[rt][ct][j] = (trans && i0 + j == col) ? 1.f : 0.f;
          else
            acc[rt][ct][j] = src ? src[(size_t)(i0 + j) * D + col] : 0.f;
        }
      }
  }

  // Operands of one chunk: Tm and PT rows (A fragments), exp(G_T) of this lane's
  // rows, and the chunk's dO tile (16-byte vectors, stored to LDS one step later).
  // Two sets alternate so that the loads for the next chunk, issued before this
  // chunk's products, are first waited on in the next step.
  auto load_a = [&](int cgl, Frag (&A)[RTW][NKD], Frag (&P)[RTW][NKC], f4 (&E)[RTW]) {
    const size_t ch = (size_t)cgl * H + h;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int i = (rgp * RTW + rt) * 16 + cl;
#pragma unroll
      for (int kk = 0; kk < NKD; ++kk) A[rt][kk] = MM::ld_nat(Tm + ch * DD + (size_t)i * D, kk * KS, lane);
      if (!trans) {
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) P[rt][kk] = MM::ld_nat(PT + ch * D * 64 + (size_t)i * 64, kk * KS, lane);
      }
      E[rt] = *(const f4*)(eGT + ch * D + (rgp * RTW + rt) * 16 + 4 * g4);
    }
  };
  auto load_do = [&](int cgl, u32x4 (&R)[NLO]) {
    const ChunkInfo ci = chunks[cgl];
#pragma unroll
    for (int l = 0; l < NLO; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (r < ci.len && !trans) x = *(const u32x4*)(dO + ((size_t)(ci.t0 + r) * H + h) * D + vv * EPV);
      R[l] = x;
    }
  };
  // One chunk, last to first: issue the next chunk's loads, publish the state (and
  // this chunk's dO tile), store dS_out, then dS <- exp(G_T) . dS + Tm dS + PT dO.
  auto step = [&](int cc, Frag (&ta)[RTW][NKD], Frag (&pa)[RTW][NKC], f4 (&eg)[RTW],
                  u32x4 (&ro)[NLO], Frag (&tn)[RTW][NKD], Frag (&pn)[RTW][NKC], f4 (&en)[RTW],
                  u32x4 (&rn)[NLO]) {
    const int cgl = gi.c0 + cc;
    const size_t ch = (size_t)cgl * H + h;
    T* sS = sS0 + (cc & 1) * (PS * D);
    T* sO = sO0 + (cc & 1) * (PO * 64);
    if (cc > 0) {  // the next chunk's operands, into the set the previous step used
      load_a(cgl - 1, tn, pn, en);
      load_do(cgl - 1, rn);
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
        store_c<T>(sS, PS, (rgp * RTW + rt) * 16, (cgp * CTW + ct) * 16, acc[rt][ct], lane);
#pragma unroll
    for (int l = 0; l < NLO; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      *(u32x4*)(sO + r * PO + vv * EPV) = ro[l];
    }
    __syncthreads();
    if constexpr (!PQ) {  // dS_out of this chunk, 16-byte rows
      T* dst = dstates + ch * DD;
#pragma unroll
      for (int l = 0; l < NLS; ++l) {
        const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
        *(uint4*)(dst + (size_t)r * D + vv * EPV) = *(const uint4*)(sS + r * PS + vv * EPV);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rt][ct][j] *= eg[rt][j];
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const Frag b = MM::ld_tr_nat(sS, PS, kk * KS, (cgp * CTW + ct) * 16, lane);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) acc[rt][ct] = MM::mma(ta[rt][kk], b, acc[rt][ct]);
      }
    }
    if (!trans) {
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) {
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          const Frag b = MM::ld_tr_nat(sO, PO, kk * KS, (cgp * CTW + ct) * 16, lane);
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) acc[rt][ct] = MM::mma(pa[rt][kk], b, acc[rt][ct]);
        }
      }
    }
  };
  Frag ta0[RTW][NKD], pa0[RTW][NKC], ta1[RTW][NKD], pa1[RTW][NKC];
  f4 eg0[RTW], eg1[RTW];
  u32x4 ro0[NLO], ro1[NLO];
  int cc = gi.cnt - 1;
  if (cc >= 0) {
    load_a(gi.c0 + cc, ta0, pa0, eg0);
    load_do(gi.c0 + cc, ro0);
  }
  for (; cc >= 1; cc -= 2) {
    step(cc, ta0, pa0, eg0, ro0, ta1, pa1, eg1, ro1);
    step(cc - 1, ta1, pa1, eg1, ro1, ta0, pa0, eg0, ro0);
  }
  if (cc == 0) step(0, ta0, pa0, eg0, ro0, ta1, pa1, eg1, ro1);
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const int r0 = (rgp * RTW + rt) * 16;
      const int c0 = (cgp * CTW + ct) * 16;
      if constexpr (PQ) {
        if (trans) store_c<T>(Pg + gh * DD, D, r0, c0, acc[rt][ct], lane);
        else store_c<float>(Qg + gh * DD, D, r0, c0, acc[rt][ct], lane);
      } else {
        if ((gi.flags & GRP_FIRST) && dh0) store_c<float>(dh0 + uh * DD, D, r0, c0, acc[rt][ct], lane);
      }
    }
}

// Group maps of the split scan with the transition and the offset in one workgroup per
// (group, head): P_g from I without the dO terms and Q_g from 0 with them, so that every
// chunk's Tm is read once for both (k_scanw<PQ> runs them as separate workgroups, which
// takes two rounds of the GPU once there are more groups than CUs).  Both states and the
// chunk's dO tile go through LDS as natural tiles of T; with three of them the tiles are
// single-buffered (two barriers per chunk), while the next chunk's operands load into the
// other register set.
template <typename T, int D>
__global__ __launch_bounds__(4 * D) void k_scanpq(
    const ChunkInfo* __restrict__ chunks, const GroupInfo* __restrict__ groups, int H,
    const T* __restrict__ Tm, const T* __restrict__ PT, const float* __restrict__ eGT,
    const T* __restrict__ dO, T* __restrict__ Pg, float* __restrict__ Qg) {
  using L = SL<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int NT = L::NT, RTW = L::RTW, CTW = L::CTW, PS = L::PS, PO = L::PO;
  constexpr int KS = MM::KS;
  constexpr int NKD = D / KS, NKC = 64 / KS;
  constexpr int EPV = 16 / L::ES;
  constexpr int VPR = D / EPV;                 // 16-byte vectors per D-long row
  constexpr int NLO = 64 * VPR / NT;           // dO vectors per thread
  static_assert(64 * VPR % NT == 0, "tile split");
  __shared__ __attribute__((aligned(16))) char smem[2 * L::S_SZ + L::O_SZ];
  T* sP = (T*)smem;
  T* sQ = (T*)(smem + L::S_SZ);
  T* sO = (T*)(smem + 2 * L::S_SZ);

  const int g = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int rgp = w & 3, cgp = w >> 2;
  const GroupInfo gi = groups[g];
  const size_t DD = (size_t)D * D;
  const size_t gh = (size_t)g * H + h;  // (group, head)

  f4 ap[RTW][CTW], aq[RTW][CTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const int i0 = (rgp * RTW + rt) * 16 + 4 * g4;
      const int col = (cgp * CTW + ct) * 16 + cl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ap[rt][ct][j] = i0 + j == col ? 1.f : 0.f;
        aq[rt][ct][j] = 0.f;
      }
    }
  auto load_a = [&](int cgl, Frag (&A)[RTW][NKD], Frag (&P)[RTW][NKC], f4 (&E)[RTW]) {
    const size_t ch = (size_t)cgl * H + h;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int i = (rgp * RTW + rt) * 16 + cl;
#pragma unroll
      for (int kk = 0; kk < NKD; ++kk) A[rt][kk] = MM::ld_nat(Tm + ch * DD + (size_t)i * D, kk * KS, lane);
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) P[rt][kk] = MM::ld_nat(PT + ch * D * 64 + (size_t)i * 64, kk * KS, lane);
      E[rt] = *(const f4*)(eGT + ch * D + (rgp * RTW + rt) * 16 + 4 * g4);
    }
  };
  auto load_do = [&](int cgl, u32x4 (&R)[NLO]) {  // rows past the chunk: zero
    const ChunkInfo ci = chunks[cgl];
#pragma unroll
    for (int l = 0; l < NLO; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (r < ci.len) x = *(const u32x4*)(dO + ((size_t)(ci.t0 + r) * H + h) * D + vv * EPV);
      R[l] = x;
    }
  };
  // One chunk, last to first: issue the next chunk's loads, publish both states and this
  // chunk's dO, then P <- exp(G_T) . P + Tm P and Q <- exp(G_T) . Q + Tm Q + PT dO.
  auto step = [&](int cc, Frag (&ta)[RTW][NKD], Frag (&pa)[RTW][NKC], f4 (&eg)[RTW],
                  u32x4 (&ro)[NLO], Frag (&tn)[RTW][NKD], Frag (&pn)[RTW][NKC], f4 (&en)[RTW],
                  u32x4 (&rn)[NLO]) {
    const int cgl = gi.c0 + cc;
    if (cc > 0) {
      load_a(cgl - 1, tn, pn, en);
      load_do(cgl - 1, rn);
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        store_c<T>(sP, PS, (rgp * RTW + rt) * 16, (cgp * CTW + ct) * 16, ap[rt][ct], lane);
        store_c<T>(sQ, PS, (rgp * RTW + rt) * 16, (cgp * CTW + ct) * 16, aq[rt][ct], lane);
      }
#pragma unroll
    for (int l = 0; l < NLO; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      *(u32x4*)(sO + r * PO + vv * EPV) = ro[l];
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ap[rt][ct][j] *= eg[rt][j];
          aq[rt][ct][j] *= eg[rt][j];
        }
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const Frag bp = MM::ld_tr_nat(sP, PS, kk * KS, (cgp * CTW + ct) * 16, lane);
        const Frag bq = MM::ld_tr_nat(sQ, PS, kk * KS, (cgp * CTW + ct) * 16, lane);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
          ap[rt][ct] = MM::mma(ta[rt][kk], bp, ap[rt][ct]);
          aq[rt][ct] = MM::mma(ta[rt][kk], bq, aq[rt][ct]);
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < NKC; ++kk) {
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const Frag b = MM::ld_tr_nat(sO, PO, kk * KS, (cgp * CTW + ct) * 16, lane);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) aq[rt][ct] = MM::mma(pa[rt][kk], b, aq[rt][ct]);
      }
    }
    __syncthreads();  // the tiles are read before the next chunk writes them
  };
  Frag ta0[RTW][NKD], pa0[RTW][NKC], ta1[RTW][NKD], pa1[RTW][NKC];
  f4 eg0[RTW], eg1[RTW];
  u32x4 ro0[NLO], ro1[NLO];
  int cc = gi.cnt - 1;
  if (cc >= 0) {
    load_a(gi.c0 + cc, ta0, pa0, eg0);
    load_do(gi.c0 + cc, ro0);
  }
  for (; cc >= 1; cc -= 2) {
    step(cc, ta0, pa0, eg0, ro0, ta1, pa1, eg1, ro1);
    step(cc - 1, ta1, pa1, eg1, ro1, ta0, pa0, eg0, ro0);
  }
  if (cc == 0) step(0, ta0, pa0, eg0, ro0, ta1, pa1, eg1, ro1);
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const int r0 = (rgp * RTW + rt) * 16;
      const int c0 = (cgp * CTW + ct) * 16;
      store_c<T>(Pg + gh * DD, D, r0, c0, ap[rt][ct], lane);
      store_c<float>(Qg + gh * DD, D, r0, c0, aq[rt][ct], lane);
    }
}

// Group boundaries of one (sequence, head).  Backward (FWD = false): B = dht at the
// end of the last group; going back, B <- P_g B + Q_g is the state gradient at the end
// of the group before, stored as bnd of that group.  Forward (FWD = true): S = h0 at the
// start of the first group; going forward, S <- P_g S + Q_g is the state at the start
// of the next group, stored as its bnd.
template <typename T, int D, bool FWD>
__global__ __launch_bounds__(4 * D) void k_scan_bnd(const int* __restrict__ grp_off, int H,
                                                    const T* __restrict__ Pg,
                                                    const float* __restrict__ Qg,
                                                    const float* __restrict__ dht,
                                                    float* __restrict__ bnd) {
  using L = SL<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int RTW = L::RTW, CTW = L::CTW, PS = L::PS;
  constexpr int KS = MM::KS, NKD = D / KS;
  __shared__ __attribute__((aligned(16))) T sS[D * PS];
  const int n = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int rgp = w & 3, cgp = w >> 2;
  const size_t DD = (size_t)D * D;
  const int gb = grp_off[n], ng = grp_off[n + 1] - gb;
  f4 acc[RTW][CTW];
  {
    const float* src = dht ? dht + ((size_t)n * H + h) * DD : nullptr;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const int i0 = (rgp * RTW + rt) * 16 + 4 * g4;
        const int col = (cgp * CTW + ct) * 16 + cl;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rt][ct][j] = src ? src[(size_t)(i0 + j) * D + col] : 0.f;
      }
  }
  for (int it = 0; it + 1 < ng; ++it) {
    const int gg = FWD ? it : ng - 1 - it;  // the group whose map is applied
    const size_t gh = (size_t)(gb + gg) * H + h;
    // backward: the state gradient at the end of group gg - 1 is P_g B + Q_g;
    // forward: the state at the start of group gg + 1 is P_g S + Q_g
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
        store_c<T>(sS, PS, (rgp * RTW + rt) * 16, (cgp * CTW + ct) * 16, acc[rt][ct], lane);
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int i = (rgp * RTW + rt) * 16 + cl;
      Frag a[NKD];
#pragma unroll
      for (int kk = 0; kk < NKD; ++kk) a[kk] = MM::ld_nat(Pg + gh * DD + (size_t)i * D, kk * KS, lane);
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const int i0 = (rgp * RTW + rt) * 16 + 4 * g4;
        const int col = (cgp * CTW + ct) * 16 + cl;
        f4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = Qg[gh * DD + (size_t)(i0 + j) * D + col];
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk)
          x = MM::mma(a[kk], MM::ld_tr_nat(sS, PS, kk * KS, (cgp * CTW + ct) * 16, lane), x);
        acc[rt][ct] = x;
      }
    }
    __syncthreads();
    const size_t bh = (size_t)(gb + (FWD ? gg + 1 : gg - 1)) * H + h;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
        store_c<float>(bnd + bh * DD, D, (rgp * RTW + rt) * 16, (cgp * CTW + ct) * 16, acc[rt][ct],
                       lane);
  }
}

// ---------------------------------------------------------------------------
// Forward state scan (the production forward).  Per (sequence, head), chunks first to
// last, with U = INV diag(beta) (V - Kd S) written as X = Uv + Wn S (Wn = -W):
//   h_saved(c) = S;   O = Qd S + Mqk X;   S <- e^{G_T} . S + Kr^T X,
// and ht = S after the last chunk.  S is carried in fp32 MFMA accumulators with the
// tiling of the backward scan (wave w: row tiles of row group w % 4, column tiles of
// column group w / 4); X and O are 64 x V, wave w holding row tile w % 4 and the
// column tiles of column group w / 4.  S and X go through LDS as natural tiles of T,
// read back as B operands; O is staged in LDS and stored as 16-byte rows a step later.
// One workgroup per chunk group of a (sequence, head) (a whole sequence unless long
// sequences are split): PQ = false scans the group from its true start state (h0 for
// the first group, else bnd) and stores O, h_saved and, for the last group, ht;
// PQ = true scans it without outputs, blockIdx.z = 0 from I without the Uv term (the
// group's transition P_g, act dtype) and blockIdx.z = 1 from 0 (its offset Q_g, fp32),
// so that the state after the group is P_g S + Q_g for the state S before it.
template <typename T, int D, bool PQ>
__global__ __launch_bounds__(4 * D) void k_fscan(
    const ChunkInfo* __restrict__ chunks, const GroupInfo* __restrict__ groups, int H,
    const T* __restrict__ Wn, const T* __restrict__ KrT, const T* __restrict__ UvT,
    const T* __restrict__ Qd, const T* __restrict__ Mq, const float* __restrict__ eGT,
    const float* __restrict__ h0, const float* __restrict__ bnd, T* __restrict__ o,
    float* __restrict__ ht, T* __restrict__ h_saved, T* __restrict__ Pg,
    float* __restrict__ Qg) {
  using L = SL<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int NT = L::NT, RTW = L::RTW, CTW = L::CTW, PS = L::PS, PO = L::PO;
  constexpr int KS = MM::KS;
  constexpr int NKD = D / KS, NKC = 64 / KS;
  constexpr int EPV = 16 / L::ES;
  constexpr int VPR = D / EPV;       // 16-byte vectors per D-long row
  constexpr int NLO = 64 * VPR / NT; // O vectors per thread
  constexpr int NLS = D * VPR / NT;  // state vectors per thread
  static_assert(64 * VPR % NT == 0 && D * VPR % NT == 0, "tile split");
  __shared__ __attribute__((aligned(16))) char smem[L::S_SZ + 2 * L::O_SZ];
  T* sS = (T*)smem;
  T* sX = (T*)(smem + L::S_SZ);
  T* sO = (T*)(smem + L::S_SZ + L::O_SZ);

  const int gidx = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int rgp = w & 3, cgp = w >> 2;
  const int xr = w & 3;  // row tile of X and O
  const size_t DD = (size_t)D * D;
  const GroupInfo gi = groups[gidx];
  const size_t uh = (size_t)gi.seq * H + h;  // (sequence, head)
  const size_t gh = (size_t)gidx * H + h;    // (group, head)
  const int cb = gi.c0, nck = gi.cnt;
  const size_t rs = (size_t)H * D;
  const bool trans = PQ && blockIdx.z == 0;  // transition: identity start, no Uv term
  if constexpr (PQ) {  // no outputs in this pass
    o = nullptr;
    h_saved = nullptr;
  }

  f4 acc[RTW][CTW];
  {
    const float* src = nullptr;
    if constexpr (!PQ) src = (gi.flags & GRP_FIRST) ? (h0 ? h0 + uh * DD : nullptr) : bnd + gh * DD;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const int i0 = (rgp * RTW + rt) * 16 + 4 * g4;
        const int col = (cgp * CTW + ct) * 16 + cl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (PQ)
            acc[rt][ct][j] = (trans && i0 + j == col) ? 1.f : 0.f;
          else
            acc[rt][ct][j] = src ? src[(size_t)(i0 + j) * D + col] : 0.f;
        }
      }
  }

  // One set of operand fragments, each part refilled for the next chunk right after its
  // last use in the current step (so that it has most of a step to land).
  Frag fw[NKD], fq[NKD], fm[NKC], fk[RTW][NKC];
  f4 fuv[CTW], fe[RTW];
  auto load_xo = [&](int cg) {  // operands of X and of Qd S
    const size_t ch = (size_t)cg * H + h;
    const int r = 16 * xr + cl;
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) {
      fw[kk] = MM::ld_nat(Wn + ch * 64 * D + (size_t)r * D, kk * KS, lane);
      fq[kk] = MM::ld_nat(Qd + ch * 64 * D + (size_t)r * D, kk * KS, lane);
    }
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {  // Uv rows 16 xr + 4 g4 .. + 3 of column col
      const int col = (cgp * CTW + ct) * 16 + cl;
      const T* src = UvT + ch * D * 64 + (size_t)col * 64 + 16 * xr + 4 * g4;
      T u4[4];
      if constexpr (L::ES == 2) *(uint2*)u4 = *(const uint2*)src;
      else *(uint4*)u4 = *(const uint4*)src;
#pragma unroll
      for (int j = 0; j < 4; ++j) fuv[ct][j] = trans ? 0.f : to_f(u4[j]);
    }
  };
  auto load_m = [&](int cg) {
    const size_t ch = (size_t)cg * H + h;
#pragma unroll
    for (int kk = 0; kk < NKC; ++kk)
      fm[kk] = MM::ld_nat(Mq + ch * 4096 + (size_t)(16 * xr + cl) * 64, kk * KS, lane);
  };
  auto load_k = [&](int cg) {
    const size_t ch = (size_t)cg * H + h;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int i = (rgp * RTW + rt) * 16 + cl;
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) fk[rt][kk] = MM::ld_nat(KrT + ch * D * 64 + (size_t)i * 64, kk * KS, lane);
      fe[rt] = *(const f4*)(eGT + ch * D + (rgp * RTW + rt) * 16 + 4 * g4);
    }
  };
  // O of chunk cg (staged in sO) out as 16-byte rows; rows past the chunk are not
  // part of the sequence
  auto store_o = [&](int cg) {
    const ChunkInfo ci = chunks[cg];
#pragma unroll
    for (int l = 0; l < NLO; ++l) {
      const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
      if (r < ci.len)
        *(uint4*)(o + ((size_t)ci.t0 + r) * rs + (size_t)h * D + vv * EPV) =
            *(const uint4*)(sO + r * PO + vv * EPV);
    }
  };
  if (nck > 0) {
    load_xo(cb);
    load_m(cb);
    load_k(cb);
  }
  for (int c = 0; c < nck; ++c) {
    const int cg = cb + c;
    const bool more = c + 1 < nck;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
        store_c<T>(sS, PS, (rgp * RTW + rt) * 16, (cgp * CTW + ct) * 16, acc[rt][ct], lane);
    __syncthreads();
    if (h_saved) {  // the state at the start of this chunk, 16-byte rows
      T* dst = h_saved + ((size_t)cg * H + h) * DD;
#pragma unroll
      for (int l = 0; l < NLS; ++l) {
        const int idx = tid + l * NT, r = idx / VPR, vv = idx % VPR;
        *(uint4*)(dst + (size_t)r * D + vv * EPV) = *(const uint4*)(sS + r * PS + vv * EPV);
      }
    }
    if (o && c > 0) store_o(cg - 1);
    // X = Uv + Wn S and the first part of O, Qd S (same B fragments)
    f4 X[CTW], Oa[CTW];
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      X[ct] = fuv[ct];
      Oa[ct] = zero4();
    }
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const Frag b = MM::ld_tr_nat(sS, PS, kk * KS, (cgp * CTW + ct) * 16, lane);
        X[ct] = MM::mma(fw[kk], b, X[ct]);
        if (o) Oa[ct] = MM::mma(fq[kk], b, Oa[ct]);
      }
    }
    if (more) load_xo(cg + 1);
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) store_c<T>(sX, PO, 16 * xr, (cgp * CTW + ct) * 16, X[ct], lane);
    __syncthreads();
    if (o) {  // O += Mqk X, staged for the next step
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) {
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
          Oa[ct] = MM::mma(fm[kk], MM::ld_tr_nat(sX, PO, kk * KS, (cgp * CTW + ct) * 16, lane), Oa[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) store_c<T>(sO, PO, 16 * xr, (cgp * CTW + ct) * 16, Oa[ct], lane);
    }
    if (more) load_m(cg + 1);
    // S <- e^{G_T} . S + Kr^T X
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rt][ct][j] *= fe[rt][j];
#pragma unroll
    for (int kk = 0; kk < NKC; ++kk) {
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const Frag b = MM::ld_tr_nat(sX, PO, kk * KS, (cgp * CTW + ct) * 16, lane);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) acc[rt][ct] = MM::mma(fk[rt][kk], b, acc[rt][ct]);
      }
    }
    if (more) load_k(cg + 1);
  }
  if (o && nck > 0) {
    __syncthreads();  // the last chunk's O staging complete
    store_o(cb + nck - 1);
  }
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const int r0 = (rgp * RTW + rt) * 16, c0 = (cgp * CTW + ct) * 16;
      if constexpr (PQ) {
        if (trans) store_c<T>(Pg + gh * DD, D, r0, c0, acc[rt][ct], lane);
        else store_c<float>(Qg + gh * DD, D, r0, c0, acc[rt][ct], lane);
      } else {
        if ((gi.flags & GRP_LAST) && ht) store_c<float>(ht + uh * DD, D, r0, c0, acc[rt][ct], lane);
      }
    }
}

// Group maps of the forward's split scan with the transition and the offset in one
// workgroup per (group, head): P from I without the Uv term, Q from 0 with it,
//   X_P = Wn P,  X_Q = Uv + Wn Q,  P <- e^{G_T} . P + Kr^T X_P,  Q <- e^{G_T} . Q + Kr^T X_Q,
// so that each chunk's Wn and Kr^T fragments are read once for both.  The two states
// and the two X tiles go through LDS (two barriers per chunk); each operand part is
// refilled for the next chunk right after its last use.
template <typename T, int D>
__global__ __launch_bounds__(4 * D) void k_fscanpq(
    const GroupInfo* __restrict__ groups, int H, const T* __restrict__ Wn,
    const T* __restrict__ KrT, const T* __restrict__ UvT, const float* __restrict__ eGT,
    T* __restrict__ Pg, float* __restrict__ Qg) {
  using L = SL<T, D>;
  using MM = Mma<T>;
  typedef typename MM::Frag Frag;
  constexpr int RTW = L::RTW, CTW = L::CTW, PS = L::PS, PO = L::PO;
  constexpr int KS = MM::KS;
  constexpr int NKD = D / KS, NKC = 64 / KS;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::S_SZ + 2 * L::O_SZ];
  T* sP = (T*)smem;
  T* sQ = (T*)(smem + L::S_SZ);
  T* sXP = (T*)(smem + 2 * L::S_SZ);
  T* sXQ = (T*)(smem + 2 * L::S_SZ + L::O_SZ);

  const int gidx = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int rgp = w & 3, cgp = w >> 2;
  const int xr = w & 3;  // row tile of X
  const size_t DD = (size_t)D * D;
  const GroupInfo gi = groups[gidx];
  const size_t gh = (size_t)gidx * H + h;  // (group, head)
  const int cb = gi.c0, nck = gi.cnt;

  f4 ap[RTW][CTW], aq[RTW][CTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const int i0 = (rgp * RTW + rt) * 16 + 4 * g4;
      const int col = (cgp * CTW + ct) * 16 + cl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ap[rt][ct][j] = i0 + j == col ? 1.f : 0.f;
        aq[rt][ct][j] = 0.f;
      }
    }
  Frag fw[NKD], fk[RTW][NKC];
  f4 fuv[CTW], fe[RTW];
  auto load_x = [&](int cg) {  // operands of X: Wn rows and Uv
    const size_t ch = (size_t)cg * H + h;
    const int r = 16 * xr + cl;
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) fw[kk] = MM::ld_nat(Wn + ch * 64 * D + (size_t)r * D, kk * KS, lane);
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {  // Uv rows 16 xr + 4 g4 .. + 3 of column col
      const int col = (cgp * CTW + ct) * 16 + cl;
      const T* src = UvT + ch * D * 64 + (size_t)col * 64 + 16 * xr + 4 * g4;
      T u4[4];
      if constexpr (L::ES == 2) *(uint2*)u4 = *(const uint2*)src;
      else *(uint4*)u4 = *(const uint4*)src;
#pragma unroll
      for (int j = 0; j < 4; ++j) fuv[ct][j] = to_f(u4[j]);
    }
  };
  auto load_k = [&](int cg) {
    const size_t ch = (size_t)cg * H + h;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int i = (rgp * RTW + rt) * 16 + cl;
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) fk[rt][kk] = MM::ld_nat(KrT + ch * D * 64 + (size_t)i * 64, kk * KS, lane);
      fe[rt] = *(const f4*)(eGT + ch * D + (rgp * RTW + rt) * 16 + 4 * g4);
    }
  };
  if (nck > 0) {
    load_x(cb);
    load_k(cb);
  }
  for (int c = 0; c < nck; ++c) {
    const int cg = cb + c;
    const bool more = c + 1 < nck;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        store_c<T>(sP, PS, (rgp * RTW + rt) * 16, (cgp * CTW + ct) * 16, ap[rt][ct], lane);
        store_c<T>(sQ, PS, (rgp * RTW + rt) * 16, (cgp * CTW + ct) * 16, aq[rt][ct], lane);
      }
    __syncthreads();
    f4 XP[CTW], XQ[CTW];
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      XP[ct] = zero4();
      XQ[ct] = fuv[ct];
    }
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        XP[ct] = MM::mma(fw[kk], MM::ld_tr_nat(sP, PS, kk * KS, (cgp * CTW + ct) * 16, lane), XP[ct]);
        XQ[ct] = MM::mma(fw[kk], MM::ld_tr_nat(sQ, PS, kk * KS, (cgp * CTW + ct) * 16, lane), XQ[ct]);
      }
    }
    if (more) load_x(cg + 1);
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      store_c<T>(sXP, PO, 16 * xr, (cgp * CTW + ct) * 16, XP[ct], lane);
      store_c<T>(sXQ, PO, 16 * xr, (cgp * CTW + ct) * 16, XQ[ct], lane);
    }
    __syncthreads();  // X tiles complete; the state tiles are dead
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ap[rt][ct][j] *= fe[rt][j];
          aq[rt][ct][j] *= fe[rt][j];
        }
#pragma unroll
    for (int kk = 0; kk < NKC; ++kk) {
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const Frag bp = MM::ld_tr_nat(sXP, PO, kk * KS, (cgp * CTW + ct) * 16, lane);
        const Frag bq = MM::ld_tr_nat(sXQ, PO, kk * KS, (cgp * CTW + ct) * 16, lane);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
          ap[rt][ct] = MM::mma(fk[rt][kk], bp, ap[rt][ct]);
          aq[rt][ct] = MM::mma(fk[rt][kk], bq, aq[rt][ct]);
        }
      }
    }
    if (more) load_k(cg + 1);
  }
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const int r0 = (rgp * RTW + rt) * 16, c0 = (cgp * CTW + ct) * 16;
      store_c<T>(Pg + gh * DD, D, r0, c0, ap[rt][ct], lane);
      store_c<float>(Qg + gh * DD, D, r0, c0, aq[rt][ct], lane);
    }
}

template <typename T, int D>
static hipError_t fscan_t(const Shape& s, const FwdPtrs& p, hipStream_t st) {
  if (s.gs > 0) {  // chunk groups side by side: P_g and Q_g, the boundaries, then the outputs
    // (P_g and Q_g in one workgroup per (group, head) when separate ones would need more
    // than one round of the GPU; KDA_SCANPQ=0 / 1 forces either form)
    int resident = 0;
    hipError_t e = resident_blocks((const void*)k_fscan<T, D, true>, SL<T, D>::NT, &resident);
    if (e != hipSuccess) return e;
    bool joint = 2 * (int64_t)s.NG * s.H > resident;
    if (const char* env = std::getenv("KDA_SCANPQ")) joint = std::atoi(env) != 0;
    if (joint) {
      hipLaunchKernelGGL((k_fscanpq<T, D>), dim3((unsigned)s.NG, (unsigned)s.H),
                         dim3(SL<T, D>::NT), 0, st, p.groups, s.H, (const T*)p.Wn, (const T*)p.KrT,
                         (const T*)p.UvT, p.eGT, (T*)p.Pg, p.Qg);
    } else {
      hipLaunchKernelGGL((k_fscan<T, D, true>), dim3((unsigned)s.NG, (unsigned)s.H, 2),
                         dim3(SL<T, D>::NT), 0, st, p.chunks, p.groups, s.H, (const T*)p.Wn,
                         (const T*)p.KrT, (const T*)p.UvT, (const T*)p.Qd, (const T*)p.Mq, p.eGT,
                         nullptr, nullptr, nullptr, nullptr, nullptr, (T*)p.Pg, p.Qg);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_scan_bnd<T, D, true>), dim3((unsigned)s.N, (unsigned)s.H),
                       dim3(SL<T, D>::NT), 0, st, p.grp_off, s.H, (const T*)p.Pg, p.Qg,
                       p.h0, p.bnd);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_fscan<T, D, false>), dim3((unsigned)s.NG, (unsigned)s.H),
                     dim3(SL<T, D>::NT), 0, st, p.chunks, p.groups, s.H, (const T*)p.Wn,
                     (const T*)p.KrT, (const T*)p.UvT, (const T*)p.Qd, (const T*)p.Mq, p.eGT, p.h0,
                     p.bnd, (T*)p.o, p.ht, (T*)p.h_saved, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_fscan(const Shape& s, const FwdPtrs& p, hipStream_t st) {
  if (s.NG == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? fscan_t<bf16, 128>(s, p, st) : fscan_t<bf16, 64>(s, p, st);
  return fscan_t<float, 64>(s, p, st);
}

template <typename T, int D>
static hipError_t scan_t(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  const dim3 gg((unsigned)s.NG, (unsigned)s.H);
  if (s.gs > 0) {
    // the group maps: transition and offset in separate workgroups while both fit one
    // round of the GPU, else in one workgroup per (group, head) (each Tm read once);
    // KDA_SCANPQ=0 / 1 forces the separate / the joint form
    int resident = 0;
    hipError_t e = resident_blocks((const void*)k_scanw<T, D, true>, SL<T, D>::NT, &resident);
    if (e != hipSuccess) return e;
    bool joint = 2 * (int64_t)s.NG * s.H > resident;
    if (const char* env = std::getenv("KDA_SCANPQ")) joint = std::atoi(env) != 0;
    if (joint) {
      hipLaunchKernelGGL((k_scanpq<T, D>), gg, dim3(SL<T, D>::NT), 0, st, p.chunks, p.groups, s.H,
                         (const T*)p.Tm, (const T*)p.PT, p.eGT, (const T*)p.dO, (T*)p.Pg, p.Qg);
    } else {
      hipLaunchKernelGGL((k_scanw<T, D, true>), dim3((unsigned)s.NG, (unsigned)s.H, 2),
                         dim3(SL<T, D>::NT), 0, st, p.chunks,
                         p.groups, s.H, (const T*)p.Tm, (const T*)p.PT, p.eGT, (const T*)p.dO,
                         nullptr, nullptr, nullptr, nullptr, (T*)p.Pg, p.Qg);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_scan_bnd<T, D, false>), dim3((unsigned)s.N, (unsigned)s.H),
                       dim3(SL<T, D>::NT), 0, st, p.grp_off, s.H,
                       (const T*)p.Pg, p.Qg, p.dht, p.bnd);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_scanw<T, D, false>), gg, dim3(SL<T, D>::NT), 0, st, p.chunks,
                     p.groups, s.H, (const T*)p.Tm, (const T*)p.PT, p.eGT, (const T*)p.dO, p.dht,
                     p.bnd, (T*)p.dstates, p.dh0, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_scan(const Shape& s, const BwdPtrs& p, hipStream_t st) {
  if (s.NG == 0) return hipSuccess;
  if (s.bf16) return s.D == 128 ? scan_t<bf16, 128>(s, p, st) : scan_t<bf16, 64>(s, p, st);
  return scan_t<float, 64>(s, p, st);
}

}  // namespace kda
