// kda_dev.h -- device helpers shared by the KDA backward kernels (gfx950).
//
// MFMA conventions (CDNA3/CDNA4 16x16 family, wave64):
//   A operand (16 x KS):  lane l holds row (l & 15), k = (l >> 4) * KPL + [0, KPL)
//   B operand (KS x 16):  lane l holds col (l & 15), k = (l >> 4) * KPL + [0, KPL)
//   C/D (16 x 16 fp32):   lane l holds col (l & 15), rows (l >> 4) * 4 + [0, 4)
// bf16 uses v_mfma_f32_16x16x32_bf16 (KS = 32, KPL = 8); fp32 uses
// v_mfma_f32_16x16x4_f32 (KS = 4, KPL = 1).  Every operand is therefore read from a
// layout in which the contraction index is contiguous: A as [m][k], B as [n][k].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes in registers

constexpr int CH = 64;      // chunk length (tokens)
constexpr int NTHR = 256;   // threads per workgroup (4 waves)
constexpr float LOG2E = 1.4426950408889634f;

// One row of the chunk table: a 64-token chunk of one sequence.
struct ChunkInfo {
  int t0;    // first token (packed index)
  int len;   // valid rows, 1..64
  int seq;   // sequence index
  int cidx;  // chunk index inside the sequence
};

// One row of the group table: a run of consecutive chunks of one sequence that the
// state-gradient scan treats as a unit (the whole sequence when it is not split).
struct GroupInfo {
  int c0;     // first chunk (index into the chunk table)
  int cnt;    // chunks in the group (0 only for an empty sequence)
  int seq;    // sequence index
  int flags;  // GRP_FIRST: first group of its sequence; GRP_LAST: last group
};
constexpr int GRP_FIRST = 1, GRP_LAST = 2;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// 2^x on the transcendental unit.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-token log decay in log2 units, g log2(e) with g = -e^{A_log} softplus(x)
// (aA = e^{A_log}).  softplus(x) log2(e) = max(x, 0) log2(e) + log2(1 + 2^{-|x| log2(e)}):
// the log's argument lies in [1, 2] and the exponent is <= 0, so the bare hardware
// log2 / exp2 apply with no range reduction.
__device__ __forceinline__ float gate_log2(float x, float aA) {
  const float t = __builtin_amdgcn_exp2f(-fabsf(x) * LOG2E);
  return -aA * fmaf(fmaxf(x, 0.f), LOG2E, __builtin_amdgcn_logf(1.f + t));
}

// Transposing LDS read (ds_read_b64_tr_b16).  Inside every group of 16 lanes, lane
// 4a + b receives element b of the 8-byte chunks that lanes a, a + 4, a + 8, a + 12
// of the group point at.  With lane 16G + s pointing at row k0 + (s >> 2), columns
// n0 + 4 (s & 3) .. + 3 of a row-major [k][n] tile, lane 16G + n therefore receives
// tile[k0 + e][n0 + n] for e = 0..3: a 4 x 16 block, read column-wise.  k0 is the
// row of the lane's own group (callers add the group offset).
typedef short s4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4v lds_s4v;
__device__ __forceinline__ bf16x4 ld_tr4(const bf16* tile, int pitch, int k0, int n0, int lane) {
  const int s = lane & 15;
  const bf16* p = tile + (k0 + (s >> 2)) * pitch + n0 + 4 * (s & 3);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)p));
}

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KS = 32, KPL = 8;
  typedef bf16x8 Frag;
  __device__ static __forceinline__ f4 mma(Frag a, Frag b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ Frag load(const bf16* p) { return *(const bf16x8*)p; }
  // Permuted contraction order for operands read across rows: lane group G holds
  // k = kb + 4G + j (j < 4) and k = kb + 16 + 4G + (j - 4) (j >= 4), so that one
  // fragment is two transposing reads of 16 consecutive rows each.  Both operands of
  // a product must use the same order.
  __device__ static __forceinline__ int kperm(int G, int j) {
    return j < 4 ? 4 * G + j : 12 + 4 * G + j;
  }
  // fragment of a row-major [k][n] LDS tile, contraction over its rows (permuted order)
  __device__ static __forceinline__ Frag ld_tr(const bf16* tile, int pitch, int kb, int n0,
                                               int lane) {
    const int G = lane >> 4;
    const bf16x4 lo = ld_tr4(tile, pitch, kb + 4 * G, n0, lane);
    const bf16x4 hi = ld_tr4(tile, pitch, kb + 16 + 4 * G, n0, lane);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Natural contraction order (lane group G holds k = kb + 8G + j): a fragment of a
  // row with contiguous k is one 16-byte load, and the matching fragment of a
  // row-major [k][n] LDS tile two transposing reads of 4 rows each.
  __device__ static __forceinline__ Frag ld_tr_nat(const bf16* tile, int pitch, int kb, int n0,
                                                   int lane) {
    const int G = lane >> 4;
    const bf16x4 lo = ld_tr4(tile, pitch, kb + 8 * G, n0, lane);
    const bf16x4 hi = ld_tr4(tile, pitch, kb + 8 * G + 4, n0, lane);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ static __forceinline__ Frag ld_nat(const bf16* row, int kb, int lane) {
    return *(const bf16x8*)(row + kb + 8 * (lane >> 4));
  }
  // fragment of a row with contiguous k (any memory), permuted order
  __device__ static __forceinline__ Frag ld_perm(const bf16* row, int kb, int lane) {
    const int G = lane >> 4;
    const bf16x4 lo = *(const bf16x4*)(row + kb + 4 * G);
    const bf16x4 hi = *(const bf16x4*)(row + kb + 16 + 4 * G);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // fragment of an fp32 row (any memory) in the permuted order, rounded to bf16
  __device__ static __forceinline__ Frag ld_perm_f32(const float* row, int kb, int lane) {
    const int G = lane >> 4;
    const f4 lo = *(const f4*)(row + kb + 4 * G);
    const f4 hi = *(const f4*)(row + kb + 16 + 4 * G);
    Frag r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
    r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
  }
  __device__ static __forceinline__ float elem(Frag f, int j) { return (float)f[j]; }
  __device__ static __forceinline__ Frag from_f32(const float* p) {
    f4 a = *(const f4*)p, b = *(const f4*)(p + 4);
    Frag r;
    r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)a[2]; r[3] = (bf16)a[3];
    r[4] = (bf16)b[0]; r[5] = (bf16)b[1]; r[6] = (bf16)b[2]; r[7] = (bf16)b[3];
    return r;
  }
  __device__ static __forceinline__ Frag from_vals(const float* v) {
    Frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (bf16)v[j];
    return r;
  }
  __device__ static __forceinline__ float dot(Frag a, Frag b) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += (float)a[j] * (float)b[j];
    return s;
  }
  // fp32-accurate product of fp32 operands on the bf16 unit: x = hi + lo with
  // hi = bf16(x), lo = bf16(x - hi); a.b ~ hi.hi + hi.lo + lo.hi (the dropped
  // lo.lo term is ~2^-16 relative).
  __device__ static __forceinline__ f4 mma3(const float* a, const float* b, f4 c) {
    Frag ah, al, bh, bl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ah[j] = (bf16)a[j];
      al[j] = (bf16)(a[j] - (float)ah[j]);
      bh[j] = (bf16)b[j];
      bl[j] = (bf16)(b[j] - (float)bh[j]);
    }
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KS = 4, KPL = 1;
  typedef float Frag;
  __device__ static __forceinline__ f4 mma(Frag a, Frag b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ Frag load(const float* p) { return *p; }
  __device__ static __forceinline__ int kperm(int G, int) { return G; }
  __device__ static __forceinline__ Frag ld_tr(const float* tile, int pitch, int kb, int n0,
                                               int lane) {
    return tile[(kb + (lane >> 4)) * pitch + n0 + (lane & 15)];
  }
  __device__ static __forceinline__ Frag ld_perm(const float* row, int kb, int lane) {
    return row[kb + (lane >> 4)];
  }
  __device__ static __forceinline__ Frag ld_tr_nat(const float* tile, int pitch, int kb, int n0,
                                                   int lane) {
    return ld_tr(tile, pitch, kb, n0, lane);
  }
  __device__ static __forceinline__ Frag ld_nat(const float* row, int kb, int lane) {
    return ld_perm(row, kb, lane);
  }
  __device__ static __forceinline__ Frag ld_perm_f32(const float* row, int kb, int lane) {
    return row[kb + (lane >> 4)];
  }
  __device__ static __forceinline__ float elem(Frag f, int) { return f; }
  __device__ static __forceinline__ Frag from_f32(const float* p) { return *p; }
  __device__ static __forceinline__ Frag from_vals(const float* v) { return v[0]; }
  __device__ static __forceinline__ float dot(Frag a, Frag b) { return a * b; }
  __device__ static __forceinline__ f4 mma3(const float* a, const float* b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
  }
};

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// 16-wide contractions (one 16-row block).  Lane group g = lane >> 4 supplies the
// four contraction indices kidx(g, j), j = 0..3, of its row (A) or column (B):
// bf16 uses one v_mfma_f32_16x16x16_bf16 (k = 4g + j), fp32 four
// v_mfma_f32_16x16x4_f32 (step j contracts k = 4j + g).  mma_sb keeps A in the
// act dtype and carries B at fp32 accuracy (bf16: B = hi + lo, two products).
template <typename T> struct M16;
template <> struct M16<bf16> {
  typedef short s4 __attribute__((ext_vector_type(4)));
  // an operand carried as hi + lo bf16 (fp32 accuracy)
  struct Op {
    bf16x4 h, l;
  };
  __device__ static __forceinline__ Op split(const float* v) {
    Op o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o.h[j] = (bf16)v[j];
      o.l[j] = (bf16)(v[j] - (float)o.h[j]);
    }
    return o;
  }
  // an operand that is exactly bf16 (lo part zero), read straight from a row
  __device__ static __forceinline__ Op ld_op(const bf16* row, int g) {
    Op o;
    o.h = *(const bf16x4*)(row + 4 * g);
    o.l = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    return o;
  }
  __device__ static __forceinline__ Op keep_if(bool c, Op o) {
    const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    Op r;
    r.h = c ? o.h : z;
    r.l = c ? o.l : z;
    return r;
  }
  __device__ static __forceinline__ f4 mm(bf16x4 a, bf16x4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a),
                                                      __builtin_bit_cast(s4, b), c, 0, 0, 0);
  }
  // A at act precision (hi only), B at fp32 accuracy
  __device__ static __forceinline__ f4 op_sb(const Op& a, const Op& b, f4 c) {
    return mm(a.h, b.h, mm(a.h, b.l, c));
  }
  // both at fp32 accuracy
  __device__ static __forceinline__ f4 op_ss(const Op& a, const Op& b, f4 c) {
    return mm(a.h, b.h, mm(a.h, b.l, mm(a.l, b.h, c)));
  }
  __device__ static __forceinline__ int kidx(int g, int j) { return 4 * g + j; }
  // operand of a row-major [k][n] LDS tile, contraction over its rows kb .. kb + 15
  __device__ static __forceinline__ void ld_tr(const bf16* tile, int pitch, int kb, int n0,
                                               int lane, float* out) {
    const bf16x4 v = ld_tr4(tile, pitch, kb + 4 * (lane >> 4), n0, lane);
    out[0] = (float)v[0]; out[1] = (float)v[1]; out[2] = (float)v[2]; out[3] = (float)v[3];
  }
  __device__ static __forceinline__ Op ld_tr_op(const bf16* tile, int pitch, int kb, int n0,
                                                int lane) {
    Op o;
    o.h = ld_tr4(tile, pitch, kb + 4 * (lane >> 4), n0, lane);
    o.l = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    return o;
  }
  __device__ static __forceinline__ void ld(const bf16* row, int g, float* out) {
    const bf16x4 v = *(const bf16x4*)(row + 4 * g);
    out[0] = (float)v[0]; out[1] = (float)v[1]; out[2] = (float)v[2]; out[3] = (float)v[3];
  }
  __device__ static __forceinline__ void ldf(const float* row, int g, float* out) {
    const f4 v = *(const f4*)(row + 4 * g);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
  __device__ static __forceinline__ f4 mma_sb(const float* a, const float* b, f4 c) {
    bf16x4 ah, bh, bl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ah[j] = (bf16)a[j];
      bh[j] = (bf16)b[j];
      bl[j] = (bf16)(b[j] - (float)bh[j]);
    }
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, ah),
                                                   __builtin_bit_cast(s4, bl), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, ah),
                                                      __builtin_bit_cast(s4, bh), c, 0, 0, 0);
  }
  // both operands at fp32 accuracy: ah.bh + ah.bl + al.bh
  __device__ static __forceinline__ f4 mma_ss(const float* a, const float* b, f4 c) {
    bf16x4 ah, al, bh, bl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ah[j] = (bf16)a[j];
      al[j] = (bf16)(a[j] - (float)ah[j]);
      bh[j] = (bf16)b[j];
      bl[j] = (bf16)(b[j] - (float)bh[j]);
    }
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, al),
                                                   __builtin_bit_cast(s4, bh), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, ah),
                                                   __builtin_bit_cast(s4, bl), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, ah),
                                                      __builtin_bit_cast(s4, bh), c, 0, 0, 0);
  }
};
template <> struct M16<float> {
  struct Op {
    float v[4];
  };
  __device__ static __forceinline__ Op split(const float* v) {
    Op o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o.v[j] = v[j];
    return o;
  }
  __device__ static __forceinline__ Op ld_op(const float* row, int g) {
    Op o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o.v[j] = row[4 * j + g];
    return o;
  }
  __device__ static __forceinline__ Op keep_if(bool c, Op o) {
    Op r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.v[j] = c ? o.v[j] : 0.f;
    return r;
  }
  __device__ static __forceinline__ f4 op_sb(const Op& a, const Op& b, f4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ f4 op_ss(const Op& a, const Op& b, f4 c) {
    return op_sb(a, b, c);
  }
  __device__ static __forceinline__ int kidx(int g, int j) { return 4 * j + g; }
  __device__ static __forceinline__ void ld_tr(const float* tile, int pitch, int kb, int n0,
                                               int lane, float* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = tile[(kb + 4 * j + (lane >> 4)) * pitch + n0 + (lane & 15)];
  }
  __device__ static __forceinline__ Op ld_tr_op(const float* tile, int pitch, int kb, int n0,
                                                int lane) {
    Op o;
    ld_tr(tile, pitch, kb, n0, lane, o.v);
    return o;
  }
  __device__ static __forceinline__ void ld(const float* row, int g, float* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = row[4 * j + g];
  }
  __device__ static __forceinline__ void ldf(const float* row, int g, float* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = row[4 * j + g];
  }
  __device__ static __forceinline__ f4 mma_sb(const float* a, const float* b, f4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ f4 mma_ss(const float* a, const float* b, f4 c) {
    return mma_sb(a, b, c);
  }
};

// Load KPL consecutive elements of type T as floats.
template <typename T, int N> __device__ __forceinline__ void load_f(const T* p, float* out) {
#pragma unroll
  for (int j = 0; j < N; ++j) out[j] = to_f(p[j]);
}

// Store a C tile (acc layout) into a row-major [m][n] array at (row0, col0).
template <typename T>
__device__ __forceinline__ void store_c(T* base, int pitch, int row0, int col0, f4 acc, int lane) {
  int col = col0 + (lane & 15), r = row0 + (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) base[(r + j) * pitch + col] = from_f<T>(acc[j]);
}
// Store the transpose of a C tile: element (m, n) goes to base[n * pitch + m].
// The 4 rows a lane holds become 4 contiguous elements.
template <typename T>
__device__ __forceinline__ void store_ct(T* base, int pitch, int row0, int col0, f4 acc, int lane);
template <>
__device__ __forceinline__ void store_ct<bf16>(bf16* base, int pitch, int row0, int col0, f4 acc,
                                               int lane) {
  int col = col0 + (lane & 15), r = row0 + (lane >> 4) * 4;
  bf16x4 v;
  v[0] = (bf16)acc[0]; v[1] = (bf16)acc[1]; v[2] = (bf16)acc[2]; v[3] = (bf16)acc[3];
  *(bf16x4*)(base + col * pitch + r) = v;
}
template <>
__device__ __forceinline__ void store_ct<float>(float* base, int pitch, int row0, int col0, f4 acc,
                                                int lane) {
  int col = col0 + (lane & 15), r = row0 + (lane >> 4) * 4;
  *(f4*)(base + col * pitch + r) = acc;
}

// Direct global -> LDS copy of a [ROWS][D] tile of T (global row stride `rs`
// elements) into an LDS tile of pitch D + PAD * 16 / sizeof(T) elements, i.e. PAD
// 16-byte pad granules per row.  global_load_lds moves 16 bytes per lane and lands
// lane l at the wave-uniform LDS base + 16 l, so each wave fills 64-granule slices of
// the padded tile (wave w: slices w, w + NW, ...) without passing through registers.
// Pad granules receive a copy of the row's last granule (never read); rows at or
// beyond `valid` are zero-filled with ordinary LDS stores instead.  The caller
// waits for vmcnt(0) and synchronises before the tile is read.
typedef __attribute__((address_space(3))) void lds_void;
// Byte offset of row r for a row stride of rsb bytes, on the full-rate 24-bit multiplier
// (a 32- or 64-bit product is a quarter-rate instruction).  The host keeps every row
// stride below 2^24 bytes, and rows inside a chunk or a state tile are below 2^7, so
// the product fits 31 bits.
// (The operands are masked to 24 bits so that the compiler can see the range; a call of
// the mul24 library function with an operand of unknown range becomes a full multiply.)
__device__ __forceinline__ unsigned row_off(unsigned r, unsigned rsb) {
  return (r & 0xffffffu) * (rsb & 0xffffffu);
}
// `base` (wave-uniform) plus a per-lane byte offset: the access can take the scalar-base
// plus 32-bit vector-offset address form instead of a 64-bit add per lane.
template <typename X> __device__ __forceinline__ X* at(X* base, unsigned off) {
  return (X*)((char*)base + off);
}
template <typename X> __device__ __forceinline__ const X* at(const X* base, unsigned off) {
  return (const X*)((const char*)base + off);
}
// floor(p / d) for 0 <= p < n as (p * m) >> 16 on the 24-bit multiplier (a division by
// a constant otherwise becomes a quarter-rate high multiply); n and d are checked at
// compile time.
constexpr unsigned div24_m(int d) { return (65536u + (unsigned)d - 1) / (unsigned)d; }
constexpr bool div24_exact(int d, int n) {
  for (int p = 0; p < n; ++p)
    if ((int)(((unsigned)p * div24_m(d)) >> 16) != p / d) return false;
  return (unsigned)n * div24_m(d) < (1u << 24);
}
template <int d, int n> __device__ __forceinline__ unsigned div24(unsigned p) {
  static_assert(div24_exact(d, n), "24-bit division exact over the range");
  return ((p & 0xffffffu) * div24_m(d)) >> 16;
}
// One 16-byte global -> LDS copy per active lane: lane l reads 16 bytes at g + off
// (g wave-uniform, in scalar registers; off this lane's byte offset) and writes LDS
// bytes [lds + 16 l, lds + 16 l + 16) (lds: a wave-uniform LDS byte address, via M0).
// Issued as inline asm so that the compiler does not hold every later LDS access
// of the wave until the copy lands: a reader of the destination calls wait_vmem()
// and then a workgroup barrier. The kernels that use it set M0 nowhere else.
__device__ __forceinline__ void g2l16(const void* g, unsigned off, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off),
               "s"(g), "s"(lds)
               : "memory");
}
//   lds0: LDS byte address of the tile (wave-uniform), lds_tile: the same tile seen
//   through a generic pointer (for the zero fill); src: the tile's first row (uniform),
//   rs: its row stride in elements.
//   [N0, N1): the part of the wave's slices to issue (a tile may be issued in parts).
template <typename T, int D, int ROWS, int NW, int N0 = 0, int N1 = 1 << 20, int PAD = 1>
__device__ __forceinline__ void g2l_tile(unsigned lds0, T* lds_tile, const T* src, unsigned rs,
                                         int valid, int w, int lane) {
  constexpr int GPR = D * (int)sizeof(T) / 16;  // data granules per row
  constexpr int GP = GPR + PAD;                 // granules per padded LDS row
  constexpr int NG = ROWS * GP;
  constexpr int NSL = (NG + 63) / 64;           // slices
  constexpr int NPW = (NSL + NW - 1) / NW;      // slices per wave (at most)
  const unsigned rsb = rs * (unsigned)sizeof(T);
#pragma unroll
  for (int n = N0; n < (N1 < NPW ? N1 : NPW); ++n) {
    const int base = (w + n * NW) * 64;
    if (base < NG) {
      const unsigned p = (unsigned)(base + lane);
      const unsigned row = div24<GP, NSL * 64>(p), gc = p - row * GP;
      if (p < (unsigned)NG) {
        if ((int)row < valid) {
          g2l16(src, row_off(row, rsb) + (gc < GPR ? gc : GPR - 1) * 16, lds0 + base * 16);
        } else {
          unsigned z;  // made here: a zero quad kept across the caller's loop gets spilled
          asm volatile("v_mov_b32 %0, 0" : "=v"(z));
          *(u32x4*)((char*)lds_tile + p * 16) = u32x4{z, z, z, z};
        }
      }
    }
  }
}
// Wait until this wave's global loads (including global -> LDS copies) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Registers filled by loads issued well before their use (a prefetch for the next
// work item): passing them through an empty asm makes the compiler wait for those
// loads here, at a point chosen where they have landed and no stores are queued
// behind them, instead of at the first use, where its wait would also cover every
// store issued in between.
__device__ __forceinline__ void settle(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle(u32x4& x) { asm volatile("" : "+v"(x)); }
template <int N> __device__ __forceinline__ void settle(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) settle(x[i]);
}
__device__ __forceinline__ void settle(f4& x) { asm volatile("" : "+v"(x)); }
template <int N> __device__ __forceinline__ void settle(f4 (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) settle(x[i]);
}
template <int N> __device__ __forceinline__ void settle(u32x4 (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) settle(x[i]);
}

// DPP lane move inside a row of 16 lanes.
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                                            0xF, true));
}
// Sum over the 16 lanes that share (lane >> 4) (i.e. over the columns of a C tile),
// on DPP: swap neighbours, swap pairs, mirror halves of 8, mirror the row.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}
// sum16 of N values at once, one DPP stage over all of them before the next: the
// independent adds between dependent ones stand in for the wait states a DPP read of a
// just-written register needs.
template <int N> __device__ __forceinline__ void sum16_n(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f<0xB1>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f<0x4E>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f<0x141>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f<0x140>(x[i]);
}
// Lane swaps across the 16-lane rows of a wave (VALU, no LDS):
//   swap32(a, b): lanes 32-63 of a <-> lanes 0-31 of b;
//   swap16(a, b): lanes 16-31 of a <-> lanes 0-15 of b, lanes 48-63 of a <-> 32-47 of b.
// Inline asm with both registers read and written: this compiler returns the first
// register for both results of the swap builtins.  A swap that reads a register written
// by a VALU instruction needs two wait states in between; the compiler cannot see into
// the asm, so each swap brings its own (s_nop 1).
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// rows_gather: r[k] = x of lane 16 k + (lane & 15), in every lane.
__device__ __forceinline__ void rows_gather(float x, float (&r)[4]) {
  float a = x, b = x;
  swap32(a, b);  // a: rows 0 1 0 1, b: rows 2 3 2 3
  float c = a, d = b;
  swap16(a, c);  // a: row 0, c: row 1
  swap16(b, d);  // b: row 2, d: row 3
  r[0] = a;
  r[1] = c;
  r[2] = b;
  r[3] = d;
}
// x summed over the four rows (the lanes l, l ^ 16, l ^ 32, l ^ 48), in every lane.
__device__ __forceinline__ float sum_rows(float x) {
  float a = x, b = x;
  swap32(a, b);
  float c = a + b, d = c;  // rows 0+2, 1+3, 0+2, 1+3
  swap16(c, d);
  return c + d;
}
// Sum over the whole wave.
__device__ __forceinline__ float sum64(float x) { return sum_rows(sum16(x)); }

// L2 normalisation of q and k per (token, head) (the Kernel-B guide, R1 computes the
// reciprocal norm of every row once and its K1, the norm's backward, reuses it):
//   xn = x r,  r = 1 / sqrt(sum_i x_i^2 + eps),   dx = r (dxn - xn (xn . dxn)).
// A row of D elements is held by LPR consecutive lanes (one 16-byte piece each) that
// form one DPP row (LPR = 16) or half row (LPR = 8).  Every kernel that normalises uses
// these helpers, so the normalised values are bit-identical wherever they are formed.
constexpr float kL2Eps = 1e-6f;
template <int LPR> __device__ __forceinline__ float sum_group(float x) {
  if constexpr (LPR == 16) return sum16(x);
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror: the 8 lanes of each half row
  return x;
}
// Normalises the lane's piece of a row in place; returns the row's reciprocal norm.
template <typename T, int LPR> __device__ __forceinline__ float l2n_piece(u32x4& piece) {
  constexpr int EPV = 16 / (int)sizeof(T);
  const T* e = (const T*)&piece;
  float v[EPV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPV; ++j) {
    v[j] = to_f(e[j]);
    ss += v[j] * v[j];
  }
  ss = sum_group<LPR>(ss);
  const float rr = __builtin_amdgcn_rsqf(ss + kL2Eps);  // argument >= eps: no scaling needed
  T out[EPV];
#pragma unroll
  for (int j = 0; j < EPV; ++j) out[j] = from_f<T>(v[j] * rr);
  piece = *(const u32x4*)out;
  return rr;
}
// xn = x rr for a raw piece whose row's reciprocal norm is already known (the same
// rounding as l2n_piece).
template <typename T> __device__ __forceinline__ u32x4 l2n_apply(u32x4 piece, float rr) {
  constexpr int EPV = 16 / (int)sizeof(T);
  const T* e = (const T*)&piece;
  T out[EPV];
#pragma unroll
  for (int j = 0; j < EPV; ++j) out[j] = from_f<T>(to_f(e[j]) * rr);
  return *(const u32x4*)out;
}
// The lane's share of xn . dxn.
template <typename T> __device__ __forceinline__ float dot_piece(u32x4 xn, u32x4 dxn) {
  constexpr int EPV = 16 / (int)sizeof(T);
  const T* a = (const T*)&xn;
  const T* g = (const T*)&dxn;
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < EPV; ++j) d += to_f(a[j]) * to_f(g[j]);
  return d;
}
// dx = rr (dxn - xn dot) for one piece.
template <typename T>
__device__ __forceinline__ u32x4 l2n_project(u32x4 xn, u32x4 dxn, float rr, float dot) {
  constexpr int EPV = 16 / (int)sizeof(T);
  const T* a = (const T*)&xn;
  const T* g = (const T*)&dxn;
  T out[EPV];
#pragma unroll
  for (int j = 0; j < EPV; ++j) out[j] = from_f<T>(rr * (to_f(g[j]) - to_f(a[j]) * dot));
  return *(const u32x4*)out;
}

// Pitches (in elements) of the LDS tiles.  Natural token-major tiles [64][D] of T
// get 16 bytes of row padding so that the 16 rows one MFMA operand reads start
// in distinct 4-bank groups of the 64-bank LDS; transposed tiles [D][64] likewise.
template <typename T, int D> struct Pitch {
  static constexpr int N = D + 16 / (int)sizeof(T);  // [64][D] of T
  static constexpr int NF = D + 4;                    // [64][D] of fp32
  static constexpr int CC = 68;                       // [64][64] of fp32
  static constexpr int TT = sizeof(T) == 2 ? 72 : 68; // [D][64] of T
  static constexpr int CT = sizeof(T) == 2 ? 72 : 68; // [64][64] of T
};

}  // namespace kda
