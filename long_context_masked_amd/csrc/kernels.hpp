// Device-side building blocks shared by the forward and backward kernels.
//
// Matrix products use the gfx950 bf16 MFMA v_mfma_f32_32x32x16_bf16 (fp32
// accumulate).  Operand/result lane layouts (wave64, lane l, h = l / 32):
//   A (32 x 16): lane l holds A[l % 32][8h .. 8h+7]
//   B (16 x 32): lane l holds B[8h .. 8h+7][l % 32]
//   C (32 x 32): lane l, register r holds C[8(r/4) + 4h + (r%4)][l % 32]
// Every kernel computes transposed products (C = rows of the *other*
// operand x columns of "its" rows) so that one lane owns one query row (or,
// in the dK/dV pass, one key) and the softmax statistics of that row stay in
// the lane.  A C result can then feed the next product directly as a B
// operand after an fp32 -> bf16 conversion, provided the partner A operand
// lists its k index in the order C hands it over: for the 16-wide k-step t
// of a 64-row tile the lane half h holds rows 16t + 4h + {0..3} and
// 16t + 8 + 4h + {0..3}.  Transposed tiles in LDS are stored in that order
// (perm16 below) so that the partner operand is one contiguous 16-byte read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcm {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// The running maximum is kept stale until the true maximum exceeds it by
// more than kRescaleSlack (log2 units); exp2 arguments are then bounded by
// kRescaleSlack, so unnormalised probabilities stay below 2^8 and the final
// O / l is unchanged (all terms of a row share the same stale maximum).
constexpr float kRescaleSlack = 8.0f;
constexpr float kMinit = -1.0e30f;  // finite start value of the running max

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                        float a5, float a6, float a7) {
  bf16x2 p0 = __builtin_convertvector((f32x2){a0, a1}, bf16x2);
  bf16x2 p1 = __builtin_convertvector((f32x2){a2, a3}, bf16x2);
  bf16x2 p2 = __builtin_convertvector((f32x2){a4, a5}, bf16x2);
  bf16x2 p3 = __builtin_convertvector((f32x2){a6, a7}, bf16x2);
  bf16x4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  bf16x4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The B operand for k-step t of a 64-row tile held as two C blocks c[0..1].
__device__ __forceinline__ bf16x8 c_to_b(const f32x16 *c, int t) {
  const f32x16 &x = c[t >> 1];
  const int o = (t & 1) * 8;
  return pack8(x[o + 0], x[o + 1], x[o + 2], x[o + 3], x[o + 4], x[o + 5], x[o + 6], x[o + 7]);
}

// Position of row k (0..63) of a tile inside a transposed LDS tile: within
// each 16-row group the two middle 4-row groups are swapped.
__device__ __forceinline__ int perm16(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Bits [lo, hi) of a 64-bit word, clipped to [0, 64).
__device__ __forceinline__ uint64_t range64(int lo, int hi) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > 64 ? 64 : hi;
  if (hi <= lo) return 0ull;
  const uint64_t top = hi == 64 ? ~0ull : ((1ull << hi) - 1ull);
  return top & ~((1ull << lo) - 1ull);
}

// Keep s where bit `bit` of `m` is set, else -inf / 0.
__device__ __forceinline__ float keep_or(uint32_t m, int bit, float s, float other) {
  return ((m >> bit) & 1u) ? s : other;
}

// --------------------------------------------------------------------------
// 64-row tile staging.  256 threads; thread t owns 16-byte chunk c = t % CPR
// (elements 8c..8c+7 of d) of RPT consecutive rows starting at RPT*(t/CPR).
// From these registers a tile can be written to LDS in natural [row][d]
// layout (pitch D+8) and/or transposed [d][perm16(row)] layout (pitch 72).
// --------------------------------------------------------------------------
template <int D>
struct Tile64 {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPT = 64 * CPR / 256; // rows per thread (4 or 2)
  static constexpr int NP = D + 8;           // natural pitch (elements)
  static constexpr int TP = 64 + 8;          // transposed pitch (elements)
  uint4 r[RPT];

  // rows row0 + [0, 64) of a [.., ld] bf16 matrix; rows >= nrows read as 0
  __device__ __forceinline__ void load(const bf16 *base, int64_t ld, int row0, int nrows) {
    const int t = threadIdx.x;
    const int c = t % CPR, g = t / CPR;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = row0 + g * RPT + i;
      if (row < nrows)
        r[i] = *reinterpret_cast<const uint4 *>(base + (int64_t)row * ld + c * 8);
      else
        r[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  __device__ __forceinline__ void store_nat(bf16 *s) const {
    const int t = threadIdx.x;
    const int c = t % CPR, g = t / CPR;
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<uint4 *>(s + (g * RPT + i) * NP + c * 8) = r[i];
  }

  __device__ __forceinline__ void store_trans(bf16 *s) const {
    const int t = threadIdx.x;
    const int c = t % CPR, g = t / CPR;
    const int pos = perm16(g * RPT);  // RPT rows stay contiguous under perm16
    const uint32_t *w[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) w[i] = reinterpret_cast<const uint32_t *>(&r[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      uint32_t lo16[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) lo16[i] = (w[i][e >> 1] >> sh) & 0xffffu;
      bf16 *dst = s + (c * 8 + e) * TP + pos;
      if constexpr (RPT == 4) {
        uint2 v;
        v.x = lo16[0] | (lo16[1] << 16);
        v.y = lo16[2] | (lo16[3] << 16);
        *reinterpret_cast<uint2 *>(dst) = v;
      } else {
        *reinterpret_cast<uint32_t *>(dst) = lo16[0] | (lo16[1] << 16);
      }
    }
  }
};

// --------------------------------------------------------------------------
// Kernel arguments (device pointers into caller buffers and the plan blob).
// --------------------------------------------------------------------------
struct MaskArgs {
  const int4 *rowb;        // [S] allowed key runs {a0, b0, a1, b1} per row
  const int4 *colb;        // [S] masked row runs {lts, lte, uts, ute} per key
  const uint8_t *bits;     // [bm_heads][nqb][nkb] or null
  const int *qblk, *kblk;  // block of each position
  const int *qoffs, *koffs;
  int nqb, nkb, bm_heads;  // bm_heads 0 = no bitmap
};

struct FwdArgs {
  const bf16 *q, *k, *v;
  bf16 *o;
  float *lse;
  int S, Hq, Hkv, G;
  float sl2;  // softmax scale * log2(e)
  const int4 *items;
  const uint32_t *list;
  MaskArgs m;
};

struct BwdArgs {
  const bf16 *q, *k, *v, *o, *dout;
  const float *lse;
  float *dws;  // D = rowsum(dO * O), [B, Hq, S]
  bf16 *dq, *dk, *dv;
  int S, Hq, Hkv, G;
  float scale, sl2;
  const int4 *fitems;  // Q-split items (dQ pass)
  const uint32_t *flist;
  const int4 *bitems;  // KV-split items (dK/dV pass)
  const uint32_t *blist;
  int n_fitems, n_bitems;
  MaskArgs m;
};

// Allowed-key bits of query row `row` over keys [t0, t0 + 64).
__device__ __forceinline__ uint64_t row_mask(const MaskArgs &m, int4 rb, int qb, int hm,
                                             int t0, int S) {
  uint64_t bits = range64(rb.x - t0, rb.y - t0) | range64(rb.z - t0, rb.w - t0);
  if (m.bm_heads) {
    const int last = (t0 + 63 < S ? t0 + 63 : S - 1);
    const int kb0 = m.kblk[t0], kb1 = m.kblk[last];
    const uint8_t *brow = m.bits + ((int64_t)hm * m.nqb + qb) * m.nkb;
    uint64_t keep = 0;
    for (int kb = kb0; kb <= kb1; ++kb)
      if (brow[kb]) keep |= range64(m.koffs[kb] - t0, m.koffs[kb + 1] - t0);
    bits &= keep;
  }
  return bits;
}

// Allowed-row bits of key `key` over query rows [r0, r0 + 64); rows >= S off.
__device__ __forceinline__ uint64_t col_mask(const MaskArgs &m, int4 cb, int kb, int hm,
                                             int r0, int S) {
  uint64_t bits = ~(range64(cb.x - r0, cb.y - r0) | range64(cb.z - r0, cb.w - r0));
  bits &= range64(0, S - r0);
  if (m.bm_heads) {
    const int last = (r0 + 63 < S ? r0 + 63 : S - 1);
    const int qb0 = m.qblk[r0], qb1 = m.qblk[last];
    const uint8_t *bcol = m.bits + (int64_t)hm * m.nqb * m.nkb + kb;
    uint64_t keep = 0;
    for (int qb = qb0; qb <= qb1; ++qb)
      if (bcol[(int64_t)qb * m.nkb]) keep |= range64(m.qoffs[qb] - r0, m.qoffs[qb + 1] - r0);
    bits &= keep;
  }
  return bits;
}

// Bitmap head of query head h (bm_heads in {1, Hkv, Hq}).
__device__ __forceinline__ int bitmap_head(int bm_heads, int h, int Hq, int G) {
  if (bm_heads <= 1) return 0;
  return bm_heads == Hq ? h : h / G;
}

}  // namespace lcm
