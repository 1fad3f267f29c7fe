// Device-side building blocks shared by the forward and backward kernels.
//
// Matrix products use the gfx950 bf16 MFMA v_mfma_f32_32x32x16_bf16 (fp32
// accumulate).  Operand/result lane layouts (wave64, lane l, h = l / 32):
//   A (32 x 16): lane l holds A[l % 32][8h .. 8h+7]
//   B (16 x 32): lane l holds B[8h .. 8h+7][l % 32]
//   C (32 x 32): lane l, register r holds C[8(r/4) + 4h + (r%4)][l % 32]
// Every kernel computes transposed products so that one lane owns one query
// row (forward, dQ) or one key (dK/dV) and the per-row softmax statistics
// stay in the lane.  A C result then feeds the next product directly as a B
// operand after an fp32 -> bf16 conversion, provided the partner A operand
// lists its k index in the order C hands it over: for the 16-wide k-step t
// of a 64-row tile, lane half h holds rows 16t + 4h + {0..3} and
// 16t + 8 + 4h + {0..3}.  That partner operand is always a tile stored in
// natural [row][d] layout in LDS and read transposed with
// ds_read_b64_tr_b16: within each group of 16 lanes, lane l receives element
// j from the address given by lane 4j + l/4, at 16-bit offset l % 4.  Giving
// source lane 4j + q the address of row (base + j), column (16-block + 4q)
// hands lane l the four rows base..base+3 at column (16-block + l).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcm {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

__device__ __forceinline__ bf16x2 cvt2(float a, float b) {
  return __builtin_convertvector((f32x2){a, b}, bf16x2);
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                        float a5, float a6, float a7) {
  const bf16x4 lo = __builtin_shufflevector(cvt2(a0, a1), cvt2(a2, a3), 0, 1, 2, 3);
  const bf16x4 hi = __builtin_shufflevector(cvt2(a4, a5), cvt2(a6, a7), 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The B operand of k-step t (t = 0, 1) held in one C block (registers 8t..8t+7).
__device__ __forceinline__ bf16x8 c_to_b(const f32x16 &x, int t) {
  const int o = t * 8;
  return pack8(x[o + 0], x[o + 1], x[o + 2], x[o + 3], x[o + 4], x[o + 5], x[o + 6], x[o + 7]);
}

// Sum of the eight bf16 values of a B operand, accumulated into acc.
__device__ __forceinline__ float sum8(bf16x8 v, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}

// max over both lane halves (lanes l and l ^ 32 hold the same row / key).
__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Bits [lo, hi) of a 64-bit word, clipped to [0, 64).
__device__ __forceinline__ uint64_t range64(int lo, int hi) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > 64 ? 64 : hi;
  if (hi <= lo) return 0ull;
  const uint64_t top = hi == 64 ? ~0ull : ((1ull << hi) - 1ull);
  return top & ~((1ull << lo) - 1ull);
}

// x where bit `bit` of m is set, else `other` (two VALU ops: a sign-extended
// one-bit field extract and a bitfield insert).
__device__ __forceinline__ float keep_or(uint32_t m, int bit, float x, float other) {
  const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)m, bit, 1);
  return __uint_as_float((sel & __float_as_uint(x)) | (~sel & __float_as_uint(other)));
}

// --------------------------------------------------------------------------
// LDS tiles of 64 rows x D bf16 in natural [row][d] layout.
//   SWZ = false: row pitch 2D+16 bytes, conflict-free 16-byte row reads.
//   SWZ = true:  row pitch 2D+64 bytes with 16-byte chunks XOR-swizzled by
//                the row; conflict-free for row reads, transposed reads and
//                the staging writes alike.
// --------------------------------------------------------------------------
template <int D, bool SWZ>
struct Lds {
  static constexpr int PITCH = SWZ ? 2 * D + 64 : 2 * D + 16;
  static constexpr int BYTES = 64 * PITCH;
  static constexpr int NCH = (2 * D / 16) < 16 ? (2 * D / 16) : 16;
  __device__ static __forceinline__ int off(int row, int cb) {
    return row * PITCH + (SWZ ? (cb ^ ((row & (NCH - 1)) << 4)) : cb);
  }
};

// A operand from a natural tile: rows row..row+31 by lane, 16 elements of d
// starting at byte cb (lane half h adds 16 bytes).
template <class L>
__device__ __forceinline__ bf16x8 lds_rows(const char *base, int row, int cb) {
  return *reinterpret_cast<const bf16x8 *>(base + L::off(row, cb));
}

// Per-lane byte offsets of the transposed reads of one d-block db (two
// halves: rows +0 and +8 of a 16-row k-step); add 16 * t * PITCH for k-step t.
template <class L>
__device__ __forceinline__ int tr_off(int lane, int db, int half) {
  const int row = 8 * half + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int cb = db * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  return L::off(row, cb);
}

// A operand (m = d within a 32-block, k = 16 tile rows of k-step t in C order)
// from a natural tile, via two transposed reads at precomputed offsets.
__device__ __forceinline__ bf16x8 lds_tr(const char *base, int off0, int off1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)((__attribute__((address_space(3))) char *)base + off0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)((__attribute__((address_space(3))) char *)base + off1));
  const s16x4 lo = a, hi = b;
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 64-row tile staging through registers.  256 threads; thread t owns 16-byte
// chunk c = t % CPR of RPT consecutive rows starting at RPT * (t / CPR):
// global loads are coalesced along d, LDS writes are whole rows.
template <int D>
struct Stage64 {
  static constexpr int CPR = D / 8;
  static constexpr int RPT = 64 * CPR / 256;
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

  template <class L>
  __device__ __forceinline__ void store(char *s) const {
    const int t = threadIdx.x;
    const int c = t % CPR, g = t / CPR;
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<uint4 *>(s + L::off(g * RPT + i, c * 16)) = r[i];
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
