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
constexpr float kEmptyRowLse2 = 1.0e30f;  // lse2 of a row with no allowed key
// dK/dV list entry: Q-tile index in bits 0-23, the query head in bits 24-30
// when the plan lists (Q-tile, head) stages, the partial flag in bit 31.
constexpr uint32_t kTileBits = 0x00ffffffu;
constexpr int kDkdvKeys = 128;      // keys per dK/dV workgroup (4 waves x 32)

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
// LDS tiles of 64 rows x D bf16 in natural [row][d] layout, rows unpadded
// (2D bytes) and 16-byte chunks XOR-swizzled by the row, so that 16-byte row
// reads (MFMA A operands), transposed reads and whole-row writes are all free
// of bank conflicts (d = 128; d = 64 keeps a two-way conflict on one kind).
// Tiles are filled by direct global -> LDS loads: one wave instruction writes
// 1 KiB of consecutive LDS bytes, lane L at byte 16 L, and each lane fetches
// the global chunk that the swizzle places at its LDS position.
// --------------------------------------------------------------------------
template <int D>
struct Tile {
  static constexpr int ROWB = 2 * D;            // bytes per row
  static constexpr int BYTES = 64 * ROWB;
  static constexpr int RPK = 1024 / ROWB;       // rows per 1 KiB load instruction
  static constexpr int LPR = 64 / RPK;          // lanes per row in one instruction
  template <int NW>
  static constexpr int NI = BYTES / 1024 / NW;  // load instructions per wave (NW waves)
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return ((r & 3) << 1) | ((r >> 2) & 1);
  }
  __device__ static __forceinline__ int off(int row, int cb) {
    return row * ROWB + (cb ^ (swz(row) << 4));
  }
};

// Issue the loads of rows row0 + [0, 64) of a [.., ld] bf16 matrix into the
// LDS tile at `dst`, shared by the NW waves of the workgroup.  Rows >= nrows
// repeat row nrows - 1 (finite values; the kernels mask them).  Completion:
// s_waitcnt vmcnt(0) then a barrier.
template <int D, int NW = 4>
__device__ __forceinline__ void dma_tile(char *dst, const bf16 *base, int64_t ld, int row0,
                                         int nrows) {
  using T = Tile<D>;
  constexpr int NI = T::template NI<NW>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = wave * NI + i;
    const int row = blk * T::RPK + lane / T::LPR;
    const int c = (lane % T::LPR) ^ T::swz(row);
    int grow = row0 + row;
    grow = grow < nrows ? grow : nrows - 1;
    __builtin_amdgcn_global_load_lds(base + (int64_t)grow * ld + c * 8,
                                     (__attribute__((address_space(3))) void *)(
                                         (__attribute__((address_space(3))) char *)dst + blk * 1024),
                                     16, 0, 0);
  }
}

// dma_tile with the per-lane addressing hoisted out of the loop: `off` holds
// the byte offset, from the tile's first row, of the global chunk that each
// of the lane's NI load instructions fetches, and the wave index is made
// uniform so that each load takes a scalar base plus a 32-bit lane offset.
// Tiles that extend past nrows (the ragged last tile) use dma_tile instead.
template <int D, int NW = 4>
struct TileDma {
  static constexpr int NI = Tile<D>::template NI<NW>;
  uint32_t off[NI];
  int lds0;  // byte offset of this wave's first 1 KiB block in the tile

  __device__ __forceinline__ void init(int64_t ld) {
    using T = Tile<D>;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (wave * NI + i) * T::RPK + lane / T::LPR;
      const int c = (lane % T::LPR) ^ T::swz(row);
      off[i] = (uint32_t)(row * ld * 2 + c * 16);
    }
    lds0 = wave * NI * 1024;
  }

  __device__ __forceinline__ void load(char *dst, const bf16 *base, int64_t ld, int row0,
                                       int nrows) const {
    using T = Tile<D>;
    if (row0 + 64 <= nrows) {
      const char *g = reinterpret_cast<const char *>(base + (int64_t)row0 * ld);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        __builtin_amdgcn_global_load_lds(
            g + off[i],
            (__attribute__((address_space(3))) void *)(
                (__attribute__((address_space(3))) char *)dst + lds0 + i * 1024),
            16, 0, 0);
    } else {
      dma_tile<D, NW>(dst, base, ld, row0, nrows);
    }
  }
};

// Wait for this wave's outstanding global -> LDS loads (and other vector
// memory operations); a barrier must follow before other waves read.
__device__ __forceinline__ void dma_wait() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Byte offset, inside a tile, of this lane's 16-byte row read for k-step ks
// (rows 32 rb + l % 32 add rb * 32 * ROWB, which leaves the swizzle alone).
template <int D>
__device__ __forceinline__ int row_off(int lane, int ks) {
  return Tile<D>::off(lane & 31, ks * 32 + (lane >> 5) * 16);
}

__device__ __forceinline__ bf16x8 lds_rows(const char *base, int off) {
  return *reinterpret_cast<const bf16x8 *>(base + off);
}

// Per-lane byte offsets of the transposed reads of one d-block db (two
// halves: rows +0 and +8 of a 16-row k-step); add 16 * t * ROWB for step t.
template <int D>
__device__ __forceinline__ int tr_off(int lane, int db, int half) {
  const int row = 8 * half + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int cb = db * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  return Tile<D>::off(row, cb);
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Transposed LDS reads are issued as inline assembly and completed by an
// explicit wait.  The compiler cannot tell which LDS bytes its own transposed
// read builtin touches, so it waits for every outstanding global -> LDS load
// before each such read, which would serialise the next tile's prefetch with
// the current tile's products.  The tiles read here were completed by
// dma_wait() and a barrier, so no wait on the prefetch is needed.
// tr_issue<OFF>(addr): one ds_read_b64_tr_b16 at LDS byte addr + OFF; the
// result is valid only after tr_wait() names it.
template <int OFF>
__device__ __forceinline__ s16x4 tr_issue(uint32_t addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Wait for all outstanding LDS reads; the listed registers are tied to the
// wait so that no use of them can be scheduled before it.
template <int N>
__device__ __forceinline__ void tr_wait(s16x4 (&x)[N]) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "tr_wait: 2, 4, 8 or 16 operands");
  if constexpr (N == 2)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]));
  else if constexpr (N == 4)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
  else if constexpr (N == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                   "+v"(x[6]), "+v"(x[7]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                   "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]),
                   "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15]));
}

// Register-class hints (no instructions): keep a value in accumulation
// registers (AGPRs, readable by MFMA as operands and accumulators) or in
// vector registers (VGPRs, where VALU instructions can use it).  They steer
// the allocator away from shuttling values between the two files.
template <class X>
__device__ __forceinline__ void in_agpr(X &x) { asm volatile("" : "+a"(x)); }
template <class X>
__device__ __forceinline__ void in_vgpr(X &x) { asm volatile("" : "+v"(x)); }

// Scheduling pattern for a block of 2*KS LDS row reads feeding 2*KS MFMAs
// (two independent accumulation chains): four reads first, then pairs of
// products each followed by the next pair of reads, so that LDS latency is
// covered by MFMA work instead of a wait before every pair.
template <int KS>
__device__ __forceinline__ void pipeline_reads_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
#pragma unroll
  for (int i = 0; i < KS - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Interleave pattern for a block that pairs NM MFMAs with VALU work of an
// independent softmax step: NDS0 DS reads first, then each MFMA followed by
// NV VALU instructions and, for the first NDS1 MFMAs, one more DS read.
// Issuing VALU between MFMAs is what lets the two run concurrently: a wave
// stalls at an MFMA while the matrix pipe is still busy with the previous one.
template <int NDS0, int NM, int NV, int NDS1>
__device__ __forceinline__ void interleave_mfma_valu() {
  __builtin_amdgcn_sched_group_barrier(0x100, NDS0, 0);  // DS read
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
    if (i < NDS1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Uniform read-only data (work lists, items) read through the constant
// address space is fetched with scalar loads, which complete on their own
// counter instead of queueing behind in-flight global -> LDS tile loads.
template <class X>
__device__ __forceinline__ const __attribute__((address_space(4))) X *as_const(const X *p) {
  return (const __attribute__((address_space(4))) X *)p;
}

// The A operand formed by two transposed reads (rows +0 and +8 of a k-step).
__device__ __forceinline__ bf16x8 tr_pair(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

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
  // or null: the bitmap part of the mask precomputed per 64-wide tile,
  // allowed keys [bm_heads][nqb][nM] and allowed rows [bm_heads][nkb][nM]
  const uint64_t *kwords, *rwords;
  int nM;
};

struct FwdArgs {
  const bf16 *q, *k, *v;
  bf16 *o;      // bf16 output, or
  float *o32;   // fp32 output (partial results that are merged later)
  float *lse;
  int S, Hq, Hkv, G;
  float sl2;  // softmax scale * log2(e)
  const int4 *items;
  const uint32_t *list;
  MaskArgs m;
};

// Backward workspace: per (b, h), S64 = S rounded up to 64 rows of
// lse * log2(e), then S64 rows of -D, D = rowsum(dO * O); pad rows hold 0.
struct BwdArgs {
  const bf16 *q, *k, *v, *o, *dout;
  const float *lse;
  float *ws;
  int S64;
  bf16 *dq, *dk, *dv;
  int S, Hq, Hkv, G;
  float scale, sl2;
  const int4 *fitems;  // Q-split items (dQ pass)
  const uint32_t *flist;
  const int4 *bitems;  // KV-split items (dK/dV pass)
  const uint32_t *blist;
  const int *bslot;     // per dK/dV item: partial slot, -1 when not split
  const int4 *breduce;  // per split item: K-tile, KV head, first slot, chunks
  float *part;          // partial dK/dV: [B][n_slots][2][128 keys][d] fp32
  float *dqacc;         // fused dQ accumulator [B][S64][Hq][d] fp32, or null
  int key_tile;         // keys per dK/dV item: 128 (four waves) or 64 (two waves)
  int head_entries;     // 1: dK/dV list entries name their query head (bits 24-30)
  int n_fitems, n_bitems, n_breduce, n_slots;
  MaskArgs m;
};

// Rebuild of a dynamic plan's work lists from a new bitmap (dyn.hip).
struct DynArgs {
  const uint8_t *src;      // new bitmap [heads][nqb][nkb], nonzero = on
  uint8_t *bits;           // the plan's copy of it, 0/1
  int64_t nbits;
  const uint8_t *base;     // base-mask micro-tile classes [nM][nM]
  const int *qblk, *kblk;  // bitmap block of each position [S]
  uint32_t *fwd_list, *bwd_list;
  int2 *slot_len;          // [n_fslots + n_bslots]: entries, partial entries
  int4 *fitems, *bitems;   // tile, head, list offset, length
  // XCD shares of each pass: share c owns item positions pos[off[c] ..
  // off[c+1]) and the items nat[off[c] ..) (natural order)
  const int *fshare, *bshare, *fpos, *bpos;
  const int4 *fnat, *bnat;
  int n_fshares, n_bshares;
  int S, nM, MR, MC, nqb, nkb, nFQ, nBK;
  int n_fslots, n_bslots, fheads, bheads;
  int copy_blocks;
  int bhe;                 // 1: dK/dV entries are (Q-tile, head) stages
  int64_t bcap;            // dK/dV list capacity per slot (nM, or nM * bheads)
  int head_major;          // 1: XCD shares hold several KV heads, sorted by head first
  int fkv;                 // query heads per KV head (forward items carry a query head)
  // bitmap words (or null): [bm_heads][nqb][nM] allowed keys, [bm_heads][nkb][nM]
  // allowed rows, rebuilt from the tiles' block segments
  uint64_t *kwords, *rwords;
  const int *kseg_off, *kseg_blk, *rseg_off, *rseg_blk;
  const uint64_t *kseg_mask, *rseg_mask;
  int bm_heads;
};

// Zeros over half hh of a D-wide row (the two lane halves split it).
template <int D, typename E>
__device__ __forceinline__ void zero_half_row(E *row, int hh) {
  constexpr int PER = 16 / sizeof(E);  // elements per 16-byte store
  E *p = row + hh * (D / 2);
#pragma unroll
  for (int i = 0; i < D / 2; i += PER) *reinterpret_cast<uint4 *>(p + i) = make_uint4(0u, 0u, 0u, 0u);
}

// Allowed-key bits of query row `row` over keys [t0, t0 + 64).
__device__ __forceinline__ uint64_t row_mask(const MaskArgs &m, int4 rb, int qb, int hm,
                                             int t0, int S) {
  uint64_t bits = range64(rb.x - t0, rb.y - t0) | range64(rb.z - t0, rb.w - t0);
  if (m.kwords) {
    bits &= m.kwords[((int64_t)hm * m.nqb + qb) * m.nM + (t0 >> 6)];
  } else if (m.bm_heads) {
    const int last = (t0 + 63 < S ? t0 + 63 : S - 1);
    const int kb0 = m.kblk[t0], kb1 = m.kblk[last];
    const uint8_t *brow = m.bits + ((int64_t)hm * m.nqb + qb) * m.nkb;
    if (kb0 == kb1) {  // the tile lies in one key block: all or nothing
      if (!brow[kb0]) bits = 0;
    } else {
      uint64_t keep = 0;
      for (int kb = kb0; kb <= kb1; ++kb)
        if (brow[kb]) keep |= range64(m.koffs[kb] - t0, m.koffs[kb + 1] - t0);
      bits &= keep;
    }
  }
  return bits;
}

// Allowed-row bits of key `key` over query rows [r0, r0 + 64); rows >= S off.
__device__ __forceinline__ uint64_t col_mask(const MaskArgs &m, int4 cb, int kb, int hm,
                                             int r0, int S) {
  uint64_t bits = ~(range64(cb.x - r0, cb.y - r0) | range64(cb.z - r0, cb.w - r0));
  bits &= range64(0, S - r0);
  if (m.rwords) {
    bits &= m.rwords[((int64_t)hm * m.nkb + kb) * m.nM + (r0 >> 6)];
  } else if (m.bm_heads) {
    const int last = (r0 + 63 < S ? r0 + 63 : S - 1);
    const int qb0 = m.qblk[r0], qb1 = m.qblk[last];
    const uint8_t *bcol = m.bits + (int64_t)hm * m.nqb * m.nkb + kb;
    if (qb0 == qb1) {  // the tile's rows lie in one row block: all or nothing
      if (!bcol[(int64_t)qb0 * m.nkb]) bits = 0;
    } else {
      uint64_t keep = 0;
      for (int qb = qb0; qb <= qb1; ++qb)
        if (bcol[(int64_t)qb * m.nkb]) keep |= range64(m.qoffs[qb] - r0, m.qoffs[qb + 1] - r0);
      bits &= keep;
    }
  }
  return bits;
}

// Bitmap head of query head h (bm_heads in {1, Hkv, Hq}).
__device__ __forceinline__ int bitmap_head(int bm_heads, int h, int Hq, int G) {
  if (bm_heads <= 1) return 0;
  return bm_heads == Hq ? h : h / G;
}

}  // namespace lcm
