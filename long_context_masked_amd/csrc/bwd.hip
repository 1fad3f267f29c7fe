// Backward kernels: a preprocess pass, a KV-split pass for dK/dV and a
// Q-split pass for dQ.
//
// Method ("FlashAttention vs. RingAttention", dtcms, FlashAttention-2 "core
// optimisations"): the backward keeps one merged softmax statistic (LSE) and
// recomputes P from it; it is parallelised over both rows and columns
// because of the dependency dQ_i = sum_j dS_ij K_j.  Here the column split
// (one workgroup per K-tile and KV head) owns dK and dV in registers and the
// row split (one workgroup per Q-tile and head group) owns dQ in registers,
// so neither needs atomics.
//
// With c = scale * log2(e) and lse2 = LSE * log2(e):
//   P  = exp2(c * Q K^T - lse2)          (masked entries 0)
//   dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O)
//   dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K
#include <type_traits>

#include "kernels.hpp"

namespace lcm {

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Workspace rows of (b, h): lse2 at ws + 2 (b Hq + h) S64, -D right after.
__device__ __forceinline__ int64_t ws_row0(int b, int h, int Hq, int S64) {
  return 2 * ((int64_t)b * Hq + h) * S64;
}

// ws <- {lse * log2(e), -D = -sum_d dO * O} per (b, h, row); rows in
// [S, S64) get zeros.  When dqacc is given, its row (b, s, h) of the fp32 dQ
// accumulator [B][S64][Hq][D] is zeroed as well.  A row with no allowed key
// (LSE = -inf) gets a large positive lse2 instead, so that the recomputed
// P = exp2(S c - lse2) is 0 on every key, masked ones (S = -inf) included,
// rather than -inf + inf.  D is stored negated so that the dK/dV pass can
// start the accumulation of dP at -D and get dP - D from the products alone.
// One group of D/8 lanes per row; the grid covers B * S64 * Hq rows in
// [b][s][h] order.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const bf16 *o, const bf16 *dout,
                                                           const float *lse, float *ws, float *dqacc,
                                                           int S, int S64, int Hq, int64_t nrows) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  const int h = (int)(r % Hq);
  const int64_t bs = r / Hq;
  const int b = (int)(bs / S64);
  const int s = (int)(bs % S64);
  const bool real = r < nrows && s < S;
  float acc = 0.f;
  if (real) {
    const int64_t g = (((int64_t)b * S + s) * Hq + h) * D + c * 8;
    const uint4 x = *reinterpret_cast<const uint4 *>(o + g);
    const uint4 y = *reinterpret_cast<const uint4 *>(dout + g);
    acc = bf_lo(x.x) * bf_lo(y.x) + bf_hi(x.x) * bf_hi(y.x) + bf_lo(x.y) * bf_lo(y.y) +
          bf_hi(x.y) * bf_hi(y.y) + bf_lo(x.z) * bf_lo(y.z) + bf_hi(x.z) * bf_hi(y.z) +
          bf_lo(x.w) * bf_lo(y.w) + bf_hi(x.w) * bf_hi(y.w);
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (dqacc && r < nrows) {  // the fp32 dQ accumulator row starts at zero
    float *z = dqacc + r * D + c * 8;
    *reinterpret_cast<f32x4 *>(z) = (f32x4){};
    *reinterpret_cast<f32x4 *>(z + 4) = (f32x4){};
  }
  if (r < nrows && c == 0) {
    const int64_t w0 = ws_row0(b, h, Hq, S64);
    const float l = real ? lse[((int64_t)b * Hq + h) * S + s] : 0.f;
    ws[w0 + s] = l > kNegInf ? l * kLog2e : kEmptyRowLse2;
    ws[w0 + S64 + s] = -acc;
  }
}

// ---------------------------------------------------------------------------
// dK / dV: one workgroup per (K-tile of 128 keys, KV head).  Wave w owns keys
// 32w .. 32w+31 of the tile (lane l: key 32w + l % 32), keeps K and V of
// those keys as MFMA operands in registers and accumulates dK^T and dV^T.
// For each listed Q-tile of 64 rows and each query head of the group (one
// stage), Q, dO, lse2 and D are loaded straight into LDS; Q^T and dO^T come
// from the same tiles by transposed reads.  Each stage is two 32-row units,
// and each unit u takes three steps:
//   A(u): S = Q K^T, dP = dO V^T                          (MFMA)
//   B(u): P = exp2(S c - lse2), dS = P (dP - D)           (VALU; the sum of
//         dP starts at -D, loaded from LDS straight into its accumulator)
//   C(u): dV^T += dO^T P, dK^T += Q^T dS                   (MFMA)
// Masking costs nothing on stages without masked entries: on a partial
// stage the accumulation of S starts at -inf on the masked entries (and at
// 0 elsewhere), so that their P is 0.
// One wave runs per SIMD, so the exponentials only overlap the products if
// the wave's own instruction stream alternates them: a wave stalls at an
// MFMA while the matrix pipe is busy with the previous one, but VALU work
// issued between two MFMAs runs while the first is in the pipe.  The steps of
// neighbouring units are therefore software-pipelined, and each phase is
// written as a fixed sequence of chunks (two MFMAs plus a slice of B's VALU
// work) fenced against reordering:
//   phase 1:  A(st, 1)     with B(st, 0)           (exponentials)
//   phase 2:  C(st, 0)     with B(st, 1) rows 0-15 (AGPR reads) and
//                               rows 0-7 (exponentials)
//   phase 3a: A(st + 1, 0) with B(st, 1) rows 8-15 (exponentials)
//   phase 3b: C(st, 1)     with B(st + 1, 0)       (AGPR reads)
// ("rows" are the 16 accumulator registers of a unit.)  Phase 3 reads the
// next stage's tiles, so stages rotate through three LDS buffers: the
// barrier before phase 3 publishes stage st + 1 and frees the buffer of
// stage st - 1, which then receives stage st + 2.
//
// FDQ: the pass also accumulates dQ = dS K (the dependency that makes the
// backward parallel over both rows and columns, "FlashAttention vs.
// RingAttention", FlashAttention-2 "core optimisations"), so that no second
// pass has to recompute S and dP.  dS has one key per lane, but dS K needs
// one query row per lane, so every wave writes its bf16 dS (the same values
// that enter dK) into an LDS tile [128 keys][64 rows] (phases 2 and 3b), and
// after the next stage's barrier each wave reads the whole tile transposed
// and computes dQ of the stage's 64 rows for its own 32 columns of d, from a
// slice of K kept in registers (phase 4, 16 products at d = 128).  The fp32
// result is added into a zeroed accumulator [B][S64][Hq][D] with atomics; a
// convert pass scales it and rounds it to bf16.  The dS tiles rotate through
// three LDS buffers: the one of stage st is read in stage st + 1 and written
// again in stage st + 3, after the barrier of stage st + 2 that every wave
// reaches only once its reads are done.
//
// A list entry names a Q-tile, run for each of the G query heads of the
// group (G stages); on plans with one bitmap per query head it names one
// (Q-tile, head) stage, the head in bits 24-30.
//
// NW = 2 (narrow items): 64 keys per work item, two waves, and two LDS stage
// buffers instead of three, so that two workgroups share a CU (one wave per
// SIMD either way).  For masks that leave one 64-key half of many 128-key
// tiles empty (64-wide bitmap blocks), a 128-key item would spend half its
// products on masked keys in those stages.  With two buffers, stage st + 2
// can only be loaded once every wave has finished reading stage st, so its
// loads are issued after a second barrier at the end of stage st, into
// stage st's buffer.
// ---------------------------------------------------------------------------
template <int D, bool FDQ, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_dkdv_kernel(BwdArgs a) {
  static_assert(NW == 4 || (NW == 2 && !FDQ), "narrow items have no fused dQ variant");
  constexpr int KT = 32 * NW;   // keys per work item
  constexpr int KS = D / 16;    // k-steps of A (two MFMAs each: S and dP)
  constexpr int DB = D / 32;    // 32-row blocks of dK^T / dV^T
  constexpr int NC = 2 * DB;    // chunks of C (two MFMAs each: dV and dK)
  using T = Tile<D>;
  using T64 = Tile<64>;
  constexpr int OFF_DO = T::BYTES, OFF_L = 2 * T::BYTES, OFF_D = OFF_L + 256;
  constexpr int STAGE = 2 * T::BYTES + 1024;
  constexpr int NBUF = NW == 4 ? 3 : 2;
  // k-steps of A operands read ahead (the fused pass gives the registers of
  // two of them to its dQ phase)
  constexpr int PF = KS < (FDQ ? 2 : 4) ? KS : (FDQ ? 2 : 4);
  constexpr int DSB = 2 * T64::BYTES;  // dS of a stage: keys 0-63, then 64-127
  constexpr int RBW = DB / 2;          // 32-row blocks of dQ per wave (d = 128: 2, d = 64: 1)
  static_assert(16 % KS == 0 && 8 % KS == 0 && 16 % NC == 0 && 8 % NC == 0, "chunking");
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE + (FDQ ? 3 * DSB : 0)];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ln = lane & 31, hh = lane >> 5;
  const int4 item = a.bitems[blockIdx.x];
  const int slot = *as_const(a.bslot + blockIdx.x);  // >= 0: one chunk of a split item
  const int b = blockIdx.y;
  const int S = a.S, G = a.G;
  const int kvh = item.y;
  const int key = item.x * KT + wave * 32 + ln;
  const bool key_ok = key < S;
  const int64_t ldq = (int64_t)a.Hq * D, ldk = (int64_t)a.Hkv * D;

  bf16x8 kv[KS], vv[KS];
  {
    const int64_t off = ((int64_t)b * S + (key_ok ? key : 0)) * ldk + (int64_t)kvh * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kv[ks] = *reinterpret_cast<const bf16x8 *>(a.k + off + ks * 16);
      vv[ks] = *reinterpret_cast<const bf16x8 *>(a.v + off + ks * 16);
      if (!key_ok) { kv[ks] = (bf16x8){}; vv[ks] = (bf16x8){}; }
    }
  }
  // FDQ: the B operand of dQ = dS K for this wave's 32 columns of d, every
  // 16-key step t of the tile: lane (ln, hh) holds K[16t + 4hh + {0..3}] and
  // K[16t + 8 + 4hh + {0..3}] at column 32 (wave % DB) + ln, the key order in
  // which the transposed reads of the dS tile hand over the k index.
  const int dqb = wave % DB, rb0 = (wave / DB) * RBW;
  bf16x8 kq[8];  // unused (and dropped) without FDQ
  if constexpr (FDQ) {
    const bf16 *kc = a.k + (int64_t)b * S * ldk + (int64_t)kvh * D + dqb * 32 + ln;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kk = item.x * 128 + 16 * t + (i < 4 ? 4 * hh + i : 8 + 4 * hh + i - 4);
        const bf16 x = kc[(int64_t)(kk < S ? kk : S - 1) * ldk];
        kq[t][i] = kk < S ? x : (bf16)0.f;
      }
    }
  }
  const int4 cb = key_ok ? a.m.colb[key] : make_int4(0, S, 0, 0);
  const int kblk = (a.m.bm_heads && key_ok) ? a.m.kblk[key] : 0;
  int roff[KS], toff[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = row_off<D>(lane, ks);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    toff[db][0] = tr_off<D>(lane, db, 0);
    toff[db][1] = tr_off<D>(lane, db, 1);
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dk[i] = (f32x16){}; dv[i] = (f32x16){}; }
  const float sl2 = a.sl2;

  const auto *list = as_const(a.blist + item.z);
  // A list entry is one Q-tile for all G query heads of the group (G stages),
  // or, with head_entries, one (Q-tile, query head) stage whose head is in
  // bits 24-30.
  const int GE = a.head_entries ? 1 : G;
  const int nst = item.w * GE;
  auto head_of = [&](int st, uint32_t ent) -> int {
    return a.head_entries ? (int)((ent >> 24) & 0x7fu) : st % G;
  };
  TileDma<D, NW> dma;
  dma.init(ldq);

  // Loads of stage st into `stg`: the Q and dO tiles of head kvh*G + g, and
  // 64 rows each of lse2 and D (32 / NW lanes of every wave, 16 bytes each),
  // so that every wave issues the same number of loads per stage.
  auto load_stage = [&](int st, char *stg, uint32_t ent) {
    const int g = head_of(st, ent);
    const int qt = (int)(ent & kTileBits);
    const int h = kvh * G + g;
    dma.load(stg, a.q + (int64_t)b * S * ldq + (int64_t)h * D, ldq, qt * 64, S);
    dma.load(stg + OFF_DO, a.dout + (int64_t)b * S * ldq + (int64_t)h * D, ldq, qt * 64, S);
    if (lane < 32 / NW) {
      const int q = wave * (32 / NW) + lane;
      const float *src =
          a.ws + ws_row0(b, h, a.Hq, a.S64) + (q >> 4) * a.S64 + qt * 64 + (q & 15) * 4;
      __builtin_amdgcn_global_load_lds(
          src,
          (__attribute__((address_space(3))) void *)((__attribute__((address_space(3))) char *)stg +
                                                      OFF_L + wave * (512 / NW)),
          16, 0, 0);
    }
  };

  // Allowed-row words of the lane's key for the two units of stage st (all
  // ones unless the tile is partial); returns whether it is partial.
  auto stage_mask = [&](int st, uint32_t ent, uint32_t (&mw)[2]) -> bool {
    const int g = head_of(st, ent);
    mw[0] = 0xffffffffu;
    mw[1] = 0xffffffffu;
    const bool part = (ent >> 31) != 0;
    if (part) {
      const int qt = (int)(ent & kTileBits);
      const int hm = bitmap_head(a.m.bm_heads, kvh * G + g, a.Hq, G);
      const uint64_t mk = key_ok ? col_mask(a.m, cb, kblk, hm, qt * 64, S) : 0ull;
      const uint64_t sh = mk >> (4 * hh);
      mw[0] = (uint32_t)sh;
      mw[1] = (uint32_t)(sh >> 32);
    }
    return part;
  };

  // The row operands of k-step ks of unit qh of `buf`.
  auto rows_q = [&](const char *buf, int qh, int ks) { return lds_rows(buf, roff[ks] + qh * 32 * T::ROWB); };
  auto rows_o = [&](const char *buf, int qh, int ks) {
    return lds_rows(buf + OFF_DO, roff[ks] + qh * 32 * T::ROWB);
  };

  // Transposed operands of C for k-step TT of unit QH of the current stage.
  uint32_t sa[DB][2];
  auto issue_tr = [&](auto qhc, auto ttc, s16x4(&x)[4 * DB]) {
    constexpr int OFF = (2 * decltype(qhc)::value + decltype(ttc)::value) * 16 * T::ROWB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      x[4 * db + 0] = tr_issue<OFF + OFF_DO>(sa[db][0]);
      x[4 * db + 1] = tr_issue<OFF + OFF_DO>(sa[db][1]);
      x[4 * db + 2] = tr_issue<OFF>(sa[db][0]);
      x[4 * db + 3] = tr_issue<OFF>(sa[db][1]);
    }
  };
  // One chunk of C: block db of k-step x.
  auto c_chunk = [&](const s16x4(&x)[4 * DB], int db, bf16x8 pb, bf16x8 dsb) {
    dv[db] = mfma32(tr_pair(x[4 * db], x[4 * db + 1]), pb, dv[db]);
    dk[db] = mfma32(tr_pair(x[4 * db + 2], x[4 * db + 3]), dsb, dk[db]);
  };

  // B pieces on accumulator register r of a unit.
  auto b_read = [&](f32x16 &s, f32x16 &dp, const f32x16 &sa_, const f32x16 &dpa, int r) {
    float x = sa_[r], y = dpa[r];
    in_vgpr(x);
    in_vgpr(y);
    s[r] = x;
    dp[r] = y;
  };
  // (Each result is pinned where it is computed: the values are consumed
  // phases later, and without the pins the compiler sinks the arithmetic
  // next to its uses, undoing the interleave.)
  auto b_exp = [&](f32x16 &s, f32x16 &dp, int r, float l) {
    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -l));
    float ds = p * dp[r];  // dp already holds dP - D
    in_vgpr(p);
    in_vgpr(ds);
    s[r] = p;
    dp[r] = ds;
  };
  auto b_pack = [&](const f32x16 &s, const f32x16 &dp, int t, bf16x8 &pb, bf16x8 &dsb) {
    pb = c_to_b(s, t);
    dsb = c_to_b(dp, t);
    in_vgpr(pb);
    in_vgpr(dsb);
  };

  // First k-step of S of a unit: the accumulation starts at 0, or, when the
  // stage is partial, at -inf on the masked entries, so that their P is 0.
  // The branch keeps the bias (and its accumulator writes) off full stages.
  auto s_first = [&](bf16x8 aq0, bool part, uint32_t mw) -> f32x16 {
    if (part) {
      __asm__ volatile("");
      f32x16 bias;
#pragma unroll
      for (int r = 0; r < 16; ++r) bias[r] = keep_or(mw, 8 * (r >> 2) + (r & 3), 0.f, kNegInf);
      return mfma32(aq0, kv[0], bias);
    }
    return mfma32(aq0, kv[0], (f32x16){});
  };

  // Start value of the dP sum of a unit: -D of its rows (the lane's 16
  // accumulator registers r hold rows 8 (r / 4) + 4 hh + r % 4).
  auto neg_d = [&](const char *buf, int qh) {
    const float *src = reinterpret_cast<const float *>(buf + OFF_D) + 32 * qh + 4 * hh;
    f32x16 x;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(src + 8 * c);
      x[4 * c] = v[0];
      x[4 * c + 1] = v[1];
      x[4 * c + 2] = v[2];
      x[4 * c + 3] = v[3];
    }
    return x;
  };

  // FDQ: dS of unit u (two k-steps t of 16 rows, as packed for dK) into the
  // dS tile of a stage.  Lane (ln, hh) of wave w holds key 32 w + ln, i.e.
  // row 32 (w % 2) + ln of 64-key tile w / 2, and rows 32 u + 16 t + 4 hh +
  // {0..3} and 32 u + 16 t + 8 + 4 hh + {0..3} of the stage in dsb[t].
  auto ds_store = [&](char *dsbuf, int u, const bf16x8 (&dsb)[2]) {
    char *tile = dsbuf + (wave >> 1) * T64::BYTES;
    const int kr = 32 * (wave & 1) + ln;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      *reinterpret_cast<bf16x4 *>(tile + T64::off(kr, 64 * u + 32 * t + 8 * hh)) =
          __builtin_shufflevector(dsb[t], dsb[t], 0, 1, 2, 3);
      *reinterpret_cast<bf16x4 *>(tile + T64::off(kr, 64 * u + 32 * t + 16 + 8 * hh)) =
          __builtin_shufflevector(dsb[t], dsb[t], 4, 5, 6, 7);
    }
  };
  // FDQ phase 4: dQ of stage sp (list entry entp, dS tile dsbuf, complete in
  // LDS for every wave) for rows 32 (rb0 + i) + [0, 32), i < RBW, and this
  // wave's 32 columns of d: A = dS rows read transposed from the tile (lane:
  // one query row, 8 keys), B = the K slice; then fp32 atomics into the
  // accumulator, unscaled.
  auto dq_phase = [&](int sp, uint32_t entp, const char *dsbuf) {
    const uint32_t base = lds_addr(dsbuf);
    const int g = head_of(sp, entp);
    const int qt = (int)(entp & kTileBits);
    const int rs = a.Hq * D;  // accumulator row stride (floats)
    // uniform base of the stage's rows for this wave's columns, plus a
    // 32-bit per-lane byte offset per atomic
    char *dst = reinterpret_cast<char *>(a.dqacc + ((int64_t)b * a.S64 + qt * 64) * rs +
                                         (int64_t)(kvh * G + g) * D + dqb * 32);
    const uint32_t loff = (uint32_t)(4 * hh * rs + ln) * 4u;
    // one 32-row block at a time; the transposed reads of 16-key step t + 1
    // (tile t / 4, its rows 16 (t % 4)) are in flight while step t's product
    // runs
    auto issue = [&](auto tc, int i, s16x4 (&x)[2]) {
      constexpr int t = decltype(tc)::value;
      constexpr int OFF = (t >> 2) * T64::BYTES + (t & 3) * 16 * T64::ROWB;
      x[0] = tr_issue<OFF>(base + tr_off<64>(lane, rb0 + i, 0));  // keys 16 t + 4 hh + {0..3}
      x[1] = tr_issue<OFF>(base + tr_off<64>(lane, rb0 + i, 1));  // keys 16 t + 8 + 4 hh + {0..3}
    };
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      f32x16 acc = (f32x16){};
      s16x4 xa[2], xb[2];
      issue(std::integral_constant<int, 0>{}, i, xa);
      tr_wait(xa);
      issue(std::integral_constant<int, 1>{}, i, xb);
      acc = mfma32(tr_pair(xa[0], xa[1]), kq[0], acc);
      tr_wait(xb);
      issue(std::integral_constant<int, 2>{}, i, xa);
      acc = mfma32(tr_pair(xb[0], xb[1]), kq[1], acc);
      tr_wait(xa);
      issue(std::integral_constant<int, 3>{}, i, xb);
      acc = mfma32(tr_pair(xa[0], xa[1]), kq[2], acc);
      tr_wait(xb);
      issue(std::integral_constant<int, 4>{}, i, xa);
      acc = mfma32(tr_pair(xb[0], xb[1]), kq[3], acc);
      tr_wait(xa);
      issue(std::integral_constant<int, 5>{}, i, xb);
      acc = mfma32(tr_pair(xa[0], xa[1]), kq[4], acc);
      tr_wait(xb);
      issue(std::integral_constant<int, 6>{}, i, xa);
      acc = mfma32(tr_pair(xb[0], xb[1]), kq[5], acc);
      tr_wait(xa);
      issue(std::integral_constant<int, 7>{}, i, xb);
      acc = mfma32(tr_pair(xa[0], xa[1]), kq[6], acc);
      tr_wait(xb);
      acc = mfma32(tr_pair(xb[0], xb[1]), kq[7], acc);
      const int row0 = 32 * (rb0 + i);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t off = loff + (uint32_t)((row0 + 8 * (r >> 2) + (r & 3)) * rs) * 4u;
        unsafeAtomicAdd(reinterpret_cast<float *>(dst + off), acc[r]);
      }
    }
  };

  f32x16 s0, dp0;  // unit (st, 0): S and dP - D in VGPRs
  uint32_t mwc[2], mwn[2];
  bool pc = false, pn = false;  // stages st and st + 1 are partial
  if (nst > 0) {
    load_stage(0, smem, list[0]);
    if (nst > 1) load_stage(1, smem + STAGE, list[1 / GE]);
    pc = stage_mask(0, list[0], mwc);
    dma_wait();
    __syncthreads();
    f32x16 sa0 = s_first(rows_q(smem, 0, 0), pc, mwc[0]), dpa0 = neg_d(smem, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks > 0) sa0 = mfma32(rows_q(smem, 0, ks), kv[ks], sa0);
      dpa0 = mfma32(rows_o(smem, 0, ks), vv[ks], dpa0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) b_read(s0, dp0, sa0, dpa0, r);
  }

  int cur = 0;  // buffer of stage st
  // FDQ: dS buffer of stage st and of stage st - 1, list entry of st - 1
  char *const dsb_base = smem + NBUF * STAGE;
  int dcur = 0, dprev = 0;
  uint32_t ent0 = nst > 0 ? list[0] : 0u, entp = 0u;
  // List entries are read a stage before they are needed, so that the
  // latency of the scalar load is covered by the products of a stage.
  uint32_t ent1 = nst > 1 ? list[1 / GE] : 0u;  // stage st + 1
  // The first operand rows and the LSE rows of a stage's phase 1 are read
  // during the previous stage's phase 3b (stage 0: here).
  f32x4 l0n[4];
  bf16x8 aqn[PF], aon[PF];
  {
    const float *sl0 = reinterpret_cast<const float *>(smem + OFF_L) + 4 * hh;
#pragma unroll
    for (int c = 0; c < 4; ++c) l0n[c] = *reinterpret_cast<const f32x4 *>(sl0 + 8 * c);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      aqn[i] = rows_q(smem, 1, i);
      aon[i] = rows_o(smem, 1, i);
    }
  }
  for (int st = 0; st < nst; ++st) {
    const uint32_t ent2 = st + 2 < nst ? list[(st + 2) / GE] : 0u;  // stage st + 2
#pragma unroll
    for (int i = 0; i < DB; ++i) { in_agpr(dk[i]); in_agpr(dv[i]); }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) { in_agpr(kv[ks]); in_agpr(vv[ks]); }
    if constexpr (FDQ) {
#pragma unroll
      for (int t = 0; t < 8; ++t) in_agpr(kq[t]);
    }
    const int nxt = cur == NBUF - 1 ? 0 : cur + 1;
    const int fre = nxt == NBUF - 1 ? 0 : nxt + 1;  // buffer of stage st - 1 = st + 2
    const char *buf = smem + cur * STAGE;
    const char *nbuf = smem + nxt * STAGE;
    if (st + 1 < nst) {
      pn = stage_mask(st + 1, ent1, mwn);
    } else {
      pn = false;
      mwn[0] = 0xffffffffu;
      mwn[1] = 0xffffffffu;
    }
    const uint32_t sbase = lds_addr(buf);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      sa[db][0] = sbase + toff[db][0];
      sa[db][1] = sbase + toff[db][1];
    }
    const float *sl = reinterpret_cast<const float *>(buf + OFF_L) + 4 * hh;
    f32x4 l0[4], l1[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) l0[c] = l0n[c];
    bf16x8 aq[KS], ao[KS];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      aq[i] = aqn[i];
      ao[i] = aon[i];
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 1: A(st, 1) with the exponentials of B(st, 0)
    f32x16 sa1 = s_first(aq[0], pc, mwc[1]), dpa1 = neg_d(buf, 1);
    bf16x8 pb0[2], dsb0[2];
    s16x4 xa[4 * DB], xb[4 * DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) {
        aq[ks + PF] = rows_q(buf, 1, ks + PF);
        ao[ks + PF] = rows_o(buf, 1, ks + PF);
      }
      if (ks == KS / 2) {
#pragma unroll
        for (int c = 0; c < 4; ++c) l1[c] = *reinterpret_cast<const f32x4 *>(sl + 32 + 8 * c);
      }
      if (ks > 0) sa1 = mfma32(aq[ks], kv[ks], sa1);
      dpa1 = mfma32(ao[ks], vv[ks], dpa1);
#pragma unroll
      for (int i = 0; i < 16 / KS; ++i) {
        const int r = ks * (16 / KS) + i;
        b_exp(s0, dp0, r, l0[r >> 2][r & 3]);
      }
      if ((ks + 1) * (16 / KS) == 8) b_pack(s0, dp0, 0, pb0[0], dsb0[0]);
      if (ks == KS - 1) {
        b_pack(s0, dp0, 1, pb0[1], dsb0[1]);
        issue_tr(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, xa);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- phase 2: C(st, 0) with B(st, 1): AGPR reads of all rows,
    // exponentials of rows 0-7
    f32x16 s1, dp1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int tt = c / DB, db = c % DB;
      if (c == 0) {
        tr_wait(xa);
        issue_tr(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, xb);
        if constexpr (FDQ) ds_store(dsb_base + dcur * DSB, 0, dsb0);
      }
      if (c == DB) tr_wait(xb);
      if (tt == 0) c_chunk(xa, db, pb0[0], dsb0[0]);
      else c_chunk(xb, db, pb0[1], dsb0[1]);
#pragma unroll
      for (int i = 0; i < 16 / NC; ++i) {
        const int r = c * (16 / NC) + i;
        b_read(s1, dp1, sa1, dpa1, r);
      }
#pragma unroll
      for (int i = 0; i < 8 / NC; ++i) {
        const int r = c * (8 / NC) + i;
        b_exp(s1, dp1, r, l1[r >> 2][r & 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pb1[2], dsb1[2];
    b_pack(s1, dp1, 0, pb1[0], dsb1[0]);

    // stage st + 1 is in LDS for every wave (three buffers: and stage st - 1's
    // buffer is free)
    dma_wait();
    __syncthreads();
    if constexpr (NBUF == 3) {
      if (st + 2 < nst) load_stage(st + 2, smem + fre * STAGE, ent2);
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      aq[i] = rows_q(nbuf, 0, i);
      ao[i] = rows_o(nbuf, 0, i);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 3a: A(st + 1, 0) with the exponentials of B(st, 1) rows 8-15
    // (after the last stage A reads a stale buffer and is discarded)
    f32x16 sa0 = s_first(aq[0], pn, mwn[0]), dpa0 = neg_d(nbuf, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) {
        aq[ks + PF] = rows_q(nbuf, 0, ks + PF);
        ao[ks + PF] = rows_o(nbuf, 0, ks + PF);
      }
      if (ks > 0) sa0 = mfma32(aq[ks], kv[ks], sa0);
      dpa0 = mfma32(ao[ks], vv[ks], dpa0);
#pragma unroll
      for (int i = 0; i < 8 / KS; ++i) {
        const int r = 8 + ks * (8 / KS) + i;
        b_exp(s1, dp1, r, l1[r >> 2][r & 3]);
      }
      if (ks == KS - 2) issue_tr(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}, xa);
      if (ks == KS - 1) b_pack(s1, dp1, 1, pb1[1], dsb1[1]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- phase 3b: C(st, 1) with B(st + 1, 0): AGPR reads
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int tt = c / DB, db = c % DB;
      if (c == 0) {
        tr_wait(xa);
        issue_tr(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, xb);
        if constexpr (FDQ) ds_store(dsb_base + dcur * DSB, 1, dsb1);
      }
      if (c == DB) tr_wait(xb);
      if (tt == 0) c_chunk(xa, db, pb1[0], dsb1[0]);
      else c_chunk(xb, db, pb1[1], dsb1[1]);
#pragma unroll
      for (int i = 0; i < 16 / NC; ++i) {
        const int r = c * (16 / NC) + i;
        b_read(s0, dp0, sa0, dpa0, r);
      }
      if (c == DB) {
        // phase 1 of stage st + 1 reads nbuf: start its first reads now
        const float *sln = reinterpret_cast<const float *>(nbuf + OFF_L) + 4 * hh;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) l0n[q4] = *reinterpret_cast<const f32x4 *>(sln + 8 * q4);
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          aqn[i] = rows_q(nbuf, 1, i);
          aon[i] = rows_o(nbuf, 1, i);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NBUF == 2) {
      // every wave is done with stage st's buffer: it receives stage st + 2
      if (st + 2 < nst) {
        __syncthreads();
        load_stage(st + 2, smem + cur * STAGE, ent2);
      }
    }
    if constexpr (FDQ) {
      // ---- phase 4: dQ of stage st - 1 (its dS tile was completed by every
      // wave before this stage's barrier)
      __builtin_amdgcn_sched_barrier(0);
      if (st >= 1) dq_phase(st - 1, entp, dsb_base + dprev * DSB);
      __builtin_amdgcn_sched_barrier(0);
      entp = ent0;
      ent0 = ent1;
      dprev = dcur;
      dcur = dcur == 2 ? 0 : dcur + 1;
    }
    mwc[0] = mwn[0];
    mwc[1] = mwn[1];
    ent1 = ent2;
    pc = pn;
    cur = nxt;
  }
  if constexpr (FDQ) {
    if (nst > 0) {
      __syncthreads();  // the last stage's dS tile, from every wave
      dq_phase(nst - 1, entp, dsb_base + dprev * DSB);
    }
  }

  if (slot >= 0) {
    // a chunk of a split item: unscaled fp32 partial sums into its slot
    float *pk = a.part + (((int64_t)b * a.n_slots + slot) * 2) * kDkdvKeys * D +
                (int64_t)(wave * 32 + ln) * D;
    float *pv = pk + (int64_t)kDkdvKeys * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = db * 32 + 8 * c + 4 * hh;
        *reinterpret_cast<f32x4 *>(pk + d0) =
            (f32x4){dk[db][4 * c], dk[db][4 * c + 1], dk[db][4 * c + 2], dk[db][4 * c + 3]};
        *reinterpret_cast<f32x4 *>(pv + d0) =
            (f32x4){dv[db][4 * c], dv[db][4 * c + 1], dv[db][4 * c + 2], dv[db][4 * c + 3]};
      }
  } else if (key_ok) {
    const int64_t off = ((int64_t)b * S + key) * ldk + (int64_t)kvh * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = db * 32 + 8 * c + 4 * hh;
        *reinterpret_cast<bf16x4 *>(a.dk + off + d0) = __builtin_shufflevector(
            cvt2(dk[db][4 * c] * sc, dk[db][4 * c + 1] * sc),
            cvt2(dk[db][4 * c + 2] * sc, dk[db][4 * c + 3] * sc), 0, 1, 2, 3);
        *reinterpret_cast<bf16x4 *>(a.dv + off + d0) = __builtin_shufflevector(
            cvt2(dv[db][4 * c], dv[db][4 * c + 1]), cvt2(dv[db][4 * c + 2], dv[db][4 * c + 3]),
            0, 1, 2, 3);
      }
  }
}

// ---------------------------------------------------------------------------
// Sum of the partial dK/dV of each split dK/dV item, over its chunks in slot
// order (so the result does not depend on scheduling), then dK * scale and
// both to bf16.  One workgroup per (split item, batch entry); a thread sums
// four consecutive values of one key at a time.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_dkdv_reduce_kernel(BwdArgs a) {
  const int4 r = a.breduce[blockIdx.x];  // K-tile, KV head, first slot, chunks
  const int b = blockIdx.y;
  const int64_t ldk = (int64_t)a.Hkv * D;
  constexpr int PER = kDkdvKeys * D / 4;  // float4 groups per output (dK or dV)
  const float *base = a.part + ((int64_t)b * a.n_slots + r.z) * 2 * kDkdvKeys * D;
  for (int i = threadIdx.x; i < 2 * PER; i += blockDim.x) {
    const int which = i / PER, j = i - which * PER;
    const int kl = j / (D / 4), d0 = (j - kl * (D / 4)) * 4;
    const int key = r.x * a.key_tile + kl;  // a slot holds 128 keys; narrow items use 64
    if (kl >= a.key_tile || key >= a.S) continue;
    const float *src = base + (int64_t)which * kDkdvKeys * D + (int64_t)kl * D + d0;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(src);
    for (int c = 1; c < r.w; ++c)
      acc += *reinterpret_cast<const f32x4 *>(src + (int64_t)c * 2 * kDkdvKeys * D);
    if (which == 0) acc *= a.scale;
    bf16 *dst = (which == 0 ? a.dk : a.dv) + ((int64_t)b * a.S + key) * ldk + (int64_t)r.y * D + d0;
    *reinterpret_cast<bf16x4 *>(dst) =
        __builtin_shufflevector(cvt2(acc[0], acc[1]), cvt2(acc[2], acc[3]), 0, 1, 2, 3);
  }
}


// ---------------------------------------------------------------------------
// dQ from the fp32 accumulator of the fused dK/dV pass: dQ = scale * acc,
// rounded to bf16.  One group of D/8 lanes per (b, s, h) row of dQ, s < S;
// bound by HBM (4 bytes read, 2 written per element).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_dq_convert_kernel(const float *acc, bf16 *dq, int S,
                                                              int S64, int Hq, float scale,
                                                              int64_t nrows) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
  if (r >= nrows) return;
  const int c = threadIdx.x % CPR;
  const int h = (int)(r % Hq);
  const int64_t bs = r / Hq;
  const int64_t b = bs / S, s = bs % S;
  const float *src = acc + ((b * S64 + s) * Hq + h) * D + c * 8;
  const f32x4 x0 = *reinterpret_cast<const f32x4 *>(src) * scale;
  const f32x4 x1 = *reinterpret_cast<const f32x4 *>(src + 4) * scale;
  *reinterpret_cast<bf16x8 *>(dq + r * D + c * 8) = pack8(x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per forward work item (Q-tile, head group); same lane
// ownership as the forward.  K and V tiles of 64 keys are loaded straight
// into LDS (natural layout, double-buffered); K^T comes from the K tile by
// transposed reads.  Each K-tile is processed as two 32-key halves:
//   S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T * (dP^T - D),  dQ^T += K^T dS^T
// ---------------------------------------------------------------------------
// MASKED = false drops the partial-tile path (plans without partial tiles).
template <int D, int HG, bool MASKED>
__global__ __launch_bounds__(256, 2) void attn_dq_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  using T = Tile<D>;
  constexpr int STAGE = 2 * T::BYTES;  // K tile, then V tile
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int ln = lane & 31, hh = lane >> 5;
  const int4 item = a.fitems[blockIdx.x];
  const int b = blockIdx.y;
  const int S = a.S;
  const int h = item.y + wave % HG;
  const int row = item.x * (128 / HG) + (wave / HG) * 32 + ln;
  const int kvh = h / a.G;
  const int64_t ldq = (int64_t)a.Hq * D, ldk = (int64_t)a.Hkv * D;
  const bf16 *kbase = a.k + (int64_t)b * S * ldk + (int64_t)kvh * D;
  const bf16 *vbase = a.v + (int64_t)b * S * ldk + (int64_t)kvh * D;
  const bool row_ok = row < S;
  if (item.w == 0) {
    // no listed tile: dQ of the item's rows is 0
    if (row_ok) zero_half_row<D>(a.dq + ((int64_t)b * S + row) * ldq + (int64_t)h * D, hh);
    return;
  }

  bf16x8 qv[KS], dov[KS];
  {
    const int64_t off = ((int64_t)b * S + (row_ok ? row : 0)) * ldq + (int64_t)h * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qv[ks] = *reinterpret_cast<const bf16x8 *>(a.q + off + ks * 16);
      dov[ks] = *reinterpret_cast<const bf16x8 *>(a.dout + off + ks * 16);
      if (!row_ok) { qv[ks] = (bf16x8){}; dov[ks] = (bf16x8){}; }
    }
  }
  float lse2 = 0.f, nD = 0.f;  // the row's lse * log2(e) and -D
  if (row_ok) {
    const int64_t w0 = ws_row0(b, h, a.Hq, a.S64);
    lse2 = a.ws[w0 + row];
    nD = a.ws[w0 + a.S64 + row];
  }
  const int4 rb = row_ok ? a.m.rowb[row] : make_int4(0, 0, 0, 0);
  const int hm = bitmap_head(a.m.bm_heads, h, a.Hq, a.G);
  const int qb = (a.m.bm_heads && row_ok) ? a.m.qblk[row] : 0;
  int roff[KS], koff[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = row_off<D>(lane, ks);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    koff[db][0] = tr_off<D>(lane, db, 0);
    koff[db][1] = tr_off<D>(lane, db, 1);
  }

  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = (f32x16){};
  const float sl2 = a.sl2;

  const auto *list = as_const(a.flist + item.z);
  const int n = item.w;
  TileDma<D> dma;
  dma.init(ldk);
  if (n > 0) {
    const int kt = (int)(list[0] & 0x7fffffffu);
    dma.load(smem, kbase, ldk, kt * 64, S);
    dma.load(smem + T::BYTES, vbase, ldk, kt * 64, S);
  }
  dma_wait();
  __syncthreads();

  // One K-tile, read from buffer BUF (tiles alternate between the two
  // buffers; with BUF a constant the buffer offset folds into the LDS
  // instructions' immediate offsets).
  const uint32_t sbase = lds_addr(smem);
  uint32_t ka[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    ka[db][0] = sbase + koff[db][0];
    ka[db][1] = sbase + koff[db][1];
  }
  auto tile = [&](int e, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const uint32_t ent = list[e];
    const int kt = (int)(ent & 0x7fffffffu);
    const bool partial = MASKED && (ent >> 31) != 0;
    char *stage = smem + BUF * STAGE;
    if (e + 1 < n) {
      const int nkt = (int)(list[e + 1] & 0x7fffffffu);
      char *next = smem + (1 - BUF) * STAGE;
      dma.load(next, kbase, ldk, nkt * 64, S);
      dma.load(next + T::BYTES, vbase, ldk, nkt * 64, S);
    }
    uint32_t mw[2] = {0xffffffffu, 0xffffffffu};
    bool active = true;
    if (partial) {
      const uint64_t mk = row_ok ? row_mask(a.m, rb, qb, hm, kt * 64, S) : 0ull;
      active = __ballot(mk != 0ull) != 0ull;
      const uint64_t sh = mk >> (4 * hh);
      mw[0] = (uint32_t)sh;
      mw[1] = (uint32_t)(sh >> 32);
    }
    if (active) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        // Two waves share each SIMD; the one computing S and dP runs at raised
        // priority, which staggers the waves so that one's products overlap
        // the other's softmax-gradient work.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = mfma32(lds_rows(stage, roff[ks] + kh * 32 * T::ROWB), qv[ks], s);
          dp = mfma32(lds_rows(stage + T::BYTES, roff[ks] + kh * 32 * T::ROWB), dov[ks], dp);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        if (partial) {  // masked scores -> -inf, so that P = 0 there
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = keep_or(mw[kh], 8 * (r >> 2) + (r & 3), s[r], kNegInf);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -lse2));
          dp[r] = p * (dp[r] + nD);
        }
        // dQ^T += K^T dS^T, one 16-key step at a time.
        auto step = [&](auto tc) {
          constexpr int t = decltype(tc)::value;  // 16-key step within the tile
          constexpr int toff = BUF * STAGE + t * 16 * T::ROWB;
          s16x4 x[2 * DB];
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            x[2 * db] = tr_issue<toff>(ka[db][0]);
            x[2 * db + 1] = tr_issue<toff>(ka[db][1]);
          }
          const bf16x8 dsb = c_to_b(dp, t & 1);
          tr_wait(x);
#pragma unroll
          for (int db = 0; db < DB; ++db) dq[db] = mfma32(tr_pair(x[2 * db], x[2 * db + 1]), dsb, dq[db]);
        };
        if (kh == 0) {
          step(std::integral_constant<int, 0>{});
          step(std::integral_constant<int, 1>{});
        } else {
          step(std::integral_constant<int, 2>{});
          step(std::integral_constant<int, 3>{});
        }
      }
    }
    dma_wait();
    __syncthreads();
  };
  int e = 0;
  for (; e + 1 < n; e += 2) {
    tile(e, std::integral_constant<int, 0>{});
    tile(e + 1, std::integral_constant<int, 1>{});
  }
  if (e < n) tile(e, std::integral_constant<int, 0>{});

  if (row_ok) {
    bf16 *qrow = a.dq + ((int64_t)b * S + row) * ldq + (int64_t)h * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = db * 32 + 8 * c + 4 * hh;
        *reinterpret_cast<bf16x4 *>(qrow + d0) = __builtin_shufflevector(
            cvt2(dq[db][4 * c] * sc, dq[db][4 * c + 1] * sc),
            cvt2(dq[db][4 * c + 2] * sc, dq[db][4 * c + 3] * sc), 0, 1, 2, 3);
      }
  }
}

// Every variant is instantiated explicitly: implicit instantiation from the
// launchers alone has left some host-side launch stubs unemitted.
template __global__ void attn_bwd_pre_kernel<128>(const bf16 *, const bf16 *, const float *,
                                                  float *, float *, int, int, int, int64_t);
template __global__ void attn_bwd_pre_kernel<64>(const bf16 *, const bf16 *, const float *,
                                                 float *, float *, int, int, int, int64_t);
template __global__ void attn_dkdv_kernel<128, false, 4>(BwdArgs);
template __global__ void attn_dkdv_kernel<64, false, 4>(BwdArgs);
template __global__ void attn_dkdv_kernel<128, true, 4>(BwdArgs);
template __global__ void attn_dkdv_kernel<64, true, 4>(BwdArgs);
template __global__ void attn_dkdv_kernel<128, false, 2>(BwdArgs);
template __global__ void attn_dkdv_kernel<64, false, 2>(BwdArgs);
template __global__ void attn_dq_convert_kernel<128>(const float *, bf16 *, int, int, int, float, int64_t);
template __global__ void attn_dq_convert_kernel<64>(const float *, bf16 *, int, int, int, float, int64_t);
template __global__ void attn_dkdv_reduce_kernel<128>(BwdArgs);
template __global__ void attn_dkdv_reduce_kernel<64>(BwdArgs);
#define LCM_DQ(D, HG)                                             \
  template __global__ void attn_dq_kernel<D, HG, true>(BwdArgs);  \
  template __global__ void attn_dq_kernel<D, HG, false>(BwdArgs);
LCM_DQ(128, 2)
LCM_DQ(128, 1)
LCM_DQ(64, 2)
LCM_DQ(64, 1)
#undef LCM_DQ

hipError_t launch_bwd_pre(const BwdArgs &a, int d, int B, hipStream_t st) {
  const int64_t nrows = (int64_t)B * a.S64 * a.Hq;
  const int rpb = 256 / (d / 8);
  const dim3 grid((unsigned)((nrows + rpb - 1) / rpb)), block(256);
  if (d == 128)
    hipLaunchKernelGGL((attn_bwd_pre_kernel<128>), grid, block, 0, st, a.o, a.dout, a.lse, a.ws,
                       a.dqacc, a.S, a.S64, a.Hq, nrows);
  else if (d == 64)
    hipLaunchKernelGGL((attn_bwd_pre_kernel<64>), grid, block, 0, st, a.o, a.dout, a.lse, a.ws,
                       a.dqacc, a.S, a.S64, a.Hq, nrows);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_dq_convert(const BwdArgs &a, int d, int B, hipStream_t st) {
  const int64_t nrows = (int64_t)B * a.S * a.Hq;
  const int rpb = 256 / (d / 8);
  const dim3 grid((unsigned)((nrows + rpb - 1) / rpb)), block(256);
  if (d == 128)
    hipLaunchKernelGGL((attn_dq_convert_kernel<128>), grid, block, 0, st, a.dqacc, a.dq, a.S, a.S64,
                       a.Hq, a.scale, nrows);
  else if (d == 64)
    hipLaunchKernelGGL((attn_dq_convert_kernel<64>), grid, block, 0, st, a.dqacc, a.dq, a.S, a.S64,
                       a.Hq, a.scale, nrows);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_dkdv(const BwdArgs &a, int d, int B, bool fused_dq, hipStream_t st) {
  const dim3 grid((unsigned)a.n_bitems, (unsigned)B), block(256), narrow(128);
  if (a.key_tile == 64 && fused_dq) return hipErrorInvalidValue;
  if (a.key_tile == 64 && d == 128) hipLaunchKernelGGL((attn_dkdv_kernel<128, false, 2>), grid, narrow, 0, st, a);
  else if (a.key_tile == 64 && d == 64) hipLaunchKernelGGL((attn_dkdv_kernel<64, false, 2>), grid, narrow, 0, st, a);
  else if (a.key_tile != 128) return hipErrorInvalidValue;
  else if (d == 128 && fused_dq) hipLaunchKernelGGL((attn_dkdv_kernel<128, true, 4>), grid, block, 0, st, a);
  else if (d == 128) hipLaunchKernelGGL((attn_dkdv_kernel<128, false, 4>), grid, block, 0, st, a);
  else if (d == 64 && fused_dq) hipLaunchKernelGGL((attn_dkdv_kernel<64, true, 4>), grid, block, 0, st, a);
  else if (d == 64) hipLaunchKernelGGL((attn_dkdv_kernel<64, false, 4>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_breduce == 0) return e;
  const dim3 rgrid((unsigned)a.n_breduce, (unsigned)B);
  if (d == 128) hipLaunchKernelGGL((attn_dkdv_reduce_kernel<128>), rgrid, block, 0, st, a);
  else hipLaunchKernelGGL((attn_dkdv_reduce_kernel<64>), rgrid, block, 0, st, a);
  return hipGetLastError();
}

template <int D, int HG>
static void launch_dq_masked(const BwdArgs &a, bool masked, dim3 grid, hipStream_t st) {
  if (masked) hipLaunchKernelGGL((attn_dq_kernel<D, HG, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attn_dq_kernel<D, HG, false>), grid, dim3(256), 0, st, a);
}

hipError_t launch_dq(const BwdArgs &a, int d, int HG, bool masked, int B, hipStream_t st) {
  const dim3 grid((unsigned)a.n_fitems, (unsigned)B);
  if (d == 128 && HG == 2) launch_dq_masked<128, 2>(a, masked, grid, st);
  else if (d == 128 && HG == 1) launch_dq_masked<128, 1>(a, masked, grid, st);
  else if (d == 64 && HG == 2) launch_dq_masked<64, 2>(a, masked, grid, st);
  else if (d == 64 && HG == 1) launch_dq_masked<64, 1>(a, masked, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lcm
