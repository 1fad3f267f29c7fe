// Forward kernel: O = softmax(mask(Q K^T * scale)) V and LSE, Q-split.
//
// Method ("FlashAttention vs. RingAttention", dtcms): tiling with online
// softmax and fused masking (FlashAttention-1, "core optimisations"); the
// output is normalised once at the end, one merged statistic (LSE) is kept,
// and the work is split along Q rows (FlashAttention-2, "core
// optimisations").
//
// One workgroup = 4 waves = one work item: (Q-tile, group of HG query heads
// that share a KV head).  Wave w owns 32 query rows of head h0 + w % HG; lane
// l owns row 32*(w / HG) + l % 32, and the two lane halves split each K-tile's
// 64 keys.  K and V tiles of 64 keys are loaded straight into LDS (natural
// layout) and shared by all heads of the item.  Per K-tile t:
//   S^T = K Q^T                  (MFMA; K row reads, Q^T in registers;
//                                 masked entries start the sum at -inf)
//   m update                     (running max kept stale within the slack)
//   P^T = exp2(S^T c - m) -> bf16, l += sum P (bf16 dot products)
//   O^T += V^T P^T               (MFMA; V^T by transposed LDS reads)
// The steps of neighbouring tiles are software-pipelined so that every run
// of products has independent VALU work between its MFMAs (a wave stalls at
// an MFMA while the matrix pipe is busy with the previous one, but VALU
// work issued between two MFMAs runs meanwhile):
//   phase A:  S^T(t + 1)     with the exponentials of key block 0 of tile t
//   phase B:  O^T += V^T(t)  with the exponentials of key block 1 of tile t
//             P^T(t)         and the maximum of S^T(t + 1)
// K tiles are read one tile ahead of V tiles, so each has its own ring of two
// LDS slots; the loads for K(t + 3) and V(t + 2) are issued after the
// barrier that ends tile t and complete by the barrier that ends tile t + 1.
#include <type_traits>

#include "kernels.hpp"

namespace lcm {

// MASKED = false drops the partial-tile path, for plans whose lists hold no
// partial tile (the code and registers it takes cost full tiles 1-2%).
template <int D, int HG, bool MASKED>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdArgs a) {
  constexpr int KS = D / 16;   // k-steps of QK^T
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int NCB = 2 * DB;  // chunks of two MFMAs in phase B (4 P^T steps)
  using T = Tile<D>;
  constexpr int VOFF = 2 * T::BYTES;  // K slots 0 and 1, then V slots 0 and 1
  static_assert(16 % KS == 0 && 16 % DB == 0, "chunking");
  __shared__ __attribute__((aligned(1024))) char smem[4 * T::BYTES];

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int ln = lane & 31, hh = lane >> 5;
  const int4 item = a.items[blockIdx.x];
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
    // no listed tile: no row of the item has an allowed key (O = 0, LSE = -inf)
    if (row_ok) {
      const int64_t o0 = ((int64_t)b * S + row) * ldq + (int64_t)h * D;
      if (a.o32) zero_half_row<D>(a.o32 + o0, hh);
      else zero_half_row<D>(a.o + o0, hh);
      if (hh == 0) a.lse[((int64_t)b * a.Hq + h) * S + row] = kNegInf;
    }
    return;
  }

  bf16x8 qv[KS];
  {
    const bf16 *qrow = a.q + ((int64_t)b * S + (row_ok ? row : 0)) * ldq + (int64_t)h * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qv[ks] = *reinterpret_cast<const bf16x8 *>(qrow + ks * 16);
      if (!row_ok) qv[ks] = (bf16x8){};
    }
  }
  const int4 rb = row_ok ? a.m.rowb[row] : make_int4(0, 0, 0, 0);
  const int hm = bitmap_head(a.m.bm_heads, h, a.Hq, a.G);
  const int qb = (a.m.bm_heads && row_ok) ? a.m.qblk[row] : 0;
  // K row reads use byte offsets from a slot; transposed V reads use LDS
  // addresses in V slot 0 (slot 1 adds a constant to the instruction)
  int koff[KS];
  uint32_t va[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = row_off<D>(lane, ks);
  {
    const uint32_t v0 = lds_addr(smem + VOFF);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      va[db][0] = v0 + tr_off<D>(lane, db, 0);
      va[db][1] = v0 + tr_off<D>(lane, db, 1);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = (f32x16){};
  float m_run = kMinit, l_run = 0.f;
  const float sl2 = a.sl2;

  const auto *list = as_const(a.list + item.z);
  const int n = item.w;
  TileDma<D> dma;
  dma.init(ldk);
  auto load_k = [&](int e, int slot) {
    dma.load(smem + slot * T::BYTES, kbase, ldk, (int)(list[e] & 0x7fffffffu) * 64, S);
  };
  auto load_v = [&](int e, int slot) {
    dma.load(smem + VOFF + slot * T::BYTES, vbase, ldk, (int)(list[e] & 0x7fffffffu) * 64, S);
  };
  // Allowed-key words of the lane's row for the two key blocks of tile e
  // (all ones unless the tile is partial); returns whether the tile needs the
  // per-entry bias.  A partial tile in which every row of the wave sees all
  // 64 keys or none (a bitmap or document edge between rows, not inside the
  // tile's keys) needs none: `dead` marks the rows that see no key, whose
  // exponentials then take a -inf offset and whose maxima are left out.
  auto tile_mask = [&](int e, uint32_t (&mw)[2], bool &dead) -> bool {
    const uint32_t ent = list[e];
    mw[0] = 0xffffffffu;
    mw[1] = 0xffffffffu;
    dead = false;
    bool part = MASKED && (ent >> 31) != 0;
    if (part) {
      const uint64_t mk = row_ok ? row_mask(a.m, rb, qb, hm, (int)(ent & 0x7fffffffu) * 64, S) : 0ull;
      dead = mk == 0ull;
      part = __ballot(mk != 0ull && mk != ~0ull) != 0ull;
      const uint64_t sh = mk >> (4 * hh);
      mw[0] = (uint32_t)sh;
      mw[1] = (uint32_t)(sh >> 32);
    }
    return part;
  };
  // First k-step of S^T for one key block: the sum starts at 0, or, on a
  // partial tile, at -inf on the masked entries (whose P is then 0).  The
  // branch keeps the bias off full tiles.
  auto s_first = [&](bf16x8 ak0, bool part, uint32_t mw) -> f32x16 {
    if (part) {
      __asm__ volatile("");
      f32x16 bias;
#pragma unroll
      for (int r = 0; r < 16; ++r) bias[r] = keep_or(mw, 8 * (r >> 2) + (r & 3), 0.f, kNegInf);
      return mfma32(ak0, qv[0], bias);
    }
    return mfma32(ak0, qv[0], (f32x16){});
  };
  // P of accumulator register r of key block kb, pinned where it is
  // computed (the compiler would otherwise sink it next to its use and undo
  // the interleave).
  float mneg = -m_run;  // -m_run, or -inf on a row that sees no key of the tile
  auto p_exp = [&](f32x16 &s, int r) {
    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, mneg));
    in_vgpr(p);
    s[r] = p;
  };
  auto p_pack = [&](const f32x16 &s, int t, bf16x8 &pb) {
    pb = c_to_b(s, t);
    in_vgpr(pb);
    l_run = sum8(pb, l_run);
  };
  // Running max after S^T of a new tile (rescaling O only past the slack).
  auto m_update = [&](float mx) {
    const float m_new = __builtin_fmaxf(m_run, max_halves(mx) * sl2);
    if (__ballot(m_new > m_run + kRescaleSlack) != 0ull) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }
  };

  // Prologue: K(0), V(0), K(1) in; S^T(0) and its max; then K(2), V(1) out.
  f32x16 sc[2];  // S^T of the current tile, then its P (exponentiated in place)
  bool dc = false;  // this row sees no key of the current tile (row-uniform tile)
  if (n > 0) {
    load_k(0, 0);
    load_v(0, 0);
    if (n > 1) load_k(1, 1);
    uint32_t mw[2];
    const bool part = tile_mask(0, mw, dc);
    dma_wait();
    __syncthreads();
    bf16x8 ak[2][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ak[0][ks] = lds_rows(smem, koff[ks]);
      ak[1][ks] = lds_rows(smem, koff[ks] + 32 * T::ROWB);
    }
    sc[0] = s_first(ak[0][0], part, mw[0]);
    sc[1] = s_first(ak[1][0], part, mw[1]);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
      sc[0] = mfma32(ak[0][ks], qv[ks], sc[0]);
      sc[1] = mfma32(ak[1][ks], qv[ks], sc[1]);
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sc[0][r]), sc[1][r]);
    m_update(dc ? kNegInf : mx);
    __syncthreads();  // every wave is done with K slot 0
    if (n > 2) load_k(2, 0);
    if (n > 1) load_v(1, 1);
  }

  // Tile t, read from K slot 1 - P (for t + 1) and V slot P; P = t % 2 is a
  // constant so that slot offsets fold into the LDS instructions.
  auto tile = [&](int t, auto pc, auto nc) {
    constexpr int P = decltype(pc)::value;
    constexpr bool NEXT = decltype(nc)::value;  // tile t + 1 exists
    const char *kslot = smem + (1 - P) * T::BYTES;
    uint32_t mw[2] = {0xffffffffu, 0xffffffffu};
    bool pn = false, dn = false;
    if constexpr (NEXT) pn = tile_mask(t + 1, mw, dn);
    mneg = dc ? kNegInf : -m_run;
    bf16x8 ak[2][KS];
    if constexpr (NEXT) {
      ak[0][0] = lds_rows(kslot, koff[0]);
      ak[1][0] = lds_rows(kslot, koff[0] + 32 * T::ROWB);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase A: S^T(t + 1) with the exponentials of key block 0 of tile t
    f32x16 sn[2];
    bf16x8 pb[4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (NEXT) {
        if (ks + 1 < KS) {
          ak[0][ks + 1] = lds_rows(kslot, koff[ks + 1]);
          ak[1][ks + 1] = lds_rows(kslot, koff[ks + 1] + 32 * T::ROWB);
        }
        if (ks == 0) {
          sn[0] = s_first(ak[0][0], pn, mw[0]);
          sn[1] = s_first(ak[1][0], pn, mw[1]);
        } else {
          sn[0] = mfma32(ak[0][ks], qv[ks], sn[0]);
          sn[1] = mfma32(ak[1][ks], qv[ks], sn[1]);
        }
      }
#pragma unroll
      for (int i = 0; i < 16 / KS; ++i) p_exp(sc[0], ks * (16 / KS) + i);
      if ((ks + 1) * (16 / KS) == 8) p_pack(sc[0], 0, pb[0]);
      if (ks == KS - 1) p_pack(sc[0], 1, pb[1]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Two waves share each SIMD (two workgroups per CU).  The wave in phase B
    // runs at raised priority, so that its products go first while the
    // other wave's phase A fills the gaps; this staggers the waves' phases.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase B: O^T += V^T P^T(t), 16 keys per step, with the
    // exponentials of key block 1 (steps 0 and 1) and the max of S^T(t + 1)
    auto issue = [&](auto stc, s16x4(&x)[2 * DB]) {
      constexpr int toff = P * T::BYTES + decltype(stc)::value * 16 * T::ROWB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        x[2 * db] = tr_issue<toff>(va[db][0]);
        x[2 * db + 1] = tr_issue<toff>(va[db][1]);
      }
    };
    s16x4 xa[2 * DB], xb[2 * DB];
    float mx = kNegInf;
    issue(std::integral_constant<int, 0>{}, xa);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int st = c / (DB / 2);         // P^T step (16 keys)
      const int d0 = (c % (DB / 2)) * 2;   // first of the chunk's two O^T blocks
      if (c % (DB / 2) == 0) {
        if (st % 2 == 0) {
          tr_wait(xa);
          if (st == 0) issue(std::integral_constant<int, 1>{}, xb);
          if (st == 2) issue(std::integral_constant<int, 3>{}, xb);
        } else {
          tr_wait(xb);
          if (st == 1) issue(std::integral_constant<int, 2>{}, xa);
        }
      }
      const s16x4(&x)[2 * DB] = (st % 2 == 0) ? xa : xb;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        o[d0 + j] = mfma32(tr_pair(x[2 * (d0 + j)], x[2 * (d0 + j) + 1]), pb[st], o[d0 + j]);
      if (c < DB) {  // steps 0 and 1: exponentials of key block 1
#pragma unroll
        for (int i = 0; i < 16 / DB; ++i) p_exp(sc[1], c * (16 / DB) + i);
        if ((c + 1) * (16 / DB) == 8) p_pack(sc[1], 0, pb[2]);
        if (c == DB - 1) p_pack(sc[1], 1, pb[3]);
      }
      if constexpr (NEXT) {
#pragma unroll
        for (int i = 0; i < 16 / NCB; ++i) {
          const int r = c * (16 / NCB) + i;
          mx = __builtin_fmaxf(__builtin_fmaxf(mx, sn[0][r]), sn[1][r]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) {
      m_update(dn ? kNegInf : mx);
      sc[0] = sn[0];
      sc[1] = sn[1];
      dc = dn;
    }

    // K(t + 2) and V(t + 1) are in LDS for every wave; K slot 1 - P and V
    // slot P are free
    dma_wait();
    __syncthreads();
    if (t + 3 < n) load_k(t + 3, 1 - P);
    if (t + 2 < n) load_v(t + 2, P);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  int t = 0;
  for (; t + 2 < n; t += 2) {
    tile(t, C0{}, Yes{});
    tile(t + 1, C1{}, Yes{});
  }
  if (t + 1 < n) {
    tile(t, C0{}, Yes{});
    tile(t + 1, C1{}, No{});
  } else if (t < n) {
    tile(t, C0{}, No{});
  }

  const float l_tot = sum_halves(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t o0 = ((int64_t)b * S + row) * ldq + (int64_t)h * D;
    if (a.o32) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int d0 = db * 32 + 8 * c + 4 * hh;
          *reinterpret_cast<f32x4 *>(a.o32 + o0 + d0) =
              (f32x4){o[db][4 * c] * inv, o[db][4 * c + 1] * inv, o[db][4 * c + 2] * inv,
                      o[db][4 * c + 3] * inv};
        }
    } else {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int d0 = db * 32 + 8 * c + 4 * hh;
          *reinterpret_cast<bf16x4 *>(a.o + o0 + d0) = __builtin_shufflevector(
              cvt2(o[db][4 * c] * inv, o[db][4 * c + 1] * inv),
              cvt2(o[db][4 * c + 2] * inv, o[db][4 * c + 3] * inv), 0, 1, 2, 3);
        }
    }
    if (hh == 0)
      a.lse[((int64_t)b * a.Hq + h) * S + row] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Merge of two attention results over disjoint key sets for the same queries
// ("FlashAttention vs. RingAttention", Ring Attention section: the Blockwise
// Parallel Transformer rescales each key block's output by the difference
// between its own softmax normaliser and the global one):
//   LSE = ln(e^LSE1 + e^LSE2),  O = e^(LSE1 - LSE) O1 + e^(LSE2 - LSE) O2.
// A row with no key in either part gets O = 0, LSE = -inf.  The parts are
// fp32; the result is fp32 (to merge further) or bf16 (OB).  One group of
// D/8 lanes per (b, s, h) row, 8 values per lane, rows in memory order;
// bound by HBM.
// ---------------------------------------------------------------------------
template <int D, bool OB>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float *o1, const float *lse1,
                                                         const float *o2, const float *lse2,
                                                         void *o, float *lse, int S, int Hq,
                                                         int64_t nrows) {
  constexpr int CPR = D / 8;      // lanes per row
  constexpr int RPB = 256 / CPR;  // rows per workgroup
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
  if (r >= nrows) return;
  const int c = threadIdx.x % CPR;
  const int h = (int)(r % Hq);
  const int64_t bs = r / Hq;  // b * S + s
  const int64_t li = ((bs / S) * Hq + h) * S + bs % S;
  const float l1 = lse1[li], l2 = lse2[li];
  const float m = __builtin_fmaxf(l1, l2);
  float w1 = 0.f, w2 = 0.f, lo = kNegInf;
  if (m > kNegInf) {
    const float e1 = __expf(l1 - m), e2 = __expf(l2 - m);  // 0 for an empty part
    const float t = e1 + e2;
    w1 = e1 / t;
    w2 = e2 / t;
    lo = m + __logf(t);
  }
  const int64_t g = r * D + c * 8;
  const f32x4 x0 = *reinterpret_cast<const f32x4 *>(o1 + g);
  const f32x4 x1 = *reinterpret_cast<const f32x4 *>(o1 + g + 4);
  const f32x4 y0 = *reinterpret_cast<const f32x4 *>(o2 + g);
  const f32x4 y1 = *reinterpret_cast<const f32x4 *>(o2 + g + 4);
  const f32x4 z0 = w1 * x0 + w2 * y0, z1 = w1 * x1 + w2 * y1;
  if constexpr (OB) {
    *reinterpret_cast<bf16x8 *>(static_cast<bf16 *>(o) + g) =
        pack8(z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]);
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + g) = z0;
    *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + g + 4) = z1;
  }
  if (c == 0) lse[li] = lo;
}

#define LCM_MERGE(D, OB)                                                                        \
  template __global__ void attn_merge_kernel<D, OB>(const float *, const float *, const float *, \
                                                    const float *, void *, float *, int, int,   \
                                                    int64_t);
LCM_MERGE(128, true)
LCM_MERGE(128, false)
LCM_MERGE(64, true)
LCM_MERGE(64, false)
#undef LCM_MERGE

hipError_t launch_merge(const float *o1, const float *lse1, const float *o2, const float *lse2,
                        void *o, bool o_bf16, float *lse, int64_t B, int S, int Hq, int d,
                        hipStream_t st) {
  const int64_t nrows = B * (int64_t)S * Hq;
  const int rpb = 256 / (d / 8);
  const dim3 grid((unsigned)((nrows + rpb - 1) / rpb)), block(256);
  if (d == 128 && o_bf16)
    hipLaunchKernelGGL((attn_merge_kernel<128, true>), grid, block, 0, st, o1, lse1, o2, lse2, o, lse, S, Hq, nrows);
  else if (d == 128)
    hipLaunchKernelGGL((attn_merge_kernel<128, false>), grid, block, 0, st, o1, lse1, o2, lse2, o, lse, S, Hq, nrows);
  else if (d == 64 && o_bf16)
    hipLaunchKernelGGL((attn_merge_kernel<64, true>), grid, block, 0, st, o1, lse1, o2, lse2, o, lse, S, Hq, nrows);
  else if (d == 64)
    hipLaunchKernelGGL((attn_merge_kernel<64, false>), grid, block, 0, st, o1, lse1, o2, lse2, o, lse, S, Hq, nrows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Every variant is instantiated explicitly: implicit instantiation from the
// launcher alone has left some host-side launch stubs unemitted.
#define LCM_FWD(D, HG)                                              \
  template __global__ void attn_fwd_kernel<D, HG, true>(FwdArgs);  \
  template __global__ void attn_fwd_kernel<D, HG, false>(FwdArgs);
LCM_FWD(128, 2)
LCM_FWD(128, 1)
LCM_FWD(64, 2)
LCM_FWD(64, 1)
#undef LCM_FWD

template <int D, int HG>
static void launch_fwd_masked(const FwdArgs &a, bool masked, dim3 grid, hipStream_t st) {
  if (masked) hipLaunchKernelGGL((attn_fwd_kernel<D, HG, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attn_fwd_kernel<D, HG, false>), grid, dim3(256), 0, st, a);
}

hipError_t launch_fwd(const FwdArgs &a, int d, int HG, bool masked, int n_items, int B,
                      hipStream_t st) {
  const dim3 grid((unsigned)n_items, (unsigned)B);
  if (d == 128 && HG == 2) launch_fwd_masked<128, 2>(a, masked, grid, st);
  else if (d == 128 && HG == 1) launch_fwd_masked<128, 1>(a, masked, grid, st);
  else if (d == 64 && HG == 2) launch_fwd_masked<64, 2>(a, masked, grid, st);
  else if (d == 64 && HG == 1) launch_fwd_masked<64, 1>(a, masked, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lcm
