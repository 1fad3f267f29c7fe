// Device side of dynamic block-sparse masks: rebuild a plan's work lists
// from a new block bitmap without going back to the host.
//
// Method: "Long-Context Attention Benchmark" review (xllm-io), paper summary,
// innovation 3 (block-sparse masks whose blocks are chosen from the input,
// so the bitmap changes every step) and section 3 "mask taxonomy" (uniform
// and variable block masks).  The mask is the plan's base mask AND the
// bitmap.  A 64x64 micro tile of mask head h is empty if its base class is
// empty or no bitmap block it touches is on, full if its base class is full
// and every block it touches is on, and partial otherwise.  A kernel tile is
// listed when some micro tile in it is non-empty for some mask head of the
// list's group, and marked partial unless all of them are full and the tile
// is whole.  These are the host compiler's rules on the same inputs (the
// base classes it stored in the plan), so the lists come out identical.
//
// One wave builds one list.  Lane l classifies tile c + l of a run of 64; a
// ballot compacts the listed tiles in order; the wave moves to the next 64.
// Where the plan lists dK/dV (Q-tile, head) stages (one bitmap per query
// head), each lane classifies its tile for every head of the group and a
// scan over the lanes places the lane's stages.
// Forward / dQ lists run over key tiles J ascending, dK/dV lists over
// Q-tiles I descending (the order the host gives them).
//
// Plans with bitmap words get a third launch that rebuilds them.
//
// A second launch puts the work items back in longest-first order, the
// order that keeps the tail of a launch short.  The item array is dealt to
// XCD shares at creation (each XCD's workgroups serve a fixed set of heads,
// so that its L2 holds their tiles); one workgroup re-sorts the items of one
// share by their new cost, 4 x tiles + partial tiles (a partial tile costs
// 1.25 full ones), ties in natural order (shares of several KV heads: by
// head first), with a bitonic sort in LDS, and
// writes them, with their new lengths, into the share's positions.  That is
// the host compiler's order whenever its deal does not depend on the costs
// (Hkv a multiple of 8, or no deal at all).
#include <algorithm>

#include "kernels.hpp"
#include "plan.hpp"

namespace lcm {

namespace {

// Class of micro tile (I, J) for mask head h; the tile's key columns touch
// bitmap column blocks [klo, khi].
__device__ __forceinline__ int micro_class(const DynArgs &a, int h, int I, int J, int klo,
                                           int khi) {
  const uint8_t b = a.base[(int64_t)I * a.nM + J];
  if (b == kEmpty) return kEmpty;
  const int r1 = min(a.S, I * kMicro + kMicro);
  const int qlo = a.qblk[I * kMicro], qhi = a.qblk[r1 - 1];
  const uint8_t *bm = a.src + (int64_t)h * a.nqb * a.nkb;
  bool any = false, all = true;
  for (int qb = qlo; qb <= qhi; ++qb)
    for (int kb = klo; kb <= khi; ++kb) {
      const bool on = bm[(int64_t)qb * a.nkb + kb] != 0;
      any |= on;
      all &= on;
    }
  return !any ? kEmpty : (all && b == kFull ? kFull : kPartial);
}

__device__ __forceinline__ int key_block_lo(const DynArgs &a, int J) { return a.kblk[J * kMicro]; }
__device__ __forceinline__ int key_block_hi(const DynArgs &a, int J) {
  return a.kblk[min(a.S, J * kMicro + kMicro) - 1];
}

// Lanes below this one whose bit is set in m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// 0/1 per byte of w: 1 where the byte is nonzero.
__device__ __forceinline__ uint32_t bytes_nonzero(uint32_t w) {
  return ((((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u) >> 7;
}

}  // namespace

__global__ __launch_bounds__(256) void attn_dyn_lists_kernel(DynArgs a) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < a.copy_blocks) {
    const int64_t n16 = a.nbits / 16, stride = (int64_t)a.copy_blocks * 256;
    const uint4 *s4 = reinterpret_cast<const uint4 *>(a.src);
    uint4 *d4 = reinterpret_cast<uint4 *>(a.bits);
    for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n16; i += stride) {
      uint4 v = s4[i];
      v.x = bytes_nonzero(v.x); v.y = bytes_nonzero(v.y);
      v.z = bytes_nonzero(v.z); v.w = bytes_nonzero(v.w);
      d4[i] = v;
    }
    for (int64_t i = n16 * 16 + (int64_t)blockIdx.x * 256 + tid; i < a.nbits; i += stride)
      a.bits[i] = a.src[i] != 0 ? 1 : 0;
    return;
  }
  const int w = ((int)blockIdx.x - a.copy_blocks) * 4 + tid / 64;
  const int lane = tid & 63;
  const int nM = a.nM;
  if (w < a.n_fslots) {
    // forward / dQ list of (group g, Q-tile qt): key tiles J ascending
    const int g = w / a.nFQ, qt = w - g * a.nFQ;
    const int I0 = qt * a.MR, I1 = min(nM, I0 + a.MR);
    uint32_t *out = a.fwd_list + (int64_t)w * nM;
    int cnt = 0, npart = 0;
    for (int c = 0; c < nM; c += 64) {
      const int J = c + lane;
      bool any = false, all = true;
      if (J < nM) {
        const int klo = key_block_lo(a, J), khi = key_block_hi(a, J);
        for (int hh = 0; hh < a.fheads; ++hh)
          for (int I = I0; I < I1; ++I) {
            const int x = micro_class(a, g * a.fheads + hh, I, J, klo, khi);
            any |= x != kEmpty;
            all &= x == kFull;
          }
      }
      const bool part = !all || (J + 1) * kFwdKeyTile > a.S;
      const uint64_t m = __ballot(any);
      if (any) out[cnt + lanes_below(m)] = (uint32_t)J | (part ? kPartialBit : 0u);
      cnt += __popcll(m);
      npart += __popcll(__ballot(any && part));
    }
    if (lane == 0) a.slot_len[w] = make_int2(cnt, npart);
  } else if (w < a.n_fslots + a.n_bslots) {
    // dK/dV list of (group g, K-tile kt): Q-tiles I descending
    const int wb = w - a.n_fslots;
    const int g = wb / a.nBK, kt = wb - g * a.nBK;
    const int J0 = kt * a.MC, J1 = min(nM, J0 + a.MC);
    uint32_t *out = a.bwd_list + (int64_t)wb * a.bcap;
    int cnt = 0, npart = 0;
    for (int c = 0; c < nM; c += 64) {
      const int I = nM - 1 - (c + lane);
      if (a.bhe) {
        // one entry per (Q-tile, head) with an allowed pair, heads ascending
        // within a Q-tile: bits of the lane's non-empty and full heads, an
        // exclusive scan of their counts over the lanes, then the writes
        uint64_t hany = 0, hfull = 0;
        if (I >= 0) {
          for (int hh = 0; hh < a.bheads; ++hh) {
            bool any = false, all = true;
            for (int J = J0; J < J1; ++J) {
              const int x = micro_class(a, g * a.bheads + hh, I, J, key_block_lo(a, J),
                                        key_block_hi(a, J));
              any |= x != kEmpty;
              all &= x == kFull;
            }
            hany |= (uint64_t)any << hh;
            hfull |= (uint64_t)(any && all) << hh;
          }
        }
        const bool ragged = (I + 1) * kBwdRowTile > a.S || (J1 - J0) < a.MC;
        if (ragged) hfull = 0;
        const int n = __popcll(hany), np = n - __popcll(hfull);
        int incl = n, pincl = np;
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(incl, d), py = __shfl_up(pincl, d);
          if (lane >= d) { incl += y; pincl += py; }
        }
        int k = cnt + incl - n;
        for (uint64_t m = hany; m; m &= m - 1) {
          const int hh = __builtin_ctzll(m);
          const bool part = ((hfull >> hh) & 1ull) == 0ull;
          out[k++] = (uint32_t)I | ((uint32_t)hh << kHeadShift) | (part ? kPartialBit : 0u);
        }
        cnt += __shfl(incl, 63);
        npart += __shfl(pincl, 63);
        continue;
      }
      bool any = false, all = true;
      if (I >= 0) {
        for (int hh = 0; hh < a.bheads; ++hh)
          for (int J = J0; J < J1; ++J) {
            const int x = micro_class(a, g * a.bheads + hh, I, J, key_block_lo(a, J),
                                      key_block_hi(a, J));
            any |= x != kEmpty;
            all &= x == kFull;
          }
      }
      const bool part = !all || (I + 1) * kBwdRowTile > a.S || (J1 - J0) < a.MC;
      const uint64_t m = __ballot(any);
      if (any) out[cnt + lanes_below(m)] = (uint32_t)I | (part ? kPartialBit : 0u);
      cnt += __popcll(m);
      npart += __popcll(__ballot(any && part));
    }
    if (lane == 0) a.slot_len[w] = make_int2(cnt, npart);
  }
}

// One workgroup per XCD share of either pass.  A share larger than
// kSortCap items keeps its items in natural order (lengths updated).
constexpr int kSortCap = 8192;
static_assert(kSortCap <= 0x10000, "share_sort_key keeps 16 bits of the natural index");
constexpr int kSortThreads = 1024;

__global__ __launch_bounds__(kSortThreads) void attn_dyn_sort_kernel(DynArgs a) {
  __shared__ uint64_t key[kSortCap];
  const int tid = threadIdx.x;
  const bool fwd = (int)blockIdx.x < a.n_fshares;
  const int c = fwd ? (int)blockIdx.x : (int)blockIdx.x - a.n_fshares;
  const int *off = fwd ? a.fshare : a.bshare;
  const int m0 = off[c], m = off[c + 1] - m0;
  const int *pos = (fwd ? a.fpos : a.bpos) + m0;
  const int4 *nat = (fwd ? a.fnat : a.bnat) + m0;
  int4 *items = fwd ? a.fitems : a.bitems;
  const int2 *len = a.slot_len + (fwd ? 0 : a.n_fslots);
  const int64_t cap = fwd ? a.nM : a.bcap;  // list capacity per slot
  if (m > kSortCap) {
    for (int i = tid; i < m; i += kSortThreads) {
      int4 it = nat[i];
      it.w = len[it.z / cap].x;
      items[pos[i]] = it;
    }
    return;
  }
  int n = 1;
  while (n < m) n <<= 1;
  // ascending order of share_sort_key: cost descending, ties in natural
  // order, or, where the share holds several KV heads, the head first (one
  // head's items together, each head's longest first: the host's order, as
  // its interleave leaves it)
  for (int i = tid; i < n; i += kSortThreads) {
    uint64_t k = ~0ull;
    if (i < m) {
      const int2 ln = len[nat[i].z / cap];
      const uint32_t cost = 4u * (uint32_t)ln.x + (uint32_t)ln.y;
      const uint32_t kvh = (uint32_t)(fwd ? nat[i].y / a.fkv : nat[i].y);
      k = share_sort_key(a.head_major != 0, kvh, cost, (uint32_t)i);
    }
    key[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n; i += kSortThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = key[i], y = key[ixj];
          if ((x > y) == ((i & k) == 0)) {
            key[i] = y;
            key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < m; i += kSortThreads) {
    int4 it = nat[share_sort_index(key[i])];
    it.w = len[it.z / cap].x;
    items[pos[i]] = it;
  }
}

// Bitmap words for the new bitmap, one thread per word: the allowed keys of
// key tile t for row block qb, [heads][nqb][nM], then the allowed rows of
// Q-tile t for key block kb, [heads][nkb][nM]; each the OR of the tile's
// block segments whose bit is on (the host's rule, on the same segments).
__global__ __launch_bounds__(256) void attn_dyn_words_kernel(DynArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nk = (int64_t)a.bm_heads * a.nqb * a.nM;
  const int64_t nr = (int64_t)a.bm_heads * a.nkb * a.nM;
  if (i < nk) {
    const int t = (int)(i % a.nM);
    const int64_t hq = i / a.nM;  // h * nqb + qb
    const uint8_t *row = a.src + hq * a.nkb;
    uint64_t w = 0;
    for (int s = a.kseg_off[t]; s < a.kseg_off[t + 1]; ++s)
      if (row[a.kseg_blk[s]]) w |= a.kseg_mask[s];
    a.kwords[i] = w;
  } else if (i < nk + nr) {
    const int64_t j = i - nk;
    const int t = (int)(j % a.nM);
    const int64_t hk = j / a.nM;  // h * nkb + kb
    const int kb = (int)(hk % a.nkb), h = (int)(hk / a.nkb);
    const uint8_t *col = a.src + (int64_t)h * a.nqb * a.nkb + kb;
    uint64_t w = 0;
    for (int s = a.rseg_off[t]; s < a.rseg_off[t + 1]; ++s)
      if (col[(int64_t)a.rseg_blk[s] * a.nkb]) w |= a.rseg_mask[s];
    a.rwords[j] = w;
  }
}

hipError_t launch_dyn(const DynArgs &a0, hipStream_t st) {
  DynArgs a = a0;
  const int64_t n16 = a.nbits / 16;
  a.copy_blocks = (int)std::max<int64_t>(1, std::min<int64_t>(256, (n16 + 255) / 256));
  const int64_t waves = (int64_t)a.n_fslots + a.n_bslots;
  const int64_t blocks = a.copy_blocks + (waves + 3) / 4;
  hipLaunchKernelGGL(attn_dyn_lists_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_dyn_sort_kernel, dim3((unsigned)(a.n_fshares + a.n_bshares)),
                     dim3(kSortThreads), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.kwords == nullptr) return e;
  const int64_t nw = (int64_t)a.bm_heads * (a.nqb + a.nkb) * a.nM;
  hipLaunchKernelGGL(attn_dyn_words_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lcm
