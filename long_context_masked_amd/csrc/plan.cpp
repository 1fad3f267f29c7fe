// Mask compiler: descriptor -> row/column bounds -> tile classes -> ordered
// work lists -> device blob.  Host only; makes no HIP call.
//
// Method sources (cited by page and section):
//  * "Long-Context Attention Benchmark" review (xllm-io), section 3 "mask
//    taxonomy" (the families) and components table (the mask generator and
//    kernel adapter that give every kernel one input representation).
//  * "FlashAttention vs. RingAttention" (dtcms), FlashAttention-2 "core
//    optimisations": Q-split forward, two-axis backward, and work
//    partitioning for load balance across thread blocks.
//
// Pipeline:
//  1. validate the shape and the descriptor;
//  2. express the base family as masked row intervals per key column
//     (col bounds, two per column) in closed form;
//  3. derive the allowed key runs of every query row (row bounds, at most two
//     per row) by a sweep over rows;
//  4. classify each 64x64 micro tile EMPTY / FULL / PARTIAL from the row
//     bounds (difference arrays), then AND in the block bitmap per mask head;
//  5. aggregate micro tiles into kernel tiles and emit per-Q-tile (forward,
//     dQ) and per-K-tile (dK/dV) lists of non-empty tiles;
//  6. order work items longest first and lay everything out in one blob.
#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <new>
#include <set>
#include <system_error>
#include <thread>

#include "plan.hpp"

namespace lcm {

static thread_local std::string g_err;

attn_status fail(attn_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

void clear_error() { g_err.clear(); }

namespace {

struct Run { int32_t a0, b0, a1, b1; };

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int32_t clamp_s(int64_t x, int64_t S) {
  return (int32_t)std::max<int64_t>(0, std::min<int64_t>(x, S));
}

attn_status check_offsets(const int32_t *off, int64_t n, int64_t S, const char *what) {
  if (!off) return fail(ATTN_ERR_INVALID, "%s is NULL", what);
  if (off[0] != 0) return fail(ATTN_ERR_INVALID, "%s[0] must be 0", what);
  for (int64_t i = 0; i < n; ++i)
    if (off[i + 1] <= off[i])
      return fail(ATTN_ERR_INVALID, "%s must be strictly increasing (at %lld)", what, (long long)i);
  if (off[n] != S)
    return fail(ATTN_ERR_INVALID, "%s must end at S=%lld (got %d)", what, (long long)S, off[n]);
  return ATTN_OK;
}

// Step 2: masked row intervals {lts, lte, uts, ute} for every key column.
attn_status build_colb(const attn_shape &sh, const attn_mask_desc &d, std::vector<int32_t> &cb) {
  const int64_t S = sh.S;
  cb.assign((size_t)S * 4, 0);
  auto put = [&](int64_t j, int64_t lts, int64_t lte, int64_t uts, int64_t ute) {
    int32_t *c = &cb[(size_t)j * 4];
    c[0] = clamp_s(lts, S); c[1] = clamp_s(lte, S);
    c[2] = clamp_s(uts, S); c[3] = clamp_s(ute, S);
  };
  switch (d.kind) {
    case ATTN_MASK_FULL:
      return ATTN_OK;
    case ATTN_MASK_CAUSAL:
      for (int64_t j = 0; j < S; ++j) put(j, 0, 0, 0, j);
      return ATTN_OK;
    case ATTN_MASK_SLIDING: {
      if (d.causal != 0 && d.causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1");
      if (d.window_left < 1) return fail(ATTN_ERR_INVALID, "window_left must be >= 1");
      if (!d.causal && d.window_right < 1)
        return fail(ATTN_ERR_INVALID, "window_right must be >= 1 when causal = 0");
      const int64_t wl = d.window_left, wr = d.window_right;
      for (int64_t j = 0; j < S; ++j) {
        // rows i >= j + wl are outside the window below the diagonal;
        // rows above the diagonal: i < j when causal, i <= j - wr otherwise.
        const int64_t up_end = d.causal ? j : std::max<int64_t>(0, j - wr + 1);
        put(j, j + wl, S, 0, up_end);
      }
      return ATTN_OK;
    }
    case ATTN_MASK_DOCUMENT:
    case ATTN_MASK_PREFIX_LM: {
      if (d.num_docs < 1) return fail(ATTN_ERR_INVALID, "num_docs must be >= 1");
      attn_status st = check_offsets(d.cu_seqlens, d.num_docs, S, "cu_seqlens");
      if (st != ATTN_OK) return st;
      const bool prefix = d.kind == ATTN_MASK_PREFIX_LM;
      if (!prefix && d.causal != 0 && d.causal != 1)
        return fail(ATTN_ERR_INVALID, "causal must be 0 or 1");
      if (prefix && !d.prefix_lens) return fail(ATTN_ERR_INVALID, "prefix_lens is NULL");
      for (int k = 0; k < d.num_docs; ++k) {
        const int64_t s = d.cu_seqlens[k], e = d.cu_seqlens[k + 1];
        int64_t p = 0;
        if (prefix) {
          p = d.prefix_lens[k];
          if (p < 0 || p > e - s)
            return fail(ATTN_ERR_INVALID, "prefix_lens[%d]=%lld outside [0, %lld]", k,
                        (long long)p, (long long)(e - s));
        }
        for (int64_t j = s; j < e; ++j) {
          // other documents are masked: rows [0, s) and [e, S);
          // inside the document, rows above the diagonal are masked unless
          // the family keeps them (full document, or a prefix key).
          int64_t up_end;
          if (prefix) up_end = (j < s + p) ? s : j;
          else up_end = d.causal ? j : s;
          put(j, e, S, 0, up_end);
        }
      }
      return ATTN_OK;
    }
    case ATTN_MASK_COLUMN_BOUNDS: {
      if (!d.col_bounds) return fail(ATTN_ERR_INVALID, "col_bounds is NULL");
      for (int64_t j = 0; j < S; ++j)
        for (int t = 0; t < 4; ++t) {
          const int32_t x = d.col_bounds[j * 4 + t];
          if (x < 0 || x > S)
            return fail(ATTN_ERR_INVALID, "col_bounds[%lld][%d]=%d outside [0, S]", (long long)j, t, x);
          cb[(size_t)j * 4 + t] = x;
        }
      return ATTN_OK;
    }
    default:
      return fail(ATTN_ERR_INVALID, "unknown mask kind %d", d.kind);
  }
}

// Step 3: allowed key runs per row.  Sweep rows top to bottom keeping, per
// column, how many masked intervals cover the current row, and the ordered
// set of positions where "allowed" changes between neighbouring columns.
attn_status rows_from_cols(int64_t S, const std::vector<int32_t> &cb, std::vector<Run> &rb,
                           int64_t &nnz) {
  std::vector<int64_t> start((size_t)S + 2, 0);
  for (int64_t j = 0; j < S; ++j)
    for (int t = 0; t < 2; ++t) {
      const int32_t a = cb[j * 4 + 2 * t], b = cb[j * 4 + 2 * t + 1];
      if (a >= b) continue;
      start[a + 1]++;
      if (b < S) start[b + 1]++;
    }
  for (int64_t i = 0; i <= S; ++i) start[i + 1] += start[i];
  std::vector<int64_t> fillp(start.begin(), start.end() - 1);
  std::vector<std::pair<int32_t, int8_t>> ev((size_t)start[S]);
  for (int64_t j = 0; j < S; ++j)
    for (int t = 0; t < 2; ++t) {
      const int32_t a = cb[j * 4 + 2 * t], b = cb[j * 4 + 2 * t + 1];
      if (a >= b) continue;
      ev[fillp[a]++] = {(int32_t)j, +1};
      if (b < S) ev[fillp[b]++] = {(int32_t)j, -1};
    }
  std::vector<int32_t> cover((size_t)S, 0);
  std::set<int32_t> edges{0, (int32_t)S};
  auto toggle = [&](int32_t p) {
    auto it = edges.find(p);
    if (it == edges.end()) edges.insert(p); else edges.erase(it);
  };
  rb.assign((size_t)S, Run{0, 0, 0, 0});
  nnz = 0;
  for (int64_t i = 0; i < S; ++i) {
    for (int64_t e = start[i]; e < start[i + 1]; ++e) {
      const int32_t j = ev[e].first;
      const bool was = cover[j] == 0;
      cover[j] += ev[e].second;
      if (was != (cover[j] == 0)) { toggle(j); toggle(j + 1); }
    }
    if (edges.size() > 4)
      return fail(ATTN_ERR_UNSUPPORTED,
                  "row %lld has %zu runs of allowed keys; at most 2 are supported",
                  (long long)i, edges.size() / 2);
    auto it = edges.begin();
    Run r{0, 0, 0, 0};
    if (edges.size() >= 2) { r.a0 = *it++; r.b0 = *it++; }
    if (edges.size() == 4) { r.a1 = *it++; r.b1 = *it++; }
    rb[i] = r;
    nnz += (r.b0 - r.a0) + (r.b1 - r.a1);
  }
  return ATTN_OK;
}

// Step 4a: micro-tile classes of the base mask from the row runs.
void classify_base(int64_t S, const std::vector<Run> &rb, std::vector<uint8_t> &cls) {
  const int64_t nM = (S + kMicro - 1) / kMicro;
  cls.assign((size_t)(nM * nM), kEmpty);
  std::vector<int32_t> full((size_t)nM + 1), touch((size_t)nM + 1);
  for (int64_t I = 0; I < nM; ++I) {
    std::fill(full.begin(), full.end(), 0);
    std::fill(touch.begin(), touch.end(), 0);
    const int64_t r0 = I * kMicro, r1 = std::min<int64_t>(S, r0 + kMicro);
    for (int64_t i = r0; i < r1; ++i) {
      const Run &r = rb[i];
      const int32_t as[2] = {r.a0, r.a1}, bs[2] = {r.b0, r.b1};
      for (int t = 0; t < 2; ++t) {
        const int64_t a = as[t], b = bs[t];
        if (a >= b) continue;
        touch[a / kMicro]++;
        touch[(b - 1) / kMicro + 1]--;
        const int64_t jlo = (a + kMicro - 1) / kMicro;
        const int64_t jhi = (b == S) ? nM - 1 : b / kMicro - 1;
        if (jlo <= jhi) { full[jlo]++; full[jhi + 1]--; }
      }
    }
    int32_t f = 0, tc = 0;
    const int32_t R = (int32_t)(r1 - r0);
    for (int64_t J = 0; J < nM; ++J) {
      f += full[J]; tc += touch[J];
      cls[I * nM + J] = tc == 0 ? kEmpty : (f == R ? kFull : kPartial);
    }
  }
}

struct Bitmap {
  int heads = 0, nqb = 0, nkb = 0;
  std::vector<uint8_t> bits;         // [heads][nqb][nkb], 0/1
  std::vector<int32_t> qoffs, koffs; // [n+1]
  std::vector<int32_t> qblk, kblk;   // block of each position [S]
};

// Step 4b: AND the bitmap of mask head hm into the base micro classes.
void classify_bitmap(int64_t S, const std::vector<uint8_t> &base, const Bitmap &bm, int hm,
                     std::vector<uint8_t> &cls) {
  const int64_t nM = (S + kMicro - 1) / kMicro;
  cls.resize(base.size());
  const uint8_t *B = bm.bits.data() + (size_t)hm * bm.nqb * bm.nkb;
  std::vector<int32_t> klo((size_t)nM), khi((size_t)nM);
  for (int64_t J = 0; J < nM; ++J) {
    klo[J] = bm.kblk[J * kMicro];
    khi[J] = bm.kblk[std::min<int64_t>(S, J * kMicro + kMicro) - 1];
  }
  for (int64_t I = 0; I < nM; ++I) {
    const int32_t qlo = bm.qblk[I * kMicro];
    const int32_t qhi = bm.qblk[std::min<int64_t>(S, I * kMicro + kMicro) - 1];
    for (int64_t J = 0; J < nM; ++J) {
      const uint8_t b = base[I * nM + J];
      if (b == kEmpty) { cls[I * nM + J] = kEmpty; continue; }
      bool any = false, all = true;
      for (int32_t qb = qlo; qb <= qhi; ++qb)
        for (int32_t kb = klo[J]; kb <= khi[J]; ++kb) {
          const bool on = B[(size_t)qb * bm.nkb + kb] != 0;
          any |= on; all &= on;
        }
      cls[I * nM + J] = !any ? kEmpty : (all && b == kFull ? kFull : kPartial);
    }
  }
}

// Exact allowed-pair count of base AND bitmap head hm.
int64_t nnz_with_bitmap(int64_t S, const std::vector<Run> &rb, const Bitmap &bm, int hm) {
  const uint8_t *B = bm.bits.data() + (size_t)hm * bm.nqb * bm.nkb;
  std::vector<int64_t> C((size_t)bm.nkb + 1);
  int64_t tot = 0;
  for (int32_t qb = 0; qb < bm.nqb; ++qb) {
    C[0] = 0;
    for (int32_t kb = 0; kb < bm.nkb; ++kb)
      C[kb + 1] = C[kb] + (B[(size_t)qb * bm.nkb + kb] ? bm.koffs[kb + 1] - bm.koffs[kb] : 0);
    // P(x) = allowed-by-bitmap keys in [0, x) for a row of block qb
    auto P = [&](int64_t x) -> int64_t {
      if (x >= S) return C[bm.nkb];
      const int32_t kb = bm.kblk[x];
      return C[kb] + (B[(size_t)qb * bm.nkb + kb] ? x - bm.koffs[kb] : 0);
    };
    for (int64_t i = bm.qoffs[qb]; i < bm.qoffs[qb + 1]; ++i) {
      const Run &r = rb[i];
      if (r.b0 > r.a0) tot += P(r.b0) - P(r.a0);
      if (r.b1 > r.a1) tot += P(r.b1) - P(r.a1);
    }
  }
  return tot;
}

struct Item { int32_t tile, head, off, len; double cost; };

// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin in
// launch order, so item b runs on XCD b % 8.  Items of one KV head stream
// the same K/V (forward, dQ) or Q/dO (dK/dV) tiles; giving each XCD the items
// of as few KV heads as possible lets its L2 serve those tiles to all of its
// workgroups.  v is in longest-first order.  When Hkv is a multiple of 8,
// XCD x takes the heads h with h % 8 == x; when Hkv divides 8, each head's
// items go to the least-loaded of the XCDs congruent to it modulo Hkv (the
// longest-processing-time rule within that set).  Otherwise the order is
// left as it is.  Each XCD's share stays in longest-first order, except that
// a share of several KV heads (Hkv > 8) runs one head's items after another,
// each head's longest first: the workgroups then in flight on the XCD walk
// the tiles of one head together.  With the share's heads mixed (MHA, a
// random bitmap per head) L2 served a third of the forward's K/V tiles and
// the rest came from HBM at two thirds of its bandwidth.  If `cls`
// is given it receives the XCD share (0 when the order is left) of every
// position of the result.
constexpr int kXcds = 8;
// The share sort's key layouts give back the natural index, and order as
// the host does: by KV head first where asked, then cost descending, then
// natural index.
static_assert(share_sort_index(share_sort_key(true, 13, 0xfffffffeu, 8191)) == 8191, "index, head-major");
static_assert(share_sort_index(share_sort_key(false, 13, 0xfffffffeu, 8191)) == 8191, "index");
static_assert(share_sort_key(true, 1, 9, 0) < share_sort_key(true, 2, 99, 0), "head first");
static_assert(share_sort_key(true, 1, 99, 5) < share_sort_key(true, 1, 9, 0), "cost descending");
static_assert(share_sort_key(false, 7, 99, 5) < share_sort_key(false, 1, 9, 0), "cost descending");
static_assert(share_sort_key(true, 1, 9, 3) < share_sort_key(true, 1, 9, 4), "natural order on ties");
void xcd_interleave(std::vector<Item> &v, int64_t Hkv, int64_t heads_per_kv,
                    std::vector<int32_t> *cls = nullptr) {
  const bool by_mod = Hkv % kXcds == 0;
  const bool spread = kXcds % Hkv == 0;
  if (!by_mod && !spread) {
    if (cls) cls->assign(v.size(), 0);
    return;
  }
  std::vector<std::vector<Item>> q(kXcds);
  std::vector<double> load(kXcds, 0.0);
  for (const Item &x : v) {
    const int64_t kvh = x.head / heads_per_kv;
    int64_t slot = kvh % kXcds;
    if (!by_mod) {
      for (int64_t c = kvh; c < kXcds; c += Hkv)
        if (load[(size_t)c] < load[(size_t)slot]) slot = c;
    }
    q[(size_t)slot].push_back(x);
    load[(size_t)slot] += x.cost;
  }
  if (by_mod && Hkv > kXcds)
    for (auto &share : q)
      std::stable_sort(share.begin(), share.end(), [&](const Item &a, const Item &b) {
        return a.head / heads_per_kv < b.head / heads_per_kv;
      });
  v.clear();
  if (cls) cls->clear();
  for (size_t i = 0;; ++i) {
    bool any = false;
    for (int x = 0; x < kXcds; ++x)
      if (i < q[x].size()) {
        v.push_back(q[x][i]);
        if (cls) cls->push_back(x);
        any = true;
      }
    if (!any) break;
  }
}

// The reorder tables of one pass of a dynamic plan: for each XCD share c,
// its item positions (ascending) at pos[off[c] .. off[c+1]) and its items in
// natural order at nat[off[c] ..).  The device sorts each share's items by
// their new cost and writes them back into the share's positions.
void share_tables(const std::vector<Item> &v, const std::vector<int32_t> &cls,
                  const std::vector<int64_t> &natural, std::vector<int32_t> &off,
                  std::vector<int32_t> &pos, std::vector<std::array<int32_t, 4>> &nat) {
  int32_t nc = 1;
  for (int32_t c : cls) nc = std::max(nc, c + 1);
  off.assign((size_t)nc + 1, 0);
  for (int32_t c : cls) off[(size_t)c + 1]++;
  for (int32_t c = 0; c < nc; ++c) off[(size_t)c + 1] += off[(size_t)c];
  std::vector<int32_t> fill(off.begin(), off.end() - 1);
  pos.assign(v.size(), 0);
  for (size_t p = 0; p < v.size(); ++p) pos[(size_t)fill[(size_t)cls[p]]++] = (int32_t)p;
  nat.assign(v.size(), {0, 0, 0, 0});
  for (int32_t c = 0; c < nc; ++c) {
    std::vector<int32_t> mem(pos.begin() + off[(size_t)c], pos.begin() + off[(size_t)c + 1]);
    std::stable_sort(mem.begin(), mem.end(),
                     [&](int32_t a, int32_t b) { return natural[(size_t)a] < natural[(size_t)b]; });
    for (size_t i = 0; i < mem.size(); ++i) {
      const Item &x = v[(size_t)mem[i]];
      nat[(size_t)off[(size_t)c] + i] = {x.tile, x.head, x.off, x.len};
    }
  }
}

}  // namespace
}  // namespace lcm

using namespace lcm;

extern "C" const char *attn_last_error(void) { return g_err.c_str(); }

extern "C" const char *attn_version(void) { return "long_context_masked_amd 0.1 (gfx950)"; }

// Host threads for plan compilation: the cores the process may use, at most
// 16 (the work units are mask heads or KV heads, and a plan's memory grows
// with the threads' scratch).
static int host_threads() {
  const unsigned hw = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(hw == 0 ? 1u : hw, 16u));
}

// f(i) for i in [0, n), on up to host_threads() threads (the caller's
// included); each thread first builds its own scratch with make().  Returns
// false if an allocation failed (the remaining work is then skipped).
template <class Make, class F>
static bool parallel_for(int n, Make make, F f) {
  const int n_threads = std::max(1, std::min(n, host_threads()));
  std::atomic<int> next{0};
  std::atomic<bool> oom{false};
  auto worker = [&]() {
    try {
      auto scratch = make();
      for (int i = next++; i < n && !oom; i = next++) f(i, scratch);
    } catch (const std::bad_alloc &) {
      oom = true;
    }
  };
  std::vector<std::thread> pool;
  try {
    for (int t = 1; t < n_threads; ++t) pool.emplace_back(worker);
  } catch (const std::system_error &) {
    // fewer threads: the ones started and the caller share the work
  }
  worker();
  for (auto &t : pool) t.join();
  return !oom;
}

static attn_status plan_create_impl(const attn_shape *shp, const attn_mask_desc *desc,
                                    attn_plan **out) {
  if (!shp || !desc || !out) return fail(ATTN_ERR_INVALID, "NULL argument");
  *out = nullptr;
  const attn_shape sh = *shp;
  if (sh.B < 1 || sh.S < 1 || sh.Hq < 1 || sh.Hkv < 1)
    return fail(ATTN_ERR_INVALID, "B, S, Hq, Hkv must be >= 1");
  if (sh.S >= (int64_t(1) << 30)) return fail(ATTN_ERR_UNSUPPORTED, "S must be < 2^30");
  if (sh.Hq % sh.Hkv) return fail(ATTN_ERR_INVALID, "Hq must be a multiple of Hkv");
  if (sh.Hq > 65535 || sh.B > 65535) return fail(ATTN_ERR_UNSUPPORTED, "Hq and B must be <= 65535");
  if (sh.d != 64 && sh.d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%lld (supported: 64, 128)", (long long)sh.d);
  if (!std::isfinite(sh.scale) || sh.scale < 0.f) return fail(ATTN_ERR_INVALID, "scale must be finite and >= 0");
  const int64_t S = sh.S;
  const int G = (int)(sh.Hq / sh.Hkv);

  // bitmap
  Bitmap bm;
  const bool has_bm = desc->block_bitmap != nullptr;
  if (desc->dynamic != 0 && desc->dynamic != 1) return fail(ATTN_ERR_INVALID, "dynamic must be 0 or 1");
  const bool dynamic = desc->dynamic == 1;
  if (dynamic && !has_bm) return fail(ATTN_ERR_INVALID, "dynamic = 1 needs a block_bitmap");
  const int want_keys = desc->bwd_key_tile;
  if (want_keys != 0 && want_keys != 64 && want_keys != 128)
    return fail(ATTN_ERR_INVALID, "bwd_key_tile must be 0, 64 or 128");
  if (has_bm) {
    const int nh = desc->bitmap_heads;
    if (nh != 1 && nh != sh.Hkv && nh != sh.Hq)
      return fail(ATTN_ERR_INVALID, "bitmap_heads must be 1, Hkv or Hq");
    if (desc->n_qblk < 1 || desc->n_kblk < 1) return fail(ATTN_ERR_INVALID, "n_qblk, n_kblk must be >= 1");
    attn_status st = check_offsets(desc->q_blk_offsets, desc->n_qblk, S, "q_blk_offsets");
    if (st != ATTN_OK) return st;
    st = check_offsets(desc->k_blk_offsets, desc->n_kblk, S, "k_blk_offsets");
    if (st != ATTN_OK) return st;
    bm.heads = nh; bm.nqb = desc->n_qblk; bm.nkb = desc->n_kblk;
    const size_t nb = (size_t)nh * bm.nqb * bm.nkb;
    bm.bits.resize(nb);
    for (size_t t = 0; t < nb; ++t) bm.bits[t] = desc->block_bitmap[t] ? 1 : 0;
    bm.qoffs.assign(desc->q_blk_offsets, desc->q_blk_offsets + bm.nqb + 1);
    bm.koffs.assign(desc->k_blk_offsets, desc->k_blk_offsets + bm.nkb + 1);
    bm.qblk.resize((size_t)S); bm.kblk.resize((size_t)S);
    for (int32_t b = 0; b < bm.nqb; ++b)
      for (int32_t x = bm.qoffs[b]; x < bm.qoffs[b + 1]; ++x) bm.qblk[x] = b;
    for (int32_t b = 0; b < bm.nkb; ++b)
      for (int32_t x = bm.koffs[b]; x < bm.koffs[b + 1]; ++x) bm.kblk[x] = b;
  }

  std::vector<int32_t> colb;
  attn_status st = build_colb(sh, *desc, colb);
  if (st != ATTN_OK) return st;
  std::vector<Run> rowb;
  int64_t nnz_base = 0;
  st = rows_from_cols(S, colb, rowb, nnz_base);
  if (st != ATTN_OK) return st;
  std::vector<uint8_t> base;
  classify_base(S, rowb, base);

  auto *p = new attn_plan();
  p->shape = sh;
  p->scale = sh.scale > 0.f ? sh.scale : (float)(1.0 / std::sqrt((double)sh.d));
  p->G = G;
  // Two query heads per forward / dQ item under GQA share each staged K/V
  // tile; with one bitmap per query head an item's list would be the union
  // of its heads' lists, so there an item takes one head (128 rows).
  const bool per_qhead = has_bm && bm.heads == sh.Hq && G > 1;
  p->HG = (G % 2 == 0 && !per_qhead) ? 2 : 1;
  p->fwd_rows = kWgRowsHeads / p->HG;
  p->bitmap_heads = has_bm ? bm.heads : 0;
  p->nqb = bm.nqb; p->nkb = bm.nkb;

  const int64_t nM = (S + kMicro - 1) / kMicro;
  const int MR = p->fwd_rows / kMicro;                     // micro rows per fwd tile
  const int64_t nFQ = (S + p->fwd_rows - 1) / p->fwd_rows;  // fwd Q tiles
  const int n_mask_heads = has_bm ? bm.heads : 1;
  auto hm_of = [&](int64_t h) -> int {
    if (!has_bm || bm.heads == 1) return 0;
    if (bm.heads == sh.Hkv) return (int)(h / G);
    return (int)h;
  };
  // Keys per dK/dV item.  A 128-key item runs both 64-key halves of every
  // listed Q-tile; where one half is empty (bitmap blocks 64 keys wide) its
  // products are masked work.  Narrow 64-key items skip such halves at the
  // price of fetching each Q/dO tile for 64 keys instead of 128, so the
  // plan takes them when, on the mask heads of the first dK/dV item group,
  // more than a quarter of the listed 128-key stages have an empty half.  A
  // dynamic plan decides on its creation bitmap: the block geometry, which
  // makes the halves empty, stays when the bits change.
  p->bwd_keys = kBwdKeyTile;
  if (want_keys != 0) {
    p->bwd_keys = want_keys;
  } else if (has_bm && nM > 1) {
    std::vector<std::vector<uint8_t>> cls0(per_qhead ? (size_t)G : 1);
    for (size_t g = 0; g < cls0.size(); ++g) classify_bitmap(S, base, bm, (int)g, cls0[g]);
    int64_t listed = 0, half = 0;
    for (int64_t I = 0; I < nM; ++I)
      for (int64_t J = 0; J + 1 < nM; J += 2) {
        bool a0 = false, a1 = false;
        for (const auto &c : cls0) {
          a0 |= c[(size_t)(I * nM + J)] != kEmpty;
          a1 |= c[(size_t)(I * nM + J + 1)] != kEmpty;
        }
        listed += a0 || a1;
        half += a0 != a1;
      }
    if (4 * half > listed) p->bwd_keys = 64;
  }
  // With one bitmap per query head, a dK/dV list of Q-tiles shared by the
  // group would run every head of a tile that any head sees; such plans list
  // (Q-tile, head) stages instead.
  p->bwd_head_entries = per_qhead && G <= (dynamic ? kMaxDynEntryHeads : kMaxEntryHeads);
  const int GE = p->bwd_head_entries ? 1 : G;                // stages per list entry
  const int MC = p->bwd_keys / kMicro;                       // micro cols per bwd tile
  const int64_t nBK = (S + p->bwd_keys - 1) / p->bwd_keys;  // bwd K tiles
  // Work lists are built per list group: the mask heads one work item covers.
  // With one bitmap per query head under GQA, a forward item covers the HG
  // mask heads of its query heads and a dK/dV item the G heads of its KV
  // head; a tile is listed if any of them allows a pair in it, and full only
  // if it is full for all of them (the kernels mask per query head).
  // Otherwise every item covers a single mask head and a group is that head.
  const int n_fgroups = per_qhead ? (int)(sh.Hq / p->HG) : n_mask_heads;
  const int n_bgroups = per_qhead ? (int)sh.Hkv : n_mask_heads;
  auto fgroup_of = [&](int64_t h0) -> int { return per_qhead ? (int)(h0 / p->HG) : hm_of(h0); };
  auto bgroup_of = [&](int64_t kvh) -> int { return per_qhead ? (int)kvh : hm_of(kvh * G); };

  std::vector<uint32_t> fwd_list, bwd_list;
  std::vector<int64_t> fwd_off((size_t)n_fgroups * nFQ), bwd_off((size_t)n_bgroups * nBK);
  std::vector<int32_t> fwd_len(fwd_off.size()), bwd_len(bwd_off.size());
  std::vector<int32_t> fwd_npart(fwd_off.size()), bwd_npart(bwd_off.size());
  std::vector<int64_t> nnz_head((size_t)n_mask_heads, nnz_base);
  // Tile class of a union over the mask heads `hs` (classifications in C):
  // bit 0 = some pair allowed, bit 1 = every pair allowed.
  // Offsets are relative to the lists passed in (one mask head's, or one KV
  // head's); the caller concatenates them in head order.
  auto lists_for = [&](const std::vector<const std::vector<uint8_t> *> &C, int64_t fslot0,
                       bool do_fwd, int64_t bslot0, bool do_bwd, std::vector<uint32_t> &fwd_list,
                       std::vector<uint32_t> &bwd_list) {
    if (do_fwd)
      for (int64_t qt = 0; qt < nFQ; ++qt) {
        const size_t slot = (size_t)(fslot0 + qt);
        fwd_off[slot] = (int64_t)fwd_list.size();
        int32_t npart = 0;
        const int64_t I0 = qt * MR, I1 = std::min<int64_t>(nM, I0 + MR);
        for (int64_t J = 0; J < nM; ++J) {
          bool any = false, all = true;
          for (const auto *c : C)
            for (int64_t I = I0; I < I1; ++I) {
              const uint8_t x = (*c)[I * nM + J];
              any |= x != kEmpty; all &= x == kFull;
            }
          if (!any) continue;
          const bool ragged = (J + 1) * kFwdKeyTile > S;
          const bool part = !all || ragged;
          npart += part;
          fwd_list.push_back((uint32_t)J | (part ? kPartialBit : 0u));
        }
        fwd_len[slot] = (int32_t)(fwd_list.size() - fwd_off[slot]);
        fwd_npart[slot] = npart;
      }
    if (do_bwd)
      for (int64_t kt = 0; kt < nBK; ++kt) {
        const size_t slot = (size_t)(bslot0 + kt);
        bwd_off[slot] = (int64_t)bwd_list.size();
        int32_t npart = 0;
        const int64_t J0 = kt * MC, J1 = std::min<int64_t>(nM, J0 + MC);
        for (int64_t I = 0; I < nM; ++I) {
          const bool ragged = (I + 1) * kBwdRowTile > S || (J1 - J0) < MC;
          if (p->bwd_head_entries) {
            // one stage per (Q-tile, query head) that has an allowed pair;
            // heads in descending order, so that the reversal below leaves
            // them ascending within a Q-tile
            for (size_t g = C.size(); g-- > 0;) {
              bool any = false, all = true;
              for (int64_t J = J0; J < J1; ++J) {
                const uint8_t x = (*C[g])[I * nM + J];
                any |= x != kEmpty; all &= x == kFull;
              }
              if (!any) continue;
              const bool part = !all || ragged;
              npart += part;
              bwd_list.push_back((uint32_t)I | ((uint32_t)g << kHeadShift) | (part ? kPartialBit : 0u));
            }
            continue;
          }
          bool any = false, all = true;
          for (const auto *c : C)
            for (int64_t J = J0; J < J1; ++J) {
              const uint8_t x = (*c)[I * nM + J];
              any |= x != kEmpty; all &= x == kFull;
            }
          if (!any) continue;
          const bool part = !all || ragged;
          npart += part;
          bwd_list.push_back((uint32_t)I | (part ? kPartialBit : 0u));
        }
        // Descending Q-tile order: the items of a K-tile band that run at once
        // then all start from the last Q-tiles (which every lower-triangular or
        // banded mask shares) and move down together, so the Q/dO tiles they
        // stream are fetched once per L2.
        std::reverse(bwd_list.begin() + bwd_off[slot], bwd_list.end());
        bwd_len[slot] = (int32_t)(bwd_list.size() - bwd_off[slot]);
        bwd_npart[slot] = npart;
      }
  };
  // Work units: one KV head (one bitmap per query head: its G
  // classifications, its forward groups and its dK/dV group) or one mask
  // head.  Units are independent; each builds its own lists, on as many host
  // threads as there are cores, and the lists are then joined in unit order,
  // so the plan does not depend on the thread count.
  const int n_units = per_qhead ? (int)sh.Hkv : n_mask_heads;
  std::vector<std::vector<uint32_t>> unit_f((size_t)n_units), unit_b((size_t)n_units);
  auto run_unit = [&](int u, std::vector<std::vector<uint8_t>> &cls) {
    if (per_qhead) {
      const int64_t kvh = u;
      for (int g = 0; g < G; ++g) {
        const int hm = (int)(kvh * G + g);
        classify_bitmap(S, base, bm, hm, cls[(size_t)g]);
        nnz_head[(size_t)hm] = nnz_with_bitmap(S, rowb, bm, hm);
      }
      for (int g0 = 0; g0 < G; g0 += p->HG) {
        std::vector<const std::vector<uint8_t> *> C;
        for (int g = g0; g < g0 + p->HG; ++g) C.push_back(&cls[(size_t)g]);
        lists_for(C, (int64_t)fgroup_of(kvh * G + g0) * nFQ, true, 0, false, unit_f[(size_t)u],
                  unit_b[(size_t)u]);
      }
      std::vector<const std::vector<uint8_t> *> C;
      for (int g = 0; g < G; ++g) C.push_back(&cls[(size_t)g]);
      lists_for(C, 0, false, (int64_t)bgroup_of(kvh) * nBK, true, unit_f[(size_t)u], unit_b[(size_t)u]);
    } else {
      const int hm = u;
      const std::vector<uint8_t> *C = &base;
      if (has_bm) {
        classify_bitmap(S, base, bm, hm, cls[0]);
        C = &cls[0];
        nnz_head[(size_t)hm] = nnz_with_bitmap(S, rowb, bm, hm);
      }
      lists_for({C}, (int64_t)hm * nFQ, true, (int64_t)hm * nBK, true, unit_f[(size_t)u],
                unit_b[(size_t)u]);
    }
  };
  if (!parallel_for(n_units, [&]() { return std::vector<std::vector<uint8_t>>(per_qhead ? (size_t)G : 1); },
                    run_unit)) {
    delete p;
    return fail(ATTN_ERR_NOMEM, "host work lists");
  }
  // Join the units' lists in unit order: a unit owns the forward slots of its
  // list groups and the dK/dV slots of its group.
  {
    const int64_t fpu = (int64_t)n_fgroups / n_units * nFQ, bpu = (int64_t)n_bgroups / n_units * nBK;
    size_t nf = 0, nb = 0;
    for (int u = 0; u < n_units; ++u) { nf += unit_f[(size_t)u].size(); nb += unit_b[(size_t)u].size(); }
    try {
      fwd_list.reserve(nf);
      bwd_list.reserve(nb);
    } catch (const std::bad_alloc &) {
      delete p;
      return fail(ATTN_ERR_NOMEM, "host work lists");
    }
    for (int u = 0; u < n_units; ++u) {
      const int64_t f0 = (int64_t)fwd_list.size(), b0 = (int64_t)bwd_list.size();
      for (int64_t sl = u * fpu; sl < (u + 1) * fpu; ++sl) fwd_off[(size_t)sl] += f0;
      for (int64_t sl = u * bpu; sl < (u + 1) * bpu; ++sl) bwd_off[(size_t)sl] += b0;
      fwd_list.insert(fwd_list.end(), unit_f[(size_t)u].begin(), unit_f[(size_t)u].end());
      bwd_list.insert(bwd_list.end(), unit_b[(size_t)u].begin(), unit_b[(size_t)u].end());
      std::vector<uint32_t>().swap(unit_f[(size_t)u]);
      std::vector<uint32_t>().swap(unit_b[(size_t)u]);
    }
  }
  if (dynamic) {
    // Every list gets room for all tiles of its row or column (dK/dV
    // (Q-tile, head) lists: for every stage), at slot * capacity, so that the
    // device can rebuild any list in place.
    const int64_t nfs = (int64_t)n_fgroups * nFQ, nbs = (int64_t)n_bgroups * nBK;
    const int64_t bcap = p->bwd_head_entries ? nM * G : nM;
    if (nfs * nM > 0x7fffffff || nbs * bcap > 0x7fffffff) {
      delete p;
      return fail(ATTN_ERR_UNSUPPORTED, "dynamic work lists would exceed 2^31 entries");
    }
    auto widen = [&](std::vector<uint32_t> &list, std::vector<int64_t> &offs,
                     const std::vector<int32_t> &lens, int64_t cap) {
      std::vector<uint32_t> w((size_t)(offs.size() * cap), 0u);
      for (size_t sl = 0; sl < offs.size(); ++sl) {
        std::copy(list.begin() + offs[sl], list.begin() + offs[sl] + lens[sl],
                  w.begin() + (int64_t)sl * cap);
        offs[sl] = (int64_t)sl * cap;
      }
      list.swap(w);
    };
    widen(fwd_list, fwd_off, fwd_len, nM);
    widen(bwd_list, bwd_off, bwd_len, bcap);
    DynInfo &D = p->dyn;
    D.on = true;
    D.nM = nM; D.nFQ = nFQ; D.nBK = nBK;
    D.n_fslots = nfs; D.n_bslots = nbs;
    D.MR = MR; D.MC = MC;
    D.fheads = per_qhead ? p->HG : 1;
    D.bheads = per_qhead ? G : 1;
    D.bhe = p->bwd_head_entries;
    D.bcap = bcap;
    D.head_major = sh.Hkv % kXcds == 0 && sh.Hkv > kXcds;
    D.fkv = G;
  }
  if (fwd_list.size() > 0x7fffffffu || bwd_list.size() > 0x7fffffffu) {
    delete p;
    return fail(ATTN_ERR_UNSUPPORTED, "work lists exceed 2^31 entries");
  }

  // Step 6: items and longest-first order.  A partial tile costs more than a
  // full one (per-element masking); an item also pays a fixed epilogue.
  const double kPartCost = 1.25, kItemCost = 0.75;
  std::vector<Item> fi, bi;
  for (int64_t h0 = 0; h0 < sh.Hq; h0 += p->HG) {
    const int fg = fgroup_of(h0);
    for (int64_t qt = 0; qt < nFQ; ++qt) {
      const size_t slot = (size_t)fg * nFQ + qt;
      const int32_t len = fwd_len[slot], np = fwd_npart[slot];
      fi.push_back({(int32_t)qt, (int32_t)h0, (int32_t)fwd_off[slot], len,
                    (len - np) + kPartCost * np + kItemCost});
    }
  }
  for (int64_t kvh = 0; kvh < sh.Hkv; ++kvh) {
    const int bg = bgroup_of(kvh);
    for (int64_t kt = 0; kt < nBK; ++kt) {
      const size_t slot = (size_t)bg * nBK + kt;
      const int32_t len = bwd_len[slot], np = bwd_npart[slot];
      bi.push_back({(int32_t)kt, (int32_t)kvh, (int32_t)bwd_off[slot], len,
                    GE * ((len - np) + kPartCost * np) + kItemCost});
    }
  }
  auto by_cost = [](const Item &a, const Item &b) { return a.cost > b.cost; };
  std::stable_sort(fi.begin(), fi.end(), by_cost);
  std::stable_sort(bi.begin(), bi.end(), by_cost);

  // Step 7: split dK/dV items that cost more than the launch's share per
  // workgroup (total / kSplitTarget) into up to kSplitMax chunks, each a run
  // of consecutive listed Q-tiles (all query heads of the group), so that no
  // single workgroup outlasts the rest (small S, or key columns that every
  // row sees).  A chunk is an item of its own over a slice of the item's
  // list, and gets a partial-result slot; slots follow list order.  Items of
  // a dynamic plan are never split: their lists change after creation.
  std::vector<int32_t> slot_of;
  std::vector<std::array<int32_t, 4>> reduce;
  std::vector<int32_t> fcls, bcls;  // XCD share of each item position
  {
    double total = 0.0;
    for (const Item &x : bi) total += x.cost;
    // two narrow workgroups are resident per CU
    const double share = total * (double)sh.B / (kSplitTarget * (kBwdKeyTile / p->bwd_keys));
    std::vector<Item> split;
    std::vector<int32_t> sl;
    int32_t slots = 0;
    for (const Item &x : bi) {
      int32_t n = 1;
      if (!dynamic && x.cost * (double)sh.B > share && x.len > 1)
        n = (int32_t)std::min<double>({(double)kSplitMax, (double)x.len,
                                       std::ceil(x.cost * (double)sh.B / share)});
      if (n <= 1) {
        split.push_back(x);
        sl.push_back(-1);
        continue;
      }
      reduce.push_back({x.tile, x.head, slots, n});
      for (int32_t c = 0; c < n; ++c) {
        const int32_t a0 = (int32_t)((int64_t)c * x.len / n), a1 = (int32_t)((int64_t)(c + 1) * x.len / n);
        int32_t np = 0;
        for (int32_t e = a0; e < a1; ++e) np += (bwd_list[(size_t)x.off + e] & kPartialBit) != 0;
        const int32_t len = a1 - a0;
        split.push_back({x.tile, x.head, x.off + a0, len, GE * ((len - np) + kPartCost * np) + kItemCost});
        sl.push_back(slots + c);
      }
      slots += n;
    }
    // longest first again, chunks included; the slot follows its item
    std::vector<size_t> idx(split.size());
    for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
    std::stable_sort(idx.begin(), idx.end(),
                     [&](size_t a, size_t b) { return split[a].cost > split[b].cost; });
    bi.clear();
    for (size_t i : idx) {
      Item y = split[i];
      y.off = (int32_t)i;  // carried through the interleave; replaced below
      bi.push_back(y);
    }
    p->n_slots = slots;
    xcd_interleave(fi, sh.Hkv, G, &fcls);  // forward items carry their first query head
    xcd_interleave(bi, sh.Hkv, 1, &bcls);  // dK/dV items carry their KV head
    for (Item &y : bi) {
      const size_t i = (size_t)y.off;
      y.off = split[i].off;
      slot_of.push_back(sl[i]);
    }
  }

  // blob layout
  Layout &L = p->lay;
  int64_t off = 0;
  auto sect = [&](int64_t bytes) { const int64_t o = off; off = align256(off + bytes); return o; };
  L.rowb = sect(S * 16);
  L.colb = sect(S * 16);
  L.n_fwd_items = (int64_t)fi.size();
  L.fwd_items = sect(L.n_fwd_items * 16);
  L.n_fwd_list = (int64_t)fwd_list.size();
  L.fwd_list = sect(std::max<int64_t>(1, L.n_fwd_list) * 4);
  L.n_bwd_items = (int64_t)bi.size();
  L.bwd_items = sect(L.n_bwd_items * 16);
  L.n_bwd_list = (int64_t)bwd_list.size();
  L.bwd_list = sect(std::max<int64_t>(1, L.n_bwd_list) * 4);
  L.bwd_slot = sect(std::max<int64_t>(1, L.n_bwd_items) * 4);
  L.n_bwd_reduce = (int64_t)reduce.size();
  L.bwd_reduce = sect(std::max<int64_t>(1, L.n_bwd_reduce) * 16);
  L.n_slots = p->n_slots;
  if (has_bm) {
    L.bits = sect((int64_t)bm.bits.size());
    L.qblk = sect(S * 4);
    L.kblk = sect(S * 4);
    L.qoffs = sect((int64_t)(bm.nqb + 1) * 4);
    L.koffs = sect((int64_t)(bm.nkb + 1) * 4);
  }
  // Bitmap words of plans whose blocks cut tiles: the mask of a partial tile
  // then costs the kernels one 8-byte load per lane instead of a walk over
  // the blocks the tile touches.  A dynamic plan also keeps each tile's block
  // segments, from which the device rebuilds the words for a new bitmap.
  bool words = false;
  struct Seg { int32_t blk; uint64_t mask; };
  std::vector<std::vector<Seg>> kseg, qseg;
  int64_t n_kseg = 0, n_qseg = 0;
  if (has_bm) {
    bool cut = false;
    for (int64_t t = 0; t < nM && !cut; ++t) {
      const int64_t a = t * kMicro, e = std::min<int64_t>(S, a + kMicro) - 1;
      cut = bm.kblk[(size_t)a] != bm.kblk[(size_t)e] || bm.qblk[(size_t)a] != bm.qblk[(size_t)e];
    }
    const int64_t bytes = (int64_t)bm.heads * (bm.nqb + bm.nkb) * nM * 8;
    words = cut && bytes <= kMaxMaskWordBytes;
    if (words) {
      L.kwords = sect((int64_t)bm.heads * bm.nqb * nM * 8);
      L.rwords = sect((int64_t)bm.heads * bm.nkb * nM * 8);
      // The blocks a 64-wide tile touches, each with the bits of the tile it
      // covers: word(tile, block line) = OR of the segments whose bitmap bit
      // is on.
      auto segments = [&](const std::vector<int32_t> &blk_of, const std::vector<int32_t> &offs,
                          int64_t &count) {
        std::vector<std::vector<Seg>> out((size_t)nM);
        for (int64_t t = 0; t < nM; ++t) {
          const int64_t a = t * kMicro, e = std::min<int64_t>(S, a + kMicro);
          for (int32_t b = blk_of[(size_t)a]; b <= blk_of[(size_t)(e - 1)]; ++b) {
            const int64_t lo = std::max<int64_t>(offs[(size_t)b], a) - a;
            const int64_t hi = std::min<int64_t>(offs[(size_t)b + 1], e) - a;
            const uint64_t top = hi == 64 ? ~0ull : ((1ull << hi) - 1ull);
            out[(size_t)t].push_back({b, top & ~((1ull << lo) - 1ull)});
            ++count;
          }
        }
        return out;
      };
      kseg = segments(bm.kblk, bm.koffs, n_kseg);
      qseg = segments(bm.qblk, bm.qoffs, n_qseg);
      if (dynamic) {
        L.dyn_kseg_off = sect((nM + 1) * 4);
        L.dyn_kseg_blk = sect(n_kseg * 4);
        L.dyn_kseg_mask = sect(n_kseg * 8);
        L.dyn_rseg_off = sect((nM + 1) * 4);
        L.dyn_rseg_blk = sect(n_qseg * 4);
        L.dyn_rseg_mask = sect(n_qseg * 8);
      }
    }
  }
  std::vector<int32_t> fsh_off, fsh_pos, bsh_off, bsh_pos;
  std::vector<std::array<int32_t, 4>> fsh_nat, bsh_nat;
  if (dynamic) {
    // natural order: forward (query-head group, Q-tile), dK/dV (KV head, K-tile)
    std::vector<int64_t> fn(fi.size()), bn(bi.size());
    for (size_t i = 0; i < fi.size(); ++i) fn[i] = (int64_t)(fi[i].head / p->HG) * nFQ + fi[i].tile;
    for (size_t i = 0; i < bi.size(); ++i) bn[i] = (int64_t)bi[i].head * nBK + bi[i].tile;
    share_tables(fi, fcls, fn, fsh_off, fsh_pos, fsh_nat);
    share_tables(bi, bcls, bn, bsh_off, bsh_pos, bsh_nat);
    p->dyn.n_fshares = (int)fsh_off.size() - 1;
    p->dyn.n_bshares = (int)bsh_off.size() - 1;
    L.dyn_base = sect(nM * nM);
    L.dyn_len = sect((p->dyn.n_fslots + p->dyn.n_bslots) * 8);
    L.dyn_fshare = sect((int64_t)fsh_off.size() * 4);
    L.dyn_fpos = sect(std::max<int64_t>(1, (int64_t)fsh_pos.size()) * 4);
    L.dyn_fnat = sect(std::max<int64_t>(1, (int64_t)fsh_nat.size()) * 16);
    L.dyn_bshare = sect((int64_t)bsh_off.size() * 4);
    L.dyn_bpos = sect(std::max<int64_t>(1, (int64_t)bsh_pos.size()) * 4);
    L.dyn_bnat = sect(std::max<int64_t>(1, (int64_t)bsh_nat.size()) * 16);
  }
  L.total = off;
  try {
    p->blob.assign((size_t)L.total, 0);
  } catch (const std::bad_alloc &) {
    delete p;
    return fail(ATTN_ERR_NOMEM, "host blob of %lld bytes", (long long)L.total);
  }
  uint8_t *blob = p->blob.data();
  std::memcpy(blob + L.rowb, rowb.data(), (size_t)S * 16);
  std::memcpy(blob + L.colb, colb.data(), (size_t)S * 16);
  int32_t *it = reinterpret_cast<int32_t *>(blob + L.fwd_items);
  int64_t ffull = 0, fpart = 0, bfull = 0, bpart = 0;
  for (const Item &x : fi) {
    *it++ = x.tile; *it++ = x.head; *it++ = x.off; *it++ = x.len;
  }
  for (int64_t h0 = 0; h0 < sh.Hq; h0 += p->HG) {
    const int fg = fgroup_of(h0);
    for (int64_t qt = 0; qt < nFQ; ++qt) {
      const size_t slot = (size_t)fg * nFQ + qt;
      fpart += fwd_npart[slot]; ffull += fwd_len[slot] - fwd_npart[slot];
    }
  }
  if (!fwd_list.empty()) std::memcpy(blob + L.fwd_list, fwd_list.data(), fwd_list.size() * 4);
  it = reinterpret_cast<int32_t *>(blob + L.bwd_items);
  for (const Item &x : bi) {
    *it++ = x.tile; *it++ = x.head; *it++ = x.off; *it++ = x.len;
  }
  if (!slot_of.empty()) std::memcpy(blob + L.bwd_slot, slot_of.data(), slot_of.size() * 4);
  it = reinterpret_cast<int32_t *>(blob + L.bwd_reduce);
  for (const auto &r : reduce)
    for (int t = 0; t < 4; ++t) *it++ = r[t];
  for (int64_t kvh = 0; kvh < sh.Hkv; ++kvh) {
    const int bg = bgroup_of(kvh);
    for (int64_t kt = 0; kt < nBK; ++kt) {
      const size_t slot = (size_t)bg * nBK + kt;
      bpart += bwd_npart[slot]; bfull += bwd_len[slot] - bwd_npart[slot];
    }
  }
  if (!bwd_list.empty()) std::memcpy(blob + L.bwd_list, bwd_list.data(), bwd_list.size() * 4);
  if (has_bm) {
    std::memcpy(blob + L.bits, bm.bits.data(), bm.bits.size());
    std::memcpy(blob + L.qblk, bm.qblk.data(), (size_t)S * 4);
    std::memcpy(blob + L.kblk, bm.kblk.data(), (size_t)S * 4);
    std::memcpy(blob + L.qoffs, bm.qoffs.data(), bm.qoffs.size() * 4);
    std::memcpy(blob + L.koffs, bm.koffs.data(), bm.koffs.size() * 4);
  }
  if (words) {
    uint64_t *kw = reinterpret_cast<uint64_t *>(blob + L.kwords);
    uint64_t *rw = reinterpret_cast<uint64_t *>(blob + L.rwords);
    // one bitmap head per task; heads fill disjoint rows of both tables
    parallel_for(bm.heads, []() { return 0; }, [&](int h, int) {
      const uint8_t *bh = bm.bits.data() + (size_t)h * bm.nqb * bm.nkb;
      for (int32_t qb = 0; qb < bm.nqb; ++qb)
        for (int64_t t = 0; t < nM; ++t) {
          uint64_t w = 0;
          for (const Seg &g : kseg[(size_t)t])
            if (bh[(size_t)qb * bm.nkb + g.blk]) w |= g.mask;
          kw[((int64_t)h * bm.nqb + qb) * nM + t] = w;
        }
      for (int32_t kb = 0; kb < bm.nkb; ++kb)
        for (int64_t t = 0; t < nM; ++t) {
          uint64_t w = 0;
          for (const Seg &g : qseg[(size_t)t])
            if (bh[(size_t)g.blk * bm.nkb + kb]) w |= g.mask;
          rw[((int64_t)h * bm.nkb + kb) * nM + t] = w;
        }
    });
    if (dynamic) {
      auto put = [&](const std::vector<std::vector<Seg>> &sg, int64_t off, int64_t blk, int64_t mask) {
        int32_t *o = reinterpret_cast<int32_t *>(blob + off);
        int32_t *b = reinterpret_cast<int32_t *>(blob + blk);
        uint64_t *m = reinterpret_cast<uint64_t *>(blob + mask);
        int32_t n = 0;
        for (int64_t t = 0; t < nM; ++t) {
          o[t] = n;
          for (const Seg &g : sg[(size_t)t]) { b[n] = g.blk; m[n] = g.mask; ++n; }
        }
        o[nM] = n;
      };
      put(kseg, L.dyn_kseg_off, L.dyn_kseg_blk, L.dyn_kseg_mask);
      put(qseg, L.dyn_rseg_off, L.dyn_rseg_blk, L.dyn_rseg_mask);
    }
  }
  if (dynamic) {
    std::memcpy(blob + L.dyn_base, base.data(), base.size());
    int32_t *ln = reinterpret_cast<int32_t *>(blob + L.dyn_len);
    for (size_t i = 0; i < fwd_len.size(); ++i) { *ln++ = fwd_len[i]; *ln++ = fwd_npart[i]; }
    for (size_t i = 0; i < bwd_len.size(); ++i) { *ln++ = bwd_len[i]; *ln++ = bwd_npart[i]; }
    std::memcpy(blob + L.dyn_fshare, fsh_off.data(), fsh_off.size() * 4);
    if (!fsh_pos.empty()) std::memcpy(blob + L.dyn_fpos, fsh_pos.data(), fsh_pos.size() * 4);
    if (!fsh_nat.empty()) std::memcpy(blob + L.dyn_fnat, fsh_nat.data(), fsh_nat.size() * 16);
    std::memcpy(blob + L.dyn_bshare, bsh_off.data(), bsh_off.size() * 4);
    if (!bsh_pos.empty()) std::memcpy(blob + L.dyn_bpos, bsh_pos.data(), bsh_pos.size() * 4);
    if (!bsh_nat.empty()) std::memcpy(blob + L.dyn_bnat, bsh_nat.data(), bsh_nat.size() * 16);
  }

  int64_t nnz_b = 0;
  for (int64_t h = 0; h < sh.Hq; ++h) nnz_b += nnz_head[hm_of(h)];
  attn_stats &s = p->stats;
  s.nnz_per_batch = nnz_b;
  s.nnz_total = nnz_b * sh.B;
  s.flops_fwd = 4.0 * (double)sh.d * (double)s.nnz_total;
  s.flops_bwd = 10.0 * (double)sh.d * (double)s.nnz_total;
  s.fwd_items = L.n_fwd_items;
  s.fwd_tiles_full = ffull;
  s.fwd_tiles_partial = fpart;
  s.bwd_items = L.n_bwd_items;
  s.bwd_tiles_full = bfull * GE;
  s.bwd_tiles_partial = bpart * GE;
  s.fwd_tile_rows = p->fwd_rows;
  s.fwd_tile_cols = kFwdKeyTile;
  s.bwd_tile_rows = kBwdRowTile;
  s.bwd_tile_cols = p->bwd_keys;
  s.heads_per_item = p->HG;
  s.device_bytes = L.total;
  s.bwd_head_entries = p->bwd_head_entries ? 1 : 0;
  *out = p;
  return ATTN_OK;
}

extern "C" attn_status attn_plan_create(const attn_shape *shape, const attn_mask_desc *desc,
                                        attn_plan **out) {
  clear_error();
  try {
    return plan_create_impl(shape, desc, out);
  } catch (const std::bad_alloc &) {
    return fail(ATTN_ERR_NOMEM, "host allocation failed while compiling the mask");
  } catch (...) {
    return fail(ATTN_ERR_INVALID, "unexpected error while compiling the mask");
  }
}

extern "C" size_t attn_plan_device_bytes(const attn_plan *plan) {
  return plan ? (size_t)plan->lay.total : 0;
}

extern "C" attn_status attn_plan_stats(const attn_plan *plan, attn_stats *out) {
  clear_error();
  if (!plan || !out) return fail(ATTN_ERR_INVALID, "NULL argument");
  *out = plan->stats;
  return ATTN_OK;
}

extern "C" attn_status attn_plan_get_layout(const attn_plan *plan, attn_plan_layout *out) {
  clear_error();
  if (!plan || !out) return fail(ATTN_ERR_INVALID, "NULL argument");
  const Layout &L = plan->lay;
  out->blob = plan->blob.data();
  out->blob_bytes = L.total;
  out->off_rowb = L.rowb; out->off_colb = L.colb;
  out->off_fwd_items = L.fwd_items; out->n_fwd_items = L.n_fwd_items;
  out->off_fwd_list = L.fwd_list; out->n_fwd_list = L.n_fwd_list;
  out->off_bwd_items = L.bwd_items; out->n_bwd_items = L.n_bwd_items;
  out->off_bwd_list = L.bwd_list; out->n_bwd_list = L.n_bwd_list;
  out->off_bits = L.bits; out->off_qblk = L.qblk; out->off_kblk = L.kblk;
  out->off_qoffs = L.qoffs; out->off_koffs = L.koffs;
  out->off_kwords = L.kwords; out->off_rwords = L.rwords;
  out->off_bwd_slot = L.bwd_slot;
  out->off_bwd_reduce = L.bwd_reduce; out->n_bwd_reduce = L.n_bwd_reduce;
  out->n_slots = L.n_slots;
  return ATTN_OK;
}

// Two fp32 values (LSE * log2 e and D) per (b, h, row), rows padded to 64,
// then the partial results of split dK/dV items.
extern "C" size_t attn_bwd_workspace_bytes(const attn_plan *plan) {
  if (!plan) return 0;
  return (size_t)(lcm::ws_stats_bytes(plan) + lcm::ws_partial_bytes(plan));
}

extern "C" size_t attn_bwd_atomic_workspace_bytes(const attn_plan *plan) {
  if (!plan) return 0;
  return (size_t)(lcm::ws_stats_bytes(plan) + lcm::ws_partial_bytes(plan) + lcm::ws_dq_bytes(plan));
}

extern "C" void attn_plan_destroy(attn_plan *plan) { delete plan; }
