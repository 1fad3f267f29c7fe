// Host-only driver for the mask compiler and the descriptor plan cache, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  It links plan.cpp and desc_cache.cpp and
// replaces the three GPU entry points the cache calls (plan upload, forward,
// backward) with host stand-ins: the upload copies the blob into the caller's
// buffer with memcpy, the launches only check their plan.  Exit status 0 and
// no sanitizer report mean that every plan lifecycle below ran clean.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "attn.h"

// ---- host stand-ins for the entry points implemented in device code ----
extern "C" attn_status attn_plan_bind(attn_plan *plan, void *dev_buf, size_t bytes,
                                      attn_stream_t) {
  const size_t need = attn_plan_device_bytes(plan);
  if (!dev_buf || bytes < need) return ATTN_ERR_INVALID;
  attn_plan_layout lay;
  if (attn_plan_get_layout(plan, &lay) != ATTN_OK) return ATTN_ERR_INVALID;
  std::memcpy(dev_buf, lay.blob, (size_t)lay.blob_bytes);
  return ATTN_OK;
}
extern "C" attn_status attn_fwd(const attn_plan *plan, const void *, const void *, const void *,
                                void *, float *, attn_stream_t) {
  return plan ? ATTN_OK : ATTN_ERR_INVALID;
}
extern "C" attn_status attn_bwd(const attn_plan *plan, const void *, const void *, const void *,
                                const void *, const float *, const void *, void *, void *,
                                void *, void *, size_t, attn_stream_t) {
  return plan ? ATTN_OK : ATTN_ERR_INVALID;
}

namespace {

std::atomic<int> g_fail{0};
volatile uint64_t g_sink = 0;  // keeps the blob reads below from being optimised away
#define EXPECT(c)                                                         \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #c); \
      ++g_fail;                                                           \
    }                                                                     \
  } while (0)

uint64_t g_rng = 0x9e3779b97f4a7c15ull;
uint32_t rnd() {
  g_rng = g_rng * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_rng >> 33);
}

attn_mask_desc blank(int kind) {
  attn_mask_desc d;
  std::memset(&d, 0, sizeof d);
  d.kind = kind;
  return d;
}

// Every byte of the plan's blob and every section of its layout is read, so
// that a size or offset past the allocation shows up under ASan.
uint64_t touch(const attn_plan *p) {
  attn_plan_layout lay;
  EXPECT(attn_plan_get_layout(p, &lay) == ATTN_OK);
  const uint8_t *b = static_cast<const uint8_t *>(lay.blob);
  uint64_t h = 0;
  for (int64_t i = 0; i < lay.blob_bytes; ++i) h = h * 31 + b[i];
  const int64_t offs[] = {lay.off_rowb, lay.off_colb, lay.off_fwd_items, lay.off_fwd_list,
                          lay.off_bwd_items, lay.off_bwd_list, lay.off_bits, lay.off_qblk,
                          lay.off_kblk, lay.off_qoffs, lay.off_koffs, lay.off_bwd_slot,
                          lay.off_bwd_reduce};
  for (int64_t o : offs) EXPECT(o < lay.blob_bytes);
  EXPECT((size_t)lay.blob_bytes <= attn_plan_device_bytes(p));
  attn_stats st;
  EXPECT(attn_plan_stats(p, &st) == ATTN_OK);
  EXPECT(st.nnz_total == st.nnz_per_batch * 1 || st.nnz_total % st.nnz_per_batch == 0);
  (void)attn_bwd_workspace_bytes(p);
  return h;
}

attn_status make(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t d,
                 const attn_mask_desc &m, bool keep_stats = true) {
  attn_shape sh{B, S, Hq, Hkv, d, 0.f};
  attn_plan *p = nullptr;
  const attn_status st = attn_plan_create(&sh, &m, &p);
  if (st == ATTN_OK) {
    EXPECT(p != nullptr);
    if (keep_stats) g_sink = g_sink + touch(p);
    attn_plan_destroy(p);
  } else {
    EXPECT(p == nullptr);
    EXPECT(attn_last_error() != nullptr && attn_last_error()[0] != 0);
  }
  return st;
}

std::vector<int32_t> partition(int S, int lo, int hi) {
  std::vector<int32_t> o{0};
  while (o.back() < S) o.push_back(std::min(S, o.back() + lo + (int)(rnd() % (hi - lo + 1))));
  return o;
}

std::vector<uint8_t> bits(int heads, int nq, int nk, int pct) {
  std::vector<uint8_t> b((size_t)heads * nq * nk);
  for (auto &x : b) x = (uint8_t)((int)(rnd() % 100) < pct);
  return b;
}

void families(int64_t S, int64_t Hq, int64_t Hkv, int64_t d) {
  EXPECT(make(1, S, Hq, Hkv, d, blank(ATTN_MASK_FULL)) == ATTN_OK);
  EXPECT(make(2, S, Hq, Hkv, d, blank(ATTN_MASK_CAUSAL)) == ATTN_OK);
  for (int causal = 0; causal < 2; ++causal) {
    attn_mask_desc m = blank(ATTN_MASK_SLIDING);
    m.causal = causal;
    m.window_left = 1 + (int)(rnd() % (S + 1));
    m.window_right = 1 + (int)(rnd() % (S + 1));
    EXPECT(make(1, S, Hq, Hkv, d, m) == ATTN_OK);
  }
  std::vector<int32_t> cu = partition((int)S, 1, (int)std::max<int64_t>(1, S / 3));
  for (int causal = 0; causal < 2; ++causal) {
    attn_mask_desc m = blank(ATTN_MASK_DOCUMENT);
    m.causal = causal;
    m.num_docs = (int)cu.size() - 1;
    m.cu_seqlens = cu.data();
    EXPECT(make(1, S, Hq, Hkv, d, m) == ATTN_OK);
  }
  std::vector<int32_t> pre;
  for (size_t k = 0; k + 1 < cu.size(); ++k) pre.push_back((int32_t)(rnd() % (cu[k + 1] - cu[k] + 1)));
  {
    attn_mask_desc m = blank(ATTN_MASK_PREFIX_LM);
    m.num_docs = (int)cu.size() - 1;
    m.cu_seqlens = cu.data();
    m.prefix_lens = pre.data();
    EXPECT(make(1, S, Hq, Hkv, d, m) == ATTN_OK);
  }
  {  // column bounds: causal plus a masked band below the diagonal (at most two runs per row)
    std::vector<int32_t> cb((size_t)S * 4);
    const int32_t w = 1 + (int32_t)(rnd() % S);
    for (int32_t j = 0; j < S; ++j) {
      cb[4 * j + 0] = std::min<int32_t>((int32_t)S, j + w);
      cb[4 * j + 1] = (int32_t)S;
      cb[4 * j + 2] = 0;
      cb[4 * j + 3] = j;
    }
    attn_mask_desc m = blank(ATTN_MASK_COLUMN_BOUNDS);
    m.col_bounds = cb.data();
    EXPECT(make(1, S, Hq, Hkv, d, m) == ATTN_OK);
  }
  // bitmaps: uniform and variable blocks, shared or distinct partitions, one
  // bitmap, one per KV head, one per query head; static and dynamic
  const int heads_opts[3] = {1, (int)Hkv, (int)Hq};
  for (int hi = 0; hi < 3; ++hi)
    for (int dyn = 0; dyn < 2; ++dyn) {
      std::vector<int32_t> qo = partition((int)S, 16, 160);
      std::vector<int32_t> ko = (rnd() & 1) ? qo : partition((int)S, 16, 160);
      const int nq = (int)qo.size() - 1, nk = (int)ko.size() - 1;
      std::vector<uint8_t> b = bits(heads_opts[hi], nq, nk, 50);
      attn_mask_desc m = blank((rnd() & 1) ? ATTN_MASK_FULL : ATTN_MASK_CAUSAL);
      m.block_bitmap = b.data();
      m.bitmap_heads = heads_opts[hi];
      m.n_qblk = nq;
      m.n_kblk = nk;
      m.q_blk_offsets = qo.data();
      m.k_blk_offsets = ko.data();
      m.dynamic = dyn;
      EXPECT(make(1, S, Hq, Hkv, d, m) == ATTN_OK);
    }
}

void errors() {
  attn_shape sh{1, 256, 4, 2, 64, 0.f};
  attn_mask_desc ok = blank(ATTN_MASK_CAUSAL);
  attn_plan *p = nullptr;
  EXPECT(attn_plan_create(nullptr, &ok, &p) == ATTN_ERR_INVALID);
  EXPECT(attn_plan_create(&sh, nullptr, &p) == ATTN_ERR_INVALID);
  EXPECT(attn_plan_create(&sh, &ok, nullptr) == ATTN_ERR_INVALID);
  EXPECT(make(0, 256, 4, 2, 64, ok) == ATTN_ERR_INVALID);
  EXPECT(make(1, 0, 4, 2, 64, ok) == ATTN_ERR_INVALID);
  EXPECT(make(1, 256, 4, 3, 64, ok) == ATTN_ERR_INVALID);
  EXPECT(make(1, 256, 4, 2, 96, ok) == ATTN_ERR_UNSUPPORTED);
  EXPECT(make(1, 256, 4, 2, 64, blank(17)) != ATTN_OK);
  attn_mask_desc sw = blank(ATTN_MASK_SLIDING);
  sw.window_left = 0;
  EXPECT(make(1, 256, 4, 2, 64, sw) == ATTN_ERR_INVALID);
  int32_t bad_cu[3] = {0, 200, 100};
  attn_mask_desc doc = blank(ATTN_MASK_DOCUMENT);
  doc.num_docs = 2;
  doc.cu_seqlens = bad_cu;
  EXPECT(make(1, 256, 4, 2, 64, doc) == ATTN_ERR_INVALID);
  doc.cu_seqlens = nullptr;
  EXPECT(make(1, 256, 4, 2, 64, doc) == ATTN_ERR_INVALID);
  int32_t cu[3] = {0, 100, 256}, pre[2] = {0, 200};
  attn_mask_desc pl = blank(ATTN_MASK_PREFIX_LM);
  pl.num_docs = 2;
  pl.cu_seqlens = cu;
  pl.prefix_lens = pre;
  EXPECT(make(1, 256, 4, 2, 64, pl) == ATTN_ERR_INVALID);
  std::vector<int32_t> cb(256 * 4, 0);
  cb[4 * 7 + 1] = 300;  // out of [0, S]
  attn_mask_desc cbd = blank(ATTN_MASK_COLUMN_BOUNDS);
  cbd.col_bounds = cb.data();
  EXPECT(make(1, 256, 4, 2, 64, cbd) == ATTN_ERR_INVALID);
  int32_t offs[3] = {0, 128, 256}, bad_offs[3] = {0, 300, 256};
  uint8_t bm[3 * 2 * 2] = {1, 0, 0, 1, 1, 1, 0, 1, 1, 0, 1, 1};
  attn_mask_desc bd = blank(ATTN_MASK_FULL);
  bd.block_bitmap = bm;
  bd.bitmap_heads = 3;  // not 1, Hkv or Hq
  bd.n_qblk = bd.n_kblk = 2;
  bd.q_blk_offsets = bd.k_blk_offsets = offs;
  EXPECT(make(1, 256, 4, 2, 64, bd) == ATTN_ERR_INVALID);
  bd.bitmap_heads = 2;
  bd.q_blk_offsets = bad_offs;
  EXPECT(make(1, 256, 4, 2, 64, bd) == ATTN_ERR_INVALID);
  bd.q_blk_offsets = offs;
  bd.dynamic = 2;
  EXPECT(make(1, 256, 4, 2, 64, bd) == ATTN_ERR_INVALID);
  attn_mask_desc dyn_nobits = blank(ATTN_MASK_CAUSAL);
  dyn_nobits.dynamic = 1;
  EXPECT(make(1, 256, 4, 2, 64, dyn_nobits) == ATTN_ERR_INVALID);
  attn_stats st;
  EXPECT(attn_plan_stats(nullptr, &st) == ATTN_ERR_INVALID);
  attn_plan_layout lay;
  EXPECT(attn_plan_get_layout(nullptr, &lay) == ATTN_ERR_INVALID);
  attn_plan_destroy(nullptr);
}

void desc_cache() {
  // more distinct masks than the cache holds, each used through the
  // descriptor calls with host buffers, then released; finally cleared
  std::vector<std::vector<uint8_t>> bufs;
  alignas(256) static uint8_t qkv[4096];
  for (int round = 0; round < 2; ++round)
    for (int i = 0; i < ATTN_DESC_CACHE_PLANS + 8; ++i) {
      attn_shape sh{1, 200 + i, 4, 2, 64, 0.f};
      attn_mask_desc m = blank(ATTN_MASK_SLIDING);
      m.causal = 1;
      m.window_left = 17 + i;
      size_t pb = 0, wb = 0;
      uint64_t hash = 0;
      EXPECT(attn_desc_plan_bytes(&sh, &m, &pb, &wb, &hash) == ATTN_OK);
      EXPECT(pb > 0);
      bufs.emplace_back(pb + 256);
      uint8_t *buf = bufs.back().data();
      buf += (256 - ((uintptr_t)buf & 255)) & 255;
      std::vector<uint8_t> ws(wb + 512);
      uint8_t *w = ws.data() + ((256 - ((uintptr_t)ws.data() & 255)) & 255);
      EXPECT(attn_fwd_desc(&sh, &m, qkv, qkv, qkv, qkv, (float *)qkv, buf, pb, nullptr) == ATTN_OK);
      EXPECT(attn_bwd_desc(&sh, &m, qkv, qkv, qkv, qkv, (const float *)qkv, qkv, qkv, qkv, qkv, w,
                           wb, buf, pb, nullptr) == ATTN_OK);
      // a too-small plan buffer and a misaligned pointer are refused
      EXPECT(attn_fwd_desc(&sh, &m, qkv, qkv, qkv, qkv, (float *)qkv, buf, pb - 1, nullptr) != ATTN_OK);
      EXPECT(attn_fwd_desc(&sh, &m, qkv + 1, qkv, qkv, qkv, (float *)qkv, buf, pb, nullptr) ==
             ATTN_ERR_INVALID);
      if (i % 3 == 0) attn_desc_release(buf);
    }
  attn_desc_cache_clear();
  attn_desc_release(nullptr);
}

// Several threads share the descriptor cache: lookups, uploads into their
// own buffers, launches, releases and (one thread) cache clears, plus plan
// creation (with bitmaps of several heads, whose lists the compiler builds
// on threads of its own) and the thread-local error string.  Run under
// ThreadSanitizer.
void threads() {
  constexpr int NT = 4, IT = 150, NMASK = 40;
  std::vector<std::thread> ts;
  std::vector<int> fails(NT, 0);
  for (int t = 0; t < NT; ++t)
    ts.emplace_back([t, &fails] {
      uint64_t r = 0x1234567ull + (uint64_t)t * 0x9e3779b97f4a7c15ull;
      auto next = [&r] {
        r = r * 6364136223846793005ull + 1442695040888963407ull;
        return (uint32_t)(r >> 33);
      };
      alignas(256) static thread_local uint8_t qkv[4096];
      std::vector<uint8_t> buf_store, ws_store;
      for (int it = 0; it < IT; ++it) {
        const int i = (int)(next() % NMASK);
        attn_shape sh{1, 150 + i, 4, 2, 64, 0.f};
        attn_mask_desc m = blank(ATTN_MASK_SLIDING);
        m.causal = 1;
        m.window_left = 9 + i;
        size_t pb = 0, wb = 0;
        if (attn_desc_plan_bytes(&sh, &m, &pb, &wb, nullptr) != ATTN_OK) { ++fails[t]; continue; }
        buf_store.assign(pb + 256, 0);
        ws_store.assign(wb + 512, 0);
        uint8_t *buf = buf_store.data() + ((256 - ((uintptr_t)buf_store.data() & 255)) & 255);
        uint8_t *w = ws_store.data() + ((256 - ((uintptr_t)ws_store.data() & 255)) & 255);
        if (attn_fwd_desc(&sh, &m, qkv, qkv, qkv, qkv, (float *)qkv, buf, pb, nullptr) != ATTN_OK) ++fails[t];
        if (attn_bwd_desc(&sh, &m, qkv, qkv, qkv, qkv, (const float *)qkv, qkv, qkv, qkv, qkv, w, wb,
                          buf, pb, nullptr) != ATTN_OK)
          ++fails[t];
        attn_desc_release(buf);  // the buffer is freed or reused next
        // an invalid call sets this thread's error string only
        attn_shape bad{1, 100, 4, 3, 64, 0.f};
        attn_plan *p = nullptr;
        if (attn_plan_create(&bad, &m, &p) != ATTN_ERR_INVALID) ++fails[t];
        const std::string e = attn_last_error();
        if (e.empty()) ++fails[t];
        if (make(1, 64 + i, 4, 2, 64, blank(ATTN_MASK_CAUSAL), false) != ATTN_OK) ++fails[t];
        if (it % 10 == 0) {
          // bitmaps of several heads: the plan compiler builds their lists on
          // host threads of its own, inside each calling thread
          const int S2 = 300 + i;
          std::vector<int32_t> qo{0};
          while (qo.back() < S2) qo.push_back(std::min(S2, qo.back() + 16 + (int)(next() % 100)));
          const int nq = (int)qo.size() - 1, heads = (it % 20 == 0) ? 8 : 2;
          std::vector<uint8_t> b((size_t)heads * nq * nq);
          for (auto &x : b) x = (uint8_t)(next() % 2);
          attn_mask_desc bm = blank(ATTN_MASK_CAUSAL);
          bm.block_bitmap = b.data();
          bm.bitmap_heads = heads;
          bm.n_qblk = bm.n_kblk = nq;
          bm.q_blk_offsets = bm.k_blk_offsets = qo.data();
          if (make(1, S2, 8, 2, 64, bm, false) != ATTN_OK) ++fails[t];
        }
        if (t == 0 && it % 37 == 36) attn_desc_cache_clear();
      }
    });
  for (auto &th : ts) th.join();
  for (int t = 0; t < NT; ++t) EXPECT(fails[t] == 0);
  attn_desc_cache_clear();
}

}  // namespace

int main(int argc, char **argv) {
  if (argc > 1 && std::string(argv[1]) == "threads") {
    threads();
    if (g_fail) return 1;
    std::printf("host sanitizer driver: threads clean\n");
    return 0;
  }
  EXPECT(attn_version() != nullptr);
  const int64_t shapes[][4] = {{1, 2, 2, 64},   {65, 4, 2, 64},  {128, 3, 1, 64},
                               {333, 2, 2, 128}, {700, 8, 1, 128}, {1024, 8, 2, 128},
                               {2111, 4, 4, 64}};
  for (auto &s : shapes) families(s[0], s[1], s[2], s[3]);
  errors();
  desc_cache();
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail.load());
    return 1;
  }
  std::printf("host sanitizer driver: all plan lifecycles clean\n");
  return 0;
}
