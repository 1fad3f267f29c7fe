// Entry points that take the mask descriptor directly, over a process-wide
// cache of compiled plans ("Long-Context Attention Benchmark" review,
// xllm-io, section 3 components table: one input representation for every
// kernel, behind the kernel adapter).  Host only; the GPU work is that of
// attn_plan_bind, attn_fwd and attn_bwd.
//
// The cache key is the canonical byte string of the shape and of everything
// the descriptor's kind reads (scalars and array contents), so a hit is an
// exact match, never a hash match.  Plans are kept least-recently-used
// first up to ATTN_DESC_CACHE_PLANS.  Caller-provided device buffers are
// tracked by address: `resident` says which cached plan's blob a buffer
// holds, so a plan is uploaded to a buffer once and reused from there.
#include <cstring>
#include <list>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>

#include "plan.hpp"

using namespace lcm;

namespace {

struct Entry {
  std::string key;
  uint64_t hash = 0;
  attn_plan *plan = nullptr;
  std::list<Entry *>::iterator lru;
};

std::mutex g_mu;
std::unordered_map<std::string, std::unique_ptr<Entry>> g_cache;
std::list<Entry *> g_lru;                        // front: most recently used
std::unordered_map<void *, Entry *> g_resident;  // plan buffer -> plan whose blob it holds

void put(std::string &s, const void *p, size_t n) { s.append(static_cast<const char *>(p), n); }
template <typename T>
void put(std::string &s, T x) { put(s, &x, sizeof x); }

uint64_t fnv1a(const std::string &s) {
  uint64_t h = 1469598103934665603ull;
  for (unsigned char c : s) {
    h ^= c;
    h *= 1099511628211ull;
  }
  return h;
}

// Canonical key of (shape, descriptor).  Reads only what the kind uses and
// checks only what it needs to read the arrays safely; the full validation
// is attn_plan_create's, on a miss.
attn_status make_key(const attn_shape *sh, const attn_mask_desc *d, std::string &k) {
  if (!sh || !d) return fail(ATTN_ERR_INVALID, "NULL argument");
  if (d->dynamic != 0)
    return fail(ATTN_ERR_INVALID, "dynamic = 1 plans are not cached: use attn_plan_create");
  if (sh->S < 1 || sh->S >= (int64_t(1) << 30)) return fail(ATTN_ERR_INVALID, "S must be in [1, 2^30)");
  const int64_t S = sh->S;
  put(k, sh->B); put(k, sh->S); put(k, sh->Hq); put(k, sh->Hkv); put(k, sh->d);
  uint32_t sc;
  std::memcpy(&sc, &sh->scale, 4);
  put(k, sc);
  put(k, d->kind); put(k, d->causal); put(k, d->window_left); put(k, d->window_right);
  put(k, d->bwd_key_tile);
  if (d->kind == ATTN_MASK_DOCUMENT || d->kind == ATTN_MASK_PREFIX_LM) {
    if (d->num_docs < 1 || !d->cu_seqlens) return fail(ATTN_ERR_INVALID, "num_docs must be >= 1 with cu_seqlens");
    put(k, d->num_docs);
    put(k, d->cu_seqlens, (size_t)(d->num_docs + 1) * 4);
    if (d->kind == ATTN_MASK_PREFIX_LM) {
      if (!d->prefix_lens) return fail(ATTN_ERR_INVALID, "prefix_lens is NULL");
      put(k, d->prefix_lens, (size_t)d->num_docs * 4);
    }
  } else if (d->kind == ATTN_MASK_COLUMN_BOUNDS) {
    if (!d->col_bounds) return fail(ATTN_ERR_INVALID, "col_bounds is NULL");
    put(k, d->col_bounds, (size_t)S * 16);
  }
  const int32_t has_bm = d->block_bitmap ? 1 : 0;
  put(k, has_bm);
  if (has_bm) {
    if (d->bitmap_heads < 1 || d->n_qblk < 1 || d->n_kblk < 1 || !d->q_blk_offsets || !d->k_blk_offsets)
      return fail(ATTN_ERR_INVALID, "bitmap_heads, n_qblk, n_kblk must be >= 1 with both offset arrays");
    put(k, d->bitmap_heads); put(k, d->n_qblk); put(k, d->n_kblk);
    put(k, d->q_blk_offsets, (size_t)(d->n_qblk + 1) * 4);
    put(k, d->k_blk_offsets, (size_t)(d->n_kblk + 1) * 4);
    const size_t nb = (size_t)d->bitmap_heads * d->n_qblk * d->n_kblk;
    const size_t k0 = k.size();
    put(k, d->block_bitmap, nb);
    for (size_t i = k0; i < k.size(); ++i) k[i] = k[i] ? 1 : 0;  // nonzero = on
  }
  return ATTN_OK;
}

void drop_residency(Entry *e) {
  for (auto it = g_resident.begin(); it != g_resident.end();)
    it = it->second == e ? g_resident.erase(it) : std::next(it);
}

// The cached plan of (shape, desc), compiled on a miss.  Caller holds g_mu.
attn_status lookup(const attn_shape *sh, const attn_mask_desc *d, Entry **out) {
  std::string key;
  attn_status st = make_key(sh, d, key);
  if (st != ATTN_OK) return st;
  auto it = g_cache.find(key);
  if (it != g_cache.end()) {
    Entry *e = it->second.get();
    g_lru.splice(g_lru.begin(), g_lru, e->lru);
    *out = e;
    return ATTN_OK;
  }
  attn_plan *p = nullptr;
  st = attn_plan_create(sh, d, &p);
  if (st != ATTN_OK) return st;
  auto e = std::make_unique<Entry>();
  e->hash = fnv1a(key);
  e->key = std::move(key);
  e->plan = p;
  g_lru.push_front(e.get());
  e->lru = g_lru.begin();
  Entry *raw = e.get();
  g_cache.emplace(raw->key, std::move(e));
  while (g_cache.size() > ATTN_DESC_CACHE_PLANS) {
    Entry *old = g_lru.back();
    g_lru.pop_back();
    drop_residency(old);
    attn_plan_destroy(old->plan);
    g_cache.erase(old->key);
  }
  *out = raw;
  return ATTN_OK;
}

// The argument checks of attn_fwd / attn_bwd, run before a possible upload
// so that on an error nothing is enqueued.
attn_status check_ptr(const void *x, const char *name, uintptr_t align) {
  if (!x) return fail(ATTN_ERR_INVALID, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(x) & (align - 1))
    return fail(ATTN_ERR_INVALID, "%s is not %u-byte aligned", name, (unsigned)align);
  return ATTN_OK;
}

#define LCM_DESC_CHECK(expr)         \
  do {                               \
    const attn_status s_ = (expr);   \
    if (s_ != ATTN_OK) return s_;    \
  } while (0)

// Point the plan at plan_buf, uploading its blob unless plan_buf holds it.
attn_status make_resident(Entry *e, void *buf, size_t bytes, attn_stream_t stream) {
  if (!buf) return fail(ATTN_ERR_INVALID, "plan_buf is NULL");
  auto it = g_resident.find(buf);
  if (it != g_resident.end() && it->second == e) {
    if (bytes < (size_t)e->plan->lay.total)
      return fail(ATTN_ERR_INVALID, "plan_buf holds %zu bytes; the plan needs %lld", bytes,
                  (long long)e->plan->lay.total);
    e->plan->dev_blob = buf;
    e->plan->dev_bytes = bytes;
    return ATTN_OK;
  }
  g_resident.erase(buf);  // whatever it held is overwritten, or in doubt on a failure
  const attn_status st = attn_plan_bind(e->plan, buf, bytes, stream);
  if (st != ATTN_OK) return st;
  g_resident[buf] = e;
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_desc_plan_bytes(const attn_shape *shape, const attn_mask_desc *desc,
                                            size_t *plan_bytes, size_t *ws_bytes,
                                            uint64_t *key_hash) {
  clear_error();
  try {
    std::lock_guard<std::mutex> lk(g_mu);
    Entry *e = nullptr;
    const attn_status st = lookup(shape, desc, &e);
    if (st != ATTN_OK) return st;
    if (plan_bytes) *plan_bytes = attn_plan_device_bytes(e->plan);
    if (ws_bytes) *ws_bytes = attn_bwd_workspace_bytes(e->plan);
    if (key_hash) *key_hash = e->hash;
    return ATTN_OK;
  } catch (const std::bad_alloc &) {
    return fail(ATTN_ERR_NOMEM, "host allocation failed in the plan cache");
  } catch (...) {
    return fail(ATTN_ERR_INVALID, "unexpected error in the plan cache");
  }
}

extern "C" attn_status attn_fwd_desc(const attn_shape *shape, const attn_mask_desc *desc,
                                     const void *q, const void *k, const void *v, void *o,
                                     float *lse, void *plan_buf, size_t plan_buf_bytes,
                                     attn_stream_t stream) {
  clear_error();
  try {
    std::lock_guard<std::mutex> lk(g_mu);
    Entry *e = nullptr;
    LCM_DESC_CHECK(lookup(shape, desc, &e));
    LCM_DESC_CHECK(check_ptr(q, "q", 16));
    LCM_DESC_CHECK(check_ptr(k, "k", 16));
    LCM_DESC_CHECK(check_ptr(v, "v", 16));
    LCM_DESC_CHECK(check_ptr(o, "o", 16));
    LCM_DESC_CHECK(check_ptr(lse, "lse", 4));
    LCM_DESC_CHECK(make_resident(e, plan_buf, plan_buf_bytes, stream));
    return attn_fwd(e->plan, q, k, v, o, lse, stream);
  } catch (const std::bad_alloc &) {
    return fail(ATTN_ERR_NOMEM, "host allocation failed in the plan cache");
  } catch (...) {
    return fail(ATTN_ERR_INVALID, "unexpected error in the plan cache");
  }
}

extern "C" attn_status attn_bwd_desc(const attn_shape *shape, const attn_mask_desc *desc,
                                     const void *q, const void *k, const void *v, const void *o,
                                     const float *lse, const void *dout, void *dq, void *dk,
                                     void *dv, void *ws, size_t ws_bytes, void *plan_buf,
                                     size_t plan_buf_bytes, attn_stream_t stream) {
  clear_error();
  try {
    std::lock_guard<std::mutex> lk(g_mu);
    Entry *e = nullptr;
    LCM_DESC_CHECK(lookup(shape, desc, &e));
    LCM_DESC_CHECK(check_ptr(q, "q", 16));
    LCM_DESC_CHECK(check_ptr(k, "k", 16));
    LCM_DESC_CHECK(check_ptr(v, "v", 16));
    LCM_DESC_CHECK(check_ptr(o, "o", 16));
    LCM_DESC_CHECK(check_ptr(lse, "lse", 4));
    LCM_DESC_CHECK(check_ptr(dout, "dout", 16));
    LCM_DESC_CHECK(check_ptr(dq, "dq", 16));
    LCM_DESC_CHECK(check_ptr(dk, "dk", 16));
    LCM_DESC_CHECK(check_ptr(dv, "dv", 16));
    LCM_DESC_CHECK(check_ptr(ws, "ws", 256));
    if (ws_bytes < attn_bwd_workspace_bytes(e->plan))
      return fail(ATTN_ERR_INVALID, "workspace holds %zu bytes; %zu needed", ws_bytes,
                  attn_bwd_workspace_bytes(e->plan));
    LCM_DESC_CHECK(make_resident(e, plan_buf, plan_buf_bytes, stream));
    return attn_bwd(e->plan, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream);
  } catch (const std::bad_alloc &) {
    return fail(ATTN_ERR_NOMEM, "host allocation failed in the plan cache");
  } catch (...) {
    return fail(ATTN_ERR_INVALID, "unexpected error in the plan cache");
  }
}

extern "C" void attn_desc_release(void *plan_buf) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_resident.erase(plan_buf);
}

extern "C" void attn_desc_cache_clear(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_resident.clear();
  g_lru.clear();
  for (auto &kv : g_cache) attn_plan_destroy(kv.second->plan);
  g_cache.clear();
}
