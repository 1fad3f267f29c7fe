// C-ABI entry points that touch the GPU: plan binding, forward, backward.
// All argument checks run before anything is enqueued.
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "kernels.hpp"
#include "plan.hpp"

namespace lcm {
hipError_t launch_fwd(const FwdArgs &a, int d, int HG, bool masked, int n_items, int B,
                      hipStream_t st);
hipError_t launch_bwd_pre(const BwdArgs &a, int d, int B, hipStream_t st);
hipError_t launch_dkdv(const BwdArgs &a, int d, int B, bool fused_dq, hipStream_t st);
hipError_t launch_dq_convert(const BwdArgs &a, int d, int B, hipStream_t st);
hipError_t launch_dq(const BwdArgs &a, int d, int HG, bool masked, int B, hipStream_t st);
hipError_t launch_merge(const float *o1, const float *lse1, const float *o2, const float *lse2,
                        void *o, bool o_bf16, float *lse, int64_t B, int S, int Hq, int d,
                        hipStream_t st);
hipError_t launch_dyn(const DynArgs &a, hipStream_t st);
}  // namespace lcm

using namespace lcm;

static_assert(kDkdvKeys == kBwdKeyTile, "dK/dV tile width of the kernels and the plan");
static_assert(kTileBits == (1u << kHeadShift) - 1u, "dK/dV list entry layout of the kernels and the plan");

namespace {

template <typename T>
const T *sect(const attn_plan *p, int64_t off) {
  return off < 0 ? nullptr
                 : reinterpret_cast<const T *>(static_cast<const uint8_t *>(p->dev_blob) + off);
}

MaskArgs mask_args(const attn_plan *p) {
  MaskArgs m{};
  m.rowb = sect<int4>(p, p->lay.rowb);
  m.colb = sect<int4>(p, p->lay.colb);
  m.bits = sect<uint8_t>(p, p->lay.bits);
  m.qblk = sect<int>(p, p->lay.qblk);
  m.kblk = sect<int>(p, p->lay.kblk);
  m.qoffs = sect<int>(p, p->lay.qoffs);
  m.koffs = sect<int>(p, p->lay.koffs);
  m.nqb = p->nqb;
  m.nkb = p->nkb;
  m.bm_heads = p->bitmap_heads;
  m.kwords = sect<uint64_t>(p, p->lay.kwords);
  m.rwords = sect<uint64_t>(p, p->lay.rwords);
  m.nM = (int)((p->shape.S + kMicro - 1) / kMicro);
  return m;
}

bool misaligned(const void *x, uintptr_t a) { return (reinterpret_cast<uintptr_t>(x) & (a - 1)) != 0; }

attn_status check_tensor(const void *x, const char *name, uintptr_t align) {
  if (!x) return fail(ATTN_ERR_INVALID, "%s is NULL", name);
  if (misaligned(x, align)) return fail(ATTN_ERR_INVALID, "%s is not %u-byte aligned", name, (unsigned)align);
  return ATTN_OK;
}

// Host-forced device error, to exercise the error path without a GPU.
bool forced_device_error() {
  const char *e = std::getenv("ATTN_FORCE_DEVICE_ERROR");
  return e && e[0] == '1';
}

// Whether the forward / dQ lists can hold partial tiles: those of a dynamic
// plan change with every bitmap, the others are fixed at creation.
bool masked_lists(const attn_plan *p) { return p->dyn.on || p->stats.fwd_tiles_partial > 0; }

attn_status check_plan(const attn_plan *p) {
  if (!p) return fail(ATTN_ERR_INVALID, "plan is NULL");
  if (!p->dev_blob) return fail(ATTN_ERR_INVALID, "plan is not bound to device memory");
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_plan_bind(attn_plan *plan, void *dev_buf, size_t bytes,
                                      attn_stream_t stream) {
  clear_error();
  if (!plan) return fail(ATTN_ERR_INVALID, "plan is NULL");
  if (!dev_buf) return fail(ATTN_ERR_INVALID, "dev_buf is NULL");
  if (misaligned(dev_buf, 256)) return fail(ATTN_ERR_INVALID, "dev_buf is not 256-byte aligned");
  if (bytes < (size_t)plan->lay.total)
    return fail(ATTN_ERR_INVALID, "dev_buf holds %zu bytes; the plan needs %lld", bytes,
                (long long)plan->lay.total);
  if (forced_device_error()) return fail(ATTN_ERR_DEVICE, "forced device error (ATTN_FORCE_DEVICE_ERROR)");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dev_buf, plan->blob.data(), (size_t)plan->lay.total,
                                hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);  // the host blob may be freed after return
  if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "plan upload failed: %s", hipGetErrorString(e));
  plan->dev_blob = dev_buf;
  plan->dev_bytes = bytes;
  return ATTN_OK;
}

extern "C" attn_status attn_plan_set_bitmap(attn_plan *plan, const uint8_t *bits,
                                            attn_stream_t stream) {
  clear_error();
  if (plan && !plan->dyn.on) return fail(ATTN_ERR_INVALID, "plan was not created with dynamic = 1");
  attn_status st0 = check_plan(plan);
  if (st0 != ATTN_OK) return st0;
  st0 = check_tensor(bits, "bits", 16);
  if (st0 != ATTN_OK) return st0;
  const int64_t nbits = (int64_t)plan->bitmap_heads * plan->nqb * plan->nkb;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(bits);
  const uintptr_t p0 = reinterpret_cast<uintptr_t>(plan->dev_blob);
  if (b0 < p0 + (uintptr_t)plan->lay.total && p0 < b0 + (uintptr_t)nbits)
    return fail(ATTN_ERR_INVALID, "bits overlaps the plan's device buffer");
  if (forced_device_error()) return fail(ATTN_ERR_DEVICE, "forced device error (ATTN_FORCE_DEVICE_ERROR)");
  const DynInfo &D = plan->dyn;
  const Layout &L = plan->lay;
  uint8_t *blob = static_cast<uint8_t *>(plan->dev_blob);
  DynArgs a{};
  a.src = bits;
  a.bits = blob + L.bits;
  a.nbits = nbits;
  a.base = blob + L.dyn_base;
  a.qblk = reinterpret_cast<const int *>(blob + L.qblk);
  a.kblk = reinterpret_cast<const int *>(blob + L.kblk);
  a.fwd_list = reinterpret_cast<uint32_t *>(blob + L.fwd_list);
  a.bwd_list = reinterpret_cast<uint32_t *>(blob + L.bwd_list);
  a.slot_len = reinterpret_cast<int2 *>(blob + L.dyn_len);
  a.fitems = reinterpret_cast<int4 *>(blob + L.fwd_items);
  a.bitems = reinterpret_cast<int4 *>(blob + L.bwd_items);
  a.fshare = reinterpret_cast<const int *>(blob + L.dyn_fshare);
  a.bshare = reinterpret_cast<const int *>(blob + L.dyn_bshare);
  a.fpos = reinterpret_cast<const int *>(blob + L.dyn_fpos);
  a.bpos = reinterpret_cast<const int *>(blob + L.dyn_bpos);
  a.fnat = reinterpret_cast<const int4 *>(blob + L.dyn_fnat);
  a.bnat = reinterpret_cast<const int4 *>(blob + L.dyn_bnat);
  a.n_fshares = D.n_fshares;
  a.n_bshares = D.n_bshares;
  a.S = (int)plan->shape.S;
  a.nM = (int)D.nM;
  a.MR = D.MR;
  a.MC = D.MC;
  a.nqb = plan->nqb;
  a.nkb = plan->nkb;
  a.nFQ = (int)D.nFQ;
  a.nBK = (int)D.nBK;
  a.n_fslots = (int)D.n_fslots;
  a.n_bslots = (int)D.n_bslots;
  a.fheads = D.fheads;
  a.bheads = D.bheads;
  a.bhe = D.bhe ? 1 : 0;
  a.bcap = D.bcap;
  a.head_major = D.head_major ? 1 : 0;
  a.fkv = D.fkv;
  a.bm_heads = plan->bitmap_heads;
  if (L.kwords >= 0) {
    a.kwords = reinterpret_cast<uint64_t *>(blob + L.kwords);
    a.rwords = reinterpret_cast<uint64_t *>(blob + L.rwords);
    a.kseg_off = reinterpret_cast<const int *>(blob + L.dyn_kseg_off);
    a.kseg_blk = reinterpret_cast<const int *>(blob + L.dyn_kseg_blk);
    a.kseg_mask = reinterpret_cast<const uint64_t *>(blob + L.dyn_kseg_mask);
    a.rseg_off = reinterpret_cast<const int *>(blob + L.dyn_rseg_off);
    a.rseg_blk = reinterpret_cast<const int *>(blob + L.dyn_rseg_blk);
    a.rseg_mask = reinterpret_cast<const uint64_t *>(blob + L.dyn_rseg_mask);
  }
  (void)hipGetLastError();
  const hipError_t e = launch_dyn(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "list rebuild launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

namespace {
attn_status fwd_impl(const attn_plan *p, const void *q, const void *k, const void *v, void *o,
                     bool o32, float *lse, attn_stream_t stream) {
  clear_error();
  attn_status s;
  if ((s = check_plan(p)) != ATTN_OK) return s;
  if ((s = check_tensor(q, "q", 16)) != ATTN_OK) return s;
  if ((s = check_tensor(k, "k", 16)) != ATTN_OK) return s;
  if ((s = check_tensor(v, "v", 16)) != ATTN_OK) return s;
  if ((s = check_tensor(o, "o", 16)) != ATTN_OK) return s;
  if ((s = check_tensor(lse, "lse", 4)) != ATTN_OK) return s;
  if (forced_device_error()) return fail(ATTN_ERR_DEVICE, "forced device error (ATTN_FORCE_DEVICE_ERROR)");
  FwdArgs a{};
  a.q = static_cast<const bf16 *>(q);
  a.k = static_cast<const bf16 *>(k);
  a.v = static_cast<const bf16 *>(v);
  if (o32) a.o32 = static_cast<float *>(o);
  else a.o = static_cast<bf16 *>(o);
  a.lse = lse;
  a.S = (int)p->shape.S;
  a.Hq = (int)p->shape.Hq;
  a.Hkv = (int)p->shape.Hkv;
  a.G = p->G;
  a.sl2 = p->scale * kLog2e;
  a.items = sect<int4>(p, p->lay.fwd_items);
  a.list = sect<uint32_t>(p, p->lay.fwd_list);
  a.m = mask_args(p);
  (void)hipGetLastError();
  const hipError_t e = launch_fwd(a, (int)p->shape.d, p->HG, masked_lists(p), (int)p->lay.n_fwd_items,
                                  (int)p->shape.B, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "forward launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}
}  // namespace

extern "C" attn_status attn_fwd(const attn_plan *p, const void *q, const void *k, const void *v,
                                void *o, float *lse, attn_stream_t stream) {
  return fwd_impl(p, q, k, v, o, false, lse, stream);
}

extern "C" attn_status attn_fwd_partial(const attn_plan *p, const void *q, const void *k,
                                        const void *v, float *o, float *lse,
                                        attn_stream_t stream) {
  return fwd_impl(p, q, k, v, o, true, lse, stream);
}

namespace {

// Fill the backward argument block; tensors the stage does not use may be
// NULL (checked by the caller).
BwdArgs bwd_args(const attn_plan *p, const void *q, const void *k, const void *v,
                 const void *o, const float *lse, const void *dout, void *dq, void *dk,
                 void *dv, const void *ws) {
  BwdArgs a{};
  a.q = static_cast<const bf16 *>(q);
  a.k = static_cast<const bf16 *>(k);
  a.v = static_cast<const bf16 *>(v);
  a.o = static_cast<const bf16 *>(o);
  a.dout = static_cast<const bf16 *>(dout);
  a.lse = lse;
  a.ws = static_cast<float *>(const_cast<void *>(ws));
  a.S64 = (int)((p->shape.S + 63) / 64 * 64);
  a.dq = static_cast<bf16 *>(dq);
  a.dk = static_cast<bf16 *>(dk);
  a.dv = static_cast<bf16 *>(dv);
  a.S = (int)p->shape.S;
  a.Hq = (int)p->shape.Hq;
  a.Hkv = (int)p->shape.Hkv;
  a.G = p->G;
  a.scale = p->scale;
  a.sl2 = p->scale * kLog2e;
  a.fitems = sect<int4>(p, p->lay.fwd_items);
  a.flist = sect<uint32_t>(p, p->lay.fwd_list);
  a.bitems = sect<int4>(p, p->lay.bwd_items);
  a.blist = sect<uint32_t>(p, p->lay.bwd_list);
  a.bslot = sect<int>(p, p->lay.bwd_slot);
  a.breduce = sect<int4>(p, p->lay.bwd_reduce);
  a.part = ws ? reinterpret_cast<float *>(static_cast<char *>(const_cast<void *>(ws)) +
                                          ws_stats_bytes(p))
              : nullptr;
  a.dqacc = ws ? reinterpret_cast<float *>(static_cast<char *>(const_cast<void *>(ws)) +
                                           ws_stats_bytes(p) + ws_partial_bytes(p))
               : nullptr;
  a.n_fitems = (int)p->lay.n_fwd_items;
  a.n_bitems = (int)p->lay.n_bwd_items;
  a.n_breduce = (int)p->lay.n_bwd_reduce;
  a.n_slots = (int)p->lay.n_slots;
  a.key_tile = p->bwd_keys;
  a.head_entries = p->bwd_head_entries ? 1 : 0;
  a.m = mask_args(p);
  return a;
}

// Workspace bytes a call uses: the statistics and partial dK/dV slots, and
// the dQ accumulator when the call zeroes, fills or reads it.
size_t ws_need(const attn_plan *p, bool dq_acc) {
  return (size_t)(ws_stats_bytes(p) + ws_partial_bytes(p) + (dq_acc ? ws_dq_bytes(p) : 0));
}

attn_status check_ws(const attn_plan *p, const void *ws, size_t ws_bytes, bool dq_acc) {
  attn_status s = check_tensor(ws, "ws", 256);
  if (s != ATTN_OK) return s;
  if (ws_bytes < ws_need(p, dq_acc))
    return fail(ATTN_ERR_INVALID, "workspace holds %zu bytes; %zu needed%s", ws_bytes, ws_need(p, dq_acc),
                dq_acc ? " (attn_bwd_atomic_workspace_bytes)" : "");
  return ATTN_OK;
}

#define LCM_CHECK(expr)              \
  do {                               \
    attn_status s_ = (expr);         \
    if (s_ != ATTN_OK) return s_;    \
  } while (0)

attn_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_bwd_preprocess(const attn_plan *p, const void *o, const float *lse,
                                           const void *dout, void *ws, size_t ws_bytes,
                                           attn_stream_t stream) {
  clear_error();
  LCM_CHECK(check_plan(p));
  LCM_CHECK(check_tensor(o, "o", 16));
  LCM_CHECK(check_tensor(lse, "lse", 4));
  LCM_CHECK(check_tensor(dout, "dout", 16));
  LCM_CHECK(check_ws(p, ws, ws_bytes, false));
  if (forced_device_error()) return fail(ATTN_ERR_DEVICE, "forced device error (ATTN_FORCE_DEVICE_ERROR)");
  BwdArgs a = bwd_args(p, nullptr, nullptr, nullptr, o, lse, dout, nullptr, nullptr,
                       nullptr, ws);
  a.dqacc = nullptr;
  (void)hipGetLastError();
  return launched(launch_bwd_pre(a, (int)p->shape.d, (int)p->shape.B,
                                 reinterpret_cast<hipStream_t>(stream)), "backward preprocess");
}

extern "C" attn_status attn_bwd_dkdv(const attn_plan *p, const void *q, const void *k,
                                     const void *v, const float *lse, const void *dout,
                                     void *dk, void *dv, const void *ws, size_t ws_bytes,
                                     attn_stream_t stream) {
  clear_error();
  LCM_CHECK(check_plan(p));
  LCM_CHECK(check_tensor(q, "q", 16));
  LCM_CHECK(check_tensor(k, "k", 16));
  LCM_CHECK(check_tensor(v, "v", 16));
  LCM_CHECK(check_tensor(lse, "lse", 4));
  LCM_CHECK(check_tensor(dout, "dout", 16));
  LCM_CHECK(check_tensor(dk, "dk", 16));
  LCM_CHECK(check_tensor(dv, "dv", 16));
  LCM_CHECK(check_ws(p, ws, ws_bytes, false));
  if (forced_device_error()) return fail(ATTN_ERR_DEVICE, "forced device error (ATTN_FORCE_DEVICE_ERROR)");
  const BwdArgs a = bwd_args(p, q, k, v, nullptr, lse, dout, nullptr, dk, dv, ws);
  (void)hipGetLastError();
  return launched(launch_dkdv(a, (int)p->shape.d, (int)p->shape.B, false,
                              reinterpret_cast<hipStream_t>(stream)), "dK/dV");
}

extern "C" attn_status attn_bwd_dq(const attn_plan *p, const void *q, const void *k,
                                   const void *v, const float *lse, const void *dout, void *dq,
                                   const void *ws, size_t ws_bytes, attn_stream_t stream) {
  clear_error();
  LCM_CHECK(check_plan(p));
  LCM_CHECK(check_tensor(q, "q", 16));
  LCM_CHECK(check_tensor(k, "k", 16));
  LCM_CHECK(check_tensor(v, "v", 16));
  LCM_CHECK(check_tensor(lse, "lse", 4));
  LCM_CHECK(check_tensor(dout, "dout", 16));
  LCM_CHECK(check_tensor(dq, "dq", 16));
  LCM_CHECK(check_ws(p, ws, ws_bytes, false));
  if (forced_device_error()) return fail(ATTN_ERR_DEVICE, "forced device error (ATTN_FORCE_DEVICE_ERROR)");
  const BwdArgs a = bwd_args(p, q, k, v, nullptr, lse, dout, dq, nullptr, nullptr, ws);
  (void)hipGetLastError();
  return launched(launch_dq(a, (int)p->shape.d, p->HG, masked_lists(p), (int)p->shape.B,
                            reinterpret_cast<hipStream_t>(stream)), "dQ");
}

namespace {
attn_status bwd_impl(const attn_plan *p, const void *q, const void *k, const void *v,
                     const void *o, const float *lse, const void *dout, void *dq, void *dk,
                     void *dv, void *ws, size_t ws_bytes, attn_stream_t stream, bool fused) {
  clear_error();
  LCM_CHECK(check_plan(p));
  LCM_CHECK(check_tensor(q, "q", 16));
  LCM_CHECK(check_tensor(k, "k", 16));
  LCM_CHECK(check_tensor(v, "v", 16));
  LCM_CHECK(check_tensor(o, "o", 16));
  LCM_CHECK(check_tensor(lse, "lse", 4));
  LCM_CHECK(check_tensor(dout, "dout", 16));
  LCM_CHECK(check_tensor(dq, "dq", 16));
  LCM_CHECK(check_tensor(dk, "dk", 16));
  LCM_CHECK(check_tensor(dv, "dv", 16));
  LCM_CHECK(check_ws(p, ws, ws_bytes, fused));
  if (fused && p->bwd_keys != kBwdKeyTile)
    return fail(ATTN_ERR_UNSUPPORTED, "the fused dQ pass needs 128-key dK/dV items (this plan has %d)",
                p->bwd_keys);
  if (forced_device_error()) return fail(ATTN_ERR_DEVICE, "forced device error (ATTN_FORCE_DEVICE_ERROR)");
  BwdArgs a = bwd_args(p, q, k, v, o, lse, dout, dq, dk, dv, ws);
  if (!fused) a.dqacc = nullptr;  // the recompute pass needs no accumulator
  const int d = (int)p->shape.d, B = (int)p->shape.B;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  LCM_CHECK(launched(launch_bwd_pre(a, d, B, st), "backward preprocess"));
  if (fused) {
    LCM_CHECK(launched(launch_dkdv(a, d, B, true, st), "dK/dV with dQ"));
    return launched(launch_dq_convert(a, d, B, st), "dQ convert");
  }
  LCM_CHECK(launched(launch_dkdv(a, d, B, false, st), "dK/dV"));
  return launched(launch_dq(a, d, p->HG, masked_lists(p), B, st), "dQ");
}
}  // namespace

extern "C" attn_status attn_bwd(const attn_plan *p, const void *q, const void *k, const void *v,
                                const void *o, const float *lse, const void *dout, void *dq,
                                void *dk, void *dv, void *ws, size_t ws_bytes,
                                attn_stream_t stream) {
  return bwd_impl(p, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream, false);
}

extern "C" attn_status attn_bwd_atomic_dq(const attn_plan *p, const void *q, const void *k,
                                          const void *v, const void *o, const float *lse,
                                          const void *dout, void *dq, void *dk, void *dv,
                                          void *ws, size_t ws_bytes, attn_stream_t stream) {
  return bwd_impl(p, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream, true);
}

extern "C" attn_status attn_merge(const float *o1, const float *lse1, const float *o2,
                                  const float *lse2, void *o, int o_bf16, float *lse, int64_t B,
                                  int64_t S, int64_t Hq, int64_t d, attn_stream_t stream) {
  clear_error();
  if (B < 1 || S < 1 || Hq < 1) return fail(ATTN_ERR_INVALID, "B, S, Hq must be >= 1");
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%lld (supported: 64, 128)", (long long)d);
  if (S >= (int64_t(1) << 30) || Hq > 65535 || B > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "S must be < 2^30, B and Hq <= 65535");
  LCM_CHECK(check_tensor(o1, "o1", 16));
  LCM_CHECK(check_tensor(o2, "o2", 16));
  LCM_CHECK(check_tensor(o, "o", 16));
  LCM_CHECK(check_tensor(lse1, "lse1", 4));
  LCM_CHECK(check_tensor(lse2, "lse2", 4));
  LCM_CHECK(check_tensor(lse, "lse", 4));
  // the outputs may not overlap the inputs (every lane of a row reads the
  // row's LSE before one of them writes it) or each other
  const uint64_t rows = (uint64_t)(B * S * Hq);
  const uint64_t ni = rows * (uint64_t)d * 4, no = rows * (uint64_t)d * (o_bf16 ? 2 : 4), nl = rows * 4;
  auto overlap = [](const void *x, uint64_t nx, const void *y, uint64_t ny) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a < b + ny && b < a + nx;
  };
  if (overlap(o, no, o1, ni) || overlap(o, no, o2, ni) || overlap(o, no, lse1, nl) ||
      overlap(o, no, lse2, nl) || overlap(lse, nl, o1, ni) || overlap(lse, nl, o2, ni) ||
      overlap(lse, nl, lse1, nl) || overlap(lse, nl, lse2, nl) || overlap(o, no, lse, nl))
    return fail(ATTN_ERR_INVALID, "outputs overlap the inputs or each other");
  if (forced_device_error()) return fail(ATTN_ERR_DEVICE, "forced device error (ATTN_FORCE_DEVICE_ERROR)");
  (void)hipGetLastError();
  return launched(launch_merge(o1, lse1, o2, lse2, o, o_bf16 != 0, lse, B, (int)S, (int)Hq, (int)d,
                               reinterpret_cast<hipStream_t>(stream)),
                  "merge");
}

// ---------------------------------------------------------------------------
// attn_bwd without a caller workspace, for callers that cannot allocate
// device memory.  The workspace of the backward (LSE * log2(e), -D and the
// partial dK/dV of split items) lives in this file-scope array instead; each
// GPU the library runs on holds one copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not a device address: the
// address of each device's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

attn_status scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(ATTN_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}
}  // namespace

extern "C" size_t attn_bwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

extern "C" attn_status attn_bwd_noalloc(const attn_plan *p, const void *q, const void *k,
                                        const void *v, const void *o, const float *lse,
                                        const void *dout, void *dq, void *dk, void *dv,
                                        attn_stream_t stream) {
  clear_error();
  LCM_CHECK(check_plan(p));
  const size_t need = ws_need(p, false);
  if (need > kScratchBytes)
    return fail(ATTN_ERR_INVALID,
                "attn_bwd_noalloc: this plan needs %zu bytes of workspace; the library's "
                "static workspace holds %zu (use attn_bwd with a caller buffer)",
                need, kScratchBytes);
  void *ws = nullptr;
  LCM_CHECK(scratch_of_current_device(&ws));
  return bwd_impl(p, q, k, v, o, lse, dout, dq, dk, dv, ws, kScratchBytes, stream, false);
}
