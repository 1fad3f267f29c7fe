// Internal plan representation shared by the mask compiler (plan.cpp) and
// the launch code (api.hip).  Not part of the public interface.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "attn.h"

namespace lcm {

// Tile geometry.  Classification runs on 64x64 "micro tiles"; every kernel
// tile is a whole number of them.
constexpr int kMicro = 64;
constexpr int kFwdKeyTile = 64;   // forward / dQ: keys per K-tile
constexpr int kBwdKeyTile = 128;  // dK/dV: keys per workgroup (4 waves x 32); narrow items: 64
constexpr int kBwdRowTile = 64;   // dK/dV: query rows per Q-tile
constexpr int kWgRowsHeads = 128; // forward / dQ: (rows x heads) per workgroup

constexpr uint32_t kPartialBit = 0x80000000u;
constexpr int kHeadShift = 24;   // dK/dV (Q-tile, head) entries: head in bits 24-30
constexpr int kMaxEntryHeads = 128;
constexpr int kMaxDynEntryHeads = 64;  // the device list compiler keeps a 64-bit head mask
constexpr int64_t kMaxMaskWordBytes = int64_t(4) << 30;  // both bitmap word tables
// Class of a 64x64 micro tile (stored as uint8 in a dynamic plan's blob).
enum : uint8_t { kEmpty = 0, kPartial = 1, kFull = 2 };

// Byte offsets of the sections of the device blob (all 256-byte aligned).
struct Layout {
  int64_t rowb = -1, colb = -1;
  int64_t fwd_items = -1, fwd_list = -1, bwd_items = -1, bwd_list = -1;
  int64_t bwd_slot = -1, bwd_reduce = -1;
  int64_t bits = -1, qblk = -1, kblk = -1, qoffs = -1, koffs = -1;
  // static plans whose bitmap blocks cut 64-wide tiles: the bitmap part of
  // the mask as 64-bit words, allowed keys of micro-tile J for row block qb
  // [heads][nqb][nM] and allowed rows of micro-tile I for key block kb
  // [heads][nkb][nM]
  int64_t kwords = -1, rwords = -1;
  // dynamic plans with bitmap words: the blocks each 64-wide tile touches,
  // with the tile bits each covers (CSR by tile: offsets [nM + 1], block
  // indices, masks), so that the device rebuilds the words for a new bitmap
  int64_t dyn_kseg_off = -1, dyn_kseg_blk = -1, dyn_kseg_mask = -1;
  int64_t dyn_rseg_off = -1, dyn_rseg_blk = -1, dyn_rseg_mask = -1;
  int64_t n_fwd_items = 0, n_fwd_list = 0, n_bwd_items = 0, n_bwd_list = 0;
  int64_t n_bwd_reduce = 0, n_slots = 0;
  // dynamic plans only: base micro-tile classes, (length, partial tiles) of
  // every list, and the per-XCD-share reorder tables of both passes
  int64_t dyn_base = -1, dyn_len = -1;
  int64_t dyn_fshare = -1, dyn_fpos = -1, dyn_fnat = -1;
  int64_t dyn_bshare = -1, dyn_bpos = -1, dyn_bnat = -1;
  int64_t total = 0;
};

// What the device list builder of a dynamic plan needs.  List group g of
// the forward covers mask heads [g * fheads, (g + 1) * fheads) and owns the
// forward lists of slots [g * nFQ, (g + 1) * nFQ), one per Q-tile; likewise
// the dK/dV groups with bheads and nBK.  Every forward list has room for nM
// entries at list + slot * nM, every dK/dV list for bcap entries at
// list + slot * bcap: nM, or nM * bheads when its entries are (Q-tile, head)
// stages (bhe).  The items of each pass are dealt to XCD shares
// (fixed at creation); a share's items are re-sorted, longest first, within
// the share's positions of the item array.
// Sort key of the device's re-sort of an XCD share (ascending order): the
// item's cost descending, ties by its natural index i < 2^16; or, when the
// share holds several KV heads, the KV head first.  share_sort_index
// recovers i from either layout.
constexpr uint64_t share_sort_key(bool head_major, uint32_t kvh, uint32_t cost, uint32_t i) {
  return head_major ? ((uint64_t)(kvh & 0xffffu) << 48) | ((uint64_t)(0xffffffffu - cost) << 16) | (i & 0xffffu)
                    : ((uint64_t)(0xffffffffu - cost) << 32) | (i & 0xffffu);
}
constexpr uint32_t share_sort_index(uint64_t key) { return (uint32_t)(key & 0xffffu); }

struct DynInfo {
  bool on = false;
  int64_t nM = 0, nFQ = 0, nBK = 0;
  int64_t n_fslots = 0, n_bslots = 0;
  int MR = 1, MC = 2, fheads = 1, bheads = 1;
  int n_fshares = 1, n_bshares = 1;
  bool bhe = false;
  int64_t bcap = 0;
  bool head_major = false;  // shares sorted by KV head, then cost (several heads per XCD)
  int fkv = 1;              // query heads per KV head
};

// dK/dV items whose work exceeds the share of one workgroup are split into
// chunks, each a run of the item's listed Q-tiles; a chunk writes fp32
// partial dK/dV into a slot of the caller's workspace and a reduce pass sums
// the chunks of each split item in a fixed order.
constexpr int kSplitTarget = 256;  // dK/dV workgroups resident at once (one per CU)
constexpr int kSplitMax = 16;      // chunks per item at most

}  // namespace lcm

struct attn_plan {
  attn_shape shape{};
  int32_t n_slots = 0;  // partial-result slots of split dK/dV items
  float scale = 0.f;
  int G = 1;            // query heads per KV head
  int HG = 1;           // query heads per forward / dQ workgroup
  int fwd_rows = 128;   // query rows per forward / dQ workgroup
  int bwd_keys = 128;   // keys per dK/dV work item: 128, or 64 (two waves)
  bool bwd_head_entries = false;  // dK/dV lists hold (Q-tile, query head) stages
  int bitmap_heads = 0; // 0 = no bitmap
  int nqb = 0, nkb = 0;
  std::vector<uint8_t> blob;  // host copy of the device blob
  lcm::Layout lay;
  lcm::DynInfo dyn;
  attn_stats stats{};
  void *dev_blob = nullptr;
  size_t dev_bytes = 0;
};

namespace lcm {
// Backward workspace: lse2 and D per (b, h, row), rows padded to 64, then
// the fp32 partial dK/dV of split items, [B][slot][dK, dV][128 keys][d].
inline int64_t ws_stats_bytes(const attn_plan *p) {
  const int64_t s64 = (p->shape.S + 63) / 64 * 64;
  return (p->shape.B * p->shape.Hq * s64 * 8 + 255) & ~int64_t(255);
}
inline int64_t ws_partial_bytes(const attn_plan *p) {
  return p->shape.B * (int64_t)p->n_slots * 2 * kBwdKeyTile * p->shape.d * 4;
}
// fp32 dQ accumulator of the fused dK/dV pass: [B][S64][Hq][d].
inline int64_t ws_dq_bytes(const attn_plan *p) {
  const int64_t s64 = (p->shape.S + 63) / 64 * 64;
  return p->shape.B * s64 * p->shape.Hq * p->shape.d * 4;
}

// Thread-local last error (defined in plan.cpp).
attn_status fail(attn_status s, const char *fmt, ...);
void clear_error();
}  // namespace lcm
