/*
 * attn.h -- masked attention, forward and backward, for MI355X (gfx950).
 *
 * Computes O = softmax(mask(Q K^T * scale)) V and its gradients, the core
 * attention of "FlashAttention vs. RingAttention" (dtcms), FlashAttention-1
 * "problem and bottleneck" (softmax(Q K^T / sqrt(d_k)) V), under the mask
 * families of the "Long-Context Attention Benchmark" review (xllm-io),
 * section 3 "mask taxonomy".  That review's kernel adapter gives all kernels
 * one input representation; this header is that representation for one GPU.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every call returns attn_status.  On any status other than ATTN_OK,
 *   attn_last_error() returns a message (thread-local, valid until the next
 *   call on the same thread).  No C++ exception crosses this interface.
 * - All validation happens before any GPU work is enqueued: on an error
 *   nothing is launched and no output buffer is written.
 * - The library allocates no device memory.  The caller allocates and owns
 *   every device buffer (tensors, workspace, the plan's device blob) and keeps
 *   it alive until the work enqueued on `stream` has completed.
 * - Device tensors are contiguous, bf16 unless stated, 16-byte aligned:
 *     Q, O, dO, dQ : [B, S, Hq,  d]   (d innermost)
 *     K, V, dK, dV : [B, S, Hkv, d]
 *     LSE          : [B, Hq, S] float32, natural log of the softmax
 *                    normaliser (the single merged statistic of
 *                    FlashAttention-2, "core optimisations"); -inf on a row
 *                    that no key may attend to (whose O row is then 0).
 *   Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 * - Sq = Sk = S: self-attention over one packed sequence per batch entry;
 *   the mask is the same for every batch entry.
 * - Supported: d in {64, 128}, Hq % Hkv == 0, 1 <= S < 2^30.
 * - Launches are asynchronous on `stream` (a hipStream_t; NULL is the null
 *   stream).  Device faults surface at the caller's next synchronisation.
 */
#ifndef LCM_ATTN_H
#define LCM_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *attn_stream_t; /* same object as hipStream_t */

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* malformed argument or descriptor            */
  ATTN_ERR_UNSUPPORTED = 2, /* well-formed but outside what is implemented */
  ATTN_ERR_NOMEM = 3,       /* host allocation failed                      */
  ATTN_ERR_DEVICE = 4       /* a HIP call or kernel launch failed          */
} attn_status;

/*
 * Mask families.  i is the query row, j the key column, both in [0, S).
 *   FULL           every pair allowed.
 *   CAUSAL         j <= i.
 *   SLIDING        i - j < window_left and j - i < window_right; with
 *                  causal = 1 also j <= i (window_right is then ignored).
 *                  CAUSAL SLIDING WINDOW w: window_left = w, causal = 1
 *                  (w keys including the diagonal); FULL SLIDING WINDOW w:
 *                  window_left = window_right = w (|i - j| < w).
 *   DOCUMENT       doc(i) == doc(j) for documents cut by cu_seqlens; with
 *                  causal = 1 also j <= i.
 *   PREFIX_LM      doc(i) == doc(j) and (j < start(doc) + prefix_lens[doc]
 *                  or j <= i).  One document of length S is PREFIX LM CAUSAL.
 *   COLUMN_BOUNDS  per key column j, four int32 {lts, lte, uts, ute}: row i
 *                  is masked for column j iff lts <= i < lte or
 *                  uts <= i < ute (the column-wise representation the review
 *                  attributes to FlashMask).  Any of the twelve static
 *                  families can be written this way; SHARED QUESTION, GLOBAL
 *                  SLIDING, CAUSAL BLOCKWISE and BLOCK CAUSAL DOCUMENT are.
 *                  Each query row must end up with at most two maximal runs
 *                  of allowed keys (true of all twelve families), else
 *                  ATTN_ERR_UNSUPPORTED.
 * Optional block bitmap (the review's dynamic block masks, uniform such as
 * 64x64 or variable-size): the final mask is base(i, j) AND
 * bitmap[hm][qblk(i)][kblk(j)], where qblk(i) is the b with
 * q_blk_offsets[b] <= i < q_blk_offsets[b+1] (likewise kblk) and hm is the
 * bitmap head of query head h: 0 if bitmap_heads == 1, h / (Hq / Hkv) if
 * bitmap_heads == Hkv, h if bitmap_heads == Hq.
 * With dynamic = 1 the plan keeps room for every work list at its largest
 * and the bitmap can be replaced on the device, without a new plan, by
 * attn_plan_set_bitmap (content-adaptive block masks, whose bitmap changes
 * from step to step).
 */
typedef enum {
  ATTN_MASK_FULL = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_SLIDING = 2,
  ATTN_MASK_DOCUMENT = 3,
  ATTN_MASK_PREFIX_LM = 4,
  ATTN_MASK_COLUMN_BOUNDS = 5
} attn_mask_kind;

typedef struct {
  int64_t B, S, Hq, Hkv, d;
  float scale; /* softmax scale; 0 selects 1/sqrt(d) */
} attn_shape;

/* All arrays are host memory, read during attn_plan_create only (copied). */
typedef struct {
  int32_t kind;                  /* attn_mask_kind                              */
  int32_t causal;                /* SLIDING, DOCUMENT: 0 or 1                   */
  int32_t window_left;           /* SLIDING: >= 1                               */
  int32_t window_right;          /* SLIDING with causal = 0: >= 1               */
  int32_t num_docs;              /* DOCUMENT, PREFIX_LM: >= 1                   */
  const int32_t *cu_seqlens;     /* [num_docs+1], 0 = c_0 < c_1 < ... = S       */
  const int32_t *prefix_lens;    /* PREFIX_LM: [num_docs], 0 <= p_k <= len_k    */
  const int32_t *col_bounds;     /* COLUMN_BOUNDS: [S][4], each in [0, S]       */
  const uint8_t *block_bitmap;   /* optional: [bitmap_heads][n_qblk][n_kblk]   */
  int32_t bitmap_heads, n_qblk, n_kblk;
  const int32_t *q_blk_offsets;  /* [n_qblk+1], 0 = o_0 < ... < o_n = S        */
  const int32_t *k_blk_offsets;  /* [n_kblk+1], likewise                       */
  int32_t dynamic;               /* 0, or 1 (needs block_bitmap): the bitmap
                                    may later be replaced by
                                    attn_plan_set_bitmap                         */
  int32_t bwd_key_tile;          /* keys per dK/dV work item: 0 lets the plan
                                    choose, else 128 or 64.  Results do not
                                    depend on it beyond fp32 summation
                                    order.                                     */
} attn_mask_desc;

typedef struct attn_plan attn_plan;

typedef struct {
  int64_t nnz_per_batch;   /* allowed (i,j) pairs summed over the Hq heads   */
  int64_t nnz_total;       /* nnz_per_batch * B                              */
  double flops_fwd;        /* 4 * d * nnz_total  (QK^T and PV)               */
  double flops_bwd;        /* 10 * d * nnz_total (five products)             */
  int64_t fwd_items, fwd_tiles_full, fwd_tiles_partial;   /* forward / dQ    */
  int64_t bwd_items, bwd_tiles_full, bwd_tiles_partial;   /* dK/dV pass      */
  int64_t fwd_tile_rows, fwd_tile_cols, bwd_tile_rows, bwd_tile_cols;
  int64_t heads_per_item;  /* query heads sharing one K/V tile in fwd / dQ   */
  int64_t device_bytes;    /* size of the device blob                        */
  int64_t bwd_head_entries; /* 1: each dK/dV list entry is one (Q-tile, query
                              head) stage, the head in bits 24-30 (one bitmap
                              per query head under GQA, static plans); 0: an
                              entry is a Q-tile for all heads of the group  */
} attn_stats;

/*
 * Compile the mask for `shape`: validate, classify every (Q-tile, K-tile)
 * pair as empty, full or partial, build the per-Q-tile (forward, dQ) and
 * per-K-tile (dK/dV) work lists and order them longest-first.  Host only: no
 * HIP call is made.  On success *out owns host memory only.  A dK/dV work
 * item spans 128 keys, or 64 (two waves) when desc->bwd_key_tile = 64 or,
 * with bwd_key_tile = 0, when more than a quarter of the listed 128-key
 * tiles of the first item group have an empty 64-key half (bitmap blocks 64
 * keys wide; a dynamic plan decides on its creation bitmap);
 * stats.bwd_tile_cols reports it.  bwd_key_tile outside {0, 64, 128} is
 * ATTN_ERR_INVALID.  The lists of different mask heads (or, with one bitmap
 * per query head, KV heads) are built on up to 16 host threads of the
 * calling process and joined in head order, so the plan is the same for any
 * thread count; the call returns after every thread has joined.
 */
attn_status attn_plan_create(const attn_shape *shape, const attn_mask_desc *desc,
                             attn_plan **out);

/* Bytes of device memory the caller must provide to attn_plan_bind. */
size_t attn_plan_device_bytes(const attn_plan *plan);

/*
 * Copy the plan's metadata (work lists, row/column bounds, bitmap) into the
 * caller's device buffer `dev_buf` (>= attn_plan_device_bytes, 256-byte
 * aligned) with an asynchronous host-to-device copy on `stream`, and record
 * the buffer in the plan.  Must precede attn_fwd / attn_bwd; binding again
 * replaces the recorded buffer.  Not thread-safe against concurrent use of
 * the same plan.
 */
attn_status attn_plan_bind(attn_plan *plan, void *dev_buf, size_t bytes,
                           attn_stream_t stream);

/*
 * Replace the block bitmap of a dynamic plan on the device and rebuild its
 * work lists there, for the dynamic block-sparse masks of the
 * "Long-Context Attention Benchmark" review (xllm-io), "paper summary",
 * innovation 3: the blocks are chosen from the input, so the bitmap changes
 * every step and the lists cannot wait for a host compile.
 *
 *   bits  device memory, uint8 [bitmap_heads][n_qblk][n_kblk] in the block
 *         partition the plan was created with; nonzero = block allowed.
 *         16-byte aligned, must not overlap the plan's device buffer; read
 *         by work enqueued on `stream` only (the caller keeps it alive and
 *         unchanged until that work has run).
 *
 * Enqueues two kernels on `stream`: the first copies the bitmap into the
 * plan's buffer and rebuilds every forward / dQ and dK/dV list, the second
 * stores each work item's new length.  The lists equal, entry for entry,
 * those attn_plan_create would build for the new bitmap; the order of the
 * work items stays the one chosen at creation, and no dK/dV item is split.
 * Later attn_fwd / attn_bwd calls on `stream` see the new mask; calls on
 * other streams must be ordered after it by the caller.  attn_plan_stats
 * and attn_plan_get_layout keep describing the creation bitmap, and binding
 * the plan again uploads that bitmap and its lists.
 *
 * Errors: ATTN_ERR_INVALID for a NULL or unbound plan, a plan created
 * without dynamic = 1, a NULL, misaligned or overlapping `bits`;
 * ATTN_ERR_DEVICE if a launch fails.  Nothing is enqueued on an error.
 */
attn_status attn_plan_set_bitmap(attn_plan *plan, const uint8_t *bits, attn_stream_t stream);

attn_status attn_plan_stats(const attn_plan *plan, attn_stats *out);

/* Host view of the device blob and its section offsets (tests, tooling). */
typedef struct {
  const void *blob;
  int64_t blob_bytes;
  int64_t off_rowb, off_colb;           /* int32 [S][4] each               */
  int64_t off_fwd_items, n_fwd_items;   /* int32 [n][4]: tile, h0, off, len */
  int64_t off_fwd_list, n_fwd_list;     /* uint32 [n]: tile | partial<<31  */
  int64_t off_bwd_items, n_bwd_items;   /* int32 [n][4]: tile, kvh, off, len */
  int64_t off_bwd_list, n_bwd_list;     /* uint32 [n]                      */
  int64_t off_bits, off_qblk, off_kblk, off_qoffs, off_koffs; /* -1 if none */
  /* int32 [n_bwd_items], parallel to the dK/dV items: the partial slot of an
   * item that is one chunk of a split (K-tile, KV head), or -1 when the item
   * writes dK/dV itself.  The chunks of a split item list consecutive runs
   * of its Q-tiles, in slot order. */
  int64_t off_bwd_slot;
  /* int32 [n][4]: K-tile, KV head, first slot, number of chunks, for each
   * dK/dV item split into chunks whose partial results are summed. */
  int64_t off_bwd_reduce, n_bwd_reduce;
  int64_t n_slots;                      /* partial slots per batch entry    */
  /* uint64 [bitmap heads][n_qblk][ceil(S/64)]: allowed keys of 64-key tile t
   * for rows of bitmap row block qb (bit c: key 64 t + c), and uint64
   * [bitmap heads][n_kblk][ceil(S/64)]: allowed rows of 64-row tile t for
   * keys of column block kb; the bitmap part of the mask only.  Plans whose
   * blocks cut 64-wide tiles, up to 4 GiB for both (dynamic plans: for the
   * creation bitmap; attn_plan_set_bitmap rebuilds them on the device);
   * else -1. */
  int64_t off_kwords, off_rwords;
} attn_plan_layout;

attn_status attn_plan_get_layout(const attn_plan *plan, attn_plan_layout *out);

/* Bytes of device workspace attn_bwd needs: per (b, h, row) the fp32 values
 * LSE * log2(e) and -D, D = rowsum(dO * O), rows padded to a multiple of 64,
 * then, when the plan split long dK/dV work items into chunks (small S, or
 * key columns seen by every row), fp32 partial dK and dV of 128 keys per
 * chunk slot and batch entry. */
size_t attn_bwd_workspace_bytes(const attn_plan *plan);
/* Bytes of device workspace attn_bwd_atomic_dq needs: attn_bwd's, then the
 * fp32 dQ accumulator [B][S rounded up to 64][Hq][d] (4 bytes per element of
 * dQ: 1.6 GB at S = 48K, Hq = 64, d = 128). */
size_t attn_bwd_atomic_workspace_bytes(const attn_plan *plan);

/*
 * Forward: O and LSE.  Q-split: one workgroup per (Q-tile, group of query
 * heads sharing a KV head), iterating over its non-empty K-tiles (the Q-split
 * of FlashAttention-2, "core optimisations"; online softmax with deferred
 * rescaling of FlashAttention-1/2).
 */
attn_status attn_fwd(const attn_plan *plan, const void *q, const void *k,
                     const void *v, void *o, float *lse, attn_stream_t stream);

/*
 * Backward: dQ, dK, dV from Q, K, V, the forward's O and LSE, and dO.  The
 * dependency dQ_i = sum_j dS_ij K_j makes the backward parallel over both
 * rows and columns ("FlashAttention vs. RingAttention", FlashAttention-2
 * "core optimisations").  Three launches on `stream`: -D, D = rowsum(dO * O),
 * and LSE * log2(e) into `ws`; a KV-split pass (one workgroup per K-tile and
 * KV head) accumulating dK and dV in registers; a Q-split pass (one
 * workgroup per Q-tile and head group) recomputing S and dP and accumulating
 * dQ = scale * sum_j dS_ij K_j in registers.  dK and dV of a KV head are
 * summed over its query-head group.  No atomics: every output is the same
 * bit for bit from run to run.  `ws` is a device buffer of at least
 * attn_bwd_workspace_bytes(plan) bytes, 256-byte aligned.
 */
attn_status attn_bwd(const attn_plan *plan, const void *q, const void *k,
                     const void *v, const void *o, const float *lse,
                     const void *dout, void *dq, void *dk, void *dv, void *ws,
                     size_t ws_bytes, attn_stream_t stream);

/*
 * attn_bwd with dQ accumulated inside the KV-split pass instead of a second
 * pass: every wave writes its bf16 dS to LDS, and after the next stage's
 * barrier computes dQ of the stage's rows for its own columns of d from the
 * transposed dS tile and a slice of K in registers, adding it into a zeroed
 * fp32 accumulator in `ws` with atomics; a last launch writes
 * dQ = scale * accumulator in bf16.  It saves the recomputation of S and dP,
 * at the price of one fp32 atomic addition per (row, key) pair at d = 128;
 * measured on MI355X it is about half as fast as attn_bwd, so attn_bwd is
 * the default.  The order of the atomic additions varies, so dQ may differ
 * in its last bit from run to run.  Same arguments as attn_bwd, with `ws` of
 * at least attn_bwd_atomic_workspace_bytes(plan) bytes.  Needs 128-key dK/dV
 * items: a plan with 64-key items returns ATTN_ERR_UNSUPPORTED before any
 * launch.
 */
attn_status attn_bwd_atomic_dq(const attn_plan *plan, const void *q, const void *k,
                               const void *v, const void *o, const float *lse,
                               const void *dout, void *dq, void *dk, void *dv, void *ws,
                               size_t ws_bytes, attn_stream_t stream);

/*
 * attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same backward, with its workspace in a static device array that the
 * library holds on every GPU it runs on until the process ends, instead of a
 * caller buffer.  The caller still passes the bound plan, the inputs and the
 * outputs.  Plans whose workspace (attn_bwd_workspace_bytes) exceeds
 * attn_bwd_noalloc_max_workspace_bytes() (128 MiB) are rejected with
 * ATTN_ERR_INVALID before anything is launched.  Calls no allocation
 * routine.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race and must
 * be serialised by the caller.  The backward writes every workspace value
 * it reads, so nothing left by an earlier call is used.  The device is the
 * current one, which must be the stream's.
 */
attn_status attn_bwd_noalloc(const attn_plan *plan, const void *q, const void *k,
                             const void *v, const void *o, const float *lse,
                             const void *dout, void *dq, void *dk, void *dv,
                             attn_stream_t stream);
size_t attn_bwd_noalloc_max_workspace_bytes(void);

/*
 * The three stages of attn_bwd, callable one at a time on the same stream
 * and in this order (attn_bwd is exactly these three calls).  They exist so
 * that callers can interleave other work between stages and time them.
 *   attn_bwd_preprocess: ws <- LSE * log2(e) and -D, D = rowsum(dO * O), fp32.
 *   attn_bwd_dkdv:       dK, dV from Q, K, V, dO and the values in ws.
 *   attn_bwd_dq:         dQ from Q, K, V, dO and the values in ws.
 * Arguments have the meaning and requirements given for attn_bwd.
 */
attn_status attn_bwd_preprocess(const attn_plan *plan, const void *o, const float *lse,
                                const void *dout, void *ws, size_t ws_bytes,
                                attn_stream_t stream);
attn_status attn_bwd_dkdv(const attn_plan *plan, const void *q, const void *k,
                          const void *v, const float *lse, const void *dout, void *dk,
                          void *dv, const void *ws, size_t ws_bytes, attn_stream_t stream);
attn_status attn_bwd_dq(const attn_plan *plan, const void *q, const void *k,
                        const void *v, const float *lse, const void *dout, void *dq,
                        const void *ws, size_t ws_bytes, attn_stream_t stream);

/*
 * Partial results for attention over chunks of the keys, the one-GPU
 * building block of ring-style sequence parallelism ("FlashAttention vs.
 * RingAttention", Ring Attention section: the Blockwise Parallel Transformer
 * computes each query block against one key/value block at a time and
 * rescales each block's output by the difference between its own softmax
 * normaliser and the global one).
 *
 * attn_fwd_partial: attn_fwd with O written in fp32 ([B, S, Hq, d], 16-byte
 * aligned): the chunk's attention output, normalised by its own sum, and its
 * LSE.  A chunk is a plan whose mask keeps only that chunk's keys (for
 * instance a block bitmap with one row block and one column block per
 * chunk).
 *
 * attn_merge: the O and LSE over the union of two disjoint key sets, from the
 * results over each set:
 *   LSE = ln(exp(LSE1) + exp(LSE2)),
 *   O   = exp(LSE1 - LSE) O1 + exp(LSE2 - LSE) O2.
 *   o1, o2:          [B, S, Hq, d] fp32, 16-byte aligned (attn_fwd_partial
 *                    results, or earlier merges);
 *   o:               [B, S, Hq, d], fp32 when o_bf16 == 0 (to merge further),
 *                    bf16 otherwise (the final O), 16-byte aligned;
 *   lse1, lse2, lse: [B, Hq, S] fp32, natural log, -inf on rows with no key
 *                    in that part, 4-byte aligned.
 * A row with no key in either part gets O = 0 and LSE = -inf.  The outputs
 * may not overlap the inputs or each other.  Allocates nothing; enqueues one
 * kernel on `stream`.  Errors: ATTN_ERR_INVALID (NULL or misaligned pointer,
 * non-positive size, overlapping buffers), ATTN_ERR_UNSUPPORTED (d not 64 or
 * 128, S >= 2^30, B or Hq > 65535), ATTN_ERR_DEVICE (launch failure).
 *
 * The backward over a chunk is attn_bwd with the chunk's plan and the merged
 * (bf16) O and LSE: it gives the chunk's share of dQ (the shares add up to
 * dQ) and dK, dV of the chunk's keys (zero for the other keys).
 */
attn_status attn_fwd_partial(const attn_plan *plan, const void *q, const void *k,
                             const void *v, float *o, float *lse, attn_stream_t stream);
attn_status attn_merge(const float *o1, const float *lse1, const float *o2, const float *lse2,
                       void *o, int o_bf16, float *lse, int64_t B, int64_t S, int64_t Hq,
                       int64_t d, attn_stream_t stream);

void attn_plan_destroy(attn_plan *plan);

/*
 * Calls that take the shape and the mask descriptor directly, for callers
 * that do not keep plans: the one input representation of the
 * "Long-Context Attention Benchmark" review (xllm-io), section 3, components
 * table (the kernel adapter), with the compiled mask cached.
 *
 * Plan cache.  The library compiles each distinct (shape, descriptor
 * content) once and keeps the host plan in a process-wide cache of at most
 * ATTN_DESC_CACHE_PLANS plans, least recently used evicted first; lookups
 * compare the full content (shape, scalars and every array the kind reads),
 * so equal masks from different arrays share a plan and different masks
 * never do.  All calls below are thread-safe against each other.
 *
 * Plan buffer.  The plan's device blob lives in `plan_buf`, device memory
 * the caller provides (>= the plan bytes that attn_desc_plan_bytes returns,
 * 256-byte aligned) and dedicates to the cache: the library records which
 * plan's blob each buffer holds and uploads (synchronising `stream`) only
 * when a call passes a buffer that holds another plan's blob or none.  The
 * caller must not write to a plan buffer, and must call
 * attn_desc_release(plan_buf) before freeing or reusing its memory.  One
 * buffer per mask avoids uploads; a single buffer shared by several masks
 * works, with an upload whenever the mask changes.
 *
 * Descriptors with dynamic = 1 are rejected (ATTN_ERR_INVALID): a dynamic
 * plan is updated in place and is not shareable.  Errors are those of
 * attn_plan_create, attn_plan_bind and attn_fwd / attn_bwd.
 */
#define ATTN_DESC_CACHE_PLANS 32

/* Compile (or find) the plan of (shape, desc).  Outputs, each optional
 * (NULL to skip): the plan buffer size, the attn_bwd workspace size, and a
 * 64-bit hash of the cache key (equal masks give equal hashes; a caller may
 * use it to keep one plan buffer per mask). */
attn_status attn_desc_plan_bytes(const attn_shape *shape, const attn_mask_desc *desc,
                                 size_t *plan_bytes, size_t *ws_bytes, uint64_t *key_hash);

/* attn_fwd on the cached plan of (shape, desc), its blob in plan_buf. */
attn_status attn_fwd_desc(const attn_shape *shape, const attn_mask_desc *desc, const void *q,
                          const void *k, const void *v, void *o, float *lse, void *plan_buf,
                          size_t plan_buf_bytes, attn_stream_t stream);

/* attn_bwd on the cached plan of (shape, desc), its blob in plan_buf. */
attn_status attn_bwd_desc(const attn_shape *shape, const attn_mask_desc *desc, const void *q,
                          const void *k, const void *v, const void *o, const float *lse,
                          const void *dout, void *dq, void *dk, void *dv, void *ws,
                          size_t ws_bytes, void *plan_buf, size_t plan_buf_bytes,
                          attn_stream_t stream);

/* Forget that plan_buf holds a plan blob (call before freeing or reusing
 * it).  Unknown buffers are ignored.  Never fails. */
void attn_desc_release(void *plan_buf);

/* Empty the plan cache (all plans destroyed, all buffers forgotten). */
void attn_desc_cache_clear(void);

const char *attn_last_error(void);

/* Library version string. */
const char *attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LCM_ATTN_H */
