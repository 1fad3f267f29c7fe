"""Mask descriptors for the LongCA-bench families.

Turns a mask spec (a plain dict: family name plus parameters, as produced by
the ``synthetic`` package or written by hand) into the C descriptor of
include/attn.h.  The regular families map to their own descriptor kinds; the
heterogeneous ones (SHARED QUESTION, GLOBAL SLIDING, CAUSAL BLOCKWISE, BLOCK
CAUSAL DOCUMENT) are written as per-column masked row intervals, the
column-wise representation that the "Long-Context Attention Benchmark"
review (xllm-io, section 3, dense-kernel table) attributes to FlashMask.

Readings of the families (the review names them only):
  CAUSAL SLIDING WINDOW w: 0 <= i - j < w;  FULL SLIDING WINDOW w: |i - j| < w.
  PREFIX LM CAUSAL p: j < p or j <= i.
  SHARED QUESTION: causal; answers see the question and themselves only.
  GLOBAL SLIDING g, w: causal; j < g or i - j < w (bidirectional variant:
    j < g or i < g or |i - j| < w).
  CAUSAL BLOCKWISE b: rows of every block but the last are causal inside their
    block; rows of the last block are causal over everything (block-causal
    variant: blk(j) <= blk(i)).
  PREFIX LM DOCUMENT: the prefix-LM rule inside each document.
  BLOCK CAUSAL DOCUMENT b: same document and blk(j) <= blk(i), blocks counted
    from the document start.
  TASK BATCH: token-level tasks fused into one launch; task t is a segment of
    kv_t context tokens whose last q_t are queries, causal inside the segment;
    its other rows have no keys.
A block bitmap, when present, is ANDed with the family.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib as L


def _i32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64).astype(np.int32))


def _cu(lens):
    return _i32(np.concatenate([[0], np.cumsum(lens)]))


def column_bounds(spec):
    """[S, 4] int32 masked row intervals {lts, lte, uts, ute} per key column
    for the families written in column form."""
    S = int(spec["S"])
    j = np.arange(S, dtype=np.int64)
    cb = np.zeros((S, 4), dtype=np.int64)
    fam = spec["family"]
    if fam == "shared_question":
        q = int(spec["question"])
        ends = np.cumsum([q] + list(spec["answers"]))
        seg_end = ends[np.searchsorted(ends, j, side="right")]  # end of j's segment
        ans = j >= q
        cb[:, 0] = np.where(ans, seg_end, 0)
        cb[:, 1] = np.where(ans, S, 0)
        cb[:, 3] = j                       # rows above the diagonal
    elif fam == "global_sliding":
        g, w = int(spec["globals"]), int(spec["window"])
        if spec.get("bidirectional", False):
            loc = j >= g
            cb[:, 0] = np.where(loc, np.minimum(S, j + w), 0)
            cb[:, 1] = np.where(loc, S, 0)
            cb[:, 2] = np.where(loc, g, 0)
            cb[:, 3] = np.where(loc, np.maximum(g, j - w + 1), 0)
        else:
            loc = j >= g
            cb[:, 0] = np.where(loc, np.minimum(S, j + w), 0)
            cb[:, 1] = np.where(loc, S, 0)
            cb[:, 3] = j
    elif fam == "causal_blockwise":
        b = int(spec["block"])
        n = (S + b - 1) // b
        blk = j // b
        if spec.get("reading", "last_block_global") == "block_causal":
            cb[:, 3] = blk * b
        else:
            s_last = (n - 1) * b
            early = blk < n - 1
            cb[:, 0] = np.where(early, np.minimum(S, (blk + 1) * b), 0)
            cb[:, 1] = np.where(early, s_last, 0)
            cb[:, 3] = j
    elif fam == "block_causal_document":
        b = int(spec["block"])
        lens = np.asarray(spec["doc_lens"], dtype=np.int64)
        ends = np.cumsum(lens)
        starts = ends - lens
        doc = np.searchsorted(ends, j, side="right")
        bstart = starts[doc] + ((j - starts[doc]) // b) * b
        cb[:, 0] = ends[doc]
        cb[:, 1] = S
        cb[:, 3] = bstart
    elif fam == "task_batch":
        lens = np.asarray(spec["kv_lens"], dtype=np.int64)
        ql = np.asarray(spec["q_lens"], dtype=np.int64)
        ends = np.cumsum(lens)
        seg = np.searchsorted(ends, j, side="right")
        cb[:, 0] = ends[seg]                              # rows after the segment
        cb[:, 1] = S
        cb[:, 3] = np.maximum(j, ends[seg] - ql[seg])     # earlier rows, non-query rows
    else:
        raise ValueError(f"family {fam!r} has its own descriptor kind")
    return _i32(cb)


class MaskDescriptor:
    """A C ``attn_mask_desc`` plus the arrays it points to (kept alive here)."""

    def __init__(self, spec):
        self.spec = spec
        self.S = int(spec["S"])
        self._keep = []
        d = L.MaskDesc()
        fam = spec["family"]
        if fam == "full":
            d.kind = L.MASK_FULL
        elif fam == "causal":
            d.kind = L.MASK_CAUSAL
        elif fam == "sliding":
            d.kind = L.MASK_SLIDING
            w = int(spec["window"])
            d.causal = 1 if spec["causal"] else 0
            d.window_left = w
            d.window_right = 1 if spec["causal"] else w
        elif fam == "document":
            d.kind = L.MASK_DOCUMENT
            d.causal = 1 if spec["causal"] else 0
            self._set_docs(d, spec["doc_lens"])
        elif fam == "prefix_lm_causal":
            d.kind = L.MASK_PREFIX_LM
            self._set_docs(d, [self.S])
            d.prefix_lens = self._ptr32(_i32([spec["prefix"]]))
        elif fam == "prefix_lm_document":
            d.kind = L.MASK_PREFIX_LM
            self._set_docs(d, spec["doc_lens"])
            d.prefix_lens = self._ptr32(_i32(spec["prefix_lens"]))
        elif fam in ("shared_question", "global_sliding", "causal_blockwise",
                     "block_causal_document", "task_batch"):
            d.kind = L.MASK_COLUMN_BOUNDS
            d.col_bounds = self._ptr32(column_bounds(spec))
        elif fam == "column_bounds":
            d.kind = L.MASK_COLUMN_BOUNDS
            d.col_bounds = self._ptr32(_i32(spec["col_bounds"]).reshape(-1, 4))
        else:
            raise ValueError(f"unknown mask family {fam!r}")
        bm = spec.get("bitmap")
        if bm is not None:
            bits = np.ascontiguousarray(bm["bits"], dtype=np.uint8)
            assert bits.ndim == 3
            self._keep.append(bits)
            d.block_bitmap = bits.ctypes.data_as(L.PU8)
            d.bitmap_heads, d.n_qblk, d.n_kblk = (int(x) for x in bits.shape)
            d.q_blk_offsets = self._ptr32(_i32(bm["q_offsets"]))
            d.k_blk_offsets = self._ptr32(_i32(bm["k_offsets"]))
        d.dynamic = 1 if spec.get("dynamic") else 0
        d.bwd_key_tile = int(spec.get("bwd_key_tile", 0))
        d._arrays = self._keep   # the struct keeps the arrays it points to alive
        self.c = d

    def _ptr32(self, arr):
        self._keep.append(arr)
        return arr.ctypes.data_as(L.P32)

    def _set_docs(self, d, lens):
        cu = _cu(lens)
        d.num_docs = len(cu) - 1
        d.cu_seqlens = self._ptr32(cu)
