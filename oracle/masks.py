"""Mask predicates mask(i, j) for the LongCA-bench families, vectorised.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The families are named in the "Long-Context Attention Benchmark" review
(xllm-io), section 3, mask taxonomy: six regular masks (FULL, CAUSAL, FULL /
CAUSAL SLIDING WINDOW, FULL / CAUSAL DOCUMENT), six heterogeneous ones (SHARED
QUESTION, GLOBAL SLIDING, CAUSAL BLOCKWISE, PREFIX LM CAUSAL, PREFIX LM
DOCUMENT, BLOCK CAUSAL DOCUMENT) and two dynamic block masks (uniform, e.g.
64x64, and variable-size blocks).  The page gives names only; each predicate
below states the reading it takes.  ``i`` is the query row, ``j`` the key
column, both in [0, S) of one packed sequence (Sq = Sk = S).

``pred`` evaluates the predicate on any broadcastable integer arrays of rows
``i`` and columns ``j``; ``allowed`` returns ``allowed[i - i0, j]`` for the
rows [i0, i1) and all S columns.
"""
from __future__ import annotations

import numpy as np


def _doc_ids(doc_lens):
    return np.repeat(np.arange(len(doc_lens)), doc_lens)


def _doc_starts(doc_lens):
    return np.concatenate([[0], np.cumsum(doc_lens)[:-1]]).astype(np.int64)


def base_pred(spec, i, j):
    """mask(i, j) of the base family of ``spec`` (no bitmap), for int64
    arrays of rows i and columns j that broadcast against each other."""
    S = int(spec["S"])
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    fam = spec["family"]

    if fam == "full":
        # FULL: every key is visible.
        return np.ones(np.broadcast_shapes(i.shape, j.shape), dtype=bool)

    if fam == "causal":
        # CAUSAL with Sq = Sk: keys up to and including the query position.
        return j <= i

    if fam == "sliding":
        # SLIDING WINDOW of width w.  Reading: CAUSAL SW keeps 0 <= i-j < w
        # (w keys including self); FULL SW keeps |i-j| < w.
        w = int(spec["window"])
        if spec["causal"]:
            return (j <= i) & (i - j < w)
        return np.abs(i - j) < w

    if fam == "document":
        # DOCUMENT (packed variable-length sequences): a token sees only its
        # own document; CAUSAL DOCUMENT additionally requires j <= i.
        doc = _doc_ids(spec["doc_lens"])
        same = doc[i] == doc[j]
        return same & (j <= i) if spec["causal"] else same

    if fam == "prefix_lm_causal":
        # PREFIX LM CAUSAL with prefix p: j < p or j <= i (prefix tokens see
        # the whole prefix bidirectionally; the rest is causal).
        p = int(spec["prefix"])
        return (j < p) | (j <= i)

    if fam == "shared_question":
        # SHARED QUESTION: a question of q tokens followed by answers laid out
        # consecutively.  Reading: causal everywhere; an answer token sees the
        # question and its own answer, never another answer.
        q = int(spec["question"])
        lens = [q] + list(spec["answers"])
        seg = _doc_ids(lens)            # 0 = question, k = answer k
        same = seg[i] == seg[j]
        return (j <= i) & ((j < q) | same)

    if fam == "global_sliding":
        # GLOBAL SLIDING with g global tokens and window w.  Reading: causal;
        # a key is visible if it is global (j < g) or inside the window
        # (i - j < w).  Alternative reading (bidirectional): j < g or i < g or
        # |i - j| < w.
        g, w = int(spec["globals"]), int(spec["window"])
        if spec.get("bidirectional", False):
            return (j < g) | (i < g) | (np.abs(i - j) < w)
        return (j <= i) & ((j < g) | (i - j < w))

    if fam == "causal_blockwise":
        # CAUSAL BLOCKWISE with block b, n = ceil(S / b) blocks.  Reading:
        # rows of blocks 0..n-2 are causal inside their own block; rows of the
        # last block are causal over the whole sequence.  Alternative reading
        # (block-causal): blk(j) <= blk(i).
        b = int(spec["block"])
        n = (S + b - 1) // b
        bi, bj = i // b, j // b
        if spec.get("reading", "last_block_global") == "block_causal":
            return bj <= bi
        return (j <= i) & ((bi == bj) | (bi == n - 1))

    if fam == "prefix_lm_document":
        # PREFIX LM DOCUMENT: the prefix-LM rule applied inside each document,
        # with that document's own prefix length.
        lens = spec["doc_lens"]
        doc = _doc_ids(lens)
        start = _doc_starts(lens)
        pre = np.asarray(spec["prefix_lens"], dtype=np.int64)
        di = doc[i]
        same = di == doc[j]
        return same & ((j < start[di] + pre[di]) | (j <= i))

    if fam == "block_causal_document":
        # BLOCK CAUSAL DOCUMENT: inside a document, blocks of b tokens counted
        # from the document start; a token sees every block up to its own.
        b = int(spec["block"])
        lens = spec["doc_lens"]
        doc = _doc_ids(lens)
        start = _doc_starts(lens)
        pos = np.arange(S, dtype=np.int64) - start[doc]
        blk = pos // b
        same = doc[i] == doc[j]
        return same & (blk[j] <= blk[i])

    if fam == "task_batch":
        # TASK BATCH: token-level core-attention tasks fused into one launch
        # ("Efficient Long-context Language Model Training by Core Attention
        # Disaggregation", abstract: core attention is composable, kernels
        # keep their efficiency on fused batches of token-level shards of
        # arbitrary length).  Reading: task t is a segment of kv_t tokens, the
        # context of a query shard (its document up to the shard's end), whose
        # last q_t tokens are the shard's queries; a query sees the keys of its
        # own segment up to itself, and the segment's other rows are not
        # queries (no keys).
        lens = spec["kv_lens"]
        seg = _doc_ids(lens)
        start = _doc_starts(lens)
        end = start + np.asarray(lens, dtype=np.int64)
        ql = np.asarray(spec["q_lens"], dtype=np.int64)
        si = seg[i]
        same = si == seg[j]
        return same & (j <= i) & (i >= end[si] - ql[si])

    raise ValueError(f"unknown mask family {fam!r}")


def bitmap_pred(bitmap, hm, i, j):
    """bits[hm][qblk(i)][kblk(j)] of a block bitmap, for broadcastable int64
    arrays of rows i and columns j.

    Uniform or variable-size blocks (page 1 section 3, dynamic masks): the
    block of a position is the b with offsets[b] <= x < offsets[b+1].
    """
    qo = np.asarray(bitmap["q_offsets"], dtype=np.int64)
    ko = np.asarray(bitmap["k_offsets"], dtype=np.int64)
    qb = np.searchsorted(qo, np.asarray(i, dtype=np.int64), side="right") - 1
    kb = np.searchsorted(ko, np.asarray(j, dtype=np.int64), side="right") - 1
    return bitmap["bits"][hm][qb, kb].astype(bool)


def mask_head(spec, h, Hq, Hkv):
    """Which bitmap head applies to query head h (bitmap heads in {1,Hkv,Hq})."""
    if "bitmap" not in spec:
        return 0
    nh = spec["bitmap"]["bits"].shape[0]
    if nh == 1:
        return 0
    if nh == Hq:
        return h
    if nh == Hkv:
        return h // (Hq // Hkv)
    raise ValueError("bitmap head count must be 1, Hkv or Hq")


def pred(spec, i, j, hm=0):
    """The full predicate, base family AND the optional bitmap, for
    broadcastable int64 arrays of rows i and columns j."""
    a = base_pred(spec, i, j)
    if "bitmap" in spec:
        a = a & bitmap_pred(spec["bitmap"], hm, i, j)
    return a


def allowed(spec, i0, i1, hm=0):
    """Full predicate rows [i0, i1) over all S columns."""
    i = np.arange(i0, i1, dtype=np.int64)[:, None]
    j = np.arange(int(spec["S"]), dtype=np.int64)[None, :]
    return pred(spec, i, j, hm)


def dense_mask(spec, hm=0):
    """The whole S x S boolean mask (small S only)."""
    return allowed(spec, 0, int(spec["S"]), hm)


def nnz(spec, hm=0, row_block=1024):
    """Number of allowed (i, j) pairs, by popcount of the predicate."""
    S = int(spec["S"])
    tot = 0
    for i0 in range(0, S, row_block):
        tot += int(allowed(spec, i0, min(S, i0 + row_block), hm).sum())
    return tot
