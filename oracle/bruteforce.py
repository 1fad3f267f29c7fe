"""Pure-Python brute force for tiny cases: scalar loops and math.fsum.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is a second, independent transcription of the same definitions as
``oracle.masks`` and ``oracle.attention`` (scalar predicate per (i, j), no
numpy), used to pin them.  Sources: "Long-Context Attention Benchmark" review
(xllm-io), section 3 mask taxonomy, for the family names; "FlashAttention vs.
RingAttention" (dtcms), FlashAttention-1 "problem and bottleneck", for
softmax(Q K^T / sqrt(d_k)) V.  The readings are the ones stated in
``oracle.masks``.
"""
from __future__ import annotations

import math


def _segment_of(x, lens):
    """Index of the segment containing position x, and that segment's start."""
    start = 0
    for idx, L in enumerate(lens):
        if x < start + L:
            return idx, start
        start += L
    raise IndexError(x)


def _block_of(x, offsets):
    for b in range(len(offsets) - 1):
        if offsets[b] <= x < offsets[b + 1]:
            return b
    raise IndexError(x)


def allowed(spec, i, j, hm=0):
    """Scalar predicate: may query row i attend to key j?"""
    fam = spec["family"]
    S = spec["S"]
    if fam == "full":
        ok = True
    elif fam == "causal":
        ok = j <= i
    elif fam == "sliding":
        w = spec["window"]
        if spec["causal"]:
            ok = 0 <= i - j < w
        else:
            ok = -w < i - j < w
    elif fam == "document":
        di, _ = _segment_of(i, spec["doc_lens"])
        dj, _ = _segment_of(j, spec["doc_lens"])
        ok = di == dj and (j <= i or not spec["causal"])
    elif fam == "prefix_lm_causal":
        ok = j < spec["prefix"] or j <= i
    elif fam == "shared_question":
        segs = [spec["question"]] + list(spec["answers"])
        si, _ = _segment_of(i, segs)
        sj, _ = _segment_of(j, segs)
        ok = j <= i and (sj == 0 or si == sj)
    elif fam == "global_sliding":
        g, w = spec["globals"], spec["window"]
        if spec.get("bidirectional", False):
            ok = j < g or i < g or abs(i - j) < w
        else:
            ok = j <= i and (j < g or i - j < w)
    elif fam == "causal_blockwise":
        b = spec["block"]
        nblk = -(-S // b)
        if spec.get("reading", "last_block_global") == "block_causal":
            ok = j // b <= i // b
        elif i // b == nblk - 1:
            ok = j <= i
        else:
            ok = j <= i and j // b == i // b
    elif fam == "prefix_lm_document":
        di, si = _segment_of(i, spec["doc_lens"])
        dj, _ = _segment_of(j, spec["doc_lens"])
        ok = di == dj and (j < si + spec["prefix_lens"][di] or j <= i)
    elif fam == "block_causal_document":
        di, si = _segment_of(i, spec["doc_lens"])
        dj, sj = _segment_of(j, spec["doc_lens"])
        b = spec["block"]
        ok = di == dj and (j - sj) // b <= (i - si) // b
    elif fam == "task_batch":
        ti, si = _segment_of(i, spec["kv_lens"])
        tj, _ = _segment_of(j, spec["kv_lens"])
        end = si + spec["kv_lens"][ti]
        ok = ti == tj and j <= i and i >= end - spec["q_lens"][ti]
    else:
        raise ValueError(fam)
    if ok and "bitmap" in spec:
        bm = spec["bitmap"]
        qb = _block_of(i, bm["q_offsets"])
        kb = _block_of(j, bm["k_offsets"])
        ok = bool(bm["bits"][hm][qb][kb])
    return ok


def attention(q, k, v, do, spec, scale=None, hm_of_head=None):
    """Forward and backward by scalar loops.

    q, do: nested lists [S][Hq][d]; k, v: [S][Hkv][d] (batch of one).
    Returns dict of nested lists o, lse, dq, dk, dv.
    """
    S = len(q)
    Hq = len(q[0])
    Hkv = len(k[0])
    d = len(q[0][0])
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    hm_of_head = hm_of_head or (lambda h: 0)
    o = [[[0.0] * d for _ in range(Hq)] for _ in range(S)]
    lse = [[0.0] * S for _ in range(Hq)]
    dq = [[[0.0] * d for _ in range(Hq)] for _ in range(S)]
    dk_terms = [[[[] for _ in range(d)] for _ in range(Hkv)] for _ in range(S)]
    dv_terms = [[[[] for _ in range(d)] for _ in range(Hkv)] for _ in range(S)]
    for h in range(Hq):
        kv = h // G
        hm = hm_of_head(h)
        for i in range(S):
            keys = [j for j in range(S) if allowed(spec, i, j, hm)]
            if not keys:
                lse[h][i] = -math.inf
                continue
            s = {j: scale * math.fsum(q[i][h][c] * k[j][kv][c] for c in range(d)) for j in keys}
            m = max(s.values())
            z = math.fsum(math.exp(s[j] - m) for j in keys)
            p = {j: math.exp(s[j] - m) / z for j in keys}
            lse[h][i] = m + math.log(z)
            for c in range(d):
                o[i][h][c] = math.fsum(p[j] * v[j][kv][c] for j in keys)
            D = math.fsum(do[i][h][c] * o[i][h][c] for c in range(d))
            for j in keys:
                dp = math.fsum(do[i][h][c] * v[j][kv][c] for c in range(d))
                ds = p[j] * (dp - D)
                for c in range(d):
                    dk_terms[j][kv][c].append(scale * ds * q[i][h][c])
                    dv_terms[j][kv][c].append(p[j] * do[i][h][c])
            for c in range(d):
                dq[i][h][c] = scale * math.fsum(
                    p[j] * (math.fsum(do[i][h][e] * v[j][kv][e] for e in range(d)) - D) * k[j][kv][c]
                    for j in keys)
    dk = [[[math.fsum(dk_terms[j][kv][c]) for c in range(d)] for kv in range(Hkv)] for j in range(S)]
    dv = [[[math.fsum(dv_terms[j][kv][c]) for c in range(d)] for kv in range(Hkv)] for j in range(S)]
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
