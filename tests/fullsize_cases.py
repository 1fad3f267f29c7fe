"""Key columns for the element-wise dK/dV check at the workloads' full sizes.

dK_j and dV_j sum over every row allowed to attend to key j, and each such
row needs its whole score row (for P_ij, D_i and the row sums of the
sensitivities), so the oracle's cost for a column is the number of rows that
see it times the keys those rows see.  Columns are taken from a candidate
list (the fixed positions 0, 1, 127, 128, S/2, S-129, S-1, then seeded
random ones) as long as the rows that see the chosen set stay within a
budget; masks whose every column is seen by most rows (FULL, block-sparse)
are checked at their smaller configured length or with a smaller budget.
"""
import numpy as np

import synthetic as syn
from oracle import masks as om

HQ, D = 64, 128


class Lazy64:
    """Array view that widens bf16 bits to float64 only where indexed."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return syn.bf16_bits_to_f32(self.bits[idx]).astype(np.float64)


def _seeing_rows(spec, Hq, Hkv, kv, col):
    """Rows allowed to attend to key ``col`` for some query head of KV group kv."""
    S = spec["S"]
    G = Hq // Hkv
    i = np.arange(S)[:, None]
    out = np.zeros(S, dtype=bool)
    for hm in sorted({om.mask_head(spec, kv * G + g, Hq, Hkv) for g in range(G)}):
        out |= om.pred(spec, i, np.array([[col]]), hm)[:, 0]
    return out


def pick_cols(spec, Hq, Hkv, kv, row_budget=4096, n_random=9, extra=(), seed=0):
    """Chosen key columns: candidates in order, each kept while the union of
    the rows that see the kept columns stays within row_budget."""
    S = spec["S"]
    rng = np.random.default_rng(seed + 7 * kv)
    cand = [0, 1, 127, 128, S // 2, S - 129, S - 1] + list(extra) + rng.integers(0, S, n_random).tolist()
    rows = np.zeros(S, dtype=bool)
    cols = []
    for c in cand:
        c = int(c)
        if c in cols or not 0 <= c < S:
            continue
        r = rows | _seeing_rows(spec, Hq, Hkv, kv, c)
        if r.sum() <= row_budget:
            rows = r
            cols.append(c)
    return sorted(cols)


def _doc_ends(spec):
    e = np.cumsum(spec["doc_lens"])
    return [int(x) for x in e]


def col_cases():
    """(label, spec, Hkv, KV heads checked, row budget, extra candidates,
    oracle row block).  About 5e9 (row, key) scores in all."""
    out = []
    dense8 = dict(syn.config_mask_specs("dense", 8192))
    dense48 = dict(syn.config_mask_specs("dense", 49152))
    # FULL: every column is seen by every row, so the whole group is formed
    out.append(("dense8K_full", dense8["full"], 8, (7,), 8192, (), 512))
    out.append(("dense8K_causal", dense8["causal"], 8, (0,), 1024, (), 512))
    out.append(("dense48K_causal", dense48["causal"], 8, (0, 7), 1024,
                (49152 - 2, 49152 - 64, 49152 - 65), 512))
    out.append(("dense48K_causal_sw1024", dense48["causal_sw1024"], 8, (7,), 4096, (), 512))
    doc = dict(syn.config_mask_specs("document"))
    ends = _doc_ends(doc["causal_document"])
    tails = [e - o for e in ends for o in (1, 129)]
    out.append(("doc64K_causal_document", doc["causal_document"], 8, (0,), 1024, tails, 512))
    lens = doc["full_document"]["doc_lens"]
    short = int(np.argmin(lens))
    s0 = int(np.sum(lens[:short]))
    out.append(("doc64K_full_document", doc["full_document"], 8, (3,), 4096,
                (s0, s0 + 1, s0 + lens[short] - 1), 512))
    het = dict(syn.config_mask_specs("hetero"))
    sq = het["shared_question"]
    q = sq["question"]
    out.append(("hetero32K_shared_question", sq, 8, (7,), 1024,
                [int(x) - o for x in np.cumsum([q] + list(sq["answers"])) for o in (1, 65)], 512))
    # global keys: every later row sees them, so their dK/dV items are split
    # into chunks whose fp32 partials a reduce pass sums
    out.append(("hetero32K_global_sliding", het["global_sliding"], 8, (0,), 40000, (5, 63), 64))
    out.append(("hetero32K_prefix_lm_causal", het["prefix_lm_causal"], 8, (7,), 512, (), 512))
    out.append(("hetero32K_causal_blockwise", het["causal_blockwise"], 8, (0,), 4096,
                (4095, 4096 * 3 + 5), 512))
    var = dict(syn.config_mask_specs("variants"))
    out.append(("variants32K_global_sliding_bidir", var["global_sliding_bidir"], 8, (0,), 4300, (), 512))
    # block-causal reading: a key of the last block is seen by every row of
    # it, each with all earlier keys; at 8K with 2K blocks to bound the cost
    bc = syn.spec_causal_blockwise(8192, 2048, reading="block_causal")
    out.append(("variants8K_causal_blockwise_block_causal", bc, 8, (0,), 2048, (), 512))
    # the longest configured sequence: S = 128K, keys near the end (few rows)
    dense128 = dict(syn.config_mask_specs("dense", 131072))
    out.append(("dense128K_causal", dense128["causal"], 8, (3,), 512,
                (131072 - 2, 131072 - 64, 131072 - 65), 512))
    spg = dict(syn.config_mask_specs("sparse", 32768, Hq=HQ, Hkv=8))
    out.append(("sparse32K_block64_50", spg["block64_50"], 8, (5,), 20000, (), 64))
    spm = dict(syn.config_mask_specs("sparse", 32768, Hq=HQ, Hkv=64))
    out.append(("sparse32K_mha_block64_50", spm["block64_50"], 64, (0, 21, 42, 63), 20000, (), 64))
    out.append(("sparse32K_mha_varblock_50", spm["varblock_50"], 64, (0, 63), 20000, (), 64))
    return out


def grad_cols_parallel(x, spec, Hq, Hkv, kvs, cols_of, row_block, workers=16):
    """oracle grad_cols for the KV heads ``kvs``, one thread per query head
    (numpy releases the GIL in its loops; BLAS runs one thread per worker),
    the heads' contributions summed in head order.  Returns {kv: result}."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import attention as ora
    G = Hq // Hkv
    lz = {n: Lazy64(x[n]) for n in ("q", "k", "v", "do")}
    jobs = [(kv, h) for kv in kvs for h in range(kv * G, kv * G + G)]

    def one(job):
        kv, h = job
        return ora.grad_cols(lz["q"], lz["k"], lz["v"], lz["do"], spec, kv, cols_of[kv],
                             row_block=row_block, heads=[h])

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=min(workers, len(jobs))) as ex:
            parts = list(ex.map(one, jobs))
    out = {}
    for (kv, h), r in zip(jobs, parts):
        if kv not in out:
            out[kv] = {n: np.zeros_like(r[n]) for n in ("dk", "dv", "m_dk", "m_dv")}
            out[kv]["pairs"] = 0
        for n in ("dk", "dv"):
            out[kv][n] += r[n]
        for n in ("m_dk", "m_dv"):
            out[kv][n] += r[n] ** 2
        out[kv]["pairs"] += r["pairs"]
    for kv in out:
        for n in ("m_dk", "m_dv"):
            out[kv][n] = np.sqrt(out[kv][n])
    return out
