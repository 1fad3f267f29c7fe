"""Seeded synthetic inputs: bf16 tensors and mask-family parameter specs.

Tensors are drawn as float32 N(0, 1) from numpy's PCG64 generator and rounded
to bfloat16 with round-to-nearest-even; they are returned as raw uint16 bit
patterns so that every consumer (fp64 oracle, GPU path) sees the exact same
bf16 values.

A *mask spec* is a plain dict naming one of the LongCA-bench mask families
(page 1, section 3, mask taxonomy) together with its parameters, e.g.
``{"family": "document", "doc_lens": [...], "causal": True}``.  A spec carries
no semantics here: what each family allows is defined separately by the oracle
(``oracle/masks.py``) and by the library's descriptor builder.

The document-length, prefix and answer samplers stand in for the pages'
mixed-dataset sampler (Pile / ProLong64K / ProLong512K, page 1 section 3
components table), whose data is not available.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_from_f32", "bf16_bits_to_f32", "normal_bf16", "attention_inputs",
    "spec_full", "spec_causal", "spec_sliding", "spec_document",
    "spec_prefix_lm_causal", "spec_shared_question", "spec_global_sliding",
    "spec_causal_blockwise", "spec_prefix_lm_document",
    "spec_block_causal_document", "spec_task_batch", "with_bitmap", "spec_seq_len",
    "sample_doc_lens", "sample_prefix", "sample_answers", "sample_tasks",
    "uniform_block_bitmap", "variable_block_bitmap", "variable_partition", "partition_bitmap",
    "config_mask_specs",
]

# ----------------------------------------------------------------------------
# bf16 tensors
# ----------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); uint16 bits.

    Inputs must be finite (normal samples always are).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = u + np.uint32(0x7FFF) + lsb
    return (r >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, seed: int, stream: int) -> np.ndarray:
    """N(0,1) float32 samples rounded to bf16, as uint16 bits.

    ``stream`` separates independent tensors drawn under one seed.
    """
    rng = np.random.default_rng([int(seed), int(stream)])
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = bf16_bits_from_f32(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def attention_inputs(B, S, Hq, Hkv, d, seed=0, with_do=True):
    """Q [B,S,Hq,d], K/V [B,S,Hkv,d] and dO [B,S,Hq,d] as bf16 bit arrays."""
    out = {
        "q": normal_bf16((B, S, Hq, d), seed, 1),
        "k": normal_bf16((B, S, Hkv, d), seed, 2),
        "v": normal_bf16((B, S, Hkv, d), seed, 3),
    }
    if with_do:
        out["do"] = normal_bf16((B, S, Hq, d), seed, 4)
    return out

# ----------------------------------------------------------------------------
# mask specs (parameters only)
# ----------------------------------------------------------------------------

def spec_full(S):
    return {"family": "full", "S": int(S)}


def spec_causal(S):
    return {"family": "causal", "S": int(S)}


def spec_sliding(S, window, causal=True):
    return {"family": "sliding", "S": int(S), "window": int(window), "causal": bool(causal)}


def spec_document(doc_lens, causal):
    doc_lens = [int(x) for x in doc_lens]
    return {"family": "document", "S": int(sum(doc_lens)), "doc_lens": doc_lens,
            "causal": bool(causal)}


def spec_prefix_lm_causal(S, prefix):
    return {"family": "prefix_lm_causal", "S": int(S), "prefix": int(prefix)}


def spec_shared_question(question, answers):
    answers = [int(a) for a in answers]
    return {"family": "shared_question", "S": int(question) + int(sum(answers)),
            "question": int(question), "answers": answers}


def spec_global_sliding(S, n_global, window, bidirectional=False):
    return {"family": "global_sliding", "S": int(S), "globals": int(n_global),
            "window": int(window), "bidirectional": bool(bidirectional)}


def spec_causal_blockwise(S, block, reading="last_block_global"):
    assert reading in ("last_block_global", "block_causal")
    return {"family": "causal_blockwise", "S": int(S), "block": int(block),
            "reading": reading}


def spec_prefix_lm_document(doc_lens, prefix_lens):
    doc_lens = [int(x) for x in doc_lens]
    prefix_lens = [int(x) for x in prefix_lens]
    assert len(prefix_lens) == len(doc_lens)
    return {"family": "prefix_lm_document", "S": int(sum(doc_lens)),
            "doc_lens": doc_lens, "prefix_lens": prefix_lens}


def spec_block_causal_document(doc_lens, block):
    doc_lens = [int(x) for x in doc_lens]
    return {"family": "block_causal_document", "S": int(sum(doc_lens)),
            "doc_lens": doc_lens, "block": int(block)}


def spec_task_batch(kv_lens, q_lens):
    """Fused batch of token-level tasks: segment t has kv_lens[t] tokens of
    context, the last q_lens[t] of them queries."""
    kv_lens = [int(x) for x in kv_lens]
    q_lens = [int(x) for x in q_lens]
    assert len(kv_lens) == len(q_lens) and all(0 <= q <= k for q, k in zip(q_lens, kv_lens))
    return {"family": "task_batch", "S": int(sum(kv_lens)), "kv_lens": kv_lens, "q_lens": q_lens}


def sample_tasks(S, shard, seed, kv_max=None):
    """Tasks that fill S tokens: query shards of `shard` tokens, each with a
    context drawn uniformly from [shard, kv_max] tokens (default 4 * shard:
    a shard at a random position in the first four shards of its document);
    the last task is cut to fit."""
    kv_max = 4 * shard if kv_max is None else int(kv_max)
    rng = np.random.default_rng(seed)
    kv, q, left = [], [], int(S)
    while left > 0:
        k = min(int(rng.integers(shard, kv_max + 1)), left)
        kv.append(k)
        q.append(min(shard, k))
        left -= k
    return kv, q


def with_bitmap(spec, q_offsets, k_offsets, bits):
    """Attach a block bitmap ``bits[hm][qb][kb]`` (uint8 0/1) to a base spec.

    ``q_offsets``/``k_offsets`` are block boundaries 0 = o_0 < ... < o_n = S.
    """
    out = dict(spec)
    out["bitmap"] = {
        "q_offsets": [int(x) for x in q_offsets],
        "k_offsets": [int(x) for x in k_offsets],
        "bits": np.ascontiguousarray(bits, dtype=np.uint8),
    }
    return out


def spec_seq_len(spec):
    return int(spec["S"])

# ----------------------------------------------------------------------------
# samplers
# ----------------------------------------------------------------------------

def sample_doc_lens(S, lo, hi, seed):
    """Document lengths round(exp(U(ln lo, ln hi))) appended until S is filled;
    the last one is truncated so that the lengths sum to S."""
    rng = np.random.default_rng(seed)
    out, tot = [], 0
    while tot < S:
        L = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = max(1, min(L, S - tot))
        out.append(L)
        tot += L
    return out


def sample_prefix(lo, hi, seed):
    """Prefix length uniform on the integers [lo, hi]."""
    rng = np.random.default_rng(seed)
    return int(rng.integers(lo, hi + 1))


def sample_answers(total, n, seed):
    """Split ``total`` tokens into ``n`` answers at n-1 sorted uniform cuts."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.integers(1, total, size=n - 1))
    edges = np.concatenate([[0], cuts, [total]])
    lens = np.diff(edges).astype(int).tolist()
    return [max(0, x) for x in lens]


def _bernoulli_bits(heads, nq, nk, density, seed, diag_on=True):
    rng = np.random.default_rng(seed)
    bits = (rng.random((heads, nq, nk)) < density).astype(np.uint8)
    if diag_on:
        r = np.arange(min(nq, nk))
        bits[:, r, r] = 1
    return bits


def uniform_block_bitmap(S, block, heads, density=0.5, seed=0):
    """Uniform ``block`` x ``block`` bitmap, Bernoulli(density) per block with
    the diagonal blocks forced on; returns (offsets, bits[heads][n][n])."""
    n = (S + block - 1) // block
    offs = [min(S, i * block) for i in range(n + 1)]
    return offs, _bernoulli_bits(heads, n, n, density, seed)


def variable_partition(S, lo, hi, seed):
    """A random partition of [0, S) into blocks of i.i.d. uniform integer size
    in [lo, hi]; the last block is truncated."""
    rng = np.random.default_rng(seed)
    offs = [0]
    while offs[-1] < S:
        offs.append(min(S, offs[-1] + int(rng.integers(lo, hi + 1))))
    return offs


def partition_bitmap(q_offsets, k_offsets, heads, density=0.5, seed=0, diag_on=True):
    """Bernoulli(density) bits over given row and column block partitions
    (which may differ), blocks (b, b) forced on when ``diag_on``."""
    return _bernoulli_bits(heads, len(q_offsets) - 1, len(k_offsets) - 1, density, seed, diag_on)


def variable_block_bitmap(S, lo, hi, heads, density=0.5, seed=0):
    """One random partition shared by rows and columns, Bernoulli(density) per
    block pair, diagonal forced on; returns (offsets, bits)."""
    offs = variable_partition(S, lo, hi, seed)
    n = len(offs) - 1
    return offs, _bernoulli_bits(heads, n, n, density, seed + 7919)

# ----------------------------------------------------------------------------
# the workloads' mask mixes
# ----------------------------------------------------------------------------

def config_mask_specs(config, S=None, Hq=64, Hkv=8, seed=0):
    """Mask specs of the named workload family at sequence length S.

    * ``tiny``: every family at S=512 with scaled-down parameters.
    * ``dense``: FULL, CAUSAL, causal sliding window w=1024.
    * ``document``: FULL / CAUSAL DOCUMENT, log-uniform lengths in [256, 16K].
    * ``hetero``: PREFIX LM CAUSAL, SHARED QUESTION, GLOBAL SLIDING,
      CAUSAL BLOCKWISE.
    * ``sparse``: uniform 64 / 128 and variable block bitmaps at 50% density,
      per KV head.
    * ``tasks``: fused batches of token-level tasks (query shards of 256, 1K
      or 4K tokens, contexts uniform in [shard, 4 shard]) filling S = 64K.
    * ``variants``: FULL SW w=1024, PREFIX LM DOCUMENT and BLOCK CAUSAL
      DOCUMENT (block 1024) over log-uniform documents in [256, 16K],
      bidirectional GLOBAL SLIDING, block-causal CAUSAL BLOCKWISE.
    Returns a list of (label, spec).
    """
    if config == "tiny":
        S = 512 if S is None else S
        docs = sample_doc_lens(S, 16, 256, seed)
        q = 64
        return [
            ("full", spec_full(S)),
            ("causal", spec_causal(S)),
            ("causal_sw64", spec_sliding(S, 64, True)),
            ("full_sw64", spec_sliding(S, 64, False)),
            ("full_document", spec_document(docs, False)),
            ("causal_document", spec_document(docs, True)),
            ("prefix_lm_causal", spec_prefix_lm_causal(S, sample_prefix(32, 128, seed))),
            ("shared_question", spec_shared_question(q, sample_answers(S - q, 4, seed))),
            ("global_sliding", spec_global_sliding(S, 8, 64)),
            ("causal_blockwise", spec_causal_blockwise(S, 128)),
            ("prefix_lm_document", spec_prefix_lm_document(
                docs, [sample_prefix(0, L, seed + i) for i, L in enumerate(docs)])),
            ("block_causal_document", spec_block_causal_document(docs, 64)),
            ("block64_50", with_bitmap(spec_full(S), *_dup(uniform_block_bitmap(S, 64, Hkv, 0.5, seed)))),
            ("varblock_50", with_bitmap(spec_full(S), *_dup(variable_block_bitmap(S, 32, 224, Hkv, 0.5, seed)))),
            ("task_batch", spec_task_batch(*sample_tasks(S, 48, seed, kv_max=200))),
        ]
    if config == "tasks":
        S = 65536 if S is None else S
        return [(f"tasks_shard{sh}", spec_task_batch(*sample_tasks(S, sh, seed + i)))
                for i, sh in enumerate((256, 1024, 4096))]
    if config == "dense":
        return [("full", spec_full(S)), ("causal", spec_causal(S)),
                ("causal_sw1024", spec_sliding(S, 1024, True))]
    if config == "document":
        S = 65536 if S is None else S
        docs = sample_doc_lens(S, 256, 16384, seed)
        return [("full_document", spec_document(docs, False)),
                ("causal_document", spec_document(docs, True))]
    if config == "hetero":
        S = 32768 if S is None else S
        q = 2048
        return [
            ("prefix_lm_causal", spec_prefix_lm_causal(S, sample_prefix(1024, 8192, seed))),
            ("shared_question", spec_shared_question(q, sample_answers(S - q, 4, seed))),
            ("global_sliding", spec_global_sliding(S, 64, 2048)),
            ("causal_blockwise", spec_causal_blockwise(S, 4096)),
        ]
    if config == "variants":
        S = 32768 if S is None else S
        docs = sample_doc_lens(S, 256, 16384, seed)
        return [
            ("full_sw1024", spec_sliding(S, 1024, False)),
            ("prefix_lm_document", spec_prefix_lm_document(
                docs, [sample_prefix(0, L, seed + i) for i, L in enumerate(docs)])),
            ("block_causal_document", spec_block_causal_document(docs, 1024)),
            ("global_sliding_bidir", spec_global_sliding(S, 64, 2048, bidirectional=True)),
            ("causal_blockwise_block_causal", spec_causal_blockwise(S, 4096, "block_causal")),
        ]
    if config == "sparse":
        S = 32768 if S is None else S
        return [
            ("block64_50", with_bitmap(spec_full(S), *_dup(uniform_block_bitmap(S, 64, Hkv, 0.5, seed)))),
            ("block128_50", with_bitmap(spec_full(S), *_dup(uniform_block_bitmap(S, 128, Hkv, 0.5, seed)))),
            ("varblock_50", with_bitmap(spec_full(S), *_dup(variable_block_bitmap(S, 32, 224, Hkv, 0.5, seed)))),
        ]
    raise ValueError(f"unknown config {config!r}")


def _dup(offs_bits):
    offs, bits = offs_bits
    return offs, offs, bits
