"""fp64 masked attention, forward and backward, by the plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition ("FlashAttention vs. RingAttention", FlashAttention-1 "problem and
bottleneck"): Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V, with the
mask applied to the score matrix before the softmax.  The method the pages
describe is exact (same page: FlashAttention "is not an approximation"), so
the oracle is the definition itself: full score rows are materialised in fp64,
masked explicitly, and normalised with an exact two-pass softmax.  There is no
tiling, no online recurrence and no reordering beyond row blocks.

Readings taken where the pages are silent:
* scale = 1/sqrt(d) with d the head dimension;
* the one merged softmax statistic kept for the backward (FlashAttention-2
  "core optimisations") is the natural-log log-sum-exp, LSE_i = m_i +
  ln sum_j exp(s_ij - m_i), stored as [B, Hq, S];
* GQA: query head h reads KV head h // (Hq / Hkv);
* a row with no allowed key has O_i = 0, LSE_i = -inf and zero gradients.

Backward (standard softmax calculus; the dQ form dQ_i = sum_j dS_ij K_j is
the dependency named in FlashAttention-2 "core optimisations"):
  D_i   = dO_i . O_i
  dP_ij = dO_i . v_j
  dS_ij = p_ij (dP_ij - D_i)
  dQ_i  = scale sum_j dS_ij k_j
  dK_j  = scale sum_i dS_ij q_i
  dV_j  = sum_i p_ij dO_i
with dK, dV of a KV head summed over the query heads of its group.

Inputs are float64 arrays already holding the bf16 values (upcast exactly).
"""
from __future__ import annotations

import math

import numpy as np

from . import masks


def _probs(s, a):
    """Exact masked softmax of score rows ``s`` under boolean ``a``.

    Returns (p, lse) with p = 0 on masked entries and on empty rows.
    """
    sm = np.where(a, s, -np.inf)
    m = sm.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.where(a, np.exp(sm - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
    lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return p, lse


def forward(q, k, v, spec, scale=None, heads=None, row_block=512):
    """O and LSE for the selected query heads.

    q: [B,S,Hq,d], k/v: [B,S,Hkv,d] float64.  ``heads`` lists the query heads
    to compute (default: all).  Returns o [B,S,len(heads),d] and
    lse [B,len(heads),S].
    """
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    heads = list(range(Hq)) if heads is None else list(heads)
    o = np.zeros((B, S, len(heads), d))
    lse = np.zeros((B, len(heads), S))
    for b in range(B):
        for hi, h in enumerate(heads):
            kv = h // G
            hm = masks.mask_head(spec, h, Hq, Hkv)
            kT = k[b, :, kv, :].T
            vv = v[b, :, kv, :]
            for i0 in range(0, S, row_block):
                i1 = min(S, i0 + row_block)
                s = (q[b, i0:i1, h, :] @ kT) * scale
                p, l = _probs(s, masks.allowed(spec, i0, i1, hm))
                o[b, i0:i1, hi, :] = p @ vv
                lse[b, hi, i0:i1] = l
    return o, lse


def merge(o_parts, lse_parts):
    """O and LSE over a union of disjoint key sets from the results over each
    set.

    "FlashAttention vs. RingAttention", Ring Attention section (Blockwise
    Parallel Transformer): the output of each key block is rescaled by the
    difference between its own softmax normaliser and the global one.  With
    LSE_c the natural-log normaliser of part c (its LSE):
        LSE = ln sum_c exp(LSE_c),   O = sum_c exp(LSE_c - LSE) O_c.
    A row with no key in any part keeps O = 0 and LSE = -inf.

    o_parts: list of [B,S,H,d] float64; lse_parts: list of [B,H,S] float64.
    """
    lse = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])  # [C,B,H,S]
    m = lse.max(axis=0)
    live = np.isfinite(m)
    m0 = np.where(live, m, 0.0)
    w = np.exp(lse - m0)                   # exp(-inf) = 0 for empty parts
    tot = np.where(live, w.sum(axis=0), 1.0)
    out_lse = np.where(live, m0 + np.log(tot), -np.inf)
    wn = np.where(live, w / tot, 0.0)      # [C,B,H,S]
    o = np.zeros_like(np.asarray(o_parts[0], dtype=np.float64))
    for c, oc in enumerate(o_parts):
        o += wn[c].transpose(0, 2, 1)[..., None] * oc
    return o, out_lse


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (8 significant
    bits, ties to even), returned as float64.  Normal-range values only."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    scaled = m * 256.0                      # 8 significant bits before the point
    r = np.round(scaled)                    # numpy rounds half to even
    return np.ldexp(r / 256.0, e)


def backward(q, k, v, do, spec, scale=None, kv_heads=None, row_block=512,
             o_for_d="exact", magnitudes=False):
    """dQ, dK, dV (and O, LSE) for the selected KV heads and their groups.

    Returns a dict with dq [B,S,G*n,d] for the query heads of the selected KV
    heads (in order), dk/dv [B,S,n,d], o and lse for the same query heads,
    and ``heads``, the query head indices covered.

    ``o_for_d``: the O entering D_i = dO_i . O_i.  "exact" uses the exact
    output; "bf16" uses it rounded to bfloat16, i.e. the O a caller holds when
    the forward returns bf16 and the backward receives that O back.

    ``magnitudes``: also return, per output element x = sum_t a_t b_t of each
    product (O = P V, dV = P^T dO, dQ = scale dS K, dK = scale dS^T Q), the
    quadratic magnitude sqrt(sum_t (a_t b_t)^2) under keys "m_o", "m_dv",
    "m_dq", "m_dk".  It sets the size of the error a product makes when one
    of its operands is rounded to a narrower format term by term.
    """
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    heads = [kv * G + g for kv in kv_heads for g in range(G)]
    nq = len(heads)
    if o_for_d not in ("exact", "bf16"):
        raise ValueError("o_for_d must be 'exact' or 'bf16'")
    dq = np.zeros((B, S, nq, d))
    dk = np.zeros((B, S, len(kv_heads), d))
    dv = np.zeros((B, S, len(kv_heads), d))
    o = np.zeros((B, S, nq, d))
    lse = np.zeros((B, nq, S))
    if magnitudes:
        m_o = np.zeros_like(o)
        m_dq = np.zeros_like(dq)
        m_dk2 = np.zeros_like(dk)
        m_dv2 = np.zeros_like(dv)
    for b in range(B):
        for hi, h in enumerate(heads):
            kvi = hi // G
            kv = kv_heads[kvi]
            hm = masks.mask_head(spec, h, Hq, Hkv)
            kk = k[b, :, kv, :]
            vv = v[b, :, kv, :]
            for i0 in range(0, S, row_block):
                i1 = min(S, i0 + row_block)
                qi = q[b, i0:i1, h, :]
                doi = do[b, i0:i1, h, :]
                s = (qi @ kk.T) * scale
                p, l = _probs(s, masks.allowed(spec, i0, i1, hm))
                oi = p @ vv
                o[b, i0:i1, hi, :] = oi
                lse[b, hi, i0:i1] = l
                od = oi if o_for_d == "exact" else round_bf16(oi)
                D = (doi * od).sum(axis=1)
                dp = doi @ vv.T
                ds = p * (dp - D[:, None])
                dq[b, i0:i1, hi, :] = (ds @ kk) * scale
                dk[b, :, kvi, :] += (ds.T @ qi) * scale
                dv[b, :, kvi, :] += p.T @ doi
                if magnitudes:
                    p2, ds2 = p * p, ds * ds
                    m_o[b, i0:i1, hi, :] = np.sqrt(p2 @ (vv * vv))
                    m_dq[b, i0:i1, hi, :] = np.sqrt(ds2 @ (kk * kk)) * scale
                    m_dk2[b, :, kvi, :] += (ds2.T @ (qi * qi)) * scale * scale
                    m_dv2[b, :, kvi, :] += p2.T @ (doi * doi)
    out = {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "heads": heads}
    if magnitudes:
        out.update(m_o=m_o, m_dq=m_dq, m_dk=np.sqrt(m_dk2), m_dv=np.sqrt(m_dv2))
    return out


def output_rows(q, k, v, spec, h, rows, scale=None):
    """O and LSE of query head ``h`` for an arbitrary set of rows only.

    Used to check sampled outputs at sizes where the whole tensor would take
    too long.  Returns o [len(rows), d], lse [len(rows)] for batch 0.
    """
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    hm = masks.mask_head(spec, h, Hq, Hkv)
    kv = h // G
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for r, i in enumerate(rows):
        s = (k[0, :, kv, :] @ q[0, i, h, :]) * scale
        p, l = _probs(s[None, :], masks.allowed(spec, i, i + 1, hm))
        o[r] = p[0] @ v[0, :, kv, :]
        lse[r] = l[0]
    return o, lse


def grad_rows(q, k, v, do, spec, h, rows, scale=None, o_for_d="exact"):
    """dQ, O and LSE of query head ``h`` for an arbitrary set of rows only
    (batch 0).  Every quantity a row's dQ needs is local to the row: its
    probabilities p_ij, D_i = dO_i . O_i and dP_ij = dO_i . v_j.  Returns
    dq [len(rows), d], o [len(rows), d], lse [len(rows)] and the quadratic
    magnitudes m_dq, m_o of the two products (see ``backward``)."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    hm = masks.mask_head(spec, h, Hq, Hkv)
    kv = h // G
    kk = k[0, :, kv, :]
    vv = v[0, :, kv, :]
    out = {n: np.zeros((len(rows), d)) for n in ("dq", "o", "m_dq", "m_o")}
    out["lse"] = np.zeros(len(rows))
    for r, i in enumerate(rows):
        s = (kk @ q[0, i, h, :]) * scale
        p, l = _probs(s[None, :], masks.allowed(spec, i, i + 1, hm))
        p = p[0]
        oi = p @ vv
        od = oi if o_for_d == "exact" else round_bf16(oi)
        Di = float(do[0, i, h, :] @ od)
        dp = vv @ do[0, i, h, :]
        ds = p * (dp - Di)
        out["dq"][r] = (ds @ kk) * scale
        out["o"][r] = oi
        out["lse"][r] = l[0]
        out["m_dq"][r] = np.sqrt((ds * ds) @ (kk * kk)) * scale
        out["m_o"][r] = np.sqrt((p * p) @ (vv * vv))
    return out
