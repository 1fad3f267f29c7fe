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


def _sensitivities(p, ds, o, do, q, k, v, scale, cols=None, rows=True):
    """First-order sensitivities of one row block's outputs to relative
    perturbations of the intermediate values that a tiled kernel rounds.

    Rows i of the block (one query head), keys j of the whole sequence.  The
    perturbations, each a relative change of one value (|.| <= u when the
    value is rounded to a format with unit roundoff u):

      delta_ij  the unnormalised probability p~_ij whose sum normalises the
                forward: O_i = sum_j p~_ij v_j / sum_j p~_ij, and
                LSE_i = m_i + ln sum_j p~_ij (so LSE_i moves by
                sum_j p_ij delta_ij and the backward's P_ij = exp(S_ij - LSE_i)
                by minus that);
      eps_id    the element O_id handed to the backward, which forms
                D_i = sum_d dO_id O_id from it;
      eta_ij    P_ij where it enters dV_j = sum_i P_ij dO_i;
      eta'_ij   dS_ij where it enters dK_j = scale sum_i dS_ij q_i;
      eta''_ij  dS_ij where it enters dQ_i = scale sum_j dS_ij k_j.

    To first order every output x moves by sum_t c_t e_t over these
    perturbations e_t; this returns the 2-norm sqrt(sum_t c_t^2) of the
    coefficient vector of every output element: for O (delta only), LSE,
    dQ, and the squared norms of this block's contributions to dK and dV
    (summed over row blocks and query heads by the caller; over every key,
    or over the key indices ``cols`` when given, False for none; the row
    outputs are left out when ``rows`` is False).  The
    closed forms below follow from D' = D + sum_j dS_ij delta_ij + sum_d dO_id O_id eps_id
    (since p_ij sum_d dO_id (v_jd - O_id) = dS_ij) and
    dS'_ij = P'_ij (dP_ij - D'_i); with the row sums
      A_i = sum_j p_ij^2, B_i = sum_j p_ij dS_ij, C_i = sum_j dS_ij^2,
      E_i = sum_d (dO_id O_id)^2, kbar_i = sum_j p_ij k_j:
      |c(O_id)|^2   = sum_j p_ij^2 (v_jd - O_id)^2
      |c(LSE_i)|^2  = A_i
      |c(dQ_id)|^2  = dQ_id^2 A_i + 2 scale dQ_id kbar_id B_i
                      + scale^2 kbar_id^2 (C_i + E_i) + scale^2 sum_j dS_ij^2 k_jd^2
      |c(dK_jd)|^2  = scale^2 sum_i q_id^2 (dS_ij^2 (A_i + 1) + 2 dS_ij p_ij B_i
                                             + p_ij^2 (C_i + E_i))
      |c(dV_jd)|^2  = sum_i p_ij^2 dO_id^2 (1 + A_i).
    """
    p2 = p * p
    A = p2.sum(axis=1)
    B = (p * ds).sum(axis=1)
    C = (ds * ds).sum(axis=1)
    E = ((do * o) ** 2).sum(axis=1)
    out = {"lse": np.sqrt(A)}
    if rows:
        m_o2 = p2 @ (v * v) - 2.0 * o * (p2 @ v) + o * o * A[:, None]
        dq = (ds @ k) * scale
        kbar = p @ k
        m_dq2 = (dq * dq * A[:, None] + 2.0 * scale * dq * kbar * B[:, None]
                 + scale * scale * kbar * kbar * (C + E)[:, None]
                 + scale * scale * ((ds * ds) @ (k * k)))
        out["o"] = np.sqrt(np.maximum(m_o2, 0.0))
        out["dq"] = np.sqrt(np.maximum(m_dq2, 0.0))
    if cols is not False:
        pc, dsc = (p, ds) if cols is None else (p[:, cols], ds[:, cols])
        w = dsc * dsc * (A + 1.0)[:, None] + 2.0 * dsc * pc * B[:, None] + pc * pc * (C + E)[:, None]
        out["dk2"] = np.maximum((w.T @ (q * q)) * scale * scale, 0.0)
        out["dv2"] = (pc * pc * (1.0 + A)[:, None]).T @ (do * do)
    return out


def backward(q, k, v, do, spec, scale=None, kv_heads=None, row_block=512,
             o_for_d="exact", magnitudes=False):
    """dQ, dK, dV (and O, LSE) for the selected KV heads and their groups.

    Returns a dict with dq [B,S,G*n,d] for the query heads of the selected KV
    heads (in order), dk/dv [B,S,n,d], o and lse for the same query heads,
    and ``heads``, the query head indices covered.

    ``o_for_d``: the O entering D_i = dO_i . O_i.  "exact" uses the exact
    output; "bf16" uses it rounded to bfloat16.

    ``magnitudes``: also return the first-order sensitivity of every output
    element to relative perturbations of the intermediate values a tiled
    kernel rounds (see ``_sensitivities``): "m_o", "m_dq", "m_dk", "m_dv"
    (same shapes as the outputs) and "m_lse" ([B, G*n, S]).
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
        m_lse = np.zeros_like(lse)
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
                    sv = _sensitivities(p, ds, oi, doi, qi, kk, vv, scale)
                    m_o[b, i0:i1, hi, :] = sv["o"]
                    m_dq[b, i0:i1, hi, :] = sv["dq"]
                    m_lse[b, hi, i0:i1] = sv["lse"]
                    m_dk2[b, :, kvi, :] += sv["dk2"]
                    m_dv2[b, :, kvi, :] += sv["dv2"]
    out = {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "heads": heads}
    if magnitudes:
        out.update(m_o=m_o, m_dq=m_dq, m_dk=np.sqrt(m_dk2), m_dv=np.sqrt(m_dv2), m_lse=m_lse)
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
    dq [len(rows), d], o [len(rows), d], lse [len(rows)] and the
    sensitivities m_dq, m_o, m_lse (see ``backward``)."""
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
    out["m_lse"] = np.zeros(len(rows))
    for r, i in enumerate(rows):
        s = (kk @ q[0, i, h, :]) * scale
        p, l = _probs(s[None, :], masks.allowed(spec, i, i + 1, hm))
        oi = p @ vv
        od = oi if o_for_d == "exact" else round_bf16(oi)
        doi = do[0, i:i + 1, h, :]
        Di = float(doi[0] @ od[0])
        dp = doi @ vv.T
        ds = p * (dp - Di)
        out["dq"][r] = (ds @ kk)[0] * scale
        out["o"][r] = oi[0]
        out["lse"][r] = l[0]
        sv = _sensitivities(p, ds, oi, doi, q[0, i:i + 1, h, :], kk, vv, scale, cols=False)
        out["m_dq"][r] = sv["dq"][0]
        out["m_o"][r] = sv["o"][0]
        out["m_lse"][r] = sv["lse"][0]
    return out


def grad_cols(q, k, v, do, spec, kv_head, cols, scale=None, row_block=512, heads=None):
    """dK and dV of KV head ``kv_head`` for chosen key columns only (batch 0),
    with their sensitivities m_dk, m_dv (see ``backward``).

    dK_j = scale sum_{h, i} dS_ij q_i and dV_j = sum_{h, i} P_ij dO_i over the
    query heads h of the group and the rows i allowed to attend to j.  Such a
    row's P_ij, D_i = dO_i . O_i and the row sums of the sensitivities need
    its whole score row, so exactly those rows are formed in full, in row
    blocks, each over the keys that some row of the block may attend to
    (P is zero on every other key); only the chosen columns' terms are
    accumulated.  ``heads``: only these query heads of the group contribute
    (default: all of them; squared sensitivities add over heads).  Returns
    dk, dv, m_dk, m_dv [len(cols), d] and ``pairs``, the number of (row, key)
    scores formed."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    cols = np.asarray(cols, dtype=np.int64)
    out = {n: np.zeros((len(cols), d)) for n in ("dk", "dv", "m_dk", "m_dv")}
    all_j = np.arange(S, dtype=np.int64)[None, :]
    pairs = 0
    for h in (range(kv_head * G, kv_head * G + G) if heads is None else heads):
        assert h // G == kv_head
        hm = masks.mask_head(spec, h, Hq, Hkv)
        rows = np.nonzero(masks.pred(spec, np.arange(S)[:, None], cols[None, :], hm).any(axis=1))[0]
        for r0 in range(0, len(rows), row_block):
            ri = rows[r0:r0 + row_block]
            a = masks.pred(spec, ri[:, None], all_j, hm)
            keys = np.nonzero(a.any(axis=0))[0]      # keys some row of the block sees
            a = a[:, keys]
            pairs += a.size
            kk = k[0, keys, kv_head, :]
            vv = v[0, keys, kv_head, :]
            qi = q[0, ri, h, :]
            doi = do[0, ri, h, :]
            p, _ = _probs((qi @ kk.T) * scale, a)
            oi = p @ vv
            D = (doi * oi).sum(axis=1)
            ds = p * (doi @ vv.T - D[:, None])
            at = np.searchsorted(keys, cols)          # chosen columns among the block's keys
            seen = (at < len(keys)) & (keys[np.minimum(at, len(keys) - 1)] == cols)
            if not seen.any():
                continue
            sel = at[seen]
            out["dk"][seen] += (ds[:, sel].T @ qi) * scale
            out["dv"][seen] += p[:, sel].T @ doi
            sv = _sensitivities(p, ds, oi, doi, qi, kk, vv, scale, cols=sel, rows=False)
            out["m_dk"][seen] += sv["dk2"]
            out["m_dv"][seen] += sv["dv2"]
    out["m_dk"] = np.sqrt(out["m_dk"])
    out["m_dv"] = np.sqrt(out["m_dv"])
    out["pairs"] = pairs
    return out
