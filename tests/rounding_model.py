"""The kernels' arithmetic as a perturbed pipeline, for pinning the parity
gate's rounding room on the CPU.

The library's kernels compute in fp32 with bf16 operands and round to bf16
at five points (the forward and backward kernels' own comments state them):

  forward   the unnormalised probabilities p~_ij, before P V and before their
            sum l_i (so LSE_i = m_i + ln l_i uses the rounded values), and
            the output O;
  backward  P_ij = exp(S_ij - LSE_i) before dV = P^T dO; dS_ij before
            dK = scale dS^T Q (dK/dV pass) and before dQ = scale dS K (dQ
            pass); and the outputs dQ, dK, dV.  D_i = dO_i . O_i uses the O
            the backward is given.

``pipeline`` computes all outputs from the full score matrices in fp64, with
either a relative perturbation or a rounding function applied at each of
those points.  With zero perturbations it is the exact definition; with
bf16 rounding at every point it is a model of the kernels' arithmetic (fp32
accumulation, whose error is about 2^-24 relative per term, is left out).

Uses: the oracle's first-order sensitivities are pinned against central
differences of this pipeline (tests/test_gate.py), and the gate is shown to
hold, with margin, on the rounded pipeline, and to fail on it with mistakes
planted in it.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import masks as om


def pipeline(q, k, v, do, spec, pert=None, rnd=None, plant=None):
    """Forward + backward of masked attention with perturbed or rounded
    intermediates.

    q, k, v, do: float64 [B, S, Hq|Hkv, d].  ``pert``: optional dict of
    relative perturbations, each applied as x -> x (1 + e):
      "delta" [B, Hq, S, S]  forward p~_ij
      "eps"   [B, S, Hq, d]  O handed to the backward
      "eta_v" [B, Hq, S, S]  P_ij entering dV
      "eta_k" [B, Hq, S, S]  dS_ij entering dK
      "eta_q" [B, Hq, S, S]  dS_ij entering dQ
    ``rnd``: a rounding function applied at the same points and to the
    outputs dQ, dK, dV (O is rounded where it is handed over).
    ``plant``: name of a deliberate mistake (see PLANTS), for tests that show
    the gate catches it.

    Returns dict o, lse, dq, dk, dv; o is the O handed to the backward.
    """
    pert = pert or {}
    r = rnd if rnd is not None else (lambda x: x)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, S, Hq, d))
    lse = np.zeros((B, Hq, S))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            hm = om.mask_head(spec, h, Hq, Hkv)
            a = om.allowed(spec, 0, S, hm)
            if plant == "drop_diagonal":
                a = a & ~np.eye(S, dtype=bool) | (a & (a.sum(axis=1, keepdims=True) == 1))
            kk, vv = k[b, :, kv], v[b, :, kv]
            s = (q[b, :, h] @ kk.T) * scale
            sm = np.where(a, s, -np.inf)
            m = sm.max(axis=1)
            live = np.isfinite(m)
            m0 = np.where(live, m, 0.0)
            pt = np.where(a, np.exp(sm - m0[:, None]), 0.0)
            if "delta" in pert:
                pt = pt * (1.0 + pert["delta"][b, h])
            pt = r(pt)
            lsum = pt.sum(axis=1)
            if plant == "normaliser_skips_last_key":
                last = np.where(a.any(axis=1), S - 1 - np.argmax(a[:, ::-1], axis=1), 0)
                lsum = lsum - np.where(a.sum(axis=1) > 1, pt[np.arange(S), last], 0.0)
            den = np.where(live, lsum, 1.0)
            oi = np.where(live[:, None], (pt @ vv) / den[:, None], 0.0)
            if "eps" in pert:
                oi = oi * (1.0 + pert["eps"][b, :, h])
            oi = r(oi)
            li = np.where(live, m0 + np.log(den), -np.inf)
            o[b, :, h] = oi
            lse[b, h] = li
            # backward, from the O and LSE just handed over
            doi = do[b, :, h]
            if plant == "d_from_other_head":
                doi_d = do[b, :, (h + 1) % Hq]
            else:
                doi_d = doi
            D = (doi_d * oi).sum(axis=1)
            lb = np.where(live, li, 0.0)
            pb = np.where(a & live[:, None], np.exp(np.where(a, s, 0.0) - lb[:, None]), 0.0)
            dp = doi @ vv.T
            ds = pb * (dp - D[:, None])
            if plant == "ds_sign":
                ds = -ds
            pv = pb * (1.0 + pert["eta_v"][b, h]) if "eta_v" in pert else pb
            dsk = ds * (1.0 + pert["eta_k"][b, h]) if "eta_k" in pert else ds
            dsq = ds * (1.0 + pert["eta_q"][b, h]) if "eta_q" in pert else ds
            dv[b, :, kv] += r(pv).T @ doi
            ksc = 1.0 if plant == "dk_unscaled" else scale
            dk[b, :, kv] += (r(dsk).T @ q[b, :, h]) * ksc
            dq[b, :, h] = (r(dsq) @ kk) * scale
    return {"o": o, "lse": lse, "dq": r(dq), "dk": r(dk), "dv": r(dv)}


# Mistakes a kernel could plausibly make, planted in the pipeline only.
PLANTS = ("drop_diagonal", "normaliser_skips_last_key", "d_from_other_head", "ds_sign",
          "dk_unscaled")


def numeric_sensitivities(q, k, v, do, spec, step=1e-6):
    """2-norms of the first-order coefficients of every output element with
    respect to every perturbation of ``pipeline``, by central differences
    (tiny inputs only: two pipeline runs per perturbed value).  O's own
    hand-over perturbation eps is its final rounding and is left out of O's
    norm, as in the oracle's sensitivities."""
    B, S, Hq, d = q.shape
    shapes = {"delta": (B, Hq, S, S), "eps": (B, S, Hq, d), "eta_v": (B, Hq, S, S),
              "eta_k": (B, Hq, S, S), "eta_q": (B, Hq, S, S)}
    names = ("o", "lse", "dq", "dk", "dv")
    acc = {n: 0.0 for n in names}
    for key, shp in shapes.items():
        for idx in np.ndindex(*shp):
            e = np.zeros(shp)
            e[idx] = step
            up = pipeline(q, k, v, do, spec, pert={key: e})
            dn = pipeline(q, k, v, do, spec, pert={key: -e})
            for n in names:
                if n == "o" and key == "eps":
                    continue
                c = (np.nan_to_num(up[n], neginf=0.0) - np.nan_to_num(dn[n], neginf=0.0)) / (2 * step)
                acc[n] = acc[n] + c * c
    return {n: np.sqrt(acc[n]) for n in names}
