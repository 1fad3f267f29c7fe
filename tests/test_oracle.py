"""Pins for the fp64 oracle: things other than the oracle itself.

* hand-drawn mask grids (tests/golden) and closed-form pair counts pin the
  mask predicates;
* the pure-Python brute force pins the vectorised fp64 forward/backward;
* central finite differences pin the backward formulas;
* closed forms (uniform V, Q = 0, single-key rows) and invariants (rows of P
  sum to one, sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, unseen keys get zero
  gradient, DOCUMENT = independent per-document attention, GQA = MHA on
  repeated K/V) pin the arithmetic end to end;
* the merge of partial results is pinned by the forward over the union of
  disjoint key sets, a two-key closed form and empty parts.
"""
import json
import math
import os

import numpy as np
import pytest

import synthetic as syn
from oracle import attention as ora
from oracle import bruteforce as bf
from oracle import masks as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_grids():
    out = []
    label, spec, rows = None, None, []
    with open(os.path.join(GOLDEN, "mask_grids_S12.txt")) as f:
        for line in f:
            line = line.rstrip("\n")
            if line.startswith("#") or not line.strip():
                continue
            if line.startswith("== "):
                if label is not None:
                    out.append((label, spec, rows))
                _, label, js = line.split(" ", 2)
                spec = json.loads(js)
                if "bitmap" in spec:
                    spec["bitmap"]["bits"] = np.array(spec["bitmap"]["bits"], dtype=np.uint8)
                rows = []
            else:
                rows.append(line)
    out.append((label, spec, rows))
    return out


GRIDS = _load_grids()


@pytest.mark.parametrize("label,spec,rows", GRIDS, ids=[g[0] for g in GRIDS])
def test_mask_grid_golden(label, spec, rows):
    want = np.array([[c == "1" for c in r] for r in rows])
    assert want.shape == (12, 12)
    got = om.dense_mask(spec)
    assert (got == want).all(), f"{label}:\n{got.astype(int)}"
    got_bf = np.array([[bf.allowed(spec, i, j) for j in range(12)] for i in range(12)])
    assert (got_bf == want).all()


def _tiny_specs(S):
    docs = [7, 13, 3, S - 23]
    q = 9
    out = [
        syn.spec_full(S), syn.spec_causal(S), syn.spec_sliding(S, 5, True),
        syn.spec_sliding(S, 4, False), syn.spec_document(docs, False),
        syn.spec_document(docs, True), syn.spec_prefix_lm_causal(S, 6),
        syn.spec_shared_question(q, [5, 0, 11, S - q - 16]),
        syn.spec_global_sliding(S, 3, 5), syn.spec_global_sliding(S, 3, 4, True),
        syn.spec_causal_blockwise(S, 8), syn.spec_causal_blockwise(S, 8, "block_causal"),
        syn.spec_prefix_lm_document(docs, [2, 13, 0, 5]),
        syn.spec_block_causal_document(docs, 4),
        syn.spec_task_batch(docs, [3, 13, 1, 4]),
    ]
    offs, bits = syn.variable_block_bitmap(S, 3, 9, 2, 0.5, seed=3)
    out.append(syn.with_bitmap(syn.spec_causal(S), offs, offs, bits))
    offs, bits = syn.uniform_block_bitmap(S, 8, 1, 0.5, seed=4)
    out.append(syn.with_bitmap(syn.spec_full(S), offs, offs, bits))
    return out


@pytest.mark.parametrize("spec", _tiny_specs(40), ids=lambda s: s["family"] + ("+bm" if "bitmap" in s else ""))
def test_predicate_matches_bruteforce(spec):
    S = spec["S"]
    nh = spec["bitmap"]["bits"].shape[0] if "bitmap" in spec else 1
    for hm in range(nh):
        got = om.dense_mask(spec, hm)
        want = np.array([[bf.allowed(spec, i, j, hm) for j in range(S)] for i in range(S)])
        assert (got == want).all()


def test_nnz_closed_forms():
    """Closed-form allowed-pair counts of each family."""
    S = 1000
    assert om.nnz(syn.spec_full(S)) == S * S
    assert om.nnz(syn.spec_causal(S)) == S * (S + 1) // 2
    w = 37
    csw = w * (w + 1) // 2 + (S - w) * w
    assert om.nnz(syn.spec_sliding(S, w, True)) == csw
    assert om.nnz(syn.spec_sliding(S, w, False)) == S * (2 * w - 1) - w * (w - 1)
    docs = syn.sample_doc_lens(S, 16, 256, seed=1)
    assert sum(docs) == S
    assert om.nnz(syn.spec_document(docs, False)) == sum(L * L for L in docs)
    assert om.nnz(syn.spec_document(docs, True)) == sum(L * (L + 1) // 2 for L in docs)
    p = 123
    assert om.nnz(syn.spec_prefix_lm_causal(S, p)) == S * (S + 1) // 2 + p * (p - 1) // 2
    q, ans = 100, [250, 0, 400, 250]
    want = q * (q + 1) // 2 + sum(a * q + a * (a + 1) // 2 for a in ans)
    assert om.nnz(syn.spec_shared_question(q, ans)) == want
    g, w = 16, 100
    csw = w * (w + 1) // 2 + (S - w) * w
    assert om.nnz(syn.spec_global_sliding(S, g, w)) == csw + g * (S - w) - g * (g - 1) // 2
    b = 200
    n = S // b
    assert om.nnz(syn.spec_causal_blockwise(S, b)) == n * b * (b + 1) // 2 + (S - b) * b
    assert om.nnz(syn.spec_causal_blockwise(S, b, "block_causal")) == b * b * n * (n + 1) // 2
    kv, ql = [300, 5, 450, 245], [300, 1, 17, 100]
    want = sum(qq * (qq + 1) // 2 + qq * (k - qq) for k, qq in zip(kv, ql))
    assert om.nnz(syn.spec_task_batch(kv, ql)) == want
    offs, bits = syn.variable_block_bitmap(S, 32, 224, 2, 0.5, seed=2)
    sizes = np.diff(offs)
    for hm in range(2):
        want = int((bits[hm] * np.outer(sizes, sizes)).sum())
        assert om.nnz(syn.with_bitmap(syn.spec_full(S), offs, offs, bits), hm) == want


def _to_f64(bits):
    return syn.bf16_bits_to_f32(bits).astype(np.float64)


def _inputs(S, Hq, Hkv, d, seed):
    t = syn.attention_inputs(1, S, Hq, Hkv, d, seed)
    return {k: _to_f64(v) for k, v in t.items()}


@pytest.mark.parametrize("spec", _tiny_specs(28)[:8] + _tiny_specs(28)[10:], ids=lambda s: s["family"])
def test_fp64_matches_bruteforce(spec):
    S, Hq, Hkv, d = spec["S"], 2, 1, 3
    x = _inputs(S, Hq, Hkv, d, seed=5)
    nh = spec["bitmap"]["bits"].shape[0] if "bitmap" in spec else 1
    hm_of = (lambda h: om.mask_head(spec, h, Hq, Hkv)) if nh > 1 else (lambda h: 0)
    if nh not in (1, Hq, Hkv):
        pytest.skip("bitmap head count")
    ref = bf.attention(x["q"][0].tolist(), x["k"][0].tolist(), x["v"][0].tolist(),
                       x["do"][0].tolist(), spec, hm_of_head=hm_of)
    o, lse = ora.forward(x["q"], x["k"], x["v"], spec)
    g = ora.backward(x["q"], x["k"], x["v"], x["do"], spec)
    np.testing.assert_allclose(o[0], np.array(ref["o"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0], np.array(ref["lse"]), rtol=1e-12, atol=1e-12)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g[name][0], np.array(ref[name]), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["o"], o, rtol=0, atol=1e-14)


def _loss(q, k, v, do, spec):
    o, _ = ora.forward(q, k, v, spec)
    return float((o * do).sum())


@pytest.mark.parametrize("spec", [syn.spec_causal(12), syn.spec_sliding(12, 3, False),
                                  syn.spec_shared_question(3, [4, 5]),
                                  syn.spec_document([5, 7], True)],
                         ids=["causal", "full_sw", "shared_question", "causal_doc"])
def test_backward_finite_differences(spec):
    """dQ, dK, dV equal the central differences of L = sum(dO * O)."""
    S, Hq, Hkv, d = spec["S"], 4, 2, 3
    rng = np.random.default_rng(11)
    q, do = rng.standard_normal((2, 1, S, Hq, d))
    k, v = rng.standard_normal((2, 1, S, Hkv, d))
    g = ora.backward(q, k, v, do, spec)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do, spec)
            x[idx] = old - eps
            lm = _loss(q, k, v, do, spec)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("spec", _tiny_specs(64), ids=lambda s: s["family"])
def test_uniform_v_closed_form(spec):
    """v_j = v for all j gives O_i = v, dQ = dK = 0, and sum_j dV_j = sum_i dO_i."""
    S, Hq, Hkv, d = spec["S"], 4, 2, 8
    x = _inputs(S, Hq, Hkv, d, seed=1)
    v = np.broadcast_to(x["v"][:, :1], x["v"].shape).copy()
    g = ora.backward(x["q"], x["k"], v, x["do"], spec)
    G = Hq // Hkv
    for h in range(Hq):
        hm = om.mask_head(spec, h, Hq, Hkv)
        rows = om.dense_mask(spec, hm).any(axis=1)
        np.testing.assert_allclose(g["o"][0, rows, h], np.broadcast_to(v[0, 0, h // G], (rows.sum(), d)), atol=1e-12)
        assert np.abs(g["o"][0, ~rows, h]).max(initial=0) == 0
    assert np.abs(g["dq"]).max() < 1e-12
    assert np.abs(g["dk"]).max() < 1e-12


@pytest.mark.parametrize("spec", _tiny_specs(64), ids=lambda s: s["family"])
def test_zero_q_closed_form(spec):
    """Q = 0 gives uniform weights: O_i = mean of allowed v_j, LSE_i = ln n_i."""
    S, Hq, Hkv, d = spec["S"], 2, 2, 4
    x = _inputs(S, Hq, Hkv, d, seed=2)
    q = np.zeros_like(x["q"])
    o, lse = ora.forward(q, x["k"], x["v"], spec)
    for h in range(Hq):
        a = om.dense_mask(spec, om.mask_head(spec, h, Hq, Hkv))
        n = a.sum(axis=1)
        for i in range(S):
            if n[i] == 0:
                assert lse[0, h, i] == -np.inf and not o[0, i, h].any()
                continue
            assert abs(lse[0, h, i] - math.log(n[i])) < 1e-12
            np.testing.assert_allclose(o[0, i, h], x["v"][0, a[i], h].mean(axis=0), atol=1e-12)


def test_single_key_row():
    """Causal row 0 sees only key 0: O_0 = v_0, LSE_0 = s_00, dQ_0 = 0."""
    S, d = 16, 8
    x = _inputs(S, 1, 1, d, seed=3)
    g = ora.backward(x["q"], x["k"], x["v"], x["do"], syn.spec_causal(S))
    np.testing.assert_allclose(g["o"][0, 0, 0], x["v"][0, 0, 0], atol=1e-14)
    s00 = float(x["q"][0, 0, 0] @ x["k"][0, 0, 0]) / math.sqrt(d)
    assert abs(g["lse"][0, 0, 0] - s00) < 1e-12
    assert np.abs(g["dq"][0, 0, 0]).max() < 1e-14


@pytest.mark.parametrize("spec", _tiny_specs(48), ids=lambda s: s["family"])
def test_gradient_invariants(spec):
    """sum_j dK_j = 0 (shift invariance in K); sum_j dV_j = sum over rows with
    an allowed key of dO_i; keys no row sees get dK = dV = 0."""
    S, Hq, Hkv, d = spec["S"], 4, 2, 5
    x = _inputs(S, Hq, Hkv, d, seed=4)
    g = ora.backward(x["q"], x["k"], x["v"], x["do"], spec)
    G = Hq // Hkv
    for kv in range(Hkv):
        assert np.abs(g["dk"][0, :, kv].sum(axis=0)).max() < 1e-10
        want = np.zeros(d)
        seen = np.zeros(S, dtype=bool)
        for h in range(kv * G, kv * G + G):
            a = om.dense_mask(spec, om.mask_head(spec, h, Hq, Hkv))
            want += x["do"][0, a.any(axis=1), h].sum(axis=0)
            seen |= a.any(axis=0)
        np.testing.assert_allclose(g["dv"][0, :, kv].sum(axis=0), want, atol=1e-10)
        assert np.abs(g["dk"][0, ~seen, kv]).max(initial=0) == 0
        assert np.abs(g["dv"][0, ~seen, kv]).max(initial=0) == 0


def test_empty_rows_and_unseen_keys():
    """A bitmap that hides a whole block row and block column."""
    S = 12
    offs = [0, 4, 8, 12]
    bits = np.array([[[1, 0, 1], [0, 0, 0], [1, 0, 1]]], dtype=np.uint8)
    spec = syn.with_bitmap(syn.spec_full(S), offs, offs, bits)
    x = _inputs(S, 1, 1, 4, seed=6)
    g = ora.backward(x["q"], x["k"], x["v"], x["do"], spec)
    assert (g["lse"][0, 0, 4:8] == -np.inf).all()
    assert not g["o"][0, 4:8].any() and not g["dq"][0, 4:8].any()
    assert not g["dk"][0, 4:8].any() and not g["dv"][0, 4:8].any()


def test_document_equals_independent_attention():
    docs = [9, 17, 6]
    x = _inputs(sum(docs), 4, 2, 6, seed=7)
    for causal in (False, True):
        spec = syn.spec_document(docs, causal)
        g = ora.backward(x["q"], x["k"], x["v"], x["do"], spec)
        s = 0
        for L in docs:
            sub = {k: v[:, s:s + L] for k, v in x.items()}
            sp = syn.spec_causal(L) if causal else syn.spec_full(L)
            gs = ora.backward(sub["q"], sub["k"], sub["v"], sub["do"], sp)
            for name in ("o", "dq", "dk", "dv"):
                np.testing.assert_allclose(g[name][:, s:s + L], gs[name], atol=1e-13)
            np.testing.assert_allclose(g["lse"][:, :, s:s + L], gs["lse"], atol=1e-13)
            s += L


def test_gqa_equals_mha_on_repeated_kv():
    S, Hq, Hkv, d = 24, 6, 2, 4
    G = Hq // Hkv
    x = _inputs(S, Hq, Hkv, d, seed=8)
    spec = syn.spec_sliding(S, 7, True)
    g = ora.backward(x["q"], x["k"], x["v"], x["do"], spec)
    kr = np.repeat(x["k"], G, axis=2)
    vr = np.repeat(x["v"], G, axis=2)
    gm = ora.backward(x["q"], kr, vr, x["do"], spec)
    np.testing.assert_allclose(g["o"], gm["o"], atol=1e-14)
    np.testing.assert_allclose(g["dq"], gm["dq"], atol=1e-13)
    np.testing.assert_allclose(g["dk"], gm["dk"].reshape(1, S, Hkv, G, d).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(g["dv"], gm["dv"].reshape(1, S, Hkv, G, d).sum(axis=3), atol=1e-13)


def test_probability_rows_sum_to_one():
    """With V = 1 every non-empty row of O is exactly the row sum of P."""
    S = 40
    for spec in _tiny_specs(S):
        x = _inputs(S, 2, 1, 3, seed=9)
        v = np.ones_like(x["v"])
        o, _ = ora.forward(x["q"], x["k"], v, spec)
        a = om.dense_mask(spec, 0).any(axis=1)
        np.testing.assert_allclose(o[0, a, 0], 1.0, atol=1e-14)


def test_output_rows_matches_forward():
    S = 96
    spec = syn.spec_global_sliding(S, 4, 9)
    x = _inputs(S, 4, 2, 8, seed=10)
    o, lse = ora.forward(x["q"], x["k"], x["v"], spec)
    rows = [0, 5, 50, 95]
    for h in (0, 3):
        orow, lrow = ora.output_rows(x["q"], x["k"], x["v"], spec, h, rows)
        np.testing.assert_allclose(orow, o[0, rows, h], atol=1e-14)
        np.testing.assert_allclose(lrow, lse[0, h, rows], atol=1e-14)


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 1.0 + 2**-8 + 2**-20], dtype=np.float32)
    b = syn.bf16_bits_to_f32(syn.bf16_bits_from_f32(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to even (1.0)
    assert b[0] == 1.0 and b[1] == 1.0 and b[2] == np.float32(1.015625)
    assert b[3] == -2.5
    assert b[5] == np.float32(1.0078125)
    assert abs(b[4] - 3.0e-3) < 3.0e-3 * 2**-8


def test_round_bf16_pins():
    """The oracle's bf16 rounding against hand values and against the input
    generator's independent implementation."""
    hand = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-30, -2.5, 0.0,
                     3.0 * 2**-140 * 2**10])
    want = np.array([1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.5, 0.0, 3.0 * 2**-130])
    np.testing.assert_array_equal(ora.round_bf16(hand), want)
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    other = syn.bf16_bits_to_f32(syn.bf16_bits_from_f32(x)).astype(np.float64)
    np.testing.assert_array_equal(ora.round_bf16(x.astype(np.float64)), other)


def test_sensitivity_special_cases():
    """First-order sensitivities (the closed forms are pinned against central
    differences in tests/test_gate.py): a row with one key has O = v exactly
    whatever its probability's rounding, so |c(O)| = 0 and |c(LSE)| = 1; the
    forward's output sensitivity vanishes under uniform V; every value is
    finite and non-negative."""
    S, d = 16, 4
    x = _inputs(S, 2, 1, d, seed=12)
    spec = syn.spec_causal(S)
    g = ora.backward(x["q"], x["k"], x["v"], x["do"], spec, magnitudes=True)
    np.testing.assert_allclose(g["m_o"][0, 0], 0.0, atol=1e-12)
    np.testing.assert_allclose(g["m_lse"][0, :, 0], 1.0, rtol=1e-14)
    assert (g["m_lse"][0, :, 1:] < 1.0).all()
    for n in ("m_o", "m_dq", "m_dk", "m_dv", "m_lse"):
        assert np.isfinite(g[n]).all() and (g[n] >= 0).all()
    v1 = np.broadcast_to(x["v"][:, :1], x["v"].shape).copy()
    g1 = ora.backward(x["q"], x["k"], v1, x["do"], spec, magnitudes=True)
    # (the closed form expands sum_j p^2 (v - O)^2, which cancels to ~1e-16
    # of sum_j p^2 v^2 in fp64)
    np.testing.assert_allclose(g1["m_o"], 0.0, atol=1e-7)


def test_o_for_d_bf16_is_exact_when_o_is_representable():
    """With V constant and bf16-representable, O is exactly representable, so
    D from the rounded O equals D from the exact O; otherwise they differ."""
    S = 40
    x = _inputs(S, 2, 1, 4, seed=13)
    spec = syn.spec_sliding(S, 9, True)
    v = np.broadcast_to(x["v"][:, :1], x["v"].shape).copy()
    a = ora.backward(x["q"], x["k"], v, x["do"], spec)
    b = ora.backward(x["q"], x["k"], v, x["do"], spec, o_for_d="bf16")
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(a[n], b[n], atol=1e-13)
    c = ora.backward(x["q"], x["k"], x["v"], x["do"], spec, o_for_d="bf16")
    e = ora.backward(x["q"], x["k"], x["v"], x["do"], spec)
    assert np.abs(c["dq"] - e["dq"]).max() > 0
    np.testing.assert_array_equal(c["dv"], e["dv"])


def test_grad_rows_matches_backward():
    """The per-row oracle path agrees with the whole-tensor backward."""
    S, Hq, Hkv, d = 80, 4, 2, 6
    x = _inputs(S, Hq, Hkv, d, seed=14)
    offs, bits = syn.variable_block_bitmap(S, 5, 20, Hkv, 0.5, seed=15)
    for spec in (syn.spec_causal(S), syn.spec_shared_question(10, [30, 40]),
                 syn.with_bitmap(syn.spec_full(S), offs, offs, bits)):
        for o_for_d in ("exact", "bf16"):
            g = ora.backward(x["q"], x["k"], x["v"], x["do"], spec, o_for_d=o_for_d, magnitudes=True)
            rows = [0, 1, 37, 79]
            for h in (0, 3):
                r = ora.grad_rows(x["q"], x["k"], x["v"], x["do"], spec, h, rows, o_for_d=o_for_d)
                np.testing.assert_allclose(r["dq"], g["dq"][0, rows, h], atol=1e-13)
                np.testing.assert_allclose(r["o"], g["o"][0, rows, h], atol=1e-14)
                np.testing.assert_allclose(r["lse"], g["lse"][0, h, rows], atol=1e-14)
                np.testing.assert_allclose(r["m_dq"], g["m_dq"][0, rows, h], atol=1e-13)
                np.testing.assert_allclose(r["m_o"], g["m_o"][0, rows, h], atol=1e-13)
                np.testing.assert_allclose(r["m_lse"], g["m_lse"][0, h, rows], atol=1e-14)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (3, 3)])
def test_grad_cols_matches_backward(Hq, Hkv):
    """The per-column oracle path (full rows of only the rows that see the
    chosen keys, over the keys their block sees) agrees with the
    whole-tensor backward: GQA and MHA, bitmaps per KV head and per query
    head, windows, rows with no key, unseen keys."""
    S, d = 80, 6
    x = _inputs(S, Hq, Hkv, d, seed=16)
    offs, bits = syn.variable_block_bitmap(S, 5, 20, Hkv, 0.5, seed=17)
    uoffs, ubits = syn.uniform_block_bitmap(S, 16, Hq, 0.4, seed=18)
    specs = (syn.spec_causal(S), syn.spec_sliding(S, 7, True),
             syn.with_bitmap(syn.spec_full(S), offs, offs, bits),
             syn.with_bitmap(syn.spec_causal(S), uoffs, uoffs, ubits),
             syn.spec_task_batch([30, 50], [10, 20]), syn.spec_global_sliding(S, 3, 9))
    cols = [0, 1, 17, 40, 63, 79]
    for spec in specs:
        g = ora.backward(x["q"], x["k"], x["v"], x["do"], spec, magnitudes=True)
        for kv in range(Hkv):
            r = ora.grad_cols(x["q"], x["k"], x["v"], x["do"], spec, kv, cols, row_block=16)
            for n in ("dk", "dv", "m_dk", "m_dv"):
                np.testing.assert_allclose(r[n], g[n][0, cols, kv], atol=1e-12, err_msg=n)


def _key_split(base, cuts):
    """Specs of base restricted to the key ranges between consecutive cuts
    (a one-row-block bitmap with column blocks at the cuts)."""
    S = base["S"]
    offs = [0] + list(cuts) + [S]
    out = []
    for c in range(len(offs) - 1):
        bits = np.zeros((1, 1, len(offs) - 1), dtype=np.uint8)
        bits[0, 0, c] = 1
        out.append(syn.with_bitmap(base, [0, S], offs, bits))
    return out


@pytest.mark.parametrize("base,cuts", [
    (syn.spec_causal(97), [40]),
    (syn.spec_full(64), [10, 33, 50]),
    (syn.spec_document([30, 20, 27], True), [25]),
    (syn.spec_sliding(80, 16, True), [8, 72]),
])
def test_merge_over_key_partition_equals_forward(base, cuts):
    """Attention over the union of disjoint key sets, from the pinned fp64
    forward over each set, equals the forward over the union; the part
    order does not matter."""
    S = base["S"]
    x = syn.attention_inputs(1, S, 4, 2, 16, seed=4)
    q, k, v = (syn.bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v"))
    parts = [ora.forward(q, k, v, sp) for sp in _key_split(base, cuts)]
    o, lse = ora.merge([p[0] for p in parts], [p[1] for p in parts])
    o_ref, lse_ref = ora.forward(q, k, v, base)
    assert np.abs(o - o_ref).max() < 1e-12
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(lse) == fin).all()
    assert np.abs(lse[fin] - lse_ref[fin]).max() < 1e-12
    o2, lse2 = ora.merge([p[0] for p in parts[::-1]], [p[1] for p in parts[::-1]])
    assert np.abs(o2 - o).max() < 1e-12 and np.abs(lse2[fin] - lse[fin]).max() < 1e-12


def test_merge_two_single_keys_closed_form():
    """Two parts of one key each: the merge is the softmax over the two
    scores written out by hand."""
    va, vb = np.array([1.0, -2.0, 0.5]), np.array([3.0, 0.25, -1.0])
    sa, sb = 0.7, -1.3
    o, lse = ora.merge([va.reshape(1, 1, 1, 3), vb.reshape(1, 1, 1, 3)],
                       [np.full((1, 1, 1), sa), np.full((1, 1, 1), sb)])
    pa = math.exp(sa) / (math.exp(sa) + math.exp(sb))
    assert np.abs(o.reshape(3) - (pa * va + (1 - pa) * vb)).max() < 1e-15
    assert abs(lse.item() - math.log(math.exp(sa) + math.exp(sb))) < 1e-15


def test_merge_empty_parts():
    """A part with no key for a row (O = 0, LSE = -inf) leaves the other part
    unchanged; rows empty in every part stay O = 0, LSE = -inf."""
    o1 = np.arange(6, dtype=np.float64).reshape(1, 2, 1, 3)
    l1 = np.array([[[0.3, -np.inf]]])
    o2 = np.zeros((1, 2, 1, 3))
    l2 = np.full((1, 1, 2), -np.inf)
    o, lse = ora.merge([o1, o2], [l1, l2])
    assert (o[0, 0] == o1[0, 0]).all() and lse[0, 0, 0] == 0.3
    assert (o[0, 1] == 0).all() and np.isneginf(lse[0, 0, 1])
