"""Pins for the parity gate's rounding room (CPU only).

* The oracle's first-order sensitivities m_x (the closed forms in
  oracle.attention._sensitivities) equal the 2-norms of the coefficients
  obtained by central differences of an independently written perturbed
  pipeline (tests/rounding_model.py), on tiny inputs covering GQA, bitmaps,
  windows and rows with no key.
* With bf16 rounding at every rounding point of the kernels, the pipeline
  passes the gate against the oracle with margin on the tiny config, ragged
  d = 128 cases and a causal block-sparse mask, chained (the backward takes
  the forward's own rounded O and LSE).
* The rounding room is needed: without its lam(N) u m_x term the same
  rounded pipeline fails on causal masks, whose first rows mix a handful of
  keys and are far larger than the tensor RMS.
* The room does not hide mistakes: each of several plausible kernel mistakes
  planted in the pipeline fails the gate.
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as ora

from gpu_util import GATE_MAX, GATE_MEAN, U_BF16, gate, room
import rounding_model as rm


def _inputs(B, S, Hq, Hkv, d, seed):
    x = syn.attention_inputs(B, S, Hq, Hkv, d, seed)
    return {n: syn.bf16_bits_to_f32(x[n]).astype(np.float64) for n in x}


def _tiny_specs(S):
    offs, bits = syn.variable_block_bitmap(S, 2, 4, 1, 0.5, seed=3)
    return [
        ("causal", syn.spec_causal(S)),
        ("sliding", syn.spec_sliding(S, 3, True)),
        ("full_bitmap", syn.with_bitmap(syn.spec_full(S), offs, offs, bits)),
        # rows with no key (context rows of a task)
        ("task_batch", syn.spec_task_batch([4, S - 4], [2, 1])),
    ]


@pytest.mark.parametrize("label,spec", _tiny_specs(7), ids=[l for l, _ in _tiny_specs(7)])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (2, 2)])
def test_sensitivities_match_central_differences(label, spec, Hq, Hkv):
    x = _inputs(1, 7, Hq, Hkv, 3, seed=21)
    ref = ora.backward(x["q"], x["k"], x["v"], x["do"], spec, magnitudes=True)
    num = rm.numeric_sensitivities(x["q"], x["k"], x["v"], x["do"], spec)
    for name, key in (("o", "m_o"), ("lse", "m_lse"), ("dq", "m_dq"), ("dk", "m_dk"), ("dv", "m_dv")):
        np.testing.assert_allclose(ref[key], num[name], rtol=2e-5, atol=1e-8, err_msg=name)


def test_pipeline_without_perturbation_is_the_oracle():
    S = 40
    x = _inputs(1, S, 4, 2, 8, seed=22)
    spec = syn.spec_causal(S)
    ref = ora.backward(x["q"], x["k"], x["v"], x["do"], spec)
    got = rm.pipeline(x["q"], x["k"], x["v"], x["do"], spec)
    for n in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(got[n], ref[n], rtol=1e-12, atol=1e-12, err_msg=n)


def _model_cases():
    tiny = [("tiny_" + l, s, (1, 512, 4, 2, 64)) for l, s in syn.config_mask_specs("tiny", Hkv=2)]
    S = 700
    docs = syn.sample_doc_lens(S, 16, 400, 3)
    ragged = [
        ("gqa700_causal", syn.spec_causal(S), (1, S, 8, 1, 128)),
        ("gqa700_causal_document", syn.spec_document(docs, True), (1, S, 8, 1, 128)),
        ("gqa700_global_sliding", syn.spec_global_sliding(S, 16, 100), (1, S, 8, 1, 128)),
        ("mha333_causal_sw", syn.spec_sliding(333, 130, True), (1, 333, 2, 2, 128)),
    ]
    # the causal block-sparse mask of the dynamic-plan tests: 128-blocks at
    # 30% density on a causal base, many rows with few keys
    offs, bits = syn.uniform_block_bitmap(640, 128, 2, 0.3, seed=5)
    sparse = [("causal_block128_30", syn.with_bitmap(syn.spec_causal(640), offs, offs, bits),
               (1, 640, 4, 2, 128))]
    return tiny + ragged + sparse


MODEL = _model_cases()
_RESULTS = {}


def _run_model(label, spec, shape, plant=None):
    key = (label, plant)
    if key not in _RESULTS:
        x = _inputs(*shape, seed=7)
        ref = ora.backward(x["q"], x["k"], x["v"], x["do"], spec, magnitudes=True)
        got = rm.pipeline(x["q"], x["k"], x["v"], x["do"], spec, rnd=ora.round_bf16, plant=plant)
        _RESULTS[key] = (got, ref)
    return _RESULTS[key]


@pytest.mark.parametrize("label,spec,shape", MODEL, ids=[c[0] for c in MODEL])
def test_rounded_pipeline_passes_the_gate(label, spec, shape):
    got, ref = _run_model(label, spec, shape)
    for n in ("o", "dq", "dk", "dv"):
        mx, mean, used = gate(n, got[n], ref[n], ref["m_" + n])
        # margin: at most 60% of the allowance is used
        assert used <= 0.6, (n, used)
    fin = np.isfinite(ref["lse"])
    assert (np.isneginf(got["lse"]) == ~fin).all()
    assert np.abs(got["lse"][fin] - ref["lse"][fin]).max() <= 5e-3


def _fails_without_rounding_room(got, ref):
    """Tensors that break the gate with the lam(N) u m_x term left out."""
    out = []
    for n in ("o", "dq", "dk", "dv"):
        rms = float(np.sqrt(np.mean(ref[n] ** 2)))
        err = np.abs(got[n] - ref[n])
        if (err > room(ref[n], None, rms)).any():
            out.append(n)
    return out


def test_gate_needs_the_rounding_room():
    """Causal masks: the literal bound plus output rounding is not enough for
    any bf16 kernel; the rounding term is what admits the rounded pipeline."""
    failing = {}
    for label, spec, shape in MODEL:
        if "causal" in label:
            got, ref = _run_model(label, spec, shape)
            failing[label] = _fails_without_rounding_room(got, ref)
    assert failing["tiny_causal"], failing
    assert sum(bool(v) for v in failing.values()) >= 3, failing


@pytest.mark.parametrize("plant", rm.PLANTS)
def test_gate_catches_planted_mistakes(plant):
    spec = syn.spec_causal(256)
    got, ref = _run_model("plant_causal256", spec, (1, 256, 4, 2, 64), plant=plant)
    caught = []
    for n in ("o", "dq", "dk", "dv"):
        try:
            gate(n, got[n], ref[n], ref["m_" + n])
        except AssertionError:
            caught.append(n)
    assert caught, plant


def test_lambda_and_unit_roundoff():
    """u is bf16's unit roundoff: the largest relative rounding error of
    round-to-nearest-even to 8 significant bits."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))
    rel = np.abs(ora.round_bf16(x) - x) / np.abs(x)
    assert rel.max() <= U_BF16 and rel.max() > 0.99 * U_BF16
    assert GATE_MAX == 2e-2 and GATE_MEAN == 2e-3
