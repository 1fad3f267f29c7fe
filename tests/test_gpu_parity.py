"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every element of O, LSE, dQ, dK and dV; they span
several tiles, ragged tails, both head dims, GQA and MHA, and every mask
family.  The gate is described in gpu_util (max-abs 2e-2 and mean-abs 2e-3
of the oracle tensor's RMS, with the rounding room bf16 itself forces,
derived and pinned in tests/test_gate.py); LSE must agree
to 5e-3 absolute and be -inf exactly on rows with no allowed key.
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as ora
from oracle import masks as om

from gpu_util import assert_within_one_ulp, gate, to_dev, to_f64, f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import long_context_masked_amd as lcm  # noqa: E402
from long_context_masked_amd import _lib as L  # noqa: E402


def run_case(spec, B, Hq, Hkv, d, seed=0, check_bwd=True, x=None):
    """Forward, then the backward chained on the forward's own O and LSE,
    against the oracle."""
    S = spec["S"]
    if x is None:
        x = syn.attention_inputs(B, S, Hq, Hkv, d, seed)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    plan = lcm.Plan(B, S, Hq, Hkv, d, spec)
    o, lse = lcm.fwd(plan, q, k, v)
    qf, kf, vf, dof = (f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = ora.backward(qf, kf, vf, dof, spec, magnitudes=True)
    if check_bwd:
        dq, dk, dv = lcm.bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    gate("O", to_f64(o), ref["o"], ref["m_o"])
    lg = lse.cpu().numpy().astype(np.float64)
    lr = ref["lse"]
    fin = np.isfinite(lr)
    assert (np.isneginf(lg) == ~fin).all()
    assert np.abs(lg[fin] - lr[fin]).max() <= 5e-3
    if check_bwd:
        gate("dQ", to_f64(dq), ref["dq"], ref["m_dq"])
        gate("dK", to_f64(dk), ref["dk"], ref["m_dk"])
        gate("dV", to_f64(dv), ref["dv"], ref["m_dv"])


TINY = syn.config_mask_specs("tiny", Hkv=2)


@pytest.mark.parametrize("label,spec", TINY, ids=[l for l, _ in TINY])
def test_tiny_config_every_family(label, spec):
    """B=1, S=512, Hq=4, Hkv=2, d=64, every mask family, fwd + bwd."""
    run_case(spec, 1, 4, 2, 64)


@pytest.mark.parametrize("label", ["causal", "causal_document", "varblock_50"])
def test_batch_of_two(label):
    spec = dict(TINY)[label]
    run_case(spec, 2, 4, 2, 64, seed=1)


def _ragged_specs(S, Hkv):
    docs = syn.sample_doc_lens(S, 16, 400, 3)
    q = 100
    offs, bits = syn.variable_block_bitmap(S, 32, 224, Hkv, 0.5, seed=2)
    uoffs, ubits = syn.uniform_block_bitmap(S, 64, Hkv, 0.5, seed=4)
    return [
        ("full", syn.spec_full(S)), ("causal", syn.spec_causal(S)),
        ("causal_sw", syn.spec_sliding(S, 130, True)), ("full_sw", syn.spec_sliding(S, 70, False)),
        ("causal_document", syn.spec_document(docs, True)),
        ("full_document", syn.spec_document(docs, False)),
        ("prefix_lm_causal", syn.spec_prefix_lm_causal(S, 150)),
        ("shared_question", syn.spec_shared_question(q, syn.sample_answers(S - q, 4, 1))),
        ("global_sliding", syn.spec_global_sliding(S, 16, 100)),
        ("causal_blockwise", syn.spec_causal_blockwise(S, 256)),
        ("block64", syn.with_bitmap(syn.spec_full(S), uoffs, uoffs, ubits)),
        ("varblock", syn.with_bitmap(syn.spec_full(S), offs, offs, bits)),
        # rows with no key inside listed tiles (each task's context rows)
        ("task_batch", syn.spec_task_batch(*syn.sample_tasks(S, 37, 5, kv_max=150))),
    ]


RAGGED_GQA = _ragged_specs(700, 1)


@pytest.mark.parametrize("label,spec", RAGGED_GQA, ids=[l for l, _ in RAGGED_GQA])
def test_d128_gqa_ragged(label, spec):
    """d=128, Hq=8 over one KV head (two query heads per workgroup), S=700."""
    run_case(spec, 1, 8, 1, 128, seed=5)


RAGGED_MHA = _ragged_specs(333, 2)


@pytest.mark.parametrize("label,spec", RAGGED_MHA, ids=[l for l, _ in RAGGED_MHA])
def test_d128_mha_ragged(label, spec):
    """d=128, MHA 2:2 (one head of 128 rows per workgroup), S=333."""
    run_case(spec, 1, 2, 2, 128, seed=6)


@pytest.mark.parametrize("S,Hq,Hkv,d,kind", [(512, 4, 2, 64, "uniform64"), (700, 8, 2, 128, "variable"),
                                               (333, 6, 2, 128, "uniform64")])
def test_per_query_head_bitmaps_under_gqa(S, Hq, Hkv, d, kind):
    """One bitmap per query head with query heads sharing KV heads: the work
    lists are unions over the heads of an item, masking is per head."""
    if kind == "uniform64":
        offs, bits = syn.uniform_block_bitmap(S, 64, Hq, 0.5, seed=11)
    else:
        offs, bits = syn.variable_block_bitmap(S, 32, 224, Hq, 0.5, seed=12)
    run_case(syn.with_bitmap(syn.spec_causal(S), offs, offs, bits), 1, Hq, Hkv, d, seed=13)


def test_d64_mha_odd_group_and_short():
    """Hq=3 over Hkv=1 (odd group), S=65 and S=1."""
    run_case(syn.spec_causal(65), 1, 3, 1, 64, seed=7)
    run_case(syn.spec_full(1), 1, 3, 1, 64, seed=8)


def test_empty_rows_and_keys():
    """A bitmap that leaves whole block rows and columns empty: O = 0,
    LSE = -inf, zero gradients there."""
    S = 256
    offs = [0, 64, 128, 192, 256]
    bits = np.array([[[1, 0, 1, 0], [0, 0, 0, 0], [1, 0, 1, 0], [0, 0, 0, 1]]], dtype=np.uint8)
    spec = syn.with_bitmap(syn.spec_full(S), offs, offs, bits)
    run_case(spec, 1, 2, 1, 64, seed=9)


def _bf16_bits(a):
    return syn.bf16_bits_from_f32(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("label,spec,Hq,Hkv,d", [
    ("full_gqa", syn.spec_full(700), 8, 1, 128), ("causal_gqa", syn.spec_causal(700), 8, 1, 128),
    ("full_mha", syn.spec_full(333), 2, 2, 128), ("causal_d64", syn.spec_causal(512), 4, 2, 64)])
def test_forward_rescales_when_later_keys_score_far_higher(label, spec, Hq, Hkv, d):
    """Rows whose later keys score tens to hundreds of log2 units above
    everything in the first key tile they read, so that the forward's running
    maximum moves past its slack and O and the row sum are rescaled (N(0, 1)
    inputs never get there).  Two constructions: keys late in the sequence
    along the sign pattern of one query row, and a first key tile that scores
    far below the rest for every row.  O and LSE are checked; the backward
    does not use the running maximum."""
    S = spec["S"]
    x = syn.attention_inputs(1, S, Hq, Hkv, d, seed=21)
    q, k = f64(x["q"]), f64(x["k"])
    for j, r in ((S - 5, 3), (S // 2 + 7, S - 1)):
        k[0, j] = 4.0 * np.sign(q[0, r, 0] + 1e-3)
    x["k"] = _bf16_bits(k)
    run_case(spec, 1, Hq, Hkv, d, x=x, check_bwd=False)
    rng = np.random.default_rng(22)
    u = np.sign(rng.standard_normal(d)) * 2.0
    q2 = u + 0.25 * rng.standard_normal((1, S, Hq, d))
    k2 = f64(x["k"]).copy()
    k2[0, :64] = -4.0 * np.sign(u) + 0.5 * rng.standard_normal((64, Hkv, d))
    x2 = dict(x, q=_bf16_bits(q2), k=_bf16_bits(k2))
    run_case(spec, 1, Hq, Hkv, d, x=x2, check_bwd=False)


def test_forward_is_deterministic():
    S = 1024
    spec = syn.spec_causal(S)
    x = syn.attention_inputs(1, S, 8, 2, 128, 0, with_do=False)
    q, k, v = (to_dev(x[n], torch) for n in ("q", "k", "v"))
    plan = lcm.Plan(1, S, 8, 2, 128, spec)
    o1, l1 = lcm.fwd(plan, q, k, v)
    o2, l2 = lcm.fwd(plan, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_backward_is_deterministic_with_split_items():
    """The partial dK/dV of split items are summed in a fixed order and dQ
    has its own pass, so two backward passes give identical bits (S = 1K
    splits every dK/dV item); with dQ accumulated by atomics, dK and dV keep
    identical bits and dQ stays within one bf16 ulp, run to run."""
    S = 1024
    spec = syn.spec_causal(S)
    plan = lcm.Plan(1, S, 8, 2, 128, spec)
    assert plan.layout()["n_slots"] > 0
    x = syn.attention_inputs(1, S, 8, 2, 128, 0)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    o, lse = lcm.fwd(plan, q, k, v)
    g1 = lcm.bwd(plan, q, k, v, o, lse, do)
    g2 = lcm.bwd(plan, q, k, v, o, lse, do)
    a1 = lcm.bwd(plan, q, k, v, o, lse, do, atomic_dq=True)
    a2 = lcm.bwd(plan, q, k, v, o, lse, do, atomic_dq=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    for a, b, c in zip(a1[1:], a2[1:], g1[1:]):
        assert torch.equal(a, b) and torch.equal(a, c)
    assert_within_one_ulp("dQ", a1[0], a2[0])


def test_atomic_and_separate_dq_paths_both_match_the_oracle():
    """attn_bwd (separate dQ pass) and attn_bwd_atomic_dq (dQ accumulated in
    the dK/dV pass) against the oracle on masks with partial tiles, GQA and
    MHA, both head dims, ragged S, rows without keys and one bitmap per query
    head."""
    po, pb = syn.uniform_block_bitmap(333, 64, 6, 0.5, seed=14)
    cases = [(syn.spec_causal(333), 1, 6, 2, 128), (RAGGED_GQA[12][1], 1, 8, 1, 128),
             (dict(TINY)["varblock_50"], 2, 4, 2, 64),
             # one bitmap per query head: (Q-tile, head) dK/dV stages
             (syn.with_bitmap(syn.spec_causal(333), po, po, pb), 1, 6, 2, 128)]
    for spec, B, Hq, Hkv, d in cases:
        spec = dict(spec, bwd_key_tile=128)  # the fused dQ pass runs on 128-key items
        S = spec["S"]
        print(f"atomic vs separate dQ: {spec['family']} S={S} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
        x = syn.attention_inputs(B, S, Hq, Hkv, d, 9)
        q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
        plan = lcm.Plan(B, S, Hq, Hkv, d, spec)
        o, lse = lcm.fwd(plan, q, k, v)
        gs = lcm.bwd(plan, q, k, v, o, lse, do)
        ga = lcm.bwd(plan, q, k, v, o, lse, do, atomic_dq=True)
        torch.cuda.synchronize()
        ref = ora.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), spec, magnitudes=True)
        for g in (gs, ga):
            gate("dQ", to_f64(g[0]), ref["dq"], ref["m_dq"])
            gate("dK", to_f64(g[1]), ref["dk"], ref["m_dk"])
            gate("dV", to_f64(g[2]), ref["dv"], ref["m_dv"])


def _narrow_cases():
    S1, S2, S3 = 1000, 1500, 900
    uo, ub = syn.uniform_block_bitmap(S2, 64, 2, 0.5, seed=31)
    vo, vb = syn.variable_block_bitmap(S3, 32, 224, 2, 0.5, seed=32)
    po, pb = syn.uniform_block_bitmap(700, 64, 8, 0.5, seed=33)
    return [
        ("causal_ragged_d64", dict(syn.spec_causal(S1), bwd_key_tile=64), 1, 4, 2, 64),
        ("block64_gqa_auto", syn.with_bitmap(syn.spec_full(S2), uo, uo, ub), 1, 8, 2, 128),
        ("varblock_mha", dict(syn.with_bitmap(syn.spec_causal(S3), vo, vo, vb), bwd_key_tile=64), 1, 2, 2, 128),
        ("per_query_head_gqa", dict(syn.with_bitmap(syn.spec_causal(700), po, po, pb), bwd_key_tile=64),
         1, 8, 2, 128),
        ("global_sliding_split", dict(syn.spec_global_sliding(2048, 64, 256), bwd_key_tile=64), 1, 16, 2, 128),
        ("document_batch2", dict(syn.spec_document(syn.sample_doc_lens(640, 8, 200, 5), True), bwd_key_tile=64),
         2, 4, 2, 64),
    ]


@pytest.mark.parametrize("label,spec,B,Hq,Hkv,d", _narrow_cases(), ids=[c[0] for c in _narrow_cases()])
def test_narrow_dkdv_items(label, spec, B, Hq, Hkv, d):
    """64-key dK/dV items (two waves, two stage buffers): ragged S, both head
    dims, GQA and MHA, bitmaps per KV head and per query head, split items
    and a batch of two, against the oracle."""
    p = lcm.Plan(B, spec["S"], Hq, Hkv, d, spec)
    assert p.stats["bwd_tile_cols"] == 64
    if label == "global_sliding_split":
        assert p.layout()["n_slots"] > 0
    run_case(spec, B, Hq, Hkv, d, seed=34)


@pytest.mark.parametrize("label,spec", [
    ("full", syn.spec_full(8192)), ("causal_sw1024", syn.spec_sliding(8192, 1024, True))])
def test_narrow_and_wide_dkdv_items_agree(label, spec):
    """Without split items, a key's dK and dV sum the same products in the
    same order whether its item spans 64 or 128 keys (a listed tile that a
    64-key item skips adds exact zeros to the 128-key item's sums), so the
    two plans give equal dK and dV; dQ has its own pass and equal bits."""
    S, Hq, Hkv, d = spec["S"], 16, 8, 128
    x = syn.attention_inputs(1, S, Hq, Hkv, d, 35)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    wide = lcm.Plan(1, S, Hq, Hkv, d, dict(spec, bwd_key_tile=128))
    narrow = lcm.Plan(1, S, Hq, Hkv, d, dict(spec, bwd_key_tile=64))
    assert wide.layout()["n_slots"] == 0 and narrow.layout()["n_slots"] == 0
    o, lse = lcm.fwd(wide, q, k, v)
    gw = lcm.bwd(wide, q, k, v, o, lse, do)
    gn = lcm.bwd(narrow, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), gw, gn):
        assert torch.equal(a, b), name
    with pytest.raises(lcm.AttnError) as ei:
        lcm.bwd(narrow, q, k, v, o, lse, do, atomic_dq=True)
    assert ei.value.status == L.ATTN_ERR_UNSUPPORTED


def test_forced_device_error_leaves_outputs_untouched(monkeypatch):
    S = 128
    plan = lcm.Plan(1, S, 2, 1, 64, syn.spec_causal(S))
    x = syn.attention_inputs(1, S, 2, 1, 64, 0, with_do=False)
    q, k, v = (to_dev(x[n], torch) for n in ("q", "k", "v"))
    plan.bind(q.device)
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, S), 3.0, device=q.device)
    monkeypatch.setenv("ATTN_FORCE_DEVICE_ERROR", "1")
    with pytest.raises(lcm.AttnError) as ei:
        lcm.fwd(plan, q, k, v, out=o, lse=lse)
    assert ei.value.status == 4
    monkeypatch.delenv("ATTN_FORCE_DEVICE_ERROR")
    torch.cuda.synchronize()
    assert (o == 7.0).all() and (lse == 3.0).all()


def test_smoke_entry_point():
    """The package's smoke check (one causal fwd + bwd at S = 512 against the
    oracle, with the gate above) passes."""
    import __graft_entry__
    __graft_entry__.smoke()


def _random_configs(n=14, seed=2026, tag="r"):
    """Seeded random shapes, masks and plan options: S in [65, 900], KV heads
    1-16 with groups of 1-4 (16 KV heads put two heads in each XCD share),
    both head dims, batches of 1-2, every base family, bitmaps per KV head
    and per query head (uniform 32/64/128 or variable blocks, distinct row
    and column partitions), and 64-key, 128-key or chosen dK/dV items."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(rng.integers(65, 901))
        Hkv = int(rng.choice([1, 2, 4, 16]))
        G = int(rng.choice([1, 2, 3, 4])) if Hkv < 16 else int(rng.choice([1, 2]))
        Hq, d, B = Hkv * G, int(rng.choice([64, 128])), int(rng.choice([1, 1, 2]))
        fam = int(rng.integers(0, 6))
        s = int(rng.integers(0, 1 << 30))
        if fam == 0:
            base = syn.spec_full(S)
        elif fam == 1:
            base = syn.spec_causal(S)
        elif fam == 2:
            base = syn.spec_sliding(S, int(rng.integers(1, S + 1)), bool(rng.integers(0, 2)))
        elif fam == 3:
            base = syn.spec_document(syn.sample_doc_lens(S, 16, max(17, S // 2), s), bool(rng.integers(0, 2)))
        elif fam == 4:
            base = syn.spec_global_sliding(S, int(rng.integers(1, 40)), int(rng.integers(8, 200)),
                                           bool(rng.integers(0, 2)))
        else:
            base = syn.spec_causal_blockwise(S, int(rng.integers(16, 300)))
        spec = base
        bm = int(rng.integers(0, 4))  # 0: none, 1: per KV head, 2: per query head, 3: distinct partitions
        heads = {1: Hkv, 2: Hq, 3: 1}.get(bm)
        if bm in (1, 2):
            if rng.integers(0, 2):
                offs, bits = syn.uniform_block_bitmap(S, int(rng.choice([32, 64, 128])), heads, 0.5, s)
            else:
                offs, bits = syn.variable_block_bitmap(S, 16, 200, heads, 0.5, s)
            spec = syn.with_bitmap(base, offs, offs, bits)
        elif bm == 3:
            qo = syn.variable_partition(S, 20, 150, s)
            ko = syn.variable_partition(S, 30, 200, s + 1)
            spec = syn.with_bitmap(base, qo, ko, syn.partition_bitmap(qo, ko, 1, 0.5, s + 2))
        tile = int(rng.choice([0, 0, 64, 128]))
        if tile:
            spec = dict(spec, bwd_key_tile=tile)
        out.append((f"{tag}{i}_S{S}_B{B}_{Hq}x{Hkv}_d{d}_{base['family']}_bm{bm}_k{tile}", spec, B, Hq, Hkv, d))
    return out


RANDOM = _random_configs() + _random_configs(16, 4049, "q")


@pytest.mark.parametrize("label,spec,B,Hq,Hkv,d", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_configurations(label, spec, B, Hq, Hkv, d):
    """Forward and chained backward against the oracle on seeded random
    configurations (shape, mask family, bitmap layout, dK/dV item width)."""
    print(f"random configuration {label}", flush=True)
    run_case(spec, B, Hq, Hkv, d, seed=int(label[1:label.index("_")]) + 40)
