"""GPU tests of dynamic block-sparse plans: attn_plan_set_bitmap rebuilds the
work lists on the device.

* The rebuilt lists equal, entry for entry, the lists the host compiler
  builds for the same bitmap (and the host compiler's lists are checked
  against the oracle's dense mask in test_host.py).
* After an update, the forward and backward agree with the fp64 oracle for
  the new mask (the gate of gpu_util; the backward runs on the oracle's bf16
  O and LSE, so that both sides form D = rowsum(dO * O) from the same O), and
  O, LSE and dQ equal bit for bit what the ordinary plan for that bitmap
  gives (same lists, same per-item arithmetic; dK/dV may differ in rounding
  where the ordinary plan splits an item).
* Several updates in a row, an all-zero bitmap, and byte values other than
  0/1 (any nonzero byte turns a block on).
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as ora

from gpu_util import gate, to_dev, to_f64, f64
from plan_util import lists_by_item

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import long_context_masked_amd as lcm  # noqa: E402


def _cases():
    out = []
    S = 700
    o = syn.uniform_block_bitmap(S, 64, 1, seed=0)[0]
    out.append(("uniform64_causal_gqa", syn.spec_causal(S), o, o, 8, 2, 128, 2))
    S = 1000
    qo = syn.variable_partition(S, 20, 150, seed=2)
    ko = syn.variable_partition(S, 40, 200, seed=3)
    out.append(("distinct_qk_partitions", syn.spec_full(S), qo, ko, 4, 2, 64, 1))
    S = 512
    o = syn.uniform_block_bitmap(S, 128, 1, seed=0)[0]
    out.append(("per_query_head_gqa", syn.spec_causal(S), o, o, 8, 2, 64, 8))
    S = 333
    o = syn.uniform_block_bitmap(S, 32, 1, seed=0)[0]
    out.append(("mha_ragged", syn.spec_full(S), o, o, 2, 2, 128, 2))
    S = 900
    o = syn.variable_partition(S, 30, 130, seed=9)
    docs = syn.sample_doc_lens(S, 64, 400, 4)
    out.append(("causal_document_base", syn.spec_document(docs, True), o, o, 4, 1, 64, 1))
    # items dealt to the 8 XCDs by KV head, and not dealt at all
    S = 700
    o = syn.uniform_block_bitmap(S, 64, 1, seed=0)[0]
    out.append(("mha8_by_head_deal", syn.spec_causal(S), o, o, 8, 8, 64, 8))
    out.append(("gqa6_3_no_deal", syn.spec_full(S), o, o, 6, 3, 128, 3))
    # two KV heads per XCD share: the share runs one head's items after the other
    out.append(("mha16_head_major_shares", syn.spec_causal(S), o, o, 16, 16, 64, 16))
    return out


CASES = _cases()


def _bits(qo, ko, heads, density, seed, diag_on=True):
    return syn.partition_bitmap(qo, ko, heads, density, seed, diag_on)


def _dev_bits(bits, scale=1):
    return torch.from_numpy(np.ascontiguousarray(bits * scale, dtype=np.uint8)).cuda()


def _rows_sorted(a):
    a = np.asarray(a)
    return a[np.lexsort(a.T[::-1])]


def _check_items(dl, fresh_layout, Hkv):
    """Device-rebuilt items against those of a dynamic plan created with the
    new bitmap: identical, order included, when the host deals items to
    XCDs by head (Hkv a multiple of 8) or not at all (8 % Hkv != 0); the
    same set otherwise (the deal is by load and stays the creation-time one)."""
    for key in ("fwd_items", "bwd_items"):
        a, b = dl[key], fresh_layout[key]
        if Hkv % 8 == 0 or 8 % Hkv != 0:
            assert np.array_equal(a, b), f"{key}: order differs from the host compiler's"
        else:
            assert np.array_equal(_rows_sorted(a), _rows_sorted(b)), f"{key} differ"


def _check_lists_equal(dyn, spec_new, B, Hq, Hkv, d, bits_new):
    # the ordinary plan for the new bitmap, with the dynamic plan's dK/dV item
    # width (chosen from its creation bitmap)
    ref = lcm.Plan(B, spec_new["S"], Hq, Hkv, d, dict(spec_new, bwd_key_tile=dyn.stats["bwd_tile_cols"]))
    rl = ref.layout()
    fs, bs = lists_by_item(rl)
    dl = dyn.device_layout()
    fd, bd = lists_by_item(dl)
    assert fd == fs, "forward / dQ lists differ from the host compiler's"
    assert bd == bs, "dK/dV lists differ from the host compiler's"
    assert ("kwords" in dl) == ("kwords" in rl)
    if "kwords" in dl:  # bitmap words rebuilt on the device, against the host's
        assert np.array_equal(dl["kwords"], rl["kwords"]) and np.array_equal(dl["rwords"], rl["rwords"])
    fresh = lcm.Plan(B, spec_new["S"], Hq, Hkv, d,
                     dict(spec_new, dynamic=True, bwd_key_tile=dyn.stats["bwd_tile_cols"]))
    _check_items(dl, fresh.layout(), Hkv)
    return ref


def _check_bits_section(dyn, bits_new):
    lay = L_layout(dyn)
    raw = dyn._dev[dyn._dev_off:dyn._dev_off + lay.blob_bytes].cpu().numpy()
    got = raw[lay.off_bits:lay.off_bits + bits_new.size]
    assert (got == (bits_new.ravel() != 0)).all()


def L_layout(plan):
    import ctypes as C
    from long_context_masked_amd import _lib as L
    lay = L.Layout()
    L.check(L.lib().attn_plan_get_layout(plan.handle, C.byref(lay)))
    return lay


def _oracle_check(plan, spec, B, Hq, Hkv, d, seed, x=None):
    """Forward, then the backward chained on the forward's own O and LSE (the
    product path), against the oracle's O, LSE and gradients."""
    S = spec["S"]
    x = syn.attention_inputs(B, S, Hq, Hkv, d, seed) if x is None else x
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    qf, kf, vf, dof = (f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = ora.backward(qf, kf, vf, dof, spec, magnitudes=True)
    o, lse = lcm.fwd(plan, q, k, v)
    dq, dk, dv = lcm.bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    gate("O", to_f64(o), ref["o"], ref["m_o"])
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref["lse"])
    assert (np.isneginf(lg) == ~fin).all()
    if fin.any():
        assert np.abs(lg[fin] - ref["lse"][fin]).max() <= 5e-3
    gate("dQ", to_f64(dq), ref["dq"], ref["m_dq"])
    gate("dK", to_f64(dk), ref["dk"], ref["m_dk"])
    gate("dV", to_f64(dv), ref["dv"], ref["m_dv"])
    return (q, k, v, do), (o, lse, dq, dk, dv)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_set_bitmap_rebuilds_host_lists_and_matches_oracle(case):
    label, base, qo, ko, Hq, Hkv, d, heads = case
    B = 1
    print(f"dynamic case {label}", flush=True)
    b1 = _bits(qo, ko, heads, 0.5, seed=1)
    b2 = _bits(qo, ko, heads, 0.3, seed=2)
    dyn = lcm.Plan(B, base["S"], Hq, Hkv, d, dict(syn.with_bitmap(base, qo, ko, b1), dynamic=True))
    dyn.bind()
    spec2 = syn.with_bitmap(base, qo, ko, b2)
    dyn.set_bitmap(_dev_bits(b2, scale=5))          # any nonzero byte is "on"
    static2 = _check_lists_equal(dyn, spec2, B, Hq, Hkv, d, b2)
    _check_bits_section(dyn, b2)
    (q, k, v, do), (o, lse, dq, dk, dv) = _oracle_check(dyn, spec2, B, Hq, Hkv, d, seed=3)
    # same lists and per-item arithmetic as the ordinary plan for b2 (whose
    # dK/dV items may be split, so dK/dV may differ in the last bits)
    o2, lse2 = lcm.fwd(static2, q, k, v)
    dq2, _, _ = lcm.bwd(static2, q, k, v, o2, lse2, do)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(dq, dq2)


@pytest.mark.parametrize("case", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_repeated_updates(case):
    """b1 -> b2 -> b3 (no diagonal: rows and columns without keys) -> b1."""
    label, base, qo, ko, Hq, Hkv, d, heads = case
    B = 2
    b1 = _bits(qo, ko, heads, 0.5, seed=11)
    b2 = _bits(qo, ko, heads, 0.8, seed=12)
    b3 = _bits(qo, ko, heads, 0.2, seed=13, diag_on=False)
    dyn = lcm.Plan(B, base["S"], Hq, Hkv, d, dict(syn.with_bitmap(base, qo, ko, b1), dynamic=True))
    dyn.bind()
    x = syn.attention_inputs(B, base["S"], Hq, Hkv, d, 21)
    for step, b in enumerate((b2, b3, b1)):
        print(f"dynamic case {label} update {step}", flush=True)
        spec = syn.with_bitmap(base, qo, ko, b)
        dyn.set_bitmap(_dev_bits(b))
        _check_lists_equal(dyn, spec, B, Hq, Hkv, d, b)
        _oracle_check(dyn, spec, B, Hq, Hkv, d, seed=0, x=x)


def test_all_zero_bitmap_then_back():
    """Every list empty: O = 0, LSE = -inf, zero gradients; then a bitmap
    with blocks on again."""
    label, base, qo, ko, Hq, Hkv, d, heads = CASES[0]
    S, B = base["S"], 1
    b1 = _bits(qo, ko, heads, 0.5, seed=31)
    dyn = lcm.Plan(B, S, Hq, Hkv, d, dict(syn.with_bitmap(base, qo, ko, b1), dynamic=True))
    dyn.bind()
    dyn.set_bitmap(torch.zeros(b1.shape, dtype=torch.bool, device="cuda"))
    dl = dyn.device_layout()
    assert (dl["fwd_items"][:, 3] == 0).all() and (dl["bwd_items"][:, 3] == 0).all()
    x = syn.attention_inputs(B, S, Hq, Hkv, d, 32)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    o, lse = lcm.fwd(dyn, q, k, v)
    dq, dk, dv = lcm.bwd(dyn, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert (o == 0).all() and torch.isneginf(lse).all()
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()
    dyn.set_bitmap(_dev_bits(b1))
    _check_lists_equal(dyn, syn.with_bitmap(base, qo, ko, b1), B, Hq, Hkv, d, b1)
    _oracle_check(dyn, syn.with_bitmap(base, qo, ko, b1), B, Hq, Hkv, d, seed=33, x=x)


def test_set_bitmap_argument_errors():
    label, base, qo, ko, Hq, Hkv, d, heads = CASES[0]
    b1 = _bits(qo, ko, heads, 0.5, seed=41)
    dyn = lcm.Plan(1, base["S"], Hq, Hkv, d, dict(syn.with_bitmap(base, qo, ko, b1), dynamic=True))
    dyn.bind()
    with pytest.raises(ValueError):
        dyn.set_bitmap(torch.zeros((heads + 1,) + b1.shape[1:], dtype=torch.uint8, device="cuda"))
    import ctypes as C
    from long_context_masked_amd import _lib as L
    t = torch.zeros(b1.size + 16, dtype=torch.uint8, device="cuda")
    assert L.lib().attn_plan_set_bitmap(dyn.handle, C.c_void_p(t.data_ptr() + 1), None) == L.ATTN_ERR_INVALID
    inside = dyn._dev.data_ptr() + dyn._dev_off   # the plan's own buffer
    assert L.lib().attn_plan_set_bitmap(dyn.handle, C.c_void_p(inside), None) == L.ATTN_ERR_INVALID
    assert b"overlaps" in L.lib().attn_last_error()


def test_autograd_refuses_a_bitmap_replaced_after_the_forward():
    """attention() on a dynamic plan: the backward raises if set_bitmap ran
    after the forward, and runs when the bitmap is the forward's."""
    label, base, qo, ko, Hq, Hkv, d, heads = CASES[0]
    b1 = _bits(qo, ko, heads, 0.5, seed=51)
    b2 = _bits(qo, ko, heads, 0.5, seed=52)
    dyn = lcm.Plan(1, base["S"], Hq, Hkv, d, dict(syn.with_bitmap(base, qo, ko, b1), dynamic=True))
    x = syn.attention_inputs(1, base["S"], Hq, Hkv, d, 53)
    q, k, v, do = (to_dev(x[n], torch).requires_grad_(n != "do") for n in ("q", "k", "v", "do"))
    o = lcm.attention(q, k, v, dyn)
    o.backward(do)
    torch.cuda.synchronize()
    o = lcm.attention(q, k, v, dyn)
    dyn.set_bitmap(_dev_bits(b2))
    with pytest.raises(RuntimeError, match="set_bitmap"):
        o.backward(do)


@pytest.mark.parametrize("blk,heads", [(64, 8), (128, 64)], ids=["block64_per_kv_head", "block128_per_query_head"])
def test_fullsize_sparse_32k_gqa(blk, heads):
    """The sparse workload's shape (S = 32K, GQA 64:8, d = 128): after an
    update the device lists equal the host compiler's for the new bitmap, O,
    LSE and dQ equal the ordinary plan's bit for bit, and dK/dV (the ordinary
    plan splits long items, with another summation order) agree to one bf16
    rounding."""
    from plan_util import concat_lists
    S, Hq, Hkv, d = 32768, 64, 8, 128
    print(f"dynamic full size S={S} block {blk} bitmap heads {heads}", flush=True)
    offs, b1 = syn.uniform_block_bitmap(S, blk, heads, 0.5, seed=1)
    _, b2 = syn.uniform_block_bitmap(S, blk, heads, 0.5, seed=2)
    base = syn.spec_full(S)
    dyn = lcm.Plan(1, S, Hq, Hkv, d, dict(syn.with_bitmap(base, offs, offs, b1), dynamic=True))
    static = lcm.Plan(1, S, Hq, Hkv, d, dict(syn.with_bitmap(base, offs, offs, b2),
                                             bwd_key_tile=dyn.stats["bwd_tile_cols"]))
    dyn.bind()
    dyn.set_bitmap(_dev_bits(b2))
    dl = dyn.device_layout()
    (fk, fl, fe), (bk, bl, be) = concat_lists(dl)
    (gk, gl, ge), (ck, cl, ce) = concat_lists(static.layout())
    assert np.array_equal(fk, gk) and np.array_equal(fl, gl) and np.array_equal(fe, ge)
    assert np.array_equal(bk, ck) and np.array_equal(bl, cl) and np.array_equal(be, ce)
    fresh = lcm.Plan(1, S, Hq, Hkv, d, dict(syn.with_bitmap(base, offs, offs, b2), dynamic=True,
                                            bwd_key_tile=dyn.stats["bwd_tile_cols"]))
    _check_items(dl, fresh.layout(), Hkv)   # longest first, as a fresh plan
    del fresh
    x = syn.attention_inputs(1, S, Hq, Hkv, d, 7)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    del x
    o1, l1 = lcm.fwd(dyn, q, k, v)
    o2, l2 = lcm.fwd(static, q, k, v)
    g1 = lcm.bwd(dyn, q, k, v, o1, l1, do)
    g2 = lcm.bwd(static, q, k, v, o1, l1, do)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(g1[0], g2[0])
    for a, b in zip(g1[1:], g2[1:]):
        a, b = a.float(), b.float()
        rms = float(b.pow(2).mean().sqrt())
        assert bool(((a - b).abs() <= 2.0 ** -7 * torch.maximum(a.abs(), b.abs()) + 1e-4 * rms).all())


def test_share_above_sort_cap_keeps_natural_order():
    """No XCD deal (Hkv = 12) and more than 8192 items in the one share: the
    items stay in natural order (query-head group, Q-tile) / (KV head,
    K-tile), with their new lengths; lists as the host compiler's."""
    S, Hq, Hkv, d = 90112, 12, 12, 64
    offs, b1 = syn.uniform_block_bitmap(S, 128, 1, 0.5, seed=51)
    _, b2 = syn.uniform_block_bitmap(S, 128, 1, 0.3, seed=52)
    base = syn.spec_causal(S)
    dyn = lcm.Plan(1, S, Hq, Hkv, d, dict(syn.with_bitmap(base, offs, offs, b1), dynamic=True))
    assert dyn.stats["fwd_items"] > 8192 and dyn.stats["bwd_items"] > 8192
    dyn.bind()
    dyn.set_bitmap(_dev_bits(b2))
    from plan_util import concat_lists
    dl = dyn.device_layout()
    fresh = lcm.Plan(1, S, Hq, Hkv, d, dict(syn.with_bitmap(base, offs, offs, b2), dynamic=True,
                                            bwd_key_tile=dyn.stats["bwd_tile_cols"]))
    fl = fresh.layout()
    for (a, b) in zip(concat_lists(dl), concat_lists(fl)):
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
    nFQ, nBK = (S + 127) // 128, (S + 127) // 128
    fi, bi = dl["fwd_items"], dl["bwd_items"]
    assert np.array_equal(fi[:, 1] * nFQ + fi[:, 0], np.arange(len(fi)))   # HG = 1 (no GQA)
    assert np.array_equal(bi[:, 1] * nBK + bi[:, 0], np.arange(len(bi)))
    assert np.array_equal(_rows_sorted(fi), _rows_sorted(fl["fwd_items"]))
    assert np.array_equal(_rows_sorted(bi), _rows_sorted(fl["bwd_items"]))


def test_random_shapes_and_partitions_lists_bit_exact():
    """Seeded random configurations: ragged S, every head grouping (bitmap
    heads 1, Hkv or Hq; odd groups), distinct random row and column block
    partitions (tiny blocks included), densities from 0 to 1, several base
    masks.  After each update the device-built lists and items equal the
    host compiler's (items in full when the host's XCD deal does not depend
    on costs, as a set otherwise)."""
    rng = np.random.default_rng(2024)
    groupings = [(4, 2), (8, 2), (3, 1), (6, 3), (8, 8), (2, 2), (12, 4)]
    for trial in range(24):
        S = int(rng.integers(65, 1500))
        Hq, Hkv = groupings[trial % len(groupings)]
        G = Hq // Hkv
        heads = [1, Hkv, Hq][int(rng.integers(0, 3))]
        lo = int(rng.choice([1, 8, 32, 64]))
        qo = syn.variable_partition(S, lo, lo + int(rng.integers(0, 200)), seed=int(rng.integers(1 << 30)))
        ko = syn.variable_partition(S, lo, lo + int(rng.integers(0, 200)), seed=int(rng.integers(1 << 30)))
        base = [syn.spec_full(S), syn.spec_causal(S), syn.spec_sliding(S, int(rng.integers(16, 400)), True),
                syn.spec_document(syn.sample_doc_lens(S, 16, 300, int(rng.integers(100))), True)][trial % 4]
        d = 64 if trial % 2 else 128
        dens = [0.0, 0.1, 0.5, 0.9, 1.0][trial % 5]
        b1 = _bits(qo, ko, heads, 0.5, seed=int(rng.integers(1 << 30)), diag_on=False)
        b2 = _bits(qo, ko, heads, dens, seed=int(rng.integers(1 << 30)), diag_on=False)
        print(f"trial {trial}: S={S} Hq={Hq} Hkv={Hkv} heads={heads} d={d} blocks {len(qo) - 1}x{len(ko) - 1} "
              f"density {dens}", flush=True)
        dyn = lcm.Plan(1, S, Hq, Hkv, d, dict(syn.with_bitmap(base, qo, ko, b1), dynamic=True))
        dyn.bind()
        dyn.set_bitmap(_dev_bits(b2))
        _check_lists_equal(dyn, syn.with_bitmap(base, qo, ko, b2), 1, Hq, Hkv, d, b2)
        _check_bits_section(dyn, b2)
