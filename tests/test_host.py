"""CPU tests of the library's host side: exports, mask compiler, scheduler,
error statuses.  No GPU work is launched here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synthetic as syn
from oracle import masks as om
from plan_util import lists_by_item

lcm = pytest.importorskip("long_context_masked_amd")
from long_context_masked_amd import _lib as L  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "attn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert "attn_fwd" in names and "attn_bwd" in names and len(names) >= 10
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, f"binding lacks {n}"
    assert b"gfx950" in lib.attn_version()


def _tiny_specs(Hkv=2):
    return syn.config_mask_specs("tiny", Hkv=Hkv)


def test_library_shares_torch_hip_runtime():
    """Loading libattn.so through the binding, with torch not yet imported,
    still leaves one HIP runtime and one HSA runtime in the process (torch's):
    two copies would each claim the GPU, and the second to start finds none."""
    import subprocess
    import sys
    code = (
        "import long_context_masked_amd._lib as L; L.lib()\n"
        "names = set(l.split()[-1] for l in open('/proc/self/maps')\n"
        "            if 'libamdhip64' in l or 'libhsa-runtime64' in l)\n"
        "print(len([n for n in names if 'amdhip64' in n]), len([n for n in names if 'hsa-runtime' in n]))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["1", "1"], r.stdout


@pytest.mark.parametrize("label,spec", _tiny_specs(), ids=[l for l, _ in _tiny_specs()])
def test_nnz_matches_oracle_popcount(label, spec):
    Hq, Hkv = 4, 2
    p = lcm.Plan(2, spec["S"], Hq, Hkv, 64, spec)
    want = sum(om.nnz(spec, om.mask_head(spec, h, Hq, Hkv)) for h in range(Hq))
    assert p.stats["nnz_per_batch"] == want
    assert p.stats["nnz_total"] == 2 * want
    assert p.stats["flops_fwd"] == 4 * 64 * 2 * want
    assert p.stats["flops_bwd"] == 10 * 64 * 2 * want


def _expand_colb(cb, S):
    i = np.arange(S)[:, None]
    m = ((i >= cb[None, :, 0]) & (i < cb[None, :, 1])) | ((i >= cb[None, :, 2]) & (i < cb[None, :, 3]))
    return ~m


def _expand_rowb(rb, S):
    j = np.arange(S)[None, :]
    return ((j >= rb[:, 0:1]) & (j < rb[:, 1:2])) | ((j >= rb[:, 2:3]) & (j < rb[:, 3:4]))


def _family_specs(S, seed):
    docs = syn.sample_doc_lens(S, 8, 300, seed)
    q = 37
    return [
        syn.spec_full(S), syn.spec_causal(S), syn.spec_sliding(S, 33, True),
        syn.spec_sliding(S, 21, False), syn.spec_document(docs, False), syn.spec_document(docs, True),
        syn.spec_prefix_lm_causal(S, 77), syn.spec_shared_question(q, syn.sample_answers(S - q, 4, seed)),
        syn.spec_global_sliding(S, 16, 50), syn.spec_global_sliding(S, 16, 50, True),
        syn.spec_causal_blockwise(S, 128), syn.spec_causal_blockwise(S, 128, "block_causal"),
        syn.spec_causal_blockwise(S, 100),
        syn.spec_prefix_lm_document(docs, [syn.sample_prefix(0, L, seed + i) for i, L in enumerate(docs)]),
        syn.spec_block_causal_document(docs, 40),
    ]


@pytest.mark.parametrize("S,seed", [(700, 0), (1024, 1), (333, 2)])
def test_encodings_match_oracle_predicate(S, seed):
    """Column bounds and row runs the compiler stores both expand to exactly
    the oracle's predicate, for every static family."""
    for spec in _family_specs(S, seed):
        p = lcm.Plan(1, S, 2, 1, 64, spec)
        lay = p.layout()
        want = om.base_pred(spec, np.arange(S)[:, None], np.arange(S)[None, :])
        assert (_expand_colb(lay["colb"], S) == want).all(), spec["family"]
        assert (_expand_rowb(lay["rowb"], S) == want).all(), spec["family"]


def _check_lists(p, spec, Hq, Hkv):
    """Every allowed pair is covered by exactly one listed tile; a tile flagged
    FULL is fully allowed; EMPTY tiles are never listed; every (tile, head)
    item appears exactly once."""
    S = spec["S"]
    G = Hq // Hkv
    lay = p.layout()
    st = p.stats
    FR, FC = st["fwd_tile_rows"], st["fwd_tile_cols"]
    BR, BC = st["bwd_tile_rows"], st["bwd_tile_cols"]
    HG = st["heads_per_item"]
    dense = {}

    def dm(h):
        hm = om.mask_head(spec, h, Hq, Hkv)
        if hm not in dense:
            dense[hm] = om.dense_mask(spec, hm)
        return dense[hm]

    seen = set()
    for qt, h0, off, n in lay["fwd_items"]:
        key = (qt, h0)
        assert key not in seen
        seen.add(key)
        ents = lay["fwd_list"][off:off + n]
        tiles = (ents & 0x7FFFFFFF).astype(int)
        assert len(set(tiles.tolist())) == len(tiles)
        r0, r1 = qt * FR, min(S, qt * FR + FR)
        # an item's list serves all its heads: a listed tile has an allowed
        # pair for some head, and a FULL tile is fully allowed for every head
        for t, e in zip(tiles, ents):
            c0, c1 = t * FC, min(S, t * FC + FC)
            blks = [dm(h)[r0:r1, c0:c1] for h in range(h0, h0 + HG)]
            assert any(b.any() for b in blks), "empty tile listed"
            if not (e >> 31):
                assert all(b.all() for b in blks) and c1 - c0 == FC, "FULL tile not fully allowed"
        for h in range(h0, h0 + HG):
            a = dm(h)[r0:r1]
            cover = np.zeros(S, dtype=bool)
            for t in tiles:
                cover[t * FC:min(S, t * FC + FC)] = True
            assert not a[:, ~cover].any(), "allowed pair outside the listed tiles"
    assert len(seen) == (Hq // HG) * ((S + FR - 1) // FR)

    # dK/dV items may be split into chunks, each a run of the item's listed
    # Q-tiles: the chunks of one (K-tile, KV head) list consecutive slices
    # that together form its list, and own consecutive partial slots, in
    # list order, that one reduce entry names.  Unsplit items have slot -1.
    groups = {}
    for (kt, kvh, off, n), slot in zip(lay["bwd_items"], lay["bwd_slot"]):
        assert n > 0
        groups.setdefault((int(kt), int(kvh)), []).append((int(off), int(n), int(slot)))
    reduce = {(int(r[0]), int(r[1])): (int(r[2]), int(r[3])) for r in lay["bwd_reduce"]}
    assert len(reduce) == len(lay["bwd_reduce"])
    slots_seen = set()
    whole = {}
    for (kt, kvh), ch in groups.items():
        ch = sorted(ch)
        assert all(c[0] + c[1] == d[0] for c, d in zip(ch, ch[1:])), "chunk slices overlap or leave gaps"
        whole[(kt, kvh)] = (ch[0][0], ch[-1][0] + ch[-1][1] - ch[0][0])
        if len(ch) == 1:
            assert ch[0][2] == -1 and (kt, kvh) not in reduce
        else:
            slot0, nch = reduce[(kt, kvh)]
            assert nch == len(ch)
            assert [c[2] for c in ch] == list(range(slot0, slot0 + nch)), "slots follow list order"
            slots_seen.update(c[2] for c in ch)
    assert slots_seen == set(range(lay["n_slots"]))
    # An entry is a Q-tile for all G heads, or (bwd_head_entries) one
    # (Q-tile, head) stage with the head in bits 24-30.
    he = bool(st["bwd_head_entries"])
    seen = set()
    for (kt, kvh), (off, n) in whole.items():
        seen.add((kt, kvh))
        ents = lay["bwd_list"][off:off + n]
        tiles = (ents & 0xFFFFFF).astype(int)
        heads = ((ents >> 24) & 0x7F).astype(int)
        if he:
            assert len(set(zip(tiles.tolist(), heads.tolist()))) == len(ents)
        else:
            assert (heads == 0).all()
        c0, c1 = kt * BC, min(S, kt * BC + BC)
        for g in range(G):
            a = dm(kvh * G + g)[:, c0:c1]
            cover = np.zeros(S, dtype=bool)
            sel = heads == g if he else np.ones(len(ents), dtype=bool)
            for t, e in zip(tiles[sel], ents[sel]):
                r0, r1 = t * BR, min(S, t * BR + BR)
                assert a[r0:r1].any() or (G > 1 and not he)
                if not (e >> 31):
                    assert a[r0:r1].all() and r1 - r0 == BR
                cover[r0:r1] = True
            assert not a[~cover].any()
    assert len(seen) == Hkv * ((S + BC - 1) // BC)


@pytest.mark.parametrize("label,spec", _tiny_specs(), ids=[l for l, _ in _tiny_specs()])
def test_work_lists_cover_mask_exactly(label, spec):
    _check_lists(lcm.Plan(1, spec["S"], 4, 2, 64, spec), spec, 4, 2)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (3, 1), (8, 2)])
def test_work_lists_ragged_and_head_groupings(Hq, Hkv):
    S = 200  # ragged against 64- and 128-wide tiles
    specs = _family_specs(S, 3)[:12]
    offs, bits = syn.variable_block_bitmap(S, 20, 90, Hkv, 0.5, seed=5)
    specs.append(syn.with_bitmap(syn.spec_causal(S), offs, offs, bits))
    # one bitmap per query head (under GQA the lists are unions over heads)
    offs, bits = syn.variable_block_bitmap(S, 20, 90, Hq, 0.5, seed=6)
    specs.append(syn.with_bitmap(syn.spec_full(S), offs, offs, bits))
    for spec in specs:
        _check_lists(lcm.Plan(1, S, Hq, Hkv, 128, spec), spec, Hq, Hkv)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (3, 1), (8, 2)])
def test_narrow_dkdv_items_cover_mask_exactly(Hq, Hkv):
    """Forced 64-key dK/dV items (bwd_key_tile = 64): the same exact-cover
    checks, over 64-key columns, for static families, ragged S and the
    bitmap head groupings."""
    S = 200
    specs = [dict(s, bwd_key_tile=64) for s in _family_specs(S, 4)[:12]]
    offs, bits = syn.variable_block_bitmap(S, 20, 90, Hkv, 0.5, seed=8)
    specs.append(dict(syn.with_bitmap(syn.spec_causal(S), offs, offs, bits), bwd_key_tile=64))
    offs, bits = syn.uniform_block_bitmap(S, 64, Hq, 0.5, seed=9)
    specs.append(dict(syn.with_bitmap(syn.spec_full(S), offs, offs, bits), bwd_key_tile=64))
    for spec in specs:
        p = lcm.Plan(1, S, Hq, Hkv, 128, spec)
        assert p.stats["bwd_tile_cols"] == 64
        _check_lists(p, spec, Hq, Hkv)


@pytest.mark.parametrize("Hq,Hkv,bm_heads", [(16, 16, 16), (16, 2, 16), (16, 2, 2)])
def test_plan_independent_of_host_threads(Hq, Hkv, bm_heads):
    """The plan compiler builds each head's lists on its own host thread and
    joins them in head order: the blob is the same on every build, and each
    head's forward entries follow the previous head's."""
    S = 1500
    offs, bits = syn.variable_block_bitmap(S, 20, 150, bm_heads, 0.5, seed=11)
    spec = syn.with_bitmap(syn.spec_causal(S), offs, offs, bits)
    blobs = []
    for _ in range(3):
        p = lcm.Plan(1, S, Hq, Hkv, 128, spec)
        lay = L.Layout()
        L.check(L.lib().attn_plan_get_layout(p.handle, C.byref(lay)))
        blobs.append(np.ctypeslib.as_array((C.c_uint8 * lay.blob_bytes).from_address(lay.blob)).copy())
        del p
    assert all(np.array_equal(blobs[0], b) for b in blobs[1:])
    p = lcm.Plan(1, S, Hq, Hkv, 128, spec)
    items = p.layout()["fwd_items"]
    first = {}
    for qt, h0, off, n in items:
        first[int(h0)] = min(first.get(int(h0), 1 << 62), int(off))
    heads = sorted(first)
    assert [first[h] for h in heads] == sorted(first[h] for h in heads)
    _check_lists(p, spec, Hq, Hkv)


@pytest.mark.parametrize("S,heads,kind", [(700, 2, "variable"), (333, 3, "distinct"), (512, 1, "uniform64"),
                                           (1000, 4, "uniform96")])
def test_bitmap_words_equal_the_bitmap(S, heads, kind):
    """The plan's bitmap words against the bitmap itself: bit c of word
    (h, qb, t) is bitmap[h][qb][kblk(64 t + c)] for keys below S, 0 beyond;
    bit r of row word (h, kb, t) is bitmap[h][qblk(64 t + r)][kb].  Plans
    whose blocks do not cut 64-wide tiles have none; dynamic plans have the
    same words for their creation bitmap."""
    if kind == "variable":
        qo = ko = syn.variable_partition(S, 20, 150, 4)
        bits = syn.partition_bitmap(qo, ko, heads, 0.5, 5)
    elif kind == "distinct":
        qo, ko = syn.variable_partition(S, 20, 90, 6), syn.variable_partition(S, 30, 120, 7)
        bits = syn.partition_bitmap(qo, ko, heads, 0.5, 8)
    else:
        qo, bits = syn.uniform_block_bitmap(S, int(kind[7:]), heads, 0.5, 9)
        ko = qo
    spec = syn.with_bitmap(syn.spec_causal(S), qo, ko, bits)
    lay = lcm.Plan(1, S, heads, heads, 64, spec).layout()
    if kind == "uniform64":
        assert "kwords" not in lay and "rwords" not in lay
        return
    kblk = np.searchsorted(np.asarray(ko), np.arange(S), side="right") - 1
    qblk = np.searchsorted(np.asarray(qo), np.arange(S), side="right") - 1
    nM = (S + 63) // 64
    pad = nM * 64 - S
    b = np.asarray(bits, dtype=bool)
    # allowed keys: [h][qb][key] -> words over 64-key tiles
    keys = np.concatenate([b[:, :, kblk], np.zeros(b.shape[:2] + (pad,), dtype=bool)], axis=2)
    rows = np.concatenate([b[:, qblk, :].transpose(0, 2, 1), np.zeros((b.shape[0], b.shape[2], pad), dtype=bool)], axis=2)

    def words(x):
        x = x.reshape(x.shape[0], x.shape[1], nM, 64).astype(np.uint64)
        return (x << np.arange(64, dtype=np.uint64)).sum(axis=3, dtype=np.uint64)

    assert np.array_equal(lay["kwords"], words(keys))
    assert np.array_equal(lay["rwords"], words(rows))
    # a dynamic plan holds the same words for its creation bitmap
    dl = lcm.Plan(1, S, heads, heads, 64, dict(spec, dynamic=True)).layout()
    assert np.array_equal(dl["kwords"], lay["kwords"]) and np.array_equal(dl["rwords"], lay["rwords"])


def _empty_half_fraction(spec, S):
    """Of the 128-key (64-row, 128-key) tiles with an allowed pair, the
    fraction whose 64-key halves are not both non-empty: brute force over
    the oracle's dense mask of mask head 0."""
    m = om.dense_mask(spec, 0)
    listed = half = 0
    for r in range(0, S, 64):
        for c in range(0, S - 127, 128):
            a0, a1 = m[r:r + 64, c:c + 64].any(), m[r:r + 64, c + 64:c + 128].any()
            listed += a0 or a1
            half += a0 != a1
    return half / listed


@pytest.mark.parametrize("label,block,density,narrow", [
    ("block64_50", 64, 0.5, True), ("block64_90", 64, 0.9, False),
    ("block128_50", 128, 0.5, False), ("block256_30", 256, 0.3, False),
])
def test_dkdv_key_tile_choice(label, block, density, narrow):
    """With bwd_key_tile = 0 the plan takes 64-key dK/dV items exactly when
    more than a quarter of the listed 128-key tiles of mask head 0 have an
    empty 64-key half (dynamic plans likewise, on their creation bitmap);
    masks without a bitmap and an explicit 128 keep 128-key items."""
    S = 2048
    offs, bits = syn.uniform_block_bitmap(S, block, 1, density, 3)
    spec = syn.with_bitmap(syn.spec_full(S), offs, offs, bits)
    frac = _empty_half_fraction(spec, S)
    assert (frac > 0.25) == narrow, frac
    assert lcm.Plan(1, S, 8, 2, 128, spec).stats["bwd_tile_cols"] == (64 if narrow else 128)
    assert lcm.Plan(1, S, 8, 2, 128, dict(spec, bwd_key_tile=128)).stats["bwd_tile_cols"] == 128
    assert lcm.Plan(1, S, 8, 2, 128, dict(spec, dynamic=True)).stats["bwd_tile_cols"] == (64 if narrow else 128)
    assert lcm.Plan(1, S, 8, 2, 128, syn.spec_causal(S)).stats["bwd_tile_cols"] == 128
    assert lcm.Plan(1, S, 8, 2, 128, dict(syn.spec_causal(S), bwd_key_tile=64)).stats["bwd_tile_cols"] == 64


def _lpt_makespan(costs, m):
    loads = np.zeros(m)
    for c in costs:
        loads[np.argmin(loads)] += c
    return loads.max()


@pytest.mark.parametrize("family", ["causal", "causal_document", "block64_50"])
def test_schedule_is_longest_first(family):
    """Workgroups are dealt to the 8 XCDs round-robin, so item b runs on XCD
    b % 8.  Each XCD's share holds the items of its KV heads (head h % 8, or
    h % Hkv when Hkv divides 8) in longest-first order.  Graham's LPT bound
    says the list-scheduling makespan on m workers is at most
    (4/3 - 1/(3m)) OPT; it is checked here against a lower bound of OPT,
    which implies it: max(total/m, largest item, p_m + p_(m+1)) with items
    sorted longest first (two of the m+1 longest items share a worker).  The
    shares are balanced to within a few percent."""
    S, Hq, Hkv = 4096, 16, 2
    G = Hq // Hkv
    if family == "causal":
        spec = syn.spec_causal(S)
    elif family == "causal_document":
        spec = syn.spec_document(syn.sample_doc_lens(S, 64, 2048, 0), True)
    else:
        offs, bits = syn.uniform_block_bitmap(S, 64, Hkv, 0.5, 0)
        spec = syn.with_bitmap(syn.spec_full(S), offs, offs, bits)
    p = lcm.Plan(1, S, Hq, Hkv, 128, spec)
    lay = p.layout()
    for kind, items, lst in (("fwd", lay["fwd_items"], lay["fwd_list"]),
                             ("bwd", lay["bwd_items"], lay["bwd_list"])):
        costs, kvh = [], []
        for i, (_, head, off, n) in enumerate(items):
            e = lst[off:off + n]
            npart = int((e >> 31).sum())
            # the plan's cost model: 1 per full tile, 1.25 per partial one
            # (dK/dV: per stage, G stages per listed tile), 0.75 per item
            if kind == "fwd":
                c = (n - npart) + 1.25 * npart + 0.75
            else:  # per stage: G stages per listed tile (a chunk is an item)
                c = G * ((n - npart) + 1.25 * npart) + 0.75
            costs.append(c)
            kvh.append(head // G if kind == "fwd" else head)
        costs, kvh = np.array(costs), np.array(kvh)
        xcd = np.arange(len(costs)) % 8
        home = kvh == xcd % Hkv
        if kind == "fwd":
            assert home.all(), "items not grouped by KV head per XCD"
        else:
            # heads split into unequal numbers of chunks run out of work at
            # different times; the interleave is exact up to that point
            cut = int(np.argmin(home)) if not home.all() else len(home)
            assert cut >= 0.9 * len(home), "items not grouped by KV head per XCD"
            costs = costs[:cut - cut % 8]
        totals = np.array([costs[x::8].sum() for x in range(8)])
        assert totals.max() <= 1.05 * totals.mean()
        for x in range(8):
            share = costs[x::8]
            assert (np.diff(share) <= 1e-9).all(), "XCD share not in non-increasing cost order"
            for m in (8, 32, 64):
                lower = max(share.sum() / m, share.max())     # <= OPT
                if len(share) > m:
                    lower = max(lower, share[m - 1] + share[m])
                assert _lpt_makespan(share, m) <= (4.0 / 3.0 - 1.0 / (3.0 * m)) * lower + 1e-9


@pytest.mark.parametrize("Hkv,dynamic", [(16, False), (64, False), (16, True)])
def test_xcd_shares_of_several_heads_run_head_by_head(Hkv, dynamic):
    """With more than 8 KV heads each XCD share (items b with b % 8 == x)
    holds the heads h % 8 == x; it runs one head's items after another, in
    ascending head order, each head's in non-increasing cost order."""
    S, G = 8192, 2  # items of about equal cost: none split, shares of equal length
    offs, bits = syn.uniform_block_bitmap(S, 128, Hkv, 0.5, 7)
    spec = syn.with_bitmap(syn.spec_full(S), offs, offs, bits)
    if dynamic:
        spec = dict(spec, dynamic=True)
    p = lcm.Plan(1, S, Hkv * G, Hkv, 128, spec)
    lay = p.layout()
    HG = p.stats["heads_per_item"]
    for kind, items, lst, per_kv in (("fwd", lay["fwd_items"], lay["fwd_list"], G),
                                      ("bwd", lay["bwd_items"], lay["bwd_list"], 1)):
        for x in range(8):
            share = items[x::8]
            kvh = share[:, 1] // per_kv
            assert (kvh % 8 == x).all(), kind
            assert (np.diff(kvh) >= 0).all(), f"{kind}: share {x} not head by head"
            for h in np.unique(kvh):
                run = share[kvh == h]
                cost = []
                for _, _, off, n in run:
                    e = lst[off:off + n]
                    npart = int((e >> 31).sum())
                    stages = G if kind == "bwd" else 1
                    cost.append(stages * ((n - npart) + 1.25 * npart))
                assert (np.diff(cost) <= 1e-9).all(), f"{kind}: head {h} not longest first"


@pytest.mark.parametrize("label,spec,S,splits", [
    ("full1K", syn.spec_full(1024), 1024, True),
    ("causal1K", syn.spec_causal(1024), 1024, True),
    ("global_sliding32K", syn.spec_global_sliding(32768, 64, 2048), 32768, True),
    ("full16K", syn.spec_full(16384), 16384, False),
    ("causal16K", syn.spec_causal(16384), 16384, False),
])
def test_dkdv_split_where_items_outlast_the_launch(label, spec, S, splits):
    """dK/dV items longer than the launch's share per resident workgroup
    (total / 256) are cut into at most 16 chunks; the rest stay whole.  At
    S = 1K the 64 items of GQA 64:8 cannot fill 256 CUs, and under global
    sliding the global key columns are seen by every row; uniform masks at
    16K have 1024 items of equal cost."""
    p = lcm.Plan(1, S, 64, 8, 128, spec)
    lay = p.layout()
    assert (lay["n_slots"] > 0) == splits
    red = lay["bwd_reduce"]
    assert (red[:, 3] >= 2).all() and (red[:, 3] <= 16).all()
    assert int(red[:, 3].sum()) == lay["n_slots"]
    assert p.workspace_bytes() >= lay["n_slots"] * 2 * 128 * 128 * 4
    if splits:  # chunks bring the longest workgroup near the launch's share
        cost = lay["bwd_items"][:, 3].astype(float)  # listed Q-tiles per item
        assert cost.max() <= max(2.0 * cost.sum() / 256, 1.0)


def _status(fn):
    try:
        fn()
    except L.AttnError as e:
        return e.status
    return L.ATTN_OK


def _create(shape, desc):
    sh = L.Shape(*shape)
    h = C.c_void_p()
    st = L.lib().attn_plan_create(C.byref(sh), C.byref(desc), C.byref(h))
    if st == L.ATTN_OK:
        L.lib().attn_plan_destroy(h)
    return st


def test_plan_create_errors():
    S = 256
    ok = lcm.MaskDescriptor(syn.spec_causal(S)).c
    assert _create((1, S, 4, 2, 64, 0.0), ok) == L.ATTN_OK
    assert _create((1, S, 4, 2, 96, 0.0), ok) == L.ATTN_ERR_UNSUPPORTED
    assert _create((1, S, 4, 3, 64, 0.0), ok) == L.ATTN_ERR_INVALID
    assert _create((0, S, 4, 2, 64, 0.0), ok) == L.ATTN_ERR_INVALID
    assert _create((1, S, 4, 2, 64, float("nan")), ok) == L.ATTN_ERR_INVALID
    assert L.lib().attn_plan_create(None, None, None) == L.ATTN_ERR_INVALID
    assert b"NULL" in L.lib().attn_last_error()

    def desc(spec, **kw):
        d = lcm.MaskDescriptor(spec)
        for k, v in kw.items():
            setattr(d.c, k, v)
        return d

    d = desc(syn.spec_sliding(S, 8, True), window_left=0)
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    d = desc(syn.spec_sliding(S, 8, False), window_right=0)
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    d = desc(syn.spec_causal(S), kind=99)
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    d = lcm.MaskDescriptor(syn.spec_document([100, 100, 56], True))
    bad = np.array([0, 150, 100, 256], dtype=np.int32)
    d.c.cu_seqlens = bad.ctypes.data_as(L.P32)
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    bad2 = np.array([0, 100, 200, 255], dtype=np.int32)
    d.c.cu_seqlens = bad2.ctypes.data_as(L.P32)
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    d = lcm.MaskDescriptor(syn.spec_prefix_lm_document([100, 156], [5, 157]))
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    cb = np.zeros((S, 4), dtype=np.int32)
    cb[3, 1] = S + 1
    d = lcm.MaskDescriptor({"family": "column_bounds", "S": S, "col_bounds": cb})
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    # a checkerboard of masked columns gives rows with many allowed runs
    cb = np.zeros((S, 4), dtype=np.int32)
    cb[1::2, 1] = S
    d = lcm.MaskDescriptor({"family": "column_bounds", "S": S, "col_bounds": cb})
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_UNSUPPORTED
    offs, bits = syn.uniform_block_bitmap(S, 64, 3, 0.5, 0)
    d = lcm.MaskDescriptor(syn.with_bitmap(syn.spec_full(S), offs, offs, bits))
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    offs, bits = syn.uniform_block_bitmap(S, 64, 4, 0.5, 0)
    d = lcm.MaskDescriptor(syn.with_bitmap(syn.spec_full(S), offs, offs, bits))
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_OK   # one bitmap per query head, GQA
    assert _create((1, S, 4, 4, 64, 0.0), d.c) == L.ATTN_OK
    bad_offs = np.array([0, 64, 64, 192, 256], dtype=np.int32)
    d.c.q_blk_offsets = bad_offs.ctypes.data_as(L.P32)
    assert _create((1, S, 4, 4, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    # keys per dK/dV item: 0, 64 or 128; 64 only on static plans
    for tile, want in ((64, L.ATTN_OK), (128, L.ATTN_OK), (32, L.ATTN_ERR_INVALID), (-1, L.ATTN_ERR_INVALID)):
        assert _create((1, S, 4, 2, 64, 0.0), desc(syn.spec_causal(S), bwd_key_tile=tile).c) == want
    offs, bits = syn.uniform_block_bitmap(S, 64, 1, 0.5, 0)
    d = desc(dict(syn.with_bitmap(syn.spec_full(S), offs, offs, bits), dynamic=True), bwd_key_tile=64)
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_OK


def test_launch_entry_points_validate_before_touching_the_gpu():
    """Invalid arguments return ATTN_ERR_INVALID without any HIP call (this
    runs on a host with no GPU)."""
    S = 128
    p = lcm.Plan(1, S, 2, 1, 64, syn.spec_causal(S))
    lib = L.lib()
    P = C.c_void_p
    a = P(4096)  # never dereferenced: validation fails first
    assert lib.attn_fwd(None, a, a, a, a, a, None) == L.ATTN_ERR_INVALID
    assert lib.attn_fwd(p.handle, a, a, a, a, a, None) == L.ATTN_ERR_INVALID  # unbound plan
    assert b"not bound" in lib.attn_last_error()
    assert lib.attn_bwd(p.handle, a, a, a, a, a, a, a, a, a, a, C.c_size_t(1 << 20), None) == L.ATTN_ERR_INVALID
    assert lib.attn_plan_bind(p.handle, None, C.c_size_t(1 << 20), None) == L.ATTN_ERR_INVALID
    assert lib.attn_plan_bind(p.handle, P(4096 + 8), C.c_size_t(1 << 20), None) == L.ATTN_ERR_INVALID
    assert lib.attn_plan_bind(p.handle, P(4096), C.c_size_t(16), None) == L.ATTN_ERR_INVALID
    os.environ["ATTN_FORCE_DEVICE_ERROR"] = "1"
    try:
        assert lib.attn_plan_bind(p.handle, P(4096), C.c_size_t(1 << 20), None) == L.ATTN_ERR_DEVICE
    finally:
        del os.environ["ATTN_FORCE_DEVICE_ERROR"]
    assert lib.attn_plan_device_bytes(None) == 0
    assert lib.attn_bwd_workspace_bytes(p.handle) >= 2 * S * 4


def test_merge_validates_before_touching_the_gpu():
    """attn_merge rejects NULL, misaligned and overlapping buffers and
    unsupported sizes before any HIP call; a forced device error is reported
    as such."""
    lib = L.lib()
    P = C.c_void_p
    B, S, H, d = 1, 64, 2, 64
    ni, no, nl = B * S * H * d * 4, B * S * H * d * 2, B * S * H * 4
    o1, o2, o = 1 << 20, 2 << 20, 3 << 20          # never dereferenced
    l1, l2, lo = 4 << 20, 5 << 20, 6 << 20

    def call(a=o1, b=l1, c=o2, e=l2, f=o, g=lo, dd=d, SS=S, ob=1):
        return lib.attn_merge(P(a), P(b), P(c), P(e), P(f), ob, P(g), B, SS, H, dd, None)

    assert call(a=0) == L.ATTN_ERR_INVALID
    assert call(g=0) == L.ATTN_ERR_INVALID
    assert call(c=o2 + 8) == L.ATTN_ERR_INVALID                 # O must be 16-byte aligned
    assert call(e=l2 + 2) == L.ATTN_ERR_INVALID                 # LSE 4-byte aligned
    assert call(f=o1) == L.ATTN_ERR_INVALID                     # in place
    assert b"overlap" in lib.attn_last_error()
    assert call(f=o2 + ni - 16) == L.ATTN_ERR_INVALID           # partial overlap
    assert call(g=o + no - 4, ob=1) == L.ATTN_ERR_INVALID       # bf16 output and LSE
    assert call(g=o + 2 * no - 4, ob=0) == L.ATTN_ERR_INVALID   # fp32 output is twice as long
    assert call(g=l1 + nl - 4) == L.ATTN_ERR_INVALID
    assert call(dd=96) == L.ATTN_ERR_UNSUPPORTED
    assert call(SS=0) == L.ATTN_ERR_INVALID
    os.environ["ATTN_FORCE_DEVICE_ERROR"] = "1"
    try:
        assert call() == L.ATTN_ERR_DEVICE
    finally:
        del os.environ["ATTN_FORCE_DEVICE_ERROR"]


def test_scale_default_and_stats_fields():
    S = 300
    p = lcm.Plan(3, S, 8, 2, 128, syn.spec_sliding(S, 40, False))
    st = p.stats
    assert st["heads_per_item"] == 2 and st["fwd_tile_rows"] == 64
    assert st["bwd_tile_cols"] == 128 and st["bwd_tile_rows"] == 64
    assert st["device_bytes"] == p.device_bytes()
    assert p.workspace_bytes() >= 3 * 8 * S * 4


def _dynamic_cases():
    S = 333
    uo, ub = syn.uniform_block_bitmap(S, 64, 2, 0.5, seed=1)
    qo = syn.variable_partition(S, 20, 150, seed=2)
    ko = syn.variable_partition(S, 40, 200, seed=3)
    vb = syn.partition_bitmap(qo, ko, 1, 0.5, seed=4)
    po, pb = syn.uniform_block_bitmap(S, 32, 8, 0.4, seed=5)
    return [
        ("uniform64_gqa", syn.with_bitmap(syn.spec_causal(S), uo, uo, ub), 4, 2),
        ("distinct_qk_partitions", syn.with_bitmap(syn.spec_full(S), qo, ko, vb), 4, 2),
        ("per_query_head_gqa", syn.with_bitmap(syn.spec_causal(S), po, po, pb), 8, 2),
        ("per_query_head_odd_group", syn.with_bitmap(syn.spec_full(S), po[:], po, pb[:3]), 3, 1),
    ]


@pytest.mark.parametrize("label,spec,Hq,Hkv", _dynamic_cases(), ids=[c[0] for c in _dynamic_cases()])
def test_dynamic_plan_lists_equal_static(label, spec, Hq, Hkv):
    """A dynamic plan lists the same tiles, entry for entry, as the ordinary
    plan for its creation bitmap; each list sits at slot * nM (room for
    every tile of its row or column) and no dK/dV item is split."""
    S = spec["S"]
    static = lcm.Plan(1, S, Hq, Hkv, 64, spec)
    dyn = lcm.Plan(1, S, Hq, Hkv, 64, dict(spec, dynamic=True))
    assert dyn.stats["bwd_tile_cols"] == static.stats["bwd_tile_cols"]
    ls, ld = static.layout(), dyn.layout()
    fs, bs = lists_by_item(ls)
    fd, bd = lists_by_item(ld)
    assert dyn.stats["bwd_head_entries"] == static.stats["bwd_head_entries"]
    assert fs == fd and bs == bd
    nM = (S + 63) // 64
    assert (ld["fwd_items"][:, 2] % nM == 0).all() and (ld["bwd_items"][:, 2] % nM == 0).all()
    assert len(set(ld["fwd_items"][:, 2].tolist())) <= ld["fwd_list"].size // nM
    assert (ld["bwd_slot"] == -1).all() and ld["n_slots"] == 0 and len(ld["bwd_reduce"]) == 0
    assert dyn.stats["nnz_total"] == static.stats["nnz_total"]
    _check_lists(dyn, spec, Hq, Hkv)


def test_dynamic_plan_errors():
    S = 256
    lib = L.lib()
    d = lcm.MaskDescriptor(dict(syn.spec_causal(S), dynamic=True))
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID   # no bitmap
    assert b"block_bitmap" in lib.attn_last_error()
    offs, bits = syn.uniform_block_bitmap(S, 64, 2, 0.5, 0)
    spec = syn.with_bitmap(syn.spec_causal(S), offs, offs, bits)
    d = lcm.MaskDescriptor(spec)
    d.c.dynamic = 2
    assert _create((1, S, 4, 2, 64, 0.0), d.c) == L.ATTN_ERR_INVALID
    a = C.c_void_p(4096)  # never dereferenced: validation fails first
    static = lcm.Plan(1, S, 4, 2, 64, spec)
    assert lib.attn_plan_set_bitmap(static.handle, a, None) == L.ATTN_ERR_INVALID
    assert b"dynamic" in lib.attn_last_error()
    dyn = lcm.Plan(1, S, 4, 2, 64, dict(spec, dynamic=True))
    assert lib.attn_plan_set_bitmap(dyn.handle, a, None) == L.ATTN_ERR_INVALID
    assert b"not bound" in lib.attn_last_error()
    assert lib.attn_plan_set_bitmap(None, a, None) == L.ATTN_ERR_INVALID


def _desc_bytes(shape, desc):
    sh = L.Shape(*shape)
    pb, wb, kh = C.c_size_t(), C.c_size_t(), C.c_uint64()
    st = L.lib().attn_desc_plan_bytes(C.byref(sh), C.byref(desc), C.byref(pb), C.byref(wb), C.byref(kh))
    return st, pb.value, wb.value, kh.value


def test_desc_plan_cache_keys_on_content():
    """Equal masks from different arrays share one cached plan (same sizes
    and key hash); any change of shape, scalar, array or bitmap bit gives
    another; the sizes are those of an ordinary plan."""
    lib = L.lib()
    lib.attn_desc_cache_clear()
    S = 300
    shape = (1, S, 4, 2, 64, 0.0)
    docs = [100, 120, 80]
    d1 = lcm.MaskDescriptor(syn.spec_document(docs, True))
    d2 = lcm.MaskDescriptor(syn.spec_document(list(docs), True))   # other arrays, same content
    st1, pb1, wb1, h1 = _desc_bytes(shape, d1.c)
    st2, pb2, wb2, h2 = _desc_bytes(shape, d2.c)
    assert st1 == st2 == L.ATTN_OK and (pb1, wb1, h1) == (pb2, wb2, h2)
    p = lcm.Plan(*shape[:5], syn.spec_document(docs, True))
    assert pb1 == p.device_bytes() and wb1 == p.workspace_bytes()
    hashes = {h1}
    for spec in (syn.spec_document(docs, False), syn.spec_document([100, 121, 79], True),
                 syn.spec_causal(S), syn.spec_sliding(S, 64, True), syn.spec_sliding(S, 65, True)):
        st, _, _, h = _desc_bytes(shape, lcm.MaskDescriptor(spec).c)
        assert st == L.ATTN_OK
        hashes.add(h)
    st, _, _, h = _desc_bytes((2, S, 4, 2, 64, 0.0), d1.c)
    hashes.add(h)
    st, _, _, h = _desc_bytes((1, S, 4, 2, 64, 0.1), d1.c)
    hashes.add(h)
    offs, bits = syn.uniform_block_bitmap(S, 64, 2, 0.5, seed=3)
    b = syn.with_bitmap(syn.spec_causal(S), offs, offs, bits)
    _, _, _, hb = _desc_bytes(shape, lcm.MaskDescriptor(b).c)
    b5 = syn.with_bitmap(syn.spec_causal(S), offs, offs, bits * 5)   # nonzero = on
    _, _, _, hb5 = _desc_bytes(shape, lcm.MaskDescriptor(b5).c)
    assert hb == hb5
    flipped = bits.copy()
    flipped[1, 2, 3] ^= 1
    _, _, _, hf = _desc_bytes(shape, lcm.MaskDescriptor(syn.with_bitmap(syn.spec_causal(S), offs, offs, flipped)).c)
    hashes.update({hb, hf})
    assert len(hashes) == 10


def test_desc_plan_cache_errors_and_eviction():
    lib = L.lib()
    S = 256
    shape = (1, S, 4, 2, 64, 0.0)
    offs, bits = syn.uniform_block_bitmap(S, 64, 2, 0.5, 0)
    dyn = lcm.MaskDescriptor(dict(syn.with_bitmap(syn.spec_causal(S), offs, offs, bits), dynamic=True))
    assert _desc_bytes(shape, dyn.c)[0] == L.ATTN_ERR_INVALID
    assert b"dynamic" in lib.attn_last_error()
    bad = lcm.MaskDescriptor(syn.spec_causal(S))
    bad.c.kind = 99
    assert _desc_bytes(shape, bad.c)[0] == L.ATTN_ERR_INVALID
    assert _desc_bytes((1, S, 4, 2, 96, 0.0), lcm.MaskDescriptor(syn.spec_causal(S)).c)[0] == L.ATTN_ERR_UNSUPPORTED
    assert lib.attn_desc_plan_bytes(None, None, None, None, None) == L.ATTN_ERR_INVALID
    # more distinct masks than the cache holds: the oldest are evicted and
    # compiled again when asked for
    first = _desc_bytes(shape, lcm.MaskDescriptor(syn.spec_sliding(S, 1, True)).c)
    for w in range(1, 45):
        st, pb, _, _ = _desc_bytes(shape, lcm.MaskDescriptor(syn.spec_sliding(S, w, True)).c)
        assert st == L.ATTN_OK and pb > 0
    again = _desc_bytes(shape, lcm.MaskDescriptor(syn.spec_sliding(S, 1, True)).c)
    assert again == first
    lib.attn_desc_cache_clear()
    lib.attn_desc_release(None)   # unknown buffers are ignored


def test_desc_calls_validate_before_touching_the_gpu():
    """Argument errors of attn_fwd_desc / attn_bwd_desc return before any
    upload or launch (this host has no GPU)."""
    lib = L.lib()
    S = 128
    sh = L.Shape(1, S, 2, 1, 64, 0.0)
    d = lcm.MaskDescriptor(syn.spec_causal(S))
    P = C.c_void_p
    a = P(4096)  # never dereferenced
    big = C.c_size_t(1 << 24)
    assert lib.attn_fwd_desc(C.byref(sh), C.byref(d.c), None, a, a, a, a, a, big, None) == L.ATTN_ERR_INVALID
    assert lib.attn_fwd_desc(C.byref(sh), C.byref(d.c), a, a, a, a, P(4098), a, big, None) == L.ATTN_ERR_INVALID
    assert lib.attn_fwd_desc(C.byref(sh), C.byref(d.c), a, a, a, a, a, None, big, None) == L.ATTN_ERR_INVALID
    assert lib.attn_fwd_desc(C.byref(sh), C.byref(d.c), a, a, a, a, a, P(4096 + 16), big, None) == L.ATTN_ERR_INVALID
    assert lib.attn_fwd_desc(C.byref(sh), C.byref(d.c), a, a, a, a, a, a, C.c_size_t(8), None) == L.ATTN_ERR_INVALID
    assert lib.attn_bwd_desc(C.byref(sh), C.byref(d.c), a, a, a, a, a, a, a, a, a, a, C.c_size_t(16), a, big,
                             None) == L.ATTN_ERR_INVALID
    assert b"workspace" in lib.attn_last_error()
    os.environ["ATTN_FORCE_DEVICE_ERROR"] = "1"
    try:
        assert lib.attn_fwd_desc(C.byref(sh), C.byref(d.c), a, a, a, a, a, a, big, None) == L.ATTN_ERR_DEVICE
    finally:
        del os.environ["ATTN_FORCE_DEVICE_ERROR"]
