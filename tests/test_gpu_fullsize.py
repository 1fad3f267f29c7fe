"""GPU parity at the workloads' full sizes, in the benchmark's launch
configuration (B=1, d=128, GQA 64:8; the block-sparse masks also under MHA
64:64 and at S = 128K).

At these sizes the fp64 oracle cannot run whole tensors, so the tests check:
* sampled rows of O, LSE and dQ, which the oracle computes one row at a time
  (everything a row's dQ needs is local to the row), against the same gate as
  the small cases;
* every row's mask coverage with Q = 0: all allowed keys then get the same
  weight, so exp(LSE_i) must equal the number of allowed keys n_i (counted
  from the oracle's predicate) and O_i the mean of the allowed v_j (beyond
  S = 64K on sampled blocks of rows, and with more than 2 bitmap heads on
  the first and last, to keep the oracle's count within seconds);
* sampled key columns of dK and dV, which the oracle computes from the full
  score rows of only the rows that see those keys (tests/fullsize_cases.py
  picks them within a cost budget), against the same gate, on both the
  unsplit dK/dV items (bf16 written by the pass itself) and the split ones
  (fp32 partials summed by the reduce pass);
* the identities sum_j dV_j = sum over query rows of the group of dO_i and
  sum_j dK_j = 0 per KV head, which hold at any size because every
  probability row sums to one (softmax is invariant to a shift of the keys);
* uniform V: O = v, dQ = dK = 0.
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as ora
from oracle import masks as om

from gpu_util import f64, gate, to_dev, to_f64
from fullsize_cases import Lazy64, col_cases, grad_cols_parallel, pick_cols

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import long_context_masked_amd as lcm  # noqa: E402

HQ, D = 64, 128
_INPUTS = {}


def inputs(S, Hkv):
    if (S, Hkv) not in _INPUTS:
        x = syn.attention_inputs(1, S, HQ, Hkv, D, seed=0)
        _INPUTS[(S, Hkv)] = (x, {n: to_dev(x[n], torch) for n in x})
    return _INPUTS[(S, Hkv)]


def _cases():
    out = []
    for label, spec in syn.config_mask_specs("dense", 49152):
        out.append(("dense48K_" + label, spec, 8))
    for label, spec in syn.config_mask_specs("document"):
        out.append(("doc64K_" + label, spec, 8))
    for label, spec in syn.config_mask_specs("hetero"):
        out.append(("hetero32K_" + label, spec, 8))
    for label, spec in syn.config_mask_specs("variants"):
        out.append(("variants32K_" + label, spec, 8))
    for label, spec in syn.config_mask_specs("tasks")[:2]:
        out.append(("tasks64K_" + label, spec, 8))
    for label, spec in syn.config_mask_specs("sparse", 32768, Hq=HQ, Hkv=8):
        out.append(("sparse32K_" + label, spec, 8))
    for label, spec in syn.config_mask_specs("sparse", 32768, Hq=HQ, Hkv=64):
        out.append(("sparse32K_mha_" + label, spec, 64))
    for label, spec in syn.config_mask_specs("sparse", 131072, Hq=HQ, Hkv=8):
        out.append(("sparse128K_" + label, spec, 8))
    # one bitmap per query head under GQA (work lists are unions over heads)
    offs, bits = syn.uniform_block_bitmap(32768, 128, HQ, 0.5, 1)
    out.append(("sparse32K_perhead_block128_50", syn.with_bitmap(syn.spec_full(32768), offs, offs, bits), 8))
    # one 128K MHA mask: its plan alone lists about 10^8 tiles per direction
    offs, bits = syn.uniform_block_bitmap(131072, 128, 64, 0.5, 0)
    out.append(("sparse128K_mha_block128_50", syn.with_bitmap(syn.spec_full(131072), offs, offs, bits), 64))
    return out


CASES = _cases()
IDS = [c[0] for c in CASES]


def _rows(S, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, S // 3, S // 2 + 7, S - 65, S - 2, S - 1]
    return sorted(set(fixed + rng.integers(0, S, 7).tolist()))


def _rows_with_keys(spec):
    """Rows with at least one allowed key, from the oracle's predicate (only
    the task-batch family has rows without keys; the others need no count)."""
    S = spec["S"]
    if spec["family"] != "task_batch" or "bitmap" in spec:
        return np.ones(S)
    out = np.zeros(S)
    for i0 in range(0, S, 2048):
        out[i0:i0 + 2048] = om.allowed(spec, i0, min(S, i0 + 2048)).any(axis=1)
    return out


@pytest.mark.parametrize("label,spec,Hkv", CASES, ids=IDS)
def test_sampled_rows(label, spec, Hkv):
    S = spec["S"]
    x, t = inputs(S, Hkv)
    plan = lcm.Plan(1, S, HQ, Hkv, D, spec)
    o, lse = lcm.fwd(plan, t["q"], t["k"], t["v"])
    dq, dk, dv = lcm.bwd(plan, t["q"], t["k"], t["v"], o, lse, t["do"])
    torch.cuda.synchronize()
    rows = _rows(S, 1)
    lz = {n: Lazy64(x[n]) for n in ("q", "k", "v", "do")}
    got = {"o": [], "dq": [], "lse": []}
    ref = {"o": [], "dq": [], "lse": [], "m_o": [], "m_dq": []}
    for h in (0, 7, 33, 63):
        r = ora.grad_rows(lz["q"], lz["k"], lz["v"], lz["do"], spec, h, rows)
        for n in ref:
            ref[n].append(r[n])
        got["o"].append(to_f64(o[0, rows, h]))
        got["dq"].append(to_f64(dq[0, rows, h]))
        got["lse"].append(lse[0, h, rows].cpu().numpy().astype(np.float64))
    g = {n: np.stack(v) for n, v in got.items()}
    rf = {n: np.stack(v) for n, v in ref.items()}
    gate("O", g["o"], rf["o"], rf["m_o"])
    gate("dQ", g["dq"], rf["dq"], rf["m_dq"])
    fin = np.isfinite(rf["lse"])
    assert (np.isneginf(g["lse"]) == ~fin).all()
    assert np.abs(g["lse"][fin] - rf["lse"][fin]).max() <= 5e-3
    # sum_j dV_j = sum of dO over the rows of the group that have a key
    dvs = dv[0].to(torch.float64).sum(dim=0)          # [Hkv, d]
    live = torch.from_numpy(_rows_with_keys(spec)).to(t["do"].device)
    dos = (t["do"][0].to(torch.float64) * live[:, None, None]).sum(dim=0)
    dos = dos.reshape(Hkv, HQ // Hkv, D).sum(dim=1)
    err = (dvs - dos).abs().max().item()
    assert err <= 1e-2 * np.sqrt(S * HQ / Hkv), err
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
    # sum_j dK_j = 0 per KV head: softmax is invariant to adding one vector
    # to every key, so the loss has zero derivative along that direction
    dks = dk[0].to(torch.float64).sum(dim=0).abs().max().item()
    assert dks <= 1e-2 * np.sqrt(S * HQ / Hkv), dks


@pytest.mark.parametrize("label,spec,Hkv", CASES, ids=IDS)
def test_mask_coverage_every_row(label, spec, Hkv):
    """Q = 0: exp(LSE_i) = n_i for every row and head (beyond S = 64K on
    sampled row blocks; with more than 2 bitmap heads on the first and last);
    O_i = mean of allowed v_j."""
    S = spec["S"]
    x, t = inputs(S, Hkv)
    plan = lcm.Plan(1, S, HQ, Hkv, D, spec)
    q0 = torch.zeros_like(t["q"])
    o, lse = lcm.fwd(plan, q0, t["k"], t["v"])
    torch.cuda.synchronize()
    nh = spec["bitmap"]["bits"].shape[0] if "bitmap" in spec else 1
    G = HQ // Hkv
    vbits = x["v"]
    # the oracle counts about 2.5e8 (row, key) pairs per second
    blocks = list(range(0, S, 2048)) if S <= 65536 else [0, S // 2 - 1024, S - 2048]
    hms = range(nh) if nh <= 2 else [0, nh - 1]
    for hm in hms:
        rows = np.concatenate([np.arange(i0, min(S, i0 + 2048)) for i0 in blocks])
        counts = np.concatenate([om.allowed(spec, i0, min(S, i0 + 2048), hm).sum(axis=1) for i0 in blocks])
        heads = [h for h in range(HQ) if om.mask_head(spec, h, HQ, Hkv) == hm]
        n_gpu = torch.exp(lse[0, heads][:, rows].to(torch.float64)).cpu().numpy()
        assert (np.rint(n_gpu) == counts[None, :]).all(), label
        has = counts > 0
        assert np.abs(n_gpu[:, has] / counts[None, has] - 1).max() < 1e-4
        # O_i = mean of the allowed v_j on sampled rows of the first head
        h = heads[0]
        rows = _rows(S, 2)
        vv = f64(vbits[0, :, h // G, :])
        a = np.stack([om.allowed(spec, i, i + 1, hm)[0] for i in rows])
        n = a.sum(axis=1, keepdims=True)
        want = (a @ vv) / np.maximum(n, 1)   # a row with no key has O = 0
        gate("O(Q=0)", to_f64(o[0, rows, h]), want)


_UNIFORM = [c for c in CASES if c[0].startswith(("dense48K_causal", "hetero32K_shared", "sparse32K_var",
                                                   "sparse128K_block64"))]


@pytest.mark.parametrize("label,spec,Hkv", _UNIFORM, ids=[c[0] for c in _UNIFORM])
def test_uniform_v_closed_form(label, spec, Hkv):
    """v_j = v for every key: O = v, and dQ = dK = 0 up to rounding."""
    S = spec["S"]
    x, t = inputs(S, Hkv)
    plan = lcm.Plan(1, S, HQ, Hkv, D, spec)
    v1 = t["v"][:, :1].expand_as(t["v"]).contiguous()
    o, lse = lcm.fwd(plan, t["q"], t["k"], v1)
    dq, dk, dv = lcm.bwd(plan, t["q"], t["k"], v1, o, lse, t["do"])
    torch.cuda.synchronize()
    want = v1[0, 0].repeat_interleave(HQ // Hkv, dim=0).to(torch.float32)  # [Hq, d]
    assert (o[0].to(torch.float32) - want[None]).abs().max().item() <= 2.0 ** -7 * want.abs().max().item()
    assert dq.abs().max().item() <= 1e-3
    assert dk.abs().max().item() <= 1e-3


COLS = col_cases()


@pytest.mark.parametrize("label,spec,Hkv,kvs,budget,extra,row_block", COLS, ids=[c[0] for c in COLS])
def test_sampled_key_columns(label, spec, Hkv, kvs, budget, extra, row_block):
    """dK and dV of sampled key columns, chained on the forward's own O and
    LSE, against the oracle; the columns cover unsplit dK/dV items and, where
    the plan splits items, split ones."""
    S = spec["S"]
    x, t = inputs(S, Hkv)
    plan = lcm.Plan(1, S, HQ, Hkv, D, spec)
    o, lse = lcm.fwd(plan, t["q"], t["k"], t["v"])
    dq, dk, dv = lcm.bwd(plan, t["q"], t["k"], t["v"], o, lse, t["do"])
    torch.cuda.synchronize()
    cols = {kv: pick_cols(spec, HQ, Hkv, kv, budget, extra=extra) for kv in kvs}
    assert all(len(c) > 0 for c in cols.values()), cols
    lay = plan.layout()
    items, slots = lay["bwd_items"], lay["bwd_slot"]
    paths = set()
    for kv, cs in cols.items():
        for c in cs:
            sel = (items[:, 0] == c // 128) & (items[:, 1] == kv)
            paths.add("split" if (slots[sel] >= 0).any() else "direct")
    assert "direct" in paths or slots.max() >= 0, paths
    print(f"{label}: columns {cols}, dK/dV paths {sorted(paths)}", flush=True)
    ref = grad_cols_parallel(x, spec, HQ, Hkv, kvs, cols, row_block)
    got = {n: np.concatenate([to_f64(g[0, cols[kv], kv]) for kv in kvs]) for n, g in (("dk", dk), ("dv", dv))}
    rf = {n: np.concatenate([ref[kv][n] for kv in kvs]) for n in ("dk", "dv", "m_dk", "m_dv")}
    gate("dK", got["dk"], rf["dk"], rf["m_dk"], quiet=False)
    gate("dV", got["dv"], rf["dv"], rf["m_dv"], quiet=False)
    if label == "hetero32K_global_sliding":
        assert "split" in paths, paths
