"""GPU parity of the partial-attention + merge path: attention over a mask
computed as the merge of fp32 partial results over disjoint chunks of the
keys (each chunk a plan whose mask keeps only those keys; the last merge
writes bf16), and the backward over the chunks with the merged O and LSE.
The oracle is the fp64 forward/backward over the whole mask and the fp64
merge of the same partial results."""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as ora

from gpu_util import f64, gate, to_dev, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import long_context_masked_amd as lcm  # noqa: E402


def key_chunks(base, cuts):
    """base restricted to the key ranges between consecutive cuts."""
    S = base["S"]
    offs = [0] + list(cuts) + [S]
    out = []
    for c in range(len(offs) - 1):
        bits = np.zeros((1, 1, len(offs) - 1), dtype=np.uint8)
        bits[0, 0, c] = 1
        out.append(syn.with_bitmap(base, [0, S], offs, bits))
    return out


CASES = [
    ("causal700_cut320", syn.spec_causal(700), [320], 1, 8, 2, 128),
    ("full512_3chunks", syn.spec_full(512), [128, 384], 1, 4, 2, 64),
    ("causal_doc600", syn.spec_document(syn.sample_doc_lens(600, 16, 300, 2), True), [256], 2, 4, 4, 64),
    ("global_sliding640", syn.spec_global_sliding(640, 16, 100), [192, 448], 1, 8, 1, 128),
]


def _run(base, cuts, B, Hq, Hkv, d, seed=3):
    S = base["S"]
    x = syn.attention_inputs(B, S, Hq, Hkv, d, seed)
    t = {n: to_dev(x[n], torch) for n in x}
    plans = [lcm.Plan(B, S, Hq, Hkv, d, sp) for sp in key_chunks(base, cuts)]
    parts = [lcm.fwd_partial(p, t["q"], t["k"], t["v"]) for p in plans]
    o, lse = parts[0]
    for c, (oc, lc) in enumerate(parts[1:]):
        o, lse = lcm.merge(o, lse, oc, lc, bf16_out=(c == len(parts) - 2))
    return x, t, plans, o, lse


@pytest.mark.parametrize("label,base,cuts,B,Hq,Hkv,d", CASES, ids=[c[0] for c in CASES])
def test_merged_forward_matches_whole_mask(label, base, cuts, B, Hq, Hkv, d):
    x, t, plans, o, lse = _run(base, cuts, B, Hq, Hkv, d)
    torch.cuda.synchronize()
    qf, kf, vf, dof = (f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = ora.backward(qf, kf, vf, dof, base, magnitudes=True)
    gate("O", to_f64(o), ref["o"], ref["m_o"])
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref["lse"])
    assert (np.isneginf(lg) == ~fin).all()
    assert np.abs(lg[fin] - ref["lse"][fin]).max() <= 5e-3


@pytest.mark.parametrize("label,base,cuts,B,Hq,Hkv,d", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_partial_forward_matches_chunk(label, base, cuts, B, Hq, Hkv, d):
    """attn_fwd_partial over one chunk: fp32 O and LSE of that chunk's mask."""
    S = base["S"]
    x = syn.attention_inputs(B, S, Hq, Hkv, d, 3)
    t = {n: to_dev(x[n], torch) for n in x}
    spec = key_chunks(base, cuts)[-1]
    o, lse = lcm.fwd_partial(lcm.Plan(B, S, Hq, Hkv, d, spec), t["q"], t["k"], t["v"])
    torch.cuda.synchronize()
    assert o.dtype == torch.float32
    ref = ora.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), spec, magnitudes=True)
    gate("O", o.double().cpu().numpy(), ref["o"], ref["m_o"])
    lg = lse.double().cpu().numpy()
    fin = np.isfinite(ref["lse"])
    assert (np.isneginf(lg) == ~fin).all()  # causal: rows before the chunk see no key
    assert np.abs(lg[fin] - ref["lse"][fin]).max() <= 5e-3


@pytest.mark.parametrize("label,base,cuts,B,Hq,Hkv,d", CASES, ids=[c[0] for c in CASES])
def test_chunked_backward_sums_to_whole_mask(label, base, cuts, B, Hq, Hkv, d):
    """attn_bwd over each chunk with the merged O and LSE: the chunks' dQ add
    up to dQ, and their dK, dV (zero outside the chunk) to dK, dV."""
    x, t, plans, o, lse = _run(base, cuts, B, Hq, Hkv, d)
    dq = dk = dv = None
    for p in plans:
        g = lcm.bwd(p, t["q"], t["k"], t["v"], o, lse, t["do"])
        g = [a.float() for a in g]
        dq, dk, dv = (g if dq is None else (dq + g[0], dk + g[1], dv + g[2]))
    torch.cuda.synchronize()
    qf, kf, vf, dof = (f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = ora.backward(qf, kf, vf, dof, base, magnitudes=True)
    tf = lambda a: a.cpu().numpy().astype(np.float64)
    gate("dQ", tf(dq), ref["dq"], ref["m_dq"])
    gate("dK", tf(dk), ref["dk"], ref["m_dk"])
    gate("dV", tf(dv), ref["dv"], ref["m_dv"])


@pytest.mark.parametrize("bf16_out", [False, True])
def test_merge_against_oracle_merge_with_empty_rows(bf16_out):
    """Random partial results, some rows empty in one part or in both: the
    kernel's merge against the fp64 merge of the same fp32 values."""
    B, S, H, d = 2, 200, 3, 128
    g = torch.Generator().manual_seed(7)
    o1 = torch.randn(B, S, H, d, generator=g)
    o2 = torch.randn(B, S, H, d, generator=g)
    l1 = torch.randn(B, H, S, generator=g) * 4
    l2 = torch.randn(B, H, S, generator=g) * 4
    l1[:, :, ::7] = -float("inf")
    l2[:, :, ::5] = -float("inf")
    o1[:, ::7] = 0
    o2[:, ::5] = 0
    dev = torch.device("cuda:0")
    o, lse = lcm.merge(o1.to(dev), l1.to(dev), o2.to(dev), l2.to(dev), bf16_out=bf16_out)
    assert o.dtype == (torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    ro, rl = ora.merge([o1.double().numpy(), o2.double().numpy()], [l1.double().numpy(), l2.double().numpy()])
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    fin = np.isfinite(rl)
    assert (np.isneginf(gl) == ~fin).all() and (~fin).any()
    assert np.abs(gl[fin] - rl[fin]).max() <= 1e-5 * (1 + np.abs(rl[fin]).max())
    assert (go[np.broadcast_to(~fin.transpose(0, 2, 1)[..., None], go.shape)] == 0).all()
    # O is a convex combination of o1 and o2: fp32 arithmetic, then (bf16_out)
    # one rounding to bf16
    rel = 2.0 ** -8 if bf16_out else 1e-6
    bound = rel * np.maximum(np.abs(o1.double().numpy()), np.abs(o2.double().numpy())) + 1e-6
    assert (np.abs(go - ro) <= bound).all()


def test_merge_full_size_sampled_rows():
    """S = 16K CAUSAL, GQA 64:8, d = 128, keys split at 8K: sampled rows of
    the merged O and LSE against the oracle's rows of the whole mask."""
    S, Hq, Hkv, d = 16384, 64, 8, 128
    base = syn.spec_causal(S)
    x, t, plans, o, lse = _run(base, [8192], 1, Hq, Hkv, d, seed=0)
    torch.cuda.synchronize()
    rows = [0, 1, 4095, 8191, 8192, 8193, 12000, S - 1]
    q, k, v = (f64(x[n]) for n in ("q", "k", "v"))
    for h in (0, 13, 63):
        ro, rl = ora.output_rows(q, k, v, base, h, rows)
        gate("O", to_f64(o[0, rows, h]), ro)
        assert np.abs(lse[0, h, rows].cpu().numpy() - rl).max() <= 5e-3
