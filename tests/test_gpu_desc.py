"""GPU tests of the descriptor calls (attn_fwd_desc / attn_bwd_desc) and
their plan cache: results equal, bit for bit, those of the same mask through
an explicit plan, and agree with the fp64 oracle; one plan buffer can serve
several masks in turn (the blob is uploaded again when the mask changes), and
a released buffer is filled again before use."""
import ctypes as C

import numpy as np
import pytest

import synthetic as syn
from oracle import attention as ora

from gpu_util import gate, to_dev, to_f64, f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import long_context_masked_amd as lcm  # noqa: E402
from long_context_masked_amd import _lib as L  # noqa: E402


def _specs(S):
    offs, bits = syn.uniform_block_bitmap(S, 64, 2, 0.5, seed=4)
    return [("causal", syn.spec_causal(S)),
            ("causal_document", syn.spec_document(syn.sample_doc_lens(S, 32, 300, 2), True)),
            ("shared_question", syn.spec_shared_question(60, syn.sample_answers(S - 60, 3, 1))),
            ("block64", syn.with_bitmap(syn.spec_full(S), offs, offs, bits))]


S, B, Hq, Hkv, d = 700, 1, 8, 2, 128
SPECS = _specs(S)


def _inputs(seed):
    x = syn.attention_inputs(B, S, Hq, Hkv, d, seed)
    return x, [to_dev(x[n], torch) for n in ("q", "k", "v", "do")]


@pytest.mark.parametrize("label,spec", SPECS, ids=[l for l, _ in SPECS])
def test_desc_calls_equal_plan_calls(label, spec):
    print(f"desc case {label}", flush=True)
    x, (q, k, v, do) = _inputs(1)
    o1, l1 = lcm.fwd_desc(q, k, v, spec)
    g1 = lcm.bwd_desc(q, k, v, o1, l1, do, spec)
    plan = lcm.Plan(B, S, Hq, Hkv, d, spec)
    o2, l2 = lcm.fwd(plan, q, k, v)
    g2 = lcm.bwd(plan, q, k, v, o2, l2, do)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(g1[0], g2[0])
    for a, b in zip(g1[1:], g2[1:]):   # both plans split the same items: same order of sums
        assert torch.equal(a, b)
    if label == "causal_document":
        qf, kf, vf, dof = (f64(x[n]) for n in ("q", "k", "v", "do"))
        ref = ora.backward(qf, kf, vf, dof, spec, magnitudes=True)
        gate("O", to_f64(o1), ref["o"], ref["m_o"])
        gate("dQ", to_f64(g1[0]), ref["dq"], ref["m_dq"])
        gate("dK", to_f64(g1[1]), ref["dk"], ref["m_dk"])
        gate("dV", to_f64(g1[2]), ref["dv"], ref["m_dv"])


def _fwd_desc_raw(spec, q, k, v, buf_ptr, nbytes):
    desc = lcm.MaskDescriptor(spec)
    sh = L.Shape(B, S, Hq, Hkv, d, 0.0)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    P = C.c_void_p
    L.check(L.lib().attn_fwd_desc(C.byref(sh), C.byref(desc.c), P(q.data_ptr()), P(k.data_ptr()),
                                  P(v.data_ptr()), P(o.data_ptr()), P(lse.data_ptr()), P(buf_ptr),
                                  C.c_size_t(nbytes), P(torch.cuda.current_stream().cuda_stream)))
    return o, lse


def test_one_plan_buffer_shared_by_several_masks():
    """A -> B -> C -> A through one buffer: each call uploads the blob it
    needs; then the buffer is released, overwritten, and used again."""
    _, (q, k, v, _) = _inputs(2)
    need = 0
    for _, spec in SPECS:
        st_sh = L.Shape(B, S, Hq, Hkv, d, 0.0)
        pb = C.c_size_t()
        L.check(L.lib().attn_desc_plan_bytes(C.byref(st_sh), C.byref(lcm.MaskDescriptor(spec).c),
                                             C.byref(pb), None, None))
        need = max(need, pb.value)
    buf = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    ptr = buf.data_ptr() + (-buf.data_ptr()) % 256
    order = [0, 1, 2, 3, 0, 2, 0]
    for i in order:
        label, spec = SPECS[i]
        print(f"shared buffer: {label}", flush=True)
        o, lse = _fwd_desc_raw(spec, q, k, v, ptr, need)
        o2, l2 = lcm.fwd(lcm.Plan(B, S, Hq, Hkv, d, spec), q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2)
    L.lib().attn_desc_release(C.c_void_p(ptr))
    buf.fill_(0xFF)      # no longer known to hold a plan: it is filled again
    torch.cuda.synchronize()
    o, lse = _fwd_desc_raw(SPECS[0][1], q, k, v, ptr, need)
    o2, l2 = lcm.fwd(lcm.Plan(B, S, Hq, Hkv, d, SPECS[0][1]), q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    L.lib().attn_desc_release(C.c_void_p(ptr))


def test_cache_clear_then_calls_again():
    _, (q, k, v, do) = _inputs(3)
    spec = SPECS[1][1]
    o1, l1 = lcm.fwd_desc(q, k, v, spec)
    lcm.desc_cache_clear()
    o2, l2 = lcm.fwd_desc(q, k, v, spec)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_python_forms_with_a_mask_and_autograd():
    """fwd(q, k, v, mask), bwd(q, k, v, o, lse, do, mask) and attention(q, k,
    v, mask) equal the Plan forms."""
    _, (q, k, v, do) = _inputs(5)
    spec = SPECS[2][1]
    plan = lcm.Plan(B, S, Hq, Hkv, d, spec)
    o1, l1 = lcm.fwd(q, k, v, spec)
    g1 = lcm.bwd(q, k, v, o1, l1, do, spec)
    o2, l2 = lcm.fwd(plan, q, k, v)
    g2 = lcm.bwd(plan, q, k, v, o2, l2, do)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    oa = lcm.attention(qa, ka, va, spec)
    oa.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(oa.detach(), o2)
    assert torch.equal(qa.grad, g2[0]) and torch.equal(ka.grad, g2[1]) and torch.equal(va.grad, g2[2])
