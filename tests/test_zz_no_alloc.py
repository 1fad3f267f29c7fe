"""attn_bwd_noalloc: the backward with its workspace in the library's static
device array, for callers that cannot allocate.  Through the C ABI, against
attn_bwd with a caller workspace (the same kernels and summation order, so
bit for bit), on two calls in a row, the second with a smaller input; and
the rejection of a plan whose workspace exceeds the array.
"""
import ctypes as C

import pytest

import synthetic as syn

from gpu_util import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import long_context_masked_amd as lcm  # noqa: E402
from long_context_masked_amd import _lib as L  # noqa: E402

P = C.c_void_p


def _run(spec, B, Hq, Hkv, d, seed):
    S = spec["S"]
    print(f"no-alloc backward: {spec['family']} B={B} S={S} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    x = syn.attention_inputs(B, S, Hq, Hkv, d, seed)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    plan = lcm.Plan(B, S, Hq, Hkv, d, spec)
    o, lse = lcm.fwd(plan, q, k, v)
    ref = lcm.bwd(plan, q, k, v, o, lse, do)
    got = [torch.full_like(t, 3.0) for t in ref]
    stream = torch.cuda.current_stream().cuda_stream
    L.check(L.lib().attn_bwd_noalloc(plan.handle, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
                                     P(o.data_ptr()), P(lse.data_ptr()), P(do.data_ptr()),
                                     P(got[0].data_ptr()), P(got[1].data_ptr()), P(got[2].data_ptr()),
                                     P(stream)))
    torch.cuda.synchronize()
    for n, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{n} of attn_bwd_noalloc differs from attn_bwd"
    return plan


def test_noalloc_backward_equals_attn_bwd_on_two_calls():
    # first call: S = 1K causal splits every dK/dV item, so the static array
    # holds partial dK/dV slots as well as the row statistics
    p1 = _run(syn.spec_causal(1024), 1, 8, 2, 128, seed=61)
    assert p1.layout()["n_slots"] > 0
    # second call, smaller: what the first left in the array must not matter
    _run(syn.spec_sliding(333, 70, True), 2, 4, 2, 64, seed=62)


def test_noalloc_rejects_a_workspace_beyond_the_array():
    cap = int(L.lib().attn_bwd_noalloc_max_workspace_bytes())
    assert cap == 128 << 20
    S, Hq = 300032, 64          # row statistics alone: 64 heads x 300032 rows x 8 bytes
    plan = lcm.Plan(1, S, Hq, 8, 128, syn.spec_sliding(S, 64, True))
    assert plan.workspace_bytes() > cap
    plan.bind()
    st = L.lib().attn_bwd_noalloc(plan.handle, *([None] * 9), None)
    assert st == L.ATTN_ERR_INVALID
    assert b"static workspace" in L.lib().attn_last_error()
