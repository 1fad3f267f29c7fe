"""HIP graph capture of the forward and backward, and one plan shared by two
streams (GPU).

Once a plan is bound, attn_fwd and attn_bwd only launch kernels on the given
stream (no allocation, no memset, no synchronisation), so a caller can
capture them in a graph and replay it.  The test captures one forward plus
backward with torch's graph API, replays it several times with eager work
and synchronisations in between, and checks every replay bit for bit against
the eager results (both passes are deterministic); then it changes the
inputs in place and checks that a replay follows them.
"""
import pytest

import synthetic as syn

from gpu_util import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import long_context_masked_amd as lcm  # noqa: E402


def _cases():
    offs, bits = syn.variable_block_bitmap(700, 32, 224, 2, 0.5, seed=3)
    return [
        # S = 1K causal splits every dK/dV item (partial slots and the reduce launch)
        ("causal_1k_gqa", syn.spec_causal(1024), 8, 2, 128),
        ("varblock_700_mha_d64", syn.with_bitmap(syn.spec_full(700), offs, offs, bits), 2, 2, 64),
    ]


CASES = _cases()


@pytest.mark.parametrize("label,spec,Hq,Hkv,d", CASES, ids=[c[0] for c in CASES])
def test_captured_forward_backward_replays_match_eager(label, spec, Hq, Hkv, d):
    print(f"graph case {label}", flush=True)
    S = spec["S"]
    x = syn.attention_inputs(1, S, Hq, Hkv, d, seed=31)
    x2 = syn.attention_inputs(1, S, Hq, Hkv, d, seed=32)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    q2 = to_dev(x2["q"], torch)
    plan = lcm.Plan(1, S, Hq, Hkv, d, spec)
    plan.bind(q.device)

    def step(qq):
        o, lse = lcm.fwd(plan, qq, k, v)
        return (o, lse) + tuple(lcm.bwd(plan, qq, k, v, o, lse, do))

    ref = [t.clone() for t in step(q)]
    ref2 = [t.clone() for t in step(q2)]
    torch.cuda.synchronize()

    qg = q.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(qg)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(qg)
    torch.cuda.synchronize()

    names = ("O", "LSE", "dQ", "dK", "dV")
    for rep in range(3):
        step(q2)  # eager work between replays, on other inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, got, want in zip(names, outs, ref):
            assert torch.equal(got, want), f"replay {rep}: {n} differs from the eager result"
    qg.copy_(q2)
    graph.replay()
    torch.cuda.synchronize()
    for n, got, want in zip(names, outs, ref2):
        assert torch.equal(got, want), f"replay on new inputs: {n} differs from the eager result"


def test_one_plan_on_two_streams_at_once():
    """A bound plan is read-only on the device, so two streams may use it at
    the same time: forward + backward on two streams concurrently, each
    against its own sequential result."""
    S, Hq, Hkv, d = 1024, 8, 2, 128
    spec = syn.spec_causal(S)
    plan = lcm.Plan(1, S, Hq, Hkv, d, spec)
    ins = []
    for seed in (41, 42):
        x = syn.attention_inputs(1, S, Hq, Hkv, d, seed=seed)
        ins.append(tuple(to_dev(x[n], torch) for n in ("q", "k", "v", "do")))
    plan.bind(ins[0][0].device)

    def step(q, k, v, do):
        o, lse = lcm.fwd(plan, q, k, v)
        return (o, lse) + tuple(lcm.bwd(plan, q, k, v, o, lse, do))

    ref = [[t.clone() for t in step(*x)] for x in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        for s, x in zip(streams, ins):
            with torch.cuda.stream(s):
                outs.append((step(*x), s))
    torch.cuda.synchronize()
    for i, (got, s) in enumerate(outs):
        for n, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, ref[i % 2]):
            assert torch.equal(a, b), f"launch {i}: {n} differs from the sequential result"
