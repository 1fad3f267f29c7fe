"""Helpers for the parity tests: bf16 transfer and the parity gate.

Parity gate per tensor X in {O, dQ, dK, dV} (bf16 outputs) against the fp64
oracle, with rms = RMS of the whole oracle tensor and N its number of
elements compared:
  * every element:  |x_gpu - x_ref| <= 2e-2 rms + u |x_ref| + lam(N) u m_x
  * mean:           mean |x_gpu - x_ref| <= 2e-3 rms   (raw, no room)
The 2e-2 / 2e-3 bounds are the target's.  The other two terms are the error
that bf16 itself forces on any kernel with these rounding points, derived
rather than tuned:
  * u = 2^-8 is bf16's unit roundoff (8 significant bits, round to nearest
    even), so rounding the exact result to bf16 moves it by at most u |x|;
  * m_x is the 2-norm of the first-order coefficients of x with respect to
    the relative rounding errors made inside the computation (the forward's
    unnormalised probabilities, the O handed to the backward, the backward's
    P and dS before their products), returned by the oracle as its
    sensitivities and pinned against central differences of a perturbed
    pipeline (tests/test_gate.py);
  * under the standard probabilistic model of rounding (Higham and Mary,
    2019: rounding errors independent, mean zero, bounded by u), Hoeffding's
    inequality gives P(|sum_t c_t e_t| >= lam u |c|) <= 2 exp(-lam^2 / 2) for
    one element, so lam(N) = sqrt(2 ln(2 N / alpha)) bounds all N elements of
    a tensor at once except with probability alpha = 2^-20.
The D-propagation is inside m_x: D_i = dO_i . O_i is formed from the O the
backward is given, whose rounding errors reach dQ and dK through D.
Where the oracle tensor is identically zero (S = 1: every row sees one key,
so dQ = dK = 0 exactly) the relative gate is undefined and an absolute bound
ZERO_REF_ABS applies instead (inputs are unit-scale N(0, 1)).
"""
import math

import numpy as np

import synthetic as syn

GATE_MAX = 2e-2
GATE_MEAN = 2e-3
U_BF16 = 2.0 ** -8
ALPHA = 2.0 ** -20
ZERO_REF_ABS = 1e-3


def to_dev(bits, torch):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def f64(bits):
    return syn.bf16_bits_to_f32(bits).astype(np.float64)


def lam(n):
    """Hoeffding multiplier for n elements at failure probability ALPHA."""
    return math.sqrt(2.0 * math.log(2.0 * max(int(n), 1) / ALPHA))


def room(ref, mag, rms, n=None):
    """Per-element allowance: the target's 2e-2 rms plus bf16's own room."""
    ref = np.asarray(ref, dtype=np.float64)
    n = ref.size if n is None else n
    r = GATE_MAX * rms + U_BF16 * np.abs(ref)
    if mag is not None:
        r = r + lam(n) * U_BF16 * np.asarray(mag, dtype=np.float64)
    return r


def gate(name, got, ref, mag=None, rms=None, n=None, quiet=True):
    """Assert the parity gate; returns (raw max-abs / rms, mean-abs / rms,
    worst fraction of the allowance used)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(ref ** 2))) if rms is None else rms
    err = np.abs(got - ref)
    if rms == 0.0:
        assert err.max() <= ZERO_REF_ABS, f"{name}: {err.max():.3e} off an all-zero reference"
        return float(err.max()), float(err.mean()), 0.0
    mx, mean = float(err.max()) / rms, float(err.mean()) / rms
    allow = room(ref, mag, rms, n)
    frac = err / allow
    worst = np.unravel_index(int(np.argmax(frac)), frac.shape)
    used = float(frac[worst])
    if not quiet:
        print(f"{name}: max {mx:.2e} mean {mean:.2e} of rms, {used:.0%} of the allowance", flush=True)
    assert used <= 1.0, (
        f"{name}: element {worst} off by {err[worst]:.3e} (ref {ref[worst]:.4e}, rms {rms:.3e}, "
        f"allowance {allow[worst]:.3e}); raw max {mx:.3e}")
    assert mean <= GATE_MEAN, f"{name}: mean-abs {mean:.3e} of rms (raw max {mx:.3e})"
    return mx, mean, used


def assert_within_one_ulp(name, a, b):
    """a and b (bf16 tensors) are equal up to one bf16 unit in the last place,
    or, for elements near zero where the summed terms cancel, to 1e-4 of the
    tensor's RMS: what two runs of the atomic dQ accumulation can differ by
    (fp32 sums in another order, about 2^-24 of the terms each, then one
    rounding to bf16)."""
    import torch
    x, y = a.to(torch.float32), b.to(torch.float32)
    floor = 1e-4 * float(x.pow(2).mean().sqrt())
    ok = (x - y).abs() <= 2.0 ** -7 * torch.maximum(x.abs(), y.abs()) + floor
    assert bool(ok.all()), f"{name}: {int((~ok).sum())} elements differ by more than one bf16 ulp"
