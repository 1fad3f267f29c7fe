"""Helpers for GPU tests: bf16 transfer and the parity gate.

Parity gate per tensor X in {O, dQ, dK, dV} (bf16 outputs) against the fp64
oracle, with rms = RMS of the whole oracle tensor:
  * every element:  |x_gpu - x_ref| <= 2e-2 * rms + eps * (|x_ref| + 2 * m_x)
  * mean:           mean |x_gpu - x_ref| <= 2e-3 * rms
eps = 2^-7 is the machine epsilon of bf16 and m_x = sqrt(sum_t (a_t b_t)^2)
is the quadratic magnitude of the product that forms x (returned by the
oracle).  The eps terms are the room the bf16 formats themselves need:
rounding the exact result to bf16 (|x_ref|) and rounding P or dS to bf16
before the product (m_x; 2 m_x is about eight standard deviations of
round-to-nearest error).  Without them the max bound is unreachable for any
bf16-output kernel on causal masks, whose first rows mix a handful of keys
and are far larger than the tensor RMS.  dQ and dK are compared with the
oracle run on the bf16 O the forward returns (D = rowsum(dO * O) uses it).
The raw max-abs / rms is reported alongside.  Where the oracle tensor is
identically zero (S = 1: every row sees one key, so dQ = dK = 0 exactly) the
relative gate is undefined and an absolute bound ZERO_REF_ABS applies
instead (inputs are unit-scale N(0, 1)).
"""
import numpy as np

import synthetic as syn

GATE_MAX = 2e-2
GATE_MEAN = 2e-3
BF16_EPS = 2.0 ** -7
ZERO_REF_ABS = 1e-3


def to_dev(bits, torch):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def f64(bits):
    return syn.bf16_bits_to_f32(bits).astype(np.float64)


def gate(name, got, ref, mag=None, rms=None):
    """Assert the parity gate; returns (raw max-abs / rms, mean-abs / rms)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(ref ** 2))) if rms is None else rms
    err = np.abs(got - ref)
    if rms == 0.0:
        assert err.max() <= ZERO_REF_ABS, f"{name}: {err.max():.3e} off an all-zero reference"
        return float(err.max()), float(err.mean())
    mx, mean = float(err.max()) / rms, float(err.mean()) / rms
    room = np.abs(ref) if mag is None else np.abs(ref) + 2.0 * np.asarray(mag)
    excess = err - (GATE_MAX * rms + BF16_EPS * room)
    worst = np.unravel_index(int(np.argmax(excess)), excess.shape)
    assert excess.max() <= 0.0, (
        f"{name}: element {worst} off by {err[worst]:.3e} (ref {ref[worst]:.4e}, rms {rms:.3e}); "
        f"raw max {mx:.3e}")
    assert mean <= GATE_MEAN, f"{name}: mean-abs {mean:.3e} of rms (raw max {mx:.3e})"
    return mx, mean
