"""The rounding model behind the bar of the bf16 sweep layers (CPU only).

On the sweep's small layers a global max|dy|/rms(y) bar does not fit: with d and
d_ff of 64, top-1 routing and a binding capacity, drops zero many rows, a few
tokens reach several times rms(y), and the bf16 rounding of the SwiGLU activation
alone (the one narrowing the kernels do before the second product) moves y by
more than 2e-2 rms(y). These tests show that on the CPU, with the float64 oracle
plus that single rounding, and that the per-element bound the GPU sweep uses holds
for the model on every bf16 sweep layer while still failing a misplaced row.
"""
import numpy as np
import pytest

import workloads as wk
from oracle import moe as om
from rounding_model import round_bf16, y_bound, y_rounded_activation
from sweep_cases import sweep_cases, sweep_workload

_SWEEP = sweep_cases(48)
_BF16 = [i for i, kw in enumerate(_SWEEP) if kw["dtype"] == wk.BF16]


def _layer(i):
    wl = sweep_workload(i, _SWEEP[i])
    inp = wk.make_inputs(wl)
    host = inp.expert_stacks()
    ex = lambda e: tuple(wk.to_f64(a[e], wl.dtype) for a in host)
    sh = inp.shared()
    sh64 = tuple(wk.to_f64(a, wl.dtype) for a in sh) if sh is not None else None
    x64 = wk.to_f64(inp.x, wl.dtype)
    ref = om.forward(x64, wk.to_f64(inp.w_router, wl.dtype), ex, wl.k, wl.gate, inp.bias,
                     wl.capacity_factor, sh64)
    keep = ref["dest"] >= 0
    model = y_rounded_activation(wl.d, x64, ref["idx"], ref["gates"], keep, ex, sh64)
    bound = y_bound(wl.d, wl.d_ff, x64, ref["idx"], ref["gates"], keep, ex, sh64,
                    wl.d_ff_shared)
    return wl, ref, model, bound, ex, x64, keep


def test_round_bf16_is_nearest_even():
    a = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -3.0e-3])
    got = round_bf16(a)
    assert got[0] == 1.0
    assert got[1] == 1.0                      # tie -> even (1.0)
    assert got[2] == 1.0 + 2 * 2.0 ** -7      # tie -> even (odd neighbour below)
    assert got[3] == 1.0
    assert abs(got[4] - a[4]) <= 2.0 ** -8 * abs(a[4])


def test_layer26_activation_rounding_alone_exceeds_the_global_bar():
    """Sweep layer 26 (300 tokens, d = d_ff = 64, 40 experts, top-1, capacity 1.25):
    the activation's bf16 rounding by itself moves y by more than 2e-2 rms(y), and by
    no more than the per-element bound anywhere."""
    wl, ref, model, bound, *_ = _layer(26)
    assert wl.dtype == wk.BF16 and wl.k == 1 and wl.capacity_factor == 1.25
    y = ref["y"]
    rms = float(np.sqrt(np.mean(y ** 2)))
    rel = float(np.max(np.abs(model - y))) / rms
    assert ref["n_dropped"] > 0
    assert rel > 2e-2, rel
    assert np.all(np.abs(model - y) <= bound)


@pytest.mark.parametrize("i", _BF16)
def test_bound_holds_for_the_model_on_every_bf16_sweep_layer(i):
    _, ref, model, bound, *_ = _layer(i)
    assert np.all(np.abs(model - ref["y"]) <= bound)


def test_bound_fails_a_misplaced_row():
    """The bound is tight enough to catch a kept row that went through the wrong
    expert, or a gate applied to the wrong slot."""
    wl, ref, model, bound, ex, x64, keep = _layer(26)
    E = wl.E
    idx = ref["idx"].copy()
    t = int(np.nonzero(keep[:, 0])[0][0])
    idx[t, 0] = (idx[t, 0] + 1) % E
    wrong = y_rounded_activation(wl.d, x64, idx, ref["gates"], keep, ex)
    assert np.any(np.abs(wrong - ref["y"]) > bound)
    g = ref["gates"].copy()
    g[t, 0] *= 0.5
    wrong = y_rounded_activation(wl.d, x64, ref["idx"], g, keep, ex)
    assert np.any(np.abs(wrong - ref["y"]) > bound)
