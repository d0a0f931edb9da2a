"""The rounding model behind the activation format and the bf16 parity bars (CPU only).

The kernels' one narrowing is the SwiGLU activation between the two expert
products. Rounded to bf16, that alone moves y by more than the 2e-2 rms(y) bar on
some layers: sweep layer 26 (d = d_ff = 64, top-1, binding capacity) and the
Switch-shaped layer at 8192 tokens (71 % of the tokens dropped, so rms(y) is low,
and a heavy-tailed activation), where the GPU's error at every token matched this
model to the last digit. Stored as IEEE half (8x finer) the same layers sit well
inside the bar. These tests show that with the float64 oracle plus those roundings
alone, and that the per-element bound the GPU tests use holds for the model on every
bf16 sweep layer while still failing a misplaced row.
"""
import numpy as np
import pytest

import workloads as wk
from oracle import moe as om
from rounding_model import round_bf16, round_f16, y_bound, y_rounded_activation
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
    return wl, ref, model, bound, ex, x64, keep, sh64


def _rel(a, y):
    return float(np.max(np.abs(a - y))) / float(np.sqrt(np.mean(y ** 2)))


def test_rounding_is_nearest_even():
    a = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -3.0e-3])
    got = round_bf16(a)
    assert got[0] == 1.0
    assert got[1] == 1.0                      # tie -> even (1.0)
    assert got[2] == 1.0 + 2 * 2.0 ** -7      # tie -> even (odd neighbour below)
    assert got[3] == 1.0
    assert abs(got[4] - a[4]) <= 2.0 ** -8 * abs(a[4])
    with np.errstate(over="ignore"):
        h = round_f16(np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 70000.0, 2.0 ** -20,
                                -3.0e-3]))
    assert h[0] == 1.0 and h[1] == 1.0 + 2 * 2.0 ** -10
    assert np.isinf(h[2])                     # above 65504
    assert h[3] == 2.0 ** -20                 # a subnormal step multiple: exact
    assert abs(h[4] + 3.0e-3) <= 2.0 ** -11 * 3.0e-3


def test_bf16_weights_widen_to_half_exactly_above_2_pow_minus_17():
    """Every bf16 value in [2^-17, 65504] is a half value; below, the error is at
    most half the subnormal step 2^-24."""
    bits = np.arange(0, 1 << 15, dtype=np.uint16)          # all non-negative bf16
    v = wk.bf16_bits_to_f32(bits).astype(np.float64)
    v = v[np.isfinite(v) & (v <= 65504.0)]
    w = round_f16(v)
    big = v >= 2.0 ** -17
    assert np.array_equal(w[big], v[big])
    assert np.max(np.abs(w[~big] - v[~big])) <= 2.0 ** -25


def test_layer26_bf16_activation_exceeds_the_bar_half_does_not():
    """Sweep layer 26 (300 tokens, d = d_ff = 64, 40 experts, top-1, capacity 1.25):
    a bf16 activation alone moves y by more than 2e-2 rms(y); the half activation of
    the kernels stays within 2e-2 rms(y) and within the per-element bound."""
    wl, ref, model, bound, ex, x64, keep, sh64 = _layer(26)
    assert wl.dtype == wk.BF16 and wl.k == 1 and wl.capacity_factor == 1.25
    assert ref["n_dropped"] > 0
    y = ref["y"]
    as_bf16 = y_rounded_activation(wl.d, x64, ref["idx"], ref["gates"], keep, ex, sh64,
                                   act="bf16")
    assert _rel(as_bf16, y) > 2e-2
    assert _rel(model, y) < 0.5e-2
    assert np.all(np.abs(model - y) <= bound)


@pytest.mark.parametrize("i", _BF16)
def test_model_within_both_bars_on_every_bf16_sweep_layer(i):
    _, ref, model, bound, *_ = _layer(i)
    assert np.all(np.abs(model - ref["y"]) <= bound)
    assert _rel(model, ref["y"]) <= 2e-2


def test_bound_fails_a_misplaced_row():
    """The bound is tight enough to catch a kept row that went through the wrong
    expert, or a gate applied to the wrong slot."""
    wl, ref, model, bound, ex, x64, keep, _ = _layer(26)
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


def test_switch_layer_needs_the_half_activation():
    """The Switch-shaped layer (8192 tokens, d 1024, 64 experts of d_ff 4096, top-1,
    capacity factor 1.0: 6470 tokens dropped) with the oracle's routing: a bf16
    activation moves y by 0.049 rms(y) (the GPU measured 0.00323 / 0.0664, the same
    figure), the half activation by less than half of the 2e-2 bar (0.0056)."""
    wl = wk.get("switch_t8192_cf1.0")
    inp = wk.make_inputs(wl)
    x64 = wk.to_f64(inp.x, wl.dtype)
    r = om.route(x64, wk.to_f64(inp.w_router, wl.dtype), wl.k, wl.gate, None)
    p = om.assign_rows(r["idx"], wl.E, wl.capacity_factor)
    keep = p["dest"][:, 0] >= 0
    y = np.zeros((wl.T, wl.d))
    yb = np.zeros_like(y)
    yh = np.zeros_like(y)
    for e in range(wl.E):
        rows = np.nonzero((r["idx"][:, 0] == e) & keep)[0]
        if rows.size == 0:
            continue
        w1, w3, w2 = (wk.to_f64(a, wl.dtype) for a in inp.expert(e))
        a = om.swiglu_hidden(x64[rows], w1, w3)
        g = r["gates"][rows, :1]
        y[rows] = g * (a @ w2.T)
        yb[rows] = g * (round_bf16(a) @ w2.T)
        yh[rows] = g * (round_f16(a) @ round_f16(w2).T)
    assert p["n_dropped"] == 6470
    assert 0.045 < _rel(yb, y) < 0.053
    assert _rel(yh, y) < 1e-2
