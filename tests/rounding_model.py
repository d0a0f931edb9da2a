"""Where the HIP path rounds, modelled on the CPU for bf16 layers (test
infrastructure, not part of the oracle).

The kernels take bf16 x and weights and accumulate both expert products in fp32.
The only narrowing on the path is the SwiGLU activation a = silu(x W1^T) * (x W3^T),
stored as IEEE half (11-bit significand, nearest-even) between the two products;
the second product widens W2 from bf16 to half (exact for |w| >= 2^-17, smaller
weights to half's subnormal step, an error <= 2^-25) and runs on half MFMAs with
fp32 accumulation. Gates, y_perm and y stay fp32. This module evaluates the layer
with exactly those roundings added to the float64 oracle (or, for comparison, with
the activation rounded to bf16 instead), and the per-element bound the parity tests
hold bf16 layers to:

  |y_gpu - y| <= (u + 2 (d + d_ff) 2^-24) sum_j |g_j| sum_f |a_jf w2_e,if|
                 + 2^-25 sum_j |g_j| sum_f |a_jf|                    (+ shared)

u = 2^-11 is the activation's rounding (nearest-even to an 11-bit significand moves
an element by at most 2^-11 of itself); (d + d_ff) 2^-24 covers the fp32
accumulation of the two products, doubled because the first product's error reaches
y through silu and the branch product with a factor below 2; the last term is the
widening of the smallest weights. The gates and the combine (fp32, at most k + 1
terms) add rounding far below these.
"""
from __future__ import annotations

import numpy as np

import workloads as wk
from oracle import moe as om

U_F16 = 2.0 ** -11   # unit roundoff of IEEE half (11-bit significand, nearest-even)
U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8-bit significand, nearest-even)
U_F32 = 2.0 ** -24
W_WIDEN_ABS = 2.0 ** -25   # bf16 -> half below 2^-17: half of the subnormal step


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 (nearest-even), widened back to float64."""
    return wk.bf16_bits_to_f32(wk.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


def round_f16(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> IEEE half (nearest-even, with subnormals), back to float64."""
    return np.asarray(a, np.float32).astype(np.float16).astype(np.float64)


def _groups(idx, keep):
    need = {}
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                need.setdefault(int(idx[t, j]), []).append((t, j))
    return need


def y_bound(d, d_ff, x64, idx, gates64, keep, expert64, shared64=None, d_ff_shared=0):
    """The per-element bound above, [T, d]; expert64(e) returns (W1, W3, W2) in float64."""
    T = x64.shape[0]
    mag = np.zeros((T, d))
    amag = np.zeros(T)
    for e, rows in sorted(_groups(idx, keep).items()):
        w1, w3, w2 = expert64(e)
        a = np.abs(om.swiglu_hidden(x64[[t for t, _ in rows]], w1, w3))
        out = a @ np.abs(w2).T
        asum = a.sum(axis=1)
        for (t, j), o, s_ in zip(rows, out, asum):
            mag[t] += abs(gates64[t, j]) * o
            amag[t] += abs(gates64[t, j]) * s_
    dff = d_ff
    if shared64 is not None:
        a = np.abs(om.swiglu_hidden(x64, shared64[0], shared64[1]))
        mag += a @ np.abs(shared64[2]).T
        amag += a.sum(axis=1)
        dff = max(dff, d_ff_shared)
    return (U_F16 + 2.0 * (d + dff) * U_F32) * mag + W_WIDEN_ABS * amag[:, None]


def y_rounded_activation(d, x64, idx, gates64, keep, expert64, shared64=None, act="f16"):
    """The layer with the kernels' roundings, all else in float64:
    y_t = sum_j g_tj r(a_tj) r(W2_e)^T (+ the shared expert likewise), where r rounds
    to IEEE half (act="f16", the kernels' format) or, for comparison, the activation
    to bf16 with W2 as stored (act="bf16")."""
    ra = round_f16 if act == "f16" else round_bf16
    rw = round_f16 if act == "f16" else (lambda w: w)
    T = x64.shape[0]
    y = np.zeros((T, d))
    for e, rows in sorted(_groups(idx, keep).items()):
        w1, w3, w2 = expert64(e)
        a = ra(om.swiglu_hidden(x64[[t for t, _ in rows]], w1, w3))
        out = a @ rw(w2).T
        for (t, j), o in zip(rows, out):
            y[t] += gates64[t, j] * o
    if shared64 is not None:
        y += ra(om.swiglu_hidden(x64, shared64[0], shared64[1])) @ rw(shared64[2]).T
    return y
