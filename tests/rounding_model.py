"""Where the HIP path rounds, modelled on the CPU for bf16 layers (test
infrastructure, not part of the oracle).

The kernels take bf16 x and weights, accumulate both expert products in fp32, and
round the SwiGLU activation a = silu(x W1^T) * (x W3^T) to bf16 before the second
product (the only narrowing on the path; gates, y_perm and y stay fp32). This
module evaluates the layer with exactly that one rounding added to the float64
oracle, and the per-element bound the parity tests hold bf16 layers to:

  |y_gpu - y|  <=  (2^-8 + 2 (d + d_ff) 2^-24) sum_j |g_j| sum_f |a_jf w2_e,if|  (+ shared)

The first term is the activation's rounding: nearest-even to an 8-bit significand
moves each element by at most 2^-8 of itself, so y moves by at most 2^-8 times the
sum of the magnitudes it adds. The second covers the fp32 accumulation of the two
products over d and d_ff terms, (d + d_ff) 2^-24 of the same magnitudes, doubled:
the first product's error reaches y through silu and the branch product with a
factor below 2. The gates and the combine (fp32, at most k + 1 terms) add rounding
far below either term.
"""
from __future__ import annotations

import numpy as np

import workloads as wk
from oracle import moe as om

U_BF16 = 2.0 ** -8    # unit roundoff of bf16 (8-bit significand, nearest-even)
U_F32 = 2.0 ** -24


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 (nearest-even), widened back to float64."""
    return wk.bf16_bits_to_f32(wk.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


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
    for e, rows in sorted(_groups(idx, keep).items()):
        w1, w3, w2 = expert64(e)
        a = np.abs(om.swiglu_hidden(x64[[t for t, _ in rows]], w1, w3))
        out = a @ np.abs(w2).T
        for (t, j), o in zip(rows, out):
            mag[t] += abs(gates64[t, j]) * o
    dff = d_ff
    if shared64 is not None:
        mag += np.abs(om.swiglu_hidden(x64, shared64[0], shared64[1])) @ np.abs(shared64[2]).T
        dff = max(dff, d_ff_shared)
    return (U_BF16 + 2.0 * (d + dff) * U_F32) * mag


def y_rounded_activation(d, x64, idx, gates64, keep, expert64, shared64=None):
    """The layer with the activation rounded to bf16 before the second product, all
    else in float64: y_t = sum_j g_tj bf16(a_tj) W2_e^T (+ bf16(a_shared) Ws2^T)."""
    T = x64.shape[0]
    y = np.zeros((T, d))
    for e, rows in sorted(_groups(idx, keep).items()):
        w1, w3, w2 = expert64(e)
        a = round_bf16(om.swiglu_hidden(x64[[t for t, _ in rows]], w1, w3))
        out = a @ w2.T
        for (t, j), o in zip(rows, out):
            y[t] += gates64[t, j] * o
    if shared64 is not None:
        y += round_bf16(om.swiglu_hidden(x64, shared64[0], shared64[1])) @ shared64[2].T
    return y
