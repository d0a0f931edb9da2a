"""Seeded synthetic inputs for the five MoE-layer workloads.

This module only draws random numbers and stores them in the formats the layer
takes (fp32, or bf16 kept as raw uint16 bit patterns). It holds none of the
layer's arithmetic: no router scores, no selection, no gates, no expert math.
Both the float64 oracle and the GPU tests/benchmark read their inputs from here,
and nothing else is shared between them.

Recipe (the shapes are the pages' own workloads; no dataset is used):

* Every tensor has its own numpy PCG64 stream, seeded with
  ``SeedSequence([config_id, tensor_id, expert_id, extra])``, so one expert's
  weights can be regenerated on their own (the oracle streams experts).
* Normal draws are float32 ziggurat samples scaled by the standard deviation in
  float32; bf16 tensors are then rounded to nearest-even. Those bits are the
  canonical inputs of both sides.
* ``N(0, v)`` means variance ``v``: weights are ``N(0, 1/fan_in)``.
* "Near-uniform" routing (Mixtral shape): the router has orthonormal rows
  (QR of a Gaussian), so for ``x ~ N(0, I)`` the scores are ``N(0, I_E)`` and
  every k-subset of experts is equally likely.
* Logit offsets (Switch skew, stress skew): a layer without a router bias can
  only be skewed through its input, so a common direction ``c`` with
  ``W_r c = o`` (minimum-norm least squares on the bf16 router) is added to
  every token before rounding.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

# tensor ids for the seed sequence
_X, _ROUTER, _BIAS, _W1, _W3, _W2, _SW1, _SW3, _SW2, _OFFSET = range(1, 11)

BF16 = "bf16"
F32 = "f32"
GATE_SELECTED = "selected"   # softmax over the k selected logits (Mixtral, DeepSeek)
GATE_ALL = "all"             # full-softmax probability of the chosen expert (Switch)


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    gate: str = GATE_SELECTED
    dtype: str = BF16
    n_shared: int = 0
    d_ff_shared: int = 0
    capacity_factor: float = 0.0      # <= 0: no capacity limit
    aux_alpha: float = 0.0
    bias_range: float = 0.0           # b ~ U(-r, r) when r > 0
    router: str = "gaussian"          # "gaussian" (N(0,1/d)) or "orthonormal"
    offsets: Optional[Tuple[float, ...]] = None  # fixed logit offsets o[E]
    offset_var: float = 0.0           # o ~ N(0, offset_var) when > 0

    def with_T(self, T: int, name: Optional[str] = None) -> "Workload":
        from dataclasses import replace
        return replace(self, T=T, name=name or self.name)


def _mk_all():
    w = {}
    w["toy_t64"] = Workload("toy_t64", 1, T=64, d=128, E=4, k=2, d_ff=256, dtype=F32)
    for T in (1, 2, 4, 8, 16, 32, 512, 4096):
        w[f"mixtral_t{T}"] = Workload(f"mixtral_t{T}", 2, T=T, d=4096, E=8, k=2, d_ff=14336,
                                      router="orthonormal")
    for cf in (1.0, 1.25, 2.0):
        w[f"switch_t8192_cf{cf}"] = Workload(
            f"switch_t8192_cf{cf}", 3, T=8192, d=1024, E=64, k=1, d_ff=4096, gate=GATE_ALL,
            capacity_factor=cf, aux_alpha=0.01, offset_var=1.5)
    for T in (1, 64, 4096):
        w[f"deepseek_t{T}"] = Workload(f"deepseek_t{T}", 4, T=T, d=7168, E=256, k=8, d_ff=2048,
                                       n_shared=1, d_ff_shared=2048, bias_range=0.1)
    w["skew_t16384"] = Workload("skew_t16384", 5, T=16384, d=4096, E=8, k=2, d_ff=14336,
                                router="orthonormal",
                                offsets=(8.0, 0.0, 0.0, 0.0, 0.0, 0.0, -8.0, -8.0))
    return w


WORKLOADS = _mk_all()


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ----------------------------------------------------------------- formats

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even), returning the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored tensor (bf16 bits or float32)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _normal(key, shape, var: float) -> np.ndarray:
    a = _rng(*key).standard_normal(shape, dtype=np.float32)
    a *= np.float32(math.sqrt(var))
    return a


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == BF16 else np.ascontiguousarray(a32, dtype=np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------- inputs

@dataclass
class Inputs:
    """Stored inputs of one workload. Expert weights are generated on demand."""
    wl: Workload
    x: np.ndarray            # [T, d]
    w_router: np.ndarray     # [E, d]
    bias: Optional[np.ndarray]  # [E] float32 or None
    _cache: dict = field(default_factory=dict, repr=False)

    # per-expert weights (stored dtype): W1, W3 [d_ff, d]; W2 [d, d_ff]
    def expert(self, e: int):
        wl = self.wl
        cid = wl.config_id
        w1 = _store(_normal((cid, _W1, e), (wl.d_ff, wl.d), 1.0 / wl.d), wl.dtype)
        w3 = _store(_normal((cid, _W3, e), (wl.d_ff, wl.d), 1.0 / wl.d), wl.dtype)
        w2 = _store(_normal((cid, _W2, e), (wl.d, wl.d_ff), 1.0 / wl.d_ff), wl.dtype)
        return w1, w3, w2

    def shared(self, s: int = 0):
        wl = self.wl
        if wl.n_shared == 0:
            return None
        cid, f = wl.config_id, wl.d_ff_shared
        w1 = _store(_normal((cid, _SW1, s), (f, wl.d), 1.0 / wl.d), wl.dtype)
        w3 = _store(_normal((cid, _SW3, s), (f, wl.d), 1.0 / wl.d), wl.dtype)
        w2 = _store(_normal((cid, _SW2, s), (wl.d, f), 1.0 / f), wl.dtype)
        return w1, w3, w2

    def expert_stacks(self, experts=None):
        """All (or the listed) experts' weights as stacks [n, d_ff, d], [n, d_ff, d], [n, d, d_ff],
        generated in parallel threads."""
        wl = self.wl
        ids = list(range(wl.E)) if experts is None else list(experts)
        sdt = np.uint16 if wl.dtype == BF16 else np.float32
        w1 = np.empty((len(ids), wl.d_ff, wl.d), sdt)
        w3 = np.empty((len(ids), wl.d_ff, wl.d), sdt)
        w2 = np.empty((len(ids), wl.d, wl.d_ff), sdt)

        def fill(i):
            a, b, c = self.expert(ids[i])
            w1[i], w3[i], w2[i] = a, b, c

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(ids))))
        return w1, w3, w2


def router_weights(wl: Workload) -> np.ndarray:
    cid = wl.config_id
    if wl.router == "orthonormal":
        g = _rng(cid, _ROUTER, 0).standard_normal((wl.d, wl.E))
        q, _ = np.linalg.qr(g)
        w = q.T.astype(np.float32)
    else:
        w = _normal((cid, _ROUTER, 0), (wl.E, wl.d), 1.0 / wl.d)
    return _store(w, wl.dtype)


def logit_offsets(wl: Workload) -> Optional[np.ndarray]:
    if wl.offsets is not None:
        return np.asarray(wl.offsets, np.float64)
    if wl.offset_var > 0:
        return _rng(wl.config_id, _OFFSET, 0).standard_normal(wl.E) * math.sqrt(wl.offset_var)
    return None


def make_inputs(wl: Workload, T: Optional[int] = None) -> Inputs:
    """Generate the workload's token block, router and bias (experts on demand)."""
    if T is not None and T != wl.T:
        wl = wl.with_T(T)
    cid = wl.config_id
    wr = router_weights(wl)
    x32 = _normal((cid, _X, 0, wl.T), (wl.T, wl.d), 1.0)
    o = logit_offsets(wl)
    if o is not None:
        w64 = to_f64(wr, wl.dtype)
        c = np.linalg.lstsq(w64, o, rcond=None)[0]   # min-norm c with W_r c = o
        x32 += c.astype(np.float32)[None, :]
    bias = None
    if wl.bias_range > 0:
        bias = _rng(cid, _BIAS, 0).uniform(-wl.bias_range, wl.bias_range, wl.E).astype(np.float32)
    return Inputs(wl=wl, x=_store(x32, wl.dtype), w_router=wr, bias=bias)
