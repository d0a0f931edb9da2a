"""Seeded parameter draws of the small-layer sweeps (no GPU, no torch): the GPU
parity sweeps and the CPU rounding-model test draw the same layers from here."""
import numpy as np

import workloads as wk


def sweep_cases(n=48, seed=2024):
    """Seeded draws over the layer's parameters (sizes the oracle finishes in seconds)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 8, 16, 40, 64, 96]))
        k = int(rng.integers(1, min(E, 8) + 1))
        kw = dict(T=int(rng.choice([1, 2, 5, 17, 64, 65, 129, 300])),
                  d=int(rng.choice([64, 128, 256])), E=E, k=k,
                  d_ff=int(rng.choice([64, 128, 192])),
                  dtype=wk.BF16 if rng.random() < 0.75 else wk.F32,
                  gate=wk.GATE_ALL if rng.random() < 0.3 else wk.GATE_SELECTED)
        if rng.random() < 0.35:
            kw.update(n_shared=1, d_ff_shared=int(rng.choice([64, 128, 256])))
        if rng.random() < 0.35:
            kw.update(capacity_factor=float(rng.choice([0.5, 1.0, 1.25])), offset_var=1.0)
        if rng.random() < 0.3:
            kw.update(bias_range=0.1)
        cases.append(kw)
    return cases


def sweep_workload(i, kw):
    """Layer i of the forward sweep as a workload (config id 200 + i)."""
    return wk.Workload(f"sweep_{i}", 200 + i, **kw)


def bwd_sweep_cases(n=8, seed=77):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 2, 8, 24, 64]))
        kw = dict(T=int(rng.choice([1, 3, 40, 129, 300])), d=int(rng.choice([256, 512])), E=E,
                  k=int(rng.integers(1, min(E, 8) + 1)), d_ff=int(rng.choice([256, 512])),
                  gate=wk.GATE_ALL if rng.random() < 0.3 else wk.GATE_SELECTED,
                  aux_alpha=0.01 if rng.random() < 0.5 else 0.0)
        if rng.random() < 0.35:
            kw.update(n_shared=1, d_ff_shared=int(rng.choice([256, 512])))
        if rng.random() < 0.35:
            kw.update(capacity_factor=float(rng.choice([0.5, 1.0, 1.25])), offset_var=1.0)
        if rng.random() < 0.3:
            kw.update(bias_range=0.1)
        cases.append(kw)
    return cases
