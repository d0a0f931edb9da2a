"""Shared helpers of the GPU parity tests: upload seeded workloads, run the HIP
library through its binding, and evaluate the float64 oracle on the same inputs.
The oracle never receives a value produced by the GPU except the GPU's own
routing indices, when a test evaluates the oracle *under that routing*
(the conditional check of a selection that near-ties can flip)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import mixture_experts_layer_31_amd as moe
import workloads as wk
from oracle import moe as om
from rounding_model import y_bound

NEAR_TIE = 1e-3          # tokens whose k-th/(k+1)-th score margin is below this are flagged
Y_TOL_F32 = 1e-5         # max|dy| <= 1e-5 * rms(y) for fp32 inputs
Y_TOL_BF16 = 2e-2        # max|dy| / rms(y) <= 2e-2 for bf16 inputs, fp32 accumulation
GATE_TOL = 1e-6          # max|dg|, gates computed in fp32 from fp32-accumulated logits


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == wk.BF16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    return t.to(dev())


class Weights:
    """A workload's expert weights on the GPU plus the host copies the oracle reads."""

    def __init__(self, wl: wk.Workload):
        t0 = time.time()
        self.wl = wl
        inp = wk.make_inputs(wl, T=1)
        self.host = inp.expert_stacks()
        self.w1, self.w3, self.w2 = (to_dev(a, wl.dtype) for a in self.host)
        sh = inp.shared()
        self.host_shared = sh
        self.s1 = self.s3 = self.s2 = None
        if sh is not None:
            self.s1, self.s3, self.s2 = (to_dev(a, wl.dtype) for a in sh)
        self.wr_host = inp.w_router
        self.wr = to_dev(inp.w_router, wl.dtype)
        self.bias_host = inp.bias
        self.bias = torch.from_numpy(inp.bias).to(dev()) if inp.bias is not None else None
        self._cache = {}
        log(f"[weights] {wl.name}: generated and uploaded in {time.time() - t0:.1f}s")

    def expert64(self, e: int):
        if e not in self._cache:
            if len(self._cache) >= 4:
                self._cache.pop(next(iter(self._cache)))
            self._cache[e] = tuple(wk.to_f64(a[e], self.wl.dtype) for a in self.host)
        return self._cache[e]

    def shared64(self):
        if self.host_shared is None:
            return None
        return tuple(wk.to_f64(a, self.wl.dtype) for a in self.host_shared)


def config_of(wl: wk.Workload, T: int) -> moe.MoeConfig:
    return moe.make_config(T, wl.d, wl.E, wl.k, wl.d_ff, n_shared=wl.n_shared,
                           d_ff_shared=wl.d_ff_shared, gate=wl.gate, dtype=wl.dtype,
                           capacity_factor=wl.capacity_factor, aux_alpha=wl.aux_alpha)


def run_forward(wl: wk.Workload, W: Weights, x_host: np.ndarray, T: int, bias="default",
                ep: int = 0, stats: str = "full"):
    """Fused moe_forward; returns numpy copies of y, idx, gates and the stats.
    stats="counts" asks only for what the index writes (expert counts, kept rows, drops,
    touched experts, busiest load over the mean); "none" for no
    statistics (the keys of what was not asked for are absent)."""
    cfg = config_of(wl, T)
    cfg.ep_ranks = ep
    x = to_dev(x_host, wl.dtype)
    y = torch.full((T, wl.d), float("nan"), dtype=torch.float32, device=dev())
    idx = torch.full((T, wl.k), -7, dtype=torch.int32, device=dev())
    gates = torch.full((T, wl.k), float("nan"), dtype=torch.float32, device=dev())
    st = moe.Stats.alloc(wl.E, groups=wl.E * (ep if ep > 1 else 1))
    ws = moe.alloc_workspace(cfg, moe.STAGE_FORWARD)
    b = W.bias if bias == "default" else bias
    if stats == "counts":
        st = moe.Stats(st.counts, st.kept, st.n_dropped, touched=st.touched,
                       max_over_mean=st.max_over_mean)
    elif stats == "none":
        st = None
    moe.forward(cfg, x, W.wr, b, W.w1, W.w3, W.w2, W.s1, W.s3, W.s2, y, idx, gates, st, ws)
    torch.cuda.synchronize()
    if st is None:
        return dict(y=y.cpu().numpy(), idx=idx.cpu().numpy().astype(np.int64),
                    gates=gates.cpu().numpy())
    if stats == "counts":
        return dict(y=y.cpu().numpy(), idx=idx.cpu().numpy().astype(np.int64),
                    gates=gates.cpu().numpy(), counts=st.counts.cpu().numpy(),
                    kept=st.kept.cpu().numpy(), n_dropped=int(st.n_dropped.cpu()[0]),
                    touched=int(st.touched.cpu()[0]),
                    max_over_mean=float(st.max_over_mean.cpu()[0]))
    return dict(y=y.cpu().numpy(), idx=idx.cpu().numpy().astype(np.int64),
                gates=gates.cpu().numpy(), counts=st.counts.cpu().numpy(),
                kept=st.kept.cpu().numpy(), n_dropped=int(st.n_dropped.cpu()[0]),
                touched=int(st.touched.cpu()[0]),
                max_over_mean=float(st.max_over_mean.cpu()[0]),
                f=st.f.cpu().numpy(), P=st.P.cpu().numpy(), aux=float(st.aux.cpu()[0]),
                z_loss=float(st.z_loss.cpu()[0]), entropy=float(st.entropy.cpu()[0]),
                max_prob=float(st.max_prob.cpu()[0]), top_gap=float(st.top_gap.cpu()[0]))


def run_staged(wl: wk.Workload, W: Weights, x_host: np.ndarray, T: int, ep: int = 0,
               keep_perm: bool = True):
    """route -> permute -> expert_ffn -> combine through the staged entry points; ep > 1
    lays the rows out as ep simulated expert-parallel ranks (and returns the send-row
    matrix as "traffic"). keep_perm=False skips the gathered rows x_perm (permute with
    no gather) and does not copy y_perm back (full-size layers)."""
    cfg = config_of(wl, T)
    cfg.ep_ranks = ep
    G = wl.E * (ep if ep > 1 else 1)
    x = to_dev(x_host, wl.dtype)
    R = T * wl.k
    idx = torch.empty((T, wl.k), dtype=torch.int32, device=dev())
    gates = torch.empty((T, wl.k), dtype=torch.float32, device=dev())
    offsets = torch.empty(G + 1, dtype=torch.int32, device=dev())
    dest = torch.empty((T, wl.k), dtype=torch.int32, device=dev())
    src = torch.empty(R, dtype=torch.int32, device=dev())
    rows = R + wl.n_shared * T
    y_perm = torch.zeros((rows, wl.d), dtype=torch.float32, device=dev())
    y = torch.empty((T, wl.d), dtype=torch.float32, device=dev())
    x_perm = torch.zeros((R, wl.d), dtype=x.dtype, device=dev()) if keep_perm else None
    st = moe.Stats.alloc(wl.E, groups=G)
    moe.route(cfg, x, W.wr, W.bias, idx, gates, st, moe.alloc_workspace(cfg, moe.STAGE_ROUTE))
    moe.permute(cfg, idx, x, offsets, dest, src, x_perm, st,
                moe.alloc_workspace(cfg, moe.STAGE_PERMUTE))
    moe.expert_ffn(cfg, x, src, offsets, W.w1, W.w3, W.w2, W.s1, W.s3, W.s2, y_perm,
                   moe.alloc_workspace(cfg, moe.STAGE_EXPERT_FFN))
    moe.combine(cfg, y_perm, dest, gates, y, moe.alloc_workspace(cfg, moe.STAGE_COMBINE))
    traffic = None
    if ep > 1:
        traffic = torch.full((ep * ep,), -1, dtype=torch.int32, device=dev())
        moe.ep_traffic(cfg, offsets, traffic)
    torch.cuda.synchronize()
    out = dict(y=y.cpu().numpy(), idx=idx.cpu().numpy().astype(np.int64), gates=gates.cpu().numpy(),
               offsets=offsets.cpu().numpy(), dest=dest.cpu().numpy(), src=src.cpu().numpy(),
               counts=st.counts.cpu().numpy(), kept=st.kept.cpu().numpy(),
               n_dropped=int(st.n_dropped.cpu()[0]), touched=int(st.touched.cpu()[0]),
               max_over_mean=float(st.max_over_mean.cpu()[0]),
               traffic=None if traffic is None else traffic.cpu().numpy().reshape(ep, ep))
    if not keep_perm:
        return out
    out["y_perm"] = y_perm.cpu().numpy()
    if wl.dtype == wk.BF16:
        out["x_perm"] = x_perm.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        out["x_perm"] = x_perm.cpu().numpy()
    return out


def oracle_route(wl: wk.Workload, W: Weights, x_host: np.ndarray):
    x64 = wk.to_f64(x_host, wl.dtype)
    wr64 = wk.to_f64(W.wr_host, wl.dtype)
    return om.route(x64, wr64, wl.k, wl.gate, W.bias_host), x64


def check_routing(wl, gpu_idx, r):
    """Selected sets equal on every token whose k-th/(k+1)-th margin is >= 1e-3; rank order
    equal where all adjacent top-k gaps are >= 1e-3 too. Returns the flagged mask."""
    flagged = r["margin"] < NEAR_TIE
    ok = ~flagged
    gs, os_ = np.sort(gpu_idx, 1), np.sort(r["idx"], 1)
    bad = np.nonzero((gs != os_).any(1) & ok)[0]
    assert bad.size == 0, f"{bad.size} unflagged tokens route differently, e.g. {bad[:5]}"
    if wl.k > 1:
        sel = np.take_along_axis(r["s"], r["idx"], 1)
        ordered = ok & (-np.diff(sel, axis=1) >= NEAR_TIE).all(1)
    else:
        ordered = ok
    assert (gpu_idx[ordered] == r["idx"][ordered]).all(), "rank order differs"
    return flagged


def check_gates(wl, gpu_idx, gpu_gates, z64):
    g64 = (om.gates_selected(z64, gpu_idx) if wl.gate == wk.GATE_SELECTED
           else om.gates_all(z64, gpu_idx))
    err = float(np.max(np.abs(gpu_gates - g64))) if g64.size else 0.0
    assert err <= GATE_TOL, f"gate error {err:.3g} > {GATE_TOL}"
    return g64, err


def check_load_summary(gpu, gpu_idx, E, counts, kept):
    """touched (experts keeping an assignment) exact; the busiest expert's load over the
    mean to fp32 rounding (the GPU divides in double and rounds once to float)."""
    T, k = gpu_idx.shape
    assert gpu["touched"] == int(np.count_nonzero(kept)), "touched"
    ref = om.max_over_mean_load(counts, T, k)
    assert abs(gpu["max_over_mean"] - ref) <= 2.0 ** -23 * ref, ("max_over_mean",
                                                                  gpu["max_over_mean"], ref)


def check_permutation(wl, T, gpu, gpu_idx):
    """Bit-exact against the oracle's histogram/capacity/permutation run on the GPU's idx."""
    p = om.assign_rows(gpu_idx, wl.E, wl.capacity_factor)
    assert np.array_equal(gpu["counts"], p["counts"]), "counts"
    assert np.array_equal(gpu["kept"], p["kept"]), "kept"
    assert gpu["n_dropped"] == p["n_dropped"], "n_dropped"
    if "touched" in gpu:
        check_load_summary(gpu, gpu_idx, wl.E, p["counts"], p["kept"])
    if "offsets" in gpu:
        assert np.array_equal(gpu["offsets"], p["offsets"]), "offsets"
        assert np.array_equal(gpu["dest"], p["dest"]), "dest"
        R = int(p["offsets"][-1])
        assert np.array_equal(gpu["src"][:R], p["src"]), "src"
    return p


def y_rounding_bound(wl, W: Weights, x64, idx, gates64, keep):
    """Per-element bound on |y_gpu - y| for bf16 layers from the kernels' rounding points
    (rounding_model.y_bound: the activation's bf16 rounding before the second product
    plus the fp32 accumulation of both products), [T, d]."""
    return y_bound(wl.d, wl.d_ff, x64, idx, gates64, keep, W.expert64, W.shared64(),
                   wl.d_ff_shared)


def check_y(wl, y_gpu, y_ref, what=""):
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.max(np.abs(y_gpu - y_ref)))
    tol = Y_TOL_F32 if wl.dtype == wk.F32 else Y_TOL_BF16
    assert np.isfinite(y_gpu).all(), "non-finite output"
    assert err <= tol * rms, f"{what} max|dy| = {err:.3g} > {tol} * rms {rms:.3g}"
    return err / rms


def oracle_y_sampled(wl, W: Weights, x64, tokens, idx, gates64, keep):
    """y for the sampled tokens straight from y = sum_j g_j f_j(x) (+ shared), one expert at
    a time (each expert's float64 weights are built once)."""
    tokens = np.asarray(tokens)
    y = np.zeros((len(tokens), wl.d))
    need = {}
    for i, t in enumerate(tokens):
        for j in range(wl.k):
            if keep[t, j]:
                need.setdefault(int(idx[t, j]), []).append((i, t, j))
    for e in sorted(need):
        w = W.expert64(e)
        rows = need[e]
        X = x64[[t for _, t, _ in rows]]
        out = om.swiglu(X, *w)
        for (i, t, j), o in zip(rows, out):
            y[i] += gates64[t, j] * o
    sh = W.shared64()
    if sh is not None:
        y += om.swiglu(x64[tokens], *sh)
    return y
