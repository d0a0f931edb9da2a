"""Python binding of the MI355X MoE-layer library (libmoe_mi355x.so).

Argument marshalling only: every entry point forwards device pointers (from
torch tensors), sizes and a HIP stream to the C ABI declared in include/moe.h.
All computation happens in the library's HIP kernels; there is no fallback.
If the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16 = 0, 1
GATE_SELECTED, GATE_ALL = 0, 1
(STAGE_ROUTE, STAGE_PERMUTE, STAGE_EXPERT_FFN, STAGE_COMBINE, STAGE_FORWARD,
 STAGE_EXPERT_GATEUP, STAGE_EXPERT_DOWN, STAGE_BACKWARD) = range(8)

EXPORTS = ("moe_status_string", "moe_last_error", "moe_workspace_size", "moe_route",
           "moe_permute", "moe_expert_ffn", "moe_expert_gateup", "moe_expert_down",
           "moe_act_stride", "moe_combine", "moe_forward", "moe_update_bias", "moe_ep_traffic",
           "moe_backward", "moe_forward_noalloc")

NOALLOC_SCRATCH_BYTES = 128 << 20   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("ep_ranks", ctypes.c_int32),
                ("capacity_factor", ctypes.c_double), ("aux_alpha", ctypes.c_float),
                ("reserved2", ctypes.c_float)]


class MoeStats(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("kept", ctypes.c_void_p),
                ("n_dropped", ctypes.c_void_p), ("f", ctypes.c_void_p),
                ("P", ctypes.c_void_p), ("aux", ctypes.c_void_p),
                ("z_loss", ctypes.c_void_p), ("entropy", ctypes.c_void_p),
                ("max_prob", ctypes.c_void_p), ("top_gap", ctypes.c_void_p),
                ("margin", ctypes.c_void_p), ("touched", ctypes.c_void_p),
                ("max_over_mean", ctypes.c_void_p)]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {message}")


_lib = None


def load(path: str = LIB_PATH):
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"MoE HIP library not built: {path} is missing "
                           "(run python -m mixture_experts_layer_31_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    cfgp = ctypes.POINTER(MoeConfig)
    stp = ctypes.POINTER(MoeStats)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_workspace_size": (ctypes.c_int, [cfgp, ctypes.c_int, ctypes.POINTER(sz)]),
        "moe_act_stride": (i32, [cfgp]),
        "moe_route": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, stp, vp, sz, vp]),
        "moe_permute": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, stp, vp, sz, vp]),
        "moe_expert_ffn": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_expert_gateup": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_expert_down": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_combine": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_forward": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       stp, vp, sz, vp]),
        "moe_update_bias": (ctypes.c_int, [cfgp, vp, ctypes.c_float, vp, vp]),
        "moe_ep_traffic": (ctypes.c_int, [cfgp, vp, vp, vp]),
        "moe_backward": (ctypes.c_int, [cfgp] + [vp] * 19 + [sz, vp]),
        "moe_forward_noalloc": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, stp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().moe_status_string(s).decode()


def _check(status: int, where: str):
    if status != OK:
        raise MoEError(status, where, load().moe_last_error().decode())


def _p(t) -> Optional[int]:
    """Device pointer of a tensor (None passes NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(T: int, d: int, E: int, k: int, d_ff: int, *, n_shared: int = 0,
                d_ff_shared: int = 0, gate: str = "selected", dtype: str = "bf16",
                capacity_factor: float = 0.0, aux_alpha: float = 0.0,
                ep_ranks: int = 0) -> MoeConfig:
    return MoeConfig(T=T, d=d, E=E, k=k, d_ff=d_ff, n_shared=n_shared, d_ff_shared=d_ff_shared,
                     gate_mode=GATE_ALL if gate == "all" else GATE_SELECTED,
                     dtype=BF16 if dtype == "bf16" else F32, ep_ranks=int(ep_ranks),
                     capacity_factor=float(capacity_factor), aux_alpha=float(aux_alpha),
                     reserved2=0.0)


def workspace_size(cfg: MoeConfig, stage: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(cfg), stage, ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def act_stride(cfg: MoeConfig) -> int:
    return load().moe_act_stride(ctypes.byref(cfg))


def alloc_workspace(cfg: MoeConfig, stage: int, device="cuda"):
    import torch
    return torch.empty(workspace_size(cfg, stage), dtype=torch.uint8, device=device)


@dataclass
class Stats:
    """Device tensors for moe_stats; build with Stats.alloc(E)."""
    counts: object = None
    kept: object = None
    n_dropped: object = None
    f: object = None
    P: object = None
    aux: object = None
    z_loss: object = None
    entropy: object = None
    max_prob: object = None
    top_gap: object = None
    margin: object = None
    touched: object = None
    max_over_mean: object = None

    @staticmethod
    def alloc(E: int, device="cuda", groups: Optional[int] = None,
              T: Optional[int] = None) -> "Stats":
        """counts/kept hold one entry per row group: E, or ep_ranks*E with the
        expert-parallel layout (pass groups=ep_ranks*E then). margin[T] is
        allocated when T is given."""
        import torch
        z = lambda n, dt: torch.zeros(n, dtype=dt, device=device)
        f1 = lambda: z(1, torch.float32)
        G = groups or E
        return Stats(z(G, torch.int32), z(G, torch.int32), z(1, torch.int32),
                     z(E, torch.float32), z(E, torch.float32), f1(), f1(), f1(), f1(), f1(),
                     z(T, torch.float32) if T is not None else None,
                     z(1, torch.int32), f1())

    def c(self) -> MoeStats:
        return MoeStats(_p(self.counts), _p(self.kept), _p(self.n_dropped), _p(self.f),
                        _p(self.P), _p(self.aux), _p(self.z_loss), _p(self.entropy),
                        _p(self.max_prob), _p(self.top_gap), _p(self.margin),
                        _p(self.touched), _p(self.max_over_mean))


def _stats_ref(stats: Optional[Stats]):
    return ctypes.byref(stats.c()) if stats is not None else None


def _ws(ws):
    return _p(ws), (ws.numel() * ws.element_size() if ws is not None and not isinstance(ws, int) else 0)


def route(cfg, x, w_router, sel_bias, idx, gates, stats: Optional[Stats] = None, ws=None,
          stream=None):
    wp, wb = _ws(ws)
    _check(load().moe_route(ctypes.byref(cfg), _p(x), _p(w_router), _p(sel_bias), _p(idx),
                            _p(gates), _stats_ref(stats), wp, wb, _stream(stream)), "moe_route")


def permute(cfg, idx, x, offsets, dest, src, x_perm=None, stats: Optional[Stats] = None,
            ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load().moe_permute(ctypes.byref(cfg), _p(idx), _p(x), _p(offsets), _p(dest), _p(src),
                              _p(x_perm), _stats_ref(stats), wp, wb, _stream(stream)),
           "moe_permute")


def expert_ffn(cfg, x, src, offsets, w1, w3, w2, ws1, ws3, ws2, y_perm, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load().moe_expert_ffn(ctypes.byref(cfg), _p(x), _p(src), _p(offsets), _p(w1), _p(w3),
                                 _p(w2), _p(ws1), _p(ws3), _p(ws2), _p(y_perm), wp, wb,
                                 _stream(stream)), "moe_expert_ffn")


def expert_gateup(cfg, x, src, offsets, w1, w3, ws1, ws3, act, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load().moe_expert_gateup(ctypes.byref(cfg), _p(x), _p(src), _p(offsets), _p(w1),
                                    _p(w3), _p(ws1), _p(ws3), _p(act), wp, wb, _stream(stream)),
           "moe_expert_gateup")


def expert_down(cfg, act, offsets, w2, ws2, y_perm, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load().moe_expert_down(ctypes.byref(cfg), _p(act), _p(offsets), _p(w2), _p(ws2),
                                  _p(y_perm), wp, wb, _stream(stream)), "moe_expert_down")


def combine(cfg, y_perm, dest, gates, y, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load().moe_combine(ctypes.byref(cfg), _p(y_perm), _p(dest), _p(gates), _p(y), wp, wb,
                              _stream(stream)), "moe_combine")


def update_bias(cfg, counts, gamma: float, bias, stream=None):
    """bias[e] -= gamma above the mean load T*k/E, += gamma below (in place)."""
    _check(load().moe_update_bias(ctypes.byref(cfg), _p(counts), ctypes.c_float(gamma), _p(bias),
                                  _stream(stream)), "moe_update_bias")


def backward(cfg, x, w_router, sel_bias, w1, w3, w2, ws1, ws3, ws2, dy, dx, dw_router, dw1, dw3,
             dw2, dws1=None, dws3=None, dws2=None, ws=None, stream=None):
    """Gradients of <dy, y> + L_aux (recomputes the forward); fp32 outputs."""
    wp, wb = _ws(ws)
    _check(load().moe_backward(ctypes.byref(cfg), _p(x), _p(w_router), _p(sel_bias), _p(w1),
                               _p(w3), _p(w2), _p(ws1), _p(ws3), _p(ws2), _p(dy), _p(dx),
                               _p(dw_router), _p(dw1), _p(dw3), _p(dw2), _p(dws1), _p(dws3),
                               _p(dws2), wp, wb, _stream(stream)), "moe_backward")


def ep_traffic(cfg, offsets, rows, stream=None):
    """rows[s*n + r]: rows source rank s sends to rank r (cfg.ep_ranks = n > 1)."""
    _check(load().moe_ep_traffic(ctypes.byref(cfg), _p(offsets), _p(rows), _stream(stream)),
           "moe_ep_traffic")


def forward(cfg, x, w_router, sel_bias, w1, w3, w2, ws1, ws3, ws2, y, idx=None, gates=None,
            stats: Optional[Stats] = None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load().moe_forward(ctypes.byref(cfg), _p(x), _p(w_router), _p(sel_bias), _p(w1),
                              _p(w3), _p(w2), _p(ws1), _p(ws3), _p(ws2), _p(y), _p(idx),
                              _p(gates), _stats_ref(stats), wp, wb, _stream(stream)),
           "moe_forward")


def forward_noalloc(cfg, x, w_router, sel_bias, w1, w3, w2, ws1, ws3, ws2, y, idx=None,
                    gates=None, stats: Optional[Stats] = None, stream=None):
    """moe_forward with the library's fixed per-GPU scratch instead of a workspace."""
    _check(load().moe_forward_noalloc(ctypes.byref(cfg), _p(x), _p(w_router), _p(sel_bias),
                                      _p(w1), _p(w3), _p(w2), _p(ws1), _p(ws3), _p(ws2), _p(y),
                                      _p(idx), _p(gates), _stats_ref(stats), _stream(stream)),
           "moe_forward_noalloc")
