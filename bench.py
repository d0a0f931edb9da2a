#!/usr/bin/env python3
"""Throughput of the MoE-layer forward pass on one MI355X.

A step is one pass of the whole layer over one batch of synthetic tokens:
route -> permute -> grouped gate/up (+SwiGLU) -> grouped down -> combine, one
moe_forward call through the library's C ABI, with inputs and weights resident
in HBM. The default workload is the Mixtral-shaped layer at T = 4096 tokens.

Prints ONE JSON line (rank 0). Besides the step throughput it reports the
same steps run as the five staged entry points (moe_route, moe_permute,
moe_expert_gateup, moe_expert_down, moe_combine), the roofline of the dominant
kernel (the grouped gate/up GEMM), timed with HIP events recorded on the
library's stream around moe_expert_gateup in every staged step, the float64
CPU oracle timed on a bounded sample of the workload, and
the ceilings this device reaches on both rooflines (an MFMA loop and a
streaming read). Steps of HBM-bound workloads start from cold caches (a 1 GiB
read between steps, outside the timed step).

After the headline workload the same line carries "configs": the fused step of
the other workloads of the metric (Mixtral-shaped decode at 1, 8 and 32 tokens and
prefill at 512, DeepSeek-shaped at 1, 64 and 4096 tokens, the skewed 16384-token
load and the Switch layer at three capacity factors, with its balance loss), each
with tokens/s, TFLOP/s, GB/s and the fractions of both rooflines; and "coverage":
the expert coverage of decode batches under the GPU's routing against 1 - 0.75^B.
The headline workload's moe_backward (the layer's gradients on the same batch) is
timed too and reported as "backward" (--no-backward leaves it out).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--ep N]
                  [--no-backward] [--no-flush] [--no-calibration] [--configs A,B,...]
  python bench.py --calibrate-copy     # plain 1 GiB copies, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "MoE-layer tokens/s at 1 GPU + % MFMA peak (prefill) / % HBM BW (decode)"
# sources of the prefill gate/up kernel: its part of gemm_bf16.hip (the one-wave-per-
# SIMD kernel, its launcher and the gate/up dispatch) and the headers with its tile
# order and helpers; the committed counter summary is used only while their hash matches
_CSRC = os.path.join(ROOT, "mixture_experts_layer_31_amd", "csrc")
GEMM_SOURCE_PARTS = [
    ("gemm_bf16.hip", "// ---------------------------------------------------------------- large tiles, one wave per SIMD",
     "// ---------------------------------------------------------------- decode tiles"),
    ("gemm_bf16.hip", "// One wave per SIMD, 256 x 256 weight-row tiles", "hipError_t launch_gemm_gateup_bf16_with_shared("),
    ("gemm_common.h", None, None),
    ("common.h", None, None),
]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemm_gateup_mixtral_t4096_counters.md")
CALIB_LIB = os.path.join(ROOT, "mixture_experts_layer_31_amd", "libmoe_calibrate.so")
# the rest of the metric, timed after the headline workload: the decode rows (HBM),
# the other prefill shapes, and the Switch layer with its balance loss
CONFIG_SWEEP = ("mixtral_t1", "mixtral_t8", "mixtral_t32", "mixtral_t512", "deepseek_t1",
                "deepseek_t64", "deepseek_t4096", "skew_t16384", "switch_t8192_cf1.0",
                "switch_t8192_cf1.25", "switch_t8192_cf2.0")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_t4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="tokens in the CPU-oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--ep", type=int, default=0,
                    help="lay the rows out as N simulated expert-parallel ranks and report "
                         "the dispatch volume per rank")
    ap.add_argument("--no-flush", action="store_true",
                    help="HBM-bound workloads: time steps back to back (warm MALL/L2)")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_backward on the same batch (the default)")
    ap.add_argument("--no-backward", action="store_true",
                    help="leave out the timing of moe_backward")
    ap.add_argument("--configs", default=",".join(CONFIG_SWEEP),
                    help="comma-separated workloads timed after the headline one (their "
                         "fused steps, from cold caches where HBM-bound); empty for none")
    ap.add_argument("--config-steps", type=int, default=20)
    return ap.parse_args()


def calibrate_copy():
    """A plain elementwise kernel of known traffic (reads 1 GiB, writes 1 GiB, five
    launches), so that rocprofv3's FETCH_SIZE / WRITE_SIZE can be scaled to bytes."""
    import torch
    n = 1 << 28                      # 2^28 fp32 = 1 GiB
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty(n, dtype=torch.float32, device="cuda")
    for _ in range(5):
        torch.add(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise add", "bytes_read": 4 * n,
                      "bytes_written": 4 * n, "launches": 5}))


def device_ceilings():
    """What this device reaches on the two rooflines, beside the nominal peaks: a
    dense MFMA loop (v_mfma_f32_32x32x16_bf16 on pseudo-random register operands, 2048
    workgroups of 4 waves) and a streaming read of 2 GiB (8x the MALL), with the
    kernels of libmoe_calibrate.so; the best of 3 timed launches each."""
    import ctypes
    import torch
    if not os.path.exists(CALIB_LIB):
        raise RuntimeError(f"{CALIB_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(CALIB_LIB)
    lib.moe_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.moe_calib_mfma_flops.restype = ctypes.c_double
    lib.moe_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best_ms(launch):
        if launch() != 0:
            raise RuntimeError("calibration kernel launch failed")
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    blocks, iters = 2048, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ms = best_ms(lambda: lib.moe_calib_mfma(blocks, iters, ctypes.c_void_p(out.data_ptr()), sp))
    tflops = lib.moe_calib_mfma_flops(blocks, iters) / (ms * 1e-3) / 1e12
    buf = torch.ones(1 << 29, dtype=torch.float32, device="cuda")     # 2 GiB
    rblocks = 4096
    outr = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda")
    ms = best_ms(lambda: lib.moe_calib_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 4,
                                            rblocks, ctypes.c_void_p(outr.data_ptr()), sp))
    gbps = buf.numel() * 4 / (ms * 1e-3) / 1e9
    del buf, out, outr
    torch.cuda.empty_cache()
    return {"mfma_loop_tflops": round(tflops, 1), "mfma_loop_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "hbm_read_gbps": round(gbps, 1), "hbm_read_frac": round(gbps / PEAK_HBM_GBPS, 4)}


def kernel_source_hash():
    h = hashlib.sha256()
    for name, start, end in GEMM_SOURCE_PARTS:
        with open(os.path.join(_CSRC, name), encoding="utf-8") as f:
            text = f.read()
        if start is not None:
            a = text.index(start)
            text = text[a:text.index(end, a)]
        h.update(text.encode("utf-8"))
    return h.hexdigest()[:16]


def counters_traffic(workload):
    """HBM bytes per launch of the gate/up kernel from the committed counter summary, or
    None if there is none for this workload or the kernel source changed since."""
    if workload != "mixtral_t4096" or not os.path.exists(COUNTERS_FILE):
        return None
    txt = open(COUNTERS_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    f = re.search(r"fetch_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    w = re.search(r"write_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m and f and w) or m.group(1) != kernel_source_hash():
        return None
    return float(f.group(1)) + float(w.group(1))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the layer runs on a single GPU here, and there is "
              "no multi-GPU path to time (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import numpy as np
    import torch

    import mixture_experts_layer_31_amd as moe
    import workloads as wk

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    moe.load()
    calib = None if args.no_calibration else device_ceilings()
    wl = wk.get(args.workload)
    T = wl.T
    t0 = time.time()
    inp = wk.make_inputs(wl)
    host = inp.expert_stacks()
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        if wl.dtype == wk.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x = up(inp.x)
    wr = up(inp.w_router)
    w1, w3, w2 = (up(a) for a in host)
    sh = inp.shared()
    s1 = s3 = s2 = None
    if sh is not None:
        s1, s3, s2 = (up(a) for a in sh)
    bias = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
    if args.no_cpu_baseline:
        del host
    log(f"[bench] {wl.name}: inputs generated and uploaded in {time.time() - t0:.1f}s")

    cfg = moe.make_config(T, wl.d, wl.E, wl.k, wl.d_ff, n_shared=wl.n_shared,
                          d_ff_shared=wl.d_ff_shared, gate=wl.gate, dtype=wl.dtype,
                          capacity_factor=wl.capacity_factor, aux_alpha=wl.aux_alpha,
                          ep_ranks=args.ep)
    G = wl.E * (args.ep if args.ep > 1 else 1)
    R = T * wl.k
    rows = R + wl.n_shared * T
    i32 = torch.int32
    idx = torch.empty((T, wl.k), dtype=i32, device=dev)
    gates = torch.empty((T, wl.k), dtype=torch.float32, device=dev)
    offsets = torch.empty(G + 1, dtype=i32, device=dev)
    dest = torch.empty((T, wl.k), dtype=i32, device=dev)
    src = torch.empty(R, dtype=i32, device=dev)
    # the SwiGLU activation between the two entry points: IEEE half for bf16 layers
    act = torch.empty((rows, moe.act_stride(cfg)),
                      dtype=torch.float16 if wl.dtype == wk.BF16 else torch.float32, device=dev)
    y_perm = torch.empty((rows, wl.d), dtype=torch.float32, device=dev)
    y = torch.empty((T, wl.d), dtype=torch.float32, device=dev)
    ws_r = moe.alloc_workspace(cfg, moe.STAGE_ROUTE)
    ws_p = moe.alloc_workspace(cfg, moe.STAGE_PERMUTE)
    ws_g = moe.alloc_workspace(cfg, moe.STAGE_EXPERT_GATEUP)
    ws_d = moe.alloc_workspace(cfg, moe.STAGE_EXPERT_DOWN)
    ws_f = moe.alloc_workspace(cfg, moe.STAGE_FORWARD)
    stream = torch.cuda.current_stream()

    def step(ev_a=None, ev_b=None, stats=None):
        moe.route(cfg, x, wr, bias, idx, gates, stats, ws_r, stream)
        moe.permute(cfg, idx, x, offsets, dest, src, None, stats, ws_p, stream)
        if ev_a is not None:
            ev_a.record(stream)
        moe.expert_gateup(cfg, x, src, offsets, w1, w3, s1, s3, act, ws_g, stream)
        if ev_b is not None:
            ev_b.record(stream)
        moe.expert_down(cfg, act, offsets, w2, s2, y_perm, ws_d, stream)
        moe.combine(cfg, y_perm, dest, gates, y, None, stream)

    # routing statistics of this batch (outside the timed region)
    st = moe.Stats.alloc(wl.E, groups=G)
    step(stats=st)
    torch.cuda.synchronize()
    kept = st.kept.cpu().numpy().astype(np.int64)
    R_kept = int(kept.sum())
    touched = int((kept > 0).sum())

    # algorithmic work, from this batch's routing
    elt = 2 if wl.dtype == wk.BF16 else 4
    d, dff, dffs, nsh = wl.d, wl.d_ff, wl.d_ff_shared, wl.n_shared
    F_step = 2.0 * T * d * wl.E + 6.0 * d * dff * R_kept + 6.0 * d * dffs * T * nsh
    B_step = (touched * 3.0 * d * dff * elt + nsh * 3.0 * d * dffs * elt + wl.E * d * elt
              + T * d * elt + T * d * 4.0)
    peak_f = PEAK_BF16_TFLOPS if wl.dtype == wk.BF16 else PEAK_F32_TFLOPS
    step_bound = "mfma" if F_step / (peak_f * 1e12) >= B_step / (PEAK_HBM_GBPS * 1e9) else "hbm"
    # HBM-bound steps start from cold caches: reading 1 GiB between steps evicts the
    # 256 MB MALL and the L2 (with clean lines: a write would leave dirty ones for
    # the step to write back), outside the timed step
    flush = step_bound == "hbm" and not args.no_flush
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev) if flush else None
    sink = torch.zeros((), dtype=torch.float32, device=dev) if flush else None

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        if flush:
            torch.sum(scratch, dim=0, out=sink)
        sev[i][0].record(stream)
        step(*evs[i])
        sev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    staged_ms_each = np.array([a.elapsed_time(b) for a, b in sev])
    # back to back, the span over the K steps; with flushes, the steps' own times
    staged_ms = float(staged_ms_each.mean()) if flush else start.elapsed_time(stop) / K
    gemm_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # the layer's own entry point, moe_forward (all six stages in one call), on the
    # same batch: K steps timed the same way (cold caches for HBM-bound workloads);
    # this is the step the headline value measures
    def fused():
        moe.forward(cfg, x, wr, bias, w1, w3, w2, s1, s3, s2, y, None, None, None, ws_f, stream)

    for _ in range(max(2, args.warmup)):
        fused()
    torch.cuda.synchronize()
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    w1t = time.perf_counter()
    f0.record(stream)
    for i in range(K):
        if flush:
            torch.sum(scratch, dim=0, out=sink)
        fev[i][0].record(stream)
        fused()
        fev[i][1].record(stream)
    f1.record(stream)
    torch.cuda.synchronize()
    wall += time.perf_counter() - w1t
    step_ms = np.array([a.elapsed_time(b) for a, b in fev])
    ms_step = float(step_ms.mean()) if flush else f0.elapsed_time(f1) / K
    del scratch, sink

    F_g = 4.0 * d * dff * R_kept + 4.0 * d * dffs * T * nsh
    B_g = (touched * 2.0 * d * dff * elt + nsh * 2.0 * d * dffs * elt + T * d * elt
           + (R_kept * dff + nsh * T * dffs) * elt)
    g_bound = "mfma" if F_g / (peak_f * 1e12) >= B_g / (PEAK_HBM_GBPS * 1e9) else "hbm"
    if g_bound == "mfma":
        achieved = F_g / (gemm_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=peak_f, unit="TFLOP/s",
                    frac=round(achieved / peak_f, 4))
    else:
        achieved = B_g / (gemm_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBPS, 4))
    tr = counters_traffic(wl.name)
    roof["traffic"] = tr
    roof["kernel"] = "moe_expert_gateup: grouped gate/up GEMM + SwiGLU"
    roof["kernel_ms"] = round(gemm_ms, 4)
    roof["algorithmic_bytes"] = B_g
    roof["algorithmic_flops"] = F_g

    step_tflops = F_step / (ms_step * 1e-3) / 1e12
    step_gbps = B_step / (ms_step * 1e-3) / 1e9

    ep_report = None
    if args.ep > 1:
        # dispatch volume of this batch in the simulated layout (the combine returns the same)
        n = args.ep
        rows = torch.empty(n * n, dtype=i32, device=dev)
        moe.ep_traffic(cfg, offsets, rows, stream)
        torch.cuda.synchronize()
        rows = rows.cpu().numpy().astype(np.int64).reshape(n, n)
        row_bytes = d * elt
        sent = (rows.sum(axis=1) - np.diag(rows)) * row_bytes
        ep_report = {"ranks": n, "max_send_bytes": int(sent.max()),
                     "mean_send_bytes": float(sent.mean()),
                     "formula_bytes": (T // n) * wl.k * (1.0 - 1.0 / n) * row_bytes,
                     "rows_per_rank_min": int(rows.sum(axis=0).min()),
                     "rows_per_rank_max": int(rows.sum(axis=0).max())}

    bwd_report = None
    # moe_backward takes bf16 layers with d, d_ff and d_ff_shared multiples of 256
    bwd_ok = (wl.dtype == "bf16" and wl.d % 256 == 0 and wl.d_ff % 256 == 0
              and wl.d_ff_shared % 256 == 0)
    if not args.no_backward and args.ep <= 1 and bwd_ok:
        bwd_report = time_backward(args, cfg, wl, x, wr, bias, (w1, w3, w2), (s1, s3, s2),
                                   R_kept, stream, peak_f)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, host, args.cpu_sample)

    configs, coverage = None, None
    names = [n for n in args.configs.split(",") if n]
    if names and args.ep <= 1:
        del x, w1, w3, w2, s1, s3, s2, y, y_perm, act, ws_f, ws_r, ws_p, ws_g, ws_d
        if not args.no_cpu_baseline:
            del host
        torch.cuda.empty_cache()
        configs, coverage = config_sweep(names, args.config_steps, args.no_flush)

    out = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "d": d, "E": wl.E, "k": wl.k, "d_ff": dff,
                   "n_shared": nsh, "d_ff_shared": dffs, "gate": wl.gate,
                   "capacity_factor": wl.capacity_factor, "kept_rows": R_kept,
                   "touched_experts": touched, "parallelism": "single GPU"},
        "step": {"tflops": round(step_tflops, 2), "gbps": round(step_gbps, 1),
                 "bound": step_bound,
                 "frac_mfma": round(step_tflops / peak_f, 4),
                 "frac_hbm": round(step_gbps / PEAK_HBM_GBPS, 4),
                 "entry_point": "moe_forward",
                 "staged_ms": round(staged_ms, 4),
                 "step_ms_median": round(float(np.median(step_ms)), 4),
                 "step_ms_min": round(float(step_ms.min()), 4),
                 "step_ms_max": round(float(step_ms.max()), 4),
                 "cold_caches": flush,
                 "wall_s": round(wall, 4)},
        "calibration": calib,
        "roofline": roof,
        "cpu_baseline": cpu,
        "expert_parallel": ep_report,
        "backward": bwd_report,
        "configs": configs,
        "coverage": coverage,
    }
    print(json.dumps(out), flush=True)


def config_sweep(names, K, no_flush):
    """The fused step (one moe_forward) of each named workload, K timed steps after 3
    warm-ups (mean, median, minimum and maximum reported); HBM-bound workloads from cold caches (a 1 GiB read before each step,
    outside its timing). Work and bytes are counted from each batch's own routing as
    for the headline. Workloads of one shape share their uploaded weights. Also the
    GPU-routing coverage of decode batches at the Mixtral shape (CME295 notes §2.3)."""
    import numpy as np
    import torch
    import mixture_experts_layer_31_amd as moe
    import workloads as wk

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    shape = None
    W = None
    out = []
    coverage = None

    def up(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == wk.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    for name in names:
        wl = wk.get(name)
        key = (wl.config_id, wl.d, wl.E, wl.d_ff, wl.n_shared)
        t0 = time.time()
        if key != shape:
            W = None
            torch.cuda.empty_cache()
            inp = wk.make_inputs(wl)
            W = {"w": tuple(up(a, wl.dtype) for a in inp.expert_stacks())}
            sh = inp.shared()
            W["s"] = tuple(up(a, wl.dtype) for a in sh) if sh is not None else (None,) * 3
            W["wr"] = up(inp.w_router, wl.dtype)
            W["bias"] = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
            shape = key
        else:
            inp = wk.make_inputs(wl)
        T = wl.T
        x = up(inp.x, wl.dtype)
        cfg = moe.make_config(T, wl.d, wl.E, wl.k, wl.d_ff, n_shared=wl.n_shared,
                              d_ff_shared=wl.d_ff_shared, gate=wl.gate, dtype=wl.dtype,
                              capacity_factor=wl.capacity_factor, aux_alpha=wl.aux_alpha)
        y = torch.empty((T, wl.d), dtype=torch.float32, device=dev)
        ws = moe.alloc_workspace(cfg, moe.STAGE_FORWARD)
        st = moe.Stats.alloc(wl.E)

        def fused(stats=None):
            moe.forward(cfg, x, W["wr"], W["bias"], *W["w"], *W["s"], y, None, None, stats, ws,
                        stream)

        fused(st)
        torch.cuda.synchronize()
        kept = st.kept.cpu().numpy().astype(np.int64)
        R_kept, touched = int(kept.sum()), int((kept > 0).sum())
        elt = 2 if wl.dtype == wk.BF16 else 4
        d, dff, dffs, nsh = wl.d, wl.d_ff, wl.d_ff_shared, wl.n_shared
        F = 2.0 * T * d * wl.E + 6.0 * d * dff * R_kept + 6.0 * d * dffs * T * nsh
        B = (touched * 3.0 * d * dff * elt + nsh * 3.0 * d * dffs * elt + wl.E * d * elt
             + T * d * elt + T * d * 4.0)
        peak_f = PEAK_BF16_TFLOPS if wl.dtype == wk.BF16 else PEAK_F32_TFLOPS
        bound = "mfma" if F / (peak_f * 1e12) >= B / (PEAK_HBM_GBPS * 1e9) else "hbm"
        flush = bound == "hbm" and not no_flush
        for _ in range(3):
            fused()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        for i in range(K):
            if flush:
                torch.sum(scratch, dim=0, out=sink)
            evs[i][0].record(stream)
            fused()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        ms_all = np.array([a.elapsed_time(b) for a, b in evs])
        ms = float(ms_all.mean())
        tf = F / (ms * 1e-3) / 1e12
        gb = B / (ms * 1e-3) / 1e9
        rec = {"workload": name, "T": T, "ms": round(ms, 4),
               "ms_median": round(float(np.median(ms_all)), 4),
               "ms_min": round(float(ms_all.min()), 4), "ms_max": round(float(ms_all.max()), 4),
               "tokens_per_s": round(T / (ms * 1e-3), 1), "tflops": round(tf, 2),
               "gbps": round(gb, 1), "bound": bound, "frac_mfma": round(tf / peak_f, 4),
               "frac_hbm": round(gb / PEAK_HBM_GBPS, 4),
               "frac_bound": round((tf / peak_f) if bound == "mfma" else (gb / PEAK_HBM_GBPS), 4),
               "cold_caches": flush, "kept_rows": R_kept, "touched_experts": touched,
               "algorithmic_flops": F, "algorithmic_bytes": B}
        if wl.capacity_factor > 0:
            rec["capacity_factor"] = wl.capacity_factor
            rec["n_dropped"] = int(st.n_dropped.cpu()[0])
        if wl.aux_alpha > 0:
            rec["aux_loss"] = round(float(st.aux.cpu()[0]), 6)
            rec["aux_alpha"] = wl.aux_alpha
        counts = st.counts.cpu().numpy().astype(np.int64)
        rec["max_over_mean_load"] = round(float(counts.max() / (T * wl.k / wl.E)), 3)
        out.append(rec)
        log(f"[bench] {name}: {ms:.4f} ms/step, {rec['frac_bound']:.3f} of the {bound} roofline "
            f"({time.time() - t0:.1f}s)")
        if wl.config_id == 2 and coverage is None:
            coverage = gpu_coverage(wl, W, stream)
        del x, y, ws, st
    del scratch, sink, W
    torch.cuda.empty_cache()
    return out, coverage


def gpu_coverage(wl, W, stream, n=2000, Bs=(1, 2, 4, 8, 16, 32)):
    """Fraction of the experts a batch of B tokens touches under the GPU's routing
    (moe_route on n * 32 seeded tokens, batches of consecutive tokens), against
    1 - (1 - k/E)^B, with the standard error of the mean from the exact variance of the
    untouched-expert count under uniform top-k choices."""
    import math
    import numpy as np
    import torch
    import mixture_experts_layer_31_amd as moe
    import workloads as wk

    dev = torch.device("cuda:0")
    T = n * max(Bs)
    cfg = moe.make_config(T, wl.d, wl.E, wl.k, wl.d_ff, gate=wl.gate, dtype=wl.dtype)
    a = np.ascontiguousarray(wk.make_inputs(wl, T=T).x)
    x = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.empty((T, wl.k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, wl.k), dtype=torch.float32, device=dev)
    moe.route(cfg, x, W["wr"], None, idx, gates, None, moe.alloc_workspace(cfg, moe.STAGE_ROUTE),
              stream)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    E, k = wl.E, wl.k
    res = {"batches": n, "B": [], "gpu": [], "closed_form": [], "se": [], "within_3se": True}
    for B in Bs:
        cov = np.array([np.unique(gi[i * B:(i + 1) * B]).size / E for i in range(n)])
        q = (1 - k / E) ** B
        q2 = (math.comb(E - 2, k) / math.comb(E, k)) ** B
        se = math.sqrt(max(E * q * (1 - q) + E * (E - 1) * (q2 - q * q), 0.0) / E ** 2 / n)
        res["B"].append(B)
        res["gpu"].append(round(float(cov.mean()), 5))
        res["closed_form"].append(round(1 - q, 5))
        res["se"].append(float(f"{se:.2e}"))
        res["within_3se"] &= bool(abs(cov.mean() - (1 - q)) <= 3 * se + 1e-12)
    return res


def time_backward(args, cfg, wl, x, wr, bias, experts, shared, R_kept, stream, peak_f):
    """moe_backward over the same batch (dy ~ N(0, 1)), K timed calls between HIP events
    on the library's stream. Algorithmic work per kept row: 12 d d_ff flop (the
    activation gradient, dx through W1/W3 and the three weight gradients; twice the
    forward's 6 d d_ff), plus 4 d d_ff to recompute h1 and h3, which the library does
    instead of keeping them from the forward."""
    import numpy as np
    import torch
    import mixture_experts_layer_31_amd as moe

    dev = x.device
    T, d, E, dff = wl.T, wl.d, wl.E, wl.d_ff
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    dy = torch.randn((T, d), generator=gen, dtype=torch.float32, device=dev)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    dx, dwr = f32(T, d), f32(E, d)
    dw1, dw3, dw2 = f32(E, dff, d), f32(E, dff, d), f32(E, d, dff)
    dws = (None, None, None)
    if wl.n_shared:
        dffs = wl.d_ff_shared
        dws = (f32(dffs, d), f32(dffs, d), f32(d, dffs))
    ws = moe.alloc_workspace(cfg, moe.STAGE_BACKWARD)

    def call():
        moe.backward(cfg, x, wr, bias, *experts, *shared, dy, dx, dwr, dw1, dw3, dw2, *dws,
                     ws, stream)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    K = args.steps
    b0.record(stream)
    for _ in range(K):
        call()
    b1.record(stream)
    torch.cuda.synchronize()
    ms = b0.elapsed_time(b1) / K
    rows_sh = wl.n_shared * T
    F = (12.0 * d * dff * R_kept + 12.0 * d * wl.d_ff_shared * rows_sh
         + 4.0 * T * d * E)
    F_re = 4.0 * d * dff * R_kept + 4.0 * d * wl.d_ff_shared * rows_sh
    tf = F / (ms * 1e-3) / 1e12
    tf_all = (F + F_re) / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "algorithmic_flops": F, "recompute_flops": F_re,
            "tflops": round(tf, 2), "frac_mfma": round(tf / peak_f, 4),
            "tflops_with_recompute": round(tf_all, 2),
            "workspace_bytes": int(ws.numel())}


def cpu_baseline(wl, inp, host, sample):
    """The float64 oracle, as it is, on the first `sample` tokens of the same batch (its
    float64 copies of the bf16 weights are made inside the timed region, one expert at a
    time, as the oracle does). Reported as tokens/s."""
    import numpy as np
    import workloads as wk
    from oracle import moe as om
    try:
        from threadpoolctl import threadpool_info
        cores = sum(p.get("num_threads", 0) for p in threadpool_info()
                    if p.get("user_api") == "blas") or (os.cpu_count() or 1)
    except Exception:
        cores = os.cpu_count() or 1
    if sample <= 0:
        sample = {4096: 4096, 16384: 4096, 8192: 8192, 512: 512}.get(wl.T, min(wl.T, 32))
        if wl.E >= 64 and wl.k >= 8:
            sample = min(sample, 64)
    S = min(sample, wl.T)
    x64 = wk.to_f64(inp.x[:S], wl.dtype)
    wr64 = wk.to_f64(inp.w_router, wl.dtype)

    def experts(e):
        return tuple(wk.to_f64(a[e], wl.dtype) for a in host)

    shared = None
    sh = inp.shared()
    t0 = time.perf_counter()
    if sh is not None:
        shared = tuple(wk.to_f64(a, wl.dtype) for a in sh)
    om.forward(x64, wr64, experts, wl.k, wl.gate, inp.bias, wl.capacity_factor, shared,
               wl.aux_alpha)
    dt = time.perf_counter() - t0
    return {"value": round(S / dt, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {S} of the {wl.T} tokens of {wl.name} (capacity, if any, "
                      f"computed on the sample), float64, {dt:.1f} s"}


if __name__ == "__main__":
    main()
