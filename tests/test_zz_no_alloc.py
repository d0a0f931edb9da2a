"""moe_forward_noalloc, the form of moe_forward for callers that cannot allocate
device memory (its scratch is a fixed array of the library on each GPU), against
moe_forward with a caller workspace: bit for bit on two calls in a row, the second
one smaller, and a layer whose scratch would exceed the fixed size is refused
before anything is launched."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_31_amd as moe
import workloads as wk
from gpu_support import Weights, config_of, dev, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.load()


def _run(wl, W, x, T, noalloc, stats):
    cfg = config_of(wl, T)
    y = torch.full((T, wl.d), float("nan"), dtype=torch.float32, device=dev())
    idx = torch.full((T, wl.k), -7, dtype=torch.int32, device=dev())
    gates = torch.full((T, wl.k), float("nan"), dtype=torch.float32, device=dev())
    st = moe.Stats.alloc(wl.E) if stats else None
    if noalloc:
        moe.forward_noalloc(cfg, x, W.wr, W.bias, W.w1, W.w3, W.w2, W.s1, W.s3, W.s2, y, idx,
                            gates, st)
    else:
        ws = moe.alloc_workspace(cfg, moe.STAGE_FORWARD)
        ws.fill_(0xA5)   # leftovers of another kind than the fixed scratch's
        moe.forward(cfg, x, W.wr, W.bias, W.w1, W.w3, W.w2, W.s1, W.s3, W.s2, y, idx, gates, st,
                    ws)
    torch.cuda.synchronize()
    out = dict(y=y.cpu().numpy(), idx=idx.cpu().numpy(), gates=gates.cpu().numpy())
    if stats:
        out.update(counts=st.counts.cpu().numpy(), kept=st.kept.cpu().numpy(),
                   aux=st.aux.cpu().numpy())
    return out


_CASES = {
    # decode-sized steps with a shared expert (the side stream beside the routed
    # product above 16 tokens) and a selection bias
    "fine_grained_shared": (dict(d=512, E=64, k=6, d_ff=256, n_shared=1, d_ff_shared=256,
                                 bias_range=0.1), (200, 40)),
    # 256-row tiles at 1024 rows, then 16-row streaming tiles at 5 tokens
    "mixtral_like": (dict(d=1024, E=8, k=2, d_ff=2048, router="orthonormal"), (512, 5)),
    # capacity with full-softmax gates and the balance loss
    "switch_like": (dict(d=256, E=16, k=1, d_ff=512, gate=wk.GATE_ALL, capacity_factor=1.0,
                         aux_alpha=0.01, offset_var=1.5), (300, 33)),
}


@pytest.mark.parametrize("case", list(_CASES))
def test_noalloc_equals_forward_on_two_calls(case):
    kw, Ts = _CASES[case]
    wl = wk.Workload(f"noalloc_{case}", 140 + list(_CASES).index(case), T=Ts[0],
                     dtype=wk.BF16, **kw)
    W = Weights(wl)
    for i, T in enumerate(Ts):
        log(f"[case] noalloc {case} call {i} T={T}")
        x = to_dev(wk.make_inputs(wl, T=T).x, wl.dtype)
        stats = i == 0
        a = _run(wl, W, x, T, True, stats)
        b = _run(wl, W, x, T, False, stats)
        for key in a:
            assert np.array_equal(a[key], b[key]), f"{case} call {i}: {key}"
        assert np.isfinite(a["y"]).all()


def test_noalloc_refuses_a_layer_above_its_scratch():
    """The Mixtral-shaped layer at 4096 tokens needs more scratch than the fixed
    array holds: refused with MOE_ERR_WORKSPACE, nothing launched, y untouched."""
    wl = wk.get("mixtral_t4096")
    cfg = config_of(wl, wl.T)
    assert moe.workspace_size(cfg, moe.STAGE_FORWARD) > moe.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.bfloat16, device=dev())
    y = torch.full((4,), 3.0, device=dev())
    with pytest.raises(moe.MoEError) as e:
        moe.forward_noalloc(cfg, t, t, None, t, t, t, None, None, None, y)
    assert e.value.status == moe.ERR_WORKSPACE
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (y == 3.0).all()
