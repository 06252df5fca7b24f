"""GPU tests of PreparedCall: an entry point's call checked and marshalled
once (prepare=True), then launched again and again on the same buffers.

Every launch of a prepared call gives the bits of the plain call on the
inputs the buffers hold at that moment: inputs are overwritten in place
between launches, and each result is compared with a plain call on the same
inputs.  Covered: the forward pass (plain, with start states and packed
sequences, with checkpoints), the fused convolution, the decode step (whose
state is updated in place), and the backward pass (also with d_state above
16, captured in a graph); the in-wave scan captured in a graph.
"""
import sys

import numpy as np
import pytest

import selective_state_space_fwd_amd as ssm
import ssm_inputs
from ssm_testutil import to_device

pytestmark = pytest.mark.gpu

KEYS = ("u", "delta", "B", "C", "z", "A", "D", "delta_bias")


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def fresh(dev, batch, d_inner, N, L, io, seed):
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True, seed=seed)
    return {k: to_device(inp.get(k), dev) for k in KEYS}


def refill(t, new):
    for k in KEYS:
        t[k].copy_(new[k])


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["plain", "ex", "ckpt", "chunked"])
def test_prepared_forward(dev, io, variant):
    import torch
    batch, d_inner, N, L = (1, 40, 16, 700) if variant == "ex" else (2, 40, 16, 700)
    K = 64 if variant == "chunked" else 0
    t = fresh(dev, batch, d_inner, N, L, io, 1)
    extra = {}
    if variant == "ex":
        cu = torch.tensor([0, 100, 100, 450, 700], dtype=torch.int32, device=dev)
        h0 = torch.randn(4, d_inner, N, device=dev)
        extra = dict(cu_seqlens=cu, initial_state=h0)
    if variant == "ckpt":
        extra = dict(ckpt=torch.empty(ssm.ckpt_shape(batch, d_inner, L), device=dev))
    args = [t[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")]
    call = ssm.ssm_scan_fwd(*args, chunk_size=K, prepare=True, **extra)
    assert isinstance(call, ssm.PreparedCall)
    y, last = call.result
    for r in range(3):
        refill(t, fresh(dev, batch, d_inner, N, L, io, 10 + r))
        got = call()
        assert got[0] is y and got[1] is last
        snap = (y.clone(), last.clone(), extra["ckpt"].clone() if "ckpt" in extra else None)
        plain_extra = dict(extra)
        if "ckpt" in extra:
            plain_extra["ckpt"] = torch.empty_like(extra["ckpt"])
        yp, lp = ssm.ssm_scan_fwd(*args, chunk_size=K, **plain_extra)
        torch.cuda.synchronize()
        assert torch.equal(snap[0], yp) and torch.equal(snap[1], lp), r
        if "ckpt" in extra:
            assert torch.equal(snap[2], plain_extra["ckpt"]), r
    say(f"prepared forward {variant} io={io}: 3 launches equal to plain calls")


def test_prepared_conv_and_backward(dev):
    import torch
    batch, d_inner, N, L = 2, 40, 16, 300
    t = fresh(dev, batch, d_inner, N, L, "f32", 3)
    w, cb = (torch.from_numpy(a).to(dev) for a in ssm_inputs.make_conv_params(d_inner, 4, seed=4))
    conv = ssm.ssm_scan_fwd_conv(t["u"], w, cb, t["delta"], t["A"], t["B"], t["C"], t["D"],
                                 t["z"], t["delta_bias"], return_u=True, prepare=True)
    dy = torch.randn(batch, d_inner, L, device=dev)
    bwd = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"],
                           t["delta_bias"], prepare=True)
    for r in range(2):
        refill(t, fresh(dev, batch, d_inner, N, L, "f32", 20 + r))
        dy.copy_(torch.randn(batch, d_inner, L, device=dev))
        yc = [x.clone() for x in conv()]
        gb = {k: (None if v is None else v.clone()) for k, v in bwd().items()}
        yc2 = ssm.ssm_scan_fwd_conv(t["u"], w, cb, t["delta"], t["A"], t["B"], t["C"], t["D"],
                                    t["z"], t["delta_bias"], return_u=True)
        gb2 = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"],
                               t["delta_bias"])
        torch.cuda.synchronize()
        for a, b in zip(yc, yc2):
            assert torch.equal(a, b), r
        for k, v in gb.items():
            if v is not None:
                assert torch.equal(v, gb2[k]), (r, k)


def test_prepared_state_update(dev):
    import torch
    batch, d_inner, N = 8, 96, 16
    inp = ssm_inputs.make_update_inputs(batch, d_inner, N, io_dtype="f32", gate=True, seed=5)
    t = {k: torch.from_numpy(inp[k]).to(dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                        "state")}
    call = ssm.ssm_state_update(t["state"], t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                t["z"], prepare=True)
    for r in range(3):
        before = t["state"].clone()
        t["u"].copy_(torch.randn_like(t["u"]))
        y = call().clone()
        after = t["state"].clone()
        twin = before.clone()
        y2 = ssm.ssm_state_update(twin, t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                  t["z"])
        torch.cuda.synchronize()
        assert torch.equal(y, y2) and torch.equal(after, twin), r


@pytest.mark.parametrize("K", [0, 1024])
def test_training_step_in_a_graph(dev, K):
    """The forward pass keeping checkpoints and the backward pass reading them,
    captured as one graph (chunked in two passes, and in one launch with
    K = 1024) and replayed three times with new inputs written in place, host
    work and synchronisation in between: every replay gives the bits of an
    eager step on the same inputs."""
    import torch
    batch, d_inner, N, L = 2, 64, 16, 4096
    t = fresh(dev, batch, d_inner, N, L, "f32", 30)
    dy = torch.randn(batch, d_inner, L, device=dev)
    ck = torch.empty(ssm.ckpt_shape(batch, d_inner, L), device=dev)
    args = [t[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")]
    fwd = ssm.ssm_scan_fwd(*args, chunk_size=K, ckpt=ck, prepare=True)
    bwd = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"],
                           t["delta_bias"], ckpt=ck, prepare=True)
    fwd(); bwd()                      # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream     # the capturing stream
        fwd(stream=cap)
        bwd(stream=cap)
    for r in range(3):
        refill(t, fresh(dev, batch, d_inner, N, L, "f32", 40 + r))
        dy.copy_(torch.randn(batch, d_inner, L, device=dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_g, h_g = (x.clone() for x in fwd.result)
        grads_g = {k: (None if v is None else v.clone()) for k, v in bwd.result.items()}
        y_e, h_e = fwd()
        grads_e = bwd()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e) and torch.equal(h_g, h_e), r
        for k, v in grads_g.items():
            if v is not None:
                assert torch.equal(v, grads_e[k]), (r, k)
        say(f"graph training step K={K} replay {r}: equal to eager")


@pytest.mark.parametrize("shape", [(1, 8192, 64, 128),   # four groups side by side
                                   (2, 40, 48, 300)])   # one group per launch
def test_backward_state_groups_in_a_graph(dev, shape):
    """The backward with d_state above 16 (start state, dlast, gate, delta
    bias) captured as a graph: gathers, the backward launches, the reduces,
    the scatters, the d(bias) additions and (side by side) the slot sums.
    Three replays with new inputs written in place, host work and
    synchronisation in between: every replay gives the bits of an eager call."""
    import torch
    batch, d_inner, N, L = shape
    say(f"bwd state groups in a graph shape={shape}")
    t = fresh(dev, batch, d_inner, N, L, "f32", 50)
    dy = torch.randn(batch, d_inner, L, device=dev)
    h0 = torch.randn(batch, d_inner, N, device=dev)
    dl = torch.randn(batch, d_inner, N, device=dev)
    bwd = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"],
                           t["delta_bias"], initial_state=h0, dlast=dl, prepare=True)
    bwd()                             # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bwd(stream=torch.cuda.current_stream().cuda_stream)
    for r in range(3):
        refill(t, fresh(dev, batch, d_inner, N, L, "f32", 60 + r))
        dy.copy_(torch.randn(batch, d_inner, L, device=dev))
        h0.copy_(torch.randn(batch, d_inner, N, device=dev))
        dl.copy_(torch.randn(batch, d_inner, N, device=dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        grads_g = {k: (None if v is None else v.clone()) for k, v in bwd.result.items()}
        grads_e = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"],
                                   t["z"], t["delta_bias"], initial_state=h0, dlast=dl)
        torch.cuda.synchronize()
        for k, v in grads_g.items():
            if v is not None:
                assert torch.equal(v, grads_e[k]), (r, k)
        say(f"  replay {r}: equal to eager")


@pytest.mark.parametrize("shape,io,K,h0", [
    ((1, 2048, 16, 4096), "bf16", 256, False),   # segments of 16: event-counter ordering
    ((2, 1536, 16, 1024), "f32", 0, True),       # segments of 8 (the library's plan), start states
])
def test_in_wave_scan_in_a_graph(dev, shape, io, K, h0):
    """The in-wave scan captured as a graph and replayed three times with new
    inputs written in place, host work and synchronisation in between: every
    replay gives the bits of an eager call on the same inputs."""
    import torch
    batch, d_inner, N, L = shape
    plan = ssm.scan_plan(batch, d_inner, N, L, 1 if io == "bf16" else 0, K)
    assert plan.startswith("in-wave"), plan
    say(f"in-wave scan in a graph shape={shape} io={io} plan '{plan}'")
    t = fresh(dev, batch, d_inner, N, L, io, 70)
    extra = dict(initial_state=torch.randn(batch, d_inner, N, device=dev)) if h0 else {}
    args = [t[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")]
    call = ssm.ssm_scan_fwd(*args, chunk_size=K, prepare=True, **extra)
    call()                            # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(stream=torch.cuda.current_stream().cuda_stream)
    for r in range(3):
        refill(t, fresh(dev, batch, d_inner, N, L, io, 80 + r))
        if h0:
            extra["initial_state"].copy_(torch.randn(batch, d_inner, N, device=dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_g, h_g = (x.clone() for x in call.result)
        y_e, h_e = ssm.ssm_scan_fwd(*args, chunk_size=K, **extra)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e) and torch.equal(h_g, h_e), r
        say(f"  replay {r}: equal to eager")


def test_training_step_split_backward_in_a_graph(dev):
    """A training step whose backward, given the checkpoints, runs the blocks
    of a whole round as one chunk and the rest in chunks (two backward
    launches, reverse aggregates for the second), captured as one graph and
    replayed three times with new inputs: every replay gives the bits of an
    eager step."""
    import torch
    batch, d_inner, N, L = 2, 24576, 16, 128
    plan = ssm.scan_bwd_plan(batch, d_inner, N, L, 0, with_ckpt=True)
    assert plan.startswith("the blocks of a whole round"), plan
    say(f"graph training step, split backward: '{plan}'")
    t = fresh(dev, batch, d_inner, N, L, "f32", 90)
    dy = torch.randn(batch, d_inner, L, device=dev)
    ck = torch.empty(ssm.ckpt_shape(batch, d_inner, L), device=dev)
    args = [t[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")]
    fwd = ssm.ssm_scan_fwd(*args, ckpt=ck, prepare=True)
    bwd = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"],
                           t["delta_bias"], ckpt=ck, prepare=True)
    fwd(); bwd()                      # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        fwd(stream=cap)
        bwd(stream=cap)
    for r in range(3):
        refill(t, fresh(dev, batch, d_inner, N, L, "f32", 91 + r))
        dy.copy_(torch.randn(batch, d_inner, L, device=dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        grads_g = {k: (None if v is None else v.clone()) for k, v in bwd.result.items()}
        fwd()
        grads_e = bwd()
        torch.cuda.synchronize()
        for k, v in grads_g.items():
            if v is not None:
                assert torch.equal(v, grads_e[k]), (r, k)
        say(f"  replay {r}: equal to eager")
