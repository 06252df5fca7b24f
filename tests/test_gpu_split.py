"""GPU parity of the balanced serial walks (quad_split_kernel): when the
16-channel blocks are not a whole number of rounds of the 1024 SIMDs, the
blocks past the last whole round run as two chunks on two wavefronts, the
second waiting for the first's end state.  Against the oracle: whole
chunks, ragged channels, the element path (inputs not 16-byte aligned),
d_state below 16, start states, exact integers bit for bit; the schedule where no chunk waits
bit-equal to the waiting one; graph replays with new inputs equal to eager
calls (the flags of a captured launch are cleared by a kernel node).
"""
import sys

import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
import ssm_inputs
from ssm_testutil import TOL, decoded, floored_err, to_device, to_f64

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


def plan_of(batch, d_inner, N, L, io):
    return ssm.scan_plan(batch, d_inner, N, L, 1 if io == "bf16" else 0, 0)


@pytest.mark.parametrize("shape,io,h0", [
    ((1, 24576, 16, 256), "f32", False),      # 1536 blocks: one round + 512 split
    ((1, 20008, 16, 304), "bf16", False),     # ragged channels
    ((2, 20480, 5, 512), "f32", True),        # d_state 5, start states, 2560 blocks
])
def test_split_against_oracle(dev, shape, io, h0):
    import torch
    batch, d_inner, N, L = shape
    plan = plan_of(batch, d_inner, N, L, io)
    say(f"split walks {shape} {io} h0={h0}: plan '{plan}', chunk "
        f"{ssm.ssm_scan_chunk_size(batch, d_inner, N, L, 1 if io == 'bf16' else 0)}")
    assert plan.startswith("one chunk, the blocks past")
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=not h0,
                                      seed=L + N, random_a=True)
    if h0:
        inp["D"] = None
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    hs = np.random.default_rng(5).standard_normal((batch, d_inner, N)).astype(np.float32) \
        if h0 else None
    y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            t["delta_bias"], initial_state=to_device(hs, dev) if h0 else None)
    y2, h2 = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                              t["delta_bias"], initial_state=to_device(hs, dev) if h0 else None,
                              independent_chunks=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(h, h2)
    f = decoded(inp)
    yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], softplus=True,
                             initial_state=None if hs is None else hs.astype(np.float64))
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    say(f"  err y={ey:.3e} last_state={eh:.3e} (tol {TOL[io]})")
    assert ey <= TOL[io] and eh <= TOL[io]


def misaligned(t):
    """A contiguous copy of t whose first element sits one element past an
    allocation's start: aligned to the element, not to 16 bytes."""
    import torch
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = flat[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_split_element_path(dev, io):
    """u, delta and y one element off 16-byte alignment: the split walks
    load and store element by element."""
    import torch
    batch, d_inner, N, L = 1, 20480, 16, 512
    assert plan_of(batch, d_inner, N, L, io).startswith("one chunk, the blocks past")
    say(f"split walks, element path, io={io}")
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True, seed=77)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    u, dl = misaligned(t["u"]), misaligned(t["delta"])
    y = misaligned(torch.empty_like(t["u"]))
    assert u.data_ptr() % 16 and dl.data_ptr() % 16 and y.data_ptr() % 16
    y, h = ssm.ssm_scan_fwd(u, dl, t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                            y=y)
    y2, h2 = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                              t["delta_bias"])
    torch.cuda.synchronize()
    f = decoded(inp)
    yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], softplus=True)
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    say(f"  err y={ey:.3e} last_state={eh:.3e} (tol {TOL[io]})")
    assert ey <= TOL[io] and eh <= TOL[io]
    # the element path and the 16-byte path run the same arithmetic
    assert torch.equal(y, y2) and torch.equal(h, h2)


def test_split_integers_bit_exact(dev):
    """Decay 1, unit step, small integers: chunk 1 starts from chunk 0's end
    state exactly, so every value matches the sequential result bit for bit."""
    import torch
    batch, d_inner, N, L = 1, 24576, 16, 300
    assert plan_of(batch, d_inner, N, L, "f32").startswith("one chunk, the blocks past")
    rng = np.random.default_rng(9)
    u = rng.integers(-2, 3, (batch, d_inner, L)).astype(np.float32)
    case = dict(u=u, delta=np.ones_like(u), A=np.zeros((d_inner, N), np.float32),
                B=rng.integers(-2, 3, (batch, N, L)).astype(np.float32),
                C=rng.integers(-2, 3, (batch, N, L)).astype(np.float32),
                D=rng.integers(-2, 3, d_inner).astype(np.float32))
    t = {k: to_device(v, dev) for k, v in case.items()}
    y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], None, None,
                            softplus=False)
    torch.cuda.synchronize()
    yr, hr = oracle.scan_fwd(case["u"], case["delta"], case["A"], case["B"], case["C"],
                             case["D"], softplus=False)
    assert np.array_equal(to_f64(y), yr)
    assert np.array_equal(to_f64(h), hr)


def test_split_graph_replays(dev):
    """The split launch captured in a HIP graph and replayed three times with
    new inputs written in place, each replay bit-equal to an eager call."""
    import torch
    batch, d_inner, N, L = 1, 24576, 16, 256
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype="bf16", gate=True, seed=1)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    ssm.ssm_scan_fwd(*args)          # load and warm up outside the capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            yg, hg = ssm.ssm_scan_fwd(*args)
    torch.cuda.synchronize()
    for r in range(3):
        new = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype="bf16", gate=True,
                                          seed=100 + r)
        for k in ("u", "delta", "B", "C", "z"):
            t[k].copy_(to_device(new[k], dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ye, he = ssm.ssm_scan_fwd(*args)
        torch.cuda.synchronize()
        assert torch.equal(yg, ye) and torch.equal(hg, he), r
        say(f"split graph replay {r}: equal to eager")
