"""GPU tests of the one-launch chunked scan (d_state <= 16, 2..32 chunks of
1024 tokens or more): chunks publish their transfer operators in the
workspace, wait for their predecessors' for a bounded time and compute any
missing one themselves.

The result must not depend on the schedule: a launch in which every chunk
computes all operators before it itself (SSM_FLAG_INDEPENDENT_CHUNKS) must
give the same bits as the waiting launch, for the lean and the extended
(packed sequences, convolution, ZOH) kernels.  Repeated launches on one
workspace (stale flags of earlier launches), a workspace full of random
bytes, and graph replays with new inputs each time must give the bits of a
fresh eager launch.  Every case is also checked against the fp64 oracle.
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


def chunks(L, K):
    return -(-L // K)


# (batch, d_inner, N, L, K): J = ceil(L / K) between 2 and 32, ragged
# channel blocks and token tails, the element (non-vector) path (L % 4 != 0)
SHAPES = [(2, 40, 16, 3000, 1024), (1, 33, 5, 5000, 1024), (3, 16, 1, 2100, 1024),
          (1, 24, 16, 32768, 1024), (1, 48, 12, 4099, 1024), (2, 130, 16, 6000, 2048)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_waiting_equals_independent_and_oracle(dev, io, shape):
    import torch
    batch, d_inner, N, L, K = shape
    assert 2 <= chunks(L, K) <= 32
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=sum(shape))
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    y1, h1 = ssm.ssm_scan_fwd(*args, chunk_size=K)
    y2, h2 = ssm.ssm_scan_fwd(*args, chunk_size=K, independent_chunks=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    f = decoded(inp)
    yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], softplus=True)
    ey, eh = floored_err(to_f64(y1), yr), floored_err(to_f64(h1), hr)
    say(f"fused io={io} {shape} J={chunks(L, K)}: err y={ey:.3e} last_state={eh:.3e}")
    assert ey <= TOL[io] and eh <= TOL[io]


@pytest.mark.parametrize("variant", ["packed", "conv", "zoh"])
def test_extended_kernel_waiting_equals_independent(dev, variant):
    """The extended instance: packed sequences with start states (boundaries
    inside chunks, on chunk edges, an empty sequence), the fused convolution,
    and ZOH."""
    import torch
    d_inner, N, K = 40, 16, 1024
    lens = [1500, 0, 700, 1, 2000, 1024, 3] if variant == "packed" else [4000]
    L = int(sum(lens))
    inp = ssm_inputs.make_scan_inputs(1, d_inner, N, L, io_dtype="f32", gate=True, seed=4)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    f = decoded(inp)
    rng = np.random.default_rng(8)
    if variant == "conv":
        w, cb = ssm_inputs.make_conv_params(d_inner, 4, seed=5)
        g = lambda a: torch.from_numpy(a).to(dev)
        run = lambda ind: ssm.ssm_scan_fwd_conv(t["u"], g(w), g(cb), t["delta"], t["A"], t["B"],
                                                t["C"], t["D"], t["z"], t["delta_bias"],
                                                chunk_size=K, independent_chunks=ind)[:2]
        ur = oracle.causal_conv1d(f["u"], w, cb, silu=True)
        yr, hr = oracle.scan_fwd(ur, f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                                 f["delta_bias"], softplus=True)
    elif variant == "packed":
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        h0 = rng.standard_normal((len(lens), d_inner, N)).astype(np.float32)
        cu_t, h0_t = torch.from_numpy(cu).to(dev), torch.from_numpy(h0).to(dev)
        run = lambda ind: ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                           t["z"], t["delta_bias"], chunk_size=K,
                                           initial_state=h0_t, cu_seqlens=cu_t,
                                           independent_chunks=ind)
        yr, hr = oracle.scan_varlen(f["u"], f["delta"], f["A"], f["B"], f["C"], cu, f["D"],
                                    f["z"], f["delta_bias"], softplus=True,
                                    initial_state=h0.astype(np.float64))
    else:
        run = lambda ind: ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                           t["z"], t["delta_bias"], chunk_size=K, zoh=True,
                                           independent_chunks=ind)
        yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                                 f["delta_bias"], softplus=True, zoh=True)
    y1, h1 = run(False)
    y2, h2 = run(True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    ey, eh = floored_err(to_f64(y1), yr), floored_err(to_f64(h1), hr)
    say(f"fused {variant}: err y={ey:.3e} last_state={eh:.3e}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_stale_and_random_workspace(dev):
    """Launches that reuse one workspace (flags of earlier launches in it), on
    changing inputs, and a workspace of random bytes, all match a launch on a
    fresh workspace bit for bit."""
    import torch
    batch, d_inner, N, L, K = 2, 64, 16, 4096, 1024
    desc = ssm.make_desc(batch, d_inner, N, L, 0, K)
    need = ssm.load_library().ssm_scan_workspace_bytes(__import__("ctypes").byref(desc))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    for it in range(4):
        inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype="f32", gate=True,
                                          seed=100 + it)
        t = {k: to_device(inp.get(k), dev) for k in KEYS}
        args = (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
        if it == 3:
            ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=dev)
        y, h = ssm.ssm_scan_fwd(*args, chunk_size=K, workspace=ws)
        yf, hf = ssm.ssm_scan_fwd(*args, chunk_size=K, independent_chunks=True)
        torch.cuda.synchronize()
        assert torch.equal(y, yf) and torch.equal(h, hf), it


def test_graph_replays_with_new_inputs(dev):
    """A captured launch replayed three times, the inputs overwritten before
    each replay and host work and synchronisation in between: every replay
    equals an eager launch on the same inputs bit for bit."""
    import torch
    batch, d_inner, N, L, K = 2, 64, 16, 4096, 1024
    def fresh(seed):
        inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype="f32", gate=True,
                                          seed=seed)
        return {k: to_device(inp.get(k), dev) for k in KEYS}
    t = fresh(200)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    ssm.ssm_scan_fwd(*args, chunk_size=K)           # load and warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        yg, hg = ssm.ssm_scan_fwd(*args, chunk_size=K)
    for r in range(3):
        new = fresh(300 + r)
        for k in KEYS:
            t[k].copy_(new[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ye, he = ssm.ssm_scan_fwd(*args, chunk_size=K)
        torch.cuda.synchronize()
        assert torch.equal(yg, ye) and torch.equal(hg, he), r
        say(f"graph replay {r}: equal to eager")


def test_long_sequence_one_launch(dev):
    """The long-sequence workload (1 x 2048 channels, N = 16, 64 Ki tokens,
    bf16) in 16 chunks of 4096 tokens: one launch.  Equal to the
    independent-chunk launch bit for bit; 64 channels spread over the row
    against the oracle (the scan of a channel depends only on its own inputs
    and the shared B, C)."""
    import torch
    K = 4096
    assert ssm.scan_plan(1, 2048, 16, 65536, 1, K).startswith("one launch")
    inp = ssm_inputs.make_scan_inputs(1, 2048, 16, 65536, io_dtype="bf16", gate=True, seed=0)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    y1, h1 = ssm.ssm_scan_fwd(*args, chunk_size=K)
    y2, h2 = ssm.ssm_scan_fwd(*args, chunk_size=K, independent_chunks=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    f = decoded(inp)
    ch = np.arange(0, 2048, 32)
    yr, hr = oracle.scan_fwd(f["u"][:, ch], f["delta"][:, ch], f["A"][ch], f["B"], f["C"],
                             f["D"][ch], f["z"][:, ch], f["delta_bias"][ch], softplus=True)
    ey = floored_err(to_f64(y1)[:, ch], yr)
    eh = floored_err(to_f64(h1)[:, ch], hr)
    say(f"long sequence auto plan: err y={ey:.3e} last_state={eh:.3e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
