"""ssm_scan_fwd_noalloc (the scan for callers that cannot allocate: its
chunked schedules use the library's own device scratch array) against
ssm_scan_fwd with a caller workspace, through the C ABI.  Same plan, same
kernels: the outputs must be bit-identical.  Two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents), and a
one-launch plan whose publication flags live in the scratch, called twice.
"""
import ctypes
import sys

import numpy as np
import pytest

import selective_state_space_fwd_amd as ssm
import ssm_inputs
from ssm_testutil import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_both(dev, shape, io, K):
    import torch
    batch, d_inner, N, L = shape
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=L + d_inner)
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    lib = ssm.load_library()
    code = 1 if io == "bf16" else 0
    plan = ssm.scan_plan(batch, d_inner, N, L, code, K)
    need = ssm.ssm_scan_workspace_bytes(batch, d_inner, N, L, code, K)
    say(f"no-alloc {shape} {io} K={K}: plan '{plan}', workspace of a plain call {need} B")
    y1, h1 = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                              t["delta_bias"], chunk_size=K)
    y2 = torch.full_like(y1, float("nan"))
    h2 = torch.full_like(h1, float("nan"))
    d = ssm.make_desc(batch, d_inner, N, L, code, K)
    stream = torch.cuda.current_stream(dev).cuda_stream
    p = lambda x: None if x is None else x.data_ptr()
    st = lib.ssm_scan_fwd_noalloc(ctypes.byref(d), p(t["u"]), p(t["delta"]), p(t["A"]),
                                  p(t["B"]), p(t["C"]), p(t["D"]), p(t["z"]),
                                  p(t["delta_bias"]), 1, p(y2), p(h2), stream)
    assert st == 0, ssm.ssm_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    return plan


def test_noalloc_matches_workspace_entry_point(dev):
    # a larger chunked call, then a smaller one on the same scratch; then a
    # one-launch plan twice (its flags are epochs new for every launch)
    plans = [run_both(dev, (1, 256, 16, 4096), "f32", 0),
             run_both(dev, (2, 40, 16, 1000), "bf16", 64),
             run_both(dev, (1, 64, 16, 8192), "f32", 1024),
             run_both(dev, (1, 48, 16, 4100), "bf16", 1024)]
    assert plans[0].startswith("two passes") and plans[2].startswith("one launch")
    # a plan without workspace touches no scratch
    run_both(dev, (1, 1024, 16, 512), "f32", 0)


def test_noalloc_rejects_plans_above_the_limit(dev):
    """65536 tokens of 2048 channels in chunks of 512 need 33 MiB of chunk
    operators and start states: refused before any launch."""
    lib = ssm.load_library()
    d = ssm.make_desc(1, 2048, 16, 65536, 1, 512)
    assert ssm.ssm_scan_workspace_bytes(1, 2048, 16, 65536, 1, 512) > 32 << 20
    st = lib.ssm_scan_fwd_noalloc(ctypes.byref(d), 16, 16, 16, 16, 16, None, None, None, 1,
                                  16, None, None)
    assert st == 5
