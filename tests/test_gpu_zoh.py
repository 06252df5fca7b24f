"""GPU parity of the zero-order-hold discretisation (SSM_FLAG_ZOH) against
the fp64 oracle: scan on both kernels, with chunking, packed sequences and
the fused convolution, the single-token update, and the accuracy of the
hold factor (exp(dt A) - 1) / A across dt A from -20 to -1e-7.
"""
import sys

import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
import ssm_inputs
from ssm_testutil import TOL, decoded, floored_err, to_device, to_f64

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


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 40])
@pytest.mark.parametrize("K", [0, 16])
def test_zoh_scan(dev, io, N, K):
    import torch
    inp = ssm_inputs.make_scan_inputs(2, 50, N, 600, io_dtype=io, gate=True, seed=N + K)
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            t["delta_bias"], chunk_size=K, zoh=True)
    torch.cuda.synchronize()
    f = decoded(inp)
    yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], softplus=True, zoh=True)
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    say(f"zoh io={io} N={N} K={K}: err y={ey:.3e} last_state={eh:.3e}")
    assert ey <= TOL[io] and eh <= TOL[io]


@pytest.mark.parametrize("N", [16, 64])
def test_zoh_with_conv_and_packing(dev, N):
    import torch
    lens = [40, 0, 3, 130, 77]
    total = sum(lens)
    inp = ssm_inputs.make_scan_inputs(1, 24, N, total, io_dtype="f32", gate=True, seed=9)
    w, cb = ssm_inputs.make_conv_params(24, 4, seed=10)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    h0 = np.random.default_rng(3).standard_normal((len(lens), 24, N)).astype(np.float32)
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    g = lambda a: torch.from_numpy(a).to(dev)
    y, h, _ = ssm.ssm_scan_fwd_conv(t["u"], g(w), g(cb), t["delta"], t["A"], t["B"], t["C"],
                                    t["D"], t["z"], t["delta_bias"], initial_state=g(h0),
                                    cu_seqlens=g(cu), chunk_size=16, zoh=True)
    torch.cuda.synchronize()
    f = decoded(inp)
    ur = oracle.causal_conv1d(f["u"], w, cb, silu=True, cu_seqlens=cu)
    yr, hr = oracle.scan_varlen(ur, f["delta"], f["A"], f["B"], f["C"], cu, f["D"], f["z"],
                                f["delta_bias"], softplus=True,
                                initial_state=h0.astype(np.float64), zoh=True)
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    say(f"zoh + conv + packed N={N}: err y={ey:.3e} last_state={eh:.3e}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 5, 64])
def test_zoh_decode(dev, io, N):
    import torch
    inp = ssm_inputs.make_update_inputs(64, 40, N, io_dtype=io, gate=True, seed=N)
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D")}
    st = torch.from_numpy(np.ascontiguousarray(inp["state"])).to(dev)
    y = ssm.ssm_state_update(st, t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                             zoh=True)
    torch.cuda.synchronize()
    f = {k: ssm_inputs.to_f64(inp.get(k)) for k in ("u", "delta", "B", "C", "z")}
    sr, yr = oracle.state_update(inp["state"], f["u"], f["delta"], inp["A"], f["B"], f["C"],
                                 inp["D"], f["z"], zoh=True)
    es, ey = floored_err(to_f64(st), sr), floored_err(to_f64(y), yr)
    say(f"zoh decode io={io} N={N}: err state={es:.3e} y={ey:.3e}")
    assert es <= TOL[io] and ey <= TOL[io]


def test_zoh_factor_accuracy(dev):
    """One token from a zero state with B = C = u = 1 and A = -1 gives
    y = (1 - exp(-dt)): the hold factor itself, for dt from 1e-7 to 20,
    including both sides of the polynomial / quotient switch at |dt A| = 1/8."""
    import torch
    dts = np.concatenate([np.logspace(-7, np.log10(20.0), 400), [0.1249, 0.125, 0.1251],
                          np.linspace(0.12, 0.2, 41)])
    n = dts.size
    one = lambda *s: torch.ones(*s, device=dev)
    delta = torch.from_numpy(dts.astype(np.float32)).to(dev).view(1, n, 1)
    A = -one(n, 1)
    y, _ = ssm.ssm_scan_fwd(one(1, n, 1), delta, A, one(1, 1, 1), one(1, 1, 1), softplus=False,
                            zoh=True)
    torch.cuda.synchronize()
    d32 = dts.astype(np.float32).astype(np.float64)
    ref = -np.expm1(-d32)
    err = np.max(np.abs(to_f64(y).ravel() - ref) / np.abs(ref))
    say(f"zoh factor: max relative error {err:.3e}")
    assert err < 2e-6
