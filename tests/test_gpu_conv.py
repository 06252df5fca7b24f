"""GPU parity of the scan with the causal conv1d fused in front
(ssm_scan_fwd_conv) against the fp64 oracle: oracle.causal_conv1d followed
by oracle.scan_fwd / oracle.scan_varlen on the unrounded convolution output.

Cases: widths 1..4, silu on and off, conv_state and initial_state, packed
sequences, chunk edges (many short chunks), both kernels (d_state <= 16 and
> 16), fp32 and bf16, the Mamba-130M-shaped layer in full, and exact-integer
inputs bit for bit.
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


def run_case(dev, batch, d_inner, N, L, io, W, silu, K, with_state, lens=None, seed=0,
             decay_kernel=True, gate=True):
    import torch
    if lens is not None:
        batch, L = 1, int(sum(lens))
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=gate, seed=seed)
    w, cb = ssm_inputs.make_conv_params(d_inner, W, seed=seed + 1, decay_kernel=decay_kernel)
    rows = batch if lens is None else len(lens)
    cu = None if lens is None else np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(seed + 2)
    cs = rng.standard_normal((rows, d_inner, W - 1)).astype(np.float32) if with_state else None
    h0 = rng.standard_normal((rows, d_inner, N)).astype(np.float32) if with_state else None
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    g = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    y, h, u = ssm.ssm_scan_fwd_conv(t["u"], g(w), g(cb), t["delta"], t["A"], t["B"], t["C"],
                                    t["D"], t["z"], t["delta_bias"], softplus=True,
                                    conv_silu=silu, conv_state=g(cs), initial_state=g(h0),
                                    cu_seqlens=g(cu), return_u=True, chunk_size=K)
    torch.cuda.synchronize()
    f = decoded(inp)
    ur = oracle.causal_conv1d(f["u"], w, cb, silu=silu, cu_seqlens=cu,
                              conv_state=None if cs is None else cs.astype(np.float64))
    h0r = None if h0 is None else h0.astype(np.float64)
    if cu is None:
        yr, hr = oracle.scan_fwd(ur, f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                                 f["delta_bias"], softplus=True, initial_state=h0r)
    else:
        yr, hr = oracle.scan_varlen(ur, f["delta"], f["A"], f["B"], f["C"], cu, f["D"], f["z"],
                                    f["delta_bias"], softplus=True, initial_state=h0r)
    eu = floored_err(to_f64(u), ur)
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    say(f"  err u={eu:.3e} y={ey:.3e} last_state={eh:.3e} (tol {TOL[io]})")
    assert eu <= TOL[io] and ey <= TOL[io] and eh <= TOL[io]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 48])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_conv_widths(dev, io, N, W):
    K = {1: 0, 2: 16, 3: 64, 4: 32}[W]
    say(f"conv io={io} N={N} W={W} K={K}")
    run_case(dev, 2, 40, N, 333, io, W, silu=True, K=K, with_state=False, seed=W)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 40])
@pytest.mark.parametrize("silu", [True, False])
def test_conv_with_start_states(dev, io, N, silu):
    say(f"conv + conv_state + initial_state io={io} N={N} silu={silu}")
    run_case(dev, 3, 33, N, 520, io, 4, silu=silu, K=16, with_state=True, seed=7,
             decay_kernel=False)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("with_state", [False, True])
def test_conv_packed_sequences(dev, io, N, with_state):
    lens = [37, 0, 1, 2, 200, 16, 0, 3, 64, 129]
    say(f"conv packed io={io} N={N} state={with_state}")
    run_case(dev, 1, 40, N, 0, io, 4, silu=True, K=16, with_state=with_state, lens=lens,
             seed=11)


def test_conv_mamba130m_layer_full(dev):
    """The Mamba-130M-shaped layer (2 x 1536 channels, N = 16, L = 2048, fp32,
    gate) with a width-4 convolution, every output compared."""
    say("conv mamba130m layer")
    run_case(dev, 2, 1536, 16, 2048, "f32", 4, silu=True, K=0, with_state=False, seed=3)


def test_conv_integer_bit_exact(dev):
    """Integer inputs and taps, unit decay, no silu: every path is exact, so the
    result must equal the oracle bit for bit at any chunking."""
    import torch
    d_inner, N, L, W = 20, 16, 300, 4
    rng = np.random.default_rng(5)
    x = rng.integers(-3, 4, size=(1, d_inner, L)).astype(np.float32)
    w = rng.integers(-2, 3, size=(d_inner, W)).astype(np.float32)
    cb = rng.integers(-2, 3, size=d_inner).astype(np.float32)
    B = rng.integers(-2, 3, size=(1, N, L)).astype(np.float32)
    C = rng.integers(-2, 3, size=(1, N, L)).astype(np.float32)
    dt = np.ones((1, d_inner, L), np.float32)
    A = np.zeros((d_inner, N), np.float32)
    ur = oracle.causal_conv1d(x, w, cb, silu=False)
    yr, hr = oracle.scan_fwd(ur, dt, A, B, C, softplus=False)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    for K in (16, 48, 0):
        y, h, u = ssm.ssm_scan_fwd_conv(g(x), g(w), g(cb), g(dt), g(A), g(B), g(C),
                                        softplus=False, conv_silu=False, return_u=True,
                                        chunk_size=K)
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(u), ur)
        assert np.array_equal(to_f64(y), yr) and np.array_equal(to_f64(h), hr)
