"""GPU parity of libssm against the fp64 oracle, called through the C ABI.

Floating point: floored relative error (see ssm_testutil.floored_err) below
1e-4 for float32 I/O and 2e-2 for bfloat16 I/O.  Exact-integer inputs must
match bit for bit.  Every workload is compared element by element, y and
last_state in full.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
import ssm_inputs
from ssm_testutil import TOL, decoded, floored_err, to_device, to_f32, to_f64

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


def run_gpu(inp, dev, chunk_size=0, last_state=True, softplus=None, **over):
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    t.update(over)
    sp = inp["softplus"] if softplus is None else softplus
    y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            t["delta_bias"], softplus=sp, return_last_state=last_state,
                            chunk_size=chunk_size)
    import torch
    torch.cuda.synchronize()
    return y, h


def check_full(inp, dev, chunk_size=0, tol=None):
    io = inp["io_dtype"]
    y, h = run_gpu(inp, dev, chunk_size)
    f = decoded(inp)
    yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], softplus=bool(f["softplus"]))
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    tol = tol or TOL[io]
    say(f"  err y={ey:.3e} last_state={eh:.3e} (tol {tol})")
    assert ey <= tol and eh <= tol
    return y, h


# ------------------------------------------------------------ workload configs

def test_config_tiny_f32(dev):
    say("config tiny f32 b=1 d=64 N=16 L=256")
    inp = ssm_inputs.make_scan_inputs(**ssm_inputs.CONFIGS["c0_tiny_f32"])
    check_full(inp, dev)


def test_config_mamba130m_f32_full(dev):
    say("config mamba-130m f32 b=2 d=1536 N=16 L=2048 (all rows)")
    inp = ssm_inputs.make_scan_inputs(**ssm_inputs.CONFIGS["c1_mamba130m_f32"])
    check_full(inp, dev)


def test_config_mamba2p8b_bf16_full(dev):
    say("config mamba-2.8b bf16 b=8 d=5120 N=16 L=2048 (every element)")
    inp = ssm_inputs.make_scan_inputs(**ssm_inputs.CONFIGS["c2_mamba2p8b_bf16"])
    check_full(inp, dev)


@pytest.fixture(scope="module")
def long_case():
    """The long-sequence workload and the oracle's y and last_state for it,
    computed once for every chunk length."""
    inp = ssm_inputs.make_scan_inputs(**ssm_inputs.CONFIGS["c3_long_bf16"])
    f = decoded(inp)
    yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], softplus=bool(f["softplus"]))
    del f
    return inp, yr, hr


@pytest.mark.parametrize("K", [256, 512, 1024, 0])
def test_config_long_bf16_chunks(dev, long_case, K):
    say(f"config long bf16 b=1 d=2048 N=16 L=65536 chunk={K or 'auto'} (every element)")
    inp, yr, hr = long_case
    y, h = run_gpu(inp, dev, K)
    ey = floored_err(to_f32(y), yr)
    eh = floored_err(to_f32(h), hr)   # float32 and bfloat16 convert to float32 exactly
    say(f"  err y={ey:.3e} last_state={eh:.3e} (tol {TOL['bf16']})")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_config_bigstate_f32_full(dev):
    say("config big-state f32 b=4 d=2048 N=256 L=4096 (every element)")
    inp = ssm_inputs.make_scan_inputs(**ssm_inputs.CONFIGS["c4_bigstate_f32"])
    check_full(inp, dev)


@pytest.mark.parametrize("gate", [False, True])
def test_config_decode_f32_full(dev, gate):
    import torch
    say(f"config decode f32 256x5120xN=16 gate={gate} (all channels)")
    inp = ssm_inputs.make_update_inputs(256, 5120, 16, gate=gate)
    st = to_device(inp["state"], dev)
    y = ssm.ssm_state_update(st, *(to_device(inp[k], dev) for k in ("u", "delta", "A", "B",
                                                                    "C", "D", "z")))
    torch.cuda.synchronize()
    sr, yr = oracle.state_update(inp["state"], *(ssm_inputs.to_f64(inp[k]) for k in
                                                 ("u", "delta", "A", "B", "C", "D", "z")))
    es, ey = floored_err(to_f64(st), sr), floored_err(to_f64(y), yr)
    say(f"  err state={es:.3e} y={ey:.3e}")
    assert es <= TOL["f32"] and ey <= TOL["f32"]


# ------------------------------------------------------------ shapes and edges

@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,K", [
    ((1, 1, 16, 1), 0), ((1, 5, 16, 17), 16), ((2, 63, 16, 100), 32), ((1, 65, 16, 777), 64),
    ((3, 100, 16, 1000), 0), ((1, 64, 16, 1000), 48), ((2, 130, 16, 513), 0),
    ((1, 64, 1, 300), 0), ((1, 33, 3, 129), 16), ((2, 40, 8, 200), 0), ((1, 64, 17, 250), 32),
    ((1, 70, 32, 260), 0), ((1, 64, 48, 99), 16), ((1, 65, 100, 120), 0),
    ((2, 64, 256, 96), 32),
])
def test_shapes_full(dev, io, shape, K):
    batch, d_inner, N, L = shape
    say(f"shape b={batch} d={d_inner} N={N} L={L} K={K or 'auto'} io={io}")
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=batch * 7 + N, random_a=True)
    check_full(inp, dev, chunk_size=K)


@pytest.mark.parametrize("opts", [
    dict(D=None), dict(z=None), dict(delta_bias=None), dict(softplus=False),
    dict(D=None, z=None, delta_bias=None),
])
def test_optional_arguments(dev, opts):
    import torch
    say(f"optional arguments {sorted(opts)}")
    inp = ssm_inputs.make_scan_inputs(2, 96, 16, 300, gate=True, seed=21)
    if opts.get("softplus") is False:
        # without softplus the raw step size is used as is: make it positive
        # and moderate, and drop the (negative) bias
        inp["delta"] = ssm_inputs.encode(np.abs(ssm_inputs.to_f64(inp["delta"])) * 0.1, "f32")
        inp["delta_bias"] = None
    for k in ("D", "z", "delta_bias"):
        if k in opts:
            inp[k] = None
    if "softplus" in opts:
        inp["softplus"] = 0
    for K in (0, 64):
        check_full(inp, dev, chunk_size=K)
    y, h = run_gpu(inp, dev, last_state=False)
    assert h is None and torch.isfinite(y).all()


def test_empty_sequence_zeroes_last_state(dev):
    import torch
    u = torch.zeros((2, 8, 0), device=dev)
    A = -torch.ones((8, 16), device=dev)
    B = torch.zeros((2, 16, 0), device=dev)
    last = torch.full((2, 8, 16), 7.0, device=dev)
    y, h = ssm.ssm_scan_fwd(u, u, A, B, B, last_state=last)
    torch.cuda.synchronize()
    assert y.shape == (2, 8, 0) and torch.equal(h, torch.zeros_like(h))


# ------------------------------------------------------------ exactness

def integer_case(batch, d_inner, N, L, seed, impulses_only=False, K=16):
    rng = np.random.default_rng(seed)
    if impulses_only:
        u = np.zeros((batch, d_inner, L), np.float32)
        for k in range(1, L // K + 1):
            for t in (k * K - 1, k * K, k * K + 1):
                if t < L:
                    u[:, :, t] = rng.integers(-2, 3, (batch, d_inner))
        u[:, :, 0] = 1
    else:
        u = rng.integers(-2, 3, (batch, d_inner, L)).astype(np.float32)
    B = rng.integers(-2, 3, (batch, N, L)).astype(np.float32)
    C = rng.integers(-2, 3, (batch, N, L)).astype(np.float32)
    D = rng.integers(-2, 3, d_inner).astype(np.float32)
    return dict(u=u, delta=np.ones_like(u), A=np.zeros((d_inner, N), np.float32), B=B, C=C,
                D=D, z=None, delta_bias=None, softplus=0)


@pytest.mark.parametrize("K", [16, 32, 48, 64, 256, 0])
@pytest.mark.parametrize("shape", [(2, 70, 16, 1000), (1, 64, 32, 333), (1, 3, 5, 64)])
def test_integer_bit_exact_f32(dev, K, shape):
    """Decay 1, unit step, small integers: every value is an exact integer
    below 2^24, so chunk boundaries and state indexing must be bit-exact."""
    batch, d_inner, N, L = shape
    say(f"integer exact f32 shape={shape} K={K or 'auto'}")
    case = integer_case(batch, d_inner, N, L, seed=K + L)
    inp = {k: (ssm_inputs.encode(v, "f32") if isinstance(v, np.ndarray) and k in
               ("u", "delta", "B", "C") else v) for k, v in case.items()}
    inp["io_dtype"] = "f32"
    y, h = run_gpu(inp, dev, chunk_size=K)
    yr, hr = oracle.scan_fwd(case["u"], case["delta"], case["A"], case["B"], case["C"],
                             case["D"], softplus=False)
    assert np.array_equal(to_f64(y), yr)
    assert np.array_equal(to_f64(h), hr)


@pytest.mark.parametrize("K", [16, 64, 0])
def test_integer_bit_exact_bf16_impulses(dev, K):
    """bf16 I/O with impulses around every chunk boundary: results stay small
    integers, exact in bf16."""
    say(f"integer exact bf16 impulses K={K or 'auto'}")
    case = integer_case(1, 64, 16, 200, seed=5, impulses_only=True, K=16)
    case["B"] = np.clip(case["B"], -1, 1)
    case["C"] = np.clip(case["C"], -1, 1)
    inp = {k: (ssm_inputs.encode(v, "bf16") if k in ("u", "delta", "B", "C") else v)
           for k, v in case.items()}
    inp["io_dtype"] = "bf16"
    y, h = run_gpu(inp, dev, chunk_size=K)
    yr, hr = oracle.scan_fwd(case["u"], case["delta"], case["A"], case["B"], case["C"],
                             case["D"], softplus=False)
    assert np.max(np.abs(yr)) < 256
    assert np.array_equal(to_f64(y), yr)
    assert np.array_equal(to_f64(h), hr)


def test_deterministic_and_batch_permutation(dev):
    import torch
    say("determinism and batch permutation")
    inp = ssm_inputs.make_scan_inputs(3, 200, 16, 700, io_dtype="bf16", gate=True, seed=3)
    y1, h1 = run_gpu(inp, dev, chunk_size=64)
    y2, h2 = run_gpu(inp, dev, chunk_size=64)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    p = [2, 0, 1]
    perm = dict(inp)
    for k in ("u", "delta", "B", "C", "z"):
        perm[k] = np.ascontiguousarray(inp[k][p])
    yp, hp = run_gpu(perm, dev, chunk_size=64)
    assert torch.equal(yp, y1[p]) and torch.equal(hp, h1[p])


# ------------------------------------------------------------ special cases

def test_zero_step_gives_skip_only(dev):
    import torch
    inp = ssm_inputs.make_scan_inputs(1, 64, 16, 100, gate=False, seed=4)
    inp["delta"] = np.zeros_like(inp["delta"])
    inp["delta_bias"] = None
    y, h = run_gpu(inp, dev, softplus=0)
    D = inp["D"].astype(np.float32)[None, :, None]
    assert np.array_equal(to_f64(y), (D * inp["u"]).astype(np.float64))
    assert torch.equal(h, torch.zeros_like(h))


def test_gate_zero_gives_zero(dev):
    import torch
    inp = ssm_inputs.make_scan_inputs(1, 64, 16, 100, gate=True, seed=5)
    inp["z"] = np.zeros_like(inp["z"])
    y, _ = run_gpu(inp, dev)
    assert torch.equal(y.abs(), torch.zeros_like(y))


def test_underflowing_decay(dev):
    """dt |A| >= 100: exp underflows to 0 and y_t = dt u_t (C_t . B_t) + D u_t."""
    rng = np.random.default_rng(6)
    b, d, N, L = 1, 64, 16, 64
    u = rng.standard_normal((b, d, L)).astype(np.float32)
    inp = dict(u=u, delta=np.full_like(u, 50.0), A=np.full((d, N), -4.0, np.float32),
               B=rng.standard_normal((b, N, L)).astype(np.float32),
               C=rng.standard_normal((b, N, L)).astype(np.float32),
               D=rng.standard_normal(d).astype(np.float32), z=None, delta_bias=None,
               softplus=0, io_dtype="f32")
    y, _ = run_gpu(inp, dev)
    cb = np.sum(inp["C"][0].astype(np.float64) * inp["B"][0], axis=0)
    ref = 50.0 * u[0] * cb[None, :] + inp["D"][:, None] * u[0]
    assert floored_err(to_f64(y)[0], ref) < 1e-5
    assert np.isfinite(to_f64(y)).all()


def test_softplus_accuracy_sweep(dev):
    """N=1, A=0, B=C=u=1, D=0, L=1: y = softplus(raw), over raw in [-40, 40]."""
    import torch
    raw = np.linspace(-40, 40, 20001).astype(np.float32)
    d = raw.size
    inp = dict(u=np.ones((1, d, 1), np.float32), delta=raw.reshape(1, d, 1),
               A=np.zeros((d, 1), np.float32), B=np.ones((1, 1, 1), np.float32),
               C=np.ones((1, 1, 1), np.float32), D=None, z=None, delta_bias=None,
               softplus=1, io_dtype="f32")
    y, _ = run_gpu(inp, dev)
    x = raw.astype(np.float64)
    ref = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
    rel = np.max(np.abs(to_f64(y).ravel() - ref) / ref)
    say(f"  softplus max relative error {rel:.3e}")
    assert rel < 2e-6


def test_gate_accuracy_sweep(dev):
    """y = u * silu(z) with the scan reduced to the skip term."""
    z = np.linspace(-30, 30, 12001).astype(np.float32)
    d = z.size
    inp = dict(u=np.ones((1, d, 1), np.float32), delta=np.zeros((1, d, 1), np.float32),
               A=np.zeros((d, 1), np.float32), B=np.ones((1, 1, 1), np.float32),
               C=np.ones((1, 1, 1), np.float32), D=np.ones(d, np.float32),
               z=z.reshape(1, d, 1), delta_bias=None, softplus=0, io_dtype="f32")
    y, _ = run_gpu(inp, dev)
    x = z.astype(np.float64)
    ref = x / (1 + np.exp(-x))
    err = np.abs(to_f64(y).ravel() - ref) / np.maximum(np.abs(ref), 1e-30)
    say(f"  silu max relative error {err.max():.3e}")
    assert err.max() < 2e-6


def test_decode_repeated_equals_scan(dev):
    """L single-token updates from a zero state reproduce the scan."""
    import torch
    inp = ssm_inputs.make_scan_inputs(2, 96, 16, 64, gate=True, seed=8)
    y, h = run_gpu(inp, dev)
    f = decoded(inp)
    dt = np.log1p(np.exp(f["delta"] + inp["delta_bias"].astype(np.float64)[None, :, None]))
    t = {k: to_device(inp[k], dev) for k in ("u", "B", "C", "z")}
    dtg = torch.from_numpy(dt.astype(np.float32)).to(dev)
    A, D = to_device(inp["A"], dev), to_device(inp["D"], dev)
    state = torch.zeros((2, 96, 16), device=dev)
    ys = []
    for i in range(64):
        ys.append(ssm.ssm_state_update(state, t["u"][..., i].contiguous(),
                                       dtg[..., i].contiguous(), A,
                                       t["B"][..., i].contiguous(), t["C"][..., i].contiguous(),
                                       D, t["z"][..., i].contiguous()))
    torch.cuda.synchronize()
    yd = torch.stack(ys, dim=-1)
    assert floored_err(to_f64(yd), to_f64(y)) < 1e-5
    assert floored_err(to_f64(state), to_f64(h)) < 1e-5


@pytest.mark.parametrize("N", [1, 3, 4, 12, 16, 17, 20, 36, 64, 256])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_shapes(dev, N, io):
    import torch
    say(f"decode N={N} io={io}")
    inp = ssm_inputs.make_update_inputs(5, 67, N, io_dtype=io, seed=N)
    st = to_device(inp["state"], dev)
    y = ssm.ssm_state_update(st, *(to_device(inp[k], dev) for k in ("u", "delta", "A", "B",
                                                                    "C", "D", "z")))
    torch.cuda.synchronize()
    sr, yr = oracle.state_update(inp["state"], *(ssm_inputs.to_f64(inp[k]) for k in
                                                 ("u", "delta", "A", "B", "C", "D", "z")))
    assert floored_err(to_f64(st), sr) <= 1e-5
    assert floored_err(to_f64(y), yr) <= TOL[io]
