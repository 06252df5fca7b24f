"""GPU parity of the in-wave scan (chunks of 128 or 256 tokens run in sequence
on one wavefront per channel, each chunk scanned by 16 time segments in
parallel) against the fp64 oracle, through the C ABI.

The library runs it for calls without packed sequences, the fused
convolution or checkpoints, when the caller asks for chunks of 128 or 256
tokens, or by its own choice when the channels are 1024 to 8192.  Cases:
whole and partial chunks, rows whose length is not a multiple of 16 (the
element path), channel counts that leave a workgroup part empty, d_state
below 16, optional arguments, start states, the zero-order-hold term, and
exact-integer inputs bit for bit.
"""
import ctypes
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


def plan_of(inp, K, zoh=False):
    batch, d_inner, N, L = inp["u"].shape[0], inp["u"].shape[1], inp["A"].shape[1], \
        inp["u"].shape[2]
    d = ssm.make_desc(batch, d_inner, N, L, 1 if inp["io_dtype"] == "bf16" else 0, K,
                      ssm.SSM_FLAG_ZOH if zoh else 0)
    return ssm.load_library().ssm_scan_plan(ctypes.byref(d)).decode()


def run_and_check(dev, inp, K, zoh=False, h0=None, softplus=None, tol=None):
    import torch
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    sp = bool(inp["softplus"] if softplus is None else softplus)
    h0t = to_device(h0, dev) if h0 is not None else None
    plan = plan_of(inp, K, zoh)
    assert plan.startswith("in-wave"), plan
    y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            t["delta_bias"], softplus=sp, chunk_size=K, zoh=zoh,
                            initial_state=h0t)
    torch.cuda.synchronize()
    f = decoded(inp)
    yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], softplus=sp, zoh=zoh,
                             initial_state=None if h0 is None else h0.astype(np.float64))
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    tol = tol or TOL[inp["io_dtype"]]
    say(f"  plan '{plan}': err y={ey:.3e} last_state={eh:.3e} (tol {tol})")
    assert ey <= tol and eh <= tol
    return y, h


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,K", [
    ((1, 4, 16, 256), 256),      # one whole chunk, one workgroup
    ((1, 5, 16, 300), 256),      # partial workgroup, partial chunk, element path
    ((2, 64, 16, 1000), 128),    # ragged tail, element path
    ((2, 64, 16, 1024), 128),    # whole chunks, 16-byte accesses
    ((1, 33, 5, 513), 256),      # d_state 5
    ((1, 8, 1, 4096), 256),      # d_state 1, many chunks
    ((3, 22, 12, 2000), 128),    # d_state 12, batch rows
    ((2, 600, 16, 2048), 0),     # the library's choice: 1200 channels, chunks of 256
    ((1, 3072, 16, 512), 0),     # the library's choice: 3072 channels, chunks of 128
    ((1, 1024, 12, 777), 0),     # the library's choice, element path
    ((1, 20, 9, 1024), 256),     # buffer views: partial workgroup, B/C rows past d_state 9 read as zeros
    ((2, 22, 3, 2048), 128),     # buffer views, segments of 8: partial workgroup, d_state 3
])
def test_tscan_shapes(dev, io, shape, K):
    batch, d_inner, N, L = shape
    say(f"in-wave b={batch} d={d_inner} N={N} L={L} K={K or 'auto'} io={io}")
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=batch * 11 + N + L, random_a=True)
    run_and_check(dev, inp, K)


@pytest.mark.parametrize("K", [128, 256])
@pytest.mark.parametrize("opts", [
    dict(D=None), dict(z=None), dict(delta_bias=None), dict(softplus=False),
    dict(D=None, z=None, delta_bias=None),
])
def test_tscan_optional_arguments(dev, K, opts):
    say(f"in-wave optional arguments {sorted(opts)} K={K}")
    inp = ssm_inputs.make_scan_inputs(2, 36, 16, 700, gate=True, seed=31)
    if opts.get("softplus") is False:
        inp["delta"] = ssm_inputs.encode(np.abs(ssm_inputs.to_f64(inp["delta"])) * 0.1, "f32")
        inp["delta_bias"] = None
    for k in ("D", "z", "delta_bias"):
        if k in opts:
            inp[k] = None
    if "softplus" in opts:
        inp["softplus"] = 0
    run_and_check(dev, inp, K)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [128, 256])
def test_tscan_initial_state(dev, io, K):
    say(f"in-wave start states io={io} K={K}")
    inp = ssm_inputs.make_scan_inputs(2, 40, 16, 1000, io_dtype=io, gate=True, seed=41)
    h0 = np.random.default_rng(42).standard_normal((2, 40, 16)).astype(np.float32)
    run_and_check(dev, inp, K, h0=h0)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,K", [((2, 50, 16, 600), 128), ((1, 64, 7, 1024), 256),
                                     ((2, 1000, 16, 640), 0)])
def test_tscan_zoh(dev, io, shape, K):
    batch, d_inner, N, L = shape
    say(f"in-wave zero-order hold b={batch} d={d_inner} N={N} L={L} K={K or 'auto'} io={io}")
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=N + L)
    run_and_check(dev, inp, K, zoh=True)


def integer_inputs(batch, d_inner, N, L, seed):
    rng = np.random.default_rng(seed)
    u = rng.integers(-2, 3, (batch, d_inner, L)).astype(np.float32)
    return dict(u=u, delta=np.ones_like(u), A=np.zeros((d_inner, N), np.float32),
                B=rng.integers(-2, 3, (batch, N, L)).astype(np.float32),
                C=rng.integers(-2, 3, (batch, N, L)).astype(np.float32),
                D=rng.integers(-2, 3, d_inner).astype(np.float32), z=None, delta_bias=None,
                softplus=0, io_dtype="f32")


@pytest.mark.parametrize("shape,K", [((2, 70, 16, 1000), 128), ((1, 64, 9, 333), 256),
                                     ((1, 1100, 16, 700), 0), ((2, 1500, 3, 1024), 0)])
def test_tscan_integers_bit_exact(dev, shape, K):
    """Decay 1, unit step, small integers: every partial sum is an exact
    integer, so the segment scan and the chunk-to-chunk carry must reproduce
    the sequential result bit for bit."""
    import torch
    batch, d_inner, N, L = shape
    say(f"in-wave integers b={batch} d={d_inner} N={N} L={L} K={K or 'auto'}")
    case = integer_inputs(batch, d_inner, N, L, seed=L + N)
    assert plan_of(case, K).startswith("in-wave")
    t = {k: to_device(case[k], dev) for k in ("u", "delta", "A", "B", "C", "D")}
    y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], None, None,
                            softplus=False, chunk_size=K)
    torch.cuda.synchronize()
    yr, hr = oracle.scan_fwd(case["u"], case["delta"], case["A"], case["B"], case["C"],
                             case["D"], softplus=False)
    assert np.array_equal(to_f64(y), yr)
    assert np.array_equal(to_f64(h), hr)


def sparse_integer_inputs(batch, d_inner, N, L, seed, n_imp=12):
    """Decay 1, unit step; u holds n_imp impulses of +-1 per channel, B and C
    take -1, 0 or 1 at every token, D small integers.  Every state is an
    integer of magnitude <= n_imp and every y one of magnitude <= N n_imp + 2
    (< 256 here): exact in bf16, while every tile's B and C rows differ."""
    rng = np.random.default_rng(seed)
    u = np.zeros((batch, d_inner, L), np.float32)
    pos = rng.integers(0, L, (batch, d_inner, n_imp))
    np.put_along_axis(u, pos, rng.choice(np.array([-1.0, 1.0], np.float32),
                                         (batch, d_inner, n_imp)), axis=2)
    return dict(u=u, delta=np.ones_like(u), A=np.zeros((d_inner, N), np.float32),
                B=rng.integers(-1, 2, (batch, N, L)).astype(np.float32),
                C=rng.integers(-1, 2, (batch, N, L)).astype(np.float32),
                D=rng.integers(-2, 3, d_inner).astype(np.float32))


@pytest.mark.parametrize("shape", [
    (1, 8, 16, 256),       # one tile
    (1, 13, 16, 512),      # two tiles; the second workgroup has 5 channels of 8
    (2, 16, 16, 800),      # three tiles and a ragged fourth, 16-byte accesses
    (2, 16, 16, 808),      # the same, element path (L not a multiple of 16)
    (1, 24, 16, 1280),     # five tiles
    (1, 64, 16, 16384),    # 64 tiles, 8 workgroups
    (1, 9, 5, 1300),       # d_state 5
])
def test_tscan_bf16_segments16_bit_exact(dev, shape):
    """bf16 I/O with segments of 16: each tile stages the next tile's B and C
    into the third of three LDS buffers and the wavefronts order their reads
    through event counters (no barrier per tile).  A row read from the wrong
    buffer or before it is written changes y; integer inputs make every value
    exact, so y and the last state must equal the oracle bit for bit."""
    import torch
    batch, d_inner, N, L = shape
    say(f"in-wave bf16 segments of 16, integers b={batch} d={d_inner} N={N} L={L}")
    case = sparse_integer_inputs(batch, d_inner, N, L, seed=L + d_inner)
    enc = {k: ssm_inputs.encode(case[k], "bf16") for k in ("u", "delta", "B", "C")}
    plan = ssm.scan_plan(batch, d_inner, N, L, 1, 256)
    assert plan.startswith("in-wave") and "segments of 16" in plan, plan
    t = {k: to_device(v, dev) for k, v in enc.items()}
    t.update({k: to_device(case[k], dev) for k in ("A", "D")})
    for rep in range(2):
        y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], None,
                                None, softplus=False, chunk_size=256)
        torch.cuda.synchronize()
        yr, hr = oracle.scan_fwd(case["u"], case["delta"], case["A"], case["B"], case["C"],
                                 case["D"], softplus=False)
        assert np.max(np.abs(yr)) < 256
        assert np.array_equal(to_f64(y), yr), rep
        assert np.array_equal(to_f64(h), hr), rep


def test_tscan_deterministic_and_matches_chunked(dev):
    """Run to run bit-identical; within the float32 bar of the two-pass
    chunked schedule on the same inputs (chunks of 512)."""
    import torch
    inp = ssm_inputs.make_scan_inputs(2, 48, 16, 2048, io_dtype="f32", gate=True, seed=51)
    y1, h1 = run_and_check(dev, inp, 256)
    y2, h2 = run_and_check(dev, inp, 256)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    y3, h3 = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                              t["delta_bias"], chunk_size=512)
    torch.cuda.synchronize()
    assert floored_err(to_f64(y3), to_f64(y1)) < 2e-5
    assert floored_err(to_f64(h3), to_f64(h1)) < 2e-5
