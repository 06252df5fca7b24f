"""GPU parity of the backward pass (ssm_scan_bwd) against the fp64 oracle's
reverse walk (oracle.scan_bwd, itself pinned to finite differences).

Every gradient is compared: du, ddelta, dz, dA, dB, dC, dD, ddelta_bias, dh0.
Cases: one chunk and many (chunk edges inside and on tile edges, ragged
tails), gate on and off, start state and upstream last-state gradient on and
off, d_state 1..16, fp32 and bf16 inputs; exact-integer inputs bit for bit;
run-to-run identity.
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

NAMES = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0")


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_case(dev, batch, d_inner, N, L, io, gate, with_state, K, seed, zoh=False):
    import torch
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=gate, seed=seed)
    rng = np.random.default_rng(seed + 100)
    dy = ssm_inputs.encode(rng.standard_normal((batch, d_inner, L)).astype(np.float32), io)
    h0 = rng.standard_normal((batch, d_inner, N)).astype(np.float32) if with_state else None
    dlast = rng.standard_normal((batch, d_inner, N)).astype(np.float32) if with_state else None
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    g = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    out = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], to_device(dy, dev),
                           t["D"], t["z"], t["delta_bias"], softplus=True, initial_state=g(h0),
                           dlast=g(dlast), chunk_size=K, zoh=zoh)
    torch.cuda.synchronize()
    f = decoded(inp)
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], ssm_inputs.to_f64(dy, io),
                          f["D"], f["z"], f["delta_bias"], softplus=True,
                          initial_state=None if h0 is None else h0.astype(np.float64),
                          dlast=None if dlast is None else dlast.astype(np.float64), zoh=zoh)
    errs = {}
    for k in NAMES:
        if out[k] is None or ref.get(k) is None:
            continue
        if k == "dh0" and h0 is None:
            continue
        errs[k] = floored_err(to_f64(out[k]), ref[k])
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return out, errs


# The gradients are computed in fp32 from the same (rounded) inputs as the
# oracle and written in fp32, so both I/O types are held to the fp32 bar.
GRAD_TOL = TOL["f32"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,K", [((2, 40, 16, 300), 0), ((2, 40, 16, 300), 16),
                                     ((1, 33, 5, 77), 32), ((3, 16, 1, 9), 0),
                                     ((2, 24, 16, 513), 64)])
@pytest.mark.parametrize("gate,with_state", [(True, True), (False, False)])
def test_backward_parity(dev, io, shape, K, gate, with_state):
    say(f"bwd io={io} shape={shape} K={K} gate={gate} state={with_state}")
    _, errs = run_case(dev, *shape, io, gate, with_state, K, seed=sum(shape) + K)
    for k, e in errs.items():
        assert e <= GRAD_TOL, (k, e)


def test_backward_mamba130m_layer(dev):
    """The Mamba-130M-shaped layer (2 x 1536 channels, N = 16, L = 2048,
    fp32, gate) with the library's own chunking, every gradient compared."""
    say("bwd mamba130m layer")
    _, errs = run_case(dev, 2, 1536, 16, 2048, "f32", True, True, 0, seed=5)
    for k, e in errs.items():
        assert e <= GRAD_TOL, (k, e)


def test_backward_integer_bit_exact_and_deterministic(dev):
    """Exact-integer inputs (unit decay, integer u, B, C, D, dy, start state
    and last-state gradient, dt = 1): every gradient is an exact integer sum,
    so all must equal the oracle bit for bit whatever the chunking, and two
    runs must agree bit for bit."""
    import torch
    batch, d_inner, N, L = 2, 40, 16, 40
    rng = np.random.default_rng(17)
    ri = lambda *s: rng.integers(-2, 3, size=s).astype(np.float32)
    u, B, C, dy = ri(batch, d_inner, L), ri(batch, N, L), ri(batch, N, L), ri(batch, d_inner, L)
    D, h0, dlast = ri(d_inner), ri(batch, d_inner, N), ri(batch, d_inner, N)
    dt = np.ones((batch, d_inner, L), np.float32)
    A = np.zeros((d_inner, N), np.float32)
    ref = oracle.scan_bwd(u, dt, A, B, C, dy, D, softplus=False, initial_state=h0, dlast=dlast)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    first = None
    for K in (16, 32, 0):
        out = ssm.ssm_scan_bwd(g(u), g(dt), g(A), g(B), g(C), g(dy), g(D), softplus=False,
                               initial_state=g(h0), dlast=g(dlast), chunk_size=K)
        torch.cuda.synchronize()
        for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
            assert np.array_equal(to_f64(out[k]), ref[k]), (K, k)
        if first is None:
            first = out
    again = ssm.ssm_scan_bwd(g(u), g(dt), g(A), g(B), g(C), g(dy), g(D), softplus=False,
                             initial_state=g(h0), dlast=g(dlast), chunk_size=16)
    torch.cuda.synchronize()
    for k in ("du", "dA", "dB", "dC"):
        assert torch.equal(again[k], first[k])


# ---------------------------------------------------------------- packed sequences

LENS = {
    "mixed": [37, 0, 1, 200, 16, 0, 64, 5, 129, 0],
    "short": [3, 1, 4, 1, 5, 9, 2, 6],
    "one": [300],
    "edges": [8, 16, 24, 40, 64, 7],     # starts on 8-token tiles and 16/32/64-token chunks
    "leading_empty": [0, 0, 77, 50],
}


def run_packed_case(dev, lens, N, io, K, with_state, seed, gate=True, zoh=False):
    import torch
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    L, n, d_inner = int(cu[-1]), len(lens), 40
    inp = ssm_inputs.make_scan_inputs(1, d_inner, N, L, io_dtype=io, gate=gate, seed=seed)
    rng = np.random.default_rng(seed + 100)
    dy = ssm_inputs.encode(rng.standard_normal((1, d_inner, L)).astype(np.float32), io)
    h0 = rng.standard_normal((n, d_inner, N)).astype(np.float32) if with_state else None
    dlast = rng.standard_normal((n, d_inner, N)).astype(np.float32) if with_state else None
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    g = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    out = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], to_device(dy, dev),
                           t["D"], t["z"], t["delta_bias"], softplus=True, initial_state=g(h0),
                           dlast=g(dlast), chunk_size=K, cu_seqlens=g(cu), zoh=zoh)
    torch.cuda.synchronize()
    f = decoded(inp)
    ref = oracle.scan_bwd_varlen(f["u"], f["delta"], f["A"], f["B"], f["C"], cu,
                                 ssm_inputs.to_f64(dy, io), f["D"], f["z"], f["delta_bias"],
                                 softplus=True,
                                 initial_state=None if h0 is None else h0.astype(np.float64),
                                 dlast=None if dlast is None else dlast.astype(np.float64),
                                 zoh=zoh)
    errs = {}
    for k in NAMES:
        if out[k] is None or ref.get(k) is None or (k == "dh0" and h0 is None):
            continue
        errs[k] = floored_err(to_f64(out[k]), ref[k])
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return out, ref, errs


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 5])
@pytest.mark.parametrize("lens", sorted(LENS))
@pytest.mark.parametrize("K,with_state", [(0, True), (16, True), (32, False), (64, True)])
def test_backward_packed_sequences(dev, io, N, lens, K, with_state):
    say(f"bwd packed {lens} io={io} N={N} K={K} state={with_state}")
    _, _, errs = run_packed_case(dev, LENS[lens], N, io, K, with_state,
                                 seed=len(LENS[lens]) + N + K)
    for k, e in errs.items():
        assert e <= GRAD_TOL, (k, e)


def test_backward_packed_integer_bit_exact(dev):
    """Exact-integer inputs (unit decay, dt = 1) packed with boundaries inside
    tiles and chunks and an empty sequence: every gradient equals the oracle
    bit for bit at every chunking."""
    import torch
    lens = [5, 0, 12, 1, 30, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d_inner, N, L, n = 24, 16, int(cu[-1]), len(lens)
    rng = np.random.default_rng(23)
    ri = lambda *s: rng.integers(-2, 3, size=s).astype(np.float32)
    u, B, C, dy = ri(1, d_inner, L), ri(1, N, L), ri(1, N, L), ri(1, d_inner, L)
    D, h0, dlast = ri(d_inner), ri(n, d_inner, N), ri(n, d_inner, N)
    dt = np.ones((1, d_inner, L), np.float32)
    A = np.zeros((d_inner, N), np.float32)
    ref = oracle.scan_bwd_varlen(u, dt, A, B, C, cu, dy, D, softplus=False, initial_state=h0,
                                 dlast=dlast)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    for K in (16, 32, 0):
        out = ssm.ssm_scan_bwd(g(u), g(dt), g(A), g(B), g(C), g(dy), g(D), softplus=False,
                               initial_state=g(h0), dlast=g(dlast), chunk_size=K,
                               cu_seqlens=g(cu))
        torch.cuda.synchronize()
        for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
            assert np.array_equal(to_f64(out[k]), ref[k]), (K, k)


def test_backward_single_sequence_packing_equals_unpacked(dev):
    """One packed sequence covering the row gives the unpacked backward's
    gradients (the two instances agree to rounding)."""
    import torch
    inp = ssm_inputs.make_scan_inputs(1, 40, 16, 300, io_dtype="f32", gate=True, seed=31)
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    rng = np.random.default_rng(32)
    dy = torch.from_numpy(rng.standard_normal((1, 40, 300)).astype(np.float32)).to(dev)
    h0 = torch.from_numpy(rng.standard_normal((1, 40, 16)).astype(np.float32)).to(dev)
    dl = torch.from_numpy(rng.standard_normal((1, 40, 16)).astype(np.float32)).to(dev)
    cu = torch.tensor([0, 300], dtype=torch.int32, device=dev)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"], t["delta_bias"])
    a = ssm.ssm_scan_bwd(*args, initial_state=h0, dlast=dl, chunk_size=32)
    b = ssm.ssm_scan_bwd(*args, initial_state=h0, dlast=dl, chunk_size=32, cu_seqlens=cu)
    torch.cuda.synchronize()
    for k in NAMES:
        assert floored_err(to_f64(b[k]), to_f64(a[k])) <= 1e-6, k


# ---------------------------------------------------------------- zero-order hold

@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,K", [((2, 40, 16, 300), 0), ((2, 40, 16, 300), 16),
                                     ((1, 33, 5, 77), 32), ((3, 16, 1, 9), 0),
                                     ((2, 24, 16, 513), 64)])
@pytest.mark.parametrize("gate,with_state", [(True, True), (False, False)])
def test_backward_zoh(dev, io, shape, K, gate, with_state):
    """SSM_FLAG_ZOH: the input factor (e^{dt A} - 1) / A and its derivatives
    (e^{dt A} for ddt, dt^2 psi(dt A) for dA) in every gradient."""
    say(f"bwd zoh io={io} shape={shape} K={K} gate={gate} state={with_state}")
    _, errs = run_case(dev, *shape, io, gate, with_state, K, seed=sum(shape) + K + 1, zoh=True)
    for k, e in errs.items():
        assert e <= GRAD_TOL, (k, e)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [0, 16])
def test_backward_zoh_packed(dev, io, K):
    say(f"bwd zoh packed io={io} K={K}")
    _, _, errs = run_packed_case(dev, LENS["mixed"], 16, io, K, True, seed=41 + K, zoh=True)
    for k, e in errs.items():
        assert e <= GRAD_TOL, (k, e)


def test_backward_zoh_random_a_small_and_large_steps(dev):
    """A drawn at random (not -(n+1)), with rows whose dt*A lies around the
    series/closed-form switch of phi and psi (|dt A| near 1/2) and far beyond."""
    import torch
    inp = ssm_inputs.make_scan_inputs(2, 40, 16, 200, io_dtype="f32", gate=True, seed=51,
                                      random_a=True)
    rng = np.random.default_rng(52)
    A = inp["A"].copy()
    A[:8] *= 20.0                      # large |dt A|
    A[8:16] *= 0.01                    # tiny |dt A|
    inp["A"] = A
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    dy = rng.standard_normal((2, 40, 200)).astype(np.float32)
    out = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"],
                           torch.from_numpy(dy).to(dev), t["D"], t["z"], t["delta_bias"],
                           softplus=True, chunk_size=32, zoh=True)
    torch.cuda.synchronize()
    f = decoded(inp)
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], dy.astype(np.float64),
                          f["D"], f["z"], f["delta_bias"], softplus=True, zoh=True)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias"):
        e = floored_err(to_f64(out[k]), ref[k])
        say(f"  {k}={e:.2e}")
        assert e <= GRAD_TOL, (k, e)


# ---------------------------------------------------------------- full-size shapes

FULL_SHAPES = {
    "mamba2p8b": (8, 5120, 16, 2048),       # bf16 I/O, gate
    "long": (1, 2048, 16, 65536),           # bf16 I/O, gate
}


@pytest.mark.parametrize("name", sorted(FULL_SHAPES))
def test_backward_full_size_sampled(dev, name):
    """The Mamba-2.8B-shaped layer and the 64 Ki-token sequence, bf16 I/O,
    with the library's own chunking and the forward pass's checkpoints.

    Per-channel gradients (du, ddelta, dz of every token, dA, dD, d(bias))
    of 24 channels spread over the layer against the oracle on those channels
    alone (a channel's gradients depend on its own inputs and the shared B, C
    only).  dB and dC sum over all channels, which no sample can check: they
    are held to their additivity over channels instead, dB(all) = dB(first
    half) + dB(second half) with the halves run as layers of their own, and
    the first 24 channels' dB, dC against the oracle on those channels."""
    import torch
    batch, d_inner, N, L = FULL_SHAPES[name]
    say(f"bwd full size {name} {FULL_SHAPES[name]}")
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype="bf16", gate=True, seed=3)
    rng = np.random.default_rng(4)
    dy = ssm_inputs.encode(rng.standard_normal((batch, d_inner, L)).astype(np.float32), "bf16")
    dlast = rng.standard_normal((batch, d_inner, N)).astype(np.float32)
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    dy_t, dlast_t = to_device(dy, dev), g(dlast)

    def backward(ch):
        """The GPU backward of the layer restricted to channels ch (None: all)."""
        sel = (lambda x: x) if ch is None else (lambda x: x[:, ch].contiguous())
        pc = (lambda x: x) if ch is None else (lambda x: x[ch].contiguous())
        u, dl, z, dyc = sel(t["u"]), sel(t["delta"]), sel(t["z"]), sel(dy_t)
        A, D, bias, dls = pc(t["A"]), pc(t["D"]), pc(t["delta_bias"]), sel(dlast_t)
        ck = torch.empty(ssm.ckpt_shape(batch, u.shape[1], L), dtype=torch.float32, device=dev)
        ssm.ssm_scan_fwd(u, dl, A, t["B"], t["C"], D, z, bias, ckpt=ck)
        out = ssm.ssm_scan_bwd(u, dl, A, t["B"], t["C"], dyc, D, z, bias, dlast=dls, ckpt=ck)
        torch.cuda.synchronize()
        return out

    full = backward(None)
    half = d_inner // 2
    lo = backward(torch.arange(0, half, device=dev))
    hi = backward(torch.arange(half, d_inner, device=dev))
    for k in ("dB", "dC"):
        e = floored_err(to_f64(lo[k]) + to_f64(hi[k]), to_f64(full[k]))
        say(f"  {k} additivity over channel halves: {e:.2e}")
        assert e <= GRAD_TOL, k

    ch = np.linspace(0, d_inner - 1, 24).astype(np.int64)
    f = decoded(inp)
    ref = oracle.scan_bwd(f["u"][:, ch], f["delta"][:, ch], f["A"][ch], f["B"], f["C"],
                          ssm_inputs.to_f64(dy, "bf16")[:, ch], f["D"][ch], f["z"][:, ch],
                          f["delta_bias"][ch], softplus=True,
                          dlast=dlast[:, ch].astype(np.float64))
    errs = {}
    for k in ("du", "ddelta", "dz"):
        errs[k] = floored_err(to_f64(full[k])[:, ch], ref[k])
    for k in ("dA", "dD", "ddelta_bias"):
        errs[k] = floored_err(to_f64(full[k])[ch], ref[k])
    first = np.arange(24)
    sub = backward(torch.from_numpy(first).to(dev))
    ref0 = oracle.scan_bwd(f["u"][:, first], f["delta"][:, first], f["A"][first], f["B"], f["C"],
                           ssm_inputs.to_f64(dy, "bf16")[:, first], f["D"][first],
                           f["z"][:, first], f["delta_bias"][first], softplus=True,
                           dlast=dlast[:, first].astype(np.float64))
    for k in ("dB", "dC"):
        errs[k + "(24 ch)"] = floored_err(to_f64(sub[k]), ref0[k])
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= GRAD_TOL, (k, e)


# ---------------------------------------------------------------- d_state > 16

@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,zoh,K", [(17, False, 0), (32, False, 64), (40, True, 0),
                                     (64, False, 32), (256, False, 0)])
@pytest.mark.parametrize("gate,with_state", [(True, True), (False, False)])
def test_backward_state_groups(dev, io, N, zoh, K, gate, with_state):
    """d_state above 16: the 16-state pass per group of 16 states, the groups'
    per-token sums added (D's terms once), the padded states of a last partial
    group left out.  Every gradient against the oracle's reverse walk."""
    d_inner, L = (24, 200) if N > 64 else (40, 300)
    say(f"bwd state groups N={N} io={io} zoh={zoh} K={K} gate={gate} state={with_state}")
    _, errs = run_case(dev, 2, d_inner, N, L, io, gate, with_state, K, seed=N + K, zoh=zoh)
    for k, e in errs.items():
        assert e <= GRAD_TOL, (k, e)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,zoh,P", [
    ((1, 8192, 64, 128), False, 4),   # four groups in one launch
    ((1, 8192, 80, 96), False, 4),    # five groups: a launch of four, then one
    ((2, 4096, 48, 64), False, 3),    # three groups side by side, two batch rows
    ((1, 8192, 32, 64), True, 2),     # zero-order hold (one wavefront per SIMD): two
])
@pytest.mark.parametrize("gate,with_state", [(True, True), (False, False)])
def test_backward_state_groups_side_by_side(dev, io, shape, zoh, P, gate, with_state):
    """d_state above 16 with enough channel blocks that P groups of 16
    states fill the GPU together: they run side by side in one launch, each
    over the whole sequence, writing du, ddelta and dz to a workspace slot per
    group; the slots are summed at the end.  Every gradient against the
    oracle's reverse walk."""
    batch, d_inner, N, L = shape
    d = ssm.make_desc(batch, d_inner, N, L, 1 if io == "bf16" else 0, 0,
                      ssm.SSM_FLAG_ZOH if zoh else 0)
    need = ssm.load_library().ssm_scan_bwd_workspace_bytes(ctypes.byref(d))
    # the groups' slots of du, ddelta and dz are part of the workspace
    assert need >= 3 * ((N + 15) // 16) * batch * d_inner * L * 4
    say(f"bwd state groups side by side shape={shape} io={io} zoh={zoh} P={P} gate={gate} "
        f"state={with_state}")
    _, errs = run_case(dev, batch, d_inner, N, L, io, gate, with_state, 0,
                       seed=N + L + batch, zoh=zoh)
    for k, e in errs.items():
        assert e <= GRAD_TOL, (k, e)


def test_backward_state_groups_integer_bit_exact(dev):
    """Exact-integer inputs with 48 states (three groups of 16, the later two
    adding their du, ddelta and dz to the first's in place): every gradient
    equals the oracle bit for bit, and two runs agree bit for bit."""
    import torch
    batch, d_inner, N, L = 2, 24, 48, 40
    rng = np.random.default_rng(29)
    ri = lambda *s: rng.integers(-2, 3, size=s).astype(np.float32)
    u, B, C, dy = ri(batch, d_inner, L), ri(batch, N, L), ri(batch, N, L), ri(batch, d_inner, L)
    D, h0, dlast = ri(d_inner), ri(batch, d_inner, N), ri(batch, d_inner, N)
    dt = np.ones((batch, d_inner, L), np.float32)
    A = np.zeros((d_inner, N), np.float32)
    ref = oracle.scan_bwd(u, dt, A, B, C, dy, D, softplus=False, initial_state=h0, dlast=dlast)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    say(f"bwd state groups, integers, N={N}")
    out = ssm.ssm_scan_bwd(g(u), g(dt), g(A), g(B), g(C), g(dy), g(D), softplus=False,
                           initial_state=g(h0), dlast=g(dlast))
    again = ssm.ssm_scan_bwd(g(u), g(dt), g(A), g(B), g(C), g(dy), g(D), softplus=False,
                             initial_state=g(h0), dlast=g(dlast))
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        assert np.array_equal(to_f64(out[k]), ref[k]), k
        assert torch.equal(out[k], again[k]), k

