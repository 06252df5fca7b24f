"""GPU tests of the forward pass's checkpoints (ssm_scan_fwd_ckpt) and of the
backward pass that reads them instead of recomputing the forward sweep.

A checkpoint is the state entering an 8-token tile of a (batch, channel) row.
It is compared with the fp64 oracle's state after the tokens before the tile
(the last state of the oracle scan over that prefix, of the tile's own
sequence when sequences are packed).  A tile that starts a sequence is not
compared: the backward restarts such a tile from the sequence's start state
and never reads its checkpoint.

Every forward schedule writes them: the chunked passes, the one-launch
chunked path, the balanced serial walks and the in-wave scan.  The backward
with checkpoints is held to the oracle's gradients at the same bar as the
backward without them, for one chunk and many, checkpoints from each of
those schedules, packed sequences and ZOH; the two backward results agree
with each other within that bar.
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


def tiles_to_check(n_ck, K):
    """Every tile of a short row; of a long one the first few, those around
    each chunk edge, the last, and an even spread in between."""
    if n_ck <= 64:
        return list(range(n_ck))
    pick = {0, 1, 2, n_ck - 2, n_ck - 1}
    if K:
        for e in range(K // 8, n_ck, K // 8):
            pick.update({e - 1, e, e + 1})
    pick.update(np.linspace(0, n_ck - 1, 24).astype(int).tolist())
    return sorted(i for i in pick if 0 <= i < n_ck)


def oracle_tile_states(f, h0, tiles, zoh, starts=None, h0_rows=None):
    """State entering tile i (token 8 i) per the oracle: the last state of the
    scan over the tokens of the tile's sequence before it.  Returns
    {i: (batch, d_inner, N)}; tiles that start a sequence are left out."""
    out = {}
    for i in tiles:
        t0 = 8 * i
        if starts is None:
            s0, init = 0, h0
        else:
            s = int(np.searchsorted(starts, t0, side="right")) - 1
            s0 = int(starts[s])
            if s0 == t0:
                continue
            init = None if h0_rows is None else h0_rows[s:s + 1]
        if t0 == s0:
            N = f["A"].shape[1]
            shape = (f["u"].shape[0], f["u"].shape[1], N)
            out[i] = np.zeros(shape) if init is None else np.array(init, dtype=np.float64)
            continue
        sl = slice(s0, t0)
        z = None if f["z"] is None else f["z"][:, :, sl]
        _, last = oracle.scan_fwd(f["u"][:, :, sl], f["delta"][:, :, sl], f["A"],
                                  f["B"][:, :, sl], f["C"][:, :, sl], f["D"], z,
                                  f["delta_bias"], softplus=True, initial_state=init, zoh=zoh)
        out[i] = last
    return out


def forward_with_ckpt(dev, t, N, L, K, zoh, h0=None, cu=None):
    import torch
    batch, d_inner = t["u"].shape[0], t["u"].shape[1]
    ck = torch.full(ssm.ckpt_shape(batch, d_inner, L), float("nan"), dtype=torch.float32,
                    device=dev)
    y, last = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                               t["delta_bias"], chunk_size=K, zoh=zoh, initial_state=h0,
                               cu_seqlens=cu, ckpt=ck)
    y2, last2 = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                 t["delta_bias"], chunk_size=K, zoh=zoh, initial_state=h0,
                                 cu_seqlens=cu)
    torch.cuda.synchronize()
    # writing the checkpoints changes nothing else
    assert torch.equal(y, y2) and torch.equal(last, last2)
    return ck


# (batch, d_inner, N, L, K): one chunk, 16- and 32-token chunks (edges on and
# between tiles of the backward), a ragged channel block and token tail, the
# element path (L % 4 != 0), the one-launch chunked path (K = 1024), and the
# vector path's buffer views with a ragged channel block and d_state 9 (the
# checkpoint stores of channels past d_inner dropped)
SHAPES = [(2, 40, 16, 300, 0), (2, 40, 16, 300, 16), (1, 33, 5, 301, 32),
          (3, 16, 1, 97, 0), (1, 24, 16, 3000, 1024), (2, 40, 9, 512, 64)]


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_forward_checkpoints_equal_oracle_states(dev, shape, io, zoh):
    import torch
    batch, d_inner, N, L, K = shape
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=sum(shape) + zoh)
    rng = np.random.default_rng(7)
    h0 = rng.standard_normal((batch, d_inner, N)).astype(np.float32)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    ck = forward_with_ckpt(dev, t, N, L, K, zoh, h0=torch.from_numpy(h0).to(dev))
    ck = ck.cpu().numpy().astype(np.float64)
    f = decoded(inp)
    tiles = tiles_to_check(ck.shape[2], K)
    ref = oracle_tile_states(f, h0.astype(np.float64), tiles, zoh)
    err = max(floored_err(ck[:, :, i, :N], r) for i, r in ref.items())
    say(f"ckpt {shape} io={io} zoh={zoh}: {len(ref)} tiles, err={err:.3e}")
    assert err <= TOL[io]
    assert np.all(ck[:, :, :, N:] == 0.0)   # states past d_state


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 24576, 16, 256), (2, 10240, 16, 512)])
def test_forward_checkpoints_split_walks(dev, shape, io):
    """Shapes that run the balanced serial walks (the blocks past the last
    whole round in two chunks, the second starting from the first's end
    state): checkpoints come from the same plan, those of the second chunk
    from its start state on.  Against the oracle's tile states, with start
    states; y and last_state bit-equal to the call without checkpoints."""
    import torch
    batch, d_inner, N, L = shape
    plan = ssm.scan_plan(batch, d_inner, N, L, 1 if io == "bf16" else 0)
    assert plan.startswith("one chunk, the blocks past"), plan
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=L + d_inner)
    h0 = np.random.default_rng(8).standard_normal((batch, d_inner, N)).astype(np.float32)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    ck = forward_with_ckpt(dev, t, N, L, 0, False, h0=torch.from_numpy(h0).to(dev))
    ck = ck.cpu().numpy().astype(np.float64)
    f = decoded(inp)
    tiles = tiles_to_check(ck.shape[2], 0)
    ref = oracle_tile_states(f, h0.astype(np.float64), tiles, False)
    err = max(floored_err(ck[:, :, i, :N], r) for i, r in ref.items())
    say(f"ckpt split walks {shape} io={io}: {len(ref)} tiles, err={err:.3e}")
    assert err <= TOL[io]


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 40, 16, 300, 256), (1, 33, 5, 301, 128),
                                   (1, 1024, 16, 512, 0)])
def test_forward_checkpoints_in_wave_scan(dev, shape, io, zoh):
    """Shapes that run the in-wave scan (chunks of 256 with a ragged token
    tail, chunks of 128 with d_state 5, and the library's own choice on 16-byte
    rows): its replay writes the checkpoints, two per segment of 16 tokens or
    one per segment of 8.  Against the oracle's tile states, with start
    states; y and last_state bit-equal to the call without checkpoints."""
    import torch
    batch, d_inner, N, L, K = shape
    plan = ssm.scan_plan(batch, d_inner, N, L, 1 if io == "bf16" else 0, K)
    assert plan.startswith("in-wave scan"), plan
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=sum(shape) + zoh)
    h0 = np.random.default_rng(9).standard_normal((batch, d_inner, N)).astype(np.float32)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    ck = forward_with_ckpt(dev, t, N, L, K, zoh, h0=torch.from_numpy(h0).to(dev))
    ck = ck.cpu().numpy().astype(np.float64)
    f = decoded(inp)
    tiles = tiles_to_check(ck.shape[2], K)
    ref = oracle_tile_states(f, h0.astype(np.float64), tiles, zoh)
    err = max(floored_err(ck[:, :, i, :N], r) for i, r in ref.items())
    say(f"ckpt in-wave scan {shape} io={io} zoh={zoh}: {len(ref)} tiles, err={err:.3e}")
    assert err <= TOL[io]
    assert np.all(ck[:, :, :, N:] == 0.0)   # states past d_state


def test_forward_checkpoints_packed_sequences(dev):
    import torch
    lens = [37, 0, 1, 200, 16, 0, 64, 5, 129, 0, 300]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    L, d_inner, N = int(cu[-1]), 40, 16
    inp = ssm_inputs.make_scan_inputs(1, d_inner, N, L, io_dtype="f32", gate=True, seed=11)
    h0 = np.random.default_rng(12).standard_normal((len(lens), d_inner, N)).astype(np.float32)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    for K in (0, 32):
        ck = forward_with_ckpt(dev, t, N, L, K, False, h0=torch.from_numpy(h0).to(dev),
                               cu=torch.from_numpy(cu).to(dev))
        ck = ck.cpu().numpy().astype(np.float64)
        ref = oracle_tile_states(decoded(inp), None, range(ck.shape[2]), False,
                                 starts=cu[:-1], h0_rows=h0.astype(np.float64))
        err = max(floored_err(ck[:, :, i, :N], r) for i, r in ref.items())
        say(f"ckpt packed K={K}: {len(ref)} tiles, err={err:.3e}")
        assert err <= TOL["f32"]
        assert np.isfinite(ck).all()   # every tile written, starts of sequences included


def backward_pair(dev, inp, io, N, L, K_fwd, K_bwd, zoh, with_state, cu=None, seed=0):
    """The backward without and with the forward's checkpoints, and the
    oracle's gradients."""
    import torch
    batch, d_inner = inp["u"].shape[0], inp["u"].shape[1]
    rows = batch if cu is None else len(cu) - 1
    rng = np.random.default_rng(seed + 100)
    dy = ssm_inputs.encode(rng.standard_normal((batch, d_inner, L)).astype(np.float32), io)
    h0 = rng.standard_normal((rows, d_inner, N)).astype(np.float32) if with_state else None
    dlast = rng.standard_normal((rows, d_inner, N)).astype(np.float32) if with_state else None
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    g = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    ck = forward_with_ckpt(dev, t, N, L, K_fwd, zoh, h0=g(h0), cu=g(cu))
    run = lambda c: ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                     to_device(dy, dev), t["D"], t["z"], t["delta_bias"],
                                     softplus=True, initial_state=g(h0), dlast=g(dlast),
                                     chunk_size=K_bwd, cu_seqlens=g(cu), zoh=zoh, ckpt=c)
    plain, fast = run(None), run(ck)
    torch.cuda.synchronize()
    f = decoded(inp)
    opt = dict(softplus=True, initial_state=None if h0 is None else h0.astype(np.float64),
               dlast=None if dlast is None else dlast.astype(np.float64), zoh=zoh)
    if cu is None:
        ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"],
                              ssm_inputs.to_f64(dy, io), f["D"], f["z"], f["delta_bias"], **opt)
    else:
        ref = oracle.scan_bwd_varlen(f["u"], f["delta"], f["A"], f["B"], f["C"], cu,
                                     ssm_inputs.to_f64(dy, io), f["D"], f["z"], f["delta_bias"],
                                     **opt)
    worst = {}
    for k in NAMES:
        if plain[k] is None or ref.get(k) is None or (k == "dh0" and h0 is None):
            continue
        e_fast = floored_err(to_f64(fast[k]), ref[k])
        e_pair = floored_err(to_f64(fast[k]), to_f64(plain[k]))
        worst[k] = (e_fast, e_pair, torch.equal(fast[k], plain[k]))
    say("  " + " ".join(f"{k}={a:.1e}/{b:.1e}{'=' if s else ''}"
                        for k, (a, b, s) in worst.items()))
    return worst


GRAD_TOL = TOL["f32"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,K_fwd,K_bwd", [((2, 40, 16, 300), 0, 0),
                                               ((2, 40, 16, 300), 16, 64),
                                               ((1, 33, 5, 301), 32, 16),
                                               ((1, 24, 16, 3000), 1024, 0),
                                               ((2, 40, 16, 300), 256, 0),
                                               ((1, 33, 5, 301), 128, 16)])
@pytest.mark.parametrize("zoh", [False, True])
def test_backward_with_checkpoints(dev, io, shape, K_fwd, K_bwd, zoh):
    batch, d_inner, N, L = shape
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=L + N + zoh)
    worst = backward_pair(dev, inp, io, N, L, K_fwd, K_bwd, zoh, True, seed=L)
    for k, (e_fast, e_pair, _) in worst.items():
        assert e_fast <= GRAD_TOL and e_pair <= GRAD_TOL, k


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,zoh", [((3, 12288, 16, 256), False), ((2, 24576, 16, 128), False),
                                       ((3, 6144, 16, 128), True)])
def test_backward_with_checkpoints_split(dev, io, shape, zoh):
    """More 16-channel blocks than one round of wavefront slots: given the
    checkpoints, the blocks of a whole round run as one chunk and the rest in
    chunks (two launches, the per-chunk sums over each channel's own chunk
    count).  Every gradient against the oracle and against the backward
    without checkpoints (which cuts every block into chunks)."""
    batch, d_inner, N, L = shape
    plan = ssm.scan_bwd_plan(batch, d_inner, N, L, 1 if io == "bf16" else 0, zoh=zoh,
                             with_ckpt=True)
    assert plan.startswith("the blocks of a whole round"), plan
    say(f"bwd with checkpoints, split: shape={shape} io={io} zoh={zoh}")
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=True,
                                      seed=L + d_inner + zoh)
    worst = backward_pair(dev, inp, io, N, L, 0, 0, zoh, True, seed=L + 1)
    for k, (e_fast, e_pair, _) in worst.items():
        assert e_fast <= GRAD_TOL and e_pair <= GRAD_TOL, k


@pytest.mark.parametrize("K_fwd,K_bwd", [(0, 0), (32, 16)])
@pytest.mark.parametrize("zoh", [False, True])
def test_backward_with_checkpoints_packed(dev, K_fwd, K_bwd, zoh):
    lens = [37, 0, 1, 200, 16, 0, 64, 5, 129, 0, 8, 16, 24, 40, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    L, N = int(cu[-1]), 16
    inp = ssm_inputs.make_scan_inputs(1, 40, N, L, io_dtype="f32", gate=True, seed=21 + zoh)
    worst = backward_pair(dev, inp, "f32", N, L, K_fwd, K_bwd, zoh, True, cu=cu, seed=21)
    for k, (e_fast, e_pair, _) in worst.items():
        assert e_fast <= GRAD_TOL and e_pair <= GRAD_TOL, k


def test_backward_with_checkpoints_deterministic(dev):
    """Two backward launches on one set of checkpoints give the same bits."""
    import torch
    batch, d_inner, N, L = 2, 64, 16, 1000
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype="bf16", gate=True, seed=5)
    t = {k: to_device(inp.get(k), dev) for k in KEYS}
    ck = forward_with_ckpt(dev, t, N, L, 0, False)
    dy = to_device(ssm_inputs.encode(np.random.default_rng(6).standard_normal(
        (batch, d_inner, L)).astype(np.float32), "bf16"), dev)
    run = lambda: ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"],
                                   t["z"], t["delta_bias"], ckpt=ck)
    a, b = run(), run()
    torch.cuda.synchronize()
    for k in NAMES:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
